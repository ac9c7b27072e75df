"""GPU parity on seeded random shapes, where the plan's rules meet: batch
1..8 with ragged lengths (single tokens included), 1..8 kv heads and groups
of 1..8 query heads, head dims 64 and 128, fp32 and bf16 KV, sinks and
windows from empty to longer than the context, automatic and explicit
split lengths (so one, two or four query heads per exact-merge block and
window splits from the batch-aware targets).  Each shape runs the fused
call and the standalone calls against the oracle (the bars of
test_gpu_parity); every third one also runs a three-layer chain
(alspec_spec_decode_layers) against the oracle and, bit for bit, against
single fused calls that use the chain's plan."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import attention_level_speculation_amd as al  # noqa: E402
import oracle  # noqa: E402
from synth import gen  # noqa: E402

from gpu_util import compare, run_fused, run_standalone, to_device  # noqa: E402

N_CASES = 24


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h = al.Handle(0)
    yield h
    h.close()


def _shape(i):
    rng = np.random.default_rng(2024 + i)
    B = int(rng.integers(1, 9))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([g for g in (1, 2, 4, 8) if g * Hkv <= 64]))
    D = int(rng.choice([64, 128]))
    dt = str(rng.choice(["f32", "bf16"]))
    L_cap = int(rng.choice([300, 2500, 6000]))
    lens = [int(x) for x in rng.integers(1, L_cap + 1, size=B)]
    lens[int(rng.integers(0, B))] = L_cap          # one entry at capacity
    S = int(rng.integers(0, 9))
    W = int(rng.choice([0, 1, 63, 128, 500, 2048]))
    if S + W == 0:
        W = 64
    lam = float(rng.choice([0.05, 0.1, 0.3]))
    split = int(rng.choice([0, 0, 256, 640]))
    wsplit = int(rng.choice([0, 0, 64, 200]))
    w = gen.Workload(f"rand{i}", B=B, Hq=G * Hkv, Hkv=Hkv, D=D, L_cap=L_cap,
                     seq_lens=lens, kv_dtype=dt, S=S, W=W, lam=lam,
                     needles=[1] * B, seed=300 + i)
    return w, split, wsplit


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(handle, i):
    w, split, wsplit = _shape(i)
    print(f"[case] rand{i}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} "
          f"{w.kv_dtype} lens={w.seq_lens} S={w.S} W={w.W} lam={w.lam} "
          f"split={split} wsplit={wsplit}", flush=True)
    p = al.params_for(w, split_tokens=split, window_split_tokens=wsplit)
    n_layers = 3 if i % 3 == 0 else 1
    refs, devs = [], []
    for layer in range(n_layers):
        q, k, v = gen.layer_inputs(w, layer)
        refs.append(oracle.spec_decode(q, k, v, w.seq_lens, w.S, w.W, w.lam))
        devs.append(to_device(q, k, v))
    got = run_fused(al, handle, p, *devs[0])
    compare(got, refs[0], w.kv_dtype, w.lam, f"rand{i}-fused")
    stand = run_standalone(al, handle, p, *devs[0])
    compare(stand, refs[0], w.kv_dtype, w.lam, f"rand{i}-standalone")
    if n_layers == 1:
        return
    wss = [al.alloc_workspace(p) for _ in range(3)]
    outs = [al.alloc_outputs(p) for _ in range(n_layers)]
    al.spec_decode_layers(handle, p, [(*d, o, wss[j % len(wss)]) for j, (d, o)
                                      in enumerate(zip(devs, outs))])
    torch.cuda.synchronize()
    ps = type(p).from_buffer_copy(p)
    ps.window_split_tokens = al.plan_splits(p, 0)[1][1]
    for j, d in enumerate(devs):
        got_j = {k_: v_.cpu().numpy() for k_, v_ in outs[j].items()}
        compare(got_j, refs[j], w.kv_dtype, w.lam, f"rand{i}-chain{j}")
        single = run_fused(al, handle, ps, *d)
        for key in single:
            assert np.array_equal(got_j[key], single[key]), (j, key)
