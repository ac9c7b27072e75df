"""The allocation-free fused call (alspec_spec_decode_noalloc), through the
C ABI, against the fused call with a caller-owned workspace: both run the
same kernels, so every output must be equal bit for bit.  Two calls in a
row share the library's static scratch, the second with a smaller input
(fewer users, shorter contexts, another head dim and KV dtype), so what the
first call left in the scratch must not leak into the second.  The outputs
are also held to the oracle's bars.  A workspace larger than the scratch
is refused before any GPU work."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import attention_level_speculation_amd as al  # noqa: E402
import oracle  # noqa: E402
from synth import gen  # noqa: E402

from gpu_util import compare, run_fused, to_device  # noqa: E402


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h = al.Handle(0)
    yield h
    h.close()


def _run_noalloc(h, p, dev, two_streams):
    out = al.alloc_outputs(p)
    if two_streams:
        sa, se = torch.cuda.Stream(), torch.cuda.Stream()
        sa.wait_stream(torch.cuda.current_stream())
        se.wait_stream(torch.cuda.current_stream())
        al.spec_decode_noalloc(h, p, *dev, out, sa, se)
        torch.cuda.current_stream().wait_stream(se)
        torch.cuda.current_stream().wait_stream(sa)
    else:
        al.spec_decode_noalloc(h, p, *dev, out)
    torch.cuda.synchronize()
    return {k_: v_.cpu().numpy() for k_, v_ in out.items()}


CASES = [
    # a larger input first, then a smaller one
    gen.Workload("noalloc_big", B=3, Hq=32, Hkv=8, D=128, L_cap=12000,
                 seq_lens=[12000, 7000, 9500], kv_dtype="bf16", S=4, W=1024,
                 lam=0.1, needles=[2, 0, 4], seed=91),
    gen.Workload("noalloc_small", B=2, Hq=8, Hkv=2, D=64, L_cap=3000,
                 seq_lens=[3000, 1700], kv_dtype="f32", S=4, W=128, lam=0.1,
                 needles=[1, 1], seed=92),
]


@pytest.mark.parametrize("overlap", [0, 1, 2])
def test_noalloc_matches_workspace_call(handle, overlap):
    for w in CASES:
        print(f"[case] noalloc {w.name} overlap={overlap}", flush=True)
        q, k, v = gen.layer_inputs(w, 0)
        dev = to_device(q, k, v)
        p = al.params_for(w, overlap=overlap)
        got = _run_noalloc(handle, p, dev, two_streams=overlap > 0)
        want = run_fused(al, handle, p, *dev, two_streams=overlap > 0)
        for key in want:
            assert np.array_equal(got[key], want[key]), (w.name, key)
        ref = oracle.spec_decode(q, k, v, w.seq_lens, w.S, w.W, w.lam)
        compare(got, ref, w.kv_dtype, w.lam, w.name + "-noalloc")


def test_noalloc_rejects_oversized_workspace(handle):
    """A plan whose workspace exceeds the 16 MiB scratch (two users at 128K
    with 64-token splits: 16.8 MiB) is refused with nothing enqueued.  The
    buffers have the plan's full sizes all the same."""
    p = al.make_params(2, 8, 1, 128, 131072, [131072] * 2, "bf16", 4, 2048,
                       0.1, split_tokens=64, window_split_tokens=64)
    assert al.workspace_size(p) > al.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((2, 8, 128), device="cuda")
    k = torch.zeros((2, 1, 131072, 128), dtype=torch.bfloat16, device="cuda")
    out = al.alloc_outputs(p)
    torch.cuda.synchronize()
    with pytest.raises(al.AlspecError) as e:
        al.spec_decode_noalloc(handle, p, q, k, k, out)
    assert e.value.status == 3
    assert "exceeds the static scratch" in al.last_error()
