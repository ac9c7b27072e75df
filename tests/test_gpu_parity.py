"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

Bars: per (user, layer) relative L2 error of O_exact and O_approx <= 1e-5
with fp32 KV and <= 2e-3 with bf16 KV (fp32 accumulation); |ratio - ratio
oracle| <= 1e-4; commit flags equal except where the oracle's ratio lies
within 1e-4 of lambda; lse within 1e-4 nats; the committed output is
exactly the approximate or the exact output.  Full-size cases use the
automatic split plan, the launch configuration the benchmark times.
"""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import attention_level_speculation_amd as al  # noqa: E402
import oracle  # noqa: E402
from synth import gen  # noqa: E402

from gpu_util import (compare, run_fused, run_standalone,  # noqa: E402
                      to_device)


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h = al.Handle(0)
    yield h
    h.close()


def _case(handle, w, layer=0, lam=None, two_streams=True, **pkw):
    lam = w.lam if lam is None else lam
    print(f"[case] {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} "
          f"lens={w.seq_lens[:4]}{'...' if w.B > 4 else ''} {w.kv_dtype} "
          f"S={w.S} W={w.W} lam={lam} layer={layer} {pkw}", flush=True)
    q, k, v = gen.layer_inputs(w, layer)
    ref = oracle.spec_decode(q, k, v, w.seq_lens, w.S, w.W, lam)
    p = al.params_for(w, lam=lam, **pkw)
    qd, kd, vd = to_device(q, k, v)
    got = run_fused(al, handle, p, qd, kd, vd, two_streams=two_streams)
    worst = compare(got, ref, w.kv_dtype, lam, w.name)
    print(f"[case] worst {worst} ratio gpu {got['ratio'][:4]} oracle "
          f"{ref['ratio'][:4]}", flush=True)
    return q, k, v, ref, got, p, (qd, kd, vd)


# ------------------------------------------------------ workload configs ---

def test_tiny_f32(handle):
    _case(handle, gen.tiny_f32_1k())


def test_tiny_f32_standalone_path(handle):
    w = gen.tiny_f32_1k()
    q, k, v = gen.layer_inputs(w, 0)
    ref = oracle.spec_decode(q, k, v, w.seq_lens, w.S, w.W, w.lam)
    p = al.params_for(w)
    qd, kd, vd = to_device(q, k, v)
    got = run_standalone(al, handle, p, qd, kd, vd)
    compare(got, ref, "f32", w.lam, "standalone")
    got2 = run_standalone(al, handle, p, qd, kd, vd, include_sink_window=True)
    compare(got2, ref, "f32", w.lam, "standalone-all-splits")
    # the exact splits recomputed over sink+window give the same bits
    assert np.array_equal(got["o_exact"], got2["o_exact"])
    fused = run_fused(al, handle, p, qd, kd, vd)
    assert np.array_equal(fused["o_approx"], got["o_approx"])
    # the standalone exact combine merges as the fused call does
    assert np.array_equal(fused["o_exact"], got["o_exact"])
    assert np.array_equal(fused["lse_exact"], got["lse_exact"])


@pytest.mark.parametrize("layer", [0, 1])
def test_llama8b_32k_layers(handle, layer):
    _case(handle, gen.llama8b_32k(), layer=layer)


def test_headline_128k_full_size(handle):
    _case(handle, gen.llama8b_128k(needles=4), layer=0)


@pytest.mark.parametrize("needles", [0, 16])
def test_headline_density_extremes_scaled(handle, needles):
    w = gen.scaled(gen.llama8b_128k(needles=needles), 20000)
    for layer in range(3):
        _case(handle, w, layer=layer)


def test_multiuser_ragged_full_size(handle):
    w = gen.multiuser_8b()
    q, k, v = gen.layer_inputs(w, 0)
    qd, kd, vd = to_device(q, k, v)
    for lam in (0.05, 0.10, 0.20):
        print(f"[case] multiuser lam={lam} lens={w.seq_lens}", flush=True)
        ref = oracle.spec_decode(q, k, v, w.seq_lens, w.S, w.W, lam)
        p = al.params_for(w, lam=lam)
        got = run_fused(al, handle, p, qd, kd, vd)
        compare(got, ref, "bf16", lam, f"multiuser lam={lam}")
        print(f"[case] commits {got['commit'].tolist()} oracle "
              f"{ref['commit'].tolist()}", flush=True)
    # the one-launch approximation (sequential mode) and the two-launch one
    # (overlapped modes) give the same bits with 8 users x 8 kv heads
    seq = run_fused(al, handle, al.params_for(w), qd, kd, vd)
    for ov in (1, 2):
        other = run_fused(al, handle, al.params_for(w, overlap=ov), qd, kd, vd)
        for key in seq:
            assert np.array_equal(seq[key], other[key]), (ov, key)
    alone = run_standalone(al, handle, al.params_for(w), qd, kd, vd)
    assert np.array_equal(alone["o_approx"], seq["o_approx"])
    assert np.array_equal(alone["o_exact"], seq["o_exact"])
    allsp = run_standalone(al, handle, al.params_for(w), qd, kd, vd,
                           include_sink_window=True)
    assert np.array_equal(allsp["o_exact"], seq["o_exact"])


def test_llama70b_full_size(handle):
    _case(handle, gen.llama70b_128k(), layer=0)


# ------------------------------------------------------------ edge cases ---

def _mk(name, B, Hq, Hkv, D, lens, dt, S, W, lam=0.1, needles=1, seed=7):
    return gen.Workload(name, B=B, Hq=Hq, Hkv=Hkv, D=D, L_cap=max(lens),
                        seq_lens=list(lens), kv_dtype=dt, S=S, W=W, lam=lam,
                        needles=[needles] * B, seed=seed)


MAX_B_LENS = [1, 2, 4, 5, 131, 132, 133] + [137 + 37 * i for i in range(57)]

EDGE = [
    # name, B, Hq, Hkv, D, lens, dtype, S, W, split, wsplit
    ("g1_d64_f32", 2, 4, 4, 64, [777, 1500], "f32", 4, 100, 0, 0),
    ("g2_d128_bf16", 2, 8, 4, 128, [3001, 65], "bf16", 4, 256, 0, 0),
    ("g4_d64_bf16", 3, 8, 2, 64, [2049, 1, 300], "bf16", 4, 128, 0, 0),
    ("g8_d128_f32", 1, 16, 2, 128, [5003], "f32", 4, 512, 256, 64),
    ("g8_d64_bf16", 2, 8, 1, 64, [4100, 999], "bf16", 2, 200, 0, 0),
    ("tiny_splits", 2, 8, 2, 128, [1234, 4321], "bf16", 4, 300, 64, 32),
    ("odd_splits", 1, 4, 2, 128, [6000], "f32", 3, 333, 777, 50),
    ("no_sink", 2, 8, 2, 128, [2000, 1500], "bf16", 0, 300, 0, 0),
    ("no_window", 2, 8, 2, 128, [2000, 1500], "bf16", 4, 0, 0, 0),
    ("short_inside_sink", 3, 8, 2, 64, [1, 2, 3], "f32", 4, 0, 0, 0),
    ("cover_exact", 2, 8, 2, 128, [132, 100], "bf16", 4, 128, 0, 0),
    ("window_only_long", 1, 8, 8, 128, [4096], "bf16", 0, 1, 0, 0),
    # maximum batch (64 users, ragged down to a single token, around the
    # sink + window boundary) and maximum kv heads
    ("max_batch_f32", 64, 8, 8, 64, MAX_B_LENS, "f32", 4, 128, 0, 0),
    ("max_batch_g4_bf16", 64, 32, 8, 128, MAX_B_LENS, "bf16", 4, 128, 0, 0),
    ("max_kv_heads", 1, 64, 64, 128, [1700], "bf16", 4, 128, 0, 0),
    # four query heads per exact-merge block (at least 128 (user, head)
    # pairs, every head's middle states in one merge round: up to 32 at
    # D = 64, 16 at D = 128), and one per block where a head has more than
    # a two-head round holds (32 at D = 128)
    ("nh4_d64_f32", 8, 16, 4, 64, [3000, 2500, 4000, 1800, 3500, 2200, 2900,
                                   4096], "f32", 4, 256, 256, 0),
    ("nh4_d128_bf16", 4, 32, 8, 128, [6000, 5000, 7000, 6500], "bf16", 4,
     512, 512, 0),
    ("nh1_many_middle", 4, 32, 8, 128, [9000] * 4, "bf16", 4, 256, 256, 0),
    # two per block (32 slots at D = 128) for a single entry
    ("nh2_d128_bf16", 1, 32, 8, 128, [40000], "bf16", 4, 1024, 2048, 0),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge_shapes(handle, case):
    name, B, Hq, Hkv, D, lens, dt, S, W, split, wsplit = case
    w = _mk(name, B, Hq, Hkv, D, lens, dt, S, W)
    q, k, v, ref, got, p, dev = _case(handle, w, split_tokens=split,
                                      window_split_tokens=wsplit)
    stand = run_standalone(al, handle, p, *dev)
    compare(stand, ref, dt, w.lam, name + "-standalone")


# Shapes that take the kernels' less common branches (plans computed on the
# host): the sink and window merge over more states than one memory round
# holds (a max pass, then rounds), the exact merge likewise over many middle
# states, and the standalone verify over more outputs per entry than its
# registers hold.
BRANCHES = [
    # name, B, Hq, Hkv, D, lens, dtype, S, W, split, wsplit
    # 70B shape at batch 1, automatic plan: 17 sink and window states
    # against 9 per round of an 8-head merge
    ("approx_rounds_g8_auto", 1, 64, 8, 128, [20000], "bf16", 4, 2048, 0, 0),
    # 33 states against 9 (G = 8) and against 18 (G = 4)
    ("approx_rounds_g8_w64", 1, 64, 8, 128, [20000], "bf16", 4, 2048, 0, 64),
    ("approx_rounds_g4_w64", 1, 32, 8, 128, [20000], "bf16", 4, 2048, 0, 64),
    # about 300 middle states per head against 64 per round, both dtypes
    ("exact_rounds_f32", 1, 8, 2, 128, [20000], "f32", 4, 1024, 64, 0),
    ("exact_rounds_bf16", 1, 8, 2, 128, [20000], "bf16", 4, 1024, 64, 0),
    ("exact_rounds_d64_f32", 1, 8, 2, 64, [20000], "f32", 4, 1024, 64, 0),
    # automatic plan: 75 middle states against 64
    ("exact_rounds_auto", 1, 8, 2, 128, [20000], "bf16", 4, 1024, 0, 0),
    # 16384 outputs per entry: the standalone verify's streaming form
    ("verify_large_entry", 2, 128, 16, 128, [700, 1500], "bf16", 4, 128, 0,
     0),
]


@pytest.mark.parametrize("case", BRANCHES, ids=[c[0] for c in BRANCHES])
def test_merge_and_verify_branches(handle, case):
    """Each branch shape through the fused call (two streams), the
    standalone calls (with the sink and window states from the
    approximation, and with every split recomputed), and a three-layer
    chain: every layer against the oracle, and the chain bit for bit
    against single fused calls with its plan."""
    name, B, Hq, Hkv, D, lens, dt, S, W, split, wsplit = case
    w = _mk(name, B, Hq, Hkv, D, lens, dt, S, W)
    q, k, v, ref, got, p, dev = _case(handle, w, split_tokens=split,
                                      window_split_tokens=wsplit)
    stand = run_standalone(al, handle, p, *dev)
    compare(stand, ref, dt, w.lam, name + "-standalone")
    allsp = run_standalone(al, handle, p, *dev, include_sink_window=True)
    compare(allsp, ref, dt, w.lam, name + "-standalone-all-splits")
    assert np.array_equal(allsp["o_exact"], got["o_exact"])
    assert np.array_equal(stand["o_approx"], got["o_approx"])
    devs = [dev] + [to_device(*gen.layer_inputs(w, l)) for l in (1, 2)]
    refs = [ref] + [oracle.spec_decode(*gen.layer_inputs(w, l), w.seq_lens,
                                       w.S, w.W, w.lam) for l in (1, 2)]
    wss = [al.alloc_workspace(p) for _ in range(3)]
    outs = [al.alloc_outputs(p) for _ in range(3)]
    al.spec_decode_layers(handle, p, [(*d, o, wss[j]) for j, (d, o) in
                                      enumerate(zip(devs, outs))])
    torch.cuda.synchronize()
    for j, d in enumerate(devs):
        got_j = {k_: v_.cpu().numpy() for k_, v_ in outs[j].items()}
        compare(got_j, refs[j], dt, w.lam, f"{name}-chain{j}")
        single = run_fused(al, handle, p, *d)
        for key in single:
            assert np.array_equal(got_j[key], single[key]), (j, key)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_full_cover_gives_ratio_exactly_zero(handle, dt):
    """S + W >= L: the middle is empty, the exact merge repeats the
    approximation's operations, so the outputs agree bit for bit and the
    ratio is exactly 0 (commit even at lambda = 0)."""
    w = _mk("cover", 3, 8, 2, 128, [200, 64, 131], dt, 4, 196, lam=0.0)
    q, k, v = gen.layer_inputs(w, 0)
    p = al.params_for(w, lam=0.0)
    dev = to_device(q, k, v)
    for two in (True, False):
        got = run_fused(al, handle, p, *dev, two_streams=two)
        assert np.array_equal(got["o_exact"], got["o_approx"])
        assert (got["ratio"] == 0).all() and (got["commit"] == 1).all()
    st = run_standalone(al, handle, p, *dev)
    assert np.array_equal(st["o_exact"], st["o_approx"])
    assert (st["ratio"] == 0).all() and (st["commit"] == 1).all()


def test_nan_user_discards_others_unchanged(handle):
    w = _mk("nan", 3, 8, 2, 128, [3000, 3000, 3000], "bf16", 4, 256)
    q, k, v = gen.layer_inputs(w, 0)
    p = al.params_for(w, lam=math.inf)
    base = run_fused(al, handle, p, *to_device(q, k, v))
    k2 = k.copy()
    v2 = v.copy()
    nan_bf16 = np.uint16(0x7FC0)
    k2[1, 0, 1500, 3] = nan_bf16       # middle key of entry 1
    v2[2, 1, 1, 0] = nan_bf16          # sink value of entry 2
    got = run_fused(al, handle, p, *to_device(q, k2, v2))
    assert got["commit"].tolist() == [1, 0, 0]
    assert math.isnan(got["ratio"][1]) and math.isnan(got["ratio"][2])
    for key in ("o_exact", "o_approx", "ratio", "o_committed"):
        assert np.array_equal(got[key][0], base[key][0])


def test_padding_rows_never_read(handle):
    """Rows at or beyond an entry's length hold NaN; nothing changes."""
    w = _mk("pad", 3, 8, 2, 128, [1000, 2500, 4096], "bf16", 4, 300)
    q, k, v = gen.layer_inputs(w, 0)
    k2 = k.copy()
    v2 = v.copy()
    for b, L in enumerate(w.seq_lens):
        k2[b, :, L:] = np.uint16(0x7FC0)
        v2[b, :, L:] = np.uint16(0x7FC0)
    p = al.params_for(w)
    a = run_fused(al, handle, p, *to_device(q, k, v))
    b_ = run_fused(al, handle, p, *to_device(q, k2, v2))
    for key in ("o_exact", "o_approx", "ratio", "commit"):
        assert np.array_equal(a[key], b_[key]), key


def test_lambda_extremes(handle):
    w = _mk("lam", 4, 8, 2, 64, [900, 1200, 50, 3000], "f32", 4, 60)
    q, k, v = gen.layer_inputs(w, 0)
    dev = to_device(q, k, v)
    g_inf = run_fused(al, handle, al.params_for(w, lam=math.inf), *dev)
    assert (g_inf["commit"] == 1).all()
    g_0 = run_fused(al, handle, al.params_for(w, lam=0.0), *dev)
    assert g_0["commit"].tolist() == [int(r == 0) for r in g_0["ratio"]]
    assert g_0["commit"][2] == 1  # L = 50 <= S + W: exact cover


def test_determinism_and_one_vs_two_streams(handle):
    w = gen.scaled(gen.llama8b_32k(), 9000, seq_lens=[9000])
    q, k, v = gen.layer_inputs(w, 0)
    p = al.params_for(w)
    dev = to_device(q, k, v)
    a = run_fused(al, handle, p, *dev, two_streams=True)
    b = run_fused(al, handle, p, *dev, two_streams=True)
    c = run_fused(al, handle, p, *dev, two_streams=False)
    d = run_fused(al, handle, al.params_for(w, overlap=1), *dev,
                  two_streams=True)
    e = run_fused(al, handle, al.params_for(w, overlap=2), *dev,
                  two_streams=True)
    f = run_fused(al, handle, al.params_for(w, overlap=2), *dev,
                  two_streams=False)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
        assert np.array_equal(a[key], c[key]), key
        assert np.array_equal(a[key], d[key]), key
        assert np.array_equal(a[key], e[key]), key
        assert np.array_equal(a[key], f[key]), key


def test_back_to_back_calls_share_workspace(handle):
    """Successive fused calls on one workspace and two streams, with
    different inputs, each match their own single-call result."""
    w = gen.scaled(gen.llama8b_32k(), 6000)
    p = al.params_for(w)
    ws = al.alloc_workspace(p)
    sa, se = torch.cuda.Stream(), torch.cuda.Stream()
    layers = [to_device(*gen.layer_inputs(w, l)) for l in range(3)]
    outs = []
    for dev in layers:
        o = al.alloc_outputs(p)
        al.spec_decode(handle, p, *dev, o, ws, sa, se)
        outs.append(o)
    torch.cuda.synchronize()
    for dev, o in zip(layers, outs):
        ref = run_fused(al, handle, p, *dev)
        for key in ref:
            assert np.array_equal(o[key].cpu().numpy(), ref[key]), key


@pytest.mark.parametrize("n_ws", [1, 2])
def test_pipelined_calls_match_single_calls(handle, n_ws):
    """Pipelined calls (exact passes back to back on one stream, merges on
    the other) over one shared or two alternating workspaces give exactly
    the single-call results."""
    w = gen.scaled(gen.llama8b_32k(), 6000)
    p = al.params_for(w, overlap=2)
    wss = [al.alloc_workspace(p) for _ in range(n_ws)]
    sa, se = torch.cuda.Stream(), torch.cuda.Stream()
    layers = [to_device(*gen.layer_inputs(w, l)) for l in range(5)]
    sa.wait_stream(torch.cuda.current_stream())
    se.wait_stream(torch.cuda.current_stream())
    outs = []
    for i, dev in enumerate(layers):
        o = al.alloc_outputs(p)
        al.spec_decode(handle, p, *dev, o, wss[i % n_ws], sa, se)
        outs.append(o)
    torch.cuda.synchronize()
    for dev, o in zip(layers, outs):
        ref = run_fused(al, handle, al.params_for(w), *dev)
        for key in ref:
            assert np.array_equal(o[key].cpu().numpy(), ref[key]), key


def test_pipelined_results_ordered_by_order_after_verify(handle):
    """Results of a pipelined call are read on the current stream after
    alspec_order_after_verify, with no device-wide synchronisation."""
    w = gen.scaled(gen.llama8b_32k(), 7000)
    q, k, v = gen.layer_inputs(w, 1)
    dev = to_device(q, k, v)
    ref = oracle.spec_decode(q, k, v, w.seq_lens, w.S, w.W, w.lam)
    p = al.params_for(w, overlap=2)
    ws = al.alloc_workspace(p)
    torch.cuda.synchronize()
    sa, se = torch.cuda.Stream(), torch.cuda.Stream()
    o = al.alloc_outputs(p)
    torch.cuda.synchronize()
    al.spec_decode(handle, p, *dev, o, ws, sa, se)
    cur = torch.cuda.current_stream()
    al.order_after_verify(handle, cur)
    cur.wait_stream(sa)
    got = {key: val.cpu().numpy() for key, val in o.items()}
    compare(got, ref, "bf16", w.lam, "pipelined-ordered")


def test_workspace_reuse_across_shapes(handle):
    big = gen.scaled(gen.llama8b_32k(), 8000)
    small = _mk("small", 2, 16, 2, 64, [700, 1300], "f32", 4, 64)
    pb = al.params_for(big)
    ps = al.params_for(small)
    ws = al.alloc_workspace(pb)
    assert ws.numel() >= al.workspace_size(ps)
    for w, p in ((big, pb), (small, ps), (big, pb)):
        q, k, v = gen.layer_inputs(w, 0)
        ref = oracle.spec_decode(q, k, v, w.seq_lens, w.S, w.W, w.lam)
        got = run_fused(al, handle, p, *to_device(q, k, v), ws=ws)
        compare(got, ref, w.kv_dtype, w.lam, "reuse " + w.name)


def test_invalid_workspace_rejected(handle):
    w = _mk("ws", 1, 8, 2, 128, [500], "bf16", 4, 64)
    q, k, v = gen.layer_inputs(w, 0)
    p = al.params_for(w)
    dev = to_device(q, k, v)
    ws = al.alloc_workspace(p)
    out = al.alloc_outputs(p)
    with pytest.raises(al.AlspecError) as e:
        al.spec_decode(handle, p, *dev, out, ws[:-256])
    assert e.value.status == 3
    with pytest.raises(al.AlspecError) as e:
        al.spec_decode(handle, p, *dev, out, ws[1:])
    assert e.value.status == 3


@pytest.mark.parametrize("overlap", [0, 1, 2])
def test_graph_capture_replays_match_eager(handle, overlap):
    """Three layers of fused calls captured into one HIP graph, replayed
    three times with the outputs cleared and another eager call on the same
    handle and workspace between replays: every replay equals the eager
    result bit for bit."""
    w = gen.scaled(gen.llama8b_32k(), 6000)
    p = al.params_for(w, overlap=overlap)
    print(f"[case] graph capture overlap={overlap} L=6000", flush=True)
    layers = [to_device(*gen.layer_inputs(w, l)) for l in range(3)]
    other = to_device(*gen.layer_inputs(w, 5))
    eager = [run_fused(al, handle, al.params_for(w), *dev) for dev in layers]
    eager_other = run_fused(al, handle, al.params_for(w), *other)
    # overlap 0 runs each call on stream_exact, so captured calls may share
    # a workspace; captured pipelined calls get one each (the library adds
    # no workspace ordering under capture)
    wss = [al.alloc_workspace(p) for _ in range(2 if overlap == 0 else 3)]
    outs = [al.alloc_outputs(p) for _ in layers]
    sa, se, cap = (torch.cuda.Stream(), torch.cuda.Stream(),
                   torch.cuda.Stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        sa.wait_stream(cap)
        se.wait_stream(cap)
        for i, dev in enumerate(layers):
            if overlap > 0 and i > 0:
                se.wait_stream(sa)    # q of layer i from approximation i-1
            al.spec_decode(handle, p, *dev, outs[i], wss[i % len(wss)],
                           sa, se)
        if overlap == 2:
            al.order_after_verify(handle, cap)
        cap.wait_stream(sa)
        cap.wait_stream(se)
    for rep in range(3):
        for o in outs:
            for t in o.values():
                t.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(cap):
            graph.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            for key in eager[i]:
                assert np.array_equal(o[key].cpu().numpy(), eager[i][key]), \
                    (rep, i, key)
        # eager work on the same handle and workspace between replays
        mid = run_fused(al, handle, p, *other, ws=wss[0])
        for key in mid:
            assert np.array_equal(mid[key], eager_other[key]), (rep, key)


def test_order_after_verify_under_capture_without_pipelined_calls(handle):
    """alspec_order_after_verify on a capturing stream when no pipelined
    call was captured: OK, nothing added; the graph replays normally."""
    x = torch.zeros(4, device="cuda")
    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        x.add_(1)
        al.order_after_verify(handle, cap)
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    assert x.tolist() == [2.0] * 4


def test_half_captured_call_rejected(handle):
    """A fused call whose approximation stream captures while its exact
    stream does not is refused before anything is enqueued."""
    w = _mk("halfcap", 1, 8, 2, 128, [900], "bf16", 4, 64)
    p = al.params_for(w, overlap=1)
    dev = to_device(*gen.layer_inputs(w, 0))
    ws = al.alloc_workspace(p)
    out = al.alloc_outputs(p)
    sa, se, cap = (torch.cuda.Stream(), torch.cuda.Stream(),
                   torch.cuda.Stream())
    x = torch.zeros(4, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    status = None
    with torch.cuda.graph(graph, stream=cap):
        x.add_(1)
        sa.wait_stream(cap)           # sa joins the capture, se does not
        try:
            al.spec_decode(handle, p, *dev, out, ws, sa, se)
        except al.AlspecError as e:
            status = e.status
        cap.wait_stream(sa)
    assert status == 1
    graph.replay()
    torch.cuda.synchronize()
    assert x.tolist() == [1.0] * 4


def _chain(handle, w, n_layers, n_ws=None, lam=None, overlap=0):
    lam = w.lam if lam is None else lam
    p = al.params_for(w, lam=lam, overlap=overlap)
    if n_ws is None:
        n_ws = al.LAYERS_WS_RING
    devs = [to_device(*gen.layer_inputs(w, l)) for l in range(n_layers)]
    wss = [al.alloc_workspace(p) for _ in range(n_ws)]
    outs = [al.alloc_outputs(p) for _ in range(n_layers)]
    return p, devs, wss, outs


def _single_with_chain_plan(p):
    """Params whose single calls use the plan spec_decode_layers takes for
    p (every entry point takes one plan), with the window split set
    explicitly, so the two agree bit for bit."""
    q = type(p).from_buffer_copy(p)
    q.window_split_tokens = al.plan_splits(p, 0)[1][1]
    assert al.plan_splits(q, 0)[1] == al.plan_splits(p, 0)[1]
    return q


@pytest.mark.parametrize("overlap", [0, 1])
@pytest.mark.parametrize("shape,n_layers", [
    ("bf16_g4", 1), ("bf16_g4", 2), ("bf16_g4", 5), ("f32_g2", 4),
    ("bf16_g8_ragged", 3), ("f32_d64_g1_ragged", 4),
    ("bf16_d64_g4_tiny", 3), ("bf16_g4", 8), ("bf16_g4", 9),
    ("bf16_g4", 17)])
def test_layers_chain_matches_single_calls(handle, shape, n_layers, overlap):
    """The layer-pipelined chain, in one launch (overlap 0: items taken
    from a queue, layers reusing a workspace waiting for the verify three
    layers back) and in one launch per layer (overlap 1), gives every layer
    exactly the outputs of a single fused call on its inputs with the same
    plan, with the smallest ring of workspaces allowed (each sized for the
    single calls' automatic plan): MFMA and
    VALU split kernels, head dims 128 and 64, users whose context is shorter
    than the sink plus window (no middle) or a single token."""
    w = {"bf16_g4": gen.scaled(gen.llama8b_32k(), 6000),
         "f32_g2": _mk("c2", 2, 8, 4, 128, [2500, 777], "f32", 4, 256),
         "bf16_g8_ragged": _mk("c8", 3, 16, 2, 128, [3000, 130, 5000],
                               "bf16", 4, 128),
         "f32_d64_g1_ragged": _mk("c1", 3, 4, 4, 64, [1777, 90, 2600],
                                  "f32", 4, 100),
         "bf16_d64_g4_tiny": _mk("c4", 4, 8, 2, 64, [1, 2049, 5, 300],
                                 "bf16", 4, 128)}[shape]
    print(f"[case] chain {shape} layers={n_layers} overlap={overlap}",
          flush=True)
    p, devs, wss, outs = _chain(handle, w, n_layers, overlap=overlap)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    al.spec_decode_layers(handle, p, [(*d, o, wss[j % len(wss)])
                                      for j, (d, o) in enumerate(zip(devs,
                                                                     outs))],
                          s)
    torch.cuda.synchronize()
    ps = _single_with_chain_plan(p)
    for j, d in enumerate(devs):
        ref = run_fused(al, handle, ps, *d)
        for key in ref:
            assert np.array_equal(outs[j][key].cpu().numpy(), ref[key]), \
                (j, key)
    # and against the oracle for the last layer
    q, k, v = gen.layer_inputs(w, n_layers - 1)
    ref = oracle.spec_decode(q, k, v, w.seq_lens, w.S, w.W, w.lam)
    compare({k_: v_.cpu().numpy() for k_, v_ in outs[-1].items()}, ref,
            w.kv_dtype, w.lam, "chain-last")


@pytest.mark.parametrize("pattern,n_layers", [
    ("ring4", 11), ("irregular", 12), ("ring3", 260)])
def test_layers_chain_workspace_patterns(handle, pattern, n_layers):
    """The one-launch chain with workspaces reused at distances other than
    three (a ring of four; an irregular assignment where a layer's latest
    predecessor on its workspace lies three to five layers back) and a chain
    longer than one launch's 256 layers: every layer bit for bit equal to a
    single fused call on its inputs."""
    w = _mk("wp", 4, 8, 2, 64, [1, 2049, 5, 300], "bf16", 4, 128)
    print(f"[case] chain workspaces {pattern} layers={n_layers}", flush=True)
    p = al.params_for(w)
    order = {"ring4": [j % 4 for j in range(n_layers)],
             "irregular": [0, 1, 2, 0, 3, 1, 4, 2, 0, 3, 1, 4],
             "ring3": [j % 3 for j in range(n_layers)]}[pattern]
    assert len(order) == n_layers
    for j, a in enumerate(order):
        assert a not in order[max(0, j - 2):j]
    wss = [al.alloc_workspace(p) for _ in range(max(order) + 1)]
    base = [to_device(*gen.layer_inputs(w, l)) for l in range(7)]
    devs = [base[j % 7] for j in range(n_layers)]
    outs = [al.alloc_outputs(p) for _ in range(n_layers)]
    al.spec_decode_layers(handle, p, [(*devs[j], outs[j], wss[order[j]])
                                      for j in range(n_layers)])
    torch.cuda.synchronize()
    ps = _single_with_chain_plan(p)
    refs = [run_fused(al, handle, ps, *d) for d in base]
    for j in range(n_layers):
        for key, want in refs[j % 7].items():
            assert np.array_equal(outs[j][key].cpu().numpy(), want), (j, key)


@pytest.mark.parametrize("shape,n_layers", [("llama8b_128k", 4),
                                             ("llama70b_128k", 3)])
def test_layers_chain_full_size(handle, shape, n_layers):
    """The chain at full size with the automatic plan, the configuration
    the benchmark times (launches with all four block ranges between the
    first and the last): every layer against the oracle, and bit for bit
    against single fused calls on its inputs with the chain's plan."""
    w = {"llama8b_128k": gen.llama8b_128k(needles=4),
         "llama70b_128k": gen.llama70b_128k()}[shape]
    p = al.params_for(w)
    print(f"[case] chain full size {shape} layers={n_layers}", flush=True)
    devs, refs = [], []
    for layer in range(n_layers):
        q, k, v = gen.layer_inputs(w, layer)
        refs.append(oracle.spec_decode(q, k, v, w.seq_lens, w.S, w.W, w.lam))
        devs.append(to_device(q, k, v))
        del q, k, v
    wss = [al.alloc_workspace(p) for _ in range(al.LAYERS_WS_RING)]
    outs = [al.alloc_outputs(p) for _ in range(n_layers)]
    al.spec_decode_layers(handle, p, [(*d, o, wss[j % len(wss)]) for j, (d, o)
                                      in enumerate(zip(devs, outs))])
    torch.cuda.synchronize()
    ps = _single_with_chain_plan(p)
    for j, d in enumerate(devs):
        got = {k_: v_.cpu().numpy() for k_, v_ in outs[j].items()}
        compare(got, refs[j], w.kv_dtype, w.lam, f"{shape} chain layer {j}")
        single = run_fused(al, handle, ps, *d)
        for key in single:
            assert np.array_equal(got[key], single[key]), (j, key)
        print(f"[case] layer {j} ratio {got['ratio'][:4]}", flush=True)


def test_layers_chain_graph_replays(handle):
    """A captured chain replays to the eager chain's outputs, three times,
    with eager chains on the same workspaces between replays."""
    w = gen.scaled(gen.llama8b_32k(), 5000)
    p, devs, wss, outs = _chain(handle, w, 4)
    eager = [al.alloc_outputs(p) for _ in devs]
    al.spec_decode_layers(handle, p, [(*d, o, wss[j % len(wss)]) for j, (d, o) in
                                      enumerate(zip(devs, eager))])
    torch.cuda.synchronize()
    want = [{k_: v_.cpu().numpy() for k_, v_ in o.items()} for o in eager]
    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        al.spec_decode_layers(handle, p, [(*d, o, wss[j % len(wss)]) for j, (d, o)
                                          in enumerate(zip(devs, outs))],
                              cap)
    for rep in range(3):
        for o in outs:
            for t in o.values():
                t.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(cap):
            graph.replay()
        torch.cuda.synchronize()
        for j, o in enumerate(outs):
            for key in want[j]:
                assert np.array_equal(o[key].cpu().numpy(), want[j][key]), \
                    (rep, j, key)
        al.spec_decode_layers(handle, p, [(*d, o, wss[j % len(wss)]) for j, (d, o)
                                          in enumerate(zip(devs, eager))])
        torch.cuda.synchronize()


def test_layers_ring_rule(handle):
    """Both forms refuse layers fewer than ALSPEC_LAYERS_WS_RING (3) apart
    on one workspace (status 3, nothing enqueued)."""
    w = _mk("ring", 1, 8, 2, 128, [1500], "bf16", 4, 128)
    dev = to_device(*gen.layer_inputs(w, 0))
    assert al.LAYERS_WS_RING == 3
    for overlap, ring, ok in ((0, 2, False), (0, 3, True),
                              (1, 2, False), (1, 3, True)):
        p = al.params_for(w, overlap=overlap)
        wss = [al.alloc_workspace(p) for _ in range(ring)]
        outs = [al.alloc_outputs(p) for _ in range(12)]
        layers = [(*dev, o, wss[j % ring]) for j, o in enumerate(outs)]
        if ok:
            al.spec_decode_layers(handle, p, layers)
            torch.cuda.synchronize()
        else:
            with pytest.raises(al.AlspecError) as e:
                al.spec_decode_layers(handle, p, layers)
            assert e.value.status == 3
