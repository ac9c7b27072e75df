"""GPU parity of the post-attention operators (alspec_post_attention)
against the float64 oracle on the same seeded inputs.

Bar: per (entry, output) relative L2 error <= 5e-6.  The kernels multiply
bf16 weights (exact in fp32) by fp32 activations and accumulate in fp32
over K <= 28672 terms: each term and partial sum is rounded to 2^-24
relative, and these errors add like a random walk, so an output's relative
error is a small multiple of 2^-24 ~ 6e-8 (observed at most 3.5e-7 over
four dependent operators at the 70B shape).  A wrong step gives errors of
order 1.  Skipped entries must be bit-for-bit untouched.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import attention_level_speculation_amd as al  # noqa: E402
import oracle.post as op  # noqa: E402
from synth import post_gen as pg  # noqa: E402

BAR = 5e-6


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h = al.Handle(0)
    yield h
    h.close()


def _dev_weights(s, w):
    return {n: torch.from_numpy(w[n].view(np.int16)).view(torch.bfloat16)
            .to("cuda").contiguous() for n in pg.NAMES}


def _rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    return [float(np.linalg.norm(got[b] - ref[b]) / np.linalg.norm(ref[b]))
            for b in range(ref.shape[0])]


def _run(handle, s, w_dev, o, h, skip=None, h_out=None, qkv=None):
    p = al.make_post_params(s.B, s.attn_dim, s.hidden, s.ffn, s.qkv_dim,
                            s.eps)
    od = torch.from_numpy(o).cuda()
    hd = torch.from_numpy(h).cuda()
    if h_out is None:
        h_out = torch.full((s.B, s.hidden), float("nan"), device="cuda")
    if qkv is None:
        qkv = torch.full((s.B, s.qkv_dim), float("nan"), device="cuda")
    ws = al.alloc_post_workspace(p)
    sk = None if skip is None else torch.tensor(skip, dtype=torch.uint8,
                                                device="cuda")
    al.post_attention(handle, p, w_dev, od, hd, h_out, qkv, ws, skip=sk)
    torch.cuda.synchronize()
    return h_out, qkv


SHAPES = [
    # name, B, attn_dim, hidden, ffn, qkv_dim: ragged rows (not multiples
    # of the 4-row wave tile or the 16-row block), short and long K
    ("ragged_small", 3, 40, 48, 136, 20),
    ("one_row_tails", 1, 8, 8, 8, 1),
    # one and two entries (the split-K forms of the gated MLP and the down
    # projection): ragged row blocks, K shorter than the four waves'
    # shares, long K
    ("b2_ragged", 2, 40, 48, 136, 20),
    ("b1_k_tail", 1, 520, 1032, 2056, 77),
    ("b2_long_k", 2, 256, 264, 14344, 9),
    # one entry: the staged row form at its largest K (next QKV, K = 4096)
    # beside the plain form just past it (output projection, K = 4104)
    ("b1_stage_edges", 1, 4104, 4096, 136, 20),
    ("k_tail", 2, 520, 1032, 2056, 77),
    ("max_batch", 8, 256, 512, 1024, 384),
    ("mid_70b_like", 4, 1024, 2048, 5632, 3072),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[c[0] for c in SHAPES])
def test_post_attention_matches_oracle(handle, shape):
    s = pg.PostShape(*shape, seed=sum(shape[1:]))
    print(f"[case] post {shape}", flush=True)
    w = pg.weights(s)
    o, h = pg.activations(s)
    ref_h, ref_q = op.post_attention(o, h, w, s.eps)
    h_out, qkv = _run(handle, s, _dev_weights(s, w), o, h)
    eh = _rel(h_out.cpu().numpy(), ref_h)
    eq = _rel(qkv.cpu().numpy(), ref_q)
    print(f"[case] worst h {max(eh):.2e} qkv {max(eq):.2e}", flush=True)
    assert max(eh) <= BAR and max(eq) <= BAR


@pytest.mark.parametrize("shape", ["llama8b", "llama70b"])
def test_post_attention_full_size(handle, shape):
    """The 8B (B = 1) and 70B (B = 4) layer shapes, the bench's launch
    configuration."""
    s = {"llama8b": pg.llama8b(B=1), "llama70b": pg.llama70b(B=4)}[shape]
    print(f"[case] post full size {shape}", flush=True)
    w = pg.weights(s)
    o, h = pg.activations(s)
    ref_h, ref_q = op.post_attention(o, h, w, s.eps)
    h_out, qkv = _run(handle, s, _dev_weights(s, w), o, h)
    eh = _rel(h_out.cpu().numpy(), ref_h)
    eq = _rel(qkv.cpu().numpy(), ref_q)
    print(f"[case] worst h {max(eh):.2e} qkv {max(eq):.2e}", flush=True)
    assert max(eh) <= BAR and max(eq) <= BAR


def test_skip_flags_and_determinism(handle):
    """Entries flagged nonzero are untouched; the others equal an unflagged
    call bit for bit; all flagged leaves everything untouched; two calls
    give identical bits."""
    s = pg.PostShape("skip", 5, 64, 128, 256, 96, seed=4)
    w = pg.weights(s)
    wd = _dev_weights(s, w)
    o, h = pg.activations(s)
    full_h, full_q = _run(handle, s, wd, o, h)
    again_h, again_q = _run(handle, s, wd, o, h)
    assert torch.equal(full_h, again_h) and torch.equal(full_q, again_q)
    flags = [1, 0, 1, 0, 0]
    prev_h = torch.full((s.B, s.hidden), 7.0, device="cuda")
    prev_q = torch.full((s.B, s.qkv_dim), -3.0, device="cuda")
    got_h, got_q = _run(handle, s, wd, o, h, skip=flags,
                        h_out=prev_h.clone(), qkv=prev_q.clone())
    for b, f in enumerate(flags):
        if f:
            assert torch.equal(got_h[b], prev_h[b])
            assert torch.equal(got_q[b], prev_q[b])
        else:
            assert torch.equal(got_h[b], full_h[b])
            assert torch.equal(got_q[b], full_q[b])
    none_h, none_q = _run(handle, s, wd, o, h, skip=[1] * s.B,
                          h_out=prev_h.clone(), qkv=prev_q.clone())
    assert torch.equal(none_h, prev_h) and torch.equal(none_q, prev_q)


def test_in_place_residual(handle):
    """h_out may be h_in when no skip flags are given."""
    s = pg.PostShape("inplace", 2, 64, 96, 160, 32, seed=6)
    w = pg.weights(s)
    wd = _dev_weights(s, w)
    o, h = pg.activations(s)
    ref_h, ref_q = _run(handle, s, wd, o, h)
    p = al.make_post_params(s.B, s.attn_dim, s.hidden, s.ffn, s.qkv_dim,
                            s.eps)
    hd = torch.from_numpy(h).cuda()
    qkv = torch.empty((s.B, s.qkv_dim), device="cuda")
    al.post_attention(handle, p, wd, torch.from_numpy(o).cuda(), hd, hd, qkv,
                      al.alloc_post_workspace(p))
    torch.cuda.synchronize()
    assert torch.equal(hd, ref_h) and torch.equal(qkv, ref_q)


@pytest.mark.parametrize("B", [1, 2])
def test_small_batch_repeats_and_skips(handle, B):
    """One or two entries (the decode step's batch) on one workspace: five
    calls in a row give identical bits, skip flags leave flagged entries
    untouched and the others equal to the unflagged call, and all entries
    flagged leaves everything as it was."""
    s = pg.PostShape("small_batch", B, 72, 136, 1000, 40, seed=11 + B)
    print(f"[case] post small batch B={B}", flush=True)
    w = pg.weights(s)
    wd = _dev_weights(s, w)
    o, h = pg.activations(s)
    p = al.make_post_params(s.B, s.attn_dim, s.hidden, s.ffn, s.qkv_dim,
                            s.eps)
    ws = al.alloc_post_workspace(p)
    od = torch.from_numpy(o).cuda()
    hd = torch.from_numpy(h).cuda()

    def call(skip=None, h0=None, q0=None):
        h_out = (torch.full((s.B, s.hidden), float("nan"), device="cuda")
                 if h0 is None else h0.clone())
        qkv = (torch.full((s.B, s.qkv_dim), float("nan"), device="cuda")
               if q0 is None else q0.clone())
        sk = None if skip is None else torch.tensor(skip, dtype=torch.uint8,
                                                    device="cuda")
        al.post_attention(handle, p, wd, od, hd, h_out, qkv, ws, skip=sk)
        torch.cuda.synchronize()
        return h_out, qkv
    first = call()
    ref_h, ref_q = op.post_attention(o, h, w, s.eps)
    assert max(_rel(first[0].cpu().numpy(), ref_h)) <= BAR
    assert max(_rel(first[1].cpu().numpy(), ref_q)) <= BAR
    for _ in range(4):
        again = call()
        assert torch.equal(again[0], first[0])
        assert torch.equal(again[1], first[1])
    prev_h = torch.full((s.B, s.hidden), 7.0, device="cuda")
    prev_q = torch.full((s.B, s.qkv_dim), -3.0, device="cuda")
    patterns = [[1], [0]] if B == 1 else [[1, 0], [0, 1], [1, 1], [0, 0]]
    for flags in patterns:
        got_h, got_q = call(flags, prev_h, prev_q)
        for b, f in enumerate(flags):
            want_h = prev_h[b] if f else first[0][b]
            want_q = prev_q[b] if f else first[1][b]
            assert torch.equal(got_h[b], want_h), (flags, b)
            assert torch.equal(got_q[b], want_q), (flags, b)
    # and once more unflagged after the flagged calls
    last = call()
    assert torch.equal(last[0], first[0]) and torch.equal(last[1], first[1])
