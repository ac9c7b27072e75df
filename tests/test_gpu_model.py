"""GPU tests of the chained decode step with speculative post-attention
work and replay on discard (attention_level_speculation_amd.runtime).

- The speculative schedule (two streams, replay gated on the device
  commit flag) gives bit for bit the result of the plain sequence "attention
  step, then post-attention on the committed output", whatever the flags.
- With lambda = 0 every layer discards: the result equals exact attention
  followed by the post-attention work (the non-speculative baseline).
- The chain matches the float64 oracle chain (oracle attention step, its
  committed output, oracle post-attention, next query) at lambda = +inf
  (every layer commits) and 0 (every layer discards), where the flags are
  not in doubt.  Bar: relative L2 <= 1e-4 on the final residual and QKV
  after 3 layers with fp32 KV (each attention output is within ~1e-6 of
  the oracle's and each post-attention step within ~1e-7; chaining through
  the layers' queries amplifies this by at most a few hundred).
- The one-stream speculative form (speculative work on o_approx before
  the exact pass, replay gated by the commit flag) gives the committed
  sequence's result, matches the oracle chain where the flags are not in
  doubt, and, captured into one HIP graph, replays to the eager result
  bit for bit, three times with eager work in between.
- With planted weights (each next query pointed at the next layer's
  planted sink direction, synth.post_gen.plant_query_direction) the later
  layers' queries find the sink as the generator's do, and at lambda 0.05
  the flags go commit, commit, discard: both forms give the committed
  sequence's bits and the oracle chain's flags and outputs.
- A captured graph of the two-stream speculative step replaying to the
  eager result is skipped: capture crashed the host inside the HIP runtime
  (see the test's reason).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import attention_level_speculation_amd as al  # noqa: E402
from attention_level_speculation_amd import runtime as rt  # noqa: E402
import oracle  # noqa: E402
import oracle.post as op  # noqa: E402
from synth import gen  # noqa: E402
from synth import post_gen as pg  # noqa: E402

N_LAYERS = 3


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h = al.Handle(0)
    yield h
    h.close()


PLANT_DIM = 7   # the residual's dominant coordinate at hidden 256


def _setup(lam, kv="f32", planted=False):
    Hq, Hkv, D, L = 8, 2, 64, 3000
    w = gen.Workload("model", B=1, Hq=Hq, Hkv=Hkv, D=D, L_cap=L,
                     seq_lens=[L], kv_dtype=kv, S=4, W=128, lam=lam,
                     needles=[0 if planted else 1], seed=31)
    ps = pg.PostShape("model", 1, Hq * D, 256, 512, (Hq + 2 * Hkv) * D,
                      seed=32)
    weights = [pg.weights(pg.PostShape(ps.name, ps.B, ps.attn_dim,
                                       ps.hidden, ps.ffn, ps.qkv_dim,
                                       ps.eps, ps.seed + l))
               for l in range(N_LAYERS)]
    h0 = pg.activations(ps)[1]
    if planted:
        for l, wt in enumerate(weights):
            # planted in float, rounded once to bf16 (the other entries
            # are bf16 values already, so rounding again keeps them)
            wq = torch.from_numpy(gen.bf16_bits_to_f32(wt["w_qkv"]).copy())
            na = torch.from_numpy(
                gen.bf16_bits_to_f32(wt["norm_attn"]).copy())
            nxt = (l + 1) % N_LAYERS
            pg.plant_query_direction(
                wq, na, [gen.head_plant(w, nxt, 0, g).u for g in range(Hkv)],
                w.const.a, D, Hq // Hkv, ps.hidden, dim=PLANT_DIM)
            wt["w_qkv"] = gen.f32_to_bf16_bits(wq.numpy())
            wt["norm_attn"] = gen.f32_to_bf16_bits(na.numpy())
        h0 = h0.copy()
        h0[0, PLANT_DIM] = pg.MASSIVE_VALUE
    host = {"kv": [gen.layer_inputs(w, l) for l in range(N_LAYERS)],
            "w": weights, "h0": h0}
    return w, ps, host


def _device(w, ps, host, lam):
    p = al.params_for(w, lam=lam)
    pp = al.make_post_params(1, ps.attn_dim, ps.hidden, ps.ffn, ps.qkv_dim,
                             ps.eps)
    wdev = [{n: torch.from_numpy(d[n].view(np.int16)).view(torch.bfloat16)
             .cuda() for n in pg.NAMES} for d in host["w"]]
    kvd = []
    for q, k, v in host["kv"]:
        kd = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).cuda() \
            if w.kv_dtype == "bf16" else torch.from_numpy(k).cuda()
        vd = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda() \
            if w.kv_dtype == "bf16" else torch.from_numpy(v).cuda()
        kvd.append((kd, vd))
    hs = [torch.from_numpy(host["h0"]).cuda()] + [
        torch.full((1, ps.hidden), float("nan"), device="cuda")
        for _ in range(N_LAYERS)]
    layers = [rt.ModelLayer(kvd[l][0], kvd[l][1],
                            al.post_weights_struct(pp, wdev[l]),
                            al.alloc_outputs(p), hs[l], hs[l + 1],
                            torch.full((1, ps.qkv_dim), float("nan"),
                                       device="cuda"))
              for l in range(N_LAYERS)]
    q0 = torch.from_numpy(host["kv"][0][0]).cuda()
    ws = (al.alloc_workspace(p), al.alloc_post_workspace(pp),
          al.alloc_post_workspace(pp))
    keep = (wdev, kvd, hs)
    return p, pp, q0, layers, ws, keep


def _run(handle, dev, **kw):
    p, pp, q0, layers, ws, _ = dev
    sa, se = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    se.wait_stream(torch.cuda.current_stream())
    rt.model_step(handle, p, pp, q0, layers, *ws, sa, se, **kw)
    torch.cuda.current_stream().wait_stream(se)
    torch.cuda.current_stream().wait_stream(sa)
    torch.cuda.synchronize()
    return (layers[-1].h_out.cpu().numpy().copy(),
            layers[-1].qkv_out.cpu().numpy().copy(),
            [int(l_.out["commit"][0].item()) for l_ in layers])


@pytest.mark.parametrize("lam", [0.0, 0.1, 0.5, float("inf")])
def test_speculative_equals_committed_sequence(handle, lam):
    w, ps, host = _setup(lam)
    dev = _device(w, ps, host, lam)
    print(f"[case] model lam={lam}", flush=True)
    hs, qs, flags = _run(handle, dev, speculative=True)
    hq, qq, flags2 = _run(handle, dev, speculative=False)
    print(f"[case] commits {flags}", flush=True)
    assert flags == flags2
    assert np.array_equal(hs, hq) and np.array_equal(qs, qq)
    if lam == 0.0:
        assert flags == [0] * N_LAYERS
        he, qe, _ = _run(handle, dev, exact_only=True)
        assert np.array_equal(he, hq) and np.array_equal(qe, qq)
    if lam == float("inf"):
        assert flags == [1] * N_LAYERS


@pytest.mark.parametrize("lam", [0.0, 0.1, 0.5, float("inf")])
def test_one_stream_equals_committed_sequence(handle, lam):
    """The one-stream form runs the separate calls (approximation, middle
    pass, combine, verify), whose outputs are the fused call's; where the
    flags agree the final residual and QKV equal the committed sequence's
    bit for bit."""
    w, ps, host = _setup(lam)
    dev = _device(w, ps, host, lam)
    print(f"[case] model one stream lam={lam}", flush=True)
    hs, qs, flags = _run(handle, dev, speculative=True, one_stream=True)
    hq, qq, flags2 = _run(handle, dev, speculative=False)
    print(f"[case] commits {flags} / {flags2}", flush=True)
    assert flags == flags2
    assert np.array_equal(hs, hq) and np.array_equal(qs, qq)


def _oracle_chain(w, ps, host, lam, ratios=None):
    q = host["kv"][0][0].astype(np.float64)
    h = host["h0"].astype(np.float64)
    for l in range(N_LAYERS):
        _, k, v = host["kv"][l]
        r = oracle.spec_decode(q.astype(np.float32), k, v, w.seq_lens, w.S,
                               w.W, lam)
        if ratios is not None:
            ratios.append(float(r["ratio"][0]))
        o = r["o_committed"].reshape(1, -1)
        h, qkv = op.post_attention(o, h, host["w"][l], ps.eps)
        q = qkv[:, :ps.attn_dim].reshape(1, w.Hq, w.D)
    return h, qkv


@pytest.mark.parametrize("lam", [0.0, float("inf")])
def test_chain_matches_oracle_chain(handle, lam):
    w, ps, host = _setup(lam)
    dev = _device(w, ps, host, lam)
    hg, qg, _ = _run(handle, dev, speculative=True)
    ho, qo = _oracle_chain(w, ps, host, lam)
    eh = np.linalg.norm(hg - ho) / np.linalg.norm(ho)
    eq = np.linalg.norm(qg - qo) / np.linalg.norm(qo)
    print(f"[case] chain vs oracle lam={lam}: h {eh:.2e} qkv {eq:.2e}",
          flush=True)
    assert eh <= 1e-4 and eq <= 1e-4


@pytest.mark.parametrize("lam", [0.0, float("inf")])
def test_one_stream_matches_oracle_chain(handle, lam):
    w, ps, host = _setup(lam)
    dev = _device(w, ps, host, lam)
    hg, qg, _ = _run(handle, dev, speculative=True, one_stream=True)
    ho, qo = _oracle_chain(w, ps, host, lam)
    eh = np.linalg.norm(hg - ho) / np.linalg.norm(ho)
    eq = np.linalg.norm(qg - qo) / np.linalg.norm(qo)
    print(f"[case] one-stream chain vs oracle lam={lam}: h {eh:.2e} "
          f"qkv {eq:.2e}", flush=True)
    assert eh <= 1e-4 and eq <= 1e-4


@pytest.mark.parametrize("one_stream", [False, True])
def test_planted_queries_mix_commits(handle, one_stream):
    lam = 0.05
    w, ps, host = _setup(lam, planted=True)
    ratios = []
    ho, qo = _oracle_chain(w, ps, host, lam, ratios)
    want = [int(r <= lam) for r in ratios]
    # the flags are not in doubt, and they mix
    assert min(abs(r - lam) for r in ratios) > 1e-4, ratios
    assert want == [1, 1, 0], ratios
    dev = _device(w, ps, host, lam)
    print(f"[case] planted model one_stream={one_stream}", flush=True)
    hs, qs, flags = _run(handle, dev, speculative=True, one_stream=one_stream)
    hq, qq, flags2 = _run(handle, dev, speculative=False)
    print(f"[case] commits {flags}, oracle ratios {ratios}", flush=True)
    assert flags == flags2 == want
    assert np.array_equal(hs, hq) and np.array_equal(qs, qq)
    eh = np.linalg.norm(hs - ho) / np.linalg.norm(ho)
    eq = np.linalg.norm(qs - qo) / np.linalg.norm(qo)
    assert eh <= 1e-4 and eq <= 1e-4, (eh, eq)


def test_one_stream_graph_replays_match_eager(handle):
    """The one-stream step over all layers captured into one HIP graph:
    three replays, each after eager work on the same buffers, give the
    eager step's bits (the commit flags at lambda 0.1 mix)."""
    w, ps, host = _setup(0.1)
    dev = _device(w, ps, host, 0.1)
    want_h, want_q, want_f = _run(handle, dev, speculative=True,
                                  one_stream=True)
    p, pp, q0, layers, ws, _ = dev
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    print("[case] capture one-stream step", flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        rt.model_step(handle, p, pp, q0, layers, *ws, cap, cap,
                      speculative=True, one_stream=True)
    for rep in range(3):
        _run(handle, dev, speculative=False)       # eager work in between
        for l_ in layers:
            l_.h_out.fill_(float("nan"))
            l_.qkv_out.fill_(float("nan"))
            l_.out["commit"].fill_(7)
        torch.cuda.synchronize()
        with torch.cuda.stream(cap):
            g.replay()
        torch.cuda.synchronize()
        print(f"[case] replay {rep}", flush=True)
        assert np.array_equal(layers[-1].h_out.cpu().numpy(), want_h), rep
        assert np.array_equal(layers[-1].qkv_out.cpu().numpy(), want_q), rep
        assert [int(l_.out["commit"][0].item()) for l_ in layers] == want_f


@pytest.mark.skip(reason="capturing this step ended in a host segmentation "
                  "fault inside hipStreamEndCapture (torch's HIP runtime): "
                  "the step makes each of its two captured streams wait on "
                  "the other in turn, which this library's own captured "
                  "schedules never do; no cause in this code was found, so "
                  "the case stays off the GPU and the step runs eagerly")
def test_graph_replays_match_eager(handle):
    w, ps, host = _setup(0.1)
    dev = _device(w, ps, host, 0.1)
    want_h, want_q, _ = _run(handle, dev, speculative=True)
    p, pp, q0, layers, ws, _ = dev
    cap, sa, se = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        sa.wait_stream(cap)
        se.wait_stream(cap)
        rt.model_step(handle, p, pp, q0, layers, *ws, sa, se,
                      speculative=True)
        cap.wait_stream(sa)
        cap.wait_stream(se)
    for rep in range(3):
        for l_ in layers:
            l_.h_out.fill_(float("nan"))
            l_.qkv_out.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(cap):
            g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(layers[-1].h_out.cpu().numpy(), want_h), rep
        assert np.array_equal(layers[-1].qkv_out.cpu().numpy(), want_q), rep
        _run(handle, dev, speculative=False)       # eager work in between
