"""Pins of the post-attention oracle (oracle/post.py) against facts other
than itself: plain-loop brute force on small shapes, closed forms of
special weights, textbook values of silu, the unit RMS of a normed vector,
the scale invariance of RMSNorm and the affinity of the residual."""
import math

import numpy as np
import pytest

import oracle.post as op
from synth import post_gen as pg
from synth.gen import f32_to_bf16_bits


def _bits(a):
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _brute(o, h_in, w, eps):
    """The decoder layer with explicit loops and indices, row n of W[n][k]
    times the input's k-th element, no numpy products."""
    def val(name):
        return op.bf16_bits_to_f64(w[name])
    Wo, gm, Wg, Wu, Wd, ga, Wq = (val(n) for n in pg.NAMES)
    B, A = o.shape
    H, F, Q = Wo.shape[0], Wg.shape[0], Wq.shape[0]
    h_out = np.zeros((B, H))
    qkv = np.zeros((B, Q))
    for b in range(B):
        h1 = [float(h_in[b, n]) + sum(Wo[n, k] * float(o[b, k])
                                      for k in range(A)) for n in range(H)]
        r = 1.0 / math.sqrt(sum(v * v for v in h1) / H + eps)
        x = [h1[k] * r * gm[k] for k in range(H)]
        m = []
        for n in range(F):
            g = sum(Wg[n, k] * x[k] for k in range(H))
            u = sum(Wu[n, k] * x[k] for k in range(H))
            m.append(g / (1.0 + math.exp(-g)) * u)
        h2 = [h1[n] + sum(Wd[n, k] * m[k] for k in range(F))
              for n in range(H)]
        r2 = 1.0 / math.sqrt(sum(v * v for v in h2) / H + eps)
        y = [h2[k] * r2 * ga[k] for k in range(H)]
        for n in range(Q):
            qkv[b, n] = sum(Wq[n, k] * y[k] for k in range(H))
        h_out[b] = h2
    return h_out, qkv


@pytest.mark.parametrize("dims", [(2, 8, 8, 16, 12), (3, 16, 8, 24, 5),
                                  (1, 8, 24, 8, 40)])
def test_brute_force(dims):
    s = pg.PostShape("t", *dims, seed=sum(dims))
    w = pg.weights(s)
    o, h = pg.activations(s)
    ho, qo = op.post_attention(o, h, w, s.eps)
    hb, qb = _brute(o, h, w, s.eps)
    assert np.allclose(ho, hb, rtol=1e-12, atol=1e-12)
    assert np.allclose(qo, qb, rtol=1e-12, atol=1e-12)


def _zero_layer(H, A, F, Q):
    return {"w_o": _bits(np.zeros((H, A))), "norm_mlp": _bits(np.ones(H)),
            "w_gate": _bits(np.zeros((F, H))), "w_up": _bits(np.zeros((F, H))),
            "w_down": _bits(np.zeros((H, F))), "norm_attn": _bits(np.ones(H)),
            "w_qkv": _bits(np.eye(Q, H))}


def test_identity_projection_and_unit_rms():
    """W_o = I and a zero MLP: h_out = h_in + o exactly; with W_qkv = I and
    unit norm weights the output is h_out / sqrt(mean(h_out^2) + eps), whose
    mean square is ms / (ms + eps)."""
    H = 16
    w = _zero_layer(H, H, 8, H)
    w["w_o"] = _bits(np.eye(H))
    rng = np.random.default_rng(3)
    o = rng.standard_normal((2, H)).astype(np.float32)
    h = rng.standard_normal((2, H)).astype(np.float32)
    eps = 1e-3
    ho, qo = op.post_attention(o, h, w, eps)
    assert np.array_equal(ho, h.astype(np.float64) + o.astype(np.float64))
    ms = np.mean(ho * ho, axis=1)
    assert np.allclose(np.mean(qo * qo, axis=1), ms / (ms + eps),
                       rtol=1e-12)


def test_silu_textbook_values():
    """h_in = 1 (so the normed input is 1 / sqrt(1 + eps) per element, eps
    negligible), gate row n picks t_n, up picks 1, W_down = I: h_out - 1 is
    silu(t).  silu(0) = 0, silu(1) = sigma(1) = 0.7310585786300049,
    silu(-1) = -0.2689414213699951, silu(2) = 2 sigma(2) = 1.7615941559557649,
    silu(+-40) = 40 and -40 e^-40 to 1e-15."""
    t = np.array([0.0, 1.0, -1.0, 2.0, 40.0, -40.0, 0.5, -0.5])
    F = H = len(t)
    w = _zero_layer(H, H, F, 1)
    g = np.zeros((F, H))
    g[:, 0] = t
    u = np.zeros((F, H))
    u[:, 0] = 1.0
    w["w_gate"], w["w_up"], w["w_down"] = _bits(g), _bits(u), _bits(np.eye(H))
    assert np.array_equal(op.bf16_bits_to_f64(w["w_gate"])[:, 0], t)
    ho, _ = op.post_attention(np.zeros((1, H), np.float32),
                              np.ones((1, H), np.float32), w, 1e-300)
    m = ho[0] - 1.0
    want = [0.0, 0.7310585786300049, -0.2689414213699951, 1.7615941559557649,
            40.0, 0.0, 0.31122966560092726, -0.18877033439907274]
    assert np.allclose(m, want, rtol=1e-13, atol=1e-15)


def test_rmsnorm_scale_invariance():
    """With W_o = 0 the MLP sees rmsnorm(h_in), unchanged by scaling h_in
    (eps negligible), so h_out(c h) - c h = h_out(h) - h."""
    s = pg.PostShape("t", 2, 8, 16, 24, 8, eps=1e-300, seed=5)
    w = pg.weights(s)
    w["w_o"] = _bits(np.zeros((16, 8)))
    o, h = pg.activations(s)
    h = h.astype(np.float64)
    a, _ = op.post_attention(o, h, w, s.eps)
    b, _ = op.post_attention(o, 3.0 * h, w, s.eps)
    assert np.allclose(b - 3.0 * h, a - h, rtol=1e-12, atol=1e-12)


def test_residual_affine_in_attention_output():
    """With a zero gate the MLP adds nothing: h_out - h_in = W_o o is
    linear in o."""
    s = pg.PostShape("t", 1, 16, 8, 8, 8, seed=9)
    w = pg.weights(s)
    w["w_gate"] = _bits(np.zeros((8, 8)))
    o1, h = pg.activations(s, 0)
    o2, _ = pg.activations(s, 1)
    f = lambda o_: op.post_attention(o_, h, w, s.eps)[0] - h  # noqa: E731
    assert np.allclose(f(o1.astype(np.float64) + o2), f(o1) + f(o2),
                       rtol=1e-12, atol=1e-12)
    # and the projection is W_o times o, row by row
    Wo = op.bf16_bits_to_f64(w["w_o"])
    assert np.allclose(f(o1)[0], [sum(Wo[n, k] * float(o1[0, k])
                                      for k in range(16)) for n in range(8)],
                       rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mistake", ["no_residual", "sigmoid", "transpose",
                                     "norm_mean", "norm_after_gain"])
def test_planted_mistakes_are_caught(mistake):
    """Each plausible slip in the definition, planted in a copy of it,
    fails the brute-force pin."""
    s = pg.PostShape("t", 2, 8, 8, 16, 12, seed=21)
    w = pg.weights(s)
    o, h = pg.activations(s)
    hb, qb = _brute(o, h, w, s.eps)

    def wrong(o_, h_, w_, eps):
        W = {n: op.bf16_bits_to_f64(v) for n, v in w_.items()}
        h1 = (0 if mistake == "no_residual" else h_) + o_ @ W["w_o"].T
        if mistake == "norm_mean":
            x = (h1 - h1.mean(-1, keepdims=True)) / np.sqrt(
                np.var(h1, -1, keepdims=True) + eps) * W["norm_mlp"]
        elif mistake == "norm_after_gain":
            v = h1 * W["norm_mlp"]
            x = v / np.sqrt(np.mean(v * v, -1, keepdims=True) + eps)
        else:
            x = op.rmsnorm(h1, W["norm_mlp"], eps)
        wg = W["w_gate"]
        act = (1 / (1 + np.exp(-(x @ wg.T))) if mistake == "sigmoid"
               else op.silu(x @ wg.T))
        m = act * (x @ W["w_up"].T)
        wd = W["w_down"]
        h2 = h1 + (m @ wd.T if mistake != "transpose"
                   else (wd @ m.T).T if wd.shape[0] == m.shape[1]
                   else m @ wd.reshape(wd.shape[1], wd.shape[0]))
        return h2, op.rmsnorm(h2, W["norm_attn"], eps) @ W["w_qkv"].T
    hw, qw = wrong(o, h, w, s.eps)
    assert not (np.allclose(hw, hb, rtol=1e-9, atol=1e-9) and
                np.allclose(qw, qb, rtol=1e-9, atol=1e-9))
