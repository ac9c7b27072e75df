"""Pins of the CPU oracle against what the pages and the mathematics fix.

The pages ('Attention-Level Speculation': atlas.scime.ai summary, sections
Summary / Approach / Key results / Limitations; ICML 2025 poster page,
abstract) describe the method in prose and print no worked example, so every
pin here is a hand-worked closed form, an identity the definitions imply, a
limit, a special case, or a brute force in high precision on tiny inputs.
Each is chosen so that a plausible slip in the oracle (a dropped sink or
window term, an off-by-one set boundary, a wrong GQA head mapping, a
transposed operand, a missing renormalisation, a per-head instead of a
per-(user, layer) norm) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _ev(expr):
    env = {"e": math.e, "ln": math.log, "sqrt": math.sqrt, "nan": math.nan,
           "exp": math.exp}
    return float(eval(str(expr), {"__builtins__": {}}, env))


def _arr(nested, dtype=np.float64):
    if isinstance(nested, list):
        return np.array([_arr(x, dtype) for x in nested], dtype=dtype)
    return _ev(nested)


def rand_problem(rng, B=2, Hq=4, Hkv=2, D=8, L_cap=40, lens=None,
                 scale=1.0):
    q = (rng.standard_normal((B, Hq, D)) * scale).astype(np.float32)
    k = (rng.standard_normal((B, Hkv, L_cap, D)) * scale).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L_cap, D)).astype(np.float32)
    if lens is None:
        lens = rng.integers(1, L_cap + 1, size=B)
    return q, k, v, np.asarray(lens, dtype=np.int32)


# ---------------------------------------------------------------- golden ----

with open(GOLDEN) as f:
    _CASES = json.load(f)["cases"]


@pytest.mark.parametrize("case", _CASES, ids=[c["name"] for c in _CASES])
def test_hand_worked(case):
    q = _arr(case["q"]).astype(np.float32)
    k = _arr(case["k"]).astype(np.float32)
    v = _arr(case["v"]).astype(np.float32)
    sm = _ev(case["sm_scale"])
    exp = case["expect"]
    for lam, flags in exp["commit_at"].items():
        r = oracle.spec_decode(q, k, v, case["seq_lens"], case["S"], case["W"],
                               float(lam), sm_scale=sm)
        assert r["commit"].tolist() == flags, (lam, r["ratio"])
    for key in ("o_exact", "o_approx", "lse_exact", "lse_approx", "mass_A",
                "ratio"):
        if key in exp:
            np.testing.assert_allclose(r[key], _arr(exp[key]), rtol=1e-6,
                                       atol=1e-7, err_msg=key)
    assert not np.isnan(r["o_exact"]).any(), "padding rows were read"
    if "o_middle" in exp:
        # attention over the middle tokens alone, for the closed form of the
        # approximation error: O_approx - O_exact = (1 - mass_A)(O_A - O_mid)
        L, S, W = case["seq_lens"][0], case["S"], case["W"]
        mid = np.arange(min(S, L), max(min(S, L), L - W))
        m, l, acc = oracle.partial(q[0, 0], k[0, 0], v[0, 0], mid, sm)
        np.testing.assert_allclose(acc / l, _arr(exp["o_middle"])[0, 0],
                                   rtol=1e-6)


# ------------------------------------------------------- high-precision brute

def _brute_mp(q, k, v, lens, S, W, sm):
    """Independent high-precision evaluation on tiny inputs.  It forms each
    softmax weight as p_j = 1 / sum_i exp(s_i - s_j) and builds the
    approximation by masking the full token range with an indicator of the
    sink and window, instead of listing the set."""
    import mpmath as mp
    mp.mp.dps = 40
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    oe = np.zeros((B, Hq, D))
    oa = np.zeros((B, Hq, D))
    ratio = np.zeros(B)
    for b in range(B):
        L = int(lens[b])
        num = mp.mpf(0)
        den = mp.mpf(0)
        for h in range(Hq):
            g = h // G
            s = [mp.mpf(sm) * mp.fsum(mp.mpf(float(q[b, h, d])) *
                                      mp.mpf(float(k[b, g, j, d]))
                                      for d in range(D)) for j in range(L)]
            ind = [1 if (j < S or j >= L - W) else 0 for j in range(L)]
            pe = [1 / mp.fsum(mp.e ** (s[i] - s[j]) for i in range(L))
                  for j in range(L)]
            pa = [ind[j] / mp.fsum(ind[i] * mp.e ** (s[i] - s[j])
                                   for i in range(L)) if ind[j] else mp.mpf(0)
                  for j in range(L)]
            for d in range(D):
                e_ = mp.fsum(pe[j] * mp.mpf(float(v[b, g, j, d]))
                             for j in range(L))
                a_ = mp.fsum(pa[j] * mp.mpf(float(v[b, g, j, d]))
                             for j in range(L))
                oe[b, h, d] = float(e_)
                oa[b, h, d] = float(a_)
                num += (a_ - e_) ** 2
                den += e_ ** 2
        ratio[b] = float(mp.sqrt(num / den))
    return oe, oa, ratio


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_high_precision(seed):
    rng = np.random.default_rng(100 + seed)
    q, k, v, lens = rand_problem(rng, B=2, Hq=4, Hkv=2, D=4, L_cap=12,
                                 lens=[12, 7], scale=1.5)
    S, W = 2, 3
    r = oracle.spec_decode(q, k, v, lens, S, W, 0.1, sm_scale=0.7)
    oe, oa, ratio = _brute_mp(q, k, v, lens, S, W, 0.7)
    np.testing.assert_allclose(r["o_exact"], oe, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["o_approx"], oa, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["ratio"], ratio, rtol=1e-10)


# ------------------------------------------------------------ identities ----

@pytest.mark.parametrize("L,S,W", [(10, 4, 6), (10, 4, 100), (3, 4, 0),
                                    (1, 1, 0), (1, 0, 1), (5, 0, 5)])
def test_full_cover_gives_identical_outputs(L, S, W):
    """S + W >= L: the approximation set is the whole context, so the two
    outputs coincide bit for bit and the ratio is 0 even for lambda = 0."""
    rng = np.random.default_rng(L * 31 + S)
    q, k, v, _ = rand_problem(rng, B=1, Hq=2, Hkv=1, D=8, L_cap=L, lens=[L])
    r = oracle.spec_decode(q, k, v, [L], S, W, 0.0)
    assert np.array_equal(r["o_exact"], r["o_approx"])
    assert r["ratio"][0] == 0.0 and r["commit"][0] == 1


def test_shift_invariance_of_keys():
    """Adding one vector t to every key adds sm_scale*<q,t> to every logit of
    a head; softmax is unchanged.  Dyadic inputs keep K + t exact in fp32."""
    rng = np.random.default_rng(7)
    B, Hq, Hkv, D, L = 1, 4, 2, 8, 33
    q = (rng.integers(-64, 64, (B, Hq, D)) / 32).astype(np.float32)
    k = (rng.integers(-64, 64, (B, Hkv, L, D)) / 32).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    t = (rng.integers(-64, 64, D) / 16).astype(np.float32)
    r0 = oracle.spec_decode(q, k, v, [L], 3, 5, 0.1)
    r1 = oracle.spec_decode(q, k + t, v, [L], 3, 5, 0.1)
    for key in ("o_exact", "o_approx", "ratio", "mass_A"):
        np.testing.assert_allclose(r1[key], r0[key], rtol=1e-12, atol=1e-14)
    # lse shifts by the logit shift
    shift = (q[0] @ t.astype(np.float64)) / math.sqrt(D)
    np.testing.assert_allclose(r1["lse_exact"][0] - r0["lse_exact"][0], shift,
                               rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_split_and_merge_equals_one_pass(seed):
    """Splitting the tokens into parts (some empty), taking each part's
    state and merging with log-sum-exp gives the one-pass softmax."""
    rng = np.random.default_rng(seed)
    L, D = 57, 16
    q = rng.standard_normal(D).astype(np.float32) * 2
    k = rng.standard_normal((L, D)).astype(np.float32)
    v = rng.standard_normal((L, D)).astype(np.float32)
    perm = rng.permutation(L)
    cuts = np.sort(rng.integers(0, L + 1, size=6))
    parts = np.split(perm, cuts)
    ms, ls, accs = [], [], []
    for p in parts:
        m, l, acc = oracle.partial(q, k, v, p, 0.25)
        if len(p) == 0:
            assert m == -math.inf and l == 0.0 and not acc.any()
        ms.append(m); ls.append(l); accs.append(acc)
    out, lse = oracle.lse_merge(ms, ls, np.stack(accs))
    m1, l1, acc1 = oracle.partial(q, k, v, np.arange(L), 0.25)
    np.testing.assert_allclose(out, acc1 / l1, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, m1 + math.log(l1), rtol=1e-14)
    # and against the spec_decode exact output for the same head
    r = oracle.spec_decode(q[None, None], k[None, None], v[None, None], [L],
                           1, 1, 0.1, sm_scale=0.25)
    np.testing.assert_allclose(r["o_exact"][0, 0], out, rtol=1e-13, atol=1e-15)


def test_lse_merge_rejects_all_empty():
    with pytest.raises(ValueError):
        oracle.lse_merge([-math.inf, -math.inf], [0.0, 0.0], np.zeros((2, 3)))


@pytest.mark.parametrize("seed", range(3))
def test_error_closed_form(seed):
    """O_approx - O_exact = (1 - mass_A) (O_approx - O_mid), with O_mid the
    softmax output over the middle tokens alone and mass_A the exact softmax
    mass on the approximation set."""
    rng = np.random.default_rng(seed)
    q, k, v, _ = rand_problem(rng, B=1, Hq=2, Hkv=1, D=8, L_cap=50, lens=[50])
    S, W = 3, 7
    sm = 1 / math.sqrt(8)
    r = oracle.spec_decode(q, k, v, [50], S, W, 0.1)
    mid = np.arange(S, 50 - W)
    for h in range(2):
        m, l, acc = oracle.partial(q[0, h], k[0, 0], v[0, 0], mid, sm)
        lhs = r["o_approx"][0, h] - r["o_exact"][0, h]
        rhs = (1 - r["mass_A"][0, h]) * (r["o_approx"][0, h] - acc / l)
        np.testing.assert_allclose(lhs, rhs, rtol=1e-10, atol=1e-14)


def test_uniform_limit_gives_means():
    """q = 0 makes every logit 0: exact attention is the mean of the values
    and the approximation is the mean over the sink and window rows."""
    rng = np.random.default_rng(3)
    q, k, v, _ = rand_problem(rng, B=1, Hq=2, Hkv=2, D=4, L_cap=20, lens=[20])
    q[:] = 0
    S, W = 2, 5
    r = oracle.spec_decode(q, k, v, [20], S, W, 0.1)
    A = list(range(S)) + list(range(20 - W, 20))
    for h in range(2):
        np.testing.assert_allclose(r["o_exact"][0, h],
                                   v[0, h].astype(np.float64).mean(0),
                                   rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(r["o_approx"][0, h],
                                   v[0, h, A].astype(np.float64).mean(0),
                                   rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(r["lse_exact"][0, h], math.log(20),
                                   rtol=1e-14)


@pytest.mark.parametrize("pos,in_window", [(30, True), (29, False)])
def test_window_boundary(pos, in_window):
    """A key 60 nats above the rest dominates.  At position L-W it is the
    first window token, so the approximation returns its value; at L-W-1 it
    is the last middle token, so only exact attention sees it."""
    L, S, W, D = 40, 2, 10, 4
    q = np.zeros((1, 1, D), np.float32); q[0, 0, 0] = 1
    k = np.zeros((1, 1, L, D), np.float32)
    v = np.zeros((1, 1, L, D), np.float32); v[0, 0, :, 1] = 1
    k[0, 0, pos, 0] = 60
    v[0, 0, pos] = [5, 0, 0, 0]
    r = oracle.spec_decode(q, k, v, [L], S, W, 0.1, sm_scale=1.0)
    np.testing.assert_allclose(r["o_exact"][0, 0], [5, 0, 0, 0], atol=1e-20 + L * math.exp(-60) * 10)
    if in_window:
        np.testing.assert_allclose(r["o_approx"][0, 0], [5, 0, 0, 0], atol=1e-20 + L * math.exp(-60) * 10)
        assert r["commit"][0] == 1
    else:
        np.testing.assert_allclose(r["o_approx"][0, 0], [0, 1, 0, 0], atol=1e-15)
        assert r["commit"][0] == 0


@pytest.mark.parametrize("pos,in_sink", [(2, True), (3, False)])
def test_sink_boundary(pos, in_sink):
    """Same with the sink: position S-1 is the last sink token, position S
    the first middle token."""
    L, S, W, D = 40, 3, 10, 4
    q = np.zeros((1, 1, D), np.float32); q[0, 0, 0] = 1
    k = np.zeros((1, 1, L, D), np.float32)
    v = np.zeros((1, 1, L, D), np.float32); v[0, 0, :, 1] = 1
    k[0, 0, pos, 0] = 60
    v[0, 0, pos] = [5, 0, 0, 0]
    r = oracle.spec_decode(q, k, v, [L], S, W, 0.1, sm_scale=1.0)
    expect_a = [5, 0, 0, 0] if in_sink else [0, 1, 0, 0]
    np.testing.assert_allclose(r["o_approx"][0, 0], expect_a, atol=1e-15)
    assert r["commit"][0] == int(in_sink)


def test_gqa_equals_repeated_mha():
    """Query head h reads kv head h // G: GQA must equal multi-head
    attention with every kv head repeated G times (in order)."""
    rng = np.random.default_rng(11)
    q, k, v, lens = rand_problem(rng, B=2, Hq=8, Hkv=2, D=8, L_cap=30)
    r = oracle.spec_decode(q, k, v, lens, 2, 6, 0.1)
    kr = np.repeat(k, 4, axis=1)
    vr = np.repeat(v, 4, axis=1)
    r2 = oracle.spec_decode(q, kr, vr, lens, 2, 6, 0.1)
    for key in ("o_exact", "o_approx", "ratio"):
        assert np.array_equal(r[key], r2[key]), key


def test_affine_in_values():
    """V -> a V + 1 b^T maps both outputs to a O + b (softmax weights sum to
    one) and scales the squared error by a^2.  Dyadic values keep a V + b
    exact in fp32."""
    rng = np.random.default_rng(5)
    q, k, v, lens = rand_problem(rng, B=1, Hq=2, Hkv=1, D=8, L_cap=25,
                                 lens=[25])
    v = (rng.integers(-128, 128, v.shape) / 32).astype(np.float32)
    a = 2.0
    bvec = (np.arange(8) / 4 - 1).astype(np.float32)
    r = oracle.spec_decode(q, k, v, lens, 2, 4, 0.1)
    r2 = oracle.spec_decode(q, k, (a * v + bvec).astype(np.float32), lens, 2,
                            4, 0.1)
    for key in ("o_exact", "o_approx"):
        np.testing.assert_allclose(r2[key], a * r[key] + bvec, rtol=1e-12,
                                   atol=1e-12)
    num = ((r["o_approx"] - r["o_exact"]) ** 2).sum()
    num2 = ((r2["o_approx"] - r2["o_exact"]) ** 2).sum()
    np.testing.assert_allclose(num2, a * a * num, rtol=1e-10)


def test_middle_permutation_invariance():
    """Reordering the middle tokens changes neither output nor the ratio."""
    rng = np.random.default_rng(9)
    L, S, W = 48, 3, 8
    q, k, v, _ = rand_problem(rng, B=1, Hq=2, Hkv=1, D=8, L_cap=L, lens=[L])
    perm = np.arange(L)
    perm[S:L - W] = rng.permutation(np.arange(S, L - W))
    r = oracle.spec_decode(q, k, v, [L], S, W, 0.1)
    r2 = oracle.spec_decode(q, k[:, :, perm], v[:, :, perm], [L], S, W, 0.1)
    for key in ("o_exact", "o_approx", "ratio"):
        np.testing.assert_allclose(r2[key], r[key], rtol=1e-12, atol=1e-15)


def test_batch_entries_independent():
    """Changing one batch entry's data leaves the others bit for bit."""
    rng = np.random.default_rng(12)
    q, k, v, lens = rand_problem(rng, B=3, Hq=4, Hkv=2, D=8, L_cap=30)
    r = oracle.spec_decode(q, k, v, lens, 2, 5, 0.1)
    k2 = k.copy(); v2 = v.copy(); q2 = q.copy()
    k2[1] = rng.standard_normal(k2[1].shape)
    v2[1] *= 3
    q2[1] += 1
    r2 = oracle.spec_decode(q2, k2, v2, lens, 2, 5, 0.1)
    for b in (0, 2):
        for key in ("o_exact", "o_approx", "ratio", "commit"):
            assert np.array_equal(r[key][b], r2[key][b])


def test_nan_discards_only_its_user():
    """A NaN in one user's keys or values makes that user's ratio NaN, which
    never commits; the other users are untouched."""
    rng = np.random.default_rng(13)
    q, k, v, lens = rand_problem(rng, B=3, Hq=2, Hkv=1, D=8, L_cap=30,
                                 lens=[30, 30, 30])
    r0 = oracle.spec_decode(q, k, v, lens, 2, 5, math.inf)
    k1 = k.copy(); k1[1, 0, 12, 3] = np.nan       # middle key of user 1
    v1 = v.copy(); v1[2, 0, 0, 0] = np.nan        # sink value of user 2
    r = oracle.spec_decode(q, k1, v1, lens, 2, 5, math.inf)
    assert r["commit"].tolist() == [1, 0, 0]
    assert math.isnan(r["ratio"][1]) and math.isnan(r["ratio"][2])
    assert np.array_equal(r["o_exact"][0], r0["o_exact"][0])


# ----------------------------------------------------------------- verify ---

def test_verify_known_relative_error():
    rng = np.random.default_rng(2)
    e = rng.standard_normal((3, 4, 8))
    d = rng.standard_normal((3, 4, 8))
    eps = np.array([0.05, 0.1, 0.3])
    a = e + eps[:, None, None] * d * (np.linalg.norm(e.reshape(3, -1), axis=1)
                                      / np.linalg.norm(d.reshape(3, -1), axis=1))[:, None, None]
    ratio, commit = oracle.verify(a, e, 0.1 + 1e-9)
    np.testing.assert_allclose(ratio, eps, rtol=1e-12)
    assert commit.tolist() == [1, 1, 0]


def test_verify_monotone_in_lambda_and_special_values():
    rng = np.random.default_rng(4)
    e = rng.standard_normal((20, 16))
    a = e + rng.standard_normal((20, 16)) * rng.uniform(0, 0.5, (20, 1))
    prev = np.zeros(20, np.uint8)
    for lam in np.linspace(0, 1, 41):
        _, c = oracle.verify(a, e, lam)
        assert (c >= prev).all()
        prev = c
    _, c = oracle.verify(a, e, math.inf)
    assert c.all()
    # lambda = 0 commits exactly the entries with zero difference
    a2 = a.copy(); a2[3] = e[3]
    r, c = oracle.verify(a2, e, 0.0)
    assert c.tolist() == [1 if i == 3 else 0 for i in range(20)] and r[3] == 0
    # zero exact output: ratio 0 if the difference is 0, else +inf
    z = np.zeros((2, 4))
    r, c = oracle.verify(np.array([[0, 0, 0, 0], [0, 1e-30, 0, 0]]), z, 1.0)
    assert r[0] == 0 and c[0] == 1 and r[1] == math.inf and c[1] == 0
    # NaN never commits, not even for lambda = inf
    a3 = a.copy(); a3[5, 2] = np.nan
    r, c = oracle.verify(a3, e, math.inf)
    assert math.isnan(r[5]) and c[5] == 0 and c.sum() == 19


def test_bf16_inputs_are_widened_exactly():
    """bf16 keys/values (as bit patterns) must give the same result as the
    same values stored in fp32."""
    rng = np.random.default_rng(8)
    q, k, v, lens = rand_problem(rng, B=2, Hq=4, Hkv=2, D=8, L_cap=20)
    kb = (k.view(np.uint32) >> 16).astype(np.uint16)
    vb = (v.view(np.uint32) >> 16).astype(np.uint16)
    kf = (kb.astype(np.uint32) << 16).view(np.float32)
    vf = (vb.astype(np.uint32) << 16).view(np.float32)
    r = oracle.spec_decode(q, kb, vb, lens, 2, 5, 0.1)
    r2 = oracle.spec_decode(q, kf, vf, lens, 2, 5, 0.1)
    for key in ("o_exact", "o_approx", "ratio"):
        assert np.array_equal(r[key], r2[key])


def test_threads_do_not_change_results():
    rng = np.random.default_rng(21)
    q, k, v, lens = rand_problem(rng, B=3, Hq=8, Hkv=2, D=16, L_cap=64)
    r1 = oracle.spec_decode(q, k, v, lens, 4, 9, 0.1, threads=1)
    r4 = oracle.spec_decode(q, k, v, lens, 4, 9, 0.1, threads=5)
    for key in r1:
        assert np.array_equal(r1[key], r4[key]), key


@pytest.mark.parametrize("bad", [
    dict(S=0, W=0), dict(lam=-0.1), dict(lam=math.nan), dict(lens=[0]),
    dict(lens=[11]), dict(sm=0.0)])
def test_rejects_invalid(bad):
    rng = np.random.default_rng(0)
    q, k, v, _ = rand_problem(rng, B=1, Hq=2, Hkv=1, D=4, L_cap=10, lens=[10])
    args = dict(S=1, W=1, lam=0.1, lens=[10], sm=0.5)
    args.update(bad)
    with pytest.raises(ValueError):
        oracle.spec_decode(q, k, v, args["lens"], args["S"], args["W"],
                           args["lam"], sm_scale=args["sm"])
