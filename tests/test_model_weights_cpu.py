"""The chained decode step's synthetic weights (host only): the planted
column of the next QKV makes each query carry a * u of its kv head's
planted direction, through the RMSNorm of a residual stream with one
dominant coordinate -- the same structure the generator gives its queries
(q = noise + a * u), so the step's layers find the planted sink."""
import math

import numpy as np
import pytest
import torch

from synth import gen
from synth import post_gen as pg


def _rmsnorm(h, w, eps=1e-5):
    return h / torch.sqrt((h * h).mean() + eps) * w


@pytest.mark.parametrize("hidden,D,Hq,Hkv", [(256, 32, 4, 2), (512, 64, 8, 2)])
def test_planted_query_carries_a_u(hidden, D, Hq, Hkv):
    G = Hq // Hkv
    g_ = torch.Generator().manual_seed(5)
    qkv_dim = (Hq + 2 * Hkv) * D
    w_qkv = torch.randn(qkv_dim, hidden, generator=g_) / hidden ** 0.5
    norm = 1.0 + 0.1 * torch.randn(hidden, generator=g_)
    rng = np.random.default_rng(3)
    dirs = []
    for _ in range(Hkv):
        z = rng.standard_normal(D)
        dirs.append(z / np.linalg.norm(z))
    a = 8.0
    dim = 7
    pg.plant_query_direction(w_qkv, norm, dirs, a, D, G, hidden, dim=dim)
    # weights as the step stores them: bf16
    w_b = w_qkv.to(torch.bfloat16).float()
    n_b = norm.to(torch.bfloat16).float()
    for trial in range(4):
        h = torch.randn(hidden, generator=g_) * (1 + 3 * trial)
        h[dim] = pg.MASSIVE_VALUE
        q = (w_b[:Hq * D] @ _rmsnorm(h, n_b)).reshape(Hq, D).double()
        for hq in range(Hq):
            u = torch.from_numpy(dirs[hq // G])
            proj = float(q[hq] @ u)
            # the rest is the random product of the small coordinates: of
            # the order of the generator's query noise (N(0,1)/sqrt(D) per
            # element, norm about 1), growing with the residual's spread
            rest = float(torch.linalg.norm(q[hq] - proj * u))
            assert rest < 1.5, (trial, hq, rest)
            # the planted part: a, within the bf16 rounding, the norm's
            # share of the other coordinates (a few 1e-3) and the noise's
            # own component along u (about rest / sqrt(D); 4 sigma)
            assert abs(proj - a) < 0.02 * a + 4 * rest / math.sqrt(D), \
                (trial, hq, proj, rest)
            # and no other kv head's direction is planted in this head
            for g in range(Hkv):
                if g != hq // G:
                    other = float(q[hq] @ torch.from_numpy(dirs[g]))
                    assert abs(other - a * float(
                        torch.from_numpy(dirs[g]) @ u)) < 0.5


def test_untouched_entries_and_norm_weight():
    hidden, D, Hq, Hkv = 128, 16, 4, 4
    w = torch.randn((Hq + 2 * Hkv) * D, hidden)
    n = torch.randn(hidden)
    w0, n0 = w.clone(), n.clone()
    dirs = [np.eye(D)[i] for i in range(Hkv)]
    pg.plant_query_direction(w, n, dirs, 8.0, D, 1, hidden, dim=3)
    assert n[3] == 1.0
    mask = torch.ones_like(w, dtype=torch.bool)
    mask[:Hq * D, 3] = False
    assert torch.equal(w[mask], w0[mask])          # only the query column
    assert torch.equal(torch.cat([n[:3], n[4:]]), torch.cat([n0[:3], n0[4:]]))
    for h in range(Hq):
        col = w[h * D:(h + 1) * D, 3]
        assert torch.allclose(col, torch.from_numpy(dirs[h]).float() *
                              8.0 / math.sqrt(hidden))


def test_generator_queries_have_the_same_structure():
    """The generator's own queries: q . u = a + noise of the base elements,
    the component the planted weights reproduce."""
    w = gen.scaled(gen.llama8b_32k(), 300)
    q = gen.q_all(w, 0)
    for g in range(w.Hkv):
        u = gen.head_plant(w, 0, 0, g).u
        for h in range(g * w.G, (g + 1) * w.G):
            assert abs(float(q[0, h] @ u) - w.const.a) < 0.5
