"""Helpers of the GPU parity tests: move seeded host inputs to the device,
run the library through its C ABI, and compare with the CPU oracle."""
import math

import numpy as np

TOL = {"f32": 1e-5, "bf16": 2e-3}   # per-entry relative L2 of outputs
RATIO_TOL = 1e-4                    # |ratio_gpu - ratio_oracle|
LSE_TOL = 1e-4                      # |lse_gpu - lse_oracle| (nats)
FLAG_BAND = 1e-4                    # flags may differ within this of lambda


def to_device(q, k, v, dev="cuda"):
    import torch
    qd = torch.from_numpy(np.ascontiguousarray(q)).to(dev)
    if k.dtype == np.uint16:
        kd = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).to(dev)
        vd = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        kd = torch.from_numpy(k).to(dev)
        vd = torch.from_numpy(v).to(dev)
    return qd, kd, vd


def run_fused(al, h, p, qd, kd, vd, two_streams=True, ws=None):
    import torch
    out = al.alloc_outputs(p)
    if ws is None:
        ws = al.alloc_workspace(p)
    if two_streams:
        sa = torch.cuda.Stream()
        se = torch.cuda.Stream()
        sa.wait_stream(torch.cuda.current_stream())
        se.wait_stream(torch.cuda.current_stream())
        al.spec_decode(h, p, qd, kd, vd, out, ws, sa, se)
        torch.cuda.current_stream().wait_stream(se)
        torch.cuda.current_stream().wait_stream(sa)
    else:
        al.spec_decode(h, p, qd, kd, vd, out, ws)
    torch.cuda.synchronize()
    return {k_: v_.cpu().numpy() for k_, v_ in out.items()}


def run_standalone(al, h, p, qd, kd, vd, include_sink_window=False):
    """sink_approx, then exact splits, lse_combine and verify, one stream."""
    import torch
    out = al.alloc_outputs(p)
    ws = al.alloc_workspace(p)
    al.sink_approx(h, p, qd, kd, vd, out["o_approx"], out["lse_approx"], ws)
    if include_sink_window:
        ws2 = al.alloc_workspace(p)
        al.flash_decode_exact(h, p, qd, kd, vd, 1, ws2)
        al.lse_combine(h, p, ws2, out["o_exact"], out["lse_exact"])
    else:
        al.flash_decode_exact(h, p, qd, kd, vd, 0, ws)
        al.lse_combine(h, p, ws, out["o_exact"], out["lse_exact"])
    al.verify(h, p, out["o_approx"], out["o_exact"], out["ratio"],
              out["commit"], out["o_committed"])
    torch.cuda.synchronize()
    return {k_: v_.cpu().numpy() for k_, v_ in out.items()}


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return np.linalg.norm(a - b) / n if n > 0 else np.linalg.norm(a - b)


# Worst errors of every compare() call in this process, by label (written
# out at the end of the session when ALSPEC_MARGINS names a file).
MARGINS = []


def compare(got, ref, kv_dtype, lam, label=""):
    """Assert parity of one call's outputs with the oracle; returns a dict
    of the worst errors.

    For O_exact and O_approx of every batch entry, three bars at the same
    tolerance tol (1e-5 fp32 KV, 2e-3 bf16 KV):
      - the entry's relative L2 error over its Hq*D outputs;
      - every query head's relative L2 error over its D outputs, so that a
        wrong head cannot hide in the entry's norm;
      - every element: |got - ref| <= tol * max|ref| over the entry, so that
        a wrong lane or element cannot either.
    Then lse within 1e-4 nats, the ratio within 1e-4, flags equal outside
    the 1e-4 band around lambda, and the committed output equal, bit for
    bit, to the output its flag selects."""
    tol = TOL[kv_dtype]
    B = ref["ratio"].shape[0]
    worst = {"o_exact": 0.0, "o_approx": 0.0, "o_exact_head": 0.0,
             "o_approx_head": 0.0, "o_exact_elem": 0.0, "o_approx_elem": 0.0,
             "ratio": 0.0, "lse": 0.0}
    for b in range(B):
        if not np.isfinite(ref["ratio"][b]):
            continue
        for key in ("o_exact", "o_approx"):
            g = np.asarray(got[key][b], np.float64)
            r = np.asarray(ref[key][b], np.float64)
            e = rel_l2(g, r)
            worst[key] = max(worst[key], e)
            assert e <= tol, f"{label} entry {b} {key} rel err {e:.3g} > {tol}"
            for h in range(r.shape[0]):
                eh = rel_l2(g[h], r[h])
                worst[key + "_head"] = max(worst[key + "_head"], eh)
                assert eh <= tol, (f"{label} entry {b} head {h} {key} rel "
                                   f"err {eh:.3g} > {tol}")
            scale = np.abs(r).max()
            de = np.abs(g - r).max() / scale if scale > 0 else \
                np.abs(g - r).max()
            worst[key + "_elem"] = max(worst[key + "_elem"], de)
            if de > tol:
                h, d = np.unravel_index(np.argmax(np.abs(g - r)), r.shape)
                raise AssertionError(
                    f"{label} entry {b} {key}[{h}][{d}] = {g[h, d]!r}, "
                    f"oracle {r[h, d]!r}: error {de:.3g} of the entry's "
                    f"largest output > {tol}")
        for gk, rk in (("lse_exact", "lse_exact"), ("lse_approx", "lse_approx")):
            d = np.abs(got[gk][b] - ref[rk][b]).max()
            worst["lse"] = max(worst["lse"], d)
            assert d <= LSE_TOL, f"{label} entry {b} {gk} err {d:.3g}"
        dr = abs(float(got["ratio"][b]) - ref["ratio"][b])
        worst["ratio"] = max(worst["ratio"], dr)
        assert dr <= RATIO_TOL, f"{label} entry {b} ratio err {dr:.3g}"
        if abs(ref["ratio"][b] - lam) > FLAG_BAND:
            assert int(got["commit"][b]) == int(ref["commit"][b]), (
                f"{label} entry {b} flag {got['commit'][b]} vs "
                f"{ref['commit'][b]} (ratio {ref['ratio'][b]:.6f})")
        sel = got["o_approx"][b] if got["commit"][b] else got["o_exact"][b]
        assert np.array_equal(got["o_committed"][b], sel), \
            f"{label} entry {b} committed output"
    MARGINS.append({"label": label, "kv_dtype": kv_dtype, "tol": tol,
                    **{k_: float(v_) for k_, v_ in worst.items()}})
    return worst


def is_close_flag_case(ref, lam):
    return bool(np.any(np.abs(ref["ratio"] - lam) <= FLAG_BAND))
