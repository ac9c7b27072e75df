#!/usr/bin/env python3
"""Benchmark of the speculative flash-decode step of attention-level
speculation (ALSpec) on one MI355X.

Workload (the headline long-context case): one user's decode token through
32 layers of Llama-3-8B-shaped attention -- 32 query heads over 8 kv heads,
head dim 128, bf16 KV with fp32 arithmetic, context 131072 (512 MiB of KV
per layer), sink 4, window 2048, lambda 0.10 -- for needle densities
0, 1, 2, 4, 8 and 16 per kv head.  All 6 x 32 layers (96 GiB) are drawn on
the device by the seeded generator and stay resident.  A step is one token
through the 32 layers of one density (densities rotate step by step); each
layer is one fused call of the library: sink+window approximation, exact
split-K pass over the middle, merge, relative-L2 verify and commit.

Schedules (overlap modes of the library):
  pipelined  -- the speculative order (overlap mode 2), captured once per
                density as a HIP graph and replayed: the exact split-K
                passes of successive layers back to back on one stream,
                each after the previous layer's approximation (under
                speculation the query comes from it); approximations on a
                second stream; merge, verify and commit on the library's
                verify stream, off the exact passes' path.  Every layer has
                its own workspace.
  pipelined_verify_on_exact_stream -- the same with overlap mode 1 (merge
                and verify between successive exact passes), as a graph.
  sequential -- every layer's approximation, exact pass and verify one
                after another on one stream (overlap mode 0), as a graph.
  pipelined_eager -- overlap mode 2 issued call by call without a graph.
  layer_pipelined -- alspec_spec_decode_layers on one stream: launch j runs
                the merge of layer j's approximation, layer j's exact
                split-K pass, layer j+1's sink and window splits and layer
                j-1's merge/verify/commit as disjoint block ranges of one
                grid; stream order carries the dependencies.  Three
                workspaces in a ring.  Issued eagerly, and
                (layer_pipelined_graph) as a graph.
  exact_only_baseline -- not speculative: exact attention over every split
                and its merge per layer (alspec_flash_decode_exact with the
                sink and window splits, alspec_lse_combine), as a graph;
                reported beside the headline as the cost of speculation.
  static_sink_baseline -- the pages' static attention-sink baseline: the
                approximation alone (alspec_sink_approx) as the layer's
                output, no exact pass and no verify, as a graph.
  fixed_layer_sink_baseline -- the pages' attention sink at fixed layers:
                the static approximation on the odd layers, exact attention
                (as in the exact-only baseline) on the even ones, as a graph.
The headline value is the throughput of the fastest speculative schedule
(named in config.schedule).  They compute the same outputs, bit for bit
(every schedule takes the same split plan).  The baselines are reported
beside it,
with each one's output error against exact attention on the same inputs.

Also reported: KV GB/s of the headline schedule's dominant kernel against
the HBM peak (for the layer-pipelined schedules its kernel in the steady
state, from HIP events around back-to-back chains of all layers and of two;
beside it the exact split-K kernel alone, from HIP events around
back-to-back launches over all resident layers), per-kernel HIP events in
eagerly issued steps of the schedules, the speculation
hit rate per density, each layer's time to its approximate and to its
verified output and the critical-path time a commit saves, the chained
decode step with the post-attention operators (model_step: eager two-stream
overlap and the one-stream form as one HIP graph, with the operators'
own HBM roofline), a two-GPU projection from the measured durations, the
HBM probe, and the CPU oracle timed on a bounded sample of the same
layers.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("spec flash-decode tokens·layers/s + KV GB/s (% HBM peak) at "
          "128K; hit rate")
HBM_PEAK_GBPS = 8000.0
EVENT_NAMES = ("approx_begin", "approx_end", "exact_begin", "exact_end",
               "verify_end")

# HBM bytes per launch of each roofline kernel on this workload, from
# rocprofv3 FETCH_SIZE and WRITE_SIZE runs, scaled by what the counters read
# for a copy kernel of known size (fetch x2.000, write x1.000).  Valid only
# for the kernel and plan sources they were taken on (sha256 of the files
# below); once those change the figures are withheld until measured again.
TRAFFIC = {"sources": ("attention_level_speculation_amd/csrc/alspec_kernels.hip",
                       "attention_level_speculation_amd/csrc/alspec_kernels.h",
                       "attention_level_speculation_amd/csrc/alspec_plan.h",
                       "attention_level_speculation_amd/csrc/alspec_plan.cpp"),
           "sha256": "ec93685d7c6304dd62558aef1d105358"
                     "0b1d6958527130677d5bc31f7a993072",
           # (fetch, write) per launch: the per-layer chain kernel in its
           # steady state (all four block ranges), the exact split-K pass,
           # the one-launch chain of the 32 layers at 128K, and the two
           # chain forms of the 32K, multi-user and 70B configurations
           # (the one-launch chain over all of their layers)
           "bytes": {"chain": (262912.0 * 1024 * 2.0, 862.6 * 1024 * 1.0),
                     "partials_middle": (258181.1 * 1024 * 2.0,
                                         520.0 * 1024 * 1.0),
                     "one_chain": (8405447.9 * 1024 * 2.0,
                                   30015.5 * 1024 * 1.0),
                     "c2_one_chain": (2114859.2 * 1024 * 2.0,
                                      29449.3 * 1024 * 1.0),
                     "c2_chain": (66303.8 * 1024 * 2.0, 846.6 * 1024 * 1.0),
                     "c4_one_chain": (51413771.4 * 1024 * 2.0,
                                      48896.1 * 1024 * 1.0),
                     "c4_chain": (1607038.4 * 1024 * 2.0, 1432.5 * 1024 * 1.0),
                     "c5_one_chain": (84013249.6 * 1024 * 2.0,
                                      186951.1 * 1024 * 1.0),
                     "c5_chain": (1050750.6 * 1024 * 2.0,
                                  2213.7 * 1024 * 1.0)}}


def measured_traffic(kernel):
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC["sources"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != TRAFFIC["sha256"] or kernel not in TRAFFIC["bytes"]:
        return None
    fetch, write = TRAFFIC["bytes"][kernel]
    return fetch + write


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=120)
    ap.add_argument("--warmup", type=int, default=12)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--densities", default="0,1,2,4,8,16")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--window-split-tokens", type=int, default=0)
    ap.add_argument("--ws-ring", type=int, default=0,
                    help="workspaces the eager pipelined schedule cycles "
                         "through (0: one per layer)")
    ap.add_argument("--chain-ring", type=int, default=6,
                    help="workspaces the layer-pipelined chains cycle "
                         "through (at least 3; from 4 on no layer's splits "
                         "wait for an earlier layer's verify)")
    ap.add_argument("--schedules",
                    default="pipe,pipe1,seq,pipe_eager,chain,chain_graph,"
                            "chainL,chainL_graph,exact,sink,fixsink",
                    help="schedules to time (the fastest is the headline)")
    ap.add_argument("--no-events", action="store_true",
                    help="skip the instrumented runs (per-layer latencies)")
    ap.add_argument("--kernel-launches", type=int, default=768,
                    help="back-to-back launches timed for the roofline: of "
                         "the exact split-K kernel, and about as many of the "
                         "layer-pipelined kernel (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--configs", default="c2,c4,c5",
                    help="other configurations timed as layer-pipelined "
                         "chains after the headline: c2 (8B shape at 32K), "
                         "c4 (8 users, ragged 64K-128K), c5 (70B shape, 4 "
                         "users at 128K, 80 layers); 'none' to skip")
    ap.add_argument("--model-steps", type=int, default=10,
                    help="timed tokens of the chained decode step with "
                         "post-attention work (0: skip)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (world size "
              f"{world}) is not supported: this path has no multi-GPU "
              "sharding: every figure is for one GPU's full share.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import attention_level_speculation_amd as al
    from attention_level_speculation_amd import _binding as B_
    from synth import device as sdev
    from synth import gen

    dens = [int(x) for x in args.densities.split(",")]
    nd = len(dens)
    nl = args.layers
    works = [gen.llama8b_128k(needles=n) for n in dens]
    w0 = works[0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs resident in HBM --------------------------------------
    t0 = time.time()
    Ks, Vs, Qs = [], [], []
    for di, w in enumerate(works):
        K = torch.empty((nl, w.B, w.Hkv, w.L_cap, w.D), dtype=torch.bfloat16,
                        device=dev)
        V = torch.empty_like(K)
        Q = torch.empty((nl, w.B, w.Hq, w.D), dtype=torch.float32, device=dev)
        for layer in range(nl):
            sdev.fill_kv(w, layer, K[layer], V[layer])
            Q[layer].copy_(torch.from_numpy(gen.q_all(w, layer)))
        torch.cuda.synchronize()
        Ks.append(K)
        Vs.append(V)
        Qs.append(Q)
        log(f"drew needles={dens[di]}: {nl} layers "
            f"({2 * K.numel() * 2 / 2**30:.1f} GiB) t={time.time() - t0:.1f}s")

    def params(overlap):
        return al.params_for(w0, split_tokens=args.split_tokens,
                             window_split_tokens=args.window_split_tokens,
                             overlap=overlap)
    # schedules: name -> (overlap mode, captured as a graph); "exact" is the
    # non-speculative baseline: exact attention over every split, no
    # approximation and no verify
    modes = {"pipe": (2, True), "pipe1": (1, True), "seq": (0, True),
             "pipe_eager": (2, False), "chain": (None, False),
             "chain_graph": (None, True), "chainL": (None, False),
             "chainL_graph": (None, True), "exact": (None, True),
             "sink": (None, True), "fixsink": (None, True)}
    P = {m: params(ov or 0) for m, (ov, _) in modes.items()}
    # the layer-pipelined chain in one launch per layer
    P["chainL"] = params(1)
    P["chainL_graph"] = params(1)
    splits, (T, Tw) = al.plan_splits(P["seq"], 0)
    n_mid = sum(1 for s in splits if s[0] == 2)
    mid_tokens = sum(e - b for k, b, e in splits if k == 2)
    a_tokens = sum(e - b for k, b, e in splits if k != 2)
    bytes_per_token = w0.Hkv * w0.D * 2 * 2           # K and V, bf16
    mid_bytes = mid_tokens * bytes_per_token * w0.B   # one exact launch
    layer_bytes = sum(w0.seq_lens) * bytes_per_token  # every KV byte
    h = al.Handle(0)
    # workspaces: the sequential schedule runs each call on one stream and
    # reuses one; each captured pipelined layer gets its own (the library
    # adds no workspace ordering under capture); the eager pipelined
    # schedule cycles through a ring, ordered by the library
    if args.chain_ring < al.LAYERS_WS_RING:
        raise SystemExit(f"--chain-ring must be at least {al.LAYERS_WS_RING}")
    ring = min(nl, args.chain_ring)
    n_ws = {"seq": 1, "pipe": nl, "pipe1": nl,
            "pipe_eager": args.ws_ring or nl, "chain": ring,
            "chain_graph": ring, "chainL": ring, "chainL_graph": ring,
            "exact": 1, "sink": 1, "fixsink": 1}
    WS = {m: [al.alloc_workspace(P[m], dev) for _ in range(n_ws[m])]
          for m in modes}
    outs = [[al.alloc_outputs(P["seq"], dev) for _ in range(nl)]
            for _ in range(nd)]
    sa = torch.cuda.Stream(device=dev)
    se = torch.cuda.Stream(device=dev)
    cap = torch.cuda.Stream(device=dev)
    cur = torch.cuda.current_stream()
    fn = B_._spec_decode

    def call_args(p, di, layer, ws):
        o = outs[di][layer]
        return [h.ptr, ctypes.byref(p), Qs[di][layer].data_ptr(),
                Ks[di][layer].data_ptr(), Vs[di][layer].data_ptr(),
                o["o_approx"].data_ptr(), o["lse_approx"].data_ptr(),
                o["o_exact"].data_ptr(), o["lse_exact"].data_ptr(),
                o["ratio"].data_ptr(), o["commit"].data_ptr(),
                o["o_committed"].data_ptr(), ws.data_ptr(), ws.numel(),
                sa.cuda_stream, se.cuda_stream]
    A = {m: [[call_args(P[m], di, l, WS[m][l % len(WS[m])])
              for l in range(nl)] for di in range(nd)] for m in modes}

    def exact_args(di, layer):
        o, ws = outs[di][layer], WS["exact"][0]
        p = ctypes.byref(P["exact"])
        return ([h.ptr, p, Qs[di][layer].data_ptr(), Ks[di][layer].data_ptr(),
                 Vs[di][layer].data_ptr(), 1, ws.data_ptr(), ws.numel(),
                 se.cuda_stream],
                [h.ptr, p, ws.data_ptr(), ws.numel(),
                 o["o_exact"].data_ptr(), o["lse_exact"].data_ptr(),
                 se.cuda_stream])
    AX = [[exact_args(di, l) for l in range(nl)] for di in range(nd)]

    def sink_args(di, layer):
        o, ws = outs[di][layer], WS["sink"][0]
        return [h.ptr, ctypes.byref(P["sink"]), Qs[di][layer].data_ptr(),
                Ks[di][layer].data_ptr(), Vs[di][layer].data_ptr(),
                o["o_approx"].data_ptr(), o["lse_approx"].data_ptr(),
                ws.data_ptr(), ws.numel(), se.cuda_stream]
    AS = [[sink_args(di, l) for l in range(nl)] for di in range(nd)]

    # layer-pipelined chains: one alspec_layer array per (schedule, density)
    AC = {m: [B_.layers_struct(P[m], [
        (Qs[di][l], Ks[di][l], Vs[di][l], outs[di][l], WS[m][l % len(WS[m])])
        for l in range(nl)]) for di in range(nd)]
        for m in ("chain", "chain_graph", "chainL", "chainL_graph")}

    def new_events():
        evs = {n: torch.cuda.Event(enable_timing=True) for n in EVENT_NAMES}
        for ev_ in evs.values():
            ev_.record(se)           # torch creates the hipEvent on record
        return B_.Events(*[evs[n].cuda_event for n in EVENT_NAMES]), evs

    # Chain events: layer l's exact pass needs its query, which under
    # speculation comes from layer l-1's approximation.  They only order
    # two streams of this device, so they are created without the
    # system-scope fence a default event takes on completion (the HIP
    # runtime torch loaded, reached by its soname).
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreateWithFlags.argtypes = [ctypes.c_void_p, ctypes.c_uint]
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_uint]
    chain = []
    for _ in range(nl):
        e_ = ctypes.c_void_p()
        if hip.hipEventCreateWithFlags(ctypes.byref(e_),
                                       0x2 | 0x20000000) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        chain.append(e_)
    sa_p, se_p = ctypes.c_void_p(sa.cuda_stream), ctypes.c_void_p(se.cuda_stream)

    def enqueue(mode, di, evrow=None):
        """One step (all layers of density di) on sa/se; evrow: per-layer
        (Events struct, dict) for instrumented runs."""
        if mode == "exact":
            for fa, la in AX[di]:
                st = B_._flash_exact(*fa) or B_._lse_combine(*la)
                if st != 0:
                    raise al.AlspecError(st, "exact-only baseline")
            return
        if mode in ("chain", "chain_graph", "chainL", "chainL_graph"):
            st = B_._spec_decode_layers(h.ptr, ctypes.byref(P[mode]), nl,
                                        AC[mode][di], se.cuda_stream)
            if st != 0:
                raise al.AlspecError(st, "alspec_spec_decode_layers")
            return
        if mode == "sink":
            for sa_ in AS[di]:
                st = B_._sink_approx(*sa_)
                if st != 0:
                    raise al.AlspecError(st, "static-sink baseline")
            return
        if mode == "fixsink":
            for layer in range(nl):
                if layer % 2:
                    st = B_._sink_approx(*AS[di][layer])
                else:
                    fa, la = AX[di][layer]
                    st = B_._flash_exact(*fa) or B_._lse_combine(*la)
                if st != 0:
                    raise al.AlspecError(st, "fixed-layer sink baseline")
            return
        for layer in range(nl):
            if mode != "seq" and layer > 0:
                # the approximation stream holds nothing after the previous
                # layer's approximation
                if (hip.hipEventRecord(chain[layer], sa_p) != 0 or
                        hip.hipStreamWaitEvent(se_p, chain[layer], 0) != 0):
                    raise RuntimeError("chain event failed")
            ev = None if evrow is None else ctypes.byref(evrow[layer][0])
            st = fn(*A[mode][di][layer], ev)
            if st != 0:
                raise al.AlspecError(st, "alspec_spec_decode")

    def issue(mode, di, evrow=None):
        """One eager step, ordered after the current stream and joined
        back into it."""
        sa.wait_stream(cur)
        se.wait_stream(cur)
        enqueue(mode, di, evrow)
        if modes[mode][0] == 2:
            al.order_after_verify(h, cur)
        cur.wait_stream(sa)
        cur.wait_stream(se)

    def capture(mode, di):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            sa.wait_stream(cap)
            se.wait_stream(cap)
            enqueue(mode, di)
            if modes[mode][0] == 2:
                al.order_after_verify(h, cap)   # joins the verify stream
            cap.wait_stream(sa)
            cap.wait_stream(se)
        return g

    torch.cuda.synchronize()
    graphs = {m: [capture(m, di) for di in range(nd)]
              for m, (_, g) in modes.items()
              if g and m in args.schedules.split(",")}
    log(f"plan: split {T} (middle splits {n_mid}), window split {Tw}; "
        f"captured {len(graphs) * nd} step graphs")

    def timed(mode):
        def step(s_):
            if mode in graphs:
                graphs[mode][s_ % nd].replay()
            else:
                issue(mode, s_ % nd)
        torch.cuda.synchronize()
        for s_ in range(args.warmup):
            step(s_)
        torch.cuda.synchronize()          # barrier: one rank
        t_start = time.perf_counter()
        for s_ in range(args.steps):
            step(s_)
        torch.cuda.synchronize()
        return time.perf_counter() - t_start

    res = {}
    sched = args.schedules.split(",")
    for mode, key in (("pipe", "pipelined"),
                      ("pipe1", "pipelined_verify_on_exact_stream"),
                      ("seq", "sequential"),
                      ("pipe_eager", "pipelined_eager"),
                      ("chain", "layer_pipelined"),
                      ("chain_graph", "layer_pipelined_graph"),
                      ("chainL", "layer_pipelined_per_layer_launch"),
                      ("chainL_graph", "layer_pipelined_per_layer_launch_graph"),
                      ("exact", "exact_only_baseline"),
                      ("sink", "static_sink_baseline"),
                      ("fixsink", "fixed_layer_sink_baseline")):
        if mode not in sched:
            continue
        wall_ = timed(mode)
        log(f"{key}: {args.steps} steps in {wall_:.3f} s")
        res[key] = {"overlap_mode": modes[mode][0],
                    "hip_graph": modes[mode][1],
                    "ms_per_step": wall_ / args.steps * 1e3,
                    "tokens_layers_per_s": w0.B * nl * args.steps / wall_}
    # headline: the fastest speculative schedule (each computes the same
    # outputs); the exact-only baseline is reported beside it
    best = max((k_ for k_ in res if not k_.endswith("_baseline")),
               key=lambda k_: res[k_]["tokens_layers_per_s"])
    wall = res[best]["ms_per_step"] * args.steps / 1e3

    # ---- instrumented runs: HIP events around every kernel --------------
    # (eager calls: the HIP runtime loaded with torch rejects event records
    # inside a stream capture, so the events bracket eagerly issued steps
    # of the same schedule, each recorded on the stream its kernel runs on)
    if not args.no_events:
        for mode, key in (("pipe", "pipelined"), ("seq", "sequential")):
            if mode not in sched:
                continue
            rows = [[new_events() for _ in range(nl)] for _ in range(nd)]
            ex, t_ap, t_ex, saved, tot = [], [], [], 0.0, 0.0
            reps = max(1, args.steps // nd)
            for rep in range(reps + 1):
                for di in range(nd):
                    torch.cuda.synchronize()
                    ref_ev = torch.cuda.Event(enable_timing=True)
                    ref_ev.record(cur)
                    issue(mode, di, rows[di])
                    torch.cuda.synchronize()
                    if rep == 0:
                        continue          # warm-up pass

                    def at(ev):
                        return ref_ev.elapsed_time(ev) * 1e3   # us
                    for layer in range(nl):
                        e = rows[di][layer][1]
                        a0, a1 = at(e["approx_begin"]), at(e["approx_end"])
                        e0, e1 = at(e["exact_begin"]), at(e["exact_end"])
                        v1 = at(e["verify_end"])
                        ex.append(e1 - e0)
                        # approximate output: its kernels' span; verified
                        # output: from the exact pass's start
                        t_ap.append(a1 - a0)
                        t_ex.append(v1 - e0)
                        if int(outs[di][layer]["commit"][0].item()):
                            saved += max(0.0, v1 - a1)
                        tot += max(v1, a1) - min(a0, e0)
            ex = np.array(ex)
            res[key].update({
                "exact_kernel_us_mean": float(ex.mean()),
                "exact_kernel_us_p10": float(np.percentile(ex, 10)),
                "exact_kernel_us_p90": float(np.percentile(ex, 90)),
                "exact_kernel_launches_timed": int(ex.size),
                "approx_latency_us_mean": float(np.mean(t_ap)),
                "exact_latency_us_mean": float(np.mean(t_ex)),
                "approx_over_exact": float(np.mean(t_ap) / np.mean(t_ex)),
                "committed_time_saved_frac": saved / tot if tot > 0 else 0.0,
                "instrumented_schedule": "eager, HIP events per kernel",
            })
        log("instrumented runs done")

    # ---- hit rate -------------------------------------------------------
    hits = {}
    allc = []
    for di, n in enumerate(dens):
        c = [int(outs[di][layer]["commit"][0].item()) for layer in range(nl)]
        hits[str(n)] = sum(c) / len(c)
        allc += c
    hit_rate = sum(allc) / len(allc)

    # ---- output error against exact attention (same inputs) -------------
    # per (user, layer), the relative L2 error of the layer's attention
    # output: the verify's ratio where the approximation stands, 0 where
    # exact attention does.  The pages score tasks, which synthetic inputs
    # cannot; this is the error the verify bounds.
    ratio = np.array([[outs[di][layer]["ratio"].cpu().numpy()
                       for layer in range(nl)] for di in range(nd)])
    commit = np.array([[outs[di][layer]["commit"].cpu().numpy()
                        for layer in range(nl)] for di in range(nd)]) != 0
    odd = (np.arange(nl) % 2 == 1)[None, :, None]

    def err_stats(e):
        return {"mean": float(e.mean()), "max": float(e.max()),
                "frac_over_lambda": float((e > w0.lam).mean())}
    quality = {
        "measure": "relative L2 error of the attention output against "
                   "exact attention, per (user, layer), over every "
                   "density and layer",
        "speculative": err_stats(np.where(commit, ratio, 0.0)),
        "static_sink_baseline": err_stats(ratio),
        "fixed_layer_sink_baseline": err_stats(np.where(odd, ratio, 0.0)),
        "exact_only_baseline": err_stats(np.zeros_like(ratio)),
    }

    out = {
        "metric": METRIC,
        "value": w0.B * nl * args.steps / wall,
        "unit": "tokens·layers/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded Philox generator, planted sink and "
                "needles; no datasets, no weights",
        "config": {
            "workload": "llama3-8b-shaped decode attention, context 131072, "
                        "batch 1, 32 q / 8 kv heads, head dim 128, bf16 KV, "
                        f"{nl} layers, sink 4, window 2048, lambda 0.10, "
                        f"needles per kv head {dens}",
            "schedule": best,
            "kv_dtype": "bf16", "arith": "f32", "context": w0.L_cap,
            "batch": w0.B, "layers": nl, "num_q_heads": w0.Hq,
            "num_kv_heads": w0.Hkv, "head_dim": w0.D, "sink": w0.S,
            "window": w0.W, "lambda": w0.lam, "split_tokens": T,
            "window_split_tokens": Tw,
            "middle_splits_per_head": n_mid,
            "generator": {"a": w0.const.a, "c_s": w0.const.c_s,
                          "tau_s": w0.const.tau_s, "c_n": w0.const.c_n,
                          "tau_n": w0.const.tau_n},
        },
        "library": _library_record(al.LIB_PATH),
        "hit_rate": hit_rate,
        "hit_rate_by_needles": hits,
        "output_error": quality,
        "kv_bytes_per_layer": layer_bytes,
        "step_kv_GBps": layer_bytes * nl * args.steps / wall / 1e9,
    }
    out["step_hbm_frac"] = out["step_kv_GBps"] / HBM_PEAK_GBPS
    out.update(res)
    # ---- the pages' measure: attention latency overhead ------------------
    # With speculation a layer's attention costs the approximation where it
    # commits and exact attention where it discards; without, always exact
    # attention.  Per-layer device times of back-to-back layers captured as
    # HIP graphs: exact attention alone (the exact-only baseline) and the
    # approximation alone (the static-sink baseline).
    if "exact_only_baseline" in res and "static_sink_baseline" in res:
        t_e = res["exact_only_baseline"]["ms_per_step"] * 1e3 / nl
        t_a = res["static_sink_baseline"]["ms_per_step"] * 1e3 / nl
        out["attention_overhead_reduction"] = {
            "value": overhead_reduction(t_e, t_a, hit_rate),
            "by_needles": {n_: overhead_reduction(t_e, t_a, h_)
                           for n_, h_ in hits.items()},
            "t_exact_us": t_e, "t_approx_us": t_a, "hit_rate": hit_rate,
            "approx_over_exact": t_a / t_e,
            "formula": "t_exact / (hit_rate * t_approx + (1 - hit_rate) "
                       "* t_exact)",
            "inputs": "per-layer device time of back-to-back layers "
                      "captured as HIP graphs: exact attention alone "
                      "(exact_only_baseline) and the approximation alone "
                      "(static_sink_baseline); hit rate of this run"}
    for key in ("pipelined", "sequential"):
        r_ = res.get(key, {})
        if "approx_latency_us_mean" in r_:
            r_["attention_overhead_reduction"] = overhead_reduction(
                r_["exact_latency_us_mean"], r_["approx_latency_us_mean"],
                hit_rate)
    if "exact_only_baseline" in res:
        # time a speculative step costs over exact attention alone
        out["speculation_cost_frac"] = (
            res[best]["ms_per_step"] /
            res["exact_only_baseline"]["ms_per_step"] - 1.0)
    # ---- roofline: the dominant kernel of the headline schedule ---------
    # (the layer-pipelined kernel for the chain schedules, else the exact
    # split-K kernel), and the exact split-K kernel alone beside it
    if args.kernel_launches > 0:
        us = kernel_timing(args, al, B_, h, P["seq"], Qs, Ks, Vs, se, nd, nl)
        achieved = mid_bytes / (us * 1e-6) / 1e9
        exact_pass = {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
            "traffic": measured_traffic("partials_middle"),
            "kernel": "partials_kernel<KvBf16,128,4,false> (exact split-K "
                      "pass over the middle)",
            "algorithmic_bytes_per_launch": mid_bytes,
            "launch_us_mean": us,
            "launches_timed": args.kernel_launches,
        }
        if best.startswith("layer_pipelined"):
            key = "chainL" if "per_layer_launch" in best else "chain"
            lus, cus, group, reps = chain_timing(args, B_, h, P[key], AC[key],
                                                 se, nl)
            if group > 1:
                # the whole chain is one launch: its bytes over its duration
                achieved = layer_bytes * group / (cus * 1e-6) / 1e9
                kern = ("one_chain_kernel<KvBf16,128,4> (the whole chain of "
                        f"{group} layers in one launch, items taken from a "
                        "queue: merges of sink and window states, sink and "
                        "window splits of the next layer, middle splits, "
                        "verifies of the layer before; the launch time "
                        "includes the layer-table writer before it)")
            else:
                achieved = layer_bytes / (lus * 1e-6) / 1e9
                kern = ("chain_kernel<KvBf16,128,4> (steady state: middle "
                        "splits of layer j, dispatched first, sink and "
                        "window splits of layer j+1, merge of layer j's "
                        "approximation, verify of layer j-1)")
                # when the approximate output is there: every block of the
                # launch is resident from its start, so layer j's merge
                # ends a few microseconds into launch j, and its verdict
                # and committed output a few into launch j+1
                res[best]["approximate_output"] = {
                    "ready": "layer j's approximate output is merged by "
                             "blocks of launch j that start with it (its "
                             "sink and window splits ran in launch j-1); "
                             "its exact output, verdict and committed "
                             "output come from blocks of launch j+1",
                    "lead_over_committed_output_us": lus,
                    "lead_measure": "one steady launch (HIP events, as "
                                    "roofline.launch_us_mean)"}
            out["roofline"] = {
                "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                "traffic": measured_traffic("one_chain" if group > 1
                                            else "chain"),
                "kernel": kern,
                "algorithmic_bytes_per_launch": layer_bytes * group,
                "launch_us_mean": cus,
                "layers_per_launch": group,
                "us_per_layer_steady": lus,
                "steady_frac": layer_bytes / (lus * 1e-6) / 1e9 /
                HBM_PEAK_GBPS,
                "chains_timed": reps * nd,
            }
            out["roofline_exact_pass"] = exact_pass
        else:
            out["roofline"] = exact_pass
        out["roofline"]["approx_tokens_per_head"] = a_tokens

    # ---- chained decode step with post-attention work -------------------
    if args.model_steps > 0:
        di4 = dens.index(4) if 4 in dens else 0
        out["model_step"] = model_timing(args, al, h, works[di4], Qs[di4],
                                         Ks[di4], Vs[di4], nl, dev)
        log("model step done")
        seq = res.get("sequential", {})
        if ("approx_latency_us_mean" in seq and
                "exact_only_baseline" in res):
            out["projection"] = projection(
                seq, res["exact_only_baseline"]["ms_per_step"] * 1e3 / nl,
                out["model_step"]["post_attention_roofline"]["us_per_layer"],
                hit_rate)

    # ---- CPU oracle baseline --------------------------------------------
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, works, dens, outs, nl, Qs,
                                           Ks, Vs)

    # ---- the other configurations (headline inputs freed first) ---------
    del graphs
    Ks.clear()
    Vs.clear()
    A.clear()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    which = [c for c in args.configs.split(",") if c and c != "none"]
    if which:
        out["configs"] = config_records(args, al, B_, h, dev, which)
        log("configurations done")

    # ---- HBM probe ------------------------------------------------------
    if not args.no_probe:
        torch.cuda.empty_cache()
        pr = sdev.probe_bandwidth()
        out["probe"] = {k: round(v["GBps"], 1) for k, v in pr.items()}
        out["probe"]["read_settings"] = {
            k: pr["read"][k] for k in ("blocks", "loads_in_flight",
                                       "nontemporal")}
        for key in ("roofline", "roofline_exact_pass"):
            if key in out:
                out[key]["frac_of_probe_read"] = (
                    out[key]["achieved"] / pr["read"]["GBps"])
        if "model_step" in out:
            out["model_step"]["post_attention_roofline"][
                "probe_at_size"] = post_probe_at_size(
                    out["model_step"]["post_attention_roofline"])
        log("probe done")

    print(json.dumps(out), flush=True)
    h.close()


def post_probe_at_size(roof):
    """The read probe at the byte count of each post-attention product (one
    launch per product, back to back over distinct slices), and the layer
    time those four probe launches take together: the ceiling that launch
    ramps and tails leave for four short HBM-bound launches."""
    from synth import device as sdev
    from synth import post_gen as pg
    ps = pg.llama8b(B=1)
    sh = ps.shapes()
    prod = {"o_proj": [sh["w_o"]], "gate_up": [sh["w_gate"], sh["w_up"]],
            "down": [sh["w_down"]], "next_qkv": [sh["w_qkv"]]}
    nbytes = {k: sum(r * c * 2 for r, c in v) for k, v in prod.items()}
    pr = sdev.probe_read_sizes(sorted(set(nbytes.values())))
    res = {}
    for k, nb in nbytes.items():
        r = pr[nb]
        res[k] = {"bytes": nb, "us": r["us"], "GBps": r["GBps"],
                  "settings": {x: r[x] for x in ("blocks", "loads_in_flight",
                                                 "nontemporal")}}
    probe_us = sum(r["us"] for r in res.values())
    res["layer_probe_us"] = probe_us
    res["layer_frac_of_probe"] = probe_us / roof["us_per_layer"]
    return res


def overhead_reduction(t_exact, t_approx, hit):
    """The pages' attention latency overhead reduction ("Attention-Level
    Speculation", atlas.scime.ai summary, Key results): attention costs
    t_exact per layer without speculation; with it, t_approx where the
    speculation commits (a fraction `hit` of the layers) and t_exact where
    it discards."""
    return t_exact / (hit * t_approx + (1.0 - hit) * t_exact)


# Link latencies swept by the projection (no second GPU here): a small
# point-to-point transfer (a commit flag or an 8-16 KiB output) and a small
# all-reduce of a tensor-parallel pair, both taken as one latency L.
LINK_US = (2.0, 5.0, 10.0, 20.0)


def project_layer(t_approx, t_exact, exact_only, post, hit, p2p, allreduce):
    """Per-layer latency of one decode token on two GPUs, projected from
    one GPU's measured durations, as the pages projected H100 ([A] Key
    results, Limitations: device durations, host and dispatch latency
    excluded):
      one_gpu  exact attention, then post-attention, in turn;
      alspec   the pages' placement ([A] Approach): GPU A runs exact
               attention and the verify, GPU B the approximation and the
               post-attention work on it.  A commit costs max(approx + post,
               exact to verified output + p2p); a discard costs exact + p2p
               + the replayed post-attention work; weighted by the hit rate;
      tp2      tensor parallel over two GPUs, no speculation: attention and
               post-attention each halved, plus two all-reduces (after the
               output projection and after the MLP)."""
    one = exact_only + post
    commit = max(t_approx + post, t_exact + p2p)
    discard = t_exact + p2p + post
    alspec = hit * commit + (1.0 - hit) * discard
    tp2 = (exact_only + post) / 2.0 + 2.0 * allreduce
    return {"one_gpu": one, "alspec_2gpu_commit": commit,
            "alspec_2gpu_discard": discard, "alspec_2gpu": alspec,
            "tp_2gpu": tp2}


def projection(seq, exact_only_us, post_us, hit):
    """project_layer over the swept link latencies, from this run's
    sequential-schedule latencies, exact-only attention and post-attention
    duration (MI355X, one GPU)."""
    t_a = seq["approx_latency_us_mean"]
    t_e = seq["exact_latency_us_mean"]
    sweep = []
    for L in LINK_US:
        u = project_layer(t_a, t_e, exact_only_us, post_us, hit, L, L)
        sweep.append({"link_us": L, "us_per_layer": u,
                      "speedup_vs_one_gpu": {
                          "alspec_2gpu": u["one_gpu"] / u["alspec_2gpu"],
                          "tp_2gpu": u["one_gpu"] / u["tp_2gpu"]}})
    return {
        "inputs_us": {"approximation": t_a,
                      "exact_to_verified_output": t_e,
                      "exact_only_attention": exact_only_us,
                      "post_attention": post_us},
        "hit_rate": hit,
        "link_sweep": sweep,
        "note": "a model, not a measurement: durations measured on one "
                "MI355X, the link latency swept (point-to-point and "
                "all-reduce both taken as it); the post-attention weights "
                "are random, the hit rate is this run's attention hit rate "
                "on the synthetic inputs",
    }


def config_records(args, al, B_, h, dev, which):
    """The other configurations as layer-pipelined chains
    (alspec_spec_decode_layers) in both its forms (one launch; one launch
    per layer), one configuration at a time, each drawn on the device and
    freed after: the chain's wall time per decode token (HIP events around
    back-to-back chains of all layers), its launch against the HBM roofline
    (as for the headline), and the hit rate; the faster form is the
    record's."""
    import torch

    from synth import device as sdev
    from synth import gen
    recs = {}
    for name in which:
        w = {"c2": gen.llama8b_32k, "c4": gen.multiuser_8b,
             "c5": gen.llama70b_128k}[name]()
        nl = w.n_layers
        t0 = time.time()
        K = torch.empty((nl, w.B, w.Hkv, w.L_cap, w.D), dtype=torch.bfloat16,
                        device=dev)
        V = torch.empty_like(K)
        Q = torch.empty((nl, w.B, w.Hq, w.D), dtype=torch.float32, device=dev)
        for layer in range(nl):
            sdev.fill_kv(w, layer, K[layer], V[layer])
            Q[layer].copy_(torch.from_numpy(gen.q_all(w, layer)))
        torch.cuda.synchronize()
        log(f"{name}: drew {nl} layers ({2 * K.numel() * 2 / 2**30:.1f} GiB) "
            f"t={time.time() - t0:.1f}s")
        layer_bytes = sum(w.seq_lens) * w.Hkv * w.D * 2 * 2
        s = torch.cuda.Stream(device=dev)
        forms = {}
        for form, overlap in (("one_launch", 0), ("per_layer_launch", 1)):
            p = al.params_for(w, overlap=overlap)
            wss = [al.alloc_workspace(p, dev)
                   for _ in range(min(nl, args.chain_ring))]
            outs = [al.alloc_outputs(p, dev) for _ in range(nl)]
            arr = B_.layers_struct(p, [(Q[l], K[l], V[l], outs[l],
                                        wss[l % len(wss)])
                                       for l in range(nl)])
            steady, launch_us, group, reps = chain_timing(args, B_, h, p,
                                                          [arr], s, nl)
            # whole chains, back to back
            e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            torch.cuda.synchronize()
            e0.record(s)
            for _ in range(reps):
                st = B_._spec_decode_layers(h.ptr, ctypes.byref(p), nl, arr,
                                            s.cuda_stream)
                if st != 0:
                    raise al.AlspecError(st, "alspec_spec_decode_layers")
            e1.record(s)
            torch.cuda.synchronize()
            chain_us = e0.elapsed_time(e1) * 1e3 / reps
            # the launch's bytes over its duration (one launch: the whole
            # chain; one launch per layer: a steady layer)
            achieved = layer_bytes * group / (launch_us * 1e-6) / 1e9
            kern = ("one_chain_kernel (the whole chain of "
                    f"{group} layers in one launch)" if group > 1 else
                    "chain_kernel (one launch per layer, steady state)")
            forms[form] = {
                "tokens_layers_per_s": w.B * nl / (chain_us * 1e-6),
                "us_per_layer": chain_us / nl,
                "chains_timed": reps,
                "roofline": {"bound": "hbm", "achieved": achieved,
                             "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": achieved / HBM_PEAK_GBPS,
                             "traffic": measured_traffic(
                                 f"{name}_{'one_chain' if group > 1 else 'chain'}"),
                             "kernel": kern,
                             "algorithmic_bytes_per_launch":
                                 layer_bytes * group,
                             "launch_us_mean": launch_us,
                             "layers_per_launch": group,
                             "us_per_layer_steady": steady,
                             "steady_frac": layer_bytes / (steady * 1e-6) /
                             1e9 / HBM_PEAK_GBPS},
                "ratio": torch.stack([o["ratio"] for o in outs]).cpu()
                .numpy(),
            }
            log(f"{name} {form}: {chain_us / nl:.1f} us per layer "
                f"({achieved / HBM_PEAK_GBPS:.3f} of peak per launch), "
                f"steady {steady:.1f} us per layer")
            del outs, wss, arr
        best = min(forms, key=lambda f: forms[f]["us_per_layer"])
        ratio = forms[best].pop("ratio")
        for f in forms.values():
            f.pop("ratio", None)
        lams = (0.05, 0.10, 0.20) if name == "c4" else (w.lam,)
        recs[name] = {
            "workload": f"{w.name}: batch {w.B}, {w.Hq} q / {w.Hkv} kv heads, "
                        f"head dim {w.D}, bf16 KV, context "
                        f"{min(w.seq_lens)}-{max(w.seq_lens)}, sink {w.S}, "
                        f"window {w.W}, {nl} layers",
            "schedule": f"layer_pipelined, {best} (alspec_spec_decode_layers,"
                        " eager, one call per decode token; the faster of "
                        "its two forms)",
            "workspaces": min(nl, args.chain_ring),
            "tokens_layers_per_s": forms[best]["tokens_layers_per_s"],
            "us_per_layer": forms[best]["us_per_layer"],
            "chains_timed": forms[best]["chains_timed"],
            "roofline": forms[best]["roofline"],
            "forms": forms,
            "hit_rate": {str(lam): float((ratio <= lam).mean())
                         for lam in lams},
        }
        del K, V, Q
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return recs


def B_params_seq(al, p):
    """p with the sequential overlap mode (the chained step's)."""
    q = type(p).from_buffer_copy(p)
    q.overlap = 0
    return q


def model_timing(args, al, h, w, Q, K, V, nl, dev):
    """One decode token through nl Llama-3-8B-shaped layers: the attention
    step on the resident 128K KV, then the post-attention operators with
    seeded random bf16 weights (o_proj, RMSNorm + gated MLP, down, RMSNorm
    + next QKV; 416 MiB per layer), layer l+1's query from layer l's QKV.

    The weights carry the structure that makes a trained model's queries
    find the sink (post_gen.plant_query_direction): the residual stream
    holds one dominant coordinate (post_gen.MASSIVE_DIM, MASSIVE_VALUE), so
    after the RMSNorm of the next QKV that coordinate is close to
    sqrt(hidden) whatever the rest holds; that norm's weight is 1 there,
    and the QKV weight's column there gives query
    head h of kv head g the entries a * u_g / sqrt(hidden), u_g being the
    planted direction of the next layer's KV cache (the generator's
    queries carry a * u_g in the same way).  The random rest of each query
    plays the part of the generator's query noise.  Without it the queries
    are unrelated to the planted sink and needles, and no layer commits.

    Timed by wall clock between synchronisations, in four forms:
      exact_only      exact attention, then post-attention on its output
      spec_sequence   attention step with verify, then post-attention on
                      the committed output, one stream
      spec_overlap    the same result with the post-attention work run on
                      o_approx beside the exact pass and replayed on o_exact
                      after a discard (runtime.model_step; eager: the two-
                      stream step cannot be captured, see the runtime
                      module)
      spec_one_stream_graph
                      the speculative work on o_approx before the exact
                      pass, on one stream, all layers captured as one HIP
                      graph
    The speculative forms at lambda 0.10 and, to bracket them, at +inf
    (every layer commits) and 0 (every layer discards).  Also the
    post-attention kernels alone against the HBM roofline (HIP events
    around back-to-back layers).
    """
    import torch

    from attention_level_speculation_amd import runtime as rt
    from synth import gen
    from synth import post_gen as pg
    ps = pg.llama8b(B=1)
    pp = al.make_post_params(1, ps.attn_dim, ps.hidden, ps.ffn, ps.qkv_dim,
                             ps.eps)
    gen_ = torch.Generator(device=dev)
    gen_.manual_seed(ps.seed)
    weights = []
    for layer in range(nl):
        d = {}
        for n_, shp in ps.shapes().items():
            if n_.startswith("norm"):
                t = 1.0 + 0.1 * torch.randn(shp, device=dev, generator=gen_)
            else:
                t = torch.randn(shp, device=dev, generator=gen_)
                t *= shp[1] ** -0.5
            d[n_] = t
        # query rows: the next layer's planted directions
        nxt = (layer + 1) % nl
        pg.plant_query_direction(
            d["w_qkv"], d["norm_attn"],
            [gen.head_plant(w, nxt, 0, g).u for g in range(w.Hkv)],
            w.const.a, w.D, w.G, ps.hidden)
        weights.append({n_: t.to(torch.bfloat16) for n_, t in d.items()})
    structs = [al.post_weights_struct(pp, d) for d in weights]
    f = dict(dtype=torch.float32, device=dev)
    hs = [torch.randn((1, ps.hidden), generator=gen_, **f)] + [
        torch.empty((1, ps.hidden), **f) for _ in range(nl)]
    hs[0][0, pg.MASSIVE_DIM] = pg.MASSIVE_VALUE
    qkvs = [torch.empty((1, ps.qkv_dim), **f) for _ in range(nl)]
    wsp = (al.alloc_post_workspace(pp, dev), al.alloc_post_workspace(pp, dev))
    sa, se = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    cur = torch.cuda.current_stream()
    res = {"workload": "llama3-8b-shaped decoder layers, batch 1: attention "
                       "over the 128K bf16 KV of one density (4 needles), "
                       "then post-attention with seeded random bf16 "
                       "weights whose next-QKV query rows point at the "
                       "next layer's planted sink direction through one "
                       "dominant residual coordinate", "layers": nl,
           "post_weight_bytes_per_layer": ps.weight_bytes(),
           "steps": args.model_steps}

    # post-attention kernels alone
    o_ = torch.randn((1, ps.attn_dim), generator=gen_, **f)
    for i in range(8):
        al.post_attention(h, pp, structs[i % nl], o_, hs[0], hs[1], qkvs[0],
                          wsp[1], stream=se)
    torch.cuda.synchronize()
    reps = max(1, args.kernel_launches // 4)
    e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
    e0.record(se)
    for i in range(reps):
        al.post_attention(h, pp, structs[i % nl], o_, hs[0], hs[1], qkvs[0],
                          wsp[1], stream=se)
    e1.record(se)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    gbps = ps.weight_bytes() / (us * 1e-6) / 1e9
    res["post_attention_roofline"] = {
        "bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS,
        "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
        "kernels": "gemv_residual (o_proj), gate_up, gemv_residual (down), "
                   "gemv_norm (next QKV), one layer",
        "algorithmic_bytes_per_layer": ps.weight_bytes(),
        "us_per_layer": us, "layers_timed": reps}

    def run(lam, graph=False, **kw):
        p = al.params_for(w, lam=lam)
        outs = [al.alloc_outputs(p, dev) for _ in range(nl)]
        layers = [rt.ModelLayer(K[l], V[l], structs[l], outs[l], hs[l],
                                hs[l + 1], qkvs[l]) for l in range(nl)]
        ws = al.alloc_workspace(p, dev)

        def issue():
            sa.wait_stream(cur)
            se.wait_stream(cur)
            rt.model_step(h, p, pp, Q[0], layers, ws, wsp[0], wsp[1], sa, se,
                          **kw)
            cur.wait_stream(sa)
            cur.wait_stream(se)
        step = issue
        if graph:
            # the one-stream form over all layers as one HIP graph
            issue()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=se):
                rt.model_step(h, p, pp, Q[0], layers, ws, wsp[0], wsp[1],
                              se, se, **kw)

            def step():
                se.wait_stream(cur)
                with torch.cuda.stream(se):
                    g.replay()
                cur.wait_stream(se)
        step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.model_steps):
            step()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / args.model_steps
        commits = [int(o["commit"][0].item()) for o in outs]
        return {"us_per_layer": wall * 1e6 / nl,
                "tokens_layers_per_s": nl / wall,
                "commit_rate": sum(commits) / nl}
    # the approximation against the exact pass inside the model step: the
    # one-stream speculative order (approximation, post-attention on it,
    # exact pass and merge, verify, post-attention replay where discarded),
    # HIP events around the approximation and around the exact pass of
    # every layer
    p = al.params_for(w)
    p0 = B_params_seq(al, p)
    outs = [al.alloc_outputs(p0, dev) for _ in range(nl)]
    ws = al.alloc_workspace(p0, dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
          for _ in range(nl)]
    t_a, t_e = [], []
    for it in range(1 + args.model_steps):
        torch.cuda.synchronize()
        q = Q[0]
        for l in range(nl):
            o = outs[l]
            ev[l][0].record(se)
            al.sink_approx(h, p0, q, K[l], V[l], o["o_approx"],
                           o["lse_approx"], ws, se)
            ev[l][1].record(se)
            al.post_attention(h, pp, structs[l], o["o_approx"].view(1, -1),
                              hs[l], hs[l + 1], qkvs[l], wsp[0], stream=se)
            ev[l][2].record(se)
            al.flash_decode_exact(h, p0, q, K[l], V[l], 0, ws, se)
            al.lse_combine(h, p0, ws, o["o_exact"], o["lse_exact"], se)
            ev[l][3].record(se)
            al.verify(h, p0, o["o_approx"], o["o_exact"], o["ratio"],
                      o["commit"], o["o_committed"], se)
            al.post_attention(h, pp, structs[l], o["o_exact"].view(1, -1),
                              hs[l], hs[l + 1], qkvs[l], wsp[1],
                              skip=o["commit"], stream=se)
            q = rt.q_view(p0, qkvs[l])
        torch.cuda.synchronize()
        if it:  # the first token warms up
            for l in range(nl):
                t_a.append(ev[l][0].elapsed_time(ev[l][1]) * 1e3)
                t_e.append(ev[l][2].elapsed_time(ev[l][3]) * 1e3)
    ta, te = sum(t_a) / len(t_a), sum(t_e) / len(t_e)
    res["attention_split"] = {
        "measure": "HIP events around the approximation call and around "
                   "the exact pass (split-K over the middle and merge) of "
                   "every layer, in the one-stream speculative order with "
                   "the post-attention work between them",
        "approx_us_mean": ta, "exact_us_mean": te,
        "approx_over_exact": ta / te, "layers_timed": len(t_a)}
    del outs, ws
    res["exact_only"] = run(w.lam, exact_only=True)
    res["exact_only"].pop("commit_rate")
    res["spec_sequence"] = run(w.lam, speculative=False)
    res["spec_overlap"] = run(w.lam, speculative=True)
    res["spec_overlap_all_commit"] = run(float("inf"), speculative=True)
    res["spec_overlap_all_discard"] = run(0.0, speculative=True)
    res["spec_one_stream_graph"] = run(w.lam, graph=True, speculative=True,
                                       one_stream=True)
    res["spec_one_stream_graph_all_commit"] = run(
        float("inf"), graph=True, speculative=True, one_stream=True)
    res["spec_one_stream_graph_all_discard"] = run(
        0.0, graph=True, speculative=True, one_stream=True)
    return res


def kernel_timing(args, al, B_, h, p, Qs, Ks, Vs, stream, nd, nl):
    """Average duration of the exact split-K kernel: back-to-back launches
    (alspec_flash_decode_exact over the middle splits) over every resident
    layer in turn, bracketed by two HIP events on the stream they run on;
    elapsed time / launches (so inter-launch gaps count against it)."""
    import torch
    ws = al.alloc_workspace(p)
    order = [(di, layer) for layer in range(nl) for di in range(nd)]
    args_ = [(h.ptr, ctypes.byref(p), Qs[di][layer].data_ptr(),
              Ks[di][layer].data_ptr(), Vs[di][layer].data_ptr(), 0,
              ws.data_ptr(), ws.numel(), stream.cuda_stream)
             for di, layer in order]
    fn = B_._flash_exact

    def run(n):
        for i in range(n):
            st = fn(*args_[i % len(args_)])
            if st != 0:
                raise al.AlspecError(st, "alspec_flash_decode_exact")
    torch.cuda.synchronize()
    run(16)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run(args.kernel_launches)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / args.kernel_launches


def chain_timing(args, B_, h, p, arrs, stream, nl):
    """Device time of the layer-pipelined chain: per call and per layer in
    its steady state.  alspec_spec_decode_layers runs back to back over all
    nl layers and, separately, over the first short_n, each bracketed by two
    HIP events on the stream it runs on; both calls hold the chain's first
    approximation and its last verify, so the difference of the two per-call
    times is nl - short_n steady layers (inter-launch gaps count against
    it).  In one launch (p.overlap 0) the per-call time is the launch's
    (with the small table writer before it) and short_n is nl / 2; in one
    launch per layer (p.overlap 1) short_n is 2 and the per-launch time is
    the per-layer one.  Returns (microseconds per steady layer,
    microseconds per launch, layers per launch, repetitions per density)."""
    import torch
    if nl < 3:
        raise SystemExit("the steady state needs at least 3 layers")
    short_n = nl // 2 if p.overlap == 0 else 2
    span = nl - short_n
    short = [(B_.Layer * short_n)(*a[:short_n]) for a in arrs]

    def run(layers, n, reps):
        for _ in range(reps):
            for arr in layers:
                st = B_._spec_decode_layers(h.ptr, ctypes.byref(p), n, arr,
                                            stream.cuda_stream)
                if st != 0:
                    raise RuntimeError(f"alspec_spec_decode_layers: {st}")
    reps = max(1, args.kernel_launches // (len(arrs) * nl))
    torch.cuda.synchronize()
    run(arrs, nl, 1)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record(stream)
    run(arrs, nl, reps)
    ev[1].record(stream)
    ev[2].record(stream)
    run(short, short_n, reps)
    ev[3].record(stream)
    torch.cuda.synchronize()
    n = reps * len(arrs)
    full = ev[0].elapsed_time(ev[1]) * 1e3 / n
    part = ev[2].elapsed_time(ev[3]) * 1e3 / n
    per_layer = (full - part) / span
    if p.overlap == 0:
        return per_layer, full, nl, reps
    return per_layer, per_layer, 1, reps


def cpu_baseline(args, works, dens, outs, nl, Qs, Ks, Vs):
    """The oracle as it stands, on all host cores, on a bounded sample of
    the same layers: whole layers, copied from the device-resident inputs
    (the generator's device twin, equal to its host definition)."""
    import numpy as np
    import torch

    import oracle
    threads = oracle.default_threads()
    secs = 0.0
    n = 0
    agree = 0
    order = [(di, layer) for layer in range(nl) for di in range(len(dens))]
    for di, layer in order:
        w = works[di]
        q = Qs[di][layer].cpu().numpy()
        k = Ks[di][layer].view(torch.int16).cpu().numpy().view(np.uint16)
        v = Vs[di][layer].view(torch.int16).cpu().numpy().view(np.uint16)
        t = time.perf_counter()
        r = oracle.spec_decode(q, k, v, w.seq_lens, w.S, w.W, w.lam,
                               threads=threads)
        secs += time.perf_counter() - t
        n += 1
        g = int(outs[di][layer]["commit"][0].item())
        agree += int(g == int(r["commit"][0]) or
                     abs(r["ratio"][0] - w.lam) <= 1e-4)
        if secs >= args.cpu_seconds:
            break
    # the same oracle on one core, one layer
    di, layer = order[0]
    w = works[di]
    q = Qs[di][layer].cpu().numpy()
    k = Ks[di][layer].view(torch.int16).cpu().numpy().view(np.uint16)
    v = Vs[di][layer].view(torch.int16).cpu().numpy().view(np.uint16)
    t = time.perf_counter()
    oracle.spec_decode(q, k, v, w.seq_lens, w.S, w.W, w.lam, threads=1)
    one = time.perf_counter() - t
    return {"value": n * works[0].B / secs, "unit": "tokens·layers/s",
            "one_core_value": works[0].B / one,
            "cores": threads, "kind": "oracle",
            "sample": f"{n} of the {len(dens) * nl} (needles, layer) pairs "
                      "of the same workload: whole layers (32 heads, context "
                      "131072), double precision, about "
                      f"{args.cpu_seconds:.0f} s of oracle time",
            "seconds": secs, "sample_flags_agree": f"{agree}/{n}",
            "cpu_model": _cpu_model()}


def _library_record(path):
    """The HIP library this run loaded: its path (relative to the
    repository when inside it) and the first 16 hex digits of its
    sha256."""
    import hashlib
    with open(path, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()[:16]
    rel = os.path.relpath(os.path.realpath(path), os.path.realpath(ROOT))
    return {"path": path if rel.startswith("..") else rel,
            "sha256_16": digest}


def _cpu_model():
    """The host CPU's model name, as the kernel reports it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
