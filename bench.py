#!/usr/bin/env python3
"""Benchmark of the MI355X MoE layer on one GPU.

A step is one forward of the layer at 2,048 pre-routing tokens per GPU
(dzen.guru page, "Что показали замеры?": 2,048 tokens before routing on each
GPU) with DeepSeek-V3-like expert shapes: d = 7168, E = 256, top-8, f = 2048,
bf16, ring capacity 1.25 x the copies.  The step runs the whole forward path:
router, counting-sort dispatch into the ring, gate/up + SwiGLU grouped GEMM,
down grouped GEMM, gate-weighted combine.  Inputs are synthetic and resident
in HBM before timing starts.

Prints ONE JSON line.  `roofline` is for the dominant kernel (the gate/up +
SwiGLU grouped GEMM), from HIP events recorded around it on the launch stream
in every timed step.  `cpu_baseline` times the fp64 oracle on the host on a
bounded sample of the same workload.  `secondary` carries the small-batch
decode (us/token, HBM fraction), the grouped GEMMs at one GPU's
expert-parallel share (MFMA fraction), and the MXFP8 forward.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-secondary]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Host threads of the oracle baseline: the CPUs this process may run on, capped by the
# OpenMP thread count the machine sets for a process's share.  The BLAS pools read these
# variables when numpy is first imported, so they are pinned here, before any import.
AFFINITY_CPUS = len(os.sched_getaffinity(0))
CPU_THREADS = min(AFFINITY_CPUS, int(os.environ.get("OMP_NUM_THREADS") or AFFINITY_CPUS))
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ[_v] = str(CPU_THREADS)

METRIC = "MoE-layer tokens/s at 2048 tok; decode µs/token; % of MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFS = 2516.6
FP8_PEAK_TFS = 5033.2


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle expert work in the CPU baseline sample")
    ap.add_argument("--only", choices=["decode", "share", "skew", "skew-no-stack", "skew-mx", "mxfp8"],
                    default=None,
                    help="run one secondary workload alone (e.g. under a profiler) and print its JSON")
    ap.add_argument("--no-fused", action="store_true",
                    help="leave out the single-launch forward (a cooperative launch, which "
                         "rocprofv3 does not survive at exit)")
    ap.add_argument("--decode-batch", type=int, choices=[1, 4, 8], default=None,
                    help="with --only decode: this batch size alone")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (reference for counter scaling)")
    return ap.parse_args()


def progress(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gemm_source_hash() -> str:
    """Hash of the grouped GEMM's sources (the counters are void once they change)."""
    h = hashlib.sha256()
    for name in ("gemm.hip", "gemm_body.h", "common.h"):
        with open(os.path.join(ROOT, "mixture_experts_layer_33_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, per_launch_alg_bytes: float):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        with open(path) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = data.get(kernel)
    if not ent or ent.get("gemm_hip_sha256_16") != gemm_source_hash():
        return None
    return ent.get("bytes_per_launch")


def fwd_step_timed(layer, inp, events):
    layer.forward(inp.x, inp.w_router, inp.b_router, inp.w_gate, inp.w_up, inp.w_down,
                  events=events)


REPEAT_BUFFERS = ("topk_idx", "topk_gate", "expert_count", "expert_offset", "copy_slot", "slot_copy",
                  "ring_x", "ring_y", "y")


def measure_forward(torch, moe, inp, cfg, steps, warmup, scales=(None, None, None), wq=None):
    """Time `steps` forwards back to back; returns (ms/step, avg GEMM-1 ms, avg GEMM-2 ms,
    layer, spread) with spread = per-step median / min / p90 (from an event at every step
    boundary) and whether every output and ring buffer of the last timed step is bitwise
    equal to the first warm-up step's."""
    layer = moe.Layer.create(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.C, dtype=cfg.dtype)
    wg, wu, wd = wq if wq is not None else (inp.w_gate, inp.w_up, inp.w_down)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    first = None
    for i in range(max(1, warmup)):
        layer.forward(inp.x, inp.w_router, inp.b_router, wg, wu, wd, scales=scales)
        if i == 0:
            first = {n: layer.bufs[n].clone() for n in REPEAT_BUFFERS if n in layer.bufs}
    torch.cuda.synchronize()
    marks[0].record()
    for i in range(steps):
        layer.forward(inp.x, inp.w_router, inp.b_router, wg, wu, wd, scales=scales, events=evs[i])
        marks[i + 1].record()
    torch.cuda.synchronize()
    ms = marks[0].elapsed_time(marks[steps]) / steps
    per = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    g1 = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    g2 = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    same = all(torch.equal(first[n].view(torch.uint8), layer.bufs[n].view(torch.uint8)) for n in first)
    spread = {"step_ms_median": round(per[len(per) // 2], 4), "step_ms_min": round(per[0], 4),
              "step_ms_p90": round(per[int(0.9 * (len(per) - 1))], 4),
              "repeat_bitwise_equal": bool(same), "repeat_buffers": sorted(first)}
    return ms, g1, g2, layer, spread


def measure_fused(torch, moe, inp, cfg, steps, warmup, chained):
    """The same forward as one kernel launch (moe_forward): ms per step back to back, the
    per-step spread, and whether every output and ring buffer equals the chained calls'
    bit for bit (`chained`: the Layer of the timed chained forward)."""
    layer = moe.Layer.create(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.C, dtype=cfg.dtype)
    args = (inp.x, inp.w_router, inp.b_router, inp.w_gate, inp.w_up, inp.w_down)
    for _ in range(max(1, warmup)):
        layer.forward_fused(*args)
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record()
    for i in range(steps):
        layer.forward_fused(*args)
        marks[i + 1].record()
    torch.cuda.synchronize()
    ms = marks[0].elapsed_time(marks[steps]) / steps
    per = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    same = all(torch.equal(layer.bufs[n].view(torch.uint8), chained.bufs[n].view(torch.uint8))
               for n in ("topk_idx", "topk_gate", "expert_count", "expert_offset", "copy_slot", "y"))
    return {"launches_per_step": 1, "ms_per_step": round(ms, 4), "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
            "step_ms_median": round(per[len(per) // 2], 4), "step_ms_min": round(per[0], 4),
            "step_ms_p90": round(per[int(0.9 * (len(per) - 1))], 4),
            "barrier_status": layer.forward_status(), "bitwise_equal_to_chained": bool(same)}


def expert_bytes(counts, d, f, elem_bytes, scale_bytes_per_elem=0.0):
    used = int((counts > 0).sum())
    per = d * f * (elem_bytes + scale_bytes_per_elem)
    return used, used * 2 * per, used * per


def cpu_baseline(inp, cfg, budget_s):
    """The oracle on the host over the whole layer: router, dispatch, ring fill, the expert
    FFN of every expert (ascending id) and combine.  Each step is repeated `reps` times so
    that about `budget_s` seconds of oracle work are timed, reps sized from an untimed
    warm-up and a timed probe of the first expert; an expert's weights are widened to
    fp64 once, outside the timed regions.  If one layer alone would exceed the budget, its
    experts are sampled in ascending id until the budget and the expert time is
    extrapolated by the sampled share of token copies.  BLAS runs on CPU_THREADS threads,
    pinned before numpy was imported."""
    import numpy as np
    import oracle
    from gen import bits16
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threadpool_limits(CPU_THREADS)
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = CPU_THREADS
    x = oracle.from_bf16_bits(bits16(inp.x))
    w_r = oracle.from_f32(inp.w_router.cpu().numpy())
    t0 = time.perf_counter()
    r = oracle.route(x, w_r, None, cfg.k)
    disp = oracle.dispatch(r.idx, cfg.E, cfg.C, 0)
    ring = oracle.ring_fill(x, disp)
    t_fixed1 = time.perf_counter() - t0
    ring_y = np.zeros((cfg.C, cfg.d))
    t_exp, rows, sampled, reps = 0.0, 0, 0, None
    for e in range(cfg.E):
        slots = oracle.segment_slots(disp, e)
        if slots.size == 0:
            continue
        w = tuple(oracle.from_bf16_bits(bits16(t[e])) for t in (inp.w_gate, inp.w_up, inp.w_down))
        if reps is None:   # size the repetition count from the first expert's cost
            oracle.swiglu(ring[slots], *w)                       # warm-up: thread pools, caches
            t1 = time.perf_counter()
            oracle.swiglu(ring[slots], *w)
            probe = (time.perf_counter() - t1) * cfg.n / slots.size + 2 * t_fixed1
            reps = int(max(1, min(50, math.ceil(budget_s / max(probe, 1e-9)))))
        if sampled % 32 == 0:
            progress(f"oracle expert {e}: {t_exp:.1f} s of expert work so far ({reps} reps)")
        t1 = time.perf_counter()
        for _ in range(reps):
            ring_y[slots] = oracle.swiglu(ring[slots], *w)
        t_exp += time.perf_counter() - t1
        rows += slots.size
        sampled += 1
        if t_exp >= budget_s and rows < cfg.n:
            break
    reps = reps or 1
    t2 = time.perf_counter()
    for i in range(reps):
        if i:   # the router, dispatch and ring fill again, once per extra repetition
            r = oracle.route(x, w_r, None, cfg.k)
            disp = oracle.dispatch(r.idx, cfg.E, cfg.C, 0)
            ring = oracle.ring_fill(x, disp)
        oracle.combine(ring_y, disp.copy_slot, r.gate)
    t_fixed = t_fixed1 + time.perf_counter() - t2
    est = t_fixed + t_exp * (cfg.n / rows)
    return {"value": round(reps * cfg.T / est, 3), "unit": "tokens/s", "cores": threads,
            "affinity_cpus": AFFINITY_CPUS, "kind": "oracle",
            "sample": (f"fp64 numpy oracle on {threads} BLAS threads, {reps} repetition(s) of each "
                       f"step: router, dispatch, ring fill and combine over all {cfg.T} tokens "
                       f"({t_fixed:.2f} s); expert SwiGLU on {sampled} of {cfg.E} experts ({rows} of "
                       f"{cfg.n} copies, {t_exp:.2f} s); {reps} full layer(s) "
                       + ("timed" if rows == cfg.n else "extrapolated by the copy share")
                       + f" in {est:.1f} s")}


def skew_fwd_bwd(torch, moe, steps, stack=True):
    """Forward (saving A|U) and backward of the skewed workload, timed separately.
    Algorithmic bytes: forward = used experts' three matrices + W_r (fp32) + x read twice
    (router, dispatch) + ring written and read + H written and read + saved A|U written +
    ring_y written and read + y written; backward = used experts' three matrices read +
    all three weight gradients written (every expert, zeros included) + dW_r (fp32) +
    dy, x, ring rows, saved A|U read + dx written."""
    import numpy as np
    from gen import SKEW_BWD, make_layer
    cfg = SKEW_BWD
    progress(f"skewed forward + backward {cfg.name}")
    inp = make_layer(cfg, "cuda")
    layer = moe.Layer.create(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.C)
    args = (inp.x, inp.w_router, inp.b_router, inp.w_gate, inp.w_up, inp.w_down)
    for _ in range(2):
        layer.forward(*args, save_au=True)
        layer.backward(inp.dy, inp.x, inp.w_router, inp.w_gate, inp.w_up, inp.w_down)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        layer.forward(*args, save_au=True)
        ev[i][1].record()
        layer.backward(inp.dy, inp.x, inp.w_router, inp.w_gate, inp.w_up, inp.w_down)
        ev[i][2].record()
    torch.cuda.synchronize()
    fwd = [e[0].elapsed_time(e[1]) for e in ev]
    bwd = [e[1].elapsed_time(e[2]) for e in ev]
    counts = layer.bufs["expert_count"].cpu().numpy()
    used = int((counts > 0).sum())
    T, d, E, k, f = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f
    n = T * k
    w_used = used * 3 * f * d * 2
    fwd_bytes = (w_used + E * d * 4 + 2 * T * d * 2 + 2 * n * d * 2 + 2 * n * f * 2 + n * 2 * f * 2
                 + 2 * n * d * 2 + T * d * 2)
    bwd_bytes = (w_used + E * 3 * f * d * 2 + E * d * 4 + 2 * T * d * 2 + n * d * 2
                 + n * 2 * f * 2 + T * d * 2)
    fwd_flops = 2.0 * n * d * 3 * f + 2.0 * T * E * d
    bwd_flops = 2 * 2.0 * n * d * 3 * f + 2 * 2.0 * n * d
    fm, bm = float(np.median(fwd)), float(np.median(bwd))
    return {"tokens": T, "fwd_ms_median": round(fm, 4), "fwd_ms_min": round(min(fwd), 4),
            "bwd_ms_median": round(bm, 4), "bwd_ms_min": round(min(bwd), 4),
            "tokens_per_s_fwd_bwd": round(T / ((fm + bm) * 1e-3), 1),
            "fwd_alg_bytes": fwd_bytes, "fwd_hbm_frac": round(fwd_bytes / (fm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "fwd_mfma_frac": round(fwd_flops / (fm * 1e-3) / 1e12 / BF16_PEAK_TFS, 4),
            "bwd_alg_bytes": bwd_bytes, "bwd_hbm_frac": round(bwd_bytes / (bm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bwd_mfma_frac": round(bwd_flops / (bm * 1e-3) / 1e12 / BF16_PEAK_TFS, 4),
            "experts_used": used, "max_load": int(counts.max()), "mean_load": round(float(n / E), 2),
            "max_over_mean": round(float(counts.max() / (n / E)), 2),
            **({"ring_stack": ring_stack(torch, moe, inp, layer, steps, fm, bm)} if stack else {})}


def skew_fwd_bwd_mx(torch, moe, steps):
    """The skewed workload in MXFP8: forward (saving A|U) and moe_backward_mx, timed apart;
    the per-step weight quantisation (forward weights along K, backward weights transposed)
    timed on its own, in one pass per weight (moe_quantize_mx_both; its bytes: every bf16
    weight read once, both MX layouts written) and, for comparison, as the two separate
    quantisers.  Algorithmic bytes: forward = used experts' MX weights (codes + one
    scale byte per 32) + W_r + x twice + ring (MX) written and read + H (MX) written and read
    + saved A|U written + ring_y written and read + y; backward = used experts' transposed
    MX weights + all three weight gradients written (bf16, every expert) + dW_r + dy and x
    read + saved A|U read + dx."""
    import numpy as np
    from gen import SKEW_BWD, make_layer
    cfg = SKEW_BWD.with_(name="skew_bwd_mx_t8192", dtype="mxfp8")
    progress(f"skewed MXFP8 forward + backward {cfg.name}")
    inp = make_layer(cfg, "cuda")
    q = [moe.quantize_mx(w) for w in (inp.w_gate, inp.w_up, inp.w_down)]
    wq, scales = tuple(c for c, _ in q), tuple(s for _, s in q)
    bw = moe.quantize_mx_t_backward_weights(inp.w_gate, inp.w_up, inp.w_down)
    layer = moe.Layer.create(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.C, dtype="mxfp8")
    fargs = (inp.x, inp.w_router, inp.b_router, *wq)
    for _ in range(2):
        layer.forward(*fargs, scales=scales, save_au=True)
        layer.backward_mx(inp.dy, inp.x, inp.w_router, *bw)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        layer.forward(*fargs, scales=scales, save_au=True)
        ev[i][1].record()
        layer.backward_mx(inp.dy, inp.x, inp.w_router, *bw)
        ev[i][2].record()
        moe.quantize_mx_training_weights(inp.w_gate, inp.w_up, inp.w_down)
        ev[i][3].record()
        for w, c, s in zip((inp.w_gate, inp.w_up, inp.w_down), wq, scales):
            moe.moe_quantize_mx(w, c, s)
        moe.quantize_mx_t_backward_weights(inp.w_gate, inp.w_up, inp.w_down)
        ev[i][4].record()
    torch.cuda.synchronize()
    fwd = [e[0].elapsed_time(e[1]) for e in ev]
    bwd = [e[1].elapsed_time(e[2]) for e in ev]
    wqt = [e[2].elapsed_time(e[3]) for e in ev]
    wqs = [e[3].elapsed_time(e[4]) for e in ev]
    counts = layer.bufs["expert_count"].cpu().numpy()
    used = int((counts > 0).sum())
    T, d, E, k, f = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f
    n = T * k
    mxb = 1 + 1 / 32
    w_used = used * 3 * f * d * mxb
    fwd_bytes = (w_used + E * d * 4 + 2 * T * d * 2 + 2 * n * d * mxb + 2 * n * f * mxb
                 + n * 2 * f * 2 + 2 * n * d * 2 + T * d * 2)
    bwd_bytes = (w_used + E * 3 * f * d * 2 + E * d * 4 + 2 * T * d * 2 + n * 2 * f * 2 + T * d * 2)
    fm, bm = float(np.median(fwd)), float(np.median(bwd))
    qm = float(np.median(wqt))
    q_bytes = 3 * E * f * d * (2 + 2 * mxb)
    return {"tokens": T, "fwd_ms_median": round(fm, 4), "fwd_ms_min": round(min(fwd), 4),
            "bwd_ms_median": round(bm, 4), "bwd_ms_min": round(min(bwd), 4),
            "weight_quant_ms_median": round(qm, 4),
            "weight_quant_hbm_frac": round(q_bytes / (qm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "weight_quant_separate_ms_median": round(float(np.median(wqs)), 4),
            "training_step_ms": round(fm + bm + qm, 4),
            "tokens_per_s_fwd_bwd": round(T / ((fm + bm) * 1e-3), 1),
            "fwd_alg_bytes": fwd_bytes, "fwd_hbm_frac": round(fwd_bytes / (fm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bwd_alg_bytes": bwd_bytes, "bwd_hbm_frac": round(bwd_bytes / (bm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "experts_used": used, "max_load": int(counts.max()),
            "max_over_mean": round(float(counts.max() / (n / E)), 2)}


def ring_stack(torch, moe, inp, layer, steps, fwd_ms_1, bwd_ms_1, L=4):
    """L layers of the skewed shape sharing one ring (the same weights in every layer): the
    forwards advance the head, the backward consumes the layers last first with nothing
    recomputed.  Reported next to the single-layer figures: per-layer time should match."""
    import numpy as np
    s1 = layer.shape
    progress(f"ring stack: {L} layers sharing one ring")
    st = moe.RingStack(L, s1.tokens, s1.hidden, s1.experts, s1.top_k, s1.ffn)
    w = [(inp.w_router, inp.b_router, inp.w_gate, inp.w_up, inp.w_down)] * L
    dw = (layer.bufs["dw_gate"], layer.bufs["dw_up"], layer.bufs["dw_down"], layer.bufs["dw_router"])
    for _ in range(2):
        st.forward(inp.x, w)
        st.backward(inp.dy, w, dw=dw)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        st.forward(inp.x, w)
        ev[i][1].record()
        st.backward(inp.dy, w, dw=dw)
        ev[i][2].record()
    torch.cuda.synchronize()
    fm = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    bm = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
    C = st.shape.capacity
    resident = C * (s1.hidden * 2 + 2 * s1.ffn * 2 + 4)   # ring rows, saved [A|U], slot map
    out = {"layers": L, "ring_rows": C, "ring_resident_bytes": resident,
           "fwd_ms_median": round(fm, 4), "bwd_ms_median": round(bm, 4),
           "fwd_ms_per_layer": round(fm / L, 4), "bwd_ms_per_layer": round(bm / L, 4),
           "fwd_per_layer_over_single": round(fm / L / fwd_ms_1, 3),
           "bwd_per_layer_over_single": round(bm / L / bwd_ms_1, 3),
           "tokens_per_s_fwd_bwd": round(s1.tokens / ((fm + bm) * 1e-3), 1)}
    del st
    torch.cuda.empty_cache()
    return out


def part_decode(torch, moe, steps, batches=(1, 4, 8)):
    """Small-batch decode, output-parallel, B = 1, 4, 8."""
    import numpy as np
    from gen import DECODE, make_layer
    dec, prev = {}, None
    for B in batches:
        cfg = DECODE(B)
        progress(f"decode B={B}")
        inp = make_layer(cfg, "cuda", reuse=prev)
        prev = inp
        layer = moe.Layer.create(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, fs=cfg.fs)
        args = (inp.x, inp.w_router, inp.b_router, inp.w_gate, inp.w_up, inp.w_down,
                inp.ws_gate, inp.ws_up, inp.ws_down)
        for _ in range(3):
            layer.decode(*args)
        torch.cuda.synchronize()
        # a decode call is short: time many back-to-back calls (about 0.1-0.5 s)
        calls = max(100, 10 * steps)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(calls):
            layer.decode(*args)
        e.record()
        torch.cuda.synchronize()
        us = s.elapsed_time(e) * 1e3 / calls
        # cold: each call timed alone after a 1 GiB fill that evicts the 256 MB Infinity
        # Cache (the fill is outside the events)
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        cold = []
        for _ in range(20):
            flush.zero_()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            layer.decode(*args)
            c1.record()
            torch.cuda.synchronize()
            cold.append(c0.elapsed_time(c1) * 1e3)
        del flush
        cold.sort()
        U = int(np.unique(layer.bufs["topk_idx"].cpu().numpy()).size)
        nbytes = (U + 1) * 3 * cfg.f * cfg.d * 2 + cfg.E * cfg.d * 4 + 2 * B * cfg.d * 2
        dec[f"B{B}"] = {"calls": calls, "us_per_call": round(us, 2), "us_per_token": round(us / B, 2),
                        "cold_us_median": round(cold[len(cold) // 2], 2), "cold_us_min": round(cold[0], 2),
                        "cold_us_p90": round(cold[int(0.9 * (len(cold) - 1))], 2),
                        "unique_experts": U, "alg_bytes": nbytes,
                        "GBps": round(nbytes / us / 1e3, 1),
                        "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
    del prev, inp, layer
    torch.cuda.empty_cache()
    return dec


def part_share(torch, moe, steps):
    """One GPU's expert-parallel share: the grouped GEMMs alone, MFMA-bound."""
    import numpy as np
    from gen import SHARE_BF16, SHARE_MXFP8, make_share
    out = {}
    for scfg, peak in ((SHARE_BF16, BF16_PEAK_TFS), (SHARE_MXFP8, FP8_PEAK_TFS)):
        progress(f"expert-parallel share {scfg.name}")
        sh = make_share(scfg, "cuda")
        mx = scfg.dtype == "mxfp8"
        shape = moe.make_shape(scfg.rows, scfg.d, scfg.E, 1, scfg.f, scfg.C, dtype=scfg.dtype)
        off = torch.tensor(np.concatenate([[0], np.cumsum(sh.counts)]), dtype=torch.int32, device="cuda")
        ws = moe.workspace(shape, moe.OP_EXPERT_FFN, "cuda")
        ring_y = torch.empty((scfg.C, scfg.d), dtype=torch.bfloat16, device="cuda")
        if mx:
            xq, xs = moe.quantize_mx(sh.ring_x)
            q = [moe.quantize_mx(w) for w in (sh.w_gate, sh.w_up, sh.w_down)]
            wargs = [c for c, _ in q] + [s for _, s in q]
        else:
            xq, xs = sh.ring_x, None
            wargs = [sh.w_gate, sh.w_up, sh.w_down, None, None, None]
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for i in range(3 + steps):
            ev = evs[i - 3] if i >= 3 else [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            moe.moe_expert_ffn_timed(shape, xq, xs, off, 0, *wargs, ring_y, None, ws, ev)
        torch.cuda.synchronize()
        g1 = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
        g2 = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
        f1 = 2.0 * scfg.rows * scfg.d * 2 * scfg.f
        f2 = 2.0 * scfg.rows * scfg.f * scfg.d
        out[scfg.name] = {"rows": scfg.rows, "experts": scfg.E, "gemm1_ms": round(g1, 4),
                          "gemm2_ms": round(g2, 4), "ffn_ms": round(g1 + g2, 4),
                          "TFLOPs": round((f1 + f2) / (g1 + g2) / 1e9, 1),
                          "mfma_frac": round((f1 + f2) / (g1 + g2) / 1e9 / peak, 4),
                          "gemm1_mfma_frac": round(f1 / g1 / 1e9 / peak, 4),
                          "gemm2_mfma_frac": round(f2 / g2 / 1e9 / peak, 4)}
        del sh, ws, ring_y, xq, xs, wargs
        torch.cuda.empty_cache()
    return out


def part_mxfp8(torch, moe, steps):
    """The MXFP8 forward at the 2,048-token shape."""
    from gen import FWD_MXFP8, make_layer
    cfg = FWD_MXFP8
    progress(f"forward {cfg.name}")
    inp = make_layer(cfg, "cuda")
    q = [moe.quantize_mx(w) for w in (inp.w_gate, inp.w_up, inp.w_down)]
    ms, g1, g2, layer, spread = measure_forward(torch, moe, inp, cfg, steps, 3,
                                                scales=tuple(s for _, s in q), wq=tuple(c for c, _ in q))
    # algorithmic bytes: E4M3 codes plus one E8M0 byte per 32 of every MX operand read once
    counts = layer.bufs["expert_count"].cpu().numpy()
    used = int((counts > 0).sum())
    n, d, f = cfg.n, cfg.d, cfg.f
    mxb = 1 + 1 / 32
    alg1 = used * 2 * f * d * mxb + n * d * mxb + n * f * mxb       # weights + ring rows + H
    alg2 = used * d * f * mxb + n * f * mxb + n * d * 2              # weights + H + ring_y bf16
    return {"tokens_per_s": round(cfg.T / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
                              "gemm1_ms": round(g1, 4), "gemm2_ms": round(g2, 4),
                              "gemm1_alg_bytes": alg1, "gemm2_alg_bytes": alg2,
                              "gemm1_hbm_frac": round(alg1 / (g1 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "gemm2_hbm_frac": round(alg2 / (g2 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "gemm_hbm_frac": round((alg1 + alg2) / ((g1 + g2) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "gemm_fp8_mfma_frac": round(2.0 * n * d * 3 * f / ((g1 + g2) * 1e-3) / 1e12 / FP8_PEAK_TFS, 4),
                              **spread}


def secondary(torch, moe, steps):
    out = {"decode": part_decode(torch, moe, steps)}
    out.update(part_share(torch, moe, steps))
    out["skew_fwd_bwd_t8192"] = skew_fwd_bwd(torch, moe, steps)
    torch.cuda.empty_cache()
    out["skew_fwd_bwd_mx_t8192"] = skew_fwd_bwd_mx(torch, moe, steps)
    torch.cuda.empty_cache()
    out["fwd_mxfp8_t2048"] = part_mxfp8(torch, moe, steps)
    return out


def calibrate_copy(torch, args):
    """A plain 1 GiB device-to-device copy: the reference for scaling the HBM counters."""
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU; the layer has no multi-GPU path "
              "(no collectives, no sharding), so --gpus must be 1.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import mixture_experts_layer_33_amd as moe
    from gen import FWD_BF16, make_layer

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.only:
        calibrate_copy(torch, args)
        steps = max(2, args.steps)
        if args.only == "decode":
            res = part_decode(torch, moe, steps,
                              (args.decode_batch,) if args.decode_batch else (1, 4, 8))
        elif args.only == "share":
            res = part_share(torch, moe, steps)
        elif args.only == "skew-mx":
            res = skew_fwd_bwd_mx(torch, moe, steps)
        elif args.only in ("skew", "skew-no-stack"):
            res = skew_fwd_bwd(torch, moe, steps, stack=args.only == "skew")
        else:
            res = part_mxfp8(torch, moe, steps)
        print(json.dumps({"only": args.only, "steps": steps, **res}), flush=True)
        return
    cfg = FWD_BF16
    progress(f"drawing inputs of {cfg.name}")
    inp = make_layer(cfg, "cuda")
    torch.cuda.synchronize()
    progress(f"timing {args.steps} steps after {args.warmup} warm-up steps")
    t0 = time.perf_counter()
    ms, g1, g2, layer, spread = measure_forward(torch, moe, inp, cfg, args.steps, args.warmup)
    wall = time.perf_counter() - t0
    counts = layer.bufs["expert_count"].cpu().numpy()
    used, w_gu, w_d = expert_bytes(counts, cfg.d, cfg.f, 2)
    n = cfg.n
    alg1 = w_gu + n * cfg.d * 2 + n * cfg.f * 2           # weights + ring rows + H
    alg2 = w_d + n * cfg.f * 2 + n * cfg.d * 2            # weights + H + ring_y
    flops1 = 2.0 * n * cfg.d * 2 * cfg.f
    flops2 = 2.0 * n * cfg.f * cfg.d
    ach1 = alg1 / (g1 * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(cfg.T / (ms * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.d, "experts": cfg.E,
                   "top_k": cfg.k, "ffn": cfg.f, "capacity": cfg.C, "ring_head": 0,
                   "step": "route+dispatch+gate/up GEMM+down GEMM+combine"},
        "roofline": {"kernel": "gg_mfma_kernel<128,256,2,4,SWIGLU,bf16> (gate/up + SwiGLU)",
                     "bound": "hbm", "achieved": round(ach1, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach1 / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("gemm1_swiglu_bf16", alg1),
                     "alg_bytes_per_launch": alg1, "avg_launch_ms": round(g1, 4),
                     "mfma_TFLOPs": round(flops1 / (g1 * 1e-3) / 1e12, 1),
                     "mfma_frac": round(flops1 / (g1 * 1e-3) / 1e12 / BF16_PEAK_TFS, 4)},
        "kernels": {"gemm2_down": {"avg_launch_ms": round(g2, 4), "alg_bytes_per_launch": alg2,
                                   "GBps": round(alg2 / (g2 * 1e-3) / 1e9, 1),
                                   "hbm_frac": round(alg2 / (g2 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                   "mfma_frac": round(flops2 / (g2 * 1e-3) / 1e12 / BF16_PEAK_TFS, 4)},
                    "experts_used": used,
                    "layer_hbm_frac": round((alg1 + alg2) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "timed_wall_s": round(wall, 3),
    }
    result.update(spread)
    if not args.no_fused:
        progress("single-launch forward (moe_forward)")
        result["fused_forward"] = measure_fused(torch, moe, inp, cfg, args.steps, args.warmup, layer)
    progress(f"forward {ms:.3f} ms/step, gate/up GEMM {g1:.3f} ms, down GEMM {g2:.3f} ms")
    calibrate_copy(torch, args)
    if not args.no_secondary:
        result["secondary"] = secondary(torch, moe, max(5, args.steps // 2))
    if not args.no_cpu_baseline:
        progress("timing the fp64 oracle on the host (bounded sample)")
        result["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
