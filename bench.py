"""Throughput of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

A step is one moe_layer_forward call (gate, top-k + softmax, dispatch,
grouped FFN, weighted combine, counts and balance loss) over
one batch of seeded synthetic inputs already resident in HBM.  W untimed
steps, then K timed steps between two device synchronisations on the
stream the library launches on; per-stage durations come from HIP events
the library records around each of its launches inside that same timed
region.  Prints one JSON line.

The default workload is the E=64, top-2, d=2048 layer (T=8192, d_ff=8192,
capacity factor 2, Zipf-skewed gate); `value` is its tokens/s.  The oracle
(CPU) is timed beside it on the same workload (the whole batch when it fits
the time budget).  Unless --only is given, every other workload (the tiny
fp32 layer, the 16-, 128- and 256-expert layers and the literal-Zipf reading
of the headline) is then timed the same way with shorter runs and reported
under "configs": ms/step, tokens/s, the grouped GEMMs' rate, the dominant
launch against its roofline and the routing / permutation / combine launches
against HBM.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd tokens/sec + grouped-GEMM % peak MFMA, E=64 top-2 d=2048"
PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15         # FLOP/s, dense bf16 matrix
PEAK_FP32 = 157.3e12       # FLOP/s, fp32
CSRC = os.path.join(ROOT, "mixture_experts_layer_26_amd", "csrc")
COPY_CALIB_BYTES = 1 << 30
# kernel-name patterns of the launches each stage makes (bf16 path)
STAGE_KERNELS = {
    "route": ("route_mfma_kernel", "gate_topk_kernel"),
    "hist": ("hist_kernel",),
    "scatter": ("scatter_kernel",),
    "gather": ("gather_kernel", "gather_tiled_kernel"),
    # the forward's GEMMs only: the 128x128 kernel (template arguments end
    # with the epilogue and the A layout) and the pipelined one with the
    # forward's operand layouts (the backward's instantiations use other
    # epilogues or layouts); GEMM1 reads x_perm row-major (moe_grouped_ffn)
    # or tiled (moe_layer_forward)
    "ffn1": (", 0, false>(moe::GemmArgs)", ", 0, true>(moe::GemmArgs)",
             ", 0, false, false, false>(moe::GemmArgs)", ", 0, true, false, false>(moe::GemmArgs)",
             # the split kernel (expert tails on 128-row tiles): <NS, EPI, AT, BKC>
             "split_kernel<4, 0, false, false>(moe::GemmArgs)", "split_kernel<4, 0, true, false>(moe::GemmArgs)"),
    "ffn2": (", 1, true>(moe::GemmArgs)", ", 1, true, false, false>(moe::GemmArgs)",
             "split_kernel<4, 1, true, false>(moe::GemmArgs)"),
    "combine": ("combine_kernel",),
}


# sources of the layer forward's kernels and their launches (the backward,
# heat map and loss-variant files build none of them)
FORWARD_SOURCES = ("combine.hip", "dispatch.hip", "ffn_bf16.hip", "ffn_fp32.hip", "ffn_sched.h", "lds_dma.h",
                   "moe_api.hip", "moe_common.h", "moe_kernels.h", "route.hip", "route_mfma.hip")


def kernel_source_hash() -> str:
    """Hash of the forward kernels' sources: counter records taken from other
    sources no longer describe the kernels that run."""
    h = hashlib.sha256()
    for name in FORWARD_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # steady state: the GEMMs settle about 4% faster after some 30 layer
    # forwards (1.495 ms/step timed after 5 warm-up steps, 1.44 ms after 30 on
    # the same box); 50 timed steps of about 1.5 ms each
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default=None)
    ap.add_argument("--cpu-seconds", type=float, default=30.0,
                    help="time budget of the oracle: the whole workload when it fits, else a scaled sample")
    ap.add_argument("--only", action="store_true",
                    help="time the one workload only (no per-workload summary of the others)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured copy and library-GEMM reference rates")
    ap.add_argument("--forward-only", action="store_true",
                    help="the timed layer forward of the one workload and nothing after it (for counter runs: "
                         "no heat map, router variants, cold combine, backward, reference rates, oracle or "
                         "other workloads)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<stage>_<workload>.json from the "
                         "counter_collection.csv of a FETCH_SIZE and a WRITE_SIZE "
                         "rocprofv3 --pmc run of this script with --copy-calib")
    return ap.parse_args()


def dispatch_block_tokens(T, E, k):
    """Tokens per histogram/scatter block, the library's rule: 1024 (512 above
    256 experts, 256 above 512), halved while a block holds more than 2048
    slots or there are fewer than 16 blocks, as long as the block count stays
    <= 256 (only the reported bytes of the two dispatch launches depend on
    it)."""
    bt = 1024 if E <= 256 else 512 if E <= 512 else 256
    while bt > 64 and (bt * k > 2048 or (T + bt - 1) // bt < 16) and (T + bt // 2 - 1) // (bt // 2) <= 256:
        bt //= 2
    return bt


def stage_bytes_flops(cfg, S, active, esz, nblk):
    """Algorithmic bytes and FLOPs of each launch (what the method must move
    or compute over the kept slots; no dense T x E work)."""
    T, d, E, k, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    return {
        "route": (T * d * esz + d * E * 4 + T * k * 8, 2 * T * d * E),
        "hist": (T * k * 4 + nblk * E * 4, 0),
        "scatter": (nblk * nblk * E * 4 + T * k * 12 + S * 8, 0),
        # every token row read once (its k copies come from cache), every
        # kept row written once, plus the permutation
        "gather": (T * d * esz + S * d * esz + S * 4, 0),
        "ffn1": (active * d * F * esz + S * d * esz + S * F * esz + active * F * 4, 2 * S * d * F),
        "ffn2": (active * F * d * esz + S * F * esz + S * d * 4 + active * d * 4, 2 * S * d * F),
        "combine": (S * d * 4 + T * d * 4 + T * k * 8, 2 * S * d),
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, budget_s):
    """Time the oracle (as it stands) over the whole workload when it fits
    the time budget: the full layer forward (gate, routing, dispatch, every
    kept slot's expert FFN, combine and the balance loss) in one call.  If a
    first timed chunk shows that the whole batch would take more than
    budget_s, the expert FFN and combine run over leading token chunks until
    the budget is spent and are scaled to all kept slots (said in `sample`)."""
    import numpy as np
    import oracle
    x, Wg, bg = inp["x"], inp["Wg"], inp["bg"]
    t0 = time.perf_counter()
    L = oracle.gate(x, Wg, bg)
    idx, w = oracle.route(L.astype(np.float32), cfg.k, cfg.temperature)
    cap = oracle.capacity(cfg.T, cfg.E, cfg.k, cfg.capacity_factor)
    dsp = oracle.dispatch(idx, cfg.E, cap)
    t_route = time.perf_counter() - t0
    S = int(dsp["offsets"][-1])
    # a first chunk sizes the rest
    probe = np.arange(0, min(cfg.T, 256), dtype=np.int32)
    t1 = time.perf_counter()
    oracle.layer_tokens(probe, x, inp["W1"], inp["b1"], inp["W2"], inp["b2"], idx, dsp["slot"], w)
    t_probe = time.perf_counter() - t1
    probe_slots = max(int((dsp["slot"][probe] >= 0).sum()), 1)
    base = {"unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle", "cpu_model": cpu_model()}
    if t_probe * S / probe_slots <= budget_s:
        t2 = time.perf_counter()
        ref = oracle.layer_forward(x, Wg, bg, inp["W1"], inp["b1"], inp["W2"], inp["b2"], cfg.k,
                                   cfg.capacity_factor, cfg.temperature, cfg.aux_lambda)
        total = time.perf_counter() - t2
        return dict(base, value=cfg.T / total, seconds_measured=round(total, 2), sample=(
            f"the whole workload: one oracle layer forward (gate, top-k, dispatch, expert FFN of all "
            f"{int(ref['offsets'][-1])} kept slots, combine, balance loss) over all {cfg.T} tokens, "
            f"{total:.2f} s; fp64, plain C + OpenMP on {oracle.threads()} threads"))
    done_tok, done_slots, t_ffn = int(probe[-1]) + 1, probe_slots, t_probe
    chunk = 64
    while done_tok < cfg.T and t_ffn < budget_s:
        toks = np.arange(done_tok, min(cfg.T, done_tok + chunk), dtype=np.int32)
        t1 = time.perf_counter()
        oracle.layer_tokens(toks, x, inp["W1"], inp["b1"], inp["W2"], inp["b2"], idx, dsp["slot"], w)
        t_ffn += time.perf_counter() - t1
        done_slots += int((dsp["slot"][toks] >= 0).sum())
        done_tok = int(toks[-1]) + 1
    total = t_route + t_ffn * (S / max(done_slots, 1))
    return dict(base, value=cfg.T / total, seconds_measured=round(t_route + t_ffn, 2), sample=(
        f"gate+top-k+dispatch over all {cfg.T} tokens ({t_route:.2f} s); expert FFN + combine over the "
        f"first {done_tok} tokens ({done_slots} of {S} kept slots, {t_ffn:.2f} s), scaled by {S}/{done_slots} "
        f"to all kept slots; fp64, plain C + OpenMP on {oracle.threads()} threads"))


def _stage_of(kernel: str):
    for stage, pats in STAGE_KERNELS.items():
        if stage.startswith("ffn"):
            if "ffn_gemm_" in kernel and any(kernel.endswith(p) for p in pats):
                return stage
        elif any(p in kernel for p in pats):
            return stage
    return None


def write_traffic(fetch_csv: str, write_csv: str, workload: str, steps: int) -> None:
    """HBM bytes per launch of each stage from the FETCH_SIZE / WRITE_SIZE
    counters (KiB per dispatch).  Each counter is scaled by what it reads for
    the plain copy of COPY_CALIB_BYTES that --copy-calib runs; the last
    `steps` dispatches of each kernel (the timed ones) are averaged."""
    import csv
    import numpy as np

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        by = {}
        for r in rows:
            by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return by

    fe, wr = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    kib = COPY_CALIB_BYTES / 1024

    def calib(by):
        vals = [v for name, vs in by.items() if "copyBuffer" in name for v in vs]
        big = max(vals)
        return kib / float(np.mean([v for v in vals if v > 0.5 * big]))

    f_fetch, f_write = calib(fe), calib(wr)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for name in fe:
        stage = _stage_of(name)
        if stage is None or name not in wr:
            continue
        fk = float(np.mean(fe[name][-steps:]))
        wk = float(np.mean(wr[name][-steps:]))
        rec = {
            "workload": workload, "stage": stage, "kernel": name,
            "bytes_per_launch": (fk * f_fetch + wk * f_write) * 1024,
            "fetch_bytes": fk * f_fetch * 1024, "write_bytes": wk * f_write * 1024,
            "fetch_kib_raw": fk, "write_kib_raw": wk,
            "calib_fetch_factor": f_fetch, "calib_write_factor": f_write,
            "dispatches_averaged": min(steps, len(fe[name])),
            "kernel_source_hash": kernel_source_hash(),
            "commands": [
                f"rocprofv3 --pmc {c} --output-format csv -d <dir> -o run -- python3 bench.py "
                f"--config {workload} --steps {steps} --warmup 1 --forward-only --copy-calib"
                for c in ("FETCH_SIZE", "WRITE_SIZE")],
        }
        with open(os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.json"), "w") as f:
            json.dump(rec, f, indent=1)
        print(f"{stage:8s} {rec['bytes_per_launch'] / 1e9:8.4f} GB/launch  "
              f"(fetch x{f_fetch:.3f}, write x{f_write:.3f})")


def load_traffic(workload: str, stage: str):
    p = os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def measured_peaks(cfg, S, active, dev):
    """What this GPU reaches on plain references, beside the published
    peaks: a device-to-device copy of 1 GiB (HBM read + write), the vendor
    library's bf16 GEMM (hipBLASLt through torch.matmul) on 8192^3, and the
    same library on the workload's expert GEMM1 shape with the kept rows
    spread evenly over the active experts (torch.bmm, contiguous operands,
    no routing, no skew, no bias or GELU).  Reference rates only."""
    import torch

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    out = {}
    src = torch.empty(COPY_CALIB_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src), 5)
    out["copy_GB/s"] = 2 * COPY_CALIB_BYTES / t / 1e9
    del src, dst
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    t = timed(lambda: torch.matmul(a, b), 5)
    out["library_gemm_bf16_8192_TFLOP/s"] = 2 * n ** 3 / t / 1e12
    del a, b
    if cfg.dtype == "bf16" and active > 0:
        m = (S + active - 1) // active
        a = torch.randn(active, m, cfg.d, device=dev, dtype=torch.bfloat16)
        b = torch.randn(active, cfg.d, cfg.d_ff, device=dev, dtype=torch.bfloat16)
        t = timed(lambda: torch.bmm(a, b), 5)
        out["library_bmm_expert_shape"] = f"{active} x [{m} x {cfg.d}] x [{cfg.d} x {cfg.d_ff}]"
        out["library_bmm_expert_shape_TFLOP/s"] = 2.0 * active * m * cfg.d * cfg.d_ff / t / 1e12
        del a, b
    torch.cuda.empty_cache()
    return out


def time_heat_map(moe, s, cfg, d, y, counts, aux, ws, stream, reps=20):
    """Routing heat map + load telemetry (moe_coactivation) on the top-k
    lists of one layer forward of the same workload; HIP events around each
    call on the call's stream.  Algorithmic bytes: read T*k indices, write
    the E x E counts and the E loads."""
    import numpy as np
    import torch
    dev = y.device
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    moe.moe_layer_forward(s, d["x"], d["Wg"], d["bg"], d["W1"], d["b1"], d["W2"], d["b2"], y,
                          counts, aux, ws, topk_idx=idx, stream=stream)
    Hm = torch.empty((cfg.E, cfg.E), dtype=torch.int32, device=dev)
    rt = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    st = torch.empty(3, dtype=torch.float32, device=dev)
    for _ in range(3):
        moe.moe_coactivation(s, idx, Hm, rt, st, stream=stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        moe.moe_coactivation(s, idx, Hm, rt, st, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * float(np.median([a.elapsed_time(b) for a, b in ev]))
    nbytes = cfg.T * cfg.k * 4 + cfg.E * cfg.E * 4 + cfg.E * 4
    stats = st.cpu().numpy()
    return {"us": us, "algorithmic_bytes": nbytes, "GB/s": nbytes / (us * 1e-6) / 1e9,
            "frac_hbm": nbytes / (us * 1e-6) / PEAK_HBM, "pairs": cfg.T * cfg.k * (cfg.k - 1) // 2,
            "load_mean": float(stats[0]), "load_var": float(stats[1]), "load_cv": float(stats[2])}


def _median_us(fn, stream, reps=20):
    import numpy as np
    import torch
    for _ in range(3):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return 1e3 * float(np.median([a.elapsed_time(b) for a, b in ev]))


def time_combine_cold(moe, s, cfg, b, stream, reps=10):
    """The combine alone (moe_combine on the forward's expert outputs, slot
    and weights), once right after a forward (out_perm written just before,
    partly still in the 256 MB MALL) and once after 1 GiB has been streamed
    through the caches (a device copy, each rep), so that out_perm comes from
    HBM.  Algorithmic bytes as the combine stage: read the kept rows' fp32
    outputs and the weights, write y."""
    import numpy as np
    import torch
    dev = b["y"].device
    T, D, k = cfg.T, cfg.d, cfg.k
    f32, i32 = torch.float32, torch.int32
    idx, w = torch.empty((T, k), dtype=i32, device=dev), torch.empty((T, k), dtype=f32, device=dev)
    ws = b["ws"]
    R = moe.moe_max_rows(s)

    def region(which, dtype, n, esz):
        off = moe.moe_workspace_offset(s, which)
        return ws[off:off + n * esz].view(dtype)

    y2 = torch.empty((T, D), dtype=f32, device=dev)
    src = torch.empty(COPY_CALIB_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    warm, cold = [], []
    for _ in range(reps):
        moe.moe_layer_forward(s, b["d"]["x"], b["d"]["Wg"], b["d"]["bg"], b["d"]["W1"], b["d"]["b1"], b["d"]["W2"],
                              b["d"]["b2"], b["y"], b["counts"], b["aux"], ws, topk_idx=idx, topk_w=w, stream=stream)
        slot = region(moe.MOE_WS_SLOT, i32, T * k, 4)
        outp = region(moe.MOE_WS_OUT, f32, R * D, 4)
        for lst, flush in ((warm, False), (cold, True)):
            if flush:
                dst.copy_(src)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            moe.moe_combine(s, outp, slot, w, y2, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            lst.append(1e3 * e0.elapsed_time(e1))
    S = int(b["counts"].sum().item())
    nbytes = S * D * 4 + T * D * 4 + T * k * 8
    out = {"algorithmic_bytes": nbytes}
    for name, lst in (("after_forward", warm), ("after_1GiB_stream", cold)):
        us = float(np.median(lst))
        out[name] = {"us": us, "GB/s": nbytes / (us * 1e-6) / 1e9, "frac_hbm": nbytes / (us * 1e-6) / PEAK_HBM}
    del src, dst
    return out


def time_router_variant(moe, s, cfg, d, ws, stream):
    """The stable layer's router on the workload's gate logits: noisy top-1
    over the full softmax (moe_route_logits_ex, writing the noisy logits)
    and the load-variance loss (moe_aux_loss_ex).  Algorithmic bytes of the
    router: read logits and noise, write the noisy logits, index and weight."""
    import numpy as np
    import torch
    dev = d["x"].device
    T, E = cfg.T, cfg.E
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    i0 = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
    w0 = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
    moe.moe_route(s, d["x"], d["Wg"], d["bg"], logits, i0, w0, ws, stream=stream)
    noise = torch.from_numpy(np.random.default_rng(11).standard_normal((T, E)).astype(np.float32)).to(dev)
    s1 = moe.shape(T, cfg.d, E, 1, cfg.d_ff, 0.0, 1.0, 0.01)
    idx = torch.empty((T, 1), dtype=torch.int32, device=dev)
    w = torch.empty((T, 1), dtype=torch.float32, device=dev)
    noisy = torch.empty((T, E), dtype=torch.float32, device=dev)
    us_route = _median_us(lambda: moe.moe_route_logits_ex(s1, moe.MOE_ROUTER_TOP1_FULL, logits, idx, w, noise=noise,
                                                          noise_scale=0.1, noisy_logits=noisy, stream=stream), stream)
    routed = torch.empty(E, dtype=torch.int32, device=dev)
    Hm = torch.empty((E, E), dtype=torch.int32, device=dev)
    moe.moe_coactivation(s1, idx, Hm, routed, stream=stream)
    aux = torch.empty(1, dtype=torch.float32, device=dev)
    us_loss = _median_us(lambda: moe.moe_aux_loss_ex(s1, moe.MOE_LOSS_VARIANCE, routed, aux, stream=stream), stream)
    state = moe.window_state(E, 100, dev)
    pbar = torch.empty(E, dtype=torch.float32, device=dev)
    aux_w = torch.empty(1, dtype=torch.float32, device=dev)
    us_window = _median_us(lambda: moe.moe_aux_loss_window(s1, routed, state, 100, aux_w, pbar, stream=stream),
                           stream)
    nbytes = 3 * T * E * 4 + 8 * T
    return {"top1_noisy_us": us_route, "top1_noisy_bytes": nbytes, "window_loss_us": us_window,
            "top1_noisy_GB/s": nbytes / (us_route * 1e-6) / 1e9,
            "top1_noisy_frac_hbm": nbytes / (us_route * 1e-6) / PEAK_HBM,
            "variance_loss_us": us_loss, "variance_loss": float(aux.cpu().numpy()[0])}


def time_backward(moe, s, cfg, d, ws, stream, reps=5):
    """moe_layer_backward after one forward of the same batch (dy seeded
    N(0,1)); HIP events around each call.  FLOPs: five GEMMs of 2 S d d_ff
    each (recompute, dh, dx_perm, dW1, dW2) plus the gate's two sums of
    2 T k d (dWg and the gate's part of dx: k nonzero logit gradients per
    token)."""
    import numpy as np
    import torch
    dev = d["x"].device
    T, E, k, D, F = cfg.T, cfg.E, cfg.k, cfg.d, cfg.d_ff
    f32, i32 = torch.float32, torch.int32
    y, counts, aux = (torch.empty((T, D), dtype=f32, device=dev), torch.empty(E, dtype=i32, device=dev),
                      torch.empty(1, dtype=f32, device=dev))
    idx, w = torch.empty((T, k), dtype=i32, device=dev), torch.empty((T, k), dtype=f32, device=dev)
    moe.moe_layer_forward(s, d["x"], d["Wg"], d["bg"], d["W1"], d["b1"], d["W2"], d["b2"], y, counts, aux, ws,
                          topk_idx=idx, topk_w=w, stream=stream)
    R = moe.moe_max_rows(s)

    def region(which, dtype, n, esz):
        off = moe.moe_workspace_offset(s, which)
        return ws[off:off + n * esz].view(dtype)

    slot = region(moe.MOE_WS_SLOT, i32, T * k, 4)
    offsets = region(moe.MOE_WS_OFFSETS, i32, E + 1, 4)
    # a bf16 forward keeps x_perm only in the tile layout: the backward copies
    # the rows itself (its time includes that copy)
    xperm = None if cfg.dtype == "bf16" else region(moe.MOE_WS_XPERM, f32, R * D, 4)
    outp = region(moe.MOE_WS_OUT, f32, R * D, 4)
    dy = torch.from_numpy(np.random.default_rng(77).standard_normal((T, D)).astype(np.float32)).to(dev)
    g = [torch.empty(sh, dtype=f32, device=dev) for sh in ((T, D), (D, E), (E,), (E, D, F), (E, F), (E, F, D), (E, D))]
    bws = moe.backward_workspace(s, dev)
    us = _median_us(lambda: moe.moe_layer_backward(s, d["x"], d["Wg"], d["W1"], d["b1"], d["W2"], dy, idx, w, slot,
                                                   offsets, xperm, outp, *g, bws, stream=stream), stream, reps)
    S = int(counts.cpu().numpy().sum())
    # five expert GEMMs over the kept rows; the gate's dWg and dx part are
    # sums over the k selected experts of each token (the other logits have
    # no gradient)
    flops = 10 * S * D * F + 4 * T * cfg.k * D
    bf16 = cfg.dtype == "bf16"
    peak = PEAK_BF16 if bf16 else PEAK_FP32
    return {"ms": us / 1e3, "tflops": flops / (us * 1e-6) / 1e12, "flops": flops,
            "peak_tflops": peak / 1e12, "frac_peak": flops / (us * 1e-6) / peak,
            "arith": ("expert GEMMs on bf16 MFMA (fp32 accumulate); gate gradients as fp32 sums over the k "
                      "selected experts" if bf16 else "fp32 vector ALUs")}


def prepare(moe, cfg, dev):
    """Seeded inputs of the workload on the device, its shape, workspace and
    outputs; returns (host inputs, device inputs, buffers, seconds taken)."""
    import numpy as np
    import torch
    from moe_inputs import make_inputs
    t_gen = time.perf_counter()
    inp = make_inputs(cfg)

    def to_dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    d = {k: to_dev(v) for k, v in inp.items()}
    s = moe.shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff, cfg.capacity_factor, cfg.temperature,
                  cfg.aux_lambda, moe.MOE_BF16 if cfg.dtype == "bf16" else moe.MOE_F32)
    b = dict(s=s, ws=moe.workspace(s, dev),
             y=torch.empty((cfg.T, cfg.d), dtype=torch.float32, device=dev),
             counts=torch.empty(cfg.E, dtype=torch.int32, device=dev),
             routed=torch.empty(cfg.E, dtype=torch.int32, device=dev),
             aux=torch.empty(1, dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    return inp, d, b, time.perf_counter() - t_gen


class TimingEvents:
    """HIP timing events created with hipEventDisableSystemFence: recording
    one skips the system-scope release (an L2 write-back and invalidate),
    which a default event pays between the launches it brackets and which
    slows the launch after it.  Read only after a device synchronisation."""
    FLAG = 0x20000000   # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        self._C = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.made = []

    def new(self) -> int:
        e = self._C.c_void_p()
        if self.hip.hipEventCreateWithFlags(self._C.byref(e), self.FLAG) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.made.append(e.value)
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = self._C.c_float()
        if self.hip.hipEventElapsedTime(self._C.byref(ms), self._C.c_void_p(a), self._C.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self):
        for e in self.made:
            self.hip.hipEventDestroy(self._C.c_void_p(e))
        self.made = []


def warm_clocks(dev, ms=60.0):
    """About `ms` of bf16 matrix-core work (the library's 8192^3 GEMM): the
    GPU's clocks follow its matrix-core load, and a forward timed right
    after host-side set-up reads its first ~30 steps slower; this brings the
    clocks to their working level without running the measured layer."""
    import torch
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    for _ in range(max(1, int(ms))):   # ~1 ms each on MI355X
        torch.matmul(a, b)
    del a, b


def make_stage_events(moe, steps):
    """Fence-free HIP events for time_forward: one set around the two GEMMs
    for each timed step, one around every stage for each step of the second
    pass."""
    names = moe.moe_stage_names()
    gemm_stages = {j for j, n in enumerate(names) if n in ("ffn1", "ffn2")}
    te = TimingEvents()

    def make(which):
        return [[te.new() if (i // 2) in which else None for i in range(2 * len(names))] for _ in range(steps)]

    return dict(te=te, names=names, gemm_stages=gemm_stages, timed=make(gemm_stages),
                all=make(set(range(len(names)))))


def time_forward(moe, cfg, d, b, stream, steps, warmup, ev=None):
    """W untimed steps, then K timed steps between two synchronisations on
    the launch stream.  The timed steps record HIP events around the two
    expert GEMMs only (the dominant launches, whose times the roofline needs
    from the timed region); the other stages are timed in a second, fully
    instrumented pass of as many steps right after.  All stage events skip
    the system-scope fence (TimingEvents) and exist before the warmup steps,
    so that nothing but the synchronisation separates the warmup from the
    timed steps.  Returns (ms per step, {stage: us})."""
    import numpy as np
    import torch
    s, ws = b["s"], b["ws"]
    ev = ev or make_stage_events(moe, steps)
    te, names, gemm_stages, ev_timed, ev_all = ev["te"], ev["names"], ev["gemm_stages"], ev["timed"], ev["all"]

    def step(events=None):
        if events is not None:
            moe.moe_set_stage_events(events)
        moe.moe_layer_forward(s, d["x"], d["Wg"], d["bg"], d["W1"], d["b1"], d["W2"], d["b2"], b["y"],
                              b["counts"], b["aux"], ws, routed=b["routed"], stream=stream)

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        step(ev_timed[i])
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    for i in range(steps):
        step(ev_all[i])
    torch.cuda.synchronize()
    moe.moe_set_stage_events([None] * (2 * len(names)))

    def stage_mean(ev, j):
        return 1e3 * float(np.mean([te.elapsed_ms(e[2 * j], e[2 * j + 1]) for e in ev]))

    out = {n: stage_mean(ev_timed if j in gemm_stages else ev_all, j) for j, n in enumerate(names)}
    te.destroy()
    return ms, out


def summarize(cfg, ms, stage_us, b):
    """Throughput, the grouped GEMMs' rate, the dominant launch against its
    roofline and the routing / permutation / combine launches against HBM."""
    c = b["counts"].cpu().numpy()
    rt = b["routed"].cpu().numpy()
    esz = 2 if cfg.dtype == "bf16" else 4
    S = int(c.sum())
    active = int((c > 0).sum())
    bt = dispatch_block_tokens(cfg.T, cfg.E, cfg.k)
    nblk = (cfg.T + bt - 1) // bt
    bf = stage_bytes_flops(cfg, S, active, esz, nblk)
    ffn_flops = 4 * S * cfg.d * cfg.d_ff
    gemm_us = stage_us["ffn1"] + stage_us["ffn2"]
    dom = max(stage_us, key=lambda n: stage_us[n])
    dbytes, dflops = bf[dom]
    t_dom = stage_us[dom] * 1e-6
    peak_mm = PEAK_BF16 if esz == 2 else PEAK_FP32
    if dbytes / PEAK_HBM >= dflops / peak_mm:
        roof = {"bound": "hbm", "achieved": dbytes / t_dom / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": dflops / t_dom / 1e12, "peak": peak_mm / 1e12,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = load_traffic(cfg.name, dom)
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = dbytes
    roof["algorithmic_flops"] = dflops
    roof["mfma_frac"] = dflops / t_dom / peak_mm
    roof["hbm_frac"] = dbytes / t_dom / PEAK_HBM
    return {
        "ms_per_step": ms,
        "tokens_per_s": cfg.T / (ms * 1e-3),
        "roofline": roof,
        "grouped_gemm": {"tflops": ffn_flops / (gemm_us * 1e-6) / 1e12,
                         "frac_peak_bf16" if esz == 2 else "frac_peak_fp32": ffn_flops / (gemm_us * 1e-6) / peak_mm,
                         "us": gemm_us},
        "stages_us": stage_us,
        # algorithmic bytes of the routing, permutation and combine launches
        # over their HIP-event times (which include the event records: a few
        # us on these short launches, see the kernel trace in profiles/)
        "stage_hbm": {n: {"us": stage_us[n], "algorithmic_bytes": bf[n][0],
                          "GB/s": bf[n][0] / (stage_us[n] * 1e-6) / 1e9,
                          "frac_hbm": bf[n][0] / (stage_us[n] * 1e-6) / PEAK_HBM}
                      for n in ("route", "hist", "scatter", "gather", "combine") if n in stage_us},
        "layer_tflops": (ffn_flops + 2 * cfg.T * cfg.d * cfg.E) / (ms * 1e-3) / 1e12,
        "kept_slots": S, "dropped_slots": cfg.T * cfg.k - S, "active_experts": active,
        "routed_cv": float(rt.std() / rt.mean()),
        "aux": float(b["aux"].cpu().numpy()[0]),
    }


def config_of(cfg):
    return {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k,
            "d_ff": cfg.d_ff, "capacity_factor": cfg.capacity_factor,
            "temperature": cfg.temperature, "seed": cfg.seed, "dtype": cfg.dtype,
            "gate_bias": (f"zipf s={cfg.zipf_s} alpha={cfg.zipf_alpha}" if cfg.zipf_s else None),
            "clustered_tokens": cfg.cluster_frac or None,
            "parallelism": "single GPU"}


def main():
    args = parse()
    if args.traffic_from:
        from moe_inputs import HEADLINE
        write_traffic(*args.traffic_from, args.config or HEADLINE, args.steps)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    import torch

    import mixture_experts_layer_26_amd as moe
    from moe_inputs import HEADLINE, WORKLOADS, get

    cfg = get(args.config or HEADLINE)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    inp, d, b, t_gen = prepare(moe, cfg, dev)
    s, ws, y, counts, aux = b["s"], b["ws"], b["y"], b["counts"], b["aux"]
    fwd_only = args.forward_only
    # The untimed measurements on the same batch run first, the backward (the
    # heaviest matrix-core work) last: the timed steps then start on a GPU at
    # the clocks it holds while it works, not right after seconds of
    # host-side set-up, where the first ~30 forwards of the 64-expert layer
    # read up to 20% slower.  W and K are unchanged.
    ev = make_stage_events(moe, args.steps)
    pre = {}
    if not fwd_only:
        pre["heat_map"] = time_heat_map(moe, s, cfg, d, y, counts, aux, ws, stream)
        if not args.no_peaks and not args.copy_calib:
            c = counts.cpu().numpy()   # the heat map's forward of the same batch
            pre["measured_peaks"] = measured_peaks(cfg, int(c.sum()), int((c > 0).sum()), dev)
        # the combine's rate with its input out of the caches (the 256 MB MALL
        # holds part of out_perm right after the forward)
        pre["combine_cold"] = time_combine_cold(moe, s, cfg, dict(b, d=d), stream)
        pre["router_variant"] = time_router_variant(moe, s, cfg, d, ws, stream)
        if not args.no_backward:
            pre["backward"] = time_backward(moe, s, cfg, d, ws, stream)
    ms, stage_us = time_forward(moe, cfg, d, b, stream, args.steps, args.warmup, ev)
    summ = summarize(cfg, ms, stage_us, b)
    out = {
        "metric": METRIC,
        "value": summ["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded numpy PCG64 inputs of the workload's shape and distributions)",
        "config": config_of(cfg),
        "roofline": summ["roofline"],
        "stages_timing": "ffn1/ffn2: HIP events inside the timed steps; other stages: a second pass of the same "
                         "number of steps with events around every launch; stage events are created with "
                         "hipEventDisableSystemFence (no cache write-back at each record)",
        "timed_after": ("the heat map, measured peaks, combine, router-variant and backward timings on the same "
                        "batch, then the W warmup steps" if pre else "the W warmup steps"),
        "setup_seconds": round(t_gen, 2),
    }
    out.update({k: v for k, v in summ.items() if k not in ("ms_per_step", "tokens_per_s", "roofline")})
    out.update(pre)
    if args.copy_calib:
        src = torch.empty(COPY_CALIB_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calib_bytes"] = COPY_CALIB_BYTES
    del d, b, s, ws, y, counts, aux
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline and not fwd_only:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    del inp
    if not args.only and not fwd_only:
        # every other workload (and the literal-Zipf reading of the headline,
        # and the naive soft layer over all 128 experts): the same timed
        # forward, shorter runs, no backward or oracle
        out["configs"] = {}
        for name in WORKLOADS + ["skewed_e64_literal", "dense_soft_e16", "dense_soft_e128"]:
            if name == cfg.name:
                continue
            c2 = get(name)
            _, d2, b2, tg = prepare(moe, c2, dev)
            w2, k2 = min(args.warmup, 10), min(args.steps, 20)
            ev2 = make_stage_events(moe, k2)
            warm_clocks(dev)
            ms2, st2 = time_forward(moe, c2, d2, b2, stream, k2, w2, ev2)
            out["configs"][name] = dict(config=config_of(c2), steps=k2, warmup=w2, dtype=c2.dtype,
                                        timed_after="60 ms of bf16 library GEMMs, then the W warmup steps",
                                        **summarize(c2, ms2, st2, b2), setup_seconds=round(tg, 2))
            del d2, b2
            torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
