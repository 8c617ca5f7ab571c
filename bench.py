"""Benchmark of the Orthros attention hot path on one MI355X.

One step = one pass over every part of the hot path on synthetic, seeded
inputs already resident in HBM:
  prefill_128k   cache append (T = 131072 rows), sliding-window prefill
                 (W = 4096, query scale-offset fused), output-stream
                 cross-attention at the last position (T_out = 1);
                 B = 1, 32 query / 8 KV heads, D = 128, bf16
  decode_pair    256 consecutive decode pair steps, B = 64 sequences with
                 32768 cached tokens each (W = 2048); the cache length is
                 rewound to 32768 at the start of every step
The reported value is prefill tokens/s (B*T over the summed time of the
three prefill launches); the decode pair's KV GB/s and latency, the full
causal run at the same T (speedup ratio), the roofline of the dominant
kernel and the fp64 CPU oracle's rate on a bounded sample are reported
beside it. Extra legs outside the timed steps: the sliding window at
W = 128, the paged ragged decode, the whole layer (projections + attention
+ W_O) at 128K, the 32K and SFT dual-stream prefills, and the training
backward at the SFT shape. All GPU times come from HIP events on the launch
stream.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-causal]
                [--no-paged] [--no-layer] [--no-backward] [--no-other-prefills]
                [--no-cpu-baseline] [--only prefill|decode]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Orthros prefill tokens/s @128K (SWA+global) + decode-pair KV GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
BAND_SRC = os.path.join(ROOT, "long_context_prefill_swa_amd", "csrc",
                        "band_persist.hip")
SPLIT_SRC = os.path.join(ROOT, "long_context_prefill_swa_amd", "csrc",
                         "splitkv_mfma.hip")
ROLL_SRC = os.path.join(ROOT, "long_context_prefill_swa_amd", "csrc",
                        "band_roll.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def band_pairs(T, W):
    """(query, key) pairs of the base stream per head: sum_t min(t+1, W)."""
    W = min(W, T)
    return W * (W + 1) // 2 + (T - W) * W


def causal_pairs(T):
    return T * (T + 1) // 2


def kernel_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(name, sha):
    """HBM bytes per launch of `name` from a committed counter summary, or
    None if there is none or it was taken on other kernel source."""
    path = os.path.join(PROFILES, f"{name}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != sha:
        return None
    return float(m_b.group(1))


def stats(xs):
    """mean, median, p10, p90 and count of a list of times (ms)."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)),
            "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def shader_clock(dev, iters=100000):
    """Average shader clock (MHz) while every compute unit runs MFMA chains
    (libclock_probe.so: shader-cycle counter over the constant-rate wall
    counter), or None if the probe is not built."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "long_context_prefill_swa_amd",
                        "libclock_probe.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.clock_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                              ctypes.POINTER(ctypes.c_int), ctypes.c_void_p]
    L.clock_probe.restype = ctypes.c_int
    n_blocks = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.zeros(3 * n_blocks, dtype=torch.int64, device=dev)
    khz = ctypes.c_int(0)
    stream = torch.cuda.current_stream(dev)
    rc = L.clock_probe(ctypes.c_void_p(out.data_ptr()), n_blocks, iters,
                       ctypes.byref(khz),
                       ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"clock probe failed: hip error {rc}")
    torch.cuda.synchronize()
    r = out.view(n_blocks, 3).cpu().double()
    cycles, ticks = r[:, 0].sum().item(), r[:, 1].sum().item()
    return cycles / (ticks / (khz.value * 1e3)) / 1e6


def hbm_reference(dev, flush, reps=10):
    """The HBM rate plain streaming kernels reach on this GPU
    (libclock_probe.so: buffer loads and stores, each launch after a MALL
    flush), as a second reference beside the published 8 TB/s: a read of
    512 MiB (the 128K cache's K and V) and a copy moving 2.68 GB (the bytes
    of the W = 128 window pass). None if the probe is not built."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "long_context_prefill_swa_amd",
                        "libclock_probe.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    L.hbm_read_probe.argtypes = [vp, sz, i32, vp, vp]
    L.hbm_copy_probe.argtypes = [vp, vp, sz, i32, vp]
    L.hbm_read_probe.restype = L.hbm_copy_probe.restype = ctypes.c_int
    stream = torch.cuda.current_stream(dev)
    st = ctypes.c_void_p(stream.cuda_stream)
    read_bytes, read_wg = 512 << 20, 256
    copy_bytes, copy_wg = 1342177280, 4096
    src = torch.ones(copy_bytes // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    sink = torch.empty(read_wg * 256 * 4, dtype=torch.int32, device=dev)

    def timed(f):
        for _ in range(2):
            if f() != 0:
                raise RuntimeError("hbm probe launch failed")
        ts = []
        for _ in range(reps):
            flush()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            f()
            b.record(stream)
            ts.append((a, b))
        torch.cuda.synchronize()
        return stats([x.elapsed_time(y) for x, y in ts])

    s_read = timed(lambda: L.hbm_read_probe(ctypes.c_void_p(src.data_ptr()),
                                            read_bytes, read_wg,
                                            ctypes.c_void_p(sink.data_ptr()), st))
    s_copy = timed(lambda: L.hbm_copy_probe(ctypes.c_void_p(src.data_ptr()),
                                            ctypes.c_void_p(dst.data_ptr()),
                                            copy_bytes, copy_wg, st))
    del src, dst, sink
    torch.cuda.empty_cache()
    read_gbps = read_bytes / (s_read["median"] * 1e-3) / 1e9
    copy_gbps = 2 * copy_bytes / (s_copy["median"] * 1e-3) / 1e9
    return {"read_GBps": read_gbps, "read_bytes": read_bytes,
            "read_ms": s_read, "copy_GBps": copy_gbps,
            "copy_bytes_moved": 2 * copy_bytes, "copy_ms": s_copy,
            "read_frac_of_peak": read_gbps / PEAK_HBM_GBPS,
            "copy_frac_of_peak": copy_gbps / PEAK_HBM_GBPS,
            "notes": "hand-written streaming read and copy kernels "
                     "(libclock_probe.so), medians, each launch after a MALL "
                     "flush"}


def run_context(dev, clock_before, clock_after):
    import torch
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rocm = ""
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    p = torch.cuda.get_device_properties(dev)
    return {"gpu": p.name, "gcn_arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count,
            "shader_clock_mhz_under_mfma_load":
                {"before": clock_before, "after": clock_after},
            "rocm": rocm, "torch": torch.__version__,
            "torch_hip": torch.version.hip, "cpu_model": cpu,
            "cpu_count": os.cpu_count(),
            "cpu_affinity": len(os.sched_getaffinity(0)),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-causal", action="store_true")
    ap.add_argument("--no-paged", action="store_true")
    ap.add_argument("--no-layer", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-other-prefills", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode"], default=None)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} "
              "is not supported (the attention path is run on one GPU's "
              "share; see the sharding notes).", file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_prefill_swa_amd as lo
    from workloads import (affine_inputs, decode_all_steps, kv_inputs,
                           prefill_inputs, workload)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lo.lib()
    stream = torch.cuda.current_stream(dev)
    run_prefill = args.only in (None, "prefill")
    run_decode = args.only in (None, "decode")

    # ---- prefill_128k inputs ------------------------------------------------
    pc, pc_id = workload("prefill_128k")
    if run_prefill:
        log(f"[bench] generating {pc.name} inputs")
        px = prefill_inputs(pc, pc_id, dev)
        kc4 = torch.empty((pc.B, pc.Hkv, pc.T, pc.D), dtype=torch.bfloat16,
                          device=dev)
        vc4 = torch.empty_like(kc4)
        cl4 = torch.zeros(pc.B, dtype=torch.int32, device=dev)
        o4 = torch.empty_like(px.q_pre)
        ox4 = torch.empty_like(px.qx_pre)
        ws4 = lo.workspace(lo.orthros_workspace_bytes(
            lo.ORTHROS_OP_GLOBAL_XATTN, pc.B, pc.Hq, pc.Hkv, pc.D, pc.T_out,
            pc.T), dev)

    # ---- decode_pair inputs -----------------------------------------------
    dc, dc_id = workload("decode_pair_b64")
    n_dec = dc.decode_steps
    if run_decode:
        log(f"[bench] generating {dc.name} inputs")
        cap3 = dc.T + n_dec
        kc3 = torch.empty((dc.B, dc.Hkv, cap3, dc.D), dtype=torch.bfloat16,
                          device=dev)
        vc3 = torch.empty_like(kc3)
        cl3 = torch.zeros(dc.B, dtype=torch.int32, device=dev)
        k0, v0 = kv_inputs(dc, dc_id, dev)
        lo.orthros_kv_append(kc3, vc3, cl3, k0, v0)
        del k0, v0
        a3, b3, ax3, bx3 = affine_inputs(dc, dc_id, dev)
        st = decode_all_steps(dc, dc_id, device=dev)
        o3 = torch.empty((dc.B, dc.Hq, dc.D), dtype=torch.bfloat16, device=dev)
        ox3 = torch.empty_like(o3)
        ws3 = lo.workspace(lo.orthros_workspace_bytes(
            lo.ORTHROS_OP_DECODE_PAIR, dc.B, dc.Hq, dc.Hkv, dc.D, 1, cap3), dev)
    torch.cuda.synchronize()

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    # The 256 MB Infinity Cache (MALL) would serve part of a memory-bound
    # pass from the previous launch's reads. Reading 1 GiB of other data
    # evicts it (and the L2s). A read, not a write: a written buffer would
    # leave dirty lines whose write-back the next pass would pay for.
    flush_buf = torch.zeros((1 << 30) // 4, dtype=torch.float32, device=dev)

    def mall_flush():
        flush_buf.sum()

    def step(record):
        marks = {}
        if run_prefill:
            cl4.zero_()
            marks["p0"] = ev()
            lo.orthros_kv_append(kc4, vc4, cl4, px.k, px.v)
            marks["p1"] = ev()
            lo.orthros_swa_prefill(px.q_pre, px.alpha, px.beta, kc4, vc4, o4,
                                   pc.W)
            marks["p2"] = ev()
            # output row right after the window pass, as a prefill runs it
            # (K/V partly still in the MALL): the warm figure
            lo.orthros_global_xattn(px.qx_pre, px.alpha_x, px.beta_x, kc4,
                                    vc4, ox4, pc.T_in, ws=ws4)
            marks["p3"] = ev()
            mall_flush()
            marks["p4"] = ev()
            # the same call from HBM: the reported figure
            lo.orthros_global_xattn(px.qx_pre, px.alpha_x, px.beta_x, kc4,
                                    vc4, ox4, pc.T_in, ws=ws4)
            marks["p5"] = ev()
        if run_decode:
            cl3.fill_(dc.T)
            mall_flush()
            dm = [ev()]
            for s in range(n_dec):
                lo.orthros_decode_pair(st.q_pre[s], st.qx_pre[s], a3, b3, ax3,
                                       bx3, st.k_new[s], st.v_new[s], kc3,
                                       vc3, cl3, o3, ox3, dc.T + s + 1, dc.W,
                                       ws=ws3)
                dm.append(ev())
            marks["d"] = dm
        if record is not None:
            record.append(marks)

    clock_before = shader_clock(dev)
    log(f"[bench] shader clock under MFMA load: {clock_before:.0f} MHz")
    log(f"[bench] warmup {args.warmup} step(s)")
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    lo.orthros_check_device_errors()

    log(f"[bench] timing {args.steps} step(s)")
    recs = []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    start_ev = ev()
    for _ in range(args.steps):
        step(recs)
    end_ev = ev()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    total_ms = start_ev.elapsed_time(end_ev)
    lo.orthros_check_device_errors()
    if run_decode:
        assert cl3.tolist() == [dc.T + n_dec] * dc.B, "decode cache lengths"
    clock_after = shader_clock(dev)

    def leg(a, b):
        return stats([r[a].elapsed_time(r[b]) for r in recs])

    out = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": total_ms / args.steps, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": "prefill_128k + decode_pair_b64",
                      "prefill_128k": "B=1 Hq=32 Hkv=8 D=128 T=131072 W=4096 T_out=1",
                      "decode_pair_b64": "B=64 Hq=32 Hkv=8 D=128 L0=32768 W=2048 steps=256",
                      "global_batch": pc.B, "seq_len": pc.T}}
    out["run"] = run_context(dev, clock_before, clock_after)
    ref = hbm_reference(dev, mall_flush)
    if ref is not None:
        out["hbm_reference"] = ref
        log(f"[bench] HBM reference: read {ref['read_GBps']:.0f} GB/s, "
            f"copy {ref['copy_GBps']:.0f} GB/s")
    log(f"[bench] wall {wall:.2f}s, events {total_ms:.1f} ms")

    if run_prefill:
        s_app, s_swa = leg("p0", "p1"), leg("p1", "p2")
        s_glob_warm, s_glob = leg("p2", "p3"), leg("p4", "p5")
        t_app, t_swa, t_glob = s_app["mean"], s_swa["mean"], s_glob["mean"]
        t_pre = t_app + t_swa + t_glob
        F_swa = 4.0 * pc.D * band_pairs(pc.T, pc.W) * pc.Hq * pc.B
        F_glob = 4.0 * pc.D * pc.T * pc.Hq * pc.B
        kv_bytes = 2.0 * pc.B * pc.Hkv * pc.T * pc.D * 2
        swa_tflops = F_swa / (t_swa * 1e-3) / 1e12
        out["value"] = pc.B * pc.T / (t_pre * 1e-3)
        out["prefill"] = {
            "ms_kv_append": t_app, "ms_swa": t_swa, "ms_global": t_glob,
            "ms_total": t_pre,
            "timing": {"kv_append": s_app, "swa": s_swa,
                       "global_from_hbm": s_glob,
                       "global_warm_after_swa": s_glob_warm},
            "attention_tflops": (F_swa + F_glob) / ((t_swa + t_glob) * 1e-3) / 1e12,
            "attention_frac_of_bf16_peak":
                (F_swa + F_glob) / ((t_swa + t_glob) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "swa_tflops": swa_tflops,
            "swa_tflops_median": F_swa / (s_swa["median"] * 1e-3) / 1e12,
            "global_GBps": kv_bytes / (t_glob * 1e-3) / 1e9,
            "global_frac_of_hbm_peak": kv_bytes / (t_glob * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "global_warm_GBps": kv_bytes / (s_glob_warm["mean"] * 1e-3) / 1e9,
            "kv_append_GBps": 2 * kv_bytes / (t_app * 1e-3) / 1e9,
            "notes": "global_from_hbm follows a 1 GiB write that evicts the "
                     "MALL; global_warm_after_swa directly follows the "
                     "window pass (extra). value uses the HBM figure."}
        sha = kernel_sha(BAND_SRC)
        out["roofline"] = {
            "kernel": "band_persist_kernel (sliding-window prefill, prefill_128k)",
            "bound": "mfma", "achieved": swa_tflops, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": swa_tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic_from_profile("band_persist_prefill_128k", sha),
            "algorithmic_flop_per_launch": F_swa,
            "avg_launch_ms": t_swa, "kernel_source_sha256": sha}
        sha_g = kernel_sha(SPLIT_SRC)
        out["roofline_global"] = {
            "kernel": "split-KV output row (prefill_128k, 131072 keys), from HBM",
            "bound": "hbm", "achieved": kv_bytes / (t_glob * 1e-3) / 1e9,
            "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": kv_bytes / (t_glob * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "traffic": traffic_from_profile("splitkv_global_128k", sha_g),
            "algorithmic_bytes_per_launch": kv_bytes,
            "avg_launch_ms": t_glob, "kernel_source_sha256": sha_g}
        if "hbm_reference" in out:  # against the measured streaming read
            out["roofline_global"]["frac_of_measured_read"] = (
                out["roofline_global"]["achieved"]
                / out["hbm_reference"]["read_GBps"])
        log(f"[bench] prefill: append {t_app:.3f} ms, swa {t_swa:.3f} ms "
            f"({swa_tflops:.1f} TFLOP/s), global {t_glob:.3f} ms from HBM, "
            f"{s_glob_warm['mean']:.3f} ms warm")

    if run_decode:
        passes = [r["d"][0].elapsed_time(r["d"][-1]) for r in recs]
        per_step = [r["d"][i].elapsed_time(r["d"][i + 1])
                    for r in recs for i in range(n_dec)]
        t_dec = sum(passes) / len(passes)
        # algorithmic bytes per step: every cached K/V row read once per
        # (sequence, KV head), plus the appended row, queries and outputs
        L_sum = sum(dc.T + s + 1 for s in range(n_dec))
        kv_read = 2.0 * dc.B * dc.Hkv * dc.D * 2 * L_sum
        small = n_dec * dc.B * (4 * dc.Hq * dc.D * 2 + 2 * dc.Hkv * dc.D * 2)
        gbps = (kv_read + small) / (t_dec * 1e-3) / 1e9
        out["decode_pair"] = {
            "ms_per_step": t_dec / n_dec, "ms_256_steps": t_dec,
            "step_latency_ms": stats(per_step),
            "pass_ms": stats(passes),
            "kv_GBps": gbps, "frac_of_hbm_peak": gbps / PEAK_HBM_GBPS,
            "algorithmic_bytes_256_steps": kv_read + small,
            "notes": "each 256-step pass follows a 1 GiB write that evicts "
                     "the MALL"}
        # The decode pair is one split-KV launch per step (the merge and
        # the length bump run in the same launch).
        sha_s = kernel_sha(SPLIT_SRC)
        step_bytes = (kv_read + small) / n_dec
        out["roofline_decode"] = {
            "kernel": "splitkv_kernel (decode pair step, B=64)",
            "bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": gbps / PEAK_HBM_GBPS,
            "traffic": traffic_from_profile("splitkv_decode_b64", sha_s),
            "algorithmic_bytes_per_launch": step_bytes,
            "avg_launch_ms": t_dec / n_dec, "kernel_source_sha256": sha_s}
        if "hbm_reference" in out:
            out["roofline_decode"]["frac_of_measured_read"] = (
                gbps / out["hbm_reference"]["read_GBps"])
        log(f"[bench] decode: {t_dec / n_dec:.3f} ms/step, {gbps:.0f} GB/s")
        if not run_prefill:
            out["value"] = None

    # ---- full causal attention at the same T (speedup ratio) --------------
    if run_prefill and not args.no_causal:
        reps = 5
        lo.orthros_swa_prefill(px.q_pre, px.alpha, px.beta, kc4, vc4, o4, pc.T)
        torch.cuda.synchronize()
        evs = [ev()]
        for _ in range(reps):
            lo.orthros_swa_prefill(px.q_pre, px.alpha, px.beta, kc4, vc4, o4,
                                   pc.T)
            evs.append(ev())
        torch.cuda.synchronize()
        sc = stats([evs[i].elapsed_time(evs[i + 1]) for i in range(reps)])
        t_c = sc["mean"]
        F_c = 4.0 * pc.D * causal_pairs(pc.T) * pc.Hq * pc.B
        out["causal"] = {"ms": t_c, "timing": sc,
                         "tflops": F_c / (t_c * 1e-3) / 1e12,
                         "speedup_vs_swa": t_c / out["prefill"]["ms_swa"],
                         "speedup_vs_swa_median":
                             sc["median"] / out["prefill"]["timing"]["swa"]["median"]}
        log(f"[bench] causal {t_c:.2f} ms, speedup {t_c / out['prefill']['ms_swa']:.1f}x")

    # ---- the window the paper trains with (W = 128) at the same T ----------
    if run_prefill:
        reps, W_s = 20, 128
        lo.orthros_swa_prefill(px.q_pre, px.alpha, px.beta, kc4, vc4, o4, W_s)
        torch.cuda.synchronize()
        ts_ = []
        for _ in range(reps):
            mall_flush()
            e0 = ev()
            lo.orthros_swa_prefill(px.q_pre, px.alpha, px.beta, kc4, vc4, o4,
                                   W_s)
            e1 = ev()
            ts_.append((e0, e1))
        torch.cuda.synchronize()
        s_w = stats([a.elapsed_time(b) for a, b in ts_])
        t_s = s_w["mean"]
        # every byte of Q, O, K and V crosses HBM once
        by = 2 * 2 * pc.B * pc.T * pc.D * (pc.Hq + pc.Hkv)
        out["swa_w128"] = {
            "ms": t_s, "timing": s_w, "notes": "each launch follows a MALL flush",
            "tokens_per_s": pc.B * pc.T / (t_s * 1e-3),
            "tflops": 4.0 * pc.D * band_pairs(pc.T, W_s) * pc.Hq * pc.B
            / (t_s * 1e-3) / 1e12,
            "algorithmic_bytes": by, "gbps": by / (t_s * 1e-3) / 1e9,
            "hbm_frac": by / (t_s * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "roofline": {
                "kernel": "band_roll_kernel (sliding window W=128, prefill_128k)",
                "bound": "hbm", "achieved": by / (t_s * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": by / (t_s * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                "traffic": traffic_from_profile("band_roll_prefill_128k_w128",
                                                kernel_sha(ROLL_SRC)),
                "kernel_source_sha256": kernel_sha(ROLL_SRC)}}
        if "hbm_reference" in out:  # against the measured copy (reads+writes)
            out["swa_w128"]["roofline"]["frac_of_measured_copy"] = (
                out["swa_w128"]["gbps"] / out["hbm_reference"]["copy_GBps"])
        log(f"[bench] swa W=128: {t_s:.3f} ms, "
            f"{out['swa_w128']['gbps']:.0f} GB/s")

    # ---- the whole layer: projections + both streams + W_O (128K) -----------
    if run_prefill and not args.no_layer:
        out["layer_forward"] = layer_forward_leg(lo, pc, pc_id, kc4, vc4, dev,
                                                 ev)

    # ---- the other prefill shapes: 32K single layer, SFT dual stream -------
    if run_prefill and not args.no_other_prefills:
        out["other_prefills"] = {
            name: prefill_leg(lo, name, dev, ev, mall_flush)
            for name in ("prefill_32k", "sft_dual_8k")}

    # ---- training backward at the SFT shape (both streams) ------------------
    if run_prefill and not args.no_backward:
        out["backward_sft"] = backward_leg(lo, dev, ev)

    # ---- paged cache, ragged lengths (variable-length batched decoding) -----
    if run_decode and not args.no_paged:
        del kc3, vc3
        torch.cuda.empty_cache()
        out["decode_pair_paged_ragged"] = paged_ragged_decode(
            lo, dc, dc_id, st, a3, b3, ax3, bx3, dev, ev, mall_flush)

    # ---- CPU oracle on a bounded sample --------------------------------------
    if run_prefill and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(px, pc)

    print(json.dumps(out), flush=True)


def backward_leg(lo, dev, ev, reps=5):
    """orthros_attn_backward at the SFT dual-stream shape (B=4, T=8192,
    T_out=2048, W=1024, 32/8 heads): forward outputs from the library, unit
    upstream gradients. Algorithmic FLOPs: 8 D per (row, key) pair of either
    stream (dV = P^T dO, dP = dO V^T, dQ = dS K, dK = dS^T Q); the score
    recomputations are not counted."""
    import torch

    from workloads import normal, prefill_inputs, workload
    c, cid = workload("sft_dual_8k")
    x = prefill_inputs(c, cid, dev)
    kc = torch.empty((c.B, c.Hkv, c.T, c.D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    cl = torch.zeros(c.B, dtype=torch.int32, device=dev)
    lo.orthros_kv_append(kc, vc, cl, x.k, x.v)
    o = torch.empty_like(x.q_pre)
    ox = torch.empty_like(x.qx_pre)
    lo.orthros_swa_prefill(x.q_pre, x.alpha, x.beta, kc, vc, o, c.W)
    lo.orthros_global_xattn(x.qx_pre, x.alpha_x, x.beta_x, kc, vc, ox, c.T_in)
    d_o = normal(tuple(o.shape), 9001, torch.bfloat16, dev)
    d_ox = normal(tuple(ox.shape), 9002, torch.bfloat16, dev)
    ws = lo.workspace(lo.orthros_backward_workspace_bytes(
        c.B, c.T, c.T_out, c.Hq, c.Hkv, c.D), dev)
    g = None

    def f():
        return lo.orthros_attn_backward(x.q_pre, x.qx_pre, x.alpha, x.beta,
                                        x.alpha_x, x.beta_x, kc, vc, o, ox,
                                        d_o, d_ox, c.W, out=g, ws=ws)
    g = f()
    torch.cuda.synchronize()
    evs = [ev()]
    for _ in range(reps):
        f()
        evs.append(ev())
    torch.cuda.synchronize()
    sb = stats([evs[i].elapsed_time(evs[i + 1]) for i in range(reps)])
    t = sb["mean"]
    pairs = band_pairs(c.T, c.W) + sum(c.T_in + r + 1 for r in range(c.T_out))
    flop = 8.0 * c.D * pairs * c.Hq * c.B
    res = {"workload": c.name, "ms": t, "timing": sb,
           "tflops": flop / (t * 1e-3) / 1e12,
           "algorithmic_tflop": flop / 1e12,
           "mfma_frac": flop / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    log(f"[bench] backward {c.name}: {t:.2f} ms, {res['tflops']:.0f} TFLOP/s")
    del x, kc, vc, o, ox, d_o, d_ox, ws, g
    torch.cuda.empty_cache()
    return res


def global_pairs(T, T_out):
    """(query, key) pairs of the output stream per head: output row r sits
    at position T - T_out + r and sees every key up to it."""
    T_in = T - T_out
    return T_out * T_in + T_out * (T_out + 1) // 2


def prefill_leg(lo, name, dev, ev, flush, reps=20):
    """One prefill of workload `name` (cache fill, sliding window, output
    stream), its attention TFLOP/s and tokens/s."""
    import torch
    from workloads import prefill_inputs, workload
    c, cid = workload(name)
    x = prefill_inputs(c, cid, dev)
    kc = torch.empty((c.B, c.Hkv, c.T, c.D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    cl = torch.zeros(c.B, dtype=torch.int32, device=dev)
    o = torch.empty_like(x.q_pre)
    ox = torch.empty_like(x.qx_pre)
    ws = lo.workspace(lo.orthros_workspace_bytes(
        lo.ORTHROS_OP_GLOBAL_XATTN, c.B, c.Hq, c.Hkv, c.D, c.T_out, c.T), dev)

    def run(marks):
        cl.zero_()
        marks.append(ev())
        lo.orthros_kv_append(kc, vc, cl, x.k, x.v)
        marks.append(ev())
        lo.orthros_swa_prefill(x.q_pre, x.alpha, x.beta, kc, vc, o, c.W)
        marks.append(ev())
        if c.T_out == 1:
            flush()      # the one-row pass is memory-bound: from HBM
        marks.append(ev())
        lo.orthros_global_xattn(x.qx_pre, x.alpha_x, x.beta_x, kc, vc, ox,
                                c.T_in, ws=ws)
        marks.append(ev())
    run([])
    torch.cuda.synchronize()
    recs = []
    for _ in range(reps):
        m = []
        run(m)
        recs.append(m)
    torch.cuda.synchronize()
    legs = [stats([r[i].elapsed_time(r[i + 1]) for r in recs])
            for i in (0, 1, 3)]
    t = [g["mean"] for g in legs]
    F_swa = 4.0 * c.D * band_pairs(c.T, c.W) * c.Hq * c.B
    F_glob = 4.0 * c.D * global_pairs(c.T, c.T_out) * c.Hq * c.B
    res = {"config": f"B={c.B} Hq={c.Hq} Hkv={c.Hkv} D={c.D} T={c.T} "
                     f"W={c.W} T_out={c.T_out}",
           "ms_kv_append": t[0], "ms_swa": t[1], "ms_global": t[2],
           "timing": {"kv_append": legs[0], "swa": legs[1],
                      "global": legs[2]},
           "tokens_per_s": c.B * c.T / (sum(t) * 1e-3),
           "swa_tflops": F_swa / (t[1] * 1e-3) / 1e12,
           "global_tflops": F_glob / (t[2] * 1e-3) / 1e12,
           "attention_tflops": (F_swa + F_glob) / ((t[1] + t[2]) * 1e-3) / 1e12}
    res["attention_frac_of_bf16_peak"] = res["attention_tflops"] / PEAK_BF16_TFLOPS
    log(f"[bench] {name}: append {t[0]:.3f} ms, swa {t[1]:.3f} ms, "
        f"global {t[2]:.3f} ms, attention {res['attention_tflops']:.0f} TFLOP/s")
    del kc, vc, x
    return res


def layer_forward_leg(lo, pc, pc_id, kc, vc, dev, ev, reps=5):
    """One Orthros layer at the 128K prefill shape (d_model = Hq*D = 4096,
    one output row): hipBLASLt projections, cache fill, both attention
    streams and W_O, at the configuration's window and at W = 128."""
    import torch

    from workloads import layer_inputs
    x = layer_inputs(pc, pc_id, None, dev)
    B, M, dm = x.x.shape
    cl = torch.zeros(B, dtype=torch.int32, device=dev)
    y = torch.empty_like(x.x)
    ws = lo.workspace(lo.orthros_layer_workspace_bytes(
        B, pc.T, pc.T_out, dm, pc.Hq, pc.Hkv, pc.D), dev)
    HqD, HkvD = pc.Hq * pc.D, pc.Hkv * pc.D
    gemm_flop = 2.0 * B * (M * dm * HqD * 2 + pc.T * dm * HkvD * 2)
    res = {"d_model": dm, "gemm_tflop": gemm_flop / 1e12}
    wq, wk, wv, wo = x.stored_weights()
    for W in (pc.W, 128):
        def f():
            lo.orthros_layer_forward(x.x, wq, wk, wv, wo, x.alpha,
                                     x.beta, x.alpha_x, x.beta_x, kc, vc, cl,
                                     y, pc.T_out, W, ws=ws)
        f()
        torch.cuda.synchronize()
        evs = [ev()]
        for _ in range(reps):
            f()
            evs.append(ev())
        torch.cuda.synchronize()
        sl = stats([evs[i].elapsed_time(evs[i + 1]) for i in range(reps)])
        t = sl["mean"]
        res[f"W{W}"] = {"ms": t, "timing": sl,
                        "tokens_per_s": B * pc.T / (t * 1e-3)}
        log(f"[bench] layer W={W}: {t:.2f} ms, "
            f"{B * pc.T / (t * 1e-3) / 1e6:.2f} M tokens/s")
    lo.orthros_check_device_errors()
    del x, y, ws
    torch.cuda.empty_cache()
    return res


def paged_ragged_decode(lo, dc, dc_id, st, a, b, ax, bx, dev, ev, flush,
                        page_size=64, reps=3):
    """256 decode pair steps on a paged cache with ragged lengths: B=64
    sequences of seeded lengths uniform in [16384, 49152] (mean 32768), page
    size 64, pages of each sequence scattered over the pool by a seeded
    permutation. Timed separately from the bench step (HIP events on the
    launch stream); reports the decode-pair step time and KV GB/s over the
    algorithmic bytes of the actual lengths."""
    import torch
    from workloads import normal
    n_dec = dc.decode_steps
    g = torch.Generator().manual_seed(1000 * dc_id + 99)
    lens = torch.randint(16384, 49153, (dc.B,), generator=g).tolist()
    pages = [(n + n_dec + page_size - 1) // page_size for n in lens]
    max_pages = max(pages)
    n_pages = sum(pages)
    perm = torch.randperm(n_pages, generator=g).to(torch.int32)
    bt = torch.zeros((dc.B, max_pages), dtype=torch.int32)
    at = 0
    for bi, npg in enumerate(pages):
        bt[bi, :npg] = perm[at:at + npg]
        at += npg
    bt = bt.to(dev)
    kp = torch.empty((n_pages, dc.Hkv, page_size, dc.D), dtype=torch.bfloat16,
                     device=dev)
    vp = torch.empty_like(kp)
    # fill each sequence's first len rows (seeded N(0,1) draws, one call per
    # sequence so no append reaches past its own pages)
    cl = torch.zeros(dc.B, dtype=torch.int32, device=dev)
    for bi, n in enumerate(lens):
        kb = normal((1, n, dc.Hkv, dc.D), 1000 * dc_id + 200 + 2 * bi,
                    torch.bfloat16, dev)
        vb = normal((1, n, dc.Hkv, dc.D), 1000 * dc_id + 201 + 2 * bi,
                    torch.bfloat16, dev)
        lo.orthros_kv_append_paged(kp, vp, bt[bi:bi + 1], cl[bi:bi + 1], kb, vb)
    del kb, vb
    cl0 = torch.tensor(lens, dtype=torch.int32, device=dev)
    o = torch.empty((dc.B, dc.Hq, dc.D), dtype=torch.bfloat16, device=dev)
    ox = torch.empty_like(o)
    max_len = max(lens) + n_dec
    ws = lo.workspace(lo.orthros_workspace_bytes(
        lo.ORTHROS_OP_DECODE_PAIR, dc.B, dc.Hq, dc.Hkv, dc.D, 1, max_len), dev)

    def run():
        cl.copy_(cl0)
        flush()
        e0 = ev()
        for s in range(n_dec):
            lo.orthros_decode_pair_paged(
                st.q_pre[s], st.qx_pre[s], a, b, ax, bx, st.k_new[s],
                st.v_new[s], kp, vp, bt, cl, o, ox, max(lens) + s + 1, dc.W,
                ws=ws)
        e1 = ev()
        return e0, e1
    run()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = run()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    lo.orthros_check_device_errors()
    assert cl.tolist() == [n + n_dec for n in lens], "paged decode lengths"
    t = sum(times) / len(times)
    sp = stats(times)
    kv = sum(2.0 * dc.Hkv * dc.D * 2 * sum(n + s + 1 for s in range(n_dec))
             for n in lens)
    small = n_dec * dc.B * (4 * dc.Hq * dc.D * 2 + 2 * dc.Hkv * dc.D * 2)
    gbps = (kv + small) / (t * 1e-3) / 1e9
    log(f"[bench] paged ragged decode: {t / n_dec:.3f} ms/step, {gbps:.0f} GB/s")
    return {"ms_per_step": t / n_dec, "pass_ms": sp, "kv_GBps": gbps,
            "frac_of_hbm_peak": gbps / PEAK_HBM_GBPS, "page_size": page_size,
            "lengths": "B=64 uniform in [16384, 49152], mean "
                       f"{sum(lens) / len(lens):.0f}",
            "algorithmic_bytes_256_steps": kv + small}


def cpu_baseline(px, pc, budget_s=12.0):
    """The fp64 oracle on host cores, on a sample of the prefill_128k
    workload: the output-stream row (all heads) once, then base-stream rows
    (all heads) at evenly spread positions until `budget_s` is spent. The
    rate is scaled to the full prefill (T base rows + one output row)."""
    import numpy as np
    import torch

    import oracle

    def f64(t):
        return t.detach().to("cpu", torch.float64).numpy()

    log("[bench] cpu baseline: copying inputs")
    k, v = f64(px.k), f64(px.v)
    a, b, ax, bx = (f64(t) for t in (px.alpha, px.beta, px.alpha_x, px.beta_x))
    t0 = time.perf_counter()
    oracle.xattn(f64(px.qx_pre), ax, bx, k, v, pc.T_in)
    t_glob = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    rows, t_rows = 0, 0.0
    W = pc.W
    while t_rows < budget_s and rows < 4096:
        t = int(rng.integers(W, pc.T))
        lo_t = t - W + 1
        q = f64(px.q_pre[:, t:t + 1])
        t0 = time.perf_counter()
        oracle.xattn(q, a, b, k[:, lo_t:t + 1], v[:, lo_t:t + 1], t - lo_t)
        t_rows += time.perf_counter() - t0
        rows += 1
    est = pc.T * (t_rows / rows) + t_glob
    return {"value": pc.B * pc.T / est, "unit": "tokens/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": (f"prefill_128k: {rows} base-stream rows (W=4096, all 32 "
                       f"heads) in {t_rows:.1f} s plus the output-stream row "
                       f"(131072 keys, all heads) in {t_glob:.1f} s; scaled to "
                       f"131072 base rows + 1 output row")}


if __name__ == "__main__":
    main()
