"""Benchmark of ordered-skipping block-sparse prefill attention on one MI355X.

One step = one cosa_osk_prefill call over a whole layer (all 32 q heads, the
128K-token sequence): the longest-first schedule kernel plus the ordered-
skipping attention kernel.  Inputs (Q, the paged K/V pool, the page table and
the computation-order mask built on the GPU by cosa_build_order_mask) are
resident in HBM before the timed region.  Also timed: the same kernel with the
dense causal mask and skipping off (the dense baseline), and the mask builder.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

Prints one JSON line.  value = effective TFLOP/s on the visited blocks:
QK^T flops of every visited (q head, block) plus P V flops of the computed ones,
each 2*b*b*128 for b-token logical blocks (b = 64, or 128 for the *_b128
workload), over the median call time.  The line's "configs" object holds the same
measurements (median / p10 / p90 ms, effective TFLOP/s and its fraction of the
bf16 peak, dense-mask speedup, skip ratio, builder time) for the other four
workloads, taken in the same run.
"""
import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
OTHER_WARM_MS = 200.0          # minimum warm-up of each non-headline workload's timed calls
TILE_FLOP = 2 * 64 * 64 * 128  # one 64x64x128 contraction


def block_flop(block_size: int) -> float:
    """One b x b x 128 contraction (QK^T or P V of one visited (q head, block))."""
    return TILE_FLOP * (block_size // 64) ** 2


KAP_STRIDE = 16
# the five measured workloads; the one named by --workload is the headline, the
# others go into the JSON line's "configs" object
OTHER_WORKLOADS = ["cfg1_2k_mha", "cfg2_16k_gqa", "cfg3_32k_structured", "cfg4_128k_structured",
                   "cfg5_paged_2seq"]
KERNEL_SOURCES = ["block_sparse_long_osk_amd/csrc/osk_prefill.hip", "block_sparse_long_osk_amd/csrc/osk_internal.h"]
# FETCH_SIZE / WRITE_SIZE summaries per workload (used while the kernel sources are unchanged)
TRAFFIC_FILES = {
    "cfg4_128k_structured": os.path.join(ROOT, "profiles", "osk_prefill_cfg4_128k_traffic.json"),
    "cfg4_128k_structured_b128": os.path.join(ROOT, "profiles", "osk_prefill_b128_cfg4_128k_traffic.json"),
}


def kernel_source_hash():
    """Hash of the kernel sources' code: comments and blank space are left out, so that
    only a change of the code itself invalidates the stored counter summaries."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def time_calls(fn, steps, warmup, warm_ms=0.0):
    """Per-call durations (ms) from HIP events on the current stream, plus the
    wall time of the whole timed region bracketed by synchronizations.  Before the
    timed calls: `warmup` untimed calls, and more until at least `warm_ms` of wall time
    has gone by (the GPU clock needs some tens of ms of back-to-back load to settle)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < warmup or (time.perf_counter() - t0) * 1e3 < warm_ms:
        fn()
        n += 1
        if warm_ms > 0 and n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    per = [a.elapsed_time(b) for a, b in evs]
    return per, wall


def calib_mode():
    """The MFMA calibration kernel with constant operands and with data-like random bf16 operands,
    in short (4096-round, a few ms) and long (114,688-round, ~0.1 s) calls: rate and the clock it
    implies at one 32x32x16 MFMA per 32 cycles on each of the 1024 SIMDs.  Under rocprofv3 --pmc
    GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES show whether a difference is the clock or the
    MFMA issue rate."""
    import ctypes
    import torch
    L = ctypes.CDLL(os.path.join(ROOT, "block_sparse_long_osk_amd", "libcosa_calib.so"))
    L.cosa_calib_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    L.cosa_calib_mfma_bf16.restype = ctypes.c_int32
    L.cosa_calib_mfma_bf16_data.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32,
                                            ctypes.c_void_p]
    L.cosa_calib_mfma_bf16_data.restype = ctypes.c_int32
    L.cosa_calib_mfma_bf16_flop.argtypes = [ctypes.c_int32, ctypes.c_int32]
    L.cosa_calib_mfma_bf16_flop.restype = ctypes.c_double
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nwg = 256 * 8
    out = torch.empty(nwg * 4, dtype=torch.float32, device="cuda")
    res = {"mode": "calib", "workgroups": nwg, "cases": []}
    for kind, iters, warm in (("constant", 4096, 2), ("data", 4096, 2), ("constant", 4096 * 28, 3),
                              ("data", 4096 * 28, 3)):
        def f():
            if kind == "constant":
                rc = L.cosa_calib_mfma_bf16(ctypes.c_void_p(out.data_ptr()), nwg, iters, stream)
            else:
                rc = L.cosa_calib_mfma_bf16_data(ctypes.c_void_p(out.data_ptr()), nwg, iters, 12345, stream)
            if rc != 0:
                raise RuntimeError("calibration launch failed")
        per, _ = time_calls(f, 5, warm)
        tf = L.cosa_calib_mfma_bf16_flop(nwg, iters) / (statistics.median(per) * 1e-3) / 1e12
        res["cases"].append({"operands": kind, "rounds": iters, "ms_median": statistics.median(per),
                             "tflops": tf, "implied_clock_ghz": tf * 1e12 / (1024 * 1024) / 1e9})
        print(f"[bench] calib {kind} {iters}: {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
    return res


def calibrate():
    """Attainable bf16 MFMA rate (independent 32x32x16 MFMA chains on every SIMD) and
    HBM streaming-read rate (2 GiB, 16-byte loads) on this device, from the
    measurement-only kernels of libcosa_calib.so, timed with events."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "block_sparse_long_osk_amd", "libcosa_calib.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m block_sparse_long_osk_amd.build`")
    L = ctypes.CDLL(path)
    L.cosa_calib_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    L.cosa_calib_mfma_bf16.restype = ctypes.c_int32
    L.cosa_calib_mfma_bf16_flop.argtypes = [ctypes.c_int32, ctypes.c_int32]
    L.cosa_calib_mfma_bf16_flop.restype = ctypes.c_double
    L.cosa_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    L.cosa_calib_read.restype = ctypes.c_int32
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nwg, iters = 256 * 8, 4096
    out = torch.empty(nwg * 4, dtype=torch.float32, device="cuda")

    def mfma():
        if L.cosa_calib_mfma_bf16(ctypes.c_void_p(out.data_ptr()), nwg, iters, stream) != 0:
            raise RuntimeError("cosa_calib_mfma_bf16 failed")
    per, _ = time_calls(mfma, 5, 2)
    mfma_tflops = L.cosa_calib_mfma_bf16_flop(nwg, iters) / (statistics.median(per) * 1e-3) / 1e12
    # sustained: data-like operands, ~100 ms per call after ~0.3 s of the same load, so the
    # clock is the one power management settles on
    L.cosa_calib_mfma_bf16_data.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32,
                                            ctypes.c_void_p]
    L.cosa_calib_mfma_bf16_data.restype = ctypes.c_int32
    long_iters = 4096 * 28

    def mfma_data():
        if L.cosa_calib_mfma_bf16_data(ctypes.c_void_p(out.data_ptr()), nwg, long_iters, 12345, stream) != 0:
            raise RuntimeError("cosa_calib_mfma_bf16_data failed")
    per, _ = time_calls(mfma_data, 5, 3)
    sustained_tflops = L.cosa_calib_mfma_bf16_flop(nwg, long_iters) / (statistics.median(per) * 1e-3) / 1e12
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    rwg = 256 * 16
    rout = torch.empty(rwg, dtype=torch.int32, device="cuda")

    def read():
        if L.cosa_calib_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(rout.data_ptr()), rwg,
                             stream) != 0:
            raise RuntimeError("cosa_calib_read failed")
    per, _ = time_calls(read, 5, 2)
    read_gbs = nbytes / (statistics.median(per) * 1e-3) / 1e9
    del buf, rout, out
    return {"mfma_bf16_tflops": mfma_tflops, "hbm_read_gbs": read_gbs,
            "mfma_bf16_tflops_sustained": sustained_tflops,
            # 1024 flop per clock per SIMD (one 32x32x16 MFMA per 32 cycles), 1024 SIMDs
            "mfma_clock_ghz_sustained": sustained_tflops * 1e12 / (1024 * 1024) / 1e9,
            "how": "independent v_mfma_f32_32x32x16_bf16 chains, 2048 workgroups x 4 waves (burst: 4096 "
                   "rounds on constant operands; sustained: 114,688 rounds, ~0.1 s per call, on data-like "
                   "random bf16 operands, after 3 such calls); 2 GiB streaming read with 16-byte loads "
                   "(libcosa_calib.so)"}


def pct(xs, p):
    xs = sorted(xs)
    k = (len(xs) - 1) * p
    lo, hi = math.floor(k), math.ceil(k)
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


def cpu_baseline(batch, wl, delta, budget_s=15.0):
    """The fp64 oracle as it stands, timed on a bounded random sample of query
    blocks (all KV heads of each), scaled to effective TFLOP/s."""
    from block_sparse_long_osk_amd import inputs
    from oracle import maskref, osk
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        blas_threads = 1
    from oracle import paging
    q = inputs.bf16_bits_to_f32(batch.q)
    k = inputs.bf16_bits_to_f32(batch.k_pool)
    v = inputs.bf16_bits_to_f32(batch.v_pool)
    B, pt = batch.block_size, batch.page_table
    if k.shape[2] != B:   # the oracle's pools at the logical block size
        k, v, pt = paging.logical_view(k, v, pt, batch.cu_seqlens, k.shape[2], block=B)
    t_mask = time.perf_counter()
    om, ml = maskref.build_order_mask(q, k, pt, batch.cu_seqlens, wl.num_kv_heads, wl.budget1, page_size=B)
    t_mask = time.perf_counter() - t_mask
    rng = np.random.default_rng(0)
    order = rng.permutation(batch.total_qblocks)
    flops = 0.0
    spent = 0.0
    n_blocks = 0
    for qb in order:
        units = [(int(qb), g) for g in range(wl.num_kv_heads)]
        t = time.perf_counter()
        res = osk.osk_reference(q, k, v, pt, batch.cu_seqlens, om, ml, delta, page_size=B, units=units)
        spent += time.perf_counter() - t
        d = res["decisions"][qb]
        flops += block_flop(B) * (float((d != 2).sum()) + float((d == 0).sum()))
        n_blocks += 1
        if spent >= budget_s:
            break
    rate = flops / spent / 1e12
    return {"value": rate, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{n_blocks} random query blocks x {wl.num_kv_heads} KV heads of {wl.name} "
                      f"(mask rows from the CPU reference builder, {t_mask:.1f} s, not timed)",
            "seconds": round(spent, 2)}


def skip_sweep(args, wl, db, om, ml, mask_kind="proxy", budget1=None):
    """Skip ratio and ms per call against Delta for two visit orders of the same page sets:
    the mask's own order (the mean-pooled proxy's score-descending order, or KAP's
    HRM-first order) and ascending page id.  tau = ln(Delta / L) is swept over a fixed
    grid; the pages' own Delta = 500, 2000 and 3000 are included.  Ends with the tau at
    which each order reaches a 52 % skip ratio."""
    rows = []
    import numpy as np
    import torch
    from block_sparse_long_osk_amd import runner
    width = om.shape[2]
    om_h = om.cpu().numpy()
    ml_h = ml.cpu().numpy()
    asc = om_h.copy()
    for idx in np.ndindex(ml_h.shape):
        n = int(ml_h[idx])
        asc[idx][:n] = np.sort(asc[idx][:n])
    orders = {mask_kind: (om, ml), "ascending": runner.upload_mask(asc, ml_h)}
    L = max(wl.seq_lens)
    deltas = [("tau", float(L * np.exp(t)), t) for t in (-1.0, -0.5, -0.3, -0.2, -0.15, -0.1, -0.05, -0.02, 0.0)]
    # the pages' own operating points (CoSA App. D.4: Delta = 500 with the remapped order,
    # about 3000 without it, for a similar skip ratio; Delta = 2000 in the main results)
    for d in (500.0, 2000.0, 3000.0):
        deltas.append(("pages_delta", d, float(np.log(d / L))))
    outs = runner.allocate_outputs(db, width, log=False)
    outs.lse = None
    ws = runner.workspace_for(db, width)
    for kind, delta, tau in deltas:
        row = {"mode": "skip-sweep", "mask": mask_kind, "workload": wl.name, "delta": delta,
               "tau_at_longest_seq": tau, "kind": kind}
        for name, (m, mlen) in orders.items():
            logged = runner.prefill(db, m, mlen, delta, log=True)
            torch.cuda.synchronize()
            dec = logged.decisions
            visited = int((dec != 2).sum().item())
            skipped = int((dec == 1).sum().item())
            del logged, dec
            per, _ = time_calls(lambda: runner.prefill(db, m, mlen, delta, outputs=outs, workspace=ws), 5, 2)
            row[name] = {"skip_ratio": skipped / max(visited, 1), "ms_per_layer": statistics.median(per)}
        row["budget1"] = budget1
        rows.append(row)
        print(json.dumps(row), flush=True)
    # tau at which each visit order reaches a 52 % skip ratio (linear interpolation over the
    # tau grid), the pages' reference level for the remapped order
    grid = sorted((r for r in rows if r["kind"] == "tau"), key=lambda r: r["tau_at_longest_seq"])
    summary = {"mode": "skip-sweep-summary", "mask": mask_kind, "workload": wl.name, "budget1": budget1,
               "target_skip": 0.52}
    for name in orders:
        hit = None
        for r0, r1 in zip(grid, grid[1:]):
            s0, s1 = r0[name]["skip_ratio"], r1[name]["skip_ratio"]
            if s0 < 0.52 <= s1:
                t0, t1 = r0["tau_at_longest_seq"], r1["tau_at_longest_seq"]
                hit = t0 + (0.52 - s0) / (s1 - s0) * (t1 - t0)
                break
        summary[name] = None if hit is None else {"tau": hit, "delta": float(L * np.exp(hit))}
    print(json.dumps(summary), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--dense-steps", type=int, default=3)
    ap.add_argument("--workload", default="cfg4_128k_structured")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="measure the --workload only, not the other four workloads")
    ap.add_argument("--other-steps", type=int, default=20,
                    help="timed calls for each of the other workloads (after at least 3 warm-up calls "
                         "and %d ms of them)" % OTHER_WARM_MS)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--budget1", default=None,
                    help="skip-sweep: comma-separated first-stage budgets to sweep (default: the workload's)")
    ap.add_argument("--mask", choices=["proxy", "kap", "union"], default="proxy",
                    help="skip-sweep: sweep with the mean-pooled proxy masks or with KAP masks (stride 16, "
                         "the workload's budget as the fixed fraction)")
    ap.add_argument("--mode", choices=["bench", "counters", "skip-sweep", "calib"], default="bench",
                    help="counters: a plain 1 GiB device copy (the counter scale reference), then "
                         "--steps OSK calls; for rocprofv3 --pmc passes.  skip-sweep: in-kernel skip "
                         "ratio and time per call against Delta, with the proxy's visit order and with "
                         "every mask row sorted ascending (one JSON line per Delta).  calib: the MFMA "
                         "calibration kernel on constant and on data-like operands, short and long "
                         "calls (one JSON line; no workload)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the kernel shards by KV head or by "
              "query-block range without exchange inside a layer, but this library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.mode == "calib":
        print(json.dumps(calib_mode()))
        return
    from block_sparse_long_osk_amd import binding, inputs, runner
    binding.lib()
    wl = inputs.WORKLOADS[args.workload]
    delta = inputs.skip_scale(args.workload)
    print(f"[bench] generating {wl.name}", file=sys.stderr, flush=True)
    batch = inputs.generate(wl)
    db = runner.upload(batch)
    torch.cuda.synchronize()

    # ---- computation-order mask on the GPU (timed separately)
    om, ml = runner.build_mask(db, wl.budget1)
    if args.mode == "counters":
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)                                                  # plain copy: reads and writes 1 GiB
        torch.cuda.synchronize()
        del src, dst
        for _ in range(args.steps):
            runner.prefill(db, om, ml, delta)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "counters", "workload": wl.name, "copy_bytes": 1 << 30,
                          "osk_calls": args.steps, "kernel_source_hash": kernel_source_hash()}))
        return
    if args.mode == "skip-sweep":
        budgets = [float(x) for x in args.budget1.split(",")] if args.budget1 else [wl.budget1]
        for b1 in budgets:
            if args.mask == "kap":
                om, ml = runner.build_kap_mask(db, KAP_STRIDE, binding.COSA_KAP_FRACTION, b1)
            else:
                om, ml = runner.build_mask(db, b1)
            skip_sweep(args, wl, db, om, ml, args.mask, b1)
            del om, ml
            torch.cuda.empty_cache()
        return
    rec = measure(args, wl, batch, db, om, ml, delta, headline=True)
    # the other workloads, each measured the same way in this run (the headline's
    # attainable rates, CPU baseline and KAP builder are not repeated)
    if args.mask == "proxy" and not args.headline_only:
        del db, om, ml
        torch.cuda.empty_cache()
        others = {}
        for name in OTHER_WORKLOADS:
            if name == wl.name:
                continue
            owl = inputs.WORKLOADS[name]
            print(f"[bench] generating {name}", file=sys.stderr, flush=True)
            obatch = inputs.generate(owl)
            odb = runner.upload(obatch)
            oom, oml = runner.build_mask(odb, owl.budget1)
            torch.cuda.synchronize()
            others[name] = measure(args, owl, obatch, odb, oom, oml, inputs.skip_scale(name), headline=False)
            del odb, oom, oml, obatch
            torch.cuda.empty_cache()
        rec["configs"] = others
    print(json.dumps(rec), flush=True)


def measure(args, wl, batch, db, om, ml, delta, headline):
    """Times one workload: the prefill over its built mask (median, p10, p90 of
    per-call HIP-event times), the dense-mask baseline and the mask builder; for the
    headline also the KAP builder, the attainable rates, the roofline and the CPU
    baseline.  Returns the record (the JSON line's body for the headline)."""
    import torch
    from block_sparse_long_osk_amd import binding, runner
    # the headline takes exactly --warmup untimed calls; the other workloads, whose calls
    # are short, are also warmed for OTHER_WARM_MS so their timed calls run at a settled clock
    steps, warmup = (args.steps, args.warmup) if headline else (args.other_steps, 3)
    warm_ms = 0.0 if headline else OTHER_WARM_MS
    # the timed prefill's mask: the mean-pooled proxy (default), KAP at the workload's budget
    # as the fixed fraction, or per-q-head sets as union rows with membership
    membership = None
    reuse = None
    if args.mask == "kap":
        om, ml = runner.build_kap_mask(db, KAP_STRIDE, binding.COSA_KAP_FRACTION, wl.budget1)
    elif args.mask == "union":
        om, ml, membership, head_len = runner.build_union_mask(db, wl.budget1)
        reuse = float(head_len.sum().item()) / float(ml.sum().item())
    width = om.shape[2]
    if args.mask == "union":
        ws_b = torch.empty(binding.cosa_build_union_mask_workspace_bytes(db.dims(width)), dtype=torch.uint8,
                           device="cuda")
        builder_ms, _ = time_calls(lambda: runner.build_union_mask(db, wl.budget1, workspace=ws_b), 5, 2)
    else:
        wb = binding.cosa_order_mask_width(db.max_blocks, wl.budget1)
        ws_b = torch.empty(binding.cosa_build_order_mask_workspace_bytes(db.dims(wb)), dtype=torch.uint8,
                           device="cuda")
        builder_ms, _ = time_calls(lambda: runner.build_mask(db, wl.budget1, workspace=ws_b), 5, 2)
    del ws_b
    kap_ms = None
    if headline and db.num_q_heads // db.num_kv_heads * (db.block_size // KAP_STRIDE) <= 32:
        # the KAP builder (CoSA section 4.2): stride 16, fixed fraction = the workload's budget, and Top-p 0.95
        kw = binding.cosa_kap_mask_width(db.max_blocks, binding.COSA_KAP_TOP_P, 0.95)
        ws_k = torch.empty(binding.cosa_build_kap_mask_workspace_bytes(db.dims(kw)), dtype=torch.uint8, device="cuda")
        kf, _ = time_calls(lambda: runner.build_kap_mask(db, KAP_STRIDE, binding.COSA_KAP_FRACTION, wl.budget1,
                                                         workspace=ws_k), 5, 2)
        kp, _ = time_calls(lambda: runner.build_kap_mask(db, KAP_STRIDE, binding.COSA_KAP_TOP_P, 0.95,
                                                         workspace=ws_k), 5, 2)
        kap_ms = {"stride": KAP_STRIDE, "fraction_ms": statistics.median(kf), "top_p_0.95_ms": statistics.median(kp)}
        del ws_k

    # ---- one logged (untimed) call: visited / computed counts for the flop count
    logged = runner.prefill(db, om, ml, delta, log=True, membership=membership)
    torch.cuda.synchronize()
    dec = logged.decisions
    visited = int((dec != 2).sum().item())
    computed = int((dec == 0).sum().item())
    # (query block, KV head, entry) visits where every q head of the group skips: their
    # V tile is gathered but no head reads it
    G = db.num_q_heads // db.num_kv_heads
    d4 = dec.view(dec.shape[0], db.num_kv_heads, G, dec.shape[2])
    kv_visits = int((d4 != 2).any(dim=2).sum().item())
    all_skip = int((d4 == 1).all(dim=2).sum().item())
    del logged, dec, d4
    B = db.block_size
    flop = block_flop(B) * (visited + computed)
    nb = [-(-L // B) for L in db.seq_lens]
    causal = sum(n * (n + 1) // 2 for n in nb) * db.num_q_heads  # (q head, block) pairs j <= i

    # ---- timed OSK calls (no logging)
    outs = runner.allocate_outputs(db, width, log=False)
    outs.lse = None
    ws = runner.workspace_for(db, width)
    step = lambda: runner.prefill(db, om, ml, delta, outputs=outs, workspace=ws, membership=membership)
    print(f"[bench] {wl.name}: timing {steps} steps", file=sys.stderr, flush=True)
    per, wall = time_calls(step, steps, warmup, warm_ms)
    med = statistics.median(per)
    ms_per_step = wall / steps
    aborts = runner.abort_count(db, ws, width)
    if aborts:
        print(f"[bench] {aborts} workgroups reported aborted inter-wave waits", file=sys.stderr)
    tflops = flop / (med * 1e-3) / 1e12
    del outs, ws

    # ---- dense-mask baseline: same kernel, every causal page, skipping off
    dense = None
    if not args.no_dense:
        dom, dml = runner.dense_mask(db)
        d_visited = int(dml.sum().item()) * (db.num_q_heads // db.num_kv_heads)
        d_flop = 2 * block_flop(B) * d_visited
        douts = runner.allocate_outputs(db, dom.shape[2], log=False)
        douts.lse = None
        dws = runner.workspace_for(db, dom.shape[2])
        print(f"[bench] {wl.name}: timing dense baseline", file=sys.stderr, flush=True)
        dper, _ = time_calls(lambda: runner.prefill(db, dom, dml, -1.0, outputs=douts, workspace=dws),
                             args.dense_steps, 1, warm_ms)
        dmed = statistics.median(dper)
        dense = {"ms_per_layer": dmed, "tflops": d_flop / (dmed * 1e-3) / 1e12,
                 "frac_of_peak": d_flop / (dmed * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                 "visited_q_head_pages": d_visited, "algorithmic_tflop": d_flop / 1e12}
        del douts, dom, dml, dws

    kv_bytes = 2 * B * 128 * 2 * kv_visits
    common = {
        "ms_per_layer_median": med, "ms_p10": pct(per, 0.1), "ms_p90": pct(per, 0.9),
        "effective_tflops": tflops, "frac_of_peak": tflops / PEAK_BF16_TFLOPS,
        "visited_q_head_pages": visited, "computed_q_head_pages": computed,
        "skip_ratio": 1.0 - computed / max(visited, 1), "algorithmic_tflop": flop / 1e12,
        # against every causal (q head, block) pair: the first stage's realized budget and the
        # share left after both stages
        "realized_stage1_budget": visited / max(causal, 1), "computed_fraction": computed / max(causal, 1),
        "all_heads_skip_fraction": all_skip / max(kv_visits, 1),
        "speedup_vs_dense": (dense["ms_per_layer"] / med) if dense else None,
        "dense": dense, "mask_builder_ms": statistics.median(builder_ms),
        "osk_plus_builder_ms": med + statistics.median(builder_ms),
        "skip_scale_delta": delta, "aborted_workgroups": aborts,
    }
    if not headline:
        common.update({"steps": steps, "warmup": warmup, "seq_lens": list(wl.seq_lens),
                       "note": "latency-bound correctness case (32 workgroups): no roofline claim"
                               if wl.num_q_heads == 1 else None})
        return common

    # ---- attainable rates on this device (measurement-only kernels)
    print(f"[bench] calibrating MFMA and HBM rates", file=sys.stderr, flush=True)
    attain = calibrate()
    if dense:
        dense["frac_of_attainable"] = dense["tflops"] / attain["mfma_bf16_tflops"]
        dense["frac_of_sustained_mfma"] = dense["tflops"] / attain["mfma_bf16_tflops_sustained"]

    # ---- roofline of the dominant kernel
    traffic = None
    tfile = TRAFFIC_FILES.get(wl.name) if args.mask == "proxy" else None  # counters taken with the proxy mask
    if tfile and os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("workload") == wl.name and tr.get("kernel_source_hash") == kernel_source_hash():
            traffic = tr.get("bytes_per_launch")
    roofline = {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                "frac_of_attainable": tflops / attain["mfma_bf16_tflops"],
                "frac_of_sustained_mfma": tflops / attain["mfma_bf16_tflops_sustained"],
                "kernel": ("osk_prefill_ring_kernel<4>" if B == 64 else "osk_prefill_b128_kernel<2>")
                          + " (+ schedule kernel, 0.2% of the call)",
                "algorithmic_flop_per_launch": flop,
                # K and V tiles of every (query block, KV head) visit, as requested from the
                # memory hierarchy (most are served by the L2s): not an HBM figure
                "kv_gather_logical_gbs": kv_bytes / (med * 1e-3) / 1e9,
                # bytes past the L2s (FETCH_SIZE + WRITE_SIZE, scaled; includes reads the
                # last-level cache serves) per launch over the median launch time
                "hbm_gbs_from_counters": (traffic / (med * 1e-3) / 1e9) if traffic else None,
                "hbm_frac_from_counters": (traffic / (med * 1e-3) / 1e9 / PEAK_HBM_GBS) if traffic else None}

    cpu = None
    if not args.no_cpu:
        print(f"[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(batch, wl, delta)
        cpu["ms_per_layer_extrapolated"] = flop / (cpu["value"] * 1e12) * 1e3

    rec = {
        "metric": "OSK prefill ms/layer + effective TFLOP/s at 128K; speedup vs dense-mask",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded structured generator; no dataset or model weights)",
        "config": {"workload": wl.name, "seq_len": wl.seq_lens[0] if len(wl.seq_lens) == 1 else list(wl.seq_lens),
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads, "head_dim": 128,
                   "page_size": int(batch.k_pool.shape[2]), "block_size": B, "budget1": wl.budget1,
                   "skip_scale_delta": delta, "mask": args.mask},
    }
    rec.update(common)
    rec.update({"kap_builder": kap_ms, "reuse_ratio": reuse, "roofline": roofline, "attainable": attain,
                "cpu_baseline": cpu})
    return rec


if __name__ == "__main__":
    main()
