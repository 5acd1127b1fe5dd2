"""Benchmark of the HyperAttention forward on one MI355X.

One step = one non-causal forward plus one causal forward (min_seq_len
4096) of a single attention layer at n = 131072: batch 1, 32 heads, d = 64,
bf16, block 256, 256 sampled columns, 7 hash bits, planted large entries
(1% of key rows are noisy copies of query rows).  Inputs are generated on
the GPU before timing and stay resident.

Prints one JSON line.  ``value`` is the effective throughput of the step:
algorithmic FLOPs (4 d B H n (b + m) per non-causal pass; for the causal
pass the same per level over n/2 query rows plus 4 d B H (n/s) s(s+1)/2 for
the exact leaves) divided by the measured step time; the timed steps run
with no per-launch instrumentation.  ``roofline`` is taken for the kernel
class with the largest share of the step, timed by HIP events that the
library records around each of its launches on the launch stream, over a
second run of the same number of steps.  ``cpu_baseline`` times the CPU
oracle on two of the 32 heads of the same workload (both passes) and
scales it to the same unit.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
MFMA_FP32_PEAK_TFLOPS = 157.3


def alg_flops(w, causal):
    """Algorithmic FLOPs of one forward (the work the method must do)."""
    d, BH, n, m = w.d, w.batch * w.heads, w.n, w.samples
    if not causal:
        b = min(w.block, n)
        return 4.0 * d * BH * n * (b + m), {"attend": 4.0 * d * BH * n * (b + m)}
    s = w.min_seq_len
    ns, levels = n, []
    while ns > s:
        ns //= 2
        levels.append(ns)
    leaf = ns
    quad = sum(4.0 * d * BH * (n / 2) * (min(w.block, seg) + m) for seg in levels)
    leaves = 4.0 * d * BH * (n / leaf) * leaf * (leaf + 1) / 2
    return quad + leaves, {"quadrant": quad, "leaf": leaves}


def alg_bytes(w, causal):
    """Algorithmic HBM bytes per kernel class for one forward: every input
    row the kernel needs read once, every output written once, the causal
    accumulator read and written once per merge (fp32 values + lse)."""
    e = 2 if str(w.dtype).endswith("bfloat16") else 4
    BH, BK, n, d = w.batch * w.heads, w.batch * w.kv_heads, w.n, w.d
    row, acc = d * e, d * 4 + 4
    out = {"hash": (BH + BK) * n * (d * e + 2)}
    if not causal:
        out["sort"] = (BH + BK) * n * (2 + 2 + 4)          # hist read, scatter read, perm write
        out["attend"] = (BH * n * (row + 4 + 4)             # Q row, its perm entry, lse
                         + BK * n * (2 * row + 4)           # K and V rows, perm entry
                         + BH * n * row)                    # output row
        return out
    L, ns = 0, n
    while ns > w.min_seq_len:
        ns //= 2
        L += 1
    out["sort"] = L * (BH + BK) * (n // 2) * (2 + 2 + 4)
    half = n // 2
    out["quadrant"] = L * (BH * half * (row + 4 + 2 * acc)  # Q row, perm, accumulator read + write
                           + BK * half * (2 * row + 4))    # K and V rows, perm
    out["leaf"] = BH * n * row + 2 * BK * n * row + BH * n * acc
    return out


CPU_HEADS = 2      # heads of the bounded oracle sample (about 10-20 s of CPU work)


def rep_times(torch, stream, fn, reps):
    """ms of each of `reps` calls of fn, from an event pair per call on `stream`,
    and their mean, median, p10 and p90."""
    import numpy as np
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    return {"mean": float(ms.mean()), "median": float(np.median(ms)), "p10": float(np.percentile(ms, 10)),
            "p90": float(np.percentile(ms, 90)), "reps": reps}


def gpu_sample(ha, torch, w_nc, w_c, q, k, v, ws, nh):
    """What the library computes on the first nh heads of the benchmark's
    inputs (outside any timed region): each pass's out and lse, the bucket
    ranks of the Q and K rows, the non-causal whole-head permutations and
    sample positions; host numpy arrays for the comparison with the oracle."""
    import numpy as np
    res = {}
    for name, w in (("noncausal", w_nc), ("causal", w_c)):
        out, lse = ha.forward(q, k, v, workspace=ws, **w.method_args())
        res[name] = (out[:, :nh].float().cpu().numpy(), lse[:, :nh].cpu().numpy())
        del out, lse
    R = ha.projections(w_nc.seed, w_nc.d, w_nc.proj_bits, q.device)
    rq = ha.hash_rows(q[0, :nh].contiguous(), R)
    rk = ha.hash_rows(k[0, :nh].contiguous(), R)
    res["rank_q"], res["rank_k"] = rq.cpu().numpy().astype(np.uint32), rk.cpu().numpy().astype(np.uint32)
    res["perm_q"] = ha.sort_ranks(rq, w_nc.proj_bits).cpu().numpy()[:, 0]
    res["perm_k"] = ha.sort_ranks(rk, w_nc.proj_bits).cpu().numpy()[:, 0]
    res["samples"] = ha.sample_indices(w_nc.seed, 1, nh, w_nc.n, w_nc.samples, device=q.device).cpu().numpy()[0, :, 0]
    torch.cuda.synchronize()
    return res


def oracle_parity(gpu, refs, w_nc, qh, kh, nh):
    """The library's results on the oracle sample's heads (gpu_sample)
    against the oracle's (refs: out and lse per pass): output and lse
    errors, and mismatch counts of ranks, permutations and samples."""
    import numpy as np
    import oracle
    if "error" in gpu:
        return {"error": gpu["error"]}
    parity = {"heads": nh}
    for name, (o_ref, l_ref) in refs.items():
        o_gpu, l_gpu = gpu[name]
        both_inf = np.isneginf(l_gpu) & np.isneginf(l_ref)
        parity[name] = {"out_max_abs": float(np.abs(o_gpu - o_ref).max()),
                        "out_rel_fro": float(np.linalg.norm(o_gpu - o_ref) / np.linalg.norm(o_ref)),
                        "lse_max_abs": float(np.where(both_inf, 0.0, np.abs(l_gpu - l_ref)).max())}
    R = oracle.projections(w_nc.seed, w_nc.d, w_nc.proj_bits)
    mism = {"rank": 0, "perm": 0, "sample": 0}
    for h in range(nh):
        for x, key in ((qh, "q"), (kh, "k")):
            rk = oracle.ranks(x[0, h], R)
            mism["rank"] += int(np.count_nonzero(gpu["rank_" + key][h] != rk))
            mism["perm"] += int(np.count_nonzero(gpu["perm_" + key][h] != oracle.sort_perm(rk)))
        ref_s = oracle.sample_positions(w_nc.seed, 0, h, 1, w_nc.n, w_nc.samples)
        mism["sample"] += int(np.count_nonzero(gpu["samples"][h] != ref_s))
    parity["mismatches"] = mism
    parity["compared"] = {"rank": 2 * nh * w_nc.n, "perm": 2 * nh * w_nc.n, "sample": nh * w_nc.samples}
    return parity


def cpu_baseline(w_nc, w_c, q, k, v, gpu=None):
    """Time the oracle on the first CPU_HEADS heads of both passes; returns
    the baseline dict.  With `gpu` (gpu_sample's arrays for the same heads)
    the dict also carries the library's agreement with that oracle run:
    output and lse errors per pass, and mismatch counts of ranks,
    permutations and sample positions (expected zero: the library computes
    these bit-exactly)."""
    import numpy as np
    import oracle
    from oracle.hyperattn import HAConfig
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    nh = min(CPU_HEADS, q.shape[1], k.shape[1])
    qh = q[:, :nh].float().cpu().numpy()
    kh = k[:, :nh].float().cpu().numpy()
    vh = v[:, :nh].float().cpu().numpy()
    flops = 0.0
    refs = {}
    t0 = time.perf_counter()
    for name, w in (("noncausal", w_nc), ("causal", w_c)):
        cfg = HAConfig(block=w.block, samples=w.samples, proj_bits=w.proj_bits, causal=w.causal,
                       min_seq_len=w.min_seq_len, seed=w.seed)
        refs[name] = oracle.forward(qh, kh, vh, cfg)
        f, _ = alg_flops(w.with_(heads=nh, kv_heads=nh), w.causal)
        flops += f
    dt = time.perf_counter() - t0
    parity = None
    if gpu is not None:
        try:
            parity = oracle_parity(gpu, refs, w_nc, qh, kh, nh)
        except Exception as e:              # the parity record is context; never lose the bench line to it
            parity = {"error": repr(e)}
    # the whole fp32 n = 1024 configuration as well (well under a second)
    from approximate_long_context_amd.workloads import WORKLOADS, make_inputs
    ws = WORKLOADS["small"]
    qs, ks, vs = (t.numpy() for t in make_inputs(ws, "cpu"))
    t1 = time.perf_counter()
    oracle.forward(qs, ks, vs, HAConfig(block=ws.block, samples=ws.samples, proj_bits=ws.proj_bits,
                                        causal=ws.causal, min_seq_len=ws.min_seq_len, seed=ws.seed))
    dt_small = time.perf_counter() - t1
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"heads 0..{nh - 1} of {w_nc.heads}, all {w_nc.n} rows, non-causal + causal passes, fp64 numpy; "
                      f"{dt:.1f} s on {os.cpu_count()} host CPUs", "seconds": dt,
            "configs_ms": {"small": dt_small * 1e3}, "parity": parity}


def traffic_record(kernel_class):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/
    traffic_long131k.json), if they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic_long131k.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    entry = rec.get("kernels", {}).get(kernel_class)
    if entry is None:
        return None
    src = "ha_hash.hip" if kernel_class == "hash" else "ha_sort.hip" if kernel_class == "sort" else "ha_attn.hip"
    sha = hashlib.sha256(open(os.path.join(ROOT, "approximate_long_context_amd", "csrc", src), "rb").read()).hexdigest()
    if entry.get("source_sha256") != sha:
        return None
    return entry.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other configurations and the error against exact attention")
    ap.add_argument("--workload", default="long131k")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run 5 device-to-device copies of MIB MiB (known HBM traffic) "
                         "to calibrate hardware byte counters")
    ap.add_argument("--gather-calibration", type=int, default=0, metavar="MIB",
                    help="also run 5 permutation gathers (hyperattn_gather) of MIB MiB of rows through a "
                         "random permutation: known HBM traffic with the row-wise access pattern of the "
                         "attention kernels, to check the byte-counter calibration")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); each head is an independent "
              "problem, so more GPUs would split the heads with no communication.", file=sys.stderr)
        sys.exit(2)

    import torch
    import approximate_long_context_amd as ha
    from approximate_long_context_amd.workloads import WORKLOADS, make_inputs

    dev = torch.device("cuda:0")
    w_nc = WORKLOADS[args.workload]
    w_c = WORKLOADS.get(args.workload + "_causal", w_nc.with_(causal=True))
    q, k, v = make_inputs(w_nc, dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    wsb = max(ha.workspace_bytes(w.batch, w.n, w.d, w.heads, w.kv_heads, w.block, w.samples, w.proj_bits,
                                 w.causal, w.min_seq_len, w.dtype) for w in (w_nc, w_c))
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def step():
        ha.forward(q, k, v, out=out, lse=lse, workspace=ws, **w_nc.method_args())
        ha.forward(q, k, v, out=out, lse=lse, workspace=ws, **w_c.method_args())

    if args.copy_calibration:
        src = torch.empty(args.copy_calibration << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.gather_calibration:
        # rows of d = 64 bf16 (128 bytes), 16 heads, one random permutation per head:
        # each gather reads and writes MIB MiB exactly once
        rows = (args.gather_calibration << 20) // 128 // 16
        src = torch.randn(16, rows, 64, device=dev).to(torch.bfloat16)
        g = torch.Generator(device=dev).manual_seed(3)
        perm = torch.stack([torch.randperm(rows, generator=g, device=dev) for _ in range(16)]).to(torch.int32)
        for _ in range(5):
            ha.gather_rows(src, perm)
        torch.cuda.synchronize()
        del src, perm

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, no per-launch timing hooks
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps

    # per-kernel durations: the same steps again, with the library recording HIP
    # events around each launch on the launch stream
    ha.timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    per_kernel = ha.timing_read()
    ha.timing_enable(False)

    # separate per-pass timing (untimed for `value`, reported for context)
    pass_ms, pass_stats = {}, {}
    for name, w in (("noncausal", w_nc), ("causal", w_c)):
        st = rep_times(torch, stream, lambda w=w: ha.forward(q, k, v, out=out, lse=lse, workspace=ws, **w.method_args()),
                       max(args.steps, 3))
        pass_ms[name] = st["mean"]
        pass_stats[name] = st

    # the library's results on the oracle sample's heads (compared in cpu_baseline)
    gpu_par = None
    if not args.no_cpu_baseline:
        try:
            gpu_par = gpu_sample(ha, torch, w_nc, w_c, q, k, v, ws, min(CPU_HEADS, w_nc.heads, w_nc.kv_heads))
        except Exception as e:              # the parity record is context; never lose the bench line to it
            gpu_par = {"error": repr(e)}

    f_nc, parts_nc = alg_flops(w_nc, False)
    f_c, parts_c = alg_flops(w_c, True)
    flops_step = f_nc + f_c
    value = flops_step / (ms_step * 1e-3) / 1e12

    # dominant kernel class and its roofline (HBM-bound when the kernel's
    # algorithmic intensity is below the MFMA/HBM ridge)
    kflops = {"attend": parts_nc["attend"], "leaf": parts_c["leaf"], "quadrant": parts_c["quadrant"]}
    bytes_nc, bytes_c = alg_bytes(w_nc, False), alg_bytes(w_c, True)
    kbytes = {}
    for dct in (bytes_nc, bytes_c):
        for kname, b in dct.items():
            kbytes[kname] = kbytes.get(kname, 0) + b
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    breakdown = {}
    for name, (ms, cnt) in per_kernel.items():
        if cnt:
            breakdown[name] = {"ms_per_step": ms / args.steps, "launches_per_step": cnt / args.steps,
                               "avg_launch_ms": ms / cnt}
    modelled = [kname for kname in breakdown if kname in kflops or kname in kbytes]
    dom = max(modelled, key=lambda kname: breakdown[kname]["ms_per_step"])
    ms_dom, cnt_dom = per_kernel[dom]
    launches = cnt_dom / args.steps
    avg_s = ms_dom / cnt_dom * 1e-3
    intensity = kflops[dom] / kbytes[dom] if dom in kflops else 0.0
    if dom in kflops and intensity >= ridge:
        per_launch = kflops[dom] / launches
        achieved = per_launch / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_BF16_PEAK_TFLOPS}
    else:
        per_launch = kbytes[dom] / launches
        achieved = per_launch / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    roof.update({"kernel": dom, "work_per_launch": per_launch, "avg_launch_ms": ms_dom / cnt_dom,
                 "intensity_flop_per_byte": intensity, "ridge_flop_per_byte": ridge})
    if dom in kflops:
        roof["mfma_tflops"] = kflops[dom] / launches / avg_s / 1e12
    roof["traffic"] = traffic_record(dom)
    for name in breakdown:
        if name in kflops:
            tot = kflops[name]
            breakdown[name]["tflops"] = tot / (breakdown[name]["ms_per_step"] * 1e-3) / 1e12
        if name in kbytes:
            breakdown[name]["gbs"] = kbytes[name] / (breakdown[name]["ms_per_step"] * 1e-3) / 1e9

    result = {
        "metric": "HyperAttention fwd ms + effective TFLOP/s at n=131072, 32 heads, causal/non",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w_nc.name}: one attention layer, batch {w_nc.batch}, {w_nc.heads} heads, "
                               f"n={w_nc.n}, d={w_nc.d}, bf16, block {w_nc.block}, samples {w_nc.samples}, "
                               f"r={w_nc.proj_bits}; step = non-causal + causal (min_seq_len "
                               f"{w_c.min_seq_len}) forward",
                   "batch": w_nc.batch, "heads": w_nc.heads, "seq_len": w_nc.n, "head_dim": w_nc.d,
                   "parallelism": "single GPU"},
        "ms_noncausal": pass_ms["noncausal"],
        "pass_ms_stats": pass_stats,
        "ms_causal": pass_ms["causal"],
        "tflops_noncausal": f_nc / (pass_ms["noncausal"] * 1e-3) / 1e12,
        "tflops_causal": f_c / (pass_ms["causal"] * 1e-3) / 1e12,
        # context only: the dense attention work the method avoids (4 B H n^2 d,
        # causal 2 B H n (n + 1) d) per pass time, and the hash arithmetic
        # (2 d r per row of Q and K, not part of `value`)
        "dense_equiv_tflops": {
            "noncausal": 4.0 * w_nc.batch * w_nc.heads * w_nc.n ** 2 * w_nc.d / (pass_ms["noncausal"] * 1e-3) / 1e12,
            "causal": 2.0 * w_c.batch * w_c.heads * w_c.n * (w_c.n + 1) * w_c.d / (pass_ms["causal"] * 1e-3) / 1e12},
        "hash_gflop_per_pass": 2.0 * w_nc.d * w_nc.proj_bits * w_nc.batch * (w_nc.heads + w_nc.kv_heads) * w_nc.n / 1e9,
        "wall_s_timed": wall,
        "roofline": roof,
        "kernels": breakdown,
    }
    if not args.no_extras:
        result["approx_rel_error"] = approx_error(ha, torch, w_nc, w_c, q, k, v, out)
        result["configs"] = other_configs(ha, torch, dev, stream)
        result["rownorm"] = {name: rownorm_bench(ha, torch, w, q, k, v, out, stream)
                             for name, w in (("noncausal", w_nc), ("causal", w_c))}
        result["diagnostics"] = diagnostics_bench(ha, torch, dev, stream)
        result["rect"] = rect_bench(ha, torch, dev, stream)
        result["gather"] = gather_bench(ha, torch, w_nc, k, stream)
        del ws
        result["backward"] = {name: backward_bench(ha, torch, w, q, k, v, out, lse, stream)
                              for name, w in (("noncausal", w_nc), ("causal", w_c))}
        result["backward"]["glm32k"] = backward_config_bench(ha, torch, "glm32k", dev, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w_nc, w_c, q, k, v, gpu_par)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


def approx_error(ha, torch, w_nc, w_c, q, k, v, out):
    """Secondary number: ||O - O_exact||_F / ||O_exact||_F of the headline
    configuration, with O_exact from the library's exact mode (block = n
    non-causal, min_seq_len = n causal; both oracle-checked at small n)."""
    res = {}
    ex = torch.empty_like(out)
    for name, w, exact in (("noncausal", w_nc, w_nc.with_(block=w_nc.n)),
                           ("causal", w_c, w_c.with_(min_seq_len=w_c.n))):
        ha.forward(q, k, v, out=out, **w.method_args())
        ha.forward(q, k, v, out=ex, **exact.method_args())
        a = out.float()
        b = ex.float()
        res[name] = float(torch.linalg.vector_norm(a - b) / torch.linalg.vector_norm(b))
        del a, b
    return res


def rect_bench(ha, torch, dev, stream, reps=5):
    """A rectangular non-causal problem shaped like a prefill chunk: 32768
    queries over 131072 keys, 32 heads, d = 64, bf16, block 256 (key
    blocks of 1024), 256 samples (not part of `value`).  FLOPs
    4 d (b_k + m) per query row."""
    B, H, nq, nk, d, block, m, r = 1, 32, 32768, 131072, 64, 256, 256, 7
    g = torch.Generator(device=dev).manual_seed(5)
    q = (torch.randn(B, H, nq, d, generator=g, device=dev) * d ** -0.25).to(torch.bfloat16)
    k = (torch.randn(B, H, nk, d, generator=g, device=dev) * d ** -0.25).to(torch.bfloat16)
    v = torch.randn(B, H, nk, d, generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    ws = torch.empty(ha.lib().hyperattn_rect_workspace_bytes(B, nq, nk, d, H, H, block, m, r, ha.HA_BF16),
                     dtype=torch.uint8, device=dev)
    args = dict(block=block, samples=m, proj_bits=r)
    ha.forward_rect(q, k, v, out=out, workspace=ws, **args)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        ha.forward_rect(q, k, v, out=out, workspace=ws, **args)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    b_k = -(-block * nk // nq)
    flops = 4.0 * d * B * H * nq * (b_k + m)
    del q, k, v, out, ws
    return {"n_q": nq, "n_k": nk, "heads": H, "head_dim": d, "block": block, "key_block": b_k, "samples": m,
            "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12}


def diagnostics_bench(ha, torch, dev, stream):
    """alpha (largest squared column norm of the exact softmax matrix; with
    and without the first 32 columns) on the 32k GQA causal configuration
    with planted attention sinks, and kappa (largest / smallest residual
    row sum outside the sortLSH blocks) on the 32k non-causal one; maxima
    over heads, and the column pass's time (not part of `value`)."""
    from approximate_long_context_amd.workloads import WORKLOADS, make_inputs
    res = {}
    w = WORKLOADS["glm32k"]
    q, k, v = make_inputs(w, dev)
    n = w.n
    lse = ha.forward(q, k, v, block=n, samples=0, proj_bits=w.proj_bits, causal=True, min_seq_len=n)[1]
    ha.column_sqmass(q, k, lse, causal=True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    _, a0 = ha.column_sqmass(q, k, lse, causal=True, skip=0)
    e1.record(stream)
    _, a32 = ha.column_sqmass(q, k, lse, causal=True, skip=32)
    torch.cuda.synchronize()
    res["glm32k_causal"] = {"alpha": float(a0.max()), "alpha_skip32": float(a32.max()),
                            "column_pass_ms": e0.elapsed_time(e1), "n": n}
    del q, k, v, lse
    w = WORKLOADS["c32k"]
    q, k, v = make_inputs(w, dev)
    B, H, n, d = q.shape
    le = ha.forward(q, k, v, block=n, samples=0, proj_bits=w.proj_bits)[1]
    R = ha.projections(w.seed, d, w.proj_bits, dev)
    perm_q = ha.sort_ranks(ha.hash_rows(q.view(-1, n, d), R), w.proj_bits).view(B * H, n)
    perm_k = ha.sort_ranks(ha.hash_rows(k.view(-1, n, d), R), w.proj_bits).view(B * w.kv_heads, n)
    idx = ha.sample_indices(w.seed, B, H, n, 16, device=dev)
    _, lb = ha.attend(q, k, v, perm_q, perm_k, idx, block=w.block, samples=16, parts=1)
    kappa = ha.residual_ratio(le.view(B * H, n), lb.reshape(B * H, n).contiguous(), perm_q.contiguous())
    res["c32k"] = {"kappa": float(kappa.max()), "block": w.block, "n": n}
    del q, k, v
    return res


def rownorm_bench(ha, torch, w, q, k, v, out, stream, reps=3):
    """The row-norm-sampling variant of the product (HA_FLAG_ROWNORM) on one
    headline pass (non-causal, or causal with every quadrant's own draws):
    ms, effective TFLOP/s counted like the forward's and its error against
    exact attention (not part of `value`)."""
    args = w.method_args()
    ws = torch.empty(ha.workspace_bytes(w.batch, w.n, w.d, w.heads, w.kv_heads, w.block, w.samples, w.proj_bits,
                                        w.causal, w.min_seq_len, w.dtype, flags=ha.HA_FLAG_ROWNORM),
                     dtype=torch.uint8, device=q.device)

    def run():
        ha.forward(q, k, v, out=out, workspace=ws, flags=ha.HA_FLAG_ROWNORM, **args)

    run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    f, _ = alg_flops(w, w.causal)
    ex = torch.empty_like(out)
    exact = w.with_(min_seq_len=w.n) if w.causal else w.with_(block=w.n)
    ha.forward(q, k, v, out=ex, **exact.method_args())
    run()
    a, b = out.float(), ex.float()
    err = float(torch.linalg.vector_norm(a - b) / torch.linalg.vector_norm(b))
    del a, b, ex, ws
    return {"ms": ms, "tflops": f / (ms * 1e-3) / 1e12, "approx_rel_error": err}


def gather_bench(ha, torch, w, k, stream, reps=5):
    """The stand-alone permutation gather (hyperattn_gather, the materialised
    mode's copy of rows into sorted order) on the headline K through its own
    LSH sort permutation: HBM bytes = rows x (row read + row written +
    4-byte permutation entry) per launch, against the 8 TB/s peak.  The
    default forward fuses this gather into the attention kernels' row loads
    (their bytes are in `kernels.attend.gbs`)."""
    R = ha.projections(w.seed, w.d, w.proj_bits, device=k.device)
    heads = w.batch * w.kv_heads
    k2 = k.reshape(heads, w.n, w.d)
    perm = ha.sort_ranks(ha.hash_rows(k2, R), w.proj_bits)[:, 0, :].contiguous()
    ha.gather_rows(k2, perm)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        ha.gather_rows(k2, perm)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = heads * w.n * (2 * w.d * k.element_size() + 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": ms, "bytes": nbytes, "gbs": gbs, "peak_gbs": HBM_PEAK_GBS, "frac": gbs / HBM_PEAK_GBS,
            "rows": heads * w.n, "row_bytes": w.d * k.element_size()}


def backward_bench(ha, torch, w, q, k, v, out, lse, stream, reps=3):
    """ms and effective TFLOP/s of the backward (dQ, dK, dV) of one pass of
    the headline configuration (not part of `value`).  Algorithmic FLOPs:
    10 d per (row, key) pair -- S, dP, dV, dQ, dK -- i.e. 2.5 times the
    forward's; the kernels recompute S and dP once more (14 d)."""
    ha.forward(q, k, v, out=out, lse=lse, **w.method_args())
    g = torch.Generator(device=q.device).manual_seed(77)
    dout = torch.randn(q.shape, generator=g, device=q.device).to(torch.bfloat16)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    ws = torch.empty(ha.backward_workspace_bytes(w.batch, w.n, w.d, w.heads, w.kv_heads, w.block, w.samples,
                                                 w.proj_bits, w.causal, w.min_seq_len),
                     dtype=torch.uint8, device=q.device)
    args = w.method_args()
    args.pop("flags", None)

    def run():
        ha.backward(q, k, v, out, lse, dout, dq=dq, dk=dk, dv=dv, workspace=ws, **args)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    ha.timing_enable(True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    per_kernel = ha.timing_read()
    ha.timing_enable(False)
    ms = e0.elapsed_time(e1) / reps
    f_fwd, _ = alg_flops(w, w.causal)
    res = {"ms": ms, "tflops": 2.5 * f_fwd / (ms * 1e-3) / 1e12, "causal": w.causal,
           "kernels": {name: t / reps for name, (t, cnt) in per_kernel.items() if cnt}}
    del dout, dq, dk, dv, ws
    return res


def backward_config_bench(ha, torch, name, dev, stream):
    """backward_bench on another named configuration (its own inputs; the
    d = 128 grouped-head causal one shows the d = 128 kernels)."""
    from approximate_long_context_amd.workloads import WORKLOADS, make_inputs
    w = WORKLOADS[name]
    q, k, v = make_inputs(w, dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    res = backward_bench(ha, torch, w, q, k, v, out, lse, stream)
    res["config"] = name
    del q, k, v, out, lse
    return res


def other_configs(ha, torch, dev, stream, reps=20):
    """ms per forward (median of `reps` after 3 warm-ups, with p10 / p90) and
    effective TFLOP/s of the other configurations: the fp32 n = 1024 single
    head (against the fp32 MFMA peak) and the bf16 ones (not part of
    `value`)."""
    from approximate_long_context_amd.workloads import WORKLOADS, make_inputs
    res = {}
    for name in ("small", "c32k", "glm32k", "stress512k"):
        w = WORKLOADS[name]
        q, k, v = make_inputs(w, dev)
        out = torch.empty_like(q)
        ws = torch.empty(ha.workspace_bytes(w.batch, w.n, w.d, w.heads, w.kv_heads, w.block, w.samples,
                                            w.proj_bits, w.causal, w.min_seq_len, w.dtype),
                         dtype=torch.uint8, device=dev)
        for _ in range(3):
            ha.forward(q, k, v, out=out, workspace=ws, **w.method_args())
        st = rep_times(torch, stream, lambda: ha.forward(q, k, v, out=out, workspace=ws, **w.method_args()), reps)
        ms = st["median"]
        # per-kernel-class ms per forward, from a separate timed set of calls
        ha.timing_enable(True)
        for _ in range(reps):
            ha.forward(q, k, v, out=out, workspace=ws, **w.method_args())
        torch.cuda.synchronize()
        kern = {kn: round(kms / reps, 4) for kn, (kms, cnt) in ha.timing_read().items() if cnt}
        ha.timing_enable(False)
        f, _ = alg_flops(w, w.causal)
        fp32 = w.dtype == torch.float32
        res[name] = {"ms": ms, "ms_p10": st["p10"], "ms_p90": st["p90"], "reps": reps,
                     "tflops": f / (ms * 1e-3) / 1e12, "causal": w.causal, "n": w.n,
                     "heads": w.heads, "kv_heads": w.kv_heads, "head_dim": w.d,
                     "block": w.block, "samples": w.samples, "dtype": "f32" if fp32 else "bf16",
                     "mfma_peak_tflops": MFMA_FP32_PEAK_TFLOPS if fp32 else MFMA_BF16_PEAK_TFLOPS,
                     "kernels_ms": kern}
        del q, k, v, out, ws
    return res


if __name__ == "__main__":
    main()
