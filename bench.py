#!/usr/bin/env python3
"""Benchmark of the latent causal attention hot path on one MI355X.

A step is one mla_latent_attn_fwd call (weight absorption, the fused causal
latent flash kernel, the up-projection) on the long-prefill workload
(bf16, B=2, T=16384, H=64, d=128, r=512), inputs resident in HBM.  The
decode workload (bf16, 64 ragged sequences of 1024..8192 cached latents,
H=32) is timed in the same run and reported in the `decode` object.

Prints ONE JSON line.  `value` is prefill TFLOP/s of the absorbed method's
algorithmic work (causal keys only); `roofline` is the flash kernel's
achieved TFLOP/s against the dense bf16 matrix-core peak, from its
average launch time measured with HIP events on the launch stream, with
`traffic` (HBM bytes per launch) and `mfma_busy` (the matrix cores' busy
fraction) read from the committed rocprofv3 counter summaries under
profiles/ while they match the library sources;
`cpu_baseline` is the fp64 CPU oracle timed on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0         # HBM3E
PEAK_FP32_TFLOPS = 157.3      # 256 CU x 2.4 GHz x 256 fp32 FLOP/clk/CU (vector ALUs)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_util.json")


def library_source_sha() -> str:
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "rank_latent_causal_mla_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when the library sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != library_source_sha():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else int(k["hbm_bytes"])


def measured_mfma_busy(kernel: str):
    """Fraction of the run's SIMD cycles the matrix cores were busy in
    `kernel` (rocprofv3 MfmaUtil, committed summary), or None when the
    library sources changed since it was taken."""
    try:
        with open(MFMA_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != library_source_sha():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else float(k["mfma_busy"])


# ---------------------------------------------------------------- algorithmic work
def gemm_flops(M: int, K: int, N: int) -> int:
    """FLOPs of an [M,K] x [K,N] product (one multiply and one add per term)."""
    return 2 * M * K * N


def prefill_flops(cfg) -> dict:
    """Absorbed-method FLOPs of one prefill call, causal keys only."""
    B, T, H, d, r = cfg.B, cfg.T, cfg.H, cfg.d, cfg.r
    absorb = H * gemm_flops(B * T, d, r)
    attn = 2 * B * H * r * T * (T + 1)          # scores + P latent over s <= t
    up = H * gemm_flops(B * T, r, d)
    down = gemm_flops(B * T, cfg.D, r) if cfg.D else 0
    return {"absorb": absorb, "attn": attn, "up": up, "down": down, "total": absorb + attn + up + down}


def masked_flops(cfg, key_mask) -> dict:
    """Absorbed-method FLOPs of one key-masked prefill call: query t of batch b
    attends the visible keys s <= t only (masked keys are skipped)."""
    B, T, H, d, r = cfg.B, cfg.T, cfg.H, cfg.d, cfg.r
    visible = int(np.cumsum(key_mask.astype(np.int64), axis=1).sum())   # sum over (b, t) of visible keys s <= t
    absorb = H * gemm_flops(B * T, d, r)
    attn = 4 * H * r * visible
    up = H * gemm_flops(B * T, r, d)
    return {"absorb": absorb, "attn": attn, "up": up, "total": absorb + attn + up}


def unabsorbed_flops(cfg) -> dict:
    """FLOPs of one prefill call in unabsorbed form: k and v materialised
    (2 B T r H d each), then causal attention at width d over t + 1 keys."""
    B, T, H, d, r = cfg.B, cfg.T, cfg.H, cfg.d, cfg.r
    kv = 2 * H * gemm_flops(B * T, r, d)
    attn = 2 * B * H * d * T * (T + 1)          # scores + P v over s <= t
    return {"materialise": kv, "attn": attn, "total": kv + attn}


def decode_bytes(cfg, lens) -> dict:
    """Algorithmic HBM bytes of one decode call: the cached latents read once,
    both up-projection weights, q and out (bf16)."""
    es = 2 if cfg.dtype == "bf16" else 4
    lat = es * cfg.r * int(np.sum(lens))
    w = 2 * es * cfg.r * cfg.H * cfg.d
    qo = 2 * es * cfg.B * cfg.H * cfg.d
    return {"latent": lat, "weights": w, "q_out": qo, "total": lat + w + qo}


def prefill_row_flops(cfg, t: int) -> int:
    """Absorbed-method FLOPs of one query row at position t."""
    return 2 * cfg.d * cfg.r + 4 * cfg.r * (t + 1) + 2 * cfg.r * cfg.d


def to_device(arr):
    """A stored input array (float32, or uint16 bf16 bit patterns) -> a device tensor."""
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16).copy()).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


# ---------------------------------------------------------------- GPU timing
MIN_TIMED_CALLS = 50   # calls timed one by one for the median and minimum
# A decode call lasts about 80 us: its mean is taken over this many calls back
# to back (16 ms), so the host's lead over the first launches, which a serving
# loop pays once, does not weigh on it.
DECODE_TIMED_CALLS = 200
# Likewise the sub-millisecond prefill workloads (bf16_prefill, the full
# paths): at least this many calls (about 45 ms at bf16_prefill).
SHORT_TIMED_CALLS = 60


def time_steps(fn, steps: int, warmup: int):
    """Mean ms per call over `steps` calls between two synchronisations (the
    headline figure), then the median and minimum of max(steps, 50) calls
    each bracketed by its own pair of events on the current stream."""
    import torch
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    mean = e0.elapsed_time(e1) / steps
    n = max(steps, MIN_TIMED_CALLS)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    each = sorted(a.elapsed_time(b) for a, b in ev)
    return mean, {"median_ms": round(float(np.median(each)), 4), "min_ms": round(each[0], 4), "calls": n}


def kernel_times(fn, steps: int):
    """Average ms per launch of each library kernel over `steps` calls (HIP events)."""
    import torch
    import rank_latent_causal_mla_amd as mla
    torch.cuda.synchronize()
    mla.mla_profile_collect()
    mla.mla_profile_enable(True)
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    mla.mla_profile_enable(False)
    stats = mla.mla_profile_collect()
    return {k: {"avg_ms": tot / n, "launches": n} for k, (tot, n) in stats.items()}


def bench_prefill(cfg, steps, warmup, unabsorbed=False, masked=False):
    import torch
    import synth
    import rank_latent_causal_mla_amd as mla
    inp = synth.make_inputs(cfg)
    dev = {k: to_device(v) for k, v in inp.items()}
    out = torch.empty_like(dev["q"])
    dt = mla.MLA_DTYPE_BF16 if cfg.dtype == "bf16" else mla.MLA_DTYPE_F32
    if masked:
        size = mla.mla_latent_attn_masked_workspace_size
        inp["key_mask"] = synth.make_key_mask(cfg, p_hole=0.05)
        kmask = torch.from_numpy(inp["key_mask"]).cuda()
    else:
        size = mla.mla_latent_attn_unabsorbed_workspace_size if unabsorbed else mla.mla_latent_attn_workspace_size
    fwd = mla.mla_latent_attn_fwd_unabsorbed if unabsorbed else mla.mla_latent_attn_fwd
    ws = torch.empty(size(cfg.B, cfg.T, cfg.H, cfg.d, cfg.r, dt), dtype=torch.uint8, device="cuda")

    def step(_i):
        if masked:
            mla.mla_latent_attn_fwd_masked(dev["q"], dev["kv_latent"], kmask, dev["w_up_k"], dev["w_up_v"], out=out,
                                           scale=cfg.scale, workspace=ws)
        else:
            fwd(dev["q"], dev["kv_latent"], dev["w_up_k"], dev["w_up_v"], out=out, scale=cfg.scale, workspace=ws)

    ms, dist = time_steps(step, steps, warmup)
    kt = kernel_times(step, steps)
    return ms, kt, inp, dist


def bench_full(cfg, steps, warmup):
    """The full path in one call (mla_latent_attn_fwd_full): down-projection into the latent cache, then the
    causal prefill."""
    import torch
    import synth
    import rank_latent_causal_mla_amd as mla
    inp = synth.make_inputs(cfg)
    dev = {k: to_device(v) for k, v in inp.items()}
    out = torch.empty_like(dev["q"])
    lat = torch.empty((cfg.B, cfg.T, cfg.r), dtype=dev["q"].dtype, device="cuda")
    dt = mla.MLA_DTYPE_BF16 if cfg.dtype == "bf16" else mla.MLA_DTYPE_F32
    ws = torch.empty(mla.mla_latent_attn_full_workspace_size(cfg.B, cfg.T, cfg.D, cfg.H, cfg.d, cfg.r, dt),
                     dtype=torch.uint8, device="cuda")

    def step(_i):
        mla.mla_latent_attn_fwd_full(dev["hidden"], dev["w_down"], dev["q"], dev["w_up_k"], dev["w_up_v"],
                                     kv_latent=lat, out=out, scale=cfg.scale, workspace=ws)

    ms, dist = time_steps(step, steps, warmup)
    return ms, kernel_times(step, steps), dist


def bench_decode_varlen(cfg, steps, warmup, copies=3):
    """The same decode over packed caches [sum L, r] with cu_seqlens (rotated copies as above)."""
    import torch
    import synth
    import rank_latent_causal_mla_amd as mla
    inp = synth.make_inputs(cfg)
    lens = inp["seq_lens"]
    dev = {k: to_device(v) for k, v in inp.items() if k not in ("seq_lens", "kv_latent")}
    packed = np.concatenate([inp["kv_latent"][b, :int(L)] for b, L in enumerate(lens)], axis=0)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    caches = [to_device(packed)]
    caches += [caches[0].clone() for _ in range(copies - 1)]
    out = torch.empty_like(dev["q"])
    ws = torch.empty(mla.mla_decode_varlen_workspace_size(cfg.B, packed.shape[0], cfg.H, cfg.d, cfg.r,
                                                          mla.MLA_DTYPE_BF16), dtype=torch.uint8, device="cuda")

    def step(i):
        mla.mla_decode_varlen_fwd(dev["q"], caches[i % copies], cu, dev["w_up_k"], dev["w_up_v"], out=out,
                                  scale=cfg.scale, workspace=ws)

    return time_steps(step, steps, warmup)


def bench_decode(cfg, steps, warmup, copies=3):
    """Decode with `copies` independent caches used in turn, so the 256 MB
    last-level cache cannot hold the ~300 MB working set between steps."""
    import torch
    import synth
    import rank_latent_causal_mla_amd as mla
    inp = synth.make_inputs(cfg)
    lens = inp["seq_lens"]
    dev = {k: to_device(v) for k, v in inp.items() if k != "seq_lens"}
    caches = [dev["kv_latent"]] + [dev["kv_latent"].clone() for _ in range(copies - 1)]
    dlens = torch.from_numpy(lens).cuda()
    out = torch.empty_like(dev["q"])
    dt = mla.MLA_DTYPE_BF16
    ws = torch.empty(mla.mla_decode_workspace_size(cfg.B, cfg.T, cfg.H, cfg.d, cfg.r, dt),
                     dtype=torch.uint8, device="cuda")

    def step(i):
        mla.mla_decode_fwd(dev["q"], caches[i % copies], dlens, dev["w_up_k"], dev["w_up_v"], out=out,
                           scale=cfg.scale, workspace=ws)

    ms, dist = time_steps(step, steps, warmup)
    kt = kernel_times(step, steps)
    return ms, kt, lens, dist


# ---------------------------------------------------------------- CPU baseline
def host_info() -> dict:
    """The host the oracle runs on: CPU model, logical CPUs, the CPUs this
    process may run on, and the threads the oracle starts by default."""
    import platform
    import oracle
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = sorted(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = []
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "affinity_cpus": len(allowed),
            "affinity": f"{allowed[0]}-{allowed[-1]}" if allowed and allowed[-1] - allowed[0] + 1 == len(allowed)
            else ",".join(map(str, allowed)), "oracle_threads": oracle.threads(0)}


def oracle_flops(groups: dict, rows_nkeys, d: int, r: int) -> int:
    """FLOPs the oracle itself executes: for each (b, h) group, k and v of its
    nk keys (2 products of 2 r d each per key), then per row of n keys the
    logits and the weighted sum of v (2 d each per key)."""
    return sum(4 * nk * d * r for nk in groups.values()) + sum(4 * d * int(n) for n in rows_nkeys)


def cpu_baseline(work):
    """The fp64 oracle, as it stands, on bounded samples of the three bf16
    workloads; each sample attends the given rows over their full causal
    key range, so the oracle materialises k and v for every key of each
    sampled (b, h) pair."""
    import oracle
    samples, tot_abs, tot_orc, tot_sec = [], 0, 0, 0.0
    for name, cfg, inp, rb, rh, nkeys, qrows, abs_flops in work:
        groups = {}
        for b, h, n in zip(rb, rh, nkeys):
            groups[(int(b), int(h))] = max(groups.get((int(b), int(h)), 0), int(n))
        t0 = time.perf_counter()
        oracle.attend_rows(qrows, rb, rh, nkeys, inp["kv_latent"], inp["w_up_k"], inp["w_up_v"], cfg.scale)
        sec = time.perf_counter() - t0
        of = oracle_flops(groups, nkeys, cfg.d, cfg.r)
        samples.append({"workload": name, "rows": len(rb), "bh_pairs": len(groups), "seconds": round(sec, 3),
                        "absorbed_tflops": round(abs_flops / sec / 1e12, 6), "oracle_tflops": round(of / sec / 1e12, 6),
                        "threads_used": min(oracle.threads(0), len(groups))})
        tot_abs += abs_flops
        tot_orc += of
        tot_sec += sec
    info = host_info()
    first = samples[0]
    return {"value": first["absorbed_tflops"], "unit": "TFLOP/s", "cores": first["threads_used"], "kind": "oracle",
            "sample": "; ".join(f"{x['workload']}: {x['rows']} query rows over {x['bh_pairs']} (b, h) pairs, "
                                f"each over its full causal key range ({x['seconds']} s)" for x in samples),
            "what": "value: absorbed-method FLOPs of the sampled rows of the headline workload per second of the "
                    "oracle's wall time; oracle_tflops: the FLOPs the oracle itself executes (k and v materialised "
                    "for every key of each sampled (b, h) pair, then d-wide products) per second",
            "oracle_tflops": first["oracle_tflops"], "seconds": round(tot_sec, 3), "samples": samples, **info}


def cpu_work(cfg, inp, dcfg):
    """The bounded samples the CPU baseline times: the headline prefill workload
    (8 heads of batch 0, 48 positions spread over the sequence), bf16_prefill
    (16 (b, h) pairs, 32 positions each) and bf16_decode (4 sequences x 8 heads)."""
    import synth
    work = []
    prefills = [(cfg, inp, [(0, h) for h in range(min(8, cfg.H))], 48)]
    if cfg.name != "bf16_prefill":
        c3 = synth.CONFIGS["bf16_prefill"]
        prefills.append((c3, synth.make_inputs(c3), [(b, h) for b in range(0, 8, 2) for h in range(0, 16, 4)], 32))
    for c, ci, heads, npos in prefills:
        ts = [int(x) for x in np.linspace(0, c.T - 1, npos).round()]
        rb = np.repeat([b for b, _ in heads], len(ts))
        rh = np.repeat([h for _, h in heads], len(ts))
        rt = np.tile(ts, len(heads))
        flops = sum(prefill_row_flops(c, int(t)) for t in rt)
        work.append((c.name, c, ci, rb, rh, rt + 1, ci["q"][rb, rt, rh], flops))
    if dcfg is not None:
        di = synth.make_inputs(dcfg)
        lens = di["seq_lens"]
        seqs = [int(x) for x in np.argsort(lens, kind="stable")[::16][:4]]   # four sequences across the length range
        rb = np.repeat(seqs, 8)
        rh = np.tile(np.arange(8), len(seqs))
        nk = lens[rb]
        flops = sum(2 * dcfg.d * dcfg.r + 4 * dcfg.r * int(n) + 2 * dcfg.r * dcfg.d for n in nk)
        work.append((dcfg.name, dcfg, di, rb, rh, nk, di["q"][rb, 0, rh], flops))
    return work


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="bf16_long_prefill")
    ap.add_argument("--decode-workload", default="bf16_decode")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unabsorbed", action="store_true", help="skip the unabsorbed prefill timing")
    ap.add_argument("--no-masked", action="store_true", help="skip the key-masked prefill timing")
    ap.add_argument("--no-full", action="store_true", help="skip the full-path (down-projection + prefill) timing")
    ap.add_argument("--no-short", action="store_true", help="skip the bf16_prefill (T=2048) timing")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import synth
    import rank_latent_causal_mla_amd as mla
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    mla.load()

    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cfg = synth.CONFIGS[args.workload]
    ms, kt, inp, dist = bench_prefill(cfg, args.steps, args.warmup)
    # the shorter workloads below (calls of 0.1-1 ms) get at least 20 warm-up
    # calls, so that the clocks have settled when their timing starts
    sub_warmup = max(args.warmup, 20)
    work = prefill_flops(cfg)
    value = work["total"] / (ms * 1e-3) / 1e12
    flash = kt.get("flash_latent_bf16")
    roof = None
    if flash:
        ach = work["attn"] / (flash["avg_ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic("flash_latent_bf16"),
                "mfma_busy": measured_mfma_busy("flash_latent_bf16"),
                "kernel": "flash_latent_bf16", "avg_ms": round(flash["avg_ms"], 4),
                "flops_per_launch": work["attn"]}
    line = {
        "metric": "latent-attn prefill TFLOP/s (decode GB/s in `decode`) at 1 GPU, % of MFMA/HBM roofline",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "H": cfg.H, "d": cfg.d, "r": cfg.r,
                   "causal": True, "flops_per_step": work["total"]},
        "roofline": roof,
        "per_call": dist,
        "kernels_ms": {k: round(v["avg_ms"], 4) for k, v in kt.items()},
    }
    if args.workload == "bf16_long_prefill" and not args.no_short:
        # the shorter bf16 prefill workload (B=8, T=2048, H=16): the same kernels at a length where each query
        # block carries 8x less work, so fixed costs per block weigh more
        scfg = synth.CONFIGS["bf16_prefill"]
        sms, skt, _, sdist = bench_prefill(scfg, max(args.steps, SHORT_TIMED_CALLS), sub_warmup)
        sw = prefill_flops(scfg)
        sfl = skt.get("flash_latent_bf16")
        ums_s, _, _, _ = bench_prefill(scfg, max(args.steps, SHORT_TIMED_CALLS), sub_warmup, unabsorbed=True)
        line["prefill_short"] = {
            "workload": scfg.name, "value": round(sw["total"] / (sms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(sms, 4), "per_call": sdist, "flops_per_step": sw["total"],
            "unabsorbed_ms_per_step": round(ums_s, 4),
            "roofline": None if not sfl else {
                "bound": "mfma", "achieved": round(sw["attn"] / (sfl["avg_ms"] * 1e-3) / 1e12, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(sw["attn"] / (sfl["avg_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "kernel": "flash_latent_bf16", "avg_ms": round(sfl["avg_ms"], 4), "flops_per_launch": sw["attn"]},
            "kernels_ms": {k: round(v["avg_ms"], 4) for k, v in skt.items()}}
    if not args.no_unabsorbed and cfg.dtype == "bf16" and \
            mla.mla_latent_attn_unabsorbed_workspace_size(cfg.B, cfg.T, cfg.H, cfg.d, cfg.r, mla.MLA_DTYPE_BF16):
        ums, ukt, _, udist = bench_prefill(cfg, args.steps, args.warmup, unabsorbed=True)
        uw = unabsorbed_flops(cfg)
        mha = ukt.get("flash_mha_bf16")
        uroof = None
        if mha:
            ach = uw["attn"] / (mha["avg_ms"] * 1e-3) / 1e12
            uroof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic("flash_mha_bf16"),
                     "mfma_busy": measured_mfma_busy("flash_mha_bf16"), "kernel": "flash_mha_bf16", "avg_ms": round(mha["avg_ms"], 4), "flops_per_launch": uw["attn"]}
        line["unabsorbed"] = {
            "what": "the same prefill with k and v materialised (mla_latent_attn_fwd_unabsorbed); value counts "
                    "that form's own FLOPs",
            "value": round(uw["total"] / (ums * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": round(ums, 4),
            "per_call": udist,
            "flops_per_step": uw["total"], "step_time_vs_absorbed": round(ms / ums, 3), "roofline": uroof,
            "kernels_ms": {k: round(v["avg_ms"], 4) for k, v in ukt.items()}}
    if not args.no_masked:
        mms, mkt, minp, mdist = bench_prefill(cfg, args.steps, args.warmup, masked=True)
        mw = masked_flops(cfg, minp["key_mask"])
        mflash = mkt.get("flash_latent_bf16_masked")
        line["masked"] = {
            "what": "the same prefill with a key mask (mla_latent_attn_fwd_masked): per batch, keys past a valid "
                    "length uniform on [T/2, T] and 5% of the rest masked; the visible keys are packed first and "
                    "masked keys are skipped; value counts the visible causal keys only",
            "value": round(mw["total"] / (mms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(mms, 4), "per_call": mdist, "flops_per_step": mw["total"],
            "roofline": None if not mflash else {
                "bound": "mfma", "achieved": round(mw["attn"] / (mflash["avg_ms"] * 1e-3) / 1e12, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(mw["attn"] / (mflash["avg_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic("flash_latent_bf16_masked"),
                "mfma_busy": measured_mfma_busy("flash_latent_bf16_masked"), "kernel": "flash_latent_bf16_masked",
                "avg_ms": round(mflash["avg_ms"], 4), "flops_per_launch": mw["attn"]},
            "kernels_ms": {k: round(v["avg_ms"], 4) for k, v in mkt.items()}}
    if not args.no_full:
        import dataclasses
        line["full_path"] = []
        for fcfg in (synth.CONFIGS["fp32_full_path"],
                     dataclasses.replace(synth.CONFIGS["bf16_prefill"], name="bf16_prefill_down1024", D=1024)):
            fms, fkt, fdist = bench_full(fcfg, max(args.steps, SHORT_TIMED_CALLS), sub_warmup)
            fw = prefill_flops(fcfg)
            down = fkt.get("down_bf16") or fkt.get("down_f32")
            if fcfg.dtype == "bf16":
                dom, dom_flops, bound, peak = fkt.get("flash_latent_bf16"), fw["attn"], "mfma", PEAK_BF16_TFLOPS
                dom_name = "flash_latent_bf16"
            else:   # float32: every product on the vector ALUs
                dom_name = "attend_f32_tiled" if "attend_f32_tiled" in fkt else "attend_simt"
                dom, dom_flops, bound, peak = fkt.get(dom_name), fw["attn"], "alu", PEAK_FP32_TFLOPS
            froof = None
            if dom:
                ach = dom_flops / (dom["avg_ms"] * 1e-3) / 1e12
                froof = {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                         "frac": round(ach / peak, 4), "traffic": None, "kernel": dom_name,
                         "avg_ms": round(dom["avg_ms"], 4), "flops_per_launch": dom_flops}
            line["full_path"].append({
                "what": "mla_latent_attn_fwd_full: kv_latent = hidden @ w_down written as the latent cache, then the "
                        "causal prefill; value counts the down-projection and the absorbed-method FLOPs",
                "workload": fcfg.name, "dtype": fcfg.dtype,
                "shape": {"B": fcfg.B, "T": fcfg.T, "D": fcfg.D, "H": fcfg.H, "d": fcfg.d, "r": fcfg.r},
                "value": round(fw["total"] / (fms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                "ms_per_step": round(fms, 4), "per_call": fdist, "flops_per_step": fw["total"],
                "down_tflops": round(fw["down"] / (down["avg_ms"] * 1e-3) / 1e12, 2) if down else None,
                "roofline": froof,
                "kernels_ms": {k: round(v["avg_ms"], 4) for k, v in fkt.items()}})
    if not args.no_decode:
        dcfg = synth.CONFIGS[args.decode_workload]
        dms, dkt, lens, ddist = bench_decode(dcfg, max(args.steps, DECODE_TIMED_CALLS), sub_warmup)
        db = decode_bytes(dcfg, lens)
        split = dkt.get("decode_split")
        droof = None
        if split:
            ach = db["latent"] / (split["avg_ms"] * 1e-3) / 1e9
            droof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": measured_traffic("decode_split"),
                     "kernel": "decode_split",
                     "avg_ms": round(split["avg_ms"], 4), "bytes_per_launch": db["latent"]}
        line["decode"] = {"workload": dcfg.name, "value": round(db["total"] / (dms * 1e-3) / 1e9, 1),
                          "unit": "GB/s", "ms_per_step": round(dms, 4), "per_call": ddist,
                          "bytes_per_step": db["total"],
                          "sum_seq_lens": int(np.sum(lens)), "roofline": droof,
                          "kernels_ms": {k: round(v["avg_ms"], 4) for k, v in dkt.items()}}
        if dcfg.dtype == "bf16":
            vms, vdist = bench_decode_varlen(dcfg, max(args.steps, DECODE_TIMED_CALLS), sub_warmup)
            line["decode"]["varlen"] = {"what": "the same decode over a packed cache (mla_decode_varlen_fwd)",
                                        "value": round(db["total"] / (vms * 1e-3) / 1e9, 1), "unit": "GB/s",
                                        "ms_per_step": round(vms, 4), "per_call": vdist}
    if not args.no_cpu_baseline:
        import synth as _synth
        line["cpu_baseline"] = cpu_baseline(cpu_work(cfg, inp, None if args.no_decode
                                                     else _synth.CONFIGS[args.decode_workload]))
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
