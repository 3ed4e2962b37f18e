"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * prefill forward, B=1, H=32, N=8192, d=128, causal, bf16 (fa_fwd), and
  * split-KV decode, B=64, Hq=32, Hkv=8, Nk=32768, d=128, 16 splits, bf16
    (fa_decode_splitkv + fa_lse_merge).
Inputs are generated once (seeded), uploaded, and stay resident in HBM.

Prints ONE JSON line.  `value` is the prefill throughput in TFLOP/s, counting
4*d FLOP per allowed (query, key) pair (2*d for Q.K, 2*d for P.V); the decode
bandwidth and every kernel's own roofline sit beside it.  Kernel durations
come from HIP events recorded on the stream the kernels run on; each timed
kernel reports mean, median, min and p90 over its launches.  Beside the
published peaks, measured ceilings are timed in the same run: a
matrix-core-only loop on random operands (the denominator the kernels are
read against: on random data the chip sustains a lower clock than on the
small constants of the same loop, which is timed too) and a streaming read.  The other workloads (d=64
self-attention, padded GQA, backward, FP8, packed, paged decode) are timed
after the step as side legs, each after its own time-based warm-up; a last leg
runs the headline kernel on all-zero operands, which shows how much of the
clock the chip's power limit takes on the random inputs.
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s & % bf16 MFMA peak (N=8K causal d=128); decode HBM GB/s"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU (published 2.5 PFLOP/s)
PEAK_FP8_TFLOPS = 5033.2   # dense FP8 MFMA: twice the bf16 rate (published 5.0 PFLOP/s)
# The FP8 forward runs Q.K^T on FP8 and P.V on bf16 matrix cores, half of its
# FLOP each: at both peaks one FLOP costs (1/2)/PEAK_FP8 + (1/2)/PEAK_BF16.
PEAK_FP8_BF16_MIX_TFLOPS = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)
PEAK_HBM_GBS = 8000.0      # HBM3E, 8 TB/s
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic_counters.json")
KERNEL_SOURCES = ["fwd_bf16.hip", "fwd_fp8.hip", "decode_bf16.hip", "bwd_bf16.hip", "fa_device.hpp"]
WARM_S = 0.5  # minimum warm-up of the main step, seconds (clocks settle after ~0.25 s of load)
SIDE_WARM_S = 0.25


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_tiled_attention_08_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def prefill_flops(B, H, Nq, Nk, d, causal):
    """4*d FLOP per allowed (query, key) pair."""
    if causal:
        pairs = (sum(max(0, min(Nk, i + (Nk - Nq) + 1)) for i in range(Nq)) if Nq != Nk
                 else Nq * (Nq + 1) // 2)
    else:
        pairs = Nq * Nk
    return 4.0 * d * B * H * pairs


def padded_causal_flops(Hq, N, lens, d):
    """4*d FLOP per allowed pair of a causal self-attention (Nq = Nk = N) whose
    sequence b has lens[b] valid keys: row i sees min(i + 1, L_b) keys."""
    pairs = 0
    for L in lens:
        L = max(0, min(int(L), N))
        pairs += L * (L + 1) // 2 + (N - L) * L
    return 4.0 * d * Hq * pairs


def decode_bytes(B, Hq, Hkv, Nk, d, elem=2):
    """Algorithmic HBM bytes: K and V read once, Q read, O and LSE written."""
    return 2 * B * Hkv * Nk * d * elem + B * Hq * d * elem * 2 + B * Hq * 4


def _counters():
    try:
        with open(PROFILE_COUNTERS) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return rec if rec.get("kernel_source_hash") == kernel_source_hash() else None


def load_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    rec = _counters()
    k = None if rec is None else rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def load_util(kernel):
    """Matrix-core busy fraction of SIMD cycles and the sustained clock during
    the kernel, from the committed counter runs on the current sources; else
    None."""
    rec = _counters()
    return None if rec is None else rec.get("utilisation", {}).get(kernel)


def stats_ms(ms):
    """mean / median / min / p90 of per-launch durations (ms)."""
    s = sorted(ms)
    n = len(s)
    p90 = s[min(n - 1, int(0.9 * (n - 1) + 0.5))]
    med = s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])
    return {"mean_ms": round(sum(s) / n, 5), "median_ms": round(med, 5), "min_ms": round(s[0], 5),
            "p90_ms": round(p90, 5), "launches": n}


def cpu_info():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def cpu_baseline(n_heads):
    """Time the fp64 oracle on a bounded sample of the prefill workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from exact_tiled_attention_08_amd import inputs
    import oracle

    q, k, v, _ = inputs.make_inputs(3)
    q64, k64, v64 = (x[:, :n_heads].to(dtype=__import__("torch").float64).numpy() for x in (q, k, v))
    t0 = time.perf_counter()
    oracle.attention_ref(q64, k64, v64, causal=True)
    dt = time.perf_counter() - t0
    flops = prefill_flops(1, n_heads, 8192, 8192, 128, True)
    info = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in info] or [1])
    blas = [f"{p.get('internal_api')} {p.get('version')} ({p.get('threading_layer')})" for p in info
            if p.get("user_api") == "blas"]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"prefill N=8192 causal d=128, {n_heads} of 32 heads (B=1), fp64 numpy; "
                      f"{dt:.1f} s; exp runs single-threaded",
            "seconds": dt, "cpu_model": cpu_info(), "blas": blas or ["unknown"],
            "affinity_cores": len(os.sched_getaffinity(0)), "numpy": np.__version__}


def warm(call, seconds=SIDE_WARM_S, min_calls=0):
    """Run `call` back to back for at least `seconds` and `min_calls` calls
    (clocks settle after a change of workload), synchronising every 10 calls.
    Returns (calls, seconds)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < min_calls or time.perf_counter() - t0 < seconds:
        for _ in range(10):
            call()
        n += 10
        torch.cuda.synchronize()
    return n, time.perf_counter() - t0


def time_calls(call, n, stream):
    """Per-call durations (ms) from HIP events around each of n calls."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in ev]


def mfma_leg(ms, flop, kernel, workload, ceiling=None, util=None, traffic=None, peak=PEAK_BF16_TFLOPS):
    """Record of a matrix-core-bound leg from its per-launch durations."""
    st = stats_ms(ms)
    tf = flop / (st["mean_ms"] * 1e-3) / 1e12
    roof = {"bound": "mfma", "kernel": kernel, "achieved": round(tf, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(tf / peak, 4), "traffic": traffic,
            "median_tflops": round(flop / (st["median_ms"] * 1e-3) / 1e12, 2)}
    if ceiling:
        roof["measured_ceiling"] = round(ceiling, 1)
        roof["frac_of_measured_ceiling"] = round(tf / ceiling, 4)
    if util:
        roof["counter_mfma_busy_frac"] = util.get("mfma_busy_frac")
        roof["counter_clock_ghz"] = util.get("clock_ghz")
    return {"value": round(tf, 2), "unit": "TFLOP/s", "workload": workload, "flop_per_call": flop, **st,
            "roofline": roof}


def ceilings(dev, stream, read_buf):
    """Measured matrix-core-only (random and constant operands) and streaming-read rates on this GPU
    (same run)."""
    import torch

    from exact_tiled_attention_08_amd import _lib
    lib = _lib.load()
    cu = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks, iters = 2 * cu, 512
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    g = torch.Generator(device="cpu").manual_seed(99)
    operands = torch.randn(blocks * 16 * 256 * 8, generator=g).to(torch.bfloat16).to(dev)
    flop = blocks * 4 * iters * 32 * 32768.0
    res = {}
    for key, src, what in (("mfma_bf16", operands.data_ptr(), "random N(0,1) bf16 operands"),
                           ("mfma_bf16_const_operands", None, "small constant operands")):
        mf = lambda: lib.fa_ceiling_mfma(src, out.data_ptr(), blocks, iters, stream.cuda_stream)  # noqa: E731
        warm(mf)
        ms = time_calls(mf, 20, stream)
        tf = flop / (min(ms) * 1e-3) / 1e12
        res[key] = {"value": round(tf, 1), "unit": "TFLOP/s", "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                    "what": f"fa_ceiling_mfma: {blocks} work-groups x 4 waves, {iters * 32} products per wave in 4 "
                            f"independent v_mfma_f32_32x32x16_bf16 chains, {what} (fastest launch)",
                    **stats_ms(ms)}
    rblocks = 2 * cu
    ro = torch.empty(rblocks * 256, dtype=torch.int32, device=dev)
    nbytes = read_buf.numel() * read_buf.element_size()
    rd = lambda: lib.fa_ceiling_read(read_buf.data_ptr(), nbytes, ro.data_ptr(), rblocks, stream.cuda_stream)  # noqa: E731
    warm(rd)
    rms = time_calls(rd, 20, stream)
    rst = stats_ms(rms)
    read_gbs = nbytes / (min(rms) * 1e-3) / 1e9
    res["hbm_read"] = {"value": round(read_gbs, 1), "unit": "GB/s", "frac_of_peak": round(read_gbs / PEAK_HBM_GBS, 4),
                       "what": f"fa_ceiling_read: {nbytes} bytes read once by {rblocks} work-groups, each a "
                               "contiguous run with eight 16-byte nontemporal loads in flight per lane (fastest launch)",
                       **rst}
    return res


def profile_only(args, dev):
    """Run one part of the step args.warmup + args.steps times (for rocprofv3)."""
    import torch

    import exact_tiled_attention_08_amd as fa
    from exact_tiled_attention_08_amd import inputs

    n = args.warmup + args.steps
    if args.only == "ceilings":
        from exact_tiled_attention_08_amd import _lib
        lib = _lib.load()
        blocks = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
        out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
        operands = torch.randn(blocks * 16 * 256 * 8, device=dev).to(torch.bfloat16)
        for src in (operands.data_ptr(), None):
            for _ in range(n):
                lib.fa_ceiling_mfma(src, out.data_ptr(), blocks, 512, None)
    elif args.only == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(n):
            dst.copy_(src)
    elif args.only == "prefill":
        q, k, v = [t.to(dev) for t in inputs.make_inputs(3)[:3]]
        for _ in range(n):
            fa.fa_fwd(q, k, v, causal=True)
    elif args.only == "prefill_zero":
        q = torch.zeros(inputs.CONFIGS[3]["B"], inputs.CONFIGS[3]["Hq"], inputs.CONFIGS[3]["Nq"],
                        inputs.CONFIGS[3]["d"], dtype=torch.bfloat16, device=dev)
        for _ in range(n):
            fa.fa_fwd(q, q, q, causal=True)
    elif args.only in ("d64", "d64nc"):
        q, k, v = [t.to(dev) for t in inputs.make_inputs(2)[:3]]
        for _ in range(n):
            fa.fa_fwd(q, k, v, causal=args.only == "d64")
    elif args.only == "gqa":
        q, k, v, lens = [t.to(dev) for t in inputs.make_inputs(4)]
        for _ in range(n):
            fa.fa_fwd(q, k, v, causal=True, kv_seqlens=lens)
    elif args.only == "fp8":
        q, k, v, _, ds = inputs.make_fp8_inputs(3, "e4m3")
        q, k, v = q.to(dev), k.to(dev), v.to(dev)
        for _ in range(n):
            fa.fa_fwd_fp8(q, k, v, *ds, causal=True)
    elif args.only == "varlen":
        lens = inputs.lengths(4, 4, 2048, 4096).tolist()
        q, k, v, cq, ck = (t.to(dev) for t in inputs.make_packed(4, lens, lens, 32, 8, 128))
        for _ in range(n):
            fa.fa_fwd_varlen(q, k, v, cq, ck, max(lens), causal=True)
    elif args.only == "paged":
        c5 = inputs.CONFIGS[5]
        q, k, v = [t.to(dev) for t in inputs.make_inputs(5)[:3]]
        kp, vp, table = paged_copy(k, v, 16, dev)
        lens = torch.full((c5["B"],), c5["Nk"], dtype=torch.int32, device=dev)
        del k, v
        for _ in range(n):
            fa.fa_decode_paged(q, kp, vp, table, lens, num_splits=c5["num_splits"])
    elif args.only == "backward":
        q, k, v = [t.to(dev) for t in inputs.make_inputs(3)[:3]]
        do = inputs.make_dout(3).to(dev)
        o, lse = fa.fa_fwd(q, k, v, causal=True)
        for _ in range(n):
            fa.fa_bwd(q, k, v, o, lse, do, causal=True)
    else:
        c5 = inputs.CONFIGS[5]
        q, k, v = [t.to(dev) for t in inputs.make_inputs(5)[:3]]
        for _ in range(n):
            fa.fa_decode(q, k, v, num_splits=c5["num_splits"])
    torch.cuda.synchronize()
    print(f"[bench] ran {args.only} x{n}", file=sys.stderr, flush=True)


def paged_copy(k, v, page, dev):
    """The cache [B, Hkv, Nk, d] scattered into a shuffled pool of pages
    [B*Nk/page, Hkv, page, d] and its block table."""
    import torch
    B, Hkv, Nk, d = k.shape
    n_pages = B * (Nk // page)
    g = torch.Generator(device=dev).manual_seed(555)
    table = torch.randperm(n_pages, generator=g, device=dev).to(torch.int32).reshape(B, Nk // page)
    idx = table.long().reshape(-1)
    kp = torch.empty((n_pages, Hkv, page, d), dtype=k.dtype, device=dev)
    vp = torch.empty_like(kp)
    kp[idx] = k.reshape(B, Hkv, Nk // page, page, d).permute(0, 2, 1, 3, 4).reshape(-1, Hkv, page, d)
    vp[idx] = v.reshape(B, Hkv, Nk // page, page, d).permute(0, 2, 1, 3, 4).reshape(-1, Hkv, page, d)
    return kp, vp, table


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help=f"untimed steps; the warm-up also lasts at least {WARM_S} s so that clocks settle")
    ap.add_argument("--cpu-heads", type=int, default=32, help="heads in the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--side-steps", type=int, default=20,
                    help="timed calls of each side leg (d=64, padded GQA, backward, paged, packed, FP8); 0 = skip")
    ap.add_argument("--only", choices=["prefill", "prefill_zero", "d64", "d64nc", "gqa", "decode", "backward", "fp8",
                                       "varlen", "paged", "copy", "ceilings"],
                    default=None,
                    help="profiling aid: run only one part (or a 1 GiB device copy used to calibrate the HBM byte "
                         "counters, or the matrix-core ceilings) and print no JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path would shard heads or batch across GPUs with no exchange).", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_tiled_attention_08_amd as fa
    from exact_tiled_attention_08_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} CUs={props.multi_processor_count}")

    if args.only is not None:
        profile_only(args, dev)
        return

    # ---- inputs (seeded, generated on the host once, resident in HBM)
    c3 = inputs.CONFIGS[3]
    q3, k3, v3, _ = (t.to(dev) if t is not None else None for t in inputs.make_inputs(3))
    o3 = torch.empty_like(q3)
    l3 = torch.empty(q3.shape[:3], dtype=torch.float32, device=dev)
    c5 = inputs.CONFIGS[5]
    log("generating decode cache (2 x 4 GiB)")
    q5, k5, v5, _ = inputs.make_inputs(5)
    q5, k5, v5 = q5.to(dev), k5.to(dev), v5.to(dev)
    S = c5["num_splits"]
    B5, Hq5, Hkv5, Nk5, d5 = c5["B"], c5["Hq"], c5["Hkv"], c5["Nk"], c5["d"]
    op = torch.empty((B5, Hq5, S, d5), dtype=torch.float32, device=dev)
    lp = torch.empty((B5, Hq5, S), dtype=torch.float32, device=dev)
    o5 = torch.empty_like(q5)
    l5 = torch.empty((B5, Hq5, 1), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.fa_fwd(q3, k3, v3, causal=True, out=o3, lse=l3)
        if ev is not None:
            ev[1].record(stream)
        fa.fa_decode_splitkv(q5, k5, v5, num_splits=S, o_part=op, lse_part=lp)
        if ev is not None:
            ev[2].record(stream)
        fa.fa_lse_merge(op, lp, dtype=torch.bfloat16, out=o5, lse=l5)
        if ev is not None:
            ev[3].record(stream)

    log(f"warmup: at least {args.warmup} steps and {WARM_S} s")
    warm_calls, warm_s = warm(step, seconds=WARM_S, min_calls=args.warmup)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [e[0].elapsed_time(e[1]) for e in events]
    split_ms = [e[1].elapsed_time(e[2]) for e in events]
    merge_ms = [e[2].elapsed_time(e[3]) for e in events]
    dec_ms = [a + b for a, b in zip(split_ms, merge_ms)]

    log("measured ceilings")
    ceil = ceilings(dev, stream, k5)
    mfma_ceiling = ceil["mfma_bf16"]["value"]
    hbm_ceiling = ceil["hbm_read"]["value"]

    f_fwd = prefill_flops(c3["B"], c3["Hq"], c3["Nq"], c3["Nk"], c3["d"], True)
    main = mfma_leg(fwd_ms, f_fwd, "fwd_bf16_pp_kernel<causal>", "prefill fwd B=1 H=32 N=8192 d=128 causal bf16",
                    mfma_ceiling, load_util("fwd_bf16_pp_kernel"), load_traffic("fwd_bf16_pp_kernel"))
    fwd_tflops = main["value"]
    dbytes = decode_bytes(B5, Hq5, Hkv5, Nk5, d5)
    dst = stats_ms(dec_ms)
    dec_gbs = dbytes / (dst["mean_ms"] * 1e-3) / 1e9
    sst = stats_ms(split_ms)
    split_gbs = (dbytes - B5 * Hq5 * d5 * 2 - B5 * Hq5 * 4) / (sst["mean_ms"] * 1e-3) / 1e9

    side = {}
    n_side = args.side_steps
    if n_side > 0:
        # ---- d=64 self-attention (B=2, H=16, N=2048), causal and not
        c2 = inputs.CONFIGS[2]
        q2, k2, v2 = [t.to(dev) for t in inputs.make_inputs(2)[:3]]
        o2, l2 = torch.empty_like(q2), torch.empty(q2.shape[:3], dtype=torch.float32, device=dev)
        side["prefill_d64"] = {}
        d64_key = {True: "fwd_bf16_kernel_d64", False: "fwd_bf16_pp_kernel_d64"}
        for causal in (True, False):
            call = lambda: fa.fa_fwd(q2, k2, v2, causal=causal, out=o2, lse=l2)  # noqa: E731
            warm(call)
            ms = time_calls(call, n_side, stream)
            fl = prefill_flops(c2["B"], c2["Hq"], c2["Nq"], c2["Nk"], c2["d"], causal)
            name = "causal" if causal else "non_causal"
            side["prefill_d64"][name] = mfma_leg(
                ms, fl, "fwd_bf16_kernel<64,causal> (256 ping-pong work-groups would not fill two per CU)"
                if causal else "fwd_bf16_pp_kernel<64,non-causal>",
                f"prefill fwd B=2 H=16 N=2048 d=64 {'causal' if causal else 'non-causal'} bf16", mfma_ceiling,
                load_util(d64_key[causal]), load_traffic(d64_key[causal]))
            log(f"d64 {name}: {side['prefill_d64'][name]['value']} TFLOP/s")
        del q2, k2, v2, o2, l2

        # ---- padded GQA (B=4, Hq=32, Hkv=8, N=4096, d=128, causal, lengths U{2048..4096})
        c4 = inputs.CONFIGS[4]
        q4, k4, v4, lens4 = [t.to(dev) for t in inputs.make_inputs(4)]
        o4, l4 = torch.empty_like(q4), torch.empty(q4.shape[:3], dtype=torch.float32, device=dev)
        call = lambda: fa.fa_fwd(q4, k4, v4, causal=True, kv_seqlens=lens4, out=o4, lse=l4)  # noqa: E731
        warm(call)
        ms = time_calls(call, n_side, stream)
        L4 = lens4.cpu().tolist()
        fl = padded_causal_flops(c4["Hq"], c4["Nq"], L4, c4["d"])
        side["prefill_gqa_padded"] = mfma_leg(
            ms, fl, "fwd_bf16_pp_kernel<causal,padded>",
            f"prefill fwd B=4 Hq=32 Hkv=8 N=4096 d=128 causal bf16, kv lengths {L4}", mfma_ceiling,
            load_util("fwd_bf16_pp_kernel_padded"), load_traffic("fwd_bf16_pp_kernel_padded"))
        log(f"gqa padded: {side['prefill_gqa_padded']['value']} TFLOP/s")
        del q4, k4, v4, o4, l4

        # ---- backward of the long-context prefill
        do3 = inputs.make_dout(3).to(dev)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(c3["B"], c3["Hq"], c3["Nq"], c3["d"]), dtype=torch.uint8,
                         device=dev)
        dq3, dk3, dv3 = torch.empty_like(q3), torch.empty_like(k3), torch.empty_like(v3)
        call = lambda: fa.fa_bwd(q3, k3, v3, o3, l3, do3, causal=True, workspace=ws, dq=dq3, dk=dk3, dv=dv3)  # noqa: E731
        warm(call)
        ms = time_calls(call, n_side, stream)
        f_bwd = 2.5 * f_fwd
        bwd = mfma_leg(ms, f_bwd, "bwd kernels (fa_bwd)",
                       "backward of prefill B=1 H=32 N=8192 d=128 causal bf16 (dQ, dK, dV)", mfma_ceiling,
                       load_util("fa_bwd"), load_traffic("fa_bwd"))
        bwd["flop_count"] = ("5 products of 2*d FLOP per visible (query, key) pair: S recomputed, dP, dV, dK, dQ "
                             "(2.5x the forward)")
        side["backward"] = bwd
        log(f"backward: {bwd['value']} TFLOP/s")
        del do3, ws, dq3, dk3, dv3

        # ---- paged decode: 16-key pages in a shuffled pool
        page = 16
        kp, vp, table = paged_copy(k5, v5, page, dev)
        lens5 = torch.full((B5,), Nk5, dtype=torch.int32, device=dev)
        wsp = torch.empty(fa.fa_decode_workspace_bytes(B5, Hq5, d5, S), dtype=torch.uint8, device=dev)
        call = lambda: fa.fa_decode_paged(q5, kp, vp, table, lens5, num_splits=S, workspace=wsp, out=o5, lse=l5)  # noqa: E731
        warm(call)
        ms = time_calls(call, n_side, stream)
        pst = stats_ms(ms)
        pbytes = dbytes + B5 * (Nk5 // page) * 4  # + the block table
        p_gbs = pbytes / (pst["mean_ms"] * 1e-3) / 1e9
        side["decode_paged"] = {
            "value": round(p_gbs, 1), "unit": "GB/s", "page_size": page, **pst,
            "workload": "split-KV decode B=64 Hq=32 Hkv=8 Nk=32768 d=128 S=16 bf16, 16-key pages in a shuffled pool",
            "algorithmic_bytes": pbytes,
            "roofline": {"bound": "hbm", "achieved": round(p_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(p_gbs / PEAK_HBM_GBS, 4), "measured_ceiling": hbm_ceiling,
                         "frac_of_measured_ceiling": round(p_gbs / hbm_ceiling, 4),
                         "traffic": load_traffic("decode_paged+lse_merge_kernel")}}
        log(f"paged decode: {p_gbs:.1f} GB/s")
        del kp, vp, wsp

        # ---- packed (variable-length) and chunked prefill, the GQA length mix
        varlen = {}
        lens = inputs.lengths(4, 4, 2048, 4096).tolist()
        for name, lq in (("packed", lens), ("chunked", [512] * len(lens))):
            qv, kv_, vv, cq, ck = (t.to(dev) for t in inputs.make_packed(4, lq, lens, 32, 8, 128))
            ov = torch.empty_like(qv)
            lv = torch.empty(qv.shape[:2], dtype=torch.float32, device=dev)
            mq = max(lq)
            call = lambda: fa.fa_fwd_varlen(qv, kv_, vv, cq, ck, mq, causal=True, out=ov, lse=lv)  # noqa: E731
            warm(call)
            ms = time_calls(call, n_side, stream)
            fl = sum(prefill_flops(1, 32, a, b, 128, True) for a, b in zip(lq, lens))
            varlen[name] = mfma_leg(
                ms, fl, "fwd_bf16_pp_kernel<causal,packed>",
                f"fa_fwd_varlen Hq=32 Hkv=8 d=128 causal bf16, key lengths {lens}, query lengths {lq}",
                mfma_ceiling, load_util("fwd_bf16_pp_kernel_packed") if name == "packed" else None,
                load_traffic("fwd_bf16_pp_kernel_packed") if name == "packed" else None)
            log(f"varlen {name}: {varlen[name]['value']} TFLOP/s")
            del qv, kv_, vv, ov, lv
        side["prefill_varlen"] = varlen

        # ---- FP8 (E4M3) prefill on the long-context shape
        q8, k8, v8, _, ds8 = inputs.make_fp8_inputs(3, "e4m3")
        q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)
        call = lambda: fa.fa_fwd_fp8(q8, k8, v8, *ds8, causal=True, out=o3, lse=l3)  # noqa: E731
        warm(call)
        ms = time_calls(call, n_side, stream)
        fp8 = mfma_leg(ms, f_fwd, "fwd_fp8_pp_kernel<e4m3,causal>",
                       "fa_fwd_fp8 E4M3 B=1 H=32 N=8192 d=128 causal (per-tensor descales), bf16 output",
                       None, load_util("fwd_fp8_pp_kernel"), load_traffic("fwd_fp8_pp_kernel"), peak=PEAK_FP8_TFLOPS)
        fp8["roofline"]["peak_note"] = "dense FP8 matrix-core peak; Q.K^T runs on FP8, P.V on bf16 matrix cores"
        fp8["roofline"]["mixed_peak"] = round(PEAK_FP8_BF16_MIX_TFLOPS, 1)
        fp8["roofline"]["frac_of_mixed_peak"] = round(fp8["value"] / PEAK_FP8_BF16_MIX_TFLOPS, 4)
        side["prefill_fp8"] = fp8
        log(f"fp8 prefill: {fp8['value']} TFLOP/s")
        del q8, k8, v8

        # ---- the headline kernel and shape on all-zero Q, K, V: the same instruction stream and
        # schedule, but operands that toggle no bits, so the chip holds a higher clock.  A check of
        # the power limit, not a workload: the metric above stays on the N(0,1) inputs.
        z3 = torch.zeros_like(q3)
        call = lambda: fa.fa_fwd(z3, z3, z3, causal=True, out=o3, lse=l3)  # noqa: E731
        warm(call, seconds=WARM_S)
        ms = time_calls(call, n_side, stream)
        zero = mfma_leg(ms, f_fwd, "fwd_bf16_pp_kernel<causal>",
                        "prefill fwd B=1 H=32 N=8192 d=128 causal bf16 on all-zero Q, K, V (power-limit check)",
                        None, load_util("fwd_bf16_pp_kernel_zero_operands"), None)
        zero["ratio_to_headline"] = round(zero["value"] / fwd_tflops, 4)
        zero["note"] = ("same kernel, shape and launch as the headline on operands that toggle no bits; the "
                        "speed-up over the N(0,1) inputs is the clock the chip's power limit takes away")
        side["prefill_zero_operands"] = zero
        log(f"prefill on zero operands: {zero['value']} TFLOP/s")
        del z3

    rec = {
        "metric": METRIC,
        "value": fwd_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_s": round(warm_s, 3),
        "warmup_steps_run": warm_calls,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs; no dataset)",
        "config": {
            "workload": "prefill fwd B=1 H=32 N=8192 d=128 causal bf16 + split-KV decode B=64 Hq=32 Hkv=8 "
                        "Nk=32768 d=128 S=16 bf16",
            "prefill": {"B": 1, "H": 32, "N": 8192, "d": 128, "causal": True, "mult": c3["mult"]},
            "decode": {"B": B5, "Hq": Hq5, "Hkv": Hkv5, "Nk": Nk5, "d": d5, "num_splits": S},
        },
        "roofline": {**main["roofline"], "flop_per_launch": f_fwd, "avg_launch_ms": main["mean_ms"]},
        "prefill_timing": {k: main[k] for k in ("mean_ms", "median_ms", "min_ms", "p90_ms", "launches")},
        "decode": {
            "value": round(dec_gbs, 1),
            "unit": "GB/s",
            "frac_of_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": dbytes,
            **dst,
            "split": stats_ms(split_ms),
            "merge": stats_ms(merge_ms),
            "split_kernel_gbs": round(split_gbs, 1),
            "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(dec_gbs / PEAK_HBM_GBS, 4), "measured_ceiling": hbm_ceiling,
                         "frac_of_measured_ceiling": round(dec_gbs / hbm_ceiling, 4),
                         "traffic": load_traffic("decode_splitkv_bf16_kernel+lse_merge_kernel")},
        },
        "measured_ceilings": ceil,
        **side,
        "device": {"name": props.name, "cus": props.multi_processor_count},
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        log(f"timing the oracle on {args.cpu_heads} heads")
        rec["cpu_baseline"] = cpu_baseline(args.cpu_heads)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
