#!/usr/bin/env python3
"""Benchmark of the ConvRot INT8 linear layer on one MI355X (gfx950).

Headline (one JSON line on stdout): the fused forward ``convrot_linear_fwd``
(online rotation + per-row activation quantization + int8 MFMA GEMM +
dequantizing epilogue) on the attention-projection workload, M = K = N = 4096
tokens x features, in TOPS = 2*M*N*K / wall time per call, with the weight
quantized beforehand (load time).  A "step" is one such call on inputs already
resident in HBM.

The same line carries
  * ``roofline``: the dominant kernel (the int8 GEMM with its epilogue) timed
    alone with HIP events on its stream, against the 5.0 POP/s dense-int8 MFMA
    peak; ``traffic`` comes from committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    counters when they were taken on the current kernel source, else null;
  * ``cpu_baseline``: the CPU oracle (plain C, OpenMP) on the full forward of
    the same workload on this host, and ``cpu_baselines``: the oracle on the
    other workloads (tiny layer in full on all threads and on one; bounded row
    samples of the MLP pair, of one packed-stream layer extrapolated to the
    252-layer pass, and of the embedding's quantizer and lookup);
  * ``extra``: the other hot-path kernels on their workloads (load-time and
    embedding quantizers, lookup, both input-gradient modes, the MLP pair, the
    252-linear packed stream and the text encoder's quantization pass).

HBM figures: the embedding quantizer moves 3 GB per call, far beyond the
256 MB last-level cache.  The lookup (~0.4 GB per call) is timed in batches of
four calls over four different id sets, each batch after a 1 GiB reduction
that reads past the cache, so its code rows come from HBM; its back-to-back
rate is reported beside it.  Both are also given as a fraction of what a plain
streaming kernel reaches for the same read/write mix on this GPU (writes stream
markedly slower than reads), measured in the same run.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only all|fwd|kernels|copy|ceilings]
(kernels: the hot kernels a few times each, for counter runs; copy: three 1 GiB
device copies, the counters' calibration; ceilings: the HBM streaming rates, the
LDS read rate per CU and the sustained int8 / bf16 MFMA rates, as one JSON line.)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E

METRIC = "fused ConvRot INT8 linear TOPS (M=K=N=4096) and % of MI355X INT8 MFMA peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clocks ramp up over the first ~35 ms of continuous work (one
    # linear_fwd call takes ~112 us cold and ~83 us once ramped), so the default
    # warmup covers ~80 ms of calls and the timed region is long enough to be
    # insensitive to the ramp's tail.
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--only", default="all",
                    choices=["all", "fwd", "copy", "kernels", "ceilings", "overlap"],
                    help="fwd: headline only; copy: a plain 1 GiB device copy (calibrates "
                         "the FETCH_SIZE / WRITE_SIZE counters against known bytes); kernels: "
                         "each hot kernel a few times on its workload and the copy, for "
                         "rocprofv3 kernel traces and counter passes; overlap: the forward with "
                         "the activation quantizer of one row chunk beside the GEMM of the "
                         "previous one on a second stream, against the two-launch call")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def warm_up(torch, fn, min_calls, min_s=0.1):
    """At least `min_calls` calls and at least `min_s` seconds of back-to-back
    calls (batches of calls, one synchronization each): the clocks ramp over the
    first ~35 ms of continuous work, so every timing starts from ramped clocks."""
    t0 = time.perf_counter()
    n = 0
    while n < min_calls or time.perf_counter() - t0 < min_s:
        for _ in range(max(1, min(min_calls, 16))):
            fn()
            n += 1
        torch.cuda.synchronize()
    return n


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the ConvRot linear runs on a single MI355X here "
              "(token-parallel sharding needs no collective and is not exercised); "
              "run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import w8a8_rotated_int8_amd as cr
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cr.lib()

    if args.only == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied 3 x 1 GiB (counter calibration: 1073741824 bytes read and written per copy)")
        return

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.only == "kernels":
        profile_kernels(cr, torch, dev, wl, to_dev)
        return

    if args.only == "overlap":
        print(json.dumps(bench_overlap(cr, torch, dev, wl)), flush=True)
        return

    if args.only == "ceilings":
        print(json.dumps({"hbm_stream_ceiling_GBps": hbm_ceiling(torch, dev),
                          "lds_read_B_per_clk_per_cu": lds_ceiling(torch, dev),
                          "mfma_sustained": mfma_ceiling(torch, dev)}), flush=True)
        return

    def time_ms(fn, warmup, iters, min_warm_s=0.08):
        # warmed up to ramped clocks even after host-side setup
        warm_up(torch, fn, warmup, min_warm_s)
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(iters):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / iters

    def dev_normal(shape, sigma, seed, outlier_cols=None):
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        v = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
        if sigma != 1.0:
            v.mul_(sigma)
        if outlier_cols is not None:
            v[:, torch.from_numpy(outlier_cols).to(dev)] *= wl.OUTLIER_GAIN
        return v.to(torch.bfloat16)

    # ------------------------------------------------------------------
    # headline: attention projection, M = K = N = 4096
    # ------------------------------------------------------------------
    log("[bench] generating the attention-projection workload (seeded, numpy recipe)")
    a = wl.attn(0)
    M, K, N = a["M"], a["K"], a["N"]
    x = to_dev(a["x"])
    w = to_dev(a["w"])
    qw, sw = cr.quantize_weight(w)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(cr.workspace_bytes(cr.OP_LINEAR_FWD, M, N, K), dtype=torch.uint8, device=dev)
    ops = 2.0 * M * N * K

    def step():
        cr.linear_fwd(x, qw, sw, out=y, workspace=ws)

    nw = warm_up(torch, step, args.warmup, 0.1)
    log(f"[bench] headline: {nw} warmup calls (>= {args.warmup} and >= 100 ms) + {args.steps} "
        f"timed linear_fwd calls")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    tops = ops / (ms_step * 1e-3) / 1e12
    log(f"[bench] linear_fwd {ms_step * 1e3:.1f} us/call  {tops:.1f} TOPS  "
        f"({100 * tops / PEAK_INT8_TOPS:.1f}% of int8 peak; host wall {wall * 1e6 / args.steps:.1f} us)")

    # dominant kernel alone: int8 GEMM + dequantizing epilogue
    qx, sx = cr.quantize_act(x)
    y2 = torch.empty_like(y)
    iters = max(args.steps, 100)
    gemm_ms = time_ms(lambda: cr.gemm_i8_bf16(qx, sx, qw, sw, out=y2), args.warmup, iters)
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    aq_ms = time_ms(lambda: cr.quantize_act(x), args.warmup, iters)
    aq_bytes = M * K * 2 + M * K + 4 * M
    log(f"[bench] gemm kernel {gemm_ms * 1e3:.1f} us ({gemm_tops:.1f} TOPS); act quant "
        f"{aq_ms * 1e3:.1f} us ({aq_bytes / (aq_ms * 1e-3) / 1e9:.0f} GB/s, MALL-resident)")

    roofline = {
        "bound": "mfma", "achieved": round(gemm_tops, 1), "peak": PEAK_INT8_TOPS, "unit": "TOPS",
        "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
        "traffic": counter_traffic("gemm_i8_attn_4096_pmc.json", ["gemm.hip", "common.h"]),
        "kernel": "gemm_kernel<dequant-bf16> (int8 MFMA 32x32x32)", "avg_launch_us": round(gemm_ms * 1e3, 2),
        "algorithmic_ops_per_launch": ops,
    }

    extra = {
        "linear_fwd_us": round(ms_step * 1e3, 2),
        "linear_fwd_pct_int8_peak": round(100 * tops / PEAK_INT8_TOPS, 2),
        "gemm_kernel_us": round(gemm_ms * 1e3, 2),
        "act_quant_us": round(aq_ms * 1e3, 2),
        "act_quant_GBps_mall_resident": round(aq_bytes / (aq_ms * 1e-3) / 1e9, 1),
    }
    # the same GEMM and call against the matrix cores' sustained rate on this
    # chip (register operands, no memory traffic), beside the datasheet peak
    mc = mfma_ceiling(torch, dev)
    extra["mfma_sustained"] = mc
    for d in ("codes", "random"):
        extra[f"gemm_pct_of_sustained_int8_{d}"] = round(100 * gemm_tops / mc[f"int8_{d}_TOPS"], 1)
        extra[f"linear_fwd_pct_of_sustained_int8_{d}"] = round(100 * tops / mc[f"int8_{d}_TOPS"], 1)
    wq_ms = time_ms(lambda: cr.quantize_weight(w, out=(qw, sw)), 3, 20)
    extra["weight_quant_attn_us"] = round(wq_ms * 1e3, 2)
    # the same forward with a rank-16 LoRA branch on the unrotated input
    lw = wl.lora_weights(K, N, 16, 0)
    la, lb = to_dev(lw["a"]), to_dev(lw["b"])
    ws_l = torch.empty(cr.workspace_bytes(cr.OP_LINEAR_FWD_LORA, M, N, K, 16), dtype=torch.uint8,
                       device=dev)
    lora_ms = time_ms(lambda: cr.linear_fwd_lora(x, qw, sw, la, lb, 1.0, out=y, workspace=ws_l), 10, 200)
    ld_ms = time_ms(lambda: cr.lora_down(x, la), 10, 200)
    extra["lora16_fwd_us"] = round(lora_ms * 1e3, 2)
    extra["lora16_fwd_tops"] = round(ops / (lora_ms * 1e-3) / 1e12, 1)
    extra["lora16_down_us"] = round(ld_ms * 1e3, 2)
    log(f"[bench] with a rank-16 LoRA branch: {lora_ms * 1e3:.1f} us/call "
        f"(down projection alone {ld_ms * 1e3:.1f} us)")
    if args.only == "all":
        extra.update(bench_vs_bf16(cr, torch, time_ms, x, w, qw, sw, ms_step))
    del x, w, ws, y, y2, qx, sx

    if args.only == "all":
        extra.update(bench_qkv(cr, torch, dev, dev_normal, time_ms, wl))
        extra.update(bench_small_m(cr, torch, dev, dev_normal, time_ms, wl))
        extra.update(bench_embedding(cr, torch, dev, dev_normal, time_ms, wl))
        extra.update(bench_mlp(cr, torch, dev, dev_normal, time_ms, wl))
        for k in ("mlp_down_dx_bf16_tops", "mlp_up_dx_bf16_tops"):
            extra[k.replace("_tops", "_pct_of_sustained_bf16")] = round(
                100 * extra[k] / mc["bf16_random_TFLOPS"], 1)
        extra.update(bench_packed(cr, torch, dev, dev_normal, time_ms, wl))
        extra.update(bench_text_encoder_quant(cr, torch, dev, dev_normal, wl))
        extra.update(bench_vendor_int8(torch, dev, time_ms, extra.get("gemm_kernel_us")))

    cpu = cpu_lines = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(a)
        if args.only == "all":
            cpu_lines = cpu_baselines(wl)

    out = {
        "metric": METRIC, "value": round(tops, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "attention projection: x bf16 [4096 tokens, 4096] ~N(0,1) with 41 "
                               "outlier channels x50, W bf16 [4096, 4096] ~N(0,0.02), block 128; "
                               "fused forward, weight pre-quantized",
                   "M": M, "K": K, "N": N, "block": 128},
        "roofline": roofline, "cpu_baseline": cpu, "cpu_baselines": cpu_lines, "extra": extra,
    }
    print(json.dumps(out), flush=True)


def source_hash(files):
    """sha256 over the named kernel sources (csrc/), in the given order."""
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "w8a8_rotated_int8_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def counter_traffic(record, sources, key="hbm_bytes_per_launch"):
    """HBM bytes (per launch, or the record's other `key`) from a committed
    rocprofv3 counter summary (profiles/<record>), if it was taken on the
    current source of the kernel; else None."""
    p = os.path.join(ROOT, "profiles", record)
    try:
        rec = json.load(open(p))
        if rec.get("source_sha256") == source_hash(sources):
            return rec.get(key)
    except (OSError, ValueError):
        pass
    return None


def bench_vs_bf16(cr, torch, time_ms, x, w, qw, sw, fwd_ms):
    """The comparison the pages make for the DiT forward (sd-scripts pull request
    2461, Verification: bf16, the ConvRot int8 path, and the eager fallback that
    dequantizes and then runs the bf16 GEMM), here for one attention-projection
    layer on this chip: the vendor bf16 GEMM (torch.mm through hipBLASLt) on the
    bf16 weight; the fallback as this library's transient dequantization
    (W_hat^T, bf16) followed by that GEMM; and the fused int8 forward.  Device
    times from graph replays: called eagerly, torch.mm spends more time on the
    host than its kernel takes, which would leave the GPU idle between calls.
    Context, not part of the layer."""
    M, K = x.shape
    N = w.shape[0]
    wt = w.t().contiguous()
    what_t = cr.dequant_weight_t(qw, sw)
    yb = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    ws = torch.empty(cr.workspace_bytes(cr.OP_LINEAR_FWD, M, N, K), dtype=torch.uint8,
                     device=x.device)

    def fallback():
        cr.dequant_weight_t(qw, sw, out=what_t)
        torch.mm(x, what_t, out=yb)

    bf16_ms = time_graph_ms(torch, lambda: torch.mm(x, wt, out=yb))
    # the same GEMM on the dequantized weight alone (the fallback's GEMM)
    mm_hat_ms = time_graph_ms(torch, lambda: torch.mm(x, what_t, out=yb))
    fb_ms = time_graph_ms(torch, fallback)
    int8_ms = time_graph_ms(torch, lambda: cr.linear_fwd(x, qw, sw, out=y, workspace=ws))
    eager_ms = time_ms(lambda: torch.mm(x, wt, out=yb), 3, 50)
    r = {
        "vendor_bf16_gemm_4096_us": round(bf16_ms * 1e3, 2),
        "vendor_bf16_gemm_4096_tflops": round(2.0 * M * N * K / (bf16_ms * 1e-3) / 1e12, 1),
        "vendor_bf16_gemm_4096_eager_us": round(eager_ms * 1e3, 2),
        "vendor_bf16_gemm_on_w_hat_4096_us": round(mm_hat_ms * 1e3, 2),
        "dequant_fallback_4096_us": round(fb_ms * 1e3, 2),
        "fused_int8_fwd_graph_us": round(int8_ms * 1e3, 2),
        "fused_int8_over_bf16_time": round(int8_ms / bf16_ms, 3),
        "dequant_fallback_over_bf16_time": round(fb_ms / bf16_ms, 3),
    }
    log(f"[bench] one 4096^3 layer, device time: bf16 GEMM {bf16_ms * 1e3:.1f} us "
        f"({mm_hat_ms * 1e3:.1f} us on W_hat; {eager_ms * 1e3:.1f} us per eager call), "
        f"dequantize + bf16 GEMM {fb_ms * 1e3:.1f} us, fused int8 forward {int8_ms * 1e3:.1f} us "
        f"({fwd_ms * 1e3:.1f} us eager)")
    return r


def bench_vendor_int8(torch, dev, time_ms, gemm_us):
    """Reference only, not part of the layer: the vendor library's int8 GEMM
    (torch._int_mm through hipBLASLt, int32 output, no epilogue) at 4096^3 and at
    8192^3, where it runs fastest among the shapes tried.  Its rate is the
    practical int8 ceiling of the chip under load, beside the datasheet peak."""
    r = {}
    for n in (4096, 8192):
        a = torch.randint(-127, 128, (n, n), dtype=torch.int8, device=dev)
        b = torch.randint(-127, 128, (n, n), dtype=torch.int8, device=dev)
        bt = b.t()
        ms = time_ms(lambda: torch._int_mm(a, bt), 3, 20)
        r[f"vendor_int8_gemm_{n}_us"] = round(ms * 1e3, 2)
        r[f"vendor_int8_gemm_{n}_tops"] = round(2 * n ** 3 / (ms * 1e-3) / 1e12, 1)
        del a, b, bt
    if gemm_us:
        ours = 2 * 4096 ** 3 / (gemm_us * 1e-6) / 1e12
        r["gemm_pct_of_vendor_best_tops"] = round(100 * ours / r["vendor_int8_gemm_8192_tops"], 1)
    log(f"[bench] vendor int8 GEMM (reference): 4096^3 {r['vendor_int8_gemm_4096_us']} us, "
        f"8192^3 {r['vendor_int8_gemm_8192_tops']} TOPS")
    return r


def profile_kernels(cr, torch, dev, wl, to_dev):
    """A short run of each hot kernel on its workload, for rocprofv3 (kernel
    traces and FETCH_SIZE / WRITE_SIZE passes): the attention forward (act
    quantizer + int8 GEMM) x 5, the 248320-row embedding quantization x 2
    (8192-row chunks), the 32768-id lookup x 4 over four id sets, and one 1 GiB
    device copy whose bytes are known (counter calibration)."""
    import numpy as np
    a = wl.attn(0)
    x, w = to_dev(a["x"]), to_dev(a["w"])
    qw, sw = cr.quantize_weight(w)
    y = torch.empty((a["M"], a["N"]), dtype=torch.bfloat16, device=dev)
    for _ in range(5):
        cr.linear_fwd(x, qw, sw, out=y)
    torch.cuda.synchronize()
    del x, w, y
    V, D, CH = wl.EMBED_V, wl.EMBED_D, wl.EMBED_CHUNK
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    E = (torch.randn((V, D), generator=g, device=dev) * wl.SIGMA_W).to(torch.bfloat16)
    qe = torch.empty((V, D), dtype=torch.int8, device=dev)
    se = torch.empty((V,), dtype=torch.float32, device=dev)
    for _ in range(2):
        cr.quantize_weight(E, chunk_rows=CH, out=(qe, se))
    torch.cuda.synchronize()
    del E
    ids0 = wl.embed_ids(0)
    out = torch.empty((wl.EMBED_T, D), dtype=torch.bfloat16, device=dev)
    for j in range(4):
        ids = torch.from_numpy(((ids0.astype(np.int64) + j * (V // 4)) % V).astype(np.int32)).to(dev)
        cr.embedding_lookup(ids, qe, se, out=out)
    torch.cuda.synchronize()
    src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    log("[bench] profiled kernels: forward 4096^3 x5, embedding quantization x2, lookup x4, "
        "1 GiB copy x1 (1073741824 bytes read and written)")


def hbm_ceiling(torch, dev):
    """Practical HBM rate of a plain streaming kernel (libhbm_probe.so, built
    from w8a8_rotated_int8_amd/probe/) for the read/write mixes of the layer's
    memory-bound kernels, in GB/s of bytes moved: reads only, one read per two
    writes (the lookup), one per one (a copy) and two per one (the quantizer).
    1 GiB of output per call, the best of three grid sizes, median of 8 calls."""
    import ctypes as C
    lib = C.CDLL(os.path.join(ROOT, "w8a8_rotated_int8_amd", "libhbm_probe.so"))
    lib.hbm_probe_stream.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int, C.c_int, C.c_void_p]
    lib.hbm_probe_stream.restype = C.c_int
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    src = torch.ones(2 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    moved = {0: 1.0, 1: 1.5, 2: 2.0, 3: 3.0}  # bytes moved per output byte
    names = {0: "read_only", 1: "read1_write2", 2: "read1_write1", 3: "read2_write1"}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for mix in (0, 1, 2, 3):
        best = 0.0
        for mult in (4, 8, 16):
            ts = []
            for it in range(10):
                e0.record()
                rc = lib.hbm_probe_stream(C.c_void_p(src.data_ptr()), C.c_void_p(dst.data_ptr()),
                                          1 << 30, mix, n_cu * mult, stream)
                e1.record()
                torch.cuda.synchronize()
                if rc != 0:
                    raise RuntimeError("hbm_probe_stream failed")
                if it >= 2:
                    ts.append(e0.elapsed_time(e1))
            ms = sorted(ts)[len(ts) // 2]
            best = max(best, moved[mix] * (1 << 30) / (ms * 1e-3) / 1e9)
        out[names[mix]] = round(best, 1)
    del src, dst
    log(f"[bench] HBM streaming ceiling (GB/s): {out}")
    return out


def lds_ceiling(torch, dev):
    """LDS read rate of one CU in bytes per shader clock (libhbm_probe.so's
    lds_probe_read: each wave streams 16-byte reads; cycles from the shader
    cycle counter between two barriers), for 1 to 16 waves per CU, one
    workgroup per CU.  Median over the CUs of the second of two launches."""
    import ctypes as C
    lib = C.CDLL(os.path.join(ROOT, "w8a8_rotated_int8_amd", "libhbm_probe.so"))
    lib.lds_probe_read.argtypes = [C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
    lib.lds_probe_read.restype = C.c_int
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(n_cu * 1024 * 16, dtype=torch.uint8, device=dev)
    cyc = torch.zeros(n_cu, dtype=torch.int64, device=dev)
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    steps = 2000
    out = {}
    for waves in (1, 2, 4, 8, 16):
        for _ in range(2):
            if lib.lds_probe_read(64 * waves, steps, n_cu, C.c_void_p(sink.data_ptr()),
                                  C.c_void_p(cyc.data_ptr()), stream) != 0:
                raise RuntimeError("lds_probe_read failed")
        torch.cuda.synchronize()
        c = sorted(cyc.tolist())[n_cu // 2]
        out[f"{waves}_waves"] = round(64 * waves * 16 * 8 * steps / c, 1)
    del sink, cyc
    log(f"[bench] LDS read rate per CU (B/clk): {out}")
    return out


def mfma_ceiling(torch, dev):
    """Sustained matrix-core rate (libhbm_probe.so's mfma_probe_run): every
    SIMD issues back-to-back independent MFMAs on register operands, four waves
    per SIMD, no memory traffic, ~10 ms per launch after at least 200 ms of the
    same load.  The chip lowers its clock to stay within its power limit, and
    how far depends on how many operand bits switch, so the int8 form runs with
    random bytes, with code-like bytes (the spread of per-row int8 codes) and
    with zero operands (no switching: the datasheet rate at full clock); the
    bf16 form with random mantissas.  Median of five timed launches; the clock
    is the median over workgroups of shader cycles against the 100 MHz
    real-time counter."""
    import ctypes as C
    lib = C.CDLL(os.path.join(ROOT, "w8a8_rotated_int8_amd", "libhbm_probe.so"))
    lib.mfma_probe_run.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p,
                                   C.c_void_p]
    lib.mfma_probe_run.restype = C.c_int
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks, threads, steps = 2 * n_cu, 512, 20000
    sink = torch.empty(blocks * threads * 64, dtype=torch.uint8, device=dev)
    stamps = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def launch(kind):
        if lib.mfma_probe_run(kind, threads, steps, blocks, C.c_void_p(sink.data_ptr()),
                              C.c_void_p(stamps.data_ptr()), stream) != 0:
            raise RuntimeError("mfma_probe_run failed")

    out = {}
    for kind, name, ops_each, unit in ((0, "int8_random", 65536, "TOPS"),
                                       (1, "int8_codes", 65536, "TOPS"),
                                       (2, "int8_zero", 65536, "TOPS"),
                                       (3, "bf16_random", 32768, "TFLOPS")):
        t_end = time.perf_counter() + 0.2
        while time.perf_counter() < t_end:
            launch(kind)
            torch.cuda.synchronize()
        ts, clocks = [], []
        for _ in range(5):
            e0.record()
            launch(kind)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
            st = stamps.view(blocks, 2).tolist()
            ghz = sorted(c / (r / 100e6) / 1e9 for c, r in st if r > 0)
            clocks.append(ghz[len(ghz) // 2])
        ms = sorted(ts)[2]
        ops = blocks * (threads // 64) * steps * 8 * ops_each
        out[f"{name}_{unit}"] = round(ops / (ms * 1e-3) / 1e12, 1)
        out[f"{name}_GHz"] = round(sorted(clocks)[2], 3)
    del sink, stamps
    log(f"[bench] sustained MFMA rate, register operands: {out}")
    return out


def bench_qkv(cr, torch, dev, dev_normal, time_ms, wl):
    """q, k, v projections of one input: three separate forwards against one
    forward on the stacked [3N, K] weight codes (one activation quantization)."""
    M, K, N = 4096, 4096, 4096
    log("[bench] shared-input q/k/v: 3 x [4096,4096] separately and stacked")
    cols = wl.outlier_columns(K, wl.n_outliers(K), 0)
    x = dev_normal((M, K), 1.0, 31, cols)
    qcat = torch.empty((3 * N, K), dtype=torch.int8, device=dev)
    scat = torch.empty((3 * N,), dtype=torch.float32, device=dev)
    for j in range(3):
        cr.quantize_weight(dev_normal((N, K), wl.SIGMA_W, 32 + j),
                           out=(qcat[j * N:(j + 1) * N], scat[j * N:(j + 1) * N]))
    y = torch.empty((M, 3 * N), dtype=torch.bfloat16, device=dev)
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    ws = torch.empty(cr.workspace_bytes(cr.OP_LINEAR_FWD, M, 3 * N, K), dtype=torch.uint8, device=dev)

    def separate():
        for j in range(3):
            cr.linear_fwd(x, qcat[j * N:(j + 1) * N], scat[j * N:(j + 1) * N], out=ys[j], workspace=ws)

    ops = 3 * 2.0 * M * N * K
    t_sep = time_ms(separate, 10, 100)
    t_cat = time_ms(lambda: cr.linear_fwd(x, qcat, scat, out=y, workspace=ws), 10, 100)
    r = {"qkv_separate_us": round(t_sep * 1e3, 1), "qkv_separate_tops": round(ops / (t_sep * 1e-3) / 1e12, 1),
         "qkv_stacked_us": round(t_cat * 1e3, 1), "qkv_stacked_tops": round(ops / (t_cat * 1e-3) / 1e12, 1)}
    log(f"[bench] qkv {r}")
    return r


def time_graph_ms(torch, fn, calls=20, replays=50):
    """Per-call device time of fn: `calls` calls captured once in a HIP graph
    and replayed, so no host launch cost sits in the timed region.  The first
    call runs outside the capture (one-time kernel attribute set-up)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.08:
        g.replay()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * calls)


def bench_small_m(cr, torch, dev, dev_normal, time_ms, wl):
    """Text-encoder shapes: one caption (M tokens) at a time, and skinny N = 32
    outputs (few-row kernel, 128 x 128 tiles or split-K).  At these sizes one call is two or
    three kernels of a few microseconds, faster than the host issues them, so
    the device time is taken from graph replays (``_us``); back-to-back eager
    calls (``_eager_us``) show the host-bound rate."""
    r = {}
    log("[bench] small-M / skinny-N forwards")
    for (M, K, N) in ((1, 4096, 4096), (77, 4096, 4096), (300, 4096, 4096), (1000, 4096, 4096),
                      (77, 4096, 12288), (300, 4096, 12288), (77, 4096, 32), (4096, 4096, 32)):
        x = dev_normal((M, K), 1.0, 41)
        qw, sw = cr.quantize_weight(dev_normal((N, K), wl.SIGMA_W, 42))
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(cr.workspace_bytes(cr.OP_LINEAR_FWD, M, N, K), dtype=torch.uint8, device=dev)
        fwd = lambda: cr.linear_fwd(x, qw, sw, out=y, workspace=ws)
        t_eager = time_ms(fwd, 10, 200)
        t = time_graph_ms(torch, fwd)
        r[f"fwd_{M}x{K}x{N}_us"] = round(t * 1e3, 2)
        r[f"fwd_{M}x{K}x{N}_eager_us"] = round(t_eager * 1e3, 2)
        r[f"fwd_{M}x{K}x{N}_GBps_weights"] = round(N * K / (t * 1e-3) / 1e9, 1)
    log(f"[bench] small-M {r}")
    return r


def bench_embedding(cr, torch, dev, dev_normal, time_ms, wl):
    V, D, CH, T = wl.EMBED_V, wl.EMBED_D, wl.EMBED_CHUNK, wl.EMBED_T
    log(f"[bench] embedding: quantize [{V},{D}] in {CH}-row chunks, lookup {T} ids")
    E = dev_normal((V, D), wl.SIGMA_W, 5)
    qe = torch.empty((V, D), dtype=torch.int8, device=dev)
    se = torch.empty((V,), dtype=torch.float32, device=dev)
    q_ms = time_ms(lambda: cr.quantize_weight(E, chunk_rows=CH, out=(qe, se)), 2, 10)
    q_bytes = V * D * 3 + 4 * V
    del E
    ids0 = wl.embed_ids(0)
    ids = torch.from_numpy(ids0).to(dev)
    out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    l_ms = time_ms(lambda: cr.embedding_lookup(ids, qe, se, out=out), 5, 50)
    l_bytes = T * (4 + D + 4 + 2 * D)
    # from HBM: before each timed batch a 1 GiB reduction reads past the 256 MB
    # last-level cache (a read leaves no dirty lines to write back during the
    # batch); the batch is four lookups of four id sets (the recipe's ids
    # shifted by a quarter of the table each), so few rows repeat across calls
    import numpy as np
    id_sets = [torch.from_numpy(((ids0.astype(np.int64) + j * (V // 4)) % V).astype(np.int32)).to(dev)
               for j in range(4)]
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cold = []
    for _ in range(20):
        flush.sum()
        e0.record()
        for j in range(4):
            cr.embedding_lookup(id_sets[j], qe, se, out=out)
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) / 4)
    lc_ms = sorted(cold)[len(cold) // 2]
    del flush, id_sets
    # torch's 1 GiB device-to-device copy, a reference rate for streaming reads
    # and writes with ordinary stores
    src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    c_ms = time_ms(lambda: dst.copy_(src), 3, 20)
    c_GBps = 2 * (1 << 30) / (c_ms * 1e-3) / 1e9
    del src, dst
    ceil = hbm_ceiling(torch, dev)
    r = {
        "embed_quant_us": round(q_ms * 1e3, 1),
        "embed_quant_GBps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
        "embed_quant_pct_hbm": round(100 * q_bytes / (q_ms * 1e-3) / 1e9 / 8000.0, 1),
        # per quantization of the whole table (31 chunk launches)
        "embed_quant_traffic_bytes": counter_traffic("rotate_quant_embed_pmc.json",
                                                     ["rotate_quant.hip", "span_quant.h", "common.h"],
                                                     "hbm_bytes_per_call"),
        "embed_lookup_from_hbm_us": round(lc_ms * 1e3, 1),
        "embed_lookup_from_hbm_GBps": round(l_bytes / (lc_ms * 1e-3) / 1e9, 1),
        "embed_lookup_from_hbm_pct_hbm": round(100 * l_bytes / (lc_ms * 1e-3) / 1e9 / 8000.0, 1),
        "embed_lookup_traffic_bytes": counter_traffic("embedding_lookup_pmc.json",
                                                      ["dequant_lookup.hip", "common.h"]),
        "embed_lookup_back_to_back_us": round(l_ms * 1e3, 1),
        "embed_lookup_back_to_back_GBps": round(l_bytes / (l_ms * 1e-3) / 1e9, 1),
        "device_copy_GBps": round(c_GBps, 1),
        "embed_quant_pct_copy": round(100 * q_bytes / (q_ms * 1e-3) / 1e9 / c_GBps, 1),
        "embed_lookup_from_hbm_pct_copy": round(100 * l_bytes / (lc_ms * 1e-3) / 1e9 / c_GBps, 1),
        "hbm_stream_ceiling_GBps": ceil,
        "embed_quant_pct_stream_ceiling": round(
            100 * q_bytes / (q_ms * 1e-3) / 1e9 / ceil["read2_write1"], 1),
        "embed_lookup_from_hbm_pct_stream_ceiling": round(
            100 * l_bytes / (lc_ms * 1e-3) / 1e9 / ceil["read1_write2"], 1),
    }
    log(f"[bench] embedding quant {r['embed_quant_us']} us ({r['embed_quant_GBps']} GB/s), lookup "
        f"from HBM {r['embed_lookup_from_hbm_us']} us ({r['embed_lookup_from_hbm_GBps']} GB/s; "
        f"back to back {r['embed_lookup_back_to_back_us']} us); device copy {r['device_copy_GBps']} GB/s")
    return r


def bench_mlp(cr, torch, dev, dev_normal, time_ms, wl):
    import numpy as np
    M, D, F = 4096, 4096, 16384
    log("[bench] MLP pair: up [16384,4096], down [4096,16384], fwd + both dX modes")
    cols = wl.outlier_columns(D, wl.n_outliers(D), 0)
    x = dev_normal((M, D), 1.0, 11, cols)
    wu = dev_normal((F, D), wl.SIGMA_W, 12)
    wd = dev_normal((D, F), wl.SIGMA_W, 13)
    qu, su = cr.quantize_weight(wu)
    qd, sd = cr.quantize_weight(wd)
    del wu, wd
    yu = cr.linear_fwd(x, qu, su)
    h = torch.nn.functional.gelu(yu.float()).to(torch.bfloat16)
    dyd = dev_normal((M, D), wl.SIGMA_DY, 14)
    dyu = dev_normal((M, F), wl.SIGMA_DY, 15)
    ops = 2.0 * M * D * F
    r = {}
    ws_u = torch.empty(cr.workspace_bytes(cr.OP_LINEAR_FWD, M, F, D), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(cr.workspace_bytes(cr.OP_LINEAR_FWD, M, D, F), dtype=torch.uint8, device=dev)
    yd = torch.empty((M, D), dtype=torch.bfloat16, device=dev)
    t = time_ms(lambda: cr.linear_fwd(x, qu, su, out=yu, workspace=ws_u), 5, 30)
    r["mlp_up_fwd_tops"] = round(ops / (t * 1e-3) / 1e12, 1)
    t = time_ms(lambda: cr.linear_fwd(h, qd, sd, out=yd, workspace=ws_d), 5, 30)
    r["mlp_down_fwd_tops"] = round(ops / (t * 1e-3) / 1e12, 1)
    dxd = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
    dxu = torch.empty((M, D), dtype=torch.bfloat16, device=dev)
    for mode, name in ((cr.BWD_INT8, "int8"), (cr.BWD_BF16, "bf16")):
        wsd = torch.empty(cr.workspace_bytes(cr.OP_LINEAR_BWD_DX, M, D, F, mode), dtype=torch.uint8, device=dev)
        wsu = torch.empty(cr.workspace_bytes(cr.OP_LINEAR_BWD_DX, M, F, D, mode), dtype=torch.uint8, device=dev)
        t = time_ms(lambda: cr.linear_bwd_dx(dyd, qd, sd, mode, out=dxd, workspace=wsd), 3, 20)
        r[f"mlp_down_dx_{name}_tops"] = round(ops / (t * 1e-3) / 1e12, 1)
        t = time_ms(lambda: cr.linear_bwd_dx(dyu, qu, su, mode, out=dxu, workspace=wsu), 3, 20)
        r[f"mlp_up_dx_{name}_tops"] = round(ops / (t * 1e-3) / 1e12, 1)
        del wsd, wsu
    log(f"[bench] MLP {r}")
    return r


def bench_packed(cr, torch, dev, dev_normal, time_ms, wl):
    T, K, N, L = 20480, 4096, 4096, 252
    log(f"[bench] packed stream: {L} linears [{N},{K}] on {T} packed tokens, fwd + int8 dX")
    cols = wl.outlier_columns(K, wl.n_outliers(K), 0)
    x = dev_normal((T, K), 1.0, 21, cols)
    dy = dev_normal((T, N), wl.SIGMA_DY, 22)
    qws, sws = [], []
    qt_ms = 0.0
    for layer in range(L):
        w = dev_normal((N, K), wl.SIGMA_W, 1000 + layer)
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        q, sc = cr.quantize_weight(w)
        e.record()
        e.synchronize()
        qt_ms += s.elapsed_time(e)
        qws.append(q)
        sws.append(sc)
        del w
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
    wsf = torch.empty(cr.workspace_bytes(cr.OP_LINEAR_FWD, T, N, K), dtype=torch.uint8, device=dev)
    wsb = torch.empty(cr.workspace_bytes(cr.OP_LINEAR_BWD_DX, T, N, K, cr.BWD_INT8), dtype=torch.uint8, device=dev)

    def stream_pass():
        for i in range(L):
            cr.linear_fwd(x, qws[i], sws[i], out=y, workspace=wsf)
            cr.linear_bwd_dx(dy, qws[i], sws[i], cr.BWD_INT8, out=dx, workspace=wsb)

    t = time_ms(stream_pass, 1, 3)
    ops = 2 * 2.0 * T * N * K * L
    wsb16 = torch.empty(cr.workspace_bytes(cr.OP_LINEAR_BWD_DX, T, N, K, cr.BWD_BF16),
                        dtype=torch.uint8, device=dev)

    def stream_pass_bf16():
        for i in range(L):
            cr.linear_fwd(x, qws[i], sws[i], out=y, workspace=wsf)
            cr.linear_bwd_dx(dy, qws[i], sws[i], cr.BWD_BF16, out=dx, workspace=wsb16)

    t16 = time_ms(stream_pass_bf16, 1, 3)
    r = {
        "packed_fwd_dx_int8_ms_per_pass": round(t, 2),
        "packed_tokens_per_s": round(T / (t * 1e-3), 0),
        "packed_tops": round(ops / (t * 1e-3) / 1e12, 1),
        "packed_fwd_dx_bf16_ms_per_pass": round(t16, 2),
        "packed_bf16_tokens_per_s": round(T / (t16 * 1e-3), 0),
        "packed_bf16_tops": round(ops / (t16 * 1e-3) / 1e12, 1),
        "packed_weight_quant_ms_total": round(qt_ms, 2),
    }
    log(f"[bench] packed {r}")
    return r


def bench_overlap(cr, torch, dev, wl):
    """The forward with its two stages overlapped across row chunks: the rows are
    cut into C chunks; a second stream quantizes chunk c + 1 while the GEMM of
    chunk c runs, each GEMM waiting on its chunk's quantizer event.  Timed with
    events on the calling stream against the two-launch call on the same
    workspace layout, outputs compared bit for bit (same codes, same GEMM)."""
    def normal(shape, sigma, seed, cols=None):
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        v = torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * sigma
        if cols is not None:
            v[:, torch.from_numpy(cols).to(dev)] *= wl.OUTLIER_GAIN
        return v.to(torch.bfloat16)

    def timed(fn, calls=20, min_s=0.1):
        warm_up(torch, fn, 3, min_s)
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(calls):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / calls * 1e3

    out = {}
    main_s = torch.cuda.current_stream()
    qs, gs = torch.cuda.Stream(), torch.cuda.Stream()
    for name, M, K, N in (("packed_20480x4096x4096", 20480, 4096, 4096),
                          ("mlp_up_4096x4096x16384", 4096, 4096, 16384)):
        cols = wl.outlier_columns(K, wl.n_outliers(K), 0)
        x = normal((M, K), 1.0, 31, cols)
        qw, sw = cr.quantize_weight(normal((N, K), wl.SIGMA_W, 32))
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(cr.workspace_bytes(cr.OP_LINEAR_FWD, M, N, K), dtype=torch.uint8,
                         device=dev)
        qx = torch.empty((M, K), dtype=torch.int8, device=dev)
        sx = torch.empty((M,), dtype=torch.float32, device=dev)
        y2 = torch.empty_like(y)
        base = timed(lambda: cr.linear_fwd(x, qw, sw, out=y, workspace=ws))
        out[f"{name}_two_launch_us"] = round(base, 1)
        for C in (2, 4, 5, 8):
            if M % C or (M // C) % 256:
                continue
            R = M // C
            evs = [torch.cuda.Event() for _ in range(C)]

            def chunked():
                qs.wait_stream(main_s)
                gs.wait_stream(main_s)
                with torch.cuda.stream(qs):
                    for c in range(C):
                        cr.quantize_act(x[c * R:(c + 1) * R], out=(qx[c * R:(c + 1) * R],
                                                                    sx[c * R:(c + 1) * R]))
                        evs[c].record(qs)
                with torch.cuda.stream(gs):
                    for c in range(C):
                        gs.wait_event(evs[c])
                        cr.gemm_i8_bf16(qx[c * R:(c + 1) * R], sx[c * R:(c + 1) * R], qw, sw,
                                        out=y2[c * R:(c + 1) * R])
                main_s.wait_stream(gs)
                main_s.wait_stream(qs)

            def serial():
                for c in range(C):
                    cr.quantize_act(x[c * R:(c + 1) * R], out=(qx[c * R:(c + 1) * R],
                                                                sx[c * R:(c + 1) * R]))
                    cr.gemm_i8_bf16(qx[c * R:(c + 1) * R], sx[c * R:(c + 1) * R], qw, sw,
                                    out=y2[c * R:(c + 1) * R])

            out[f"{name}_chunks{C}_one_stream_us"] = round(timed(serial), 1)
            t = timed(chunked)
            torch.cuda.synchronize()
            same = bool(torch.equal(y.view(torch.int16), y2.view(torch.int16)))
            out[f"{name}_chunks{C}_us"] = round(t, 1)
            out[f"{name}_chunks{C}_bit_identical"] = same
            log(f"[bench] overlap {name}: two-launch {base:.1f} us, {C} chunks on two streams "
                f"{t:.1f} us, identical={same}")
        del x, qw, sw, y, y2, ws, qx, sx
    return out


def bench_text_encoder_quant(cr, torch, dev, dev_normal, wl):
    """The text encoder's load-time quantization pass: its 200 Linear layers (a
    stand-in for their shapes, workloads.text_encoder_linear_shapes) and the
    248320 x 4096 token embedding in 8192-row chunks, quantized back to back on
    one stream, every weight resident beforehand (~16 GB of bf16)."""
    shapes = wl.text_encoder_linear_shapes()
    V, D, CH = wl.EMBED_V, wl.EMBED_D, wl.EMBED_CHUNK
    log(f"[bench] text-encoder quantization pass: {len(shapes)} linears + [{V},{D}] embedding")
    ws = [dev_normal(tuple(sh), wl.SIGMA_W, 3000 + i) for i, sh in enumerate(shapes)]
    E = dev_normal((V, D), wl.SIGMA_W, 6)
    qs = [(torch.empty(tuple(sh), dtype=torch.int8, device=dev),
           torch.empty((sh[0],), dtype=torch.float32, device=dev)) for sh in shapes]
    qe = torch.empty((V, D), dtype=torch.int8, device=dev)
    se = torch.empty((V,), dtype=torch.float32, device=dev)

    def qpass():
        for w, out in zip(ws, qs):
            cr.quantize_weight(w, out=out)
        cr.quantize_weight(E, chunk_rows=CH, out=(qe, se))

    qpass()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(3):
        e0.record()
        qpass()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    t = sorted(times)[1]
    nbytes = sum(a * b * 3 + 4 * a for a, b in shapes) + V * D * 3 + 4 * V
    r = {"te_quant_pass_ms": round(t, 2), "te_quant_pass_GBps": round(nbytes / (t * 1e-3) / 1e9, 1),
         "te_quant_pass_pct_hbm": round(100 * nbytes / (t * 1e-3) / 1e9 / 8000.0, 1),
         "te_quant_pass_bytes": nbytes}
    log(f"[bench] text-encoder quantization {r}")
    del ws, E, qs, qe, se
    torch.cuda.empty_cache()
    return r


def cpu_baselines(wl):
    """The oracle (unmodified) on the other workloads, on bounded samples so that
    the whole set takes seconds; each line states its sample and scaling."""
    import numpy as np

    import oracle
    nthr = oracle.num_threads()
    out = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    # tiny layer: forward + both input gradients in full, median of 20 runs
    t = wl.tiny(0)
    oq, os_, _ = oracle.rotate_quantize(t["w"])
    ops1 = 3 * 2.0 * t["M"] * t["N"] * t["K"]

    def c1():
        oracle.linear_fwd(t["x"], oq, os_)
        oracle.bwd_dx_int8(t["dy"], oq, os_)
        oracle.bwd_dx_bf16(t["dy"], oq, os_)

    for threads in (nthr, 1):
        oracle.set_num_threads(threads)
        ts = sorted(timed(c1) for _ in range(20))
        dt = ts[10]
        out[f"tiny_{threads}thr"] = {
            "value": round(ops1 / dt / 1e12, 6), "unit": "TOPS", "cores": threads, "kind": "oracle",
            "ms": round(dt * 1e3, 3),
            "sample": "tiny layer in full (x [64,256], W [256,256]): forward + int8 dX + bf16 dX, "
                      "median of 20 runs"}
    oracle.set_num_threads(nthr)

    # MLP pair: 256 of the 4096 tokens through both forwards and both int8
    # gradients (weights quantized beforehand, not timed)
    rows = 64
    x = wl.activations(4096, 4096, wl.n_outliers(4096), base=0)[:rows]
    w = wl.mlp_weights(0)
    h = wl.mlp_down_input(x, w["w_up"])
    g = wl.mlp_grads(4096, 0)
    qu, su, _ = oracle.rotate_quantize(w["w_up"])
    qd, sd, _ = oracle.rotate_quantize(w["w_down"])
    del w

    def c3():
        oracle.linear_fwd(x, qu, su)
        oracle.linear_fwd(h, qd, sd)
        oracle.bwd_dx_int8(g["dy_down"][:rows], qd, sd)
        oracle.bwd_dx_int8(g["dy_up"][:rows], qu, su)

    dt = timed(c3)
    ops3 = 4 * 2.0 * rows * 4096 * 16384
    out["mlp_pair"] = {
        "value": round(ops3 / dt / 1e12, 6), "unit": "TOPS", "cores": nthr, "kind": "oracle",
        "seconds": round(dt, 2),
        "sample": f"MLP pair, {rows} of the 4096 tokens: up and down forwards + int8 dX of both "
                  "(rate per token is independent of the token count)"}
    del qu, su, qd, sd, h, g

    # packed stream: one layer's forward + int8 dX on 256 of the 20480 tokens,
    # extrapolated to the 252-layer pass over all tokens
    p = wl.packed(0)
    xs, dys = p["x"][:rows], p["dy"][:rows]
    del p
    w0 = wl.packed_weight(0, 0)
    q0, s0, _ = oracle.rotate_quantize(w0)

    def c4():
        oracle.linear_fwd(xs, q0, s0)
        oracle.bwd_dx_int8(dys, q0, s0)

    dt = timed(c4)
    scale = (20480 / rows) * 252
    out["packed_stream_extrapolated"] = {
        "value": round(20480 / (dt * scale), 3), "unit": "tokens/s", "cores": nthr, "kind": "oracle",
        "seconds_per_pass_extrapolated": round(dt * scale, 1), "extrapolated": True,
        "sample": f"one layer's forward + int8 dX on {rows} of the 20480 packed tokens, "
                  f"x {scale:.0f} for the 252-layer pass"}

    # embedding: quantize one 8192-row chunk; look up 4096 ids in that chunk
    E = wl.embed_table(0, V=8192)
    dt = timed(lambda: oracle.rotate_quantize(E))
    qb = 8192 * 4096 * 3 + 4 * 8192
    out["embed_quant_chunk"] = {
        "value": round(qb / dt / 1e9, 3), "unit": "GB/s", "cores": nthr, "kind": "oracle",
        "seconds": round(dt, 2),
        "sample": "one 8192-row chunk of the 248320 x 4096 embedding (31 such chunks)"}
    qe, se, _ = oracle.rotate_quantize(E)
    ids = wl.token_ids(4096, 8192, base=0)
    dt = timed(lambda: oracle.embedding_lookup(ids, qe, se))
    lb = 4096 * (4 + 4096 + 4 + 2 * 4096)
    out["embed_lookup"] = {
        "value": round(lb / dt / 1e9, 3), "unit": "GB/s", "cores": nthr, "kind": "oracle",
        "seconds": round(dt, 2),
        "sample": "4096 ids into one quantized 8192-row chunk (the workload looks up 32768)"}
    log(f"[bench] CPU oracle lines: " + ", ".join(f"{k} {v['value']} {v['unit']}"
                                                   for k, v in out.items()))
    return out


def cpu_baseline(a):
    import numpy as np

    import oracle
    log("[bench] CPU oracle on the full attention-projection forward")
    oq, os_, _ = oracle.rotate_quantize(a["w"])   # load time, not timed
    t0 = time.perf_counter()
    oracle.linear_fwd(a["x"], oq, os_)
    dt = time.perf_counter() - t0
    ops = 2.0 * a["M"] * a["N"] * a["K"]
    r = {"value": round(ops / dt / 1e12, 5), "unit": "TOPS", "cores": oracle.num_threads(),
         "kind": "oracle", "seconds": round(dt, 2),
         "sample": "full attention-projection forward (M=K=N=4096: rotate+quantize x, int32 "
                   "triple-loop GEMM, fp64 epilogue), weight quantized beforehand"}
    log(f"[bench] CPU oracle {dt:.1f} s -> {r['value']} TOPS on {r['cores']} threads")
    return r


if __name__ == "__main__":
    main()
