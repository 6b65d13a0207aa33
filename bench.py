"""Benchmark of the quantized attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline]
                    [--promote [--low4] | --adaptive TAU | --stripes THETA]
                    [--mask pooled|lowbit] [--patterns NV NS]

A step is one pass of the whole path over one batch of the workload's seeded
synthetic input (already resident in HBM): qattn_smooth_quant, then
qattn_block_mask for the block-sparse workload, then qattn_fwd. The default
workload is the Llama-3.1-8B-shaped causal prefill (B=1, Hq=32, Hkv=8,
N=8192, d=128, bf16).

Before the W counted warmup steps, whole steps run untimed for at least
--prewarm-ms (default 250 ms; their count is ``prewarm_steps``): under load the
GPU clock settles only after tens of milliseconds, and a handful of warmup
steps would time the transient instead of the steady state.

Prints one JSON line. ``value`` is the attention metric 4*N^2*d*H*B / step time
in TOPS (dense-equivalent operation count, the whole step in the denominator).
``roofline`` describes the dominant kernel (attn_fwd): its algorithmic
operations per launch (causal: 4*d*H*B*N(N+1)/2; sparse: 4*d*64*rows over the
kept tiles) over its average launch time, measured with HIP events on the
launch stream, against the INT8 dense matrix peak. ``cpu_baseline`` times the
CPU oracle on a bounded sample of the same workload.

With ``--promote`` the attention step is qattn_fwd_promoted: the blocks the
mask keeps (the workload's keep ratio, else first + diagonal + top 10 %) run at
16-bit Q K^T and every other visible block through the INT8 path. Its
algorithmic operations are those of the dense problem (4*d per visible pair),
of which 2*d per promoted pair and 2*d per pair for P V are 16-bit; the peak
is the matrix bound of that mix (INT8 and 16-bit work each at its own peak).
With ``--low4`` as well the call is qattn_fwd_promoted_fp4: the other blocks
take MX FP4 Q K^T (2*d per pair at the FP4 peak) instead of INT8, and the
attention launch time includes the call's MX FP4 quantization of Q and K.

With ``--mask lowbit`` the kept lists come from qattn_block_mask_lowbit (the
element-level 4-bit estimator) instead of qattn_block_mask (pooled block
means); the mask launch is part of the step either way. ``--patterns NV NS``
adds qattn_block_mask_patterns to the step: each head's NV vertical and NS
slash lines, predicted from the votes of the mask's selections, join every
query block's kept list before the attention (its pairs are counted over the
extended lists).

With ``--adaptive TAU`` the step runs qattn_head_error after the smoothing
(its per-head INT8 logit error on a fixed sample) and then qattn_fwd_adaptive:
the heads whose error exceeds TAU take 16-bit Q K^T on every block, the rest
INT8. Operations and peak are counted the same way.

With ``--stripes THETA`` the step is qattn_smooth_quant, qattn_stripe_select
(each query block keeps the first 64 keys, its own 128 positions and every key
whose pooled score comes within THETA of the anchor, up to --stripe-keys keys)
and qattn_fwd_stripes over the gathered keys. Its algorithmic operations are
4*d per visible (query, listed key) pair, against the INT8 peak as for the
dense and block-sparse paths.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0       # MI355X dense INT8 matrix peak (TOPS)
PEAK_BF16_TFLOPS = 2500.0     # dense FP16/BF16 matrix peak
PEAK_FP4_TFLOPS = 10100.0     # dense FP4 (MX) matrix peak
PEAK_HBM_GBS = 8000.0
# half the attention's operations (Q K^T) at the INT8 peak, half (P V) at the
# 16-bit peak
BLENDED_PEAK_TOPS = 1.0 / (0.5 / PEAK_INT8_TOPS + 0.5 / PEAK_BF16_TFLOPS)


# file-name slugs of the workloads (profile summaries are named after them)
SLUG = {1: "tiny_noncausal_n256", 2: "llama8b_causal_n8192", 3: "vision_noncausal_n4096",
        4: "llama8b_causal_n65536", 5: "sparse_causal_n32768"}
KERNEL_SOURCES = [os.path.join(ROOT, "bit_quantized_attention_amd", "csrc", f)
                  for f in ("attn_fwd.hip", "device_util.h", "qattn_internal.h")] + \
                 [os.path.join(ROOT, "include", "qattn.h")]


def kernel_code_hash() -> str:
    """sha256 over the attention kernel's sources with comments and blank space
    removed: it changes when the code changes, not when a comment does."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(re.sub(r"\s+", " ", text).strip().encode())
    return h.hexdigest()


def counted_traffic(cfg: int, kind: str = "attn_fwd"):
    """HBM-side bytes per attn_fwd launch from the committed counter summary of
    this workload (profiles/<kind>_<slug>_traffic.txt): FETCH_SIZE and
    WRITE_SIZE per dispatch, each scaled by what the counter reads for a plain
    copy of known size. None when there is no summary or when the kernel code
    has changed since the counters were taken (its hash is recorded)."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{SLUG[cfg]}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    if kv.get("kernel_code_sha256") != kernel_code_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(mib: int, reps: int):
    """A plain device copy of known size, run under rocprofv3 --pmc to calibrate
    FETCH_SIZE / WRITE_SIZE (each launch reads and writes mib MiB)."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": reps}))


PEAK_KINDS = [
    # (kind, param, name, unit of the rate, divisor to that unit)
    (0, 0, "mfma_i8_32x32x32", "TOPS", 1e12),
    (1, 0, "mfma_bf16_32x32x16", "TFLOP/s", 1e12),
    (2, 0, "mfma_mix_1i8_2bf16", "TOPS", 1e12),
    (14, 0, "mfma_fp4_32x32x64", "TOPS", 1e12),
    (15, 0, "mfma_fp4_32x32x64_vgpr_scales", "TOPS", 1e12),
    (3, 0, "valu_fma_f32", "G lane-instr/s", 1e9),
    (4, 0, "valu_exp_f32", "G lane-instr/s", 1e9),
    *[(5, n, f"coissue_bf16_mfma_plus_{n}_exp_1wave_per_simd", "TFLOP/s", 1e12)
      for n in (0, 2, 4, 6, 8, 12, 16)],
    *[(6, n, f"coissue_bf16_mfma_plus_{n}_fma_1wave_per_simd", "TFLOP/s", 1e12)
      for n in (2, 4, 6, 8, 12, 16)],
    *[(10, n, f"coissue_mfma16x16x32_bf16_plus_{n}_fma_1wave_per_simd", "TFLOP/s", 1e12)
      for n in (0, 1, 2, 3, 4)],
    *[(11, n, f"coissue_mfma_i8_plus_{n}_fma_1wave_per_simd", "TOPS", 1e12)
      for n in (0, 2, 4, 6, 8)],
    *[(12, n, f"split_waves_bf16_mfma_vs_{n}_fma_per_mfma", "TFLOP/s", 1e12)
      for n in (0, 2, 4, 6, 8)],
    *[(13, n, f"split_waves_bf16_mfma_vs_{n}_exp_per_mfma", "TFLOP/s", 1e12)
      for n in (2, 4, 6)],
    (7, 0, "lds_read_b128", "GB/s", 1e9),
    (8, 0, "lds_read_b64_tr_b16", "GB/s", 1e9),
    (9, 0, "hbm_copy_1gib_read_plus_write", "GB/s", 1e9),
]


def run_peaks():
    """The peak-rate micro-benchmarks of libqattn_peaks.so, one JSON line each:
    the rate, the kernel time, the shader clock under that load and the cycles
    one loop iteration of the first wave took (its own s_memtime)."""
    import ctypes
    import torch
    from bit_quantized_attention_amd import build as _b
    torch.cuda.init()
    lib = ctypes.CDLL(_b.PEAKS_LIB)
    lib.qattn_peak.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.qattn_peak.restype = ctypes.c_int
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    for kind, param, name, unit, div in PEAK_KINDS:
        res = (ctypes.c_double * 4)()
        rc = lib.qattn_peak(kind, param, res)
        if rc != 0:
            raise SystemExit(f"peak benchmark {name} failed with HIP error {rc}")
        rate, ms, ghz, cyc = res[0], res[1], res[2], res[3]
        line = {"peak": name, "rate": rate / div, "unit": unit, "kernel_ms": ms,
                "clock_ghz": ghz, "cycles_per_iteration_wave0": cyc}
        if ghz > 0:
            line["per_cu_per_clock"] = rate / (ncu * ghz * 1e9)
        print(json.dumps(line), flush=True)


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prewarm-ms", type=float, default=250.0,
                    help="untimed whole steps for at least this long before the warmup steps "
                         "(the GPU clock settles under load)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--promote", action="store_true",
                    help="promote the kept blocks to 16-bit Q K^T instead of skipping the rest")
    ap.add_argument("--low4", action="store_true",
                    help="with --promote: the blocks not promoted at MX FP4 Q K^T instead of INT8")
    ap.add_argument("--mask", choices=["pooled", "lowbit"], default="pooled",
                    help="block scores from pooled block means or element-level 4-bit estimates")
    ap.add_argument("--patterns", type=int, nargs=2, default=None, metavar=("NV", "NS"),
                    help="extend the kept lists with NV vertical and NS slash lines per head")
    ap.add_argument("--adaptive", type=float, default=None, metavar="TAU",
                    help="per-head precision: heads whose sampled INT8 logit error exceeds TAU "
                         "(log2 units) run at 16-bit Q K^T")
    ap.add_argument("--stripes", type=float, default=None, metavar="THETA",
                    help="anchor-based stripes: keep the keys whose pooled score is within THETA "
                         "of the anchor and attend over the gathered keys")
    ap.add_argument("--stripe-keys", type=int, default=3072,
                    help="capacity of a query block's stripe key list (192..3072)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--peaks", action="store_true",
                    help="only run the peak-rate micro-benchmarks (matrix, vector, LDS, HBM)")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the 64K (long-context causal) forward that the default 8K line "
                         "reports beside its own")
    return ap.parse_args(argv)


def roofline_fracs(alg_ops: float, ms: float, traffic):
    """The attention forward's rate against each bound: the INT8 matrix peak
    (the metric's fraction), the 16-bit matrix peak for its P V half, the
    blended matrix bound (half the operations at each peak) and, from the
    counted bytes, the HBM peak."""
    tops = alg_ops / (ms * 1e-3) / 1e12
    out = {"frac_int8": tops / PEAK_INT8_TOPS,
           "frac_fp16_pv_half": (tops / 2) / PEAK_BF16_TFLOPS,
           "frac_blended": tops / BLENDED_PEAK_TOPS,
           "hbm_frac": None if traffic is None else traffic / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    return out


def measure_long_context(warmup: int = 1, steps: int = 3):
    """The metric's second point: the 64K causal workload (B1 Hq32 Hkv8
    N65536 d128 bf16), smoothing + quantization, then the dense forward timed
    with events on its launch stream (outside the main timed region)."""
    import torch
    import bit_quantized_attention_amd as qa
    from synthetic import make_config
    p, t = make_config(4)
    dev = torch.device("cuda:0")
    q, k, v = (t[x].to(dev) for x in "qkv")
    del t
    plan = qa.Plan(qa.problem(p.B, p.Hq, p.Hkv, p.N, p.d, p.dtype, p.causal), dev)
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    plan.smooth_quant(q, k)
    for _ in range(warmup):
        plan.fwd(v, o)
    torch.cuda.synchronize()
    ms = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        plan.fwd(v, o)
        b.record(stream)
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    fwd = float(np.mean(ms))
    alg = dense_algorithmic_ops(p)
    literal = 4.0 * p.N * p.N * p.d * p.Hq * p.B
    traffic = counted_traffic(4)
    rec = {"workload": p.name, "N": p.N, "fwd_ms": fwd, "fwd_ms_min": float(np.min(ms)),
           "steps": steps, "fwd_tops_literal": literal / (fwd * 1e-3) / 1e12,
           "fwd_tops_algorithmic": alg / (fwd * 1e-3) / 1e12,
           "literal_frac_int8": literal / (fwd * 1e-3) / 1e12 / PEAK_INT8_TOPS,
           "traffic": traffic}
    rec.update(roofline_fracs(alg, fwd, traffic))
    del q, k, v, o, plan
    torch.cuda.empty_cache()
    return rec


def dense_algorithmic_ops(p) -> float:
    """Operations the method performs on a dense problem: 2*d per (query,
    visible key) for Q K^T and 2*d for P V (causal: key <= query)."""
    pairs = p.N * (p.N + 1) / 2 if p.causal else float(p.N) * p.N
    return 4.0 * p.d * pairs * p.Hq * p.B


def sparse_pairs(kv_idx: np.ndarray, kv_cnt: np.ndarray, causal: bool) -> float:
    """Visible (query, key) pairs under a keep list [B,Hq,nqb,mk]."""
    total = 0
    B, H, nqb, _ = kv_idx.shape
    rows = np.arange(128)
    for i in range(nqb):
        q = 128 * i + rows
        lst = kv_idx[:, :, i, :]
        cnt = kv_cnt[:, :, i]
        for j in np.unique(lst[lst >= 0]):
            keys = 64 * j + np.arange(64)
            vis = int((keys[None, :] <= q[:, None]).sum()) if causal else 128 * 64
            # number of (b, h) rows keeping block j
            n = int(((lst == j) & (np.arange(lst.shape[-1])[None, None, :] < cnt[..., None])).sum())
            total += vis * n
    return float(total)


def stripe_pairs(key_idx: np.ndarray, key_cnt: np.ndarray, causal: bool) -> float:
    """Visible (query, key) pairs under stripe key lists [B,Hq,nqb,mk]: a listed
    key k of query block i is seen by the block's rows r >= k (causal)."""
    B, H, nqb, mk = key_idx.shape
    valid = np.arange(mk)[None, None, None, :] < key_cnt[..., None]
    if causal:
        r0 = 128 * np.arange(nqb, dtype=np.int64)[None, None, :, None]
        vis = np.clip(r0 + 128 - np.maximum(key_idx.astype(np.int64), r0), 0, 128)
    else:
        vis = np.full(key_idx.shape, 128, dtype=np.int64)
    return float(np.where(valid, vis, 0).sum())


def run_cpu_baseline(p, t, target_s: float, keep=None, promote: bool = False, adaptive=None,
                     mask: str = "pooled", stripes=None, low4: bool = False, patterns=None):
    """The oracle, as it stands, on a bounded sample: every query block of as many
    query heads as fit in about target_s seconds (after the head's group is
    smoothed and quantized, and masked when sparse)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()]
        threads = max([n for _, n in blas if n] or [1])
    except Exception:  # pragma: no cover
        blas, threads = [], 1
    b = 0
    done_ops = 0.0
    heads_done = 0
    t0 = time.perf_counter()
    nqb = p.N // 128
    for hk in range(p.Hkv):
        hqs = list(range(hk * p.group, (hk + 1) * p.group))
        q = t["q"][b:b + 1, hqs].contiguous()
        k = t["k"][b:b + 1, hk:hk + 1].contiguous()
        v = t["v"][b:b + 1, hk:hk + 1].contiguous()
        sparse = keep is not None
        sq = oracle.smooth_quant(q, k, pools=sparse or stripes is not None)
        idx = cnt = None
        if sparse and mask == "pooled":
            num, den = keep
            idx, cnt, _ = oracle.block_mask(sq["q_pool"], sq["k_pool"], len(hqs), 1, p.causal,
                                            num, den)
            if patterns is not None:
                _, idx, cnt = oracle.predict_patterns(idx, cnt, p.N, p.causal, *patterns)
        if adaptive is not None:
            err = oracle.head_error(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], q, k,
                                    sq["k_mean"], len(hqs), 1)
            idx, cnt = oracle.adaptive_lists(err > adaptive, p.N, p.causal)
        for n in range(len(hqs)):
            blocks = [(0, n, i) for i in range(nqb)]
            if sparse and mask == "lowbit":
                idx, cnt, _, _ = oracle.lowbit_block_mask(q, k, len(hqs), 1, p.causal, keep[0],
                                                          keep[1], k_mean=sq["k_mean"],
                                                          heads=[(0, n)])
                if patterns is not None:
                    _, idx, cnt = oracle.predict_patterns(idx, cnt, p.N, p.causal, *patterns)
            if stripes is not None:
                theta, mk = stripes
                sidx, scnt, _ = oracle.stripe_select(sq["q_pool"][:, n:n + 1], sq["k_i8"],
                                                     sq["k_scale"], 1, 1, p.causal, theta, mk)
                oracle.emulate_stripe_attention(sq["q_i8"][:, n:n + 1], sq["q_scale"][:, n:n + 1],
                                                sq["k_i8"], sq["k_scale"], v, p.causal, 1, 1,
                                                sidx, scnt)
            elif low4:
                oracle.emulate_promoted_fp4_attention(q, k, sq["k_mean"], v, p.causal, len(hqs),
                                                      1, idx, cnt, blocks=blocks)
            elif promote or adaptive is not None:
                oracle.emulate_promoted_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"],
                                                  sq["k_scale"], q, k, sq["k_mean"], v, p.causal,
                                                  len(hqs), 1, idx, cnt, blocks=blocks)
            else:
                oracle.emulate_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], v,
                                         p.causal, len(hqs), 1, kv_idx=idx, kv_cnt=cnt,
                                         blocks=blocks)
            heads_done += 1
            if stripes is not None:
                done_ops += 4.0 * p.d * stripe_pairs(sidx, scnt, p.causal)
            elif sparse and not promote and adaptive is None:
                done_ops += 4.0 * p.d * sparse_pairs(idx[:, n:n + 1], cnt[:, n:n + 1], p.causal)
            else:
                pairs = p.N * (p.N + 1) / 2 if p.causal else float(p.N) ** 2
                done_ops += 4.0 * p.d * pairs
            if time.perf_counter() - t0 >= target_s:
                break
        if time.perf_counter() - t0 >= target_s:
            break
    el = time.perf_counter() - t0
    return {
        "value": done_ops / el / 1e12,
        "unit": "TOPS (algorithmic)",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"oracle smooth_quant + "
                  f"{('lowbit_block_mask + ' if mask == 'lowbit' else 'block_mask + ') if sparse else ''}"
                  f"{'predict_patterns + ' if patterns is not None else ''}"
                  f"{'head_error + ' if adaptive is not None else ''}"
                  f"{'stripe_select + emulate_stripe_attention' if stripes is not None else ('emulate_promoted_fp4_attention' if low4 else 'emulate_promoted_attention' if promote or adaptive is not None else 'emulate_attention')} "
                  f"over all {nqb} query blocks of {heads_done} query head(s) of batch 0 "
                  f"({el:.1f} s); numpy BLAS {blas}",
    }


def workload_keep(args, p):
    """The keep ratio the step's mask uses (None: no mask), after the checks of
    the option combinations (host only, before any GPU work)."""
    if sum([args.promote, args.adaptive is not None, args.stripes is not None]) > 1:
        raise SystemExit("--promote, --adaptive and --stripes are exclusive")
    if args.low4 and not args.promote:
        raise SystemExit("--low4 is the low path of --promote")
    if args.adaptive is not None or args.stripes is not None:
        keep = None
    else:
        keep = p.sparse if (p.sparse is not None or not args.promote) else (1, 10)
    if args.patterns is not None:
        if keep is None:
            raise SystemExit("--patterns extends a block mask (a sparse workload or --promote)")
        if not all(0 <= n <= 64 for n in args.patterns):
            raise SystemExit("--patterns: NV and NS in [0, 64]")
    return keep


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        print("bench.py: only --gpus 1 is supported (single-GPU library)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(1, args.steps))
        return
    if args.peaks:
        run_peaks()
        return
    import torch
    import bit_quantized_attention_amd as qa
    from synthetic import make_config

    p, t = make_config(args.config)
    keep = workload_keep(args, p)
    adaptive = args.adaptive is not None
    stripes = args.stripes is not None
    qa.load()
    dev = torch.device("cuda:0")
    q, k, v = (t[x].to(dev) for x in "qkv")
    plan = qa.Plan(qa.problem(p.B, p.Hq, p.Hkv, p.N, p.d, p.dtype, p.causal), dev,
                   sparse=keep, promote=args.promote, low4=args.low4,
                   pools=True if stripes else None,
                   patterns=tuple(args.patterns) if args.patterns is not None else None)
    o = torch.empty_like(q)
    head_err = torch.empty((p.B, p.Hq), dtype=torch.float32, device=dev)
    head_hi = torch.empty((p.B, p.Hq), dtype=torch.int32, device=dev)
    nqb = p.N // 128
    key_idx = torch.empty((p.B, p.Hq, nqb, args.stripe_keys), dtype=torch.int32, device=dev)
    key_cnt = torch.empty((p.B, p.Hq, nqb), dtype=torch.int32, device=dev)
    lowbit_ws = None
    if args.mask == "lowbit" and keep is not None:
        lowbit_ws = torch.empty(qa.qattn_lowbit_workspace_bytes(plan.p), dtype=torch.uint8,
                                device=dev)

    def block_mask():
        if lowbit_ws is not None:
            qa.qattn_block_mask_lowbit(plan.p, q, k, plan.k_mean, keep[0], keep[1], plan.mask_keep,
                                       plan.mask_idx, plan.mask_cnt, None, lowbit_ws)
            if args.patterns is not None:
                plan.extend_patterns()
        else:
            plan.block_mask()

    def head_precision():
        qa.qattn_head_error(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, q, k,
                            plan.k_mean, args.adaptive, head_err, head_hi)

    def stripe_select():
        qa.qattn_stripe_select(plan.p, plan.q_pool, plan.k_i8, plan.k_scale, args.stripes,
                               args.stripe_keys, key_idx, key_cnt)

    def attention():
        if stripes:
            qa.qattn_fwd_stripes(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, v,
                                 key_idx, key_cnt, args.stripe_keys, o, plan.lse)
        elif args.low4:
            plan.fwd_promoted_fp4(q, k, v, o)
        elif args.promote:
            plan.fwd_promoted(q, k, v, o)
        elif adaptive:
            qa.qattn_fwd_adaptive(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, q,
                                  k, plan.k_mean, v, head_hi, o, plan.lse)
        else:
            plan.fwd(v, o)
    stream = torch.cuda.current_stream()

    def one_step():
        plan.smooth_quant(q, k)
        if keep is not None:
            block_mask()
        if adaptive:
            head_precision()
        if stripes:
            stripe_select()
        attention()

    # The GPU's clock settles only after tens of milliseconds under load (at
    # N = 8192 the attention kernel runs about 15 % slower over the first 25
    # steps than after 70): whole untimed steps for at least --prewarm-ms
    # first, synchronized every few steps so that the wall time is GPU time,
    # then the W counted warmup steps.
    prewarm_steps = 0
    t_pw = time.perf_counter()
    while (time.perf_counter() - t_pw) * 1e3 < args.prewarm_ms:
        one_step()
        prewarm_steps += 1
        if prewarm_steps % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    # timed region: K whole steps; the attention kernel's own launches are
    # bracketed by events on the same stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    sq_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        sq_ev[s][0].record(stream)
        plan.smooth_quant(q, k)
        if keep is not None:
            block_mask()
        if adaptive:
            head_precision()
        if stripes:
            stripe_select()
        sq_ev[s][1].record(stream)
        ev[s][0].record(stream)
        attention()
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    fwd_ms = np.array([a.elapsed_time(b) for a, b in ev])
    pre_ms = np.array([a.elapsed_time(b) for a, b in sq_ev])
    fwd_avg = float(fwd_ms.mean())

    # smoothing + quantization again, each run after writing a 512 MiB
    # scratch buffer, so that its inputs come from HBM and not from the
    # 256 MB Infinity Cache (information only, outside the timed region)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flushed = []
    for _ in range(5):
        scratch.fill_(1)
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_ev.record(stream)
        plan.smooth_quant(q, k)
        b_ev.record(stream)
        torch.cuda.synchronize()
        flushed.append(a_ev.elapsed_time(b_ev))
    del scratch
    pre_flushed_ms = float(np.median(flushed))

    literal = 4.0 * p.N * p.N * p.d * p.Hq * p.B
    peak = PEAK_INT8_TOPS
    promote_info = None
    if args.promote or adaptive:
        # every visible pair: 2*d for Q K^T (INT8, or 16-bit when promoted) and
        # 2*d for P V (16-bit)
        alg = dense_algorithmic_ops(p)
        if adaptive:
            prom = (alg / (4.0 * p.d)) * float(head_hi.float().mean().item())
        else:
            prom = sparse_pairs(plan.kv_idx.cpu().numpy(), plan.kv_cnt.cpu().numpy(), p.causal)
        ops_16 = alg / 2 + 2.0 * p.d * prom
        ops_i8 = alg - ops_16
        low_peak = PEAK_FP4_TFLOPS if args.low4 else PEAK_INT8_TOPS
        peak = alg / (ops_i8 / low_peak + ops_16 / PEAK_BF16_TFLOPS)
        promote_info = {"keep": list(keep) if keep else None,
                        "promoted_pair_fraction": prom / (alg / (4.0 * p.d)),
                        "low_path": "mxfp4" if args.low4 else "int8",
                        ("ops_fp4_per_launch" if args.low4 else "ops_int8_per_launch"): ops_i8,
                        "ops_16bit_per_launch": ops_16}
        if adaptive:
            he = head_err.cpu().numpy()
            promote_info.update({"threshold": args.adaptive, "heads_16bit": int(head_hi.sum()),
                                 "heads": int(head_hi.numel()),
                                 "head_error_min": float(he.min()),
                                 "head_error_max": float(he.max())})
    elif stripes:
        pairs = stripe_pairs(key_idx.cpu().numpy(), key_cnt.cpu().numpy(), p.causal)
        alg = 4.0 * p.d * pairs
        vis = p.N * (p.N + 1) / 2 if p.causal else float(p.N) ** 2
        promote_info = {"theta": args.stripes, "max_keys": args.stripe_keys,
                        "kept_pair_fraction": pairs / (vis * p.Hq * p.B),
                        "mean_list_length": float(key_cnt.float().mean().item()),
                        "lists_at_capacity": int((key_cnt == args.stripe_keys).sum().item())}
    elif p.sparse is not None:
        pairs = sparse_pairs(plan.kv_idx.cpu().numpy(), plan.kv_cnt.cpu().numpy(), p.causal)
        alg = 4.0 * p.d * pairs
    else:
        alg = dense_algorithmic_ops(p)
    achieved = alg / (fwd_avg * 1e-3) / 1e12
    traffic = counted_traffic(args.config, "attn_fwd_stripes" if stripes else
                              "attn_fwd_promoted_fp4" if args.low4 else
                              "attn_fwd_promoted" if args.promote else "attn_fwd")
    # Q: read 2 B + write 1 B per element; K: two reads of 2 B + write 1 B
    pre_bytes = (p.B * p.Hq * p.N * p.d * 3 + p.B * p.Hkv * p.N * p.d * 5)
    res = {
        "metric": "attention TOPS (4*N^2*d*H/s) at N=8K and 64K; % of INT8 MFMA peak",
        "value": literal / (ms_step * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_steps": prewarm_steps,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8+bf16" if p.dtype == "bf16" else "i8+f16",
        "data": "synthetic (seeded Gaussian Q/K/V with per-channel K offsets and outlier channels)",
        "config": {"workload": p.name + (" (kept blocks promoted to 16-bit QK^T, the rest "
                                         f"{'MX FP4' if args.low4 else 'INT8'})"
                                         if args.promote else "") +
                   (f" (per-head precision, error threshold {args.adaptive})" if adaptive else "") +
                   (f" (anchor stripes, threshold {args.stripes}, up to {args.stripe_keys} keys)"
                    if stripes else ""),
                   "B": p.B, "Hq": p.Hq, "Hkv": p.Hkv, "N": p.N, "d": p.d,
                   "causal": p.causal,
                   "sparse": None if (args.promote or adaptive or stripes) else p.sparse,
                   "promote": list(keep) if args.promote else None,
                   "low_path": ("mxfp4" if args.low4 else "int8") if args.promote else None,
                   "adaptive_threshold": args.adaptive,
                   "stripes": [args.stripes, args.stripe_keys] if stripes else None,
                   "mask": args.mask if keep is not None else None,
                   "patterns": list(args.patterns) if args.patterns is not None else None,
                   "input_dtype": p.dtype},
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": peak,
            # tera-operations per second: INT8 and 16-bit multiply-adds count 2
            "unit": "TOP/s",
            "frac": achieved / peak,
            "traffic": traffic,
            "kernel": "attn_fwd",
            "algorithmic_ops_per_launch": alg,
            "avg_launch_ms": fwd_avg,
            **({} if (args.promote or adaptive) else roofline_fracs(alg, fwd_avg, traffic)),
        },
        "fwd_ms": fwd_avg,
        "fwd_tops_literal": literal / (fwd_avg * 1e-3) / 1e12,
        "fwd_tops_algorithmic": achieved,
        "preprocess_ms": float(pre_ms.mean()),
        "preprocess_gbs_algorithmic": pre_bytes / (float(pre_ms.mean()) * 1e-3) / 1e9
        if keep is None and not adaptive and not stripes else None,
        "fwd_ms_median": float(np.median(fwd_ms)),
        "smooth_quant_ms_cache_flushed": pre_flushed_ms,
        "smooth_quant_gbs_cache_flushed": pre_bytes / (pre_flushed_ms * 1e-3) / 1e9,
        "smooth_quant_hbm_frac_cache_flushed": pre_bytes / (pre_flushed_ms * 1e-3) / 1e9
        / PEAK_HBM_GBS,
        "blended_mfma_peak_tops": BLENDED_PEAK_TOPS,
    }
    if (args.config == 2 and not (args.promote or adaptive or stripes) and not args.no_long):
        # the metric is quoted at 8K and 64K: the 64K forward beside the 8K line
        res["long_context"] = measure_long_context()
    if promote_info is not None:
        res["adaptive" if adaptive else "stripes" if stripes else "promote"] = promote_info
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = run_cpu_baseline(p, t, args.cpu_seconds, keep, args.promote,
                                               args.adaptive, args.mask,
                                               (args.stripes, args.stripe_keys) if stripes else None,
                                               low4=args.low4, patterns=args.patterns)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
