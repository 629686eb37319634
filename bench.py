#!/usr/bin/env python3
"""Benchmark of the Dobb optimizer step on one MI355X: the GPT-2 XL matrix set.

Workload (synthetic, fixed shapes): 48 layers x {qkv 4800x1600, proj 1600x1600, fc 6400x1600,
fc-proj 1600x6400} = 192 weights, 1.4746 B parameters, B = 16 blocks per weight (nb = 100, and 400
for fc-proj).  W, G, M, A and Q are fp32; activations are bf16, 16384 tokens per capture, with a
15 % effective-rank power-law spectrum.  One benchmark step is the whole hot path with a refresh
every step: capture (accumulate + EMA) -> basis refresh (warm-started orthogonal iteration, k = 1,
Householder) -> the Dobb step (momentum, projection, sign, reconstruction, weight update).  The
first refresh (setup, untimed) is exact.  The headline comes from events around K timed steps with
the library's kernel timer off, each step a replay of a HIP graph of the step (``--eager``: launched
from the host instead; both times are in the breakdown); a second pass over K more steps, launched
from the host with the timer on (an event pair around every launch, on its stream), attributes the
time to kernels.  The CPU oracle is timed on a
bounded sample, threaded over the host's cores.

The default workload is the GPT-2 XL set.  ``--workload gpt2small`` runs the GPT-2 Small set (12 layers x
{qkv 2304x768, proj 768x768, fc 3072x768, fc-proj 768x3072}, B = 16, fp32 state, bf16 activations of
8192 tokens) and ``--workload llama7b`` the 7B-style stack (32 layers x {q, k, v, o 4096x4096, gate/up
11008x4096, down 4096x11008}, nb = 128, bf16 W and G, fp32 M, A and Q; the pages give no token count
for it, so a capture here is 4096 tokens).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--layers L] [--copy-mib C] [--eager]
                       [--workload gpt2xl|gpt2small|llama7b|single768_b4|single768_b1]
       python bench.py --pmc-summary FETCH_CSV WRITE_CSV [--copy-mib C]
       python bench.py --mfma-summary COUNTER_CSV
       python bench.py --counter-summary COUNTER_CSV [COUNTER_CSV ...]
       python bench.py --streams 2 | --compare-streams   (the two-stream schedule of DobbGroup)
"""
from __future__ import annotations

import argparse
import collections
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Dobb optimizer-step ms for GPT-2-XL-shaped matrix set; MFMA %peak, HBM %peak"
# MI355X published peaks (dense)
PEAK_HBM = 8.0e12            # B/s
PEAK_BF16_MFMA = 2.5e15      # flop/s, bf16 and fp16
PEAK_FP32_MFMA = 157.3e12    # flop/s
PEAK_FP32_VALU = 157.3e12    # flop/s
PEAK_FP64_VALU = 78.6e12     # flop/s
JACOBI_KERNELS = ("jacobi_sweep", "jacobi_sweep_fp64", "jacobi_rotate_v", "jacobi_block_sub", "jacobi_block_apply")
LDS_BYTES = 160 * 1024


def block_jacobi(nb):
    """Whether the library runs block Jacobi for nb (its fp32 element-wise working matrix exceeds the
    LDS), and then its geometry (m index blocks of b), as the library chooses them."""
    nbp = (nb + 1) // 2 * 2
    if ((nbp // 2) * 16 + 4 + 15) // 16 * 16 + nbp * nbp * 4 <= LDS_BYTES:
        return None
    m = 2 * ((nb + 79) // 80)
    b = (-(-nb // m) + 3) // 4 * 4
    return m, b


def jacobi_sweep_flops(nb):
    """fp64 flops of one sweep on one block.  Element-wise: nb (nb - 1) / 2 rotations, each combining
    rows p, q and columns p, q of A (4 nb entries, 3 flops each) and columns p, q of V (2 nb entries):
    9 nb^2 (nb - 1).  Block Jacobi: m - 1 rounds, each with m / 2 sub-problem sweeps of size 2b (the
    same count at 2b) and the tile products R_p^T A R_q for the (m/2)(m/2 - 1)/2 off-diagonal pairs
    (2 (2b)^3 twice) and V R_q for the m / 2 pair sets (2 nb (2b)^2)."""
    g = block_jacobi(nb)
    if g is None:
        return 9.0 * nb * nb * (nb - 1)
    m, b = g
    b2, h = 2 * b, m // 2
    per_round = h * 9.0 * b2 * b2 * (b2 - 1) + h * (h - 1) / 2 * 4.0 * b2 ** 3 + h * 2.0 * nb * b2 * b2
    return (m - 1) * per_round
BLOCKS = 16
QR_PANEL = 32                # Householder panel width of the refresh
QR_SINGLE_LAUNCH_MAX_NB = 128  # blocks up to this width are factored in one launch (Z in LDS)
STEP_ROWS_MAX_NB = 128        # blocks up to this width keep Q resident in LDS in the step kernels (no split_q)
STEP_FUSED_MAX_NB = 128       # ... and up to this width (nb % 4 == 0) the one-pass step kernel

# Matrix sets.  per_layer: weights per layer; tokens: activations per capture; config: seed namespace;
# cpu_rows / cpu_tokens: the oracle sample (1/cpu_rows of each weight's rows, cpu_tokens of the tokens).
WORKLOADS = {
    "gpt2xl": dict(specs="gpt2_xl_set", arg=BLOCKS, layers=48, per_layer=4, tokens=16384, w_dtype="float32",
                   config=4, lr=2.5e-3, cpu_rows=1, cpu_tokens=16384, cpu_layers=4,
                   text="GPT-2 XL matrix set ({L} layers x qkv 4800x1600, proj 1600x1600, fc 6400x1600, "
                        "fc-proj 1600x6400; B=16, nb=100/400), fp32 W/G/M/A/Q, bf16 activations {N} tokens"),
    "gpt2small": dict(specs="gpt2_small_set", arg=BLOCKS, layers=12, per_layer=4, tokens=8192, w_dtype="float32",
                      config=3, lr=3.54e-3, cpu_rows=1, cpu_tokens=8192,
                      text="GPT-2 Small matrix set ({L} layers x qkv 2304x768, proj 768x768, fc 3072x768, "
                           "fc-proj 768x3072; B=16, nb=48/192), fp32 W/G/M/A/Q, bf16 activations {N} tokens"),
    "llama7b": dict(specs="llama7b_set", arg=128, layers=32, per_layer=7, tokens=4096, w_dtype="bfloat16",
                    config=5, lr=2.5e-3, cpu_rows=16, cpu_tokens=512,
                    text="Llama-7B-style stack ({L} layers x q,k,v,o 4096x4096, gate/up 11008x4096, down "
                         "4096x11008; nb=128), bf16 W/G, fp32 M/A/Q, bf16 activations {N} tokens"),
    # single 768x768 weights: launch-latency bound, reported for completeness
    "single768_b4": dict(specs="single_768_set", arg=4, layers=1, per_layer=1, tokens=4096, w_dtype="float32",
                         x_dtype="float32", config=1, lr=2.5e-3, cpu_rows=1, cpu_tokens=4096,
                         text="single 768x768 weight (B=4, nb=192), fp32 W/G/M/A/Q, fp32 activations {N} tokens"),
    "single768_b1": dict(specs="single_768_set", arg=1, layers=1, per_layer=1, tokens=4096, w_dtype="float32",
                         x_dtype="float32", config=2, lr=2.5e-3, cpu_rows=1, cpu_tokens=4096,
                         text="single 768x768 weight (B=1, nb=768), fp32 W/G/M/A/Q, fp32 activations {N} tokens"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel from the host each step instead of replaying a HIP graph of the step")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="gpt2xl")
    ap.add_argument("--layers", type=int, default=0, help="layers of the matrix set (default: all)")
    ap.add_argument("--norm", choices=["sign", "col_l2"], default="sign",
                    help="normalisation of the coefficients: sign (Dobb) or column-l2 (Dobb-l2, Tables 11-12)")
    ap.add_argument("--orth-iters", type=int, default=1, help="orthogonal-iteration steps per refresh (Table 15)")
    ap.add_argument("--qr", choices=["householder", "cholesky"], default="householder",
                    help="QR routine of the orthogonal-iteration refresh (Table 16: Householder is the principal)")
    ap.add_argument("--basis", choices=["fp32", "bf16"], default="fp32",
                    help="storage of the block bases (Table 18: bf16 is the pages' principal setting)")
    ap.add_argument("--streams", type=int, choices=[1, 2], default=1,
                    help="2: the weights with blocks of at most 128 columns and the wider ones on two streams in "
                         "the timed region (kernels then share the GPU, so per-launch times are not each "
                         "kernel's own)")
    ap.add_argument("--compare-streams", action="store_true",
                    help="also time the full step with the other stream schedule (breakdown_ms); off by default, "
                         "so that a profiled run's kernel durations are those of the timed schedule only")
    ap.add_argument("--mfma-summary", metavar="COUNTER_CSV",
                    help="per-kernel MFMA utilisation and issued MFMA flops from a rocprofv3 --pmc run of "
                         "MfmaUtil MfmaFlopsBF16 MfmaFlopsF16 MfmaFlopsF32")
    ap.add_argument("--counter-summary", nargs="+", metavar="COUNTER_CSV",
                    help="print per-kernel stall and cache ratios from rocprofv3 --pmc runs and exit")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the per-kernel HBM traffic table from two rocprofv3 --pmc CSVs and exit")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain device-to-device copy of this many MiB first (a known-size kernel "
                         "for calibrating hardware byte counters)")
    return ap.parse_args()


def capture_splits(n, nb, count, n_tokens, bf16):
    """Token splits of one capture launch group (count weights of width n, blocks of nb), as the
    library plans them: bf16 blocks 128 < nb <= 512 (nb % 8 == 0) take the wide kernel, whose splits
    hold at most 4096 tokens and give about 1024 workgroups of 8 waves (one per 8 groups of 2 x 4
    tiles of 32 x 32 over the upper triangle); the others split until about 512 (bf16) or 1024 (fp32)
    tile pairs of 128 or 64 columns, at least 256 tokens each."""
    cnt = min(count, 48)
    B = n // nb
    if bf16 and 128 < nb <= 512 and nb % 8 == 0:
        t32 = -(-nb // 32)
        groups = sum(len(range(r, t32, 4)) for r in range(0, t32, 2))
        wgtot = -(-groups // 8) * B * cnt
        ns = min(-(-1024 // wgtot), n_tokens // 256)
        ns = max(ns, -(-n_tokens // 4096), 1)
        length = -(-(-(-n_tokens // ns)) // 64) * 64
        return -(-n_tokens // length)
    tile = 128 if bf16 else 64
    T = -(-nb // tile)
    tiles = T * (T + 1) // 2 * B * cnt
    ns = max(min(-(-(512 if bf16 else 1024) // tiles), n_tokens // 256, 64), 1)
    length = -(-(-(-n_tokens // ns)) // 64) * 64
    return -(-n_tokens // length)


def kernel_work(specs, n_tokens, g_bytes=4, w_bytes=4, norm="sign", orth_iters=1, x_bytes=2, qr="householder"):
    """Per-step work of each kernel of the path, summed over the matrix set.

    Per kernel: algorithmic HBM bytes (each operand read or written once), algorithmic flops with the
    peak of the precision they stand for, and the matrix-core flops the kernel actually issues with
    that dtype's peak.  Units (per weight m x n with B = n / nb blocks):
      accumulate_syrk_*     X read once: 2 N n bytes; N nb (nb + 1) B flops (unique entries of X_b^T X_b);
                            "wide" for bf16 blocks 128 < nb <= 512, nb % 8 == 0; fp32 activations
                            (x_bytes = 4): accumulate_syrk, 4 N n bytes, fp32 MFMA
      accumulate_reduce     A read + written: 8 nb^2 B bytes, where the capture splits its tokens over
                            workgroups (capture_splits); otherwise the EMA is in the capture kernel
                            and these bytes are its own
      refresh_gemm          Z = A Q: 2 nb^3 B flops (fp32); A, Q read, Z written: 12 nb^2 B bytes
      qr_block              nb <= 128, the whole Householder QR in one launch: 8/3 nb^3 B flops
      qr_update / qr_form   nb > 128, factor updates (a launch per panel) / formation (one launch for
                            all panels): 4/3 nb^3 B flops each (fp32)
      qr_panel              nb > 128, panel factorisation: about QR_PANEL nb^2 B flops (fp32 vector ALU)
      split_q               nb > 128 only, Q read, five 2-byte planes written: (4 + 10) nb^2 B bytes
      project_f16x3         nb <= 416: M read + written, G read: (8 + g) m n bytes of the method (the
                            projection's share of the step's G + M + W traffic); the sign byte it
                            writes per entry is traffic of this implementation ("impl_bytes");
                            2 m n nb flops (fp32 contraction), issued as three fp16 products
      project_bf16x6        nb > 416 (staged kernels): same bytes and flops, issued as six bf16 products
      reconstruct_f16x2     W read + written: 2 w m n bytes of the method, plus the sign byte read
                            (implementation); 2 m n nb flops (fp32 contraction), issued as two fp16
                            products
      step_fused_f16        nb <= 128, nb % 4 = 0: the one-pass step kernel: G read, M read + written,
                            W read + written: (8 + g + 2 w) m n bytes, no sign bytes; 4 m n nb flops
                            issued as five fp16 products over the padded block (16 ceil(nb / 16) basis
                            rows, 32 ceil(nb / 32) deep)
      step_wide_fused_f16   128 < nb <= 416, nb % 4 = 0: the one-pass wide kernel, same bytes and flops
                            (after split_q), five fp16 products over 32 ceil(nb / 32) basis rows and a
                            16 ceil(nb / 16)-deep contraction; project_f16x3 and reconstruct_f16x2 are
                            the two-kernel path a coefficient output takes
    Column-l2 normalisation (norm="col_l2") takes, for 128 < nb <= 416, split_q, project_l2_f16x3 (M
    read + written, G read, C written: (12 + g) m n bytes), colnorm and reconstruct_l2_f16x3 (C read,
    W read + written) on the wide kernels, and otherwise the plain fp32 kernels instead of the last four:
      momentum              G read, M read + written: (8 + g) m n bytes
      project               M read, C written: 8 m n bytes; 2 m n nb fp32 MFMA flops
      colnorm               C read: 4 m n bytes
      reconstruct           C read, W read + written: (4 + 2 w) m n bytes; 2 m n nb fp32 MFMA flops
      for nb <= 128 (nb % 4 == 0) the split-fp16 rows kernels instead:
      project_l2_f16x3      M read + written, G read, C written: (12 + g) m n bytes; three fp16 products
      colscale              the tiles' column sums of squares read: 8 ceil(m / 128) n bytes
      reconstruct_l2_f16x3  C read, W read + written: (4 + 2 w) m n bytes; three fp16 products
    The refresh kernels run orth_iters times per refresh.  With qr="cholesky" (Table 16) the refresh is
    Z = A Q and two Cholesky QR passes, each a Gram product Z^T Z, the factor R with its inverse and
    the product Z R^{-1}:
      refresh_gemm          five nb^3 products: 10 nb^3 B flops (fp32)
      cholqr_factor         R (nb^3 / 3) and R^{-1} (nb^3 / 3) twice: 4/3 nb^3 B flops
    """
    w = {}

    def add(name, nbytes=0.0, flops=0.0, flops_peak=PEAK_FP32_MFMA, issued=0.0, issued_peak=PEAK_BF16_MFMA,
            compute="mfma", impl=0.0):
        e = w.setdefault(name, dict(bytes=0.0, flops=0.0, flops_peak=flops_peak, issued=0.0,
                                    issued_peak=issued_peak, compute=compute, impl_bytes=0.0))
        e["bytes"] += nbytes; e["flops"] += flops; e["issued"] += issued; e["impl_bytes"] += impl

    shapes = collections.Counter((s.n, s.nb) for s in specs)
    for s in specs:
        B, nb, mn = s.n // s.nb, s.nb, s.m * s.n
        split = capture_splits(s.n, nb, shapes[(s.n, s.nb)], n_tokens, x_bytes == 2) > 1
        if x_bytes == 4:
            add("accumulate_syrk", 4.0 * n_tokens * s.n + (0.0 if split else 8.0 * nb * nb * B),
                n_tokens * nb * (nb + 1) * B, PEAK_FP32_MFMA)
        else:
            syrk = "accumulate_syrk_wide" if 128 < nb <= 512 and nb % 8 == 0 else "accumulate_syrk_bf16"
            add(syrk, 2.0 * n_tokens * s.n + (0.0 if split else 8.0 * nb * nb * B),
                n_tokens * nb * (nb + 1) * B, PEAK_BF16_MFMA)
        if split:
            add("accumulate_reduce", 8.0 * nb * nb * B)
        k = orth_iters
        if qr == "cholesky":
            add("refresh_gemm", k * 5 * 12.0 * nb * nb * B, k * 10.0 * nb ** 3 * B)
            add("cholqr_factor", 0.0, k * 4.0 / 3.0 * nb ** 3 * B)
        else:
            add("refresh_gemm", k * 12.0 * nb * nb * B, k * 2.0 * nb ** 3 * B)
        if qr == "cholesky":
            pass
        elif nb <= QR_SINGLE_LAUNCH_MAX_NB:
            add("qr_block", 0.0, k * 8.0 / 3.0 * nb ** 3 * B)
        else:
            add("qr_update", 0.0, k * 4.0 / 3.0 * nb ** 3 * B)
            add("qr_form", 0.0, k * 4.0 / 3.0 * nb ** 3 * B)
            add("qr_panel", 0.0, k * QR_PANEL * nb * nb * B, PEAK_FP32_VALU, compute="alu")
        if norm == "col_l2":
            if nb <= STEP_ROWS_MAX_NB and nb % 4 == 0 and s.n % 4 == 0:
                add("project_l2_f16x3", (12.0 + g_bytes) * mn, 2.0 * mn * nb, PEAK_FP32_MFMA, 3 * 2.0 * mn * nb)
                add("colscale", 8.0 * -(-s.m // 128) * s.n)
                add("reconstruct_l2_f16x3", (4.0 + 2 * w_bytes) * mn, 2.0 * mn * nb, PEAK_FP32_MFMA, 3 * 2.0 * mn * nb)
            elif STEP_ROWS_MAX_NB < nb <= 416 and nb % 4 == 0:
                add("split_q", 14.0 * nb * nb * B)
                add("project_l2_f16x3", (12.0 + g_bytes) * mn, 2.0 * mn * nb, PEAK_FP32_MFMA, 3 * 2.0 * mn * nb)
                add("colnorm", 4.0 * mn)
                add("reconstruct_l2_f16x3", (4.0 + 2 * w_bytes) * mn, 2.0 * mn * nb, PEAK_FP32_MFMA, 3 * 2.0 * mn * nb)
            else:
                add("momentum", (8.0 + g_bytes) * mn)
                add("project", 8.0 * mn, 2.0 * mn * nb)
                add("colnorm", 4.0 * mn)
                add("reconstruct", (4.0 + 2 * w_bytes) * mn, 2.0 * mn * nb)
            continue
        if nb <= STEP_FUSED_MAX_NB and nb % 4 == 0:
            rows, kp = 16 * -(-nb // 16), 32 * -(-nb // 32)   # basis rows and contraction depth, padded
            add("step_fused_f16", (8.0 + g_bytes + 2 * w_bytes) * mn, 4.0 * mn * nb, PEAK_FP32_MFMA,
                5 * 2.0 * s.m * B * rows * kp)
            continue
        if STEP_ROWS_MAX_NB < nb <= 416 and nb % 4 == 0:
            rows, kp = 32 * -(-nb // 32), 16 * -(-nb // 16)   # basis rows and contraction depth, padded
            add("split_q", 14.0 * nb * nb * B)
            add("step_wide_fused_f16", (8.0 + g_bytes + 2 * w_bytes) * mn, 4.0 * mn * nb, PEAK_FP32_MFMA,
                5 * 2.0 * s.m * B * rows * kp)
            continue
        if nb > STEP_ROWS_MAX_NB:
            add("split_q", 14.0 * nb * nb * B)
        if nb <= 416:
            add("project_f16x3", (8.0 + g_bytes) * mn, 2.0 * mn * nb, PEAK_FP32_MFMA, 3 * 2.0 * mn * nb, impl=mn)
        else:
            add("project_bf16x6", (8.0 + g_bytes) * mn, 2.0 * mn * nb, PEAK_FP32_MFMA, 6 * 2.0 * mn * nb, impl=mn)
        add("reconstruct_f16x2", 2.0 * w_bytes * mn, 2.0 * mn * nb, PEAK_FP32_MFMA, 2 * 2.0 * mn * nb, impl=mn)
    return w


def jacobi_entry(kernels, infos, nbs, total_ms):
    """The exact refresh's work against the fp64 vector peak (every Jacobi stage computes in fp64; the
    element-wise first stage only stores its working matrix in fp32): jacobi_sweep_flops per block and
    sweep, counted over the sweeps each block reports in info (those that rotated)."""
    sweeps = [i.clamp(min=0).double() for i in infos]
    flops = sum(jacobi_sweep_flops(nb) * float(sw.sum()) for sw, nb in zip(sweeps, nbs))
    jac_ms = sum(kernels.get(k, (0, 0.0))[1] for k in JACOBI_KERNELS)
    rate = flops / (jac_ms / 1e3) if jac_ms > 0 else 0.0
    n_blocks = sum(sw.numel() for sw in sweeps)
    return {"ms": round(total_ms, 1), "jacobi_kernels_ms": round(jac_ms, 1),
            "sweeps_mean": round(sum(float(sw.sum()) for sw in sweeps) / n_blocks, 2),
            "sweeps_max": int(max(float(sw.max()) for sw in sweeps)),
            "bound": "alu", "achieved": round(rate / 1e12, 4), "peak": PEAK_FP64_VALU / 1e12, "unit": "TFLOP/s",
            "frac": round(rate / PEAK_FP64_VALU, 5), "flops": flops}


def roofline_entry(work, seconds):
    """The binding resource of the kernel as built, and the fraction of its peak reached.

    Time at peak: HBM bytes / 8 TB/s against matrix-core time, which is the issued products at
    their dtype's peak for the split-precision kernels and the algorithmic flops at the fp32 peak
    otherwise.  "achieved" is algorithmic bytes per second when HBM binds, else the flops rate
    (issued products for the split kernels, with the algorithmic fp32-equivalent rate beside it)."""
    t_hbm = work["bytes"] / PEAK_HBM
    if work["issued"]:
        t_cmp, rate, peak = work["issued"] / work["issued_peak"], work["issued"] / seconds, work["issued_peak"]
    else:
        t_cmp, rate, peak = work["flops"] / work["flops_peak"], work["flops"] / seconds, work["flops_peak"]
    if t_hbm >= t_cmp:
        ent = {"bound": "hbm", "achieved": work["bytes"] / seconds / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    else:
        ent = {"bound": work["compute"], "achieved": rate / 1e12, "peak": peak / 1e12, "unit": "TFLOP/s"}
    ent["frac"] = ent["achieved"] / ent["peak"]
    ent["hbm_frac"] = work["bytes"] / seconds / PEAK_HBM
    if work.get("impl_bytes"):
        ent["impl_bytes_per_step"] = work["impl_bytes"]
    if work["issued"]:
        ent["mfma_issued_frac"] = work["issued"] / seconds / work["issued_peak"]
        ent["fp32_equiv_tflops"] = work["flops"] / seconds / 1e12
    return ent


# ---- measured HBM traffic (rocprofv3 counters), tied to the kernel sources they were taken on ----
CSRC = os.path.join(ROOT, "block_diagonal_eigenbasis_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_gpt2xl_step.md")
# library kernel name -> (regular expression on the device symbol, source file)
KERNEL_SYMBOLS = {
    "accumulate_syrk_bf16": (r"k_syrk_(bf16<|narrow_dma)", "k_accumulate.hip"),
    "accumulate_syrk_wide": (r"k_syrk_wide", "k_accumulate.hip"),
    "accumulate_reduce": (r"k_syrk_reduce", "k_accumulate.hip"),
    "refresh_gemm": (r"k_bgemm(_t)?<", "k_refresh.hip"),
    "qr_block": (r"k_qr_block<", "k_qr.hip"),
    "qr_panel": (r"k_qr_panel<", "k_qr.hip"),
    "qr_update": (r"k_qr_apply<\d+, true,", "k_qr.hip"),
    "qr_form": (r"k_qr_form<", "k_qr.hip"),
    "split_q": (r"k_split_(q|wide)", ("k_step_bf16.hip", "k_step_wide.hip")),
    "project_f16x3": (r"k_proj_wide<", ("k_step_wide.hip", "step_common.h")),
    "step_fused_f16": (r"k_step_fused<", ("k_step_fused.hip", "step_common.h")),
    "step_wide_fused_f16": (r"k_step_wide_fused<", ("k_step_wide.hip", "step_common.h")),
    "project_bf16x6": (r"k_proj_bf16<", ("k_step_bf16.hip", "step_common.h")),
    "reconstruct_f16x2": (r"k_recon_(bf16|wide)<", ("k_step_bf16.hip", "k_step_wide.hip", "step_common.h")),
    "project_l2_f16x3": (r"k_proj_rows<", ("k_step_rows.hip", "step_common.h")),
    "reconstruct_l2_f16x3": (r"k_recon_rows<", ("k_step_rows.hip", "step_common.h")),
    "cholqr_factor": (r"k_chol_inv", "k_cholqr.hip"),
}


def source_digest(kernel):
    """Digest of the source file that defines a kernel plus the shared internal header."""
    import hashlib
    h = hashlib.sha256()
    src = KERNEL_SYMBOLS[kernel][1]
    for f in (*(src if isinstance(src, tuple) else (src,)), "dobb_internal.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch (fetched + written) from the committed counter summary, or None when the
    kernel's source has changed since the counters were taken."""
    if kernel not in KERNEL_SYMBOLS or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            f = line.strip().strip("|").split("|")
            f = [x.strip() for x in f]
            if len(f) >= 5 and f[0] == kernel:
                if f[1].strip("`") != source_digest(kernel):
                    return None
                return float(f[3]) + float(f[4])
    return None


def pmc_summary(fetch_csv, write_csv, copy_mib):
    """Per-kernel HBM bytes per launch from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, in
    KiB per dispatch).  Each counter is scaled so that the largest device copy (the calibration copy of
    copy_mib MiB run by --copy-mib) reads and writes exactly its size."""
    import csv
    import collections

    def per_kernel(fn):
        rows = list(csv.DictReader(open(fn)))
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        ref = max(copies)
        scale = copy_mib * 1024.0 / ref
        acc = collections.defaultdict(list)
        for r in rows:
            for name, (sym, _) in KERNEL_SYMBOLS.items():
                if re.search(sym, r["Kernel_Name"]):
                    acc[name].append(float(r["Counter_Value"]) * scale * 1024.0)
        return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}, scale, ref

    fetch, fscale, fref = per_kernel(fetch_csv)
    write, wscale, wref = per_kernel(write_csv)
    print(f"calibration: {copy_mib} MiB copy read {fref:.0f} KiB (FETCH_SIZE), wrote {wref:.0f} KiB (WRITE_SIZE); "
          f"scale factors {fscale:.3f} and {wscale:.3f}")
    print()
    print("| kernel | source digest | launches | fetched bytes/launch | written bytes/launch |")
    print("|---|---|---|---|---|")
    for name in KERNEL_SYMBOLS:
        if name in fetch and name in write:
            print(f"| {name} | `{source_digest(name)}` | {fetch[name][1]} | {fetch[name][0]:.0f} | {write[name][0]:.0f} |")


def mfma_summary(counter_csv):
    """Per-kernel matrix-core figures from one rocprofv3 --pmc run of the derived counters MfmaUtil
    (MFMA-busy SIMD cycles over active cycles x SIMDs, percent) and MfmaFlops{BF16,F16,F32} (issued
    MFMA operations x 512, per dispatch), averaged over each kernel's dispatches."""
    import csv
    import collections
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(counter_csv)):
        for name, (sym, _) in KERNEL_SYMBOLS.items():
            if re.search(sym, r["Kernel_Name"]):
                acc[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
    print("| kernel | source digest | launches | MFMA busy (% of SIMD cycles) | bf16 MFMA flop/launch | "
          "fp16 MFMA flop/launch | fp32 MFMA flop/launch |")
    print("|---|---|---|---|---|---|---|")
    for name in KERNEL_SYMBOLS:
        c = acc.get(name)
        if not c:
            continue
        avg = lambda k: (sum(c[k]) / len(c[k])) if c.get(k) else float("nan")
        print(f"| {name} | `{source_digest(name)}` | {len(c.get('MfmaUtil', []))} | {avg('MfmaUtil'):.1f} | "
              f"{avg('MfmaFlopsBF16'):.4g} | {avg('MfmaFlopsF16'):.4g} | {avg('MfmaFlopsF32'):.4g} |")


def counter_summary(counter_csvs):
    """Per-kernel stall and cache figures from rocprofv3 --pmc runs (one CSV per pass), by kernel
    function (the narrow and wide instances of a bench.py kernel apart): each counter averaged over
    the kernel's dispatches in its pass, then the ratios below where their counters were taken.
      dependency wait   SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (wave-cycles waiting for an operand or a
                        counter, e.g. a load in flight)
      any wait          SQ_WAIT_ANY / SQ_WAVE_CYCLES (also barriers)
      issuing           SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES
      LDS conflicts     SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS
      L2 read latency   TCP_TCC_READ_REQ_LATENCY_sum / TCP_TCC_READ_REQ_sum (cycles, as seen by L1)
      L2 hit rate       TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)"""
    import csv
    import collections
    csv.field_size_limit(1 << 30)
    sums = collections.defaultdict(lambda: collections.defaultdict(float))
    counts = collections.defaultdict(lambda: collections.defaultdict(set))
    for path in counter_csvs:
        for r in csv.DictReader(open(path)):
            mt = re.search(r"\b(k_[a-z0-9_]+)", r["Kernel_Name"])
            if not mt or "dobb" not in r["Kernel_Name"]:
                continue
            k, c = mt.group(1), r["Counter_Name"]
            sums[k][c] += float(r["Counter_Value"])
            counts[k][c].add((path, r["Dispatch_Id"]))
    avg = lambda k, c: sums[k][c] / len(counts[k][c]) if counts[k].get(c) else None

    def ratio(k, a, b, scale=100.0):
        x, y = avg(k, a), avg(k, b)
        return None if x is None or not y else scale * x / y

    def hit(k):
        h, m_ = avg(k, "TCC_HIT_sum"), avg(k, "TCC_MISS_sum")
        return None if h is None or m_ is None or h + m_ == 0 else 100.0 * h / (h + m_)
    cols = [("dependency wait %", lambda k: ratio(k, "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES")),
            ("any wait %", lambda k: ratio(k, "SQ_WAIT_ANY", "SQ_WAVE_CYCLES")),
            ("issuing %", lambda k: ratio(k, "SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES")),
            ("LDS conflict %", lambda k: ratio(k, "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS")),
            ("L2 read latency (cycles)", lambda k: ratio(k, "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum", 1.0)),
            ("L2 hit %", hit)]
    print("| kernel function | launches | " + " | ".join(c for c, _ in cols) + " |")
    print("|---|---|" + "---|" * len(cols))
    for k in sorted(sums, key=lambda k: -(avg(k, "SQ_WAVE_CYCLES") or 0.0)):
        n = max(len(v) for v in counts[k].values())   # dispatches in a pass
        vals = [f(k) for _, f in cols]
        print(f"| `{k}` | {n} | " + " | ".join("–" if v is None else f"{v:.0f}" for v in vals) + " |")


def host_cores():
    """Threads for the CPU baseline: the CPUs this process may run on, at most 16 (the host share of
    one GPU), and the facts reported with them."""
    try:
        aff = sorted(os.sched_getaffinity(0))
    except AttributeError:
        aff = list(range(os.cpu_count() or 1))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    ranges, start = [], None
    for i, c in enumerate(aff):
        if start is None:
            start = c
        if i + 1 == len(aff) or aff[i + 1] != c + 1:
            ranges.append(f"{start}-{c}" if c > start else f"{start}")
            start = None
    return min(len(aff), 16), {"nproc": os.cpu_count(), "affinity": ",".join(ranges), "cpu_model": model}


def cpu_baseline(group, xs, specs, wl, layers, col_l2=False, k_orth=1):
    """Time the oracle, threaded over the host's cores (row chunks of the step, blocks of the capture
    and of the refresh), on the weights of cpu_layers evenly spaced layers (the first and the last
    among them): the step on 1/cpu_rows of each weight's rows, the capture on cpu_tokens of the
    tokens, the orthogonal-iteration refresh on every block; scale linearly to the full set (every
    term is linear in rows, tokens and layers)."""
    import oracle
    cores, facts = host_cores()
    rows_frac, tok = wl["cpu_rows"], wl["cpu_tokens"]
    n_tokens = wl["tokens"]
    per = wl["per_layer"]
    k = min(wl.get("cpu_layers", 2), layers)
    picked = [0] if k <= 1 else sorted({round(i * (layers - 1) / (k - 1)) for i in range(k)})
    sample = [per * l + j for l in picked for j in range(per)]
    t_meas = 0.0
    s_total = 0.0
    for i in sample:
        s = specs[i]
        r = s.m // rows_frac
        W = group.W[i][:r].cpu(); G = group.G[i][:r].cpu(); M = group.M[i][:r].cpu()
        Q = group.Q[i].cpu()
        X = xs[i][:tok].cpu()
        A = group.A[i].cpu()
        t0 = time.perf_counter()
        oracle.step(W, G, M, Q, s.nb, 2.5e-3, 0.1, 0.9, 0.2, norm=oracle.NORM_COL_L2 if col_l2 else oracle.NORM_SIGN,
                    cores=cores)
        t1 = time.perf_counter()
        oracle.accumulate(X, s.nb, cores=cores)
        t2 = time.perf_counter()
        oracle.orth_iter(A, Q, k=k_orth, cores=cores)
        t3 = time.perf_counter()
        t_meas += t3 - t0
        s_total += (t1 - t0) * (s.m / r) + (t2 - t1) * (n_tokens / tok) + (t3 - t2)
    total_s = s_total * layers / len(picked)
    return {"value": round(total_s * 1e3, 1), "unit": "ms", "cores": cores, "kind": "oracle",
            "sample": (f"the {len(sample)} weights of layers {', '.join(str(l) for l in picked)} "
                       f"of {layers}: step on 1/{rows_frac} of each weight's rows, capture on {tok} of {n_tokens} "
                       f"tokens, orthogonal-iteration refresh (k={k_orth}) on every block; measured "
                       f"{t_meas:.1f} s on {cores} threads, scaled linearly (rows, tokens, layers)"),
            "seconds_measured": round(t_meas, 2), **facts}


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.copy_mib or 1024)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the Dobb step here is the single-GPU kernel path "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import workload
    import block_diagonal_eigenbasis_amd as dobb
    from block_diagonal_eigenbasis_amd.optimizer import DobbGroup

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_mib:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy: {args.copy_mib} MiB read, {args.copy_mib} MiB written", file=sys.stderr,
              flush=True)
        del src, dst
    wl = WORKLOADS[args.workload]
    layers = args.layers or wl["layers"]
    n_tokens = wl["tokens"]
    specs = getattr(workload, wl["specs"])(wl["arg"])[: wl["per_layer"] * layers]
    w_dtype = getattr(torch, wl["w_dtype"])
    print(f"[bench] {len(specs)} weights, {workload.param_count(specs) / 1e9:.4f} B params", file=sys.stderr, flush=True)

    # ---- inputs (seeded, synthetic) -------------------------------------------------------------
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    Ws, Gs = [], []
    for s in specs:
        Ws.append((0.02 * torch.randn(s.m, s.n, device=dev, generator=gen)).to(w_dtype))
        Gs.append(torch.randn(s.m, s.n, device=dev, generator=gen).to(w_dtype))
    bases = {}
    xs = []
    for li, s in enumerate(specs):
        X, basis = workload.activations_torch(n_tokens, s.n, 0.15,
                                              seed=workload.seed_for(wl["config"], li // wl["per_layer"],
                                                                     li % wl["per_layer"]),
                                              device=dev, dtype=getattr(torch, wl.get("x_dtype", "bfloat16")),
                                              basis=bases.get(s.n))
        bases[s.n] = basis
        xs.append(X)
    del bases
    torch.cuda.synchronize()
    print("[bench] inputs ready", file=sys.stderr, flush=True)

    col_l2 = args.norm == "col_l2"
    # Table 9: the applied scale is tau sqrt(max(m, n)/m) on the sign update U, tau sqrt(max(m, n)) on
    # the column-l2 one
    scales = [0.2 * (max(s.m, s.n) / (1.0 if col_l2 else s.m)) ** 0.5 for s in specs]
    group = DobbGroup(Ws, [s.nb for s in specs], grads=Gs, n_tokens=n_tokens, lr=wl["lr"], weight_decay=0.1,
                      momentum=0.9, norm=dobb.DOBB_NORM_COL_L2 if col_l2 else dobb.DOBB_NORM_SIGN,
                      update_scales=scales, streams=args.streams,
                      basis_dtype=torch.bfloat16 if args.basis == "bf16" else torch.float32)
    K_ORTH = args.orth_iters
    REFRESH_MODE = dobb.DOBB_REFRESH_ORTH_ITER_CHOLQR if args.qr == "cholesky" else dobb.DOBB_REFRESH_ORTH_ITER
    beta = 0.9
    # setup: first capture and the exact refresh (untimed, but measured once)
    group.accumulate(xs, 0.0)
    torch.cuda.synchronize()
    nbs = [s.nb for s in specs]
    dobb.dobb_profile_reset()
    dobb.dobb_profile_enable(True)
    t0 = time.perf_counter()
    group.refresh(dobb.DOBB_REFRESH_EXACT, 0, warm_start=False)
    torch.cuda.synchronize()
    exact_ms = (time.perf_counter() - t0) * 1e3
    dobb.dobb_profile_enable(False)
    jac_cold = jacobi_entry(dobb.dobb_profile_read(), [i.cpu() for i in group.info], nbs, exact_ms)
    dobb.dobb_profile_reset()
    info = torch.cat([i for i in group.info]).cpu()
    print(f"[bench] exact refresh {exact_ms:.1f} ms, sweeps min/max {int(info.min())}/{int(info.max())}",
          file=sys.stderr, flush=True)

    def full_step():
        group.refresh_step(xs, beta, REFRESH_MODE, K_ORTH)

    for _ in range(args.warmup):
        full_step()
    torch.cuda.synchronize()
    # the step as a HIP graph (the same kernels on the same buffers, without the host launch work and
    # the gaps between launches), and the non-refresh step likewise
    if args.eager:
        step_fn, nonrefresh_fn = full_step, group.step
    else:
        graph_full = group.capture_refresh_step(xs, beta, REFRESH_MODE, K_ORTH)
        graph_step = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph_step):
            group.step()
        step_fn, nonrefresh_fn = graph_full.replay, graph_step.replay
        step_fn()
        nonrefresh_fn()
        torch.cuda.synchronize()

    # ---- timed region: K whole steps, kernel timer off -------------------------------------------
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step_fn()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] {ms_per_step:.3f} ms per step", file=sys.stderr, flush=True)
    # ---- the same K steps again with the kernel timer on: per-launch durations from event pairs on
    # each kernel's own stream
    dobb.dobb_profile_reset()
    dobb.dobb_profile_enable(True)
    ev2, ev3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev2.record(stream)
    for _ in range(args.steps):
        full_step()
    ev3.record(stream)
    torch.cuda.synchronize()
    dobb.dobb_profile_enable(False)
    ms_per_step_timer = ev2.elapsed_time(ev3) / args.steps
    kernels = dobb.dobb_profile_read()
    dobb.dobb_profile_reset()
    print(f"[bench] {ms_per_step_timer:.3f} ms per step with the kernel timer on", file=sys.stderr, flush=True)

    # ---- the same pieces without the timer: non-refresh step, capture, refresh ----------------
    def timed(fn, reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps
    reps = max(3, args.steps)
    full_ms_untimed = timed(step_fn, reps)
    full_ms_eager = timed(full_step, reps)
    step_ms = timed(nonrefresh_fn, reps)
    acc_ms = timed(lambda: group.accumulate(xs, beta), reps)
    ref_ms = timed(lambda: group.refresh(REFRESH_MODE, K_ORTH), reps)
    # the exact refresh warm-started from the current basis (the exact mode's steady state)
    dobb.dobb_profile_reset()
    dobb.dobb_profile_enable(True)
    warm_ms = timed(lambda: group.refresh(dobb.DOBB_REFRESH_EXACT, 0, warm_start=True), 1)
    dobb.dobb_profile_enable(False)
    jac_warm = jacobi_entry(dobb.dobb_profile_read(), [i.cpu() for i in group.info], nbs, warm_ms)
    dobb.dobb_profile_reset()
    # the other schedule: one stream, or the narrow and the wide blocks on two overlapping streams
    other = 3 - args.streams
    other_ms = None
    if args.compare_streams:
        group.set_streams(other)
        other_ms = timed(full_step, reps)
        group.set_streams(args.streams)

    # ---- roofline: every kernel with a work model; the dominant one (most time) is reported --------
    g_bytes = Gs[0].element_size()
    w_bytes = Ws[0].element_size()
    work = kernel_work(specs, n_tokens, g_bytes, w_bytes, args.norm, K_ORTH, xs[0].element_size(), args.qr)
    per_kernel = {}
    for name, (launches, total_ms) in kernels.items():
        ent = {"launches_per_step": launches / args.steps, "ms_per_step": round(total_ms / args.steps, 4),
               "avg_launch_ms": round(total_ms / launches, 5)}
        if name in work:
            ent.update({k: (round(v, 4) if isinstance(v, float) else v)
                        for k, v in roofline_entry(work[name], total_ms / args.steps / 1e3).items()})
        per_kernel[name] = ent
    dom = max((k for k in per_kernel if k in work), key=lambda k: per_kernel[k]["ms_per_step"])
    d = per_kernel[dom]
    launches = d["launches_per_step"]
    unit_work = work[dom]["bytes"] if d["bound"] == "hbm" else work[dom]["flops"]
    roofline = {"kernel": dom, "bound": d["bound"], "achieved": d["achieved"], "peak": d["peak"], "unit": d["unit"],
                "frac": d["frac"],
                # counters were taken on the full GPT-2 XL set only
                "traffic": (measured_traffic(dom) if args.workload == "gpt2xl" and layers == 48
                            and args.norm == "sign" and K_ORTH == 1 and args.qr == "householder" else None),
                "work_per_launch": unit_work / launches,
                "work_unit": "bytes" if d["bound"] == "hbm" else "flop",
                "impl_bytes_per_launch": work[dom].get("impl_bytes", 0.0) / launches,
                "avg_launch_ms": d["avg_launch_ms"], "launches_per_step": launches}

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(group, xs, specs, wl, layers, col_l2, K_ORTH)

    amort = lambda T: (ms_per_step + (T - 1) * step_ms) / T
    out = {
        "metric": METRIC, "value": round(ms_per_step, 3), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl["text"].format(L=layers, N=n_tokens) + f"; capture + orthogonal-iteration "
                               f"refresh (k={K_ORTH}, {args.qr} QR) + step every step"
                               + ("; column-l2 normalisation" if col_l2 else "")
                               + ("; bf16 basis" if args.basis == "bf16" else ""),
                   "matrices": len(specs), "params": workload.param_count(specs), "tokens": n_tokens,
                   "refresh_period": 1, "streams": args.streams, "basis": args.basis, "qr": args.qr,
                   "launch": "eager" if args.eager else "hip graph"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "breakdown_ms": {"full_step_kernel_timer_on": round(ms_per_step_timer, 3),
                         "full_step_again": round(full_ms_untimed, 3),
                         "full_step_eager": round(full_ms_eager, 3),
                         f"full_step_{other}_stream{'s' if other > 1 else ''}":
                             None if other_ms is None else round(other_ms, 3),
                         "step_nonrefresh": round(step_ms, 3),
                         "accumulate": round(acc_ms, 3), f"refresh_orth_iter_k{K_ORTH}": round(ref_ms, 3),
                         "refresh_exact_cold": round(exact_ms, 1), "refresh_exact_warm": round(warm_ms, 1),
                         "amortized_T10": round(amort(10), 3),
                         "amortized_T9": round(amort(9), 3)},
        "kernels": per_kernel,
        # the exact refresh (setup from the identity, and warm-started from the current basis): the
        # Jacobi kernels' rotation work against the fp64 vector peak
        "refresh_exact": {"cold": jac_cold, "warm": jac_warm},
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
