"""Host-side measurement logic of bench.py (CPU only): the per-kernel work model against the totals
the GPT-2 XL matrix set fixes independently, the exact refresh's flop count, and the counter
summary's parsing and ratios on a synthetic rocprofv3 CSV."""
import csv
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workload  # noqa: E402


def test_work_model_gpt2xl_totals():
    specs = workload.gpt2_xl_set(16)
    P = workload.param_count(specs)
    assert P == 1_474_560_000
    w = bench.kernel_work(specs, 16384)
    # projection and reconstruction: 2 m n nb flops each, 4 m n nb together = 1.180e12 for this set
    gemm = w["step_wide_fused_f16"]["flops"] + w["step_fused_f16"]["flops"]
    assert gemm == pytest.approx(1.17965e12, rel=1e-4)
    # the split products actually issued: five fp16 products in each one-pass kernel, the nb = 100
    # blocks padded to 112 basis rows and a contraction 128 deep, the nb = 400 blocks to 416 rows and
    # a contraction 400 deep
    assert w["step_fused_f16"]["issued"] == pytest.approx(2.5 * w["step_fused_f16"]["flops"] * 112 * 128 / 100 ** 2)
    assert w["step_wide_fused_f16"]["issued"] == pytest.approx(2.5 * w["step_wide_fused_f16"]["flops"] * 416 / 400)
    # the method's bytes: M read + written, G read (12 B per parameter with fp32 G); W read + written
    # (8 B per parameter with fp32 W): together the step's 20 B per parameter, with no sign bytes in
    # either one-pass kernel
    P_wide = 48 * 1600 * 6400
    assert w["step_wide_fused_f16"]["bytes"] == 20 * P_wide
    assert w["step_fused_f16"]["bytes"] == 20 * (P - P_wide)
    assert w["step_fused_f16"]["impl_bytes"] == 0 and w["step_wide_fused_f16"]["impl_bytes"] == 0
    assert "project_f16x3" not in w and "reconstruct_f16x2" not in w
    # capture: bf16 activations of 16384 tokens for all 192 weights, 17.6 GB read once.  The nb = 100
    # launches (768 tile pairs each) run unsplit, so the EMA's A read + write is theirs; the wide
    # nb = 400 launch splits its tokens four ways (fp32 sums of at most 4096 tokens), and the reduce
    # kernel reads and writes A for it
    A_100 = 8.0 * 100 * 100 * 16 * 144
    x_bytes = w["accumulate_syrk_bf16"]["bytes"] - A_100 + w["accumulate_syrk_wide"]["bytes"]
    assert x_bytes == pytest.approx(17.6e9, rel=2e-3)
    assert bench.capture_splits(1600, 100, 48, 16384, True) == 1
    assert bench.capture_splits(6400, 400, 48, 16384, True) == 4
    assert w["accumulate_reduce"]["bytes"] == 8.0 * 400 * 400 * 16 * 48
    # only the nb = 400 weights (fc-proj) take the wide capture kernel and the split basis planes
    assert w["accumulate_syrk_wide"]["bytes"] == 2 * 16384 * 6400 * 48
    assert w["split_q"]["bytes"] == 14 * 400 * 400 * 16 * 48
    # k = 2 doubles every refresh kernel's work and nothing else
    w2 = bench.kernel_work(specs, 16384, orth_iters=2)
    for k in ("refresh_gemm", "qr_block", "qr_update", "qr_form", "qr_panel"):
        assert w2[k]["flops"] == 2 * w[k]["flops"]
    assert w2["step_wide_fused_f16"] == w["step_wide_fused_f16"]


def test_jacobi_flop_count():
    # nb = 2: one pair, so a sweep is one rotation; it combines 2 rows and 2 columns of A (8 entries)
    # and 2 columns of V (4 entries), 3 flops each: 36 flops
    kern = {"jacobi_sweep": (5, 1.0), "jacobi_rotate_v": (5, 1.0)}
    e = bench.jacobi_entry(kern, [torch.tensor([3, -1, 2], dtype=torch.int32)], [2], 10.0)
    assert e["flops"] == 36 * (3 + 0 + 2)        # a block that did not converge (-1) counts no sweep
    assert e["jacobi_kernels_ms"] == 2.0
    assert e["sweeps_mean"] == pytest.approx(5 / 3, abs=0.01) and e["sweeps_max"] == 3
    # 9 nb^2 (nb - 1) per sweep for a wider block; the rate counts the Jacobi kernels' time only
    kern = {"jacobi_sweep": (1, 5e-4), "jacobi_sweep_fp64": (1, 3e-4), "jacobi_rotate_v": (1, 2e-4),
            "refresh_gemm": (1, 5.0)}
    e = bench.jacobi_entry(kern, [torch.tensor([1], dtype=torch.int32)], [100], 1.0)
    assert e["flops"] == 9 * 100 * 100 * 99
    assert e["achieved"] == pytest.approx(9 * 100 * 100 * 99 / 1e-6 / 1e12, rel=1e-3)   # TFLOP/s
    assert e["frac"] == pytest.approx(e["achieved"] / 78.6, rel=1e-3) and e["bound"] == "alu"
    # nb = 400 runs block Jacobi (its fp32 working matrix, 640 KB, exceeds the LDS): 10 index blocks
    # of 40, 9 rounds of 5 sub-problem sweeps at 80 (9 80^2 79 each), 10 tile pairs (4 80^3 each) and
    # 5 V updates (2 400 80^2 each); its kernels' time is counted
    assert bench.block_jacobi(192) is None and bench.block_jacobi(400) == (10, 40)
    assert bench.block_jacobi(300) == (8, 40) and bench.block_jacobi(301) == (8, 40)
    per_round = 5 * 9 * 80 * 80 * 79 + 10 * 4 * 80 ** 3 + 5 * 2 * 400 * 80 * 80
    kern = {"jacobi_block_sub": (9, 20.0), "jacobi_block_apply": (9, 10.0), "jacobi_init": (1, 5.0)}
    e = bench.jacobi_entry(kern, [torch.tensor([10, 9], dtype=torch.int32)], [400], 40.0)
    assert e["flops"] == pytest.approx(9 * per_round * 19)
    assert e["jacobi_kernels_ms"] == pytest.approx(30.0)


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        wr.writerows(rows)


def test_counter_summary_ratios(tmp_path, capsys):
    wide = "void dobb::(anonymous namespace)::k_proj_wide<13, 0, false>(long, long, int)"
    rows_k = "void dobb::(anonymous namespace)::k_proj_rows<4, 128, 0, false, false>(long, long)"
    other = "void at::native::elementwise_kernel<128, 4>(int)"
    a = []
    for d, k, wait in [(1, wide, 30), (2, wide, 50), (3, rows_k, 20), (4, other, 99)]:
        a += [dict(Dispatch_Id=d, Kernel_Name=k, Counter_Name="SQ_WAVE_CYCLES", Counter_Value=100),
              dict(Dispatch_Id=d, Kernel_Name=k, Counter_Name="SQ_WAIT_INST_ANY", Counter_Value=wait)]
    b = []
    for d, k in [(1, wide), (2, wide), (3, rows_k)]:
        b += [dict(Dispatch_Id=d, Kernel_Name=k, Counter_Name="TCC_HIT_sum", Counter_Value=3),
              dict(Dispatch_Id=d, Kernel_Name=k, Counter_Name="TCC_MISS_sum", Counter_Value=1)]
    _write_csv(tmp_path / "a.csv", a)
    _write_csv(tmp_path / "b.csv", b)
    bench.counter_summary([str(tmp_path / "a.csv"), str(tmp_path / "b.csv")])
    out = capsys.readouterr().out.strip().splitlines()
    assert out[0].startswith("| kernel function | launches | dependency wait %")
    table = {ln.split("|")[1].strip(): [c.strip() for c in ln.split("|")[2:-1]] for ln in out[2:]}
    assert set(table) == {"`k_proj_wide`", "`k_proj_rows`"}      # not a library kernel: left out
    assert table["`k_proj_wide`"][0] == "2"                        # two dispatches
    assert table["`k_proj_wide`"][1] == "40"                       # (30 + 50) / (100 + 100)
    assert table["`k_proj_rows`"][1] == "20"
    assert table["`k_proj_wide`"][-1] == "75"                      # L2 hits 3 of 4
    assert table["`k_proj_wide`"][4] == "–"                        # counter not taken


def test_host_cores_reports_affinity_and_model():
    cores, facts = bench.host_cores()
    assert 1 <= cores <= 16
    assert facts["nproc"] >= 1 and facts["affinity"] and facts["cpu_model"]
    n_aff = sum(int(r.split("-")[1]) - int(r.split("-")[0]) + 1 if "-" in r else 1
                for r in facts["affinity"].split(","))
    assert cores == min(n_aff, 16)
