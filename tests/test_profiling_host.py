"""Host-side arithmetic of the counter summaries kept in profiles/: the
per-kernel-group sums, the share of wave cycles and the instructions per
MFMA, on a small synthetic rocprofv3 counter_collection / kernel_stats pair."""
import csv

from decoder_only_pretraining_amd import profiling as P


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def test_counter_table_sums_and_ratios(tmp_path):
    head = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    gemm = "void gk::gemm_kmaj_kernel<256, gk::EpPart, 0, gk::NoDeq, true>(...)"
    attn = "void gk::attn_bwd_pair_kernel<128>(...)"
    # pass 1: wave cycles and a wait counter; pass 2: instruction counts
    _write(tmp_path / "p1.csv", head, [
        [1, gemm, "SQ_WAVE_CYCLES", 1000.0], [1, gemm, "SQ_WAIT_ANY", 250.0],
        [2, gemm, "SQ_WAVE_CYCLES", 1000.0], [2, gemm, "SQ_WAIT_ANY", 150.0],
        [3, attn, "SQ_WAVE_CYCLES", 500.0]])
    _write(tmp_path / "p2.csv", head, [
        [1, gemm, "SQ_INSTS_MFMA", 100.0], [1, gemm, "SQ_INSTS_VALU", 150.0],
        [1, gemm, "SQ_VALU_MFMA_BUSY_CYCLES", 3200.0],
        [2, gemm, "SQ_INSTS_MFMA", 100.0], [2, gemm, "SQ_INSTS_VALU", 250.0],
        [2, gemm, "SQ_VALU_MFMA_BUSY_CYCLES", 3200.0]])
    _write(tmp_path / "stats.csv", ["Name", "Calls", "TotalDurationNs"], [
        [gemm, 4, 400000.0], [attn, 2, 300000.0]])
    lines = P.counter_table([str(tmp_path / "p1.csv"), str(tmp_path / "p2.csv")],
                            str(tmp_path / "stats.csv"))
    text = "\n".join(lines)
    gemm_label = "gemm weight gradients, token-major K-major kernel"
    assert f"== {gemm_label}: 2 dispatches, 100.0 us avg" in text
    assert "== attn_bwd_pair (dK/dV + dQ): 1 dispatches, 150.0 us avg" in text
    # 400 of 2000 wave cycles waiting
    assert any("SQ_WAIT_ANY" in l and "400" in l and "20.0% of wave cycles" in l for l in lines)
    # 400 VALU over 200 MFMA; 6400 busy cycles over 200 MFMA
    assert any("per MFMA: VALU 2.00" in l and "MFMA-busy cycles per MFMA 32.0" in l for l in lines)
    # groups with no counters are left out
    assert "mix_norm" not in text
