"""Host logic of the profile summariser: stage assignment, the w13/w2 split of
the grouped-GEMM launches, per-pass sums of multi-kernel stages, and the copy
calibration of the HBM counters (synthetic CSVs, no GPU)."""
import csv
import json

from fp8_grouped_gemm_select_amd import profsum

KERNELS = ["void moe::(anonymous namespace)::select_experts_kernel<4>(float const*, int)",
           "void moe::(anonymous namespace)::pr_count_kernel(int const*)",
           "void moe::(anonymous namespace)::pr_scatter_quant_kernel<1>(void const*)",
           "void moe::(anonymous namespace)::grouped_gemm_kernel<false>(unsigned char const*)",
           "void moe::(anonymous namespace)::act_requant_kernel<1>(void const*)",
           "void moe::(anonymous namespace)::grouped_gemm_kernel<false>(unsigned char const*)",
           "void moe::(anonymous namespace)::post_reorder_kernel(void const*)"]


def _write_counter(path, counter, values, copy_kib):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        did = 1
        for _ in range(2):  # two layer passes
            for k, v in zip(KERNELS, values):
                w.writerow({"Dispatch_Id": did, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})
                did += 1
        w.writerow({"Dispatch_Id": did, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter,
                    "Counter_Value": copy_kib})


def test_short_names_and_stages():
    assert profsum.short_name(KERNELS[0]) == "select_experts_kernel<4>"
    assert [profsum.stage_of(k) for k in KERNELS] == ["select", "pre_reorder", "pre_reorder", "gemm",
                                                      "act_requant", "gemm", "post_reorder"]
    assert profsum.stage_of("__amd_rocclr_copyBuffer") is None
    assert profsum.stage_of("void moe::(anonymous namespace)::select_rows_kernel<16>(float const*)") == "select"
    # kernels in a top-level anonymous namespace (the ceilings library) keep their names
    assert profsum.short_name("(anonymous namespace)::copy_kernel(HIP_vector_type<unsigned int, 4u> const*, long)") \
        == "copy_kernel"


def test_traffic_calibration_and_split(tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # KiB per dispatch; the 1 MiB copy reads as 512 KiB fetched and 1024 KiB written
    _write_counter(fetch, "FETCH_SIZE", [1, 2, 3, 100, 5, 50, 7], 512)
    _write_counter(write, "WRITE_SIZE", [1, 1, 1, 10, 2, 20, 3], 1024)
    t = profsum.traffic(str(fetch), str(write), 1 << 20, "tiny", "cmd")
    assert abs(t["fetch_factor"] - 2.0) < 1e-12 and abs(t["write_factor"] - 1.0) < 1e-12
    s = t["stages"]
    assert s["gemm_w13"]["fetch_bytes"] == 100 * 1024 * 2 and s["gemm_w2"]["fetch_bytes"] == 50 * 1024 * 2
    assert s["pre_reorder"]["fetch_bytes"] == (2 + 3) * 1024 * 2   # both kernels of a pass
    assert s["pre_reorder"]["write_bytes"] == 2 * 1024
    assert s["gemm_w2"]["traffic_bytes"] == 50 * 2048 + 20 * 1024
    assert s["gemm_w13"]["source_sha256"] == profsum.source_hash("gemm_w13")
    json.dumps(t)


def test_trace_table(tmp_path):
    path = tmp_path / "t.csv"
    cols = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        t, did = 0, 1
        for _ in range(3):
            for k, dur in zip(KERNELS, [10, 20, 30, 400, 40, 200, 50]):
                w.writerow({"Dispatch_Id": did, "Kernel_Name": k, "Start_Timestamp": t,
                            "End_Timestamp": t + dur * 1000})
                did += 1
                t += dur * 1000 + 5
    md = profsum.trace_md(str(path), "tiny", "cmd")
    assert "| gemm_w13 | 3 | 400.00 |" in md
    assert "| gemm_w2 | 3 | 200.00 |" in md
    assert "| pre_reorder | 3 | 50.00 |" in md


def test_counter_table(tmp_path):
    """MFMA busy over one XCD's share of GRBM_GUI_ACTIVE, FP8 flop from the MOPS
    counter, L2 hit rate, and stage 2's kernels summed per layer pass."""
    path = tmp_path / "c.csv"
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        did, t = 1, 0
        for _ in range(3):  # three layer passes
            for k, dur in zip(KERNELS, [10, 20, 30, 400, 40, 200, 50]):
                gemm = "grouped_gemm" in k
                vals = {"GRBM_GUI_ACTIVE": 8 * 1000, "SQ_VALU_MFMA_BUSY_CYCLES": 512 * 1000 if gemm else 0,
                        "SQ_INSTS_VALU_MFMA_MOPS_F8": 2e6 if gemm else 0, "TCC_HIT_sum": 3, "TCC_MISS_sum": 1}
                for name, v in vals.items():
                    w.writerow({"Dispatch_Id": did, "Kernel_Name": k, "Counter_Name": name, "Counter_Value": v,
                                "Start_Timestamp": t, "End_Timestamp": t + dur * 1000})
                did += 1
                t += dur * 1000 + 5
    md = profsum.counters_md([str(path)], "tiny", ["cmd"])
    # 512e3 busy cycles over (8e3 / 8 XCDs) x 1024 SIMDs = 50 %; 2e6 MOPS x 512 = 1.024 GFLOP
    assert "| gemm_w13 | 3 | 400.0 | 50.0 % | 1.0 | 75.0 % |" in md
    assert "| pre_reorder | 6 | 50.0 | 0.0 % | 0.0 | 75.0 % |" in md
