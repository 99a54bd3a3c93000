"""The profile tables' generator (host only): kernel names lose only their
parameter list and the library's namespace, and a kernel-trace table lists every
kernel by total time with the stats file's figures in microseconds."""
import csv
import os

from block_sparse_cross_amd import counter_summary as cs


def test_strip_params_keeps_template_arguments():
    assert cs.strip_params("attn_fwd_bf16_kernel<128, unsigned short>(unsigned short const*, int)") \
        == "attn_fwd_bf16_kernel<128, unsigned short>"
    # parentheses inside template arguments stay; only the trailing list goes
    name = "k<4, f(at::T&)::{lambda(float)#1}>(int, char*)"
    assert cs.strip_params(name) == "k<4, f(at::T&)::{lambda(float)#1}>"
    assert cs.strip_params("__amd_rocclr_fillBufferAligned") == "__amd_rocclr_fillBufferAligned"


def test_trace_table(tmp_path):
    d = tmp_path / "kt"
    os.makedirs(d)
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
                    "StdDev"])
        w.writerow(["void splitkv::(anonymous namespace)::lse_merge_kernel<8>(float const*, int)",
                    "2", "3000", "1500", "10.0", "1000", "2000", "1"])
        w.writerow(["void splitkv::(anonymous namespace)::attn_bwd_dkdv_kernel<128>(int)",
                    "4", "27000", "6750", "90.0", "6000", "7000", "1"])
    lines = cs.trace_table(str(d)).strip().split("\n")
    assert lines[2] == "| attn_bwd_dkdv_kernel<128> | 4 | 27.0 | 6.8 | 6.0 | 7.0 | 90.00 |"
    assert lines[3] == "| lse_merge_kernel<8> | 2 | 3.0 | 1.5 | 1.0 | 2.0 | 10.00 |"
