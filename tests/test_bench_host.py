"""Host-side pieces of bench.py (no GPU): the algorithmic byte and flop counts it divides
by, the instance label it reports, and the one-GPU guard."""
import os
import subprocess
import sys

import kda_synth as ks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_of_the_long_workload():
    wl = ks.WORKLOADS["long"]
    ht = 4 * 32 * 16384
    # q, k, z, v, o at 128 bf16 each, beta 2 B; two fp32 states of 128 x 128 per head; A_log and dt_bias
    assert bench.algorithmic_bytes(wl) == ht * 1282 + 2 * 128 * 128 * 128 * 4 + 32 * 4 + 32 * 128 * 4 == 2705342592
    # scalar-decay gate: one bf16 gate value per head-token, one bias per head
    assert bench.algorithmic_bytes(wl, scalar_gate=True) == ht * 1028 + 2 * 128 * 128 * 128 * 4 + 32 * 4 + 32 * 4


def test_forward_flops_per_head_token():
    # 6KV + (C-1)K + (C+1)(K+V) + (C-1)(K+V) + C^2/3 at K = V = 128, C = 64
    assert abs(bench.forward_flops_per_head_token(128, 128, 64) - 140501.333) < 1e-2


def test_kernel_labels_follow_the_forward_plan():
    W = ks.WORKLOADS
    assert bench.kernel_label(W["long"]) == bench.KERNEL_NAME == "kda::chunk_fwd_pc_kernel<128,64,32,false,false>"
    assert bench.kernel_label(W["long"], True) == "kda::chunk_fwd_pc_kernel<128,64,32,true,false>"
    assert bench.kernel_label(W["long"], norm=True) == "kda::chunk_fwd_pc_kernel<128,64,32,false,true>"
    assert bench.kernel_label(W["nano"]) == "kda::chunk_fwd_pc_kernel<64,64,32,false,false>"
    assert bench.block_tokens(W["long"]) == 32 and bench.block_tokens(W["tiny"]) == 16
    assert bench.kernel_label(W["tiny"]) == "kda::chunk_fwd_kernel<float,16,16,16>"
    assert bench.kernel_label(W["adjoint"]) == "kda::chunk_fwd_kernel<float,128,16,32>"


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2 and "one GPU" in p.stderr
