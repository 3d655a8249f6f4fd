"""Host checks of bench.py: the algorithmic byte counts behind the roofline
object, worked out here from the workload shapes, and the one-GPU contract."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench      # noqa: E402
import workloads  # noqa: E402


def test_attention_bytes_chain_bf16():
    # 24/4 heads, head dim 256, 8 verify rows over 4096 cached positions:
    # every key and value row of the 4104 positions of each KV head read once
    # (2 B per bf16 value), the 8 x 24 query rows read and output rows written,
    # one fp32 log-sum-exp per row
    cfg = workloads.CONFIGS["C2"]
    kv = 4104 * 4 * (256 * 2) * 2
    q_out = 2 * (8 * 24 * 256 * 2)
    lse = 8 * 24 * 4
    assert bench.attn_algorithmic_bytes(cfg, np.array([4096])) == kv + q_out + lse == 17007360


def test_attention_bytes_4bit_and_window():
    # 4-bit cache: per position and KV head 128 code bytes + 8 fp16 scales, K and V
    cfg = workloads.CONFIGS["C4"]
    per_pos = 2 * (128 + 8 * 2)
    q_out = 2 * (16 * 24 * 256 * 2)
    lse = 16 * 24 * 4
    assert bench.attn_algorithmic_bytes(cfg, np.array([131072])) == 131088 * 4 * per_pos + q_out + lse
    # a window keeps only the last W key rows of the sequence
    assert bench.attn_algorithmic_bytes(cfg, np.array([131072]), window=2048) == 2048 * 4 * per_pos + q_out + lse


def test_attention_bytes_batch_sums_sequences():
    cfg = workloads.CONFIGS["C5"]
    lens = np.array([1000, 5000, 16000, 1024, 77, 3000, 9000, 12345])
    one = [bench.attn_algorithmic_bytes(workloads.small_variant(cfg, batch=1), np.array([L])) for L in lens]
    q_out_lse = 2 * (4 * 32 * 128 * 2) + 4 * 32 * 4           # per sequence
    kv = sum(o - q_out_lse for o in one)
    assert bench.attn_algorithmic_bytes(cfg, lens) == kv + 8 * q_out_lse


def test_delta_bytes_tree22():
    # one layer of the 22-node tree: committed fp32 state read (48 value heads,
    # 128 x 128), q and k (16 key heads) and v (48 value heads) of every node in
    # bf16, decay and beta fp32 per node and value head, outputs written in bf16,
    # every node's f16 state written
    cfg = workloads.DELTA_CONFIGS["D2"]
    s0 = 48 * 128 * 128 * 4
    qkv = 22 * (2 * 16 * 128 + 48 * 128) * 2
    gb = 22 * 48 * 8
    out = 22 * 48 * 128 * 2
    states = 22 * 48 * 128 * 128 * 2
    assert bench.delta_algorithmic_bytes(cfg) == s0 + qkv + gb + out + states == 38478080


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_attention_flops_and_binding_roof():
    # Q K^T and P V: 2 + 2 flops per (row, key, head-dim) element, rows =
    # 6 query heads x 16 nodes per KV head, 4 KV heads, 131088 keys
    cfg = workloads.CONFIGS["C4"]
    flops = bench.attn_algorithmic_flops(cfg, np.array([131072]))
    assert flops == 4 * (6 * 16) * 4 * 131088 * 256 == 51_545_899_008
    # at peak the matrix cores need longer than HBM needs for the bytes:
    # the 4-bit block is matrix-bound, the 4K bf16 chain HBM-bound
    t_mfma = flops / (bench.MFMA_PEAK_TFLOPS * 1e12)
    t_hbm = bench.attn_algorithmic_bytes(cfg, np.array([131072])) / (bench.HBM_PEAK_GBPS * 1e9)
    assert t_mfma > t_hbm and bench.uses_matrix_cores(cfg)
    c2 = workloads.CONFIGS["C2"]
    assert (bench.attn_algorithmic_flops(c2, np.array([4096])) / (bench.MFMA_PEAK_TFLOPS * 1e12)
            < bench.attn_algorithmic_bytes(c2, np.array([4096])) / (bench.HBM_PEAK_GBPS * 1e9))
    assert not bench.uses_matrix_cores(workloads.CONFIGS["C1"])          # fp32, 2 rows: vector ALU
