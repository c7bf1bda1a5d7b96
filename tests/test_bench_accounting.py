"""bench.py's host-side accounting, on the CPU: the algorithmic bytes and
flops its rooflines divide by, the workspace record it prices the kernels'
counter traffic against, and the one-GPU contract of its command line."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_record_bytes_matches_the_layout():
    # w, Q e^Gam, K~^T (64 x d_k each) and u (64 x d_v) in bf16, the six
    # lower A_qk fragments of 512 elements, and e^{Gam_C} (d_k fp32)
    assert bench.record_bytes(128, 128, 2) == (3 * 64 * 128 + 64 * 128 + 6 * 512) * 2 + 128 * 4 == 72192
    assert bench.record_bytes(64, 128, 4) == (64 * (3 * 64 + 128) + 6 * 512) * 4 + 64 * 4


def test_path_bytes_of_the_single_sequence_and_the_packed_chunk():
    # one 8192-row sequence, H = 32, d = 128, bf16: q, k, v (bf16), g (fp32),
    # beta (fp32) in, o (bf16) out, the final state (fp32) out
    per_row_head = 2 * 128 * 2 + 128 * 2 + 128 * 4 + 4 + 128 * 2
    state = 32 * 128 * 128 * 4
    single = bench.path_bytes(8192, 32, 128, 128, 2, 1, False, True)
    assert single == 8192 * 32 * per_row_head + state == 405_798_912
    # 16 packed sequences with their states gathered from and scattered to
    # the pool
    packed = bench.path_bytes(8192, 32, 128, 128, 2, 16, True, True)
    assert packed == 8192 * 32 * per_row_head + 2 * 16 * state == 470_810_624


def test_kernel_bytes_add_up_to_the_path_and_the_records():
    # the intra kernel reads the inputs and writes one record per (chunk,
    # head); the scan reads the records back, reads and writes the states
    # and writes o: together the path's bytes plus the records twice
    lengths = [28, 288, 498, 773, 330, 211, 505, 1313, 311, 179, 1, 716, 138, 272, 2330, 299]
    T, H = sum(lengths), 32
    n = bench.chunk_count(lengths)
    assert n == sum(-(-L // 64) for L in lengths) == 137
    intra = bench.intra_bytes(T, H, 128, 128, 2, n)
    scan = bench.scan_bytes(T, H, 128, 128, 2, n, 16, True, True)
    rec = n * H * bench.record_bytes(128, 128, 2)
    assert intra + scan == bench.path_bytes(T, H, 128, 128, 2, 16, True, True) + 2 * rec


def test_path_flops_of_one_full_chunk():
    # one 64-row chunk, one head, d_k = d_v = d: A_kk and A_qk over the lower
    # triangle (with the diagonal), w and u through the triangular inverse,
    # the inverse itself (about C^3 / 3), then w S, Q~ S, A_qk U and K~^T U
    C, d, tri = 64, 128, 64 * 65 // 2
    intra = 2 * tri * d * 2 + 2 * tri * (d + d) + C ** 3 // 3
    scan = 2 * C * d * d * 2 + 2 * tri * d + 2 * C * d * d
    assert bench.path_flops([64], 1, d, d, intra_only=True) == intra
    assert bench.path_flops([64], 1, d, d) == intra + scan
    # a ragged last chunk counts its own rows only, and heads multiply
    assert bench.path_flops([64 + 10], 3, d, d) == 3 * (bench.path_flops([64], 1, d, d)
                                                         + bench.path_flops([10], 1, d, d))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    for argv in (["--gpus", "2"], ["--gpus", "8"]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2
        assert "one GPU only" in r.stderr
        assert r.stdout == ""
