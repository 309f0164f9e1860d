"""The benchmark's algorithmic byte counts (the numerator of every GB/s it prints),
against the t4096 workload's byte totals worked out by hand: each HBM byte a call
must move counted once, reads and writes, to 0.1 MB.

t4096: T = 4096 tokens, H = 7168 (a bf16 row is 14,336 B), E = 256 experts in
G = 8 groups, top-8. Per-expert rows R = T*K = 32,768; per-group rows at the
expected deduplicated count P = 21,687 (5.2947 groups per token).
"""
import pytest

import bench

T, H, E, G, K = 4096, 7168, 256, 8, 8
R, P = T * K, 21687


def mb(n):
    return round(n / 1e6, 1)


def test_dispatch_bytes_per_expert_bf16():
    # reads: x 58.72 MB + weights and indices 0.26 MB + slot_e 0.13 MB;
    # writes: 32,768 rows of 14,336 B plus 64 B of weights and indices
    r, w = bench.dispatch_bytes(T, H, K, G, R, "expert")
    assert (mb(r), mb(w), mb(r + w)) == (59.1, 471.9, 531.0)


def test_dispatch_bytes_per_group_bf16():
    r, w = bench.dispatch_bytes(T, H, K, G, P, "group")
    assert (mb(r), mb(w), mb(r + w)) == (59.1, 312.3, 371.4)


def test_dispatch_bytes_fp8():
    # a receive row: 7,168 e4m3 bytes + 56 fp32 scales + 64 B of metadata
    r, w = bench.dispatch_bytes(T, H, K, G, R, "expert", fp8=True)
    assert (mb(r), mb(w), mb(r + w)) == (59.1, 244.3, 303.4)
    r, w = bench.dispatch_bytes(T, H, K, G, P, "group", fp8=True)
    assert (mb(w), mb(r + w)) == (161.7, 220.8)


@pytest.mark.parametrize("rows,total", [(R, 528.7), (P, 369.9)])
def test_combine_bytes(rows, total):
    # reads: each distinct receive row once + weights + slots; writes: T bf16 rows
    r, w = bench.combine_bytes(T, H, K, rows)
    assert mb(w) == 58.7
    assert mb(r + w) == total


def test_layout_bytes_is_the_index_read_plus_the_layout_arrays():
    # reads topk_idx (128 KiB); writes counts/offsets, tok_group_mask, slot_e,
    # slot_g, recv_src_e (3 x 128 KiB), slot_tg (128 KiB) and recv_src_g (P ints)
    b = bench.layout_bytes(T, K, E, G, P)
    assert b == 4 * (T * K + 2 * E + 2 * G + 2 + T + 3 * T * K + T * G + P)
    assert mb(b) == 0.8
