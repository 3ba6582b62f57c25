"""The bench's algorithmic counts (the numerators of its roofline figures),
checked against closed forms for the workloads it reports (CPU)."""
import bench


def test_dsv3_scan_counts_closed_form():
    B, H, T = 64, 128, 4096
    c = bench.algorithmic_counts(B, 1, H, [T] * B, causal=False)
    # every head scores 576 and averages 512 columns of every cached row
    assert c["flops_scan"] == 2 * B * H * T * (576 + 512) == 73_014_444_032
    # cache rows once (1152 B), latent queries in, latent outputs out (bf16)
    assert c["bytes_scan"] == B * T * 1152 + B * H * 1152 + B * H * 1024 == 319_815_680
    # the step adds the two absorption products (2 x 128 x 512 MACs per head and row)
    assert c["flops_step"] - c["flops_scan"] == 2 * 2 * B * H * 128 * 512


def test_causal_pairs_and_fp8_rows():
    # s_q = 4 causal: query j of a sequence of T rows sees T - 3 + j rows
    c = bench.algorithmic_counts(2, 4, 8, [10, 7], causal=True)
    pairs = sum(T - 4 + j + 1 for T in (10, 7) for j in range(4))
    assert c["flops_scan"] == pairs * 8 * (2 * 576 + 2 * 512)
    # an e4m3 row is 576 one-byte codes and a 4-byte scale
    f = bench.algorithmic_counts(2, 1, 8, [10, 7], causal=False, cache_elem_bytes=1, scale_bytes=4)
    assert f["bytes_cache"] == 17 * 580
