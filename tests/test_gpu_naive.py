"""Parity of the naive (expand-then-attend) ablation, through the C ABI, with
the fp64 oracle's naive form, and agreement with the absorbed path on the same
inputs (the two bracketings compute the same attention).

Bars as for the absorbed path: max-abs <= 2e-2 beyond the final bf16 output
rounding and relative L2 <= 5e-3; FP8 caches max-abs <= 6e-2.
"""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from head_latent_attention_mla_amd import workloads as W

from test_gpu_parity import SCALE, MAX_ABS, _assert_close, _f64, small

pytestmark = pytest.mark.gpu

KINDS = ["contig", "tiny", "tiny_unit", "paged", "verify", "verify_h", "fp8", "fp8_paged"]


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from head_latent_attention_mla_amd import mla as m
    return m


@pytest.mark.parametrize("kind", KINDS)
def test_naive_vs_oracle_and_absorbed(mla, kind):
    w = small(kind)
    print(f"[naive] {kind} {w}", flush=True)
    inp = W.generate(w)
    q, w_uk, w_uv, cache = W.to_torch(inp)
    fp8 = w.cache_dtype == "fp8"
    out_n = mla.naive_decode(q, cache, w_uk, w_uv, SCALE, w.causal)
    out_a = mla.decode(q, cache, w_uk, w_uv, SCALE, w.causal)
    torch.cuda.synchronize()
    ref = O.naive_decode(inp, SCALE)
    m = _assert_close(_f64(out_n), ref, fp8=fp8, what="naive vs oracle")
    print(f"[naive] {kind}: {m}", flush=True)
    # both bracketings on the GPU agree with each other within the combined bar
    d = np.abs(_f64(out_n) - _f64(out_a)) - 2.0 ** -7 * np.abs(ref)
    assert float(np.max(d)) <= 2 * (6e-2 if fp8 else MAX_ABS), kind


def test_naive_workspace_and_limits(mla):
    # transposed W_UV + fp32 scores [2, 1, 128, 256] + row sums [2, 1, 128]
    assert mla.naive_workspace_bytes(2, 1, 128, 256) == 128 * 128 * 512 * 2 + 2 * 128 * 256 * 4 + 1024
    assert mla.naive_workspace_bytes(0, 1, 128, 256) == 0
    w = small("verify").with_(s_q=5)
    inp = W.generate(w)
    q, w_uk, w_uv, cache = W.to_torch(inp)
    with pytest.raises(mla.MLAError, match="UNSUPPORTED"):
        mla.naive_decode(q, cache, w_uk, w_uv, SCALE, True)


def test_naive_full_size(mla):
    """The DeepSeek-V3-shaped workload at full size (B=64, H=128, T=4096):
    every output against the oracle's absorbed form in fp64 (pinned equal to
    the naive form by associativity), and sampled (sequence, head) pairs
    against the naive form itself."""
    w = W.WORKLOADS["dsv3"]
    print(f"[naive] full {w}", flush=True)
    inp = W.generate(w)
    q, w_uk, w_uv, cache = W.to_torch(inp)
    out = mla.naive_decode(q, cache, w_uk, w_uv, SCALE, w.causal)
    torch.cuda.synchronize()
    got = _f64(out)
    m = _assert_close(got, O.absorbed_decode(inp, SCALE), what="naive full vs absorbed fp64")
    print(f"[naive] full: {m}", flush=True)
    rng = np.random.default_rng(7)
    pairs = [(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(4)]
    ref = O.naive_decode(inp, SCALE, pairs=pairs)
    for b, h in pairs:
        _assert_close(got[b, :, h], ref[b, :, h], what=f"naive full ({b},{h})")
