"""Split-T scan with FP8 arithmetic (mla_decode_partial_fp8) on FP8 caches,
through the C ABI, against the fp64 oracle, on the FP8 bar: max-abs <= 6e-2
beyond the final bf16 output rounding, for every case.  The E4M3 rounding of
queries and weights averages out only over many comparable weights; where a
query row's largest probability exceeds 1/32 of its total (few rows, a
peaked softmax) the call recomputes that (sequence, row group) with bf16
arithmetic -- those outputs are then the bf16-arithmetic path's, bit for
bit.  Relative L2 is reported and held to 6e-2 (E4M3 queries
and weights cost a few 1e-2 of it where nothing is flagged)."""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from head_latent_attention_mla_amd import workloads as W

from test_gpu_parity import SCALE, _assert_close, _f64

pytestmark = pytest.mark.gpu
REL_L2_FP8_MATH = 6e-2


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from head_latent_attention_mla_amd import mla as m
    return m


CASES = dict(
    contig=W.Workload("f8m_contig", B=3, H=128, s_q=1, causal=False, T=700, cache_dtype="fp8", seed=71),
    verify=W.Workload("f8m_verify", B=2, H=128, s_q=2, causal=True, T=333, cache_dtype="fp8", T_stride=350, seed=72),
    paged=W.Workload("f8m_paged", B=4, H=128, s_q=1, causal=False, T_range=(70, 900), paged=True,
                     cache_dtype="fp8", seed=73),
    heads40=W.Workload("f8m_h40", B=2, H=40, s_q=3, causal=True, T=130, cache_dtype="fp8", seed=74),
    short=W.Workload("f8m_short", B=5, H=16, s_q=1, causal=False, T_range=(1, 63), cache_dtype="fp8", seed=75),
    literal=W.Workload("f8m_lit", B=2, H=128, s_q=1, causal=False, T=256, cache_dtype="fp8", scaling="literal",
                       seed=76),
)


def _run(mla, inp, num_splits=0):
    q, w_uk, w_uv, cache = W.to_torch(inp)
    w = inp["workload"]
    out = mla.decode(q, cache, w_uk, w_uv, SCALE, causal=w.causal, num_splits=num_splits, fp8_math=True)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("kind", list(CASES))
def test_fp8_math_vs_oracle(mla, kind):
    w = CASES[kind]
    print(f"[fp8 math] {kind} {w}", flush=True)
    inp = W.generate(w)
    got = _f64(_run(mla, inp))
    ref = O.naive_decode(inp, SCALE, causal=w.causal)
    m = _assert_close(got, ref, fp8=True, what=kind)
    print(f"[fp8 math] {kind}: {m}", flush=True)
    assert m["rel_l2"] <= REL_L2_FP8_MATH, (kind, m)


def test_fp8_math_split_counts(mla):
    w = CASES["contig"]
    inp = W.generate(w)
    ref = O.naive_decode(inp, SCALE, causal=False)
    for ns in (1, 3, 11):
        m = _assert_close(_f64(_run(mla, inp, num_splits=ns)), ref, fp8=True, what=f"ns={ns}")
        assert m["rel_l2"] <= REL_L2_FP8_MATH


def test_fp8_math_peaked_softmax(mla):
    """Queries scaled two-fold: the softmax is peaked enough that E4M3
    queries and weights alone miss the FP8 bar; the recomputed rows meet it."""
    w = W.Workload("f8m_peak2", B=2, H=128, s_q=1, causal=False, T=600, cache_dtype="fp8", seed=77)
    inp = W.generate(w)
    inp["q"] = W.to_bf16_bits(O.bf16_to_f64(inp["q"]) * 2.0)
    got = _f64(_run(mla, inp))
    m = _assert_close(got, O.naive_decode(inp, SCALE, causal=False), fp8=True, what="two-fold queries")
    print(f"[fp8 math] two-fold: {m}", flush=True)
    assert m["rel_l2"] <= REL_L2_FP8_MATH, m


def test_fp8_math_large_score_range(mla):
    """Queries scaled six-fold: the softmax reference moves several times
    (steps of 2^8) and every row is recomputed with bf16 arithmetic -- the
    output equals that scan's bit for bit.  At six-fold scores the bf16
    storage of the latent query and of the dequantised cached values alone
    moves the peaked outputs by up to 0.114 (a CPU model of exactly those
    roundings with exact fp64 bookkeeping), beyond the FP8 max-abs bar for
    any bf16-precision path, so here the oracle comparison holds relative
    L2 (model: 0.008) and finiteness; the two-fold case above holds max-abs."""
    w = W.Workload("f8m_range", B=2, H=128, s_q=1, causal=False, T=600, cache_dtype="fp8", seed=77)
    inp = W.generate(w)
    inp["q"] = W.to_bf16_bits(O.bf16_to_f64(inp["q"]) * 6.0)
    q, w_uk, w_uv, cache = W.to_torch(inp)
    a = mla.decode(q, cache, w_uk, w_uv, SCALE, causal=False, fp8_math=True)
    b = mla.decode(q, cache, w_uk, w_uv, SCALE, causal=False, fp8_math=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.view(torch.int16).cpu().numpy(), b.view(torch.int16).cpu().numpy())
    m = O.compare(_f64(a), O.naive_decode(inp, SCALE, causal=False))
    print(f"[fp8 math] six-fold: {m}", flush=True)
    assert m["nonfinite"] == 0 and m["rel_l2"] <= REL_L2_FP8_MATH, m


def test_fp8_math_flagged_groups_take_the_bf16_arithmetic(mla):
    """Sequences of 1..24 rows: every query row's largest probability is at
    least 1/24 of its total, so every (sequence, row group) is recomputed --
    the output equals the bf16-arithmetic scan's bit for bit.  One sequence
    of 4096 unit-scale rows (scanned in 64 parts of 64 rows: the check is on
    the whole row, not the part) keeps the E4M3 arithmetic, so its output
    differs from the bf16-arithmetic one."""
    short = W.Workload("f8m_flag", B=4, H=128, s_q=1, causal=False, T_range=(1, 24), cache_dtype="fp8", seed=81)
    inp = W.generate(short)
    q, w_uk, w_uv, cache = W.to_torch(inp)
    a = mla.decode(q, cache, w_uk, w_uv, SCALE, causal=False, fp8_math=True)
    b = mla.decode(q, cache, w_uk, w_uv, SCALE, causal=False, fp8_math=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.view(torch.int16).cpu().numpy(), b.view(torch.int16).cpu().numpy())
    long = W.Workload("f8m_long", B=1, H=128, s_q=1, causal=False, T=4096, cache_dtype="fp8", seed=82)
    inp = W.generate(long)
    q, w_uk, w_uv, cache = W.to_torch(inp)
    a = mla.decode(q, cache, w_uk, w_uv, SCALE, causal=False, fp8_math=True)
    b = mla.decode(q, cache, w_uk, w_uv, SCALE, causal=False, fp8_math=False)
    torch.cuda.synchronize()
    assert not torch.equal(a, b)
    _assert_close(_f64(a), O.naive_decode(inp, SCALE, causal=False), fp8=True, what="long, E4M3 arithmetic")


def test_fp8_math_full_size(mla):
    """B=64, H=128, s_q=2 causal, T=16384 FP8 cache: every output against the
    oracle's absorbed form in fp64, and sampled (sequence, head) pairs
    against the naive form."""
    from test_gpu_parity import full_inputs
    w = W.WORKLOADS["fp8_cache"]
    print(f"[fp8 math] full {w}", flush=True)
    inp = full_inputs("fp8_cache")
    got = _f64(_run(mla, inp))
    m = _assert_close(got, O.absorbed_decode(inp, SCALE, causal=True), fp8=True, what="fp8 math full")
    print(f"[fp8 math] full: {m}", flush=True)
    rng = np.random.default_rng(3)
    pairs = [(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(3)] + [(0, 0), (w.B - 1, w.H - 1)]
    ref = O.naive_decode(inp, SCALE, causal=True, pairs=pairs)
    for b, h in pairs:
        _assert_close(got[b, :, h], ref[b, :, h], fp8=True, what=f"full ({b},{h})")
