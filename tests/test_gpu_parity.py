"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bars (floating point, bf16 inputs, fp32 accumulation): every element within
max-abs 2e-2 of the oracle, plus -- for outputs stored as bf16 -- that
element's own rounding to bf16, |bf16(ref) - ref|; relative L2 <= 5e-3 over
the tensor with no allowance.  FP8 caches: max-abs 6e-2 on the same terms.
Small cases span several 64-row tiles, a ragged tail, partial row groups and
every cache kind; the full-size workloads are checked over the whole output
tensor, in the launch configuration the benchmark times.
"""
import functools
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import mla_oracle as O
from head_latent_attention_mla_amd import workloads as W

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(192.0)
MAX_ABS, REL_L2, MAX_ABS_FP8 = 2e-2, 5e-3, 6e-2
FP8_READY = True


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from head_latent_attention_mla_amd import mla as m
    return m


def _bits(t):
    return W.bf16_tensor_to_numpy_bits(t)


def _f64(t):
    if t.dtype == torch.bfloat16:
        return O.bf16_to_f64(_bits(t))
    return t.detach().double().cpu().numpy()


def bf16_rounding(ref):
    """|bf16(ref) - ref| element by element: the part of an output's error
    that its final rounding to bf16 accounts for (at most 2^-9 |ref|)."""
    r = np.asarray(ref, np.float64)
    return np.abs(O.bf16_to_f64(W.to_bf16_bits(r)) - r)


def materialisation_bound(inp, scale, causal=None, u=2.0 ** -9, pairs=None):
    """First-order bound, per output element, of the effect of storing every
    expanded key and value element in bf16 (relative rounding <= u), as the
    expand path and the naive ablation do (their keys and values are
    materialised in bf16 before the attention).  With p = softmax(s),
    s_t = scale <q, k_t> and out = sum_t p_t V_t:
      values:  |sum_t p_t V_t eps_t|              <= u sum_t p_t |V_t|
      keys:    |sum_t p_t ds_t (V_t - out)|       <= u sum_t p_t a_t |V_t - out|,
               a_t = scale sum_k |q_k K_nope[t, k]| (the rope keys are copied).
    Computed from the fp64 expansion of the oracle's inputs, for the listed
    (b, h) pairs only when ``pairs`` is given (zero elsewhere)."""
    w = inp["workload"]
    causal = w.causal if causal is None else causal
    q = O.bf16_to_f64(inp["q"])
    w_uk, w_uv = O.bf16_to_f64(inp["w_uk"]), O.bf16_to_f64(inp["w_uv"])
    B, s_q, H, _ = q.shape
    bound = np.zeros((B, s_q, H, 128))
    pairs = [(b, h) for b in range(B) for h in range(H)] if pairs is None else list(pairs)
    for b in sorted({pb for pb, _ in pairs}):
        T = int(inp["seqlens"][b])
        C = O.sequence_rows(inp, b)
        lat, rope = C[:, :512], C[:, 512:]
        for h in sorted({ph for pb, ph in pairs if pb == b}):
            K = lat @ w_uk[h].T
            V = lat @ w_uv[h]
            for j in range(s_q):
                n = O.visible_rows(T, s_q, j, causal)
                s = (K[:n] @ q[b, j, h, :128] + rope[:n] @ q[b, j, h, 128:]) * scale
                p = np.exp(s - s.max())
                p /= p.sum()
                out = p @ V[:n]
                a = scale * (np.abs(K[:n]) @ np.abs(q[b, j, h, :128]))
                bound[b, j, h] = u * (p @ np.abs(V[:n]) + (p * a) @ np.abs(V[:n] - out))
    return bound


def _assert_close(got, ref, fp8=False, what="", out_bf16=True, extra_allow=None):
    """Every finite reference element: |got - ref| <= bar + |bf16(ref) - ref|
    (the second term only for bf16 outputs) + extra_allow (the bound of a
    path's stated intermediate rounding, where it has one); relative L2 over
    the tensor as stated, without allowance.  Returns the metrics with the
    raw max-abs."""
    m = oracle.compare(got, ref)
    assert m["nonfinite"] == 0, (what, m)
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    err = np.abs(got[fin] - ref[fin])
    allow = bf16_rounding(ref[fin]) if out_bf16 else np.zeros_like(err)
    if extra_allow is not None:
        allow = allow + np.broadcast_to(extra_allow, ref.shape)[fin]
    bar = MAX_ABS_FP8 if fp8 else MAX_ABS
    m["max_abs_beyond_rounding"] = float(np.max(err - allow)) if err.size else 0.0
    m["elements"] = int(err.size)
    bad = int(np.count_nonzero(err > bar + allow))
    assert bad == 0, (what, f"{bad} elements beyond the bar", m)
    if not fp8:
        assert m["rel_l2"] <= REL_L2, (what, m)
    return m


def small(kind, **kw):
    base = dict(
        contig=W.Workload("contig", B=3, H=128, s_q=1, causal=False, T=200, T_stride=230),
        tiny=W.WORKLOADS["tiny"],
        tiny_unit=W.WORKLOADS["tiny"].with_(scaling="unit", seed=101),
        paged=W.Workload("paged", B=4, H=128, s_q=1, causal=False, T_range=(70, 400), paged=True, seed=33),
        verify=W.Workload("verify", B=2, H=128, s_q=4, causal=True, T=301, seed=44),
        verify_h=W.Workload("verify_h", B=2, H=40, s_q=3, causal=True, T=130, seed=45),
        # R = 132 query rows per sequence: a second row group of 4 rows (the
        # partial store writes only the rows that exist)
        groups_ragged=W.Workload("groups_ragged", B=3, H=66, s_q=2, causal=True, T=150, T_stride=160, seed=46),
        fp8=W.Workload("fp8", B=2, H=128, s_q=2, causal=True, T=333, cache_dtype="fp8", T_stride=350, seed=55),
        fp8_paged=W.Workload("fp8_paged", B=3, H=64, s_q=1, causal=False, T_range=(60, 300), paged=True,
                             cache_dtype="fp8", seed=56),
        # enough query rows for the merge + projection to run on 32-row blocks
        # (H x ceil(N / 32) >= 256 work-groups), the second block partial (N =
        # 40): three parts per sequence (the four-split path), seven (the
        # many-split path), and four query tokens per sequence
        wide=W.Workload("wide", B=40, H=128, s_q=1, causal=False, T=150, seed=57),
        wide_many=W.Workload("wide_many", B=40, H=128, s_q=1, causal=False, T=600, seed=58),
        wide_verify=W.Workload("wide_verify", B=10, H=128, s_q=4, causal=True, T=100, seed=59),
    )[kind]
    return base.with_(**kw) if kw else base


BF16_KINDS = ["contig", "tiny", "tiny_unit", "paged", "verify", "verify_h", "groups_ragged"]
ALL_KINDS = BF16_KINDS + ["fp8", "fp8_paged"]


def _run_steps(mla, inp, num_splits=0):
    q, w_uk, w_uv, cache = W.to_torch(inp)
    if cache.fp8 and not FP8_READY:
        pytest.skip("FP8 cache path not built yet")
    w = inp["workload"]
    B, s_q, H = w.B, w.s_q, w.H
    q_lat = mla.absorb_q(q.view(B * s_q, H, -1), w_uk).view(B, s_q, H, -1)
    o_lat, lse = mla.decode_attn(q_lat, cache, SCALE, w.causal, num_splits=num_splits)
    out = mla.absorb_out(o_lat.view(B * s_q, H, -1), w_uv).view(B, s_q, H, -1)
    torch.cuda.synchronize()
    return q_lat, o_lat, lse, out


@pytest.mark.parametrize("kind", ALL_KINDS)
def test_steps_and_pipeline_vs_oracle(mla, kind):
    w = small(kind)
    print(f"[parity] {kind} {w}", flush=True)
    inp = W.generate(w)
    q_lat, o_lat, lse, out = _run_steps(mla, inp)
    fp8 = w.cache_dtype == "fp8"
    B, s_q, H = w.B, w.s_q, w.H

    # step 1 against the oracle's absorb_q on the same bf16 inputs
    q64 = O.bf16_to_f64(inp["q"]).reshape(B * s_q, H, 192)
    ql_ref = O.absorb_q(q64, O.bf16_to_f64(inp["w_uk"])).reshape(B, s_q, H, 576)
    ql_got = _f64(q_lat)
    _assert_close(ql_got, ql_ref, what="absorb_q")
    # bf16 output rounding: every element within 2^-8 relative (+ accumulation slack)
    assert np.all(np.abs(ql_got - ql_ref) <= 2.0 ** -8 * np.abs(ql_ref) + 1e-3)
    np.testing.assert_array_equal(_bits(q_lat)[..., 512:], inp["q"][..., 128:])

    # steps 2-3 against single-latent attention fed with the GPU's own q_lat
    o_ref, lse_ref = O.latent_attention(inp, ql_got, SCALE)
    _assert_close(_f64(o_lat), o_ref, fp8=fp8, what="decode_attn o_lat", out_bf16=False)
    np.testing.assert_allclose(_f64(lse), lse_ref, rtol=0, atol=2e-3 if not fp8 else 5e-3)

    # step 4 against the oracle's absorb_out on the GPU's own o_lat
    out_ref4 = O.absorb_out(_f64(o_lat).reshape(B * s_q, H, 512), O.bf16_to_f64(inp["w_uv"]))
    _assert_close(_f64(out).reshape(B * s_q, H, 128), out_ref4, what="absorb_out")

    # whole path against the naive definition
    ref = O.naive_decode(inp, SCALE)
    m = _assert_close(_f64(out), ref, fp8=fp8, what="pipeline vs naive")
    print(f"[parity] {kind}: {m}", flush=True)


@pytest.mark.parametrize("kind", ["contig", "verify", "paged"])
def test_split_count_invariance_and_determinism(mla, kind):
    inp = W.generate(small(kind))
    results = {}
    for ns in (1, 2, 3, 0):
        _, o_lat, lse, out = _run_steps(mla, inp, num_splits=ns)
        results[ns] = (_f64(o_lat), _f64(out))
    # different split plans round the bf16 probabilities against different
    # softmax references: allow one bf16 unit of the value on top of 2e-3
    base = results[1][0]
    for ns, (o, _) in results.items():
        assert np.max(np.abs(o - base) - 2.0 ** -8 * np.abs(base)) < 2e-3, ns
    # fixed split plan: bitwise identical run to run
    _, o2, _, out2 = _run_steps(mla, inp, num_splits=0)
    np.testing.assert_array_equal(_f64(o2), results[0][0])
    np.testing.assert_array_equal(_f64(out2), results[0][1])


@pytest.mark.parametrize("kind", ["contig", "tiny", "verify", "verify_h", "groups_ragged", "paged", "fp8",
                                  "wide", "wide_many", "wide_verify"])
@pytest.mark.parametrize("o_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("part", [torch.float32, torch.bfloat16])
def test_combine_out_equals_separate_steps(mla, kind, o_dtype, part):
    """The fused merge + projection gives the bits of the merge followed by
    the projection, with and without writing o_lat and lse, for fp32 and
    bf16 split partials, on each of its paths: 8-row blocks (the small
    kinds), 32-row blocks with at most four parts per sequence (wide,
    wide_verify) and with more (wide_many)."""
    w = small(kind)
    inp = W.generate(w)
    q, w_uk, w_uv, cache = W.to_torch(inp)
    B, s_q, H = w.B, w.s_q, w.H
    q_lat = mla.absorb_q(q.view(B * s_q, H, -1), w_uk).view(B, s_q, H, -1)
    ws = mla.decode_partial(q_lat, cache, SCALE, w.causal, part_dtype=part)
    lse1 = torch.empty((B, s_q, H), dtype=torch.float32, device=q.device)
    o1, _ = mla.decode_combine(ws, B, s_q, H, cache.max_seqlen, o_dtype=o_dtype, lse=lse1, part_dtype=part)
    out1 = mla.absorb_out(o1.view(B * s_q, H, -1), w_uv)
    o2, lse2 = torch.full_like(o1, float("nan")), torch.full_like(lse1, float("nan"))
    out2 = mla.decode_combine_out(ws, w_uv, B, s_q, H, cache.max_seqlen, o_dtype=o_dtype, o_lat=o2, lse=lse2,
                                  part_dtype=part)
    out3 = mla.decode_combine_out(ws, w_uv, B, s_q, H, cache.max_seqlen, o_dtype=o_dtype, part_dtype=part)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(out2), _bits(out1))
    np.testing.assert_array_equal(_bits(out3), _bits(out1))
    np.testing.assert_array_equal(o2.view(torch.int16 if o_dtype == torch.bfloat16 else torch.int32).cpu().numpy(),
                                  o1.view(torch.int16 if o_dtype == torch.bfloat16 else torch.int32).cpu().numpy())
    np.testing.assert_array_equal(lse2.cpu().numpy(), lse1.cpu().numpy())
    ref = O.naive_decode(inp, SCALE)
    _assert_close(_f64(out2).reshape(ref.shape), ref, fp8=w.cache_dtype == "fp8", what=f"combine_out {kind}")


@pytest.mark.parametrize("fp8", [False, True])
def test_paged_equals_contiguous_bitwise(mla, fp8):
    w = small("fp8_paged" if fp8 else "paged")
    inp = W.generate(w)
    a = _run_steps(mla, inp)
    b = _run_steps(mla, W.as_contiguous(inp))
    for x, y in zip(a, b):
        np.testing.assert_array_equal(_f64(x), _f64(y))


def test_masked_rows_do_not_leak(mla):
    """Rows only later query tokens may see, and NaN pad rows, never reach
    earlier tokens' outputs."""
    w = small("verify")
    inp = W.generate(w)
    _, _, _, out_a = _run_steps(mla, inp)
    T = int(inp["seqlens"][0])
    inp["rows"][:, T - 3:T] = W.to_bf16_bits(np.full((w.B, 3, 576), 9.0, np.float32))
    _, _, _, out_b = _run_steps(mla, inp)
    a, b = _f64(out_a), _f64(out_b)
    np.testing.assert_array_equal(a[:, 0], b[:, 0])       # query 0 sees rows < T - 3
    assert not np.allclose(a[:, 3], b[:, 3])


def test_sequences_are_independent(mla):
    inp = W.generate(small("contig"))
    _, _, _, out_a = _run_steps(mla, inp)
    inp["rows"][1, :200] = inp["rows"][2, :200]
    _, _, _, out_b = _run_steps(mla, inp)
    np.testing.assert_array_equal(_f64(out_a)[[0, 2]], _f64(out_b)[[0, 2]])


@pytest.mark.parametrize("T,s_q", [(1, 1), (4, 4), (64, 1), (65, 2), (129, 3)])
def test_edge_lengths(mla, T, s_q):
    w = W.Workload("edge", B=2, H=128, s_q=s_q, causal=True, T=T, T_stride=T + 5, seed=T)
    inp = W.generate(w)
    *_, out = _run_steps(mla, inp)
    _assert_close(_f64(out), O.naive_decode(inp, SCALE), what=f"T={T}")


def test_large_score_range_rescale(mla):
    """Scores that jump by far more than the 2^64 reference step inside a
    split still give the exact softmax (the rescale path)."""
    w = W.Workload("jump", B=1, H=128, s_q=1, causal=False, T=300, seed=7)
    inp = W.generate(w)
    rows = O.bf16_to_f64(inp["rows"]).astype(np.float32)
    rows[0, 200:, 512:] *= 60.0     # rope keys of late rows: scores ~ 60x larger
    inp["rows"] = W.to_bf16_bits(rows)
    *_, out = _run_steps(mla, inp, num_splits=1)
    _assert_close(_f64(out), O.naive_decode(inp, SCALE), what="rescale")


# ----------------------------------------------------------------------------
# full-size workloads, whole output tensors
# ----------------------------------------------------------------------------
@functools.lru_cache(maxsize=1)
def full_inputs(name):
    """Seeded inputs of a full-size workload (the FP8 one takes a while to
    draw, so the last one is kept for the next test that needs it)."""
    return W.generate(W.WORKLOADS[name])


def run_timed_configuration(mla, inp):
    """The launch configuration the benchmark times: absorb_q, the split-T
    scan with bf16 partials, then the fused merge + W_UV projection (asked to
    also write the fp32 latent output and the log-sum-exps)."""
    w = inp["workload"]
    q, w_uk, w_uv, cache = W.to_torch(inp)
    B, s_q, H = w.B, w.s_q, w.H
    N = B * s_q
    q_lat = mla.absorb_q(q.view(N, H, -1), w_uk).view(B, s_q, H, -1)
    ws = mla.decode_partial(q_lat, cache, SCALE, w.causal, part_dtype=torch.bfloat16)
    o_lat = torch.empty((B, s_q, H, 512), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, s_q, H), dtype=torch.float32, device=q.device)
    out = mla.decode_combine_out(ws, w_uv, B, s_q, H, cache.max_seqlen, o_lat=o_lat, lse=lse,
                                 part_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    return q_lat, o_lat, lse, out.view(B, s_q, H, 128)


@pytest.mark.parametrize("name", ["tiny", "dsv3", "mtp_verify", "ragged_paged", "fp8_cache"])
def test_full_size(mla, name):
    """Every (sequence, query token, head) of the full-size workload: the
    latent queries against the oracle's absorption, the latent output and
    log-sum-exp against single-latent attention on the GPU's own latent
    queries, the projected output against the oracle's projection of the
    GPU's own latent output; and the whole path against the naive
    definition on sampled (sequence, head) pairs."""
    w = W.WORKLOADS[name]
    print(f"[parity-full] {name}", flush=True)
    inp = full_inputs(name)
    fp8 = w.cache_dtype == "fp8"
    B, s_q, H = w.B, w.s_q, w.H
    q_lat, o_lat, lse, out = run_timed_configuration(mla, inp)

    q64 = O.bf16_to_f64(inp["q"]).reshape(B * s_q, H, 192)
    ql_ref = O.absorb_q(q64, O.bf16_to_f64(inp["w_uk"])).reshape(B, s_q, H, 576)
    ql_got = _f64(q_lat)
    m = _assert_close(ql_got, ql_ref, what=f"{name} absorb_q")
    print(f"[parity-full] {name} q_lat: {m}", flush=True)

    o_ref, lse_ref = O.latent_attention(inp, ql_got, SCALE)
    m = _assert_close(_f64(o_lat), o_ref, fp8=fp8, what=f"{name} o_lat", out_bf16=False)
    print(f"[parity-full] {name} o_lat: {m}", flush=True)
    np.testing.assert_allclose(_f64(lse), lse_ref, rtol=0, atol=2e-3 if not fp8 else 5e-3)

    out_ref = O.absorb_out(_f64(o_lat).reshape(B * s_q, H, 512), O.bf16_to_f64(inp["w_uv"]))
    m = _assert_close(_f64(out).reshape(B * s_q, H, 128), out_ref, what=f"{name} out")
    print(f"[parity-full] {name} out: {m}", flush=True)

    rng = np.random.default_rng(123)
    pairs = [(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(4)]
    pairs += [(0, 0), (w.B - 1, w.H - 1)]
    ref = O.naive_decode(inp, SCALE, pairs=pairs)
    got = _f64(out)
    sel = np.zeros(got.shape, bool)
    for b, h in pairs:
        sel[b, :, h] = True
    m = _assert_close(got[sel], ref[sel], fp8=fp8, what=f"{name} vs naive")
    print(f"[parity-full] {name} end to end: {m}", flush=True)


# ----------------------------------------------------------------------------
# the balanced work plan over ragged lengths
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("case", ["many_short", "very_ragged", "very_ragged_paged"])
@pytest.mark.parametrize("ns", [0, 1, 3])
def test_ragged_work_plan(mla, case, ns):
    """Sequences of very different lengths share the equal tile ranges: each
    tile is scanned exactly once and each sequence's parts merge to the
    oracle, for more sequences than scan chunks and for forced split counts."""
    w = dict(
        many_short=W.Workload("many_short", B=300, H=16, s_q=1, causal=False, T_range=(1, 300), seed=71),
        very_ragged=W.Workload("very_ragged", B=7, H=128, s_q=2, causal=True, T_range=(2, 2000), seed=72),
        very_ragged_paged=W.Workload("very_ragged_paged", B=7, H=64, s_q=1, causal=False, T_range=(1, 2000),
                                     paged=True, seed=73),
    )[case]
    print(f"[parity] plan {case} ns={ns} lengths={W.generate(w)['seqlens'][:8]}", flush=True)
    inp = W.generate(w)
    *_, out = _run_steps(mla, inp, num_splits=ns)
    _assert_close(_f64(out), O.naive_decode(inp, SCALE), what=f"{case} ns={ns}")
