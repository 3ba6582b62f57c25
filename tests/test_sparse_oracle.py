"""Pins of the oracle's sparse top-k decode ("Why MLA and MTP Fight Each
Other", section 6: attention runs over the selected latents only) against the
dense naive form, which the other oracle tests pin."""
import copy
import math

import numpy as np
import pytest

from oracle import mla_oracle as O
from head_latent_attention_mla_amd import workloads as W

SCALE = 1.0 / math.sqrt(192.0)


def _inp(seed=11, B=3, H=4, T=40, s_q=1, paged=False, fp8=False):
    w = W.Workload("sp", B=B, H=H, s_q=s_q, causal=False, T=T, paged=paged,
                   cache_dtype="fp8" if fp8 else "bf16", seed=seed)
    return W.generate(w)


@pytest.mark.parametrize("paged,fp8", [(False, False), (True, False), (False, True)])
def test_selecting_everything_in_order_is_the_dense_form(paged, fp8):
    inp = _inp(paged=paged, fp8=fp8)
    B, T = 3, 40
    sel = np.tile(np.arange(T, dtype=np.int32), (B, 1))
    cnt = np.full(B, T, dtype=np.int32)
    np.testing.assert_array_equal(O.sparse_decode(inp, sel, cnt, SCALE), O.naive_decode(inp, SCALE, causal=False))


def test_selection_order_does_not_matter():
    inp = _inp()
    sel, cnt = W.generate_selection(inp, k=17)
    perm = sel.copy()
    rng = np.random.default_rng(0)
    for b in range(3):
        perm[b, : cnt[b]] = rng.permutation(perm[b, : cnt[b]])
    np.testing.assert_allclose(O.sparse_decode(inp, perm, cnt, SCALE), O.sparse_decode(inp, sel, cnt, SCALE),
                               rtol=1e-12, atol=1e-14)


def test_gather_equals_dense_form_on_the_compacted_cache():
    inp = _inp(s_q=2)
    sel, cnt = W.generate_selection(inp, k=13)
    comp = copy.copy(inp)
    comp["rows"] = np.stack([inp["rows"][b, sel[b, : cnt[b]]] for b in range(3)])
    comp["seqlens"] = cnt.copy()
    comp["T_stride"] = int(cnt.max())
    ref = O.naive_decode(comp, SCALE, causal=False)
    np.testing.assert_allclose(O.sparse_decode(inp, sel, cnt, SCALE), ref, rtol=1e-12, atol=1e-14)


def test_a_repeated_row_counts_twice():
    """Selecting row t twice equals a dense cache holding a second copy of it."""
    inp = _inp(B=1, T=20)
    sel = np.array([[0, 3, 7, 7, 12]], dtype=np.int32)
    cnt = np.array([5], dtype=np.int32)
    dup = copy.copy(inp)
    dup["rows"] = inp["rows"][:, [0, 3, 7, 7, 12]]
    dup["seqlens"] = np.array([5], dtype=np.int32)
    np.testing.assert_allclose(O.sparse_decode(inp, sel, cnt, SCALE), O.naive_decode(dup, SCALE, causal=False),
                               rtol=1e-12, atol=1e-14)


def test_single_selected_row_returns_its_value():
    inp = _inp(B=2, T=30)
    sel = np.array([[9], [29]], dtype=np.int32)
    cnt = np.array([1, 1], dtype=np.int32)
    out = O.sparse_decode(inp, sel, cnt, SCALE)
    w_uv = O.bf16_to_f64(inp["w_uv"])
    for b in range(2):
        lat = O.sequence_rows(inp, b)[sel[b, 0], :512]
        for h in range(4):
            np.testing.assert_allclose(out[b, 0, h], lat @ w_uv[h], rtol=1e-12, atol=1e-14)


def test_selection_generator():
    inp = _inp(B=4, T=50)
    sel, cnt = W.generate_selection(inp, k=60)
    assert list(cnt) == [50] * 4                      # capped by the length
    sel2, cnt2 = W.generate_selection(inp, k=10)
    assert list(cnt2) == [10] * 4
    for b in range(4):
        row = sel2[b, :10]
        assert np.all(np.diff(row) > 0) and row.min() >= 0 and row.max() < 50
    np.testing.assert_array_equal(sel2, W.generate_selection(inp, k=10)[0])   # deterministic
