"""The seeded generator: shapes, structure and distributions of the inputs (CPU)."""
import math

import numpy as np

from oracle import mla_oracle as O
from head_latent_attention_mla_amd import workloads as W


def test_deterministic_per_seed():
    w = W.WORKLOADS["tiny"]
    a, b = W.generate(w), W.generate(w)
    for k in ("q", "w_uk", "w_uv", "rows"):
        np.testing.assert_array_equal(a[k], b[k])
    c = W.generate(w, seed=99)
    assert not np.array_equal(a["q"], c["q"])


def test_shapes_of_every_workload_scaled_down():
    for name, w in W.WORKLOADS.items():
        small = w.with_(B=2, H=8, s_q=min(w.s_q, 60), T=None if w.paged else 100,
                        T_range=(70, 200) if w.paged else None)
        inp = W.generate(small)
        assert inp["q"].shape == (2, small.s_q, 8, 192)
        assert inp["w_uk"].shape == (8, 128, 512) and inp["w_uv"].shape == (8, 512, 128)
        if w.paged:
            nblk = (inp["seqlens"] + 63) // 64
            used = np.concatenate([inp["block_table"][b, :n] for b, n in enumerate(nblk)])
            assert sorted(used.tolist()) == list(range(inp["rows"].shape[0]))   # a permutation of the pool
            assert np.all(inp["block_table"][0, nblk[0]:] == -1)
            assert np.all((70 <= inp["seqlens"]) & (inp["seqlens"] <= 200))
        else:
            assert inp["rows"].shape == (2, 100, 576)
        if w.cache_dtype == "fp8":
            assert inp["rows"].dtype == np.uint8 and inp["row_scale"] is not None
        else:
            assert inp["rows"].dtype == np.uint16


def test_pad_rows_are_nan():
    w = W.Workload("p", B=2, H=2, s_q=1, causal=False, T=10, T_stride=16)
    inp = W.generate(w)
    assert np.all(np.isnan(O.bf16_to_f64(inp["rows"][:, 10:])))
    assert np.all(np.isfinite(O.bf16_to_f64(inp["rows"][:, :10])))


def test_unit_scaling_gives_unit_score_variance():
    w = W.WORKLOADS["dsv3"].with_(B=4, T=512)
    inp = W.generate(w)
    q = O.bf16_to_f64(inp["q"]).reshape(4, 128, 192)
    ql = O.absorb_q(q, O.bf16_to_f64(inp["w_uk"]))
    s = []
    for b in range(4):
        s.append((ql[b] @ O.sequence_rows(inp, b).T).ravel() / math.sqrt(192))
    sd = np.std(np.concatenate(s))
    assert 0.9 < sd < 1.1


def test_literal_scaling_gives_nearly_flat_scores():
    inp = W.generate(W.WORKLOADS["tiny"])
    q = O.bf16_to_f64(inp["q"]).reshape(2, 16, 192)
    ql = O.absorb_q(q, O.bf16_to_f64(inp["w_uk"]))
    s = (ql[0] @ O.sequence_rows(inp, 0).T) / math.sqrt(192)
    assert np.std(s) < 0.01
