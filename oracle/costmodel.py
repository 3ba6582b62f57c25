"""Analytic FLOP and byte counts for decode attention -- TEST INFRASTRUCTURE.

Counting rules (same on every page): a multiply-add is 2 FLOPs, a contraction
costs 2 x (product of output dims) x (contracted dim) ("MLA, dim by dim",
"Tensor View"; "Why MLA and MTP Fight Each Other", section 2.1); softmax,
scaling and masking are not counted (section 1 there; "Notation and
Preliminaries" in "MLA, dim by dim").  Only the attention term that grows
with the cache length is counted unless a function says otherwise.

The tests pin every function here to a number the pages print.
"""
from __future__ import annotations


def gqa_decode_cached_token(n_q: int, n_kv: int, d_h: int, T: int, b: float):
    """Grouped-query decode attention over T cached tokens of one layer.

    Each KV head stores d_h key + d_h value elements per token; each of its
    n_q/n_kv query heads does a d_h dot product and a d_h multiply-add.
    ("Decode attention intensity...", "A strong answer".)  -> (bytes, flops, AI)
    """
    byts = 2 * T * d_h * b * n_kv
    flops = 4 * n_q * T * d_h
    return byts, flops, flops / byts


def mla_absorbed_cached_token(H: int, d_c: int, d_r: int, b: float, s_q: int = 1):
    """Absorbed MLA: per cached row every head scores over d_c + d_r and
    aggregates over d_c; the row is read once (b bytes per element).
    ("Decode attention intensity...", "A strong answer"; "Why MLA and MTP
    Fight Each Other", Appendix A.)  -> (bytes, flops, AI)
    """
    byts = (d_c + d_r) * b
    flops = s_q * H * (2 * (d_c + d_r) + 2 * d_c)
    return byts, flops, flops / byts


def mla_tp_intensity(H: int, d_c: int, d_r: int, b: float, tp: int) -> float:
    """Tensor parallelism over heads replicates the latent on every rank: the
    bytes stay, each rank keeps H/tp heads."""
    return mla_absorbed_cached_token(H // tp, d_c, d_r, b)[2]


def naive_expand_flops_per_cached_token(H: int, d_c: int, d_k: int, d_v: int) -> int:
    """Re-expanding one cached latent into per-head keys and values."""
    return 2 * d_c * H * (d_k + d_v)


def mla_fixed_flops(d_model: int, H: int, d_c: int, d_k: int, d_v: int) -> int:
    """Length-independent work of one decode step ("Why MLA and MTP Fight Each
    Other", section 4.1): latent down-projection, query projection, W_UK
    absorption into the query, W_UV projection of the latent output."""
    return 2 * d_model * d_c + 2 * d_model * H * d_k + 2 * H * d_k * d_c + 2 * H * d_c * d_v


def mla_per_length_flops(H: int, d_c: int) -> int:
    """Length-proportional work per cached token without rope: 4 H d_c."""
    return 4 * H * d_c


def decode_algorithms(H: int, d_c: int, d_k: int, d_v: int, L: int, S: int = 1, b: float = 2):
    """(MLA algorithm, MHA algorithm) FLOPs and bytes for S query tokens over L
    cached tokens ("Why MLA and MTP Fight Each Other", sections 5.3-5.5):

    absorb: per-query projection 2 H S d_c (d_k+d_v) + pairs 2 H S L (2 d_c);
    expand: per-cached-token projection 2 H L d_c (d_k+d_v) + pairs 2 H S L (d_k+d_v).
    Bytes: the absorbed form reads the latent once; the expanded form also
    moves the per-head keys and values.
    """
    f_mla = 2 * H * S * d_c * (d_k + d_v) + 2 * H * S * L * 2 * d_c
    f_mha = 2 * H * L * d_c * (d_k + d_v) + 2 * H * S * L * (d_k + d_v)
    by_mla = L * d_c * b
    by_mha = L * d_c * b + H * L * (d_k + d_v) * b
    return (f_mla, by_mla), (f_mha, by_mha)


def crossover_S(d_c: int, d_k: int, d_v: int, L: float) -> float:
    """S where the two algorithms cost the same FLOPs (H cancels)."""
    return L * d_c * (d_k + d_v) / (d_c * (d_k + d_v) + L * (2 * d_c - d_k - d_v))


def per_pair_macs(d_c: int, d_k: int, d_v: int, d_r: int = 0):
    """(absorbed, expanded) MACs per query/cached-token pair (Appendix A.3)."""
    return 2 * d_c + d_r, d_k + d_r + d_v


def sparse_mla_flops(H: int, d_c: int, d_k: int, d_v: int, k: int) -> int:
    """Absorbed MLA over k gathered rows, one query (section 6)."""
    return 2 * H * d_c * (d_k + d_v) + 4 * H * k * d_c


def cache_bytes(numbers_per_token: int, T: int, layers: int, b: float = 2) -> float:
    return numbers_per_token * T * layers * b


def ridge(peak_flops: float, bw_bytes: float) -> float:
    return peak_flops / bw_bytes
