"""fp64 CPU oracle for MLA decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never calls it, and it shares no code,
tables or constants with that path; the two meet only at the arrays drawn by
``head_latent_attention_mla_amd.workloads``.

What it computes -- the plain, slow definition, in float64:

* ``naive_decode``: the up-project-then-attend form.  Every cached latent is
  expanded per head into a key (latent part through W_UK, joined with the
  row's shared rope key) and a value (through W_UV); then ordinary softmax
  attention with the 192-wide query.  This is the form written out first in
  "The MLA decode speedup hiding in your model card" ("The naive form, written
  out"), with the decoupled rope channel added as in "MLA, dim by dim" ("Why
  RoPE Gets in the Way": score = absorbed content term + rope term) and in
  "Why MLA and MTP Fight Each Other" (Appendix A: the rope segment is shared
  by all heads and scores only, it has no value).
* ``absorb_q`` / ``latent_attention`` / ``absorb_out``: the three absorbed
  steps, each on its own, following "MLA, dim by dim" ("MLA Decode": decode
  score order (q W_UK^T) C^T, decode value order (p C) W_UV) and "Why MLA and
  MTP Fight Each Other" (sections 3.1 and 3.2).  They exist so each boundary
  call can be compared alone; chained they equal ``naive_decode`` by
  associativity.

Readings the pages leave open (each is a documented choice, not page text):

* cached row = [latent 0..511 | rope key 512..575]; query = [nope 0..127 |
  rope 128..191]; latent query = [q_abs 0..511 | q_rope 512..575];
* W_UK stored (head, d_nope, d_c), W_UV stored (head, d_c, d_v);
* scores are scaled by the caller's ``scale`` (1/sqrt(192): absorption keeps
  the pre-absorption scale, as both forms in the substack post divide by the
  square root of the head width);
* rope rotation is applied upstream: the cached rope key and the query's rope
  part arrive already rotated;
* causal (speculative verification with s_q query tokens): ``seqlens[b]``
  counts the s_q new rows, and query j sees rows 0 .. T - s_q + j;
* FP8 rows are OCP E4M3 codes times one fp32 scale per row.

Parity unpinned: nothing here is unpinned -- every function is checked by the
CPU tests against closed forms, a library reduction or brute force.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

D_NOPE = 128
D_ROPE = 64
D_C = 512
D_V = 128
ROW = D_C + D_ROPE


# ----------------------------------------------------------------------------
# storage decoders
# ----------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 ("e4m3fn") codes -> float64, from the format definition.

    sign = bit 7, exponent = bits 6..3 (bias 7), mantissa = bits 2..0.
    exponent 0: subnormal, (m/8) * 2^(1-7); otherwise (1 + m/8) * 2^(e-7).
    exponent 15 with mantissa 7 is NaN; there is no infinity.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.power(2.0, e - 7.0))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return s * mag


# ----------------------------------------------------------------------------
# cache access
# ----------------------------------------------------------------------------
def sequence_rows(inp: dict, b: int, upto: Optional[int] = None) -> np.ndarray:
    """Logical cached rows 0..T_b-1 of sequence b as float64 [T_b, 576].

    Paged caches are walked block by block through the block table; FP8 rows
    are decoded and multiplied by their per-row scale.
    """
    T = int(inp["seqlens"][b]) if upto is None else int(upto)
    rows, scale, table = inp["rows"], inp.get("row_scale"), inp.get("block_table")
    if table is None:
        raw = rows[b, :T]
        sc = None if scale is None else scale[b, :T]
    else:
        bs = int(inp["block_size"])
        raw_parts, sc_parts = [], []
        for i in range((T + bs - 1) // bs):
            phys = int(table[b, i])
            n = min(bs, T - i * bs)
            raw_parts.append(rows[phys, :n])
            if scale is not None:
                sc_parts.append(scale[phys, :n])
        raw = np.concatenate(raw_parts, axis=0) if raw_parts else rows[:0, 0]
        sc = None if scale is None else (np.concatenate(sc_parts) if sc_parts else np.zeros(0))
    if scale is None:
        return bf16_to_f64(raw)
    return e4m3_to_f64(raw) * np.asarray(sc, dtype=np.float64)[:, None]


def visible_rows(T: int, s_q: int, j: int, causal: bool) -> int:
    """Number of leading rows query j may attend to (rows 0 .. n-1)."""
    return T - s_q + j + 1 if causal else T


def _softmax_weights(scores: np.ndarray) -> Tuple[np.ndarray, float]:
    """Softmax of a 1-D score vector with the maximum subtracted; also its log-sum-exp."""
    m = np.max(scores)
    e = np.exp(scores - m)
    z = np.sum(e)
    return e / z, float(m + math.log(z))


# ----------------------------------------------------------------------------
# the naive (expand) form: the definition
# ----------------------------------------------------------------------------
def naive_decode(inp: dict, scale: float, causal: Optional[bool] = None,
                 pairs: Optional[Iterable[Tuple[int, int]]] = None) -> np.ndarray:
    """out[b, j, h, :] for MLA decode, by expanding every cached latent per head.

    For head h and cached row c_t:
        key_t   = [ W_UK[h] c_t[0:512]  |  c_t[512:576] ]          (192 wide)
        value_t =   c_t[0:512]^T W_UV[h]                           (128 wide)
        s_t     = scale * <q[b, j, h], key_t>
        out     = sum_t softmax(s)_t value_t   over the visible rows.
    ``pairs`` restricts the work to the listed (b, h); other entries stay NaN.
    """
    w = inp["workload"]
    causal = w.causal if causal is None else causal
    q = bf16_to_f64(inp["q"])
    w_uk = bf16_to_f64(inp["w_uk"])
    w_uv = bf16_to_f64(inp["w_uv"])
    B, s_q, H, _ = q.shape
    out = np.full((B, s_q, H, D_V), np.nan)
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(H)]
    by_b = {}
    for b, h in pairs:
        by_b.setdefault(b, []).append(h)
    for b, heads in by_b.items():
        T = int(inp["seqlens"][b])
        C = sequence_rows(inp, b)
        lat, rope = C[:, :D_C], C[:, D_C:]
        for h in heads:
            k_nope = lat @ w_uk[h].T            # [T, 128]: expand keys
            keys = np.concatenate([k_nope, rope], axis=1)  # [T, 192]
            vals = lat @ w_uv[h]                # [T, 128]: expand values
            for j in range(s_q):
                n = visible_rows(T, s_q, j, causal)
                s = (keys[:n] @ q[b, j, h]) * scale
                p, _ = _softmax_weights(s)
                out[b, j, h] = p @ vals[:n]
    return out


# ----------------------------------------------------------------------------
# sparse top-k decode: attention over a selected subset of the cached rows
# ----------------------------------------------------------------------------
def sparse_decode(inp: dict, sel_idx: np.ndarray, sel_count: np.ndarray, scale: float,
                  pairs: Optional[Iterable[Tuple[int, int]]] = None) -> np.ndarray:
    """out[b, j, h, :] attending only over the selected cached rows of sequence b.

    "Why MLA and MTP Fight Each Other", section 6: a selector keeps the top-k
    cached latents and attention runs over those alone, gathered by index
    (the cost goes from the context length to k).  Here the selection of
    sequence b is the positions sel_idx[b, :sel_count[b]] of its cache, shared
    by its s_q query tokens, and it is the whole visible set (no further
    mask).  The arithmetic is the expand form of ``naive_decode`` applied to
    the gathered rows, in the listed order (repeats count once each).
    """
    q = bf16_to_f64(inp["q"])
    w_uk = bf16_to_f64(inp["w_uk"])
    w_uv = bf16_to_f64(inp["w_uv"])
    B, s_q, H, _ = q.shape
    out = np.full((B, s_q, H, D_V), np.nan)
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(H)]
    by_b = {}
    for b, h in pairs:
        by_b.setdefault(b, []).append(h)
    for b, heads in by_b.items():
        n = int(sel_count[b])
        C = sequence_rows(inp, b)[np.asarray(sel_idx[b, :n], dtype=np.int64)]
        lat, rope = C[:, :D_C], C[:, D_C:]
        for h in heads:
            keys = np.concatenate([lat @ w_uk[h].T, rope], axis=1)
            vals = lat @ w_uv[h]
            for j in range(s_q):
                p, _ = _softmax_weights((keys @ q[b, j, h]) * scale)
                out[b, j, h] = p @ vals
    return out


# ----------------------------------------------------------------------------
# the three absorbed steps, each alone
# ----------------------------------------------------------------------------
def absorb_q(q: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """q [N, H, 192] f64, W_UK [H, 128, 512] f64 -> latent query [N, H, 576].

    q_abs[n, h, c] = sum_k q[n, h, k] W_UK[h, k, c] for the 128 no-rope dims;
    the 64 rope dims of q are carried over unchanged after it.
    """
    N, H, _ = q.shape
    out = np.empty((N, H, ROW))
    for h in range(H):
        out[:, h, :D_C] = q[:, h, :D_NOPE] @ w_uk[h]
        out[:, h, D_C:] = q[:, h, D_NOPE:]
    return out


def latent_attention(inp: dict, q_lat: np.ndarray, scale: float,
                     causal: Optional[bool] = None,
                     pairs: Optional[Iterable[Tuple[int, int]]] = None):
    """Single-latent attention: every head scores its 576-wide latent query
    against the same cached rows and averages the rows' 512 latent columns.

    q_lat [B, s_q, H, 576] f64.  Returns (o_lat [B, s_q, H, 512], lse [B, s_q, H])
    with lse the natural log-sum-exp of the scaled scores.
    """
    w = inp["workload"]
    causal = w.causal if causal is None else causal
    B, s_q, H, _ = q_lat.shape
    o = np.full((B, s_q, H, D_C), np.nan)
    lse = np.full((B, s_q, H), np.nan)
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(H)]
    by_b = {}
    for b, h in pairs:
        by_b.setdefault(b, []).append(h)
    for b, heads in by_b.items():
        T = int(inp["seqlens"][b])
        C = sequence_rows(inp, b)
        for j in range(s_q):
            n = visible_rows(T, s_q, j, causal)
            S = (q_lat[b, j, heads] @ C[:n].T) * scale     # [len(heads), n]
            P = np.empty_like(S)
            for i, h in enumerate(heads):
                P[i], lse[b, j, h] = _softmax_weights(S[i])
            # every head's weighted sum of the same latent rows: one product
            o[b, j, heads] = P @ C[:n, :D_C]
    return o, lse


def absorb_out(o_lat: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """o_lat [N, H, 512] f64, W_UV [H, 512, 128] -> out [N, H, 128] = o_lat[h] W_UV[h]."""
    N, H, _ = o_lat.shape
    out = np.empty((N, H, D_V))
    for h in range(H):
        out[:, h] = o_lat[:, h] @ w_uv[h]
    return out


def absorbed_decode(inp: dict, scale: float, causal: Optional[bool] = None) -> np.ndarray:
    """The three absorbed steps chained in fp64 (equal to ``naive_decode``)."""
    q = bf16_to_f64(inp["q"])
    B, s_q, H, _ = q.shape
    q_lat = absorb_q(q.reshape(B * s_q, H, -1), bf16_to_f64(inp["w_uk"])).reshape(B, s_q, H, ROW)
    o_lat, _ = latent_attention(inp, q_lat, scale, causal)
    out = absorb_out(o_lat.reshape(B * s_q, H, D_C), bf16_to_f64(inp["w_uv"]))
    return out.reshape(B, s_q, H, D_V)


# ----------------------------------------------------------------------------
# comparison metrics
# ----------------------------------------------------------------------------
def compare(got: np.ndarray, ref: np.ndarray) -> dict:
    """max-abs and relative-L2 error of ``got`` against ``ref`` (finite entries of ref)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mask = np.isfinite(ref)
    d = got[mask] - ref[mask]
    nrm = float(np.linalg.norm(ref[mask]))
    return dict(max_abs=float(np.max(np.abs(d))) if d.size else 0.0,
                rel_l2=float(np.linalg.norm(d) / nrm) if nrm > 0 else float(np.linalg.norm(d)),
                nonfinite=int(np.count_nonzero(~np.isfinite(got[mask]))))
