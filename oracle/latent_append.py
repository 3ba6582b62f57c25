"""fp64 CPU oracle for the latent append step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; the HIP product path never does and
shares no code with it.

What it computes: the step that produces a cached row for each new token.
"Why MLA and MTP Fight Each Other" (section 3) and "MLA, dim by dim" ("MLA
Decode") compress the token's hidden state x (d_model wide) through W_DKV
into the 512-wide latent c = x W_DKV, which is appended to the latent cache;
Appendix A of the first page and "Why RoPE Gets in the Way" on the second add
a 64-wide rope key, shared by all heads, that carries the rotation R_i of the
token's position i and is stored beside the latent.

Readings the pages leave open (documented choices, not page text):

* the two projections are one weight ``w_dkr`` [576, d_model] in (out, in)
  order: rows 0..511 give the latent, rows 512..575 the rope key before its
  rotation (the row order of the cache, [latent | rope key]);
* no normalisation is applied to the latent (the pages write c = x W_DKV);
* R_i is the rotary embedding on consecutive pairs (2k, 2k + 1) of the rope
  key, turned by the angle i * base^(-2k / 64), k = 0..31 (the pages' own
  formulas for the rotation are not legible); ``base`` is an argument;
* storage: bf16 rounds each value to nearest even; FP8 stores OCP E4M3 codes
  with one fp32 scale per row, scale = amax / 448 rounded to fp32 (1 for an
  all-zero row), code = the E4M3 value nearest to value / scale, ties to the
  even mantissa, magnitudes past 448 clamped to 448.

Every function below is pinned by CPU tests against closed forms, rotation
invariants, a library conversion or brute force.
"""
from __future__ import annotations

import numpy as np

D_C = 512
D_ROPE = 64
ROW = D_C + D_ROPE
E4M3_MAX = 448.0


def rope_angles(pos: np.ndarray, base: float) -> np.ndarray:
    """[N] positions -> [N, 32] angles pos * base^(-2k/64) (float64)."""
    k = np.arange(D_ROPE // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * k / D_ROPE)
    return np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]


def rope_rotate(v: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Turn each pair (v[2k], v[2k+1]) of [N, 64] rows by its angle."""
    v = np.asarray(v, dtype=np.float64)
    ang = rope_angles(pos, base)
    c, s = np.cos(ang), np.sin(ang)
    a, b = v[:, 0::2], v[:, 1::2]
    out = np.empty_like(v)
    out[:, 0::2] = a * c - b * s
    out[:, 1::2] = a * s + b * c
    return out


def append_rows(x: np.ndarray, w_dkr: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """x [N, d] f64, w_dkr [576, d] f64 -> the new cached rows [N, 576] (f64).

    latent = x W_DKV (rows 0..511 of w_dkr); rope key = R_pos (x W_KR).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_dkr, dtype=np.float64)
    rows = x @ w.T
    rows[:, D_C:] = rope_rotate(rows[:, D_C:], pos, base)
    return rows


# ----------------------------------------------------------------------------
# storage roundings, each by nearest-value search over the format's values
# ----------------------------------------------------------------------------
def _e4m3_table():
    """Non-negative finite E4M3 values (codes 0x00..0x7E) from the definition."""
    codes = np.arange(0x7F, dtype=np.int64)
    e = codes >> 3
    m = (codes & 7).astype(np.float64)
    vals = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.power(2.0, e - 7.0))
    return codes, vals


def e4m3_nearest(v: np.ndarray) -> np.ndarray:
    """float64 -> E4M3 codes: nearest value, ties to the code with an even
    mantissa, magnitudes beyond 448 clamped to 448; the sign bit follows the
    sign of v (a negative value that rounds to zero keeps it)."""
    v = np.asarray(v, dtype=np.float64)
    codes, vals = _e4m3_table()
    a = np.minimum(np.abs(v), E4M3_MAX).ravel()
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    out = codes[idx].astype(np.uint8).reshape(v.shape)
    return out | (np.signbit(v).astype(np.uint8) << np.uint8(7))


def quantize_rows(rows: np.ndarray):
    """Rows [N, 576] f64 -> (codes uint8 [N, 576], scale fp32 [N])."""
    rows = np.asarray(rows, dtype=np.float64)
    amax = np.max(np.abs(rows), axis=1)
    scale = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)
    return e4m3_nearest(rows / scale.astype(np.float64)[:, None]), scale


def bf16_nearest(v: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, nearest value with ties to an even
    mantissa (finite inputs within the bf16 range)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, E = np.frexp(a)                                   # a = f * 2^E, f in [0.5, 1)
    e = np.maximum(E - 1, -126)                          # subnormals share the 2^-126 binade
    quantum = np.ldexp(1.0, e - 7)
    m = np.rint(a / quantum)                             # half to even
    val = m * quantum
    f32 = val.astype(np.float32)                         # exact: val has <= 8 significant bits
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return bits | (np.signbit(v).astype(np.uint16) << np.uint16(15))
