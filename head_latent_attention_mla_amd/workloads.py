"""Seeded synthetic inputs for absorbed MLA decode.

This module only *draws* inputs: Gaussian tensors, sequence lengths, a block
permutation for the paged cache, and the storage encodings of those draws
(bf16 bit patterns, OCP FP8-E4M3 codes with a per-row fp32 scale).  It holds
none of the attention arithmetic, so both the CPU oracle and the GPU path can
consume its arrays without sharing any of the method's code.

Shapes and names follow the pages' notation (MLA, dim by dim -- "Notation and
Preliminaries"; inferenceinterviews, "A strong answer"):

* ``q``        [B, s_q, H, 192]  bf16 bits, [nope 0..127 | rope 128..191]
* ``w_uk``     [H, 128, 512]     bf16 bits, (head, d_nope, d_c)
* ``w_uv``     [H, 512, 128]     bf16 bits, (head, d_c, d_v)
* ``rows``     contiguous [B, T_stride, 576] or paged pool [n_blocks, 64, 576];
               bf16 bits, or e4m3 codes with ``row_scale`` fp32 of matching
               leading shape.  A row is [latent 0..511 | rope key 512..575].
* ``seqlens``  int32 [B], rows per sequence (the s_q new rows included).
* ``block_table`` int32 [B, max_blocks] for the paged cache, else None.

Pad rows (beyond ``seqlens[b]``) are filled with NaN so that any read of a row
that must be masked shows up in the result.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

D_NOPE = 128
D_ROPE = 64
D_QK = D_NOPE + D_ROPE          # 192: per-head query/key width before absorption
D_C = 512                       # latent width
D_V = 128                       # per-head value width
ROW = D_C + D_ROPE              # 576: cached row = latent + decoupled rope key
BLOCK = 64                      # paged-cache block size (rows)

BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)
E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One decode workload: shapes, cache kind and input distribution."""
    name: str
    B: int
    H: int
    s_q: int
    causal: bool
    T: Optional[int] = None                    # fixed length for every sequence
    T_range: Optional[Tuple[int, int]] = None  # ragged: integer-uniform, inclusive
    paged: bool = False
    cache_dtype: str = "bf16"                  # "bf16" | "fp8"
    scaling: str = "unit"                      # "unit" | "literal"
    seed: int = 0
    T_stride: Optional[int] = None             # contiguous row stride (>= T); pad rows NaN
    topk: Optional[int] = None                 # sparse decode: rows selected per sequence

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def max_T(self) -> int:
        return self.T if self.T is not None else self.T_range[1]


# The five workloads.  Sizes follow the DeepSeek-V3 attention shape (H=128,
# 512-wide latent + 64-wide rope key, d_nope = d_v = 128).
WORKLOADS = {
    # Tiny: tensors drawn N(0,1) * width^-1/2 ("literal" scaling).
    "tiny": Workload("tiny", B=2, H=16, s_q=1, causal=False, T=256,
                     scaling="literal", seed=1),
    # DeepSeek-V3-shaped decode, contiguous bf16 latent cache [64, 4096, 576].
    "dsv3": Workload("dsv3", B=64, H=128, s_q=1, causal=False, T=4096, seed=2),
    # Ragged long-context decode over a paged cache of 64-row blocks.
    "ragged_paged": Workload("ragged_paged", B=16, H=128, s_q=1, causal=False,
                             T_range=(8192, 32768), paged=True, seed=3),
    # Speculative verification: 4 query tokens per sequence, causal among them.
    "mtp_verify": Workload("mtp_verify", B=32, H=128, s_q=4, causal=True, T=8192,
                           seed=4),
    # FP8-E4M3 latent cache with one fp32 scale per row, 2 query tokens.
    "fp8_cache": Workload("fp8_cache", B=64, H=128, s_q=2, causal=True, T=16384,
                          cache_dtype="fp8", seed=5),
    # Sparse top-k decode: 2048 of 16384 cached rows selected per sequence.
    "sparse_topk": Workload("sparse_topk", B=64, H=128, s_q=1, causal=False, T=16384,
                            topk=2048, seed=6),
    # prefill of two 4096-token prompts: every cached row is also a query row
    "prefill": Workload("prefill", B=2, H=128, s_q=4096, causal=True, T=4096, seed=8),
}


# ----------------------------------------------------------------------------
# storage encodings of the draws
# ----------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32/fp64 values -> bf16 bit patterns, round-to-nearest-even (via fp32)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    rounded = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Finite values -> OCP FP8 E4M3 ("e4m3fn") codes.

    Round to nearest, ties to even mantissa; magnitudes beyond 448 saturate to
    448 (the format has no infinity; S.1111.111 is NaN and is never produced
    here).  Exponent bias 7, three mantissa bits, subnormal quantum 2^-9.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, E = np.frexp(a)                       # a = f * 2^E, f in [0.5, 1)
    e = np.clip(E - 1, -6, 8)                # unbiased exponent, subnormals pinned at -6
    quantum = np.ldexp(1.0, e - 3)
    m = np.rint(a / quantum)                 # numpy rint rounds half to even
    carry = m >= 16                          # rounding overflowed into the next binade
    m = np.where(carry, 8, m)
    e = np.where(carry, e + 1, e)
    normal = m >= 8
    exp_field = np.where(normal, e + 7, 0).astype(np.uint8)
    man_field = np.where(normal, m - 8, m).astype(np.uint8)
    return sign | (exp_field << np.uint8(3)) | man_field


def quantize_rows_e4m3(rows: np.ndarray):
    """Per-row scale = amax/448 (1 for an all-zero row); codes = E4M3(row/scale)."""
    rows = np.asarray(rows, dtype=np.float64)
    amax = np.max(np.abs(rows), axis=-1)
    scale = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)
    codes = to_e4m3_codes(rows / scale.astype(np.float64)[..., None])
    return codes, scale


# ----------------------------------------------------------------------------
# generator
# ----------------------------------------------------------------------------
def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def _stds(w: Workload):
    """(q, latent row, W_UK, W_UV) standard deviations.

    Weights are always N(0,1) * (last-axis width)^-1/2.  "literal" scaling
    applies the same rule to q (width 192) and the cached rows (width 576);
    "unit" scaling draws q and rows N(0,1), which gives scaled scores of unit
    variance: (128 * 512/512 + 64) / 192 = 1.
    """
    w_uk, w_uv = D_C ** -0.5, D_V ** -0.5
    if w.scaling == "literal":
        return D_QK ** -0.5, ROW ** -0.5, w_uk, w_uv
    if w.scaling == "unit":
        return 1.0, 1.0, w_uk, w_uv
    raise ValueError(f"unknown scaling {w.scaling!r}")


def generate(w: Workload, seed: Optional[int] = None, fill_pad: bool = True) -> dict:
    """Draw every input of workload ``w`` from ``seed`` (default ``w.seed``).

    Draw order: W_UK, W_UV, q, then per-sequence lengths (ragged), then the
    cached rows sequence by sequence, then the physical block permutation
    (paged).  FP8 quantisation is deterministic and draws nothing.
    """
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    sd_q, sd_row, sd_uk, sd_uv = _stds(w)
    B, H, s_q = w.B, w.H, w.s_q

    w_uk = to_bf16_bits(_normal(rng, (H, D_NOPE, D_C), sd_uk))
    w_uv = to_bf16_bits(_normal(rng, (H, D_C, D_V), sd_uv))
    q = to_bf16_bits(_normal(rng, (B, s_q, H, D_QK), sd_q))

    if w.T is not None:
        seqlens = np.full(B, w.T, dtype=np.int32)
    else:
        lo, hi = w.T_range
        seqlens = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    if np.any(seqlens < s_q):
        raise ValueError("every sequence must hold at least s_q rows")

    fp8 = w.cache_dtype == "fp8"
    enc_dtype = np.uint8 if fp8 else np.uint16
    pad_val = E4M3_NAN if fp8 else BF16_NAN

    def encode(block_f32):
        if fp8:
            return quantize_rows_e4m3(block_f32)
        return to_bf16_bits(block_f32), None

    out = dict(workload=w, seed=seed, q=q, w_uk=w_uk, w_uv=w_uv, seqlens=seqlens,
               cache_dtype=w.cache_dtype, paged=w.paged)

    if not w.paged:
        T_stride = w.T_stride or int(seqlens.max())
        rows = np.empty((B, T_stride, ROW), dtype=enc_dtype)
        scale = np.ones((B, T_stride), dtype=np.float32) if fp8 else None
        for b in range(B):
            T = int(seqlens[b])
            codes, sc = encode(_normal(rng, (T, ROW), sd_row))
            rows[b, :T] = codes
            if fp8:
                scale[b, :T] = sc
            if T < T_stride:
                rows[b, T:] = pad_val if fill_pad else 0
                if fp8:
                    scale[b, T:] = np.nan if fill_pad else 1.0
        out.update(rows=rows, row_scale=scale, block_table=None,
                   block_size=BLOCK, T_stride=T_stride)
        return out

    # paged: logical rows of each sequence, scattered into a permuted block pool
    nblk = (seqlens + BLOCK - 1) // BLOCK
    n_blocks = int(nblk.sum())
    max_blocks = (w.max_T + BLOCK - 1) // BLOCK
    logical = []
    for b in range(B):
        logical.append(encode(_normal(rng, (int(seqlens[b]), ROW), sd_row)))
    perm = rng.permutation(n_blocks).astype(np.int32)
    block_table = np.full((B, max_blocks), -1, dtype=np.int32)
    pool = np.full((n_blocks, BLOCK, ROW), pad_val if fill_pad else 0, dtype=enc_dtype)
    pscale = np.full((n_blocks, BLOCK), np.nan if fill_pad else 1.0, dtype=np.float32) if fp8 else None
    k = 0
    for b in range(B):
        codes, sc = logical[b]
        for i in range(int(nblk[b])):
            phys = int(perm[k]); k += 1
            block_table[b, i] = phys
            t0, t1 = i * BLOCK, min((i + 1) * BLOCK, int(seqlens[b]))
            pool[phys, : t1 - t0] = codes[t0:t1]
            if fp8:
                pscale[phys, : t1 - t0] = sc[t0:t1]
    out.update(rows=pool, row_scale=pscale, block_table=block_table,
               block_size=BLOCK, max_blocks=max_blocks)
    return out


def generate_selection(inp: dict, k: Optional[int] = None, seed: Optional[int] = None):
    """A sparse selection for sparse decode: per sequence, min(k, T_b) distinct
    cached positions drawn uniformly without replacement, in increasing order.
    Returns (sel_idx int32 [B, k_max] padded with -1, sel_count int32 [B]).
    Drawn from ``seed`` (default: the workload seed + 1000), after and apart
    from the other inputs."""
    w = inp["workload"]
    k = w.topk if k is None else k
    rng = np.random.default_rng(w.seed + 1000 if seed is None else seed)
    seqlens = inp["seqlens"]
    B = len(seqlens)
    counts = np.minimum(k, seqlens).astype(np.int32)
    k_max = int(counts.max())
    sel = np.full((B, k_max), -1, dtype=np.int32)
    for b in range(B):
        sel[b, : counts[b]] = np.sort(rng.choice(int(seqlens[b]), size=int(counts[b]), replace=False))
    return sel, counts


def as_contiguous(inp: dict) -> dict:
    """Re-lay a paged input as a contiguous cache (same logical rows)."""
    if not inp["paged"]:
        return inp
    seqlens = inp["seqlens"]
    B = len(seqlens)
    T_stride = int(seqlens.max())
    rows = inp["rows"]
    fp8 = inp["row_scale"] is not None
    crow = np.zeros((B, T_stride, ROW), dtype=rows.dtype)
    cscale = np.ones((B, T_stride), dtype=np.float32) if fp8 else None
    bs = inp["block_size"]
    for b in range(B):
        T = int(seqlens[b])
        for i in range((T + bs - 1) // bs):
            phys = inp["block_table"][b, i]
            t0, t1 = i * bs, min((i + 1) * bs, T)
            crow[b, t0:t1] = rows[phys, : t1 - t0]
            if fp8:
                cscale[b, t0:t1] = inp["row_scale"][phys, : t1 - t0]
    out = dict(inp)
    out.update(rows=crow, row_scale=cscale, block_table=None, paged=False, T_stride=T_stride)
    out.pop("max_blocks", None)
    return out


def to_torch(inp: dict, device="cuda"):
    """Copy a generated input set to device tensors (bit-exact): returns
    (q, w_uk, w_uv, cache) with cache a ``mla.LatentCache``."""
    import torch
    from . import mla

    def bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)

    q, w_uk, w_uv = bf16(inp["q"]), bf16(inp["w_uk"]), bf16(inp["w_uv"])
    if inp["row_scale"] is not None:
        rows = torch.from_numpy(inp["rows"]).to(device)
        scale = torch.from_numpy(inp["row_scale"]).to(device)
    else:
        rows, scale = bf16(inp["rows"]), None
    table = None if inp["block_table"] is None else torch.from_numpy(inp["block_table"]).to(device)
    cache = mla.LatentCache(rows=rows, seqlens=torch.from_numpy(inp["seqlens"]).to(device),
                            max_seqlen=int(inp["seqlens"].max()), row_scale=scale, block_table=table)
    return q, w_uk, w_uv, cache


def bf16_tensor_to_numpy_bits(t) -> np.ndarray:
    """bf16 device tensor -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(dtype=__import__("torch").int16).cpu().numpy().view(np.uint16)


# ----------------------------------------------------------------------------
# latent append inputs
# ----------------------------------------------------------------------------
D_MODEL = 7168                  # DeepSeek-V3 hidden width


@dataclasses.dataclass(frozen=True)
class AppendWorkload:
    """One latent-append step: N new tokens of width d_model written into a
    cache of B sequences with T_cap row slots each."""
    name: str
    N: int
    d_model: int
    B: int
    T_cap: int
    paged: bool = True
    cache_dtype: str = "fp8"
    seed: int = 0


APPEND_WORKLOADS = {
    # one decode step of DeepSeek-V3 shape: 64 sequences append one token each
    # into a paged FP8 cache of 4096 slots per sequence
    "latent_append": AppendWorkload("latent_append", N=64, d_model=D_MODEL, B=64, T_cap=4096, seed=7),
}


def generate_append(w: AppendWorkload, seed: Optional[int] = None, distinct: bool = True) -> dict:
    """Draw x [N, d] ~ N(0, 1) and w_dkr [576, d] ~ N(0, 1/d) (bf16 bits), so
    every projected value is about N(0, 1); token n goes to sequence
    seq_id[n] (uniform) at a uniform position below T_cap, all (sequence,
    position) slots distinct when ``distinct``.  Draw order: w_dkr, x,
    seq_id, pos."""
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    w_dkr = to_bf16_bits(_normal(rng, (ROW, w.d_model), w.d_model ** -0.5))
    x = to_bf16_bits(_normal(rng, (w.N, w.d_model), 1.0))
    if distinct:
        if w.N > w.B * w.T_cap:
            raise ValueError("more tokens than slots")
        slots = rng.choice(w.B * w.T_cap, size=w.N, replace=False)
        seq_id = (slots // w.T_cap).astype(np.int32)
        pos = (slots % w.T_cap).astype(np.int32)
    else:
        seq_id = rng.integers(0, w.B, size=w.N).astype(np.int32)
        pos = rng.integers(0, w.T_cap, size=w.N).astype(np.int32)
    return dict(workload=w, seed=seed, x=x, w_dkr=w_dkr, seq_id=seq_id, pos=pos)
