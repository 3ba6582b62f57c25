"""ctypes binding of libmla (include/mla.h): argument marshalling only.

Every step of the path runs in the HIP kernels of ``libmla.so``; this module
checks tensor shapes, dtypes and devices, allocates outputs and workspaces with
PyTorch (device memory and streams are all PyTorch is used for) and passes raw
pointers and the current stream to the C ABI.  There is no CPU fallback: if the
library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

D_NOPE, D_ROPE, D_C, D_V = 128, 64, 512, 128
ROW = D_C + D_ROPE
BLOCK = 64
DEFAULT_SCALE = 1.0 / math.sqrt(D_NOPE + D_ROPE)

MLA_BF16, MLA_FP8_E4M3, MLA_FP32 = 0, 1, 2
_STATUS = {0: "MLA_OK", 1: "MLA_ERR_ARG", 2: "MLA_ERR_UNSUPPORTED", 3: "MLA_ERR_WORKSPACE", 4: "MLA_ERR_HIP"}


class MLAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_lib.mla_status_string(status).decode()}")


class KVDesc(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_void_p),
        ("row_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seqlens", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("T_stride", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32),
    ]


# name -> (restype, argtypes); mirrors include/mla.h
_VP, _I32, _SZ, _F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
SIGNATURES = {
    "mla_absorb_q": (_I32, [_VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _VP]),
    "mla_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "mla_decode_workspace_bytes_ex": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "mla_decode_num_splits": (_I32, [_I32, _I32, _I32, _I32, _I32]),
    "mla_decode_attn": (_I32, [_VP, ctypes.POINTER(KVDesc), _I32, _I32, _I32, _F32, _I32, _VP, _I32,
                               _VP, _VP, _SZ, _VP]),
    "mla_decode_attn_ex": (_I32, [_VP, ctypes.POINTER(KVDesc), _I32, _I32, _I32, _F32, _I32, _VP, _I32,
                                  _VP, _VP, _SZ, _I32, _VP]),
    "mla_decode_partial": (_I32, [_VP, ctypes.POINTER(KVDesc), _I32, _I32, _I32, _F32, _I32, _VP, _SZ, _I32,
                                  _I32, _VP]),
    "mla_decode_partial_fp8": (_I32, [_VP, ctypes.POINTER(KVDesc), _I32, _I32, _I32, _F32, _I32, _VP, _SZ,
                                      _I32, _I32, _VP]),
    "mla_decode_combine": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _VP, _SZ, _VP, _I32, _VP, _VP]),
    "mla_absorb_out": (_I32, [_VP, _I32, _VP, _VP, _I32, _I32, _I32, _I32, _VP]),
    "mla_decode_combine_out": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _VP, _SZ, _VP, _VP, _VP, _I32, _VP,
                                      _VP]),
    "mla_sparse_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "mla_sparse_decode_partial": (_I32, [_VP, ctypes.POINTER(KVDesc), _VP, _VP, _I32, _I32, _I32, _I32, _F32,
                                         _VP, _SZ, _I32, _I32, _VP]),
    "mla_sparse_decode_attn": (_I32, [_VP, ctypes.POINTER(KVDesc), _VP, _VP, _I32, _I32, _I32, _I32, _F32,
                                      _VP, _I32, _VP, _VP, _SZ, _I32, _VP]),
    "mla_naive_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "mla_naive_decode": (_I32, [_VP, ctypes.POINTER(KVDesc), _VP, _VP, _I32, _I32, _I32, _F32, _I32, _VP,
                                _VP, _SZ, _VP]),
    "mla_append_workspace_bytes": (_SZ, [_I32, _I32]),
    "mla_latent_append": (_I32, [_VP, _VP, _I32, _I32, _VP, _VP, _F32, ctypes.POINTER(KVDesc), _I32, _VP, _SZ,
                                 _VP]),
    "mla_prefill_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "mla_prefill_expand": (_I32, [_VP, ctypes.POINTER(KVDesc), _VP, _VP, _I32, _I32, _I32, _F32, _I32, _VP,
                                  _VP, _SZ, _VP]),
    "mla_attend_uses_expand": (_I32, [_I32, _I32]),
    "mla_attend_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "mla_attend": (_I32, [_VP, ctypes.POINTER(KVDesc), _VP, _VP, _I32, _I32, _I32, _F32, _I32, _VP, _VP, _SZ,
                          _VP]),
    "mla_validate_kv": (_I32, [ctypes.POINTER(KVDesc), _I32, _I32, ctypes.c_int64, _VP]),
    "mla_validate_kv_host": (_I32, [ctypes.POINTER(KVDesc), _VP, _VP, _I32, _I32, ctypes.c_int64]),
    "mla_decode_noalloc_max_bytes": (_SZ, []),
    "mla_decode_attn_noalloc": (_I32, [_VP, ctypes.POINTER(KVDesc), _I32, _I32, _I32, _F32, _I32, _VP, _I32,
                                       _VP, _VP]),
    "mla_status_string": (ctypes.c_char_p, [_I32]),
}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"libmla.so not built at {path}; run `python -m head_latent_attention_mla_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = load_library()


def _check(status: int, what: str):
    if status != 0:
        raise MLAError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _empty(shape, dtype, device, stream=None) -> torch.Tensor:
    """torch.empty on ``stream`` (the current stream when None): the caching
    allocator then hands the memory to other work only once ``stream`` has
    passed the kernels that use it."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


# MLA_VALIDATE=1: check the device-resident preconditions of every cache
# before the calls that read it (mla_validate_kv; synchronises, for debugging)
VALIDATE = os.environ.get("MLA_VALIDATE", "0") not in ("", "0")


def _maybe_validate(cache: "LatentCache", s_q: int, stream=None):
    if VALIDATE:
        cache.validate(s_q, stream)


def _require(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


@dataclasses.dataclass
class LatentCache:
    """Device latent cache: contiguous [B, T_stride, 576] or a paged pool
    [n_blocks, 64, 576] with an int32 block table [B, max_blocks]; bf16 rows,
    or uint8 E4M3 codes with an fp32 per-row scale."""
    rows: torch.Tensor
    seqlens: torch.Tensor
    max_seqlen: int
    row_scale: Optional[torch.Tensor] = None
    block_table: Optional[torch.Tensor] = None

    @property
    def fp8(self) -> bool:
        return self.row_scale is not None

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    @property
    def B(self) -> int:
        return int(self.seqlens.shape[0])

    def desc(self) -> KVDesc:
        _require(self.seqlens, "seqlens", torch.int32)
        if self.fp8:
            _require(self.rows, "rows", torch.uint8)
            _require(self.row_scale, "row_scale", torch.float32, self.rows.shape[:2])
        else:
            _require(self.rows, "rows", torch.bfloat16)
        if self.rows.dim() != 3 or self.rows.shape[2] != ROW:
            raise ValueError(f"rows must be [*, *, {ROW}]")
        d = KVDesc()
        d.rows = self.rows.data_ptr()
        d.row_scale = self.row_scale.data_ptr() if self.fp8 else None
        d.seqlens = self.seqlens.data_ptr()
        d.dtype = MLA_FP8_E4M3 if self.fp8 else MLA_BF16
        d.max_seqlen = int(self.max_seqlen)
        if self.paged:
            _require(self.block_table, "block_table", torch.int32)
            if self.block_table.shape[0] != self.B:
                raise ValueError("block_table must have one row per sequence")
            if self.rows.shape[1] != BLOCK:
                raise ValueError(f"paged pool must be [n_blocks, {BLOCK}, {ROW}]")
            d.block_table = self.block_table.data_ptr()
            d.block_size = BLOCK
            d.max_blocks = int(self.block_table.shape[1])
            d.T_stride = 0
        else:
            if self.rows.shape[0] != self.B:
                raise ValueError("contiguous rows must be [B, T_stride, 576]")
            d.block_table = None
            d.T_stride = int(self.rows.shape[1])
            d.block_size = 0
            d.max_blocks = 0
        return d

    def validate(self, s_q: int = 1, stream=None) -> None:
        """Check the device-resident preconditions (lengths within bounds,
        block ids inside the pool) with mla_validate_kv; raises MLAError."""
        kv = self.desc()
        n_pool = int(self.rows.shape[0]) if self.paged else 0
        _check(_lib.mla_validate_kv(ctypes.byref(kv), self.B, int(s_q), n_pool, _stream(stream)),
               "mla_validate_kv")


def absorb_q(q: torch.Tensor, w_uk: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q [N, H, 192] bf16, W_UK [H, 128, 512] bf16 -> latent query [N, H, 576] bf16."""
    N, H = q.shape[0], q.shape[1]
    _require(q, "q", torch.bfloat16, (N, H, D_NOPE + D_ROPE))
    _require(w_uk, "w_uk", torch.bfloat16, (H, D_NOPE, D_C))
    if out is None:
        out = _empty((N, H, ROW), torch.bfloat16, q.device, stream)
    _require(out, "q_lat", torch.bfloat16, (N, H, ROW))
    _check(_lib.mla_absorb_q(_ptr(q), _ptr(w_uk), _ptr(out), N, H, D_NOPE, D_ROPE, D_C, _stream(stream)),
           "mla_absorb_q")
    return out


def decode_workspace_bytes(B: int, s_q: int, H: int, max_seqlen: int, num_splits: int = 0) -> int:
    if num_splits == 0:
        return int(_lib.mla_decode_workspace_bytes(B, s_q, H, max_seqlen))
    return int(_lib.mla_decode_workspace_bytes_ex(B, s_q, H, max_seqlen, num_splits))


def decode_num_splits(B: int, s_q: int, H: int, max_seqlen: int, num_splits: int = 0) -> int:
    return int(_lib.mla_decode_num_splits(B, s_q, H, max_seqlen, num_splits))


def decode_attn(q_lat: torch.Tensor, cache: LatentCache, scale: float = DEFAULT_SCALE, causal: bool = False,
                o_dtype=torch.float32, num_splits: int = 0, o_lat: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                workspace: Optional[torch.Tensor] = None, stream=None):
    """Latent attention: q_lat [B, s_q, H, 576] bf16 against the shared cache.
    Returns (o_lat [B, s_q, H, 512] in o_dtype, lse [B, s_q, H] fp32 or None)."""
    B, s_q, H = q_lat.shape[0], q_lat.shape[1], q_lat.shape[2]
    _require(q_lat, "q_lat", torch.bfloat16, (B, s_q, H, ROW))
    if cache.B != B:
        raise ValueError("cache holds a different number of sequences")
    kv = cache.desc()
    dt = {torch.float32: MLA_FP32, torch.bfloat16: MLA_BF16}[o_dtype]
    if o_lat is None:
        o_lat = _empty((B, s_q, H, D_C), o_dtype, q_lat.device, stream)
    _require(o_lat, "o_lat", o_dtype, (B, s_q, H, D_C))
    if lse is None and want_lse:
        lse = _empty((B, s_q, H), torch.float32, q_lat.device, stream)
    if lse is not None:
        _require(lse, "lse", torch.float32, (B, s_q, H))
    need = decode_workspace_bytes(B, s_q, H, cache.max_seqlen, num_splits)
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, q_lat.device, stream)
    _maybe_validate(cache, s_q, stream)
    if num_splits == 0:
        _check(_lib.mla_decode_attn(_ptr(q_lat), ctypes.byref(kv), B, s_q, H, float(scale), int(bool(causal)),
                                    _ptr(o_lat), dt, _ptr(lse), _ptr(workspace), workspace.numel(),
                                    _stream(stream)), "mla_decode_attn")
    else:
        _check(_lib.mla_decode_attn_ex(_ptr(q_lat), ctypes.byref(kv), B, s_q, H, float(scale), int(bool(causal)),
                                       _ptr(o_lat), dt, _ptr(lse), _ptr(workspace), workspace.numel(), num_splits,
                                       _stream(stream)), "mla_decode_attn_ex")
    return o_lat, lse


def decode_attn_noalloc(q_lat: torch.Tensor, cache: LatentCache, scale: float = DEFAULT_SCALE,
                        causal: bool = False, o_lat: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, stream=None):
    """decode_attn with the split workspace inside the library (no
    allocation by the library; the outputs must be given).  Calls that
    overlap on one GPU race on that workspace."""
    B, s_q, H = q_lat.shape[0], q_lat.shape[1], q_lat.shape[2]
    _require(q_lat, "q_lat", torch.bfloat16, (B, s_q, H, ROW))
    if o_lat is None:
        raise ValueError("decode_attn_noalloc needs its output tensor")
    dt = {torch.float32: MLA_FP32, torch.bfloat16: MLA_BF16}[o_lat.dtype]
    _require(o_lat, "o_lat", o_lat.dtype, (B, s_q, H, D_C))
    if lse is not None:
        _require(lse, "lse", torch.float32, (B, s_q, H))
    kv = cache.desc()
    _maybe_validate(cache, s_q, stream)
    _check(_lib.mla_decode_attn_noalloc(_ptr(q_lat), ctypes.byref(kv), B, s_q, H, float(scale),
                                        int(bool(causal)), _ptr(o_lat), dt, _ptr(lse), _stream(stream)),
           "mla_decode_attn_noalloc")
    return o_lat, lse


def _part_code(part_dtype) -> int:
    """Element type of the split partials: torch.float32 or torch.bfloat16."""
    return {torch.float32: MLA_FP32, torch.bfloat16: MLA_BF16}[part_dtype]


def decode_partial(q_lat: torch.Tensor, cache: LatentCache, scale: float = DEFAULT_SCALE, causal: bool = False,
                   num_splits: int = 0, workspace: Optional[torch.Tensor] = None, stream=None,
                   fp8_math: bool = False, part_dtype=torch.float32) -> torch.Tensor:
    """Phase 1 of decode_attn: the split-T scan into a workspace (returned).
    fp8_math (FP8 caches only): E4M3 matrix arithmetic (mla_decode_partial_fp8).
    part_dtype: element type of the partials (pass the same to the merge)."""
    B, s_q, H = q_lat.shape[0], q_lat.shape[1], q_lat.shape[2]
    _require(q_lat, "q_lat", torch.bfloat16, (B, s_q, H, ROW))
    kv = cache.desc()
    need = decode_workspace_bytes(B, s_q, H, cache.max_seqlen, num_splits)
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, q_lat.device, stream)
    _maybe_validate(cache, s_q, stream)
    fn, name = ((_lib.mla_decode_partial_fp8, "mla_decode_partial_fp8") if fp8_math
                else (_lib.mla_decode_partial, "mla_decode_partial"))
    _check(fn(_ptr(q_lat), ctypes.byref(kv), B, s_q, H, float(scale), int(bool(causal)),
              _ptr(workspace), workspace.numel(), num_splits, _part_code(part_dtype), _stream(stream)), name)
    return workspace


def decode_combine(workspace: torch.Tensor, B: int, s_q: int, H: int, max_seqlen: int, num_splits: int = 0,
                   o_dtype=torch.float32, o_lat: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, stream=None, part_dtype=torch.float32):
    """Phase 2 of decode_attn: merge the split partials held in ``workspace``."""
    dt = {torch.float32: MLA_FP32, torch.bfloat16: MLA_BF16}[o_dtype]
    if o_lat is None:
        o_lat = _empty((B, s_q, H, D_C), o_dtype, workspace.device, stream)
    _require(o_lat, "o_lat", o_dtype, (B, s_q, H, D_C))
    if lse is not None:
        _require(lse, "lse", torch.float32, (B, s_q, H))
    _check(_lib.mla_decode_combine(B, s_q, H, max_seqlen, num_splits, _part_code(part_dtype), _ptr(workspace),
                                   workspace.numel(),
                                   _ptr(o_lat), dt, _ptr(lse), _stream(stream)), "mla_decode_combine")
    return o_lat, lse


def decode_combine_out(workspace: torch.Tensor, w_uv: torch.Tensor, B: int, s_q: int, H: int, max_seqlen: int,
                       num_splits: int = 0, o_dtype=torch.float32, out: Optional[torch.Tensor] = None,
                       o_lat: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None,
                       part_dtype=torch.float32):
    """Phases 2 + 4 fused: merge the split partials and project through W_UV.
    Returns out [B * s_q, H, 128] bf16; o_lat and lse are written when given."""
    dt = {torch.float32: MLA_FP32, torch.bfloat16: MLA_BF16}[o_dtype]
    _require(w_uv, "w_uv", torch.bfloat16, (H, D_C, D_V))
    if out is None:
        out = _empty((B * s_q, H, D_V), torch.bfloat16, workspace.device, stream)
    _require(out, "out", torch.bfloat16, (B * s_q, H, D_V))
    if o_lat is not None:
        _require(o_lat, "o_lat", o_dtype, (B, s_q, H, D_C))
    if lse is not None:
        _require(lse, "lse", torch.float32, (B, s_q, H))
    _check(_lib.mla_decode_combine_out(B, s_q, H, max_seqlen, num_splits, _part_code(part_dtype), _ptr(workspace),
                                       workspace.numel(),
                                       _ptr(w_uv), _ptr(out), _ptr(o_lat), dt, _ptr(lse), _stream(stream)),
           "mla_decode_combine_out")
    return out


def absorb_out(o_lat: torch.Tensor, w_uv: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """o_lat [N, H, 512] (fp32 or bf16), W_UV [H, 512, 128] bf16 -> out [N, H, 128] bf16."""
    N, H = o_lat.shape[0], o_lat.shape[1]
    dt = {torch.float32: MLA_FP32, torch.bfloat16: MLA_BF16}[o_lat.dtype]
    _require(o_lat, "o_lat", o_lat.dtype, (N, H, D_C))
    _require(w_uv, "w_uv", torch.bfloat16, (H, D_C, D_V))
    if out is None:
        out = _empty((N, H, D_V), torch.bfloat16, o_lat.device, stream)
    _require(out, "out", torch.bfloat16, (N, H, D_V))
    _check(_lib.mla_absorb_out(_ptr(o_lat), dt, _ptr(w_uv), _ptr(out), N, H, D_C, D_V, _stream(stream)),
           "mla_absorb_out")
    return out


def decode(q: torch.Tensor, cache: LatentCache, w_uk: torch.Tensor, w_uv: torch.Tensor,
           scale: float = DEFAULT_SCALE, causal: bool = False, o_dtype=torch.float32,
           num_splits: int = 0, fused: bool = True, stream=None, fp8_math: bool = False,
           part_dtype=torch.bfloat16) -> torch.Tensor:
    """Absorbed MLA decode: q [B, s_q, H, 192] -> out [B, s_q, H, 128] bf16.
    fused: merge and project in one pass (mla_decode_combine_out) with split
    partials of part_dtype; otherwise mla_decode_attn (partials in o_dtype)
    then mla_absorb_out.  Both give the same bits when part_dtype == o_dtype."""
    B, s_q, H = q.shape[0], q.shape[1], q.shape[2]
    q_lat = absorb_q(q.view(B * s_q, H, -1), w_uk, stream=stream).view(B, s_q, H, ROW)
    if fused or fp8_math:
        ws = decode_partial(q_lat, cache, scale, causal, num_splits, stream=stream, fp8_math=fp8_math,
                            part_dtype=part_dtype)
        out = decode_combine_out(ws, w_uv, B, s_q, H, cache.max_seqlen, num_splits, o_dtype, stream=stream,
                                 part_dtype=part_dtype)
        return out.view(B, s_q, H, D_V)
    o_lat, _ = decode_attn(q_lat, cache, scale, causal, o_dtype, num_splits, want_lse=False, stream=stream)
    return absorb_out(o_lat.view(B * s_q, H, D_C), w_uv, stream=stream).view(B, s_q, H, D_V)


def sparse_workspace_bytes(B: int, s_q: int, H: int, k_max: int, num_splits: int = 0, fp8: bool = False) -> int:
    return int(_lib.mla_sparse_workspace_bytes(B, s_q, H, k_max, num_splits, MLA_FP8_E4M3 if fp8 else MLA_BF16))


def _sparse_args(q_lat, cache, sel_idx, sel_count):
    B, s_q, H = q_lat.shape[0], q_lat.shape[1], q_lat.shape[2]
    _require(q_lat, "q_lat", torch.bfloat16, (B, s_q, H, ROW))
    if sel_idx.dim() != 2 or sel_idx.shape[0] != B:
        raise ValueError("sel_idx must be [B, k_max]")
    _require(sel_idx, "sel_idx", torch.int32, tuple(sel_idx.shape))
    _require(sel_count, "sel_count", torch.int32, (B,))
    return B, s_q, H, int(sel_idx.shape[1])


def sparse_decode_partial(q_lat: torch.Tensor, cache: LatentCache, sel_idx: torch.Tensor, sel_count: torch.Tensor,
                          scale: float = DEFAULT_SCALE, num_splits: int = 0,
                          workspace: Optional[torch.Tensor] = None, stream=None,
                          part_dtype=torch.float32) -> torch.Tensor:
    """Sparse top-k scan into a workspace (returned): attention over the rows
    sel_idx[b, :sel_count[b]] of each sequence.  Merge with decode_combine /
    decode_combine_out using k_max = sel_idx.shape[1] as max_seqlen."""
    B, s_q, H, k_max = _sparse_args(q_lat, cache, sel_idx, sel_count)
    kv = cache.desc()
    need = sparse_workspace_bytes(B, s_q, H, k_max, num_splits, cache.fp8)
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, q_lat.device, stream)
    _check(_lib.mla_sparse_decode_partial(_ptr(q_lat), ctypes.byref(kv), _ptr(sel_idx), _ptr(sel_count), k_max,
                                          B, s_q, H, float(scale), _ptr(workspace), workspace.numel(), num_splits,
                                          _part_code(part_dtype), _stream(stream)), "mla_sparse_decode_partial")
    return workspace


def sparse_decode_attn(q_lat: torch.Tensor, cache: LatentCache, sel_idx: torch.Tensor, sel_count: torch.Tensor,
                       scale: float = DEFAULT_SCALE, o_dtype=torch.float32, num_splits: int = 0,
                       want_lse: bool = True, workspace: Optional[torch.Tensor] = None, stream=None):
    """Sparse top-k latent attention: returns (o_lat [B, s_q, H, 512], lse [B, s_q, H] or None)."""
    B, s_q, H, k_max = _sparse_args(q_lat, cache, sel_idx, sel_count)
    kv = cache.desc()
    dt = {torch.float32: MLA_FP32, torch.bfloat16: MLA_BF16}[o_dtype]
    o_lat = _empty((B, s_q, H, D_C), o_dtype, q_lat.device, stream)
    lse = _empty((B, s_q, H), torch.float32, q_lat.device, stream) if want_lse else None
    need = sparse_workspace_bytes(B, s_q, H, k_max, num_splits, cache.fp8)
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, q_lat.device, stream)
    _check(_lib.mla_sparse_decode_attn(_ptr(q_lat), ctypes.byref(kv), _ptr(sel_idx), _ptr(sel_count), k_max,
                                       B, s_q, H, float(scale), _ptr(o_lat), dt, _ptr(lse), _ptr(workspace),
                                       workspace.numel(), num_splits, _stream(stream)), "mla_sparse_decode_attn")
    return o_lat, lse


def sparse_decode(q: torch.Tensor, cache: LatentCache, sel_idx: torch.Tensor, sel_count: torch.Tensor,
                  w_uk: torch.Tensor, w_uv: torch.Tensor, scale: float = DEFAULT_SCALE, num_splits: int = 0,
                  stream=None, part_dtype=torch.bfloat16) -> torch.Tensor:
    """Sparse absorbed decode: q [B, s_q, H, 192] -> out [B, s_q, H, 128] bf16."""
    B, s_q, H = q.shape[0], q.shape[1], q.shape[2]
    q_lat = absorb_q(q.view(B * s_q, H, -1), w_uk, stream=stream).view(B, s_q, H, ROW)
    ws = sparse_decode_partial(q_lat, cache, sel_idx, sel_count, scale, num_splits, stream=stream,
                               part_dtype=part_dtype)
    out = decode_combine_out(ws, w_uv, B, s_q, H, int(sel_idx.shape[1]), num_splits, stream=stream,
                             part_dtype=part_dtype)
    return out.view(B, s_q, H, D_V)


def naive_workspace_bytes(B: int, s_q: int, H: int, max_seqlen: int) -> int:
    return int(_lib.mla_naive_workspace_bytes(B, s_q, H, max_seqlen))


def naive_decode(q: torch.Tensor, cache: LatentCache, w_uk: torch.Tensor, w_uv: torch.Tensor,
                 scale: float = DEFAULT_SCALE, causal: bool = False, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Ablation: expand every cached row per head, then attend. Same I/O as decode()."""
    B, s_q, H = q.shape[0], q.shape[1], q.shape[2]
    _require(q, "q", torch.bfloat16, (B, s_q, H, D_NOPE + D_ROPE))
    _require(w_uk, "w_uk", torch.bfloat16, (H, D_NOPE, D_C))
    _require(w_uv, "w_uv", torch.bfloat16, (H, D_C, D_V))
    kv = cache.desc()
    if out is None:
        out = _empty((B, s_q, H, D_V), torch.bfloat16, q.device, stream)
    need = naive_workspace_bytes(B, s_q, H, cache.max_seqlen)
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, q.device, stream)
    _maybe_validate(cache, s_q, stream)
    _check(_lib.mla_naive_decode(_ptr(q), ctypes.byref(kv), _ptr(w_uk), _ptr(w_uv), B, s_q, H, float(scale),
                                 int(bool(causal)), _ptr(out), _ptr(workspace), workspace.numel(),
                                 _stream(stream)), "mla_naive_decode")
    return out


def append_workspace_bytes(N: int, d_model: int) -> int:
    return int(_lib.mla_append_workspace_bytes(N, d_model))


def latent_append(x: torch.Tensor, w_dkr: torch.Tensor, seq_id: torch.Tensor, pos: torch.Tensor,
                  cache: LatentCache, rope_base: float = 10000.0, workspace: Optional[torch.Tensor] = None,
                  stream=None) -> None:
    """Write the cached rows of N new tokens: x [N, d] bf16 hidden states,
    w_dkr [576, d] bf16 (W_DKV^T over W_KR^T); token n goes to position
    pos[n] of sequence seq_id[n] of ``cache`` (its rows and scales are
    written in place; its seqlens are not touched)."""
    N, d = int(x.shape[0]), int(x.shape[1])
    _require(x, "x", torch.bfloat16, (N, d))
    _require(w_dkr, "w_dkr", torch.bfloat16, (ROW, d))
    _require(seq_id, "seq_id", torch.int32, (N,))
    _require(pos, "pos", torch.int32, (N,))
    kv = cache.desc()
    need = append_workspace_bytes(N, d)
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, x.device, stream)
    _check(_lib.mla_latent_append(_ptr(x), _ptr(w_dkr), N, d, _ptr(seq_id), _ptr(pos), float(rope_base),
                                  ctypes.byref(kv), cache.B, _ptr(workspace), workspace.numel(),
                                  _stream(stream)), "mla_latent_append")


def prefill_workspace_bytes(B: int, s_q: int, H: int, max_seqlen: int) -> int:
    return int(_lib.mla_prefill_workspace_bytes(B, s_q, H, max_seqlen))


def _attend_args(q, cache, w_uk, w_uv, out, stream=None):
    B, s_q, H = q.shape[0], q.shape[1], q.shape[2]
    _require(q, "q", torch.bfloat16, (B, s_q, H, D_NOPE + D_ROPE))
    _require(w_uk, "w_uk", torch.bfloat16, (H, D_NOPE, D_C))
    _require(w_uv, "w_uv", torch.bfloat16, (H, D_C, D_V))
    kv = cache.desc()
    if out is None:
        out = _empty((B, s_q, H, D_V), torch.bfloat16, q.device, stream)
    _require(out, "out", torch.bfloat16, (B, s_q, H, D_V))
    return B, s_q, H, kv, out


def prefill_expand(q: torch.Tensor, cache: LatentCache, w_uk: torch.Tensor, w_uv: torch.Tensor,
                   scale: float = DEFAULT_SCALE, causal: bool = True, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Expand path: every cached row expanded per head into K and V, then
    attention with the 192-wide queries. Same I/O as decode()/naive_decode()."""
    B, s_q, H, kv, out = _attend_args(q, cache, w_uk, w_uv, out, stream)
    need = prefill_workspace_bytes(B, s_q, H, cache.max_seqlen)
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, q.device, stream)
    _maybe_validate(cache, s_q, stream)
    _check(_lib.mla_prefill_expand(_ptr(q), ctypes.byref(kv), _ptr(w_uk), _ptr(w_uv), B, s_q, H, float(scale),
                                   int(bool(causal)), _ptr(out), _ptr(workspace), workspace.numel(),
                                   _stream(stream)), "mla_prefill_expand")
    return out


def attend_uses_expand(s_q: int, max_seqlen: int) -> bool:
    r = int(_lib.mla_attend_uses_expand(s_q, max_seqlen))
    if r < 0:
        raise ValueError("invalid sizes")
    return bool(r)


def attend_workspace_bytes(B: int, s_q: int, H: int, max_seqlen: int) -> int:
    return int(_lib.mla_attend_workspace_bytes(B, s_q, H, max_seqlen))


def attend(q: torch.Tensor, cache: LatentCache, w_uk: torch.Tensor, w_uv: torch.Tensor,
           scale: float = DEFAULT_SCALE, causal: bool = True, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Absorbed or expand path, whichever costs fewer FLOPs for s_q query
    tokens against max_seqlen cached rows."""
    B, s_q, H, kv, out = _attend_args(q, cache, w_uk, w_uv, out, stream)
    need = attend_workspace_bytes(B, s_q, H, cache.max_seqlen)
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, q.device, stream)
    _maybe_validate(cache, s_q, stream)
    _check(_lib.mla_attend(_ptr(q), ctypes.byref(kv), _ptr(w_uk), _ptr(w_uv), B, s_q, H, float(scale),
                           int(bool(causal)), _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)),
           "mla_attend")
    return out
