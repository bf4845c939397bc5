"""ctypes binding of libsmla.so (the gfx950 sparse MLA library).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/smla.h. PyTorch provides device
memory and the current stream. If the library is missing the calls raise;
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsmla.so")

KV_BF16 = 0
KV_FP8_PER_TENSOR = 1
KV_FP8_GROUP128 = 2
KV_FP8_DS_MLA = 3          # packed 656-byte rows: 512 E4M3 codes | 4 fp32 scales | 64 bf16 rope
DS_MLA_ROW_BYTES = 656

SMLA_OK = 0

EXPORTED = (
    "smla_convert_indices",
    "smla_decode_workspace_size",
    "smla_decode_num_splits",
    "smla_decode_fwd",
    "smla_prefill_fwd",
    "smla_cache_write",
    "smla_set_timing_events",
    "smla_last_error",
    "smla_version",
    "smla_attn_args_size",
    "smla_dcp_filter_convert",
    "smla_merge_partials",
    "smla_planned_valid_counts",
    "smla_gather_upconvert",
    "smla_decode_fwd_noalloc",
)


class SmlaError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("q_nope", ctypes.c_void_p),
        ("q_nope_stride_tok", ctypes.c_int64),
        ("q_nope_stride_head", ctypes.c_int64),
        ("q_rope", ctypes.c_void_p),
        ("q_rope_stride_tok", ctypes.c_int64),
        ("q_rope_stride_head", ctypes.c_int64),
        ("num_tokens", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("kv_cache", ctypes.c_void_p),
        ("num_slots", ctypes.c_int64),
        ("kv_row_stride_bytes", ctypes.c_int64),
        ("kv_format", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("group_scales", ctypes.c_void_p),
        ("indices", ctypes.c_void_p),
        ("indices_stride", ctypes.c_int64),
        ("topk", ctypes.c_int32),
        ("topk_length", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
        ("out", ctypes.c_void_p),
        ("out_stride_tok", ctypes.c_int64),
        ("out_stride_head", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        ("lse_stride_tok", ctypes.c_int64),
        ("num_splits", ctypes.c_int32),
        ("req_id", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("num_reqs", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("bt_row_stride", ctypes.c_int64),
        ("block_size", ctypes.c_int32),
        ("block_stride_rows", ctypes.c_int32),
        ("softcap", ctypes.c_float),
        ("sinks", ctypes.c_void_p),
        ("group_scales_stride", ctypes.c_int64),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load libsmla.so (built in-tree by ``python -m sparse_mla_attention_top_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sparse_mla_attention_top_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.smla_convert_indices.argtypes = [vp, vp, i32, i32, i64, vp, i64, i32, i32, i32, i32, vp, i64, vp, vp]
    lib.smla_convert_indices.restype = ctypes.c_int
    lib.smla_dcp_filter_convert.argtypes = [vp, vp, i32, i32, i64, vp, i64, i32, i32, i32, i32, i32, i32, i32, i32,
                                            vp, i64, vp, vp]
    lib.smla_dcp_filter_convert.restype = ctypes.c_int
    lib.smla_merge_partials.argtypes = [vp, i64, i64, i64, vp, i64, i64, i32, i32, i32, vp, i64, i64, vp, i64, vp]
    lib.smla_merge_partials.restype = ctypes.c_int
    lib.smla_planned_valid_counts.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp]
    lib.smla_planned_valid_counts.restype = ctypes.c_int
    lib.smla_gather_upconvert.argtypes = [vp, i64, i64, i32, vp, i32, i32, i64, i32, i32, vp, vp, i32, vp, i64, i64,
                                          vp]
    lib.smla_gather_upconvert.restype = ctypes.c_int
    lib.smla_decode_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.smla_decode_workspace_size.restype = sz
    lib.smla_decode_num_splits.argtypes = [i32, i32, i32, i32]
    lib.smla_decode_num_splits.restype = i32
    lib.smla_decode_fwd.argtypes = [ctypes.POINTER(AttnArgs), vp, sz, vp]
    lib.smla_decode_fwd.restype = ctypes.c_int
    lib.smla_decode_fwd_noalloc.argtypes = [ctypes.POINTER(AttnArgs), vp]
    lib.smla_decode_fwd_noalloc.restype = ctypes.c_int
    lib.smla_prefill_fwd.argtypes = [ctypes.POINTER(AttnArgs), vp]
    lib.smla_prefill_fwd.restype = ctypes.c_int
    lib.smla_cache_write.argtypes = [vp, i64, vp, i64, vp, i32, i32, i32, f32, vp, i64, i64, vp, i64, vp]
    lib.smla_cache_write.restype = ctypes.c_int
    lib.smla_set_timing_events.argtypes = [vp, vp]
    lib.smla_set_timing_events.restype = ctypes.c_int
    lib.smla_attn_args_size.argtypes = []
    lib.smla_attn_args_size.restype = sz
    if lib.smla_attn_args_size() != ctypes.sizeof(AttnArgs):
        raise RuntimeError(f"{LIB_PATH}: smla_attn_args is {lib.smla_attn_args_size()} bytes, "
                           f"the binding lays out {ctypes.sizeof(AttnArgs)}: rebuild the library")
    lib.smla_last_error.argtypes = []
    lib.smla_last_error.restype = ctypes.c_char_p
    lib.smla_version.argtypes = []
    lib.smla_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(fn: str, rc: int) -> None:
    if rc != SMLA_OK:
        raise SmlaError(fn, rc, load().smla_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


# ---------------------------------------------------------------------------
# index conversion
# ---------------------------------------------------------------------------

def _bt_row_stride(block_table: torch.Tensor) -> int:
    """Row stride of a [R, max_blocks] block table; a one-row table may carry any
    stride for its size-1 dimension, so its row length is passed instead."""
    return block_table.stride(0) if block_table.shape[0] > 1 else block_table.shape[1]


def convert_indices(req_id: torch.Tensor, block_table: torch.Tensor, topk_local: torch.Tensor,
                    block_size: int = 64, block_stride_rows: int = 0,
                    out: Optional[torch.Tensor] = None, valid_counts: Optional[torch.Tensor] = None,
                    want_valid_counts: bool = True, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Request-local top-k indices -> global cache slots (+ valid counts)."""
    _need(topk_local.dtype == torch.int32 and req_id.dtype == torch.int32 and block_table.dtype == torch.int32,
          "int32 tensors expected")
    _need(topk_local.dim() == 2 and topk_local.stride(1) == 1, "topk_local must be [T, K] with unit column stride")
    _need(block_table.dim() == 2 and block_table.stride(1) == 1, "block_table must be [R, max_blocks]")
    T, K = topk_local.shape
    if out is None:
        out = torch.empty((T, K), dtype=torch.int32, device=topk_local.device)
    if valid_counts is None and want_valid_counts:
        valid_counts = torch.empty((T,), dtype=torch.int32, device=topk_local.device)
    rc = load().smla_convert_indices(_ptr(req_id), _ptr(block_table), block_table.shape[0], block_table.shape[1],
                                     _bt_row_stride(block_table), _ptr(topk_local), topk_local.stride(0), T, K,
                                     block_size, block_stride_rows, _ptr(out), out.stride(0), _ptr(valid_counts),
                                     _stream(stream))
    _check("smla_convert_indices", rc)
    return out, valid_counts


def dcp_filter_convert(req_id: torch.Tensor, block_table: torch.Tensor, topk_tokens: torch.Tensor,
                       dcp_size: int, dcp_rank: int, interleave: int, block_size: int = 64,
                       block_stride_rows: int = 0, compact_valid_to_front: bool = False,
                       out: Optional[torch.Tensor] = None, valid_counts: Optional[torch.Tensor] = None,
                       want_valid_counts: bool = True, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One context-parallel rank's local cache slots for top-k rows of request
    token positions (-1 where the position is on another rank)."""
    _need(topk_tokens.dtype == torch.int32 and req_id.dtype == torch.int32 and block_table.dtype == torch.int32,
          "int32 tensors expected")
    _need(topk_tokens.dim() == 2 and topk_tokens.stride(1) == 1, "topk_tokens must be [T, K] with unit column stride")
    _need(block_table.dim() == 2 and block_table.stride(1) == 1, "block_table must be [R, max_blocks]")
    T, K = topk_tokens.shape
    if out is None:
        out = torch.empty((T, K), dtype=torch.int32, device=topk_tokens.device)
    if valid_counts is None and want_valid_counts:
        valid_counts = torch.empty((T,), dtype=torch.int32, device=topk_tokens.device)
    rc = load().smla_dcp_filter_convert(_ptr(req_id), _ptr(block_table), block_table.shape[0], block_table.shape[1],
                                        _bt_row_stride(block_table), _ptr(topk_tokens), topk_tokens.stride(0), T, K,
                                        dcp_size, dcp_rank, interleave, block_size, block_stride_rows,
                                        1 if compact_valid_to_front else 0, _ptr(out), out.stride(0),
                                        _ptr(valid_counts), _stream(stream))
    _check("smla_dcp_filter_convert", rc)
    return out, valid_counts


def merge_partials(part_out: torch.Tensor, part_lse: torch.Tensor, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, return_lse: bool = True,
                   stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Merge partials part_out [P, T, h, 512] bf16 / part_lse [P, T, h] fp32
    by their LSE. Returns (out [T, h, 512] bf16, lse [T, h] fp32 or None)."""
    _need(part_out.dtype == torch.bfloat16 and part_out.dim() == 4 and part_out.shape[3] == 512
          and part_out.stride(3) == 1, "part_out must be bf16 [P, T, h, 512] with unit channel stride")
    P, T, H, _ = part_out.shape
    _need(part_lse.dtype == torch.float32 and part_lse.shape == (P, T, H) and part_lse.stride(2) == 1,
          "part_lse must be fp32 [P, T, h]")
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=part_out.device)
    _need(out.dtype == torch.bfloat16 and out.shape == (T, H, 512) and out.stride(2) == 1, "out must be bf16 [T, h, 512]")
    if lse is None and return_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=part_out.device)
    rc = load().smla_merge_partials(_ptr(part_out), part_out.stride(0), part_out.stride(1), part_out.stride(2),
                                    _ptr(part_lse), part_lse.stride(0), part_lse.stride(1), P, T, H,
                                    _ptr(out), out.stride(0), out.stride(1), _ptr(lse),
                                    lse.stride(0) if lse is not None else 0, _stream(stream))
    _check("smla_merge_partials", rc)
    return out, lse


def planned_valid_counts(seq_lens: torch.Tensor, query_start_loc: torch.Tensor, req_id: torch.Tensor, topk: int,
                         kpool: int, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Valid count of every query row from the batch layout (int32 [T])."""
    for name, t in (("seq_lens", seq_lens), ("query_start_loc", query_start_loc), ("req_id", req_id)):
        _need(t.dtype == torch.int32 and t.dim() == 1 and t.is_contiguous(), f"{name} must be contiguous int32 [n]")
    R, T = seq_lens.shape[0], req_id.shape[0]
    _need(query_start_loc.shape[0] == R + 1, "query_start_loc must be int32 [num_reqs + 1]")
    if out is None:
        out = torch.empty((T,), dtype=torch.int32, device=req_id.device)
    _need(out.dtype == torch.int32 and out.numel() == T and out.is_contiguous(), "out must be int32 [T]")
    rc = load().smla_planned_valid_counts(_ptr(seq_lens), _ptr(query_start_loc), _ptr(req_id), R, T, int(topk),
                                          int(kpool), _ptr(out), _stream(stream))
    _check("smla_planned_valid_counts", rc)
    return out


def gather_upconvert(kv_cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                     workspace_starts: torch.Tensor, max_seq_len: int, workspace: torch.Tensor,
                     block_size: int = 64, block_stride_rows: int = 0, stream=None) -> torch.Tensor:
    """Gather each request's context rows from a packed FP8 cache into the bf16
    workspace [W, 576] at workspace_starts[r] + position."""
    S, row_stride, width = _kv_geometry(kv_cache)
    _check_kv(kv_cache, KV_FP8_DS_MLA, width, S, None)
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.stride(1) == 1,
          "block_table must be int32 [num_reqs, max_blocks]")
    R = block_table.shape[0]
    for name, t in (("seq_lens", seq_lens), ("workspace_starts", workspace_starts)):
        _need(t.dtype == torch.int32 and t.numel() == R and t.is_contiguous(), f"{name} must be contiguous int32 [R]")
    _need(workspace.dtype == torch.bfloat16 and workspace.dim() == 2 and workspace.shape[1] >= 576
          and workspace.stride(1) == 1, "workspace must be bf16 [W, >= 576]")
    rc = load().smla_gather_upconvert(_ptr(kv_cache), S, row_stride, KV_FP8_DS_MLA, _ptr(block_table), R,
                                      block_table.shape[1], _bt_row_stride(block_table), int(block_size),
                                      int(block_stride_rows), _ptr(seq_lens), _ptr(workspace_starts), int(max_seq_len),
                                      _ptr(workspace), workspace.shape[0], workspace.stride(0), _stream(stream))
    _check("smla_gather_upconvert", rc)
    return workspace


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _kv_geometry(kv_cache: torch.Tensor):
    """(num_slots, row_stride_bytes, row_width) of a [..., S, D] or [blocks, B, D] cache."""
    if kv_cache.dim() == 3:
        nb, bs, d = kv_cache.shape
        _need(kv_cache.stride(2) == 1 and kv_cache.stride(0) == bs * kv_cache.stride(1),
              "paged cache must be [num_blocks, block_size, D] with contiguous blocks")
        return nb * bs, kv_cache.stride(1) * kv_cache.element_size(), d
    _need(kv_cache.dim() == 2 and kv_cache.stride(1) == 1, "cache must be [S, D] or [blocks, B, D]")
    return kv_cache.shape[0], kv_cache.stride(0) * kv_cache.element_size(), kv_cache.shape[1]


def _group_scales_stride(group_scales: Optional[torch.Tensor], S: int, d: int) -> int:
    """Row stride (floats) of a [num_slots, >= ceil(d/128)] fp32 group-scale
    array whose rows are those of the cache's slots; d = 512 + d_rope, the
    channels the call reads."""
    G = (d + 127) // 128
    _need(group_scales is not None and group_scales.dtype == torch.float32 and group_scales.dim() == 2
          and group_scales.shape[0] >= S and group_scales.shape[1] >= G and group_scales.stride(1) == 1,
          f"group_scales must be fp32 [num_slots, >= {G}] with unit column stride")
    return group_scales.stride(0)


def _check_kv(kv_cache: torch.Tensor, kv_format: int, width: int, S: int,
              group_scales: Optional[torch.Tensor]) -> None:
    """Storage type of the cache and the group-scale array for kv_format."""
    if kv_format == KV_BF16:
        _need(kv_cache.dtype == torch.bfloat16, "a bf16-format cache must be a bf16 tensor")
    else:
        _need(kv_cache.dtype == torch.uint8, "an FP8-format cache must be a uint8 tensor of E4M3FN codes")
    if kv_format == KV_FP8_GROUP128:
        _need(group_scales is not None, "group_scales is required for the group-scaled FP8 format")
    if kv_format == KV_FP8_DS_MLA:
        _need(width >= DS_MLA_ROW_BYTES and group_scales is None,
              "a packed FP8 cache is uint8 [..., >= 656] with its scales in the row (no group_scales)")


def _attn_args(q_nope, q_rope, kv_cache, kv_format, indices, softmax_scale, topk_length, k_scale,
               group_scales, out, lse, num_splits, block_table=None, req_id=None, block_size=64,
               block_stride_rows=0, softcap=0.0, sinks=None) -> Tuple[AttnArgs, torch.Tensor, Optional[torch.Tensor]]:
    _need(q_nope.dtype == torch.bfloat16 and q_nope.dim() == 3 and q_nope.shape[2] == 512 and q_nope.stride(2) == 1,
          "q_nope must be bf16 [T, h, 512] with unit channel stride")
    T, H, _ = q_nope.shape
    d_rope = 0 if q_rope is None else q_rope.shape[2]
    if q_rope is not None:
        _need(q_rope.dtype == torch.bfloat16 and q_rope.shape[:2] == (T, H) and q_rope.stride(2) == 1,
              "q_rope must be bf16 [T, h, d_rope]")
    _need(indices.dtype == torch.int32 and indices.dim() == 2 and indices.shape[0] == T and indices.stride(1) == 1,
          "indices must be int32 [T, topk]")
    if topk_length is not None:
        _need(topk_length.dtype == torch.int32 and topk_length.numel() == T, "topk_length must be int32 [T]")
    S, row_stride, width = _kv_geometry(kv_cache)
    _check_kv(kv_cache, kv_format, width, S, group_scales)
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=q_nope.device)
    _need(out.dtype == torch.bfloat16 and out.shape == (T, H, 512) and out.stride(2) == 1, "out must be bf16 [T, h, 512]")
    a = AttnArgs()
    a.q_nope = _ptr(q_nope)
    a.q_nope_stride_tok, a.q_nope_stride_head = q_nope.stride(0), q_nope.stride(1)
    a.q_rope = _ptr(q_rope)
    a.q_rope_stride_tok = q_rope.stride(0) if q_rope is not None else 0
    a.q_rope_stride_head = q_rope.stride(1) if q_rope is not None else 0
    a.num_tokens, a.num_heads, a.d_rope = T, H, d_rope
    a.kv_cache = _ptr(kv_cache)
    a.num_slots = S
    a.kv_row_stride_bytes = row_stride
    a.kv_format = kv_format
    a.k_scale = float(k_scale)
    a.group_scales = _ptr(group_scales)
    if kv_format == KV_FP8_GROUP128:
        a.group_scales_stride = _group_scales_stride(group_scales, S, 512 + d_rope)
    a.indices = _ptr(indices)
    a.indices_stride = indices.stride(0)
    a.topk = indices.shape[1]
    a.topk_length = _ptr(topk_length)
    a.softmax_scale = float(softmax_scale)
    a.out = _ptr(out)
    a.out_stride_tok, a.out_stride_head = out.stride(0), out.stride(1)
    a.lse = _ptr(lse)
    a.lse_stride_tok = lse.stride(0) if lse is not None else 0
    a.num_splits = int(num_splits)
    a.softcap = float(softcap)
    if sinks is not None:
        _need(sinks.dtype == torch.float32 and sinks.numel() == H and sinks.is_contiguous(),
              "sinks must be contiguous fp32 [h]")
        a.sinks = _ptr(sinks)
    if block_table is not None:
        _need(req_id is not None and req_id.dtype == torch.int32 and req_id.numel() == T and req_id.is_contiguous(),
              "req_id must be contiguous int32 [T] with a block table")
        _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.stride(1) == 1,
              "block_table must be int32 [num_reqs, max_blocks]")
        a.req_id = _ptr(req_id)
        a.block_table = _ptr(block_table)
        a.num_reqs, a.max_blocks = block_table.shape
        a.bt_row_stride = _bt_row_stride(block_table)
        a.block_size = int(block_size)
        a.block_stride_rows = int(block_stride_rows)
    return a, out, lse


def decode_workspace_size(num_tokens: int, num_heads: int, topk: int, num_splits: int = 0) -> int:
    return int(load().smla_decode_workspace_size(num_tokens, num_heads, topk, num_splits))


def decode_num_splits(num_tokens: int, num_heads: int, topk: int, num_splits: int = 0) -> int:
    return int(load().smla_decode_num_splits(num_tokens, num_heads, topk, num_splits))


def decode_fwd(q_nope, q_rope, kv_cache, indices, softmax_scale, kv_format=KV_BF16, topk_length=None,
               k_scale=1.0, group_scales=None, out=None, lse=None, return_lse=True, num_splits=0,
               workspace=None, stream=None, block_table=None, req_id=None, block_size=64, block_stride_rows=0,
               softcap=0.0, sinks=None):
    """Sparse MLA decode forward. Returns (out [T,h,512] bf16, lse [T,h] fp32 or None).
    With ``block_table`` (and ``req_id``), ``indices`` are request-local and are
    converted inside the attention kernel. ``softcap`` > 0 caps the scaled
    logits (c tanh(z / c)); ``sinks`` (fp32 [h]) adds one logit per head with a
    zero value row to each softmax."""
    T, H = q_nope.shape[:2]
    if lse is None and return_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q_nope.device)
    a, out, lse = _attn_args(q_nope, q_rope, kv_cache, kv_format, indices, softmax_scale, topk_length,
                             k_scale, group_scales, out, lse, num_splits, block_table, req_id, block_size,
                             block_stride_rows, softcap, sinks)
    need = decode_workspace_size(T, H, indices.shape[1], num_splits) if T > 0 else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_nope.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load().smla_decode_fwd(ctypes.byref(a), _ptr(workspace), ws_bytes, _stream(stream))
    _check("smla_decode_fwd", rc)
    return out, lse


def decode_fwd_noalloc(q_nope, q_rope, kv_cache, indices, softmax_scale, out, lse=None, kv_format=KV_BF16,
                       topk_length=None, k_scale=1.0, group_scales=None, num_splits=0, stream=None,
                       block_table=None, req_id=None, block_size=64, block_stride_rows=0, softcap=0.0, sinks=None):
    """decode_fwd without a workspace: the split partials live in the library's
    static device scratch (smla_decode_fwd_noalloc), and the caller passes the
    output (and LSE, or None) buffers, so nothing is allocated."""
    _need(out is not None, "decode_fwd_noalloc writes into a caller-owned out buffer (bf16 [T, h, 512])")
    a, out, lse = _attn_args(q_nope, q_rope, kv_cache, kv_format, indices, softmax_scale, topk_length,
                             k_scale, group_scales, out, lse, num_splits, block_table, req_id, block_size,
                             block_stride_rows, softcap, sinks)
    rc = load().smla_decode_fwd_noalloc(ctypes.byref(a), _stream(stream))
    _check("smla_decode_fwd_noalloc", rc)
    return out, lse


def prefill_fwd(q_nope, q_rope, kv_cache, indices, softmax_scale, kv_format=KV_BF16, topk_length=None,
                k_scale=1.0, group_scales=None, out=None, lse=None, return_lse=False, stream=None,
                block_table=None, req_id=None, block_size=64, block_stride_rows=0, softcap=0.0, sinks=None):
    """Sparse MLA prefill forward (no split). Returns (out, lse or None). ``block_table``,
    ``softcap`` and ``sinks`` as for decode_fwd."""
    T, H = q_nope.shape[:2]
    if lse is None and return_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q_nope.device)
    a, out, lse = _attn_args(q_nope, q_rope, kv_cache, kv_format, indices, softmax_scale, topk_length,
                             k_scale, group_scales, out, lse, 0, block_table, req_id, block_size,
                             block_stride_rows, softcap, sinks)
    rc = load().smla_prefill_fwd(ctypes.byref(a), _stream(stream))
    _check("smla_prefill_fwd", rc)
    return out, lse


# ---------------------------------------------------------------------------
# cache write
# ---------------------------------------------------------------------------

def cache_write(kv_c: torch.Tensor, k_pe: Optional[torch.Tensor], slot_mapping: torch.Tensor,
                kv_cache: torch.Tensor, kv_format: int = KV_BF16, k_scale: float = 1.0,
                group_scales: Optional[torch.Tensor] = None, stream=None) -> None:
    """Write [kv_c | k_pe] rows into the cache at slot_mapping (negative = skip)."""
    _need(kv_c.dtype == torch.bfloat16 and kv_c.dim() == 2 and kv_c.shape[1] == 512 and kv_c.stride(1) == 1,
          "kv_c must be bf16 [T, 512]")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == kv_c.shape[0], "slot_mapping must be int64 [T]")
    d_rope = 0 if k_pe is None else k_pe.shape[1]
    if k_pe is not None:
        _need(k_pe.dtype == torch.bfloat16 and k_pe.stride(1) == 1, "k_pe must be bf16 [T, d_rope]")
    S, row_stride, width = _kv_geometry(kv_cache)
    _check_kv(kv_cache, kv_format, width, S, group_scales)
    gs_stride = _group_scales_stride(group_scales, S, 512 + d_rope) if kv_format == KV_FP8_GROUP128 else 0
    rc = load().smla_cache_write(_ptr(kv_c), kv_c.stride(0), _ptr(k_pe), k_pe.stride(0) if k_pe is not None else 0,
                                 _ptr(slot_mapping), kv_c.shape[0], d_rope, kv_format, float(k_scale),
                                 _ptr(kv_cache), S, row_stride, _ptr(group_scales), gs_stride, _stream(stream))
    _check("smla_cache_write", rc)


def set_timing_events(start=None, end=None) -> None:
    """Record torch.cuda.Event pair around the main attention kernel of the
    following calls on this thread (None, None clears)."""
    rc = load().smla_set_timing_events(None if start is None else start.cuda_event,
                                       None if end is None else end.cuda_event)
    _check("smla_set_timing_events", rc)


def version() -> str:
    return load().smla_version().decode()
