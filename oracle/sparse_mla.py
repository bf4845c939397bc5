"""Plain fp64 oracle of the sparse MLA forward path, in numpy.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark. The library and its Python binding never
import it, and it shares no code with them.

What is computed, with the passage each step follows:

* ``convert_indices`` -- request-local top-k index -> global cache slot via
  the block table: slot = block_table[req, idx // B] * B + idx % B, -1 stays
  -1, and the per-row count of valid entries (vLLM "Sparse MLA on Hopper"
  branch, test_cutlass_fa3_sparse_backend.py, TEST 2.5 "Valid Counts from
  Index Conversion" and TEST 2.9 "Full fix flow"; cutlass_fa3_sparse.py,
  ``forward_mqa`` step 2).
* ``dequantize_rows`` -- cache rows to fp64: bf16 exactly; E4M3FN bytes times
  the per-tensor scale or the per-token x 128-channel-group scale
  (flashinfer_mla_sparse_sm90.py, module docstring).
* ``dequantize_rows`` for the packed 656-byte format (FlashMLA sparse
  backend: 656 bytes per token for its FP8 cache; CUTLASS FA3 sparse backend
  docstring, "Key differences"). The pages give the size only; the reading
  used is the split the size allows with the group scales of the other FP8
  format: bytes 0..511 the E4M3FN codes of the 512 latent channels, bytes
  512..527 four little-endian fp32 scales (latent group g = channels
  128g..128g+127), bytes 528..655 the 64 rope channels as plain bf16.
* ``attention`` -- per query token and head: scores over the token's valid
  top-k slots, s = scale * q . k over all D channels, softmax, output
  sum_j p_j * k[:512] in the 512-dim latent space, and LSE = ln sum exp(s)
  (FA3 kernel test file, ``test_fa3_mla_correctness_vs_reference``: the
  gathered K = [c_kv | k_rope], V = c_kv, SDPA with the given scale; FlashMLA
  sparse API docs, ``_forward_fp8_kv_mixed_batch``: LSE per (token, head),
  rows with no valid slot give (0, -inf)). Two options of the FA3 API
  (``flash_attn_with_kvcache`` arguments ``softcap`` and ``sinks``), whose
  formulas the pages do not print, are read as: softcap c > 0 replaces each
  scaled logit z by c * tanh(z / c) (0 disables it); a sink is one logit per
  head that joins the softmax denominator with a zero value row, so
  out = sum_j e^z_j v_j / (sum_j e^z_j + e^sink) and LSE = ln of that
  denominator; an empty row then gives (0, sink).
* ``dcp_filter_convert`` -- one context-parallel rank's share of a top-k row
  of request token positions: the positions this rank stores, converted to
  its local cache slots through its own block table, -1 elsewhere, optionally
  compacted to the front (vLLM FlashMLA sparse backend, ``forward_mqa``: the
  ``triton_filter_and_convert_dcp_index`` call with dcp_size, dcp_rank,
  cp_kv_cache_interleave_size and compact_valid_to_front). The pages do not
  print the placement; the reading used here is the plain interleave: with
  interleave I over W ranks, position p is on rank (p // I) % W at local
  position (p // (I W)) I + p % I.
* ``merge_partials`` -- combine partial (out, lse) pairs computed over
  disjoint slices of a row: the identity element is (0, -inf) (FlashMLA
  sparse API docs, ``_forward_fp8_kv_mixed_batch``, the cross-rank LSE merge).
* ``planned_valid_counts`` -- each query row's valid count from the batch
  layout alone: a row for the j-th query token of request i sees
  ctx = seq_len[i] - q_len[i] + j + 1 tokens, and the pooled indexer keeps
  ctx of them when ctx <= topk, else topk + ctx % kpool (FlashInfer sparse SM90
  backend, ``_kv_lens_host`` and ``_clamp_work_kv_end``).
  ``indexer_selection`` simulates the selection that docstring describes (whole
  context up to topk; else the best topk / kpool complete pools of kpool
  consecutive positions, expanded, plus the trailing incomplete pool), to pin
  the count.
* ``gather_upconvert`` -- the FP8 prefill design of the FlashMLA sparse backend
  (``forward_mqa``, the ``cp_gather_and_upconvert_fp8_kv_cache`` call): each
  request's context rows, in position order, are gathered from the packed FP8
  cache through the block table into a bf16 workspace at workspace_starts[r],
  and the bf16 kernel then runs over the workspace. The pages do not print
  the conversion; the reading is value = bf16_rne(fl32(e4m3 * scale)) per latent
  channel and the rope channels copied.
* ``cache_write`` -- write [kv_c(512) | k_pe(d_rope)] rows at slot_mapping,
  negative slots skipped; bf16 copy, or E4M3 with a given per-tensor scale,
  or E4M3 with per-token x 128-channel-group scales absmax/448 computed here
  (branch diff, ``do_kv_cache_update`` / ``concat_and_cache_mla``;
  flashinfer_mla_sparse_sm90.py docstring on the group-scale layout).

Readings where the pages are silent (each also listed in the design notes):
entries past the row length, negative entries, out-of-range local indices,
negative block-table entries and global slots >= num_slots are all invalid
and skipped; duplicates each count; LSE is the natural log of the scaled
logits; the FP8 quantizer divides in fp32 and rounds to nearest even with
saturation at 448.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from . import e4m3

KV_BF16 = 0
KV_FP8_PER_TENSOR = 1
KV_FP8_GROUP128 = 2
KV_FP8_DS_MLA = 3
D_V = 512
GROUP = 128
# packed row: [512 E4M3FN codes | 4 fp32 group scales | 64 bf16 rope channels]
DS_MLA_SCALES_AT = 512
DS_MLA_ROPE_AT = 528
DS_MLA_ROW_BYTES = 656


# ---------------------------------------------------------------------------
# bf16 <-> float
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the upper half of an IEEE binary32: value = float32(bits << 16)."""
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# index conversion
# ---------------------------------------------------------------------------

def convert_indices(req_id: np.ndarray, block_table: np.ndarray, topk_local: np.ndarray,
                    block_size: int, block_stride_rows: Optional[int] = None):
    """Returns (global [T, K] int32, valid_counts [T] int32).

    slot = block_table[req, l // block_size] * block_stride_rows + l % block_size
    for every entry l >= 0 whose block number is inside the table and whose
    table entry is >= 0; every other entry is -1. valid_counts[t] counts the
    entries that are not -1."""
    stride = block_size if block_stride_rows is None else block_stride_rows
    req_id = np.asarray(req_id, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    loc = np.asarray(topk_local, dtype=np.int64)
    T, K = loc.shape
    max_blocks = bt.shape[1]
    out = np.full((T, K), -1, dtype=np.int64)
    for t in range(T):
        row = loc[t]
        ok = row >= 0
        blk = np.where(ok, row // block_size, 0)
        ok &= blk < max_blocks
        blk = np.where(ok, blk, 0)
        entry = bt[req_id[t], blk]
        ok &= entry >= 0
        out[t] = np.where(ok, entry * stride + row % block_size, -1)
    valid = (out >= 0).sum(axis=1)
    return out.astype(np.int32), valid.astype(np.int32)


# ---------------------------------------------------------------------------
# dequantization
# ---------------------------------------------------------------------------

def pack_ds_mla(codes: np.ndarray, scales: np.ndarray, rope_bits: np.ndarray) -> np.ndarray:
    """Packed rows [n, 656] uint8 from latent codes [n, 512] uint8, group
    scales [n, 4] fp32 and rope bf16 bits [n, 64]."""
    n = codes.shape[0]
    out = np.empty((n, DS_MLA_ROW_BYTES), dtype=np.uint8)
    out[:, :DS_MLA_SCALES_AT] = codes
    out[:, DS_MLA_SCALES_AT:DS_MLA_ROPE_AT] = np.ascontiguousarray(scales, dtype="<f4").view(np.uint8)
    out[:, DS_MLA_ROPE_AT:] = np.ascontiguousarray(rope_bits, dtype="<u2").view(np.uint8)
    return out


def unpack_ds_mla(rows: np.ndarray):
    """(codes [n, 512], scales [n, 4] fp32, rope bf16 bits [n, 64]) of packed
    rows (the first 656 bytes of each row are used)."""
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.uint8)[:, :DS_MLA_ROW_BYTES])
    codes = rows[:, :DS_MLA_SCALES_AT]
    scales = np.ascontiguousarray(rows[:, DS_MLA_SCALES_AT:DS_MLA_ROPE_AT]).view("<f4")
    rope = np.ascontiguousarray(rows[:, DS_MLA_ROPE_AT:]).view("<u2")
    return codes, scales.astype(np.float32), rope.astype(np.uint16)


def dequantize_rows(cache: np.ndarray, kv_format: int, slots: np.ndarray,
                    k_scale: float = 1.0, group_scales: Optional[np.ndarray] = None,
                    d: Optional[int] = None) -> np.ndarray:
    """Rows ``slots`` of a flat cache ([S, D] uint16 bf16 bits, [S, D] uint8
    E4M3FN codes, or [S, >= 656] uint8 packed rows) as float64 values."""
    slots = np.asarray(slots, dtype=np.int64)
    if kv_format == KV_BF16:
        return bf16_bits_to_f64(cache[slots])
    if kv_format == KV_FP8_DS_MLA:
        codes, sc, rope = unpack_ds_mla(cache[slots])
        lat = e4m3.decode(codes) * np.repeat(sc.astype(np.float64), GROUP, axis=1)
        return np.concatenate([lat, bf16_bits_to_f64(rope)], axis=1)
    vals = e4m3.decode(cache[slots])
    if kv_format == KV_FP8_PER_TENSOR:
        return vals * float(np.float32(k_scale))
    if kv_format == KV_FP8_GROUP128:
        D = vals.shape[1]
        sc = np.asarray(group_scales, dtype=np.float32)[slots].astype(np.float64)
        per_channel = np.repeat(sc, GROUP, axis=1)[:, :D]
        return vals * per_channel
    raise ValueError(kv_format)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def valid_entries(idx_row: np.ndarray, length: Optional[int], num_slots: int) -> np.ndarray:
    """Entries of one global index row that take part: position < length
    (when a length is given) and 0 <= slot < num_slots."""
    row = np.asarray(idx_row, dtype=np.int64)
    n = row.shape[0] if length is None else max(0, min(int(length), row.shape[0]))
    row = row[:n]
    return row[(row >= 0) & (row < num_slots)]


def attention_rows(q_t: np.ndarray, rows: np.ndarray, scale: float, d_v: int = D_V,
                   magnitude: bool = False, softcap: float = 0.0,
                   sinks: Optional[np.ndarray] = None):
    """One query token: q_t [h, D] and its gathered rows [v, D] (fp64).
    Returns out [h, d_v], lse [h]; with ``magnitude`` also
    mag [h, d_v] = sum_j p_j |v_j|, the size against which rounding of the
    terms p_j v_j of the output is measured (0 for an empty row).
    softcap > 0: logits z = softcap * tanh(scale q.k / softcap). sinks [h]:
    one extra logit per head in the denominator, with a zero value row."""
    h = q_t.shape[0]
    sink = None if sinks is None else np.asarray(sinks, dtype=np.float64).reshape(h)
    if rows.shape[0] == 0:
        lse0 = np.full(h, -np.inf) if sink is None else sink.copy()
        empty = (np.zeros((h, d_v)), lse0)
        return empty + (np.zeros((h, d_v)),) if magnitude else empty
    s = scale * (q_t @ rows.T)                      # [h, v]
    if softcap > 0:
        s = softcap * np.tanh(s / softcap)
    m = s.max(axis=1, keepdims=True)
    if sink is not None:
        m = np.maximum(m, sink[:, None])
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    if sink is not None:
        l = l + np.exp(sink[:, None] - m)
    out = (p @ rows[:, :d_v]) / l
    lse = (m + np.log(l))[:, 0]
    if magnitude:
        return out, lse, (p @ np.abs(rows[:, :d_v])) / l
    return out, lse


def attention(q: np.ndarray, cache: np.ndarray, kv_format: int, indices: np.ndarray,
              softmax_scale: float, topk_length: Optional[np.ndarray] = None,
              k_scale: float = 1.0, group_scales: Optional[np.ndarray] = None,
              tokens: Optional[np.ndarray] = None, d_v: int = D_V, softcap: float = 0.0,
              sinks: Optional[np.ndarray] = None):
    """Sparse MLA forward over global slot indices.

    q: [T, h, D] float64 (already the bf16 values); cache: flat [S, D] in the
    storage format; indices: [T, K] global slots. Only the listed ``tokens``
    (default all) are computed. Returns out [n, h, d_v], lse [n, h] fp64.
    ``softcap`` and ``sinks`` [h] as in ``attention_rows``."""
    res = _attention(q, cache, kv_format, indices, softmax_scale, topk_length, k_scale, group_scales,
                     tokens, d_v, False, softcap, sinks)
    return res[0], res[1]


def attention_with_magnitude(q: np.ndarray, cache: np.ndarray, kv_format: int, indices: np.ndarray,
                             softmax_scale: float, topk_length: Optional[np.ndarray] = None,
                             k_scale: float = 1.0, group_scales: Optional[np.ndarray] = None,
                             tokens: Optional[np.ndarray] = None, d_v: int = D_V,
                             softcap: float = 0.0, sinks: Optional[np.ndarray] = None):
    """``attention`` plus mag [n, h, d_v] = sum_j p_j |v_j| per output element
    (the softmax-weighted sum of the magnitudes of the value rows)."""
    return _attention(q, cache, kv_format, indices, softmax_scale, topk_length, k_scale, group_scales,
                      tokens, d_v, True, softcap, sinks)


def _attention(q, cache, kv_format, indices, softmax_scale, topk_length, k_scale, group_scales,
               tokens, d_v, magnitude, softcap=0.0, sinks=None):
    tokens = np.arange(q.shape[0]) if tokens is None else np.asarray(tokens)
    S = cache.shape[0]
    outs, lses, mags = [], [], []
    for t in tokens:
        length = None if topk_length is None else int(topk_length[t])
        sel = valid_entries(indices[t], length, S)
        rows = dequantize_rows(cache, kv_format, sel, k_scale, group_scales)
        r = attention_rows(q[t], rows, softmax_scale, d_v, magnitude, softcap, sinks)
        outs.append(r[0])
        lses.append(r[1])
        if magnitude:
            mags.append(r[2])
    h = q.shape[1]
    if not outs:
        return np.zeros((0, h, d_v)), np.zeros((0, h)), np.zeros((0, h, d_v))
    return np.stack(outs), np.stack(lses), (np.stack(mags) if magnitude else None)


def planned_valid_counts(seq_lens: np.ndarray, query_start_loc: np.ndarray, req_id: np.ndarray,
                         topk: int, kpool: int) -> np.ndarray:
    """Valid count of every query row t (request r = req_id[t], rows of request
    r are query_start_loc[r] .. query_start_loc[r+1]-1): with
    ctx = seq_lens[r] - query_start_loc[r+1] + t + 1, ctx if ctx <= topk,
    else topk + ctx % kpool. A request id outside [0, R) or ctx <= 0 gives 0.
    int32 [T]."""
    seq = np.asarray(seq_lens, dtype=np.int64)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    req = np.asarray(req_id, dtype=np.int64)
    ok = (req >= 0) & (req < seq.shape[0])
    rq = np.where(ok, req, 0)
    rows = np.arange(req.shape[0], dtype=np.int64)
    ctx = np.where(ok, seq[rq] - qsl[rq + 1] + rows + 1, 0)
    ctx = np.maximum(ctx, 0)
    return np.where(ctx <= topk, ctx, topk + ctx % kpool).astype(np.int32)


def indexer_selection(ctx: int, topk: int, kpool: int, pool_scores: np.ndarray) -> np.ndarray:
    """Positions a pooled top-k indexer keeps for a context of ctx tokens:
    all of them when ctx <= topk; otherwise the topk // kpool complete pools
    (kpool consecutive positions each) with the highest pool_scores, expanded
    to their positions, plus every position of the trailing incomplete pool."""
    if ctx <= topk:
        return np.arange(ctx)
    assert topk % kpool == 0
    full = ctx // kpool
    best = np.argsort(-np.asarray(pool_scores)[:full], kind="stable")[:topk // kpool]
    kept = (best[:, None] * kpool + np.arange(kpool)[None, :]).ravel()
    tail = np.arange(full * kpool, ctx)
    return np.concatenate([kept, tail])


def upconvert_rows(cache: np.ndarray, slots: np.ndarray) -> np.ndarray:
    """Packed FP8 rows -> bf16 bit patterns [n, 576]: latent channel c is
    bf16_rne(fl32(e4m3(code) * scale[c // 128])), the rope channels are copied."""
    codes, sc, rope = unpack_ds_mla(np.asarray(cache)[np.asarray(slots, dtype=np.int64)])
    lat = (e4m3.decode(codes).astype(np.float32) * np.repeat(sc, GROUP, axis=1)).astype(np.float32)
    return np.concatenate([f32_to_bf16_bits(lat), rope], axis=1)


def gather_upconvert(cache: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray,
                     workspace_starts: np.ndarray, block_size: int, workspace: np.ndarray,
                     block_stride_rows: Optional[int] = None) -> None:
    """Row workspace_starts[r] + p of ``workspace`` (bf16 bits [W, 576]) gets
    request r's context position p < seq_lens[r] (and p < max_blocks * B), read
    from the packed cache at slot block_table[r][p // B] * stride + p % B and
    upconverted. A negative table entry or a slot past the cache gives a zero
    row; rows that fall outside the workspace are not written."""
    stride = block_size if block_stride_rows is None else block_stride_rows
    bt = np.asarray(block_table, dtype=np.int64)
    S, W = cache.shape[0], workspace.shape[0]
    for r in range(bt.shape[0]):
        n = min(int(seq_lens[r]), bt.shape[1] * block_size)
        for pos in range(max(n, 0)):
            w = int(workspace_starts[r]) + pos
            if w < 0 or w >= W:
                continue
            e = bt[r, pos // block_size]
            slot = e * stride + pos % block_size
            if e < 0 or slot >= S:
                workspace[w] = 0
            else:
                workspace[w] = upconvert_rows(cache, [slot])[0]


def dcp_owner_local(pos: np.ndarray, dcp_size: int, interleave: int):
    """(rank, local position) of request token positions pos >= 0 under the
    interleaved placement: runs of ``interleave`` consecutive positions go to
    ranks 0, 1, ..., W-1 in turn, and each rank stores its runs back to back."""
    pos = np.asarray(pos, dtype=np.int64)
    run = pos // interleave
    rank = run % dcp_size
    local = (run // dcp_size) * interleave + pos % interleave
    return rank, local


def dcp_filter_convert(req_id: np.ndarray, block_table: np.ndarray, topk_tokens: np.ndarray,
                       dcp_size: int, dcp_rank: int, interleave: int, block_size: int,
                       block_stride_rows: Optional[int] = None, compact_valid_to_front: bool = False):
    """Rank ``dcp_rank``'s view of top-k rows of request token positions.
    Returns (local slots [T, K] int32, valid_counts [T] int32).

    An entry p < 0, or a position stored on another rank, becomes -1. A
    position this rank stores is converted like ``convert_indices`` from its
    local position, through this rank's block table. With
    ``compact_valid_to_front`` the valid entries of a row come first, in
    their order, followed by -1."""
    loc = np.asarray(topk_tokens, dtype=np.int64)
    rank, local = dcp_owner_local(np.maximum(loc, 0), dcp_size, interleave)
    mine = (loc >= 0) & (rank == dcp_rank)
    local = np.where(mine, local, -1)
    out, valid = convert_indices(req_id, block_table, local, block_size, block_stride_rows)
    if compact_valid_to_front:
        packed = np.full_like(out, -1)
        for t in range(out.shape[0]):
            keep = out[t][out[t] >= 0]
            packed[t, :keep.size] = keep
        out = packed
    return out, valid


def merge_partials(outs: np.ndarray, lses: np.ndarray):
    """Merge P partial results over disjoint slices: outs [P, ..., d],
    lses [P, ...]. lse = ln sum_p exp(lse_p); out = sum_p exp(lse_p - lse) out_p.
    (0, -inf) is the identity; all-identity stays (0, -inf)."""
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    m = lses.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - m_safe), 0.0)     # [P, ...]
    tot = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    out = np.where(finite[..., None],
                   (w[..., None] * outs).sum(axis=0) / np.where(finite, tot, 1.0)[..., None],
                   0.0)
    return out, lse


# ---------------------------------------------------------------------------
# FP8 quantizer and cache write
# ---------------------------------------------------------------------------

def quantize_per_tensor(x_bits: np.ndarray, k_scale: float) -> np.ndarray:
    """bf16 rows -> E4M3FN codes of fl32(x / k_scale)."""
    x = bf16_bits_to_f32(x_bits)
    y = (x / np.float32(k_scale)).astype(np.float32)
    return e4m3.encode_rne(y)


def group_scale(absmax: np.ndarray) -> np.ndarray:
    """fl32(absmax / 448), and 1.0 where a group is all zero."""
    a = np.asarray(absmax, dtype=np.float32)
    s = (a / np.float32(448.0)).astype(np.float32)
    return np.where(a == 0, np.float32(1.0), s).astype(np.float32)


def quantize_group128(x_bits: np.ndarray):
    """bf16 rows [n, D] -> (codes [n, D] uint8, scales [n, ceil(D/128)] fp32).
    Group g covers channels [128 g, min(128 g + 128, D))."""
    x = bf16_bits_to_f32(x_bits)
    n, D = x.shape
    G = (D + GROUP - 1) // GROUP
    codes = np.empty((n, D), dtype=np.uint8)
    scales = np.empty((n, G), dtype=np.float32)
    for g in range(G):
        c0, c1 = g * GROUP, min(D, (g + 1) * GROUP)
        xs = x[:, c0:c1]
        sc = group_scale(np.abs(xs).max(axis=1))
        scales[:, g] = sc
        codes[:, c0:c1] = e4m3.encode_rne((xs / sc[:, None]).astype(np.float32))
    return codes, scales


def cache_write(kv_c_bits: np.ndarray, k_pe_bits: Optional[np.ndarray], slot_mapping: np.ndarray,
                kv_format: int, cache: np.ndarray, k_scale: float = 1.0,
                group_scales: Optional[np.ndarray] = None) -> None:
    """Write rows [kv_c | k_pe] into ``cache`` (flat [S, D]: uint16 bf16 bits or
    uint8 codes; packed format: [S, >= 656] uint8) at slot_mapping; slots < 0
    are skipped. In group mode the per-row scales go to ``group_scales``
    [S, ceil(D/128)]; the packed format quantizes the 512 latent channels per
    128-channel group with the same scale rule, stores the scales in the row
    and copies the 64 rope channels as bf16."""
    kv_c = np.asarray(kv_c_bits).view(np.uint16)
    rows = kv_c if k_pe_bits is None or np.asarray(k_pe_bits).shape[-1] == 0 else \
        np.concatenate([kv_c, np.asarray(k_pe_bits).view(np.uint16)], axis=1)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    rows, slots = rows[keep], slots[keep]
    if kv_format == KV_BF16:
        cache[slots] = rows
    elif kv_format == KV_FP8_PER_TENSOR:
        cache[slots] = quantize_per_tensor(rows, k_scale)
    elif kv_format == KV_FP8_GROUP128:
        codes, sc = quantize_group128(rows)
        cache[slots] = codes
        group_scales[slots] = sc
    elif kv_format == KV_FP8_DS_MLA:
        if rows.shape[1] != D_V + 64:
            raise ValueError("the packed format holds 512 latent + 64 rope channels")
        codes, sc = quantize_group128(rows[:, :D_V])
        cache[slots, :DS_MLA_ROW_BYTES] = pack_ds_mla(codes, sc, rows[:, D_V:])
    else:
        raise ValueError(kv_format)
