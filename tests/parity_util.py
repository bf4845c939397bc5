"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import sys
from typing import Optional

import numpy as np
import torch

from oracle import sparse_mla as O
from sparse_mla_attention_top_amd import smla

OUT_TOL = 1e-2      # max-abs on the bf16 output vs the fp64 oracle, plus the
U_BF16 = 2.0 ** -8  # rounding of bf16 operands and results (unit roundoff 2^-8):
                    # |gpu - ref| <= 1e-2 + u (|ref| + k * sum_j p_j |v_j|), where the
                    # output itself is rounded once to bf16 (u |ref|) and every term
                    # p_j v_j of the P.V sum carries k bf16 roundings of p_j: k = 1 for
                    # bf16 and per-tensor FP8 caches (P enters the MFMA in bf16), k = 2
                    # for the group-scaled FP8 cache (P times the row's group scale is
                    # rounded again). sum_j p_j |v_j| is given by the oracle. Outputs of
                    # ordinary size are held to the plain 1e-2.
LSE_TOL = 1e-3      # max-abs on the LSE


def say(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (CPU)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def q_f64(q: torch.Tensor) -> np.ndarray:
    return O.bf16_bits_to_f64(bits(q))


def compare(out_gpu: torch.Tensor, lse_gpu: Optional[torch.Tensor], ref, what: str, k: int = 1):
    """ref = (out, lse, mag) from oracle_for; k = bf16 roundings of each P term."""
    out_ref, lse_ref, mag_ref = ref
    o = out_gpu.float().cpu().numpy().astype(np.float64)
    assert o.shape == out_ref.shape, (what, o.shape, out_ref.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    diff = np.abs(o - out_ref)
    err = diff.max() if o.size else 0.0
    bound = OUT_TOL + U_BF16 * (np.abs(out_ref) + k * mag_ref)
    excess = (diff - bound).max() if o.size else 0.0
    assert excess <= 0, (f"{what}: out err {err:.3e} exceeds 1e-2 + 2^-8 (|ref| + {k} sum p|v|) "
                         f"(worst excess {excess:.3e})")
    lerr = 0.0
    if lse_gpu is not None and lse_ref is not None:
        l = lse_gpu.float().cpu().numpy().astype(np.float64)
        assert l.shape == lse_ref.shape
        inf_ref = np.isneginf(lse_ref)
        assert (np.isneginf(l) == inf_ref).all(), f"{what}: -inf pattern of LSE differs"
        if (~inf_ref).any():
            lerr = np.abs(l[~inf_ref] - lse_ref[~inf_ref]).max()
        assert lerr <= LSE_TOL, f"{what}: lse max-abs err {lerr:.3e} > {LSE_TOL}"
    return err, lerr


def oracle_for(q: torch.Tensor, cache_bits: np.ndarray, global_idx: np.ndarray, scale: float,
               lengths: Optional[np.ndarray] = None, tokens=None, kv_format: int = O.KV_BF16,
               k_scale: float = 1.0, group_scales: Optional[np.ndarray] = None, softcap: float = 0.0,
               sinks: Optional[np.ndarray] = None):
    sel = np.arange(q.shape[0]) if tokens is None else np.asarray(tokens)
    qf = q_f64(q[torch.as_tensor(sel)])
    idx = global_idx[sel]
    ln = None if lengths is None else np.asarray(lengths)[sel]
    return O.attention_with_magnitude(qf, cache_bits, kv_format, idx, scale, topk_length=ln,
                                      k_scale=k_scale, group_scales=group_scales, softcap=softcap, sinks=sinks)


def cache_for(kv_src: torch.Tensor, kv_format: int, device: str = "cuda"):
    """The cache of one format built from bf16 rows [S, D]: (the cache as the
    oracle reads it, the device cache, device group scales or None, k_scale,
    the bf16 roundings k of each P term for compare)."""
    from sparse_mla_attention_top_amd import inputs as I
    rows = bits(kv_src)
    if kv_format == O.KV_BF16:
        return rows, kv_src.to(device), None, 1.0, 1
    if kv_format == O.KV_FP8_PER_TENSOR:
        ks = I.per_tensor_scale_from_absmax(kv_src)
        codes = O.quantize_per_tensor(rows, ks)
        return codes, torch.from_numpy(codes).to(device), None, ks, 1
    if kv_format == O.KV_FP8_GROUP128:
        codes, sc = O.quantize_group128(rows)
        return codes, torch.from_numpy(codes).to(device), torch.from_numpy(sc).to(device), 1.0, 2
    packed = np.zeros((rows.shape[0], O.DS_MLA_ROW_BYTES), np.uint8)
    O.cache_write(rows[:, :512], rows[:, 512:], np.arange(rows.shape[0]), O.KV_FP8_DS_MLA, packed)
    return packed, torch.from_numpy(packed).to(device), None, 1.0, 2
