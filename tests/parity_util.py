"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import sys
from typing import Optional

import numpy as np
import torch

from oracle import sparse_mla as O
from sparse_mla_attention_top_amd import smla

OUT_TOL = 1e-2      # max-abs on the output vs the fp64 oracle, before the output's own rounding:
                    # the bar is 1e-2 + half a bf16 ulp at |ref| (no bf16 value is closer than
                    # that to an arbitrary real; 0.0039 at |ref| in [1, 2), 0.0156 in [4, 8))
LSE_TOL = 1e-3      # max-abs on the LSE
U_BF16 = 2.0 ** -8  # bf16 unit roundoff (half an ulp relative to the binade's lower end)


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Largest round-to-nearest error of a bf16 value near |x|: 2^(e - 8) for
    |x| in [2^e, 2^(e+1)) (normal range; 2^-134 below it)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def say(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (CPU)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def q_f64(q: torch.Tensor) -> np.ndarray:
    return O.bf16_bits_to_f64(bits(q))


def compare(out_gpu: torch.Tensor, lse_gpu: Optional[torch.Tensor], ref, what: str, k: int = 1,
            stress: bool = False):
    """ref = (out, lse) or (out, lse, mag) from oracle_for. The output is held to
    max-abs 1e-2 plus half a bf16 ulp at |ref| (the rounding every bf16 output
    carries); the LSE to 1e-3. NaN must appear exactly where the oracle has it.

    k is the number of bf16 roundings each P term takes before the P.V MFMA:
    1 for bf16 and per-tensor FP8 caches (p -> bf16), 2 for the group-scaled FP8
    formats (then bf16(p) * the row's group scale -> bf16 again). The bar above
    absorbs one rounding; a second adds up to 2^-8 sum_j p_j |v_j| (mag), which
    k = 2 allows on top. ``stress`` (inputs built far outside the N(0,1)
    workloads, e.g. group scales spread over 2^-6 .. 2^6, where one rounding of P
    alone exceeds 1e-2) allows 2^-8 k mag. Prints the measured errors, and how
    far the worst element is from the plain bar (1e-2 + half an ulp)."""
    out_ref, lse_ref = ref[0], ref[1]
    o = out_gpu.float().cpu().numpy().astype(np.float64)
    assert o.shape == out_ref.shape, (what, o.shape, out_ref.shape)
    nan_ref = np.isnan(out_ref)
    assert (np.isnan(o) == nan_ref).all(), f"{what}: NaN pattern of the output differs (unwritten or wrong elements)"
    assert np.isfinite(o[~nan_ref]).all(), f"{what}: non-finite output"
    fin = ~nan_ref                           # elements with a number to compare
    diff = np.abs(o[fin] - out_ref[fin])
    err = diff.max() if diff.size else 0.0
    plain = OUT_TOL + half_ulp_bf16(out_ref[fin])
    bound = plain
    if stress or k > 1:
        assert len(ref) > 2 and ref[2] is not None, "this comparison needs the magnitude (oracle_for magnitude=True)"
        bound = bound + U_BF16 * (k if stress else k - 1) * ref[2][fin]
    excess = (diff - bound).max() if diff.size else 0.0
    plain_excess = (diff - plain).max() if diff.size else 0.0
    small = np.abs(out_ref[fin]) < 1.0
    small_err = diff[small].max() if small.any() else 0.0
    if excess > 0:
        at = int(np.argmax(diff - bound))
        print(f"[parity] {what}: worst element |ref| {abs(out_ref[fin][at]):.4f}, gpu {o[fin][at]:.4f}, "
              f"err {diff[at]:.3e}, bound {bound[at]:.3e}"
              + (f", sum p|v| {ref[2][fin][at]:.4f}" if len(ref) > 2 and ref[2] is not None else ""), flush=True)
    assert excess <= 0, (f"{what}: out err {err:.3e} exceeds the bar (1e-2 + half a bf16 ulp at |ref|"
                         f"{', + 2^-8 k sum p|v|' if stress else (', + 2^-8 (k-1) sum p|v|' if k > 1 else '')}); "
                         f"worst excess {excess:.3e}")
    lerr = 0.0
    if lse_gpu is not None and lse_ref is not None:
        l = lse_gpu.float().cpu().numpy().astype(np.float64)
        assert l.shape == lse_ref.shape
        assert (np.isnan(l) == np.isnan(lse_ref)).all(), f"{what}: NaN pattern of LSE differs"
        inf_ref = np.isneginf(lse_ref)
        assert (np.isneginf(l) == inf_ref).all(), f"{what}: -inf pattern of LSE differs"
        fl = np.isfinite(lse_ref)
        if fl.any():
            lerr = np.abs(l[fl] - lse_ref[fl]).max()
        assert lerr <= LSE_TOL, f"{what}: lse max-abs err {lerr:.3e} > {LSE_TOL}"
    print(f"[parity] {what}: out max-abs {err:.3e} (|ref| < 1: {small_err:.3e}; worst margin to 1e-2 + half ulp "
          f"{-plain_excess:+.3e}), lse max-abs {lerr:.3e}", flush=True)
    return err, lerr


def oracle_for(q: torch.Tensor, cache_bits: np.ndarray, global_idx: np.ndarray, scale: float,
               lengths: Optional[np.ndarray] = None, tokens=None, kv_format: int = O.KV_BF16,
               k_scale: float = 1.0, group_scales: Optional[np.ndarray] = None, softcap: float = 0.0,
               sinks: Optional[np.ndarray] = None, magnitude: Optional[bool] = None):
    """The oracle's (out, lse) for the selected tokens, and sum_j p_j |v_j| with
    ``magnitude`` (default: for the group-scaled FP8 formats, whose comparisons
    allow for the second rounding of P)."""
    if magnitude is None:
        magnitude = kv_format in (O.KV_FP8_GROUP128, O.KV_FP8_DS_MLA)
    sel = np.arange(q.shape[0]) if tokens is None else np.asarray(tokens)
    qf = q_f64(q[torch.as_tensor(sel)])
    idx = global_idx[sel]
    ln = None if lengths is None else np.asarray(lengths)[sel]
    if magnitude:
        return O.attention_with_magnitude(qf, cache_bits, kv_format, idx, scale, topk_length=ln, k_scale=k_scale,
                                          group_scales=group_scales, softcap=softcap, sinks=sinks)
    return O.attention(qf, cache_bits, kv_format, idx, scale, topk_length=ln, k_scale=k_scale,
                       group_scales=group_scales, softcap=softcap, sinks=sinks)


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


# ---------------------------------------------------------------------------
# the library's attention calls with every output buffer filled with NaN first,
# so that an element the GPU path leaves unwritten cannot pass as a value left
# over from an earlier call
# ---------------------------------------------------------------------------

def nan_fill(t: Optional[torch.Tensor]) -> None:
    if t is None:
        return
    if t.dtype == torch.uint8:
        t.fill_(0xFF)                     # all-ones bytes: NaN as bf16 and as fp32
    else:
        t.fill_(float("nan"))


def _prepared(q_nope, kw, want_lse: bool):
    T, H = q_nope.shape[:2]
    dev = q_nope.device
    if kw.get("out") is None:
        kw["out"] = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    nan_fill(kw["out"])
    if kw.get("lse") is None and want_lse:
        kw["lse"] = torch.empty((T, H), dtype=torch.float32, device=dev)
    nan_fill(kw.get("lse"))
    return T, H


def decode_fwd(q_nope, q_rope, kv_cache, indices, softmax_scale, **kw):
    """smla.decode_fwd with NaN-filled out, LSE and split workspace."""
    T, H = _prepared(q_nope, kw, kw.get("return_lse", True))
    need = smla.decode_workspace_size(T, H, indices.shape[1], kw.get("num_splits", 0)) if T > 0 else 0
    if kw.get("workspace") is None and need > 0:
        kw["workspace"] = torch.empty(need, dtype=torch.uint8, device=q_nope.device)
    nan_fill(kw.get("workspace"))
    return smla.decode_fwd(q_nope, q_rope, kv_cache, indices, softmax_scale, **kw)


def prefill_fwd(q_nope, q_rope, kv_cache, indices, softmax_scale, **kw):
    """smla.prefill_fwd with NaN-filled out and LSE."""
    _prepared(q_nope, kw, kw.get("return_lse", False))
    return smla.prefill_fwd(q_nope, q_rope, kv_cache, indices, softmax_scale, **kw)


def merge_partials(part_out, part_lse, **kw):
    """smla.merge_partials with NaN-filled out and LSE."""
    P, T, H, _ = part_out.shape
    if kw.get("out") is None:
        kw["out"] = torch.empty((T, H, 512), dtype=torch.bfloat16, device=part_out.device)
    nan_fill(kw["out"])
    if kw.get("lse") is None and kw.get("return_lse", True):
        kw["lse"] = torch.empty((T, H), dtype=torch.float32, device=part_out.device)
    nan_fill(kw.get("lse"))
    return smla.merge_partials(part_out, part_lse, **kw)
