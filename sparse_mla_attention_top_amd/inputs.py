"""Seeded synthetic workloads for sparse MLA attention.

This module only draws random inputs with the shapes and structure of the
sparse-MLA decode and prefill workloads; it holds none of the attention
arithmetic, the index conversion or the FP8 quantizer. Both the GPU path
(through the C ABI) and the fp64 oracle consume what it produces.

Structure follows what the pages state about the inputs:
  * the latent cache is paged, ``[num_blocks, block_size=64, 576]`` bf16
    (512 latent channels followed by 64 rope channels), or 512 channels in
    the NoPE variant (vLLM "Sparse MLA on Hopper" branch diff,
    cutlass_fa3_sparse.py, ``get_kv_cache_shape``; flashinfer_mla_sparse_sm90.py
    module docstring);
  * each query token carries a request-local top-k row of slot indices with
    -1 past its valid count, drawn as distinct uniform slots in random order
    the way the kernel tests use ``torch.randperm`` (FA3 kernel test file,
    ``test_fa3_mla_with_invalid_indices`` / ``test_fa3_valid_counts_correctness``);
  * a per-request block table maps request-local block numbers to cache
    blocks; ``req_id_per_token`` names each token's request (same branch,
    ``CutlassFA3MLASparseMetadata``).

Values are N(0,1) drawn in fp32 and rounded to bf16 (round to nearest even,
torch's ``.to(torch.bfloat16)``).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

BLOCK_SIZE = 64
D_LATENT = 512

# kv formats (mirror the C enum values)
KV_BF16 = 0
KV_FP8_PER_TENSOR = 1
KV_FP8_GROUP128 = 2
KV_FP8_DS_MLA = 3          # packed 656-byte rows


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    name: str
    seed: int
    num_requests: int
    tokens_per_req: int
    first_pos: int            # position of each request's first query token
    ctx_len: int              # context length per request (slots it owns)
    heads: int
    d_rope: int               # 64, or 0 for NoPE
    kv_format: int
    topk: int
    softmax_scale: float
    valid_rule: str           # "min_pos" : v = min(topk, pos+1) from [0, pos]
                              # "range"   : v ~ U{lo..hi} from [0, pos]
    valid_lo: int = 0
    valid_hi: int = 0
    identity_blocks: bool = False

    @property
    def d(self) -> int:
        return D_LATENT + self.d_rope

    @property
    def num_tokens(self) -> int:
        return self.num_requests * self.tokens_per_req

    @property
    def blocks_per_req(self) -> int:
        return (self.ctx_len + BLOCK_SIZE - 1) // BLOCK_SIZE

    @property
    def num_blocks(self) -> int:
        return self.num_requests * self.blocks_per_req

    @property
    def num_slots(self) -> int:
        return self.num_blocks * BLOCK_SIZE

    def scaled(self, **kw) -> "WorkloadSpec":
        return dataclasses.replace(self, **kw)


# The five workloads (decode and prefill shapes of the pages). Scales: the
# tiny case uses 576**-0.5; the bf16 decode case the literal 0.0723; the
# others 192**-0.5, the scale the pages' DeepSeek-V3.2 sparse path passes.
SPECS = {
    "tiny": WorkloadSpec("tiny", 101, 1, 4, 0, 256, 16, 64, KV_BF16, 64,
                         576 ** -0.5, "min_pos", identity_blocks=True),
    "tiny_late": WorkloadSpec("tiny_late", 111, 1, 4, 252, 256, 16, 64, KV_BF16, 64,
                              576 ** -0.5, "min_pos", identity_blocks=True),
    "decode_bf16": WorkloadSpec("decode_bf16", 202, 32, 1, 8191, 8192, 128, 64, KV_BF16,
                                2048, 0.0723, "min_pos"),
    "nope_fp8": WorkloadSpec("nope_fp8", 303, 128, 1, 16383, 16384, 64, 0,
                             KV_FP8_PER_TENSOR, 2048, 192 ** -0.5, "range", 512, 2048),
    "prefill_bf16": WorkloadSpec("prefill_bf16", 404, 1, 4096, 0, 4096, 128, 64, KV_BF16,
                                 2048, 192 ** -0.5, "min_pos", identity_blocks=True),
    "longctx_fp8": WorkloadSpec("longctx_fp8", 505, 64, 4, 65532, 65536, 128, 64,
                                KV_FP8_GROUP128, 2048, 192 ** -0.5, "min_pos"),
    # the long-context decode shape on the packed 656-byte FP8 rows of the
    # FlashMLA sparse backend (heads padded to 64 / 128 there; here h = 128)
    "longctx_ds_mla": WorkloadSpec("longctx_ds_mla", 606, 64, 4, 65532, 65536, 128, 64,
                                   KV_FP8_DS_MLA, 2048, 192 ** -0.5, "min_pos"),
    # the bf16 prefill shape on packed FP8 rows (the FP8 prefill of the pages'
    # FlashMLA sparse backend)
    "prefill_ds_mla": WorkloadSpec("prefill_ds_mla", 707, 1, 4096, 0, 4096, 128, 64, KV_FP8_DS_MLA,
                                   2048, 192 ** -0.5, "min_pos", identity_blocks=True),
}


@dataclasses.dataclass
class Workload:
    spec: WorkloadSpec
    q: torch.Tensor                 # [T, h, D] bf16
    kv_src: torch.Tensor            # [S, D] bf16: the cache rows (bf16 format) or the
                                    # values that the cache write quantizes (fp8 formats)
    k_scale: float                  # per-tensor scale (fp8 per-tensor), else 1.0
    req_id: torch.Tensor            # [T] int32
    block_table: torch.Tensor       # [R, blocks_per_req] int32
    topk_local: torch.Tensor        # [T, topk] int32, request-local, -1 tail
    positions: torch.Tensor         # [T] int64
    valid: torch.Tensor             # [T] int32, length of each row's valid prefix


def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + stream)
    return g


def _bf16_normal(shape, seed: int, stream: int, device, chunk_rows: int = 1 << 20):
    """N(0,1) fp32 draws rounded to bf16, generated in row chunks."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    g = _gen(seed, stream, device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = torch.randn((r1 - r0, flat.shape[1]), generator=g,
                                  dtype=torch.float32, device=device).to(torch.bfloat16)
    return out


def normal_bf16_rows(n: int, d: int, seed: int, stream: int = 0, device="cpu") -> torch.Tensor:
    """[n, d] N(0,1) values rounded to bf16 from generator (seed, stream)."""
    return _bf16_normal((n, d), seed, 1000 + stream, device)


def per_tensor_scale_from_absmax(kv_src: torch.Tensor) -> float:
    """Calibrated per-tensor scale of the input recipe: fl32(absmax / 448)."""
    amax = np.float32(kv_src.abs().max().float().item())
    if amax == 0:
        return 1.0
    return float(np.float32(amax) / np.float32(448.0))


def generate(spec: WorkloadSpec, device="cpu", kv_device=None, with_values: bool = True) -> Workload:
    """Draw one workload. Index structures are drawn on the CPU (they are small);
    Q and the cache rows on ``kv_device`` (defaults to ``device``). With
    ``with_values=False`` only the index structures are drawn (q and kv_src
    are empty placeholders)."""
    kv_device = device if kv_device is None else kv_device
    T, R, K = spec.num_tokens, spec.num_requests, spec.topk
    gi = _gen(spec.seed, 1, "cpu")

    # block table: identity or a random permutation of all blocks
    if spec.identity_blocks:
        bt = torch.arange(spec.num_blocks, dtype=torch.int32).view(R, spec.blocks_per_req)
    else:
        bt = torch.randperm(spec.num_blocks, generator=_gen(spec.seed, 2, "cpu"))
        bt = bt.to(torch.int32).view(R, spec.blocks_per_req)

    req_id = torch.arange(R, dtype=torch.int32).repeat_interleave(spec.tokens_per_req)
    positions = (spec.first_pos + torch.arange(spec.tokens_per_req)).repeat(R)

    topk_local = torch.full((T, K), -1, dtype=torch.int32)
    valid = torch.empty(T, dtype=torch.int32)
    for t in range(T):
        pos = int(positions[t])
        visible = min(pos + 1, spec.ctx_len)
        if spec.valid_rule == "min_pos":
            v = min(K, visible)
        elif spec.valid_rule == "range":
            v = int(torch.randint(spec.valid_lo, spec.valid_hi + 1, (1,), generator=gi))
            v = min(v, visible)
        else:
            raise ValueError(spec.valid_rule)
        topk_local[t, :v] = torch.randperm(visible, generator=gi)[:v].to(torch.int32)
        valid[t] = v

    if with_values:
        q = _bf16_normal((T, spec.heads, spec.d), spec.seed, 3, kv_device)
        kv_src = _bf16_normal((spec.num_slots, spec.d), spec.seed, 4, kv_device)
        k_scale = per_tensor_scale_from_absmax(kv_src) if spec.kv_format == KV_FP8_PER_TENSOR else 1.0
    else:
        q = torch.empty((0,), dtype=torch.bfloat16)
        kv_src = torch.empty((0,), dtype=torch.bfloat16)
        k_scale = 1.0
    return Workload(spec, q, kv_src, k_scale, req_id.to(device), bt.to(device),
                    topk_local.to(device), positions, valid.to(device))


def algorithmic_flops(spec: WorkloadSpec, valid: torch.Tensor) -> float:
    """2*h*v_t*(D + 512) summed over tokens: QK^T over D channels plus P.V over
    the 512 latent channels, true heads and valid entries only."""
    return float(2 * spec.heads * (spec.d + D_LATENT) * int(valid.sum()))


def kv_row_bytes(spec: WorkloadSpec) -> int:
    if spec.kv_format == KV_BF16:
        return 2 * spec.d
    if spec.kv_format == KV_FP8_PER_TENSOR:
        return spec.d
    if spec.kv_format == KV_FP8_DS_MLA:
        return 656
    return spec.d + 4 * math.ceil(spec.d / 128)


@dataclasses.dataclass
class RandomCase:
    q: torch.Tensor          # [T, h, 512 + d_rope] bf16
    kv_src: torch.Tensor     # [S, 512 + d_rope] bf16
    indices: torch.Tensor    # [T, topk] int32 global slots, -1 = invalid
    lengths: torch.Tensor    # [T] int32, length of each row's valid prefix


def random_case(T: int, h: int, d_rope: int, topk: int, num_slots: int, seed: int,
                lengths=None, device="cpu") -> RandomCase:
    """Small synthetic case with global slot indices: row t lists lengths[t]
    distinct uniform slots (random order) followed by -1. ``lengths`` defaults
    to topk for every row (capped at num_slots)."""
    g = torch.Generator().manual_seed(seed)
    D = D_LATENT + d_rope
    q = torch.randn((T, h, D), generator=g).to(torch.bfloat16)
    kv = torch.randn((num_slots, D), generator=g).to(torch.bfloat16)
    if lengths is None:
        lengths = [min(topk, num_slots)] * T
    lengths = [int(v) for v in lengths]
    idx = torch.full((T, topk), -1, dtype=torch.int32)
    for t, v in enumerate(lengths):
        idx[t, :v] = torch.randperm(num_slots, generator=g)[:v].to(torch.int32)
    return RandomCase(q.to(device), kv.to(device), idx.to(device),
                      torch.tensor(lengths, dtype=torch.int32).to(device))


def draw_cache_copy(spec: WorkloadSpec, copy: int, device) -> torch.Tensor:
    """Another independent draw of the cache rows ([S, D] bf16) of ``spec``
    (copy 0 is the one ``generate`` returns); used to rotate inputs so that
    repeated steps do not find their rows in the last-level cache."""
    stream = 4 if copy == 0 else 100 + copy
    return _bf16_normal((spec.num_slots, spec.d), spec.seed, stream, device)
