"""GPU parity of the packed 656-byte FP8 rows (512 E4M3FN latent codes, four
fp32 group scales, 64 bf16 rope channels per row) and of their cache write,
against the fp64 oracle.

The packed caches fed to the attention tests are written by the oracle's own
cache write, never by the GPU's, so every oracle input is independent of the
HIP path. The bar is that of the group-scaled FP8 tests: max-abs 1e-2 on the
output before its own bf16 rounding, plus the second rounding of P (P times
the row's group scale is rounded to bf16 again, k = 2), 1e-3 on the LSE; the
cache write is compared bit for bit."""
import numpy as np
import pytest
import torch

from oracle import e4m3
from oracle import sparse_mla as O
import parity_util as PU
from parity_util import bits, compare, oracle_for, say
from sparse_mla_attention_top_amd import inputs as I
from sparse_mla_attention_top_amd import smla

pytestmark = pytest.mark.gpu
DEV = "cuda"
FMT = O.KV_FP8_DS_MLA
K_ROUND = 2


def _pack(rows_bits: np.ndarray, width: int = O.DS_MLA_ROW_BYTES) -> np.ndarray:
    """Oracle cache write of bf16 rows [n, 576] into packed rows [n, width]."""
    n = rows_bits.shape[0]
    cache = np.zeros((n, width), np.uint8)
    O.cache_write(rows_bits[:, :512], rows_bits[:, 512:], np.arange(n), FMT, cache)
    return cache


def _attend(entry, q, cache_dev, idx_dev, scale, lengths_dev=None, num_splits=0, **conv):
    qd = q.to(DEV)
    qn, qr = qd[..., :512], qd[..., 512:]
    if entry == "decode":
        out, lse = PU.decode_fwd(qn, qr, cache_dev, idx_dev, scale, kv_format=FMT, topk_length=lengths_dev,
                                 num_splits=num_splits, **conv)
    else:
        out, lse = PU.prefill_fwd(qn, qr, cache_dev, idx_dev, scale, kv_format=FMT, topk_length=lengths_dev,
                                  return_lse=True, **conv)
    torch.cuda.synchronize()
    return out, lse


def _run(c, cache, scale, entry, use_lengths=True, num_splits=0, stress=False):
    ln = c.lengths if use_lengths else None
    out, lse = _attend(entry, c.q, torch.from_numpy(cache).to(DEV), c.indices.to(DEV), scale,
                       None if ln is None else ln.to(DEV), num_splits)
    ref = oracle_for(c.q, cache, c.indices.numpy(), scale, None if ln is None else ln.numpy(), kv_format=FMT)
    return out, lse, compare(out, lse, ref, f"packed fp8 {entry}", K_ROUND, stress)


def test_every_code_single_slot_is_exact():
    """Token t attends to slot t alone, so its output is that row's latent
    values; with power-of-two group scales every code times its scale is
    exact in bf16, so the output equals the decoded row bit for bit. Rows
    cycle through all 254 non-NaN codes; the rope part is plain bf16."""
    S = 256
    codes = ((np.arange(S)[:, None] + np.arange(512)[None, :]) % 256).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00
    rng = np.random.default_rng(5)
    scales = np.ldexp(1.0, rng.integers(-4, 5, (S, 4))).astype(np.float32)
    rope = bits(torch.randn((S, 64), generator=torch.Generator().manual_seed(6)).to(torch.bfloat16))
    cache = O.pack_ds_mla(codes, scales, rope)
    T, h = S, 16
    q = torch.randn((T, h, 576), generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    idx = torch.full((T, 8), -1, dtype=torch.int32)
    idx[:, 5] = torch.arange(T, dtype=torch.int32)
    vals = e4m3.decode(codes) * np.repeat(scales.astype(np.float64), 128, axis=1)
    say("packed fp8 every code")
    for entry in ("prefill", "decode"):
        out, lse = _attend(entry, q, torch.from_numpy(cache).to(DEV), idx.to(DEV), 0.05)
        got = out.float().cpu().numpy().astype(np.float64)
        bad = np.argwhere(got != vals[:, None, :])
        assert not len(bad), f"{entry}: {len(bad)} outputs differ from the decoded rows (first {bad[0]})"
        ref = oracle_for(q, cache, idx.numpy(), 0.05, kv_format=FMT)
        compare(out, lse, ref, f"packed every code {entry}", K_ROUND)


@pytest.mark.parametrize("h", [16, 64, 128])
def test_packed_heads(h):
    say(f"packed fp8 h={h}")
    c = I.random_case(T=3, h=h, d_rope=64, topk=200, num_slots=700, seed=90 + h, lengths=[200, 77, 129])
    cache = _pack(bits(c.kv_src))
    for entry in ("prefill", "decode"):
        _run(c, cache, 192 ** -0.5, entry)


@pytest.mark.parametrize("topk,lengths", [(1, [1, 0]), (33, [33, 32]), (2048, [2048, 1111])])
def test_packed_topk_widths_and_splits(topk, lengths):
    say(f"packed fp8 topk={topk}")
    c = I.random_case(T=2, h=128, d_rope=64, topk=topk, num_slots=4096, seed=95 + topk, lengths=lengths)
    cache = _pack(bits(c.kv_src))
    _run(c, cache, 192 ** -0.5, "prefill")
    for splits in (1, 3, 8):
        _run(c, cache, 192 ** -0.5, "decode", num_splits=splits)


def test_packed_scattered_invalid_empty_rows_and_row_padding():
    """-1 and out-of-range entries anywhere, an empty row, and rows padded to
    672 bytes (the cache row stride is not the row size)."""
    say("packed fp8 scattered invalid, padded rows")
    c = I.random_case(T=4, h=64, d_rope=64, topk=160, num_slots=400, seed=97)
    g = torch.Generator().manual_seed(98)
    c.indices[torch.rand(c.indices.shape, generator=g) < 0.3] = -1
    c.indices[1, 5] = 400
    c.indices[3, :] = -1
    cache = _pack(bits(c.kv_src), width=672)
    cache[:, 656:] = 0x7F                               # padding bytes (NaN codes) must not be read
    for entry in ("prefill", "decode"):
        out, lse, _ = _run(c, cache, 0.1, entry, use_lengths=False)
        assert (out[3].float() == 0).all() and torch.isneginf(lse[3]).all()


def test_packed_group_scale_spread_and_zero_groups():
    say("packed fp8 group scale spread")
    c = I.random_case(T=3, h=64, d_rope=64, topk=128, num_slots=300, seed=99)
    x = c.kv_src.float()
    mult = torch.tensor([2.0 ** -6, 1.0, 2.0 ** 6, 0.0, 2.0 ** 3]).repeat_interleave(128)[:576]
    x = x * mult
    x[::7, 128:256] = 0.0
    c.kv_src = x.to(torch.bfloat16)
    cache = _pack(bits(c.kv_src))
    _, sc, _ = O.unpack_ds_mla(cache)
    assert (sc[:, 3] == 1.0).all()
    for entry in ("prefill", "decode"):       # values up to 2^6 * 4: the stress allowance
        _run(c, cache, 0.05, entry, stress=True)


@pytest.mark.parametrize("alpha", [1.2, 4.0])
def test_packed_large_logit_jump(alpha):
    """alpha = 1.2: the rerun's reference from the flagged pass's row sums;
    alpha = 4: p overflows and a max-only pass finds the maximum."""
    say(f"packed fp8 large logit jump alpha={alpha}")
    c = I.random_case(T=2, h=32, d_rope=64, topk=128, num_slots=256, seed=100)
    for t in range(2):
        s = int(c.indices[t, 100])
        c.kv_src[s] = (c.q[t, 0].float() * alpha).to(torch.bfloat16)
    cache = _pack(bits(c.kv_src))
    for entry in ("prefill", "decode"):       # a row of 4 q (values to ~16): the stress allowance
        _run(c, cache, 0.1, entry, stress=True)


# ---------------------------------------------------------------------------
# the long-context decode workload on packed rows, full size, every token
# ---------------------------------------------------------------------------

POOL = 65536


def _distinct_packed_copies(pc: np.ndarray, reps: int) -> np.ndarray:
    """Copy k of the packed pool: the latent codes of every 128-channel group
    and the 64 bf16 rope channels rotated by k (the group scales stay right),
    so no two slots a multiple of the pool apart hold the same row."""
    P = pc.shape[0]
    out = np.empty((reps * P, pc.shape[1]), np.uint8)
    rope = np.ascontiguousarray(pc[:, O.DS_MLA_ROPE_AT:O.DS_MLA_ROW_BYTES]).view(np.uint16)
    for k in range(reps):
        dst = out[k * P:(k + 1) * P]
        dst[:] = pc
        for c0 in range(0, 512, 128):
            dst[:, c0:c0 + 128] = np.roll(pc[:, c0:c0 + 128], k, axis=1)
        dst[:, O.DS_MLA_ROPE_AT:O.DS_MLA_ROW_BYTES] = np.roll(rope, k, axis=1).view(np.uint8)
    return out


def test_longctx_ds_mla_full_size():
    """256 tokens x h=128, 64 requests x 65536 context on packed rows (copies
    of a packed pool of 65536 rows, each copy rotated inside its groups),
    request-local indices through a random block table, every token checked,
    in the benchmark's launch configuration; the fused conversion must give
    the same bits."""
    spec = I.SPECS["longctx_ds_mla"]
    w = I.generate(spec, with_values=False)
    pool = I.normal_bf16_rows(POOL, spec.d, spec.seed, 1)
    q = I.normal_bf16_rows(spec.num_tokens * spec.heads, spec.d, spec.seed, 2).view(
        spec.num_tokens, spec.heads, spec.d)
    pc = _pack(bits(pool))
    reps = spec.num_slots // POOL
    codes = _distinct_packed_copies(pc, reps)
    assert not (codes[:POOL] == codes[POOL:2 * POOL]).all(axis=1).any()
    kv = torch.from_numpy(codes).to(DEV).view(spec.num_blocks, I.BLOCK_SIZE, O.DS_MLA_ROW_BYTES)
    gidx, vcnt = smla.convert_indices(w.req_id.to(DEV), w.block_table.to(DEV), w.topk_local.to(DEV))
    say("packed fp8 full size longctx_ds_mla")
    out, lse = _attend("decode", q, kv, gidx, spec.softmax_scale, vcnt)
    go, vo = O.convert_indices(w.req_id.numpy(), w.block_table.numpy(), w.topk_local.numpy(), I.BLOCK_SIZE)
    assert (gidx.cpu().numpy() == go).all()
    ref = oracle_for(q, codes, go, spec.softmax_scale, vo, kv_format=FMT)
    err, lerr = compare(out, lse, ref, "longctx_ds_mla", K_ROUND)
    print(f"longctx_ds_mla full size, every token: out err {err:.2e} lse err {lerr:.2e}")
    say("packed fp8 full size longctx_ds_mla, fused conversion")
    out2, lse2 = _attend("decode", q, kv, w.topk_local.to(DEV), spec.softmax_scale,
                         block_table=w.block_table.to(DEV), req_id=w.req_id.to(DEV), block_size=I.BLOCK_SIZE)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)) and torch.equal(lse, lse2)


# ---------------------------------------------------------------------------
# cache write (bit-exact)
# ---------------------------------------------------------------------------

def _write_case(T, S, seed, kv_c=None, kpe=None, width=O.DS_MLA_ROW_BYTES):
    g = torch.Generator().manual_seed(seed)
    if kv_c is None:
        kv_c = torch.randn((T, 512), generator=g).to(torch.bfloat16)
    if kpe is None:
        kpe = torch.randn((T, 64), generator=g).to(torch.bfloat16)
    slots = torch.randperm(S, generator=g)[:T].to(torch.int64)
    slots[torch.rand(T, generator=g) < 0.1] = -1
    init = torch.randint(0, 256, (S, width), generator=g, dtype=torch.int32).to(torch.uint8).numpy().copy()
    cache = torch.from_numpy(init.copy()).to(DEV)
    say(f"packed cache write T={T} width={width}")
    smla.cache_write(kv_c.to(DEV), kpe.to(DEV), slots.to(DEV), cache, FMT)
    torch.cuda.synchronize()
    ref = init.copy()
    O.cache_write(bits(kv_c), bits(kpe), slots.numpy(), FMT, ref)
    got = cache.cpu().numpy()
    assert np.array_equal(got, ref), f"packed rows differ ({int((got != ref).any(1).sum())} rows)"


def test_packed_cache_write_bitexact():
    _write_case(T=300, S=1000, seed=110)
    _write_case(T=40, S=64, seed=111, width=672)                  # padded rows: bytes past 656 untouched


def test_packed_cache_write_special_values():
    """Saturation-free extremes per group (the group scale absorbs them),
    rounding ties, signed zeros, subnormal codes and all-zero groups."""
    T = 64
    g = torch.Generator().manual_seed(112)
    x = torch.randn((T, 576), generator=g)
    x[0, :] = 0.0
    x[1, :] = -0.0
    x[2, :128] = 0.0
    x[3, :] = torch.linspace(-1000.0, 1000.0, 576)
    x[4, :8] = torch.tensor([1.0625, 1.1875, -1.0625, 2.125, 0.0029296875, 0.0009765625, 240.0, 448.0])
    x[5, :] = torch.ldexp(torch.ones(576), torch.randint(-14, -6, (576,), generator=g))
    xb = x.to(torch.bfloat16)
    _write_case(T=T, S=T, seed=113, kv_c=xb[:, :512], kpe=xb[:, 512:])
