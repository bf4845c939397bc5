"""GPU parity of the FP8 E4M3FN cache formats (one per-tensor scale; per-row
x 128-channel-group scales) and of the cache write, against the fp64 oracle.

The FP8 caches fed to the attention tests are made by the oracle's quantizer
(never by the GPU cache write), so every oracle input is independent of the
HIP path. Attention is held to the bar of the bf16 tests (max-abs 1e-2 on the
output before its own bf16 rounding, 1e-3 on the LSE); in the group format
each P term is rounded to bf16 twice (k = 2), and the second rounding is
allowed for (parity_util.compare). The cache write is compared bit for bit."""
import numpy as np
import pytest
import torch

from oracle import e4m3
from oracle import sparse_mla as O
import parity_util as PU
from parity_util import bits, compare, oracle_for, q_f64, say
from sparse_mla_attention_top_amd import inputs as I
from sparse_mla_attention_top_amd import smla

pytestmark = pytest.mark.gpu
DEV = "cuda"
FMTS = [O.KV_FP8_PER_TENSOR, O.KV_FP8_GROUP128]


def _k(kv_format: int) -> int:
    """bf16 roundings of each P term in the P.V sum (2 in the group format)."""
    return 2 if kv_format == O.KV_FP8_GROUP128 else 1


def _quantize(rows_bits: np.ndarray, kv_format: int, k_scale: float = 1.0):
    """Oracle quantizer: (codes [n, D] uint8, group scales [n, G] fp32 or None)."""
    if kv_format == O.KV_FP8_PER_TENSOR:
        return O.quantize_per_tensor(rows_bits, k_scale), None
    return O.quantize_group128(rows_bits)


def _attend(entry, q, codes_dev, scales_dev, kv_format, k_scale, idx_dev, scale, lengths_dev=None,
            num_splits=0, **conv):
    d_rope = q.shape[2] - 512
    qd = q.to(DEV)
    qn, qr = qd[..., :512], (qd[..., 512:] if d_rope else None)
    if entry == "decode":
        out, lse = PU.decode_fwd(qn, qr, codes_dev, idx_dev, scale, kv_format=kv_format,
                                 topk_length=lengths_dev, k_scale=k_scale, group_scales=scales_dev,
                                 num_splits=num_splits, **conv)
    else:
        out, lse = PU.prefill_fwd(qn, qr, codes_dev, idx_dev, scale, kv_format=kv_format,
                                  topk_length=lengths_dev, k_scale=k_scale, group_scales=scales_dev,
                                  return_lse=True, **conv)
    torch.cuda.synchronize()
    return out, lse


def _case(kv_format, T, h, d_rope, topk, num_slots, seed, lengths=None):
    c = I.random_case(T=T, h=h, d_rope=d_rope, topk=topk, num_slots=num_slots, seed=seed, lengths=lengths)
    k_scale = I.per_tensor_scale_from_absmax(c.kv_src) if kv_format == O.KV_FP8_PER_TENSOR else 1.0
    codes, scales = _quantize(bits(c.kv_src), kv_format, k_scale)
    return c, codes, scales, k_scale


def _run_case(kv_format, c, codes, scales, k_scale, scale, entry, use_lengths=True, num_splits=0, stress=False):
    ln = c.lengths if use_lengths else None
    out, lse = _attend(entry, c.q, torch.from_numpy(codes).to(DEV),
                       None if scales is None else torch.from_numpy(scales).to(DEV), kv_format, k_scale,
                       c.indices.to(DEV), scale, None if ln is None else ln.to(DEV), num_splits)
    ref = oracle_for(c.q, codes, c.indices.numpy(), scale, None if ln is None else ln.numpy(),
                     kv_format=kv_format, k_scale=k_scale, group_scales=scales, magnitude=stress or None)
    return out, lse, compare(out, lse, ref, f"fp8 fmt={kv_format} {entry}", _k(kv_format), stress)


# ---------------------------------------------------------------------------
# dequantisation of every code through the whole path
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kv_format,d_rope", [(O.KV_FP8_PER_TENSOR, 0), (O.KV_FP8_GROUP128, 64)])
def test_every_code_single_slot_is_exact(kv_format, d_rope):
    """Token t attends to slot t alone, so its output is that row's latent
    values: with k_scale = 1 (per-tensor) or power-of-two group scales every
    E4M3FN value times its scale is exact in bf16, so the output must equal
    the decoded row bit for bit. Rows cycle through all 254 non-NaN codes."""
    D = 512 + d_rope
    S = 256
    c_idx = (np.arange(S)[:, None] + np.arange(D)[None, :]) % 256
    codes = c_idx.astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00          # no NaN in a cache
    rng = np.random.default_rng(3)
    G = (D + 127) // 128
    scales = None
    if kv_format == O.KV_FP8_GROUP128:
        scales = np.ldexp(1.0, rng.integers(-4, 5, (S, G))).astype(np.float32)
    T, h = S, 16
    g = torch.Generator().manual_seed(4)
    q = torch.randn((T, h, D), generator=g).to(torch.bfloat16)
    idx = torch.full((T, 8), -1, dtype=torch.int32)
    idx[:, 3] = torch.arange(T, dtype=torch.int32)     # one valid entry, not first in its row
    say(f"fp8 every code fmt={kv_format} d_rope={d_rope}")
    for entry in ("prefill", "decode"):
        out, lse = _attend(entry, q, torch.from_numpy(codes).to(DEV),
                           None if scales is None else torch.from_numpy(scales).to(DEV), kv_format, 1.0,
                           idx.to(DEV), 0.05)
        vals = e4m3.decode(codes[:, :512])
        if scales is not None:
            vals = vals * np.repeat(scales.astype(np.float64), 128, axis=1)[:, :512]
        got = out.float().cpu().numpy().astype(np.float64)
        bad = np.argwhere(got != vals[:, None, :])
        if len(bad):
            t, hh, c = bad[0]
            raise AssertionError(f"{entry}: {len(bad)} outputs differ from the decoded row; first token {t} "
                                 f"head {hh} channel {c} code {codes[t, c]:#04x}: {got[t, hh, c]} != {vals[t, c]}")
        ref = oracle_for(q, codes, idx.numpy(), 0.05, kv_format=kv_format, k_scale=1.0, group_scales=scales)
        compare(out, lse, ref, f"every code {entry}", _k(kv_format))


# ---------------------------------------------------------------------------
# small and ragged cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kv_format", FMTS)
@pytest.mark.parametrize("d_rope", [0, 64])
@pytest.mark.parametrize("h", [16, 64, 128])
def test_fp8_heads_formats(kv_format, d_rope, h):
    say(f"fp8 fmt={kv_format} d_rope={d_rope} h={h}")
    c, codes, scales, k_scale = _case(kv_format, T=3, h=h, d_rope=d_rope, topk=200, num_slots=700,
                                      seed=31 + h + d_rope + kv_format, lengths=[200, 77, 129])
    for entry in ("prefill", "decode"):
        _run_case(kv_format, c, codes, scales, k_scale, 192 ** -0.5, entry)


@pytest.mark.parametrize("kv_format", FMTS)
@pytest.mark.parametrize("topk,lengths", [(1, [1, 0]), (33, [33, 32]), (2048, [2048, 1111])])
def test_fp8_topk_widths_and_splits(kv_format, topk, lengths):
    say(f"fp8 fmt={kv_format} topk={topk}")
    c, codes, scales, k_scale = _case(kv_format, T=2, h=128, d_rope=64, topk=topk, num_slots=4096,
                                      seed=topk + kv_format, lengths=lengths)
    _run_case(kv_format, c, codes, scales, k_scale, 192 ** -0.5, "prefill")
    for splits in (1, 3, 8):
        _run_case(kv_format, c, codes, scales, k_scale, 192 ** -0.5, "decode", num_splits=splits)


@pytest.mark.parametrize("kv_format", FMTS)
def test_fp8_scattered_invalid_and_empty_rows(kv_format):
    say(f"fp8 scattered invalid fmt={kv_format}")
    c, codes, scales, k_scale = _case(kv_format, T=4, h=64, d_rope=64, topk=160, num_slots=400, seed=41)
    g = torch.Generator().manual_seed(42)
    c.indices[torch.rand(c.indices.shape, generator=g) < 0.3] = -1
    c.indices[1, 5] = 400
    c.indices[3, :] = -1
    for entry in ("prefill", "decode"):
        out, lse, _ = _run_case(kv_format, c, codes, scales, k_scale, 0.1, entry, use_lengths=False)
        assert (out[3].float() == 0).all() and torch.isneginf(lse[3]).all()


def test_fp8_group_scale_spread_and_zero_groups():
    """Groups of one row with scales far apart (rows multiplied per group by
    2^-6 .. 2^6 before quantising) and all-zero groups (scale 1)."""
    say("fp8 group scale spread")
    c = I.random_case(T=3, h=64, d_rope=64, topk=128, num_slots=300, seed=51)
    x = c.kv_src.float()
    mult = torch.tensor([2.0 ** -6, 1.0, 2.0 ** 6, 0.0, 2.0 ** 3]).repeat_interleave(128)[:576]
    x = x * mult
    x[::7, 128:256] = 0.0
    c.kv_src = x.to(torch.bfloat16)
    codes, scales = _quantize(bits(c.kv_src), O.KV_FP8_GROUP128)
    assert (scales[:, 3] == 1.0).all()
    for entry in ("prefill", "decode"):       # values up to 2^6 * 4: the stress allowance
        _run_case(O.KV_FP8_GROUP128, c, codes, scales, 1.0, 0.05, entry, stress=True)


@pytest.mark.parametrize("alpha", [1.2, 4.0])
@pytest.mark.parametrize("kv_format", FMTS)
def test_fp8_large_logit_jump(kv_format, alpha):
    """alpha = 1.2: a jump of about 90 (base 2), the rerun's reference comes from
    the flagged pass's row sums; alpha = 4: about 330, p overflows and a
    max-only pass finds the maximum."""
    say(f"fp8 large logit jump fmt={kv_format} alpha={alpha}")
    c = I.random_case(T=2, h=32, d_rope=64, topk=128, num_slots=256, seed=61)
    for t in range(2):
        s = int(c.indices[t, 100])
        c.kv_src[s] = (c.q[t, 0].float() * alpha).to(torch.bfloat16)
    k_scale = I.per_tensor_scale_from_absmax(c.kv_src) if kv_format == O.KV_FP8_PER_TENSOR else 1.0
    codes, scales = _quantize(bits(c.kv_src), kv_format, k_scale)
    for entry in ("prefill", "decode"):       # a row of 4 q (values to ~16): the stress allowance
        _run_case(kv_format, c, codes, scales, k_scale, 0.1, entry, stress=True)


# ---------------------------------------------------------------------------
# the two FP8 workloads at full size (cache rows are copies of a quantised
# pool, each copy with the channels of every scale group rotated by its copy
# number, so that no two slots a multiple of the pool apart hold the same row)
# ---------------------------------------------------------------------------

POOL = 65536


def distinct_copies(pool: np.ndarray, reps: int, groups, cols=None) -> np.ndarray:
    """[reps * P, W] array whose copy k (rows kP .. kP + P - 1) is the pool with
    the columns of each (c0, c1) group rotated by k; columns outside every
    group are copied. A rotation inside a scale group keeps the group's scale
    right: copy k holds the quantisation of the pool's rows with their
    channels permuted."""
    P, W = pool.shape
    out = np.empty((reps * P, W), pool.dtype)
    for k in range(reps):
        dst = out[k * P:(k + 1) * P]
        dst[:] = pool
        for c0, c1 in groups:
            dst[:, c0:c1] = np.roll(pool[:, c0:c1], k, axis=1)
    return out


def scale_groups(d: int):
    return [(c0, min(d, c0 + 128)) for c0 in range(0, d, 128)]


def _full_size(name):
    spec = I.SPECS[name]
    w = I.generate(spec, with_values=False)
    pool = I.normal_bf16_rows(POOL, spec.d, spec.seed, 1)
    q = I.normal_bf16_rows(spec.num_tokens * spec.heads, spec.d, spec.seed, 2).view(
        spec.num_tokens, spec.heads, spec.d)
    k_scale = I.per_tensor_scale_from_absmax(pool) if spec.kv_format == O.KV_FP8_PER_TENSOR else 1.0
    pc, ps = _quantize(bits(pool), spec.kv_format, k_scale)
    reps = spec.num_slots // POOL
    assert reps * POOL == spec.num_slots and reps <= 64
    codes = distinct_copies(pc, reps, scale_groups(spec.d))
    scales = None if ps is None else np.tile(ps, (reps, 1))
    assert not (codes[:POOL] == codes[POOL:2 * POOL]).all(axis=1).any()
    kv = torch.from_numpy(codes).to(DEV).view(spec.num_blocks, I.BLOCK_SIZE, spec.d)
    gs = None if scales is None else torch.from_numpy(scales).to(DEV)
    gidx, vcnt = smla.convert_indices(w.req_id.to(DEV), w.block_table.to(DEV), w.topk_local.to(DEV))
    say(f"fp8 full size {name}")
    out, lse = _attend("decode", q, kv, gs, spec.kv_format, k_scale, gidx, spec.softmax_scale, vcnt)
    go, vo = O.convert_indices(w.req_id.numpy(), w.block_table.numpy(), w.topk_local.numpy(), I.BLOCK_SIZE)
    assert (gidx.cpu().numpy() == go).all()
    ref = oracle_for(q, codes, go, spec.softmax_scale, vo, kv_format=spec.kv_format,
                     k_scale=k_scale, group_scales=scales)
    err, lerr = compare(out, lse, ref, name, _k(spec.kv_format))
    print(f"{name} full size, every token: out err {err:.2e} lse err {lerr:.2e}")
    # the same launch with the conversion done by the attention kernel: the
    # same global rows in the same order, so the same bits
    say(f"fp8 full size {name}, fused conversion")
    out2, lse2 = _attend("decode", q, kv, gs, spec.kv_format, k_scale, w.topk_local.to(DEV), spec.softmax_scale,
                         block_table=w.block_table.to(DEV), req_id=w.req_id.to(DEV), block_size=I.BLOCK_SIZE)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)) and torch.equal(lse, lse2)


def test_nope_fp8_full_size():
    """NoPE decode, per-tensor FP8 (128 tokens x h=64, 128 requests x 16384
    context, top-k 2048, valid counts U[512, 2048] with a -1 tail), every
    token, in the benchmark's launch configuration."""
    _full_size("nope_fp8")


def test_longctx_fp8_full_size():
    """Long-context group-scaled FP8 (256 tokens x h=128, D=576, 64 requests x
    65536 context, request-local indices through a random block table), every
    token, in the benchmark's launch configuration."""
    _full_size("longctx_fp8")


# ---------------------------------------------------------------------------
# cache write / quantise (bit-exact)
# ---------------------------------------------------------------------------

def _cache_write_case(kv_format, d_rope, T, S, seed, k_scale=None, kv_c=None, kpe=None, row_pad=0):
    g = torch.Generator().manual_seed(seed)
    if kv_c is None:
        kv_c = torch.randn((T, 512 + row_pad), generator=g).to(torch.bfloat16)[:, :512]
    if kpe is None and d_rope:
        kpe = torch.randn((T, d_rope), generator=g).to(torch.bfloat16)
    slots = torch.randperm(S, generator=g)[:T].to(torch.int64)
    slots[torch.rand(T, generator=g) < 0.1] = -1
    D = 512 + d_rope
    if kv_format == O.KV_BF16:
        init = torch.randint(-32768, 32767, (S, D), generator=g, dtype=torch.int32).to(torch.int16)
        init_np = init.numpy().view(np.uint16).copy()
        cache = init.view(torch.bfloat16).to(DEV)
    else:
        init_np = torch.randint(0, 256, (S, D), generator=g, dtype=torch.int32).to(torch.uint8).numpy().copy()
        cache = torch.from_numpy(init_np.copy()).to(DEV)
    G = (D + 127) // 128
    sc_np = np.full((S, G), -1.0, dtype=np.float32)
    sc = torch.from_numpy(sc_np.copy()).to(DEV) if kv_format == O.KV_FP8_GROUP128 else None
    if k_scale is None:
        k_scale = 1.0
        if kv_format == O.KV_FP8_PER_TENSOR:
            both = kv_c.float() if kpe is None else torch.cat([kv_c.float(), kpe.float()], 1)
            k_scale = I.per_tensor_scale_from_absmax(both)
    say(f"cache write fmt={kv_format} d_rope={d_rope} T={T}")
    smla.cache_write(kv_c.to(DEV), None if kpe is None else kpe.to(DEV), slots.to(DEV), cache, kv_format,
                     k_scale, sc)
    torch.cuda.synchronize()
    ref = init_np.copy()
    O.cache_write(bits(kv_c), None if kpe is None else bits(kpe), slots.numpy(), kv_format, ref, k_scale,
                  sc_np if kv_format == O.KV_FP8_GROUP128 else None)
    got = bits(cache) if kv_format == O.KV_BF16 else cache.cpu().numpy()
    assert np.array_equal(got, ref), f"cache rows differ ({int((got != ref).any(1).sum())} rows)"
    if kv_format == O.KV_FP8_GROUP128:
        gs = sc.cpu().numpy()
        assert np.array_equal(gs.view(np.uint32), sc_np.view(np.uint32)), "group scales differ"


@pytest.mark.parametrize("kv_format", [O.KV_BF16] + FMTS)
@pytest.mark.parametrize("d_rope", [0, 64])
def test_cache_write_bitexact(kv_format, d_rope):
    _cache_write_case(kv_format, d_rope, T=300, S=1000, seed=70 + kv_format + d_rope)


def test_cache_write_strided_rows():
    g = torch.Generator().manual_seed(77)
    base = torch.randn((50, 640), generator=g).to(torch.bfloat16)
    for fmt in [O.KV_BF16] + FMTS:
        _cache_write_case(fmt, 64, T=50, S=64, seed=78, kv_c=base[:, :512], kpe=base[:, 576:640])


@pytest.mark.parametrize("kv_format", FMTS)
def test_cache_write_special_values(kv_format):
    """Saturation (|x / scale| above 448), rounding ties, signed zeros,
    E4M3 subnormals and all-zero groups."""
    T = 64
    x = torch.zeros((T, 576), dtype=torch.float32)
    g = torch.Generator().manual_seed(80)
    x[:] = torch.randn((T, 576), generator=g)
    x[0, :] = 0.0
    x[1, :] = -0.0
    x[2, :128] = 0.0                                    # one all-zero group
    x[3, :] = torch.linspace(-1000.0, 1000.0, 576)      # beyond 448 at k_scale 1
    # exact midpoints between neighbouring E4M3 values (1 + 1/16 = halfway 1 .. 1.125)
    x[4, :8] = torch.tensor([1.0625, 1.1875, -1.0625, 2.125, 0.0029296875, 0.0009765625, 240.0, 464.0])
    x[5, :] = torch.ldexp(torch.ones(576), torch.randint(-14, -6, (576,), generator=g))  # subnormal range
    xb = x.to(torch.bfloat16)
    _cache_write_case(kv_format, 64, T=T, S=T, seed=81, k_scale=1.0, kv_c=xb[:, :512], kpe=xb[:, 512:])
