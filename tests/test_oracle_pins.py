"""Pins of the fp64 oracle against facts that do not come from the oracle itself:
the pages' worked examples, library routines, closed forms, invariants and
brute force on tiny inputs. CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import e4m3
from oracle import sparse_mla as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x_f32: torch.Tensor) -> np.ndarray:
    """bf16 bit patterns of fp32 values rounded by torch."""
    return x_f32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rand_bf16(rng, shape):
    return _bits(torch.from_numpy(rng.standard_normal(shape).astype(np.float32)))


# ---------------------------------------------------------------------------
# index conversion
# ---------------------------------------------------------------------------

def test_convert_worked_examples():
    cases = json.load(open(os.path.join(GOLDEN, "convert_examples.json")))
    for c in cases["cases"]:
        g, v = O.convert_indices(np.array(c["req_id"]), np.array(c["block_table"]),
                                 np.array(c["topk_local"]), c["block_size"])
        assert g.tolist() == c["expect_global"], c["name"]
        assert v.tolist() == c["expect_valid"], c["name"]


def test_convert_valid_count_case():
    c = json.load(open(os.path.join(GOLDEN, "convert_examples.json")))["valid_count_case"]
    rng = np.random.default_rng(25)
    T, K, NB, B = c["T"], c["topk"], c["num_blocks"], c["block_size"]
    loc = np.full((T, K), -1, dtype=np.int32)
    for i, nv in enumerate(c["expect_valid"]):
        loc[i, :nv] = rng.integers(0, NB * B, nv)
    g, v = O.convert_indices(np.zeros(T, np.int32), np.arange(NB)[None], loc, B)
    assert v.tolist() == c["expect_valid"]
    for i, nv in enumerate(c["expect_valid"]):
        assert (g[i, nv:] == -1).all()
        assert (g[i, :nv] == loc[i, :nv]).all()     # identity table


def test_convert_brute_force_random_tables():
    """Pure-Python per-entry evaluation, including invalid corners: negative
    entries, local indices past the table, negative table entries."""
    rng = np.random.default_rng(7)
    R, MB, B, T, K = 3, 5, 16, 6, 12
    bt = rng.permutation(R * MB).reshape(R, MB).astype(np.int32)
    bt[1, 2] = -1
    req = rng.integers(0, R, T).astype(np.int32)
    loc = rng.integers(-3, MB * B + 10, (T, K)).astype(np.int32)
    for stride in (B, 2 * B):
        g, v = O.convert_indices(req, bt, loc, B, stride)
        for t in range(T):
            cnt = 0
            for j in range(K):
                l = int(loc[t, j])
                if l < 0 or l // B >= MB or bt[req[t], l // B] < 0:
                    want = -1
                else:
                    want = int(bt[req[t], l // B]) * stride + l % B
                    cnt += 1
                assert g[t, j] == want
            assert v[t] == cnt


# ---------------------------------------------------------------------------
# E4M3FN format and quantizer
# ---------------------------------------------------------------------------

def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.DECODE_TABLE
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert (ours[~nan] == ref[~nan]).all()
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x38] == 1.0


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(3)
    y = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 40,
        rng.uniform(-447.9, 447.9, 50000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-3).astype(np.float32),
        # exact midpoints between neighbouring codes (ties to even)
        ((e4m3.DECODE_TABLE[1:0x7E] + e4m3.DECODE_TABLE[2:0x7F]) / 2).astype(np.float32),
        e4m3.DECODE_TABLE[:0x7F].astype(np.float32),
    ])
    ours = e4m3.encode_rne(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (ours == ref).all()


def test_e4m3_encode_saturates_and_nan():
    y = np.array([448.0, 449.0, 463.9, 464.0, 1e6, np.inf, -1e6, -np.inf, np.nan], np.float32)
    c = e4m3.encode_rne(y)
    assert c[:6].tolist() == [0x7E] * 6
    assert c[6:8].tolist() == [0xFE] * 2
    assert c[8] & 0x7F == 0x7F


def test_group_quantizer_roundtrip_bound():
    """Every group's absmax element lands on +-448 and the decoded value is
    within half an E4M3 ulp of x / scale."""
    rng = np.random.default_rng(11)
    x = _rand_bf16(rng, (64, 576))
    codes, sc = O.quantize_group128(x)
    assert sc.shape == (64, 5)
    xf = O.bf16_bits_to_f32(x).astype(np.float64)
    dec = e4m3.decode(codes)
    for g in range(5):
        c0, c1 = 128 * g, min(576, 128 * g + 128)
        amax = np.abs(xf[:, c0:c1]).max(axis=1)
        assert np.allclose(sc[:, g], (amax / 448.0).astype(np.float32), rtol=0, atol=0)
        y = xf[:, c0:c1] / sc[:, g:g + 1]
        assert (np.abs(dec[:, c0:c1]).max(axis=1) == 448.0).all()
        # relative spacing of E4M3 normals is 1/8 -> error <= 1/16 relative (+ subnormal floor)
        err = np.abs(dec[:, c0:c1] - y)
        assert (err <= np.abs(y) / 16 + 2.0 ** -10 + 1e-12).all()


def test_group_quantizer_zero_group_scale_is_one():
    x = np.zeros((2, 512), np.uint16)
    codes, sc = O.quantize_group128(x)
    assert (sc == 1.0).all() and (codes == 0).all()


def _division_ties(rng, n: int):
    """(bf16 bits x, fp32 scales s) such that fl32(x / s) is exactly the midpoint
    of two neighbouring E4M3 values while the exact quotient is not: a quantizer
    that rounds the exact (fp64) quotient goes to the nearer code, one that
    divides in fp32 takes the tie to the even code. Built as s = fl32(x / m)
    for random bf16 x and midpoints m, keeping the pairs with that property."""
    mids = ((e4m3.DECODE_TABLE[8:0x7D] + e4m3.DECODE_TABLE[9:0x7E]) / 2)
    xb = _rand_bf16(rng, (20000,))
    x32 = O.bf16_bits_to_f32(xb)
    m = rng.choice(mids, 20000) * np.sign(x32)
    s = (x32 / m.astype(np.float32)).astype(np.float32)
    ok = (s > 0) & np.isfinite(s)
    q32 = (x32 / np.where(ok, s, 1)).astype(np.float32)
    exact = x32.astype(np.float64) / np.where(ok, s, 1).astype(np.float64)
    ok &= (q32.astype(np.float64) == m) & (exact != m)
    idx = np.nonzero(ok)[0][:n]
    assert idx.size == n
    return xb[idx], s[idx]


def _torch_codes(x_bits: np.ndarray, s) -> np.ndarray:
    """torch: fp32 x / fp32 scale, cast to float8_e4m3fn."""
    q = torch.from_numpy(O.bf16_bits_to_f32(x_bits)) / torch.as_tensor(np.asarray(s, np.float32))
    return q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _nearest_code_f64(v: np.ndarray) -> np.ndarray:
    """E4M3FN code nearest to each fp64 value (ties to even), no fp32 step."""
    pos = e4m3.DECODE_TABLE[:0x7F]
    a = np.minimum(np.abs(v), 448.0)
    hi = np.clip(np.searchsorted(pos, a), 1, 0x7E)
    lo = hi - 1
    dl, dh = a - pos[lo], pos[hi] - a
    code = np.where((dh < dl) | ((dh == dl) & (hi % 2 == 0)), hi, lo)
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def test_per_tensor_quantizer_matches_torch():
    """The per-tensor quantizer against torch: (x_fp32 / k_scale) in fp32, then
    torch's cast to float8_e4m3fn (round to nearest even), for quotients up to
    464 where torch saturates to 448 as well; beyond that torch gives NaN and
    the oracle saturates at +-448 (checked apart). Scales of the workloads'
    absmax / 448 kind and quotients that land exactly on an E4M3 tie in fp32
    (but not in exact arithmetic) are included, so a quantizer that multiplies
    by the scale or divides in fp64 fails."""
    rng = np.random.default_rng(21)
    x = _rand_bf16(rng, (256, 576))
    for k_scale in (float(np.float32(np.abs(O.bf16_bits_to_f32(x)).max() / np.float32(448))),
                    0.0123, 1.0, 3.0e-3):
        ref = (torch.from_numpy(O.bf16_bits_to_f32(x)) / torch.tensor(k_scale, dtype=torch.float32))
        inside = ref.abs() <= 464
        ours = O.quantize_per_tensor(x, k_scale)
        theirs = ref.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert (ours[inside.numpy()] == theirs[inside.numpy()]).all(), k_scale
        if (~inside).any():
            out = ours[~inside.numpy()]
            assert ((out & 0x7F) == 0x7E).all()
            assert ((out >> 7) == (ref[~inside].numpy() < 0)).all()
    xt, st = _division_ties(rng, 64)
    ours = np.array([O.quantize_per_tensor(np.array([[xb]], np.uint16), float(sc))[0, 0] for xb, sc in zip(xt, st)])
    assert (ours == _torch_codes(xt, st)).all()
    assert (ours % 2 == 0).all()                      # every one of them a tie, taken to the even code


def test_per_tensor_quantizer_planted_mistakes_are_caught(monkeypatch):
    """A quantizer that multiplies by the scale, or divides in fp64, disagrees
    with torch on the pin's inputs."""
    rng = np.random.default_rng(22)
    x = _rand_bf16(rng, (64, 512))
    ks = 0.0123
    theirs = (torch.from_numpy(O.bf16_bits_to_f32(x)) / torch.tensor(ks, dtype=torch.float32)
              ).to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    def times_scale(x_bits, k_scale):
        return e4m3.encode_rne((O.bf16_bits_to_f32(x_bits) * np.float32(k_scale)).astype(np.float32))

    assert not (times_scale(x, ks) == theirs).all()
    xt, st = _division_ties(rng, 64)
    fp64 = _nearest_code_f64(O.bf16_bits_to_f64(xt) / st.astype(np.float64))
    assert (fp64 != _torch_codes(xt, st)).any()


def test_cache_write_bf16_roundtrip_and_skip():
    """Cache write then read back equals the written rows, negative slots are
    skipped (branch diff, test_kv_cache_write_read_consistency)."""
    rng = np.random.default_rng(5)
    S, T = 16, 5
    kv_c, k_pe = _rand_bf16(rng, (T, 512)), _rand_bf16(rng, (T, 64))
    slots = np.array([3, -1, 0, 15, 7])
    cache = np.zeros((S, 576), np.uint16)
    O.cache_write(kv_c, k_pe, slots, O.KV_BF16, cache)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        assert (cache[s, :512] == kv_c[t]).all() and (cache[s, 512:] == k_pe[t]).all()
    untouched = [s for s in range(S) if s not in slots]
    assert (cache[untouched] == 0).all()


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _setup(rng, T=3, h=4, D=576, S=200, K=40):
    q = O.bf16_bits_to_f64(_rand_bf16(rng, (T, h, D)))
    cache = _rand_bf16(rng, (S, D))
    idx = np.stack([rng.permutation(S)[:K] for _ in range(T)]).astype(np.int32)
    return q, cache, idx


def test_dense_special_case_matches_sdpa():
    """Index rows listing every context slot = dense attention (the pages'
    kernel tests use SDPA as the reference)."""
    rng = np.random.default_rng(1)
    T, h, D, S = 2, 8, 576, 96
    q = O.bf16_bits_to_f64(_rand_bf16(rng, (T, h, D)))
    cache = _rand_bf16(rng, (S, D))
    idx = np.stack([rng.permutation(S) for _ in range(T)]).astype(np.int32)
    out, lse = O.attention(q, cache, O.KV_BF16, idx, 0.07)
    kv = torch.from_numpy(O.bf16_bits_to_f64(cache))
    for t in range(T):
        qt = torch.from_numpy(q[t])[None, :, None, :]             # [1, h, 1, D]
        k = kv[None, None].expand(1, h, S, D)
        v = kv[None, None, :, :512].expand(1, h, S, 512)
        ref = F.scaled_dot_product_attention(qt, k, v, scale=0.07)[0, :, 0]
        assert np.abs(out[t] - ref.numpy()).max() < 1e-12
        ref_lse = torch.logsumexp(0.07 * (torch.from_numpy(q[t]) @ kv.T), dim=-1)
        assert np.abs(lse[t] - ref_lse.numpy()).max() < 1e-12


def test_magnitude_is_sdpa_over_absolute_values():
    """sum_j p_j |v_j|: dense attention (SDPA) with the value rows replaced by
    their absolute values and the same weights; equals the output where every
    value is >= 0 and bounds |out| everywhere."""
    rng = np.random.default_rng(21)
    T, h, D, S = 2, 8, 576, 80
    q = O.bf16_bits_to_f64(_rand_bf16(rng, (T, h, D)))
    cache = _rand_bf16(rng, (S, D))
    idx = np.stack([rng.permutation(S) for _ in range(T)]).astype(np.int32)
    out, lse, mag = O.attention_with_magnitude(q, cache, O.KV_BF16, idx, 0.07)
    out2, lse2 = O.attention(q, cache, O.KV_BF16, idx, 0.07)
    assert (out == out2).all() and (lse == lse2).all()
    kv = torch.from_numpy(O.bf16_bits_to_f64(cache))
    for t in range(T):
        qt = torch.from_numpy(q[t])[None, :, None, :]
        k = kv[None, None].expand(1, h, S, D)
        v = kv[None, None, :, :512].abs().expand(1, h, S, 512)
        ref = F.scaled_dot_product_attention(qt, k, v, scale=0.07)[0, :, 0]
        assert np.abs(mag[t] - ref.numpy()).max() < 1e-12
    assert (mag >= np.abs(out) - 1e-12).all()
    pos = O.bf16_bits_to_f64(cache)
    pos_bits = _bits(torch.from_numpy(np.abs(pos).astype(np.float32)))
    o3, _, m3 = O.attention_with_magnitude(q, pos_bits, O.KV_BF16, idx, 0.07)
    assert np.abs(o3 - m3).max() < 1e-12
    e_o, e_l, e_m = O.attention_with_magnitude(q, cache, O.KV_BF16, np.full((T, 4), -1, np.int32), 0.07)
    assert (e_m == 0).all() and (e_o == 0).all() and np.isneginf(e_l).all()


def test_permutation_invariance():
    rng = np.random.default_rng(2)
    q, cache, idx = _setup(rng)
    out, lse = O.attention(q, cache, O.KV_BF16, idx, 0.05)
    perm = np.stack([rng.permutation(row) for row in idx])
    out2, lse2 = O.attention(q, cache, O.KV_BF16, perm, 0.05)
    assert np.abs(out - out2).max() < 1e-12 and np.abs(lse - lse2).max() < 1e-12


def test_single_valid_slot_is_that_row():
    rng = np.random.default_rng(3)
    q, cache, idx = _setup(rng)
    idx[:, 1:] = -1
    out, lse = O.attention(q, cache, O.KV_BF16, idx, 0.05)
    for t in range(q.shape[0]):
        row = O.bf16_bits_to_f64(cache[idx[t, 0]])
        assert (out[t] == row[None, :512]).all()
        assert np.allclose(lse[t], 0.05 * q[t] @ row, rtol=0, atol=1e-12)


def test_lse_closed_forms():
    rng = np.random.default_rng(4)
    q, cache, idx = _setup(rng, K=10)
    # all entries the same slot: lse = s + ln v, out = that row
    same = np.repeat(idx[:, :1], 10, axis=1)
    out, lse = O.attention(q, cache, O.KV_BF16, same, 0.05)
    for t in range(q.shape[0]):
        row = O.bf16_bits_to_f64(cache[same[t, 0]])
        assert np.allclose(lse[t], 0.05 * q[t] @ row + math.log(10), atol=1e-12)
        assert np.allclose(out[t], row[None, :512], atol=1e-12)
    # small logits: ln sum exp without max subtraction
    out, lse = O.attention(q, cache, O.KV_BF16, idx, 1e-3)
    for t in range(q.shape[0]):
        rows = O.bf16_bits_to_f64(cache[idx[t]])
        direct = np.log(np.exp(1e-3 * q[t] @ rows.T).sum(axis=1))
        assert np.abs(lse[t] - direct).max() < 1e-12


def test_minus_one_insensitivity_and_length_bound():
    rng = np.random.default_rng(5)
    q, cache, idx = _setup(rng, K=20)
    out, lse = O.attention(q, cache, O.KV_BF16, idx, 0.05)
    # scatter -1 (and other negatives, and out-of-range slots) between entries
    wide = np.full((idx.shape[0], 50), -1, np.int32)
    for t in range(idx.shape[0]):
        pos = np.sort(rng.choice(50, 20, replace=False))
        wide[t, pos] = idx[t]
        holes = np.setdiff1d(np.arange(50), pos)
        wide[t, holes[:3]] = [-7, 10 ** 6, cache.shape[0]]
    out2, lse2 = O.attention(q, cache, O.KV_BF16, wide, 0.05)
    assert np.abs(out - out2).max() < 1e-12 and np.abs(lse - lse2).max() < 1e-12
    # a row length bounds the scan: the tail past it is ignored whatever it holds
    tail = np.concatenate([idx, idx[:, :5]], axis=1)
    out3, lse3 = O.attention(q, cache, O.KV_BF16, tail, 0.05,
                             topk_length=np.full(idx.shape[0], 20))
    assert np.abs(out - out3).max() < 1e-12 and np.abs(lse - lse3).max() < 1e-12


def test_empty_row_is_merge_identity():
    rng = np.random.default_rng(6)
    q, cache, idx = _setup(rng)
    idx[1, :] = -1
    out, lse = O.attention(q, cache, O.KV_BF16, idx, 0.05, topk_length=np.array([40, 40, 0]))
    assert (out[1] == 0).all() and np.isneginf(lse[1]).all()
    assert (out[2] == 0).all() and np.isneginf(lse[2]).all()
    assert np.isfinite(lse[0]).all()


def test_brute_force_tiny():
    """Nested Python loops over the definition softmax_j = exp(s_j)/sum exp(s)."""
    rng = np.random.default_rng(8)
    for h, K in ((1, 1), (2, 5), (2, 8)):
        T, D, S = 2, 576, 30
        q, cache, idx = _setup(rng, T=T, h=h, D=D, S=S, K=K)
        idx[0, -1] = -1
        out, lse = O.attention(q, cache, O.KV_BF16, idx, 0.04)
        kv = O.bf16_bits_to_f64(cache)
        for t in range(T):
            for i in range(h):
                ss = []
                for j in range(K):
                    g = int(idx[t, j])
                    if g < 0:
                        continue
                    ss.append((0.04 * sum(q[t, i, d] * kv[g, d] for d in range(D)), g))
                if not ss:
                    assert np.isneginf(lse[t, i]) and (out[t, i] == 0).all()
                    continue
                tot = sum(math.exp(s) for s, _ in ss)
                assert abs(lse[t, i] - math.log(tot)) < 1e-10
                for c in range(0, 512, 37):
                    want = sum(math.exp(s) * kv[g, c] for s, g in ss) / tot
                    assert abs(out[t, i, c] - want) < 1e-10


def test_heads_are_independent():
    """A subset of heads gives the same result as the full set (head padding
    with zero rows only adds heads that are then dropped)."""
    rng = np.random.default_rng(9)
    q, cache, idx = _setup(rng, h=6)
    out, lse = O.attention(q, cache, O.KV_BF16, idx, 0.05)
    out2, lse2 = O.attention(q[:, 2:5], cache, O.KV_BF16, idx, 0.05)
    assert (out[:, 2:5] == out2).all() and (lse[:, 2:5] == lse2).all()
    qp = np.concatenate([q, np.zeros((q.shape[0], 58, q.shape[2]))], axis=1)
    out3, lse3 = O.attention(qp, cache, O.KV_BF16, idx, 0.05)
    assert (out3[:, :6] == out).all() and (lse3[:, :6] == lse).all()


def test_split_merge_identity():
    rng = np.random.default_rng(10)
    q, cache, idx = _setup(rng, K=40)
    out, lse = O.attention(q, cache, O.KV_BF16, idx, 0.05)
    parts_o, parts_l = [], []
    for a, b in ((0, 7), (7, 7), (7, 30), (30, 40)):     # includes an empty slice
        sl = np.full_like(idx, -1)
        sl[:, a:b] = idx[:, a:b]
        o, l = O.attention(q, cache, O.KV_BF16, sl, 0.05)
        parts_o.append(o)
        parts_l.append(l)
    mo, ml = O.merge_partials(np.stack(parts_o), np.stack(parts_l))
    assert np.abs(mo - out).max() < 1e-12 and np.abs(ml - lse).max() < 1e-12
    eo, el = O.merge_partials(np.zeros((2, 1, 3)), np.full((2, 1), -np.inf))
    assert (eo == 0).all() and np.isneginf(el).all()


# ---------------------------------------------------------------------------
# context-parallel (DCP) shard filter and merge
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("W,I", [(1, 1), (2, 1), (3, 2), (4, 64), (8, 16)])
def test_dcp_placement_partitions_positions(W, I):
    """Every position is stored by exactly one rank, and each rank's local
    positions of a request's first N tokens are exactly 0 .. N_r - 1 in
    token order (no gap, no collision)."""
    for N in (1, 7, 63, 64, 65, 300, 1000):
        pos = np.arange(N)
        rank, local = O.dcp_owner_local(pos, W, I)
        assert ((rank >= 0) & (rank < W)).all()
        total = 0
        for r in range(W):
            lr = local[rank == r]
            assert lr.tolist() == list(range(lr.size))          # in order, dense
            total += lr.size
        assert total == N


def test_dcp_single_rank_is_plain_conversion():
    rng = np.random.default_rng(21)
    R, MB, B, T, K = 3, 9, 16, 13, 70
    bt = rng.permutation(R * MB).reshape(R, MB).astype(np.int32)
    req = rng.integers(0, R, T)
    loc = rng.integers(-2, MB * B + 4, (T, K))
    for I in (1, 5, 64):
        g1, v1 = O.dcp_filter_convert(req, bt, loc, 1, 0, I, B)
        g0, v0 = O.convert_indices(req, bt, loc, B)
        assert (g1 == g0).all() and (v1 == v0).all()


def test_dcp_ranks_split_the_valid_entries_and_compaction_keeps_order():
    rng = np.random.default_rng(22)
    W, I, R, MB, B, T, K = 4, 3, 2, 12, 16, 9, 50
    req = rng.integers(0, R, T)
    loc = rng.integers(-1, W * MB * B, (T, K))
    counts = np.zeros(T, dtype=np.int64)
    for r in range(W):
        bt = rng.permutation(R * MB).reshape(R, MB).astype(np.int32)
        g, v = O.dcp_filter_convert(req, bt, loc, W, r, I, B)
        gc, vc = O.dcp_filter_convert(req, bt, loc, W, r, I, B, compact_valid_to_front=True)
        assert (v == vc).all()
        for t in range(T):
            assert gc[t, :v[t]].tolist() == g[t][g[t] >= 0].tolist() and (gc[t, v[t]:] == -1).all()
        counts += v
    # every non-negative position inside the tables is valid on exactly one rank
    assert (counts == (loc >= 0).sum(axis=1)).all()


def test_dcp_sharded_attention_merges_to_the_whole():
    """A request's cache spread over W ranks by the placement, each rank's
    attention over its filtered indices, merged by LSE: the unsharded result
    (rows a rank does not see come out as the merge identity (0, -inf))."""
    rng = np.random.default_rng(23)
    W, I, B, N, T, h, K, scale = 3, 4, 8, 200, 5, 4, 48, 0.07
    rows = _rand_bf16(rng, (N, 576))                       # token position p -> row
    q = O.bf16_bits_to_f64(_rand_bf16(rng, (T, h, 576)))
    topk = np.stack([rng.permutation(N)[:K] for _ in range(T)])
    topk[1, 10:] = -1
    topk[2, :] = I * np.arange(K) * W % N                  # only rank 0's runs ...
    topk[2] = np.where(topk[2] // I % W == 0, topk[2], -1)  # ... so ranks 1, 2 see an empty row
    req = np.zeros(T, dtype=np.int64)
    whole_bt = np.arange((N + B - 1) // B, dtype=np.int32)[None]
    whole_cache = np.zeros((whole_bt.size * B, 576), dtype=np.uint16)
    whole_cache[:N] = rows
    g, _ = O.convert_indices(req, whole_bt, topk, B)
    out, lse = O.attention(q, whole_cache, O.KV_BF16, g, scale)
    rank, local = O.dcp_owner_local(np.arange(N), W, I)
    parts_o, parts_l = [], []
    for r in range(W):
        n_r = int((rank == r).sum())
        nb = (n_r + B - 1) // B
        bt = rng.permutation(nb + 2)[:nb].astype(np.int32)[None]      # scattered blocks
        cache_r = np.zeros(((nb + 2) * B, 576), dtype=np.uint16)
        for p in np.nonzero(rank == r)[0]:
            cache_r[bt[0, local[p] // B] * B + local[p] % B] = rows[p]
        g_r, _ = O.dcp_filter_convert(req, bt, topk, W, r, I, B)
        o, l = O.attention(q, cache_r, O.KV_BF16, g_r, scale)
        if r > 0:
            assert (o[2] == 0).all() and np.isneginf(l[2]).all()
        parts_o.append(o)
        parts_l.append(l)
    mo, ml = O.merge_partials(np.stack(parts_o), np.stack(parts_l))
    assert np.abs(mo - out).max() < 1e-12 and np.abs(ml - lse).max() < 1e-12


def test_fp8_per_tensor_dequant_is_code_times_scale():
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 256, (8, 512)).astype(np.uint8)
    codes[codes & 0x7F == 0x7F] = 0
    v = O.dequantize_rows(codes, O.KV_FP8_PER_TENSOR, np.arange(8), k_scale=0.01)
    ref = codes.view(np.uint8)
    ref = torch.from_numpy(ref).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert (v == ref * float(np.float32(0.01))).all()


def test_fp8_group_dequant_uses_row_group_scale():
    rng = np.random.default_rng(13)
    codes = rng.integers(0, 0x7E, (6, 576)).astype(np.uint8)
    scales = rng.uniform(0.001, 0.02, (10, 5)).astype(np.float32)
    slots = np.array([9, 0, 4])
    v = O.dequantize_rows(np.concatenate([codes, codes[:4]]), O.KV_FP8_GROUP128, slots,
                          group_scales=scales)
    full = np.concatenate([codes, codes[:4]])
    for r, s in enumerate(slots):
        for c in (0, 127, 128, 300, 511, 512, 575):
            assert v[r, c] == e4m3.DECODE_TABLE[full[s, c]] * float(scales[s, c // 128])


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
# ---------------------------------------------------------------------------

def test_planted_mistakes_are_caught(monkeypatch):
    rng = np.random.default_rng(14)
    q, cache, idx = _setup(rng, T=1, h=2, K=6)
    kv = O.bf16_bits_to_f64(cache)

    def brute(t, i):
        ss = [(0.05 * float(q[t, i] @ kv[g]), g) for g in idx[t] if g >= 0]
        tot = sum(math.exp(s) for s, _ in ss)
        return math.log(tot), sum(math.exp(s) * kv[g, :512] for s, g in ss) / tot

    good_out, good_lse = O.attention(q, cache, O.KV_BF16, idx, 0.05)
    bl, bo = brute(0, 1)
    assert abs(good_lse[0, 1] - bl) < 1e-10 and np.abs(good_out[0, 1] - bo).max() < 1e-10

    real = O.attention_rows

    def no_max_in_lse(q_t, rows, scale, d_v=512, magnitude=False, *opts):   # dropped term
        o, l = real(q_t, rows, scale, d_v)
        s = scale * (q_t @ rows.T)
        return o, l - s.max(axis=1)

    def rope_dropped(q_t, rows, scale, d_v=512, magnitude=False, *opts):     # wrong channel range
        return real(q_t[:, :512], rows[:, :512], scale, d_v)

    for bad in (no_max_in_lse, rope_dropped):
        monkeypatch.setattr(O, "attention_rows", bad)
        o, l = O.attention(q, cache, O.KV_BF16, idx, 0.05)
        assert abs(l[0, 1] - bl) > 1e-6 or np.abs(o[0, 1] - bo).max() > 1e-6
        monkeypatch.setattr(O, "attention_rows", real)


# ---------------------------------------------------------------------------
# packed 656-byte FP8 rows (layout read from the size: 512 codes, 4 fp32
# group scales, 64 bf16 rope channels)
# ---------------------------------------------------------------------------

def test_ds_mla_hand_built_row():
    """A row assembled byte by byte decodes to the values worked out by hand."""
    import struct
    row = bytearray(656)
    row[0] = 0x38            # 1.0      (group 0)
    row[127] = 0xC0          # -2.0     (group 0)
    row[128] = 0x7E          # 448      (group 1)
    row[300] = 0x01          # 2^-9     (group 2)
    row[511] = 0x30          # 0.5      (group 3)
    row[512:528] = struct.pack("<4f", 0.5, 0.25, 2.0, 8.0)
    row[528:530] = bytes([0x80, 0x3F])    # rope channel 0 = bf16 1.0
    row[654:656] = bytes([0x40, 0xC0])    # rope channel 63 = bf16 -3.0
    cache = np.zeros((3, 656), np.uint8)
    cache[2] = np.frombuffer(bytes(row), np.uint8)
    v = O.dequantize_rows(cache, O.KV_FP8_DS_MLA, np.array([2, 0]))
    assert v.shape == (2, 576)
    expect = np.zeros(576)
    expect[0], expect[127], expect[128], expect[300], expect[511] = 0.5, -1.0, 112.0, 2.0 ** -8, 4.0
    expect[512], expect[575] = 1.0, -3.0
    assert (v[0] == expect).all()
    assert (v[1] == 0).all()
    assert O.DS_MLA_ROW_BYTES == 512 + 4 * 4 + 64 * 2 == 656   # the pages' bytes per token


def test_ds_mla_cache_write_roundtrip():
    """Packed write then read back: latent within half an E4M3 step of x per
    group scale (each group's absmax lands on +-448 scale), rope exact,
    negative slots skipped, bytes past 656 untouched."""
    rng = np.random.default_rng(21)
    T = 40
    kv_c = _rand_bf16(rng, (T, 512))
    k_pe = _rand_bf16(rng, (T, 64))
    kv_c[3, 128:256] = 0                                  # an all-zero group
    slots = rng.permutation(64)[:T].astype(np.int64)
    slots[5] = -1
    cache = np.full((64, 672), 0xAB, np.uint8)
    O.cache_write(kv_c, k_pe, slots, O.KV_FP8_DS_MLA, cache)
    keep = slots >= 0
    assert (cache[:, 656:] == 0xAB).all()
    untouched = np.setdiff1d(np.arange(64), slots[keep])
    assert (cache[untouched] == 0xAB).all()
    v = O.dequantize_rows(cache, O.KV_FP8_DS_MLA, slots[keep])
    x = O.bf16_bits_to_f64(np.concatenate([kv_c, k_pe], axis=1))[keep]
    assert (v[:, 512:] == x[:, 512:]).all()
    codes, sc, rope = O.unpack_ds_mla(cache[slots[keep]])
    for g in range(4):
        c0, c1 = 128 * g, 128 * g + 128
        amax = np.abs(x[:, c0:c1]).max(axis=1)
        expect_sc = np.where(amax == 0, 1.0, (amax / 448.0).astype(np.float32))
        assert (sc[:, g] == expect_sc.astype(np.float32)).all()
        y = x[:, c0:c1] / sc[:, g:g + 1].astype(np.float64)
        dec = v[:, c0:c1] / sc[:, g:g + 1].astype(np.float64)
        assert (np.abs(dec - y) <= np.abs(y) / 16 + 2.0 ** -10 + 1e-12).all()
        nz = amax > 0
        assert (np.abs(dec[nz]).max(axis=1) == 448.0).all()


def test_ds_mla_latent_matches_group_format():
    """The packed latent decodes like the separate-scale group format with the
    same codes and scales; the rope part like a bf16 cache."""
    rng = np.random.default_rng(22)
    codes = rng.integers(0, 0x7E, (7, 512)).astype(np.uint8)
    codes[:, ::5] |= 0x80
    scales = rng.uniform(0.001, 0.05, (7, 4)).astype(np.float32)
    rope = _rand_bf16(rng, (7, 64))
    packed = O.pack_ds_mla(codes, scales, rope)
    slots = np.array([6, 1, 3])
    a = O.dequantize_rows(packed, O.KV_FP8_DS_MLA, slots)
    b = O.dequantize_rows(codes, O.KV_FP8_GROUP128, slots, group_scales=scales)
    c = O.dequantize_rows(rope, O.KV_BF16, slots)
    assert (a[:, :512] == b).all() and (a[:, 512:] == c).all()


# ---------------------------------------------------------------------------
# logit softcap and attention sinks
# ---------------------------------------------------------------------------

def test_softcap_closed_forms():
    """One slot: out = its value row, lse = c tanh(s / c). Two slots: the
    weights are e^{c tanh(s_j / c)}, written out with scalar math."""
    rng = np.random.default_rng(23)
    q, cache, _ = _setup(rng, T=1, h=3, K=2)
    kv = O.bf16_bits_to_f64(cache)
    scale, cap = 0.3, 2.5
    idx1 = np.array([[7, -1]], np.int32)
    o, l = O.attention(q, cache, O.KV_BF16, idx1, scale, softcap=cap)
    for i in range(3):
        s = scale * float(q[0, i] @ kv[7])
        assert abs(l[0, i] - cap * math.tanh(s / cap)) < 1e-12
        assert np.abs(o[0, i] - kv[7, :512]).max() < 1e-12
    idx2 = np.array([[7, 11]], np.int32)
    o, l = O.attention(q, cache, O.KV_BF16, idx2, scale, softcap=cap)
    for i in range(3):
        z = [cap * math.tanh(scale * float(q[0, i] @ kv[g]) / cap) for g in (7, 11)]
        w = [math.exp(zz) for zz in z]
        assert abs(l[0, i] - math.log(w[0] + w[1])) < 1e-12
        ref = (w[0] * kv[7, :512] + w[1] * kv[11, :512]) / (w[0] + w[1])
        assert np.abs(o[0, i] - ref).max() < 1e-12


def test_softcap_bounds_logits_and_vanishes_for_large_caps():
    rng = np.random.default_rng(24)
    q, cache, idx = _setup(rng, T=2, h=4, K=30)
    o0, l0 = O.attention(q, cache, O.KV_BF16, idx, 0.05)
    o1, l1 = O.attention(q, cache, O.KV_BF16, idx, 0.05, softcap=1e7)
    assert np.abs(o1 - o0).max() < 1e-9 and np.abs(l1 - l0).max() < 1e-9
    # a tiny cap squeezes every logit into (-c, c): lse within ln(v) +- c
    cap = 1e-3
    _, lc = O.attention(q, cache, O.KV_BF16, idx, 50.0, softcap=cap)
    v = np.array([(idx[t] >= 0).sum() for t in range(2)], np.float64)
    assert (np.abs(lc - np.log(v)[:, None]) <= cap + 1e-12).all()


def test_sink_closed_forms_and_identity():
    rng = np.random.default_rng(25)
    q, cache, idx = _setup(rng, T=2, h=3, K=12)
    kv = O.bf16_bits_to_f64(cache)
    scale = 0.07
    # sink = -inf is no sink at all
    o0, l0 = O.attention(q, cache, O.KV_BF16, idx, scale)
    o1, l1 = O.attention(q, cache, O.KV_BF16, idx, scale, sinks=np.full(3, -np.inf))
    assert (o1 == o0).all() and (l1 == l0).all()
    # one slot: lse = ln(e^s + e^sink), out = V e^s / (e^s + e^sink)
    sinks = np.array([-1.0, 0.5, 3.0])
    o, l = O.attention(q[:1], cache, O.KV_BF16, np.array([[5, -1]], np.int32), scale, sinks=sinks)
    for i in range(3):
        s = scale * float(q[0, i] @ kv[5])
        den = math.exp(s) + math.exp(sinks[i])
        assert abs(l[0, i] - math.log(den)) < 1e-12
        assert np.abs(o[0, i] - kv[5, :512] * math.exp(s) / den).max() < 1e-12
    # empty row: (0, sink)
    o, l = O.attention(q[:1], cache, O.KV_BF16, np.full((1, 4), -1, np.int32), scale, sinks=sinks)
    assert (o == 0).all() and (l[0] == sinks).all()


def test_sink_is_a_merge_with_a_zero_partial():
    """The sink acts as one more partial result (0, sink) merged by LSE."""
    rng = np.random.default_rng(26)
    q, cache, idx = _setup(rng, T=3, h=4, K=25)
    sinks = np.array([-2.0, 0.0, 1.5, 8.0])
    o0, l0 = O.attention(q, cache, O.KV_BF16, idx, 0.05, softcap=4.0)
    o1, l1 = O.attention(q, cache, O.KV_BF16, idx, 0.05, softcap=4.0, sinks=sinks)
    zero = np.zeros_like(o0)
    mo, ml = O.merge_partials(np.stack([o0, zero]), np.stack([l0, np.broadcast_to(sinks, l0.shape)]))
    assert np.abs(mo - o1).max() < 1e-12 and np.abs(ml - l1).max() < 1e-12


# ---------------------------------------------------------------------------
# planned valid counts (pooled indexer) and the FP8 prefill upconvert
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("topk,kpool", [(64, 1), (64, 4), (256, 64), (2048, 64)])
def test_planned_counts_match_a_simulated_pooled_indexer(topk, kpool):
    """For every query row, the count of positions the simulated indexer keeps
    (distinct, inside the row's context) equals the planned count."""
    rng = np.random.default_rng(27 + kpool)
    q_lens = rng.integers(1, 5, 6)
    seq = np.array([int(rng.integers(q, q + 3 * topk)) for q in q_lens])
    seq[0] = q_lens[0]                                   # a request that is all new tokens
    qsl = np.concatenate([[0], np.cumsum(q_lens)])
    req = np.repeat(np.arange(6), q_lens)
    planned = O.planned_valid_counts(seq, qsl, req, topk, kpool)
    for t in range(req.size):
        r = req[t]
        ctx = int(seq[r] - q_lens[r] + (t - qsl[r]) + 1)
        sel = O.indexer_selection(ctx, topk, kpool, rng.standard_normal(ctx // kpool + 1))
        assert np.unique(sel).size == sel.size and sel.min() >= 0 and sel.max() < ctx
        assert sel.size == planned[t], (t, ctx, sel.size, planned[t])
    if kpool == 1:
        ctx_all = seq[req] - qsl[req + 1] + np.arange(req.size) + 1
        assert (planned == np.minimum(ctx_all, topk)).all()


def test_upconvert_is_the_bf16_rounding_of_the_decoded_value():
    """Latent: torch's bf16 rounding of e4m3 * scale (exact in fp64, so the
    fp32 product rounds the same way); power-of-two scales stay exact; the rope
    bits are copied."""
    rng = np.random.default_rng(28)
    n = 40
    codes = rng.integers(0, 256, (n, 512)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    scales = rng.uniform(1e-3, 10.0, (n, 4)).astype(np.float32)
    scales[:5] = np.ldexp(1.0, rng.integers(-8, 8, (5, 4))).astype(np.float32)
    rope = _rand_bf16(rng, (n, 64))
    cache = O.pack_ds_mla(codes, scales, rope)
    slots = rng.permutation(n)
    got = O.upconvert_rows(cache, slots)
    exact = O.dequantize_rows(cache, O.KV_FP8_DS_MLA, slots)
    ref = torch.from_numpy(exact[:, :512]).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (got[:, :512] == ref).all()
    assert (got[:, 512:] == rope[slots]).all()
    p2 = np.isin(slots, np.arange(5))
    assert (O.bf16_bits_to_f64(got[p2]) == exact[p2]).all()


def test_gather_upconvert_places_each_position():
    """Request r's position p lands in workspace row starts[r] + p, read through
    the block table; rows outside the requests' ranges stay untouched."""
    rng = np.random.default_rng(29)
    B, nblk = 4, 12
    rows = _rand_bf16(rng, (nblk * B, 576))
    cache = np.zeros((nblk * B, 656), np.uint8)
    O.cache_write(rows[:, :512], rows[:, 512:], np.arange(nblk * B), O.KV_FP8_DS_MLA, cache)
    bt = rng.permutation(nblk).reshape(3, 4).astype(np.int32)
    seq = np.array([5, 16, 0])
    starts = np.array([0, 8, 30])
    ws = np.full((32, 576), 0xABCD, np.uint16)
    O.gather_upconvert(cache, bt, seq, starts, B, ws)
    for r in range(3):
        for pos in range(seq[r]):
            slot = bt[r, pos // B] * B + pos % B
            assert (ws[starts[r] + pos] == O.upconvert_rows(cache, [slot])[0]).all()
    assert (ws[5:8] == 0xABCD).all() and (ws[24:] == 0xABCD).all()
