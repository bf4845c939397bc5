"""GPU tests of the context-parallel pieces (through the C ABI): the shard
filter against the oracle (bit-exact), the LSE merge against the oracle, and
a context sharded over simulated ranks on one GPU, each rank's decode merged,
against the unsharded result."""
import numpy as np
import pytest
import torch

from oracle import sparse_mla as O
import parity_util as PU
from parity_util import LSE_TOL, OUT_TOL, bits, compare, oracle_for, say
from sparse_mla_attention_top_amd import smla

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("W,rank,I,compact", [(1, 0, 1, False), (2, 1, 1, False), (4, 3, 64, True),
                                              (3, 2, 5, True), (8, 5, 16, False), (4, 0, 1, True)])
def test_dcp_filter_bitexact(W, rank, I, compact):
    """Rows wider than one pass of the kernel (2048 entries), -1 and negative
    positions, positions past the tables, -1 table entries."""
    rng = np.random.default_rng(31 + 7 * W + rank)
    R, MB, B, T, K = 3, 40, 16, 17, 2500
    bt = rng.permutation(R * MB).reshape(R, MB).astype(np.int32)
    bt[1, 3] = -1
    req = rng.integers(0, R, T).astype(np.int32)
    pos = rng.integers(-2, W * MB * B + 50, (T, K)).astype(np.int32)
    pos[4, :] = -1
    say(f"dcp filter W={W} rank={rank} I={I} compact={compact}")
    g, v = smla.dcp_filter_convert(torch.from_numpy(req).to(DEV), torch.from_numpy(bt).to(DEV),
                                   torch.from_numpy(pos).to(DEV), W, rank, I, block_size=B,
                                   compact_valid_to_front=compact)
    torch.cuda.synchronize()
    go, vo = O.dcp_filter_convert(req, bt, pos, W, rank, I, B, compact_valid_to_front=compact)
    assert (g.cpu().numpy() == go).all() and (v.cpu().numpy() == vo).all()


def test_merge_partials_matches_oracle():
    """Strided partials with empty parts ((0, -inf)) and a row empty in every
    part."""
    rng = np.random.default_rng(32)
    P, T, H = 5, 7, 20
    buf = torch.from_numpy(rng.standard_normal((P, T, H, 640)).astype(np.float32)).to(torch.bfloat16)
    po = buf[..., :512]
    pl = torch.from_numpy((rng.standard_normal((P, T, H)) * 3).astype(np.float32))
    pl[1, 2] = -np.inf
    po[1, 2] = 0
    pl[:, 5, 3] = -np.inf
    po[:, 5, 3] = 0
    say("merge partials")
    out, lse = PU.merge_partials(po.to(DEV), pl.to(DEV))
    torch.cuda.synchronize()
    ro, rl = O.merge_partials(po.float().numpy().astype(np.float64), pl.numpy().astype(np.float64))
    err = np.abs(out.float().cpu().numpy() - ro)
    assert (err <= 1e-6 + 2.0 ** -8 * np.abs(ro)).all(), err.max()
    l = lse.cpu().numpy()
    fin = np.isfinite(rl)
    assert (np.isneginf(l) == ~fin).all() and np.abs(l[fin] - rl[fin]).max() <= 1e-5
    assert (out[5, 3] == 0).all()


def _shard(rows, W, I, B, rng):
    """Spread a request's token rows (position p -> rows[p]) over W ranks:
    per rank a cache [slots, D] and a block table [1, nb] (scattered blocks)."""
    N = rows.shape[0]
    rank, local = O.dcp_owner_local(np.arange(N), W, I)
    caches, tables = [], []
    for r in range(W):
        n_r = int((rank == r).sum())
        nb = max(1, (n_r + B - 1) // B)
        bt = rng.permutation(nb + 3)[:nb].astype(np.int32)[None]
        cache = torch.zeros(((nb + 3) * B, rows.shape[1]), dtype=torch.bfloat16)
        own = np.nonzero(rank == r)[0]
        cache[torch.from_numpy(bt[0, local[own] // B] * B + local[own] % B)] = rows[torch.from_numpy(own)]
        caches.append(cache)
        tables.append(bt)
    return caches, tables


@pytest.mark.parametrize("W,I", [(4, 64), (3, 1), (2, 16)])
def test_dcp_sharded_decode_matches_whole(W, I):
    """One request's context spread over W simulated ranks; each rank runs the
    filter and decode on its shard, the partials are merged: the unsharded
    decode's result within the tolerance, and the oracle's. Row 0 selects
    only rank 0's positions, so the other ranks see an empty row."""
    rng = np.random.default_rng(33 + W)
    N, T, h, K, B, scale = 3000, 6, 128, 512, 64, 0.07
    g = torch.Generator().manual_seed(34 + W)
    rows = torch.randn((N, 576), generator=g).to(torch.bfloat16)
    q = torch.randn((T, h, 576), generator=g).to(torch.bfloat16)
    pos = np.stack([rng.permutation(N)[:K] for _ in range(T)]).astype(np.int32)
    own0 = np.nonzero(O.dcp_owner_local(np.arange(N), W, I)[0] == 0)[0]
    pos[0] = rng.permutation(own0)[:K]
    pos[3, 300:] = -1
    req = torch.zeros(T, dtype=torch.int32)
    qd = q.to(DEV)
    say(f"dcp sharded decode W={W} I={I}")
    parts_o, parts_l = [], []
    caches, tables = _shard(rows, W, I, B, rng)
    for r in range(W):
        loc, _ = smla.dcp_filter_convert(req.to(DEV), torch.from_numpy(tables[r]).to(DEV),
                                         torch.from_numpy(pos).to(DEV), W, r, I, block_size=B)
        o, l = PU.decode_fwd(qd[..., :512], qd[..., 512:], caches[r].to(DEV), loc, scale)
        parts_o.append(o)
        parts_l.append(l)
    torch.cuda.synchronize()
    for r in range(1, W):
        assert (parts_o[r][0] == 0).all() and torch.isneginf(parts_l[r][0]).all()
    mo, ml = PU.merge_partials(torch.stack(parts_o), torch.stack(parts_l))
    # the whole context on one rank: position p at slot p
    wo, wl = PU.decode_fwd(qd[..., :512], qd[..., 512:], rows.to(DEV), torch.from_numpy(pos).to(DEV), scale)
    torch.cuda.synchronize()
    ref = oracle_for(q, bits(rows), pos, scale)
    compare(wo, wl, ref, "dcp whole")
    # the merged result: two bf16 roundings (rank output, then merge) on top of the kernel's
    compare(mo, ml, ref, f"dcp merged W={W}")
    assert (mo.float() - wo.float()).abs().max().item() <= 2 * OUT_TOL
    assert (ml - wl).abs().max().item() <= 2 * LSE_TOL


def test_dcp_packed_fp8_ranks_with_sink_merge_to_the_whole():
    """The pages' context-parallel path runs on the packed FP8 cache: each rank
    holds its share of the positions as packed rows (written by the oracle),
    filters and decodes it; the rank partials, merged with the sink given as
    one more partial (0, sink), equal the whole context's attention with that
    sink, and the oracle's."""
    rng = np.random.default_rng(35)
    W, I, B = 4, 64, 64
    N, T, h, K, scale = 4096, 5, 64, 700, 192 ** -0.5
    g = torch.Generator().manual_seed(36)
    rows = torch.randn((N, 576), generator=g).to(torch.bfloat16)
    q = torch.randn((T, h, 576), generator=g).to(torch.bfloat16)
    sinks = torch.linspace(-2.0, 3.0, h)
    pos = np.stack([rng.permutation(N)[:K] for _ in range(T)]).astype(np.int32)
    pos[2, 400:] = -1
    rb = bits(rows)
    packed = np.zeros((N, 656), np.uint8)
    O.cache_write(rb[:, :512], rb[:, 512:], np.arange(N), O.KV_FP8_DS_MLA, packed)
    # rank caches as packed rows, laid out by the placement
    rank, local = O.dcp_owner_local(np.arange(N), W, I)
    req = torch.zeros(T, dtype=torch.int32, device=DEV)
    qd = q.to(DEV)
    parts_o, parts_l = [], []
    say("dcp packed fp8 ranks")
    for r in range(W):
        own = np.nonzero(rank == r)[0]
        nb = (own.size + B - 1) // B
        bt = rng.permutation(nb + 2)[:nb].astype(np.int32)[None]
        cache = np.zeros(((nb + 2) * B, 656), np.uint8)
        cache[bt[0, local[own] // B] * B + local[own] % B] = packed[own]
        loc, _ = smla.dcp_filter_convert(req, torch.from_numpy(bt).to(DEV), torch.from_numpy(pos).to(DEV), W, r, I,
                                         block_size=B, compact_valid_to_front=True)
        o, l = PU.decode_fwd(qd[..., :512], qd[..., 512:], torch.from_numpy(cache).to(DEV), loc, scale,
                             kv_format=smla.KV_FP8_DS_MLA)
        parts_o.append(o)
        parts_l.append(l)
    parts_o.append(torch.zeros_like(parts_o[0]))                 # the sink as a partial (0, sink)
    parts_l.append(sinks.to(DEV)[None, :].expand(T, h).contiguous())
    mo, ml = PU.merge_partials(torch.stack(parts_o), torch.stack(parts_l))
    wo, wl = PU.decode_fwd(qd[..., :512], qd[..., 512:], torch.from_numpy(packed).to(DEV),
                           torch.from_numpy(pos).to(DEV), scale, kv_format=smla.KV_FP8_DS_MLA,
                           sinks=sinks.to(DEV))
    torch.cuda.synchronize()
    ref = oracle_for(q, packed, pos, scale, kv_format=O.KV_FP8_DS_MLA, sinks=sinks.numpy().astype(np.float64))
    compare(wo, wl, ref, "packed whole with sink", 2)
    compare(mo, ml, ref, "packed ranks merged with sink", 2)
