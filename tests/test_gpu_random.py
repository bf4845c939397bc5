"""Seeded random configurations.

Attention against the fp64 oracle: cache format, NoPE or rope, head count,
top-k width, row lengths with scattered invalid entries, decode (with a random
split count) or prefill, softcap and sinks, drawn together so that
combinations no targeted test names are exercised too; and request-local
indices converted inside the kernel through random block tables (block size,
row stride, bad request ids, entries past the table); and rows that repeat
slots (each entry counts). Each case is small
enough for the oracle to check every output; the bar is the one of the other
parity tests (max-abs 1e-2 plus the bf16 allowance on the output, 1e-3 on the
LSE).

Index work, bit-exact against the oracle: the context-parallel filter and the
planned valid counts."""
import numpy as np
import pytest
import torch

from oracle import sparse_mla as O
import parity_util as PU
from parity_util import bits, cache_for, compare, oracle_for, say
from sparse_mla_attention_top_amd import inputs as I
from sparse_mla_attention_top_amd import smla

pytestmark = pytest.mark.gpu
DEV = "cuda"
FORMATS = [O.KV_BF16, O.KV_FP8_PER_TENSOR, O.KV_FP8_GROUP128, O.KV_FP8_DS_MLA]


def _draw(seed: int) -> dict:
    r = np.random.default_rng(seed)
    fmt = FORMATS[r.integers(len(FORMATS))]
    d_rope = 64 if fmt == O.KV_FP8_DS_MLA else int(r.choice([0, 64]))
    topk = int(r.choice([1, 2, 31, 32, 33, 64, 95, 128, 200, 257, 480, 700]))
    T = int(r.integers(1, 6))
    lengths = [int(r.integers(0, topk + 1)) if r.random() < 0.7 else topk for _ in range(T)]
    return dict(fmt=fmt, d_rope=d_rope, h=int(r.integers(1, 129)), T=T, topk=topk,
                num_slots=int(r.integers(topk, 3 * topk + 64)), lengths=lengths,
                holes=float(r.choice([0.0, 0.0, 0.2, 0.6])), use_lengths=bool(r.random() < 0.7),
                entry=str(r.choice(["decode", "prefill"])), splits=int(r.integers(0, 7)),
                softcap=float(r.choice([0.0, 0.0, 0.0, 2.5, 15.0])), sinks=bool(r.random() < 0.3),
                scale=float(r.uniform(0.03, 0.12)))


@pytest.mark.parametrize("seed", range(1000, 1160))
def test_random_configuration(seed):
    cfg = _draw(seed)
    say(f"random seed={seed} {cfg}")
    c = I.random_case(T=cfg["T"], h=cfg["h"], d_rope=cfg["d_rope"], topk=cfg["topk"],
                      num_slots=cfg["num_slots"], seed=seed, lengths=cfg["lengths"])
    if cfg["holes"] > 0:                                   # invalid entries inside the rows
        g = torch.Generator().manual_seed(seed + 1)
        c.indices[torch.rand(c.indices.shape, generator=g) < cfg["holes"]] = -1
    host, kv, gs, ks, k = cache_for(c.kv_src, cfg["fmt"], DEV)
    q = c.q.to(DEV)
    qn, qr = q[..., :512], (q[..., 512:] if cfg["d_rope"] else None)
    ln = c.lengths.to(DEV) if cfg["use_lengths"] else None
    sinks = None
    if cfg["sinks"]:
        sinks = np.random.default_rng(seed + 2).normal(0.0, 2.0, cfg["h"]).astype(np.float32)
    kw = dict(kv_format=cfg["fmt"], k_scale=ks, group_scales=gs, topk_length=ln, softcap=cfg["softcap"],
              sinks=None if sinks is None else torch.from_numpy(sinks).to(DEV))
    if cfg["entry"] == "decode":
        out, lse = PU.decode_fwd(qn, qr, kv, c.indices.to(DEV), cfg["scale"], num_splits=cfg["splits"], **kw)
    else:
        out, lse = PU.prefill_fwd(qn, qr, kv, c.indices.to(DEV), cfg["scale"], return_lse=True, **kw)
    torch.cuda.synchronize()
    ref = oracle_for(c.q, host, c.indices.numpy(), cfg["scale"], c.lengths.numpy() if cfg["use_lengths"] else None,
                     kv_format=cfg["fmt"], k_scale=ks, group_scales=None if gs is None else gs.cpu().numpy(),
                     softcap=cfg["softcap"], sinks=None if sinks is None else sinks.astype(np.float64))
    compare(out, lse, ref, f"random seed={seed}", k)


@pytest.mark.parametrize("seed", range(2000, 2032))
def test_random_block_tables_converted_in_kernel(seed):
    """Request-local indices through a random block table, converted in the
    kernel: the oracle's conversion rule, then its attention."""
    r = np.random.default_rng(seed)
    B = int(r.choice([1, 16, 48, 64, 100]))
    stride = B + int(r.choice([0, 0, 8]))
    R, MB = int(r.integers(1, 5)), int(r.integers(1, 12))
    T, h, K = int(r.integers(1, 6)), int(r.integers(1, 129)), int(r.choice([32, 96, 300, 512]))
    num_slots = R * MB * stride
    bt = r.permutation(R * MB).astype(np.int32).reshape(R, MB)
    req = r.integers(-1, R + 1, T).astype(np.int32)          # -1 and R are bad request ids
    loc = r.integers(-1, MB * B + B, (T, K)).astype(np.int32)  # past the table for some entries
    entry = str(r.choice(["decode", "prefill"]))
    splits = int(r.integers(0, 5))
    say(f"random block table seed={seed} B={B} stride={stride} R={R} MB={MB} T={T} h={h} K={K} {entry} splits={splits}")
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((T, h, 576), generator=g).to(torch.bfloat16)
    kv = torch.randn((num_slots, 576), generator=g).to(torch.bfloat16)
    good = (req >= 0) & (req < R)                            # a bad request id leaves its row empty
    go, _ = O.convert_indices(np.where(good, req, 0), bt, loc, B, block_stride_rows=stride)
    qd = q.to(DEV)
    kvd = kv.to(DEV)
    kw = dict(block_table=torch.from_numpy(bt).to(DEV), req_id=torch.from_numpy(req).to(DEV), block_size=B,
              block_stride_rows=stride)
    if entry == "decode":
        out, lse = PU.decode_fwd(qd[..., :512], qd[..., 512:], kvd, torch.from_numpy(loc).to(DEV), 0.07,
                                 num_splits=splits, **kw)
    else:
        out, lse = PU.prefill_fwd(qd[..., :512], qd[..., 512:], kvd, torch.from_numpy(loc).to(DEV), 0.07,
                                  return_lse=True, **kw)
    torch.cuda.synchronize()
    keep = np.nonzero(good)[0]
    if keep.size:
        ref = oracle_for(q[torch.from_numpy(keep)], bits(kv), go[keep], 0.07)
        kd = torch.from_numpy(keep).to(DEV)
        compare(out[kd], lse[kd], ref, f"random block table seed={seed}")
    bad = torch.from_numpy(np.nonzero(~good)[0]).to(DEV)
    assert (out[bad] == 0).all() and torch.isneginf(lse[bad]).all()


@pytest.mark.parametrize("seed", range(3000, 3024))
def test_random_context_parallel_filter(seed):
    """One rank's filter and conversion of top-k positions, bit-exact: random
    rank count, rank, interleave, block size, row widths past one pass of the
    kernel, positions outside every table, -1 table entries, compaction."""
    r = np.random.default_rng(seed)
    W = int(r.integers(1, 9))
    rank = int(r.integers(0, W))
    IL = int(r.choice([1, 2, 16, 64]))
    B = int(r.choice([1, 16, 64]))
    R, MB = int(r.integers(1, 5)), int(r.integers(1, 40))
    T, K = int(r.integers(1, 20)), int(r.choice([1, 64, 700, 2048, 2500]))
    compact = bool(r.random() < 0.5)
    bt = r.permutation(R * MB).astype(np.int32).reshape(R, MB)
    bt[r.random(bt.shape) < 0.05] = -1
    req = r.integers(0, R, T).astype(np.int32)
    pos = r.integers(-2, W * MB * B + 50, (T, K)).astype(np.int32)
    say(f"random dcp filter seed={seed} W={W} rank={rank} I={IL} B={B} T={T} K={K} compact={compact}")
    g, v = smla.dcp_filter_convert(torch.from_numpy(req).to(DEV), torch.from_numpy(bt).to(DEV),
                                   torch.from_numpy(pos).to(DEV), W, rank, IL, block_size=B,
                                   compact_valid_to_front=compact)
    torch.cuda.synchronize()
    go, vo = O.dcp_filter_convert(req, bt, pos, W, rank, IL, B, compact_valid_to_front=compact)
    assert (g.cpu().numpy() == go).all() and (v.cpu().numpy() == vo).all()


@pytest.mark.parametrize("seed", range(4000, 4024))
def test_random_planned_counts(seed):
    """Valid counts planned from the batch layout, bit-exact: random request
    count, query lengths, contexts (some shorter than their queries), top-k,
    pool size and bad request ids."""
    r = np.random.default_rng(seed)
    R = int(r.integers(1, 60))
    topk = int(r.choice([1, 64, 256, 2048]))
    kpool = int(r.choice([1, 4, 64]))
    q_lens = r.integers(0, 9, R)
    seq = q_lens + r.integers(-2, 3 * topk, R)
    qsl = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    req = np.repeat(np.arange(R), q_lens).astype(np.int32)
    if req.size:
        req[r.random(req.size) < 0.05] = R + 1
    say(f"random planned counts seed={seed} R={R} topk={topk} kpool={kpool} tokens={req.size}")
    if req.size == 0:
        return
    got = smla.planned_valid_counts(torch.from_numpy(seq.astype(np.int32)).to(DEV), torch.from_numpy(qsl).to(DEV),
                                    torch.from_numpy(req).to(DEV), topk, kpool)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), O.planned_valid_counts(seq, qsl, req, topk, kpool))


@pytest.mark.parametrize("seed", range(5000, 5008))
def test_random_rows_with_duplicate_slots(seed):
    """Rows drawn with replacement from a small pool of slots, so that a slot
    repeats within a tile, across tiles and across splits: every entry counts
    (the oracle's reading), in decode with splits and in prefill."""
    r = np.random.default_rng(seed)
    T, h, K = int(r.integers(1, 5)), int(r.choice([16, 64, 128])), int(r.choice([64, 300, 1024]))
    pool = int(r.choice([1, 3, 40]))
    fmt = FORMATS[r.integers(len(FORMATS))]
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((T, h, 576), generator=g).to(torch.bfloat16)
    kv = torch.randn((pool + 5, 576), generator=g).to(torch.bfloat16)
    idx = r.integers(0, pool, (T, K)).astype(np.int32)
    idx[r.random((T, K)) < 0.1] = -1
    say(f"duplicate slots seed={seed} T={T} h={h} K={K} pool={pool} fmt={fmt}")
    host, kvd, gs, ks, k = cache_for(kv, fmt, DEV)
    qd = q.to(DEV)
    kw = dict(kv_format=fmt, k_scale=ks, group_scales=gs)
    ref = oracle_for(q, host, idx, 0.06, kv_format=fmt, k_scale=ks, group_scales=None if gs is None else gs.cpu().numpy())
    for splits in (1, 3):
        out, lse = PU.decode_fwd(qd[..., :512], qd[..., 512:], kvd, torch.from_numpy(idx).to(DEV), 0.06,
                                 num_splits=splits, **kw)
        torch.cuda.synchronize()
        compare(out, lse, ref, f"duplicates decode splits={splits}", k)
    out, lse = PU.prefill_fwd(qd[..., :512], qd[..., 512:], kvd, torch.from_numpy(idx).to(DEV), 0.06,
                              return_lse=True, **kw)
    torch.cuda.synchronize()
    compare(out, lse, ref, "duplicates prefill", k)
