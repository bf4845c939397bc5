"""GPU parity of the planning and FP8 prefill pieces around the attention:
valid counts planned from the batch layout (bit-exact, and equal to the
conversion's counts on rows shaped like the pooled indexer's selection), and the
gather-and-upconvert of packed FP8 context rows into a bf16 workspace
(bit-exact), with the bf16 prefill over that workspace against the oracle."""
import numpy as np
import pytest
import torch

from oracle import sparse_mla as O
import parity_util as PU
from parity_util import bits, compare, oracle_for, say
from sparse_mla_attention_top_amd import inputs as I
from sparse_mla_attention_top_amd import smla

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32)).to(DEV)


@pytest.mark.parametrize("topk,kpool", [(64, 1), (2048, 64), (256, 4)])
def test_planned_counts_bitexact(topk, kpool):
    rng = np.random.default_rng(200 + kpool)
    R = 37
    q_lens = rng.integers(1, 9, R)
    seq = q_lens + rng.integers(0, 3 * topk, R)
    seq[3] = 0                                               # inconsistent request: ctx <= 0
    qsl = np.concatenate([[0], np.cumsum(q_lens)])
    req = np.repeat(np.arange(R), q_lens)
    req[5] = R + 3                                           # bad request ids
    req[6] = -1
    say(f"planned counts topk={topk} kpool={kpool}")
    got = smla.planned_valid_counts(_i32(seq), _i32(qsl), _i32(req), topk, kpool)
    torch.cuda.synchronize()
    ref = O.planned_valid_counts(seq, qsl, req, topk, kpool)
    assert np.array_equal(got.cpu().numpy(), ref)


def test_planned_counts_match_conversion_on_indexer_shaped_rows():
    """Rows built by the simulated pooled indexer (request-local positions in
    random order, -1 tail): the conversion's valid counts equal the planned
    counts, and the attention bounded by either gives the same bits."""
    rng = np.random.default_rng(210)
    topk, kpool, B, R, h = 256, 16, 64, 4, 64
    q_lens = np.array([3, 1, 5, 2])
    seq = np.array([200, 1000, 300, 5000])
    qsl = np.concatenate([[0], np.cumsum(q_lens)])
    req = np.repeat(np.arange(R), q_lens).astype(np.int32)
    T = req.size
    mb = (seq.max() + B - 1) // B
    bt = rng.permutation(R * mb).reshape(R, mb).astype(np.int32)
    loc = np.full((T, topk + kpool), -1, np.int32)
    for t in range(T):
        r = req[t]
        ctx = int(seq[r] - q_lens[r] + (t - qsl[r]) + 1)
        sel = O.indexer_selection(ctx, topk, kpool, rng.standard_normal(ctx // kpool + 1))
        loc[t, :sel.size] = rng.permutation(sel)
    say("planned counts vs conversion")
    planned = smla.planned_valid_counts(_i32(seq), _i32(qsl), _i32(req), topk, kpool)
    gidx, vcnt = smla.convert_indices(_i32(req), _i32(bt), _i32(loc))
    torch.cuda.synchronize()
    assert torch.equal(planned, vcnt)
    g = torch.Generator().manual_seed(211)
    S = R * mb * B
    kv = torch.randn((S, 576), generator=g).to(torch.bfloat16).to(DEV)
    q = torch.randn((T, h, 576), generator=g).to(torch.bfloat16).to(DEV)
    o1, l1 = PU.decode_fwd(q[..., :512], q[..., 512:], kv, gidx, 0.07, topk_length=planned)
    o2, l2 = PU.decode_fwd(q[..., :512], q[..., 512:], kv, gidx, 0.07, topk_length=vcnt)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    go, vo = O.convert_indices(req, bt, loc, B)
    compare(o1, l1, oracle_for(q.cpu(), bits(kv), go, 0.07, vo), "planned counts attention")


def _packed_cache(n_rows, seed, width=656):
    g = torch.Generator().manual_seed(seed)
    rows = torch.randn((n_rows, 576), generator=g).to(torch.bfloat16)
    rb = bits(rows)
    cache = np.zeros((n_rows, width), np.uint8)
    O.cache_write(rb[:, :512], rb[:, 512:], np.arange(n_rows), O.KV_FP8_DS_MLA, cache)
    return cache


@pytest.mark.parametrize("width,block_stride", [(656, 0), (672, 96)])
def test_gather_upconvert_bitexact(width, block_stride):
    """Random block tables, ragged contexts (one empty, one past the table),
    a negative table entry (zero row), a request placed partly outside the
    workspace, padded workspace rows; untouched rows keep their bytes."""
    rng = np.random.default_rng(220 + width)
    B, R, mb = 16, 5, 9
    stride_rows = block_stride or B
    S = R * mb * stride_rows
    cache = _packed_cache(S, 221, width)
    bt = rng.permutation(R * mb).reshape(R, mb).astype(np.int32)
    bt[2, 1] = -4
    seq = np.array([37, 0, 100, 9 * 16 + 20, 50], np.int32)
    starts = np.array([0, 40, 40, 150, 300], np.int32)      # request 4 runs past the 320-row workspace
    W = 320
    init = rng.integers(0, 65536, (W, 584)).astype(np.uint16)
    ws = torch.from_numpy(init.view(np.int16).copy()).view(torch.bfloat16).to(DEV)
    say(f"gather upconvert width={width}")
    smla.gather_upconvert(torch.from_numpy(cache).to(DEV), _i32(bt), _i32(seq), _i32(starts), int(seq.max()),
                          ws, block_size=B, block_stride_rows=block_stride)
    torch.cuda.synchronize()
    ref = init.copy()
    view = ref[:, :576]
    tmp = view.copy()
    O.gather_upconvert(cache, bt, seq, starts, B, tmp, block_stride_rows=stride_rows)
    ref[:, :576] = tmp
    got = bits(ws)
    assert np.array_equal(got, ref), f"{int((got != ref).any(1).sum())} workspace rows differ"


def test_fp8_prefill_by_upconvert_full_size_sampled():
    """The packed FP8 prefill workload (4096 tokens x h=128, top-k 2048, causal
    indices) run both ways: the FP8 kernel on the packed cache against the
    oracle's exact FP8 attention, and gather-upconvert + the bf16 kernel on the
    workspace against the oracle's attention over its own upconverted rows."""
    spec = I.SPECS["prefill_ds_mla"]
    w = I.generate(spec, kv_device=DEV)
    rb = bits(w.kv_src)
    cache = np.zeros((spec.num_slots, 656), np.uint8)
    O.cache_write(rb[:, :512], rb[:, 512:], np.arange(spec.num_slots), O.KV_FP8_DS_MLA, cache)
    kv = torch.from_numpy(cache).to(DEV).view(spec.num_blocks, I.BLOCK_SIZE, 656)
    q = w.q
    qn, qr = q[..., :512], q[..., 512:]
    req, bt, loc = w.req_id.to(DEV), w.block_table.to(DEV), w.topk_local.to(DEV)
    say("fp8 prefill, in-LDS dequant")
    o1, l1 = PU.prefill_fwd(qn, qr, kv, loc, spec.softmax_scale, kv_format=smla.KV_FP8_DS_MLA, return_lse=True,
                            block_table=bt, req_id=req, block_size=I.BLOCK_SIZE)
    # the workspace: request r's context at starts[r] (block-aligned), read through a workspace block table
    seq = torch.full((spec.num_requests,), spec.ctx_len, dtype=torch.int32, device=DEV)
    starts = torch.zeros((spec.num_requests,), dtype=torch.int32, device=DEV)
    ws = torch.empty((spec.num_slots, 576), dtype=torch.bfloat16, device=DEV)
    ws_bt = torch.arange(spec.num_blocks, dtype=torch.int32, device=DEV).view(spec.num_requests, -1)
    say("fp8 prefill, gather-upconvert + bf16")
    smla.gather_upconvert(kv, bt, seq, starts, spec.ctx_len, ws, block_size=I.BLOCK_SIZE)
    o2, l2 = PU.prefill_fwd(qn, qr, ws.view(spec.num_blocks, I.BLOCK_SIZE, 576), loc, spec.softmax_scale,
                            return_lse=True, block_table=ws_bt, req_id=req, block_size=I.BLOCK_SIZE)
    torch.cuda.synchronize()
    ws_ref = np.zeros((spec.num_slots, 576), np.uint16)
    O.gather_upconvert(cache, w.block_table.numpy(), seq.cpu().numpy(), starts.cpu().numpy(), I.BLOCK_SIZE, ws_ref)
    assert np.array_equal(bits(ws), ws_ref)
    go, vo = O.convert_indices(w.req_id.numpy(), w.block_table.numpy(), w.topk_local.numpy(), I.BLOCK_SIZE)
    toks = [0, 1, 31, 32, 100, 2047, 2048, 3000, 4095]
    st = torch.as_tensor(toks, device=DEV)
    ref1 = oracle_for(q.cpu(), cache, go, spec.softmax_scale, vo, tokens=toks, kv_format=O.KV_FP8_DS_MLA)
    compare(o1[st], l1[st], ref1, "fp8 prefill in-LDS", 2)
    ref2 = oracle_for(q.cpu(), ws_ref, go,
                      spec.softmax_scale, vo, tokens=toks)
    compare(o2[st], l2[st], ref2, "fp8 prefill upconvert")
