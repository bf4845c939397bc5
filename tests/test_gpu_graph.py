"""The library's calls captured in a HIP graph (through torch.cuda.graph): every
replay, with eager work and synchronisations between the replays, must give the
bits of the eager calls. Covered: decode with the conversion inside the kernel,
splits and the split merge (bf16 and packed FP8 rows, with softcap and sinks),
prefill, the context-parallel filter + decode + merge, the planned counts, and
the FP8 prefill by gather-upconvert. The eager result is itself checked against
the oracle on a sample, so the graph results are held to the parity bar too."""
import numpy as np
import pytest
import torch

from oracle import sparse_mla as O
from parity_util import bits, compare, nan_fill, oracle_for, say
from sparse_mla_attention_top_amd import inputs as I
from sparse_mla_attention_top_amd import smla

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check_graph(run, outs, replays=3):
    """run(): enqueue the calls on the current stream, writing into `outs`.
    Eager reference, capture, then replays interleaved with eager runs. The
    outputs are filled with NaN (all-ones bytes) before the eager reference
    and before every replay, outside the capture, so an element a call does
    not write shows up."""
    for o in outs:
        o.view(torch.uint8).fill_(0xFF)
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        run()                                      # warm the capture stream
        torch.cuda.current_stream().synchronize()
        with torch.cuda.graph(g, stream=side):
            run()
    torch.cuda.synchronize()
    for k in range(replays):
        for o in outs:
            o.view(torch.uint8).fill_(0xFF)
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), f"replay {k} differs from the eager result"
        run()                                      # eager work between the replays
        torch.cuda.synchronize()
    return ref


def test_graph_decode_fused_conversion_and_merge():
    spec = I.SPECS["decode_bf16"].scaled(num_requests=8, seed=230)
    w = I.generate(spec, kv_device=DEV)
    kv = w.kv_src.view(spec.num_blocks, I.BLOCK_SIZE, spec.d)
    q = w.q
    req, bt, loc = w.req_id.to(DEV), w.block_table.to(DEV), w.topk_local.to(DEV)
    T, H = spec.num_tokens, spec.heads
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    ws = torch.empty(smla.decode_workspace_size(T, H, spec.topk, 4), dtype=torch.uint8, device=DEV)
    nan_fill(ws)
    sinks = torch.linspace(-1.0, 2.0, H, device=DEV)
    say("graph decode bf16")

    def run():
        smla.decode_fwd(q[..., :512], q[..., 512:], kv, loc, spec.softmax_scale, out=out, lse=lse, workspace=ws,
                        num_splits=4, block_table=bt, req_id=req, block_size=I.BLOCK_SIZE, softcap=20.0, sinks=sinks)

    _check_graph(run, [out, lse])
    go, vo = O.convert_indices(w.req_id.numpy(), w.block_table.numpy(), w.topk_local.numpy(), I.BLOCK_SIZE)
    toks = [0, 3, 7]
    ref = oracle_for(q.cpu(), bits(w.kv_src), go, spec.softmax_scale, vo, tokens=toks, softcap=20.0,
                     sinks=sinks.cpu().numpy().astype(np.float64))
    st = torch.as_tensor(toks, device=DEV)
    compare(out[st], lse[st], ref, "graph decode")


def test_graph_packed_fp8_decode_and_prefill():
    c = I.random_case(T=5, h=128, d_rope=64, topk=700, num_slots=3000, seed=231, lengths=[700, 650, 1, 0, 333])
    rb = bits(c.kv_src)
    cache = np.zeros((3000, 656), np.uint8)
    O.cache_write(rb[:, :512], rb[:, 512:], np.arange(3000), O.KV_FP8_DS_MLA, cache)
    kv = torch.from_numpy(cache).to(DEV)
    q = c.q.to(DEV)
    idx, ln = c.indices.to(DEV), c.lengths.to(DEV)
    o1 = torch.empty((5, 128, 512), dtype=torch.bfloat16, device=DEV)
    l1 = torch.empty((5, 128), dtype=torch.float32, device=DEV)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    ws = torch.empty(smla.decode_workspace_size(5, 128, 700, 3), dtype=torch.uint8, device=DEV)
    nan_fill(ws)
    say("graph packed fp8")

    def run():
        smla.decode_fwd(q[..., :512], q[..., 512:], kv, idx, 0.07, kv_format=smla.KV_FP8_DS_MLA, topk_length=ln,
                        out=o1, lse=l1, workspace=ws, num_splits=3)
        smla.prefill_fwd(q[..., :512], q[..., 512:], kv, idx, 0.07, kv_format=smla.KV_FP8_DS_MLA, topk_length=ln,
                         out=o2, lse=l2)

    _check_graph(run, [o1, l1, o2, l2])
    ref = oracle_for(c.q, cache, c.indices.numpy(), 0.07, c.lengths.numpy(), kv_format=O.KV_FP8_DS_MLA)
    compare(o1, l1, ref, "graph packed decode", 2)
    compare(o2, l2, ref, "graph packed prefill", 2)


def test_graph_context_parallel_step():
    """One rank's filter, its decode and the merge of all ranks' partials."""
    rng = np.random.default_rng(232)
    W, IL, B, N, T, h, K = 4, 64, 64, 4096, 6, 64, 512
    pos = np.stack([rng.permutation(N)[:K] for _ in range(T)]).astype(np.int32)
    req = torch.zeros(T, dtype=torch.int32, device=DEV)
    n_local = N // W
    bt = torch.from_numpy(rng.permutation(n_local // B).astype(np.int32)[None, :]).to(DEV)
    g = torch.Generator().manual_seed(233)
    kv = torch.randn((n_local, 576), generator=g).to(torch.bfloat16).to(DEV)
    q = torch.randn((T, h, 576), generator=g).to(torch.bfloat16).to(DEV)
    parts_o = torch.randn((W, T, h, 512), generator=g).to(torch.bfloat16).to(DEV)
    parts_l = torch.randn((W, T, h), generator=g).to(DEV)
    loc = torch.empty((T, K), dtype=torch.int32, device=DEV)
    out = torch.empty((T, h, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, h), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(smla.decode_workspace_size(T, h, K), 16), dtype=torch.uint8, device=DEV)
    nan_fill(ws)
    posd = torch.from_numpy(pos).to(DEV)
    say("graph context-parallel step")

    def run():
        smla.dcp_filter_convert(req, bt, posd, W, 0, IL, block_size=B, out=loc, want_valid_counts=False,
                                compact_valid_to_front=True)
        smla.decode_fwd(q[..., :512], q[..., 512:], kv.view(-1, B, 576), loc, 0.07, out=parts_o[0], lse=parts_l[0],
                        workspace=ws)
        smla.merge_partials(parts_o, parts_l, out=out, lse=lse)

    _check_graph(run, [loc, out, lse])


def test_graph_fp8_prefill_by_upconvert_and_planned_counts():
    spec = I.SPECS["prefill_ds_mla"].scaled(num_requests=1, tokens_per_req=600, ctx_len=600, seed=234)
    w = I.generate(spec, kv_device=DEV)
    rb = bits(w.kv_src)
    cache = np.zeros((spec.num_slots, 656), np.uint8)
    O.cache_write(rb[:, :512], rb[:, 512:], np.arange(spec.num_slots), O.KV_FP8_DS_MLA, cache)
    kv = torch.from_numpy(cache).to(DEV).view(spec.num_blocks, I.BLOCK_SIZE, 656)
    q = w.q
    req, bt, loc = w.req_id.to(DEV), w.block_table.to(DEV), w.topk_local.to(DEV)
    seq = torch.full((1,), spec.ctx_len, dtype=torch.int32, device=DEV)
    qsl = torch.tensor([0, spec.num_tokens], dtype=torch.int32, device=DEV)
    starts = torch.zeros((1,), dtype=torch.int32, device=DEV)
    wsb = torch.zeros((spec.num_slots, 576), dtype=torch.bfloat16, device=DEV)   # rows past the context stay 0
    ws_bt = torch.arange(spec.num_blocks, dtype=torch.int32, device=DEV).view(1, -1)
    counts = torch.empty((spec.num_tokens,), dtype=torch.int32, device=DEV)
    out = torch.empty((spec.num_tokens, spec.heads, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((spec.num_tokens, spec.heads), dtype=torch.float32, device=DEV)
    say("graph fp8 prefill by upconvert")

    def run():
        smla.planned_valid_counts(seq, qsl, req, spec.topk, 1, out=counts)
        smla.gather_upconvert(kv, bt, seq, starts, spec.ctx_len, wsb, block_size=I.BLOCK_SIZE)
        smla.prefill_fwd(q[..., :512], q[..., 512:], wsb.view(spec.num_blocks, I.BLOCK_SIZE, 576), loc,
                         spec.softmax_scale, out=out, lse=lse, topk_length=counts, block_table=ws_bt, req_id=req,
                         block_size=I.BLOCK_SIZE)

    _check_graph(run, [counts, wsb, out, lse])
    # the causal prefill's rows hold min(top-k, pos + 1) entries, which is what the layout plans
    assert np.array_equal(counts.cpu().numpy(), w.valid.numpy())
    go, vo = O.convert_indices(w.req_id.numpy(), w.block_table.numpy(), w.topk_local.numpy(), I.BLOCK_SIZE)
    ws_ref = np.zeros((spec.num_slots, 576), np.uint16)
    O.gather_upconvert(cache, w.block_table.numpy(), [spec.ctx_len], [0], I.BLOCK_SIZE, ws_ref)
    toks = [0, 1, 255, 599]
    ref = oracle_for(q.cpu(), ws_ref, go, spec.softmax_scale, vo, tokens=toks)
    st = torch.as_tensor(toks, device=DEV)
    compare(out[st], lse[st], ref, "graph fp8 prefill upconvert")
