"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Bit-exact for index conversion; for attention max-abs 1e-2 on the output
before its own bf16 rounding (1e-2 + half a bf16 ulp at |ref|) and 1e-3 on the
LSE, every output and LSE buffer filled with NaN before the call. The
workloads are checked on every token at full size."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import sparse_mla as O
import parity_util as PU
from parity_util import LSE_TOL, OUT_TOL, bits, compare, oracle_for, q_f64, say
from sparse_mla_attention_top_amd import inputs as I
from sparse_mla_attention_top_amd import smla

pytestmark = pytest.mark.gpu
DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _gpu_convert(req, bt, loc, block_size=64, stride=0):
    g, v = smla.convert_indices(req.to(DEV), bt.to(DEV), loc.to(DEV), block_size=block_size,
                                block_stride_rows=stride)
    torch.cuda.synchronize()
    return g.cpu().numpy(), v.cpu().numpy()


# ---------------------------------------------------------------------------
# index conversion (bit-exact)
# ---------------------------------------------------------------------------

def test_convert_golden_examples():
    cases = json.load(open(os.path.join(GOLDEN, "convert_examples.json")))["cases"]
    for c in cases:
        say(f"convert golden {c['name']}")
        g, v = _gpu_convert(torch.tensor(c["req_id"], dtype=torch.int32),
                            torch.tensor(c["block_table"], dtype=torch.int32),
                            torch.tensor(c["topk_local"], dtype=torch.int32), c["block_size"])
        assert g.tolist() == c["expect_global"], c["name"]
        assert v.tolist() == c["expect_valid"], c["name"]


@pytest.mark.parametrize("name", ["tiny", "tiny_late", "decode_bf16", "nope_fp8", "prefill_bf16", "longctx_fp8"])
def test_convert_workloads_bitexact(name):
    w = I.generate(I.SPECS[name], with_values=False)
    say(f"convert workload {name}")
    g, v = _gpu_convert(w.req_id, w.block_table, w.topk_local)
    go, vo = O.convert_indices(w.req_id.numpy(), w.block_table.numpy(), w.topk_local.numpy(), 64)
    assert (g == go).all() and (v == vo).all()
    assert (v == w.valid.numpy()).all()


def test_convert_invalid_corners_bitexact():
    rng = np.random.default_rng(17)
    R, MB, B, T, K = 5, 7, 16, 37, 300
    bt = rng.permutation(R * MB).reshape(R, MB).astype(np.int32)
    bt[2, 3] = -1
    bt[4, 0] = -5
    req = rng.integers(0, R, T).astype(np.int32)
    loc = rng.integers(-3, MB * B + 10, (T, K)).astype(np.int32)
    for stride in (0, 3 * B):
        say(f"convert corners stride={stride}")
        g, v = _gpu_convert(torch.from_numpy(req), torch.from_numpy(bt), torch.from_numpy(loc), B, stride)
        go, vo = O.convert_indices(req, bt, loc, B, B if stride == 0 else stride)
        assert (g == go).all() and (v == vo).all()


@pytest.mark.parametrize("max_blocks", [4096, 4097, 9000])
def test_convert_long_block_tables_bitexact(max_blocks):
    """Block-table rows up to 4096 entries are staged in LDS, longer ones are
    read entry by entry; both sides of that limit, with a top-k wider than
    one pass of the kernel (2048 entries), invalid entries and a bad request."""
    rng = np.random.default_rng(18 + max_blocks)
    R, B, T, K = 3, 16, 9, 2500
    bt = rng.permutation(R * max_blocks).reshape(R, max_blocks).astype(np.int32)
    bt[1, ::7] = -1
    req = rng.integers(0, R, T).astype(np.int32)
    loc = rng.integers(-2, max_blocks * B + 5, (T, K)).astype(np.int32)
    go, vo = O.convert_indices(req, bt, loc, B)
    req[4] = R                     # outside [0, num_reqs): the kernel gives the row all -1
    say(f"convert long table max_blocks={max_blocks}")
    g, v = _gpu_convert(torch.from_numpy(req), torch.from_numpy(bt), torch.from_numpy(loc), B)
    keep = np.arange(T) != 4
    assert (g[keep] == go[keep]).all() and (v[keep] == vo[keep]).all()
    assert (g[4] == -1).all() and v[4] == 0


def _fused_vs_separate(q, kv, req, bt, loc, scale, entry, block_size, stride=0, num_splits=0):
    """(out, lse) of convert + attention and of attention with the conversion
    fused, on the same inputs."""
    qd = q.to(DEV)
    qn, qr = qd[..., :512], (qd[..., 512:] if q.shape[2] > 512 else None)
    kvd, reqd, btd, locd = kv.to(DEV), req.to(DEV), bt.to(DEV), loc.to(DEV)
    gidx, vcnt = smla.convert_indices(reqd, btd, locd, block_size=block_size, block_stride_rows=stride)
    conv = dict(block_table=btd, req_id=reqd, block_size=block_size, block_stride_rows=stride)
    # no row lengths on either side: invalid entries need not form a tail here
    if entry == "decode":
        a = PU.decode_fwd(qn, qr, kvd, gidx, scale, num_splits=num_splits)
        b = PU.decode_fwd(qn, qr, kvd, locd, scale, num_splits=num_splits, **conv)
    else:
        a = PU.prefill_fwd(qn, qr, kvd, gidx, scale, return_lse=True)
        b = PU.prefill_fwd(qn, qr, kvd, locd, scale, return_lse=True, **conv)
    torch.cuda.synchronize()
    return a, b, gidx, vcnt


@pytest.mark.parametrize("name,entry", [("tiny", "decode"), ("tiny_late", "prefill"), ("decode_bf16", "decode"),
                                        ("prefill_bf16", "prefill")])
def test_fused_conversion_is_bitexact(name, entry):
    """Attention with the index conversion done by the attention kernel gives
    the same bits as smla_convert_indices followed by attention on global
    indices (the same rows, in the same order, through the same arithmetic)."""
    spec = I.SPECS[name]
    say(f"fused conversion {name} {entry}")
    w = I.generate(spec)
    kv = w.kv_src.view(spec.num_blocks, I.BLOCK_SIZE, spec.d)
    (o1, l1), (o2, l2), _, _ = _fused_vs_separate(w.q, kv, w.req_id, w.block_table, w.topk_local,
                                                  spec.softmax_scale, entry, I.BLOCK_SIZE)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("block_size,stride", [(16, 0), (48, 0), (16, 40)])
def test_fused_conversion_invalid_corners(block_size, stride):
    """Fused conversion with a table holding -1 and negative entries, local
    indices below 0 and past the table, a request id out of range (its row
    becomes empty: out 0, LSE -inf), a block size that is not a power of two
    and a table stride other than the block size; bit-exact against the
    separate path and within tolerance of the oracle."""
    rng = np.random.default_rng(19 + block_size + stride)
    R, MB, T, K = 4, 9, 11, 300
    rows = (stride if stride else block_size)
    S = R * MB * rows + block_size
    bt = rng.permutation(R * MB).reshape(R, MB).astype(np.int32)
    bt[1, 2] = -1
    bt[3, 0] = -7
    req = rng.integers(0, R, T).astype(np.int32)
    loc = rng.integers(-3, MB * block_size + 9, (T, K)).astype(np.int32)
    g = torch.Generator().manual_seed(20 + block_size)
    q = torch.randn((T, 64, 576), generator=g).to(torch.bfloat16)
    kv = torch.randn((S, 576), generator=g).to(torch.bfloat16)
    go, vo = O.convert_indices(req, bt, loc, block_size, stride if stride else block_size)
    req_bad = req.copy()
    req_bad[5] = R
    say(f"fused conversion corners B={block_size} stride={stride}")
    for entry, splits in (("decode", 3), ("prefill", 0)):
        (o1, l1), (o2, l2), _, _ = _fused_vs_separate(q, kv, torch.from_numpy(req_bad), torch.from_numpy(bt),
                                                      torch.from_numpy(loc), 0.06, entry, block_size, stride, splits)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
        keep = np.arange(T) != 5
        ref = oracle_for(q[torch.from_numpy(np.nonzero(keep)[0])], bits(kv), go[keep], 0.06)
        compare(o2[torch.as_tensor(np.nonzero(keep)[0], device=DEV)],
                l2[torch.as_tensor(np.nonzero(keep)[0], device=DEV)], ref, f"fused {entry}")
        assert (o2[5] == 0).all() and torch.isneginf(l2[5]).all()


# ---------------------------------------------------------------------------
# attention on the workload specs
# ---------------------------------------------------------------------------

def _run_workload(w, entry, tokens=None, num_splits=0, scale=None, chunk=512):
    """The workload through convert + attention on the GPU, checked against the
    oracle on ``tokens`` (default every token), ``chunk`` tokens at a time.
    Returns the worst output and LSE errors."""
    spec = w.spec
    scale = spec.softmax_scale if scale is None else scale
    q = w.q.to(DEV)
    kv = w.kv_src.to(DEV).view(spec.num_blocks, I.BLOCK_SIZE, spec.d)
    gidx, vcnt = smla.convert_indices(w.req_id.to(DEV), w.block_table.to(DEV), w.topk_local.to(DEV))
    qn, qr = q[..., :512], (q[..., 512:] if spec.d_rope else None)
    if entry == "decode":
        out, lse = PU.decode_fwd(qn, qr, kv, gidx, scale, topk_length=vcnt, num_splits=num_splits)
    else:
        out, lse = PU.prefill_fwd(qn, qr, kv, gidx, scale, topk_length=vcnt, return_lse=True)
    torch.cuda.synchronize()
    go, vo = O.convert_indices(w.req_id.cpu().numpy(), w.block_table.cpu().numpy(), w.topk_local.cpu().numpy(), 64)
    assert (gidx.cpu().numpy() == go).all() and (vcnt.cpu().numpy() == vo).all()
    sel = np.arange(spec.num_tokens) if tokens is None else np.asarray(tokens)
    q_cpu, cache_bits = w.q.cpu(), bits(w.kv_src)
    err = lerr = 0.0
    for c0 in range(0, len(sel), chunk):
        part = sel[c0:c0 + chunk]
        # the oracle gathers only the rows it needs
        ref = oracle_for(q_cpu, cache_bits, go, scale, vo, tokens=part)
        st = torch.as_tensor(part, device=DEV)
        e, le = compare(out[st], lse[st], ref, f"{spec.name}/{entry} tokens {part[0]}..{part[-1]}")
        err, lerr = max(err, e), max(lerr, le)
    return err, lerr


@pytest.mark.parametrize("name", ["tiny", "tiny_late"])
@pytest.mark.parametrize("entry", ["decode", "prefill"])
def test_tiny_workload(name, entry):
    say(f"attention {name} {entry}")
    w = I.generate(I.SPECS[name])
    _run_workload(w, entry)


def test_decode_bf16_full_size():
    """The bf16 decode workload (32 requests x 8192 context, h=128, top-k 2048)
    at full size, every output element, in the launch configuration the
    benchmark times (automatic splits)."""
    spec = I.SPECS["decode_bf16"]
    say("attention decode_bf16 full")
    w = I.generate(spec)
    err, lerr = _run_workload(w, "decode")
    print(f"decode_bf16 full: out err {err:.2e} lse err {lerr:.2e}")


@pytest.mark.parametrize("splits", [1, 2, 3, 8])
def test_decode_splits(splits):
    spec = I.SPECS["decode_bf16"].scaled(num_requests=6, seed=212)
    say(f"attention decode splits={splits}")
    w = I.generate(spec)
    _run_workload(w, "decode", num_splits=splits)


def test_prefill_bf16_full_size():
    """The bf16 prefill workload (4096 tokens, h=128, top-k 2048, causal
    indices, valid = min(2048, pos + 1)) at full size, every token against the
    oracle (FA3 kernel test file, test_fa3_mla_prefill_short_sequence: every
    output of a causal prefill checked)."""
    spec = I.SPECS["prefill_bf16"]
    say("attention prefill_bf16 full, every token")
    w = I.generate(spec, kv_device=DEV)
    err, lerr = _run_workload(w, "prefill")
    print(f"prefill_bf16 full: out err {err:.2e} lse err {lerr:.2e}")


# ---------------------------------------------------------------------------
# edge shapes with global indices
# ---------------------------------------------------------------------------

def _run_case(c, scale, entry="prefill", topk_length="lengths", num_splits=0, slots_view=None, stress=False):
    q = c.q.to(DEV)
    d_rope = q.shape[2] - 512
    kv = c.kv_src.to(DEV)
    idx = c.indices.to(DEV)
    ln = c.lengths.to(DEV) if topk_length == "lengths" else None
    qn, qr = q[..., :512], (q[..., 512:] if d_rope else None)
    if entry == "decode":
        out, lse = PU.decode_fwd(qn, qr, kv, idx, scale, topk_length=ln, num_splits=num_splits)
    else:
        out, lse = PU.prefill_fwd(qn, qr, kv, idx, scale, topk_length=ln, return_lse=True)
    torch.cuda.synchronize()
    ref = oracle_for(c.q, bits(c.kv_src), c.indices.numpy(), scale, None if ln is None else c.lengths.numpy(),
                     magnitude=stress)
    return out, lse, compare(out, lse, ref, "edge", stress=stress)


@pytest.mark.parametrize("h", [1, 16, 33, 64, 100, 128])
@pytest.mark.parametrize("d_rope", [64, 0])
def test_heads_and_nope(h, d_rope):
    say(f"edge heads h={h} d_rope={d_rope}")
    c = I.random_case(T=3, h=h, d_rope=d_rope, topk=100, num_slots=500, seed=h * 10 + d_rope,
                      lengths=[100, 37, 64])
    for entry in ("prefill", "decode"):
        _run_case(c, 0.07, entry)


@pytest.mark.parametrize("topk,lengths", [(1, [1, 0, 1]), (31, [31, 5, 30]), (33, [33, 32, 1]),
                                          (257, [257, 200, 129]), (2048, [2048, 1500, 33])])
def test_topk_widths_and_ragged_tails(topk, lengths):
    say(f"edge topk={topk} lengths={lengths}")
    c = I.random_case(T=3, h=128, d_rope=64, topk=topk, num_slots=4096, seed=topk, lengths=lengths)
    for entry in ("prefill", "decode"):
        _run_case(c, 192 ** -0.5, entry)


def test_scattered_invalid_without_lengths():
    """-1, other negatives and slots >= num_slots anywhere in the row are
    skipped when no length array is passed."""
    say("edge scattered invalid")
    c = I.random_case(T=4, h=64, d_rope=64, topk=200, num_slots=300, seed=5)
    g = torch.Generator().manual_seed(6)
    mask = torch.rand(c.indices.shape, generator=g) < 0.3
    c.indices[mask] = -1
    c.indices[0, 7] = -9
    c.indices[1, 3] = 300
    c.indices[2, 150] = 2 ** 31 - 1
    for entry in ("prefill", "decode"):
        _run_case(c, 0.1, entry, topk_length=None)


def test_empty_rows_give_merge_identity():
    say("edge empty rows")
    c = I.random_case(T=3, h=64, d_rope=64, topk=64, num_slots=100, seed=8, lengths=[64, 0, 10])
    c.indices[2, :] = -1
    for entry in ("prefill", "decode"):
        out, lse, _ = _run_case(c, 0.1, entry)
        assert (out[1:].float() == 0).all() and torch.isneginf(lse[1:]).all()


def test_leading_invalid_tiles():
    """Rows (and decode splits) whose first tiles hold no valid entry, with
    valid entries after them: the softmax reference cannot come from the
    first tile, and the LSE must still be that of the valid entries."""
    say("edge leading invalid tiles")
    c = I.random_case(T=4, h=64, d_rope=64, topk=256, num_slots=600, seed=13)
    c.indices[0, :32] = -1                 # tile 0 invalid
    c.indices[1, :100] = -1                # tiles 0-2 invalid, tile 3 partly
    c.indices[2, :64] = -1                 # split 2 of 2 starts with two invalid tiles too
    c.indices[2, 128:192] = -1
    c.indices[3, 200:] = -1                # an invalid tail only
    for entry, splits in (("prefill", 0), ("decode", 1), ("decode", 2), ("decode", 4)):
        _run_case(c, 0.08, entry, topk_length=None, num_splits=splits)


@pytest.mark.parametrize("alpha", [1.2, 4.0])
def test_large_logit_jump_reruns(alpha):
    """A slot whose score exceeds the first tile's maximum by far more than the
    reference headroom of 64 (base 2): the result must still match the oracle.
    alpha = 1.2 puts the jump near 90 (base 2): the flagged pass's row sums
    stay finite and give the rerun's reference directly. alpha = 4 puts it
    near 330: some p overflows, and a max-only pass finds the maximum."""
    say(f"edge large logit jump, alpha={alpha}")
    c = I.random_case(T=2, h=32, d_rope=64, topk=128, num_slots=256, seed=9)
    # make slot used at position 100 of each row strongly aligned with head 0's query
    for t in range(2):
        s = int(c.indices[t, 100])
        c.kv_src[s] = (c.q[t, 0].float() * alpha).to(torch.bfloat16)
    for entry in ("prefill", "decode"):       # a row of 4 q (values to ~16): the stress allowance
        _run_case(c, 0.1, entry, stress=True)


@pytest.mark.parametrize("qmul,softcap", [(20.0, 0.0), (60.0, 0.0), (20.0, 30.0)])
def test_reruns_over_many_heads(qmul, softcap):
    """Q scaled up so that many heads' later scores exceed the tile-0 reference
    by more than 64 (base 2). With Q x 20 about a sixth of the (head, split)
    pairs jump that far and their row sums stay finite (the rerun takes its
    reference from them); with Q x 60 most do and many overflow past 2^128
    (a max-only pass comes first); softcap 30 bounds the logits. Decode with
    1 and 2 splits and prefill, against the oracle."""
    say(f"reruns over many heads qmul={qmul} softcap={softcap}")
    c = I.random_case(T=4, h=64, d_rope=64, topk=512, num_slots=2048, seed=77)
    c.q = (c.q.float() * qmul).to(torch.bfloat16)
    q, kv, idx = c.q.to(DEV), c.kv_src.to(DEV), c.indices.to(DEV)
    ref = oracle_for(c.q, bits(c.kv_src), c.indices.numpy(), 0.07, softcap=softcap)
    for entry, splits in (("decode", 1), ("decode", 2), ("prefill", 0)):
        if entry == "decode":
            out, lse = PU.decode_fwd(q[..., :512], q[..., 512:], kv, idx, 0.07, num_splits=splits, softcap=softcap)
        else:
            out, lse = PU.prefill_fwd(q[..., :512], q[..., 512:], kv, idx, 0.07, return_lse=True, softcap=softcap)
        torch.cuda.synchronize()
        compare(out, lse, ref, f"reruns x{qmul} softcap={softcap} {entry}/{splits}")


def test_deterministic_bitwise():
    say("determinism")
    c = I.random_case(T=8, h=128, d_rope=64, topk=512, num_slots=2048, seed=12)
    q, kv, idx = c.q.to(DEV), c.kv_src.to(DEV), c.indices.to(DEV)
    a, la = PU.decode_fwd(q[..., :512], q[..., 512:], kv, idx, 0.07, num_splits=4)
    b, lb = PU.decode_fwd(q[..., :512], q[..., 512:], kv, idx, 0.07, num_splits=4)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


@pytest.mark.parametrize("splits", [2, 8, 64])
def test_splits_share_the_valid_prefix(splits):
    """Splits divide the entries up to the last valid one: rows of 2048, 700,
    100, 33, 1 and 0 valid entries (a -1 tail, no row lengths given), so
    that short rows leave some splits empty."""
    say(f"splits share the valid prefix, splits={splits}")
    c = I.random_case(T=6, h=64, d_rope=64, topk=2048, num_slots=4096, seed=40 + splits,
                      lengths=[2048, 700, 100, 33, 1, 0])
    q, kv, idx = c.q.to(DEV), c.kv_src.to(DEV), c.indices.to(DEV)
    o, l = PU.decode_fwd(q[..., :512], q[..., 512:], kv, idx, 0.07, num_splits=splits)
    torch.cuda.synchronize()
    compare(o, l, oracle_for(c.q, bits(c.kv_src), c.indices.numpy(), 0.07), f"prefix splits={splits}")


def test_split_workspace_reused_across_shapes():
    """One caller-owned workspace serves decode calls of different shapes and
    split counts: 4 splits with each token's workgroups on one XCD (8 tokens),
    then 64 splits (the most a top-k of 2048 allows) with 3 tokens spread over
    XCDs, then the first case again."""
    say("split workspace reuse")
    ca = I.random_case(T=8, h=128, d_rope=64, topk=1024, num_slots=3000, seed=15)
    cb = I.random_case(T=3, h=64, d_rope=64, topk=2048, num_slots=5000, seed=16, lengths=[2048, 1500, 37])
    need = max(smla.decode_workspace_size(8, 128, 1024, 4), smla.decode_workspace_size(3, 64, 2048, 64))
    assert smla.decode_num_splits(3, 64, 2048, 64) == 64
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    for c, splits in ((ca, 4), (cb, 64), (ca, 4)):
        q, kv, idx, ln = c.q.to(DEV), c.kv_src.to(DEV), c.indices.to(DEV), c.lengths.to(DEV)
        o, l = PU.decode_fwd(q[..., :512], q[..., 512:], kv, idx, 0.07, topk_length=ln,
                             num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        compare(o, l, oracle_for(c.q, bits(c.kv_src), c.indices.numpy(), 0.07, c.lengths.numpy()),
                f"ws splits={splits}")


def test_strided_query_and_output_views():
    """q_nope / q_rope as views of one [T, h, 576] tensor and an output with a
    padded head stride."""
    say("strided views")
    c = I.random_case(T=5, h=20, d_rope=64, topk=96, num_slots=640, seed=13)
    q = c.q.to(DEV)
    big = torch.zeros((5, 20, 640), dtype=torch.bfloat16, device=DEV)
    out = big[:, :, :512]
    o, l = PU.prefill_fwd(q[..., :512], q[..., 512:], c.kv_src.to(DEV), c.indices.to(DEV), 0.05,
                          out=out, return_lse=True)
    torch.cuda.synchronize()
    ref = oracle_for(c.q, bits(c.kv_src), c.indices.numpy(), 0.05)
    compare(out, l, ref, "strided")
    assert (big[:, :, 512:] == 0).all()


def test_decode_matches_prefill():
    say("decode vs prefill")
    c = I.random_case(T=6, h=128, d_rope=64, topk=1024, num_slots=3000, seed=14, lengths=[1024, 900, 513, 64, 33, 1])
    q, kv, idx, ln = c.q.to(DEV), c.kv_src.to(DEV), c.indices.to(DEV), c.lengths.to(DEV)
    a, la = PU.prefill_fwd(q[..., :512], q[..., 512:], kv, idx, 0.07, topk_length=ln, return_lse=True)
    b, lb = PU.decode_fwd(q[..., :512], q[..., 512:], kv, idx, 0.07, topk_length=ln, num_splits=4)
    torch.cuda.synchronize()
    assert (a.float() - b.float()).abs().max().item() <= 2 * OUT_TOL
    assert (la - lb).abs().max().item() <= 2 * LSE_TOL
