"""GPU parity of the softmax options of the attention entry points -- the
logit softcap and the per-head attention sinks of the FA3 API -- against the
fp64 oracle, on every cache format, with and without decode splits (where the
sink enters at the merge). Bar: max-abs 1e-2 (+ the bf16 allowance of
parity_util) on the output, 1e-3 on the LSE."""
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


def _run(c, kv_format, scale, entry, softcap=0.0, sinks=None, num_splits=0, use_lengths=True):
    host, kv, sc, ks, k = cache_for(c.kv_src, kv_format, DEV)
    q = c.q.to(DEV)
    d_rope = q.shape[2] - 512
    qn, qr = q[..., :512], (q[..., 512:] if d_rope else None)
    ln = c.lengths.to(DEV) if use_lengths else None
    sk = None if sinks is None else torch.as_tensor(sinks, dtype=torch.float32).to(DEV)
    kw = dict(kv_format=kv_format, k_scale=ks, group_scales=sc, topk_length=ln, softcap=softcap, sinks=sk)
    if entry == "decode":
        out, lse = PU.decode_fwd(qn, qr, kv, c.indices.to(DEV), scale, num_splits=num_splits, **kw)
    else:
        out, lse = PU.prefill_fwd(qn, qr, kv, c.indices.to(DEV), scale, return_lse=True, **kw)
    torch.cuda.synchronize()
    ref = oracle_for(c.q, host, c.indices.numpy(), scale, c.lengths.numpy() if use_lengths else None,
                     kv_format=kv_format, k_scale=ks, group_scales=None if sc is None else sc.cpu().numpy(),
                     softcap=softcap,
                     sinks=None if sinks is None else np.asarray(sinks, np.float64))
    compare(out, lse, ref, f"fmt={kv_format} {entry} softcap={softcap} sinks={sinks is not None}", k)
    return out, lse


@pytest.mark.parametrize("softcap", [0.5, 3.0, 30.0])
def test_softcap_bf16(softcap):
    """Caps that flatten the logits (0.5), bend them (3) and barely touch
    them (30); the scale spreads the raw logits to a few units."""
    say(f"softcap {softcap}")
    c = I.random_case(T=3, h=128, d_rope=64, topk=300, num_slots=900, seed=120, lengths=[300, 150, 33])
    for entry, splits in (("prefill", 0), ("decode", 1), ("decode", 3)):
        _run(c, O.KV_BF16, 0.12, entry, softcap=softcap, num_splits=splits)


def test_softcap_with_large_logits_takes_the_exact_path():
    """A wide cap over logits far above the first tile's maximum: the rerun
    with the exact maximum must apply the cap to it as well."""
    say("softcap large logits")
    c = I.random_case(T=2, h=32, d_rope=64, topk=128, num_slots=256, seed=121)
    for t in range(2):
        s = int(c.indices[t, 100])
        c.kv_src[s] = (c.q[t, 0].float() * 4.0).to(torch.bfloat16)
    for entry in ("prefill", "decode"):
        _run(c, O.KV_BF16, 0.1, entry, softcap=200.0)


@pytest.mark.parametrize("h", [16, 64, 128])
def test_sinks_bf16(h):
    say(f"sinks h={h}")
    c = I.random_case(T=3, h=h, d_rope=64, topk=256, num_slots=800, seed=130 + h, lengths=[256, 100, 7])
    sinks = np.random.default_rng(131).normal(0.0, 2.0, h).astype(np.float32)
    for entry, splits in (("prefill", 0), ("decode", 1), ("decode", 2), ("decode", 8)):
        _run(c, O.KV_BF16, 0.08, entry, sinks=sinks, num_splits=splits)


def test_sinks_extreme_values_and_empty_rows():
    """Sinks far above every logit (the output shrinks towards 0, the LSE
    follows the sink), far below (no effect), -inf (no sink), and rows with no
    valid entry, which give (0, sink)."""
    say("sinks extreme")
    c = I.random_case(T=3, h=64, d_rope=64, topk=96, num_slots=300, seed=140, lengths=[96, 0, 40])
    sinks = np.zeros(64, np.float32)
    sinks[0::4] = 60.0
    sinks[1::4] = -60.0
    sinks[2::4] = -np.inf
    sinks[3::4] = 1.5
    for entry, splits in (("prefill", 0), ("decode", 1), ("decode", 3)):
        out, lse = _run(c, O.KV_BF16, 0.08, entry, sinks=sinks, num_splits=splits)
        assert (out[1].float() == 0).all()
        l1 = lse[1].cpu().numpy()
        assert np.array_equal(np.isneginf(l1), np.isneginf(sinks))
        fin = np.isfinite(sinks)
        assert np.abs(l1[fin] - sinks[fin]).max() < 1e-4


@pytest.mark.parametrize("kv_format,d_rope", [(O.KV_FP8_PER_TENSOR, 0), (O.KV_FP8_GROUP128, 64),
                                              (O.KV_FP8_DS_MLA, 64)])
def test_softcap_and_sinks_fp8_formats(kv_format, d_rope):
    say(f"softcap + sinks fmt={kv_format}")
    c = I.random_case(T=3, h=64, d_rope=d_rope, topk=200, num_slots=700, seed=150 + kv_format,
                      lengths=[200, 77, 129])
    sinks = np.random.default_rng(151).normal(0.0, 1.0, 64).astype(np.float32)
    for entry, splits in (("prefill", 0), ("decode", 1), ("decode", 3)):
        _run(c, kv_format, 192 ** -0.5, entry, softcap=2.0, sinks=sinks, num_splits=splits)


def test_options_with_fused_conversion_and_scattered_invalid():
    """Softcap and sinks with request-local indices converted in the kernel:
    the same bits as with global indices, and the oracle's result."""
    say("options fused conversion")
    rng = np.random.default_rng(160)
    R, MB, B, T, K, h = 3, 10, 64, 6, 320, 128
    S = R * MB * B
    bt = rng.permutation(R * MB).reshape(R, MB).astype(np.int32)
    req = rng.integers(0, R, T).astype(np.int32)
    loc = np.stack([rng.permutation(MB * B)[:K] for _ in range(T)]).astype(np.int32)
    loc[rng.random((T, K)) < 0.25] = -1
    loc[2, :64] = -1
    g = torch.Generator().manual_seed(161)
    q = torch.randn((T, h, 576), generator=g).to(torch.bfloat16)
    kv = torch.randn((S, 576), generator=g).to(torch.bfloat16)
    sinks = torch.from_numpy(rng.normal(0, 1, h).astype(np.float32))
    go, _ = O.convert_indices(req, bt, loc, B)
    qd = q.to(DEV)
    kvd = kv.to(DEV).view(R * MB, B, 576)
    args = dict(softcap=5.0, sinks=sinks.to(DEV))
    o1, l1 = PU.decode_fwd(qd[..., :512], qd[..., 512:], kvd, torch.from_numpy(go).to(DEV), 0.09, **args)
    o2, l2 = PU.decode_fwd(qd[..., :512], qd[..., 512:], kvd, torch.from_numpy(loc).to(DEV), 0.09,
                           block_table=torch.from_numpy(bt).to(DEV), req_id=torch.from_numpy(req).to(DEV),
                           block_size=B, **args)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    ref = oracle_for(q, bits(kv), go, 0.09, softcap=5.0, sinks=sinks.numpy().astype(np.float64))
    compare(o2, l2, ref, "options fused")
