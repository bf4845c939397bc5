"""The allocation-free decode (smla_decode_fwd_noalloc, split partials in the
library's static device scratch) against the workspace decode
(smla_decode_fwd) on the same inputs, through the C ABI. Both run the same
kernels with the same split plan, so the bits must agree; the first result is
also checked against the oracle. Two calls in a row, the second with a
smaller input (fewer tokens, heads and splits), so the second reads a scratch
that still holds the first call's partials."""
import numpy as np
import pytest
import torch

import parity_util as PU
from parity_util import bits, compare, oracle_for, say
from sparse_mla_attention_top_amd import inputs as I
from sparse_mla_attention_top_amd import smla

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(c, scale, splits=0):
    q, kv, idx, ln = c.q.to(DEV), c.kv_src.to(DEV), c.indices.to(DEV), c.lengths.to(DEV)
    T, H = q.shape[:2]
    ref_o, ref_l = PU.decode_fwd(q[..., :512], q[..., 512:], kv, idx, scale, topk_length=ln, num_splits=splits)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    PU.nan_fill(out)
    PU.nan_fill(lse)
    smla.decode_fwd_noalloc(q[..., :512], q[..., 512:], kv, idx, scale, out, lse, topk_length=ln,
                            num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), "output differs from smla_decode_fwd"
    assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)), "LSE differs from smla_decode_fwd"
    return out, lse


def test_noalloc_decode_matches_the_workspace_decode_twice():
    big = I.random_case(T=32, h=128, d_rope=64, topk=2048, num_slots=16384, seed=950,
                        lengths=[2048] * 30 + [1500, 1])
    small = I.random_case(T=5, h=64, d_rope=64, topk=700, num_slots=3000, seed=951, lengths=[700, 650, 1, 0, 333])
    assert smla.decode_num_splits(32, 128, 2048) == 4 and smla.decode_num_splits(5, 64, 700) == 2
    say("no-alloc decode: 32 tokens x 128 heads, 4 splits")
    o1, l1 = _both(big, 0.0723)
    toks = [0, 17, 30, 31]
    ref = oracle_for(big.q, bits(big.kv_src), big.indices.numpy(), 0.0723, big.lengths.numpy(), tokens=toks)
    st = torch.as_tensor(toks, device=DEV)
    compare(o1[st], l1[st], ref, "no-alloc decode, first call")
    say("no-alloc decode: 5 tokens x 64 heads, 2 splits (second, smaller call)")
    o2, l2 = _both(small, 0.07)
    compare(o2, l2, oracle_for(small.q, bits(small.kv_src), small.indices.numpy(), 0.07, small.lengths.numpy()),
            "no-alloc decode, second call")
    say("no-alloc decode: 5 tokens, one split (no scratch used)")
    _both(small, 0.07, splits=1)
