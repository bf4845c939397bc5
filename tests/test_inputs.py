"""Structure of the seeded synthetic workloads (host only)."""
import numpy as np
import pytest
import torch

from sparse_mla_attention_top_amd import inputs as I


@pytest.mark.parametrize("name", ["tiny", "tiny_late", "decode_bf16", "nope_fp8"])
def test_index_rows_structure(name):
    spec = I.SPECS[name]
    if spec.num_slots > 1 << 22:
        pytest.skip("large cache")
    w = I.generate(spec.scaled(num_requests=min(spec.num_requests, 8)))
    T = w.spec.num_tokens
    loc = w.topk_local.numpy()
    for t in range(T):
        v = int(w.valid[t])
        row = loc[t]
        assert (row[v:] == -1).all() and (row[:v] >= 0).all()
        assert len(set(row[:v].tolist())) == v                 # distinct
        assert row[:v].max(initial=-1) <= int(w.positions[t])  # slots <= pos
        if spec.valid_rule == "min_pos":
            assert v == min(spec.topk, int(w.positions[t]) + 1)
        else:
            assert spec.valid_lo <= v <= spec.valid_hi
    assert w.q.shape == (T, spec.heads, spec.d) and w.q.dtype == torch.bfloat16
    assert w.kv_src.shape == (w.spec.num_slots, spec.d)
    bt = w.block_table.numpy()
    assert sorted(bt.ravel().tolist()) == list(range(w.spec.num_blocks))


def test_seeded_reproducible():
    a = I.generate(I.SPECS["tiny"])
    b = I.generate(I.SPECS["tiny"])
    assert torch.equal(a.q, b.q) and torch.equal(a.kv_src, b.kv_src)
    assert torch.equal(a.topk_local, b.topk_local)


def test_tiny_positions():
    w = I.generate(I.SPECS["tiny"])
    assert w.valid.tolist() == [1, 2, 3, 4]
    w = I.generate(I.SPECS["tiny_late"])
    assert w.valid.tolist() == [64, 64, 64, 64]
