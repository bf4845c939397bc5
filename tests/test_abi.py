"""Host-only checks of the C ABI library: it loads, exports every symbol the
header declares, and rejects bad arguments without touching the GPU."""
import ctypes
import os
import re

import pytest

from sparse_mla_attention_top_amd import smla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "smla.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|int32_t|const char\*)\s+(smla_\w+)\s*\(", text, re.M)))


def test_header_declares_expected_entry_points():
    assert set(_declared_symbols()) == set(smla.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(smla.LIB_PATH)
    for name in _declared_symbols():
        assert hasattr(lib, name), name


def test_version_and_last_error():
    lib = smla.load()
    assert b"gfx950" in lib.smla_version()
    assert isinstance(lib.smla_last_error(), bytes)


def _args(**kw):
    a = smla.AttnArgs()
    a.num_tokens, a.num_heads, a.d_rope, a.topk = 1, 16, 64, 64
    a.softmax_scale = 0.1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,code", [
    ("num_heads", 0, -2), ("num_heads", 129, -2), ("d_rope", 32, -2), ("topk", 0, -2),
    ("topk", 4096, -2), ("kv_format", 7, -1), ("num_tokens", -1, -1),
])
def test_attention_rejects_bad_shapes(field, value, code):
    lib = smla.load()
    a = _args(**{field: value})
    assert lib.smla_prefill_fwd(ctypes.byref(a), None) == code
    assert lib.smla_last_error()


def test_attention_rejects_null_pointers_and_bad_strides():
    lib = smla.load()
    a = _args()                                   # all pointers NULL
    assert lib.smla_decode_fwd(ctypes.byref(a), None, 0, None) == -1
    a = _args(q_nope=16, q_rope=16, kv_cache=16, indices=16, out=16, num_slots=10,
              kv_row_stride_bytes=1000, indices_stride=64, out_stride_head=512)
    assert lib.smla_prefill_fwd(ctypes.byref(a), None) == -1   # row stride not a multiple of 16
    assert b"kv_row_stride" in lib.smla_last_error()
    a = _args(q_nope=16, q_rope=16, kv_cache=16, indices=16, out=16, num_slots=10,
              kv_row_stride_bytes=1152, indices_stride=64, out_stride_head=512, num_splits=4)
    assert lib.smla_decode_fwd(ctypes.byref(a), None, 0, None) == -3  # workspace too small


def test_zero_tokens_is_a_no_op():
    lib = smla.load()
    a = _args(num_tokens=0)
    assert lib.smla_prefill_fwd(ctypes.byref(a), None) == 0
    assert lib.smla_decode_fwd(ctypes.byref(a), None, 0, None) == 0
    assert lib.smla_convert_indices(None, None, 1, 1, 1, None, 0, 0, 0, 64, 0, None, 0, None, None) == 0
    assert lib.smla_cache_write(None, 512, None, 0, None, 0, 64, 0, 1.0, None, 1, 1152, None, 0, None) == 0


def test_convert_and_cache_write_reject_bad_args():
    lib = smla.load()
    assert lib.smla_convert_indices(16, 16, 1, 4, 4, 16, 8, 2, 8, 0, 0, 16, 8, None, None) == -1   # block_size 0
    assert lib.smla_convert_indices(16, 16, 1, 4, 2, 16, 8, 2, 8, 64, 0, 16, 8, None, None) == -1  # bt stride
    assert lib.smla_cache_write(16, 512, 16, 64, 16, 2, 64, 1, 0.0, 16, 4, 576, None, 0, None) == -1  # k_scale 0
    assert lib.smla_cache_write(16, 512, 16, 64, 16, 2, 64, 2, 1.0, 16, 4, 576, None, 0, None) == -1  # no scales
    assert lib.smla_cache_write(16, 512, 16, 64, 16, 2, 48, 0, 1.0, 16, 4, 1152, None, 0, None) == -2  # d_rope


def test_split_plan_is_shape_only():
    assert smla.decode_num_splits(32, 128, 2048) == 4      # 32 tokens x 2 head blocks x 4 = 256
    assert smla.decode_num_splits(128, 64, 2048) == 2      # 128 tokens x 1 head block x 2 = 256
    assert smla.decode_num_splits(48, 128, 2048) == 2      # never more than one round of 256
    assert smla.decode_num_splits(4096, 128, 2048) == 1
    assert smla.decode_num_splits(1, 128, 64) == 1
    assert smla.decode_num_splits(32, 128, 2048, 3) == 3
    assert smla.decode_workspace_size(32, 128, 2048) == 4 * 32 * 128 * (512 * 2 + 4)
    assert smla.decode_workspace_size(4096, 128, 2048) == 0


def test_dcp_filter_and_merge_reject_bad_arguments():
    lib = smla.load()
    # dcp_rank outside 0..dcp_size-1, interleave 0
    assert lib.smla_dcp_filter_convert(None, None, 1, 1, 1, None, 4, 1, 4, 2, 2, 1, 64, 0, 0, None, 4, None, None) == -1
    assert lib.smla_dcp_filter_convert(None, None, 1, 1, 1, None, 4, 1, 4, 2, 0, 0, 64, 0, 0, None, 4, None, None) == -1
    assert lib.smla_dcp_filter_convert(None, None, 1, 1, 1, None, 4, 1, 4, 2, 0, 1, 64, 0, 0, None, 4, None, None) == -1
    assert lib.smla_last_error()
    # no parts, and NULL pointers with tokens to merge
    assert lib.smla_merge_partials(None, 0, 0, 0, None, 0, 0, 0, 1, 1, None, 0, 0, None, 0, None) == -1
    assert lib.smla_merge_partials(None, 0, 0, 512, None, 0, 1, 2, 1, 1, None, 512, 512, None, 1, None) == -1
    # zero tokens is a no-op
    assert lib.smla_merge_partials(None, 0, 0, 512, None, 0, 1, 2, 0, 1, None, 512, 512, None, 1, None) == 0


def test_softcap_and_sinks_reject_bad_arguments():
    lib = smla.load()
    base = dict(q_nope=16, q_rope=16, kv_cache=16, indices=16, out=16, num_slots=10, indices_stride=64,
                out_stride_head=512, kv_row_stride_bytes=1152)
    for cap in (-1.0, float("nan"), float("inf")):
        a = _args(softcap=cap, **base)
        assert lib.smla_prefill_fwd(ctypes.byref(a), None) == -1
        assert b"softcap" in lib.smla_last_error()
    a = _args(sinks=18, **base)
    assert lib.smla_prefill_fwd(ctypes.byref(a), None) == -1
    assert b"sinks" in lib.smla_last_error()


def test_packed_fp8_format_rejects_bad_arguments():
    lib = smla.load()
    base = dict(q_nope=16, q_rope=16, kv_cache=16, indices=16, out=16, num_slots=10, indices_stride=64,
                out_stride_head=512, kv_format=3)
    a = _args(kv_row_stride_bytes=656, d_rope=0, **{k: v for k, v in base.items() if k != "q_rope"})
    assert lib.smla_prefill_fwd(ctypes.byref(a), None) == -2          # needs the rope part
    a = _args(kv_row_stride_bytes=640, **base)
    assert lib.smla_prefill_fwd(ctypes.byref(a), None) == -1          # row shorter than 656 bytes
    assert b"656" in lib.smla_last_error()
    a = _args(kv_row_stride_bytes=656, group_scales=16, **base)
    assert lib.smla_prefill_fwd(ctypes.byref(a), None) == -1          # scales live in the row
    assert b"group_scales" in lib.smla_last_error()
    assert lib.smla_cache_write(16, 512, 16, 64, 16, 2, 64, 3, 1.0, 16, 4, 576, None, 0, None) == -1  # stride < 656
    assert lib.smla_cache_write(16, 512, None, 0, 16, 2, 0, 3, 1.0, 16, 4, 656, None, 0, None) == -2  # no rope


def test_planned_counts_and_upconvert_reject_bad_arguments():
    lib = smla.load()
    assert lib.smla_planned_valid_counts(16, 16, 16, 0, 4, 64, 1, 16, None) == -1     # no requests
    assert lib.smla_planned_valid_counts(16, 16, 16, 2, 4, 64, 0, 16, None) == -1     # kpool 0
    assert lib.smla_planned_valid_counts(None, None, None, 2, 0, 64, 1, None, None) == 0  # no rows: no-op
    # only the packed format; row stride; workspace stride
    assert lib.smla_gather_upconvert(16, 10, 656, 2, 16, 1, 4, 4, 64, 0, 16, 16, 8, 16, 8, 576, None) == -2
    assert lib.smla_gather_upconvert(16, 10, 640, 3, 16, 1, 4, 4, 64, 0, 16, 16, 8, 16, 8, 576, None) == -1
    assert lib.smla_gather_upconvert(16, 10, 656, 3, 16, 1, 4, 4, 64, 0, 16, 16, 8, 16, 8, 570, None) == -1
    assert lib.smla_gather_upconvert(16, 10, 656, 3, 16, 1, 4, 2, 64, 0, 16, 16, 8, 16, 8, 576, None) == -1
    assert lib.smla_last_error()


def test_noalloc_decode_rejects_partials_beyond_its_scratch():
    """A split plan whose partials exceed the 32 MiB static scratch is refused
    before anything is launched (host-side check, no GPU call)."""
    lib = smla.load()
    a = _args(q_nope=16, q_rope=16, kv_cache=16, indices=16, out=16, num_slots=10, kv_row_stride_bytes=1152,
              indices_stride=2048, out_stride_tok=128 * 512, out_stride_head=512, num_tokens=256, num_heads=128,
              topk=2048, num_splits=64, q_nope_stride_tok=128 * 576, q_nope_stride_head=576,
              q_rope_stride_tok=128 * 576, q_rope_stride_head=576)
    assert lib.smla_decode_fwd_noalloc(ctypes.byref(a), None) == -3
    assert b"scratch" in lib.smla_last_error()
    a.num_tokens = 0
    assert lib.smla_decode_fwd_noalloc(ctypes.byref(a), None) == 0
