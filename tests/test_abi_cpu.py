"""Host-side checks of the C ABI library: it loads, exports every symbol its header
declares, sizes workspaces consistently and rejects invalid arguments before touching a
device.  No compute call is made.

The validation cases pass fake device addresses that are never dereferenced because
every case must fail validation; on a host with a GPU they are skipped so that a
validation bug can never turn into a launch with a bogus pointer.
"""
import ctypes as C
import os
import re

import pytest
import torch

from dflash2_block_drafter_amd import binding as B
from dflash2_block_drafter_amd import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash2.h")

needs_no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake pointers only on GPU-less hosts")
FAKE = 0x10000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dfl_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = B.lib()
    names = declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), f"{n} declared in dflash2.h but not exported"
    assert sorted(B.exported_symbols()) == names, "binding and header disagree"


def test_workspace_sizes_are_consistent():
    assert B.dfl_linear_workspace_bytes(128, 6144, 5120) >= 0
    assert B.dfl_linear_workspace_bytes(128, 6144, 100) == 0          # K not a multiple of 64
    assert B.dfl_conv_prepare_workspace_bytes(1024, 5120, 16) >= 1024 * 640 * 4
    a = B.dfl_attention_workspace_bytes(8, 16, 32, 8, 128, 2048)
    b = B.dfl_attention_workspace_bytes(8, 16, 32, 8, 128, 8192)
    assert 0 < a <= b
    assert B.dfl_candidates_workspace_bytes(120, 248320, 16) == 120 * 970 * 4   # one fp32 max per 256-column tile
    assert B.dfl_draft_workspace_bytes(None, 8, 16, 2048) == 0         # no handle


def _err(code):
    return code, B.lib().dfl_last_error().decode()


@needs_no_gpu
def test_validation_errors_before_any_launch():
    L = B.lib()
    P = FAKE
    # top_k above the supported 32
    assert _err(L.dfl_compute_candidates(P, 4, 100, 40, P, P, P, 1 << 20, None))[0] == B.DFL_E_UNSUPPORTED
    # workspace too small
    assert L.dfl_compute_candidates(P, 4, 248320, 16, P, P, P, 16, None) == B.DFL_E_WORKSPACE
    # the allocation-free variant: more tile maxima than its static scratch holds (1082 rows
    # x 970 tiles > 2^20), or a bad K, are refused before any device call
    assert L.dfl_compute_candidates_static(P, 1082, 248320, 16, P, P, None) == B.DFL_E_WORKSPACE
    assert L.dfl_compute_candidates_static(P, 4, 100, 40, P, P, None) == B.DFL_E_UNSUPPORTED
    assert L.dfl_compute_candidates_static(None, 4, 100, 4, P, P, None) == B.DFL_E_INVALID
    # the fused selection: K above 16, R not a multiple of 4 or above 64, more than 64 slots
    sel = lambda S, K, R, pred=P: L.dfl_select_tokens(P, P, 2, S, 1000, K, P, R, P, pred, P, P, P, None, P, None)
    assert sel(15, 32, 64) == B.DFL_E_UNSUPPORTED
    assert sel(15, 16, 62) == B.DFL_E_UNSUPPORTED
    assert sel(15, 16, 128) == B.DFL_E_UNSUPPORTED
    assert sel(65, 16, 64) == B.DFL_E_UNSUPPORTED
    assert sel(15, 16, 64, pred=None) == B.DFL_E_INVALID
    # without tile maxima the row's scan keeps them on chip: at most 4096 tiles (V <= 2^20)
    assert L.dfl_select_tokens(P, None, 2, 15, 4096 * 256 + 1, 16, P, 64, P, P, P, P, P, None, P,
                               None) == B.DFL_E_UNSUPPORTED
    # the selection with its projection: H not a multiple of 128, R above 64, a NULL input
    selp = lambda H, R, h=P: L.dfl_select_tokens_projected(P, 2, 15, 1000, 16, h, H, P, R, P, P, P, P, P, P, None,
                                                           P, None)
    assert selp(200, 64) == B.DFL_E_UNSUPPORTED
    assert selp(256, 128) == B.DFL_E_UNSUPPORTED
    assert selp(256, 64, h=None) == B.DFL_E_INVALID
    # null pointers
    assert L.dfl_select_path(None, P, 1, 1, 4, P, None) == B.DFL_E_INVALID
    # K not a multiple of 64
    assert L.dfl_linear(P, 4, 100, 100, P, 8, P, 8, 1, None, 0, None) == B.DFL_E_UNSUPPORTED
    # rows that are not whole blocks
    code, msg = _err(L.dfl_conv_finish(P, P, P, 30, 512, 16, 16, None, P, None))
    assert code == B.DFL_E_SHAPE and "block" in msg
    # group not a multiple of 8
    assert L.dfl_conv_finish(P, P, P, 32, 512, 16, 4, None, P, None) == B.DFL_E_UNSUPPORTED
    # finish may not convolve in place
    assert L.dfl_conv_finish(P, P, P, 32, 512, 16, 16, None, P, None) == B.DFL_E_INVALID
    # head_dim not 64/128
    assert L.dfl_head_norm_rope(P, 4, 2, 96, 192, P, 1e-6, 1e4, P, 4, None) == B.DFL_E_UNSUPPORTED
    # more than 64 query rows per KV head
    assert L.dfl_block_attention(P, 8192, P, P, 8192, P, P, 10, 10, P, None, 0, 1, 32, 32, 8, 128, P, 4096, P,
                                 1 << 30, None) == B.DFL_E_UNSUPPORTED
    # a sliding window needs the block positions, and a window is never negative
    assert L.dfl_block_attention(P, 8192, P, P, 8192, P, P, 10, 10, P, None, 64, 1, 16, 32, 8, 128, P, 4096, P,
                                 1 << 30, None) == B.DFL_E_INVALID
    assert L.dfl_block_attention(P, 8192, P, P, 8192, P, P, 10, 10, P, P, -1, 1, 16, 32, 8, 128, P, 4096, P,
                                 1 << 30, None) == B.DFL_E_INVALID
    # misaligned workspace
    assert L.dfl_compute_candidates(P, 4, 100, 4, P, P, P + 8, 1 << 20, None) == B.DFL_E_INVALID
    # ragged append: offsets that decrease, and rows past the cache
    offs = (C.c_int32 * 3)(0, 4, 2)
    st = (C.c_int32 * 2)(0, 0)
    ptrs = (C.c_void_p * 1)(P)
    assert L.dfl_context_append(P, P, offs, st, 2, 64, ptrs, ptrs, P, 1 << 20, None) == B.DFL_E_SHAPE
    offs = (C.c_int32 * 3)(0, 4, 8)
    st = (C.c_int32 * 2)(0, 61)
    assert L.dfl_context_append(P, P, offs, st, 2, 64, ptrs, ptrs, P, 1 << 20, None) == B.DFL_E_SHAPE


def _config(**kw):
    d = configs.TINY_DIMS
    cfg, keep = B.make_config(d, kw.pop("tap_layer_ids", None))
    for k, v in kw.items():
        setattr(cfg, k, v)
    return cfg, keep


@needs_no_gpu
@pytest.mark.parametrize("field,value,code", [
    ("conv_taps", 3, B.DFL_E_UNSUPPORTED),      # two-tap only
    ("block_size", 1, B.DFL_E_UNSUPPORTED),     # zero draft rows
    ("kv_heads", 3, B.DFL_E_SHAPE),             # heads not a multiple of kv_heads
    ("head_dim", 80, B.DFL_E_UNSUPPORTED),
    ("top_k", 33, B.DFL_E_UNSUPPORTED),
    ("conv_group", 12, B.DFL_E_UNSUPPORTED),
    ("hidden", 0, B.DFL_E_INVALID),
    ("sliding_window", -1, B.DFL_E_INVALID),
])
def test_load_rejects_bad_config(field, value, code):
    cfg, keep = _config(**{field: value})
    out = C.c_void_p()
    w = B.dfl_weights()
    assert B.lib().dfl_drafter_load(C.byref(cfg), C.byref(w), None, C.byref(out)) == code
    assert out.value is None


@needs_no_gpu
def test_load_rejects_repeated_tap_ids():
    cfg, keep = _config(tap_layer_ids=[5, 5])
    out = C.c_void_p()
    w = B.dfl_weights()
    code, msg = _err(B.lib().dfl_drafter_load(C.byref(cfg), C.byref(w), None, C.byref(out)))
    assert code == B.DFL_E_UNSUPPORTED and "repeats" in msg


@needs_no_gpu
def test_load_rejects_null_weights():
    cfg, keep = _config()
    out = C.c_void_p()
    w = B.dfl_weights()
    assert B.lib().dfl_drafter_load(C.byref(cfg), C.byref(w), None, C.byref(out)) == B.DFL_E_INVALID


@needs_no_gpu
def test_load_rejects_null_q4_weight():
    # a 4-bit drafter: the bf16 projection pointers are not needed, every 4-bit field is
    cfg, keep = _config()
    d = configs.TINY_DIMS
    layers = (B.dfl_layer_weights * d.layers)()
    q4 = (B.dfl_q4_layer * d.layers)()
    for i in range(d.layers):
        for f in B.LAYER_FIELDS:
            if f not in B.Q4_FIELDS:
                setattr(layers[i], f, FAKE)
        for f in B.Q4_FIELDS:
            setattr(q4[i], f, B.dfl_q4_weight(FAKE, FAKE, FAKE))
    q4[d.layers - 1].down_proj.biases = None
    w = B.dfl_weights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, C.cast(layers, C.POINTER(B.dfl_layer_weights)),
                      C.cast(q4, C.POINTER(B.dfl_q4_layer)))
    out = C.c_void_p()
    code, msg = _err(B.lib().dfl_drafter_load(C.byref(cfg), C.byref(w), None, C.byref(out)))
    assert code == B.DFL_E_INVALID and "4-bit" in msg
    assert out.value is None
