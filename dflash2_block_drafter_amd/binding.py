"""ctypes binding of libdflash2.so with the C ABI's names.

Argument marshalling only: tensors become device pointers, the stream is torch's current
HIP stream, and a non-zero status raises DflError with dfl_last_error().  Every step of
the path runs in the library's kernels; there is no fallback.  PyTorch only allocates the
device memory the calls read and write.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdflash2.so")

DFL_OK, DFL_E_INVALID, DFL_E_SHAPE, DFL_E_UNSUPPORTED = 0, -1, -2, -3
DFL_E_WORKSPACE, DFL_E_NOMEM, DFL_E_DEVICE = -4, -5, -6

KERNEL_CLASSES = ["gemm_head", "gemm_gateup", "gemm_down", "gemm_qkv", "gemm_o", "gemm_kproj",
                  "gemm_selproj", "gemm_context", "attention", "conv_prepare", "conv_finish",
                  "rmsnorm", "rope", "topk", "score_edges", "select_path", "select"]


class DflError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dflash2 error {code}: {msg}")
        self.code = code


class dfl_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in
                ("hidden", "layers", "heads", "kv_heads", "head_dim", "intermediate", "n_taps",
                 "block_size", "conv_taps", "conv_group", "top_k", "rank", "vocab")] + \
               [("rms_eps", C.c_float), ("rope_theta", C.c_float),
                ("tap_layer_ids", C.POINTER(C.c_int32)), ("sliding_window", C.c_int32),
                ("sliding_layers", C.POINTER(C.c_int32))]


LAYER_FIELDS = ("input_norm", "post_norm", "q_proj", "k_proj", "v_proj", "o_proj", "q_norm",
                "k_norm", "gate_proj", "up_proj", "down_proj", "attn_base", "attn_kproj",
                "mlp_base", "mlp_kproj")


class dfl_layer_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in LAYER_FIELDS]


class dfl_q4_weight(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("packed", "scales", "biases")]


Q4_FIELDS = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")


class dfl_q4_layer(C.Structure):
    _fields_ = [(n, dfl_q4_weight) for n in Q4_FIELDS]


class dfl_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("fc", "hidden_norm", "norm", "sel_proj", "pred", "succ")] + \
               [("layers", C.POINTER(dfl_layer_weights)), ("q4_layers", C.POINTER(dfl_q4_layer))]


TRACE_FIELDS = ("x_in", "n", "coef", "a", "coef1", "qkv", "attn", "u", "x_mid", "m", "coef_mlp", "i",
                "coef1_mlp", "p", "f", "x_out", "n_next", "h", "tile_max", "cand", "unary", "z", "scores")


class dfl_trace(C.Structure):
    _fields_ = [("layer", C.c_int32)] + [(n, C.c_void_p) for n in TRACE_FIELDS]


CONTEXT_TRACE_FIELDS = ("fc_out", "c", "kv")


class dfl_context_trace(C.Structure):
    _fields_ = [("layer", C.c_int32)] + [(n, C.c_void_p) for n in CONTEXT_TRACE_FIELDS]


_P, _I, _F, _Z = C.c_void_p, C.c_int, C.c_float, C.c_size_t
_SIGS = {
    "dfl_last_error": (C.c_char_p, []),
    "dfl_drafter_load": (_I, [C.POINTER(dfl_config), C.POINTER(dfl_weights), _P, C.POINTER(_P)]),
    "dfl_drafter_free": (None, [_P]),
    "dfl_context_workspace_bytes": (_Z, [_P, _I, _I]),
    "dfl_context_materialize": (_I, [_P, _P, _I, _I, _I, _I, C.POINTER(_P), C.POINTER(_P), _P, _Z, _P]),
    "dfl_draft_workspace_bytes": (_Z, [_P, _I, _I, _I]),
    "dfl_draft_block": (_I, [_P, _P, _P, _I, _I, C.POINTER(_P), C.POINTER(_P), _I, _I, _P, _P, _P,
                             _P, _P, _P, _Z, _P]),
    "dfl_draft_block_traced": (_I, [_P, _P, _P, _I, _I, C.POINTER(_P), C.POINTER(_P), _I, _I, _P, _P, _P,
                                    _P, _P, _P, _Z, C.POINTER(dfl_trace), _P]),
    "dfl_context_materialize_traced": (_I, [_P, _P, _I, _I, _I, _I, C.POINTER(_P), C.POINTER(_P), _P, _Z,
                                            C.POINTER(dfl_context_trace), _P]),
    "dfl_context_append_traced": (_I, [_P, _P, _P, _P, _I, _I, _P, _P, _P, _Z, C.POINTER(dfl_context_trace), _P]),
    "dfl_block_layer": (_I, [_P, _I, _P, _P, _I, _I, _P, _P, _I, _I, _P, _P, _P, _Z, _P]),
    "dfl_rms_norm": (_I, [_P, _I, _I, _I, _P, _F, _P, _I, _P]),
    "dfl_linear_workspace_bytes": (_Z, [_I, _I, _I]),
    "dfl_linear": (_I, [_P, _I, _I, _I, _P, _I, _P, _I, _I, _P, _Z, _P]),
    "dfl_head_norm_rope": (_I, [_P, _I, _I, _I, _I, _P, _F, _F, _P, _I, _P]),
    "dfl_attention_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I]),
    "dfl_block_attention": (_I, [_P, _I, _P, _P, _I, _P, _P, _I, _I, _P, _P, _I, _I, _I, _I, _I, _I, _P,
                                 _I, _P, _Z, _P]),
    "dfl_conv_prepare_workspace_bytes": (_Z, [_I, _I, _I]),
    "dfl_conv_prepare": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _Z, _P]),
    "dfl_conv_finish": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "dfl_candidates_workspace_bytes": (_Z, [_I, _I, _I]),
    "dfl_compute_candidates": (_I, [_P, _I, _I, _I, _P, _P, _P, _Z, _P]),
    "dfl_compute_candidates_static": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "dfl_selector_project_workspace_bytes": (_Z, [_I, _I, _I]),
    "dfl_selector_project": (_I, [_P, _I, _I, _P, _I, _P, _P, _Z, _P]),
    "dfl_score_edges": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _P, _P]),
    "dfl_select_path": (_I, [_P, _P, _I, _I, _I, _P, _P]),
    "dfl_tile_maxima": (_I, [_P, _I, _I, _P, _P]),
    "dfl_select_tokens": (_I, [_P, _P, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    "dfl_select_tokens_projected": (_I, [_P, _I, _I, _I, _I, _P, _I, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "dfl_bind_target": (_I, [_P, _P, _P, _I, _P]),
    "dfl_context_append_workspace_bytes": (_Z, [_P, _I, _I]),
    "dfl_linear_q4": (_I, [_P, _I, _I, _I, _P, _P, _P, _I, _P, _I, _I, _P, _Z, _P]),
    "dfl_context_append": (_I, [_P, _P, _P, _P, _I, _I, _P, _P, _P, _Z, _P]),
    "dfl_set_timed_kernel": (_I, [_P, _I]),
    "dfl_read_kernel_time": (_I, [_P, C.POINTER(C.c_double), C.POINTER(C.c_int64),
                                  C.POINTER(C.c_double)]),
}

_lib = None


def lib() -> C.CDLL:
    """Load libdflash2.so (built in-tree by the package's build step); fail loudly if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() first")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_symbols() -> list[str]:
    return list(_SIGS)


def _check(code: int) -> None:
    if code != DFL_OK:
        raise DflError(code, lib().dfl_last_error().decode())


def _ptr(t: torch.Tensor | None, dtype=None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _bf(t):
    return _ptr(t, torch.bfloat16)


def _f32(t):
    return _ptr(t, torch.float32)


def _i32(t):
    return _ptr(t, torch.int32)


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr_array(ts) -> C.Array:
    arr = (C.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _bf(t)
    return arr


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Device workspace of at least nbytes (256-byte aligned by the caching allocator)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------- config/load

def make_config(dims, tap_layer_ids=None) -> tuple[dfl_config, object]:
    ids = None
    if tap_layer_ids is not None:
        ids = (C.c_int32 * len(tap_layer_ids))(*tap_layer_ids)
    kinds = None
    if getattr(dims, "sliding_layers", None) is not None:
        kinds = (C.c_int32 * dims.layers)(*[1 if f else 0 for f in dims.sliding_layers])
    cfg = dfl_config(dims.hidden, dims.layers, dims.heads, dims.kv_heads, dims.head_dim,
                     dims.intermediate, dims.n_taps, dims.block_size, dims.conv_taps,
                     dims.conv_group, dims.top_k, dims.rank, dims.vocab, dims.rms_eps,
                     dims.rope_theta, C.cast(ids, C.POINTER(C.c_int32)) if ids is not None else None,
                     int(getattr(dims, "sliding_window", 0) or 0),
                     C.cast(kinds, C.POINTER(C.c_int32)) if kinds is not None else None)
    return cfg, (ids, kinds)


def dfl_drafter_load(dims, weights: dict, tap_layer_ids=None, stream=None, q4_weights=None) -> int:
    """weights: checkpoint name -> bf16 device tensor (the drafter's checkpoint names).
    q4_weights: None, or checkpoint name of a layer projection without ".weight" ->
    (packed int32 [N, K/8], scales bf16 [N, K/64], biases bf16 [N, K/64]); the projections
    then load from these and their bf16 entries in `weights` are not read."""
    cfg, keep = make_config(dims, tap_layer_ids)
    layers = (dfl_layer_weights * dims.layers)()
    q4_layers = None
    names = {"input_norm": "input_layernorm.weight", "post_norm": "post_attention_layernorm.weight",
             "q_proj": "self_attn.q_proj.weight", "k_proj": "self_attn.k_proj.weight",
             "v_proj": "self_attn.v_proj.weight", "o_proj": "self_attn.o_proj.weight",
             "q_norm": "self_attn.q_norm.weight", "k_norm": "self_attn.k_norm.weight",
             "gate_proj": "mlp.gate_proj.weight", "up_proj": "mlp.up_proj.weight",
             "down_proj": "mlp.down_proj.weight", "attn_base": "attention_conv.base_kernel",
             "attn_kproj": "attention_conv.kernel_projection.weight",
             "mlp_base": "mlp_conv.base_kernel", "mlp_kproj": "mlp_conv.kernel_projection.weight"}
    for i in range(dims.layers):
        for f, n in names.items():
            if q4_weights is not None and f in Q4_FIELDS:
                continue
            setattr(layers[i], f, _bf(weights[f"layers.{i}.{n}"]))
    if q4_weights is not None:
        q4_layers = (dfl_q4_layer * dims.layers)()
        for i in range(dims.layers):
            for f in Q4_FIELDS:
                packed, sc, bi = q4_weights[f"layers.{i}.{names[f][:-len('.weight')]}"]
                setattr(q4_layers[i], f, dfl_q4_weight(_i32(packed), _bf(sc), _bf(bi)))
    w = dfl_weights(_bf(weights["fc.weight"]), _bf(weights["hidden_norm.weight"]),
                    _bf(weights["norm.weight"]),
                    _bf(weights["candidate_selector.hidden_projection.weight"]),
                    _bf(weights["candidate_selector.predecessor_codebook"]),
                    _bf(weights["candidate_selector.successor_codebook"]),
                    C.cast(layers, C.POINTER(dfl_layer_weights)),
                    C.cast(q4_layers, C.POINTER(dfl_q4_layer)) if q4_layers is not None else None)
    h = C.c_void_p()
    _check(lib().dfl_drafter_load(C.byref(cfg), C.byref(w), _stream(stream), C.byref(h)))
    del keep
    return h.value


def dfl_drafter_free(handle: int) -> None:
    if handle:
        lib().dfl_drafter_free(handle)


def dfl_context_workspace_bytes(handle, B, L) -> int:
    return lib().dfl_context_workspace_bytes(handle, B, L)


def dfl_context_materialize(handle, taps, B, L, row_offset, Lcap, K: list, V: list, ws, stream=None):
    _check(lib().dfl_context_materialize(handle, _bf(taps), B, L, row_offset, Lcap, _ptr_array(K),
                                         _ptr_array(V), _ptr(ws), ws.numel(), _stream(stream)))


def dfl_context_append_workspace_bytes(handle, B, rows) -> int:
    return lib().dfl_context_append_workspace_bytes(handle, B, rows)


def dfl_context_append(handle, taps, row_offsets, starts, B, Lcap, K: list, V: list, ws, stream=None):
    """row_offsets, starts: host integer sequences (B+1 and B entries)."""
    offs = (C.c_int32 * (B + 1))(*[int(x) for x in row_offsets])
    st = (C.c_int32 * B)(*[int(x) for x in starts])
    _check(lib().dfl_context_append(handle, _bf(taps), C.cast(offs, C.c_void_p), C.cast(st, C.c_void_p), B, Lcap,
                                    _ptr_array(K), _ptr_array(V), _ptr(ws), ws.numel(), _stream(stream)))


def dfl_draft_workspace_bytes(handle, B, G, Lmax) -> int:
    return lib().dfl_draft_workspace_bytes(handle, B, G, Lmax)


def dfl_draft_block(handle, embeds, anchors, B, G, K: list, V: list, Lcap, Lmax, ctx_len, pos0,
                    lm_head, tokens, logits_out, ws, stream=None):
    kp = _ptr_array(K) if K else None
    vp = _ptr_array(V) if V else None
    _check(lib().dfl_draft_block(handle, _bf(embeds), _i32(anchors), B, G, kp, vp, Lcap, Lmax,
                                 _i32(ctx_len), _i32(pos0), _bf(lm_head), _i32(tokens),
                                 _f32(logits_out), _ptr(ws), ws.numel(), _stream(stream)))


def dfl_draft_block_traced(handle, embeds, anchors, B, G, K: list, V: list, Lcap, Lmax, ctx_len, pos0,
                           lm_head, tokens, logits_out, ws, layer: int, stages: dict, stream=None):
    """dfl_draft_block that also copies the stages named in `stages` (dfl_trace field name ->
    device tensor of that stage's shape and dtype) of layer `layer` and of the tail."""
    unknown = set(stages) - set(TRACE_FIELDS)
    if unknown:
        raise ValueError(f"unknown trace stages {sorted(unknown)}")
    tr = dfl_trace(int(layer), *[_ptr(stages.get(n)) for n in TRACE_FIELDS])
    kp = _ptr_array(K) if K else None
    vp = _ptr_array(V) if V else None
    _check(lib().dfl_draft_block_traced(handle, _bf(embeds), _i32(anchors), B, G, kp, vp, Lcap, Lmax,
                                        _i32(ctx_len), _i32(pos0), _bf(lm_head), _i32(tokens),
                                        _f32(logits_out), _ptr(ws), ws.numel(), C.byref(tr), _stream(stream)))


def dfl_context_materialize_traced(handle, taps, B, L, row_offset, Lcap, K: list, V: list, ws, layer: int,
                                   stages: dict, stream=None):
    unknown = set(stages) - set(CONTEXT_TRACE_FIELDS)
    if unknown:
        raise ValueError(f"unknown context trace stages {sorted(unknown)}")
    tr = dfl_context_trace(int(layer), *[_ptr(stages.get(n)) for n in CONTEXT_TRACE_FIELDS])
    _check(lib().dfl_context_materialize_traced(handle, _bf(taps), B, L, row_offset, Lcap, _ptr_array(K),
                                                _ptr_array(V), _ptr(ws), ws.numel(), C.byref(tr), _stream(stream)))


def dfl_context_append_traced(handle, taps, row_offsets, starts, B, Lcap, K: list, V: list, ws, layer: int,
                              stages: dict, stream=None):
    unknown = set(stages) - set(CONTEXT_TRACE_FIELDS)
    if unknown:
        raise ValueError(f"unknown context trace stages {sorted(unknown)}")
    tr = dfl_context_trace(int(layer), *[_ptr(stages.get(n)) for n in CONTEXT_TRACE_FIELDS])
    offs = (C.c_int32 * (B + 1))(*[int(x) for x in row_offsets])
    st = (C.c_int32 * B)(*[int(x) for x in starts])
    _check(lib().dfl_context_append_traced(handle, _bf(taps), C.cast(offs, C.c_void_p), C.cast(st, C.c_void_p), B,
                                           Lcap, _ptr_array(K), _ptr_array(V), _ptr(ws), ws.numel(), C.byref(tr),
                                           _stream(stream)))


def dfl_block_layer(handle, layer, x_in, x_out, B, G, K, V, Lcap, Lmax, ctx_len, pos0, ws, stream=None):
    _check(lib().dfl_block_layer(handle, layer, _bf(x_in), _bf(x_out), B, G, _bf(K), _bf(V), Lcap, Lmax,
                                 _i32(ctx_len), _i32(pos0), _ptr(ws), ws.numel(), _stream(stream)))


def dfl_rms_norm(x, rows, H, ldx, gamma, eps, y, ldy, stream=None):
    _check(lib().dfl_rms_norm(_bf(x), rows, H, ldx, _bf(gamma), eps, _bf(y), ldy, _stream(stream)))


def dfl_linear_workspace_bytes(M, N, K) -> int:
    return lib().dfl_linear_workspace_bytes(M, N, K)


def dfl_linear(x, M, K, ldx, W, N, y, ldy, out_f32, ws, stream=None):
    _check(lib().dfl_linear(_bf(x), M, K, ldx, _bf(W), N, _ptr(y, torch.float32 if out_f32 else torch.bfloat16),
                            ldy, int(out_f32), _ptr(ws) if ws is not None else None,
                            ws.numel() if ws is not None else 0, _stream(stream)))


def dfl_linear_q4(x, M, K, ldx, packed, scales, biases, N, y, ldy, out_f32, ws, stream=None):
    """packed: int32 tensor [N, K/8] of 4-bit fields (bit patterns of the uint32 words)."""
    _check(lib().dfl_linear_q4(_bf(x), M, K, ldx, _i32(packed), _bf(scales), _bf(biases), N,
                               _ptr(y, torch.float32 if out_f32 else torch.bfloat16), ldy, int(out_f32),
                               _ptr(ws) if ws is not None else None, ws.numel() if ws is not None else 0,
                               _stream(stream)))


def dfl_head_norm_rope(x, rows, heads, D, ldx, gamma, eps, theta, pos0, rows_per_req, stream=None):
    _check(lib().dfl_head_norm_rope(_bf(x), rows, heads, D, ldx, _bf(gamma), eps, theta, _i32(pos0),
                                    rows_per_req, _stream(stream)))


def dfl_attention_workspace_bytes(B, G, NH, NKV, D, Lmax) -> int:
    return lib().dfl_attention_workspace_bytes(B, G, NH, NKV, D, Lmax)


def dfl_block_attention(q, ldq, kb, vb, ldkv, K, V, Lcap, Lmax, ctx_len, B, G, NH, NKV, D, out, ldo, ws,
                        stream=None, pos0=None, window=0):
    _check(lib().dfl_block_attention(_bf(q), ldq, _bf(kb), _bf(vb), ldkv, _bf(K), _bf(V), Lcap, Lmax,
                                     _i32(ctx_len), _i32(pos0), int(window), B, G, NH, NKV, D, _bf(out), ldo,
                                     _ptr(ws), ws.numel(), _stream(stream)))


def dfl_conv_prepare_workspace_bytes(T, H, grp) -> int:
    return lib().dfl_conv_prepare_workspace_bytes(T, H, grp)


def dfl_conv_prepare(x, T, H, G, grp, kproj, base, out, coef1, ws, stream=None):
    _check(lib().dfl_conv_prepare(_bf(x), T, H, G, grp, _bf(kproj), _bf(base), _bf(out), _f32(coef1),
                                  _ptr(ws), ws.numel(), _stream(stream)))


def dfl_conv_finish(y, coef1, base, T, H, G, grp, residual, out, stream=None):
    _check(lib().dfl_conv_finish(_bf(y), _f32(coef1), _bf(base), T, H, G, grp, _bf(residual), _bf(out),
                                 _stream(stream)))


def dfl_candidates_workspace_bytes(N, V, K) -> int:
    return lib().dfl_candidates_workspace_bytes(N, V, K)


def dfl_compute_candidates(logits, N, V, K, ids, unary, ws, stream=None):
    _check(lib().dfl_compute_candidates(_f32(logits), N, V, K, _i32(ids), _f32(unary), _ptr(ws), ws.numel(),
                                        _stream(stream)))


CANDIDATES_STATIC_MAX_TILES = 1 << 20


def dfl_compute_candidates_static(logits, N, V, K, ids, unary, stream=None):
    _check(lib().dfl_compute_candidates_static(_f32(logits), N, V, K, _i32(ids), _f32(unary), _stream(stream)))


def dfl_selector_project_workspace_bytes(N, H, R) -> int:
    return lib().dfl_selector_project_workspace_bytes(N, H, R)


def dfl_selector_project(h, N, H, proj, R, z, ws, stream=None):
    _check(lib().dfl_selector_project(_bf(h), N, H, _bf(proj), R, _f32(z), _ptr(ws) if ws is not None else None,
                                      ws.numel() if ws is not None else 0, _stream(stream)))


def dfl_score_edges(cand, unary, z, anchors, B, S, K, R, pred, succ, V, scores, stream=None):
    _check(lib().dfl_score_edges(_i32(cand), _f32(unary), _f32(z), _i32(anchors), B, S, K, R, _bf(pred),
                                 _bf(succ), V, _f32(scores), _stream(stream)))


def dfl_select_path(scores, cand, B, S, K, tokens, stream=None):
    _check(lib().dfl_select_path(_f32(scores), _i32(cand), B, S, K, _i32(tokens), _stream(stream)))


def dfl_tile_maxima(logits, N, V, tile_max, stream=None):
    _check(lib().dfl_tile_maxima(_f32(logits), N, V, _f32(tile_max), _stream(stream)))


def dfl_select_tokens(logits, tile_max, B, S, V, K, z, R, anchors, pred, succ, cand, unary, scores, tokens,
                      stream=None):
    _check(lib().dfl_select_tokens(_f32(logits), _f32(tile_max), B, S, V, K, _f32(z), R, _i32(anchors), _bf(pred),
                                   _bf(succ), _i32(cand), _f32(unary), _f32(scores), _i32(tokens), _stream(stream)))


def dfl_select_tokens_projected(logits, B, S, V, K, h, H, proj, R, z, anchors, pred, succ, cand, unary, scores,
                                tokens, stream=None):
    _check(lib().dfl_select_tokens_projected(_f32(logits), B, S, V, K, _bf(h), H, _bf(proj), R, _f32(z),
                                             _i32(anchors), _bf(pred), _bf(succ), _i32(cand), _f32(unary),
                                             _f32(scores), _i32(tokens), _stream(stream)))


def dfl_bind_target(handle, lm_head, vocab_ids=None, stream=None):
    """vocab_ids: optional host sequence of token ids (a draft vocabulary)."""
    ids = None
    if vocab_ids is not None:
        ids = (C.c_int32 * len(vocab_ids))(*[int(i) for i in vocab_ids])
    _check(lib().dfl_bind_target(handle, _bf(lm_head), C.cast(ids, C.c_void_p) if ids is not None else None,
                                 len(vocab_ids) if vocab_ids is not None else 0, _stream(stream)))


def dfl_set_timed_kernel(handle, kclass: int | str):
    k = KERNEL_CLASSES.index(kclass) if isinstance(kclass, str) else kclass
    _check(lib().dfl_set_timed_kernel(handle, k))


def dfl_read_kernel_time(handle) -> tuple[float, int, float]:
    ms, n, by = C.c_double(), C.c_int64(), C.c_double()
    _check(lib().dfl_read_kernel_time(handle, C.byref(ms), C.byref(n), C.byref(by)))
    return ms.value, n.value, by.value
