"""ctypes binding of libpe.so (include/pe.h).

Argument marshalling only: each function takes torch tensors (device memory)
and Python ints, passes their data pointers and the current HIP stream to the
library, and raises PeError on a non-OK status.  No step of the drafter runs
here.  The library must have been built (``python -m drafter_pe_build_amd.build``);
importing this module without it raises immediately.
"""
import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpe.so")

PE_F32, PE_BF16 = 0, 1
PE_PADDING_SLOT_ID = -1
STATUS = {0: "PE_OK", 1: "PE_ERR_INVALID_ARG", 2: "PE_ERR_UNSUPPORTED", 3: "PE_ERR_DEVICE"}


class PeError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__("%s failed: %s" % (fn, STATUS.get(code, code)))
        self.code = code


class PeDims(ctypes.Structure):
    _fields_ = [("hidden", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("ffn", c_int32), ("vocab", c_int32),
                ("mask_token_id", c_int32), ("eps", c_float), ("dtype", c_int)]


class PeWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("embed", "stream_gain", "w_fc", "attn_gain", "w_qkv", "w_o",
                                         "mlp_gain", "w_gate", "w_up", "w_down", "final_gain", "w_lm")]


class PeBatchOut(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("draft_ids", "draft_pos", "slot_mapping", "hidden_src", "req_of_row",
                                         "rejected", "masked", "query_rows", "cu_draft", "draft_hidden")]


class PeAttnArgs(ctypes.Structure):
    _fields_ = [("num_q", c_int32), ("num_seg", c_int32), ("q_per_seg", c_int32), ("num_kv_rows", c_int32),
                ("n_q_heads", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32), ("scale", c_float),
                ("dtype", c_int), ("q", c_void_p), ("q_row_stride", c_int64), ("q_rows", c_void_p),
                ("k", c_void_p), ("v", c_void_p), ("seg_kv_base", c_void_p), ("q_start", c_void_p),
                ("q_depth", c_void_p), ("q_self_row", c_void_p), ("kv_parent", c_void_p),
                ("max_prefix", c_int32), ("split_len", c_int32), ("out", c_void_p), ("lse", c_void_p),
                ("dbg_count", c_void_p), ("dbg_hash", c_void_p), ("window_sink", c_int32), ("window_len", c_int32),
                ("max_depth", c_int32)]


class PeAttnBwdArgs(ctypes.Structure):
    _fields_ = [("num_rows", c_int32), ("n_pos", c_int32), ("n_groups", c_int32), ("n_q_heads", c_int32),
                ("n_kv_heads", c_int32), ("head_dim", c_int32), ("scale", c_float), ("dtype", c_int),
                ("group_off", c_void_p), ("start", c_void_p), ("depth", c_void_p), ("q", c_void_p),
                ("k", c_void_p), ("v", c_void_p), ("out", c_void_p), ("dout", c_void_p), ("lse", c_void_p),
                ("q_begin", c_int32), ("q_end", c_int32), ("dq", c_void_p), ("dk", c_void_p), ("dv", c_void_p)]


EXPORTS = {
    "pe_status_string": (c_char_p, [c_int]),
    "pe_version": (c_char_p, []),
    "pe_build_draft_batch": (c_int, [POINTER(PeDims), c_int32, c_int32, c_int32, c_int32] + [c_void_p] * 11
                             + [POINTER(PeBatchOut), c_void_p]),
    "pe_packed_weight_bytes": (c_int, [c_int, c_int32, c_int32, POINTER(c_size_t)]),
    "pe_pack_weight": (c_int, [c_int, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    "pe_fuse_hidden": (c_int, [POINTER(PeDims), POINTER(PeWeights), c_int32, c_void_p, c_void_p, c_void_p,
                               c_void_p, c_void_p, c_size_t, c_void_p]),
    "pe_fuse_hidden_workspace": (c_int, [POINTER(PeDims), c_int32, POINTER(c_size_t)]),
    "pe_draft_attention": (c_int, [POINTER(PeAttnArgs), c_void_p, c_size_t, c_void_p]),
    "pe_draft_attention_workspace": (c_int, [POINTER(PeAttnArgs), POINTER(c_size_t)]),
    "pe_draft_layer": (c_int, [POINTER(PeDims), POINTER(PeWeights), c_int32, c_int32, c_int32, c_void_p,
                               POINTER(PeBatchOut), c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                               c_void_p, c_size_t, c_void_p]),
    "pe_draft_layer_workspace": (c_int, [POINTER(PeDims), c_int32, c_int32, c_int32, c_int32, POINTER(c_size_t)]),
    "pe_lm_head_argmax": (c_int, [POINTER(PeDims), POINTER(PeWeights), c_int32, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_size_t, c_void_p]),
    "pe_lm_head_argmax_workspace": (c_int, [POINTER(PeDims), c_int32, POINTER(c_size_t)]),
    "pe_lm_head_argmax_noalloc": (c_int, [POINTER(PeDims), POINTER(PeWeights), c_int32, c_void_p, c_void_p,
                                          c_void_p, c_void_p]),
    "pe_lm_head_loss": (c_int, [POINTER(PeDims), POINTER(PeWeights), c_int32, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_size_t, c_void_p]),
    "pe_lm_head_loss_workspace": (c_int, [POINTER(PeDims), c_int32, POINTER(c_size_t)]),
    "pe_lm_head_kl": (c_int, [POINTER(PeDims), POINTER(PeWeights), c_int32, c_void_p, c_int32, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "pe_lm_head_kl_workspace": (c_int, [POINTER(PeDims), c_int32, POINTER(c_size_t)]),
    "pe_draft_attention_backward": (c_int, [POINTER(PeAttnBwdArgs), c_void_p, c_size_t, c_void_p]),
    "pe_draft_attention_backward_workspace": (c_int, [POINTER(PeAttnBwdArgs), POINTER(c_size_t)]),
}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libpe.so is not built: run `python -m drafter_pe_build_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn, code):
    if code != 0:
        raise PeError(fn, code)


def ptr(t):
    """Device pointer of a tensor (None -> NULL).  Host tensors are refused."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libpe takes device tensors only")
    return ctypes.c_void_p(t.data_ptr())


def stream_handle(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def dims_struct(hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, mask_token_id, eps, dtype):
    return PeDims(hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, mask_token_id, eps,
                  PE_BF16 if dtype == "bf16" else PE_F32)


def weights_struct(w):
    """``w``: dict of device tensors named as the fields of pe_drafter_weights.
    The struct keeps references to the tensors it points at."""
    st = PeWeights(*[ptr(w.get(n)) for n, _ in PeWeights._fields_])
    st._refs = [w.get(n) for n, _ in PeWeights._fields_]
    return st


def batch_struct(b):
    st = PeBatchOut(*[ptr(b[n]) for n, _ in PeBatchOut._fields_])
    st._refs = [b[n] for n, _ in PeBatchOut._fields_]
    return st


def _workspace(nbytes, device, workspace=None):
    if workspace is not None:
        return workspace
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def pe_version():
    return lib().pe_version().decode()


def pe_build_draft_batch(dims, R, K, total_window_rows, target_rows, cu_window, n_rej, kv_len, kv_base,
                         window_ids, window_pos, window_hrow, new_token, ctx_hrow, target_hidden, h_shared,
                         out, stream=None):
    b = out if isinstance(out, PeBatchOut) else batch_struct(out)
    _check("pe_build_draft_batch", lib().pe_build_draft_batch(
        ctypes.byref(dims), R, K, total_window_rows, target_rows, ptr(cu_window), ptr(n_rej), ptr(kv_len),
        ptr(kv_base), ptr(window_ids), ptr(window_pos), ptr(window_hrow), ptr(new_token), ptr(ctx_hrow),
        ptr(target_hidden), ptr(h_shared), ctypes.byref(b), stream_handle(stream)))


def pe_packed_weight_bytes(dtype, N, K):
    n = c_size_t()
    _check("pe_packed_weight_bytes", lib().pe_packed_weight_bytes(dtype, N, K, ctypes.byref(n)))
    return n.value


def pe_pack_weight(w, stream=None):
    """Packed copy (new uint8 device tensor) of the row-major [N, K] device weight w."""
    dt = PE_BF16 if w.dtype == torch.bfloat16 else PE_F32
    if w.dtype not in (torch.bfloat16, torch.float32) or w.dim() != 2 or not w.is_contiguous():
        raise ValueError("pe_pack_weight takes a contiguous 2-D bf16 or f32 tensor")
    N, K = w.shape
    out = torch.empty(pe_packed_weight_bytes(dt, N, K), dtype=torch.uint8, device=w.device)
    _check("pe_pack_weight", lib().pe_pack_weight(dt, N, K, ptr(w), ptr(out), stream_handle(stream)))
    return out


def pe_fuse_hidden_workspace(dims, T):
    n = c_size_t()
    _check("pe_fuse_hidden_workspace", lib().pe_fuse_hidden_workspace(ctypes.byref(dims), T, ctypes.byref(n)))
    return n.value


def pe_fuse_hidden(dims, weights, T, draft_hidden, rejected, ids, x0, workspace=None, stream=None):
    ws = _workspace(pe_fuse_hidden_workspace(dims, T), x0.device, workspace)
    w = weights if isinstance(weights, PeWeights) else weights_struct(weights)
    _check("pe_fuse_hidden", lib().pe_fuse_hidden(
        ctypes.byref(dims), ctypes.byref(w), T, ptr(draft_hidden), ptr(rejected), ptr(ids), ptr(x0),
        ptr(ws), ws.numel(), stream_handle(stream)))


def attn_args(**kw):
    """pe_attn_args from keyword values; tensors become device pointers and
    stay referenced by the returned struct for as long as it lives."""
    a = PeAttnArgs()
    refs = []
    for name, _ in PeAttnArgs._fields_:
        if name in kw:
            v = kw[name]
            if isinstance(v, torch.Tensor):
                refs.append(v)
                v = ptr(v)
            setattr(a, name, v)
    a._refs = refs
    return a


def attn_bwd_args(**kw):
    """pe_attn_bwd_args from keyword values (tensors become device pointers)."""
    a = PeAttnBwdArgs()
    refs = []
    for name, _ in PeAttnBwdArgs._fields_:
        if name in kw:
            v = kw[name]
            if isinstance(v, torch.Tensor):
                refs.append(v)
                v = ptr(v)
            setattr(a, name, v)
    a._refs = refs
    return a


def pe_draft_attention_backward_workspace(args):
    n = c_size_t()
    _check("pe_draft_attention_backward_workspace",
           lib().pe_draft_attention_backward_workspace(ctypes.byref(args), ctypes.byref(n)))
    return n.value


def pe_draft_attention_backward(args, device, workspace=None, stream=None):
    ws = _workspace(pe_draft_attention_backward_workspace(args), device, workspace)
    _check("pe_draft_attention_backward", lib().pe_draft_attention_backward(
        ctypes.byref(args), ptr(ws), ws.numel(), stream_handle(stream)))


def pe_draft_attention_workspace(args):
    n = c_size_t()
    _check("pe_draft_attention_workspace", lib().pe_draft_attention_workspace(ctypes.byref(args), ctypes.byref(n)))
    return n.value


def pe_draft_attention(args, device, workspace=None, stream=None):
    ws = _workspace(pe_draft_attention_workspace(args), device, workspace)
    _check("pe_draft_attention", lib().pe_draft_attention(ctypes.byref(args), ptr(ws), ws.numel(),
                                                          stream_handle(stream)))


def pe_draft_layer_workspace(dims, T, R, K, max_pos):
    n = c_size_t()
    _check("pe_draft_layer_workspace", lib().pe_draft_layer_workspace(ctypes.byref(dims), T, R, K, max_pos,
                                                                      ctypes.byref(n)))
    return n.value


def pe_draft_layer(dims, weights, T, R, K, x0, batch, kv_base, k_cache, v_cache, kv_rows, max_pos, x_out,
                   workspace=None, stream=None):
    ws = _workspace(pe_draft_layer_workspace(dims, T, R, K, max_pos), x0.device, workspace)
    w = weights if isinstance(weights, PeWeights) else weights_struct(weights)
    b = batch if isinstance(batch, PeBatchOut) else batch_struct(batch)
    _check("pe_draft_layer", lib().pe_draft_layer(
        ctypes.byref(dims), ctypes.byref(w), T, R, K, ptr(x0), ctypes.byref(b), ptr(kv_base), ptr(k_cache),
        ptr(v_cache), kv_rows, max_pos, ptr(x_out), ptr(ws), ws.numel(), stream_handle(stream)))


def pe_lm_head_argmax_workspace(dims, n):
    m = c_size_t()
    _check("pe_lm_head_argmax_workspace", lib().pe_lm_head_argmax_workspace(ctypes.byref(dims), n, ctypes.byref(m)))
    return m.value


def pe_lm_head_loss_workspace(dims, n):
    m = c_size_t()
    _check("pe_lm_head_loss_workspace", lib().pe_lm_head_loss_workspace(ctypes.byref(dims), n, ctypes.byref(m)))
    return m.value


def pe_lm_head_loss(dims, weights, n, x, targets, lse=None, loss=None, workspace=None, stream=None):
    ws = _workspace(pe_lm_head_loss_workspace(dims, n), x.device, workspace)
    w = weights if isinstance(weights, PeWeights) else weights_struct(weights)
    _check("pe_lm_head_loss", lib().pe_lm_head_loss(
        ctypes.byref(dims), ctypes.byref(w), n, ptr(x), ptr(targets), ptr(lse), ptr(loss), ptr(ws), ws.numel(),
        stream_handle(stream)))


def pe_lm_head_kl_workspace(dims, n):
    m = c_size_t()
    _check("pe_lm_head_kl_workspace", lib().pe_lm_head_kl_workspace(ctypes.byref(dims), n, ctypes.byref(m)))
    return m.value


def pe_lm_head_kl(dims, weights, n, x, k, target_ids, target_probs, kl, lse=None, w_lm_rows=None, workspace=None,
                  stream=None):
    ws = _workspace(pe_lm_head_kl_workspace(dims, n), x.device, workspace)
    w = weights if isinstance(weights, PeWeights) else weights_struct(weights)
    _check("pe_lm_head_kl", lib().pe_lm_head_kl(
        ctypes.byref(dims), ctypes.byref(w), n, ptr(x), k, ptr(target_ids), ptr(target_probs), ptr(w_lm_rows),
        ptr(lse), ptr(kl), ptr(ws), ws.numel(), stream_handle(stream)))


def pe_lm_head_argmax_noalloc(dims, weights, n, x, tokens, logits=None, stream=None):
    """pe_lm_head_argmax with the library's fixed device array as workspace
    (allocates nothing)."""
    w = weights if isinstance(weights, PeWeights) else weights_struct(weights)
    _check("pe_lm_head_argmax_noalloc", lib().pe_lm_head_argmax_noalloc(
        ctypes.byref(dims), ctypes.byref(w), n, ptr(x), ptr(tokens), ptr(logits), stream_handle(stream)))


def pe_lm_head_argmax(dims, weights, n, x, tokens, logits=None, workspace=None, stream=None):
    ws = _workspace(pe_lm_head_argmax_workspace(dims, n), x.device, workspace)
    w = weights if isinstance(weights, PeWeights) else weights_struct(weights)
    _check("pe_lm_head_argmax", lib().pe_lm_head_argmax(
        ctypes.byref(dims), ctypes.byref(w), n, ptr(x), ptr(tokens), ptr(logits), ptr(ws), ws.numel(),
        stream_handle(stream)))
