"""One drafter forward (all K draft tokens of every request) through libpe.

``DraftStep`` uploads a drafter's weights and one decode step's inputs to
device memory once, preallocates every output and workspace, and ``run()``
issues the four stage calls on the current stream:
pe_build_draft_batch -> pe_fuse_hidden -> pe_draft_layer -> pe_lm_head_argmax.
Host code here only moves arrays and passes pointers.
"""
import numpy as np
import torch

from . import _lib as L


def to_device(a, device, dtype=None):
    """numpy array -> device tensor.  uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


WEIGHT_NAMES = ("embed", "stream_gain", "w_fc", "attn_gain", "w_qkv", "w_o", "mlp_gain", "w_gate", "w_up",
                "w_down", "final_gain", "w_lm", "h_shared")
LINEAR_NAMES = ("w_fc", "w_qkv", "w_o", "w_gate", "w_up", "w_down", "w_lm")


def upload_weights(weights, device):
    """Device copies of the drafter parameters, linear weights packed by libpe."""
    out = {}
    for k in WEIGHT_NAMES:
        t = to_device(weights[k], device)
        if k in LINEAR_NAMES:
            t = L.pe_pack_weight(t)
        out[k] = t
    torch.cuda.synchronize(device)
    return out


class DraftStep:
    def __init__(self, dims, weights, case, device="cuda", weights_on_device=None):
        """dims: object with hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab,
        mask_token_id, eps, dtype ("f32" | "bf16").  weights: dict of numpy
        arrays (storage dtype; gains float32).  case: the decode-step inputs
        (cu_window, n_rej, kv_len, kv_base, window_ids/pos/hrow, new_token,
        ctx_hrow, target_hidden, k_cache, v_cache, R, K, kv_rows)."""
        self.dims = dims
        self.device = torch.device(device)
        dev = self.device
        self.cdims = L.dims_struct(dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ffn,
                                   dims.vocab, dims.mask_token_id, dims.eps, dims.dtype)
        if weights_on_device is None:
            weights_on_device = upload_weights(weights, dev)
        self.w = weights_on_device
        self.cw = L.weights_struct(self.w)
        c = case
        self.R, self.K = int(c["R"]), int(c["K"])
        self.total_w = int(c["cu_window"][-1])
        self.T = self.total_w + self.R * self.K
        self.kv_rows = int(c["kv_rows"])
        self.target_rows = int(c["target_hidden"].shape[0])
        W = np.diff(c["cu_window"])
        self.max_pos = int(np.max(c["kv_len"].astype(np.int64) + W + self.K))
        i32 = torch.int32
        self.inp = {k: to_device(c[k].astype(np.int32), dev) for k in
                    ("cu_window", "n_rej", "kv_len", "kv_base", "window_ids", "window_pos", "window_hrow",
                     "new_token", "ctx_hrow")}
        self.target_hidden = to_device(c["target_hidden"], dev)
        self.k_cache = to_device(c["k_cache"].view(np.uint16) if dims.dtype == "bf16" else c["k_cache"], dev)
        self.v_cache = to_device(c["v_cache"].view(np.uint16) if dims.dtype == "bf16" else c["v_cache"], dev)
        T, RK, d = self.T, self.R * self.K, dims.hidden
        sdt = torch.bfloat16 if dims.dtype == "bf16" else torch.float32
        self.batch = {
            "draft_ids": torch.empty(T, dtype=i32, device=dev),
            "draft_pos": torch.empty(T, dtype=i32, device=dev),
            "slot_mapping": torch.empty(T, dtype=i32, device=dev),
            "hidden_src": torch.empty(T, dtype=i32, device=dev),
            "req_of_row": torch.empty(T, dtype=i32, device=dev),
            "rejected": torch.empty(T, dtype=torch.uint8, device=dev),
            "masked": torch.empty(T, dtype=torch.uint8, device=dev),
            "query_rows": torch.empty(RK, dtype=i32, device=dev),
            "cu_draft": torch.empty(self.R + 1, dtype=i32, device=dev),
            "draft_hidden": torch.empty((T, 3, d), dtype=sdt, device=dev),
        }
        self.cbatch = L.batch_struct(self.batch)
        self.x0 = torch.zeros((T, d), dtype=torch.float32, device=dev)
        self.x_out = torch.empty((RK, d), dtype=torch.float32, device=dev)
        self.tokens = torch.empty(RK, dtype=i32, device=dev)
        self.ws_fuse = torch.empty(L.pe_fuse_hidden_workspace(self.cdims, T), dtype=torch.uint8, device=dev)
        self.ws_layer = torch.empty(L.pe_draft_layer_workspace(self.cdims, T, self.R, self.K, self.max_pos),
                                    dtype=torch.uint8, device=dev)
        self.ws_lm = torch.empty(L.pe_lm_head_argmax_workspace(self.cdims, RK), dtype=torch.uint8, device=dev)
        self.logits = None

    def build_batch(self):
        i = self.inp
        L.pe_build_draft_batch(self.cdims, self.R, self.K, self.total_w, self.target_rows, i["cu_window"],
                               i["n_rej"], i["kv_len"], i["kv_base"], i["window_ids"] if self.total_w else None,
                               i["window_pos"] if self.total_w else None,
                               i["window_hrow"] if self.total_w else None, i["new_token"], i["ctx_hrow"],
                               self.target_hidden, self.w["h_shared"], self.cbatch)

    def fuse(self):
        L.pe_fuse_hidden(self.cdims, self.cw, self.T, self.batch["draft_hidden"], self.batch["rejected"],
                         self.batch["draft_ids"], self.x0, workspace=self.ws_fuse)

    def layer(self):
        L.pe_draft_layer(self.cdims, self.cw, self.T, self.R, self.K, self.x0, self.cbatch, self.inp["kv_base"],
                         self.k_cache, self.v_cache, self.kv_rows, self.max_pos, self.x_out, workspace=self.ws_layer)

    def lm_head(self, with_logits=False):
        if with_logits and self.logits is None:
            self.logits = torch.empty((self.R * self.K, self.dims.vocab), dtype=torch.float32, device=self.device)
        L.pe_lm_head_argmax(self.cdims, self.cw, self.R * self.K, self.x_out, self.tokens,
                            self.logits if with_logits else None, workspace=self.ws_lm)

    def run(self, with_logits=False):
        self.build_batch()
        self.fuse()
        self.layer()
        self.lm_head(with_logits)
        return self.tokens


class GraphStep:
    """A DraftStep captured once into a HIP graph (torch.cuda.CUDAGraph) and
    replayed.  Every stage call only launches kernels on the current stream
    and uses preallocated buffers, so the whole drafter forward replays as
    one graph launch."""

    def __init__(self, step, warmup=2):
        self.step = step
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(warmup):
                step.run()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            step.run()
        torch.cuda.synchronize()

    def replay(self):
        self.graph.replay()
        return self.step.tokens
