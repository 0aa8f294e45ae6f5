"""Torch-side conveniences over the C ABI: device memory, streams and argument
structs.  Nothing here computes any part of the layer; every step of the
forward pass runs in libecf's kernels (or its host expert threads)."""
from __future__ import annotations

import torch

from . import _lib as L

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _ptr(t):
    return 0 if t is None else int(t.data_ptr())


def blob_sections(shape: L.Shape):
    """[(name, byte offset)] of one expert blob, in ecf_expert_layout order."""
    offs = L.ecf_expert_layout(shape)
    names = ["w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"]
    n = 6 if shape.w_dtype == L.ECF_MXFP4 else 3
    return list(zip(names[:n], offs[:n]))


def pack_expert(shape: L.Shape, tensors: dict, blob: torch.Tensor):
    """Copy one expert's tensors into a uint8 blob view at the layout offsets."""
    for name, off in blob_sections(shape):
        t = tensors[name].contiguous()
        raw = t.view(torch.uint8).reshape(-1)
        blob[off:off + raw.numel()].copy_(raw)


class ExpertPool:
    """All experts of one layer resident in one device buffer [E, slot_bytes]."""

    def __init__(self, shape: L.Shape, device="cuda", n_experts=None):
        self.shape = shape
        self.slot_bytes = L.ecf_expert_bytes(shape)
        E = n_experts or shape.n_experts
        self.buf = torch.empty((E, self.slot_bytes), dtype=torch.uint8, device=device)
        base = self.buf.data_ptr()
        self.ptrs = torch.tensor([base + e * self.slot_bytes for e in range(E)], dtype=torch.int64,
                                 device=device)

    def load(self, e: int, tensors: dict):
        pack_expert(self.shape, tensors, self.buf[e])


class Layer:
    """One MoE layer call site: owns its workspace and builds LayerArgs.

    LayerArgs carries raw device addresses only: every tensor passed to args()
    must stay referenced until the forward call's work has finished on the
    stream (a temporary such as `w.cuda()` would be freed, and its memory
    reused, while the kernels still read it)."""

    def __init__(self, shape: L.Shape, max_tokens: int, device="cuda"):
        self.shape = shape
        self.max_tokens = max_tokens
        self.ws_bytes = L.ecf_workspace_bytes(shape, max_tokens)
        self.ws = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=device)
        base = self.ws.data_ptr()
        self.ws_ptr = (base + 255) & ~255
        self.device = device

    def args(self, *, layer=0, router_w=None, router_logits=None, expert_ptrs=None, cache=None,
             b_p=0.4, b_h=1.0, q_mode=L.ECF_Q_AUTO, q_fixed=0, path=L.ECF_PATH_AUTO, stream=None,
             copy_stream=None, residual=None, out_act=None, topk_idx=None, topk_gate=None, counts=None,
             perm=None, logits_out=None) -> L.LayerArgs:
        a = L.LayerArgs()
        a.shape = self.shape
        a.layer = layer
        a.d_router_w = _ptr(router_w) or None
        a.d_router_logits = _ptr(router_logits) or None
        a.d_expert_ptrs = _ptr(expert_ptrs) or None
        a.cache = cache or None
        a.b_p, a.b_h = float(b_p), float(b_h)
        a.q_mode, a.q_fixed, a.path = int(q_mode), int(q_fixed), int(path)
        a.d_ws = self.ws_ptr
        a.ws_bytes = self.ws_bytes
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        a.stream = st.cuda_stream or None
        a.copy_stream = (copy_stream.cuda_stream or None) if copy_stream is not None else None
        a.d_residual = _ptr(residual) or None
        a.d_out_act = _ptr(out_act) or None
        a.d_topk_idx = _ptr(topk_idx) or None
        a.d_topk_gate = _ptr(topk_gate) or None
        a.d_counts = _ptr(counts) or None
        a.d_perm = _ptr(perm) or None
        a.d_logits = _ptr(logits_out) or None
        return a

    def forward(self, args: L.LayerArgs, x: torch.Tensor, out: torch.Tensor, want_stats=True):
        T = x.shape[0]
        if T > self.max_tokens:
            raise ValueError(f"{T} tokens > workspace capacity {self.max_tokens}")
        assert x.is_contiguous() and out.is_contiguous() and out.dtype == torch.float32
        return L.moe_layer_forward(args, x.data_ptr(), T, out.data_ptr(), want_stats)
