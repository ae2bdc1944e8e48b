"""A packed MoE layer held in device memory: weights packed once with ``moe_pack``, then
``moe_layer_forward`` (or the four stage entry points) per call. Allocation and marshalling
only; the computation is in the library's kernels.
"""
from __future__ import annotations

import torch

from . import native as N


def pack(fmt: str, codes: torch.Tensor, scales, K: int, N_: int):
    """Pack `codes.shape[0]` stored K x N matrices; returns (packed, packed_scales or None)."""
    count = codes.shape[0] if codes.dim() == 3 else 1
    b, sb = N.moe_pack_size(fmt, count, K, N_)
    packed = torch.empty(b, dtype=torch.uint8, device=codes.device)
    pscale = torch.empty(sb, dtype=torch.uint8, device=codes.device) if sb else None
    N.moe_pack(fmt, count, K, N_, codes, scales, packed, pscale)
    return packed, pscale


def pack_expert_set(stored: dict, fmt: str, H: int, I: int) -> dict:
    out = {}
    for name, (K, Nn) in (("gate", (H, I)), ("up", (H, I)), ("down", (I, H))):
        out[name], out[name + "_scale"] = pack(fmt, stored[name], stored[name + "_scale"], K, Nn)
    return out


class PackedLayer:
    """Device-resident packed weights of one layer and a workspace sized for T tokens."""

    def __init__(self, spec, Wr: torch.Tensor, routed: dict, shared: dict | None, T: int | None = None,
                 path: str = "auto"):
        self.spec = spec
        self.shape = N.shape_from_spec(spec, T, path)
        H, I, E = spec.H, spec.I, spec.E
        self.Wr, _ = pack(spec.act, Wr.reshape(1, H, E), None, H, E)
        self.routed = pack_expert_set(routed, spec.w_routed, H, I)
        self.shared = pack_expert_set(shared, spec.w_shared, H, I) if spec.shared else None
        self.ws = torch.empty(N.moe_workspace_size(self.shape), dtype=torch.uint8, device=Wr.device)

    def set_tokens(self, T: int, path: str | None = None):
        p = {0: "auto", 1: "decode", 2: "prefill"}[self.shape.path] if path is None else path
        self.shape = N.shape_from_spec(self.spec, T, p)
        need = N.moe_workspace_size(self.shape)
        if need > self.ws.numel():
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.ws.device)

    def forward_hash(self, x, bias, token_ids, hash_table, y, topk_idx=None, topk_w=None, stream=None):
        N.moe_layer_forward_hash(self.shape, x, self.Wr, bias, token_ids, hash_table, self.routed, self.shared, y,
                                 topk_idx, topk_w, self.ws, stream)
        return y

    def forward(self, x, bias, y, topk_idx=None, topk_w=None, stream=None):
        N.moe_layer_forward(self.shape, x, self.Wr, bias, self.routed, self.shared, y, topk_idx, topk_w,
                            self.ws, stream)
        return y
