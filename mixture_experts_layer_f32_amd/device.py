"""Device-memory plumbing around the C ABI: upload host arrays with torch,
hold a plan and its workspace, and enqueue forwards.  No arithmetic of the
layer happens here."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import (MOE_PATH_AUTO, Plan, mat, moe_forward, moe_forward_block, moe_plan, moe_plan_set,
               moe_workspace_h_offset, moe_workspace_size)


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Host numpy array -> device tensor of the same bytes (uint16 bf16 bits kept as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    elif a.dtype == np.uint32:
        t = torch.from_numpy(a.view(np.int32))
    else:
        t = torch.from_numpy(a)
    return t.to(device)


@dataclass
class DeviceWeights:
    """One layer's weights in device memory: router f32 [E, d] and the three
    expert matrix families (codes + scales, leading expert axis)."""
    w_router: torch.Tensor
    gate_q: torch.Tensor
    gate_s: torch.Tensor
    up_q: torch.Tensor
    up_s: torch.Tensor
    down_q: torch.Tensor
    down_s: torch.Tensor

    @classmethod
    def upload(cls, w_router, gate_q, gate_s, up_q, up_s, down_q, down_s, device="cuda"):
        return cls(*(to_dev(a, device) for a in (w_router, gate_q, gate_s, up_q, up_s, down_q,
                                                  down_s)))

    def mats(self):
        return (mat(self.gate_q, self.gate_s), mat(self.up_q, self.up_s),
                mat(self.down_q, self.down_s))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.w_router, self.gate_q, self.gate_s, self.up_q, self.up_s, self.down_q,
                    self.down_s))


class Runner:
    """A plan for one layer shape plus a workspace sized for `max_tokens`."""

    def __init__(self, d: int, f: int, E: int, k: int, fmt: str, renorm: bool, max_tokens: int,
                 path: int = MOE_PATH_AUTO, device="cuda", act_fmt: int = 0,
                 options: Optional[dict] = None, shared_expert: bool = False):
        self.d, self.f, self.E, self.k = d, f, E, k
        self.device = device
        self.plan: Plan = moe_plan(d, f, E, k, max_tokens, fmt, renorm, path, act_fmt,
                                   shared_expert)
        for opt, val in (options or {}).items():
            moe_plan_set(self.plan, opt, val)
        self.max_tokens = max_tokens
        nbytes = max(moe_workspace_size(self.plan, max_tokens), 256)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)

    def outputs(self, T: int):
        dev = self.device
        return dict(
            out=torch.empty((T, self.d), dtype=torch.float32, device=dev),
            topk_ids=torch.empty((T, self.k), dtype=torch.int32, device=dev),
            topk_w=torch.empty((T, self.k), dtype=torch.float32, device=dev),
            counts=torch.empty((self.E,), dtype=torch.int32, device=dev),
            offsets=torch.empty((self.E + 1,), dtype=torch.int32, device=dev),
            perm=torch.empty((T * self.k,), dtype=torch.int32, device=dev),
        )

    def forward(self, W: DeviceWeights, x: torch.Tensor, bias: Optional[torch.Tensor], outs: dict,
                stream=None) -> None:
        T = x.shape[0]
        g, u, dn = W.mats()
        moe_forward(self.plan, T, x, W.w_router, bias, g, u, dn, outs["out"],
                    outs.get("topk_ids"), outs.get("topk_w"), outs.get("counts"),
                    outs.get("offsets"), outs.get("perm"), self.workspace,
                    self.workspace.numel(), stream)

    def forward_block(self, W: DeviceWeights, WS: DeviceWeights, x: torch.Tensor,
                      bias: Optional[torch.Tensor], residual: torch.Tensor,
                      out_bf16: torch.Tensor, outs: dict, stream=None) -> None:
        """The layer with the shared expert WS (one expert) and the residual
        add: out_bf16 = bf16(residual + routed + shared); outs["out"] gets
        routed + shared in f32 (if present)."""
        T = x.shape[0]
        g, u, dn = W.mats()
        moe_forward_block(self.plan, T, x, W.w_router, bias, g, u, dn, WS.mats(), residual,
                          out_bf16, outs.get("out"), outs.get("topk_ids"), outs.get("topk_w"),
                          outs.get("counts"), outs.get("offsets"), outs.get("perm"),
                          self.workspace, self.workspace.numel(), stream)

    def h(self, T: int) -> torch.Tensor:
        """The workspace's h (bf16 bits as int16 [T*k, f], sorted-slot order)."""
        off = moe_workspace_h_offset(self.plan, T)
        n = T * self.k * self.f
        return self.workspace[off:off + 2 * n].view(torch.int16).view(T * self.k, self.f)
