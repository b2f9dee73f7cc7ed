"""Helpers for the GPU parity tests: move a seeded workload to the device, run
the C-ABI entry points, bring results back.  Imports torch lazily."""
from __future__ import annotations

import sys

import numpy as np


def say(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def device():
    import torch
    return torch.device("cuda", 0)


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device())


class GpuLayer:
    """One workload layer on the device: inputs, arena, buffers."""

    def __init__(self, lay, T=None, x_bits=None, expert_slot=None, arena=None, act_format=0):
        import torch
        from resident_expert_routing_amd import runtime as R
        self.lay = lay
        cfg = lay.cfg
        self.x_bits = lay.x_bits if x_bits is None else x_bits
        self.T = self.x_bits.shape[0] if T is None else T
        self.H, self.E, self.k, self.I = cfg.H, cfg.E, cfg.k, cfg.I
        self.expert_slot_np = lay.expert_slot if expert_slot is None else expert_slot
        self.S = lay.S
        self.x = to_dev(self.x_bits.view(np.int16)) if self.T else \
            torch.empty((0, self.H), dtype=torch.int16, device=device())
        self.w_router = to_dev(lay.w_router)
        self.bias = to_dev(lay.bias)
        self.expert_slot = to_dev(self.expert_slot_np.astype(np.int32))
        self.buf = R.LayerBuffers(self.T, self.H, self.E, self.k, self.I, self.S, device(),
                                  act_format=act_format)
        if arena is None:
            lay.prepack()
            arena = R.Arena(self.S, self.H, self.I, device())
            arena.upload(lambda s: lay.content_bytes(lay.slot_content()[s]))
        self.arena = arena
        self.hist = torch.zeros(self.E, dtype=torch.float64, device=device())

    def route(self, stream=None):
        from resident_expert_routing_amd import runtime as R
        R.route(self.buf, self.x, self.w_router, self.bias, self.expert_slot, stream)

    def demand(self, stream=None):
        from resident_expert_routing_amd import runtime as R
        R.demand(self.buf, self.hist, stream)

    def experts(self, stream=None):
        from resident_expert_routing_amd import runtime as R
        R.experts(self.buf, self.arena.ptr(), self.arena.stride, stream)

    def sync(self):
        import torch
        torch.cuda.synchronize()

    def routing(self) -> dict:
        self.sync()
        b = self.buf
        f = lambda t: t.cpu().numpy()
        return {"topk_expert": f(b.topk_expert), "topk_score": f(b.topk_score),
                "sel_expert": f(b.sel_expert), "sel_weight": f(b.sel_weight),
                "sel_slot": f(b.sel_slot), "slot_offsets": f(b.slot_offsets),
                "perm": f(b.perm), "xq": f(b.xq)}

    def out_f64(self) -> np.ndarray:
        self.sync()
        bits = self.buf.out.cpu().numpy().view(np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    def slot_bytes_fn(self):
        lay = self.lay
        sc = lay.slot_content()
        return lambda s: lay.content_bytes(sc[s])
