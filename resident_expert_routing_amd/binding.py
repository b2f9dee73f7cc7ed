"""ctypes binding of libmoe_arena.so -- argument marshalling only.

Every function here has the name and argument order of the C entry point it
wraps (include/moe_arena.h) and returns that entry point's status code.
Pointer arguments accept an int address, None (NULL) or any object with a
data_ptr() method (a torch tensor); stream arguments accept an int handle,
None (the null stream) or an object with a cuda_stream attribute (a torch
stream); event arguments accept an int, None or an object with cuda_event.
No computation of the layer happens in Python.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_arena.so")

MOE_OK = 0
MOE_EINVAL = -1
MOE_EUNSUPPORTED = -2
MOE_EWORKSPACE = -3
MOE_EHIP = -4
MOE_ESCRATCH = -5
MOE_EIO = -6
MOE_EFORMAT = -7
MOE_NOALLOC_SCRATCH_BYTES = 16 << 20
MOE_OP_ROUTE = 0
MOE_OP_DEMAND = 1
MOE_OP_EXPERTS = 2
MOE_OP_HOT_PICK = 3
MOE_OP_EXPERTS_SHARED = 4
MOE_OP_ACT_MXFP6 = 0x10
MOE_ACT_MXFP4 = 0
MOE_ACT_MXFP6 = 1
MOE_MAX_E = 1024
MOE_MAX_K = 32
MOE_MAX_S = 8192
MOE_MAX_RING_PAIRS = 16384
MOE_MAX_RING = 1024
MOE_MAX_RING_PER_STEP = 64

EXPORTS = ("moe_status_string", "moe_mxfp4_row_bytes", "moe_act_row_bytes", "moe_slot_bytes",
           "moe_slot_sections",
           "moe_workspace_bytes", "moe_route", "moe_demand_accumulate", "moe_experts_forward",
           "moe_experts_forward_noalloc", "moe_ring_plan", "moe_ring_install",
           "moe_history_save", "moe_history_load", "moe_boot_plan", "moe_history_scale",
           "arena_load_slot", "moe_hot_pick", "moe_hot_install", "moe_replan", "moe_test_mxfp4_probe",
           "moe_test_stream_read", "moe_test_mfma_loop")


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


class RouteArgs(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int), ("H", ctypes.c_int), ("E", ctypes.c_int),
                ("k", ctypes.c_int), ("S", ctypes.c_int),
                ("x", ctypes.c_void_p), ("w_router", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("expert_slot", ctypes.c_void_p), ("topk_expert", ctypes.c_void_p),
                ("topk_score", ctypes.c_void_p), ("sel_expert", ctypes.c_void_p),
                ("sel_weight", ctypes.c_void_p), ("sel_slot", ctypes.c_void_p),
                ("slot_offsets", ctypes.c_void_p), ("perm", ctypes.c_void_p),
                ("xq", ctypes.c_void_p), ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t),
                ("stage_events", ctypes.c_void_p), ("hist_row", ctypes.c_void_p),
                ("delta", ctypes.c_void_p), ("reuse_logits", ctypes.c_int),
                ("act_format", ctypes.c_int)]


class ExpertsArgs(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int), ("H", ctypes.c_int), ("I", ctypes.c_int),
                ("k", ctypes.c_int), ("S", ctypes.c_int),
                ("xq", ctypes.c_void_p), ("arena", ctypes.c_void_p),
                ("slot_stride", ctypes.c_size_t), ("slot_offsets", ctypes.c_void_p),
                ("perm", ctypes.c_void_p), ("sel_slot", ctypes.c_void_p),
                ("sel_weight", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t),
                ("stage_events", ctypes.c_void_p), ("defer_slot", ctypes.c_int),
                ("defer_event", ctypes.c_void_p), ("shared_expert", ctypes.c_void_p),
                ("act_format", ctypes.c_int)]


MOE_STAGE_EVENTS = 5
_lib = None


def load() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python resident_expert_routing_amd/build.py`")
    # torch ships its own HIP runtime (libamdhip64.so, soname libamdhip64.so.7).  Loading
    # torch first makes this library's libamdhip64.so.7 dependency resolve to that same
    # copy, so device pointers and streams from torch are valid here; loading this
    # library first would map a second, independent HIP runtime into the process.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.moe_status_string.argtypes = [i]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_mxfp4_row_bytes.argtypes = [i]
    lib.moe_mxfp4_row_bytes.restype = sz
    lib.moe_act_row_bytes.argtypes = [i, i]
    lib.moe_act_row_bytes.restype = sz
    lib.moe_slot_bytes.argtypes = [i, i]
    lib.moe_slot_bytes.restype = sz
    lib.moe_slot_sections.argtypes = [i, i, ctypes.POINTER(sz)]
    lib.moe_slot_sections.restype = i
    lib.moe_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.moe_workspace_bytes.restype = sz
    lib.moe_route.argtypes = [ctypes.POINTER(RouteArgs), vp]
    lib.moe_route.restype = i
    lib.moe_demand_accumulate.argtypes = [vp, vp, i, i, i, vp, vp, vp, sz, vp]
    lib.moe_demand_accumulate.restype = i
    lib.moe_experts_forward.argtypes = [ctypes.POINTER(ExpertsArgs), vp]
    lib.moe_experts_forward.restype = i
    lib.moe_experts_forward_noalloc.argtypes = [ctypes.POINTER(ExpertsArgs), vp]
    lib.moe_experts_forward_noalloc.restype = i
    lib.arena_load_slot.argtypes = [vp, sz, i, i, vp, sz, vp, vp]
    lib.arena_load_slot.restype = i
    lib.moe_hot_pick.argtypes = [vp, vp, i, i, i, vp, i, i, vp, ctypes.c_double, vp, vp, sz,
                                 vp]
    lib.moe_hot_pick.restype = i
    lib.moe_hot_install.argtypes = [vp, vp, i, i, i, vp, vp]
    lib.moe_hot_install.restype = i
    lib.moe_replan.argtypes = [vp, vp, i, i, i, i, vp, vp, vp, ctypes.POINTER(i)]
    lib.moe_replan.restype = i
    lib.moe_ring_plan.argtypes = [vp, vp, i, i, vp, i, i, i, vp, vp]
    lib.moe_ring_plan.restype = i
    lib.moe_ring_install.argtypes = [vp, vp, i, i, vp, i, i, vp]
    lib.moe_ring_install.restype = i
    lib.moe_history_save.argtypes = [ctypes.c_char_p, vp, i, i, ctypes.c_uint64]
    lib.moe_history_save.restype = i
    lib.moe_history_load.argtypes = [ctypes.c_char_p, vp, i, i, ctypes.POINTER(ctypes.c_uint64)]
    lib.moe_history_load.restype = i
    lib.moe_boot_plan.argtypes = [vp, i, i, i, i, vp]
    lib.moe_boot_plan.restype = i
    lib.moe_history_scale.argtypes = [vp, sz, ctypes.c_double, vp]
    lib.moe_history_scale.restype = i
    lib.moe_test_mxfp4_probe.argtypes = [i, vp, vp, vp, vp, vp, vp]
    lib.moe_test_mxfp4_probe.restype = i
    lib.moe_test_stream_read.argtypes = [vp, ctypes.c_size_t, vp, i, vp]
    lib.moe_test_stream_read.restype = i
    lib.moe_test_mfma_loop.argtypes = [i, i, vp, i, vp]
    lib.moe_test_mfma_loop.restype = i
    _lib = lib
    return lib


def _ptr(p) -> int | None:
    if p is None:
        return None
    if isinstance(p, int):
        return p
    return int(p.data_ptr())


def _host(a) -> int | None:
    """Address of a host buffer: None, an int, or a C-contiguous numpy array."""
    if a is None or isinstance(a, int):
        return a
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("host arrays must be C-contiguous")
    return int(a.ctypes.data)


def _stream(s) -> int | None:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _event(e) -> int | None:
    if e is None:
        return None
    if isinstance(e, int):
        return e
    h = int(e.cuda_event)
    if h == 0:
        # torch creates the HIP event on its first record; a null handle would
        # make the library skip the record and a later wait on it a no-op
        raise ValueError("torch.cuda.Event has no HIP event yet: record it once before passing it")
    return h


def _events(evs):
    """Sequence of MOE_STAGE_EVENTS events -> (ctypes array, its address) or (None, None)."""
    if evs is None:
        return None, None
    if len(evs) != MOE_STAGE_EVENTS:
        raise ValueError(f"stage_events needs {MOE_STAGE_EVENTS} events")
    arr = (ctypes.c_void_p * MOE_STAGE_EVENTS)(*[_event(e) for e in evs])
    return arr, ctypes.addressof(arr)


load_lib = load


def status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


moe_status_string = status_string


def moe_mxfp4_row_bytes(K: int) -> int:
    return int(load().moe_mxfp4_row_bytes(int(K)))


def moe_act_row_bytes(K: int, act_format: int) -> int:
    return int(load().moe_act_row_bytes(int(K), int(act_format)))


def moe_slot_bytes(H: int, I: int) -> int:
    return int(load().moe_slot_bytes(int(H), int(I)))


def moe_slot_sections(H: int, I: int):
    out = (ctypes.c_size_t * 6)()
    st = load().moe_slot_sections(int(H), int(I), out)
    if st != MOE_OK:
        raise MoeError(st, "moe_slot_sections")
    return [int(v) for v in out]


def moe_workspace_bytes(op: int, T: int, H: int, E: int, k: int, I: int, S: int) -> int:
    return int(load().moe_workspace_bytes(op, T, H, E, k, I, S))


def moe_route(T, H, E, k, S, x, w_router, bias, expert_slot, topk_expert, topk_score,
              sel_expert, sel_weight, sel_slot, slot_offsets, perm, xq, ws, ws_bytes,
              stream=None, stage_events=None, hist_row=None, delta=None,
              reuse_logits=False, act_format=MOE_ACT_MXFP4) -> int:
    keep, evp = _events(stage_events)
    a = RouteArgs(int(T), int(H), int(E), int(k), int(S), _ptr(x), _ptr(w_router), _ptr(bias),
                  _ptr(expert_slot), _ptr(topk_expert), _ptr(topk_score), _ptr(sel_expert),
                  _ptr(sel_weight), _ptr(sel_slot), _ptr(slot_offsets), _ptr(perm), _ptr(xq),
                  _ptr(ws), int(ws_bytes), evp, _ptr(hist_row), _ptr(delta),
                  1 if reuse_logits else 0, int(act_format))
    return int(load().moe_route(ctypes.byref(a), _stream(stream)))


def moe_demand_accumulate(topk_expert, topk_score, T, k, E, hist_row, delta, ws, ws_bytes,
                          stream=None) -> int:
    return int(load().moe_demand_accumulate(_ptr(topk_expert), _ptr(topk_score), int(T), int(k),
                                            int(E), _ptr(hist_row), _ptr(delta), _ptr(ws),
                                            int(ws_bytes), _stream(stream)))


def moe_experts_forward(T, H, I, k, S, xq, arena, slot_stride, slot_offsets, perm, sel_slot,
                        sel_weight, out, ws, ws_bytes, stream=None, stage_events=None,
                        defer_slot=-1, defer_event=None, shared_expert=None,
                        act_format=MOE_ACT_MXFP4) -> int:
    keep, evp = _events(stage_events)
    a = ExpertsArgs(int(T), int(H), int(I), int(k), int(S), _ptr(xq), _ptr(arena),
                    int(slot_stride), _ptr(slot_offsets), _ptr(perm), _ptr(sel_slot),
                    _ptr(sel_weight), _ptr(out), _ptr(ws), int(ws_bytes), evp,
                    int(defer_slot), _event(defer_event), _ptr(shared_expert), int(act_format))
    return int(load().moe_experts_forward(ctypes.byref(a), _stream(stream)))


def moe_experts_forward_noalloc(T, H, I, k, S, xq, arena, slot_stride, slot_offsets, perm,
                                sel_slot, sel_weight, out, stream=None, stage_events=None,
                                defer_slot=-1, defer_event=None, ws=None, ws_bytes=0,
                                shared_expert=None, act_format=MOE_ACT_MXFP4) -> int:
    """moe_experts_forward with the library's own scratch (ws must stay None / 0)."""
    keep, evp = _events(stage_events)
    a = ExpertsArgs(int(T), int(H), int(I), int(k), int(S), _ptr(xq), _ptr(arena),
                    int(slot_stride), _ptr(slot_offsets), _ptr(perm), _ptr(sel_slot),
                    _ptr(sel_weight), _ptr(out), _ptr(ws), int(ws_bytes), evp,
                    int(defer_slot), _event(defer_event), _ptr(shared_expert), int(act_format))
    return int(load().moe_experts_forward_noalloc(ctypes.byref(a), _stream(stream)))


def arena_load_slot(arena, slot_stride, num_slots, slot, host_src, nbytes, side_stream=None,
                    done=None) -> int:
    return int(load().arena_load_slot(_ptr(arena), int(slot_stride), int(num_slots), int(slot),
                                      _ptr(host_src), int(nbytes), _stream(side_stream),
                                      _event(done)))


def moe_hot_pick(topk_expert, topk_score, T, k, E, expert_slot, S, n_arena, hist_row, threshold,
                 out, ws=None, ws_bytes=0, stream=None) -> int:
    return int(load().moe_hot_pick(_ptr(topk_expert), _ptr(topk_score), int(T), int(k), int(E),
                                   _ptr(expert_slot), int(S), int(n_arena), _ptr(hist_row),
                                   float(threshold), _ptr(out), _ptr(ws), int(ws_bytes),
                                   _stream(stream)))


def moe_hot_install(pick, expert_slot, E, S, n_arena, slot_out=None, stream=None) -> int:
    return int(load().moe_hot_install(_ptr(pick), _ptr(expert_slot), int(E), int(S),
                                      int(n_arena), _ptr(slot_out), _stream(stream)))


def moe_replan(hist, expert_slot, L, E, k, n_swap, evict, load, new_expert_slot, n_done) -> int:
    """Host function: hist, expert_slot, evict, load, new_expert_slot are host
    buffers (numpy arrays or addresses); n_done is a ctypes.c_int."""
    return int(load_lib().moe_replan(_host(hist), _host(expert_slot), int(L), int(E), int(k),
                                     int(n_swap), _host(evict), _host(load),
                                     _host(new_expert_slot), ctypes.byref(n_done)))


def moe_ring_plan(miss_weight, expert_slot, L, E, ring, R, ring_slot0, per_step, plan,
                  stream=None) -> int:
    return int(load().moe_ring_plan(_ptr(miss_weight), _ptr(expert_slot), int(L), int(E),
                                    _ptr(ring), int(R), int(ring_slot0), int(per_step),
                                    _ptr(plan), _stream(stream)))


def moe_ring_install(plan, expert_slot, L, E, ring, R, ring_slot0, stream=None) -> int:
    return int(load().moe_ring_install(_ptr(plan), _ptr(expert_slot), int(L), int(E), _ptr(ring),
                                       int(R), int(ring_slot0), _stream(stream)))


def moe_history_save(path: str, hist, L, E, tokens: int = 0) -> int:
    """Host function: hist is a host float64 [L][E] array."""
    return int(load_lib().moe_history_save(os.fsencode(path), _host(hist), int(L), int(E),
                                            ctypes.c_uint64(int(tokens))))


def moe_history_load(path: str, hist, L, E, tokens=None) -> int:
    """Host function: fills the host float64 [L][E] array `hist`; `tokens`, if
    given, is a ctypes.c_uint64 that receives the stored token count."""
    return int(load_lib().moe_history_load(os.fsencode(path), _host(hist), int(L), int(E),
                                            ctypes.byref(tokens) if tokens is not None else None))


def moe_boot_plan(hist, L, E, k, n_slots, expert_slot) -> int:
    """Host function: hist float64 [L][E] in, expert_slot int32 [L][E] out."""
    return int(load_lib().moe_boot_plan(_host(hist), int(L), int(E), int(k), int(n_slots),
                                         _host(expert_slot)))


def moe_history_scale(hist, n, factor, stream=None) -> int:
    return int(load().moe_history_scale(_ptr(hist), int(n), float(factor), _stream(stream)))


def moe_test_mxfp4_probe(shape, a, a_scale, b, b_scale, d, stream=None) -> int:
    return int(load().moe_test_mxfp4_probe(int(shape), _ptr(a), _ptr(a_scale), _ptr(b),
                                           _ptr(b_scale), _ptr(d), _stream(stream)))


def check(status: int, what: str = "moe") -> None:
    if status != MOE_OK:
        raise MoeError(status, what)


def moe_test_stream_read(src, nbytes, sink, grid, stream=None) -> int:
    return int(load().moe_test_stream_read(_ptr(src), int(nbytes), _ptr(sink), int(grid),
                                           _stream(stream)))


def moe_test_mfma_loop(iters, sink, grid, stream=None, act_format=MOE_ACT_MXFP4) -> int:
    return int(load().moe_test_mfma_loop(int(iters), int(act_format), _ptr(sink), int(grid),
                                         _stream(stream)))
