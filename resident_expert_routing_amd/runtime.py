"""torch plumbing around the C ABI: device buffers, arena upload, one layer step.

torch supplies device memory and streams only; every step of the layer runs in
libmoe_arena's HIP kernels through the functions of binding.py.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import binding as B


class PinnedCopies:
    """Page-locked copies of host byte arrays for arena_load_slot, made once per
    array object (experts that share one packed array share one copy).  An
    entry holds its array, so the array's id names that entry for as long as it
    lives.  Past `budget` bytes the least recently used entries are dropped,
    each only once every copy that reads it has completed (the events recorded
    after those copies)."""

    def __init__(self, budget: int = 16 << 30):
        from collections import OrderedDict
        self.entries = OrderedDict()  # id(array) -> [array, page-locked copy, [events]]
        self.bytes = 0
        self.budget = int(budget)

    def get(self, host: np.ndarray) -> torch.Tensor:
        key = id(host)
        e = self.entries.get(key)
        if e is None:
            e = [host, torch.from_numpy(np.ascontiguousarray(host)).pin_memory(), []]
            self.entries[key] = e
            self.bytes += e[1].numel()
            self._trim(keep=key)
        else:
            self.entries.move_to_end(key)
        return e[1]

    def used_on(self, host: np.ndarray, stream) -> None:
        """A copy reading host's page-locked copy is enqueued on `stream`."""
        e = self.entries[id(host)]
        e[2] = [ev for ev in e[2] if not ev.query()]
        ev = torch.cuda.Event()
        ev.record(stream)
        e[2].append(ev)

    def _trim(self, keep: int) -> None:
        for key in list(self.entries):
            if self.bytes <= self.budget:
                return
            if key == keep:
                continue
            _, pinned, events = self.entries[key]
            if all(ev.query() for ev in events):
                del self.entries[key]
                self.bytes -= pinned.numel()


def _ws(nbytes: int, device) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    # torch allocations are 256-byte aligned (caching allocator blocks are 512-aligned)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


@dataclass
class LayerBuffers:
    """Outputs and workspaces of one layer call of shape (T, H, E, k, I, S)."""
    T: int
    H: int
    E: int
    k: int
    I: int
    S: int
    device: torch.device
    shared: bool = False    # workspace for a shared expert too
    act_format: int = 0     # B.MOE_ACT_MXFP4 or B.MOE_ACT_MXFP6 (xq and h rows)

    def __post_init__(self):
        T, H, E, k, I, S, dev = self.T, self.H, self.E, self.k, self.I, self.S, self.device
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.topk_expert = torch.empty((T, k), **i32)
        self.topk_score = torch.empty((T, k), **f32)
        self.sel_expert = torch.empty((T, k), **i32)
        self.sel_weight = torch.empty((T, k), **f32)
        self.sel_slot = torch.empty((T, k), **i32)
        self.slot_offsets = torch.empty(S + 1, **i32)
        self.perm = torch.empty(T * k, **i32)
        self.xq_row = B.moe_act_row_bytes(H, self.act_format)
        if self.xq_row == 0:
            raise ValueError(f"activation format {self.act_format} with H={H}")
        self.xq = torch.empty((T, self.xq_row), dtype=torch.uint8, device=dev)
        self.out = torch.empty((T, H), dtype=torch.int16, device=dev)  # bf16 bits
        self.delta = torch.empty(E, **f32)
        self.ws_route_bytes = B.moe_workspace_bytes(B.MOE_OP_ROUTE, T, H, E, k, I, S)
        self.ws_demand_bytes = B.moe_workspace_bytes(B.MOE_OP_DEMAND, T, H, E, k, I, S)
        op = B.MOE_OP_EXPERTS_SHARED if self.shared else B.MOE_OP_EXPERTS
        if self.act_format == B.MOE_ACT_MXFP6:
            op |= B.MOE_OP_ACT_MXFP6
        self.ws_experts_bytes = B.moe_workspace_bytes(op, T, H, E, k, I, S)
        self.ws_route = _ws(self.ws_route_bytes, dev)
        self.ws_demand = _ws(self.ws_demand_bytes, dev)
        self.ws_experts = _ws(self.ws_experts_bytes, dev)


class Arena:
    """S expert slots of slot_stride bytes in one device allocation."""

    def __init__(self, S: int, H: int, I: int, device, stride: int | None = None):
        self.H, self.I, self.S = H, I, S
        self.slot_bytes = B.moe_slot_bytes(H, I)
        self.stride = stride or self.slot_bytes
        assert self.stride % 256 == 0 and self.stride >= self.slot_bytes
        self.mem = torch.empty(S * self.stride, dtype=torch.uint8, device=device)

    def upload(self, slot_bytes_fn, slots=None, stream=None):
        """Copy packed host bytes into slots (plain torch copies, setup only)."""
        slots = range(self.S) if slots is None else slots
        # one page-locked copy per distinct host array; the array itself is held
        # next to it, so its id cannot be reused by another array meanwhile
        cache = {}
        for s in slots:
            host = slot_bytes_fn(s)
            key = id(host)
            if key not in cache:
                cache[key] = (host, torch.from_numpy(np.ascontiguousarray(host)).pin_memory())
            self.mem[s * self.stride: s * self.stride + self.slot_bytes].copy_(cache[key][1],
                                                                            non_blocking=True)
        torch.cuda.current_stream(self.mem.device).synchronize()

    def ptr(self) -> int:
        return self.mem.data_ptr()


def route(buf: LayerBuffers, x, w_router, bias, expert_slot, stream=None,
          stage_events=None, hist_row=None, reuse_logits=False, delta=None) -> None:
    """moe_route; with hist_row it also accumulates this batch's demand, and
    writes the per-call demand to `delta` (default: buf.delta).
    reuse_logits: the previous route on these buffers had the same x and
    w_router (only the routable set changed): skip the router's products."""
    if delta is None and hist_row is not None:
        delta = buf.delta
    B.check(B.moe_route(buf.T, buf.H, buf.E, buf.k, buf.S, x, w_router, bias, expert_slot,
                        buf.topk_expert, buf.topk_score, buf.sel_expert, buf.sel_weight,
                        buf.sel_slot, buf.slot_offsets, buf.perm, buf.xq, buf.ws_route,
                        buf.ws_route_bytes, stream, stage_events, hist_row, delta, reuse_logits,
                        buf.act_format),
            "moe_route")


def demand(buf: LayerBuffers, hist_row, stream=None, delta=True) -> None:
    B.check(B.moe_demand_accumulate(buf.topk_expert, buf.topk_score, buf.T, buf.k, buf.E,
                                    hist_row, buf.delta if delta else None, buf.ws_demand,
                                    buf.ws_demand_bytes, stream), "moe_demand_accumulate")


def experts(buf: LayerBuffers, arena_ptr, slot_stride: int, stream=None,
            stage_events=None, defer_slot: int = -1, defer_event=None,
            shared_expert=None) -> None:
    """moe_experts_forward; shared_expert: a device tensor holding the layer's
    shared expert in the slot format (buf must be made with shared=True)."""
    B.check(B.moe_experts_forward(buf.T, buf.H, buf.I, buf.k, buf.S, buf.xq, arena_ptr,
                                  slot_stride, buf.slot_offsets, buf.perm, buf.sel_slot,
                                  buf.sel_weight, buf.out, buf.ws_experts, buf.ws_experts_bytes,
                                  stream, stage_events, defer_slot, defer_event,
                                  shared_expert, buf.act_format),
            "moe_experts_forward")


class HotReader:
    """Host side of the hot read for one layer.

    The decision and the slot-table update run on the GPU (moe_hot_pick, then
    moe_hot_install on the layer's stream); the host reads the decision from a
    page-locked buffer, copies the missing expert's bytes from page-locked
    memory into the slot it now owns with arena_load_slot on a side stream.
    """

    def __init__(self, expert_slot_host: np.ndarray, n_arena: int, device, threshold: float = 0.2):
        self.es = np.asarray(expert_slot_host, dtype=np.int32).copy()
        self.n_arena = int(n_arena)
        self.threshold = float(threshold)
        self.device = device
        # (e*, c) from moe_hot_pick, then the slot moe_hot_install gave e* (-1: none)
        self.out = torch.empty(3, dtype=torch.int32, device=device)
        self.out_host = torch.empty(3, dtype=torch.int32).pin_memory()
        self.out_ready = torch.cuda.Event()
        self.installed = torch.cuda.Event()
        self.side = torch.cuda.Stream(device)   # default priority
        self.done = torch.cuda.Event()
        self.done.record(self.side)   # creates the HIP event the library records after a copy
        self.pins = PinnedCopies()
        self.ws = None   # token-pass partials of moe_hot_pick, grown to the largest batch seen

    def workspace(self, T: int) -> torch.Tensor:
        need = B.moe_workspace_bytes(B.MOE_OP_HOT_PICK, T, 0, 0, 0, 0, 0)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self.ws

    def pinned(self, e: int, expert_bytes_fn) -> torch.Tensor:
        """Page-locked copy of expert e's packed bytes (PinnedCopies)."""
        return self.pins.get(expert_bytes_fn(e))

    def enqueue_decision(self, buf: LayerBuffers, expert_slot_dev, hist_row, stream) -> None:
        """Enqueues the decision and the table update on `stream` and records
        `installed` after them; read_decision() then copies the decision to
        page-locked host memory on the side stream."""
        ws = self.workspace(buf.T)
        B.check(B.moe_hot_pick(buf.topk_expert, buf.topk_score, buf.T, buf.k, buf.E,
                               expert_slot_dev, buf.S, self.n_arena, hist_row, self.threshold,
                               self.out, ws, ws.numel(), stream), "moe_hot_pick")
        B.check(B.moe_hot_install(self.out, expert_slot_dev, buf.E, buf.S, self.n_arena,
                                  self.out[2:], stream), "moe_hot_install")
        self.installed.record(stream)

    def read_decision(self) -> None:
        """The decision's copy to the host, on the side stream after `installed`
        (so the layer's stream can go on meanwhile); the side stream is then
        also ordered after everything enqueued on the layer's stream before the
        decision -- the copy into a slot must follow every kernel that reads it."""
        self.side.wait_event(self.installed)
        with torch.cuda.stream(self.side):
            self.out_host.copy_(self.out, non_blocking=True)
            self.out_ready.record(self.side)

    def wait_decision(self):
        """Waits for the enqueued decision: (e_star, c, slot), or None when
        nothing is read (the table was left as it was)."""
        self.out_ready.synchronize()
        e_star, c, slot = (int(v) for v in self.out_host)
        if slot < 0:
            return None
        self.es[e_star], self.es[c] = slot, -1
        return e_star, c, slot

    def decide(self, buf: LayerBuffers, expert_slot_dev, hist_row, stream):
        """enqueue_decision() and wait_decision(): returns (e_star, c, slot), or
        None.  The device table already routes e_star to `slot` when this returns."""
        self.enqueue_decision(buf, expert_slot_dev, hist_row, stream)
        self.read_decision()
        return self.wait_decision()

    def load(self, picked, arena: Arena, expert_bytes_fn) -> None:
        """Enqueues the copy of the picked expert's bytes into its slot on the
        side stream; `done` is recorded after it."""
        e_star, _, slot = picked
        host = expert_bytes_fn(e_star)
        src = self.pins.get(host)
        B.check(B.arena_load_slot(arena.mem, arena.stride, arena.S, slot, src, arena.slot_bytes,
                                  self.side, self.done), "arena_load_slot")
        self.pins.used_on(host, self.side)

    def pick_and_load(self, buf: LayerBuffers, expert_slot_dev, hist_row, arena: Arena,
                      expert_bytes_fn, stream):
        """decide() and load(): returns (e_star, c, slot) after enqueueing the
        copy, or None."""
        picked = self.decide(buf, expert_slot_dev, hist_row, stream)
        if picked is not None:
            self.load(picked, arena, expert_bytes_fn)
        return picked


def layer_step_hot(buf: LayerBuffers, x, w_router, bias, expert_slot_dev, hist_row,
                   arena: Arena, hot: HotReader, expert_bytes_fn, stream=None):
    """One layer call with a hot read before the experts (long prefill chunks).

    Route with demand; decide and update the slot table on the device; route
    again over the table as it now stands (the router's products reused) while
    the decision travels to the host on the side stream; start the copy on the
    side stream; run the experts with the loaded slot deferred: the other
    slots' gate/up products run while the copy finishes, that slot's after it.
    The second routing is enqueued before the decision is known, so the layer's
    stream never waits for the host; when nothing qualifies it repeats the first
    routing's result (the table is unchanged), one selection and bucketing pass
    spent for nothing.
    """
    stream = stream if stream is not None else torch.cuda.current_stream(hot.device)
    route(buf, x, w_router, bias, expert_slot_dev, stream, hist_row=hist_row)
    hot.enqueue_decision(buf, expert_slot_dev, hist_row, stream)
    route(buf, x, w_router, bias, expert_slot_dev, stream, reuse_logits=True)
    hot.read_decision()
    picked = hot.wait_decision()
    if picked is None:
        experts(buf, arena.ptr(), arena.stride, stream)
        return None
    hot.load(picked, arena, expert_bytes_fn)
    experts(buf, arena.ptr(), arena.stride, stream, defer_slot=picked[2], defer_event=hot.done)
    return picked


def layer_step(buf: LayerBuffers, x, w_router, bias, expert_slot, hist_row, arena_ptr,
               slot_stride, stream=None, fused_demand=True) -> None:
    """One pass of the whole layer: route, demand, experts and combine.

    fused_demand: demand is accumulated by moe_route (same result as the
    separate moe_demand_accumulate call, one launch fewer for small batches).
    """
    if fused_demand:
        route(buf, x, w_router, bias, expert_slot, stream, hist_row=hist_row)
    else:
        route(buf, x, w_router, bias, expert_slot, stream)
        demand(buf, hist_row, stream)
    experts(buf, arena_ptr, slot_stride, stream)


class SharedArena:
    """One arena shared by L layers: the [L][E] slot table and the [L][E]
    float64 demand history on the device, plus the re-plan flow.

    Layer l routes with expert_slot = table[l] and accumulates demand into
    hist[l] (both contiguous rows).  replan() reads the history (80 KB at
    40 x 256), lets moe_replan pick the swaps, copies every loaded expert into
    its new slot with arena_load_slot on a side stream, and installs the new
    table on the layer stream after the copies.
    """

    def __init__(self, S: int, H: int, I: int, table_host: np.ndarray, device):
        self.arena = Arena(S, H, I, device)
        self.L, self.E = table_host.shape
        self.table_host = np.ascontiguousarray(table_host, dtype=np.int32).copy()
        self.table = torch.from_numpy(self.table_host.copy()).to(device)
        self.hist = torch.zeros((self.L, self.E), dtype=torch.float64, device=device)
        self.device = device
        self.side = torch.cuda.Stream(device)   # default priority
        self.done = torch.cuda.Event()
        self.done.record(self.side)   # creates the HIP event the library records after a copy
        self.pins = PinnedCopies()

    def upload(self, pair_bytes_fn) -> None:
        """Fill every slot with the bytes of the (layer, expert) it holds."""
        l_idx, e_idx = np.nonzero(self.table_host >= 0)
        owner = {int(self.table_host[l, e]): (int(l), int(e)) for l, e in zip(l_idx, e_idx)}
        self.arena.upload(lambda s: pair_bytes_fn(*owner[s]), slots=sorted(owner))

    def load_pair(self, slot: int, l: int, e: int, pair_bytes_fn, stream, done_event=None) -> None:
        """Enqueue the copy of pair (l, e)'s packed bytes into `slot` on `stream`
        (from its page-locked copy, PinnedCopies)."""
        host = pair_bytes_fn(l, e)
        a = self.arena
        B.check(B.arena_load_slot(a.mem, a.stride, a.S, slot, self.pins.get(host), a.slot_bytes,
                                  stream, done_event), "arena_load_slot")
        self.pins.used_on(host, stream)

    def replan(self, k: int, n_swap: int, pair_bytes_fn, stream=None, gain_only: bool = False):
        """Returns (evict [(l,e)], load [(l,e)]) once the copies are enqueued and
        the new table is ordered after them on `stream`.  gain_only: keep only
        the leading swaps whose loaded pair has a larger history than the pair
        it evicts (the lists run coldest / hottest first, so gains shrink)."""
        import ctypes
        stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        with torch.cuda.stream(stream):
            hist = self.hist.cpu().numpy()                    # waits for the layers' demand
        ev = np.empty((max(n_swap, 1), 2), dtype=np.int32)
        ld = np.empty((max(n_swap, 1), 2), dtype=np.int32)
        new = np.empty_like(self.table_host)
        n_done = ctypes.c_int(0)
        B.check(B.moe_replan(hist, self.table_host, self.L, self.E, k, n_swap, ev, ld, new,
                             n_done), "moe_replan")
        n = n_done.value
        if gain_only:
            g = 0
            while g < n and hist[ld[g, 0], ld[g, 1]] > hist[ev[g, 0], ev[g, 1]]:
                g += 1
            if g < n:   # the first g swaps of a longer plan are the plan of g swaps
                B.check(B.moe_replan(hist, self.table_host, self.L, self.E, k, g, ev, ld, new,
                                     n_done), "moe_replan")
                n = n_done.value
        if n == 0:
            return [], []
        self.side.wait_stream(stream)       # nothing still reads an evicted slot
        a = self.arena
        for i in range(n):
            slot = int(self.table_host[ev[i, 0], ev[i, 1]])
            self.load_pair(slot, int(ld[i, 0]), int(ld[i, 1]), pair_bytes_fn, self.side,
                           self.done if i == n - 1 else None)
        stream.wait_event(self.done)
        self.table_host = new
        staged = torch.from_numpy(new.copy()).pin_memory()
        with torch.cuda.stream(stream):
            self.table.copy_(staged, non_blocking=True)
        self._staged = staged                   # kept alive until the copy has run
        return ([tuple(map(int, p)) for p in ev[:n]], [tuple(map(int, p)) for p in ld[:n]])


class HotRing:
    """The asynchronous hot ring of a shared arena (TideLM README, "How adaptive
    expert loading works", item 3, DeepSeek bullet).

    R ring entries are the arena's slots ring_slot0 .. ring_slot0 + R - 1, on
    top of the resident budget.  Per step s the caller runs
        ring.before_step(s)      # installs the plan of step s - 2 (its copies done)
        ... every layer l: route(..., hist_row=hist[l], delta=ring.delta_row(l)) + experts ...
        ring.after_step(s)       # plans step s's heaviest misses on the GPU
                                 # (evictions take effect at once), then enqueues
                                 # the copies of step s - 1's plan on the side stream
    so the misses of step s are copied while step s + 1 runs and are routable
    from step s + 2 on.  The plan is taken on the device (moe_ring_plan); the
    host only reads its few picks back -- one step late, so it never waits for
    the step it has just enqueued -- and issues arena_load_slot for each.
    keep_picks: keep every step's picks in `picks` (tests); otherwise only their
    count, `n_picks`, so a long serving run holds no growing log.
    """

    def __init__(self, sa: "SharedArena", ring_slot0: int, R: int, per_step: int,
                 pair_bytes_fn, device, keep_picks: bool = False):
        assert 0 < per_step <= R and 2 * per_step <= R, "a plan must not wrap onto the last one"
        assert ring_slot0 + R <= sa.arena.S
        self.sa, self.slot0, self.R, self.per_step = sa, int(ring_slot0), int(R), int(per_step)
        self.pair_bytes = pair_bytes_fn
        self.device = device
        L, E = sa.L, sa.E
        self.delta = torch.zeros((L, E), dtype=torch.float32, device=device)
        self.ring = torch.full((1 + R,), -1, dtype=torch.int32, device=device)
        self.ring[0] = 0
        n = 1 + 3 * per_step
        self.plan = [torch.zeros(n, dtype=torch.int32, device=device) for _ in range(2)]
        self.plan_host = [torch.zeros(n, dtype=torch.int32).pin_memory() for _ in range(2)]
        self.planned = [torch.cuda.Event() for _ in range(2)]
        self.copied = [torch.cuda.Event() for _ in range(2)]
        self.side = torch.cuda.Stream(device)      # default priority
        self.n_copies = [0, 0]                      # copies issued for the plan in each buffer
        self.read_through = -1                      # the last step whose plan was read back
        self.picks = {} if keep_picks else None     # step -> [(r, l, e)], when kept
        self.n_picks = 0
        self.bytes_copied = 0

    def delta_row(self, l: int) -> torch.Tensor:
        return self.delta[l]

    def before_step(self, s: int, stream=None) -> None:
        stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        b = (s - 2) % 2
        if s >= 2 and self.n_copies[b]:
            stream.wait_event(self.copied[b])
            B.check(B.moe_ring_install(self.plan[b], self.sa.table, self.sa.L, self.sa.E,
                                       self.ring, self.R, self.slot0, stream), "moe_ring_install")

    def after_step(self, s: int, stream=None) -> None:
        stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        b = s % 2
        B.check(B.moe_ring_plan(self.delta, self.sa.table, self.sa.L, self.sa.E, self.ring,
                                self.R, self.slot0, self.per_step, self.plan[b], stream),
                "moe_ring_plan")
        with torch.cuda.stream(stream):
            self.plan_host[b].copy_(self.plan[b], non_blocking=True)
        self.planned[b].record(stream)
        self.n_copies[b] = 0
        if s >= 1:
            self._copy(s - 1)

    def finish(self, s_last: int) -> None:
        """After the last step: issue the copies of its plan too (they are then
        routable from the step after, if the caller runs one)."""
        self._copy(s_last)

    def _copy(self, s: int) -> None:
        b = s % 2
        if s <= self.read_through:
            return
        self.read_through = s
        self.planned[b].synchronize()            # the end of step s (already past, or nearly)
        n = int(self.plan_host[b][0])
        picks = [tuple(int(v) for v in self.plan_host[b][1 + 3 * i: 4 + 3 * i]) for i in range(n)]
        if self.picks is not None:
            self.picks[s] = picks
        self.n_picks += n
        if not picks:
            return
        self.side.wait_event(self.planned[b])    # the evicted entries are no longer read
        for r, l, e in picks:
            self.sa.load_pair(self.slot0 + r, l, e, self.pair_bytes, self.side)
            self.bytes_copied += self.sa.arena.slot_bytes
        self.copied[b].record(self.side)
        self.n_copies[b] = len(picks)


# How much of the history each re-plan keeps (the sensitivity setting: how
# fast the resident set follows new traffic).
SENSITIVITY_DECAY = {"low": 1.0, "medium": 0.9, "high": 0.75}


def load_history(path: str, L: int, E: int, default: np.ndarray | None = None):
    """(history [L][E] float64, tokens seen) from a history file; a missing
    file gives `default` (e.g. a bundled starting history) or zeros.  A damaged
    file or one of another shape raises."""
    import ctypes
    import os
    hist = np.zeros((L, E), dtype=np.float64)
    tok = ctypes.c_uint64(0)
    if not os.path.exists(path):
        return (np.array(default, dtype=np.float64) if default is not None else hist), 0
    B.check(B.moe_history_load(path, hist, L, E, tok), f"moe_history_load({path})")
    return hist, int(tok.value)


def boot_table(hist: np.ndarray, k: int, n_slots: int) -> np.ndarray:
    """The arena filled from a history at boot (moe_boot_plan)."""
    hist = np.ascontiguousarray(hist, dtype=np.float64)
    L, E = hist.shape
    table = np.empty((L, E), dtype=np.int32)
    B.check(B.moe_boot_plan(hist, L, E, k, n_slots, table), "moe_boot_plan")
    return table


class AdaptiveArena:
    """The demand-history planner around a SharedArena (TideLM README, "How
    adaptive expert loading works", item 1: a history that persists across
    restarts, the arena filled from it at boot, and re-planned after each
    prompt's prefill, every few hundred generated tokens during long answers,
    and between requests).

    Each re-plan first scales the device history by the sensitivity's factor
    (moe_history_scale: older traffic weighs less), then swaps up to
    `swap_frac` of the arena's slots, keeping only the swaps that gain.
    The caller reports serving events: on_prefill(), on_tokens(n) with the
    tokens generated since the last call, on_request_end().
    """

    def __init__(self, sa: "SharedArena", k: int, pair_bytes_fn, every: int = 200,
                 sensitivity: str = "medium", swap_frac: float = 0.05, n_arena: int | None = None,
                 tokens_seen: int = 0):
        self.sa, self.k, self.pair_bytes = sa, int(k), pair_bytes_fn
        self.every = int(every)
        self.factor = SENSITIVITY_DECAY[sensitivity]
        n_arena = int((sa.table_host >= 0).sum()) if n_arena is None else int(n_arena)
        self.n_swap = max(1, int(swap_frac * n_arena))
        self.since = 0
        self.tokens_seen = int(tokens_seen)
        self.replans = []           # (reason, evicted, loaded) per re-plan

    def replan(self, reason: str, stream=None):
        stream = stream if stream is not None else torch.cuda.current_stream(self.sa.device)
        B.check(B.moe_history_scale(self.sa.hist, self.sa.hist.numel(), self.factor, stream),
                "moe_history_scale")
        ev, ld = self.sa.replan(self.k, self.n_swap, self.pair_bytes, stream, gain_only=True)
        self.replans.append((reason, ev, ld))
        self.since = 0
        return ev, ld

    def on_prefill(self, tokens: int, stream=None):
        self.tokens_seen += int(tokens)
        return self.replan("prefill", stream)

    def on_tokens(self, n: int, stream=None):
        self.tokens_seen += int(n)
        self.since += int(n)
        if self.since >= self.every:
            return self.replan("tokens", stream)
        return None

    def on_request_end(self, stream=None):
        if self.since > 0:
            return self.replan("between requests", stream)
        return None

    def save(self, path: str, stream=None) -> None:
        stream = stream if stream is not None else torch.cuda.current_stream(self.sa.device)
        with torch.cuda.stream(stream):
            hist = np.ascontiguousarray(self.sa.hist.cpu().numpy())
        B.check(B.moe_history_save(path, hist, self.sa.L, self.sa.E, self.tokens_seen),
                f"moe_history_save({path})")
