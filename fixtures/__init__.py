"""Seeded synthetic inputs for the resident-expert MoE layer.

This module is the one piece shared by the GPU path's tests/bench and by the
CPU oracle's tests.  It draws random numbers and lays them out; it computes
nothing the layer computes (no router, no softmax, no top-k, no FFN, no
activation quantiser).  The single piece of number formatting it does is the
*offline* packing of synthetic expert weights into the MXFP4 checkpoint format
(E2M1 codes plus one E8M0 scale byte per 32 values), which is how a model's
routed experts arrive on disk (TideLM README, "Profile" table: the ds41-mxfp4
profile serves "native MXFP4" routed experts).  The layer never packs weights.

Workloads (sizes from the routed-expert MoE layer of the TideLM README, the
"How adaptive expert loading works" section, and the colibri cluster page's
prefill-chunk paragraph for the 8192-token chunk):

  tiny       T=64,   H=256,  E=16,  k=4, I=128,  10 of 16 resident (uniform)
  decode     T=8,    H=4096, E=256, k=8, I=2048, 166 resident + 64 ring slots
  prefill    T=2048, H=4096, E=256, k=8, I=2048, 166 resident
  long       T=8192, H=6144, E=192, k=8, I=2048, 130 resident, one hot read
  arena40    40 layers x 256 experts, T=32 per step, one shared 6666-slot arena

Every random stream is a numpy PCG64 generator keyed by (seed, purpose, ...),
so any array can be regenerated on its own.
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import dataclass, field

import numpy as np

# ----------------------------------------------------------------------------
# random streams
# ----------------------------------------------------------------------------
_PURPOSE = {
    "x": 1,
    "router": 2,
    "popularity": 3,
    "residency": 4,
    "expert": 5,
    "content_map": 6,
    "layer_split": 7,
}


def rng(seed: int, purpose: str, *key: int) -> np.random.Generator:
    """Independent PCG64 stream for (seed, purpose, key...)."""
    ss = np.random.SeedSequence([int(seed), _PURPOSE[purpose], *[int(v) for v in key]])
    return np.random.Generator(np.random.PCG64(ss))


# ----------------------------------------------------------------------------
# bf16 helpers (storage format of activations)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest even); returns uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# offline MXFP4 weight packing (checkpoint format, not part of the layer)
# ----------------------------------------------------------------------------
# E2M1 magnitudes in code order 0..7.
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
# Upper edge of each magnitude code's rounding interval, and whether that edge
# itself belongs to the code below it (ties go to the even mantissa: codes
# 0, 2, 4, 6 have an even mantissa bit).
_EDGES = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
_EDGE_GOES_DOWN = np.array([True, False, True, False, True, False, True])


def _e2m1_magnitude_code(a: np.ndarray) -> np.ndarray:
    """Nearest E2M1 magnitude code for |q| values in [0, 8), ties to even."""
    idx = np.searchsorted(_EDGES, a, side="left")  # first edge >= a
    # a equal to an edge: searchsorted(left) puts it *below* that edge; move it
    # up when the tie belongs to the upper code.
    on_edge = np.zeros(a.shape, dtype=bool)
    inb = idx < len(_EDGES)
    on_edge[inb] = a[inb] == _EDGES[idx[inb]]
    up = on_edge & ~_EDGE_GOES_DOWN[np.minimum(idx, len(_EDGES) - 1)]
    return (idx + up).astype(np.uint8)


def pack_mxfp4_rows(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Pack float32 rows [N, K] (K % 32 == 0) along K.

    Returns (codes uint8 [N, K/2], scales uint8 [N, K/32]).  Per 32-block the
    shared scale is 2**(floor(log2(amax)) - 2) clamped to the E8M0 range
    (OCP MX v1.0), every element is divided by it and rounded to the nearest
    E2M1 value (ties to even, magnitudes above 6 saturate), element 2i goes in
    the low nibble of byte i, and an all-zero block gets scale byte 0.
    """
    w = np.asarray(w, dtype=np.float32)
    n, kdim = w.shape
    assert kdim % 32 == 0
    blk = w.astype(np.float64).reshape(n, kdim // 32, 32)
    amax = np.abs(blk).max(axis=2)
    _, ex = np.frexp(amax)  # amax = m * 2**ex, m in [0.5, 1)
    se = np.clip(ex.astype(np.int64) - 3, -127, 127)  # floor(log2 amax) - 2
    zero_blk = amax == 0
    se = np.where(zero_blk, -127, se)
    q = np.ldexp(blk, (-se)[..., None])
    mag = _e2m1_magnitude_code(np.minimum(np.abs(q), 7.9999))
    code = mag | (np.signbit(q).astype(np.uint8) << 3)
    code = np.where(zero_blk[..., None], 0, code).astype(np.uint8)
    code = code.reshape(n, kdim)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    scales = (se + 127).astype(np.uint8)
    return packed, scales


# ----------------------------------------------------------------------------
# slot byte layout (the arena format, documented in include/moe_arena.h)
# ----------------------------------------------------------------------------
def _up256(v: int) -> int:
    return (v + 255) // 256 * 256


@dataclass(frozen=True)
class SlotLayout:
    H: int
    I: int

    @property
    def sections(self) -> dict:
        H, I = self.H, self.I
        sizes = [
            ("gate_codes", I * H // 2),
            ("gate_scales", I * H // 32),
            ("up_codes", I * H // 2),
            ("up_scales", I * H // 32),
            ("down_codes", H * I // 2),
            ("down_scales", H * I // 32),
        ]
        out, off = {}, 0
        for name, sz in sizes:
            out[name] = (off, sz)
            off = _up256(off + sz)
        return out

    @property
    def nbytes(self) -> int:
        off, sz = self.sections["down_scales"]
        return _up256(off + sz)


def tile_codes(codes: np.ndarray) -> np.ndarray:
    """Row-major packed codes [N, B] (N % 16 == 0, B bytes a row) -> the slot's
    code order: row blocks of 16 rows, each a run of tiles of 64 code bytes
    (128 elements) of all 16 rows (the last tile of a block narrower when B %
    64 != 0), a tile's rows one after another."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, nb = codes.shape
    assert n % 16 == 0
    full = nb // 64 * 64
    blocks = codes.reshape(n // 16, 16, nb)
    head = blocks[:, :, :full].reshape(n // 16, 16, full // 64, 64).transpose(0, 2, 1, 3)
    parts = [head.reshape(n // 16, -1)]
    if full < nb:
        parts.append(blocks[:, :, full:].reshape(n // 16, -1))
    return np.concatenate(parts, axis=1).reshape(-1)


def pack_expert(wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """Pack one SwiGLU expert (gate [I,H], up [I,H], down [H,I]) into slot bytes:
    codes in tiles of 16 rows x 64 bytes (tile_codes), scales row by row."""
    I, H = wg.shape
    lay = SlotLayout(H, I)
    buf = np.zeros(lay.nbytes, dtype=np.uint8)
    for mat, cname, sname in ((wg, "gate_codes", "gate_scales"),
                              (wu, "up_codes", "up_scales"),
                              (wd, "down_codes", "down_scales")):
        c, s = pack_mxfp4_rows(mat)
        co, cs = lay.sections[cname]
        so, ss = lay.sections[sname]
        buf[co:co + cs] = tile_codes(c)
        buf[so:so + ss] = s.reshape(-1)
    return buf


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    resident: int
    ring: int = 0
    zipf: bool = False
    zipf_s: float = 1.1
    beta_key: str = ""          # which calibrated Zipf beta to use
    contents: int = 0           # distinct expert contents (0 = one per expert)
    seed: int = 0
    weight_std: float = 0.02
    router_std: float = 0.02
    layers: int = 1

    @property
    def S(self) -> int:
        return self.resident + self.ring

    @property
    def A(self) -> int:
        return self.T * self.k

    @property
    def n_contents(self) -> int:
        return self.contents or self.E

    @property
    def slot_bytes(self) -> int:
        return SlotLayout(self.H, self.I).nbytes


CONFIGS = {
    "tiny": LayerConfig("tiny", T=64, H=256, E=16, k=4, I=128, resident=10, seed=101),
    "decode": LayerConfig("decode", T=8, H=4096, E=256, k=8, I=2048, resident=166, ring=64,
                          zipf=True, beta_key="prefill", contents=24, seed=202),
    "prefill": LayerConfig("prefill", T=2048, H=4096, E=256, k=8, I=2048, resident=166,
                           zipf=True, beta_key="prefill", contents=24, seed=202),
    "long": LayerConfig("long", T=8192, H=6144, E=192, k=8, I=2048, resident=130,
                        zipf=True, beta_key="long", contents=16, seed=404),
    "arena40": LayerConfig("arena40", T=32, H=4096, E=256, k=8, I=2048, resident=6666,
                           zipf=True, beta_key="prefill", contents=24, seed=505, layers=40),
}

# The decode and prefill workloads share one model layer (router, bias,
# residency and expert contents); their tokens differ.
_MODEL_SEED = {"decode": 202, "prefill": 202}
_X_SEED = {"decode": 2021, "prefill": 2022}

_BETA_FILE = os.path.join(os.path.dirname(__file__), "zipf_beta.json")


def zipf_beta(key: str) -> float:
    """Calibrated Zipf bias strength (written by the oracle's calibration script)."""
    with open(_BETA_FILE) as f:
        return float(json.load(f)[key]["beta"])


def popularity_ranks(seed: int, E: int, layer: int = 0) -> np.ndarray:
    """Popularity rank r_e in 1..E for every expert (a seeded permutation)."""
    return (1 + rng(seed, "popularity", layer).permutation(E)).astype(np.int64)


def zipf_bias(ranks: np.ndarray, beta: float, s: float = 1.1) -> np.ndarray:
    """Per-expert router bias b_e = -beta * s * ln(r_e), as float32."""
    return (-beta * s * np.log(ranks.astype(np.float64))).astype(np.float32)


def residency_order(seed: int, ranks: np.ndarray | None, E: int, layer: int = 0,
                    s: float = 1.1) -> np.ndarray:
    """Experts in the order they are drawn into the arena.

    With popularity ranks: weighted sampling without replacement in proportion
    to the Zipf probability r**-s (Efraimidis-Spirakis keys ln(u)/w, largest
    first).  Without: a uniform random order.
    """
    g = rng(seed, "residency", layer)
    if ranks is None:
        return g.permutation(E).astype(np.int64)
    w = ranks.astype(np.float64) ** (-s)
    w /= w.sum()
    u = g.random(E)
    keys = np.log(u) / w
    return np.argsort(-keys, kind="stable").astype(np.int64)


def content_map(seed: int, E: int, n_contents: int, layer: int = 0) -> np.ndarray:
    """Which distinct weight content each expert holds (balanced, shuffled)."""
    if n_contents >= E:
        return np.arange(E, dtype=np.int64)
    return (rng(seed, "content_map", layer).permutation(E) % n_contents).astype(np.int64)


def expert_weights(seed: int, content: int, H: int, I: int, std: float = 0.02):
    """float32 (gate [I,H], up [I,H], down [H,I]) drawn N(0, std^2)."""
    g = rng(seed, "expert", content)
    wg = g.standard_normal((I, H), dtype=np.float32) * np.float32(std)
    wu = g.standard_normal((I, H), dtype=np.float32) * np.float32(std)
    wd = g.standard_normal((H, I), dtype=np.float32) * np.float32(std)
    return wg, wu, wd


_PACK_CACHE: dict = {}


def _pack_one(args):
    seed, content, H, I, std = args
    return pack_expert(*expert_weights(seed, content, H, I, std))


def packed_expert(seed: int, content: int, H: int, I: int, std: float = 0.02) -> np.ndarray:
    key = (seed, content, H, I, std)
    if key not in _PACK_CACHE:
        _PACK_CACHE[key] = _pack_one(key)
    return _PACK_CACHE[key]


def prepack(seed: int, contents, H: int, I: int, std: float = 0.02, workers: int | None = None):
    """Pack many expert contents in parallel worker processes (fills the cache)."""
    todo = [(seed, int(c), H, I, std) for c in contents
            if (seed, int(c), H, I, std) not in _PACK_CACHE]
    if not todo:
        return
    if workers is None:
        workers = min(len(todo), len(os.sched_getaffinity(0)), 16)
    if workers <= 1 or len(todo) == 1:
        for key in todo:
            _PACK_CACHE[key] = _pack_one(key)
        return
    # A fresh interpreter per worker ('spawn'): the caller may already have
    # initialised the GPU, and a forked copy of such a process must not run.
    # The pool is closed and joined, so no worker ends by a signal.
    import multiprocessing as mp
    pool = mp.get_context("spawn").Pool(workers)
    try:
        bufs = pool.map(_pack_one, todo)
        pool.close()
    except BaseException:
        pool.terminate()
        raise
    finally:
        pool.join()
    for key, buf in zip(todo, bufs):
        _PACK_CACHE[key] = buf


@dataclass
class Layer:
    """One MoE layer's inputs, all host numpy arrays."""
    cfg: LayerConfig
    x_bits: np.ndarray          # uint16 [T,H] bf16 bits
    w_router: np.ndarray        # float32 [E,H]
    bias: np.ndarray            # float32 [E]
    expert_slot: np.ndarray     # int32 [E], -1 = not routable
    slot_expert: np.ndarray     # int32 [S]
    expert_content: np.ndarray  # int64 [E]
    ranks: np.ndarray | None
    order: np.ndarray           # residency draw order
    model_seed: int
    beta: float = 0.0
    extra: dict = field(default_factory=dict)

    @property
    def S(self) -> int:
        return int(self.slot_expert.shape[0])

    def slot_content(self) -> np.ndarray:
        return self.expert_content[self.slot_expert]

    def content_bytes(self, c: int) -> np.ndarray:
        cfg = self.cfg
        return packed_expert(self.model_seed, int(c), cfg.H, cfg.I, cfg.weight_std)

    def expert_bytes(self, e: int) -> np.ndarray:
        return self.content_bytes(self.expert_content[e])

    def prepack(self, experts=None):
        """Pack the contents of the given experts (default: all slotted) in parallel."""
        cfg = self.cfg
        cs = self.slot_content() if experts is None else self.expert_content[np.asarray(experts)]
        prepack(self.model_seed, np.unique(cs), cfg.H, cfg.I, cfg.weight_std)

    def arena_host(self) -> np.ndarray:
        """All slots packed back to back (uint8 [S, slot_bytes])."""
        cfg = self.cfg
        self.prepack()
        out = np.empty((self.S, cfg.slot_bytes), dtype=np.uint8)
        for s, c in enumerate(self.slot_content()):
            out[s] = self.content_bytes(c)
        return out


def draw_tokens(seed: int, T: int, H: int, stream: int = 0) -> np.ndarray:
    """T token rows of N(0,1) activations rounded to bf16 (uint16 bits)."""
    x = rng(seed, "x", stream).standard_normal((T, H), dtype=np.float32)
    return f32_to_bf16_bits(x)


def make_layer(name: str, T: int | None = None, x_stream: int = 0, beta: float | None = None,
               layer: int = 0) -> Layer:
    cfg = CONFIGS[name]
    T = cfg.T if T is None else T
    mseed = _MODEL_SEED.get(name, cfg.seed)
    xseed = _X_SEED.get(name, cfg.seed + 7)
    E, H = cfg.E, cfg.H
    w_router = rng(mseed, "router", layer).standard_normal((E, H), dtype=np.float32) \
        * np.float32(cfg.router_std)
    if cfg.zipf:
        ranks = popularity_ranks(mseed, E, layer)
        if beta is None:
            beta = zipf_beta(cfg.beta_key)
        bias = zipf_bias(ranks, beta, cfg.zipf_s)
    else:
        ranks, beta = None, 0.0
        bias = np.zeros(E, dtype=np.float32)
    order = residency_order(mseed, ranks, E, layer, cfg.zipf_s)
    nres = min(cfg.resident, E)
    nring = min(cfg.ring, E - nres)
    routable = order[:nres + nring]
    expert_slot = np.full(E, -1, dtype=np.int32)
    expert_slot[routable] = np.arange(nres + nring, dtype=np.int32)
    slot_expert = routable.astype(np.int32)
    x_bits = draw_tokens(xseed, T, H, x_stream + 1000 * layer)
    return Layer(cfg=cfg, x_bits=x_bits, w_router=w_router, bias=bias, expert_slot=expert_slot,
                 slot_expert=slot_expert,
                 expert_content=content_map(mseed, E, cfg.n_contents, layer),
                 ranks=ranks, order=order, model_seed=mseed, beta=float(beta),
                 extra={"n_resident": nres, "n_ring": nring})


def tiny_layer(T: int, H: int, E: int, k: int, I: int, n_routable: int, seed: int,
               bias_scale: float = 0.0, n_contents: int = 0) -> Layer:
    """Small ad-hoc layer for property tests (any shape with H, I multiples of 32)."""
    cfg = LayerConfig(f"adhoc{seed}", T=T, H=H, E=E, k=k, I=I, resident=n_routable,
                      contents=n_contents, seed=seed)
    w_router = rng(seed, "router", 0).standard_normal((E, H), dtype=np.float32) * np.float32(0.02)
    bias = (rng(seed, "popularity", 0).standard_normal(E) * bias_scale).astype(np.float32)
    order = residency_order(seed, None, E)
    expert_slot = np.full(E, -1, dtype=np.int32)
    expert_slot[order[:n_routable]] = np.arange(n_routable, dtype=np.int32)
    return Layer(cfg=cfg, x_bits=draw_tokens(seed, T, H), w_router=w_router, bias=bias,
                 expert_slot=expert_slot, slot_expert=order[:n_routable].astype(np.int32),
                 expert_content=content_map(seed, E, cfg.n_contents), ranks=None, order=order,
                 model_seed=seed)


def arena40_layer_counts(seed: int = 505, L: int = 40, E: int = 256, total: int = 6666,
                         alpha: float = 20.0, lo_frac: float = 0.4, hi_frac: float = 0.9) -> np.ndarray:
    """Per-layer resident counts for the 40-layer shared arena.

    Dirichlet(alpha * 1_L) shares of the total, clamped to
    [ceil(lo*E), floor(hi*E)] and rebalanced by largest remainder so that the
    counts sum to the total.
    """
    g = rng(seed, "layer_split", 0)
    share = g.dirichlet(np.full(L, alpha))
    lo, hi = math.ceil(lo_frac * E), math.floor(hi_frac * E)
    if not L * lo <= total <= L * hi:
        raise ValueError(f"{total} residents cannot be split over {L} layers within [{lo}, {hi}]")
    raw = share * total
    cnt = np.clip(np.floor(raw), lo, hi).astype(np.int64)
    rem = raw - np.floor(raw)
    by_rem_desc = np.argsort(-rem, kind="stable")
    while cnt.sum() != total:
        diff = total - int(cnt.sum())
        if diff > 0:
            cand = [i for i in by_rem_desc if cnt[i] < hi][:diff]
            cnt[cand] += 1
        else:
            cand = [i for i in by_rem_desc[::-1] if cnt[i] > lo][:-diff]
            cnt[cand] -= 1
    return cnt


# ----------------------------------------------------------------------------
# several layers sharing one arena
# ----------------------------------------------------------------------------
@dataclass
class ArenaModel:
    """L layers of one model sharing one arena of S slots.

    layers[l] holds layer l's router, bias and contents; its expert_slot holds
    global slot ids (layer-major: layer 0's residents first).  Tokens of a step
    are shared by all layers.
    """
    cfg: LayerConfig
    layers: list
    counts: np.ndarray          # resident experts per layer
    x_seed: int

    @property
    def L(self) -> int:
        return len(self.layers)

    @property
    def S(self) -> int:
        return int(self.counts.sum())

    def expert_slot_table(self) -> np.ndarray:
        return np.stack([lay.expert_slot for lay in self.layers]).astype(np.int32)

    def tokens(self, step: int, T: int | None = None) -> np.ndarray:
        return draw_tokens(self.x_seed, self.cfg.T if T is None else T, self.cfg.H, step)

    def pair_bytes(self, l: int, e: int) -> np.ndarray:
        return self.layers[l].expert_bytes(e)

    def slot_pairs(self, table: np.ndarray | None = None) -> np.ndarray:
        """[S, 2] (layer, expert) held by each slot under a slot table."""
        table = self.expert_slot_table() if table is None else table
        out = np.full((self.S, 2), -1, dtype=np.int64)
        l, e = np.nonzero(table >= 0)
        out[table[l, e]] = np.stack([l, e], axis=1)
        return out

    def prepack(self):
        for lay in self.layers:
            prepack(lay.model_seed, np.unique(lay.expert_content), self.cfg.H, self.cfg.I,
                    self.cfg.weight_std)


def make_arena_model(cfg: LayerConfig | str = "arena40", distinct_layers: bool = False) -> ArenaModel:
    """Per-layer routers, Zipf biases, residency draws and contents; one arena.

    distinct_layers: layer l draws its contents from its own range of content
    ids (no two layers share weights); otherwise the n_contents contents are
    reused by every layer (addresses stay distinct, so traffic is unchanged).
    """
    cfg = CONFIGS[cfg] if isinstance(cfg, str) else cfg
    L, E, H = cfg.layers, cfg.E, cfg.H
    counts = arena40_layer_counts(cfg.seed, L, E, cfg.resident)
    beta = zipf_beta(cfg.beta_key) if cfg.zipf else 0.0
    layers, nxt = [], 0
    for l in range(L):
        w_router = rng(cfg.seed, "router", l).standard_normal((E, H), dtype=np.float32) \
            * np.float32(cfg.router_std)
        if cfg.zipf:
            ranks = popularity_ranks(cfg.seed, E, l)
            bias = zipf_bias(ranks, beta, cfg.zipf_s)
        else:
            ranks, bias = None, np.zeros(E, dtype=np.float32)
        order = residency_order(cfg.seed, ranks, E, l, cfg.zipf_s)
        c = int(counts[l])
        expert_slot = np.full(E, -1, dtype=np.int32)
        expert_slot[order[:c]] = np.arange(nxt, nxt + c, dtype=np.int32)
        nxt += c
        layers.append(Layer(cfg=cfg, x_bits=np.zeros((0, H), np.uint16), w_router=w_router,
                            bias=bias, expert_slot=expert_slot,
                            slot_expert=order[:c].astype(np.int32),
                            expert_content=content_map(cfg.seed, E, cfg.n_contents, l)
                            + (l * cfg.n_contents if distinct_layers else 0),
                            ranks=ranks, order=order, model_seed=cfg.seed, beta=float(beta),
                            extra={"n_resident": c, "n_ring": 0, "layer": l}))
    return ArenaModel(cfg=cfg, layers=layers, counts=counts, x_seed=cfg.seed + 7)
