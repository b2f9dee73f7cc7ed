"""The routed-expert MoE layer against a partially resident arena -- oracle side.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  numpy float64 throughout.

Steps, in the order the TideLM README's "How adaptive expert loading works"
section describes them:
  O1 router logits          z = x W_r^T + b
  O2 probabilities          p = softmax over all experts
  O3 unrestricted top-k     the k best experts by (higher z, then lower id)
  O4 demand                 every wanted pick, resident or not, weighted by its
                            routing score p (item 1: "recorded per (layer,
                            expert), weighted by its routing score")
  O5 routable set           experts with a slot (arena or hot ring)
  O6 masked top-k           the router only picks routable experts, a missing
                            pick replaced by the next-best routable one (item 2)
  O7 renormalise            weights = p over the picks, divided by their sum
  O8 bucket                 assignments sorted stably by slot; rows named by
                            index (colibri cluster page, COLIEX01 v2 paragraph)
  O9 MXFP4 activations      see oracle/mxfp4.py
  O10 expert FFN            SwiGLU: down(q(silu(gate(q(x))) * up(q(x))))
  O11 combine               sum over picks in ascending expert id (the cluster
                            page's fixed summation order)
Picks of a token are always emitted in ascending expert id.
"""
from __future__ import annotations

import math

import numpy as np

from . import mxfp4, mxfp6


# ----------------------------------------------------------------------------
# inputs
# ----------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def slot_sections(H: int, I: int) -> dict:
    """Byte offsets of the six sections of one packed expert.

    gate codes [I, H/2], gate scales [I, H/32], up codes, up scales,
    down codes [H, I/2], down scales [H, I/32]; each section starts on a
    256-byte boundary.
    """
    def up(v):
        return -(-v // 256) * 256
    off = 0
    out = {}
    for name, rows, cols in (("gate_codes", I, H // 2), ("gate_scales", I, H // 32),
                             ("up_codes", I, H // 2), ("up_scales", I, H // 32),
                             ("down_codes", H, I // 2), ("down_scales", H, I // 32)):
        out[name] = (off, rows, cols)
        off = up(off + rows * cols)
    out["total"] = off
    return out


def code_position(n: np.ndarray, j: np.ndarray, nbytes: int) -> np.ndarray:
    """Offset, within a code section, of byte j of row n's packed codes (a row
    has nbytes code bytes).  The section is cut into row blocks of 16 rows;
    a block holds, one after another, the tiles of its rows' bytes
    [64c, 64c + w_c) for c = 0, 1, ... (w_c = 64, or what is left for the
    last), and a tile stores its 16 rows one after another, w_c bytes each.
    """
    c = j // 64
    w = np.minimum(64, nbytes - 64 * c)
    return (n // 16) * (16 * nbytes) + c * (16 * 64) + (n % 16) * w + (j - 64 * c)


def decode_expert(slot_bytes: np.ndarray, H: int, I: int):
    """Packed slot bytes -> float64 (Wg [I,H], Wu [I,H], Wd [H,I]).

    Codes are read at code_position (tiles of 16 rows); scales are row by row."""
    sec = slot_sections(H, I)
    b = np.asarray(slot_bytes, dtype=np.uint8)

    def mat(prefix):
        co, r, c = sec[prefix + "_codes"]
        so, rs, cs = sec[prefix + "_scales"]
        pos = code_position(np.arange(r)[:, None], np.arange(c)[None, :], c)
        codes = b[co:co + r * c][pos]
        scales = b[so:so + rs * cs].reshape(rs, cs)
        return mxfp4.decode(codes, scales)
    return mat("gate"), mat("up"), mat("down")


# ----------------------------------------------------------------------------
# O1-O7 routing
# ----------------------------------------------------------------------------
def router_logits(x_bits, w_router, bias=None) -> np.ndarray:
    """O1: z[t,e] = sum_h x[t,h] W_r[e,h] + b[e], float64."""
    x = bf16_to_f64(x_bits)
    w = np.asarray(w_router, dtype=np.float32).astype(np.float64)
    z = x @ w.T
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return z


def softmax(z: np.ndarray) -> np.ndarray:
    """O2: softmax over experts, max-subtracted."""
    m = z.max(axis=1, keepdims=True)
    ez = np.exp(z - m)
    return ez / ez.sum(axis=1, keepdims=True)


def rank_order(z_row: np.ndarray, allowed: np.ndarray | None = None) -> np.ndarray:
    """Experts sorted by key (-z, e): higher logit first, ties to the lower id."""
    ids = np.arange(z_row.shape[0]) if allowed is None else np.flatnonzero(allowed)
    order = np.argsort(-z_row[ids], kind="stable")
    return ids[order]


def topk(z: np.ndarray, k: int) -> np.ndarray:
    """O3: unrestricted top-k per token, ascending expert id, int64 [T,k]."""
    T, E = z.shape
    out = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        out[t] = np.sort(rank_order(z[t])[:k])
    return out


def routable(expert_slot: np.ndarray) -> np.ndarray:
    """O5: experts that hold a slot (arena or ring)."""
    return np.asarray(expert_slot) >= 0


def masked_topk(z: np.ndarray, expert_slot: np.ndarray, k: int) -> np.ndarray:
    """O6: top-min(k,|R|) over routable experts, ascending id, padded with -1."""
    T, E = z.shape
    R = routable(expert_slot)
    n = min(k, int(R.sum()))
    out = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        out[t, :n] = np.sort(rank_order(z[t], R)[:n])
    return out


def gather(p: np.ndarray, picks: np.ndarray) -> np.ndarray:
    """p[t, picks[t,j]] with 0 where the pick is -1."""
    safe = np.where(picks >= 0, picks, 0)
    vals = np.take_along_axis(p, safe, axis=1)
    return np.where(picks >= 0, vals, 0.0)


def renormalise(p: np.ndarray, picks: np.ndarray) -> np.ndarray:
    """O7: w[t,j] = p[t,e_j] / sum_j' p[t,e_j'] over present picks; 0 for padding."""
    v = gather(p, picks)
    s = v.sum(axis=1, keepdims=True)
    return np.where(picks >= 0, v / np.where(s > 0, s, 1.0), 0.0)


def demand(topk_expert: np.ndarray, topk_score: np.ndarray, E: int) -> np.ndarray:
    """O4: delta[e] = sum over tokens (ascending) of the score of pick e."""
    delta = np.zeros(E, dtype=np.float64)
    for t in range(topk_expert.shape[0]):
        for j in range(topk_expert.shape[1]):
            e = int(topk_expert[t, j])
            if e >= 0:
                delta[e] += float(topk_score[t, j])
    return delta


def demand_fast(topk_expert: np.ndarray, topk_score: np.ndarray, E: int) -> np.ndarray:
    """O4, vectorised per token (same order of additions: ascending t)."""
    delta = np.zeros(E, dtype=np.float64)
    te = np.asarray(topk_expert)
    ts = np.asarray(topk_score, dtype=np.float64)
    for t in range(te.shape[0]):
        m = te[t] >= 0
        delta[te[t][m]] += ts[t][m]
    return delta


def bucket(sel_slot: np.ndarray, S: int):
    """O8: per-slot counts, exclusive offsets [S+1] and the stable permutation.

    Assignment a = t*k + j.  perm lists the assignments sorted by slot, and
    within a slot by ascending a; entries past offsets[S] (padded picks) are -1.
    """
    flat = np.asarray(sel_slot).reshape(-1)
    valid = flat >= 0
    counts = np.bincount(flat[valid], minlength=S)[:S]
    offsets = np.zeros(S + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    idx = np.flatnonzero(valid)
    perm = np.full(flat.shape[0], -1, dtype=np.int64)
    perm[:idx.size] = idx[np.argsort(flat[idx], kind="stable")]
    return counts, offsets, perm


def route(x_bits, w_router, bias, expert_slot, k):
    """O1-O8 for one layer call."""
    z = router_logits(x_bits, w_router, bias)
    p = softmax(z)
    te = topk(z, k)
    ts = gather(p, te)
    se = masked_topk(z, expert_slot, k)
    sw = renormalise(p, se)
    es = np.asarray(expert_slot, dtype=np.int64)
    ss = np.where(se >= 0, es[np.where(se >= 0, se, 0)], -1)
    S = int(es.max()) + 1 if (es >= 0).any() else 0
    return {"z": z, "p": p, "topk_expert": te, "topk_score": ts, "sel_expert": se,
            "sel_weight": sw, "sel_slot": ss, "S_min": S}


# ----------------------------------------------------------------------------
# O9-O11 experts and combine
# ----------------------------------------------------------------------------
def silu(v: np.ndarray) -> np.ndarray:
    return v / (1.0 + np.exp(-v))


def quantise_rows(x: np.ndarray, act: str = "mxfp4") -> np.ndarray:
    """O9 applied along each row: activations in MXFP4, or in MXFP6 (E2M3) for
    the activation-format variant; act='bf16' is the no-quantiser diagnostic."""
    if act == "bf16":
        return np.asarray(x, dtype=np.float64)
    if act == "mxfp4":
        return mxfp4.quantise(x)
    if act == "mxfp6":
        return mxfp6.quantise(x)
    raise ValueError(f"unknown activation format {act!r}")


def expert_ffn(xhat: np.ndarray, weights, act: str = "mxfp4") -> np.ndarray:
    """O10: y = q(silu(xhat Wg^T) * (xhat Wu^T)) Wd^T for rows of xhat, float64."""
    wg, wu, wd = weights
    g = xhat @ wg.T
    u = xhat @ wu.T
    h = silu(g) * u
    return quantise_rows(h, act) @ wd.T


def combine(y: np.ndarray, sel_weight: np.ndarray, sel_expert: np.ndarray) -> np.ndarray:
    """O11: out[t] = sum_j w[t,j] y[t,j], j ascending (ascending expert id).

    y is [T, k, H]; padded picks (expert -1) are skipped.
    """
    T, k, H = y.shape
    out = np.zeros((T, H), dtype=np.float64)
    for j in range(k):
        live = sel_expert[:, j] >= 0
        out[live] += sel_weight[live, j][:, None] * y[live, j]
    return out


def experts_forward(x_bits, sel_expert, sel_weight, sel_slot, slot_bytes_fn, H, I,
                    act: str = "mxfp4", tokens=None, decoded=None, shared_bytes=None):
    """O9-O11.  slot_bytes_fn(s) returns slot s's packed bytes.

    tokens: optional subset of token indices to evaluate (sampled parity);
    returns (out [len(tokens), H], y [len(tokens), k, H]).
    decoded: optional dict kept by the caller across calls; the decoded
    weights of each packed byte buffer are stored there (with the buffer, so
    its id stays valid) and reused.  Decoding is exact, so results are the
    same with or without it.
    shared_bytes: optional packed bytes of the layer's shared expert (the
    colibri cluster page's shared-expert item: it takes every row, unweighted,
    and its row is added at one fixed point).  Reading: its output is added
    after the routed picks, with weight 1 -- see shared_combine.
    """
    T, k = sel_expert.shape
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    xhat = quantise_rows(bf16_to_f64(np.asarray(x_bits)[tok]), act)
    y = np.zeros((tok.size, k, H), dtype=np.float64)
    ss = np.asarray(sel_slot)[tok]
    # slots whose byte buffers are the same object are decoded once
    slots = sorted((int(s) for s in np.unique(ss[ss >= 0])), key=lambda s: id(slot_bytes_fn(s)))
    cached_key, cached = None, None
    for s in slots:
        rows, cols = np.nonzero(ss == s)
        src = slot_bytes_fn(s)
        if id(src) != cached_key:
            if decoded is not None:
                if id(src) not in decoded:
                    decoded[id(src)] = (src, decode_expert(src, H, I))
                cached = decoded[id(src)][1]
            else:
                cached = decode_expert(src, H, I)
            cached_key = id(src)
        y[rows, cols] = expert_ffn(xhat[rows], cached, act)
    out = combine(y, np.asarray(sel_weight)[tok], np.asarray(sel_expert)[tok])
    if shared_bytes is not None:
        out = shared_combine(out, expert_ffn(xhat, decode_expert(shared_bytes, H, I), act))
    return out, y


def shared_combine(routed_out: np.ndarray, y_shared: np.ndarray) -> np.ndarray:
    """The shared expert's row joins a token's output unweighted, after the
    routed picks' weighted sum (the one fixed point where it is added)."""
    return routed_out + y_shared


def layer(x_bits, w_router, bias, expert_slot, k, slot_bytes_fn, H, I, act="mxfp4",
          tokens=None, shared_bytes=None):
    """The whole layer call: O1-O11 (with the shared expert, if given)."""
    r = route(x_bits, w_router, bias, expert_slot, k)
    r["delta"] = demand_fast(r["topk_expert"], r["topk_score"], r["p"].shape[1])
    out, y = experts_forward(x_bits, r["sel_expert"], r["sel_weight"], r["sel_slot"],
                             slot_bytes_fn, H, I, act, tokens, shared_bytes=shared_bytes)
    r["out"] = out
    r["y"] = y
    return r


def bf16_round(v: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value (ties to even), returned as float64.

    Rounds directly from the float64 value (no intermediate float32 rounding).
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                      # v = m * 2**e, |m| in [0.5, 1)
    scaled = np.ldexp(m, 8)                 # 8 significant bits
    r = np.round(scaled)                    # numpy rounds half to even
    return np.ldexp(r, e - 8)


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def fsum_dot(a, b) -> float:
    """Correctly rounded dot product of two float sequences (math.fsum)."""
    return math.fsum(float(u) * float(v) for u, v in zip(a, b))
