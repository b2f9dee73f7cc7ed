"""C-ABI contract on the CPU: the library loads, exports every declared symbol,
and rejects bad arguments with the documented codes before touching HIP."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_arena.h")

import resident_expert_routing_amd as m  # noqa: E402
from resident_expert_routing_amd import binding as B  # noqa: E402
import fixtures  # noqa: E402
from oracle import moe as omoe  # noqa: E402

FAKE = 1 << 20  # a non-null, 256-aligned address that is never dereferenced on reject paths


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    lib = B.load()
    names = declared_functions()
    assert set(names) == set(B.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_no_unexpected_exports():
    out = os.popen(f"nm -D --defined-only {B.LIB_PATH}").read()
    syms = {l.split()[-1] for l in out.splitlines() if " T " in l}
    ours = {s for s in syms if s.startswith(("moe_", "arena_"))}
    assert ours == set(B.EXPORTS)


def test_status_strings():
    for code in (B.MOE_OK, B.MOE_EINVAL, B.MOE_EUNSUPPORTED, B.MOE_EWORKSPACE, B.MOE_EHIP):
        s = B.status_string(code)
        assert s.startswith("MOE_")
    assert B.status_string(12345) == "unknown moe status"


def test_layout_helpers_match_documented_format():
    assert B.moe_mxfp4_row_bytes(4096) == 2176
    assert B.moe_mxfp4_row_bytes(256) == 144
    assert B.moe_mxfp4_row_bytes(100) == 0
    for H, I in ((256, 128), (4096, 2048), (6144, 2048), (96, 64)):
        lay = fixtures.SlotLayout(H, I)
        assert B.moe_slot_bytes(H, I) == lay.nbytes
        assert B.moe_slot_sections(H, I) == [lay.sections[n][0] for n in (
            "gate_codes", "gate_scales", "up_codes", "up_scales", "down_codes", "down_scales")]
        sec = omoe.slot_sections(H, I)
        assert sec["total"] == lay.nbytes
    assert B.moe_slot_bytes(100, 64) == 0
    with pytest.raises(B.MoeError):
        B.moe_slot_sections(64, 48)


def test_activation_row_bytes():
    """MXFP4 rows as moe_mxfp4_row_bytes; MXFP6 rows 24 code bytes per block of
    32 then a scale byte per block, padded to 16."""
    from oracle import mxfp6
    assert B.moe_act_row_bytes(4096, B.MOE_ACT_MXFP4) == B.moe_mxfp4_row_bytes(4096)
    for K in (32, 96, 512, 2048, 4096, 7168):
        want = (mxfp6.row_bytes(K) + 15) // 16 * 16
        assert B.moe_act_row_bytes(K, B.MOE_ACT_MXFP6) == want
    assert B.moe_act_row_bytes(4096, B.MOE_ACT_MXFP6) == 3200
    assert B.moe_act_row_bytes(100, B.MOE_ACT_MXFP6) == 0
    assert B.moe_act_row_bytes(0, B.MOE_ACT_MXFP4) == 0
    assert B.moe_act_row_bytes(4096, 2) == 0
    assert B.moe_act_row_bytes(4096, -1) == 0


def test_workspace_sizes():
    ws = B.moe_workspace_bytes
    assert ws(B.MOE_OP_ROUTE, 0, 4096, 256, 8, 0, 230) == 0
    # float64 logits, demand partials (chunks of 64 tokens x 256 experts), then
    # bucket counts (chunks of 64 tokens x slots, 256-byte aligned)
    up = lambda v: (v + 255) // 256 * 256
    assert ws(B.MOE_OP_ROUTE, 8, 4096, 256, 8, 0, 230) == 8 * 256 * 8 + up(230 * 4)
    # larger batches with H a multiple of 512 add the certified router's
    # ||w_e||^2 (float64 [E]), the flagged-token list ([1 + T] int32)
    assert ws(B.MOE_OP_ROUTE, 2048, 4096, 256, 8, 0, 166) == \
        2048 * 256 * 8 + 32 * 256 * 8 + up(32 * 166 * 4) + up(256 * 8) + up(2049 * 4) \
        + 3 * 256 * 4096 * 2 + 3 * 2048 * 8 \
        + 4 * 2048 * 256 * 8       # bf16 planes of w, per-token bounds, four K parts of z
    assert ws(B.MOE_OP_ROUTE, 100, 96, 16, 4, 0, 10) == \
        up(100 * 16 * 8) + 2 * 16 * 8 + up(2 * 10 * 4)   # H % 64 != 0: no certification
    assert ws(B.MOE_OP_DEMAND, 64, 0, 256, 8, 0, 0) == 0
    assert ws(B.MOE_OP_DEMAND, 65, 0, 256, 8, 0, 0) == 2 * 256 * 8
    e = ws(B.MOE_OP_EXPERTS, 8, 4096, 0, 8, 2048, 230)
    assert e >= 64 * (1088 + 4096 * 4) and e % 256 == 0
    assert ws(7, 8, 4096, 256, 8, 2048, 230) == (1 << 64) - 1
    # MXFP6 activations: h rows of 3I/4 + I/32 bytes; the flag only with the experts ops
    f6 = ws(B.MOE_OP_EXPERTS | B.MOE_OP_ACT_MXFP6, 8, 4096, 0, 8, 2048, 230)
    assert f6 >= 64 * (1600 + 4096 * 4) and f6 > e and f6 % 256 == 0
    assert ws(B.MOE_OP_EXPERTS_SHARED | B.MOE_OP_ACT_MXFP6, 8, 4096, 0, 8, 2048, 230) >= \
        72 * (1600 + 4096 * 4)
    assert ws(B.MOE_OP_ROUTE | B.MOE_OP_ACT_MXFP6, 8, 4096, 256, 8, 0, 230) == (1 << 64) - 1
    # the pipelined family's tile list is absent for MXFP6 (small-batch kernels only)
    big4 = ws(B.MOE_OP_EXPERTS, 4096, 4096, 0, 8, 2048, 166)
    big6 = ws(B.MOE_OP_EXPERTS | B.MOE_OP_ACT_MXFP6, 4096, 4096, 0, 8, 2048, 166)
    assert big6 > 0 and big4 > 0
    assert ws(B.MOE_OP_ROUTE, 8, 100, 256, 8, 0, 230) == (1 << 64) - 1


def _route(**kw):
    a = dict(T=8, H=256, E=16, k=4, S=10, x=FAKE, w_router=FAKE, bias=None, expert_slot=FAKE,
             topk_expert=FAKE, topk_score=FAKE, sel_expert=FAKE, sel_weight=FAKE, sel_slot=FAKE,
             slot_offsets=FAKE, perm=FAKE, xq=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return B.moe_route(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), B.MOE_EINVAL),
    (dict(w_router=None), B.MOE_EINVAL),
    (dict(slot_offsets=None), B.MOE_EINVAL),
    (dict(perm=None), B.MOE_EINVAL),
    (dict(xq=None), B.MOE_EINVAL),
    (dict(T=-1), B.MOE_EINVAL),
    (dict(H=0), B.MOE_EINVAL),
    (dict(H=100), B.MOE_EUNSUPPORTED),
    (dict(k=17), B.MOE_EUNSUPPORTED),
    (dict(k=33, E=64), B.MOE_EUNSUPPORTED),
    (dict(E=2048), B.MOE_EUNSUPPORTED),
    (dict(S=9000), B.MOE_EUNSUPPORTED),
    (dict(ws_bytes=16), B.MOE_EWORKSPACE),
    (dict(ws=None), B.MOE_EINVAL),
    (dict(x=FAKE + 2), B.MOE_EINVAL),
    (dict(xq=FAKE + 8), B.MOE_EINVAL),
    (dict(act_format=2), B.MOE_EINVAL),
    (dict(act_format=-1), B.MOE_EINVAL),
])
def test_route_rejects(kw, code):
    assert _route(**kw) == code


def test_route_null_args_struct():
    assert B.load().moe_route(None, None) == B.MOE_EINVAL


def test_demand_rejects():
    d = B.moe_demand_accumulate
    assert d(FAKE, FAKE, 8, 4, 16, None, None, None, 0) == B.MOE_EINVAL
    assert d(None, FAKE, 8, 4, 16, FAKE, None, None, 0) == B.MOE_EINVAL
    assert d(FAKE, FAKE, 8, 40, 16, FAKE, None, None, 0) == B.MOE_EUNSUPPORTED
    assert d(FAKE, FAKE, 8, 4, 2000, FAKE, None, None, 0) == B.MOE_EUNSUPPORTED
    assert d(FAKE, FAKE, 100, 4, 16, FAKE, None, None, 0) == B.MOE_EWORKSPACE
    assert d(FAKE, FAKE, 100, 4, 16, FAKE, None, None, 1 << 20) == B.MOE_EINVAL
    assert d(FAKE, FAKE, -1, 4, 16, FAKE, None, None, 0) == B.MOE_EINVAL


def _experts(**kw):
    a = dict(T=8, H=256, I=128, k=4, S=10, xq=FAKE, arena=FAKE, slot_stride=52224,
             slot_offsets=FAKE, perm=FAKE, sel_slot=FAKE, sel_weight=FAKE, out=FAKE, ws=FAKE,
             ws_bytes=1 << 30)
    a.update(kw)
    return B.moe_experts_forward(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(xq=None), B.MOE_EINVAL),
    (dict(arena=None), B.MOE_EINVAL),
    (dict(out=None), B.MOE_EINVAL),
    (dict(perm=None), B.MOE_EINVAL),
    (dict(I=100), B.MOE_EUNSUPPORTED),
    (dict(H=96 + 8), B.MOE_EUNSUPPORTED),
    (dict(slot_stride=52224 - 256), B.MOE_EINVAL),
    (dict(slot_stride=52224 + 16), B.MOE_EINVAL),
    (dict(arena=FAKE + 16), B.MOE_EINVAL),
    (dict(ws_bytes=100), B.MOE_EWORKSPACE),
    (dict(ws=None), B.MOE_EINVAL),
    (dict(S=9000), B.MOE_EUNSUPPORTED),
    (dict(k=0), B.MOE_EINVAL),
    (dict(defer_slot=10), B.MOE_EINVAL),
    (dict(defer_slot=-2), B.MOE_EINVAL),
    (dict(defer_slot=3), B.MOE_EINVAL),  # a deferred slot needs an event
    (dict(act_format=2), B.MOE_EINVAL),
    (dict(act_format=B.MOE_ACT_MXFP6), B.MOE_EUNSUPPORTED),  # H, I not multiples of 512
    (dict(act_format=B.MOE_ACT_MXFP6, H=512, I=512, slot_stride=B.moe_slot_bytes(512, 512),
          ws_bytes=100), B.MOE_EWORKSPACE),
])
def test_experts_rejects(kw, code):
    assert _experts(**kw) == code


def test_experts_empty_batch_is_ok_without_hip():
    assert _experts(T=0, xq=None, arena=None, out=None, ws=None, ws_bytes=0) == B.MOE_OK


def test_arena_load_rejects():
    buf = np.zeros(512, dtype=np.uint8)
    host = buf.ctypes.data
    L = B.arena_load_slot
    assert L(None, 256, 4, 0, host, 256) == B.MOE_EINVAL
    assert L(FAKE, 256, 4, 0, None, 256) == B.MOE_EINVAL
    assert L(FAKE, 256, 4, 4, host, 256) == B.MOE_EINVAL
    assert L(FAKE, 256, 4, -1, host, 256) == B.MOE_EINVAL
    assert L(FAKE, 256, 4, 0, host, 257) == B.MOE_EINVAL
    assert L(FAKE, 256, 4, 0, host, 0) == B.MOE_EINVAL
    assert L(FAKE, 300, 4, 0, host, 200) == B.MOE_EINVAL
    assert L(FAKE, 256, 0, 0, host, 200) == B.MOE_EINVAL


def test_probe_rejects():
    assert B.moe_test_mxfp4_probe(0, None, FAKE, FAKE, FAKE, FAKE) == B.MOE_EINVAL
    assert B.moe_test_mxfp4_probe(1, FAKE + 4, FAKE, FAKE, FAKE, FAKE) == B.MOE_EINVAL
    assert B.moe_test_mxfp4_probe(2, FAKE, FAKE, FAKE, FAKE, FAKE) == B.MOE_EINVAL
    # microbenchmarks: validation before any HIP call
    assert B.moe_test_stream_read(None, 256, FAKE, 4) == B.MOE_EINVAL
    assert B.moe_test_stream_read(FAKE, 0, FAKE, 4) == B.MOE_EINVAL
    assert B.moe_test_stream_read(FAKE, 24, FAKE, 4) == B.MOE_EINVAL
    assert B.moe_test_stream_read(FAKE + 8, 256, FAKE, 4) == B.MOE_EINVAL
    assert B.moe_test_stream_read(FAKE, 256, FAKE, 0) == B.MOE_EINVAL
    assert B.moe_test_mfma_loop(10, None, 4) == B.MOE_EINVAL
    assert B.moe_test_mfma_loop(0, FAKE, 4) == B.MOE_EINVAL
    assert B.moe_test_mfma_loop(10, FAKE, 70000) == B.MOE_EINVAL
    assert B.moe_test_mfma_loop(10, FAKE, 4, act_format=2) == B.MOE_EINVAL


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(ImportError):
        B.load()


def hip_runtimes_mapped():
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            p = line.split()[-1]
            if "libamdhip64" in p:
                paths.add(os.path.realpath(p))
    return paths


def test_single_hip_runtime_in_process():
    """The library must share torch's HIP runtime, never map a second one."""
    B.load()
    import torch  # noqa: F401
    assert len(hip_runtimes_mapped()) == 1, hip_runtimes_mapped()


def test_hot_pick_rejects():
    h = B.moe_hot_pick
    assert h(FAKE, FAKE, 8, 4, 16, None, 10, 10, FAKE, 0.2, FAKE) == B.MOE_EINVAL
    assert h(FAKE, FAKE, 8, 4, 16, FAKE, 10, 10, None, 0.2, FAKE) == B.MOE_EINVAL
    assert h(FAKE, FAKE, 8, 4, 16, FAKE, 10, 10, FAKE, 0.2, None) == B.MOE_EINVAL
    assert h(None, FAKE, 8, 4, 16, FAKE, 10, 10, FAKE, 0.2, FAKE) == B.MOE_EINVAL
    assert h(FAKE, FAKE, 8, 40, 16, FAKE, 10, 10, FAKE, 0.2, FAKE) == B.MOE_EUNSUPPORTED
    assert h(FAKE, FAKE, 8, 4, 16, FAKE, 10, 10, FAKE, float("nan"), FAKE) == B.MOE_EINVAL
    assert h(FAKE, FAKE, 8, 4, 16, FAKE, -1, 10, FAKE, 0.2, FAKE) == B.MOE_EINVAL
    for bad in range(3):  # a misaligned topk_expert, topk_score or expert_slot
        args = [FAKE, FAKE, FAKE]
        args[bad] = FAKE + 2
        assert h(args[0], args[1], 8, 4, 16, args[2], 10, 10, FAKE, 0.2, FAKE, FAKE, 256) \
            == B.MOE_EINVAL
    need = B.moe_workspace_bytes(B.MOE_OP_HOT_PICK, 8, 0, 0, 0, 0, 0)
    assert need == 256
    assert h(FAKE, FAKE, 8, 4, 16, FAKE, 10, 10, FAKE, 0.2, FAKE, FAKE, need - 1) == B.MOE_EWORKSPACE
    assert h(FAKE, FAKE, 8, 4, 16, FAKE, 10, 10, FAKE, 0.2, FAKE, None, need) == B.MOE_EINVAL
    assert h(FAKE, FAKE, 8, 4, 16, FAKE, 10, 10, FAKE, 0.2, FAKE, FAKE + 8, need) == B.MOE_EINVAL
    assert B.moe_workspace_bytes(B.MOE_OP_HOT_PICK, 0, 0, 0, 0, 0, 0) == 0
    assert B.moe_workspace_bytes(B.MOE_OP_HOT_PICK, 10 ** 7, 0, 0, 0, 0, 0) == 256 * 16


def test_hot_install_rejects():
    h = B.moe_hot_install
    assert h(None, FAKE, 16, 10, 10) == B.MOE_EINVAL
    assert h(FAKE, None, 16, 10, 10) == B.MOE_EINVAL
    assert h(FAKE + 2, FAKE, 16, 10, 10) == B.MOE_EINVAL
    assert h(FAKE, FAKE + 2, 16, 10, 10) == B.MOE_EINVAL
    assert h(FAKE, FAKE, 16, 10, 10, FAKE + 2) == B.MOE_EINVAL
    assert h(FAKE, FAKE, 0, 10, 10) == B.MOE_EINVAL
    assert h(FAKE, FAKE, 16, -1, 10) == B.MOE_EINVAL
    assert h(FAKE, FAKE, 16, 10, -1) == B.MOE_EINVAL
    assert h(FAKE, FAKE, B.MOE_MAX_E + 1, 10, 10) == B.MOE_EUNSUPPORTED


def test_unrecorded_torch_event_is_refused():
    """A torch.cuda.Event gets its HIP event on its first record; passing one
    before that would hand the library a null event (no record after a copy,
    so a later wait on it would order nothing): the binding refuses it."""
    class Unrecorded:
        cuda_event = 0

    class Recorded:
        cuda_event = 0x1000

    with pytest.raises(ValueError):
        B._event(Unrecorded())
    assert B._event(Recorded()) == 0x1000
    assert B._event(None) is None


def test_noalloc_rejects_before_any_hip_call():
    """moe_experts_forward_noalloc: a workspace argument, or a batch larger
    than the library's scratch, is refused without touching HIP (CPU)."""
    T, H, k, I, S = 2048, 4096, 8, 2048, 166
    assert B.moe_workspace_bytes(B.MOE_OP_EXPERTS, T, H, 0, k, I, S) > \
        B.MOE_NOALLOC_SCRATCH_BYTES
    args = (H, I, k, S, FAKE, FAKE, B.moe_slot_bytes(H, I), FAKE, FAKE, FAKE, FAKE, FAKE)
    assert B.moe_experts_forward_noalloc(T, *args) == B.MOE_ESCRATCH
    assert B.moe_experts_forward_noalloc(8, *args, ws=FAKE, ws_bytes=1 << 24) == B.MOE_EINVAL
    assert B.moe_experts_forward_noalloc(8, 4096, 2048, 8, 230, 0, FAKE, B.moe_slot_bytes(
        4096, 2048), FAKE, FAKE, FAKE, FAKE, FAKE) == B.MOE_EINVAL          # null xq
    assert B.moe_experts_forward_noalloc(8, 4080, 2048, 8, 230, FAKE, FAKE, 1 << 24, FAKE,
                                         FAKE, FAKE, FAKE, FAKE) == B.MOE_EUNSUPPORTED
    assert B.moe_experts_forward_noalloc(0, *args) == B.MOE_OK           # empty batch: nothing
    assert B.status_string(B.MOE_ESCRATCH).startswith("MOE_ESCRATCH")
