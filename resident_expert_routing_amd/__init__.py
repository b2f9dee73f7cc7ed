"""MI355X-native routed-expert MoE layer against a partially resident expert arena.

The layer (TideLM README, "How adaptive expert loading works", items 1-3) runs
in libmoe_arena.so's HIP kernels for gfx950, behind the C ABI declared in
include/moe_arena.h.  `binding` wraps that ABI with ctypes; `runtime` adds the
torch plumbing (device buffers, arena upload).  Importing the package loads the
library and fails loudly if it has not been built.
"""
from . import binding
from .binding import (MOE_OP_DEMAND, MOE_OP_EXPERTS, MOE_OP_HOT_PICK, MOE_OP_ROUTE, MoeError,
                      arena_load_slot, check, moe_demand_accumulate,
                      moe_experts_forward, moe_hot_install, moe_hot_pick, moe_mxfp4_row_bytes, moe_replan, moe_route,
                      moe_slot_bytes, moe_slot_sections, moe_status_string,
                      moe_test_mfma_loop, moe_test_mxfp4_probe, moe_test_stream_read,
                      moe_workspace_bytes)

binding.load()

__all__ = ["binding", "MOE_OP_DEMAND", "MOE_OP_EXPERTS", "MOE_OP_HOT_PICK", "MOE_OP_ROUTE",
           "MoeError", "arena_load_slot", "check", "moe_demand_accumulate",
           "moe_experts_forward", "moe_hot_install", "moe_hot_pick", "moe_mxfp4_row_bytes", "moe_replan", "moe_route", "moe_slot_bytes",
           "moe_slot_sections", "moe_status_string", "moe_test_mfma_loop", "moe_test_mxfp4_probe",
           "moe_test_stream_read", "moe_workspace_bytes"]
