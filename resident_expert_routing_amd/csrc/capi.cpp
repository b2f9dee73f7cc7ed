// Host-only parts of the C ABI: status text, format sizes, workspace sizing,
// and arena_load_slot (one host-to-device copy of a host-read expert into a
// slot on a side stream, TideLM README "How adaptive expert loading works",
// item 3).
#include "common.hpp"

size_t moe_route_ws_bytes_internal(int T, int H, int E, int S);
size_t moe_demand_ws_bytes_internal(int T, int E);
size_t moe_experts_ws_bytes_internal(int T, int H, int k, int I, int S, bool shared, int fmt);
size_t moe_hot_pick_ws_bytes_internal(int T);

using namespace moe;

extern "C" MOE_EXPORT const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK: success";
    case MOE_EINVAL: return "MOE_EINVAL: null pointer, bad size or misaligned pointer";
    case MOE_EUNSUPPORTED:
      return "MOE_EUNSUPPORTED: H or I not a multiple of 32, k > min(E, 32), E > 1024 or S > 8192";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace smaller than moe_workspace_bytes()";
    case MOE_EHIP: return "MOE_EHIP: a HIP launch or copy failed";
    case MOE_EIO: return "MOE_EIO: a history file could not be opened, read, written or renamed";
    case MOE_EFORMAT: return "MOE_EFORMAT: not a history file of this shape, or a damaged one";
    case MOE_ESCRATCH:
      return "MOE_ESCRATCH: the batch needs more workspace than the library's own scratch "
             "(MOE_NOALLOC_SCRATCH_BYTES) holds";
    default: return "unknown moe status";
  }
}

extern "C" MOE_EXPORT size_t moe_mxfp4_row_bytes(int K) {
  if (K <= 0 || K % 32 != 0) return 0;
  return mxfp4_row_bytes(K);
}

extern "C" MOE_EXPORT size_t moe_act_row_bytes(int K, int act_format) {
  if (K <= 0 || K % 32 != 0) return 0;
  if (act_format != MOE_ACT_MXFP4 && act_format != MOE_ACT_MXFP6) return 0;
  return act_row_bytes(K, act_format);
}

extern "C" MOE_EXPORT size_t moe_slot_bytes(int H, int I) {
  if (H <= 0 || I <= 0 || H % 32 != 0 || I % 32 != 0) return 0;
  return slot_layout(H, I).total;
}

extern "C" MOE_EXPORT int moe_slot_sections(int H, int I, size_t* out6) {
  if (!out6) return MOE_EINVAL;
  if (H <= 0 || I <= 0 || H % 32 != 0 || I % 32 != 0) return MOE_EUNSUPPORTED;
  const SlotLayout L = slot_layout(H, I);
  for (int j = 0; j < 6; ++j) out6[j] = L.off[j];
  return MOE_OK;
}

extern "C" MOE_EXPORT size_t moe_workspace_bytes(int op, int T, int H, int E, int k, int I,
                                                 int S) {
  const size_t bad = (size_t)-1;
  if (T < 0) return bad;
  // MOE_OP_ACT_MXFP6 selects the MXFP6 activation rows of the experts' workspace
  const int fmt = (op & MOE_OP_ACT_MXFP6) ? MOE_ACT_MXFP6 : MOE_ACT_MXFP4;
  op &= ~MOE_OP_ACT_MXFP6;
  if (fmt == MOE_ACT_MXFP6 && op != MOE_OP_EXPERTS && op != MOE_OP_EXPERTS_SHARED) return bad;
  switch (op) {
    case MOE_OP_ROUTE:
      if (H <= 0 || E <= 0 || H % 32 != 0) return bad;
      return moe_route_ws_bytes_internal(T, H, E, S);
    case MOE_OP_DEMAND:
      if (E <= 0) return bad;
      return moe_demand_ws_bytes_internal(T, E);
    case MOE_OP_EXPERTS:
    case MOE_OP_EXPERTS_SHARED:
      if (H <= 0 || I <= 0 || k <= 0 || S < 0 || H % 32 != 0 || I % 32 != 0) return bad;
      return moe_experts_ws_bytes_internal(T, H, k, I, S, op == MOE_OP_EXPERTS_SHARED, fmt);
    case MOE_OP_HOT_PICK:
      return moe_hot_pick_ws_bytes_internal(T);
    default:
      return bad;
  }
}

extern "C" MOE_EXPORT int arena_load_slot(uint8_t* arena, size_t slot_stride, int num_slots,
                                          int slot, const void* host_src, size_t bytes,
                                          hipStream_t side_stream, hipEvent_t done) {
  if (!arena || !host_src) return MOE_EINVAL;
  if (num_slots <= 0 || slot < 0 || slot >= num_slots) return MOE_EINVAL;
  if (slot_stride == 0 || slot_stride % 256 != 0 || bytes == 0 || bytes > slot_stride)
    return MOE_EINVAL;
  uint8_t* dst = arena + (size_t)slot * slot_stride;
  if (hipMemcpyAsync(dst, host_src, bytes, hipMemcpyHostToDevice, side_stream) != hipSuccess)
    return MOE_EHIP;
  if (done && hipEventRecord(done, side_stream) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}
