// moe_replan: host-side re-plan of one arena shared by all layers (TideLM
// README, "How adaptive expert loading works", item 1).  The coldest resident
// (layer, expert) pairs give their slots to the hottest non-resident pairs,
// never taking a layer below k resident experts.
#include <algorithm>
#include <cmath>
#include <vector>

#include "common.hpp"

namespace {

struct Pair {
  double h;
  int32_t l, e;
};

}  // namespace

extern "C" MOE_EXPORT int moe_replan(const double* hist, const int32_t* expert_slot, int L, int E,
                                     int k, int n_swap, int32_t* evict, int32_t* load,
                                     int32_t* new_expert_slot, int* n_done) {
  if (!hist || !expert_slot || !new_expert_slot || !n_done) return MOE_EINVAL;
  if (L <= 0 || E <= 0 || k <= 0 || n_swap < 0) return MOE_EINVAL;
  if (E > MOE_MAX_E || k > MOE_MAX_K) return MOE_EUNSUPPORTED;
  if (n_swap > 0 && (!evict || !load)) return MOE_EINVAL;
  const size_t n = (size_t)L * (size_t)E;

  std::vector<Pair> res, non;
  std::vector<int32_t> slots;
  std::vector<int> count((size_t)L, 0);
  res.reserve(n);
  non.reserve(n);
  for (int l = 0; l < L; ++l) {
    for (int e = 0; e < E; ++e) {
      const size_t i = (size_t)l * E + e;
      const double h = hist[i];
      if (std::isnan(h)) return MOE_EINVAL;
      if (expert_slot[i] >= 0) {
        res.push_back({h, l, e});
        slots.push_back(expert_slot[i]);
        ++count[(size_t)l];
      } else {
        non.push_back({h, l, e});
      }
    }
  }
  std::sort(slots.begin(), slots.end());
  if (std::adjacent_find(slots.begin(), slots.end()) != slots.end()) return MOE_EINVAL;

  // coldest first; equal histories (+0 and -0 included) go to the lower (l, e)
  std::sort(res.begin(), res.end(), [](const Pair& a, const Pair& b) {
    if (a.h != b.h) return a.h < b.h;
    if (a.l != b.l) return a.l < b.l;
    return a.e < b.e;
  });
  // hottest first, equal histories to the lower (l, e)
  std::sort(non.begin(), non.end(), [](const Pair& a, const Pair& b) {
    if (a.h != b.h) return a.h > b.h;
    if (a.l != b.l) return a.l < b.l;
    return a.e < b.e;
  });

  int taken = 0;
  for (const Pair& p : res) {
    if (taken == n_swap) break;
    if (count[(size_t)p.l] - 1 < k) continue;  // the layer keeps at least k residents
    --count[(size_t)p.l];
    evict[2 * taken] = p.l;
    evict[2 * taken + 1] = p.e;
    ++taken;
  }
  taken = std::min<int>(taken, (int)non.size());

  std::copy(expert_slot, expert_slot + n, new_expert_slot);
  for (int i = 0; i < taken; ++i) {
    const Pair& p = non[(size_t)i];
    load[2 * i] = p.l;
    load[2 * i + 1] = p.e;
    const size_t from = (size_t)evict[2 * i] * E + evict[2 * i + 1];
    new_expert_slot[(size_t)p.l * E + p.e] = expert_slot[from];
    new_expert_slot[from] = -1;
  }
  *n_done = taken;
  return MOE_OK;
}
