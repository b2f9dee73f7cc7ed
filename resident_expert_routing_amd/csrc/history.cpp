// The demand history across restarts and the arena filled from it at boot
// (TideLM README, "How adaptive expert loading works", item 1: the history
// persists across restarts and the arena is filled from it at boot;
// "Settings worth knowing": the learned history lives in a state file).
// Host code only: no HIP call.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "common.hpp"

namespace {

constexpr char kMagic[8] = {'M', 'O', 'E', 'H', 'I', 'S', 'T', 1};
constexpr size_t kHeader = 24;  // magic, L, E, tokens

uint64_t fnv1a(const uint8_t* p, size_t n, uint64_t h = 0xcbf29ce484222325ull) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 0x100000001b3ull;
  }
  return h;
}

void put_u32(std::vector<uint8_t>& b, size_t at, uint32_t v) {
  for (int i = 0; i < 4; ++i) b[at + i] = (uint8_t)(v >> (8 * i));
}
void put_u64(std::vector<uint8_t>& b, size_t at, uint64_t v) {
  for (int i = 0; i < 8; ++i) b[at + i] = (uint8_t)(v >> (8 * i));
}
uint32_t get_u32(const std::vector<uint8_t>& b, size_t at) {
  uint32_t v = 0;
  for (int i = 0; i < 4; ++i) v |= (uint32_t)b[at + i] << (8 * i);
  return v;
}
uint64_t get_u64(const std::vector<uint8_t>& b, size_t at) {
  uint64_t v = 0;
  for (int i = 0; i < 8; ++i) v |= (uint64_t)b[at + i] << (8 * i);
  return v;
}

bool valid_value(double v) { return std::isfinite(v) && v >= 0.0; }

}  // namespace

extern "C" MOE_EXPORT int moe_history_save(const char* path, const double* hist, int L, int E,
                                           uint64_t tokens) {
  if (!path || !hist || L <= 0 || E <= 0) return MOE_EINVAL;
  const size_t n = (size_t)L * (size_t)E;
  for (size_t i = 0; i < n; ++i)
    if (!valid_value(hist[i])) return MOE_EINVAL;
  std::vector<uint8_t> b(kHeader + 8 * n + 8);
  std::memcpy(b.data(), kMagic, 8);
  put_u32(b, 8, (uint32_t)L);
  put_u32(b, 12, (uint32_t)E);
  put_u64(b, 16, tokens);
  for (size_t i = 0; i < n; ++i) {
    uint64_t bits;
    std::memcpy(&bits, &hist[i], 8);
    put_u64(b, kHeader + 8 * i, bits);
  }
  put_u64(b, kHeader + 8 * n, fnv1a(b.data(), kHeader + 8 * n));
  // written beside the target and renamed over it: a reader sees the old file
  // or the new one, never half of one
  const std::string tmp = std::string(path) + ".tmp";
  FILE* f = std::fopen(tmp.c_str(), "wb");
  if (!f) return MOE_EIO;
  const bool ok = std::fwrite(b.data(), 1, b.size(), f) == b.size();
  const bool closed = std::fclose(f) == 0;
  if (!ok || !closed || std::rename(tmp.c_str(), path) != 0) {
    std::remove(tmp.c_str());
    return MOE_EIO;
  }
  return MOE_OK;
}

extern "C" MOE_EXPORT int moe_history_load(const char* path, double* hist, int L, int E,
                                           uint64_t* tokens) {
  if (!path || !hist || L <= 0 || E <= 0) return MOE_EINVAL;
  const size_t n = (size_t)L * (size_t)E;
  FILE* f = std::fopen(path, "rb");
  if (!f) return MOE_EIO;
  std::vector<uint8_t> b(kHeader + 8 * n + 8);
  const size_t got = std::fread(b.data(), 1, b.size(), f);
  const int extra = std::fgetc(f);  // the file must end exactly here
  const bool read_error = std::ferror(f) != 0;
  std::fclose(f);
  if (read_error) return MOE_EIO;
  if (got < kHeader || std::memcmp(b.data(), kMagic, 8) != 0) return MOE_EFORMAT;
  if (get_u32(b, 8) != (uint32_t)L || get_u32(b, 12) != (uint32_t)E) return MOE_EFORMAT;
  if (got != b.size() || extra != EOF) return MOE_EFORMAT;
  if (get_u64(b, kHeader + 8 * n) != fnv1a(b.data(), kHeader + 8 * n)) return MOE_EFORMAT;
  std::vector<double> v(n);
  for (size_t i = 0; i < n; ++i) {
    const uint64_t bits = get_u64(b, kHeader + 8 * i);
    std::memcpy(&v[i], &bits, 8);
    if (!valid_value(v[i])) return MOE_EFORMAT;
  }
  std::copy(v.begin(), v.end(), hist);  // the output is written only for a good file
  if (tokens) *tokens = get_u64(b, 16);
  return MOE_OK;
}

extern "C" MOE_EXPORT int moe_boot_plan(const double* hist, int L, int E, int k, int n_slots,
                                        int32_t* expert_slot) {
  if (!hist || !expert_slot || L <= 0 || E <= 0 || k <= 0 || n_slots < 0) return MOE_EINVAL;
  if (E > MOE_MAX_E || k > MOE_MAX_K) return MOE_EUNSUPPORTED;
  const size_t n = (size_t)L * (size_t)E;
  for (size_t i = 0; i < n; ++i)
    if (std::isnan(hist[i])) return MOE_EINVAL;
  const int floor = std::min(k, E);
  if ((size_t)n_slots < (size_t)L * floor) return MOE_EINVAL;
  const size_t want = std::min((size_t)n_slots, n);

  // rank of every expert inside its layer: larger history first, then lower id
  std::vector<int32_t> rank(n);
  std::vector<int32_t> order((size_t)E);
  for (int l = 0; l < L; ++l) {
    const double* h = hist + (size_t)l * E;
    for (int e = 0; e < E; ++e) order[(size_t)e] = e;
    std::sort(order.begin(), order.end(), [h](int32_t a, int32_t b) {
      if (h[a] != h[b]) return h[a] > h[b];
      return a < b;
    });
    for (int r = 0; r < E; ++r) rank[(size_t)l * E + order[(size_t)r]] = r;
  }
  // every layer's floor, then the rest by (larger history, rank, lower layer)
  std::vector<uint8_t> chosen(n, 0);
  std::vector<size_t> rest;
  rest.reserve(n);
  size_t taken = 0;
  for (size_t i = 0; i < n; ++i) {
    if (rank[i] < floor) {
      chosen[i] = 1;
      ++taken;
    } else {
      rest.push_back(i);
    }
  }
  std::sort(rest.begin(), rest.end(), [&](size_t a, size_t b) {
    if (hist[a] != hist[b]) return hist[a] > hist[b];
    if (rank[a] != rank[b]) return rank[a] < rank[b];
    return a / (size_t)E < b / (size_t)E;
  });
  for (size_t j = 0; j < rest.size() && taken < want; ++j, ++taken) chosen[rest[j]] = 1;
  // slots in ascending (layer, expert)
  int32_t s = 0;
  for (size_t i = 0; i < n; ++i) expert_slot[i] = chosen[i] ? s++ : -1;
  return MOE_OK;
}
