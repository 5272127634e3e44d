// ffa_dispatch.hip - host-side context-parallel dispatch (no device code).
//
// MagiAttention blog deep-dive, section "Dispatch Solver": the query sequence is
// cut into chunks of chunk_size tokens; every chunk has an attention area (its
// valid (query, key) pairs); the chunks go to cp_size buckets with equal chunk
// counts so that the largest bucket area is as small as possible, which the
// pages solve greedily with a min-heap of buckets in O(n log n).  The rank-local
// slice table (queries of the rank's chunks, keys remapped into a receive
// buffer of the key ranges the rank needs) is what a rank hands to
// ffa_build_block_meta after fetching those keys (section "通信与重叠",
// GroupCast: only the key ranges a rank's slices touch are sent to it).
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <queue>
#include <utility>
#include <vector>

#include "ffa_internal.hpp"

namespace {

struct HSlice {
  int32_t q0, q1, k0, k1, t;
};

bool read_slices(const int32_t* p, int32_t n, int32_t Tq, int32_t Tk, std::vector<HSlice>& out) {
  out.resize(n);
  for (int32_t s = 0; s < n; ++s) {
    const HSlice h{p[5 * s], p[5 * s + 1], p[5 * s + 2], p[5 * s + 3], p[5 * s + 4]};
    if (h.q0 < 0 || h.q0 > h.q1 || h.q1 > Tq || h.k0 < 0 || h.k0 > h.k1 || h.k1 > Tk) return false;
    if (h.t < FFA_FULL || h.t > FFA_BI_CAUSAL) return false;
    out[s] = h;
  }
  return true;
}

// Valid keys of query i in slice h: [lo, hi] inclusive, empty when lo > hi.
// With r = i - q0 the rule bounds c = j - k0 from below by r (INV-CAUSAL,
// BI-CAUSAL) and from above by r + Lk - Lq (CAUSAL, BI-CAUSAL).
inline void row_keys(const HSlice& h, int64_t i, int64_t& lo, int64_t& hi) {
  const int64_t r = i - h.q0, Lq = h.q1 - h.q0, Lk = h.k1 - h.k0;
  lo = h.k0 + ((h.t == FFA_INV_CAUSAL || h.t == FFA_BI_CAUSAL) ? r : 0);
  hi = h.k1 - 1;
  if (h.t == FFA_CAUSAL || h.t == FFA_BI_CAUSAL) hi = std::min(hi, h.k0 + r + Lk - Lq);
}

// Valid pairs of slice h on queries [a, b).
int64_t rows_area(const HSlice& h, int64_t a, int64_t b) {
  a = std::max<int64_t>(a, h.q0);
  b = std::min<int64_t>(b, h.q1);
  int64_t area = 0;
  for (int64_t i = a; i < b; ++i) {
    int64_t lo, hi;
    row_keys(h, i, lo, hi);
    if (hi >= lo) area += hi - lo + 1;
  }
  return area;
}

}  // namespace

extern "C" {

FFA_API ffa_status ffa_chunk_areas(const int32_t* host_slices, int32_t num_slices,
                                   int32_t seqlen_q, int32_t seqlen_k, int32_t chunk_size,
                                   int64_t* areas) {
  if (num_slices < 0 || seqlen_q < 0 || seqlen_k < 0 || chunk_size <= 0) return FFA_ERR_INVALID_ARGUMENT;
  if ((num_slices > 0 && !host_slices) || (seqlen_q > 0 && !areas)) return FFA_ERR_INVALID_ARGUMENT;
  std::vector<HSlice> sl;
  if (!read_slices(host_slices, num_slices, seqlen_q, seqlen_k, sl)) return FFA_ERR_BAD_SLICES;
  const int64_t n = ((int64_t)seqlen_q + chunk_size - 1) / chunk_size;
  std::vector<int64_t> acc(n, 0);
  for (const HSlice& h : sl)
    for (int64_t c = h.q0 / chunk_size; c < n && c * chunk_size < h.q1; ++c)
      acc[c] += rows_area(h, c * chunk_size, (c + 1) * chunk_size);
  if (n > 0) std::memcpy(areas, acc.data(), n * sizeof(int64_t));
  return FFA_OK;
}

FFA_API ffa_status ffa_dispatch_chunks(const int64_t* areas, int32_t num_chunks, int32_t cp_size,
                                       int32_t* bucket) {
  if (!areas || !bucket || num_chunks <= 0 || cp_size <= 0 || num_chunks % cp_size != 0)
    return FFA_ERR_INVALID_ARGUMENT;
  for (int32_t c = 0; c < num_chunks; ++c)
    if (areas[c] < 0) return FFA_ERR_INVALID_ARGUMENT;
  const int32_t cap = num_chunks / cp_size;
  std::vector<int32_t> order(num_chunks);
  for (int32_t c = 0; c < num_chunks; ++c) order[c] = c;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t x, int32_t y) { return areas[x] > areas[y]; });
  // min-heap of (load, bucket); a bucket leaves the heap once it is full
  using Entry = std::pair<int64_t, int32_t>;
  std::priority_queue<Entry, std::vector<Entry>, std::greater<Entry>> heap;
  for (int32_t b = 0; b < cp_size; ++b) heap.push({0, b});
  std::vector<int32_t> count(cp_size, 0);
  for (int32_t c : order) {
    const Entry e = heap.top();
    heap.pop();
    bucket[c] = e.second;
    if (++count[e.second] < cap) heap.push({e.first + areas[c], e.second});
  }
  return FFA_OK;
}

FFA_API ffa_status ffa_rank_slices(const int32_t* host_slices, int32_t num_slices,
                                   int32_t seqlen_q, int32_t seqlen_k, int32_t chunk_size,
                                   const int32_t* chunks, int32_t num_chunks,
                                   int32_t* local_slices, int32_t max_local, int32_t* num_local,
                                   int32_t* kv_ranges, int32_t max_kv, int32_t* num_kv) {
  if (num_slices < 0 || seqlen_q < 0 || seqlen_k < 0 || chunk_size <= 0 || num_chunks < 0 ||
      max_local < 0 || max_kv < 0 || !num_local || !num_kv)
    return FFA_ERR_INVALID_ARGUMENT;
  if ((num_slices > 0 && !host_slices) || (num_chunks > 0 && !chunks)) return FFA_ERR_INVALID_ARGUMENT;
  std::vector<HSlice> sl;
  if (!read_slices(host_slices, num_slices, seqlen_q, seqlen_k, sl)) return FFA_ERR_BAD_SLICES;
  const int64_t n = ((int64_t)seqlen_q + chunk_size - 1) / chunk_size;
  std::vector<char> seen(n, 0);
  for (int32_t i = 0; i < num_chunks; ++i) {
    if (chunks[i] < 0 || chunks[i] >= n || seen[chunks[i]]) return FFA_ERR_INVALID_ARGUMENT;
    seen[chunks[i]] = 1;
  }

  // cut every slice to each owned chunk; local query rows follow the chunk order
  std::vector<HSlice> loc;    // q in local rows, k still global
  int64_t row0 = 0;
  for (int32_t i = 0; i < num_chunks; ++i) {
    const int64_t a = (int64_t)chunks[i] * chunk_size;
    const int64_t b = std::min<int64_t>(a + chunk_size, seqlen_q);
    for (const HSlice& h : sl) {
      const int64_t qa = std::max<int64_t>(a, h.q0), qb = std::min<int64_t>(b, h.q1);
      if (qa >= qb || rows_area(h, qa, qb) == 0) continue;
      HSlice c = h;
      if (h.t == FFA_INV_CAUSAL || h.t == FFA_BI_CAUSAL) c.k0 = (int32_t)(h.k0 + (qa - h.q0));
      if (h.t == FFA_CAUSAL || h.t == FFA_BI_CAUSAL) c.k1 = (int32_t)(h.k1 - (h.q1 - qb));
      c.q0 = (int32_t)(row0 + (qa - a));
      c.q1 = (int32_t)(row0 + (qb - a));
      loc.push_back(c);
    }
    row0 += b - a;
  }

  // the key ranges they touch, merged (overlapping or adjacent) and packed
  std::vector<std::pair<int32_t, int32_t>> kr;
  for (const HSlice& c : loc) kr.push_back({c.k0, c.k1});
  std::sort(kr.begin(), kr.end());
  std::vector<std::pair<int32_t, int32_t>> merged;
  for (const auto& r : kr) {
    if (!merged.empty() && r.first <= merged.back().second)
      merged.back().second = std::max(merged.back().second, r.second);
    else
      merged.push_back(r);
  }

  *num_local = (int32_t)loc.size();
  *num_kv = (int32_t)merged.size();
  if ((int64_t)loc.size() > max_local || (int64_t)merged.size() > max_kv) return FFA_ERR_WORKSPACE_TOO_SMALL;
  if ((!loc.empty() && !local_slices) || (!merged.empty() && !kv_ranges)) return FFA_ERR_INVALID_ARGUMENT;

  std::vector<int32_t> base(merged.size());
  int32_t off = 0;
  for (size_t m = 0; m < merged.size(); ++m) {
    base[m] = off;
    kv_ranges[3 * m] = merged[m].first;
    kv_ranges[3 * m + 1] = merged[m].second;
    kv_ranges[3 * m + 2] = off;
    off += merged[m].second - merged[m].first;
  }
  for (size_t s = 0; s < loc.size(); ++s) {
    const HSlice& c = loc[s];
    // the merged range holding [k0, k1): the last one starting at or before k0
    size_t m = std::upper_bound(merged.begin(), merged.end(), std::make_pair(c.k0, INT32_MAX)) -
               merged.begin() - 1;
    const int32_t shift = base[m] - merged[m].first;
    local_slices[5 * s] = c.q0;
    local_slices[5 * s + 1] = c.q1;
    local_slices[5 * s + 2] = c.k0 + shift;
    local_slices[5 * s + 3] = c.k1 + shift;
    local_slices[5 * s + 4] = c.t;
  }
  return FFA_OK;
}

}  // extern "C"
