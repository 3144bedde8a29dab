// Issue order of the bf16 forward's query tiles and how they are dealt to
// the XCDs (host only).
//
// The forward runs one workgroup per query tile, heaviest frames first
// (frames that see the most key frames), and each XCD starts its next
// workgroup whenever one of its slots frees up, so every XCD works through
// its own list in order. Tiles of one (frame, head) group stream the same
// keys and values, so they are kept together on one XCD, whose L2 then
// serves them once; but whole groups can leave the XCDs with unequal work
// when the groups' costs differ (four heads of frames that see 4, 3 and 2
// key frames, for instance, give half of the XCDs a list that ends a whole
// tile later). The groups are therefore dealt in chunks of C tiles, C
// chosen with a model of the dispatch: each XCD's tiles, in order, go to
// whichever of its slots frees first, a tile costing its 32-key steps plus
// a fixed overhead. The largest chunk whose modelled finish is within a
// small margin of the best is used (larger chunks share more K/V in L2).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <functional>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "fsattn_internal.h"

namespace fsattn {

bool frame_issue_order(const fsattn_mask *m, uint8_t *order) {
  if (m->num_frames > kMaxOrderedFrames) return false;
  int n = 0;
  int64_t most = 0;
  for (int f = 0; f < m->num_frames; ++f) most = std::max(most, live_frame_count(m, f));
  for (int64_t c = most; c >= 1 && n < m->num_frames; --c)
    for (int f = 0; f < m->num_frames; ++f)
      if (live_frame_count(m, f) == c) order[n++] = (uint8_t)f;
  return true;
}

namespace {

// Fixed cost of a tile in 32-key steps (query load, filling the staging
// ring, storing the output).
constexpr double kTileOverhead = 2.0;
// A smaller chunk must beat whole groups' modelled finish by this much.
constexpr double kMargin = 0.005;
// Longest list (tiles per slot) that is modelled; beyond it the imbalance
// is a small share of the launch and whole groups are dealt.
constexpr int64_t kMaxRounds = 64;

// Finish time of `cost` list-scheduled in order on S slots.
double list_finish(const std::vector<double> &cost, int S) {
  std::vector<double> t(S, 0.0);   // min-heap of slot free times
  for (double c : cost) {
    std::pop_heap(t.begin(), t.end(), std::greater<double>());
    t.back() += c;
    std::push_heap(t.begin(), t.end(), std::greater<double>());
  }
  return *std::max_element(t.begin(), t.end());
}

using Key = std::tuple<int, int, int, int, int, int, int, int, int, int, int>;
std::mutex g_mu;
std::map<Key, int> g_cache;

}  // namespace

int choose_deal_chunk(const fsattn_shape *s, const fsattn_mask *m, const FwdConfig &c, int override) {
  const int BH = s->batch * s->heads;
  const int rows = 16 * c.m16 * c.waves;
  const int TPF = (m->tokens_per_frame + rows - 1) / rows;
  if (override == 15) return TPF;
  if (override > 0) return 1 << (override - 1);
  const int64_t G = (int64_t)m->num_frames * BH * TPF;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < kXcds)
    return TPF;
  const int occ = fwd_bf16_occupancy(c, s->head_dim);
  if (occ <= 0) return TPF;
  const int S = cus / kXcds * occ;   // slots per XCD
  if (G > kMaxRounds * kXcds * S) return TPF;

  const Key key{m->num_frames, m->tokens_per_frame, m->window_before, m->window_after, m->ref_frame,
                m->ref_queries_global, m->ref_count, BH, rows, s->head_dim, S};
  {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_cache.find(key);
    if (it != g_cache.end()) return it->second;
  }
  uint8_t order[kMaxOrderedFrames];
  const bool ordered = frame_issue_order(m, order);
  std::vector<double> frame_cost(m->num_frames);
  for (int f = 0; f < m->num_frames; ++f)
    frame_cost[f] = (double)live_frame_count(m, f) * m->tokens_per_frame / 32.0 + kTileOverhead;
  auto finish = [&](int64_t C) {
    double end = 0.0;
    std::vector<double> cost;
    for (int x = 0; x < kXcds; ++x) {
      const int64_t n = xcd_tile_count(G, C, x);
      cost.resize(n);
      for (int64_t t = 0; t < n; ++t) {
        const int64_t g = dealt_tile(G, C, x, t);
        const int fr = (int)(g / TPF / BH);
        cost[t] = frame_cost[ordered ? order[fr] : fr];
      }
      end = std::max(end, list_finish(cost, S));
    }
    return end;
  };
  // candidates from whole groups down to single tiles, largest first
  std::vector<int> cand{TPF};
  for (int C = TPF / 2; C >= 1; C /= 2) cand.push_back(C);
  std::vector<double> fin;
  for (int C : cand) fin.push_back(finish(C));
  const double best = *std::min_element(fin.begin(), fin.end());
  int chosen = TPF;
  if (best < fin[0] * (1.0 - kMargin))
    for (size_t i = 0; i < cand.size(); ++i)
      if (fin[i] <= best * (1.0 + kMargin)) {
        chosen = cand[i];
        break;
      }
  {
    std::lock_guard<std::mutex> lock(g_mu);
    g_cache[key] = chosen;
  }
  return chosen;
}

}  // namespace fsattn
