// Pulsar's Phase-1 prefix on the host: Max-IDF chunk summaries of every
// block and the per-block prefix table [sink || summaries of earlier blocks]
// (Pith review of "Dropping the Anchor: Statistical Context Summarization
// for Distributed Systems via Pulsar Attention", "What carries the
// argument", "Core claim", "Assumptions & free parameters").  Integer work
// over the token ids only; the pages run it on the CPU.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <unordered_map>
#include <vector>

#include "../../include/star_attn.h"

namespace {

struct Chunk {
  double score;
  int64_t c0, c1;
};

}  // namespace

extern "C" int star_pulsar_prefix(const int32_t* tokens, int64_t L, int64_t block_b,
                                  int32_t chunk_m, int32_t sink, int32_t k, int64_t* rows,
                                  int64_t rows_cap, int64_t* n_rows, int64_t* prefix_start,
                                  int64_t* prefix_len, int32_t nblocks) {
  if (n_rows == nullptr) return STAR_ERR_NULL;
  if (L < 0 || block_b < 1 || chunk_m < 1 || sink < 0 || k < 0 || rows_cap < 0)
    return STAR_ERR_SHAPE;
  const int64_t n = (L + block_b - 1) / block_b;
  if (nblocks != n) return STAR_ERR_SHAPE;
  if (n == 0) {
    *n_rows = 0;
    return STAR_OK;
  }
  if (tokens == nullptr || prefix_start == nullptr || prefix_len == nullptr) return STAR_ERR_NULL;
  try {
    // df(t): number of blocks that contain t.  Token ids of a real
    // vocabulary are small non-negative integers: then one pass with a
    // dense count and the last block that counted each id; otherwise a
    // hash map over each block's distinct ids.
    int32_t tmin = INT32_MAX, tmax = INT32_MIN;
    for (int64_t t = 0; t < L; ++t) {
      tmin = std::min(tmin, tokens[t]);
      tmax = std::max(tmax, tokens[t]);
    }
    const bool dense = tmin >= 0 && tmax < (1 << 24);
    std::vector<int64_t> df_dense;
    std::unordered_map<int32_t, int64_t> df_map;
    if (dense) {
      df_dense.assign((size_t)tmax + 1, 0);
      std::vector<int64_t> last((size_t)tmax + 1, -1);
      for (int64_t i = 0; i < n; ++i) {
        const int64_t s = i * block_b, e = std::min(s + block_b, L);
        for (int64_t t = s; t < e; ++t) {
          const int32_t id = tokens[t];
          if (last[(size_t)id] != i) {
            last[(size_t)id] = i;
            ++df_dense[(size_t)id];
          }
        }
      }
    } else {
      df_map.reserve((size_t)std::min<int64_t>(L, 1 << 22));
      std::vector<int32_t> blk;
      for (int64_t i = 0; i < n; ++i) {
        const int64_t s = i * block_b, e = std::min(s + block_b, L);
        blk.assign(tokens + s, tokens + e);
        std::sort(blk.begin(), blk.end());
        blk.erase(std::unique(blk.begin(), blk.end()), blk.end());
        for (int32_t t : blk) ++df_map[t];
      }
    }
    auto df = [&](int32_t id) -> int64_t {
      return dense ? df_dense[(size_t)id] : df_map[id];
    };
    const int64_t sink_n = std::min<int64_t>(std::min<int64_t>(sink, block_b), L);
    // summary of every block but the last (no later block reads it)
    std::vector<std::vector<int64_t>> summary(n);
    std::vector<Chunk> cand;
    for (int64_t i = 0; i + 1 < n; ++i) {
      const int64_t s = i * block_b, e = std::min(s + block_b, L);
      cand.clear();
      for (int64_t c0 = s; c0 < e; c0 += chunk_m) {
        if (i == 0 && c0 < sink_n) continue;     // already in the sink
        const int64_t c1 = std::min<int64_t>(c0 + chunk_m, e);
        int64_t dmin = INT64_MAX;
        for (int64_t t = c0; t < c1; ++t) dmin = std::min(dmin, df(tokens[t]));
        // max over the chunk of log(n / max(df, 1)) is reached at the
        // smallest df
        cand.push_back({std::log((double)n / (double)std::max<int64_t>(dmin, 1)), c0, c1});
      }
      std::sort(cand.begin(), cand.end(), [](const Chunk& x, const Chunk& y) {
        return x.score != y.score ? x.score > y.score : x.c0 < y.c0;
      });
      if ((int64_t)cand.size() > k) cand.resize((size_t)k);
      std::sort(cand.begin(), cand.end(), [](const Chunk& x, const Chunk& y) { return x.c0 < y.c0; });
      for (const Chunk& c : cand)
        for (int64_t t = c.c0; t < c.c1; ++t) summary[i].push_back(t);
    }
    int64_t total = sink_n;
    for (int64_t i = 0; i + 1 < n; ++i) total += (int64_t)summary[i].size();
    *n_rows = total;
    if (total > rows_cap) return STAR_ERR_SHAPE;
    if (total > 0 && rows == nullptr) return STAR_ERR_NULL;
    int64_t w = 0;
    for (int64_t t = 0; t < sink_n; ++t) rows[w++] = t;
    prefix_start[0] = 0;
    prefix_len[0] = 0;
    int64_t acc = sink_n;
    for (int64_t i = 1; i < n; ++i) {
      for (int64_t t : summary[i - 1]) rows[w++] = t;
      acc += (int64_t)summary[i - 1].size();
      prefix_start[i] = 0;
      prefix_len[i] = acc;
    }
    return STAR_OK;
  } catch (...) {
    return STAR_ERR_UNSUPPORTED;  // allocation failure
  }
}
