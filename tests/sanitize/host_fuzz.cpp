// Host-side fuzz of the library's geometry, sizing and argument checks, built
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code only
// (tests/test_host_sanitize.py).  No kernel is launched: the launchers are
// stubs that abort, and every entry point called here must fail validation.
//
// For seeded random problems (up to the int32 limits of the index tensors):
//   * fsa_get_sizes / compute_geometry return a documented status and never
//     overflow (UBSan traps signed overflow);
//   * for valid problems the workspace layout is ordered, aligned and large
//     enough for the rows the kernels address: partial rows (pair * g + j)
//     and the dump rows below the queue counters, stats pairs likewise, the
//     aux blob's regions in order;
//   * the work-list and slot arithmetic stays in bounds for the largest
//     selection the problem allows: segment counts at their per-block bound
//     (tokens from the block's start to its sequence's end) until max_pairs
//     is reached, and random counts below it: the items
//     sum ceil(count / CT) <= max_work, and every backward chunk slot
//     offsets[f] / CT + f + chunk < kv_slots.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "fsa_internal.h"

#define CHECK(c)                                                            \
  do {                                                                      \
    if (!(c)) {                                                             \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      std::abort();                                                         \
    }                                                                       \
  } while (0)

namespace {

void check_counts(const fsa::Geometry& geo, const std::vector<int32_t>& cu, std::vector<int64_t> cnt) {
  const int64_t CT = geo.chunk_tokens, M = (int64_t)geo.H * geo.NB;
  CHECK((int64_t)cnt.size() == M);
  int64_t off = 0, items = 0, max_slot = -1;
  for (int64_t f = 0; f < M; ++f) {
    const int64_t chunks = (cnt[f] + CT - 1) / CT;
    items += chunks;
    if (chunks > 0) max_slot = std::max(max_slot, off / CT + f + chunks - 1);
    off += cnt[f];
  }
  CHECK(off <= geo.max_pairs);
  CHECK(items <= geo.max_work);
  CHECK(max_slot < geo.kv_slots);
  // partial rows of the last pair and the dump rows fit below the queue counters
  const size_t s_p = geo.partial_dtype == FSA_PARTIAL_FP32 ? 4 : 2;
  CHECK(((size_t)off * geo.g + 32) * geo.d * s_p <= geo.partial_queue_off);
  CHECK(((size_t)geo.dump_row + 32) * geo.d * s_p <= geo.partial_queue_off);
  CHECK(((size_t)geo.dump_row + 32) * 8 <= geo.stats_queue_off);
  CHECK(geo.partial_queue_off + (size_t)fsa::kQueueInts * 4 <= geo.partial_ws_bytes);
  CHECK(geo.stats_queue_off + (size_t)fsa::kQueueInts * 4 <= geo.stats_ws_bytes);
}

// Largest per-segment counts: block e of sequence s can be selected by the
// L_s - e * B_K tokens from its start to the end of the sequence, and a token
// of local block b selects at most min(T, b + 1) blocks; fill segments in a
// seeded order up to those bounds until max_pairs entries are used.
std::vector<int64_t> heavy_counts(const fsa::Geometry& geo, const std::vector<int32_t>& cu, std::mt19937_64& rng,
                                  bool random_fill) {
  std::vector<int64_t> bound;
  for (int h = 0; h < geo.H; ++h)
    for (int s = 0; s < geo.num_seqs; ++s) {
      const int64_t L = cu[s + 1] - cu[s];
      for (int64_t e = 0; e * geo.BK < L; ++e) bound.push_back(L - e * geo.BK);
    }
  std::vector<int64_t> cnt(bound.size(), 0);
  std::vector<size_t> order(bound.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = i;
  std::shuffle(order.begin(), order.end(), rng);
  int64_t left = geo.max_pairs;
  for (size_t i : order) {
    int64_t c = std::min(bound[i], left);
    if (random_fill && c > 0) c = (int64_t)(rng() % (uint64_t)(c + 1));
    cnt[i] = c;
    left -= c;
  }
  return cnt;
}

int32_t pick(std::mt19937_64& rng, std::initializer_list<int32_t> xs) {
  return *(xs.begin() + rng() % xs.size());
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 3000;
  std::mt19937_64 rng(20260);
  int valid = 0, by_status[16] = {0};
  for (int it = 0; it < iters; ++it) {
    // shapes: mostly plausible, some at the edges of what the ABI accepts
    const int B = 1 + (int)(rng() % 6);
    std::vector<int32_t> cu(B + 1, 0);
    const bool huge = rng() % 8 == 0;
    for (int s = 0; s < B; ++s) {
      int64_t L = huge ? (int64_t)(rng() % (1u << 22)) : (int64_t)(rng() % 5000);
      if (rng() % 10 == 0) L = 0;
      cu[s + 1] = (int32_t)std::min<int64_t>(cu[s] + L, INT32_MAX);
    }
    if (rng() % 50 == 0) cu[0] = 1;                              // malformed
    if (rng() % 50 == 0 && B > 1) std::swap(cu[1], cu[B]);       // decreasing
    fsa_problem p{};
    p.num_seqs = rng() % 40 == 0 ? 0 : B;
    p.cu_seqlens_host = cu.data();
    p.cu_seqlens_dev = nullptr;
    p.num_kv_heads = rng() % 20 == 0 ? (int32_t)(rng() % 4096) : 1 + (int32_t)(rng() % 16);
    p.gqa_group = rng() % 20 == 0 ? (int32_t)(rng() % 40) - 2 : 1 + (int32_t)(rng() % 16);
    p.head_dim = rng() % 10 == 0 ? (int32_t)(rng() % 300) : pick(rng, {64, 128, 256});
    p.block_size = rng() % 10 == 0 ? (int32_t)(rng() % 300) : pick(rng, {64, 128});
    p.topk = rng() % 10 == 0 ? (int32_t)(rng() % 300) - 10 : 1 + (int32_t)(rng() % 48);
    p.softmax_scale = rng() % 20 == 0 ? -1.f : 0.f;
    p.dtype = rng() % 30 == 0 ? 5 : (int32_t)(rng() % 2);
    p.partial_dtype = rng() % 30 == 0 ? 9 : (int32_t)(rng() % 2);
    fsa_sizes sz;
    const int32_t st = fsa_get_sizes(&p, &sz);
    CHECK(st >= 0 && st <= FSA_ERR_SCRATCH);
    ++by_status[st];
    fsa::Geometry geo;
    CHECK(fsa::compute_geometry(&p, &geo) == st);
    if (st != FSA_OK) continue;
    ++valid;
    // sizes and layout
    CHECK(sz.counts_bytes >= 4 && sz.qidx_bytes >= 4 && sz.slot_bytes >= 4);
    CHECK(sz.offsets_bytes == ((size_t)geo.H * geo.NB + 1) * 4);
    CHECK(sz.total_tokens == cu[B] && sz.num_blocks == geo.NB);
    CHECK(geo.aux_seq_gboff < geo.aux_nwork && geo.aux_nwork < geo.aux_loc && geo.aux_loc < geo.aux_nloc &&
          geo.aux_nloc < geo.aux_work_sorted && geo.aux_work_sorted < geo.aux_bytes);
    CHECK(geo.aux_work_sorted % 256 == 0 && geo.partial_queue_off % 256 == 0 && geo.stats_queue_off % 256 == 0);
    CHECK((int64_t)geo.H * geo.ntiles * geo.NB <= fsa::kMaxTileHist || geo.N == 0);
    CHECK(geo.win_max >= 1 && geo.win_max <= fsa::kWinMax);
    CHECK(!geo.bwd_ok || (geo.bwd_queue_off >= geo.bwd_kv_off + (size_t)geo.kv_slots * 2 * geo.BK * geo.d * 4 &&
                          geo.bwd_ws_bytes >= geo.bwd_queue_off + (size_t)fsa::kQueueInts * 4));
    CHECK(geo.bwd_kv_off >= geo.bwd_dq_off + geo.partial_rows_bytes);
    // work-list and slot bounds for the heaviest and for random selections
    if ((int64_t)geo.H * geo.NB <= (1 << 22)) {
      check_counts(geo, cu, heavy_counts(geo, cu, rng, false));
      check_counts(geo, cu, heavy_counts(geo, cu, rng, true));
    }
    // entry points refuse before any launch (NULL / misaligned arguments)
    int32_t dummy[64] = {0};
    fsa_index idx{dummy, dummy, dummy, dummy, nullptr};
    CHECK(fsa_build_index(&p, dummy, &idx, dummy, 1 << 20, nullptr) == FSA_ERR_NULL);  // cu_seqlens_dev NULL
    p.cu_seqlens_dev = dummy;
    CHECK(fsa_build_index(&p, dummy, &idx, dummy, 1 << 20, nullptr) == FSA_ERR_NULL);  // aux NULL
    CHECK(fsa_build_index_noalloc(&p, dummy, &idx, nullptr) == FSA_ERR_NULL);
    CHECK(fsa_softmax_stats(&p, nullptr, dummy, &idx, nullptr, nullptr, dummy, 0, nullptr) == FSA_ERR_NULL ||
          geo.N == 0);
  }
  std::printf("iterations %d valid %d statuses", iters, valid);
  for (int s = 0; s <= FSA_ERR_SCRATCH; ++s) std::printf(" %d:%d", s, by_status[s]);
  std::printf("\n");
  CHECK(valid > iters / 4);
  return 0;
}
