// NSA block selection on gfx950: Sel rows from per-block importance scores.
//
// The pages give the selection's hyper-parameters (Flash-Sparse-Attention
// README, Usage: topk, init_blocks, local_blocks) and say that every query
// token picks T KV blocks per KV head (FSA paper notes, Background and
// motivation); the scores (NSA's compressed attention) are an input.  Row
// (h, t), own block b:
//   positions [0, Kf)         the forced blocks: initial blocks 0 .. init-1
//                             (those <= b), then b, b-1, .. (local blocks not
//                             already initial), truncated to T;
//   positions [Kf, Kf + m)    the other blocks e <= b by score descending, ties
//                             to the smaller e, NaN counting as -inf;
//   positions [Kf + m, T)     -1.
//
// One wave per row.  Each candidate becomes a 64-bit key (order-preserving
// image of the float score << 32 | ~e), so the wanted order is the unsigned
// integer order and no floating-point operation touches the scores (-0 is
// folded into +0 and NaN into -inf on the bit pattern).  A lane holds the
// keys of blocks lane, lane + 64, .. and tracks its three best.  Each round
// takes the wave-wide maximum of the lanes' bests (DPP on the score half, a
// ballot for the owning lane, no LDS), emits its block, and the owner moves
// to its next best; it rescans below the winner only when it wins a fourth
// time.  Groups of 64 blocks wholly past the own block are skipped
// (wave-uniform).  Rows of up to 64 * kSelRegs candidates keep their keys in
// registers; longer rows rescan from memory.  A row's score loads are all
// issued before its first key is built.
#include "fsa_internal.h"

namespace fsa {
namespace {

constexpr int kSelWaves = 4;
constexpr int kSelRegs = kSelRegBlocks / 64;  // candidate keys per lane kept in registers

// Order-preserving unsigned image of a float score; NaN as -inf, -0 as +0.
// Every real score maps above 0, which marks "no candidate".
__device__ __forceinline__ uint32_t score_order(uint32_t u) {
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) u = 0xFF800000u;  // NaN -> -inf
  if (u == 0x80000000u) u = 0u;                          // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Key of block e from the bit pattern of its score.
__device__ __forceinline__ uint64_t cand_key(uint32_t score_bits, int e) {
  return ((uint64_t)score_order(score_bits) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint32_t score_bits(const float* __restrict__ row_scores, int e) {
  return __builtin_bit_cast(uint32_t, row_scores[e]);
}

// Rows past kSelRegBlocks blocks stream their scores in batches of
// kSelBatch groups of 64, every load of a batch issued before its first use.
constexpr int kSelBatch = 8;

// One step of a wave-wide unsigned maximum: the DPP-moved neighbour's value
// (0, the identity, in rows outside ROW_MASK) against the lane's own; the
// compiler folds the move into a DPP-modified v_max_u32.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t x) {
  const uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, false);
  return x > y ? x : y;
}

// Maximum over the wave, returned as a scalar: quad swaps, half-row and row
// mirrors (each 16-lane row then holds its maximum), row_bcast15 /
// row_bcast31 carry rows 0-2 into row 3, and lane 63 is read back.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = dpp_max_step<0xB1, 0xF>(x);   // quad_perm [1, 0, 3, 2]
  x = dpp_max_step<0x4E, 0xF>(x);   // quad_perm [2, 3, 0, 1]
  x = dpp_max_step<0x141, 0xF>(x);  // row_half_mirror
  x = dpp_max_step<0x140, 0xF>(x);  // row_mirror
  x = dpp_max_step<0x142, 0xA>(x);  // row_bcast15 into rows 1, 3
  x = dpp_max_step<0x143, 0xC>(x);  // row_bcast31 into rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

template <bool IN_REGS>
__global__ __launch_bounds__(kSelWaves * 64) void k_select(const float* __restrict__ scores, int64_t S,
                                                           const int32_t* __restrict__ cu, int num_seqs, int N,
                                                           int H, int BK, int T, int init_blocks, int local_blocks,
                                                           int32_t* __restrict__ sel) {
  const int lane = threadIdx.x & 63;
  // wave-uniform row, held in scalar registers so the sequence lookup uses
  // scalar loads; below 2^32 since rows < 2^31
  const int64_t row =
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(blockIdx.x * kSelWaves + (threadIdx.x >> 6)));
  if (row >= (int64_t)H * N) return;  // wave-uniform; no barrier in this kernel
  const int t = (int)(row % N);
  const int s = seq_of_token(cu, num_seqs, t);
  const int own = (t - cu[s]) / BK;
  if (IN_REGS != (own + 1 <= 64 * kSelRegs)) return;  // the other instantiation takes this row
  const float* const rs = scores + row * S;
  int32_t* const out = sel + row * T;

  // forced blocks: n_init initial ones, then the local ones not already initial
  const int n_init = min(init_blocks, own + 1);
  const int n_loc = max(0, min(local_blocks, own - init_blocks + 1));
  const int kf = min(n_init + n_loc, T);
  for (int p = lane; p < kf; p += 64) out[p] = p < n_init ? p : own - (p - n_init);
  // A candidate is a causal block that is neither initial nor local:
  // init <= e <= own - local (own - e >= local already implies e <= own),
  // tested with one unsigned compare when the range is not empty.
  const int cand_hi = own - local_blocks;
  const uint32_t cand_span = (uint32_t)(cand_hi - init_blocks);
  const bool any_cand = cand_hi >= init_blocks;
  auto candidate = [&](int e) { return any_cand && (uint32_t)(e - init_blocks) <= cand_span; };

  const int want = T - kf;
  int picked = 0;
  if (want > 0) {
    // Each lane tracks its three best keys; after its best is taken, the
    // next ones move up, and only when all three are gone does it rescan.
    uint64_t keys[IN_REGS ? kSelRegs : 1];
    uint64_t best = 0, second = 0, third = 0;
    auto offer = [&](uint64_t k) {  // selects only: no branch per key
      const uint64_t lo1 = k < best ? k : best;
      best = k > best ? k : best;
      const uint64_t lo2 = lo1 < second ? lo1 : second;
      second = lo1 > second ? lo1 : second;
      third = lo2 > third ? lo2 : third;
    };
    // every score load of the row goes out before the first key is built
    // (a key built right after its load would wait for each group in turn)
    auto scan = [&](uint64_t below) {  // offers the candidate keys < below
      for (int e0 = 0; e0 <= own; e0 += 64 * kSelBatch) {
        uint32_t raw[kSelBatch];
#pragma unroll
        for (int u = 0; u < kSelBatch; ++u) {
          const int e = e0 + lane + 64 * u;
          raw[u] = candidate(e) ? score_bits(rs, e) : 0u;
        }
#pragma unroll
        for (int u = 0; u < kSelBatch; ++u) {
          const int e = e0 + lane + 64 * u;
          const uint64_t k = candidate(e) ? cand_key(raw[u], e) : 0;
          offer(k < below ? k : 0);
        }
      }
    };
    if constexpr (IN_REGS) {
      uint32_t raw[kSelRegs];
#pragma unroll
      for (int j = 0; j < kSelRegs; ++j) {
        const int e = lane + 64 * j;
        // groups wholly past the own block load nothing (wave-uniform)
        raw[j] = 64 * j <= own && candidate(e) ? score_bits(rs, e) : 0u;
      }
#pragma unroll
      for (int j = 0; j < kSelRegs; ++j) {
        const int e = lane + 64 * j;
        keys[j] = 64 * j <= own && candidate(e) ? cand_key(raw[j], e) : 0;
        if (64 * j <= own) offer(keys[j]);
      }
    } else {
      scan(~uint64_t(0));
    }
    int exact = 2;  // how many of (second, third) are the lane's next keys below best
    for (; picked < want; ++picked) {
      // the wave's largest key: maximum of the score halves, then among the
      // lanes holding that score (nearly always one) the largest index half
      const uint32_t best_hi = (uint32_t)(best >> 32);
      const uint32_t win_hi = wave_max_u32(best_hi);
      if (win_hi == 0) break;  // no candidate left (wave-uniform)
      const uint64_t tied = __ballot(best_hi == win_hi);
      const uint32_t win_lo = __popcll(tied) == 1
                                  ? (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)best, __ffsll((long long)tied) - 1)
                                  : wave_max_u32(best_hi == win_hi ? (uint32_t)best : 0u);
      const uint64_t win = ((uint64_t)win_hi << 32) | win_lo;
      if (lane == 0) out[kf + picked] = (int32_t)(0xFFFFFFFFu - win_lo);
      if (best == win) {  // keys are unique: exactly one lane owned the winner
        if (exact > 0) {
          best = second;
          second = third;
          third = 0;
          --exact;
        } else {
          best = second = third = 0;
          if constexpr (IN_REGS) {
#pragma unroll
            for (int j = 0; j < kSelRegs; ++j)
              if (64 * j <= own) offer(keys[j] < win ? keys[j] : 0);
          } else {
            scan(win);
          }
          exact = 2;
        }
      }
    }
  }
  for (int p = kf + picked + lane; p < T; p += 64) out[p] = -1;
}

}  // namespace

hipError_t launch_select(const Geometry& geo, const int32_t* cu_dev, const float* scores, int64_t S, int init_blocks,
                         int local_blocks, int32_t* sel, hipStream_t stream) {
  const int64_t rows = (int64_t)geo.H * geo.N;
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows + kSelWaves - 1) / kSelWaves;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_select<true>), dim3((unsigned)blocks), dim3(kSelWaves * 64), 0, stream, scores, S, cu_dev,
                     geo.num_seqs, geo.N, geo.H, geo.BK, geo.T, init_blocks, local_blocks, sel);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !geo.select_long_rows) return e;
  hipLaunchKernelGGL((k_select<false>), dim3((unsigned)blocks), dim3(kSelWaves * 64), 0, stream, scores, S, cu_dev,
                     geo.num_seqs, geo.N, geo.H, geo.BK, geo.T, init_blocks, local_blocks, sel);
  return hipGetLastError();
}

}  // namespace fsa
