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
// keys of blocks lane, lane + 64, ..; each round takes the wave-wide maximum
// of the lanes' current bests, emits its block, and only the lane that owned
// it rescans for its best key below the winner.  Rows of up to 64 * kSelRegs
// candidates keep their keys in registers; longer rows rescan from memory.
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

__device__ __forceinline__ uint64_t cand_key(const float* __restrict__ row_scores, int e) {
  const uint32_t u = __builtin_bit_cast(uint32_t, row_scores[e]);
  return ((uint64_t)score_order(u) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t y = __shfl_xor(x, m, 64);
    x = y > x ? y : x;
  }
  return x;
}

template <bool IN_REGS>
__global__ __launch_bounds__(kSelWaves * 64) void k_select(const float* __restrict__ scores, int64_t S,
                                                           const int32_t* __restrict__ cu, int num_seqs, int N,
                                                           int H, int BK, int T, int init_blocks, int local_blocks,
                                                           int32_t* __restrict__ sel) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kSelWaves + (threadIdx.x >> 6);
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
  auto candidate = [&](int e) { return e <= own && e >= init_blocks && own - e >= local_blocks; };

  const int want = T - kf;
  int picked = 0;
  if (want > 0) {
    uint64_t keys[IN_REGS ? kSelRegs : 1];
    uint64_t best = 0;
    if constexpr (IN_REGS) {
#pragma unroll
      for (int j = 0; j < kSelRegs; ++j) {
        const int e = lane + 64 * j;
        keys[j] = candidate(e) ? cand_key(rs, e) : 0;
        best = keys[j] > best ? keys[j] : best;
      }
    } else {
      for (int e = lane; e <= own; e += 64)
        if (candidate(e)) {
          const uint64_t k = cand_key(rs, e);
          best = k > best ? k : best;
        }
    }
    for (; picked < want; ++picked) {
      const uint64_t win = wave_max_u64(best);
      if (win == 0) break;  // no candidate left (wave-uniform)
      if (lane == 0) out[kf + picked] = (int32_t)(0xFFFFFFFFu - (uint32_t)win);
      if (best == win) {  // keys are unique: exactly one lane owned the winner
        uint64_t nb = 0;
        if constexpr (IN_REGS) {
#pragma unroll
          for (int j = 0; j < kSelRegs; ++j) nb = (keys[j] < win && keys[j] > nb) ? keys[j] : nb;
        } else {
          for (int e = lane; e <= own; e += 64)
            if (candidate(e)) {
              const uint64_t k = cand_key(rs, e);
              nb = (k < win && k > nb) ? k : nb;
            }
        }
        best = nb;
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
