// Backward pass of selected attention on gfx950, in the KV-block-outer order
// of the forward (FSA paper notes, Key designs 1-3: per KV block, the block
// is loaded once and the queries that select it stream through; the README's
// Usage and Evaluation sections train the module and check its gradients).
//
//   k_bwd_delta      D[t, hq] = sum_d dO * O  (fp32).
//   k_bwd_main       per work item (KV head, block, query chunk): each lane
//                    keeps the K and V fragments of its key and the K^T
//                    fragments of its dQ d tiles in registers for the whole
//                    item; the item's query rows stream through in 32-row
//                    tiles staged row-major in LDS.  Wave w owns keys
//                    16w .. 16w+15 (4 waves for 64-key blocks, 8 for
//                    128-key blocks): it forms S = Q K^T and dP = dO V^T for its
//                    keys, P = exp(S - lse), dS = P (dP - D), and accumulates
//                    dV^T += dO^T P and dK^T += Q^T dS in registers over the
//                    chunk, reading dO^T and Q^T with LDS transpose reads.
//                    dS of all the keys meets in LDS and dQ^T = K^T dS^T
//                    (split over d across the waves) is staged in LDS and
//                    written as whole rows to the compact partial rows of
//                    the forward.  At the end of the
//                    item the block's dK / dV partial goes to the item's slot
//                    offsets[f] / CT + f + chunk.
//   k_reduce         (the forward's reduction) sums each (token, KV head)'s dQ
//                    partial rows in slot order.
//   k_bwd_kv_reduce  per key row of every block: dK, dV = sum over the
//                    block's chunk slots in chunk order.
// No atomics; every sum has a fixed order, so the gradients are deterministic.
//
// MFMA layouts (wave64, l = lane, u = l / 16).  v_mfma_f32_16x16x32: lane l
// supplies A[l % 16][8u + e] and B[8u + e][l % 16] (e < 8) and receives
// C[4u + r][l % 16] (r < 4).  S = Q K^T over a 16-row block therefore leaves
// lane l with key l % 16 and rows 4u + r.  For dV^T = dO^T P and
// dK^T = Q^T dS, which contract over a 32-row tile, the lane's k range 8u + e
// is taken to mean row 4u + e of the first 16-row block (e < 4) and row
// 4u + e - 4 of the second: the lane's own P / dS values of both blocks form
// the B operand as they are, with no transpose.
#include <math.h>

#include "fsa_internal.h"

namespace fsa {
namespace {

constexpr float kBwdLog2e = 1.4426950408889634f;
// One wave per 16 keys of the block: 4 waves (256 threads) for B_K = 64,
// 8 waves (512 threads) for B_K = 128.
template <int BK>
constexpr int bwd_threads() {
  return BK * 4;
}
constexpr int kBwdRows = 32;  // query rows per tile: two 16-row MFMA blocks
constexpr int kBwdRowTable = kRowsPerItem + kBwdRows;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Vec4;
template <>
struct Vec4<__bf16> {
  using type = bf16x4;
};
template <>
struct Vec4<_Float16> {
  using type = f16x4;
};

__device__ __forceinline__ f32x4 mfma_k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type bld8(const T* p) {
  return *reinterpret_cast<const typename Vec8<T>::type*>(p);
}
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// i % 4 of the 8-byte chunks addressed by lanes i / 4, i / 4 + 4, i / 4 + 8
// and i / 4 + 12 of the group.  When lane n of group u addresses row
// 4u + n / 4, columns c0 + 4 (n % 4) .. +3 of a row-major tile, lane i gets
// rows 4u .. 4u + 3 of column c0 + i: the A operand of a 16x16x16 MFMA that
// contracts over the rows of the transposed tile.
template <typename T>
__device__ __forceinline__ typename Vec4<T>::type read_tr4(const T* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(typename Vec4<T>::type, r);
}
template <typename V4>
__device__ __forceinline__ auto cat8(V4 a, V4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// LDS pitches (elements).  K: [B_K][D + 8]; Q, dO tiles: [32][D + 8]; dS:
// [32][B_K + 8].
template <int D>
constexpr int b_kld() { return D + 8; }
template <int BK>
constexpr int s_ld() {
  return BK + 8;
}

// ---- D = rowsum(dO * O) -------------------------------------------------------
// D / 8 lanes per row, 16-byte loads, a butterfly over those lanes.
// Workgroup 0 also zeroes the queue counters of k_bwd_main, which runs next.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_bwd_delta(const T* __restrict__ out, const T* __restrict__ dout,
                                                   float* __restrict__ delta, int64_t rows,
                                                   int32_t* __restrict__ queue) {
  constexpr int LPR = D / 8;  // lanes per row (8, 16 or 32)
  if (blockIdx.x == 0) clear_queue(queue);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / LPR;
  const int c = (int)(idx % LPR);
  float acc = 0.f;
  if (row < rows) {
    const auto o = bld8(out + row * D + c * 8);
    const auto g = bld8(dout + row * D + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && c == 0) delta[row] = acc;
}

// ---- main ---------------------------------------------------------------------
// One row tile's gather data in registers: this thread's Q / dO vectors
// (zero for rows past the chunk) and, for threads < kBwdRows, its row's lse
// and D.
// Rows past the chunk load nothing (masked off, rather than a stand-in row
// that every workgroup's tail tile would read) and nothing consumes a loaded
// value before put(), so the loads stay in flight while the previous tile
// computes; the row mask and the base-2 scaling of lse are applied in put().
template <typename T, int D, int NT>
struct BwdTile {
  using V8 = typename Vec8<T>::type;
  static constexpr int PER = kBwdRows * D / 8;  // vectors of one tensor's tile
  static constexpr int NV = 2 * PER / NT;       // Q and dO tiles over the NT threads
  static_assert(2 * PER % NT == 0, "whole vectors per thread");
  V8 x[NV];
  bool ok[NV];  // the vector's row is a row of the chunk
  float lraw, draw;
  bool live;

  __device__ __forceinline__ void load(const T* __restrict__ q, const T* __restrict__ dout,
                                       const float* __restrict__ lse, const float* __restrict__ delta,
                                       const int* __restrict__ rtok, int tile, int h, int g, int HQ) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = threadIdx.x + i * NT;
      const int tensor = vi / PER, e = vi % PER;
      const int row = e / (D / 8), c = e % (D / 8);
      const int r = tile * kBwdRows + row;
      const int t = rtok[r];
      const size_t qrow = t >= 0 ? (size_t)t * HQ + h * g + r % g : 0;
      x[i] = t >= 0 ? bld8((tensor == 0 ? q : dout) + qrow * D + c * 8) : V8{};
      ok[i] = t >= 0;
    }
    // threads < kBwdRows keep the lse and D of tile row threadIdx.x; the
    // others load a row's values too (unused), so no branch surrounds the
    // loads; rows past the chunk load nothing
    const int r = tile * kBwdRows + (threadIdx.x & (kBwdRows - 1));
    const int t = rtok[r];
    live = t >= 0;
    const size_t qrow = live ? (size_t)t * HQ + h * g + r % g : 0;
    lraw = live ? lse[qrow] : 0.f;
    draw = live ? delta[qrow] : 0.f;
  }

  __device__ __forceinline__ void put(T* __restrict__ Qs, T* __restrict__ Ds, float* __restrict__ tab_l,
                                      float* __restrict__ tab_d) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = threadIdx.x + i * NT;
      const int tensor = vi / PER, e = vi % PER;
      const int row = e / (D / 8), c = e % (D / 8);
      *reinterpret_cast<V8*>((tensor == 0 ? Qs : Ds) + row * b_kld<D>() + c * 8) = ok[i] ? x[i] : V8{};
    }
    if (threadIdx.x < kBwdRows) {
      tab_l[threadIdx.x] = live ? lraw * kBwdLog2e : 0.f;
      tab_d[threadIdx.x] = live ? draw : 0.f;
    }
  }
};

// Waves per SIMD: two up to d = 128.  At d = 256 the item's K / V fragments
// and the dK / dV accumulators need more than 256 registers per lane, so one
// wave per SIMD takes the whole register file (accumulators in AGPRs); the
// LDS tiles (~110 KB) allow one workgroup per CU anyway.
template <int D>
constexpr int bwd_waves_per_eu() {
  return D == 256 ? 1 : 2;
}

template <typename T, int D, int BK, typename PT>
__global__ __launch_bounds__(bwd_threads<BK>()) __attribute__((amdgpu_waves_per_eu(bwd_waves_per_eu<D>()))) void k_bwd_main(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ qidx, const int4* __restrict__ work,
    const int32_t* __restrict__ nwork, int32_t* __restrict__ queue, PT* __restrict__ dq_part,
    float* __restrict__ kv_part, int H, int g, int NB, int CT, float scale, float scale_log2) {
  using V8 = typename Vec8<T>::type;
  using V4 = typename Vec4<T>::type;
  constexpr int NT = bwd_threads<BK>();
  constexpr int W = NT / 64;           // waves, 16 keys each
  constexpr int KS = D / 32;           // 32-wide contraction steps over d
  constexpr int MT = D / 16;           // 16-wide d tiles
  // dQ^T work of a tile: 2 row blocks x MT d tiles over the W waves.  With
  // W <= MT a wave takes MT / W d tiles of both row blocks; with W = 2 MT
  // (B_K = 128, d = 64) one d tile of one row block.
  constexpr int RBW = W > MT ? 1 : 2;  // row blocks per wave
  constexpr int MW = W > MT ? 1 : MT / W;  // d tiles per wave
  constexpr int KB = BK / 32;          // 32-key contraction steps of dQ^T
  constexpr int SLD = s_ld<BK>();
  constexpr int C8 = D / 8;
  constexpr int KV = BK * C8 / NT;     // K vectors staged per thread
  constexpr int RT = (kBwdRowTable + NT - 1) / NT;
  static_assert(W <= MT ? MT % W == 0 : W == 2 * MT, "dQ tiles split evenly over the waves");
  static_assert(BK * C8 % NT == 0, "whole K vectors per thread");
  __shared__ __attribute__((aligned(16))) T Ks[BK * b_kld<D>()];
  __shared__ __attribute__((aligned(16))) T Qs[kBwdRows * b_kld<D>()];
  __shared__ __attribute__((aligned(16))) T Ds[kBwdRows * b_kld<D>()];
  __shared__ __attribute__((aligned(16))) T Ss[kBwdRows * SLD];
  constexpr int QOLD = D + 16 / (int)sizeof(PT);  // dQ stage pitch (elements): rows 16 bytes apart in banks
  __shared__ __attribute__((aligned(16))) PT Qo[kBwdRows * QOLD];
  __shared__ __attribute__((aligned(16))) int rtok[kBwdRowTable];
  __shared__ __attribute__((aligned(16))) float tab_l[kBwdRows];
  __shared__ __attribute__((aligned(16))) float tab_d[kBwdRows];

  __shared__ int s_items[2];
  ItemChain ch(queue, nwork[0], s_items);
  const int HQ = H * g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kl = lane & 15, u = lane >> 4;
  const int key = wave * 16 + kl;  // this lane's key within the block (S, dP, dK, dV)
  // d tile of this wave's m-th dQ^T tile, and its row block when RBW = 1
  auto mt_of = [&](int m) { return W > MT ? wave % MT : wave + W * m; };
  const int rb_own = W > MT ? wave / MT : 0;
  // Writes the staged dQ rows of tile `tl` of the current item as whole rows
  // (consecutive threads, consecutive 16-byte pieces; non-temporal).
  auto flush_dq = [&](int tl, int pair0, int nrows) {
    constexpr int CPR = D * (int)sizeof(PT) / 16;  // 16-byte pieces per row
    constexpr int EPC = 16 / (int)sizeof(PT);      // elements per piece
#pragma unroll
    for (int j = 0; j < (kBwdRows * CPR + NT - 1) / NT; ++j) {
      const int pc = threadIdx.x + j * NT;
      if (kBwdRows * CPR % NT != 0 && pc >= kBwdRows * CPR) break;
      const int row = pc / CPR, col = pc % CPR;
      const int r = tl * kBwdRows + row;
      if (r < nrows)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(Qo + row * QOLD + col * EPC),
                                    reinterpret_cast<u32x4*>(dq_part + ((size_t)pair0 * g + r) * D + col * EPC));
    }
  };
  // transposed-read address of this lane in a 16-row block of a tile (see read_tr4)
  const int tr_off = (4 * u + (kl >> 2)) * b_kld<D>() + 4 * (kl & 3);
  while (ch.cur >= 0) {
    const int wi = ch.cur;
    const int4 wraw = work[wi];
    const Item it = read_item(work, counts, offsets, wi, NB, CT, BK);
    const int nrows = it.ntok * g, ntile = (nrows + kBwdRows - 1) / kBwdRows;
    // Item operands that stay in registers for all of its tiles: the B
    // fragments of this lane's key for S = Q K^T and dP = dO V^T (16-byte
    // loads straight from K / V; keys past a partial last block repeat the
    // last key and are masked), and below, the K^T fragments of dQ.
    const size_t krow = ((size_t)(it.bs + min(key, it.nkeys - 1)) * H + it.h) * D;
    V8 kb[KS], vb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kb[ks] = bld8(k + krow + 32 * ks + 8 * u);
      vb[ks] = bld8(v + krow + 32 * ks + 8 * u);
    }
    V8 kst[KV];
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int vi = threadIdx.x + i * NT;
      kst[i] = bld8(k + ((size_t)(it.bs + min(vi / C8, it.nkeys - 1)) * H + it.h) * D + (vi % C8) * 8);
    }
    int tk[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int r = threadIdx.x + i * NT;
      tk[i] = qidx[it.pair0 + min(r / g, it.ntok - 1)];
    }
    __syncthreads();  // every wave is done with the previous item's K and row table
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int vi = threadIdx.x + i * NT;
      *reinterpret_cast<V8*>(Ks + (vi / C8) * b_kld<D>() + (vi % C8) * 8) = kst[i];
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int r = threadIdx.x + i * NT;
      if (r < kBwdRowTable) rtok[r] = r < nrows ? tk[i] : -1;
    }
    ch.publish(s_items);
    __syncthreads();
    const int after = ch.after(s_items);
    // K^T fragments of dQ^T = K^T dS^T: lane (kl, u) of d tile mt holds
    // K[32 ks + 8u + e][16 mt + kl], e < 8.
    V8 kt[MW][KB];
#pragma unroll
    for (int m = 0; m < MW; ++m)
#pragma unroll
      for (int ks = 0; ks < KB; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) kt[m][ks][e] = Ks[(32 * ks + 8 * u + e) * b_kld<D>() + 16 * mt_of(m) + kl];

    BwdTile<T, D, NT> tl;
    tl.load(q, dout, lse, delta, rtok, 0, it.h, g, HQ);
    f32x4 dk[MT], dv[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) dk[mt] = dv[mt] = f32x4{};

    for (int tile = 0; tile < ntile; ++tile) {
      tl.put(Qs, Ds, tab_l, tab_d);
      __syncthreads();  // tile in LDS; every wave is past the previous tile's dQ
      if (tile + 1 < ntile) tl.load(q, dout, lse, delta, rtok, tile + 1, it.h, g, HQ);
      if (tile > 0) flush_dq(tile - 1, it.pair0, nrows);  // the stage is rewritten only after the next barrier

      // S = Q K^T and dP = dO V^T for rows 16 rb + 4u + r and this lane's key.
      f32x4 s[2] = {}, dp[2] = {};
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s[rb] = mfma_k32(bld8(Qs + (16 * rb + kl) * b_kld<D>() + 32 * ks + 8 * u), kb[ks], s[rb]);
          dp[rb] = mfma_k32(bld8(Ds + (16 * rb + kl) * b_kld<D>() + 32 * ks + 8 * u), vb[ks], dp[rb]);
        }
      V4 p4[2], ds4[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int4 tq = *reinterpret_cast<const int4*>(rtok + tile * kBwdRows + 16 * rb + 4 * u);
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(tab_l + 16 * rb + 4 * u);
        const f32x4 dd = *reinterpret_cast<const f32x4*>(tab_d + 16 * rb + 4 * u);
        const int tks[4] = {tq.x, tq.y, tq.z, tq.w};
        f32x4 p, ds;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // key visible iff it is in the row's causal past (rows past the chunk: token -1)
          const bool vis = tks[r] >= 0 && key <= tks[r] - it.bs;
          p[r] = vis ? __builtin_amdgcn_exp2f(fmaf(s[rb][r], scale_log2, -l2[r])) : 0.f;
          ds[r] = p[r] * (dp[rb][r] - dd[r]);
        }
        p4[rb] = __builtin_convertvector(p, V4);
        ds4[rb] = __builtin_convertvector(ds, V4);
      }
      // dV^T += dO^T P and dK^T += Q^T dS, contracting over the tile's 32
      // rows: element e of a lane's k range is row 4u + e of block 0 (e < 4)
      // or of block 1 (e >= 4), for the transposed reads and P / dS alike.
      const V8 pb = cat8(p4[0], p4[1]), dsb = cat8(ds4[0], ds4[1]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const V8 a_do = cat8(read_tr4(Ds + tr_off + 16 * mt), read_tr4(Ds + 16 * b_kld<D>() + tr_off + 16 * mt));
        const V8 a_q = cat8(read_tr4(Qs + tr_off + 16 * mt), read_tr4(Qs + 16 * b_kld<D>() + tr_off + 16 * mt));
        dv[mt] = mfma_k32(a_do, pb, dv[mt]);
        dk[mt] = mfma_k32(a_q, dsb, dk[mt]);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) Ss[(16 * rb + 4 * u + r) * SLD + key] = ds4[rb][r];
      __syncthreads();  // dS of all the block's keys in LDS

      // dQ^T = K^T dS^T for the d tiles of this wave, staged in LDS; lane:
      // row 16 rb + kl, d = 16mt + 4u + r.
#pragma unroll
      for (int rbi = 0; rbi < RBW; ++rbi)
#pragma unroll
        for (int m = 0; m < MW; ++m) {
          const int rb = RBW == 1 ? rb_own : rbi;
          f32x4 acc = {};
#pragma unroll
          for (int ks = 0; ks < KB; ++ks)
            acc = mfma_k32(kt[m][ks], bld8(Ss + (16 * rb + kl) * SLD + 32 * ks + 8 * u), acc);
          PT* const o = Qo + (16 * rb + kl) * QOLD + 16 * mt_of(m) + 4 * u;
          if constexpr (sizeof(PT) == 4) {
            *reinterpret_cast<f32x4*>(o) = acc * scale;
          } else {
            typedef PT P4 __attribute__((ext_vector_type(4)));
            *reinterpret_cast<P4*>(o) = __builtin_convertvector(acc * scale, P4);
          }
        }
    }
    __syncthreads();  // the last tile's dQ is staged
    flush_dq(ntile - 1, it.pair0, nrows);

    // The block's dK (scaled) / dV partial of this chunk: slot [2][B_K][D] fp32.
    const int64_t slot = (int64_t)(offsets[wraw.x] / CT) + wraw.x + wraw.y / CT;
    float* const kvp = kv_part + slot * 2 * BK * D + (size_t)key * D + 4 * u;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      *reinterpret_cast<f32x4*>(kvp + 16 * mt) = dk[mt] * scale;
      *reinterpret_cast<f32x4*>(kvp + BK * D + 16 * mt) = dv[mt];
    }
    ch.advance(after);
  }
}

// ---- dK, dV = ordered sum of the block's chunk slots --------------------------
// One thread per (segment f, key, 4 columns); keys past the sequence end are
// skipped, keys of blocks nobody selects get zero.
template <typename T, int D, int BK>
__global__ __launch_bounds__(256) void k_bwd_kv_reduce(const int32_t* __restrict__ counts,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ gboff,
                                                       const int32_t* __restrict__ cu, int num_seqs,
                                                       const float* __restrict__ kv_part, T* __restrict__ dk,
                                                       T* __restrict__ dv, int H, int NB, int CT) {
  typedef T T4 __attribute__((ext_vector_type(4)));
  constexpr int C4 = D / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)H * NB * BK * C4) return;
  const int c4 = (int)(idx % C4);
  const int key = (int)((idx / C4) % BK);
  const int f = (int)(idx / ((int64_t)C4 * BK));
  const int h = f / NB, gb = f - h * NB;
  const int s = seq_of_block(gboff, num_seqs, gb);
  const int token = cu[s] + (gb - gboff[s]) * BK + key;
  if (token >= cu[s + 1]) return;
  const int nch = (counts[f] + CT - 1) / CT;
  const int64_t slot0 = (int64_t)(offsets[f] / CT) + f;
  // Eight chunks' loads are issued together (indices clamped to the last
  // chunk), then added in chunk order; the order of the sum is unchanged.
  constexpr int U = 8;
  f32x4 sk = {}, sv = {};
  for (int c = 0; c < nch; c += U) {
    f32x4 xk[U], xv[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const float* p = kv_part + (slot0 + min(c + j, nch - 1)) * 2 * BK * D + (size_t)key * D + 4 * c4;
      xk[j] = *reinterpret_cast<const f32x4*>(p);
      xv[j] = *reinterpret_cast<const f32x4*>(p + BK * D);
    }
#pragma unroll
    for (int j = 0; j < U; ++j)
      if (c + j < nch) {
        sk += xk[j];
        sv += xv[j];
      }
  }
  const size_t o = ((size_t)token * H + h) * D + 4 * c4;
  *reinterpret_cast<T4*>(dk + o) = __builtin_convertvector(sk, T4);
  *reinterpret_cast<T4*>(dv + o) = __builtin_convertvector(sv, T4);
}

template <typename T, int D, int BK, typename PT>
hipError_t bwd_typed(const Geometry& geo, const int32_t* cu_dev, const void* q, const void* k, const void* v,
                     const void* out, const void* dout, const float* lse, const fsa_index& idx, void* dq, void* dk,
                     void* dv, void* ws, hipStream_t stream) {
  char* wsb = static_cast<char*>(ws);
  float* delta = reinterpret_cast<float*>(wsb);
  PT* dq_part = reinterpret_cast<PT*>(wsb + geo.bwd_dq_off);
  float* kv_part = reinterpret_cast<float*>(wsb + geo.bwd_kv_off);
  const char* aux = static_cast<const char*>(idx.aux);
  const int4* work = reinterpret_cast<const int4*>(aux + geo.aux_work_sorted);
  const int32_t* nwork = reinterpret_cast<const int32_t*>(aux + geo.aux_nwork);
  const int32_t* gboff = reinterpret_cast<const int32_t*>(aux + geo.aux_seq_gboff);
  int32_t* queue = reinterpret_cast<int32_t*>(wsb + geo.bwd_queue_off);

  const int64_t rows = (int64_t)geo.N * geo.HQ;
  const int64_t dthreads = rows * (D / 8);
  hipLaunchKernelGGL((k_bwd_delta<T, D>), dim3((unsigned)((dthreads + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const T*>(out), static_cast<const T*>(dout), delta, rows, queue);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int NT = bwd_threads<BK>();
  hipLaunchKernelGGL((k_bwd_main<T, D, BK, PT>), dim3(persistent_grid(k_bwd_main<T, D, BK, PT>, NT, geo.max_work)),
                     dim3(NT), 0,
                     stream, static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     static_cast<const T*>(dout), lse, delta, idx.counts, idx.offsets, idx.qidx, work, nwork, queue, dq_part,
                     kv_part, geo.H, geo.g, geo.NB, geo.chunk_tokens, geo.scale, geo.scale * kBwdLog2e);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_reduce(geo, idx, dq_part, dq, false, nullptr, nullptr, nullptr, stream);
  if (e != hipSuccess) return e;
  const int64_t kthreads = (int64_t)geo.H * geo.NB * BK * (D / 4);
  if (kthreads > 0)
    hipLaunchKernelGGL((k_bwd_kv_reduce<T, D, BK>), dim3((unsigned)((kthreads + 255) / 256)), dim3(256), 0, stream,
                       idx.counts, idx.offsets, gboff, cu_dev, geo.num_seqs, kv_part, static_cast<T*>(dk),
                       static_cast<T*>(dv), geo.H, geo.NB, geo.chunk_tokens);
  return hipGetLastError();
}

template <typename T, typename PT>
hipError_t bwd_d(const Geometry& geo, const int32_t* cu_dev, const void* q, const void* k, const void* v,
                 const void* out, const void* dout, const float* lse, const fsa_index& idx, void* dq, void* dk,
                 void* dv, void* ws, hipStream_t s) {
  if (geo.BK == 128) {  // d <= 128 (checked by the caller)
    if (geo.d == 64) return bwd_typed<T, 64, 128, PT>(geo, cu_dev, q, k, v, out, dout, lse, idx, dq, dk, dv, ws, s);
    return bwd_typed<T, 128, 128, PT>(geo, cu_dev, q, k, v, out, dout, lse, idx, dq, dk, dv, ws, s);
  }
  if (geo.d == 64) return bwd_typed<T, 64, 64, PT>(geo, cu_dev, q, k, v, out, dout, lse, idx, dq, dk, dv, ws, s);
  if (geo.d == 256) return bwd_typed<T, 256, 64, PT>(geo, cu_dev, q, k, v, out, dout, lse, idx, dq, dk, dv, ws, s);
  return bwd_typed<T, 128, 64, PT>(geo, cu_dev, q, k, v, out, dout, lse, idx, dq, dk, dv, ws, s);
}

}  // namespace

hipError_t launch_bwd(const Geometry& geo, const int32_t* cu_dev, const void* q, const void* k, const void* v,
                      const void* out, const void* dout, const float* lse, const fsa_index& idx, void* dq, void* dk,
                      void* dv, void* ws, hipStream_t stream) {
  if (geo.N == 0) return hipSuccess;
  const bool f32 = geo.partial_dtype == FSA_PARTIAL_FP32;
  if (geo.dtype == FSA_DTYPE_BF16)
    return f32 ? bwd_d<__bf16, float>(geo, cu_dev, q, k, v, out, dout, lse, idx, dq, dk, dv, ws, stream)
               : bwd_d<__bf16, __bf16>(geo, cu_dev, q, k, v, out, dout, lse, idx, dq, dk, dv, ws, stream);
  return f32 ? bwd_d<_Float16, float>(geo, cu_dev, q, k, v, out, dout, lse, idx, dq, dk, dv, ws, stream)
             : bwd_d<_Float16, _Float16>(geo, cu_dev, q, k, v, out, dout, lse, idx, dq, dk, dv, ws, stream);
}

}  // namespace fsa
