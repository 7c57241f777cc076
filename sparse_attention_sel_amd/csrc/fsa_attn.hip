// Attention kernels on gfx950 for the FSA selected-attention forward:
//
//   k_stats    online-softmax statistics, KV-block-outer (paper notes, Key
//              design 4): per (KV head, block, query chunk) the block's K is
//              staged in LDS once and each query row gets the block's max and
//              exp-sum; k_stats_combine merges a query's blocks into the row
//              max and log-sum-exp.
//   k_main     token-selection kernel (paper notes, Key designs 1-3; README,
//              Method): per (KV head, block, query chunk) K and V are staged
//              in LDS once, the block's query list streams through MFMA tiles
//              (S^T = K Q^T, then O^T = V^T P^T), and the pre-scaled partial
//              rows exp(s - lse) @ V are written contiguously into the
//              compact buffer at the segment's offset.
//   k_reduce   reduction kernel (Key design 3): each (token, KV head) sums its
//              partial rows in slot order; no atomics.
//   k_stats_local, k_main_local
//              the same for the entries of a query's own, previous and first
//              blocks, computed per query block (one partial row per query).
//
// One-pass variant (FUSED, fsa_selected_attn_fwd_onepass): k_main and
// k_main_local take each row's max and sum over the block's visible keys
// from the score tile they already hold (probs_stats: the statistics kernel's
// terms in its order), write the block's softmax average of V and the
// (max, sum) pair, and k_reduce merges the pairs in slot order into row max
// and lse while it sums the weighted partial rows; no statistics pass runs.
//
// Work items come from the index builder: (segment f, first query of the
// chunk, block start token, sequence end).  Rows of a chunk are
// (query, group head) pairs, query-major: row = i * g + j.  A row table in
// LDS gives each row its Q / lse row index and its token.
//
// Q tiles.  A 32-row tile is gathered with coalesced 16-byte loads (lanes in
// row order, so one load instruction reads whole rows: for g = 4 and d = 128,
// one token's four head rows, 1 KB), staged in a per-wave LDS tile, and read
// back in the MFMA operand layout.  The same LDS tile later stages the output
// tile for row-contiguous stores.
//
// MFMA tiling (v_mfma_f32_32x32x16, wave64).  A 32-row query tile meets the
// block's keys as S^T (keys x rows) so that each lane ends up owning one query
// row: lane l holds column l % 32 of S^T.  The same registers, cast to 16-bit,
// are the B operand of O^T = V^T P^T, so P never leaves the registers.  V is
// staged transposed (Vt[d][key]) with the keys of every 16-key group permuted
// so that the 8 keys a lane contributes to one MFMA are adjacent in LDS.
#include <algorithm>
#include <cstdlib>

#include "fsa_internal.h"

namespace fsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWaves = kAttnThreads / 64;
constexpr int kRowTable = kRowsPerItem + 32;  // rows of the last tile past the chunk included

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type load8(const T* p) {
  return *reinterpret_cast<const typename Vec8<T>::type*>(p);
}

template <typename T>
__device__ __forceinline__ uint16_t bits16(T x) {
  return __builtin_bit_cast(uint16_t, x);
}

// LDS layouts (elements).  K: [BK][D + 8]; Vt: [D][BK + 8]; per-wave tile:
// [32][D + 8].  The 8-element pads spread the 16-byte reads of consecutive
// rows over all banks.
template <int D>
constexpr int k_ld() { return D + 8; }
template <int BK>
constexpr int vt_ld() { return BK + 8; }
template <int D>
constexpr int tile_ld() { return D + 8; }

// Position of key w (within its 16-key group) in the permuted Vt row: lane half
// hl contributes keys {4hl..4hl+3, 8+4hl..8+4hl+3} as MFMA elements e = 0..7.
__device__ __forceinline__ int vt_pos(int key) {
  const int w = key & 15;
  return (key & ~15) + ((w >> 2) & 1) * 8 + (w >> 3) * 4 + (w & 3);
}

// The same for the 16-row tiles of v_mfma_f32_16x16x32: within each 32-key
// group, lane group u (lanes 16u..16u+15) contributes keys {4u..4u+3,
// 16+4u..16+4u+3} as MFMA elements e = 0..7, the keys its S^T tiles hold.
__device__ __forceinline__ int vt_pos16(int key) {
  const int w = key & 31;
  return (key & ~31) + ((w >> 2) & 3) * 8 + (w >> 4) * 4 + (w & 3);
}

// Coalesced gather of the Q rows of one 32-row tile: vector v of lane l holds
// tile elements (v*64 + l)*8 .. +8, i.e. row (v*64 + l)*8 / D, column
// (v*64 + l)*8 % D.
template <typename T, int D>
__device__ __forceinline__ void load_q_tile(const T* __restrict__ q, const int* __restrict__ ridx, int tile,
                                            int lane, typename Vec8<T>::type* qv) {
#pragma unroll
  for (int v = 0; v < D / 16; ++v) {
    const int e = (v * 64 + lane) * 8;
    const int r = e / D, c = e % D;
    qv[v] = load8(q + (size_t)ridx[tile * 32 + r] * D + c);
  }
}

template <typename T, int D>
__device__ __forceinline__ void put_q_tile(T* __restrict__ qt, int lane, const typename Vec8<T>::type* qv) {
#pragma unroll
  for (int v = 0; v < D / 16; ++v) {
    const int e = (v * 64 + lane) * 8;
    *reinterpret_cast<typename Vec8<T>::type*>(qt + (e / D) * tile_ld<D>() + e % D) = qv[v];
  }
}

// S^T tile from the staged Q tile: s[kt][r] = (K Q^T)[key = kt*32 + 8*(r/4) +
// 4*hl + r%4][row = l%32].  Lane half hl supplies the contraction elements
// ks*16 + hl*8 .. +8 of both operands.
template <typename T, int D, int BK>
__device__ __forceinline__ void qk_tile(const T* __restrict__ Ks, const T* __restrict__ qt, int lr, int hl,
                                        f32x16* s) {
  constexpr int KS = D / 16, KT = BK / 32;
  typename Vec8<T>::type b[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) b[ks] = load8(qt + lr * tile_ld<D>() + ks * 16 + hl * 8);
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    f32x16 acc = {};
    const T* kp = Ks + (kt * 32 + lr) * k_ld<D>() + hl * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = mfma32(load8(kp + ks * 16), b[ks], acc);
    s[kt] = acc;
  }
}

// Gather of one 32-row Q tile straight into the B-operand layout of
// S^T = K Q^T: lane (lr, hl) holds row lr, elements ks*16 + hl*8 .. +8 for
// every ks (each load covers 32 bytes of each of the tile's 32 rows).
template <typename T, int D>
__device__ __forceinline__ void load_q_frag(const T* __restrict__ q, const int* __restrict__ ridx, int tile, int lr,
                                            int hl, typename Vec8<T>::type* b) {
  const T* row = q + (size_t)ridx[tile * 32 + lr] * D + hl * 8;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) b[ks] = load8(row + ks * 16);
}

// S^T tile from a gathered B operand (as qk_tile, without the LDS tile).
template <typename T, int D, int BK>
__device__ __forceinline__ void qk_frag(const T* __restrict__ Ks, const typename Vec8<T>::type* b, int lr, int hl,
                                        f32x16* s) {
  constexpr int KS = D / 16, KT = BK / 32;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) s[kt] = f32x16{};
  const T* kp = Ks + lr * k_ld<D>() + hl * 8;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) s[kt] = mfma32(load8(kp + kt * 32 * k_ld<D>() + ks * 16), b[ks], s[kt]);
}

// O^T += V^T P^T over one key block: o[mt] holds O^T rows (d) mt*32.. of the
// lane's query row; pb are the 16-bit probabilities of probs().
template <typename T, int D, int BK>
__device__ __forceinline__ void pv_tile(const T* __restrict__ Vt, const typename Vec8<T>::type* pb, int lr, int hl,
                                        f32x16* o) {
  constexpr int KK = BK / 16, MT = D / 32;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] = mfma32(load8(Vt + (mt * 32 + lr) * vt_ld<BK>() + kk * 16 + hl * 8), pb[kk], o[mt]);
}

// x combined with the same register of lane l ^ 32 by a commutative op:
// v_permlane32_swap of x with itself hands each lane the values of lanes
// l % 32 (first result) and l % 32 + 32 (second result).  The compiler treats
// the two results of a swap of one value with itself as equal and would fold
// the combination away, so they pass through an empty asm statement first.
__device__ __forceinline__ float2 xhalf_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  uint32_t lo = r[0], hi = r[1];
  asm volatile("" : "+v"(lo), "+v"(hi));
  return make_float2(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
}
__device__ __forceinline__ float xhalf_max(float x) {
  const float2 p = xhalf_pair(x);
  return fmaxf(p.x, p.y);
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const float2 p = xhalf_pair(x);
  return p.x + p.y;
}

// The staging data of one work item held in registers while the previous item
// computes: this thread's share of the K block (and of V, for the main
// kernel) and the query tokens of its rows of the row table.  Loads use
// clamped indices so that they are unconditional: keys past a partial last
// block are only ever seen by rows that take the causal mask (their values
// get weight zero), rows past the chunk are marked with token -1.
template <typename T, int D, int BK, bool WITH_V, int NT, bool SPLIT = false, bool VT16 = false>
struct ItemStage {
  using V8 = typename Vec8<T>::type;
  static constexpr int KV = BK * D / 8 / NT;                        // K vectors per thread
  static constexpr int VP = WITH_V ? (BK / 2) * (D / 8) / NT : 1;   // V key pairs per thread
  static constexpr int RT = (kRowTable + NT - 1) / NT;              // table rows per thread
  static_assert(BK * D / 8 % NT == 0 && (BK / 2) * (D / 8) % NT == 0, "whole vectors");
  Item it;
  V8 k[KV];
  V8 va[VP], vb[VP];
  int tok[RT];

  __device__ __forceinline__ void load(const T* __restrict__ kg, const T* __restrict__ vg, const int32_t* __restrict__ qidx,
                                       const int4* __restrict__ work, const int32_t* __restrict__ counts,
                                       const int32_t* __restrict__ offsets, int wi, int H, int g, int NB, int CT) {
    it = SPLIT ? read_item_half(work, counts, offsets, wi, NB, CT) : read_item(work, counts, offsets, wi, NB, CT, BK);
    constexpr int C8 = D / 8;
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int vi = threadIdx.x + i * NT;
      const int key = min(vi / C8, it.nk - 1), c = vi % C8;
      k[i] = load8(kg + ((size_t)(it.kb + key) * H + it.h) * D + c * 8);
    }
    if constexpr (WITH_V) {
      constexpr int KP = BK / 2;
#pragma unroll
      for (int i = 0; i < VP; ++i) {
        const int vi = threadIdx.x + i * NT;
        const int c = vi / KP, key = 2 * (vi % KP);
        va[i] = load8(vg + ((size_t)(it.kb + min(key, it.nk - 1)) * H + it.h) * D + c * 8);
        vb[i] = load8(vg + ((size_t)(it.kb + min(key + 1, it.nk - 1)) * H + it.h) * D + c * 8);
      }
    }
    // Nothing here consumes the loaded values (the row bound is applied at
    // commit), so the loads stay in flight while the current item computes.
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int r = threadIdx.x + i * NT;
      tok[i] = qidx[it.pair0 + min(r / g, it.ntok - 1)];
    }
  }

  __device__ __forceinline__ void commit(T* __restrict__ Ks, T* __restrict__ Vt, int* __restrict__ ridx,
                                         int* __restrict__ rtok, int g, int HQ) const {
    constexpr int C8 = D / 8;
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int vi = threadIdx.x + i * NT;
      *reinterpret_cast<V8*>(Ks + (vi / C8) * k_ld<D>() + (vi % C8) * 8) = k[i];
    }
    if constexpr (WITH_V) {
      constexpr int KP = BK / 2;
#pragma unroll
      for (int i = 0; i < VP; ++i) {
        const int vi = threadIdx.x + i * NT;
        const int c = vi / KP, key = 2 * (vi % KP);
        const int pos = VT16 ? vt_pos16(key) : vt_pos(key);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t packed = (uint32_t)bits16(va[i][e]) | ((uint32_t)bits16(vb[i][e]) << 16);
          *reinterpret_cast<uint32_t*>(Vt + (c * 8 + e) * vt_ld<BK>() + pos) = packed;
        }
      }
    }
    const int nrows = it.ntok * g;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int r = threadIdx.x + i * NT;
      if (r < kRowTable) {
        const bool ok = r < nrows;
        ridx[r] = (ok ? tok[i] : 0) * HQ + it.h * g + (ok ? r % g : 0);
        rtok[r] = ok ? tok[i] : -1;
      }
    }
  }
};

// Waves per SIMD the register budget aims for: two (<= 256 registers) where
// the tile state fits, one (<= 512) for the wide head dim / long blocks.
template <int D, int BK>
constexpr int attn_waves_per_eu() { return (D >= 256 || (D >= 128 && BK >= 128)) ? 1 : 2; }

// The statistics kernel's shapes.  Small tiles (d * B_K below 128 * 128)
// gather each Q tile with coalesced loads and pass it through an LDS tile to
// the MFMA B operand, two waves per SIMD.  Wider tiles gather the B operand
// straight into registers (32 bytes of each row per load): with no Q tiles in
// LDS, two workgroups fit a CU, two waves per SIMD where one fit before, and
// the next item's K is loaded at the item boundary instead of into registers
// during the current item (the other workgroup covers that latency).  At
// d = 256, B_K = 128 the scores take the registers, one wave per SIMD, and
// the prefetch stays.  Measured on the statistics stage: d = 256 B_K = 64
// 4.98 -> 4.51 ms, d = 256 B_K = 128 0.52 -> 0.42 ms, d = 128 B_K = 128
// 0.47 -> 0.43 ms; the register gather at d = 128 B_K = 64 (occupancy
// unchanged, four times the load instructions) ran 14% slower.
template <int D, int BK>
constexpr int stats_threads() { return kAttnThreads; }
template <int D, int BK>
constexpr bool stats_gather_b() { return D * BK >= 128 * 128; }
template <int D, int BK>
constexpr int stats_waves_per_eu() { return D == 256 && BK == 128 ? 1 : 2; }
template <int D, int BK>
constexpr bool stats_prefetch() { return !stats_gather_b<D, BK>() || (D == 256 && BK == 128); }
// Shapes whose three-pass main kernel is k_main16: those where k_main's
// 32-row tiles need more than 256 registers (one wave per SIMD).
template <int D, int BK, bool FUSED>
constexpr bool main16() { return !FUSED && ((D == 256 && BK == 64) || (D == 128 && BK == 128)); }
template <int D, int BK>
constexpr int stats_local_waves_per_eu() { return stats_gather_b<D, BK>() ? 2 : attn_waves_per_eu<D, BK>(); }
// k_stats_local stages its up to three key blocks at once (d <= 128, 64-key
// blocks: 52 KB of LDS at d = 128).
template <int D, int BK>
constexpr bool stats_local_all() { return D <= 128 && BK == 64; }

// Every key of the block is visible to every row of the tile: the block lies
// entirely before each row's token (rows of a chunk are in token order, so
// only the first tiles of a query's own block need the causal mask).
template <int BK>
__device__ __forceinline__ bool tile_unmasked(int tok, int bs) {
  return __all(tok < 0 || tok - bs >= BK - 1);
}

// scale * max over visible keys and the exp-sum relative to it, in base 2,
// for the lane's row (lanes l and l + 32 hold the two key halves).
template <int BK, bool MASKED>
__device__ __forceinline__ float2 row_stats(const f32x16* s, int hl, int lim, float c) {
  constexpr int KT = BK / 32;
  float m = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kt * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
      if (!MASKED || key <= lim) m = fmaxf(m, s[kt][r]);
    }
  m = xhalf_max(m) * c;
  float l = 0.f;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kt * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
      const float e = __builtin_amdgcn_exp2f(fmaf(s[kt][r], c, -m));
      l += (!MASKED || key <= lim) ? e : 0.f;
    }
  l = xhalf_sum(l);
  return make_float2(m, l);
}

// ---- statistics -------------------------------------------------------------
template <typename T, int D, int BK>
__global__ __launch_bounds__((stats_threads<D, BK>())) __attribute__((amdgpu_waves_per_eu(stats_waves_per_eu<D, BK>()))) void k_stats(
    const T* __restrict__ q, const T* __restrict__ k, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ qidx, const int4* __restrict__ work,
    const int32_t* __restrict__ nwork, int32_t* __restrict__ queue, float2* __restrict__ st, size_t dump_row, int H,
    int g, int NB, int CT, float scale_log2) {
  using V8 = typename Vec8<T>::type;
  constexpr int KS = D / 16, KT = BK / 32;
  constexpr int NT = stats_threads<D, BK>(), NW = NT / 64;
  constexpr bool FRAG = stats_gather_b<D, BK>(), PRE = stats_prefetch<D, BK>();
  __shared__ __attribute__((aligned(16))) T Ks[BK * k_ld<D>()];
  __shared__ __attribute__((aligned(16))) T Qt[FRAG ? 8 : NW * 32 * tile_ld<D>()];
  __shared__ int ridx[kRowTable], rtok[kRowTable];
  __shared__ int s_items[2];
  ItemChain ch(queue, nwork[2], s_items);  // the forward list
  const int4* const wl = work + nwork[0];
  if (ch.cur < 0) return;
  const int HQ = H * g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, hl = lane >> 5;
  T* const qt = Qt + (FRAG ? 0 : wave * 32 * tile_ld<D>());
  ItemStage<T, D, BK, false, NT> pre;
  if constexpr (PRE) pre.load(k, nullptr, qidx, wl, counts, offsets, ch.cur, H, g, NB, CT);
  while (ch.cur >= 0) {
    __syncthreads();  // the previous item's LDS reads are done
    if constexpr (!PRE) pre.load(k, nullptr, qidx, wl, counts, offsets, ch.cur, H, g, NB, CT);
    pre.commit(Ks, nullptr, ridx, rtok, g, HQ);
    ch.publish(s_items);
    const Item it = pre.it;
    __syncthreads();
    const int after = ch.after(s_items);
    const int nrows = it.ntok * g, ntile = (nrows + 31) / 32;

    auto stats_of = [&](int tl, const f32x16* s) {
      const int row = tl * 32 + lr;
      const int tok = rtok[row];
      float2 ml;
      if (tile_unmasked<BK>(tok, it.bs)) ml = row_stats<BK, false>(s, hl, 0, scale_log2);
      else ml = row_stats<BK, true>(s, hl, tok < 0 ? -1 : tok - it.bs, scale_log2);
      // lanes l and l + 32 store the same pair; rows past the chunk go to the dump
      st[tok >= 0 ? (size_t)it.pair0 * g + row : dump_row + lr] = ml;
    };
    if constexpr (FRAG) {
      // Q pipeline: two register sets, each a tile's B operand gathered
      // straight from memory; tile i + 1 is in flight while tile i computes.
      auto tile = [&](int tl, const V8* b) {
        f32x16 s[KT];
        qk_frag<T, D, BK>(Ks, b, lr, hl, s);
        stats_of(tl, s);
      };
      V8 qa[KS], qb[KS];
      if (wave < ntile) load_q_frag<T, D>(q, ridx, wave, lr, hl, qa);
      if constexpr (PRE)
        if (ch.nxt >= 0) pre.load(k, nullptr, qidx, wl, counts, offsets, ch.nxt, H, g, NB, CT);
      for (int tl = wave; tl < ntile; tl += 2 * NW) {
        if (tl + NW < ntile) load_q_frag<T, D>(q, ridx, tl + NW, lr, hl, qb);
        tile(tl, qa);
        if (tl + NW >= ntile) break;
        if (tl + 2 * NW < ntile) load_q_frag<T, D>(q, ridx, tl + 2 * NW, lr, hl, qa);
        tile(tl + NW, qb);
      }
    } else {
      // Q pipeline: one register set of coalesced loads plus the wave's LDS
      // tile.  At each tile the registers (tile i, loaded during tile i - 1)
      // go to LDS and are refilled with tile i + 1 while tile i computes from
      // LDS.  The next item's staging loads are issued after the first Q
      // tile's.  (A second register set, two gathers in flight per wave, ran
      // no faster at d = 128.)
      V8 qv[KS];
      if (wave < ntile) load_q_tile<T, D>(q, ridx, wave, lane, qv);
      if (ch.nxt >= 0) pre.load(k, nullptr, qidx, wl, counts, offsets, ch.nxt, H, g, NB, CT);
      for (int tl = wave; tl < ntile; tl += NW) {
        put_q_tile<T, D>(qt, lane, qv);
        if (tl + NW < ntile) load_q_tile<T, D>(q, ridx, tl + NW, lane, qv);
        f32x16 s[KT];
        qk_tile<T, D, BK>(Ks, qt, lr, hl, s);
        stats_of(tl, s);
      }
    }
    ch.advance(after);
  }
}

// One thread per (token, query head): merge the token's local (max, sum) pair
// (at the row of its designated local entry) and the per-block pairs of its
// other selecting entries, in slot order, into the row max and lse (stored in
// natural-log units).  Slots are read 8 at a time and their pairs loaded
// together, the loads of empty and local slots masked off (a stand-in load of
// one fixed row from every thread would make that row a hot spot).
__global__ __launch_bounds__(256) void k_stats_combine(const int32_t* __restrict__ slot,
                                                       const float2* __restrict__ st,
                                                       const int32_t* __restrict__ loc,
                                                       float* __restrict__ row_max, float* __restrict__ lse, int N,
                                                       int H, int g, int T) {
  const int HQ = H * g;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)N * HQ) return;
  const int t = (int)(idx / HQ), hq = (int)(idx - (int64_t)t * HQ);
  const int h = hq / g, j = hq - h * g;
  const int32_t* sl = slot + ((size_t)h * N + t) * T;
  const unsigned word = (unsigned)loc[(size_t)h * N + t];
  float M = -INFINITY, L = 0.f;
  if (word != 0u) {
    const float2 v = st[(size_t)sl[local_designated(word)] * g + j];
    M = v.x;
    L = v.y;
  }
  for (int j0 = 0; j0 < T; j0 += 8) {
    int sv[8];
    float2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) sv[u] = j0 + u < T && !local_entry(word, j0 + u) ? sl[j0 + u] : -1;
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = sv[u] >= 0 ? st[(size_t)sv[u] * g + j] : float2{};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (sv[u] >= 0) {
        const float mn = fmaxf(M, v[u].x);
        L = L * __builtin_amdgcn_exp2f(M - mn) + v[u].y * __builtin_amdgcn_exp2f(v[u].x - mn);
        M = mn;
      }
    }
  }
  if (L > 0.f) {
    row_max[idx] = M * kLn2;
    lse[idx] = (M + log2f(L)) * kLn2;
  } else {
    row_max[idx] = -INFINITY;
    lse[idx] = -INFINITY;
  }
}

// ---- main -------------------------------------------------------------------
// Output tile epilogue.  The O^T accumulators give each lane 4 consecutive
// head-dim values of one row, 8 values apart.  Each wave passes its 32 x D
// output tile through its LDS tile (row pitch (D + 8) * 2 bytes: all D
// columns of 16-bit partials at once, or D/2 columns of fp32 partials twice)
// and writes it back row-contiguously with 16 bytes per lane, so that every
// store instruction covers whole rows.  Partial rows are written once and
// read once by the reduction, so the stores are non-temporal.  Rows past the
// chunk are written to the dump rows after the last partial row, so every
// lane stores unconditionally.
template <typename PT, int D>
struct Stage {
  static constexpr int CW = sizeof(PT) == 4 ? D / 2 : D;  // columns per pass
  static constexpr int P = CW + 16 / (int)sizeof(PT);      // row pitch (elements)
};

template <typename PT>
__device__ __forceinline__ void stage_write4(PT* p, f32x4 x);
template <>
__device__ __forceinline__ void stage_write4<float>(float* p, f32x4 x) {
  *reinterpret_cast<f32x4*>(p) = x;
}
template <>
__device__ __forceinline__ void stage_write4<__bf16>(__bf16* p, f32x4 x) {
  typedef __bf16 v4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, __builtin_convertvector(x, v4));
}
template <>
__device__ __forceinline__ void stage_write4<_Float16>(_Float16* p, f32x4 x) {
  typedef _Float16 v4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, __builtin_convertvector(x, v4));
}

// o[mt][r] holds O^T[d = mt*32 + 8*(r/4) + 4*hl + r%4][row = lane % 32].
// Writes rows [0, rows) of the tile to dst (row-major, pitch D), the others
// to the matching rows of dump.
template <typename PT, int D>
__device__ __forceinline__ void store_tile(PT* __restrict__ stage, const f32x16* o, int lane, int rows,
                                           PT* __restrict__ dst, PT* __restrict__ dump) {
  constexpr int CW = Stage<PT, D>::CW, P = Stage<PT, D>::P;
  constexpr int EPL = 16 / (int)sizeof(PT);  // elements per 16-byte lane store
  constexpr int LPR = CW / EPL;              // lanes per staged row
  constexpr int RPI = 64 / LPR;              // rows per store instruction
  const int lr = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int c = 0; c < D / CW; ++c) {
#pragma unroll
    for (int m = 0; m < CW / 32; ++m)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16& acc = o[(CW / 32) * c + m];
        stage_write4<PT>(stage + lr * P + m * 32 + 8 * q4 + 4 * hl,
                         f32x4{acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]});
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = i * RPI + lane / LPR, col = (lane % LPR) * EPL;
      const u32x4 val = *reinterpret_cast<const u32x4*>(stage + row * P + col);
      PT* base = row < rows ? dst : dump;
      __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(base + (size_t)row * D + c * CW + col));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// store_tile with a destination row per tile row: lane l < 32 holds in `drow`
// the partial row (of `partial`, pitch D) of tile row l, or -1 to send it to
// the matching dump row.  Each row is still written as whole 16-byte pieces.
template <typename PT, int D>
__device__ __forceinline__ void store_tile_rows(PT* __restrict__ stage, const f32x16* o, int lane, int64_t drow,
                                                PT* __restrict__ partial, PT* __restrict__ dump) {
  constexpr int CW = Stage<PT, D>::CW, P = Stage<PT, D>::P;
  constexpr int EPL = 16 / (int)sizeof(PT);
  constexpr int LPR = CW / EPL;
  constexpr int RPI = 64 / LPR;
  const int lr = lane & 31, hl = lane >> 5;
  const int dlo = (int)(uint32_t)(uint64_t)drow, dhi = (int)(uint32_t)((uint64_t)drow >> 32);
#pragma unroll
  for (int c = 0; c < D / CW; ++c) {
#pragma unroll
    for (int m = 0; m < CW / 32; ++m)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16& acc = o[(CW / 32) * c + m];
        stage_write4<PT>(stage + lr * P + m * 32 + 8 * q4 + 4 * hl,
                         f32x4{acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]});
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = i * RPI + lane / LPR, col = (lane % LPR) * EPL;
      const int64_t r = (int64_t)(((uint64_t)(uint32_t)__shfl(dhi, row, 64) << 32) | (uint32_t)__shfl(dlo, row, 64));
      const u32x4 val = *reinterpret_cast<const u32x4*>(stage + row * P + col);
      PT* dst = r >= 0 ? partial + (size_t)r * D : dump + (size_t)row * D;
      __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(dst + c * CW + col));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// P = exp2(s * c - lse2) as the 16-bit B operand of O^T = V^T P^T: element e
// of pb[2*kt + u] is register r = 8*u + e of key tile kt.
template <typename T, int BK, bool MASKED>
__device__ __forceinline__ void probs(const f32x16* s, float c, float l2, int hl, int lim,
                                      typename Vec8<T>::type* pb) {
#pragma unroll
  for (int kt = 0; kt < BK / 32; ++kt)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * u + e;
        const int key = kt * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][r], c, -l2));
        x[e] = (!MASKED || key <= lim) ? p : 0.f;
      }
      pb[2 * kt + u] = __builtin_convertvector(x, typename Vec8<T>::type);
    }
}

// probs() with the row's own statistics (the one-pass forward): the max m of
// the visible scaled scores and l = sum exp(s - m), computed exactly as
// row_stats() computes them (same terms, same order), so the pair matches the
// statistics kernel's bit for bit.  The probabilities handed to the PV MFMA
// are exp(s - max(m, mprev)), the running max mprev of earlier blocks
// (-inf: none), as exp(s - m) * exp(m - max(m, mprev)).
template <typename T, int BK, bool MASKED>
__device__ __forceinline__ float2 probs_stats(const f32x16* s, float c, int hl, int lim, float mprev,
                                              typename Vec8<T>::type* pb) {
  float m = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < BK / 32; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kt * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
      if (!MASKED || key <= lim) m = fmaxf(m, s[kt][r]);
    }
  m = xhalf_max(m) * c;
  const float mx = fmaxf(m, mprev);
  const float scale = m == mx ? 1.f : __builtin_amdgcn_exp2f(m - mx);
  float l = 0.f;
#pragma unroll
  for (int kt = 0; kt < BK / 32; ++kt)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * u + e;
        const int key = kt * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][r], c, -m));
        const float pv = (!MASKED || key <= lim) ? p : 0.f;
        l += pv;
        x[e] = pv * scale;
      }
      pb[2 * kt + u] = __builtin_convertvector(x, typename Vec8<T>::type);
    }
  return make_float2(m, xhalf_sum(l));
}

// FUSED (the one-pass forward): instead of reading lse, each row takes the
// (max, sum) of its scores over this block, P = exp(s - max), and the
// partial row is divided by the sum, so it holds the block's own softmax
// average of V; the (max, sum) pair goes to `st` as the statistics kernel
// would write it, and the reduction weighs the partial rows by it.  The
// three-pass forward at d = 256 with 64-key blocks runs k_main16 instead.
// The LDS of k_main (also that of k_main_mixed, whose local items use the
// first three arrays as k_main_local does).
template <typename T, int D, int BK>
struct MainLds {
  alignas(16) T Ks[BK * k_ld<D>()];
  alignas(16) T Vt[D * vt_ld<BK>()];
  alignas(16) T Qt[kWaves * 32 * tile_ld<D>()];
  int ridx[kRowTable], rtok[kRowTable];
  int s_items[2];
  int s_local;  // k_main_mixed: the workgroup's current local item
};

// k_main's persistent loop over the block-outer items of the forward list.
template <typename T, int D, int BK, typename PT, bool FUSED>
__device__ __forceinline__ void main_items(MainLds<T, D, BK>& sm, const T* __restrict__ q,
                                           const T* __restrict__ k, const T* __restrict__ v,
                                           const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
                                           const int32_t* __restrict__ qidx, const int4* __restrict__ work,
                                           const int32_t* __restrict__ nwork, int32_t* __restrict__ queue,
                                           const float* __restrict__ lse, float2* __restrict__ st,
                                           PT* __restrict__ partial, size_t dump_row, int H, int g, int NB, int CT,
                                           float scale_log2) {
  using V8 = typename Vec8<T>::type;
  constexpr int KS = D / 16, KT = BK / 32, KK = BK / 16, MT = D / 32;
  constexpr int NT = kAttnThreads, NW = kWaves;
  static_assert(32 * Stage<PT, D>::P * sizeof(PT) <= 32 * tile_ld<D>() * sizeof(T), "stage fits the Q tile");
  T* const Ks = sm.Ks;
  T* const Vt = sm.Vt;
  T* const Qt = sm.Qt;
  int* const ridx = sm.ridx;
  int* const rtok = sm.rtok;
  int* const s_items = sm.s_items;
  ItemChain ch(queue, nwork[2], s_items);  // the forward list
  const int4* const wl = work + nwork[0];
  if (ch.cur < 0) return;
  const int HQ = H * g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, hl = lane >> 5;
  T* const qt = Qt + wave * 32 * tile_ld<D>();
  PT* const stage = reinterpret_cast<PT*>(qt);
  PT* const dump = partial + dump_row * D;
  ItemStage<T, D, BK, true, NT> pre;
  pre.load(k, v, qidx, wl, counts, offsets, ch.cur, H, g, NB, CT);
  while (ch.cur >= 0) {
    __syncthreads();  // the previous item's LDS reads are done
    pre.commit(Ks, Vt, ridx, rtok, g, HQ);
    ch.publish(s_items);
    const Item it = pre.it;
    __syncthreads();
    const int after = ch.after(s_items);
    const int nrows = it.ntok * g, ntile = (nrows + 31) / 32;

    // Q pipeline: one register set plus the wave's LDS tile (as in k_stats);
    // the lse of tile i + 1 is loaded with its Q rows.
    V8 qv[KS];
    float lnext = 0.f;
    if (wave < ntile) {
      load_q_tile<T, D>(q, ridx, wave, lane, qv);
      if constexpr (!FUSED) lnext = lse[ridx[wave * 32 + lr]];
    }
    if (ch.nxt >= 0) pre.load(k, v, qidx, wl, counts, offsets, ch.nxt, H, g, NB, CT);
    for (int tl = wave; tl < ntile; tl += NW) {
      put_q_tile<T, D>(qt, lane, qv);
      const float l2 = lnext * kLog2e;
      if (tl + NW < ntile) {
        load_q_tile<T, D>(q, ridx, tl + NW, lane, qv);
        if constexpr (!FUSED) lnext = lse[ridx[(tl + NW) * 32 + lr]];
      }
      f32x16 s[KT];
      qk_tile<T, D, BK>(Ks, qt, lr, hl, s);
      const int row = tl * 32 + lr;
      const int tok = rtok[row];
      const bool unmasked = tile_unmasked<BK>(tok, it.bs);
      const int lim = tok < 0 ? -1 : tok - it.bs;
      float inv = 1.f;
      V8 pb[KK];
      if constexpr (FUSED) {
        const float2 ml = unmasked ? probs_stats<T, BK, false>(s, scale_log2, hl, 0, -INFINITY, pb)
                                   : probs_stats<T, BK, true>(s, scale_log2, hl, lim, -INFINITY, pb);
        inv = ml.y > 0.f ? 1.f / ml.y : 0.f;
        st[tok >= 0 ? (size_t)it.pair0 * g + row : dump_row + lr] = ml;
      } else {
        if (unmasked) probs<T, BK, false>(s, scale_log2, l2, hl, 0, pb);
        else probs<T, BK, true>(s, scale_log2, l2, hl, lim, pb);
      }
      f32x16 o[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[mt] = f32x16{};
      pv_tile<T, D, BK>(Vt, pb, lr, hl, o);
      if constexpr (FUSED) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) o[mt] *= inv;
      }
      store_tile<PT, D>(stage, o, lane, min(32, nrows - tl * 32),
                        partial + ((size_t)it.pair0 * g + (size_t)tl * 32) * D,
                        dump);
    }
    ch.advance(after);
  }
}

template <typename T, int D, int BK, typename PT, bool FUSED>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(attn_waves_per_eu<D, BK>()))) void k_main(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ qidx, const int4* __restrict__ work,
    const int32_t* __restrict__ nwork, int32_t* __restrict__ queue, const float* __restrict__ lse,
    float2* __restrict__ st, PT* __restrict__ partial, size_t dump_row, int H, int g, int NB, int CT,
    float scale_log2) {
  __shared__ __attribute__((aligned(16))) MainLds<T, D, BK> sm;
  main_items<T, D, BK, PT, FUSED>(sm, q, k, v, counts, offsets, qidx, work, nwork, queue, lse, st, partial, dump_row,
                                  H, g, NB, CT, scale_log2);
}

// ---- main kernel with 16-row tiles ------------------------------------------------
// v_mfma_f32_16x16x32 (lane l: A row / B column l % 16, contraction elements
// 8u .. 8u + 7 with u = l / 16; result column l % 16, rows 4u .. 4u + 3).
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// P = exp2(s * c - l2) of the lane's query row as the B operands of
// O^T = V^T P^T: s[kt][r] is key kt*16 + 4u + r; element e of pb[kk] is key
// 32kk + 16 (e / 4) + 4u + e % 4, the order vt_pos16 gives V^T.
template <typename T, int BK, bool MASKED>
__device__ __forceinline__ void probs16(const f32x4* s, float c, float l2, int u, int lim,
                                        typename Vec8<T>::type* pb) {
#pragma unroll
  for (int kk = 0; kk < BK / 32; ++kk) {
    typename Vec8<T>::type x;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kt = 2 * kk + (e >> 2), r = e & 3;
      const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][r], c, -l2));
      x[e] = (T)((!MASKED || kt * 16 + 4 * u + r <= lim) ? p : 0.f);
    }
    pb[kk] = x;
  }
}

// o[m][r] = O^T[d = C0 + 16m + 4u + r][row = l % 16] for the NC columns
// C0 .. C0 + NC of a 16-row tile: staged row-major in the wave's LDS stage,
// then written as whole 16-byte pieces (rows [0, rows) to dst, pitch D; the
// others to the matching rows of dump).
template <typename PT, int D, int NC, int C0>
__device__ __forceinline__ void store_tile16(PT* __restrict__ stage, const f32x4* o, int lane, int rows,
                                             PT* __restrict__ dst, PT* __restrict__ dump) {
  constexpr int P = NC + 16 / (int)sizeof(PT);  // stage pitch: rows 16 bytes apart in banks
  constexpr int EPL = 16 / (int)sizeof(PT), LPR = NC / EPL, RPI = 64 / LPR;
  const int lr = lane & 15, u = lane >> 4;
#pragma unroll
  for (int m = 0; m < NC / 16; ++m) stage_write4<PT>(stage + lr * P + m * 16 + 4 * u, o[m]);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < 16 / RPI; ++i) {
    const int row = i * RPI + lane / LPR, col = (lane % LPR) * EPL;
    const u32x4 val = *reinterpret_cast<const u32x4*>(stage + row * P + col);
    PT* base = row < rows ? dst : dump;
    __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(base + (size_t)row * D + C0 + col));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// store_tile16 with a destination row per tile row: lane l < 16 holds in
// `drow` the partial row (pitch D) of tile row l, or -1 to send it to the
// matching dump row.
template <typename PT, int D, int NC, int C0>
__device__ __forceinline__ void store_tile16_rows(PT* __restrict__ stage, const f32x4* o, int lane, int64_t drow,
                                                  PT* __restrict__ partial, PT* __restrict__ dump) {
  constexpr int P = NC + 16 / (int)sizeof(PT);
  constexpr int EPL = 16 / (int)sizeof(PT), LPR = NC / EPL, RPI = 64 / LPR;
  const int lr = lane & 15, u = lane >> 4;
  const int dlo = (int)(uint32_t)(uint64_t)drow, dhi = (int)(uint32_t)((uint64_t)drow >> 32);
#pragma unroll
  for (int m = 0; m < NC / 16; ++m) stage_write4<PT>(stage + lr * P + m * 16 + 4 * u, o[m]);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < 16 / RPI; ++i) {
    const int row = i * RPI + lane / LPR, col = (lane % LPR) * EPL;
    const int64_t r = (int64_t)(((uint64_t)(uint32_t)__shfl(dhi, row, 64) << 32) | (uint32_t)__shfl(dlo, row, 64));
    const u32x4 val = *reinterpret_cast<const u32x4*>(stage + row * P + col);
    PT* dst = r >= 0 ? partial + (size_t)r * D : dump + (size_t)row * D;
    __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(dst + C0 + col));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The three-pass main kernel where k_main's 32-row tiles run one wave per
// SIMD: d = 256 with 64-key blocks (SPLIT: the halves of 128-key blocks) and
// d = 128 with 128-key blocks.  There a lane of k_main holds 128 registers of
// O^T (d = 256) or 64 of scores plus 64 of O^T (B_K = 128); with 16-row tiles
// it holds a quarter of the scores and of each O^T half, so eight waves of a
// workgroup share the staged K and V at two waves per SIMD.  Each wave walks 16-row tiles; the Q rows of
// a tile are gathered straight into the B operand of S^T = K Q^T (64
// contiguous bytes of each row per load), tile i + 1 in flight while tile i
// computes; O^T is accumulated and stored in two 128-column halves.
// The LDS of k_main16 (also that of k_main_local16 and k_main_mixed16, whose
// local items use the first three arrays).
template <typename T, int D, int BK, typename PT>
struct Main16Lds {
  static constexpr int SP = D / 2 + 16 / (int)sizeof(PT);  // stage pitch of store_tile16
  alignas(16) T Ks[BK * k_ld<D>()];
  alignas(16) T Vt[D * vt_ld<BK>()];
  alignas(16) PT Stg[8 * 16 * SP];
  int ridx[kRowTable], rtok[kRowTable];
  int s_items[2];
  int s_local;  // k_main_mixed16: the workgroup's current local item
};

// k_main16's persistent loop over the block-outer items of the forward list.
template <typename T, int D, int BK, typename PT, bool SPLIT>
__device__ __forceinline__ void main16_items(Main16Lds<T, D, BK, PT>& sm, const T* __restrict__ q,
                                             const T* __restrict__ k, const T* __restrict__ v,
                                             const int32_t* __restrict__ counts,
                                             const int32_t* __restrict__ offsets, const int32_t* __restrict__ qidx,
                                             const int4* __restrict__ work, const int32_t* __restrict__ nwork,
                                             int32_t* __restrict__ queue, const float* __restrict__ lse,
                                             PT* __restrict__ partial, size_t dump_row, size_t half_rows, int H,
                                             int g, int NB, int CT, float scale_log2) {
  using V8 = typename Vec8<T>::type;
  constexpr int NT = 512, NW = NT / 64;
  constexpr int KS = D / 32;   // contraction steps of S^T
  constexpr int KT = BK / 16;  // key tiles of S^T
  constexpr int KK = BK / 32;  // contraction steps of O^T
  constexpr int MH = D / 32;   // 16-column O^T tiles per half
  constexpr int SP = Main16Lds<T, D, BK, PT>::SP;
  T* const Ks = sm.Ks;
  T* const Vt = sm.Vt;
  PT* const Stg = sm.Stg;
  int* const ridx = sm.ridx;
  int* const rtok = sm.rtok;
  int* const s_items = sm.s_items;
  ItemChain ch(queue, SPLIT ? 2 * nwork[2] : nwork[2], s_items);  // the forward list
  const int4* const wl = work + nwork[0];
  if (ch.cur < 0) return;
  const int HQ = H * g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, u = lane >> 4;
  PT* const stage = Stg + wave * 16 * SP;
  PT* const dump = partial + dump_row * D;
  ItemStage<T, D, BK, true, NT, SPLIT, true> pre;
  pre.load(k, v, qidx, wl, counts, offsets, ch.cur, H, g, NB, CT);
  while (ch.cur >= 0) {
    __syncthreads();  // the previous item's LDS reads are done
    pre.commit(Ks, Vt, ridx, rtok, g, HQ);
    ch.publish(s_items);
    const Item it = pre.it;
    __syncthreads();
    const int after = ch.after(s_items);
    const int nrows = it.ntok * g, ntile = (nrows + 15) / 16;

    auto ld = [&](int tl, V8* b, float& l) {
      const int qr = ridx[tl * 16 + lr];
      const T* row = q + (size_t)qr * D + 8 * u;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) b[ks] = load8(row + ks * 32);
      l = lse[qr];
    };
    auto tile = [&](int tl, const V8* b, float lrow) {
      f32x4 s[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) s[kt] = f32x4{};
      const T* kp = Ks + lr * k_ld<D>() + 8 * u;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) s[kt] = mfma16(load8(kp + kt * 16 * k_ld<D>() + ks * 32), b[ks], s[kt]);
      const int tok = rtok[tl * 16 + lr];
      V8 pb[KK];
      if (tile_unmasked<BK>(tok, it.bs)) probs16<T, BK, false>(s, scale_log2, lrow * kLog2e, u, 0, pb);
      else probs16<T, BK, true>(s, scale_log2, lrow * kLog2e, u, tok < 0 ? -1 : tok - it.bs, pb);
      PT* const dst = partial + ((size_t)it.half * half_rows + (size_t)it.pair0 * g + (size_t)tl * 16) * D;
      const int rows = min(16, nrows - tl * 16);
      const T* vp = Vt + lr * vt_ld<BK>() + 8 * u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 o[MH];
#pragma unroll
        for (int m = 0; m < MH; ++m) o[m] = f32x4{};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
          for (int m = 0; m < MH; ++m)
            o[m] = mfma16(load8(vp + ((h * MH + m) * 16) * vt_ld<BK>() + kk * 32), pb[kk], o[m]);
        if (h == 0) store_tile16<PT, D, D / 2, 0>(stage, o, lane, rows, dst, dump);
        else store_tile16<PT, D, D / 2, D / 2>(stage, o, lane, rows, dst, dump);
      }
    };
    V8 qa[KS], qb[KS];
    float la = 0.f, lb = 0.f;
    if (wave < ntile) ld(wave, qa, la);
    if (ch.nxt >= 0) pre.load(k, v, qidx, wl, counts, offsets, ch.nxt, H, g, NB, CT);
    for (int tl = wave; tl < ntile; tl += 2 * NW) {
      if (tl + NW < ntile) ld(tl + NW, qb, lb);
      tile(tl, qa, la);
      if (tl + NW >= ntile) break;
      if (tl + 2 * NW < ntile) ld(tl + 2 * NW, qa, la);
      tile(tl + NW, qb, lb);
    }
    ch.advance(after);
  }
}

template <typename T, int D, int BK, typename PT, bool SPLIT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void k_main16(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ qidx, const int4* __restrict__ work,
    const int32_t* __restrict__ nwork, int32_t* __restrict__ queue, const float* __restrict__ lse,
    PT* __restrict__ partial, size_t dump_row, size_t half_rows, int H, int g, int NB, int CT, float scale_log2) {
  __shared__ __attribute__((aligned(16))) Main16Lds<T, D, BK, PT> sm;
  main16_items<T, D, BK, PT, SPLIT>(sm, q, k, v, counts, offsets, qidx, work, nwork, queue, lse, partial, dump_row,
                                    half_rows, H, g, NB, CT, scale_log2);
}

// ---- local entries, per query block ---------------------------------------------
// The entries of a query's own, previous and first block (its local entries)
// are computed per query block: one workgroup per (KV head, query block, group
// of kLocalTiles 32-row tiles of the block's rows), wave w taking tile w of the
// group.  The block's queries are contiguous, so their Q rows are gathered
// once and kept in registers (the B operand of S^T = K Q^T) while the block's
// local key blocks (kinds 0 .. min(e, 2): own, previous, first) are staged in
// LDS one after another; a row uses the key blocks its token selects (its
// local word), the own block causally.  Statistics: the rows' (max, sum) over
// those blocks, merged, go to one (max, sum) pair per row.  Main: the rows'
// exp(s - lse) V over those blocks, summed in registers, go to one partial row
// per row.  Both land at the rows of the token's designated local entry
// (its own-block entry, else previous, else first; k_main skips local entries,
// so those rows are free), so the combine and the reduction read one local
// row instead of up to three.
constexpr int kLocalTiles = kWaves;
constexpr int kLocalRows = 32 * kLocalTiles;

struct LocalItem {
  int h, e, bs, ntok, seq_lo, seq_hi, row0, rows;
};

// Workgroup i runs on XCD i % 8.  The row groups of kLocalUnit consecutive
// query blocks (one unit) go to one XCD, so the key blocks they share (their
// own blocks, each other's previous blocks and the first block) are fetched
// into that XCD's L2 once instead of by every XCD.
constexpr int kLocalUnit = 4;

// Local item of workgroup i = (KV head, global block, row group); rows = 0
// when the group lies past the block's rows or past the last block.
__device__ __forceinline__ LocalItem local_item(int i, const int32_t* __restrict__ cu,
                                                const int32_t* __restrict__ gboff, int num_seqs, int NB, int BK, int g,
                                                int groups, int nblocks) {
  LocalItem it;
  const int per_unit = kLocalUnit * groups, k = i >> 3;
  const int u = (k / per_unit) * 8 + (i & 7), w = k % per_unit;
  const int f = u * kLocalUnit + w / groups, grp = w % groups;
  if (f >= nblocks) {
    it.rows = 0;
    return it;
  }
  it.h = f / NB;
  const int gb = f - it.h * NB;
  const int sq = seq_of_block(gboff, num_seqs, gb);
  it.e = gb - gboff[sq];
  it.seq_lo = cu[sq];
  it.seq_hi = cu[sq + 1];
  it.bs = it.seq_lo + it.e * BK;
  it.ntok = min(BK, it.seq_hi - it.bs);
  it.row0 = grp * kLocalRows;
  it.rows = max(0, min(kLocalRows, it.ntok * g - it.row0));
  return it;
}

// Q / lse row of row r (within the item) of a local item; rows past the
// item map to its first row, so that every gather stays in bounds.
__device__ __forceinline__ int local_qrow(const LocalItem& it, int r, int g, int HQ) {
  const int row = it.row0 + (r < it.rows ? r : 0);
  return (it.bs + row / g) * HQ + it.h * g + row % g;
}

// The wave's Q tile of a local item (item rows 32 * wave + 0..31), in the
// row-contiguous layout of load_q_tile.
template <typename T, int D>
__device__ __forceinline__ void load_q_local(const T* __restrict__ q, const LocalItem& it, int wave, int lane, int g,
                                             int HQ, typename Vec8<T>::type* qv) {
#pragma unroll
  for (int v = 0; v < D / 16; ++v) {
    const int e = (v * 64 + lane) * 8;
    qv[v] = load8(q + (size_t)local_qrow(it, wave * 32 + e / D, g, HQ) * D + e % D);
  }
}

// The wave's Q tile of a local item gathered straight into the B-operand
// layout of S^T = K Q^T (as load_q_frag).
template <typename T, int D>
__device__ __forceinline__ void load_q_local_frag(const T* __restrict__ q, const LocalItem& it, int wave, int lr,
                                                  int hl, int g, int HQ, typename Vec8<T>::type* b) {
  const T* row = q + (size_t)local_qrow(it, wave * 32 + lr, g, HQ) * D + hl * 8;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) b[ks] = load8(row + ks * 16);
}

// One key block of head h in registers, then in LDS: K as [key][D + 8] and,
// WITH_V, V transposed and key-permuted as in ItemStage.  Keys past nk repeat
// the last key (only the own block can be short, and there the causal mask
// hides them).  load() only issues the loads, so they stay in flight while the
// previous block computes; commit() writes them to LDS.
template <typename T, int D, int BK, bool WITH_V, int NT = kAttnThreads, bool VT16 = false>
struct BlockStage {
  using V8 = typename Vec8<T>::type;
  static constexpr int C8 = D / 8, KV = BK * C8 / NT, KP = BK / 2;
  static constexpr int VP = WITH_V ? KP * C8 / NT : 1;
  static_assert(BK * C8 % NT == 0 && (!WITH_V || KP * C8 % NT == 0), "whole vectors");
  V8 kr[KV], va[VP], vb[VP];

  __device__ __forceinline__ void load(const T* __restrict__ kg, const T* __restrict__ vg, int H, int h, int kbs,
                                       int nk) {
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int vi = threadIdx.x + i * NT;
      kr[i] = load8(kg + ((size_t)(kbs + min(vi / C8, nk - 1)) * H + h) * D + (vi % C8) * 8);
    }
    if constexpr (WITH_V) {
#pragma unroll
      for (int i = 0; i < VP; ++i) {
        const int vi = threadIdx.x + i * NT;
        const int c = vi / KP, key = 2 * (vi % KP);
        va[i] = load8(vg + ((size_t)(kbs + min(key, nk - 1)) * H + h) * D + c * 8);
        vb[i] = load8(vg + ((size_t)(kbs + min(key + 1, nk - 1)) * H + h) * D + c * 8);
      }
    }
  }

  __device__ __forceinline__ void commit(T* __restrict__ Ks, T* __restrict__ Vt) const {
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int vi = threadIdx.x + i * NT;
      *reinterpret_cast<V8*>(Ks + (vi / C8) * k_ld<D>() + (vi % C8) * 8) = kr[i];
    }
    if constexpr (WITH_V) {
#pragma unroll
      for (int i = 0; i < VP; ++i) {
        const int vi = threadIdx.x + i * NT;
        const int c = vi / KP, key = 2 * (vi % KP);
        const int pos = VT16 ? vt_pos16(key) : vt_pos(key);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t packed = (uint32_t)bits16(va[i][e]) | ((uint32_t)bits16(vb[i][e]) << 16);
          *reinterpret_cast<uint32_t*>(Vt + (c * 8 + e) * vt_ld<BK>() + pos) = packed;
        }
      }
    }
  }
};

// Visible-key limit of a row for local kind `kind`: -1 when the row's token
// does not select that block (or the row is past the item), the key offset
// of the token in its own block for kind 0, the whole block otherwise.
template <int BK>
__device__ __forceinline__ int local_lim(int tok, unsigned word, int kind, int kbs) {
  if (tok < 0 || !local_has(word, kind)) return -1;
  return kind == 0 ? tok - kbs : BK - 1;
}

// Row (slot * g + j) of a local item's row r where its token's local row
// goes: the partial / statistics row of the token's designated local entry;
// -1 for rows past the item and tokens without local entries.
__device__ __forceinline__ int64_t local_dst(const LocalItem& it, int r, int tok, unsigned word,
                                             const int32_t* __restrict__ slot, int N, int T, int g) {
  if (tok < 0 || word == 0u) return -1;
  const int p = slot[((size_t)it.h * N + tok) * T + local_designated(word)];
  return (int64_t)p * g + (it.row0 + r) % g;
}

// queue: the statistics kernel's work-queue counters, cleared by workgroup 0
// (this kernel runs first in the statistics call).
template <typename T, int D, int BK>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(stats_local_waves_per_eu<D, BK>()))) void k_stats_local(
    const T* __restrict__ q, const T* __restrict__ k, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ gboff, int num_seqs, const int32_t* __restrict__ loc,
    const int32_t* __restrict__ slot, float2* __restrict__ st, int32_t* __restrict__ queue, int N, int H, int g,
    int Tn, int NB, int groups, float scale_log2) {
  using V8 = typename Vec8<T>::type;
  constexpr int KS = D / 16, KT = BK / 32;
  // ALL (d <= 128): the item's up to three key blocks are loaded at once and
  // staged side by side, so the item waits for memory once instead of once
  // per block; the Q tile is then kept as the B operand in registers (the
  // three blocks fill the LDS that its tile would take).  Wide tiles keep
  // the Q tile in registers as well, as the statistics kernel does.
  constexpr bool ALL = stats_local_all<D, BK>();
  constexpr bool FRAG = ALL || stats_gather_b<D, BK>();
  constexpr int KB = BK * k_ld<D>();  // one staged key block
  __shared__ __attribute__((aligned(16))) T Ks[(ALL ? 3 : 1) * KB];
  __shared__ __attribute__((aligned(16))) T Qt[FRAG ? 8 : kWaves * 32 * tile_ld<D>()];
  if (blockIdx.x == 0) clear_queue(queue);
  const LocalItem it = local_item(blockIdx.x, cu, gboff, num_seqs, NB, BK, g, groups, H * NB);
  if (it.rows == 0) return;
  const int HQ = H * g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, hl = lane >> 5;
  const bool busy = wave * 32 < it.rows;
  T* const qt = Qt + (FRAG ? 0 : wave * 32 * tile_ld<D>());
  const int kinds = min(it.e, 2) + 1;
  if constexpr (ALL) {
    BlockStage<T, D, BK, false> b0, b1, b2;
    b0.load(k, nullptr, H, it.h, it.bs, it.ntok);
    if (kinds > 1) b1.load(k, nullptr, H, it.h, it.seq_lo + local_block(1, it.e) * BK, BK);
    if (kinds > 2) b2.load(k, nullptr, H, it.h, it.seq_lo + local_block(2, it.e) * BK, BK);
    V8 qv[KS];
    if (busy) load_q_local_frag<T, D>(q, it, wave, lr, hl, g, HQ, qv);
    const int row = wave * 32 + lr;
    const int qrow = local_qrow(it, row, g, HQ);
    const int tok = row < it.rows ? qrow / HQ : -1;
    const unsigned word = tok >= 0 ? (unsigned)loc[(size_t)it.h * N + tok] : 0u;
    b0.commit(Ks, nullptr);
    if (kinds > 1) b1.commit(Ks + KB, nullptr);
    if (kinds > 2) b2.commit(Ks + 2 * KB, nullptr);
    __syncthreads();
    if (!busy) return;
    // the blocks merge in the order own, previous, first, as below
    float M = -INFINITY, L = 0.f;
    for (int kind = 0; kind < kinds; ++kind) {
      f32x16 s[KT];
      qk_frag<T, D, BK>(Ks + kind * KB, qv, lr, hl, s);
      const int lim = local_lim<BK>(tok, word, kind, it.seq_lo + local_block(kind, it.e) * BK);
      const float2 ml = kind == 0 ? row_stats<BK, true>(s, hl, lim, scale_log2)
                                  : row_stats<BK, false>(s, hl, 0, scale_log2);
      if (lim >= 0) {
        const float mn = fmaxf(M, ml.x);
        L = L * __builtin_amdgcn_exp2f(M - mn) + ml.y * __builtin_amdgcn_exp2f(ml.x - mn);
        M = mn;
      }
    }
    const int64_t dst = local_dst(it, row, tok, word, slot, N, Tn, g);
    if (hl == 0 && dst >= 0) st[dst] = make_float2(M, L);
    return;
  }
  // every load of the item's start goes out here: the own block's K, the Q
  // tile and the row's local word
  BlockStage<T, D, BK, false> pre;
  pre.load(k, nullptr, H, it.h, it.bs, it.ntok);
  V8 qv[KS];
  if (busy) {
    if constexpr (FRAG) load_q_local_frag<T, D>(q, it, wave, lr, hl, g, HQ, qv);
    else load_q_local<T, D>(q, it, wave, lane, g, HQ, qv);
  }
  const int row = wave * 32 + lr;
  const int qrow = local_qrow(it, row, g, HQ);
  const int tok = row < it.rows ? qrow / HQ : -1;
  const unsigned word = tok >= 0 ? (unsigned)loc[(size_t)it.h * N + tok] : 0u;
  float M = -INFINITY, L = 0.f;
  for (int kind = 0; kind < kinds; ++kind) {
    const int kbs = it.seq_lo + local_block(kind, it.e) * BK;
    __syncthreads();  // the previous block's K reads are done
    pre.commit(Ks, nullptr);
    __syncthreads();
    if (kind + 1 < kinds) pre.load(k, nullptr, H, it.h, it.seq_lo + local_block(kind + 1, it.e) * BK, BK);
    if (!busy) continue;
    f32x16 s[KT];
    if constexpr (FRAG) {
      qk_frag<T, D, BK>(Ks, qv, lr, hl, s);
    } else {
      if (kind == 0) put_q_tile<T, D>(qt, lane, qv);
      qk_tile<T, D, BK>(Ks, qt, lr, hl, s);
    }
    const int lim = local_lim<BK>(tok, word, kind, kbs);
    const float2 ml = kind == 0 ? row_stats<BK, true>(s, hl, lim, scale_log2)
                                : row_stats<BK, false>(s, hl, 0, scale_log2);
    if (lim >= 0) {
      const float mn = fmaxf(M, ml.x);
      L = L * __builtin_amdgcn_exp2f(M - mn) + ml.y * __builtin_amdgcn_exp2f(ml.x - mn);
      M = mn;
    }
  }
  const int64_t dst = local_dst(it, row, tok, word, slot, N, Tn, g);
  if (busy && hl == 0 && dst >= 0) st[dst] = make_float2(M, L);
}

// One local item of the main stage (rows > 0); Ks, Vt and Qt are the
// workgroup's LDS arrays, whose earlier readers finish before its first
// barrier.
template <typename T, int D, int BK, typename PT, bool FUSED>
__device__ __forceinline__ void local_main_item(const LocalItem& it, T* Ks, T* Vt, T* Qt, const T* __restrict__ q,
                                                const T* __restrict__ k, const T* __restrict__ v,
                                                const int32_t* __restrict__ loc, const int32_t* __restrict__ slot,
                                                const float* __restrict__ lse, float2* __restrict__ st,
                                                PT* __restrict__ partial, PT* __restrict__ dump, int N, int H, int g,
                                                int Tn, float scale_log2) {
  using V8 = typename Vec8<T>::type;
  constexpr int KS = D / 16, KT = BK / 32, KK = BK / 16, MT = D / 32;
  const int HQ = H * g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, hl = lane >> 5;
  const bool busy = wave * 32 < it.rows;
  T* const qt = Qt + wave * 32 * tile_ld<D>();
  const int kinds = min(it.e, 2) + 1;
  // every load of the item's start goes out here: the own block's K and V,
  // the Q tile, the row's local word and lse
  BlockStage<T, D, BK, true> pre;
  pre.load(k, v, H, it.h, it.bs, it.ntok);
  V8 qv[KS];
  if (busy) load_q_local<T, D>(q, it, wave, lane, g, HQ, qv);
  const int row = wave * 32 + lr;
  const int qrow = local_qrow(it, row, g, HQ);
  const int tok = row < it.rows ? qrow / HQ : -1;
  const unsigned word = tok >= 0 ? (unsigned)loc[(size_t)it.h * N + tok] : 0u;
  const float l2 = !FUSED && tok >= 0 ? lse[qrow] * kLog2e : 0.f;
  float M = -INFINITY, L = 0.f;
  f32x16 o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = f32x16{};
  for (int kind = 0; kind < kinds; ++kind) {
    const int kbs = it.seq_lo + local_block(kind, it.e) * BK;
    __syncthreads();  // the previous block's K / V reads are done
    pre.commit(Ks, Vt);
    __syncthreads();
    if (kind + 1 < kinds) pre.load(k, v, H, it.h, it.seq_lo + local_block(kind + 1, it.e) * BK, BK);
    if (!busy) continue;
    if (kind == 0) put_q_tile<T, D>(qt, lane, qv);
    f32x16 s[KT];
    qk_tile<T, D, BK>(Ks, qt, lr, hl, s);
    const int lim = local_lim<BK>(tok, word, kind, kbs);
    V8 pb[KK];
    if constexpr (FUSED) {
      // rows that do not select this block (lim < 0) get no probabilities
      // and keep their statistics
      const float2 ml = __all(lim == BK - 1) ? probs_stats<T, BK, false>(s, scale_log2, hl, 0, M, pb)
                                             : probs_stats<T, BK, true>(s, scale_log2, hl, lim, M, pb);
      if (lim >= 0) {
        const float mn = fmaxf(M, ml.x);
        const float alpha = __builtin_amdgcn_exp2f(M - mn);  // 0 while M is -inf
        L = L * alpha + ml.y * __builtin_amdgcn_exp2f(ml.x - mn);
        M = mn;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) o[mt] *= alpha;
      }
    } else {
      if (__all(lim == BK - 1)) probs<T, BK, false>(s, scale_log2, l2, hl, 0, pb);
      else probs<T, BK, true>(s, scale_log2, l2, hl, lim, pb);
    }
    pv_tile<T, D, BK>(Vt, pb, lr, hl, o);
  }
  const int64_t dst = local_dst(it, row, tok, word, slot, N, Tn, g);
  if constexpr (FUSED) {
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] *= inv;
    if (busy && hl == 0 && dst >= 0) st[dst] = make_float2(M, L);
  }
  if (busy) store_tile_rows<PT, D>(reinterpret_cast<PT*>(qt), o, lane, dst, partial, dump);
}

// FUSED: the rows' (max, sum) run over the local blocks as in k_stats_local
// (the same merge, so the pair written to st is the one it writes) and the
// accumulator is rescaled when the max grows; the partial row is divided by
// the final sum.  queue: the main kernel's work-queue counters, cleared by
// workgroup 0 (this kernel runs first in the forward call).
template <typename T, int D, int BK, typename PT, bool FUSED>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(attn_waves_per_eu<D, BK>()))) void k_main_local(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ gboff, int num_seqs, const int32_t* __restrict__ loc,
    const int32_t* __restrict__ slot, const float* __restrict__ lse, float2* __restrict__ st,
    PT* __restrict__ partial, PT* __restrict__ dump, int32_t* __restrict__ queue, int N, int H, int g, int Tn, int NB,
    int groups, float scale_log2) {
  __shared__ __attribute__((aligned(16))) T Ks[BK * k_ld<D>()];
  __shared__ __attribute__((aligned(16))) T Vt[D * vt_ld<BK>()];
  __shared__ __attribute__((aligned(16))) T Qt[kWaves * 32 * tile_ld<D>()];
  if (blockIdx.x == 0) clear_queue(queue);
  const LocalItem it = local_item(blockIdx.x, cu, gboff, num_seqs, NB, BK, g, groups, H * NB);
  if (it.rows == 0) return;
  local_main_item<T, D, BK, PT, FUSED>(it, Ks, Vt, Qt, q, k, v, loc, slot, lse, st, partial, dump, N, H, g, Tn,
                                       scale_log2);
}

// Counter of k_main_mixed's local items within each XCD queue's line (the
// block-outer items count at offset 0).
constexpr int kLocalCounter = kQueueStride / 2;

// Thread 0: the next local item of a mixed launch, or -1 once none is left.
// Claim c of XCD x is local item 8c + x, the order of the local kernels'
// grid, so a unit's items stay on its XCD while that XCD has items left;
// then the other XCDs' items are taken.
__device__ __forceinline__ int claim_local(int32_t* __restrict__ queue, int per_xcd, int& tried) {
  const int x = blockIdx.x & (kQueues - 1);
  while (tried < kQueues) {
    const int xx = (x + tried) & (kQueues - 1);
    const int c = atomicAdd(queue + xx * kQueueStride + kLocalCounter, 1);
    if (c < per_xcd) return 8 * c + xx;
    ++tried;
  }
  return -1;
}

// A workgroup's loop over local items until none is left: run(i) for each
// claimed item i; thread 0 claims the next item while the current one runs.
// s_local: a __shared__ int of the workgroup.
template <typename F>
__device__ __forceinline__ void local_loop(int* s_local, int32_t* __restrict__ queue, int per_xcd, F&& run) {
  int tried = 0;
  if (threadIdx.x == 0) *s_local = claim_local(queue, per_xcd, tried);
  __syncthreads();
  int cur = __builtin_amdgcn_readfirstlane(*s_local);
  while (cur >= 0) {
    int nxt = -1;
    if (threadIdx.x == 0) nxt = claim_local(queue, per_xcd, tried);
    run(cur);
    __syncthreads();  // every thread has read the current item
    if (threadIdx.x == 0) *s_local = nxt;
    __syncthreads();
    cur = __builtin_amdgcn_readfirstlane(*s_local);
  }
}

// The three-pass main stage at d = 64 and 128 with 64-key blocks as one
// persistent launch over both kinds of items: k_main_local's and k_main's.
// A local item walks up to three dependent blocks and is bound by latency; a
// block-outer item is bound by its Q gather and partial-row traffic.  Run
// side by side, the local items' latency hides under the block-outer items'
// traffic instead of filling a launch of its own.  Workgroup b starts on the
// local items when its place in its XCD's share, b >> 3, is a multiple of
// local_every, the others on the block-outer items, and each goes on to the
// other kind when its first kind runs out, so neither kind waits on the
// other.  With every other workgroup starting local, a CU's two workgroups
// hold one of each kind whatever order the dispatcher fills CUs in (taking
// the first half of each share instead measured 0.3-1% slower).  The
// counters of both kinds are cleared by the launch before this one.
template <typename T, int D, int BK, typename PT>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(attn_waves_per_eu<D, BK>()))) void k_main_mixed(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ qidx, const int4* __restrict__ work,
    const int32_t* __restrict__ nwork, int32_t* __restrict__ queue, const float* __restrict__ lse,
    PT* __restrict__ partial, size_t dump_row, const int32_t* __restrict__ cu, const int32_t* __restrict__ gboff,
    int num_seqs, const int32_t* __restrict__ loc, const int32_t* __restrict__ slot, int N, int H, int g, int Tn,
    int NB, int CT, int groups, int local_per_xcd, int local_every, float scale_log2) {
  __shared__ __attribute__((aligned(16))) MainLds<T, D, BK> sm;
  PT* const dump = partial + dump_row * D;
  auto run = [&](int i) {
    const LocalItem it = local_item(i, cu, gboff, num_seqs, NB, BK, g, groups, H * NB);
    if (it.rows > 0)
      local_main_item<T, D, BK, PT, false>(it, sm.Ks, sm.Vt, sm.Qt, q, k, v, loc, slot, lse, nullptr, partial, dump,
                                           N, H, g, Tn, scale_log2);
  };
  if ((int)(blockIdx.x >> 3) % local_every == 0) local_loop(&sm.s_local, queue, local_per_xcd, run);
  main_items<T, D, BK, PT, false>(sm, q, k, v, counts, offsets, qidx, work, nwork, queue, lse, nullptr, partial,
                                  dump_row, H, g, NB, CT, scale_log2);
  local_loop(&sm.s_local, queue, local_per_xcd, run);
}

// The three-pass local main kernel at d = 256 (k_main_local's items, 128
// rows each): eight waves with one 16-row tile each, so that a lane's O^T
// over the whole head dimension takes 64 registers and two waves fit a SIMD
// (k_main_local's 32-row tiles take 128, one wave per SIMD).  The layouts are
// k_main16's; the accumulation over the local blocks and the designated-row
// stores are k_main_local's.
template <typename T, typename PT>
__device__ __forceinline__ void local16_item(const LocalItem& it, Main16Lds<T, 256, 64, PT>& sm,
                                             const T* __restrict__ q, const T* __restrict__ k,
                                             const T* __restrict__ v, const int32_t* __restrict__ loc,
                                             const int32_t* __restrict__ slot, const float* __restrict__ lse,
                                             PT* __restrict__ partial, PT* __restrict__ dump, int N, int H, int g,
                                             int Tn, float scale_log2) {
  using V8 = typename Vec8<T>::type;
  constexpr int D = 256, BK = 64, NT = 512, NW = NT / 64;
  constexpr int KS = D / 32, KT = BK / 16, MT = D / 16;
  constexpr int SP = Main16Lds<T, D, BK, PT>::SP;
  static_assert(NW * 16 == kLocalRows, "one 16-row tile per wave");
  T* const Ks = sm.Ks;
  T* const Vt = sm.Vt;
  PT* const Stg = sm.Stg;
  const int HQ = H * g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, u = lane >> 4;
  const bool busy = wave * 16 < it.rows;
  PT* const stage = Stg + wave * 16 * SP;
  const int kinds = min(it.e, 2) + 1;
  // every load of the item's start goes out here: the own block's K and V,
  // the Q rows (the B operand of S^T = K Q^T), the row's local word and lse
  BlockStage<T, D, BK, true, NT, true> pre;
  pre.load(k, v, H, it.h, it.bs, it.ntok);
  const int row = wave * 16 + lr;
  const int qrow = local_qrow(it, row, g, HQ);
  V8 qv[KS];
  if (busy) {
    const T* qp = q + (size_t)qrow * D + 8 * u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qv[ks] = load8(qp + ks * 32);
  }
  const int tok = row < it.rows ? qrow / HQ : -1;
  const unsigned word = tok >= 0 ? (unsigned)loc[(size_t)it.h * N + tok] : 0u;
  const float l2 = tok >= 0 ? lse[qrow] * kLog2e : 0.f;
  f32x4 o[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) o[m] = f32x4{};
  for (int kind = 0; kind < kinds; ++kind) {
    const int kbs = it.seq_lo + local_block(kind, it.e) * BK;
    __syncthreads();  // the previous block's K / V reads are done
    pre.commit(Ks, Vt);
    __syncthreads();
    if (kind + 1 < kinds) pre.load(k, v, H, it.h, it.seq_lo + local_block(kind + 1, it.e) * BK, BK);
    if (!busy) continue;
    f32x4 s[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) s[kt] = f32x4{};
    const T* kp = Ks + lr * k_ld<D>() + 8 * u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) s[kt] = mfma16(load8(kp + kt * 16 * k_ld<D>() + ks * 32), qv[ks], s[kt]);
    const int lim = local_lim<BK>(tok, word, kind, kbs);
    V8 pb[2];
    if (__all(lim == BK - 1)) probs16<T, BK, false>(s, scale_log2, l2, u, 0, pb);
    else probs16<T, BK, true>(s, scale_log2, l2, u, lim, pb);
    const T* vp = Vt + lr * vt_ld<BK>() + 8 * u;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int m = 0; m < MT; ++m) o[m] = mfma16(load8(vp + m * 16 * vt_ld<BK>() + kk * 32), pb[kk], o[m]);
  }
  const int64_t dst = local_dst(it, row, tok, word, slot, N, Tn, g);
  if (busy) {
    store_tile16_rows<PT, D, D / 2, 0>(stage, o, lane, dst, partial, dump);
    store_tile16_rows<PT, D, D / 2, D / 2>(stage, o + MT / 2, lane, dst, partial, dump);
  }
}

template <typename T, typename PT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void k_main_local16(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ gboff, int num_seqs, const int32_t* __restrict__ loc,
    const int32_t* __restrict__ slot, const float* __restrict__ lse, PT* __restrict__ partial,
    PT* __restrict__ dump, int32_t* __restrict__ queue, int N, int H, int g, int Tn, int NB, int groups,
    float scale_log2) {
  __shared__ __attribute__((aligned(16))) Main16Lds<T, 256, 64, PT> sm;
  if (blockIdx.x == 0) clear_queue(queue);
  const LocalItem it = local_item(blockIdx.x, cu, gboff, num_seqs, NB, 64, g, groups, H * NB);
  if (it.rows == 0) return;
  local16_item<T, PT>(it, sm, q, k, v, loc, slot, lse, partial, dump, N, H, g, Tn, scale_log2);
}

// k_main_mixed at d = 256: k_main_local16's items and k_main16's block-outer
// items (64-key blocks) in one persistent launch.  Here a workgroup fills a
// CU, so the two kinds share the chip by CUs rather than within one.
template <typename T, typename PT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void k_main_mixed16(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ qidx, const int4* __restrict__ work,
    const int32_t* __restrict__ nwork, int32_t* __restrict__ queue, const float* __restrict__ lse,
    PT* __restrict__ partial, size_t dump_row, const int32_t* __restrict__ cu, const int32_t* __restrict__ gboff,
    int num_seqs, const int32_t* __restrict__ loc, const int32_t* __restrict__ slot, int N, int H, int g, int Tn,
    int NB, int CT, int groups, int local_per_xcd, int local_every, float scale_log2) {
  __shared__ __attribute__((aligned(16))) Main16Lds<T, 256, 64, PT> sm;
  PT* const dump = partial + dump_row * 256;
  auto run = [&](int i) {
    const LocalItem it = local_item(i, cu, gboff, num_seqs, NB, 64, g, groups, H * NB);
    if (it.rows > 0) local16_item<T, PT>(it, sm, q, k, v, loc, slot, lse, partial, dump, N, H, g, Tn, scale_log2);
  };
  if ((int)(blockIdx.x >> 3) % local_every == 0) local_loop(&sm.s_local, queue, local_per_xcd, run);
  main16_items<T, 256, 64, PT, false>(sm, q, k, v, counts, offsets, qidx, work, nwork, queue, lse, partial, dump_row,
                                      0, H, g, NB, CT, scale_log2);
  local_loop(&sm.s_local, queue, local_per_xcd, run);
}

// ---- reduce -----------------------------------------------------------------
template <typename PT>
struct Part8;
template <>
struct Part8<float> {
  struct type {
    f32x4 a, b;
  };
  static __device__ __forceinline__ type load(const float* p) {
    return type{__builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p)),
                __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1)};
  }
  static __device__ __forceinline__ float at(const type& x, int i) { return i < 4 ? x.a[i] : x.b[i - 4]; }
};
template <>
struct Part8<__bf16> {
  using type = bf16x8;
  static __device__ __forceinline__ type load(const __bf16* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
  }
  static __device__ __forceinline__ float at(const type& x, int i) { return (float)x[i]; }
};
template <>
struct Part8<_Float16> {
  using type = f16x8;
  static __device__ __forceinline__ type load(const _Float16* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f16x8*>(p));
  }
  static __device__ __forceinline__ float at(const type& x, int i) { return (float)x[i]; }
};

// Items (token t, KV head h), t-major so that the outputs of consecutive items
// are adjacent.  TPI threads per item, each owning 8-element vectors of the
// g*D outputs.  With LOCAL (the forward), the sum starts from the item's local
// partial row group and skips the local slots; the backward's dQ reduction
// sums every slot.  Slots are taken 8 at a time; the 8 partial loads are
// issued together, those of empty and local slots masked off (loading row 0
// in their place made that row a hot spot: 64K g = 4 reduction 0.728 ->
// 0.707 ms), and summed in slot order.
// FUSED (the one-pass forward): the partial rows are per-block softmax
// averages o_b with (max, sum) pairs (m_b, l_b); O = sum_b l_b 2^(m_b - m) o_b
// / l with the row's merged (m, l), also written out as row max and lse.
// SPLIT (B_K = 128 with d = 256): every slot has two partial rows, one per
// key half, the second half_elems elements after the first; both are added,
// the first half first.
template <typename T, typename PT, bool LOCAL, bool FUSED, bool SPLIT = false>
__global__ __launch_bounds__(kReduceThreads) void k_reduce(const int32_t* __restrict__ slot,
                                                           const PT* __restrict__ partial,
                                                           const int32_t* __restrict__ loc, T* __restrict__ out,
                                                           const float2* __restrict__ st,
                                                           float* __restrict__ row_max, float* __restrict__ lse,
                                                           int N, int H, int g, int D, int Tn, int TPI,
                                                           size_t half_elems) {
  static_assert(!SPLIT || (!LOCAL && !FUSED), "split rows only in the three-pass forward without local rows");
  const int ipb = kReduceThreads / TPI;
  const int local = threadIdx.x / TPI;
  if (local >= ipb) return;
  const int64_t item = (int64_t)blockIdx.x * ipb + local;
  if (item >= (int64_t)N * H) return;
  const int t = (int)(item / H), h = (int)(item - (int64_t)t * H);
  const int sub = threadIdx.x - local * TPI;
  const int GD = g * D, nvec = GD / 8;
  const int32_t* sl = slot + ((size_t)h * N + t) * Tn;
  const unsigned word = LOCAL ? (unsigned)loc[(size_t)h * N + t] : 0u;
  // The local row group is at the rows of the designated local entry, whose
  // slot is taken from the first batch of slot loads (the position is below 8
  // unless Sel puts its local blocks late), so its load issues together with
  // that batch's partial loads.
  const int des = LOCAL && word != 0u ? local_designated(word) : 0;
  T* dst = out + ((size_t)t * H + h) * GD;
  for (int vec = sub; vec < nvec; vec += TPI) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if constexpr (FUSED) {
      // One pass in slot order: the row's running max M and sum L (base 2,
      // scaled scores) merge each pair as k_stats_combine does, and the
      // accumulator, kept relative to M, is rescaled when M grows; O = acc / L.
      const int j = vec * 8 / D;  // query head of the vector within the group
      const size_t r = ((size_t)t * H + h) * g + j;
      float M = -INFINITY, L = 0.f;
      for (int j0 = 0; j0 < Tn; j0 += 8) {
        int raw[8], sv[8];
        float2 v[8];
        typename Part8<PT>::type x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) raw[u] = j0 + u < Tn ? sl[j0 + u] : -1;
#pragma unroll
        for (int u = 0; u < 8; ++u) sv[u] = LOCAL && local_entry(word, j0 + u) ? -1 : raw[u];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          v[u] = sv[u] >= 0 ? st[(size_t)sv[u] * g + j] : float2{};
          x[u] = sv[u] >= 0 ? Part8<PT>::load(partial + (size_t)sv[u] * GD + vec * 8) : typename Part8<PT>::type{};
        }
        if (LOCAL && j0 == 0 && word != 0u) {
          int lrow = 0;
#pragma unroll
          for (int u = 0; u < 8; ++u) lrow = des == u ? raw[u] : lrow;
          if (des >= 8) lrow = sl[des];
          const float2 vl = st[(size_t)lrow * g + j];
          const auto xl = Part8<PT>::load(partial + (size_t)lrow * GD + vec * 8);
          M = vl.x;
          L = vl.y;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = Part8<PT>::at(xl, i) * vl.y;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (sv[u] >= 0) {
            const float mn = fmaxf(M, v[u].x);
            const float a = __builtin_amdgcn_exp2f(M - mn);  // 0 while M is -inf
            const float b = v[u].y * __builtin_amdgcn_exp2f(v[u].x - mn);
            L = L * a + b;
            M = mn;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = fmaf(Part8<PT>::at(x[u], i), b, acc[i] * a);
          }
        }
      }
      const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= inv;
      if (vec * 8 % D == 0) {
        row_max[r] = L > 0.f ? M * kLn2 : -INFINITY;
        lse[r] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
      }
    } else {
      for (int j0 = 0; j0 < Tn; j0 += 8) {
        int raw[8], sv[8];
        typename Part8<PT>::type x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) raw[u] = j0 + u < Tn ? sl[j0 + u] : -1;
#pragma unroll
        for (int u = 0; u < 8; ++u) sv[u] = LOCAL && local_entry(word, j0 + u) ? -1 : raw[u];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          x[u] = sv[u] >= 0 ? Part8<PT>::load(partial + (size_t)sv[u] * GD + vec * 8) : typename Part8<PT>::type{};
        if constexpr (SPLIT) {
          typename Part8<PT>::type y[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            y[u] = sv[u] >= 0 ? Part8<PT>::load(partial + half_elems + (size_t)sv[u] * GD + vec * 8)
                              : typename Part8<PT>::type{};
#pragma unroll
          for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              acc[i] += sv[u] >= 0 ? Part8<PT>::at(x[u], i) : 0.f;
              acc[i] += sv[u] >= 0 ? Part8<PT>::at(y[u], i) : 0.f;
            }
          continue;
        }
        if (LOCAL && j0 == 0 && word != 0u) {
          int lrow = 0;
#pragma unroll
          for (int u = 0; u < 8; ++u) lrow = des == u ? raw[u] : lrow;
          if (des >= 8) lrow = sl[des];
          const auto xl = Part8<PT>::load(partial + (size_t)lrow * GD + vec * 8);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = Part8<PT>::at(xl, i);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += sv[u] >= 0 ? Part8<PT>::at(x[u], i) : 0.f;
      }
    }
    typename Vec8<T>::type o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (T)acc[i];
    *reinterpret_cast<typename Vec8<T>::type*>(dst + vec * 8) = o;
  }
}

// ---- dispatch -------------------------------------------------------------------
template <typename T>
struct Ptrs {
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* qidx;
  const int4* work;
  const int32_t* nwork;
  const int32_t* gboff;
  const int32_t* loc;
};

inline Ptrs<int> index_ptrs(const Geometry& geo, const fsa_index& idx) {
  const char* aux = static_cast<const char*>(idx.aux);
  return Ptrs<int>{idx.counts,
                   idx.offsets,
                   idx.qidx,
                   reinterpret_cast<const int4*>(aux + geo.aux_work_sorted),
                   reinterpret_cast<const int32_t*>(aux + geo.aux_nwork),
                   reinterpret_cast<const int32_t*>(aux + geo.aux_seq_gboff),
                   reinterpret_cast<const int32_t*>(aux + geo.aux_loc)};
}

// Zeroes a persistent kernel's queue counters where no local kernel runs
// before it (the local kernels clear them otherwise).
__global__ __launch_bounds__(256) void k_clear_queue(int32_t* __restrict__ queue) { clear_queue(queue); }

// One workgroup of k_main_mixed in kLocalFirstShare (every other one) starts
// on the local items.
// The mixed launch is taken where the local items fill at least
// kMixedMinRounds rounds of its workgroups; with fewer, both kinds take about
// one round each and the two launches in a row measured faster (at 8K tokens,
// 4 KV heads, g = 2: 84 us against 97 us for the main stage).
constexpr int kLocalFirstShare = 2;
constexpr unsigned kMixedMinRounds = 4;

// FSA_MAIN_MIXED=0 keeps the two launches, =1 takes the mixed launch wherever
// both kinds of items exist; unset (or any other value): the rounds rule.
// Both give the same bits: each item runs the same code either way.
inline int mixed_main_override() {
  const char* e = std::getenv("FSA_MAIN_MIXED");
  return e != nullptr && (e[0] == '0' || e[0] == '1') && e[1] == 0 ? e[0] - '0' : -1;
}

// Workgroups of the local kernels, one per item (KV head, global block, row
// group), in whole units per XCD (local_item); the surplus returns at once.
inline unsigned local_grid(const Geometry& geo, int* groups) {
  *groups = (geo.BK * geo.g + kLocalRows - 1) / kLocalRows;
  const int64_t units = ((int64_t)geo.H * geo.NB + kLocalUnit - 1) / kLocalUnit;
  return (unsigned)(((units + 7) / 8) * 8 * kLocalUnit * *groups);
}

template <typename T, int D, int BK>
void stats_typed(const Geometry& geo, const int32_t* cu, const void* q, const void* k, const fsa_index& idx,
                 void* ws, hipStream_t stream) {
  const auto p = index_ptrs(geo, idx);
  const float sl2 = geo.scale * kLog2e;
  float2* st = static_cast<float2*>(ws);
  int32_t* const queue = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + geo.stats_queue_off);
  // the local kernel (or the clear kernel) runs first: it zeroes the queue counters
  if (geo.local) {
    int groups = 0;
    const unsigned grid = local_grid(geo, &groups);
    hipLaunchKernelGGL((k_stats_local<T, D, BK>), dim3(grid), dim3(kAttnThreads), 0, stream,
                       static_cast<const T*>(q), static_cast<const T*>(k), cu, p.gboff, geo.num_seqs, p.loc, idx.slot,
                       st, queue, geo.N, geo.H, geo.g, geo.T, geo.NB, groups, sl2);
  } else {
    hipLaunchKernelGGL(k_clear_queue, dim3(1), dim3(256), 0, stream, queue);
  }
  if (geo.max_work > 0)
    hipLaunchKernelGGL((k_stats<T, D, BK>),
                       dim3(persistent_grid(k_stats<T, D, BK>, stats_threads<D, BK>(), geo.max_work)),
                       dim3(stats_threads<D, BK>()), 0, stream, static_cast<const T*>(q), static_cast<const T*>(k), p.counts,
                       p.offsets, p.qidx, p.work, p.nwork, queue, st, (size_t)geo.dump_row, geo.H, geo.g, geo.NB,
                       geo.chunk_tokens, sl2);
}

// Main kernels.  With `st` (a statistics workspace) the one-pass variant:
// no lse is read, and the per-block (max, sum) pairs go to `st`.
template <typename T, int D, int BK, typename PT, bool FUSED, bool SPLIT = false>
void main_launch(const Geometry& geo, const int32_t* cu, const void* q, const void* k, const void* v,
                 const fsa_index& idx, const float* lse, void* st_ws, void* partial, hipStream_t stream) {
  const auto p = index_ptrs(geo, idx);
  const float sl2 = geo.scale * kLog2e;
  PT* const part = static_cast<PT*>(partial);
  PT* const dump = part + geo.dump_row * geo.d;
  float2* const st = static_cast<float2*>(st_ws);
  int32_t* const queue = reinterpret_cast<int32_t*>(static_cast<char*>(partial) + geo.partial_queue_off);
  if constexpr (!FUSED && BK == 64 && !SPLIT) {
    int groups = 0;
    const unsigned lgrid = geo.local ? local_grid(geo, &groups) : 0;
    unsigned grid = 0;
    if (geo.local && geo.max_work > 0) {
      if constexpr (D == 256) grid = persistent_grid(k_main_mixed16<T, PT>, 512, geo.max_work + lgrid);
      else grid = persistent_grid(k_main_mixed<T, D, BK, PT>, kAttnThreads, geo.max_work + lgrid);
    }
    const int ov = mixed_main_override();
    if (grid > 0 && (ov == 1 || (ov != 0 && lgrid >= kMixedMinRounds * grid))) {
      // both kinds of items in one persistent launch (see k_main_mixed); the
      // clear kernel zeroes the counters of both
      hipLaunchKernelGGL(k_clear_queue, dim3(1), dim3(256), 0, stream, queue);
      const int per_xcd = (int)(lgrid / 8);
      if constexpr (D == 256)
        hipLaunchKernelGGL((k_main_mixed16<T, PT>), dim3(grid), dim3(512), 0, stream, static_cast<const T*>(q),
                           static_cast<const T*>(k), static_cast<const T*>(v), p.counts, p.offsets, p.qidx, p.work,
                           p.nwork, queue, lse, part, (size_t)geo.dump_row, cu, p.gboff, geo.num_seqs, p.loc, idx.slot,
                           geo.N, geo.H, geo.g, geo.T, geo.NB, geo.chunk_tokens, groups, per_xcd,
                           kLocalFirstShare, sl2);
      else
        hipLaunchKernelGGL((k_main_mixed<T, D, BK, PT>), dim3(grid), dim3(kAttnThreads), 0, stream,
                           static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), p.counts,
                           p.offsets, p.qidx, p.work, p.nwork, queue, lse, part, (size_t)geo.dump_row, cu, p.gboff,
                           geo.num_seqs, p.loc, idx.slot, geo.N, geo.H, geo.g, geo.T, geo.NB, geo.chunk_tokens,
                           groups, per_xcd, kLocalFirstShare, sl2);
      return;
    }
  }
  // the local kernel (or the clear kernel) runs first: it zeroes the queue counters
  if (!geo.local) {
    hipLaunchKernelGGL(k_clear_queue, dim3(1), dim3(256), 0, stream, queue);
  } else if constexpr (D == 256 && BK == 64 && !FUSED) {
    // 16-row tiles, eight waves (see k_main_local16)
    int groups = 0;
    const unsigned grid = local_grid(geo, &groups);
    hipLaunchKernelGGL((k_main_local16<T, PT>), dim3(grid), dim3(512), 0, stream, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), cu, p.gboff, geo.num_seqs, p.loc, idx.slot,
                       lse, part, dump, queue, geo.N, geo.H, geo.g, geo.T, geo.NB, groups, sl2);
  } else {
    int groups = 0;
    const unsigned grid = local_grid(geo, &groups);
    hipLaunchKernelGGL((k_main_local<T, D, BK, PT, FUSED>), dim3(grid), dim3(kAttnThreads), 0, stream,
                       static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), cu, p.gboff,
                       geo.num_seqs, p.loc, idx.slot, lse, st, part, dump, queue, geo.N, geo.H, geo.g, geo.T,
                       geo.NB, groups, sl2);
  }
  if (geo.max_work <= 0) return;
  if constexpr (main16<D, BK, FUSED>()) {
    // 16-row tiles, eight waves (see k_main16)
    hipLaunchKernelGGL((k_main16<T, D, BK, PT, SPLIT>),
                       dim3(persistent_grid(k_main16<T, D, BK, PT, SPLIT>, 512, (SPLIT ? 2 : 1) * geo.max_work)),
                       dim3(512),
                       0, stream, static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                       p.counts, p.offsets, p.qidx, p.work, p.nwork, queue, lse, part, (size_t)geo.dump_row,
                       (size_t)geo.split_half_rows, geo.H, geo.g, geo.NB, geo.chunk_tokens, sl2);
  } else {
    static_assert(!SPLIT, "split items only at d = 256");
    hipLaunchKernelGGL((k_main<T, D, BK, PT, FUSED>),
                       dim3(persistent_grid(k_main<T, D, BK, PT, FUSED>, kAttnThreads, geo.max_work)),
                       dim3(kAttnThreads), 0, stream, static_cast<const T*>(q), static_cast<const T*>(k),
                       static_cast<const T*>(v), p.counts, p.offsets, p.qidx, p.work, p.nwork, queue, lse, st, part,
                       (size_t)geo.dump_row, geo.H, geo.g, geo.NB, geo.chunk_tokens, sl2);
  }
}

template <typename T, int D, int BK, typename PT>
void main_typed(const Geometry& geo, const int32_t* cu, const void* q, const void* k, const void* v,
                const fsa_index& idx, const float* lse, void* st_ws, void* partial, hipStream_t stream) {
  if constexpr (D == 256 && BK == 128) {
    // 128-key blocks at d = 256: two 64-key halves per item (three-pass forward only)
    main_launch<T, 256, 64, PT, false, true>(geo, cu, q, k, v, idx, lse, nullptr, partial, stream);
  } else {
    if (st_ws != nullptr) main_launch<T, D, BK, PT, true>(geo, cu, q, k, v, idx, lse, st_ws, partial, stream);
    else main_launch<T, D, BK, PT, false>(geo, cu, q, k, v, idx, lse, nullptr, partial, stream);
  }
}

// Reduction.  With `st_ws` the one-pass variant, which also writes row_max
// and lse.
template <typename T, typename PT>
void reduce_typed(const Geometry& geo, const fsa_index& idx, const void* partial, void* out, bool local,
                  const void* st_ws, float* row_max, float* lse, hipStream_t stream) {
  const int nvec = geo.g * geo.d / 8;
  const int tpi = nvec < kReduceThreads ? nvec : kReduceThreads;
  const int ipb = kReduceThreads / tpi;
  const int64_t items = (int64_t)geo.N * geo.H;
  const unsigned blocks = (unsigned)((items + ipb - 1) / ipb);
  const PT* const part = static_cast<const PT*>(partial);
  const auto p = index_ptrs(geo, idx);
  const float2* const st = static_cast<const float2*>(st_ws);
  T* const o = static_cast<T*>(out);
  if (st_ws != nullptr) {
    if (local)
      hipLaunchKernelGGL((k_reduce<T, PT, true, true>), dim3(blocks), dim3(kReduceThreads), 0, stream, idx.slot, part,
                         p.loc, o, st, row_max, lse, geo.N, geo.H, geo.g, geo.d, geo.T, tpi, (size_t)0);
    else
      hipLaunchKernelGGL((k_reduce<T, PT, false, true>), dim3(blocks), dim3(kReduceThreads), 0, stream, idx.slot,
                         part, nullptr, o, st, row_max, lse, geo.N, geo.H, geo.g, geo.d, geo.T, tpi, (size_t)0);
  } else if (local && geo.split_halves) {
    // the forward at B_K = 128, d = 256: two rows per slot (no local rows at B_K = 128)
    hipLaunchKernelGGL((k_reduce<T, PT, false, false, true>), dim3(blocks), dim3(kReduceThreads), 0, stream,
                       idx.slot, part, nullptr, o, nullptr, nullptr, nullptr, geo.N, geo.H, geo.g, geo.d, geo.T, tpi,
                       (size_t)geo.split_half_rows * geo.d);
  } else if (local) {
    hipLaunchKernelGGL((k_reduce<T, PT, true, false>), dim3(blocks), dim3(kReduceThreads), 0, stream, idx.slot, part,
                       p.loc, o, nullptr, nullptr, nullptr, geo.N, geo.H, geo.g, geo.d, geo.T, tpi, (size_t)0);
  } else {
    hipLaunchKernelGGL((k_reduce<T, PT, false, false>), dim3(blocks), dim3(kReduceThreads), 0, stream, idx.slot,
                       part, nullptr, o, nullptr, nullptr, nullptr, geo.N, geo.H, geo.g, geo.d, geo.T, tpi,
                       (size_t)0);
  }
}

template <typename T, int BK>
void stats_d(const Geometry& geo, const int32_t* cu, const void* q, const void* k, const fsa_index& idx, void* ws,
             hipStream_t s) {
  switch (geo.d) {
    case 64: stats_typed<T, 64, BK>(geo, cu, q, k, idx, ws, s); break;
    case 128: stats_typed<T, 128, BK>(geo, cu, q, k, idx, ws, s); break;
    default: stats_typed<T, 256, BK>(geo, cu, q, k, idx, ws, s); break;
  }
}

template <typename T, int BK, typename PT>
void main_d(const Geometry& geo, const int32_t* cu, const void* q, const void* k, const void* v, const fsa_index& idx,
            const float* lse, void* st_ws, void* partial, hipStream_t s) {
  switch (geo.d) {
    case 64: main_typed<T, 64, BK, PT>(geo, cu, q, k, v, idx, lse, st_ws, partial, s); break;
    case 128: main_typed<T, 128, BK, PT>(geo, cu, q, k, v, idx, lse, st_ws, partial, s); break;
    default: main_typed<T, 256, BK, PT>(geo, cu, q, k, v, idx, lse, st_ws, partial, s); break;
  }
}

template <typename T, typename PT>
void main_bk(const Geometry& geo, const int32_t* cu, const void* q, const void* k, const void* v,
             const fsa_index& idx, const float* lse, void* st_ws, void* partial, hipStream_t s) {
  if (geo.BK == 64) main_d<T, 64, PT>(geo, cu, q, k, v, idx, lse, st_ws, partial, s);
  else main_d<T, 128, PT>(geo, cu, q, k, v, idx, lse, st_ws, partial, s);
}

}  // namespace

hipError_t launch_stats(const Geometry& geo, const int32_t* cu_dev, const void* q, const void* k,
                        const fsa_index& idx, float* row_max, float* lse, void* ws, hipStream_t stream) {
  if (geo.N == 0) return hipSuccess;
  if (geo.dtype == FSA_DTYPE_BF16) {
    if (geo.BK == 64) stats_d<__bf16, 64>(geo, cu_dev, q, k, idx, ws, stream);
    else stats_d<__bf16, 128>(geo, cu_dev, q, k, idx, ws, stream);
  } else {
    if (geo.BK == 64) stats_d<_Float16, 64>(geo, cu_dev, q, k, idx, ws, stream);
    else stats_d<_Float16, 128>(geo, cu_dev, q, k, idx, ws, stream);
  }
  const auto p = index_ptrs(geo, idx);
  const int64_t n = (int64_t)geo.N * geo.HQ;
  hipLaunchKernelGGL(k_stats_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, idx.slot,
                     static_cast<const float2*>(ws), p.loc, row_max, lse, geo.N, geo.H, geo.g, geo.T);
  return hipGetLastError();
}

hipError_t launch_main(const Geometry& geo, const int32_t* cu_dev, const void* q, const void* k, const void* v,
                       const fsa_index& idx, const float* lse, void* st_ws, void* partial, hipStream_t stream) {
  if (geo.N == 0) return hipSuccess;
  const bool p32 = geo.partial_dtype == FSA_PARTIAL_FP32;
  if (geo.dtype == FSA_DTYPE_BF16) {
    if (p32) main_bk<__bf16, float>(geo, cu_dev, q, k, v, idx, lse, st_ws, partial, stream);
    else main_bk<__bf16, __bf16>(geo, cu_dev, q, k, v, idx, lse, st_ws, partial, stream);
  } else {
    if (p32) main_bk<_Float16, float>(geo, cu_dev, q, k, v, idx, lse, st_ws, partial, stream);
    else main_bk<_Float16, _Float16>(geo, cu_dev, q, k, v, idx, lse, st_ws, partial, stream);
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const Geometry& geo, const fsa_index& idx, const void* partial, void* out, bool local,
                         const void* st_ws, float* row_max, float* lse, hipStream_t stream) {
  if (geo.N == 0) return hipSuccess;
  const bool p32 = geo.partial_dtype == FSA_PARTIAL_FP32;
  if (geo.dtype == FSA_DTYPE_BF16) {
    if (p32) reduce_typed<__bf16, float>(geo, idx, partial, out, local, st_ws, row_max, lse, stream);
    else reduce_typed<__bf16, __bf16>(geo, idx, partial, out, local, st_ws, row_max, lse, stream);
  } else {
    if (p32) reduce_typed<_Float16, float>(geo, idx, partial, out, local, st_ws, row_max, lse, stream);
    else reduce_typed<_Float16, _Float16>(geo, idx, partial, out, local, st_ws, row_max, lse, stream);
  }
  return hipGetLastError();
}

}  // namespace fsa
