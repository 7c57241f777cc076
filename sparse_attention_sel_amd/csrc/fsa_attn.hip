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
//
// Work items come from the index builder: (segment f, first query of the
// chunk, block start token, sequence end).  Rows of a chunk are
// (query, group head) pairs, query-major: row = i * g + j.
//
// MFMA tiling (v_mfma_f32_32x32x16, wave64).  A 32-row query tile meets the
// block's keys as S^T (keys x rows) so that each lane ends up owning one query
// row: lane l holds column l % 32 of S^T.  The same registers, cast to 16-bit,
// are the B operand of O^T = V^T P^T, so P never leaves the registers.  The
// head dimension is the contraction of S^T; lane half hl = l / 32 supplies
// d in [hl * D/2, (hl + 1) * D/2), a permutation of the contraction index that
// A (K from LDS) and B (Q from HBM) share, so each lane reads one contiguous
// half row of Q.  V is staged transposed (Vt[d][key]) with the keys of every
// 16-key group permuted so that the 8 keys a lane contributes to one MFMA are
// adjacent in LDS.
#include "fsa_internal.h"

namespace fsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type zero8() {
  typename Vec8<T>::type z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (T)0.0f;
  return z;
}

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type load8(const T* p) {
  return *reinterpret_cast<const typename Vec8<T>::type*>(p);
}

template <typename T>
__device__ __forceinline__ uint16_t bits16(T x) {
  return __builtin_bit_cast(uint16_t, x);
}

// LDS layouts (elements).  K: [BK][D + 8]; Vt: [D][BK + 8].  The 8-element
// pads spread the 16-byte reads of 32 consecutive rows over all banks.
template <int D>
constexpr int k_ld() { return D + 8; }
template <int BK>
constexpr int vt_ld() { return BK + 8; }

// Position of key w (within its 16-key group) in the permuted Vt row: lane half
// hl contributes keys {4hl..4hl+3, 8+4hl..8+4hl+3} as MFMA elements e = 0..7.
__device__ __forceinline__ int vt_pos(int key) {
  const int w = key & 15;
  return (key & ~15) + ((w >> 2) & 1) * 8 + (w >> 3) * 4 + (w & 3);
}

template <typename T, int D, int BK>
__device__ __forceinline__ void stage_k(T* __restrict__ Ks, const T* __restrict__ k, int bs, int nkeys, int H,
                                        int h) {
  constexpr int C8 = D / 8;
  for (int vi = threadIdx.x; vi < BK * C8; vi += kAttnThreads) {
    const int key = vi / C8, c = vi - key * C8;
    typename Vec8<T>::type val = zero8<T>();
    if (key < nkeys) val = load8(k + ((size_t)(bs + key) * H + h) * D + c * 8);
    *reinterpret_cast<typename Vec8<T>::type*>(Ks + key * k_ld<D>() + c * 8) = val;
  }
}

template <typename T, int D, int BK>
__device__ __forceinline__ void stage_vt(T* __restrict__ Vt, const T* __restrict__ v, int bs, int nkeys, int H,
                                         int h) {
  constexpr int KP = BK / 2;
  for (int vi = threadIdx.x; vi < KP * (D / 8); vi += kAttnThreads) {
    const int c = vi / KP, kp = vi - c * KP;
    const int key = 2 * kp;
    typename Vec8<T>::type a = zero8<T>(), b = zero8<T>();
    if (key < nkeys) a = load8(v + ((size_t)(bs + key) * H + h) * D + c * 8);
    if (key + 1 < nkeys) b = load8(v + ((size_t)(bs + key + 1) * H + h) * D + c * 8);
    const int pos = vt_pos(key);  // even; key + 1 lands at pos + 1
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t packed = (uint32_t)bits16(a[i]) | ((uint32_t)bits16(b[i]) << 16);
      *reinterpret_cast<uint32_t*>(Vt + (c * 8 + i) * vt_ld<BK>() + pos) = packed;
    }
  }
}

// S^T tile: s[kt][r] = (K Q^T)[key = kt*32 + 8*(r/4) + 4*hl + r%4][row = l%32].
template <typename T, int D, int BK>
__device__ __forceinline__ void qk_tile(const T* __restrict__ Ks, const typename Vec8<T>::type* qf, int lr, int hl,
                                        f32x16* s) {
  constexpr int KS = D / 16, KT = BK / 32;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    f32x16 acc = {};
    const T* kp = Ks + (kt * 32 + lr) * k_ld<D>() + hl * (D / 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = mfma32(load8(kp + ks * 8), qf[ks], acc);
    s[kt] = acc;
  }
}

template <typename T, int D>
__device__ __forceinline__ void load_q_half(const T* __restrict__ q, int t, int hq, int HQ, int hl, bool valid,
                                            typename Vec8<T>::type* qf) {
  constexpr int KS = D / 16;
  const T* qp = q + ((size_t)t * HQ + hq) * D + hl * (D / 2);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = valid ? load8(qp + ks * 8) : zero8<T>();
}

struct Item {
  int h, ntok, pair0, bs, nkeys;
};

__device__ __forceinline__ Item read_item(const int4* __restrict__ work, const int32_t* __restrict__ counts,
                                          const int32_t* __restrict__ offsets, int wi, int NB, int CT, int BK) {
  const int4 it = work[wi];
  Item r;
  r.h = it.x / NB;
  r.ntok = min(CT, counts[it.x] - it.y);
  r.pair0 = offsets[it.x] + it.y;
  r.bs = it.z;
  r.nkeys = min(BK, it.w - it.z);
  return r;
}

// One query row of a 32-row tile, as seen by lane l (row = tile*32 + l%32):
// its position ti in the chunk's query list, its group head j and its token.
struct Row {
  int row, ti, j, t;
  bool valid;
};

__device__ __forceinline__ Row row_of(int tile, int lr, int nrows, int g, const int32_t* __restrict__ qidx,
                                      int pair0) {
  Row r;
  r.row = tile * 32 + lr;
  r.valid = r.row < nrows;
  r.ti = r.row / g;
  r.j = r.row - r.ti * g;
  r.t = r.valid ? qidx[pair0 + r.ti] : 0;
  return r;
}

// Work-item order.  Workgroup i runs on XCD i % 8 (round-robin dispatch); XCD x
// takes the contiguous range [x * per, (x + 1) * per) of the work list, in
// order, so that neighbouring blocks (which share most of their query rows)
// meet in the same L2.  The grid is a multiple of 8 covering 8 * per items.
__device__ __forceinline__ int xcd_item(int nwork_total) {
  const int per = (nwork_total + 7) >> 3;
  const int i = blockIdx.x;
  const int k = i >> 3;
  const int wi = (i & 7) * per + k;
  return (k < per && wi < nwork_total) ? wi : -1;
}

// Each wave walks the tiles wave, wave + 4, ...; the Q half-row and lse of the
// next tile and the token of the tile after it are loaded while the current
// tile computes, so the gathers overlap the MFMA work.
constexpr int kWaves = kAttnThreads / 64;

// Waves per SIMD the register budget aims for: two (<= 256 registers) where
// the tile state fits, one (<= 512) for the wide head dim / long blocks.
template <int D, int BK>
constexpr int attn_waves_per_eu() { return (D >= 256 || (D >= 128 && BK >= 128)) ? 1 : 2; }

// ---- statistics -------------------------------------------------------------
template <typename T, int D, int BK>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(attn_waves_per_eu<D, BK>()))) void k_stats(
    const T* __restrict__ q, const T* __restrict__ k, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ qidx, const int4* __restrict__ work,
    const int32_t* __restrict__ nwork, float2* __restrict__ st, int H, int g, int NB, int CT, float scale_log2) {
  using V8 = typename Vec8<T>::type;
  constexpr int KS = D / 16, KT = BK / 32;
  __shared__ __attribute__((aligned(16))) T Ks[BK * k_ld<D>()];
  const int wi = xcd_item(nwork[0]);
  if (wi < 0) return;
  const Item it = read_item(work, counts, offsets, wi, NB, CT, BK);
  stage_k<T, D, BK>(Ks, k, it.bs, it.nkeys, H, it.h);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, hl = lane >> 5;
  const int HQ = H * g, nrows = it.ntok * g, ntile = (nrows + 31) / 32;
  Row r0 = row_of(wave, lr, nrows, g, qidx, it.pair0);
  Row r1 = row_of(wave + kWaves, lr, nrows, g, qidx, it.pair0);
  V8 qf[KS];
  load_q_half<T, D>(q, r0.t, it.h * g + r0.j, HQ, hl, r0.valid, qf);
  __syncthreads();
  for (int tile = wave; tile < ntile; tile += kWaves) {
    V8 qn[KS];
    load_q_half<T, D>(q, r1.t, it.h * g + r1.j, HQ, hl, r1.valid, qn);
    const Row r2 = row_of(tile + 2 * kWaves, lr, nrows, g, qidx, it.pair0);

    f32x16 s[KT];
    qk_tile<T, D, BK>(Ks, qf, lr, hl, s);
    const int lim = r0.valid ? r0.t - it.bs : -1;  // key (block-local) visible iff key <= lim
    float m = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (key <= lim) m = fmaxf(m, s[kt][r] * scale_log2);
      }
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    float l = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (key <= lim) l += __builtin_amdgcn_exp2f(s[kt][r] * scale_log2 - m);
      }
    l += __shfl_xor(l, 32, 64);
    if (r0.valid && hl == 0) st[(size_t)it.pair0 * g + r0.row] = make_float2(m, l);

#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = qn[ks];
    r0 = r1;
    r1 = r2;
  }
}

// One thread per (token, query head): merge the per-block (max, sum) pairs of
// the token's selecting entries, in slot order, into the row max and lse
// (stored in natural-log units).  Slots are read 8 at a time and the pairs
// loaded unconditionally (row 0 stands in for empty slots) so that the loads
// are independent.
__global__ __launch_bounds__(256) void k_stats_combine(const int32_t* __restrict__ slot,
                                                       const float2* __restrict__ st, float* __restrict__ row_max,
                                                       float* __restrict__ lse, int N, int H, int g, int T) {
  const int HQ = H * g;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)N * HQ) return;
  const int t = (int)(idx / HQ), hq = (int)(idx - (int64_t)t * HQ);
  const int h = hq / g, j = hq - h * g;
  const int32_t* sl = slot + ((size_t)h * N + t) * T;
  float M = -INFINITY, L = 0.f;
  for (int j0 = 0; j0 < T; j0 += 8) {
    int sv[8];
    float2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) sv[u] = j0 + u < T ? sl[j0 + u] : -1;
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = st[(size_t)max(sv[u], 0) * g + j];
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
// head-dim values of one row, 8 values apart, which would make 8-byte stores
// 256 bytes apart.  Each wave instead passes its 32 x D tile through a private
// LDS buffer, 64 columns at a time, and writes it back row-contiguously with
// 16 bytes per lane: every store instruction covers whole 128-byte lines.
// Partial rows are written once and read once by the reduction, so the
// stores are non-temporal (they should not evict the gathered Q rows).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kStageCols = 64;

template <typename PT>
constexpr int stage_pitch() { return kStageCols + 16 / (int)sizeof(PT); }

template <typename PT>
__device__ __forceinline__ void stage_write4(PT* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void stage_write4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}
template <>
__device__ __forceinline__ void stage_write4<__bf16>(__bf16* p, float a, float b, float c, float d) {
  typedef __bf16 v4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, v4{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d});
}
template <>
__device__ __forceinline__ void stage_write4<_Float16>(_Float16* p, float a, float b, float c, float d) {
  typedef _Float16 v4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, v4{(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d});
}

// o[mt][r] holds O^T[d = mt*32 + 8*(r/4) + 4*hl + r%4][row = lane % 32].
// Writes rows [0, rows) of the tile to dst (row-major, pitch D).
template <typename PT, int D>
__device__ __forceinline__ void store_tile(PT* __restrict__ stage, const f32x16* o, int lane, int rows,
                                           PT* __restrict__ dst) {
  constexpr int P = stage_pitch<PT>();
  constexpr int EPL = 16 / (int)sizeof(PT);  // elements per 16-byte lane store
  constexpr int LPR = kStageCols / EPL;      // lanes per staged row
  constexpr int RPI = 64 / LPR;              // rows per store instruction
  const int lr = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int c = 0; c < D / kStageCols; ++c) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16& acc = o[2 * c + m];
        stage_write4<PT>(stage + lr * P + m * 32 + 8 * q4 + 4 * hl, acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2],
                         acc[4 * q4 + 3]);
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = i * RPI + lane / LPR, col = (lane % LPR) * EPL;
      const u32x4 val = *reinterpret_cast<const u32x4*>(stage + row * P + col);
      if (row < rows) __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(dst + (size_t)row * D + c * kStageCols + col));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

template <typename T, int D, int BK, typename PT>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(attn_waves_per_eu<D, BK>()))) void k_main(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ qidx, const int4* __restrict__ work,
    const int32_t* __restrict__ nwork, const float* __restrict__ lse, PT* __restrict__ partial, int H, int g,
    int NB, int CT, float scale_log2) {
  using V8 = typename Vec8<T>::type;
  constexpr int KS = D / 16, KT = BK / 32, KK = BK / 16, MT = D / 32;
  __shared__ __attribute__((aligned(16))) T Ks[BK * k_ld<D>()];
  __shared__ __attribute__((aligned(16))) T Vt[D * vt_ld<BK>()];
  __shared__ __attribute__((aligned(16))) PT Ot[kWaves * 32 * stage_pitch<PT>()];
  const int wi = xcd_item(nwork[0]);
  if (wi < 0) return;
  const Item it = read_item(work, counts, offsets, wi, NB, CT, BK);
  stage_k<T, D, BK>(Ks, k, it.bs, it.nkeys, H, it.h);
  stage_vt<T, D, BK>(Vt, v, it.bs, it.nkeys, H, it.h);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, hl = lane >> 5;
  const int HQ = H * g, nrows = it.ntok * g, ntile = (nrows + 31) / 32;
  Row r0 = row_of(wave, lr, nrows, g, qidx, it.pair0);
  Row r1 = row_of(wave + kWaves, lr, nrows, g, qidx, it.pair0);
  V8 qf[KS];
  load_q_half<T, D>(q, r0.t, it.h * g + r0.j, HQ, hl, r0.valid, qf);
  float l2 = r0.valid ? lse[(size_t)r0.t * HQ + it.h * g + r0.j] * kLog2e : 0.f;
  __syncthreads();
  for (int tile = wave; tile < ntile; tile += kWaves) {
    V8 qn[KS];
    load_q_half<T, D>(q, r1.t, it.h * g + r1.j, HQ, hl, r1.valid, qn);
    const float l2n = r1.valid ? lse[(size_t)r1.t * HQ + it.h * g + r1.j] * kLog2e : 0.f;
    const Row r2 = row_of(tile + 2 * kWaves, lr, nrows, g, qidx, it.pair0);

    f32x16 s[KT];
    qk_tile<T, D, BK>(Ks, qf, lr, hl, s);
    const int lim = r0.valid ? r0.t - it.bs : -1;
    V8 pb[KK];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        const float p = key <= lim ? __builtin_amdgcn_exp2f(s[kt][r] * scale_log2 - l2) : 0.f;
        pb[2 * kt + (r >> 3)][r & 7] = (T)p;
      }
    f32x16 o[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const V8 a = load8(Vt + (mt * 32 + lr) * vt_ld<BK>() + kk * 16 + hl * 8);
        o[mt] = mfma32(a, pb[kk], o[mt]);
      }
    }
    store_tile<PT, D>(Ot + wave * 32 * stage_pitch<PT>(), o, lane, min(32, nrows - tile * 32),
                      partial + ((size_t)it.pair0 * g + (size_t)tile * 32) * D);

#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = qn[ks];
    l2 = l2n;
    r0 = r1;
    r1 = r2;
  }
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
// g*D outputs.  Slots are taken 8 at a time; the 8 partial loads are issued
// together (row 0 stands in for empty slots) and summed in slot order.
template <typename T, typename PT>
__global__ __launch_bounds__(kReduceThreads) void k_reduce(const int32_t* __restrict__ slot,
                                                           const PT* __restrict__ partial, T* __restrict__ out,
                                                           int N, int H, int g, int D, int Tn, int TPI) {
  const int ipb = kReduceThreads / TPI;
  const int local = threadIdx.x / TPI;
  if (local >= ipb) return;
  const int64_t item = (int64_t)blockIdx.x * ipb + local;
  if (item >= (int64_t)N * H) return;
  const int t = (int)(item / H), h = (int)(item - (int64_t)t * H);
  const int sub = threadIdx.x - local * TPI;
  const int GD = g * D, nvec = GD / 8;
  const int32_t* sl = slot + ((size_t)h * N + t) * Tn;
  T* dst = out + ((size_t)t * H + h) * GD;
  for (int vec = sub; vec < nvec; vec += TPI) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < Tn; j0 += 8) {
      int sv[8];
      typename Part8<PT>::type x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) sv[u] = j0 + u < Tn ? sl[j0 + u] : -1;
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = Part8<PT>::load(partial + (size_t)max(sv[u], 0) * GD + vec * 8);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += sv[u] >= 0 ? Part8<PT>::at(x[u], i) : 0.f;
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
};

inline Ptrs<int> index_ptrs(const Geometry& geo, const fsa_index& idx) {
  const char* aux = static_cast<const char*>(idx.aux);
  return Ptrs<int>{idx.counts, idx.offsets, idx.qidx, reinterpret_cast<const int4*>(aux + geo.aux_work),
                   reinterpret_cast<const int32_t*>(aux + geo.aux_nwork)};
}

template <typename T, int D, int BK>
void stats_typed(const Geometry& geo, const void* q, const void* k, const fsa_index& idx, float2* st,
                 hipStream_t stream) {
  const auto p = index_ptrs(geo, idx);
  const float sl2 = geo.scale * kLog2e;
  hipLaunchKernelGGL((k_stats<T, D, BK>), dim3((unsigned)((geo.max_work + 7) / 8 * 8)), dim3(kAttnThreads), 0, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), p.counts, p.offsets, p.qidx, p.work, p.nwork,
                     st, geo.H, geo.g, geo.NB, geo.chunk_tokens, sl2);
}

template <typename T, int D, int BK, typename PT>
void main_typed(const Geometry& geo, const void* q, const void* k, const void* v, const fsa_index& idx,
                const float* lse, void* partial, hipStream_t stream) {
  const auto p = index_ptrs(geo, idx);
  const float sl2 = geo.scale * kLog2e;
  hipLaunchKernelGGL((k_main<T, D, BK, PT>), dim3((unsigned)((geo.max_work + 7) / 8 * 8)), dim3(kAttnThreads), 0, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), p.counts,
                     p.offsets, p.qidx, p.work, p.nwork, lse, static_cast<PT*>(partial), geo.H, geo.g, geo.NB,
                     geo.chunk_tokens, sl2);
}

template <typename T, typename PT>
void reduce_typed(const Geometry& geo, const fsa_index& idx, const void* partial, void* out, hipStream_t stream) {
  const int nvec = geo.g * geo.d / 8;
  const int tpi = nvec < kReduceThreads ? nvec : kReduceThreads;
  const int ipb = kReduceThreads / tpi;
  const int64_t items = (int64_t)geo.N * geo.H;
  const unsigned blocks = (unsigned)((items + ipb - 1) / ipb);
  hipLaunchKernelGGL((k_reduce<T, PT>), dim3(blocks), dim3(kReduceThreads), 0, stream, idx.slot,
                     static_cast<const PT*>(partial), static_cast<T*>(out), geo.N, geo.H, geo.g, geo.d, geo.T, tpi);
}

template <typename T, int BK>
void stats_d(const Geometry& geo, const void* q, const void* k, const fsa_index& idx, float2* st,
             hipStream_t s) {
  switch (geo.d) {
    case 64: stats_typed<T, 64, BK>(geo, q, k, idx, st, s); break;
    case 128: stats_typed<T, 128, BK>(geo, q, k, idx, st, s); break;
    default:
      if constexpr (BK == 64) stats_typed<T, 256, BK>(geo, q, k, idx, st, s);
      break;
  }
}

template <typename T, int BK, typename PT>
void main_d(const Geometry& geo, const void* q, const void* k, const void* v, const fsa_index& idx,
            const float* lse, void* partial, hipStream_t s) {
  switch (geo.d) {
    case 64: main_typed<T, 64, BK, PT>(geo, q, k, v, idx, lse, partial, s); break;
    case 128: main_typed<T, 128, BK, PT>(geo, q, k, v, idx, lse, partial, s); break;
    default:
      if constexpr (BK == 64) main_typed<T, 256, BK, PT>(geo, q, k, v, idx, lse, partial, s);
      break;
  }
}

template <typename T, typename PT>
void main_bk(const Geometry& geo, const void* q, const void* k, const void* v, const fsa_index& idx,
             const float* lse, void* partial, hipStream_t s) {
  if (geo.BK == 64) main_d<T, 64, PT>(geo, q, k, v, idx, lse, partial, s);
  else main_d<T, 128, PT>(geo, q, k, v, idx, lse, partial, s);
}

}  // namespace

hipError_t launch_stats(const Geometry& geo, const void* q, const void* k, const fsa_index& idx, float* row_max,
                        float* lse, void* ws, hipStream_t stream) {
  if (geo.N == 0) return hipSuccess;
  float2* st = static_cast<float2*>(ws);
  if (geo.max_work > 0) {
    if (geo.dtype == FSA_DTYPE_BF16) {
      if (geo.BK == 64) stats_d<__bf16, 64>(geo, q, k, idx, st, stream);
      else stats_d<__bf16, 128>(geo, q, k, idx, st, stream);
    } else {
      if (geo.BK == 64) stats_d<_Float16, 64>(geo, q, k, idx, st, stream);
      else stats_d<_Float16, 128>(geo, q, k, idx, st, stream);
    }
  }
  const int64_t n = (int64_t)geo.N * geo.HQ;
  hipLaunchKernelGGL(k_stats_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, idx.slot, st, row_max,
                     lse, geo.N, geo.H, geo.g, geo.T);
  return hipGetLastError();
}

hipError_t launch_main(const Geometry& geo, const void* q, const void* k, const void* v, const fsa_index& idx,
                       const float* lse, void* partial, hipStream_t stream) {
  if (geo.N == 0 || geo.max_work == 0) return hipSuccess;
  const bool p32 = geo.partial_dtype == FSA_PARTIAL_FP32;
  if (geo.dtype == FSA_DTYPE_BF16) {
    if (p32) main_bk<__bf16, float>(geo, q, k, v, idx, lse, partial, stream);
    else main_bk<__bf16, __bf16>(geo, q, k, v, idx, lse, partial, stream);
  } else {
    if (p32) main_bk<_Float16, float>(geo, q, k, v, idx, lse, partial, stream);
    else main_bk<_Float16, _Float16>(geo, q, k, v, idx, lse, partial, stream);
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const Geometry& geo, const fsa_index& idx, const void* partial, void* out,
                         hipStream_t stream) {
  if (geo.N == 0) return hipSuccess;
  const bool p32 = geo.partial_dtype == FSA_PARTIAL_FP32;
  if (geo.dtype == FSA_DTYPE_BF16) {
    if (p32) reduce_typed<__bf16, float>(geo, idx, partial, out, stream);
    else reduce_typed<__bf16, __bf16>(geo, idx, partial, out, stream);
  } else {
    if (p32) reduce_typed<_Float16, float>(geo, idx, partial, out, stream);
    else reduce_typed<_Float16, _Float16>(geo, idx, partial, out, stream);
  }
  return hipGetLastError();
}

}  // namespace fsa
