// Query-outer selected attention: the vanilla NSA loop order that FSA
// replaces (FSA paper notes, Background and motivation and Key design 1;
// README, Method).  It is the baseline the KV-block-outer path is measured
// against and a second, independent GPU implementation of the same forward.
//
// One wave per (query token, KV head), head-major.  The g <= 16 query heads
// of the group (fsa_problem limits g to 16) are the rows of a 16-row MFMA tile
// (v_mfma_f32_16x16x32), padded with zero rows when g < 16: this padding is
// the waste the KV-block-outer order removes for small g.  The wave walks the
// token's selected blocks (valid entries, first occurrence) with an online
// softmax: S^T = K Q^T over the block's keys (K rows read from global memory
// as the A operand), running max / sum update, then O^T += V^T P^T with the
// block's V staged transposed in the wave's own LDS.  Output and log-sum-exp
// are written directly: no index, partial buffer or reduction is involved.
//
// 16x16x32 layouts (wave64): lane l supplies A[l % 16][8 * (l / 16) + e] and
// B[8 * (l / 16) + e][l % 16] (e = 0..7) and receives
// C[4 * (l / 16) + r][l % 16] (r = 0..3).  In S^T (keys x rows) lane l owns
// query row l % 16 and keys 4 * (l / 16) + r of every 16-key tile.
#include <math.h>

#include "fsa_internal.h"

namespace fsa {
namespace {

constexpr float kNsaLog2e = 1.4426950408889634f;
constexpr float kNsaLn2 = 0.6931471805599453f;
constexpr int kNsaWaves = 4;

typedef float f32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type nsa_ld8(const T* p) {
  return *reinterpret_cast<const typename Vec8<T>::type*>(p);
}

template <typename T>
__device__ __forceinline__ uint32_t nsa_bits(T x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, x);
}

// Within each 32-key step, key w is stored at position
// 8 * ((w / 4) % 4) + 4 * (w / 16) + w % 4, so that the 8 keys lane half u
// contracts over ({4u..4u+3} and {16+4u..16+4u+3}, the keys its S^T
// fragments hold) are adjacent.  Even/odd key pairs stay adjacent.
__device__ __forceinline__ int nsa_vt_pos(int key) {
  const int w = key & 31;
  return (key & ~31) + ((w >> 2) & 3) * 8 + (w >> 4) * 4 + (w & 3);
}

template <int BK>
constexpr int nsa_vt_ld() {
  return BK + 8;
}

// Mask of the valid, first-occurrence Sel entries j0 .. j0+63 of one row
// (bit i = entry j0 + i).  Valid: 0 <= e <= own block; first occurrence: no
// earlier entry of the row holds the same block.
__device__ __forceinline__ unsigned long long nsa_keep_mask(const int32_t* __restrict__ row, int Tn, int j0,
                                                            int own, int lane) {
  const int j = j0 + lane;
  const int e = j < Tn ? row[j] : -1;
  bool ok = e >= 0 && e <= own;
  const int n = min(64, Tn - j0);
  for (int i = 0; i < n; ++i) {
    const int ei = __shfl(e, i, 64);
    ok = ok && !(i < lane && ei == e);
  }
  for (int jp = 0; jp < j0; ++jp) ok = ok && row[jp] != e;
  return __ballot(ok);
}

// Walk over the kept Sel entries of one row in order: the current 64-entry
// group and its remaining keep bits.
struct NsaCursor {
  int j0;
  unsigned long long kb;
};

// Next kept entry index, or -1 after the last (wave-uniform).
__device__ __forceinline__ int nsa_next(NsaCursor& c, const int32_t* __restrict__ row, int Tn, int own, int lane) {
  while (c.kb == 0) {
    c.j0 += 64;
    if (c.j0 >= Tn) return -1;
    c.kb = nsa_keep_mask(row, Tn, c.j0, own, lane);
  }
  const int jl = __builtin_ctzll(c.kb);
  c.kb &= c.kb - 1;
  return c.j0 + jl;
}

// One block's K (in the A-operand layout of S^T = K Q^T) and V (the lane's
// share of the key pairs of the transposed staging) in registers.  Key
// indices are clamped to the sequence (nkeys keys exist from bs on); clamped
// keys are masked by causality.
template <typename T, int D, int BK>
struct NsaKV {
  using V8 = typename Vec8<T>::type;
  static constexpr int KS = D / 32, KT = BK / 16;
  static constexpr int VI = (BK / 2) * (D / 8) / 64;  // key pairs x 8-column chunks per lane
  static_assert((BK / 2) * (D / 8) % 64 == 0, "whole iterations");
  V8 kf[KT][KS];
  V8 va[VI], vb[VI];
  int bs;

  __device__ __forceinline__ void load_k(const T* __restrict__ k, int nkeys, int H, int h, int lane) {
    const int lr = lane & 15, hu = lane >> 4;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const T* kp = k + ((size_t)(bs + min(kt * 16 + lr, nkeys - 1)) * H + h) * D + 8 * hu;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[kt][ks] = nsa_ld8(kp + ks * 32);
    }
  }

  __device__ __forceinline__ void load_v(const T* __restrict__ v, int nkeys, int H, int h, int lane) {
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int vi = lane + 64 * i;
      const int c = vi / (BK / 2), key = 2 * (vi - c * (BK / 2));
      va[i] = nsa_ld8(v + ((size_t)(bs + min(key, nkeys - 1)) * H + h) * D + c * 8);
      vb[i] = nsa_ld8(v + ((size_t)(bs + min(key + 1, nkeys - 1)) * H + h) * D + c * 8);
    }
  }

  __device__ __forceinline__ void put_vt(T* __restrict__ Vt, int lane) const {
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int vi = lane + 64 * i;
      const int c = vi / (BK / 2), key = 2 * (vi - c * (BK / 2));
      const int pos = nsa_vt_pos(key);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint32_t*>(Vt + (c * 8 + e) * nsa_vt_ld<BK>() + pos) =
            nsa_bits(va[i][e]) | (nsa_bits(vb[i][e]) << 16);
    }
  }
};

// V block -> the wave's LDS, transposed (Vt[d][pos(key)], key pairs packed),
// one key pair and 8-column chunk per lane and iteration.
template <typename T, int D, int BK>
__device__ __forceinline__ void nsa_stage_vt(const T* __restrict__ v, int bs, int nkeys, int H, int h, int lane,
                                             T* __restrict__ Vt) {
  using V8 = typename Vec8<T>::type;
  for (int vi = lane; vi < (BK / 2) * (D / 8); vi += 64) {
    const int c = vi / (BK / 2), key = 2 * (vi - c * (BK / 2));
    const V8 a = nsa_ld8(v + ((size_t)(bs + min(key, nkeys - 1)) * H + h) * D + c * 8);
    const V8 b = nsa_ld8(v + ((size_t)(bs + min(key + 1, nkeys - 1)) * H + h) * D + c * 8);
    const int pos = nsa_vt_pos(key);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<uint32_t*>(Vt + (c * 8 + e) * nsa_vt_ld<BK>() + pos) = nsa_bits(a[e]) | (nsa_bits(b[e]) << 16);
  }
}

// The 32 keys [k0, k0 + 32) of a V block as register pairs (the lane's share
// of the transposed staging of one 32-key step), and their LDS writes.
template <typename T, int D>
struct NsaVHalf {
  using V8 = typename Vec8<T>::type;
  static constexpr int VI = 16 * (D / 8) / 64;  // key pairs x 8-column chunks per lane
  V8 va[VI], vb[VI];
  __device__ __forceinline__ void load(const T* __restrict__ v, int bs, int k0, int nkeys, int H, int h, int lane) {
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int vi = lane + 64 * i;
      const int c = vi / 16, key = k0 + 2 * (vi - c * 16);
      va[i] = nsa_ld8(v + ((size_t)(bs + min(key, nkeys - 1)) * H + h) * D + c * 8);
      vb[i] = nsa_ld8(v + ((size_t)(bs + min(key + 1, nkeys - 1)) * H + h) * D + c * 8);
    }
  }
  template <int LDH>
  __device__ __forceinline__ void put(T* __restrict__ Vt, int lane) const {
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int vi = lane + 64 * i;
      const int c = vi / 16, key = 2 * (vi - c * 16);
      const int pos = nsa_vt_pos(key);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint32_t*>(Vt + (c * 8 + e) * LDH + pos) = nsa_bits(va[i][e]) | (nsa_bits(vb[i][e]) << 16);
    }
  }
};

template <int D, int BK>
constexpr bool nsa_halves() { return D <= 128 && BK == 64; }

template <typename T, int D, int BK>
__global__ __launch_bounds__(kNsaWaves * 64) void k_nsa(const T* __restrict__ q, const T* __restrict__ k,
                                                        const T* __restrict__ v, const int32_t* __restrict__ sel,
                                                        const int32_t* __restrict__ cu, int num_seqs, int N, int H,
                                                        int g, int Tn, float scale_log2, T* __restrict__ out,
                                                        float* __restrict__ lse_out) {
  using V8 = typename Vec8<T>::type;
  typedef T V4 __attribute__((ext_vector_type(4)));
  constexpr int KS = D / 32;   // contraction steps of S^T over d
  constexpr int KT = BK / 16;  // 16-key tiles of a block
  constexpr int MT = D / 16;   // 16-column tiles of O^T
  constexpr int KK = BK / 32;  // 32-key contraction steps of O^T
  // With HALVES (64-key blocks, d <= 128) the block's V goes through the
  // wave's LDS 32 keys at a time: both halves are loaded at the block start,
  // the first staged before S, the second (held in registers) after the
  // first half's PV (15.2 -> 14.3 ms at 64K tokens; forcing three waves per
  // SIMD with the smaller LDS tile gained nothing more).
  constexpr bool HALVES = nsa_halves<D, BK>();
  constexpr int LD = HALVES ? 32 + 8 : nsa_vt_ld<BK>();
  __shared__ __attribute__((aligned(16))) T Vt_all[kNsaWaves * D * LD];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t item = (int64_t)blockIdx.x * kNsaWaves + wave;
  if (item >= (int64_t)N * H) return;  // wave-uniform; the kernel has no workgroup barrier
  // head-major: neighbouring waves take consecutive tokens of one KV head,
  // which select mostly the same blocks, so their K / V reads share the caches
  const int h = (int)(item / N), t = (int)(item - (int64_t)h * N);
  const int lr = lane & 15, hu = lane >> 4;
  const int HQ = H * g;
  const bool row_ok = lr < g;  // row lr is query head h*g + lr
  T* const Vt = Vt_all + wave * D * LD;

  const int s = seq_of_token(cu, num_seqs, t);
  const int c0 = cu[s], c1 = cu[s + 1];
  const int own = (t - c0) / BK;
  const int32_t* const srow = sel + ((size_t)h * N + t) * Tn;

  // Q^T as the B operand: column lr = query head h*g + lr, rows d = ks*32 + 8*hu + e.
  V8 qb[KS];
  {
    const T* qp = q + ((size_t)t * HQ + h * g + (row_ok ? lr : 0)) * D + 8 * hu;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      V8 x = {};
      if (row_ok) x = nsa_ld8(qp + ks * 32);
      qb[ks] = x;
    }
  }

  float m_run = -INFINITY, l_run = 0.f;  // row lr, base-2 units of the scaled score
  f32x4 o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = f32x4{};

  // Blocks in Sel order.  Per block: V is loaded and staged transposed in
  // the wave's LDS, then K is loaded in the A-operand layout next to the
  // MFMAs.  For d = 256 the K loads are issued together with V (one memory
  // round trip per block), which measured faster there; for the smaller head
  // dims the later K loads measured faster.
  NsaCursor cur{0, nsa_keep_mask(srow, Tn, 0, own, lane)};
  for (int j = nsa_next(cur, srow, Tn, own, lane); j >= 0; j = nsa_next(cur, srow, Tn, own, lane)) {
    NsaKV<T, D, BK> cb;
    cb.bs = c0 + srow[j] * BK;
    const int nkeys = min(BK, c1 - cb.bs);
    const int lim = t - cb.bs;  // block-local key visible iff key <= lim
    NsaVHalf<T, D> vh;
    if constexpr (D >= 256) {
      cb.load_k(k, nkeys, H, h, lane);
      cb.load_v(v, nkeys, H, h, lane);
      cb.put_vt(Vt, lane);
    } else if constexpr (HALVES) {
      NsaVHalf<T, D> v0;
      v0.load(v, cb.bs, 0, nkeys, H, h, lane);
      vh.load(v, cb.bs, 32, nkeys, H, h, lane);
      v0.template put<LD>(Vt, lane);
    } else {
      nsa_stage_vt<T, D, BK>(v, cb.bs, nkeys, H, h, lane, Vt);
    }

    // S^T = K Q^T: lane supplies K[key kt*16 + lr][ks*32 + 8*hu + e] (for
    // d < 256 loaded here, next to the MFMAs that consume it).
    f32x4 st[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const T* kp = k + ((size_t)(cb.bs + min(kt * 16 + lr, nkeys - 1)) * H + h) * D + 8 * hu;
      f32x4 acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma16(D >= 256 ? cb.kf[kt][ks] : nsa_ld8(kp + ks * 32), qb[ks], acc);
      st[kt] = acc;
    }

    // Online softmax update for row lr over keys kt*16 + 4*hu + r.
    float mb = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (kt * 16 + 4 * hu + r <= lim) mb = fmaxf(mb, st[kt][r]);
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    // key 0 of a valid block is always visible, so mb is finite
    const float m_new = fmaxf(m_run, mb * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float ls = 0.f;
    V8 pb[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      f32x8 x;
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const int kt = 2 * kk + (e8 >> 2), r = e8 & 3;
        const int key = kt * 16 + 4 * hu + r;
        const float p = key <= lim ? __builtin_amdgcn_exp2f(fmaf(st[kt][r], scale_log2, -m_new)) : 0.f;
        ls += p;
        x[e8] = p;
      }
      pb[kk] = __builtin_convertvector(x, V8);
    }
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    l_run = l_run * alpha + ls;
    m_run = m_new;

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O^T = alpha O^T + V^T P^T: lane supplies Vt[mt*16 + lr][kk*32 + 8*hu + e].
    if constexpr (HALVES) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[mt] = mfma16(nsa_ld8(Vt + (mt * 16 + lr) * LD + hu * 8), pb[0], o[mt] * alpha);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      vh.template put<LD>(Vt, lane);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[mt] = mfma16(nsa_ld8(Vt + (mt * 16 + lr) * LD + hu * 8), pb[1], o[mt]);
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc = o[mt] * alpha;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) acc = mfma16(nsa_ld8(Vt + (mt * 16 + lr) * LD + kk * 32 + hu * 8), pb[kk], acc);
        o[mt] = acc;
      }
    }
    // the next block's staging writes come after these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // O = O^T / l for rows lr < g (lane holds d = mt*16 + 4*hu + r); lse = (m + log2 l) ln 2.
  if (row_ok) {
    const size_t row = (size_t)t * HQ + h * g + lr;
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    T* op = out + row * D + 4 * hu;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<V4*>(op + mt * 16) = __builtin_convertvector(o[mt] * inv, V4);
    if (hu == 0) lse_out[row] = l_run > 0.f ? (m_run + __builtin_log2f(l_run)) * kNsaLn2 : -INFINITY;
  }
}

template <typename T, int D, int BK>
hipError_t nsa_typed(const Geometry& geo, const int32_t* cu_dev, const void* q, const void* k, const void* v,
                     const int32_t* sel, void* out, float* lse, hipStream_t stream) {
  const int64_t items = (int64_t)geo.N * geo.H;
  const int64_t blocks = (items + kNsaWaves - 1) / kNsaWaves;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_nsa<T, D, BK>), dim3((unsigned)blocks), dim3(kNsaWaves * 64), 0, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), sel, cu_dev,
                     geo.num_seqs, geo.N, geo.H, geo.g, geo.T, geo.scale * kNsaLog2e, static_cast<T*>(out), lse);
  return hipGetLastError();
}

template <typename T>
hipError_t nsa_dispatch(const Geometry& geo, const int32_t* cu_dev, const void* q, const void* k, const void* v,
                        const int32_t* sel, void* out, float* lse, hipStream_t s) {
  if (geo.BK == 64) {
    if (geo.d == 64) return nsa_typed<T, 64, 64>(geo, cu_dev, q, k, v, sel, out, lse, s);
    if (geo.d == 128) return nsa_typed<T, 128, 64>(geo, cu_dev, q, k, v, sel, out, lse, s);
    return nsa_typed<T, 256, 64>(geo, cu_dev, q, k, v, sel, out, lse, s);
  }
  if (geo.d == 64) return nsa_typed<T, 64, 128>(geo, cu_dev, q, k, v, sel, out, lse, s);
  return nsa_typed<T, 128, 128>(geo, cu_dev, q, k, v, sel, out, lse, s);
}

}  // namespace

hipError_t launch_nsa(const Geometry& geo, const int32_t* cu_dev, const void* q, const void* k, const void* v,
                      const int32_t* sel, void* out, float* lse, hipStream_t stream) {
  if (geo.N == 0) return hipSuccess;
  if (geo.dtype == FSA_DTYPE_BF16) return nsa_dispatch<__bf16>(geo, cu_dev, q, k, v, sel, out, lse, stream);
  return nsa_dispatch<_Float16>(geo, cu_dev, q, k, v, sel, out, lse, stream);
}

}  // namespace fsa
