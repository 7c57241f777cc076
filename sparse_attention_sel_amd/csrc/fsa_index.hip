// Index precompute on gfx950: Sel[h_K, N, T] -> counts (N_valid), offsets
// (compact output offsets O_i), qidx (query lists I_i) and slot (per-entry
// position), as described in the FSA paper notes, Overall framework and Key
// design 2.  A stable counting sort in four launches:
//
//   seq_table  per-sequence global-block offsets (one workgroup)
//   hist       per (KV head, token tile): LDS histogram of the selected blocks
//   tile_scan  per (KV head, block): exclusive scan of the tile histograms
//              over tiles -> tile bases; totals -> counts
//   offsets    one workgroup: exclusive scan of counts -> offsets, and the
//              work-item list (segment, query chunk) for the attention kernels
//   scatter    per (KV head, token tile): walks its tokens in order and places
//              each selecting entry at offsets + tile base + rank in the tile
//
// Integer atomics only count (their result does not depend on order); ranks
// come from per-step bit masks, so the output is bit-exact and deterministic.
#include "fsa_internal.h"

namespace fsa {
namespace {

// ---- seq_table ------------------------------------------------------------
__global__ __launch_bounds__(kBuildThreads) void k_seq_table(const int32_t* __restrict__ cu, int num_seqs,
                                                             int BK, int32_t* __restrict__ gboff) {
  __shared__ int buf[kBuildThreads];
  const int tid = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < num_seqs; base += kBuildThreads) {
    const int s = base + tid;
    const int nb = s < num_seqs ? (cu[s + 1] - cu[s] + BK - 1) / BK : 0;
    buf[tid] = nb;
    __syncthreads();
    for (int off = 1; off < kBuildThreads; off <<= 1) {
      const int v = tid >= off ? buf[tid - off] : 0;
      __syncthreads();
      buf[tid] += v;
      __syncthreads();
    }
    if (s < num_seqs) gboff[s] = carry + buf[tid] - nb;
    carry += buf[kBuildThreads - 1];
    __syncthreads();
  }
  if (tid == 0) gboff[num_seqs] = carry;
}

struct TileWindow {
  int t_lo, t_hi;  // token range of the tile
  int gb_lo, win;  // global blocks [gb_lo, gb_lo + win) the tile can select
};

__device__ __forceinline__ TileWindow tile_window(const int32_t* __restrict__ cu,
                                                  const int32_t* __restrict__ gboff, int num_seqs, int N,
                                                  int TT, int BK, int tile) {
  TileWindow w;
  w.t_lo = tile * TT;
  w.t_hi = min(w.t_lo + TT, N);
  const int s0 = seq_of_token(cu, num_seqs, w.t_lo);
  const int s1 = seq_of_token(cu, num_seqs, w.t_hi - 1);
  w.gb_lo = gboff[s0];
  w.win = gboff[s1] + (w.t_hi - 1 - cu[s1]) / BK - w.gb_lo + 1;
  return w;
}

// ---- hist -------------------------------------------------------------------
// grid (ntiles, H); dynamic LDS: win_max ints.
__global__ __launch_bounds__(kBuildThreads) void k_hist(const int32_t* __restrict__ sel,
                                                        const int32_t* __restrict__ cu,
                                                        const int32_t* __restrict__ gboff, int num_seqs, int N,
                                                        int T, int BK, int TT, int ntiles, int NB,
                                                        int32_t* __restrict__ tile_hist) {
  extern __shared__ int hist[];
  const int tile = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const TileWindow w = tile_window(cu, gboff, num_seqs, N, TT, BK, tile);
  for (int i = tid; i < w.win; i += kBuildThreads) hist[i] = 0;
  __syncthreads();
  const int n_entries = (w.t_hi - w.t_lo) * T;
  const int32_t* rows = sel + ((size_t)h * N + w.t_lo) * T;
  for (int i = tid; i < n_entries; i += kBuildThreads) {
    const int tl = i / T, j = i - tl * T;
    const int t = w.t_lo + tl;
    const int32_t* row = rows + (size_t)tl * T;
    const int e = row[j];
    if (e < 0) continue;
    const int s = seq_of_token(cu, num_seqs, t);
    if (e > (t - cu[s]) / BK) continue;
    bool dup = false;
    for (int jj = 0; jj < j; ++jj) dup |= (row[jj] == e);
    if (dup) continue;
    atomicAdd(&hist[gboff[s] + e - w.gb_lo], 1);
  }
  __syncthreads();
  int32_t* out = tile_hist + ((size_t)h * ntiles + tile) * NB + w.gb_lo;
  for (int i = tid; i < w.win; i += kBuildThreads) out[i] = hist[i];
}

// ---- tile_scan --------------------------------------------------------------
// One thread per (h, gb).  Tiles outside [tile of the block's first token, tile
// of the sequence's last token] hold no entries for gb and are not touched;
// every tile inside that range has gb in its window, so its entry was written
// by k_hist.
__global__ __launch_bounds__(kBuildThreads) void k_tile_scan(int32_t* __restrict__ tile_hist,
                                                             const int32_t* __restrict__ cu,
                                                             const int32_t* __restrict__ gboff, int num_seqs,
                                                             int H, int NB, int BK, int TT, int ntiles,
                                                             int32_t* __restrict__ counts) {
  const int idx = blockIdx.x * kBuildThreads + threadIdx.x;
  if (idx >= H * NB) return;
  const int h = idx / NB, gb = idx - h * NB;
  const int s = seq_of_block(gboff, num_seqs, gb);
  const int bs = cu[s] + (gb - gboff[s]) * BK;
  const int se = cu[s + 1];
  const int tau0 = bs / TT, tau1 = (se - 1) / TT;
  int32_t* p = tile_hist + ((size_t)h * ntiles) * NB + gb;
  int run = 0;
  int tau = tau0;
  constexpr int U = 8;
  for (; tau + U - 1 <= tau1; tau += U) {
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[(size_t)(tau + u) * NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      p[(size_t)(tau + u) * NB] = run;
      run += v[u];
    }
  }
  for (; tau <= tau1; ++tau) {
    const int v = p[(size_t)tau * NB];
    p[(size_t)tau * NB] = run;
    run += v;
  }
  counts[idx] = run;
}

// ---- offsets + work list ------------------------------------------------------
// One workgroup.  Exclusive scan of counts (-> offsets) and of the number of
// query chunks per segment (-> work-item positions), both in one 64-bit scan:
// high word = pair count, low word = chunk count (neither total reaches 2^32).
__device__ __forceinline__ int64_t wave_inclusive_scan(int64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

constexpr int kScanItems = 4;

__global__ __launch_bounds__(kScanThreads) void k_offsets(const int32_t* __restrict__ counts, int M,
                                                          int CT, const int32_t* __restrict__ cu,
                                                          const int32_t* __restrict__ gboff, int num_seqs,
                                                          int NB, int BK, int32_t* __restrict__ offsets,
                                                          int4* __restrict__ work, int32_t* __restrict__ nwork) {
  __shared__ int64_t wave_tot[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t carry = 0;
  for (int base = 0; base < M; base += kScanThreads * kScanItems) {
    int c[kScanItems];
    int64_t local = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
      const int f = base + tid * kScanItems + i;
      c[i] = f < M ? counts[f] : 0;
      local += ((int64_t)c[i] << 32) + (c[i] + CT - 1) / CT;
    }
    const int64_t incl = wave_inclusive_scan(local);
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int64_t before = 0, total = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) {
      const int64_t t = wave_tot[w];
      if (w < wave) before += t;
      total += t;
    }
    int64_t run = carry + before + incl - local;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
      const int f = base + tid * kScanItems + i;
      if (f < M) {
        offsets[f] = (int32_t)(run >> 32);
        const int nch = (c[i] + CT - 1) / CT;
        if (nch > 0) {
          const int gb = f % NB;
          const int s = seq_of_block(gboff, num_seqs, gb);
          const int bs = cu[s] + (gb - gboff[s]) * BK;
          const int se = cu[s + 1];
          int4* wp = work + (uint32_t)run;
          for (int ch = 0; ch < nch; ++ch) wp[ch] = make_int4(f, ch * CT, bs, se);
        }
        run += ((int64_t)c[i] << 32) + (c[i] + CT - 1) / CT;
      }
    }
    carry += total;
    __syncthreads();
  }
  if (tid == 0) {
    offsets[M] = (int32_t)(carry >> 32);
    nwork[0] = (int32_t)(uint32_t)carry;
    nwork[1] = (int32_t)(carry >> 32);
  }
}

// ---- scatter ------------------------------------------------------------------
// grid (ntiles, H).  LDS: cursor[win_max], mark[win_max], row buffer.
// Each step takes TPS consecutive tokens of the tile, one lane per entry
// (lane = token_in_step * Tp + j).  A block's lanes set bit token_in_step in
// mark[block]; a lane's rank among the step's selectors of its block is the
// number of lower bits, so ranks follow token order.  The highest selector
// then advances the block's cursor.
__global__ __launch_bounds__(kBuildThreads) void k_scatter(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cu, const int32_t* __restrict__ gboff,
    int num_seqs, int N, int T, int Tp, int TPS, int BK, int TT, int ntiles, int NB, int win_max,
    const int32_t* __restrict__ tile_base, const int32_t* __restrict__ offsets, int32_t* __restrict__ qidx,
    int32_t* __restrict__ slot) {
  extern __shared__ int lds[];
  int* cursor = lds;
  unsigned* mark = reinterpret_cast<unsigned*>(lds + win_max);
  int* rowbuf = lds + 2 * win_max;
  const int tile = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const TileWindow w = tile_window(cu, gboff, num_seqs, N, TT, BK, tile);
  {
    const int32_t* tb = tile_base + ((size_t)h * ntiles + tile) * NB + w.gb_lo;
    const int32_t* of = offsets + (size_t)h * NB + w.gb_lo;
    for (int i = tid; i < w.win; i += kBuildThreads) {
      cursor[i] = of[i] + tb[i];
      mark[i] = 0u;
    }
  }
  __syncthreads();
  const int my_tok = tid / Tp, my_j = tid - my_tok * Tp;
  for (int t0 = w.t_lo; t0 < w.t_hi; t0 += TPS) {
    const int t = t0 + my_tok;
    const bool active = my_tok < TPS && my_j < T && t < w.t_hi;
    int e = -1;
    if (active) e = sel[((size_t)h * N + t) * T + my_j];
    rowbuf[tid] = e;
    __syncthreads();
    bool valid = false;
    int wi = 0;
    if (active && e >= 0) {
      const int s = seq_of_token(cu, num_seqs, t);
      if (e <= (t - cu[s]) / BK) {
        bool dup = false;
        for (int jj = 0; jj < my_j; ++jj) dup |= (rowbuf[my_tok * Tp + jj] == e);
        if (!dup) {
          valid = true;
          wi = gboff[s] + e - w.gb_lo;
          atomicOr(&mark[wi], 1u << my_tok);
        }
      }
    }
    __syncthreads();
    unsigned m = 0;
    if (active) {
      int pos = -1;
      if (valid) {
        m = mark[wi];
        pos = cursor[wi] + __popc(m & ((1u << my_tok) - 1u));
        qidx[pos] = t;
      }
      slot[((size_t)h * N + t) * T + my_j] = pos;
    }
    __syncthreads();
    if (valid && (m >> my_tok) == 1u) {
      cursor[wi] += __popc(m);
      mark[wi] = 0u;
    }
    __syncthreads();
  }
}

// ---- work order -------------------------------------------------------------
// One workgroup.  Reorders the work list by (KV head, first query token of the
// chunk) with a bucket sort (bucket = token >> shift), so that the items that
// run together on one XCD gather a narrow window of query rows, which then
// stays in that XCD's L2.  Within a bucket the order depends on atomics; the
// order only affects scheduling: every item writes its own partial rows and
// the reduction sums in slot order, so all outputs are unchanged.
__global__ __launch_bounds__(kScanThreads) void k_work_sort(const int4* __restrict__ work_in,
                                                            const int32_t* __restrict__ nwork,
                                                            const int32_t* __restrict__ qidx,
                                                            const int32_t* __restrict__ offsets, int NB, int shift,
                                                            int nbh, int nbuckets, int4* __restrict__ work_out) {
  extern __shared__ int cnt[];
  __shared__ int64_t wave_tot[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int W = nwork[0];
  for (int i = tid; i < nbuckets; i += kScanThreads) cnt[i] = 0;
  __syncthreads();
  auto key_of = [&](const int4& it) {
    const int h = it.x / NB;
    return h * nbh + (qidx[offsets[it.x] + it.y] >> shift);
  };
  for (int w = tid; w < W; w += kScanThreads) atomicAdd(&cnt[key_of(work_in[w])], 1);
  __syncthreads();
  // exclusive scan of the bucket counts, kScanItems buckets per thread per pass
  int64_t carry = 0;
  for (int base = 0; base < nbuckets; base += kScanThreads * kScanItems) {
    int c[kScanItems];
    int64_t local = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
      const int b = base + tid * kScanItems + i;
      c[i] = b < nbuckets ? cnt[b] : 0;
      local += c[i];
    }
    const int64_t incl = wave_inclusive_scan(local);
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int64_t before = 0, total = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) {
      if (w < wave) before += wave_tot[w];
      total += wave_tot[w];
    }
    int64_t run = carry + before + incl - local;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
      const int b = base + tid * kScanItems + i;
      if (b < nbuckets) cnt[b] = (int)run;
      run += c[i];
    }
    carry += total;
    __syncthreads();
  }
  for (int w = tid; w < W; w += kScanThreads) {
    const int4 it = work_in[w];
    work_out[atomicAdd(&cnt[key_of(it)], 1)] = it;
  }
}

}  // namespace

hipError_t launch_build_index(const Geometry& geo, const int32_t* cu_dev, const int32_t* sel,
                              const fsa_index& idx, void* ws, hipStream_t stream) {
  char* aux = static_cast<char*>(idx.aux);
  int32_t* gboff = reinterpret_cast<int32_t*>(aux + geo.aux_seq_gboff);
  int32_t* nwork = reinterpret_cast<int32_t*>(aux + geo.aux_nwork);
  int4* work = reinterpret_cast<int4*>(aux + geo.aux_work);
  int4* work_sorted = reinterpret_cast<int4*>(aux + geo.aux_work_sorted);
  int32_t* tile_hist = static_cast<int32_t*>(ws);
  const int M = geo.H * geo.NB;

  hipLaunchKernelGGL(k_seq_table, dim3(1), dim3(kBuildThreads), 0, stream, cu_dev, geo.num_seqs, geo.BK, gboff);
  if (geo.N > 0) {
    hipLaunchKernelGGL(k_hist, dim3(geo.ntiles, geo.H), dim3(kBuildThreads), geo.win_max * sizeof(int), stream,
                       sel, cu_dev, gboff, geo.num_seqs, geo.N, geo.T, geo.BK, geo.tile_tokens, geo.ntiles, geo.NB,
                       tile_hist);
    hipLaunchKernelGGL(k_tile_scan, dim3((M + kBuildThreads - 1) / kBuildThreads), dim3(kBuildThreads), 0, stream,
                       tile_hist, cu_dev, gboff, geo.num_seqs, geo.H, geo.NB, geo.BK, geo.tile_tokens, geo.ntiles,
                       idx.counts);
  }
  hipLaunchKernelGGL(k_offsets, dim3(1), dim3(kScanThreads), 0, stream, idx.counts, M, geo.chunk_tokens, cu_dev,
                     gboff, geo.num_seqs, geo.NB > 0 ? geo.NB : 1, geo.BK, idx.offsets, work, nwork);
  if (geo.N > 0) {
    int Tp = 1;
    while (Tp < geo.T) Tp <<= 1;
    const int tps = min(32, kBuildThreads / Tp);
    const size_t lds = (size_t)(2 * geo.win_max + kBuildThreads) * sizeof(int);
    hipLaunchKernelGGL(k_scatter, dim3(geo.ntiles, geo.H), dim3(kBuildThreads), lds, stream, sel, cu_dev, gboff,
                       geo.num_seqs, geo.N, geo.T, Tp, tps, geo.BK, geo.tile_tokens, geo.ntiles, geo.NB, geo.win_max,
                       tile_hist, idx.offsets, idx.qidx, idx.slot);
    hipLaunchKernelGGL(k_work_sort, dim3(1), dim3(kScanThreads), geo.sort_buckets * sizeof(int), stream, work, nwork,
                       idx.qidx, idx.offsets, geo.NB, geo.sort_shift, geo.sort_buckets_per_head, geo.sort_buckets,
                       work_sorted);
  }
  return hipGetLastError();
}

}  // namespace fsa
