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
//   work order bucket sort of the work list by (KV head, first query token)
//
// Integer atomics only count (their result does not depend on order); ranks
// come from per-step bit masks, so the output is bit-exact and deterministic.
#include "fsa_internal.h"

namespace fsa {
namespace {

// ---- seq_table ------------------------------------------------------------
__global__ __launch_bounds__(kBuildThreads) void k_seq_table(const int32_t* __restrict__ cu, int num_seqs,
                                                             int BK, int32_t* __restrict__ gboff,
                                                             int32_t* __restrict__ queue) {
  __shared__ int buf[kBuildThreads];
  const int tid = threadIdx.x;
  for (int i = tid; i < kQueueKinds * kQueueInts; i += kBuildThreads) queue[i] = 0;
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
// grid (ntiles, H); dynamic LDS: win_max ints of histogram, then a staging
// buffer of kHistStage ints for the Sel rows of kHistStage / T tokens at a time
// (the first-occurrence check reads earlier entries of the row from LDS).
constexpr int kHistStage = 4096;

__global__ __launch_bounds__(kBuildThreads) void k_hist(const int32_t* __restrict__ sel,
                                                        const int32_t* __restrict__ cu,
                                                        const int32_t* __restrict__ gboff, int num_seqs, int N,
                                                        int T, int BK, int TT, int ntiles, int NB, int win_max,
                                                        int32_t* __restrict__ tile_hist) {
  extern __shared__ int lds[];
  int* hist = lds;
  int* rows = lds + win_max;
  const int tile = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const TileWindow w = tile_window(cu, gboff, num_seqs, N, TT, BK, tile);
  for (int i = tid; i < w.win; i += kBuildThreads) hist[i] = 0;
  const int chunk = max(1, kHistStage / T);  // tokens per staging round
  for (int c0 = w.t_lo; c0 < w.t_hi; c0 += chunk) {
    const int nt = min(chunk, w.t_hi - c0);
    const int32_t* src = sel + ((size_t)h * N + c0) * T;
    __syncthreads();  // previous round's reads done (and the histogram zeroed)
    for (int i = tid; i < nt * T; i += kBuildThreads) rows[i] = src[i];
    __syncthreads();
    for (int i = tid; i < nt * T; i += kBuildThreads) {
      const int tl = i / T, j = i - tl * T;
      const int t = c0 + tl;
      const int* row = rows + tl * T;
      const int e = row[j];
      if (e < 0) continue;
      const int s = seq_of_token(cu, num_seqs, t);
      if (e > (t - cu[s]) / BK) continue;
      bool dup = false;
      for (int jj = 0; jj < j; ++jj) dup |= (row[jj] == e);
      if (dup) continue;
      atomicAdd(&hist[gboff[s] + e - w.gb_lo], 1);
    }
  }
  __syncthreads();
  int32_t* out = tile_hist + ((size_t)h * ntiles + tile) * NB + w.gb_lo;
  for (int i = tid; i < w.win; i += kBuildThreads) out[i] = hist[i];
}

// ---- tile_scan --------------------------------------------------------------
// Exclusive scan over tiles of each (h, gb) column of the tile histograms ->
// tile bases, totals -> counts.  Tiles outside [tile of the block's first
// token, tile of the sequence's last token] hold no entries for gb and are not
// touched; every tile inside that range has gb in its window, so its entry was
// written by k_hist.  A workgroup takes 16 columns; 16 threads split each
// column's tile range into segments, scan them, and add the segment prefixes.
constexpr int kScanSegs = 16;

__global__ __launch_bounds__(kBuildThreads) void k_tile_scan(int32_t* __restrict__ tile_hist,
                                                             const int32_t* __restrict__ cu,
                                                             const int32_t* __restrict__ gboff, int num_seqs,
                                                             int H, int NB, int BK, int TT, int ntiles,
                                                             int32_t* __restrict__ counts) {
  __shared__ int seg_tot[kBuildThreads / kScanSegs][kScanSegs];
  const int col_local = threadIdx.x / kScanSegs, seg = threadIdx.x % kScanSegs;
  const int idx = blockIdx.x * (kBuildThreads / kScanSegs) + col_local;
  const bool active = idx < H * NB;
  int tau0 = 0, len = 0;
  int32_t* p = tile_hist;
  if (active) {
    const int h = idx / NB, gb = idx - h * NB;
    const int s = seq_of_block(gboff, num_seqs, gb);
    const int bs = cu[s] + (gb - gboff[s]) * BK;
    const int se = cu[s + 1];
    const int t0 = bs / TT, t1 = (se - 1) / TT;
    const int per = (t1 - t0 + kScanSegs) / kScanSegs;
    tau0 = t0 + seg * per;
    len = max(0, min(per, t1 + 1 - tau0));
    p = tile_hist + ((size_t)h * ntiles) * NB + gb;
  }
  int run = 0;
  for (int i = 0; i < len; ++i) run += p[(size_t)(tau0 + i) * NB];
  seg_tot[col_local][seg] = run;
  __syncthreads();
  int base = 0, total = 0;
  for (int k = 0; k < kScanSegs; ++k) {
    const int v = seg_tot[col_local][k];
    if (k < seg) base += v;
    total += v;
  }
  run = base;
  for (int i = 0; i < len; ++i) {
    const int v = p[(size_t)(tau0 + i) * NB];
    p[(size_t)(tau0 + i) * NB] = run;
    run += v;
  }
  if (active && seg == 0) counts[idx] = total;
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
                                                          int4* __restrict__ work, int32_t* __restrict__ nwork,
                                                          int32_t* __restrict__ buckets, int nbuckets) {
  __shared__ int64_t wave_tot[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int b = tid; b < nbuckets; b += kScanThreads) buckets[b] = 0;
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
// Reorders the work list by (KV head, first query token of the chunk) with a
// bucket sort (bucket = token >> shift), so that the items that run together
// on one XCD gather a narrow window of query rows, which then stays in that
// XCD's L2.  Three grid-wide steps: count items per bucket, exclusive scan of
// the bucket counts (one workgroup), place items at their bucket's cursor.
// Within a bucket the order depends on atomics; the order only affects
// scheduling: every item writes its own partial rows and the reduction sums
// in slot order, so all outputs are unchanged.
__device__ __forceinline__ int work_key(const int4& it, const int32_t* __restrict__ qidx,
                                        const int32_t* __restrict__ offsets, int NB, int shift, int nbh) {
  return (it.x / NB) * nbh + (qidx[offsets[it.x] + it.y] >> shift);
}

__global__ __launch_bounds__(kBuildThreads) void k_work_count(const int4* __restrict__ work,
                                                              const int32_t* __restrict__ nwork,
                                                              const int32_t* __restrict__ qidx,
                                                              const int32_t* __restrict__ offsets, int NB, int shift,
                                                              int nbh, int32_t* __restrict__ buckets) {
  const int w = blockIdx.x * kBuildThreads + threadIdx.x;
  if (w >= nwork[0]) return;
  atomicAdd(&buckets[work_key(work[w], qidx, offsets, NB, shift, nbh)], 1);
}

__global__ __launch_bounds__(kScanThreads) void k_bucket_scan(int32_t* __restrict__ buckets, int nbuckets) {
  __shared__ int64_t wave_tot[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t carry = 0;
  for (int base = 0; base < nbuckets; base += kScanThreads * kScanItems) {
    int c[kScanItems];
    int64_t local = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
      const int b = base + tid * kScanItems + i;
      c[i] = b < nbuckets ? buckets[b] : 0;
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
      if (b < nbuckets) buckets[b] = (int32_t)run;
      run += c[i];
    }
    carry += total;
    __syncthreads();
  }
}

__global__ __launch_bounds__(kBuildThreads) void k_work_place(const int4* __restrict__ work,
                                                              const int32_t* __restrict__ nwork,
                                                              const int32_t* __restrict__ qidx,
                                                              const int32_t* __restrict__ offsets, int NB, int shift,
                                                              int nbh, int32_t* __restrict__ buckets,
                                                              int4* __restrict__ work_out) {
  const int w = blockIdx.x * kBuildThreads + threadIdx.x;
  if (w >= nwork[0]) return;
  const int4 it = work[w];
  work_out[atomicAdd(&buckets[work_key(it, qidx, offsets, NB, shift, nbh)], 1)] = it;
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
  int32_t* buckets = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + geo.build_ws_buckets);
  const int M = geo.H * geo.NB;

  hipLaunchKernelGGL(k_seq_table, dim3(1), dim3(kBuildThreads), 0, stream, cu_dev, geo.num_seqs, geo.BK, gboff,
                     reinterpret_cast<int32_t*>(aux + geo.aux_queue));
  if (geo.N > 0) {
    hipLaunchKernelGGL(k_hist, dim3(geo.ntiles, geo.H), dim3(kBuildThreads),
                       (geo.win_max + kHistStage) * sizeof(int), stream, sel, cu_dev, gboff, geo.num_seqs, geo.N, geo.T,
                       geo.BK, geo.tile_tokens, geo.ntiles, geo.NB, geo.win_max, tile_hist);
    constexpr int cols = kBuildThreads / kScanSegs;
    hipLaunchKernelGGL(k_tile_scan, dim3((M + cols - 1) / cols), dim3(kBuildThreads), 0, stream,
                       tile_hist, cu_dev, gboff, geo.num_seqs, geo.H, geo.NB, geo.BK, geo.tile_tokens, geo.ntiles,
                       idx.counts);
  }
  hipLaunchKernelGGL(k_offsets, dim3(1), dim3(kScanThreads), 0, stream, idx.counts, M, geo.chunk_tokens, cu_dev,
                     gboff, geo.num_seqs, geo.NB > 0 ? geo.NB : 1, geo.BK, idx.offsets, work, nwork, buckets,
                     geo.N > 0 ? geo.sort_buckets : 0);
  if (geo.N > 0) {
    int Tp = 1;
    while (Tp < geo.T) Tp <<= 1;
    const int tps = min(32, kBuildThreads / Tp);
    const size_t lds = (size_t)(2 * geo.win_max + kBuildThreads) * sizeof(int);
    hipLaunchKernelGGL(k_scatter, dim3(geo.ntiles, geo.H), dim3(kBuildThreads), lds, stream, sel, cu_dev, gboff,
                       geo.num_seqs, geo.N, geo.T, Tp, tps, geo.BK, geo.tile_tokens, geo.ntiles, geo.NB, geo.win_max,
                       tile_hist, idx.offsets, idx.qidx, idx.slot);
    const unsigned wg = (unsigned)((geo.max_work + kBuildThreads - 1) / kBuildThreads);
    if (wg > 0) {
      hipLaunchKernelGGL(k_work_count, dim3(wg), dim3(kBuildThreads), 0, stream, work, nwork, idx.qidx, idx.offsets,
                         geo.NB, geo.sort_shift, geo.sort_buckets_per_head, buckets);
      hipLaunchKernelGGL(k_bucket_scan, dim3(1), dim3(kScanThreads), 0, stream, buckets, geo.sort_buckets);
      hipLaunchKernelGGL(k_work_place, dim3(wg), dim3(kBuildThreads), 0, stream, work, nwork, idx.qidx, idx.offsets,
                         geo.NB, geo.sort_shift, geo.sort_buckets_per_head, buckets, work_sorted);
    }
  }
  return hipGetLastError();
}

}  // namespace fsa
