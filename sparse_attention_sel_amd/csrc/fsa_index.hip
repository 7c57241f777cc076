// Index precompute on gfx950: Sel[h_K, N, T] -> counts (N_valid), offsets
// (compact output offsets O_i), qidx (query lists I_i) and slot (per-entry
// position), as described in the FSA paper notes, Overall framework and Key
// design 2.  A stable counting sort in seven launches:
//
//   seq_table  per-sequence global-block offsets (one workgroup)
//   hist       per (KV head, token tile): LDS histogram of the selected blocks
//   tile_scan  per (KV head, block): exclusive scan of the tile histograms
//              over tiles -> tile bases; totals -> counts
//   offsets    one workgroup: exclusive scan of counts -> offsets, and the
//              work-item list (segment, query chunk) for the attention kernels
//   scatter    per (KV head, token tile): walks its tokens in order and places
//              each selecting entry at offsets + tile base + rank in the tile;
//              the entries that start a work item count it into its bucket
//   work order bucket sort of the work list by (KV head, first query token)
//
// Integer atomics only count (their result does not depend on order); ranks
// come from per-step bit masks, so the output is bit-exact and deterministic.
#include <algorithm>

#include "fsa_internal.h"

namespace fsa {
namespace {

// ---- seq_table ------------------------------------------------------------
// Every workgroup clears its share of the per-segment local counts (which
// k_hist accumulates); workgroup 0 also builds the per-sequence block offsets.
__global__ __launch_bounds__(kBuildThreads) void k_seq_table(const int32_t* __restrict__ cu, int num_seqs,
                                                             int BK, int32_t* __restrict__ gboff,
                                                             int32_t* __restrict__ nloc, int M) {
  __shared__ int buf[kBuildThreads];
  const int tid = threadIdx.x;
  for (int i = blockIdx.x * kBuildThreads + tid; i < M; i += gridDim.x * kBuildThreads) nloc[i] = 0;
  if (blockIdx.x != 0) return;
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
// grid (ntiles, H).  The tile's tokens are taken in rounds of up to
// kRoundTokens tokens (kHistStage Sel ints): the round's Sel rows and, per
// token, its own block and the window slot of its sequence's first block are
// staged in LDS (one parallel lookup per token); one thread per token then
// turns its row into window slots (validity, first-occurrence dedupe) and
// counts them into the LDS histogram over the tile's block window.
// Besides the tile histogram it writes each token's local word and adds, for
// every block e >= 1, the number of local entries (tokens of blocks e and e + 1
// selecting e) to nloc; those are the first entries of the block's query list.
// LDS (ints): hist[win_max], lhist[win_max], rows[kHistStage + kRoundTokens]
// (padded stride), own, base and lword [kRoundTokens] each.
constexpr int kHistStage = 4096;
constexpr int kRoundTokens = 512;

__device__ __forceinline__ int round_tokens(int T) { return max(1, min(kRoundTokens, kHistStage / T)); }

// Staged Sel rows use an odd stride (T, or T + 1 for even T), so that the
// threads of a wave reading one row each hit distinct LDS banks.
__device__ __forceinline__ int row_stride(int T) { return T | 1; }

// Copies the Sel rows of tokens c0 .. c0 + nt - 1 (contiguous, T ints each)
// into rows at the padded stride.  i / T by a float reciprocal: exact here
// (i < 4096, T <= 256, so the quotient's fraction is at least 0.5 / T away
// from an integer, far beyond float rounding).
__device__ __forceinline__ void stage_rows(const int32_t* __restrict__ src, int nt, int T, int* __restrict__ rows) {
  const int RS = row_stride(T);
  const float inv = 1.0f / (float)T;
  for (int i = threadIdx.x; i < nt * T; i += blockDim.x) {
    const int tl = (int)(((float)i + 0.5f) * inv);
    rows[tl * RS + (i - tl * T)] = src[i];
  }
}

// Own block and window slot of the first block of the sequence of tokens
// t0 + i, i < nt (one thread per token).
__device__ __forceinline__ void token_info(const int32_t* __restrict__ cu, const int32_t* __restrict__ gboff,
                                           int num_seqs, int BK, int gb_lo, int t0, int nt, int* __restrict__ own,
                                           int* __restrict__ base) {
  for (int i = threadIdx.x; i < nt; i += blockDim.x) {
    const int t = t0 + i;
    const int s = seq_of_token(cu, num_seqs, t);
    own[i] = (t - cu[s]) / BK;
    base[i] = gboff[s] - gb_lo;
  }
}

// Replaces each staged Sel entry of tokens tl < nt by the window slot of the
// block it selects (base + e), or -1 when it selects nothing (negative, past
// the own block, or a repeat of an earlier entry of its row).  One thread per
// token row: up to 16 entries in registers; longer rows are visited from the
// last entry to the first, so the earlier entries the repeat test reads are
// still block indices.
__device__ __forceinline__ void entry_slots(int* __restrict__ rows, const int* __restrict__ own,
                                            const int* __restrict__ base, int nt, int T) {
  for (int tl = threadIdx.x; tl < nt; tl += blockDim.x) {
    int* row = rows + tl * row_stride(T);
    const int ob = own[tl], bs = base[tl];
    if (T <= 16) {
      int e[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) e[j] = j < T ? row[j] : -1;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        bool dup = false;
#pragma unroll
        for (int jj = 0; jj < j; ++jj) dup |= e[jj] == e[j];
        if (j < T) row[j] = e[j] >= 0 && e[j] <= ob && !dup ? bs + e[j] : -1;
      }
    } else {
      for (int j = T - 1; j >= 0; --j) {
        const int e = row[j];
        bool dup = false;
        for (int jj = 0; jj < j; ++jj) dup |= row[jj] == e;
        row[j] = e >= 0 && e <= ob && !dup ? bs + e : -1;
      }
    }
  }
}

__global__ __launch_bounds__(kBuildThreads) void k_hist(const int32_t* __restrict__ sel,
                                                        const int32_t* __restrict__ cu,
                                                        const int32_t* __restrict__ gboff, int num_seqs, int N,
                                                        int T, int BK, int TT, int ntiles, int NB, int win_max,
                                                        int32_t* __restrict__ tile_hist, int32_t* __restrict__ loc,
                                                        int32_t* __restrict__ nloc, int use_local) {
  extern __shared__ int lds[];
  int* hist = lds;
  int* lhist = hist + win_max;
  int* rows = lhist + win_max;
  int* own = rows + kHistStage + kRoundTokens;
  int* base = own + kRoundTokens;
  unsigned* lword = reinterpret_cast<unsigned*>(base + kRoundTokens);
  const int tile = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const TileWindow w = tile_window(cu, gboff, num_seqs, N, TT, BK, tile);
  for (int i = tid; i < w.win; i += kBuildThreads) hist[i] = lhist[i] = 0;
  const int chunk = round_tokens(T);
  for (int c0 = w.t_lo; c0 < w.t_hi; c0 += chunk) {
    const int nt = min(chunk, w.t_hi - c0);
    const int32_t* src = sel + ((size_t)h * N + c0) * T;
    __syncthreads();  // previous round's reads done (and the histograms zeroed)
    stage_rows(src, nt, T, rows);
    token_info(cu, gboff, num_seqs, BK, w.gb_lo, c0, nt, own, base);
    __syncthreads();
    entry_slots(rows, own, base, nt, T);
    __syncthreads();
    // one thread per token: histogram its selected blocks, build its local word
    for (int tl = tid; tl < nt; tl += kBuildThreads) {
      const int* row = rows + tl * row_stride(T);
      const int ob = own[tl], bs = base[tl];
      unsigned word = 0u;
      for (int j = 0; j < T; ++j) {
        const int wi = row[j];
        if (wi < 0) continue;
        atomicAdd(&hist[wi], 1);
        const int kind = use_local ? local_kind(wi - bs, ob) : -1;
        if (kind >= 0) {
          word |= (unsigned)(j + 1) << (9 * kind);
          if (kind < 2 && wi > bs) atomicAdd(&lhist[wi], 1);
        }
      }
      lword[tl] = word;
    }
    __syncthreads();
    for (int i = tid; i < nt; i += kBuildThreads) loc[(size_t)h * N + c0 + i] = (int32_t)lword[i];
  }
  __syncthreads();
  int32_t* out = tile_hist + ((size_t)h * ntiles + tile) * NB + w.gb_lo;
  for (int i = tid; i < w.win; i += kBuildThreads) {
    out[i] = hist[i];
    if (lhist[i] != 0) atomicAdd(&nloc[(size_t)h * NB + w.gb_lo + i], lhist[i]);
  }
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

// ---- offsets + work-list bases ------------------------------------------------
// One workgroup.  Exclusive scan of counts (-> offsets) and of the number of
// query chunks per segment (-> the segment's first work item, cb_full), both
// in one 64-bit scan: high word = pair count, low word = chunk count (neither
// total reaches 2^32).  A second scan gives the forward list's bases (cb_fwd):
// its chunks of a segment start after the segment's local entries.  The items
// themselves are derived from these bases by the work-order kernels.
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

// Local entries at the head of segment f with `count` entries: all of them for
// the first block of a sequence (every query's first block), else the count
// k_hist gathered (queries of the block and of the next one); none when the
// problem does not use the local path.
__device__ __forceinline__ int segment_local(int f, int count, const int32_t* __restrict__ nloc,
                                             const int32_t* __restrict__ gboff, int num_seqs, int NB,
                                             int use_local) {
  if (count == 0 || !use_local) return 0;
  const int gb = f % NB;
  const int s = seq_of_block(gboff, num_seqs, gb);
  return gb == gboff[s] ? count : min(count, nloc[f]);
}

__global__ __launch_bounds__(kScanThreads) void k_offsets(const int32_t* __restrict__ counts,
                                                          const int32_t* __restrict__ nloc, int M, int CT,
                                                          const int32_t* __restrict__ gboff, int num_seqs,
                                                          int NB, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ cb_full,
                                                          int32_t* __restrict__ cb_fwd, int32_t* __restrict__ nwork,
                                                          int32_t* __restrict__ buckets, int nbuckets, int use_local) {
  __shared__ int64_t wave_tot[2][kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int b = tid; b < 2 * nbuckets; b += kScanThreads) buckets[b] = 0;
  int64_t carry = 0, carry_f = 0;
  for (int base = 0; base < M; base += kScanThreads * kScanItems) {
    int c[kScanItems], cf[kScanItems];
    int64_t local = 0, local_f = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
      const int f = base + tid * kScanItems + i;
      c[i] = f < M ? counts[f] : 0;
      cf[i] = c[i] - segment_local(f, c[i], nloc, gboff, num_seqs, NB, use_local);
      local += ((int64_t)c[i] << 32) + (c[i] + CT - 1) / CT;
      local_f += (cf[i] + CT - 1) / CT;
    }
    const int64_t incl = wave_inclusive_scan(local);
    const int64_t incl_f = wave_inclusive_scan(local_f);
    if (lane == 63) {
      wave_tot[0][wave] = incl;
      wave_tot[1][wave] = incl_f;
    }
    __syncthreads();
    int64_t before = 0, total = 0, before_f = 0, total_f = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) {
      const int64_t t = wave_tot[0][w], tf = wave_tot[1][w];
      if (w < wave) {
        before += t;
        before_f += tf;
      }
      total += t;
      total_f += tf;
    }
    int64_t run = carry + before + incl - local;
    int64_t run_f = carry_f + before_f + incl_f - local_f;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
      const int f = base + tid * kScanItems + i;
      if (f < M) {
        offsets[f] = (int32_t)(run >> 32);
        cb_full[f] = (int32_t)(uint32_t)run;
        cb_fwd[f] = (int32_t)run_f;
        run += ((int64_t)c[i] << 32) + (c[i] + CT - 1) / CT;
        run_f += (cf[i] + CT - 1) / CT;
      }
    }
    carry += total;
    carry_f += total_f;
    __syncthreads();
  }
  if (tid == 0) {
    offsets[M] = (int32_t)(carry >> 32);
    cb_full[M] = (int32_t)(uint32_t)carry;
    cb_fwd[M] = (int32_t)carry_f;
    nwork[0] = (int32_t)(uint32_t)carry;
    nwork[1] = (int32_t)(carry >> 32);
    nwork[2] = (int32_t)carry_f;
    nwork[3] = 0;
  }
}

// ---- scatter ------------------------------------------------------------------
// grid (ntiles, H).  The tile's tokens in rounds as in k_hist (Sel rows turned
// into window slots in LDS), each round in steps of TPS consecutive tokens,
// one lane per entry (lane = token_in_step * Tp + j).  A block's lanes set bit
// token_in_step in mark[block]; a lane's rank among the step's selectors of
// its block is the number of lower bits, so ranks follow token order.  The
// highest selector then advances the block's cursor.
// Work items start at the chunk boundaries of each segment's query list (rank
// a multiple of CT in the full list, CT past the local head in the forward
// list), so the entry placed there counts its item into the work-order bucket
// of its (KV head, token bucket) for k_work_place.
// LDS (ints): cursor, two mark sets, lstart, segoff [win_max] each,
// rows[kHistStage + kRoundTokens] (padded stride), own and base
// [kRoundTokens] each.
constexpr int kScatterThreads = 512;  // 32 tokens per step at T = 16

__global__ __launch_bounds__(kScatterThreads) void k_scatter(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cu, const int32_t* __restrict__ gboff,
    int num_seqs, int N, int T, int Tp, int TPS, int BK, int TT, int ntiles, int NB, int win_max,
    const int32_t* __restrict__ tile_base, const int32_t* __restrict__ offsets, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ nloc, int use_local, int CT, int shift, int nbh, int nbuckets,
    int32_t* __restrict__ buckets, int32_t* __restrict__ qidx, int32_t* __restrict__ slot) {
  extern __shared__ int lds[];
  int* cursor = lds;  // next rank within the segment
  unsigned* mark = reinterpret_cast<unsigned*>(cursor + win_max);  // two sets, by step parity
  int* lstart = reinterpret_cast<int*>(mark + 2 * win_max);        // local entries at the segment's head
  int* segoff = lstart + win_max;                                   // offsets[f]
  int* rows = segoff + win_max;
  int* own = rows + kHistStage + kRoundTokens;
  int* base = own + kRoundTokens;
  const int tile = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const TileWindow w = tile_window(cu, gboff, num_seqs, N, TT, BK, tile);
  {
    const int32_t* tb = tile_base + ((size_t)h * ntiles + tile) * NB + w.gb_lo;
    for (int i = tid; i < w.win; i += kScatterThreads) {
      const int f = h * NB + w.gb_lo + i;
      cursor[i] = tb[i];
      mark[i] = mark[win_max + i] = 0u;
      segoff[i] = offsets[f];
      lstart[i] = segment_local(f, counts[f], nloc, gboff, num_seqs, NB, use_local);
    }
  }
  const int RS = row_stride(T);
  const int my_tok = tid / Tp, my_j = tid - my_tok * Tp;
  const int chunk = max(TPS, round_tokens(T));
  for (int c0 = w.t_lo; c0 < w.t_hi; c0 += chunk) {
    const int nt = min(chunk, w.t_hi - c0);
    __syncthreads();  // previous round's reads done (and the cursors initialised)
    stage_rows(sel + ((size_t)h * N + c0) * T, nt, T, rows);
    token_info(cu, gboff, num_seqs, BK, w.gb_lo, c0, nt, own, base);
    __syncthreads();
    entry_slots(rows, own, base, nt, T);
    __syncthreads();
    // Step k sets bits in mark set k % 2 (atomicOr), reads them after a
    // barrier, and its highest selectors advance the cursors and clear their
    // marks after the next barrier; step k + 1 uses the other set, and step
    // k + 2 reaches this set only after step k + 1's first barrier, which all
    // of step k's clears precede.
    for (int s0 = 0, par = 0; s0 < nt; s0 += TPS, par ^= 1) {
      unsigned* mk = mark + par * win_max;
      const int tl = s0 + my_tok;
      const bool active = my_tok < TPS && my_j < T && tl < nt;
      const int wi = active ? rows[tl * RS + my_j] : -1;
      const bool valid = wi >= 0;
      if (valid) atomicOr(&mk[wi], 1u << my_tok);
      __syncthreads();
      unsigned m = 0;
      if (active) {
        int pos = -1;
        if (valid) {
          m = mk[wi];
          const int r = cursor[wi] + __popc(m & ((1u << my_tok) - 1u));
          const int t = c0 + tl;
          pos = segoff[wi] + r;
          qidx[pos] = t;
          const int key = h * nbh + (t >> shift);
          if (r % CT == 0) atomicAdd(&buckets[key], 1);
          const int l0 = lstart[wi];
          if (r >= l0 && (r - l0) % CT == 0) atomicAdd(&buckets[nbuckets + key], 1);
        }
        slot[((size_t)h * N + c0 + tl) * T + my_j] = pos;
      }
      __syncthreads();
      if (valid && (m >> my_tok) == 1u) {
        cursor[wi] += __popc(m);
        mk[wi] = 0u;
      }
    }
  }
}

// ---- work order -------------------------------------------------------------
// Reorders the work list by (KV head, first query token of the chunk) with a
// bucket sort (bucket = token >> shift), so that the items that run together
// on one XCD gather a narrow window of query rows, which then stays in that
// XCD's L2.  Three steps: count items per bucket (in k_scatter, by the entry
// that starts each item), exclusive scan of the bucket counts (one
// workgroup), place items at their bucket's cursor.
// Within a bucket the order depends on atomics; the order only affects
// scheduling: every item writes its own partial rows and the reduction sums
// in slot order, so all outputs are unchanged.
__device__ __forceinline__ int work_key(const int4& it, const int32_t* __restrict__ qidx,
                                        const int32_t* __restrict__ offsets, int NB, int shift, int nbh) {
  return (it.x / NB) * nbh + (qidx[offsets[it.x] + it.y] >> shift);
}

// Item w of the two lists: the full list's items come first (nwork[0] of them,
// buckets [0, nbuckets)), then the forward list's (nwork[2], buckets
// [nbuckets, 2 nbuckets)), so one scan of both bucket arrays places the
// forward list right after the full one.  An item's segment is the last f with
// cb[f] <= its index in the list (binary search); its chunk starts at
// (index - cb[f]) * CT queries, after the local entries in the forward list.
struct ListArgs {
  const int32_t* counts;
  const int32_t* nloc;
  const int32_t* cb_full;
  const int32_t* cb_fwd;
  const int32_t* nwork;
  const int32_t* cu;
  const int32_t* gboff;
  int num_seqs, M, NB, BK, CT, nbuckets, use_local;
};

__device__ __forceinline__ bool list_item(const ListArgs& a, int w, int4* it, int* bucket0) {
  const int nfull = a.nwork[0];
  const bool fwd = w >= nfull;
  if (fwd) w -= nfull;
  if (w >= (fwd ? a.nwork[2] : nfull)) return false;
  const int32_t* cb = fwd ? a.cb_fwd : a.cb_full;
  int lo = 0, hi = a.M;  // last f in [lo, hi) with cb[f] <= w
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cb[mid] <= w) lo = mid; else hi = mid;
  }
  const int f = lo;
  const int gb = f % a.NB;
  const int s = seq_of_block(a.gboff, a.num_seqs, gb);
  const int first =
      fwd ? segment_local(f, a.counts[f], a.nloc, a.gboff, a.num_seqs, a.NB, a.use_local) : 0;
  *it = make_int4(f, first + (w - cb[f]) * a.CT, a.cu[s] + (gb - a.gboff[s]) * a.BK, a.cu[s + 1]);
  *bucket0 = fwd ? a.nbuckets : 0;
  return true;
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

__global__ __launch_bounds__(kBuildThreads) void k_work_place(ListArgs a, const int32_t* __restrict__ qidx,
                                                              const int32_t* __restrict__ offsets, int shift, int nbh,
                                                              int32_t* __restrict__ buckets,
                                                              int4* __restrict__ work_out) {
  int4 it;
  int b0;
  if (!list_item(a, blockIdx.x * kBuildThreads + threadIdx.x, &it, &b0)) return;
  work_out[atomicAdd(&buckets[b0 + work_key(it, qidx, offsets, a.NB, shift, nbh)], 1)] = it;
}

}  // namespace

hipError_t launch_build_index(const Geometry& geo, const int32_t* cu_dev, const int32_t* sel,
                              const fsa_index& idx, void* ws, hipStream_t stream) {
  char* aux = static_cast<char*>(idx.aux);
  int32_t* gboff = reinterpret_cast<int32_t*>(aux + geo.aux_seq_gboff);
  int32_t* nwork = reinterpret_cast<int32_t*>(aux + geo.aux_nwork);
  int32_t* loc = reinterpret_cast<int32_t*>(aux + geo.aux_loc);
  int32_t* nloc = reinterpret_cast<int32_t*>(aux + geo.aux_nloc);
  int4* work_sorted = reinterpret_cast<int4*>(aux + geo.aux_work_sorted);
  char* wsb = static_cast<char*>(ws);
  int32_t* tile_hist = reinterpret_cast<int32_t*>(wsb);
  int32_t* buckets = reinterpret_cast<int32_t*>(wsb + geo.build_ws_buckets);
  int32_t* cb_full = reinterpret_cast<int32_t*>(wsb + geo.build_ws_cb);
  const int M = geo.H * geo.NB;
  int32_t* cb_fwd = cb_full + (M + 1);
  const int nbk = geo.N > 0 ? geo.sort_buckets : 0;
  const int NB1 = geo.NB > 0 ? geo.NB : 1;

  const unsigned zero_wg = (unsigned)std::min<int64_t>(64, (int64_t)M / (4 * kBuildThreads) + 1);
  hipLaunchKernelGGL(k_seq_table, dim3(zero_wg), dim3(kBuildThreads), 0, stream, cu_dev, geo.num_seqs, geo.BK, gboff,
                     nloc, M);
  if (geo.N > 0) {
    hipLaunchKernelGGL(k_hist, dim3(geo.ntiles, geo.H), dim3(kBuildThreads),
                       (2 * geo.win_max + kHistStage + 4 * kRoundTokens) * sizeof(int), stream, sel, cu_dev, gboff,
                       geo.num_seqs,
                       geo.N, geo.T, geo.BK, geo.tile_tokens, geo.ntiles, geo.NB, geo.win_max, tile_hist, loc, nloc,
                       (int)geo.local);
    constexpr int cols = kBuildThreads / kScanSegs;
    hipLaunchKernelGGL(k_tile_scan, dim3((M + cols - 1) / cols), dim3(kBuildThreads), 0, stream,
                       tile_hist, cu_dev, gboff, geo.num_seqs, geo.H, geo.NB, geo.BK, geo.tile_tokens, geo.ntiles,
                       idx.counts);
  }
  hipLaunchKernelGGL(k_offsets, dim3(1), dim3(kScanThreads), 0, stream, idx.counts, nloc, M, geo.chunk_tokens,
                     gboff, geo.num_seqs, NB1, idx.offsets, cb_full, cb_fwd, nwork, buckets, nbk, (int)geo.local);
  if (geo.N > 0) {
    int Tp = 1;
    while (Tp < geo.T) Tp <<= 1;
    const int tps = min(32, kScatterThreads / Tp);
    const size_t lds = (size_t)(5 * geo.win_max + kHistStage + 3 * kRoundTokens) * sizeof(int);
    hipLaunchKernelGGL(k_scatter, dim3(geo.ntiles, geo.H), dim3(kScatterThreads), lds, stream, sel, cu_dev, gboff,
                       geo.num_seqs, geo.N, geo.T, Tp, tps, geo.BK, geo.tile_tokens, geo.ntiles, geo.NB, geo.win_max,
                       tile_hist, idx.offsets, idx.counts, nloc, (int)geo.local, geo.chunk_tokens, geo.sort_shift,
                       geo.sort_buckets_per_head, nbk, buckets, idx.qidx, idx.slot);
    if (geo.max_work > 0) {
      const ListArgs la{idx.counts, nloc, cb_full, cb_fwd, nwork, cu_dev, gboff, geo.num_seqs, M, NB1, geo.BK,
                        geo.chunk_tokens, nbk, (int)geo.local};
      const unsigned wg = (unsigned)((2 * geo.max_work + kBuildThreads - 1) / kBuildThreads);
      hipLaunchKernelGGL(k_bucket_scan, dim3(1), dim3(kScanThreads), 0, stream, buckets, 2 * nbk);
      hipLaunchKernelGGL(k_work_place, dim3(wg), dim3(kBuildThreads), 0, stream, la, idx.qidx, idx.offsets,
                         geo.sort_shift, geo.sort_buckets_per_head, buckets, work_sorted);
    }
  }
  return hipGetLastError();
}

}  // namespace fsa
