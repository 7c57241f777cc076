// Internal declarations shared by the gfx950 kernels and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fsa.h"

namespace fsa {

// ---------------------------------------------------------------------------
// Tunables
// ---------------------------------------------------------------------------
constexpr int kBuildThreads = 256;     // workgroup of the index kernels
constexpr int kScanThreads = 1024;     // single-workgroup offsets scan
constexpr int kMinTileTokens = 256;    // tokens per histogram tile (grows for long inputs)
constexpr int64_t kMaxTileHist = int64_t(1) << 24;  // cap on h_K * tiles * NB entries
constexpr int kWinMax = 6912;          // max global blocks one tile can touch (LDS of k_scatter: 5 ints each)
constexpr int kAttnThreads = 256;      // 4 waves per main / stats workgroup
constexpr int kRowsPerItem = 1024;     // target query rows (tokens * g) per work item
constexpr int kReduceThreads = 256;
constexpr int kSortBucketsMax = 16384;  // buckets of the work-order sort
constexpr int kSelRegBlocks = 1024;     // block selection keeps rows up to this many blocks in registers

// ---------------------------------------------------------------------------
// Problem geometry, computed once on the host from fsa_problem.
// ---------------------------------------------------------------------------
struct Geometry {
  int32_t num_seqs;
  int32_t N;      // total tokens
  int32_t H;      // KV heads
  int32_t g;      // GQA group
  int32_t HQ;     // query heads
  int32_t d;      // head dim
  int32_t BK;     // block size
  int32_t T;      // Sel entries per row
  int32_t NB;     // global blocks per head
  int64_t max_seq_blocks;  // blocks of the longest sequence
  bool select_long_rows;   // some sequence has more than kSelRegBlocks blocks
  int32_t tile_tokens;   // tokens per index tile
  int32_t ntiles;        // index tiles
  int32_t win_max;       // largest block window of any tile
  int32_t chunk_tokens;  // query tokens per work item
  bool split_halves;     // B_K = 128 with d = 256: the main kernel takes each 128-key block as two 64-key
                         // halves (K and V of a whole block do not fit in LDS next to the query tiles), each
                         // with its own partial rows: half 1's rows follow half 0's (split_half_rows apart)
  int64_t split_half_rows;
  bool local;            // local entries are computed per query block (B_K = 64, g >= 2: there the
                         // block's rows fill the local kernels' tiles; elsewhere the block-outer
                         // kernels take every entry, the local words stay zero)
  int32_t dtype;
  int32_t partial_dtype;
  float scale;           // softmax scale (natural units)
  int64_t max_pairs;
  int64_t max_work;
  int64_t dump_row;      // first of 32 rows after the partial / stats rows that take the
                         // stores of rows past a chunk's end (never read)
  // aux blob layout (byte offsets)
  size_t aux_seq_gboff;  // int32 [B+1] exclusive prefix of per-sequence block counts
  size_t aux_nwork;      // int32 [4]: items of the full work list, P, items of the forward list, spare
  size_t aux_loc;        // int32 [H][N]: local word of each (KV head, token), see local_entry()
  size_t aux_nloc;       // int32 [H * NB]: local entries at the head of each segment (blocks >= 1)
  size_t aux_work_sorted;// int4 [2 * max_work]: work items (segment, first query of the chunk, block
                         // start, seq end) of the full and the forward list, each ordered by
                         // (KV head, first query token); the forward list from index nwork[0] on
  int32_t sort_shift;    // work-order bucket = query token >> sort_shift
  int32_t sort_buckets_per_head;
  int32_t sort_buckets;
  size_t aux_bytes;
  size_t build_ws_bytes;
  size_t build_ws_buckets;  // byte offset of the work-order bucket counters in the build workspace
  size_t build_ws_cb;       // byte offset of the work-list bases cb_full, cb_fwd (int32 [H * NB + 1] each)
  // Statistics workspace: (max, sum) float2 per partial row, then the work-queue
  // counters of the statistics kernel.  Partial workspace: the partial rows
  // (dump_row + 32 rows of d elements), then the counters of the main kernel.
  // A query's local row (its own, previous and first block, computed per query
  // block) sits at the rows of its designated local entry (local_designated).
  size_t stats_ws_bytes;
  size_t stats_queue_off;   // byte offset of the statistics kernel's queue counters
  size_t partial_rows_bytes;
  size_t partial_ws_bytes;
  size_t partial_queue_off; // byte offset of the main kernel's queue counters
  // backward workspace: delta [N, HQ] fp32 | dQ partial rows (partial_rows_bytes) |
  // dK / dV slots: fp32 [kv_slots][2][BK][d], slot = offsets[f] / CT + f + chunk | queue counters
  bool bwd_ok;           // a backward kernel is compiled for (d, BK)
  int64_t kv_slots;
  size_t bwd_dq_off, bwd_kv_off, bwd_queue_off, bwd_ws_bytes;
};

int32_t compute_geometry(const fsa_problem* prob, Geometry* geo);

// ---------------------------------------------------------------------------
// Launchers (defined next to their kernels); all enqueue on `stream` and
// return hipSuccess or the launch error.
// ---------------------------------------------------------------------------
hipError_t launch_build_index(const Geometry& geo, const int32_t* cu_dev, const int32_t* sel,
                              const fsa_index& idx, void* ws, hipStream_t stream);
hipError_t launch_stats(const Geometry& geo, const int32_t* cu_dev, const void* q, const void* k,
                        const fsa_index& idx, float* row_max, float* lse, void* ws, hipStream_t stream);
// st_ws == nullptr: the main kernels of the three-pass forward (P = exp(s -
// lse) from the given lse).  Otherwise the one-pass variant: per-block
// softmax averages, their (max, sum) pairs written to st_ws (laid out as the
// statistics workspace); lse is not read.
hipError_t launch_main(const Geometry& geo, const int32_t* cu_dev, const void* q, const void* k, const void* v,
                       const fsa_index& idx, const float* lse, void* st_ws, void* partial, hipStream_t stream);
// local: the forward's reduction (local partial rows plus the other slots);
// otherwise every slot is summed (the backward's dQ).  With st_ws (one-pass
// forward) the rows are weighted by their pairs and row_max / lse written.
hipError_t launch_reduce(const Geometry& geo, const fsa_index& idx, const void* partial, void* out, bool local,
                         const void* st_ws, float* row_max, float* lse, hipStream_t stream);
hipError_t launch_bwd(const Geometry& geo, const int32_t* cu_dev, const void* q, const void* k, const void* v,
                      const void* out, const void* dout, const float* lse, const fsa_index& idx, void* dq, void* dk,
                      void* dv, void* ws, hipStream_t stream);
hipError_t launch_select(const Geometry& geo, const int32_t* cu_dev, const float* scores, int64_t S, int init_blocks,
                         int local_blocks, int32_t* sel, hipStream_t stream);
hipError_t launch_nsa(const Geometry& geo, const int32_t* cu_dev, const void* q, const void* k, const void* v,
                      const int32_t* sel, void* out, float* lse, hipStream_t stream);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Vec8;
template <>
struct Vec8<__bf16> {
  using type = bf16x8;
};
template <>
struct Vec8<_Float16> {
  using type = f16x8;
};

// D = A * B + C on one 32x32x16 tile (gfx950 MFMA, fp32 accumulate).
// Lane l supplies A[l % 32][8 * (l / 32) + e] and B[8 * (l / 32) + e][l % 32],
// e = 0..7; it receives C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32], r = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Sequence that holds global token t: the last s with cu[s] <= t (skips empty
// sequences).  cu has num_seqs + 1 entries.
__device__ __forceinline__ int seq_of_token(const int32_t* __restrict__ cu, int num_seqs, int t) {
  int lo = 0, hi = num_seqs;  // answer in [lo, hi)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Sequence that holds global block gb: the last s with gboff[s] <= gb.
__device__ __forceinline__ int seq_of_block(const int32_t* __restrict__ gboff, int num_seqs, int gb) {
  return seq_of_token(gboff, num_seqs, gb);
}

// Local entries.  NSA keeps a query's first block and its own and previous
// blocks in every selection, so the selected entries of those blocks ("local"
// entries) belong to every query of a query block.  The forward computes them
// per query block, where the block's queries are contiguous and share the
// three key blocks, and writes one partial row (and one (max, sum) pair) per
// query instead of three; the block-outer kernels take the other entries.
// The local word of a (KV head, token) packs, for each kind k (0: own block,
// 1: previous block, 2: block 0 of the sequence when it is neither), 1 + the
// Sel index of the token's valid entry of that block in bits [9k, 9k + 9), or
// 0 when the token does not select it (Sel rows have at most 256 entries).
__device__ __forceinline__ int local_kind(int e, int own) {
  return e == own ? 0 : e == own - 1 ? 1 : e == 0 ? 2 : -1;
}
__device__ __forceinline__ bool local_has(uint32_t word, int kind) { return ((word >> (9 * kind)) & 511u) != 0u; }
// The designated local entry of a (KV head, token) with local word `word` != 0:
// its own-block entry, else its previous-block entry, else its first-block
// entry (the Sel position).  Its partial row (slot * g + j) and statistics
// row hold the token's local row: k_main does not write the partial rows of
// local entries, so that row is free.
__device__ __forceinline__ int local_designated(uint32_t word) {
  const uint32_t f = (word & 511u) != 0u ? word : (word & (511u << 9)) != 0u ? word >> 9 : word >> 18;
  return (int)(f & 511u) - 1;
}
__device__ __forceinline__ bool local_entry(uint32_t word, int j) {
  const uint32_t x = (uint32_t)j + 1u;
  return (word & 511u) == x || ((word >> 9) & 511u) == x || ((word >> 18) & 511u) == x;
}
// Key block of local kind k for query block e (kinds 0 .. min(e, 2)).
__device__ __forceinline__ int local_block(int kind, int e) { return kind == 0 ? e : kind == 1 ? e - 1 : 0; }

// One work item of the attention kernels: KV head, number of query tokens,
// first pair (position in qidx), block start token and keys in the block.
struct Item {
  int h, ntok, pair0, bs, nkeys;
  int kb, nk;  // first token and count (>= 1) of the key rows loaded: bs and nkeys unless the item has no keys
  int half;    // key half of a 128-key block (split items), else 0
};

// Work item wi = (segment f, first query of the chunk within the segment,
// block start token, sequence end) of the index builder's work list.
__device__ __forceinline__ Item read_item(const int4* __restrict__ work, const int32_t* __restrict__ counts,
                                          const int32_t* __restrict__ offsets, int wi, int NB, int CT, int BK) {
  const int4 it = work[wi];
  Item r;
  r.h = it.x / NB;
  r.ntok = min(CT, counts[it.x] - it.y);
  r.pair0 = offsets[it.x] + it.y;
  r.bs = it.z;
  r.nkeys = min(BK, it.w - it.z);
  r.kb = r.bs;
  r.nk = r.nkeys;
  r.half = 0;
  return r;
}

// Item wi2 of the split list: work item wi2 / 2 taken over the 64 keys of
// half wi2 % 2 of its 128-key block.  A second half past the sequence end has
// no keys: its rows see no key (every query of such a block lies before the
// half), and its key loads use the block's first row.
__device__ __forceinline__ Item read_item_half(const int4* __restrict__ work, const int32_t* __restrict__ counts,
                                               const int32_t* __restrict__ offsets, int wi2, int NB, int CT) {
  Item r = read_item(work, counts, offsets, wi2 >> 1, NB, CT, 128);
  r.half = wi2 & 1;
  const int4 it = work[wi2 >> 1];
  r.bs = it.z + 64 * r.half;
  r.nkeys = min(64, it.w - r.bs);
  r.kb = r.nkeys > 0 ? r.bs : it.z;
  r.nk = max(r.nkeys, 1);
  return r;
}

// Persistent workgroups take their items from dynamic work queues.  The grid
// is a multiple of 8 and workgroup i runs on XCD x = i % 8 (round-robin
// dispatch).  The token-ordered work list is dealt to the queues in stripes of
// kStripe consecutive items (stripe s to queue s % 8), so each XCD works on
// runs of neighbouring items (query rows that its L2 may already hold) while
// all eight XCDs stay within one window of the list (one KV head and stretch
// of tokens, whose Q rows the memory-side cache can hold; splitting the list
// into eight contiguous ranges instead ran 1-3% slower).  The workgroups of
// XCD x claim the items of queue x in order with an atomic counter, then move
// on to the other queues in turn, so every workgroup stays busy while any item
// is left (item sizes vary).  Which workgroup takes an item changes no
// output.  The
// counters live in the workspace of the call (statistics, forward or backward
// workspace), cleared by the kernel that runs before the persistent one, so
// the index is read-only after it is built and calls that use one index with
// different workspaces may overlap.
constexpr int kQueues = 8;
constexpr int kQueueStride = 32;  // ints between counters: one 128-byte line each
constexpr int kQueueInts = kQueues * kQueueStride;

constexpr int kStripe = 64;

struct WorkQueue {
  int32_t* q;
  int total, x, tried;
  __device__ __forceinline__ WorkQueue(int32_t* counters, int total_items) : q(counters), total(total_items) {
    x = blockIdx.x & (kQueues - 1);
    tried = 0;
  }
  // One thread per workgroup: the next item, or -1 once every queue is empty.
  // Claim i of queue qq is item ((i / S) * kQueues + qq) * S + i % S, which
  // increases with i, so the first claim past the end ends the queue (each
  // workgroup overshoots a queue at most once: the counters stay far below
  // 2^31 for any list the index can hold).
  __device__ __forceinline__ int claim() {
    while (tried < kQueues) {
      const int qq = (x + tried) & (kQueues - 1);
      const int i = atomicAdd(q + qq * kQueueStride, 1);
      const int w = ((i / kStripe) * kQueues + qq) * kStripe + i % kStripe;
      if (w < total) return w;
      ++tried;
    }
    return -1;
  }
};

// Zeroes a launch's queue counters; run by one workgroup of the kernel that
// precedes the persistent kernel on the same stream in the same call.
__device__ __forceinline__ void clear_queue(int32_t* __restrict__ q) {
  for (int i = threadIdx.x; i < kQueueInts; i += blockDim.x) q[i] = 0;
}

// The item chain of one persistent workgroup: every thread knows the current
// item and the next one (whose staging loads run during the current item);
// thread 0 keeps the claim of the item after those in flight across a whole
// item, so the atomic's latency is hidden.  `s` is a __shared__ int[2].
struct ItemChain {
  WorkQueue wq;
  int cur, nxt, pending;
  __device__ __forceinline__ ItemChain(int32_t* counters, int total, int* s) : wq(counters, total) {
    if (threadIdx.x == 0) {
      const int a = wq.claim();
      s[0] = a;
      s[1] = a >= 0 ? wq.claim() : -1;
    }
    __syncthreads();
    cur = __builtin_amdgcn_readfirstlane(s[0]);
    nxt = __builtin_amdgcn_readfirstlane(s[1]);
    pending = -1;
    if (threadIdx.x == 0 && nxt >= 0) pending = wq.claim();
  }
  // Between the two barriers at the top of an item.
  __device__ __forceinline__ void publish(int* s) const {
    if (threadIdx.x == 0) s[0] = pending;
  }
  // After the second barrier: the item after `nxt`; thread 0 claims the next.
  __device__ __forceinline__ int after(const int* s) {
    const int a = __builtin_amdgcn_readfirstlane(s[0]);
    if (threadIdx.x == 0) pending = a >= 0 ? wq.claim() : -1;
    return a;
  }
  __device__ __forceinline__ void advance(int a) {
    cur = nxt;
    nxt = a;
  }
};

// Persistent grid: as many workgroups of `threads` as fit on the device at
// once (a multiple of 8, one share per XCD), at most one per work item.
template <typename K>
inline unsigned persistent_grid(K kernel, int threads, int64_t max_work) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || cus <= 0 ||
      per_cu <= 0) {
    cus = 256;
    per_cu = 1;
  }
  int64_t want = (int64_t)cus * per_cu;
  if (want > (max_work + 7) / 8 * 8) want = (max_work + 7) / 8 * 8;
  want = (want + 7) / 8 * 8;
  return (unsigned)(want < 8 ? 8 : want);
}

}  // namespace fsa
