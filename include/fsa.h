/*
 * fsa.h - C ABI of the MI355X (gfx950) selected-attention library.
 *
 * The library computes the forward pass (and its gradient) of the
 * token-selection ("selected attention") branch of Native Sparse Attention in
 * the KV-block-outer loop order of Flash Sparse Attention (FSA):
 *
 *   - "FSA: An Alternative Efficient Implementation of Native Sparse Attention
 *     Kernel", paper notes (papernotes.org, ICLR 2026): Overall framework
 *     (flowchart: index precompute -> token-selection kernel -> compact buffer
 *     -> reduction kernel, with the online-softmax kernel feeding both) and
 *     Key designs 1-4;
 *   - Flash-Sparse-Attention README (airanks.app mirror): Method (three
 *     kernels: main, reduction, online softmax), Features (fp16/bf16, head dim
 *     up to 256, GQA groups 1..16) and Usage (packed sequences, cu_seqlens,
 *     block_size, topk).
 *
 * Problem.  Packed sequences s = 0..B-1 occupy tokens [cu[s], cu[s+1]).
 * Q is [N, h_K*g, d], K and V are [N, h_K, d], all row-major, fp16 or bf16.
 * Query head h*g + j (j < g) belongs to KV head h.  Sel is int32
 * [h_K, N, T]: for KV head h and query token t, T block indices local to t's
 * sequence (block e covers tokens cu[s] + [e*B_K, (e+1)*B_K)).  Each of the g
 * query heads of the group attends to the union of the selected blocks,
 * restricted causally to keys k <= t.  Entries that are negative, beyond the
 * token's own block, or repeat an earlier entry of the row select nothing;
 * such entries are data, not errors.  A query with no keys gets O = 0 and
 * row max = lse = -inf.
 *
 * Calls, in order (each enqueues kernels on `stream`, never synchronises):
 *   fsa_get_sizes          host only: byte sizes of every buffer below.
 *   fsa_build_index        Sel -> index tensors I_i / N_valid / O_i.
 *                          (fsa_build_index_noalloc: the same without a
 *                          workspace, for callers that cannot allocate.)
 *   fsa_softmax_stats      per-query row max and log-sum-exp.
 *   fsa_selected_attn_fwd  main kernel (partials) + reduction -> O.
 *                          (= fsa_selected_attn_main then _reduce.)
 *   fsa_selected_attn_fwd_onepass  statistics fused into the main kernel
 *                          and the reduction: row max, lse and O in two
 *                          passes (replaces the two calls above).
 *   fsa_selected_attn_bwd  dQ, dK, dV for an output gradient dO, from the
 *                          same index, O and lse.
 *   fsa_nsa_selected_attn_fwd  the same forward in the query-outer order of
 *                          vanilla NSA (baseline; needs no index).
 *   fsa_select_blocks      Sel from per-block scores (top-k with forced
 *                          initial and local blocks), the step before the path.
 *
 * Ownership.  The caller allocates and owns every buffer (device memory
 * unless marked host).  The library allocates nothing, keeps no pointer
 * after a call returns, holds no mutable global state (except the per-device
 * address of fsa_build_index_noalloc's static scratch, looked up once) and
 * may be called from several host threads.  Buffers must stay alive until the stream has
 * executed the enqueued work.  The `fsa_index` buffers and its `aux` blob
 * belong together: build them once, reuse them for the stats and forward
 * calls of the same problem and Sel.  After fsa_build_index the index is only
 * read: the compute calls (stats, forward, backward) keep their work-queue
 * counters in their own workspace, so calls that share one index may run
 * concurrently (other streams, other threads) as long as each uses its own
 * workspace; calls that share a workspace must not overlap.
 *
 * Errors.  Every call returns FSA_OK (0) or a nonzero fsa_status.  Argument
 * checks run before anything is enqueued: on any status other than
 * FSA_ERR_HIP nothing has been enqueued.  FSA_ERR_HIP means a kernel launch
 * failed; earlier kernels of the same call may have been enqueued.
 *
 * Empty problems.  With no tokens (N = 0) the per-token data buffers (Q, K,
 * V, O, dO, lse, row max, Sel, scores, dQ, dK, dV) are empty and may be NULL;
 * workspaces and index buffers are never empty (fsa_get_sizes reports at
 * least one element) and stay required.  fsa_build_index still writes
 * offsets[0] = 0 (P = 0).
 */
#ifndef FSA_H_
#define FSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FSA_ABI_VERSION 2

typedef enum {
  FSA_OK = 0,
  FSA_ERR_NULL = 1,        /* a required pointer is NULL */
  FSA_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes */
  FSA_ERR_DTYPE = 3,       /* unknown dtype / partial dtype code */
  FSA_ERR_UNSUPPORTED = 4, /* valid shape, but no compiled kernel for it */
  FSA_ERR_WORKSPACE = 5,   /* a workspace is smaller than fsa_get_sizes asks */
  FSA_ERR_HIP = 6,         /* a HIP launch failed */
  FSA_ERR_ALIGN = 7,       /* a pointer is not aligned as documented */
  FSA_ERR_SCRATCH = 8      /* fsa_build_index_noalloc: the problem needs more build
                              scratch than FSA_NOALLOC_BUILD_SCRATCH_BYTES */
} fsa_status;

/* Build scratch held per GPU by fsa_build_index_noalloc (16 MiB). */
#define FSA_NOALLOC_BUILD_SCRATCH_BYTES (16u << 20)

typedef enum { FSA_DTYPE_BF16 = 0, FSA_DTYPE_FP16 = 1 } fsa_dtype;

/* Storage type of the compact partial buffer written by the main kernel. */
typedef enum {
  FSA_PARTIAL_FP32 = 0,  /* fp32 partial rows (4 bytes per element) */
  FSA_PARTIAL_INPUT = 1  /* partial rows in the input dtype (2 bytes) */
} fsa_partial_dtype;

typedef struct {
  int32_t num_seqs;               /* B >= 1 packed sequences */
  const int32_t* cu_seqlens_host; /* host [B+1]: 0 = cu[0] <= cu[1] <= ... = N */
  const int32_t* cu_seqlens_dev;  /* device [B+1], same values (kernels read it) */
  int32_t num_kv_heads;           /* h_K >= 1 */
  int32_t gqa_group;              /* g in [1, 16]; query heads = h_K * g */
  int32_t head_dim;               /* d: 64, 128 or 256 (same for Q, K, V) */
  int32_t block_size;             /* B_K: 64 or 128 */
  int32_t topk;                   /* T in [1, 256] entries per Sel row */
  float softmax_scale;            /* > 0, or <= 0 for 1/sqrt(d) */
  int32_t dtype;                  /* fsa_dtype of Q, K, V and O */
  int32_t partial_dtype;          /* fsa_partial_dtype */
} fsa_problem;

typedef struct {
  int64_t total_tokens;   /* N */
  int64_t num_blocks;     /* NB = sum_s ceil(L_s / B_K) global KV blocks per head */
  int64_t max_pairs;      /* upper bound of P, the number of selecting entries */
  int64_t max_work_items; /* upper bound of (KV head, block, query chunk) items */
  size_t counts_bytes;    /* int32 [h_K * NB] */
  size_t offsets_bytes;   /* int32 [h_K * NB + 1] */
  size_t qidx_bytes;      /* int32 [max_pairs] (at least one element) */
  size_t slot_bytes;      /* int32 [h_K, N, T] */
  size_t aux_bytes;       /* library-private blob that travels with the index */
  size_t build_ws_bytes;  /* scratch for fsa_build_index only */
  size_t stats_ws_bytes;  /* scratch for fsa_softmax_stats only */
  size_t partial_ws_bytes;/* scratch for fsa_selected_attn_fwd / _main / _reduce */
  size_t bwd_ws_bytes;    /* scratch for fsa_selected_attn_bwd; 0 where no backward
                             kernel is compiled for the shape (see that call) */
} fsa_sizes;

/*
 * Index tensors (paper notes, Key design 2), in a canonical layout:
 *   segment f = h * NB + gb, gb = global block = (blocks of earlier sequences) + e;
 *   counts[f]  = N_valid of segment f: how many query tokens select block gb of KV head h;
 *   offsets[f] = exclusive prefix sum of counts over f, offsets[h_K*NB] = P
 *                (the compact output offsets O_i: segment f owns partial rows
 *                [offsets[f], offsets[f+1]));
 *   qidx[offsets[f] + r] = the r-th smallest global query token of segment f (I_i);
 *   slot[h, t, j] = offsets[f] + r for the entry that selects segment f
 *                   (first occurrence in the row), -1 for entries that select nothing.
 * All int32, 4-byte aligned; aux 256-byte aligned.
 */
typedef struct {
  int32_t* counts;
  int32_t* offsets;
  int32_t* qidx;
  int32_t* slot;
  void* aux;
} fsa_index;

/* Version of this header's ABI (FSA_ABI_VERSION). */
int32_t fsa_abi_version(void);

/* Static text for a status code; never NULL. */
const char* fsa_status_string(int32_t status);

/*
 * Host-only: validate `prob` and fill `out` with every buffer size.
 * Touches no device memory and needs no GPU.  cu_seqlens_dev may be NULL here.
 */
int32_t fsa_get_sizes(const fsa_problem* prob, fsa_sizes* out);

/*
 * Index precompute (paper notes, Overall framework: "precompute index tensors
 * I_i / O_i" from the selection tensor; Key design 2).
 *   sel  device int32 [h_K, N, T], 4-byte aligned.
 *   idx  device buffers sized by fsa_get_sizes (counts, offsets, qidx, slot, aux).
 *   ws   device scratch of at least build_ws_bytes (256-byte aligned); free to
 *        reuse once the stream has passed this call.
 * Bit-exact and deterministic: counting sort without order-deciding atomics.
 */
int32_t fsa_build_index(const fsa_problem* prob, const int32_t* sel, const fsa_index* idx,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * fsa_build_index without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, outputs and errors as
 * fsa_build_index; the build scratch lives instead in a static device array
 * of FSA_NOALLOC_BUILD_SCRATCH_BYTES that each GPU the library runs on holds
 * until the process ends (its device address is looked up once per device).
 * Nothing is allocated.  Problems whose build_ws_bytes (fsa_get_sizes)
 * exceed that size return FSA_ERR_SCRATCH before anything is enqueued (about
 * 4 MiB at 64K tokens and 4 KV heads, 8 MiB at 2 x 32K tokens and 8 KV heads).
 * The scratch needs no clearing (every call writes what it reads), but all
 * calls on one GPU share it: calls that overlap in time on one GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 */
int32_t fsa_build_index_noalloc(const fsa_problem* prob, const int32_t* sel, const fsa_index* idx, void* stream);

/*
 * Online-softmax statistics (paper notes, Key design 4; README, Method
 * "online softmax kernel"): for every query token t and query head hq,
 *   row_max[t, hq] = max over visible keys of scale * q.k,
 *   lse[t, hq]     = row_max + ln(sum exp(scale * q.k - row_max)),
 * natural log, fp32 [N, h_K*g].  q, k: device, 16-byte aligned.
 *   ws  device scratch of at least stats_ws_bytes (16-byte aligned).
 */
int32_t fsa_softmax_stats(const fsa_problem* prob, const void* q, const void* k, const fsa_index* idx,
                          float* row_max, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * Forward output (README, Method: main kernel + reduction kernel; paper
 * notes, Key designs 1-3): out[t, hq, :] = sum over visible keys of
 * exp(scale * q.k - lse) * v, in the input dtype (round to nearest even).
 *   q, k, v, out  device, 16-byte aligned; out is [N, h_K*g, d].
 *   lse           device fp32 [N, h_K*g] from fsa_softmax_stats.
 *   partial_ws    device scratch of at least partial_ws_bytes (16-byte aligned).
 * Equivalent to fsa_selected_attn_main followed by fsa_selected_attn_reduce.
 */
int32_t fsa_selected_attn_fwd(const fsa_problem* prob, const void* q, const void* k, const void* v,
                              const fsa_index* idx, const float* lse, void* out, void* partial_ws,
                              size_t partial_ws_bytes, void* stream);

/*
 * One-pass forward: the statistics and the output of fsa_softmax_stats
 * followed by fsa_selected_attn_fwd, in two kernel passes instead of three.
 * The pages run a separate online-softmax kernel first because thread blocks
 * that each see one KV block cannot know a query's running max (paper notes,
 * Key design 4).  Here each (block, query) pair instead keeps its own
 * softmax: the main kernel writes the block's softmax average of V,
 *   o_b = sum_k exp(s_k - m_b) v_k / l_b  over the block's visible keys,
 * and the pair's (m_b, l_b); the reduction merges the pairs of a query in
 * slot order (the statistics kernel's merge, so row_max and lse are the
 * values fsa_softmax_stats returns) and sums l_b exp(m_b - m) / l * o_b.
 * The same outputs within rounding: o_b is rounded to the partial dtype
 * before its weight is applied instead of after.
 *   q, k, v, out  device, 16-byte aligned; row_max, lse: device fp32
 *                 [N, h_K*g], written.
 *   stats_ws      device scratch of at least stats_ws_bytes (16-byte aligned).
 *   partial_ws    device scratch of at least partial_ws_bytes (16-byte aligned).
 * B_K = 128 with d = 256 returns FSA_ERR_UNSUPPORTED.
 */
int32_t fsa_selected_attn_fwd_onepass(const fsa_problem* prob, const void* q, const void* k, const void* v,
                                      const fsa_index* idx, float* row_max, float* lse, void* out,
                                      void* stats_ws, size_t stats_ws_bytes, void* partial_ws,
                                      size_t partial_ws_bytes, void* stream);

/*
 * Main (token-selection) kernel alone (paper notes, Key designs 1-3): one
 * workgroup per (KV head, KV block, query chunk) stages the block's K and V
 * once, streams the block's query list, and writes the pre-scaled partial
 * rows exp(scale*q.k - lse) @ v contiguously to partial_ws rows
 * [offsets[f] * g, offsets[f+1] * g) (row = pair * g + j, d columns, in the
 * partial dtype).  For B_K = 64 and g >= 2 the entries of a query's own,
 * previous and first block (its local entries) are computed per query block
 * instead: their sum is written to the rows of one of them (the own-block
 * entry, else the previous-block one, else the first-block one) and the
 * other local entries' rows are left unwritten.  With B_K = 128 and d = 256
 * each block runs as two 64-key halves: the first half's rows are as above,
 * the second half's lie max_pairs * g rows further on, and the reduction adds
 * both.  partial_ws is otherwise private to the library (it also holds the
 * main kernel's work-queue counters after the rows);
 * fsa_selected_attn_reduce reads it as written.  With local entries the
 * per-query-block work and the block-outer work can run in one
 * persistent launch or in two launches in a row; the library picks by the
 * amount of per-query-block work, and the environment variable
 * FSA_MAIN_MIXED (read at each call) forces one launch (1) or two (0).  The
 * results are the same bits either way.
 */
int32_t fsa_selected_attn_main(const fsa_problem* prob, const void* q, const void* k, const void* v,
                               const fsa_index* idx, const float* lse, void* partial_ws,
                               size_t partial_ws_bytes, void* stream);

/*
 * Reduction kernel alone (paper notes, Key design 3): out[t, h*g + r, :] =
 * the sum, over the valid Sel entries j of row (h, t) in ascending j order,
 * of partial row slot[h, t, j] * g + r (the local entries counted once,
 * through the rows that hold their sum; see fsa_selected_attn_main); no
 * atomics.
 */
int32_t fsa_selected_attn_reduce(const fsa_problem* prob, const fsa_index* idx, const void* partial_ws,
                                 size_t partial_ws_bytes, void* out, void* stream);

/*
 * Backward pass (gradient of the forward above for an output gradient dO;
 * README, Usage and Evaluation: the module trains and its tests compare
 * backward outputs).  With P = exp(scale * q.k - lse) over each row's visible
 * keys:  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
 *        dQ = scale * dS K,  dK = scale * sum dS^T Q,  dV = sum P^T dO.
 * KV-block-outer like the forward: per (KV head, block, query chunk) the
 * block's K and V are staged once; dK and dV of the block accumulate in
 * registers over the chunk's queries and are summed over the chunks in chunk
 * order; dQ goes through the compact partial rows and the forward's ordered
 * reduction.  No atomics; deterministic.
 *   q, k, v, out, dout  device, input dtype, 16-byte aligned (out and lse as
 *                       returned by the forward for this problem and index);
 *   lse                 device fp32 [N, h_K*g], 4-byte aligned;
 *   dq                  device [N, h_K*g, d]; dk, dv device [N, h_K, d]; input
 *                       dtype, 16-byte aligned, fully written;
 *   ws                  device scratch of at least bwd_ws_bytes, 256-byte aligned.
 * Compiled for every shape the forward supports except B_K = 128 with
 * d = 256, which returns FSA_ERR_UNSUPPORTED (fsa_get_sizes reports
 * bwd_ws_bytes = 0 for it).
 */
int32_t fsa_selected_attn_bwd(const fsa_problem* prob, const void* q, const void* k, const void* v,
                              const void* out, const void* dout, const float* lse, const fsa_index* idx,
                              void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, void* stream);

/*
 * Block selection, the step that produces Sel (README, Usage: topk,
 * init_blocks, local_blocks; paper notes, Background and motivation: every
 * query token picks T KV blocks per KV head).  The scores are an input (the
 * pages do not describe NSA's compressed-attention scoring):
 *   scores  device fp32 [h_K, N, score_stride]: scores[h, t, e] for the local
 *           blocks e of t's sequence; entries e > t's own block are ignored.
 *           score_stride >= the block count of the longest sequence.
 *   sel     device int32 [h_K, N, T], written: for own block b, the forced
 *           blocks (0 .. init_blocks-1 that are <= b, then b, b-1, .. for
 *           local_blocks, each once, truncated to T), then the other blocks
 *           e <= b by score descending with ties to the smaller e (NaN counts
 *           as -inf, -0 as +0), then -1.
 * init_blocks, local_blocks >= 0.  Bit-exact and deterministic.
 */
int32_t fsa_select_blocks(const fsa_problem* prob, const float* scores, int64_t score_stride, int32_t init_blocks,
                          int32_t local_blocks, int32_t* sel, void* stream);

/*
 * Query-outer forward, the loop order of vanilla NSA selected attention
 * (paper notes, Background and motivation; Key design 1 names the loop order
 * this path is compared with).  One wave per (token, KV head, up to 16 query
 * heads) walks the token's selected blocks with an online softmax; the query
 * heads of a group are padded to 16 MFMA rows.  Needs no index and no
 * workspace.  Computes the same function as fsa_softmax_stats +
 * fsa_selected_attn_fwd:
 *   out[t, hq, :] in the input dtype, [N, h_K*g, d];
 *   lse[t, hq]    natural-log log-sum-exp, fp32 [N, h_K*g] (-inf and a zero
 *                 output row for a row with no valid Sel entry).
 *   q, k, v, out  device, 16-byte aligned;  sel  device int32 [h_K, N, T],
 *                 4-byte aligned;  lse  device, 4-byte aligned.
 * Returns FSA_ERR_NULL / _ALIGN / _SHAPE / _UNSUPPORTED (also for B_K = 128
 * with d = 256) before any launch, FSA_ERR_HIP if the launch fails.
 */
int32_t fsa_nsa_selected_attn_fwd(const fsa_problem* prob, const void* q, const void* k, const void* v,
                                  const int32_t* sel, float* lse, void* out, void* stream);

/*
 * Measurement: `workgroups` workgroups of four waves each run `iters`
 * rounds of eight independent v_mfma_f32_32x32x16 (bf16 or fp16, per
 * fsa_dtype) instructions per wave, for timing the sustained matrix-core
 * rate, 2 * 32 * 32 * 16 * 8 * iters * 4 * workgroups flops per call.  For
 * benchmarks that report kernels against a measured peak next to the nominal
 * one; computes nothing else.
 *   sink  device fp32 [256], never written for these inputs (keeps the loop).
 * Returns FSA_ERR_NULL / _SHAPE / _DTYPE before the launch, FSA_ERR_HIP if
 * it fails.
 */
int32_t fsa_mfma_loop(int32_t dtype, int32_t workgroups, int32_t iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FSA_H_ */
