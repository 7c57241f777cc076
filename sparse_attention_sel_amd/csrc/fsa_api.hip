// C-ABI entry points: argument validation, buffer sizing and kernel dispatch.
// Every check runs before the first launch, so a call that returns an error
// other than FSA_ERR_HIP has enqueued nothing.  Nothing here allocates.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "fsa_internal.h"

// Build scratch of fsa_build_index_noalloc: one copy per GPU, held from the
// library's first use on that GPU until the process ends.  Host code never
// passes this name to a kernel: on the host it is a stand-in, not the device
// address, which hipGetSymbolAddress returns per device (scratch_of_device).
static __device__ __align__(256) unsigned char scratch[FSA_NOALLOC_BUILD_SCRATCH_BYTES];

namespace fsa {
namespace {

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

int32_t scratch_of_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return FSA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FSA_OK;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

int32_t compute_geometry(const fsa_problem* p, Geometry* geo) {
  if (p == nullptr || geo == nullptr || p->cu_seqlens_host == nullptr) return FSA_ERR_NULL;
  if (p->num_seqs < 1) return FSA_ERR_SHAPE;
  if (p->dtype != FSA_DTYPE_BF16 && p->dtype != FSA_DTYPE_FP16) return FSA_ERR_DTYPE;
  if (p->partial_dtype != FSA_PARTIAL_FP32 && p->partial_dtype != FSA_PARTIAL_INPUT) return FSA_ERR_DTYPE;
  if (p->num_kv_heads < 1 || p->gqa_group < 1 || p->gqa_group > 16) return FSA_ERR_SHAPE;
  if (p->head_dim < 16 || p->head_dim > 256 || p->head_dim % 16 != 0) return FSA_ERR_SHAPE;
  if (p->block_size < 1 || p->topk < 1 || p->topk > 256) return FSA_ERR_SHAPE;
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256) return FSA_ERR_UNSUPPORTED;
  if (p->block_size != 64 && p->block_size != 128) return FSA_ERR_UNSUPPORTED;
  float scale = p->softmax_scale;
  if (std::isnan(scale) || std::isinf(scale)) return FSA_ERR_SHAPE;
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt((float)p->head_dim);

  const int32_t* cu = p->cu_seqlens_host;
  const int B = p->num_seqs;
  if (cu[0] != 0) return FSA_ERR_SHAPE;
  for (int s = 0; s < B; ++s)
    if (cu[s + 1] < cu[s]) return FSA_ERR_SHAPE;
  const int64_t N = cu[B];
  const int64_t H = p->num_kv_heads, g = p->gqa_group, T = p->topk, BK = p->block_size;
  if (H * N * T >= (int64_t(1) << 31)) return FSA_ERR_SHAPE;  // slot positions are int32
  if (H * g * N >= (int64_t(1) << 31)) return FSA_ERR_SHAPE;

  std::memset(geo, 0, sizeof(*geo));
  geo->num_seqs = B;
  geo->N = (int32_t)N;
  geo->H = (int32_t)H;
  geo->g = (int32_t)g;
  geo->HQ = (int32_t)(H * g);
  geo->d = p->head_dim;
  geo->BK = (int32_t)BK;
  geo->T = (int32_t)T;
  geo->dtype = p->dtype;
  geo->partial_dtype = p->partial_dtype;
  geo->scale = scale;
  geo->chunk_tokens = (int32_t)((kRowsPerItem + g - 1) / g);
  const int64_t CT = geo->chunk_tokens;
  geo->local = BK == 64 && g >= 2;

  // Blocks, the bound on selecting entries (a token of local block e selects
  // at most min(T, e + 1) distinct blocks) and the bound on work items (block
  // e of a sequence can be selected by at most the L - e*BK tokens from its
  // start to the end of the sequence).
  int64_t NB = 0, pairs = 0, work = 0, max_nb = 0;
  for (int s = 0; s < B; ++s) {
    const int64_t L = cu[s + 1] - cu[s];
    const int64_t nb = (L + BK - 1) / BK;
    NB += nb;
    max_nb = std::max(max_nb, nb);
    for (int64_t e = 0; e < nb; ++e) {
      const int64_t ntok = std::min(BK, L - e * BK);
      pairs += ntok * std::min(T, e + 1);
      work += (L - e * BK + CT - 1) / CT;
    }
  }
  if (H * NB >= (int64_t(1) << 30)) return FSA_ERR_SHAPE;
  geo->NB = (int32_t)NB;
  geo->max_seq_blocks = max_nb;
  geo->select_long_rows = max_nb > kSelRegBlocks;
  geo->max_pairs = H * pairs;
  geo->max_work = std::min(H * work, (geo->max_pairs + CT - 1) / CT + H * NB);
  if (geo->max_work >= (int64_t(1) << 31)) return FSA_ERR_SHAPE;

  // Histogram tiles: grow the tile until the tile-by-block histogram is bounded.
  int64_t TT = kMinTileTokens;
  while (N > 0 && H * ((N + TT - 1) / TT) * NB > kMaxTileHist) TT *= 2;
  geo->tile_tokens = (int32_t)TT;
  geo->ntiles = (int32_t)((N + TT - 1) / TT);
  // Largest block window of any tile: from the first block of its first
  // token's sequence to the own block of its last token.
  {
    std::vector<int64_t> gboff(B + 1, 0);
    for (int s = 0; s < B; ++s) gboff[s + 1] = gboff[s] + (cu[s + 1] - cu[s] + BK - 1) / BK;
    auto seq_of = [&](int64_t t) {
      int lo = 0, hi = B;
      while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (cu[mid] <= t) lo = mid; else hi = mid;
      }
      return lo;
    };
    int64_t win_max = 1;
    for (int64_t tile = 0; tile < geo->ntiles; ++tile) {
      const int64_t t_lo = tile * TT, t_hi = std::min(t_lo + TT, N);
      const int s0 = seq_of(t_lo), s1 = seq_of(t_hi - 1);
      const int64_t win = gboff[s1] + (t_hi - 1 - cu[s1]) / BK - gboff[s0] + 1;
      win_max = std::max(win_max, win);
    }
    if (win_max > kWinMax) return FSA_ERR_UNSUPPORTED;
    geo->win_max = (int32_t)win_max;
  }

  size_t off = 0;
  geo->aux_seq_gboff = off;
  off = round_up(off + (size_t)(B + 1) * 4, 256);
  geo->aux_nwork = off;
  off = round_up(off + 16, 256);
  geo->aux_loc = off;
  off = round_up(off + (size_t)std::max<int64_t>(H * N, 1) * 4, 256);
  geo->aux_nloc = off;
  off = round_up(off + (size_t)std::max<int64_t>(H * NB, 1) * 4, 256);
  // full and forward lists: the forward list's chunks of a segment are no
  // more than its full list's, so both fit max_work
  geo->aux_work_sorted = off;
  off = round_up(off + 2 * (size_t)std::max<int64_t>(geo->max_work, 1) * 16, 256);
  {
    int shift = 6;
    while (H * ((N + (int64_t(1) << shift) - 1) >> shift) > kSortBucketsMax) ++shift;
    geo->sort_shift = shift;
    geo->sort_buckets_per_head = (int32_t)std::max<int64_t>((N + (int64_t(1) << shift) - 1) >> shift, 1);
    geo->sort_buckets = (int32_t)(H * geo->sort_buckets_per_head);
  }
  geo->aux_bytes = off;
  geo->build_ws_buckets = round_up((size_t)std::max<int64_t>(H * geo->ntiles * NB, 1) * 4, 256);
  geo->build_ws_cb = round_up(geo->build_ws_buckets + 2 * (size_t)std::max(geo->sort_buckets, 1) * 4, 256);
  geo->build_ws_bytes = round_up(geo->build_ws_cb + 2 * (size_t)(H * NB + 1) * 4, 256);
  // One partial row per (selecting entry, query head): rows pair * g + j, the
  // compact output of the pages' index O_i, plus 32 dump rows; no other region
  // (a query's local row uses the rows of its designated local entry).
  geo->split_halves = BK == 128 && geo->d == 256;
  geo->split_half_rows = std::max<int64_t>(geo->max_pairs, 1) * g;
  geo->dump_row = (geo->split_halves ? 2 : 1) * geo->split_half_rows;
  const size_t rows = (size_t)geo->dump_row + 32;
  const size_t s_p = geo->partial_dtype == FSA_PARTIAL_FP32 ? 4 : 2;
  const size_t queue_bytes = (size_t)kQueueInts * 4;
  geo->stats_queue_off = round_up(rows * 8, 256);
  geo->stats_ws_bytes = round_up(geo->stats_queue_off + queue_bytes, 256);
  geo->partial_rows_bytes = round_up(rows * (size_t)geo->d * s_p, 256);
  geo->partial_queue_off = geo->partial_rows_bytes;
  geo->partial_ws_bytes = round_up(geo->partial_queue_off + queue_bytes, 256);
  // Backward: the chunk slot offsets[f] / CT + f + c (c < ceil(count_f / CT))
  // is injective and below max_pairs / CT + M + 2.
  geo->bwd_ok = !geo->split_halves;  // no backward kernel for B_K = 128 with d = 256
  geo->kv_slots = geo->max_pairs / geo->chunk_tokens + H * NB + 2;
  geo->bwd_dq_off = round_up((size_t)N * H * g * 4, 256);
  geo->bwd_kv_off = round_up(geo->bwd_dq_off + geo->partial_rows_bytes, 256);
  geo->bwd_queue_off = round_up(geo->bwd_kv_off + (size_t)geo->kv_slots * 2 * BK * geo->d * 4, 256);
  geo->bwd_ws_bytes = geo->bwd_ok ? round_up(geo->bwd_queue_off + queue_bytes, 256) : 0;
  return FSA_OK;
}

namespace {

int32_t check_index(const fsa_index* idx) {
  if (idx == nullptr || idx->counts == nullptr || idx->offsets == nullptr || idx->qidx == nullptr ||
      idx->slot == nullptr || idx->aux == nullptr)
    return FSA_ERR_NULL;
  if (!aligned(idx->counts, 4) || !aligned(idx->offsets, 4) || !aligned(idx->qidx, 4) || !aligned(idx->slot, 4) ||
      !aligned(idx->aux, 256))
    return FSA_ERR_ALIGN;
  return FSA_OK;
}

int32_t prepare(const fsa_problem* prob, Geometry* geo) {
  const int32_t st = compute_geometry(prob, geo);
  if (st != FSA_OK) return st;
  if (prob->cu_seqlens_dev == nullptr) return FSA_ERR_NULL;
  if (!aligned(prob->cu_seqlens_dev, 4)) return FSA_ERR_ALIGN;
  return FSA_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? FSA_OK : FSA_ERR_HIP; }

// A per-token data buffer (Q, K, V, O, lse, Sel, scores, gradients) is
// required unless the problem has no tokens, where it is empty and may be
// NULL (workspaces and index buffers are never empty and stay required).
bool data(const void* p, const Geometry& geo) { return p != nullptr || geo.N == 0; }

int32_t check_main_args(const Geometry& geo, const void* q, const void* k, const void* v, const fsa_index* idx,
                        const float* lse, const void* partial, size_t partial_bytes) {
  if (!data(q, geo) || !data(k, geo) || !data(v, geo) || !data(lse, geo) || partial == nullptr) return FSA_ERR_NULL;
  int32_t st = check_index(idx);
  if (st != FSA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(lse, 4) || !aligned(partial, 16))
    return FSA_ERR_ALIGN;
  if (partial_bytes < geo.partial_ws_bytes) return FSA_ERR_WORKSPACE;
  return FSA_OK;
}

int32_t check_reduce_args(const Geometry& geo, const fsa_index* idx, const void* partial, size_t partial_bytes,
                          const void* out) {
  if (partial == nullptr || !data(out, geo)) return FSA_ERR_NULL;
  int32_t st = check_index(idx);
  if (st != FSA_OK) return st;
  if (!aligned(partial, 16) || !aligned(out, 16)) return FSA_ERR_ALIGN;
  if (partial_bytes < geo.partial_ws_bytes) return FSA_ERR_WORKSPACE;
  return FSA_OK;
}

}  // namespace
}  // namespace fsa

using namespace fsa;

extern "C" {

int32_t fsa_abi_version(void) { return FSA_ABI_VERSION; }

const char* fsa_status_string(int32_t status) {
  switch (status) {
    case FSA_OK: return "ok";
    case FSA_ERR_NULL: return "a required pointer is NULL";
    case FSA_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case FSA_ERR_DTYPE: return "unknown dtype or partial dtype";
    case FSA_ERR_UNSUPPORTED: return "no compiled kernel for this head dim / block size / sequence length";
    case FSA_ERR_WORKSPACE: return "workspace smaller than fsa_get_sizes requires";
    case FSA_ERR_HIP: return "HIP kernel launch failed";
    case FSA_ERR_ALIGN: return "pointer misaligned";
    case FSA_ERR_SCRATCH:
      return "the index build needs more scratch than fsa_build_index_noalloc holds "
             "(FSA_NOALLOC_BUILD_SCRATCH_BYTES); use fsa_build_index with a workspace";
    default: return "unknown status";
  }
}

int32_t fsa_get_sizes(const fsa_problem* prob, fsa_sizes* out) {
  if (out == nullptr) return FSA_ERR_NULL;
  Geometry geo;
  const int32_t st = compute_geometry(prob, &geo);
  if (st != FSA_OK) return st;
  std::memset(out, 0, sizeof(*out));
  out->total_tokens = geo.N;
  out->num_blocks = geo.NB;
  out->max_pairs = geo.max_pairs;
  out->max_work_items = geo.max_work;
  const size_t M = (size_t)geo.H * geo.NB;
  out->counts_bytes = std::max<size_t>(M, 1) * 4;
  out->offsets_bytes = (M + 1) * 4;
  out->qidx_bytes = (size_t)std::max<int64_t>(geo.max_pairs, 1) * 4;
  out->slot_bytes = std::max<size_t>((size_t)geo.H * geo.N * geo.T, 1) * 4;
  out->aux_bytes = geo.aux_bytes;
  out->build_ws_bytes = geo.build_ws_bytes;
  out->stats_ws_bytes = geo.stats_ws_bytes;
  out->partial_ws_bytes = geo.partial_ws_bytes;
  out->bwd_ws_bytes = geo.bwd_ws_bytes;
  return FSA_OK;
}

int32_t fsa_build_index(const fsa_problem* prob, const int32_t* sel, const fsa_index* idx, void* ws,
                        size_t ws_bytes, void* stream) {
  Geometry geo;
  int32_t st = prepare(prob, &geo);
  if (st != FSA_OK) return st;
  if (!data(sel, geo) || ws == nullptr) return FSA_ERR_NULL;
  st = check_index(idx);
  if (st != FSA_OK) return st;
  if (!aligned(sel, 4) || !aligned(ws, 256)) return FSA_ERR_ALIGN;
  if (ws_bytes < geo.build_ws_bytes) return FSA_ERR_WORKSPACE;
  return hip_status(launch_build_index(geo, prob->cu_seqlens_dev, sel, *idx, ws, static_cast<hipStream_t>(stream)));
}

int32_t fsa_build_index_noalloc(const fsa_problem* prob, const int32_t* sel, const fsa_index* idx, void* stream) {
  Geometry geo;
  int32_t st = prepare(prob, &geo);
  if (st != FSA_OK) return st;
  if (!data(sel, geo)) return FSA_ERR_NULL;
  st = check_index(idx);
  if (st != FSA_OK) return st;
  if (!aligned(sel, 4)) return FSA_ERR_ALIGN;
  if (geo.build_ws_bytes > (size_t)FSA_NOALLOC_BUILD_SCRATCH_BYTES) return FSA_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_of_device(&ws);
  if (st != FSA_OK) return st;
  return hip_status(launch_build_index(geo, prob->cu_seqlens_dev, sel, *idx, ws, static_cast<hipStream_t>(stream)));
}

int32_t fsa_softmax_stats(const fsa_problem* prob, const void* q, const void* k, const fsa_index* idx,
                          float* row_max, float* lse, void* ws, size_t ws_bytes, void* stream) {
  Geometry geo;
  int32_t st = prepare(prob, &geo);
  if (st != FSA_OK) return st;
  if (!data(q, geo) || !data(k, geo) || !data(row_max, geo) || !data(lse, geo) || ws == nullptr) return FSA_ERR_NULL;
  st = check_index(idx);
  if (st != FSA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(row_max, 4) || !aligned(lse, 4) || !aligned(ws, 16))
    return FSA_ERR_ALIGN;
  if (ws_bytes < geo.stats_ws_bytes) return FSA_ERR_WORKSPACE;
  return hip_status(launch_stats(geo, prob->cu_seqlens_dev, q, k, *idx, row_max, lse, ws,
                                 static_cast<hipStream_t>(stream)));
}

int32_t fsa_selected_attn_main(const fsa_problem* prob, const void* q, const void* k, const void* v,
                               const fsa_index* idx, const float* lse, void* partial_ws, size_t partial_ws_bytes,
                               void* stream) {
  Geometry geo;
  int32_t st = prepare(prob, &geo);
  if (st != FSA_OK) return st;
  st = check_main_args(geo, q, k, v, idx, lse, partial_ws, partial_ws_bytes);
  if (st != FSA_OK) return st;
  return hip_status(
      launch_main(geo, prob->cu_seqlens_dev, q, k, v, *idx, lse, nullptr, partial_ws, static_cast<hipStream_t>(stream)));
}

int32_t fsa_selected_attn_reduce(const fsa_problem* prob, const fsa_index* idx, const void* partial_ws,
                                 size_t partial_ws_bytes, void* out, void* stream) {
  Geometry geo;
  int32_t st = prepare(prob, &geo);
  if (st != FSA_OK) return st;
  st = check_reduce_args(geo, idx, partial_ws, partial_ws_bytes, out);
  if (st != FSA_OK) return st;
  return hip_status(
      launch_reduce(geo, *idx, partial_ws, out, true, nullptr, nullptr, nullptr, static_cast<hipStream_t>(stream)));
}

int32_t fsa_selected_attn_fwd(const fsa_problem* prob, const void* q, const void* k, const void* v,
                              const fsa_index* idx, const float* lse, void* out, void* partial_ws,
                              size_t partial_ws_bytes, void* stream) {
  Geometry geo;
  int32_t st = prepare(prob, &geo);
  if (st != FSA_OK) return st;
  st = check_main_args(geo, q, k, v, idx, lse, partial_ws, partial_ws_bytes);
  if (st != FSA_OK) return st;
  st = check_reduce_args(geo, idx, partial_ws, partial_ws_bytes, out);
  if (st != FSA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(launch_main(geo, prob->cu_seqlens_dev, q, k, v, *idx, lse, nullptr, partial_ws, s));
  if (st != FSA_OK) return st;
  return hip_status(launch_reduce(geo, *idx, partial_ws, out, true, nullptr, nullptr, nullptr, s));
}

int32_t fsa_selected_attn_fwd_onepass(const fsa_problem* prob, const void* q, const void* k, const void* v,
                                      const fsa_index* idx, float* row_max, float* lse, void* out, void* stats_ws,
                                      size_t stats_ws_bytes, void* partial_ws, size_t partial_ws_bytes,
                                      void* stream) {
  Geometry geo;
  int32_t st = prepare(prob, &geo);
  if (st != FSA_OK) return st;
  if (geo.split_halves) return FSA_ERR_UNSUPPORTED;  // no one-pass kernels for B_K = 128 with d = 256
  if (!data(row_max, geo) || !data(lse, geo) || stats_ws == nullptr) return FSA_ERR_NULL;
  // lse is an output here; the main-kernel checks only need a non-null pointer
  st = check_main_args(geo, q, k, v, idx, lse, partial_ws, partial_ws_bytes);
  if (st != FSA_OK) return st;
  st = check_reduce_args(geo, idx, partial_ws, partial_ws_bytes, out);
  if (st != FSA_OK) return st;
  if (!aligned(row_max, 4) || !aligned(stats_ws, 16)) return FSA_ERR_ALIGN;
  if (stats_ws_bytes < geo.stats_ws_bytes) return FSA_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(launch_main(geo, prob->cu_seqlens_dev, q, k, v, *idx, nullptr, stats_ws, partial_ws, s));
  if (st != FSA_OK) return st;
  return hip_status(launch_reduce(geo, *idx, partial_ws, out, true, stats_ws, row_max, lse, s));
}

int32_t fsa_selected_attn_bwd(const fsa_problem* prob, const void* q, const void* k, const void* v,
                              const void* out, const void* dout, const float* lse, const fsa_index* idx,
                              void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, void* stream) {
  Geometry geo;
  int32_t st = prepare(prob, &geo);
  if (st != FSA_OK) return st;
  if (!geo.bwd_ok) return FSA_ERR_UNSUPPORTED;
  if (!data(q, geo) || !data(k, geo) || !data(v, geo) || !data(out, geo) || !data(dout, geo) || !data(lse, geo) ||
      !data(dq, geo) || !data(dk, geo) || !data(dv, geo) || ws == nullptr)
    return FSA_ERR_NULL;
  st = check_index(idx);
  if (st != FSA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(ws, 256))
    return FSA_ERR_ALIGN;
  if (ws_bytes < geo.bwd_ws_bytes) return FSA_ERR_WORKSPACE;
  return hip_status(launch_bwd(geo, prob->cu_seqlens_dev, q, k, v, out, dout, lse, *idx, dq, dk, dv, ws,
                               static_cast<hipStream_t>(stream)));
}

int32_t fsa_select_blocks(const fsa_problem* prob, const float* scores, int64_t score_stride, int32_t init_blocks,
                          int32_t local_blocks, int32_t* sel, void* stream) {
  Geometry geo;
  const int32_t st = prepare(prob, &geo);
  if (st != FSA_OK) return st;
  if (!data(scores, geo) || !data(sel, geo)) return FSA_ERR_NULL;
  if (init_blocks < 0 || local_blocks < 0 || score_stride < geo.max_seq_blocks || score_stride < 1)
    return FSA_ERR_SHAPE;
  if (!aligned(scores, 4) || !aligned(sel, 4)) return FSA_ERR_ALIGN;
  return hip_status(launch_select(geo, prob->cu_seqlens_dev, scores, score_stride, init_blocks, local_blocks, sel,
                                  static_cast<hipStream_t>(stream)));
}

int32_t fsa_nsa_selected_attn_fwd(const fsa_problem* prob, const void* q, const void* k, const void* v,
                                  const int32_t* sel, float* lse, void* out, void* stream) {
  Geometry geo;
  const int32_t st = prepare(prob, &geo);
  if (st != FSA_OK) return st;
  if (geo.BK == 128 && geo.d == 256) return FSA_ERR_UNSUPPORTED;  // V of four waves' blocks exceeds LDS
  if (!data(q, geo) || !data(k, geo) || !data(v, geo) || !data(sel, geo) || !data(lse, geo) || !data(out, geo))
    return FSA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(sel, 4) ||
      !aligned(lse, 4))
    return FSA_ERR_ALIGN;
  return hip_status(launch_nsa(geo, prob->cu_seqlens_dev, q, k, v, sel, out, lse, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
