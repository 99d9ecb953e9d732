// Host side of the C ABI declared in include/orthrus.h: argument validation
// (before any HIP call), launch planning from the descriptor alone, and
// stream-ordered launches.  No allocation, no synchronisation, no state.
#include "../../include/orthrus.h"
#include "common.h"
#include "block_order.h"

#include <math.h>
#include <atomic>
#include <mutex>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

// Scratch of orthrus_block_attn_noalloc: the workspace of every such call on a
// device (each device holds its own copy from library load to process end).
// Host code never passes this name to a kernel -- on the host it is only a
// stand-in for the symbol -- but the device address looked up below.
static __device__ __align__(256) uint8_t scratch[ORTHRUS_NOALLOC_SCRATCH_BYTES];

namespace orthrus {
namespace {

constexpr size_t kAlign = 256;

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int env_int(const char* name, int fallback) {
  const char* s = getenv(name);
  if (s == nullptr || *s == '\0') return fallback;
  const int v = atoi(s);
  return v > 0 ? v : fallback;
}

orthrus_status check_desc(const orthrus_attn_desc* d) {
  if (d == nullptr) return ORTHRUS_ERR_NULL_PTR;
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->block_k < 1 ||
      d->max_len < 0 || d->head_dim < 1)
    return ORTHRUS_ERR_BAD_SHAPE;
  if (d->n_q_heads % d->n_kv_heads != 0) return ORTHRUS_ERR_BAD_SHAPE;
  if (!(isfinite(d->softmax_scale) && d->softmax_scale >= 0.0f)) return ORTHRUS_ERR_BAD_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return ORTHRUS_ERR_UNSUPPORTED;
  if (d->block_k > 128) return ORTHRUS_ERR_UNSUPPORTED;
  // cache positions, split bounds and tile starts are int in the kernels: with
  // at most 2^30 rows every such sum stays below 2^31
  if (d->max_len > (1 << 30)) return ORTHRUS_ERR_UNSUPPORTED;
  // every element offset must fit comfortably in 63 bits and every grid dimension in range
  const long long rows = (long long)(d->n_q_heads / d->n_kv_heads) * d->block_k;
  if ((long long)d->batch * d->n_kv_heads > 65535LL || rows > (1LL << 20)) return ORTHRUS_ERR_BAD_SHAPE;
  return ORTHRUS_OK;
}

AttnPlan make_plan(const orthrus_attn_desc* d) {
  AttnPlan p{};
  const int G = d->n_q_heads / d->n_kv_heads;
  p.rows = G * d->block_k;
  // more than 128 rows: 256-row work-groups whose waves each take a query
  // block over whole tiles, so the cache is streamed once per 256 rows
  p.qblocks = p.rows <= 32 ? 1 : (p.rows <= 64 ? 2 : (p.rows <= 128 || env_int("ORTHRUS_ROWS128", 0) == 1 ? 4 : 8));
  p.rows_per_wg = 32 * p.qblocks;
  p.row_groups = (p.rows + p.rows_per_wg - 1) / p.rows_per_wg;
  const long long groups = (long long)d->batch * d->n_kv_heads * p.row_groups;
  long long s = kPlanCUs / groups;
  const long long max_tiles = ((long long)d->max_len + kTileKeys - 1) / kTileKeys;
  if (s > max_tiles) s = max_tiles;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  p.splits = (int)s;
  // several sequences: a balanced launch writes up to one partial per
  // work-group plus one per group boundary inside a work-group's range
  const size_t slots = ((size_t)groups * p.splits + (d->batch > 1 ? (size_t)groups : 0)) * p.rows_per_wg;
  p.ml_bytes = round_up(slots * 2 * sizeof(float), kAlign);
  p.acc_bytes = round_up(slots * d->head_dim * sizeof(uint16_t), kAlign);
  p.tab_bytes = round_up((size_t)groups * 2 * sizeof(int32_t), kAlign);  // first and last slot per group
  p.ws_bytes = p.ml_bytes + p.acc_bytes + p.tab_bytes;
  return p;
}

// Compute units of the current device, cached per device ordinal (a benign,
// idempotent cache: every thread that fills a slot writes the same value).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return -1;
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// phases: 1 = partial (stream cache + block), 2 = merge, 3 = both
orthrus_status run_attn(const orthrus_attn_desc* d, int mode, const uint16_t* q, const uint16_t* k_blk,
                        const uint16_t* v_blk, const uint16_t* k_cache, const uint16_t* v_cache,
                        const int32_t* cache_len, uint16_t* out, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream, int phases, const uint64_t* block_mask = nullptr,
                        const int32_t* blk_len = nullptr) {
  const orthrus_status st = check_desc(d);
  if (st != ORTHRUS_OK) return st;
  if (mode != ORTHRUS_MASK_DIFF_BIDIR && mode != ORTHRUS_MASK_VERIFY_CAUSAL && mode != ORTHRUS_MASK_EXPLICIT)
    return ORTHRUS_ERR_BAD_SHAPE;
  if (mode == ORTHRUS_MASK_EXPLICIT) {
    if (!block_mask && (phases & 1)) return ORTHRUS_ERR_NULL_PTR;
    if ((phases & 1) && !aligned4(block_mask)) return ORTHRUS_ERR_MISALIGNED;
    if (d->block_k > 64) return ORTHRUS_ERR_UNSUPPORTED;
  }
  if (!workspace) return ORTHRUS_ERR_NULL_PTR;
  if ((phases & 1) && (!q || !k_blk || !v_blk || !k_cache || !v_cache || !cache_len))
    return ORTHRUS_ERR_NULL_PTR;
  if ((phases & 2) && !out) return ORTHRUS_ERR_NULL_PTR;
  if (!aligned16(workspace)) return ORTHRUS_ERR_MISALIGNED;
  if ((phases & 1) && (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_cache) ||
                       !aligned16(v_cache) || !aligned4(cache_len)))
    return ORTHRUS_ERR_MISALIGNED;
  if ((phases & 2) && (!aligned16(out) || (lse && !aligned4(lse)))) return ORTHRUS_ERR_MISALIGNED;
  if (blk_len && !aligned4(blk_len)) return ORTHRUS_ERR_MISALIGNED;
  const AttnPlan plan = make_plan(d);
  if (workspace_bytes < plan.ws_bytes) return ORTHRUS_ERR_WORKSPACE_TOO_SMALL;
  const int cus = device_cus();
  if (cus < 1) return ORTHRUS_ERR_HIP;

  AttnArgs a{};
  a.q = q;
  a.k_blk = k_blk;
  a.v_blk = v_blk;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cache_len = cache_len;
  a.out = out;
  a.lse = lse;
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  a.ws_ml = reinterpret_cast<float*>(ws);
  a.ws_acc = reinterpret_cast<uint16_t*>(ws + plan.ml_bytes);
  a.ws_tab = reinterpret_cast<int2*>(ws + plan.ml_bytes + plan.acc_bytes);
  a.batch = d->batch;
  a.n_q_heads = d->n_q_heads;
  a.n_kv_heads = d->n_kv_heads;
  a.group = d->n_q_heads / d->n_kv_heads;
  a.block_k = d->block_k;
  a.head_dim = d->head_dim;
  a.max_len = d->max_len;
  a.causal = mode == ORTHRUS_MASK_VERIFY_CAUSAL ? 1 : 0;
  set_decode_strides(a);
  a.blk_mask = mode == ORTHRUS_MASK_EXPLICIT ? block_mask : nullptr;
  a.blk_len = blk_len;
  a.splits = attn_launch_splits(plan, d->batch, d->n_kv_heads, d->max_len, cus);
  const int cap = env_int("ORTHRUS_MAX_SPLITS", a.splits);  // tuning: may only lower the split count
  if (cap < a.splits) a.splits = cap;
  // several sequences: the launch's work-groups share one list of tiles
  a.ragged = (d->batch > 1 && d->batch <= kRaggedMaxSeqs && a.splits > 1 &&
              env_int("ORTHRUS_EVEN_SPLITS", 0) == 0) ? 1 : 0;
  a.nwg = d->batch * d->n_kv_heads * plan.row_groups * a.splits;
  // one work-group per group (no split): the sequences are taken longest first
  a.rank_blocks = (a.splits == 1 && d->batch > 1 && d->batch <= kRankMaxBlocks) ? 1 : 0;
  const float scale = d->softmax_scale > 0.0f ? d->softmax_scale : 1.0f / sqrtf((float)d->head_dim);
  a.scale_log2 = scale * 1.4426950408889634f;
  if ((phases & 1) && getenv("ORTHRUS_DEBUG") != nullptr)
    fprintf(stderr, "[orthrus] attn mode=%d B=%d Hq=%d Hkv=%d D=%d K=%d max_len=%d rows=%d qblocks=%d "
            "row_groups=%d splits=%d ragged=%d ws=%zu\n", mode, d->batch, d->n_q_heads, d->n_kv_heads,
            d->head_dim, d->block_k, d->max_len, plan.rows, plan.qblocks, plan.row_groups,
            a.splits, a.ragged, plan.ws_bytes);
  const hipError_t e = launch_block_attention(a, plan, phases, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_HIP;
}

// Vocabularies up to 2^30 entries: every int sum of a vocabulary index and a
// chunk or stride length in the kernels and plans then stays below 2^31.
constexpr int32_t kMaxVocab = 1 << 30;

orthrus_status check_consensus_sizes(int32_t B, int32_t K, int32_t V) {
  if (B < 1 || K < 1 || V < 1) return ORTHRUS_ERR_BAD_SHAPE;
  if (K > 128 || V > kMaxVocab) return ORTHRUS_ERR_UNSUPPORTED;
  if ((long long)B * K > 65535LL) return ORTHRUS_ERR_BAD_SHAPE;
  return ORTHRUS_OK;
}

ConsensusPlan make_consensus_plan(int32_t B, int32_t K, int32_t V) {
  ConsensusPlan p{};
  const long long rows = (long long)B * K;
  long long gc = (1024 + rows - 1) / rows;
  long long gmax = V / 1024;
  if (gmax < 1) gmax = 1;
  if (gc > gmax) gc = gmax;
  if (gc < 1) gc = 1;
  p.greedy_chunks = (int)gc;
  long long sc = ((long long)V + 4095) / 4096;
  if (sc > 256) sc = 256;
  if (sc < 1) sc = 1;
  p.sample_chunks = (int)sc;
  p.greedy_bytes = round_up((size_t)rows * p.greedy_chunks * 8, kAlign);
  p.sample_bytes = round_up((size_t)B * p.sample_chunks * 2 * 8 + (size_t)B * 4, kAlign);
  p.ws_bytes = p.greedy_bytes > p.sample_bytes ? p.greedy_bytes : p.sample_bytes;
  return p;
}

orthrus_status check_commit_desc(const orthrus_commit_desc* d) {
  if (d == nullptr) return ORTHRUS_ERR_NULL_PTR;
  if (d->n_layers < 1 || d->batch < 1 || d->n_kv_heads < 1 || d->head_dim < 1 || d->block_k < 1 ||
      d->max_len < 0)
    return ORTHRUS_ERR_BAD_SHAPE;
  if (d->head_dim % 8 != 0 || d->head_dim > 1024 || d->block_k > 1024 || d->max_len > (1 << 30))
    return ORTHRUS_ERR_UNSUPPORTED;
  const long long lb = (long long)d->n_layers * d->batch;  // below 2^62: no overflow
  if (lb > 0x7fffffffLL || lb * d->n_kv_heads > 0x7fffffffLL) return ORTHRUS_ERR_BAD_SHAPE;
  return ORTHRUS_OK;
}

orthrus_status check_kl_sizes(int32_t rows, int32_t vocab, int dtype) {
  if (dtype != ORTHRUS_DTYPE_F32 && dtype != ORTHRUS_DTYPE_BF16) return ORTHRUS_ERR_BAD_SHAPE;
  if (rows < 1 || vocab < 1) return ORTHRUS_ERR_BAD_SHAPE;
  if (rows > 65535 || vocab > kMaxVocab) return ORTHRUS_ERR_UNSUPPORTED;
  return ORTHRUS_OK;
}

struct KlPlan {
  int esize;
  bool vec;
  size_t ws_bytes;
};

KlPlan make_kl_plan(int32_t rows, int32_t vocab, int dtype) {
  (void)rows;
  KlPlan p{};
  p.esize = dtype == ORTHRUS_DTYPE_F32 ? 4 : 2;
  p.vec = ((size_t)vocab * p.esize) % 16 == 0;
  // the row-wise kernel keeps its statistics in registers; the workspace
  // argument stays in the interface, one alignment unit of it reserved
  p.ws_bytes = kAlign;
  return p;
}

// Rows of the AR (clean, causal) part are processed in groups of this many:
// group m is a verify-mode block of rows [32m, 32m+32) over the cache [0, 32m).
constexpr int kTrainArGroup = 32;

orthrus_status check_train_desc(const orthrus_train_attn_desc* d) {
  if (d == nullptr) return ORTHRUS_ERR_NULL_PTR;
  if (d->seq_len < 1 || d->n_blocks < 0 || d->block_k < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 ||
      d->head_dim < 1)
    return ORTHRUS_ERR_BAD_SHAPE;
  if (d->n_q_heads % d->n_kv_heads != 0) return ORTHRUS_ERR_BAD_SHAPE;
  if (!(isfinite(d->softmax_scale) && d->softmax_scale >= 0.0f)) return ORTHRUS_ERR_BAD_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return ORTHRUS_ERR_UNSUPPORTED;
  if (d->block_k > 32 || d->seq_len % kTrainArGroup != 0) return ORTHRUS_ERR_UNSUPPORTED;
  const long long G = d->n_q_heads / d->n_kv_heads;
  if (G * 32 > (1LL << 20)) return ORTHRUS_ERR_BAD_SHAPE;
  if ((long long)(d->seq_len / kTrainArGroup) * d->n_kv_heads > 65535LL ||
      (long long)d->n_blocks * d->n_kv_heads > 65535LL)
    return ORTHRUS_ERR_BAD_SHAPE;
  return ORTHRUS_OK;
}

// One single-split block-attention launch of the training forward.
orthrus_status run_train_part(const orthrus_train_attn_desc* d, int batch, int block_k, int causal,
                              AttnArgs a, void* stream) {
  orthrus_attn_desc ad{};
  ad.batch = batch;
  ad.n_q_heads = d->n_q_heads;
  ad.n_kv_heads = d->n_kv_heads;
  ad.head_dim = d->head_dim;
  ad.block_k = block_k;
  ad.max_len = d->seq_len;
  ad.softmax_scale = d->softmax_scale;
  const AttnPlan plan = make_plan(&ad);
  a.batch = batch;
  a.n_q_heads = d->n_q_heads;
  a.n_kv_heads = d->n_kv_heads;
  a.group = d->n_q_heads / d->n_kv_heads;
  a.block_k = block_k;
  a.head_dim = d->head_dim;
  a.max_len = d->seq_len;
  a.causal = causal;
  a.splits = 1;  // every work-group streams its whole prefix and writes its rows itself
  const float scale = d->softmax_scale > 0.0f ? d->softmax_scale : 1.0f / sqrtf((float)d->head_dim);
  a.scale_log2 = scale * 1.4426950408889634f;
  const hipError_t e = launch_block_attention(a, plan, 3, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_HIP;
}

// Host-side pointer checks of a block-attention call (every one that
// run_attn makes before its first HIP call, for the entry points that must
// finish them before looking anything up on the device).
orthrus_status check_attn_ptrs(const uint16_t* q, const uint16_t* k_blk, const uint16_t* v_blk,
                               const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* cache_len,
                               const uint16_t* out, const float* lse) {
  if (!q || !k_blk || !v_blk || !k_cache || !v_cache || !cache_len || !out) return ORTHRUS_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned4(cache_len) || !aligned16(out) || (lse && !aligned4(lse)))
    return ORTHRUS_ERR_MISALIGNED;
  return ORTHRUS_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; NULL if the lookup failed.
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = e == hipSuccess ? ptr : nullptr;
  });
  return g_scratch_ptr[dev];
}

// true if the byte ranges [p, p+n) and [q, q+m) overlap
bool overlaps(const void* p, size_t n, const void* q, size_t m) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + m && b < a + n;
}

orthrus_status run_greedy(int32_t batch, int32_t block_k, int32_t vocab, const float* logits, const int32_t* cand,
                          const int32_t* blk_len, int32_t* accept_len, int32_t* row_argmax, int32_t* correction,
                          void* workspace, size_t workspace_bytes, void* stream) {
  const orthrus_status st = check_consensus_sizes(batch, block_k, vocab);
  if (st != ORTHRUS_OK) return st;
  if (!logits || !cand || !accept_len || !correction || !workspace) return ORTHRUS_ERR_NULL_PTR;
  if (!aligned16(logits) || !aligned4(cand) || !aligned4(accept_len) || !aligned4(correction) ||
      (row_argmax && !aligned4(row_argmax)) || (blk_len && !aligned4(blk_len)) || !aligned16(workspace))
    return ORTHRUS_ERR_MISALIGNED;
  const ConsensusPlan plan = make_consensus_plan(batch, block_k, vocab);
  if (workspace_bytes < plan.ws_bytes) return ORTHRUS_ERR_WORKSPACE_TOO_SMALL;
  const hipError_t e = launch_consensus_greedy(batch, block_k, vocab, logits, cand, blk_len, accept_len,
                                               row_argmax, correction, workspace, plan,
                                               reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_HIP;
}

orthrus_status run_sample(int32_t batch, int32_t block_k, int32_t vocab, const float* p_target, const float* q_draft,
                          const int32_t* cand, const float* uniforms, const int32_t* blk_len, int32_t* accept_len,
                          int32_t* correction, void* workspace, size_t workspace_bytes, void* stream) {
  const orthrus_status st = check_consensus_sizes(batch, block_k, vocab);
  if (st != ORTHRUS_OK) return st;
  if (!p_target || !q_draft || !cand || !uniforms || !accept_len || !correction || !workspace)
    return ORTHRUS_ERR_NULL_PTR;
  if (!aligned16(p_target) || !aligned16(q_draft) || !aligned4(cand) || !aligned4(uniforms) ||
      !aligned4(accept_len) || !aligned4(correction) || (blk_len && !aligned4(blk_len)) || !aligned16(workspace))
    return ORTHRUS_ERR_MISALIGNED;
  const ConsensusPlan plan = make_consensus_plan(batch, block_k, vocab);
  if (workspace_bytes < plan.ws_bytes) return ORTHRUS_ERR_WORKSPACE_TOO_SMALL;
  const hipError_t e = launch_consensus_sample(batch, block_k, vocab, p_target, q_draft, cand, uniforms, blk_len,
                                               accept_len, correction, workspace, plan,
                                               reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_HIP;
}

orthrus_status run_commit(const orthrus_commit_desc* d, uint16_t* k_cache, uint16_t* v_cache,
                          const uint16_t* k_blk, const uint16_t* v_blk, int32_t* cache_len,
                          const int32_t* accept_len, const int32_t* correction, const int32_t* cand,
                          int32_t* next_anchor, int32_t* tokens, int32_t* n_tokens, int32_t* blk_len,
                          int32_t* accept_stat, int k_min, void* stream) {
  const orthrus_status st = check_commit_desc(d);
  if (st != ORTHRUS_OK) return st;
  if (!k_cache || !v_cache || !k_blk || !v_blk || !cache_len || !accept_len || !correction || !cand ||
      !next_anchor || !tokens || !n_tokens)
    return ORTHRUS_ERR_NULL_PTR;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_blk) || !aligned16(v_blk) ||
      !aligned4(cache_len) || !aligned4(accept_len) || !aligned4(correction) || !aligned4(cand) ||
      !aligned4(next_anchor) || !aligned4(tokens) || !aligned4(n_tokens) || (blk_len && !aligned4(blk_len)) ||
      (accept_stat && !aligned4(accept_stat)))
    return ORTHRUS_ERR_MISALIGNED;
  // the copies read the block while writing the cache: the two must not share memory
  const size_t planes = (size_t)d->n_layers * d->batch * d->n_kv_heads;
  const size_t cache_bytes = planes * d->max_len * d->head_dim * sizeof(uint16_t);
  const size_t blk_bytes = planes * d->block_k * d->head_dim * sizeof(uint16_t);
  if (overlaps(k_cache, cache_bytes, k_blk, blk_bytes) || overlaps(k_cache, cache_bytes, v_blk, blk_bytes) ||
      overlaps(v_cache, cache_bytes, k_blk, blk_bytes) || overlaps(v_cache, cache_bytes, v_blk, blk_bytes) ||
      overlaps(k_cache, cache_bytes, v_cache, cache_bytes))
    return ORTHRUS_ERR_BAD_SHAPE;
  const hipError_t e = launch_cache_commit(d->n_layers, d->batch, d->n_kv_heads, d->head_dim, d->block_k,
                                           d->max_len, k_cache, v_cache, k_blk, v_blk, cache_len, accept_len,
                                           correction, cand, next_anchor, tokens, n_tokens, blk_len, accept_stat,
                                           k_min, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_HIP;
}

}  // namespace
}  // namespace orthrus

using namespace orthrus;

extern "C" {

size_t orthrus_attn_workspace_size(const orthrus_attn_desc* d) {
  if (check_desc(d) != ORTHRUS_OK) return 0;
  return make_plan(d).ws_bytes;
}

int32_t orthrus_attn_num_splits(const orthrus_attn_desc* d) {
  if (check_desc(d) != ORTHRUS_OK) return -1;
  return make_plan(d).splits;
}

orthrus_status orthrus_block_attn(const orthrus_attn_desc* d, int32_t mode, const uint16_t* q,
                                  const uint16_t* k_blk, const uint16_t* v_blk, const uint16_t* k_cache,
                                  const uint16_t* v_cache, const int32_t* cache_len, uint16_t* out,
                                  float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return run_attn(d, (int)mode, q, k_blk, v_blk, k_cache, v_cache, cache_len, out, lse, workspace,
                  workspace_bytes, stream, 3);
}

orthrus_status orthrus_block_attn_dyn(const orthrus_attn_desc* d, int32_t mode, const uint16_t* q,
                                      const uint16_t* k_blk, const uint16_t* v_blk, const uint16_t* k_cache,
                                      const uint16_t* v_cache, const int32_t* cache_len, const int32_t* blk_len,
                                      uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (mode != ORTHRUS_MASK_DIFF_BIDIR && mode != ORTHRUS_MASK_VERIFY_CAUSAL) return ORTHRUS_ERR_BAD_SHAPE;
  if (!blk_len) return ORTHRUS_ERR_NULL_PTR;
  return run_attn(d, (int)mode, q, k_blk, v_blk, k_cache, v_cache, cache_len, out, lse, workspace,
                  workspace_bytes, stream, 3, nullptr, blk_len);
}

orthrus_status orthrus_block_attn_masked(const orthrus_attn_desc* d, const uint16_t* q, const uint16_t* k_blk,
                                         const uint16_t* v_blk, const uint16_t* k_cache, const uint16_t* v_cache,
                                         const int32_t* cache_len, const uint64_t* block_mask, uint16_t* out,
                                         float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return run_attn(d, ORTHRUS_MASK_EXPLICIT, q, k_blk, v_blk, k_cache, v_cache, cache_len, out, lse, workspace,
                  workspace_bytes, stream, 3, block_mask);
}

orthrus_status orthrus_block_attn_partial(const orthrus_attn_desc* d, int32_t mode,
                                          const uint16_t* q, const uint16_t* k_blk, const uint16_t* v_blk,
                                          const uint16_t* k_cache, const uint16_t* v_cache,
                                          const int32_t* cache_len, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  return run_attn(d, (int)mode, q, k_blk, v_blk, k_cache, v_cache, cache_len, nullptr, nullptr, workspace,
                  workspace_bytes, stream, 1);
}

orthrus_status orthrus_block_attn_merge(const orthrus_attn_desc* d, uint16_t* out, float* lse,
                                        const void* workspace, size_t workspace_bytes, void* stream) {
  return run_attn(d, ORTHRUS_MASK_DIFF_BIDIR, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, out, lse,
                  const_cast<void*>(workspace), workspace_bytes, stream, 2);
}

orthrus_status orthrus_block_attn_diff(const orthrus_attn_desc* d, const uint16_t* q, const uint16_t* k_blk,
                                       const uint16_t* v_blk, const uint16_t* k_cache,
                                       const uint16_t* v_cache, const int32_t* cache_len, uint16_t* out,
                                       float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return run_attn(d, ORTHRUS_MASK_DIFF_BIDIR, q, k_blk, v_blk, k_cache, v_cache, cache_len, out, lse,
                  workspace, workspace_bytes, stream, 3);
}

orthrus_status orthrus_block_attn_verify(const orthrus_attn_desc* d, const uint16_t* q,
                                         const uint16_t* k_blk, const uint16_t* v_blk,
                                         const uint16_t* k_cache, const uint16_t* v_cache,
                                         const int32_t* cache_len, uint16_t* out, float* lse,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  return run_attn(d, ORTHRUS_MASK_VERIFY_CAUSAL, q, k_blk, v_blk, k_cache, v_cache, cache_len, out, lse,
                  workspace, workspace_bytes, stream, 3);
}

orthrus_status orthrus_block_attn_noalloc(const orthrus_attn_desc* d, int32_t mode, const uint16_t* q,
                                          const uint16_t* k_blk, const uint16_t* v_blk, const uint16_t* k_cache,
                                          const uint16_t* v_cache, const int32_t* cache_len, uint16_t* out,
                                          float* lse, void* stream) {
  const orthrus_status st = check_desc(d);
  if (st != ORTHRUS_OK) return st;
  if (mode != ORTHRUS_MASK_DIFF_BIDIR && mode != ORTHRUS_MASK_VERIFY_CAUSAL) return ORTHRUS_ERR_BAD_SHAPE;
  if (make_plan(d).ws_bytes > ORTHRUS_NOALLOC_SCRATCH_BYTES) return ORTHRUS_ERR_UNSUPPORTED;
  const orthrus_status pst = check_attn_ptrs(q, k_blk, v_blk, k_cache, v_cache, cache_len, out, lse);
  if (pst != ORTHRUS_OK) return pst;
  void* ws = scratch_address();
  if (ws == nullptr) return ORTHRUS_ERR_HIP;
  return run_attn(d, (int)mode, q, k_blk, v_blk, k_cache, v_cache, cache_len, out, lse, ws,
                  ORTHRUS_NOALLOC_SCRATCH_BYTES, stream, 3);
}

size_t orthrus_consensus_workspace_size(int32_t batch, int32_t block_k, int32_t vocab) {
  if (check_consensus_sizes(batch, block_k, vocab) != ORTHRUS_OK) return 0;
  return make_consensus_plan(batch, block_k, vocab).ws_bytes;
}

orthrus_status orthrus_consensus_greedy(int32_t batch, int32_t block_k, int32_t vocab, const float* logits,
                                        const int32_t* cand, int32_t* accept_len, int32_t* row_argmax,
                                        int32_t* correction, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  return run_greedy(batch, block_k, vocab, logits, cand, nullptr, accept_len, row_argmax, correction, workspace,
                    workspace_bytes, stream);
}

orthrus_status orthrus_consensus_greedy_dyn(int32_t batch, int32_t block_k, int32_t vocab, const float* logits,
                                            const int32_t* cand, const int32_t* blk_len, int32_t* accept_len,
                                            int32_t* row_argmax, int32_t* correction, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  if (!blk_len) return ORTHRUS_ERR_NULL_PTR;
  return run_greedy(batch, block_k, vocab, logits, cand, blk_len, accept_len, row_argmax, correction, workspace,
                    workspace_bytes, stream);
}

orthrus_status orthrus_consensus_sample(int32_t batch, int32_t block_k, int32_t vocab, const float* p_target,
                                        const float* q_draft, const int32_t* cand, const float* uniforms,
                                        int32_t* accept_len, int32_t* correction, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return run_sample(batch, block_k, vocab, p_target, q_draft, cand, uniforms, nullptr, accept_len, correction,
                    workspace, workspace_bytes, stream);
}

orthrus_status orthrus_consensus_sample_dyn(int32_t batch, int32_t block_k, int32_t vocab, const float* p_target,
                                            const float* q_draft, const int32_t* cand, const float* uniforms,
                                            const int32_t* blk_len, int32_t* accept_len, int32_t* correction,
                                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!blk_len) return ORTHRUS_ERR_NULL_PTR;
  return run_sample(batch, block_k, vocab, p_target, q_draft, cand, uniforms, blk_len, accept_len, correction,
                    workspace, workspace_bytes, stream);
}

orthrus_status orthrus_cache_commit(const orthrus_commit_desc* d, uint16_t* k_cache, uint16_t* v_cache,
                                    const uint16_t* k_blk, const uint16_t* v_blk, int32_t* cache_len,
                                    const int32_t* accept_len, const int32_t* correction,
                                    const int32_t* cand, int32_t* next_anchor, int32_t* tokens,
                                    int32_t* n_tokens, void* stream) {
  return run_commit(d, k_cache, v_cache, k_blk, v_blk, cache_len, accept_len, correction, cand, next_anchor,
                    tokens, n_tokens, nullptr, nullptr, 1, stream);
}

orthrus_status orthrus_cache_commit_dyn(const orthrus_commit_desc* d, uint16_t* k_cache, uint16_t* v_cache,
                                        const uint16_t* k_blk, const uint16_t* v_blk, int32_t* cache_len,
                                        const int32_t* accept_len, const int32_t* correction,
                                        const int32_t* cand, int32_t* next_anchor, int32_t* tokens,
                                        int32_t* n_tokens, int32_t* blk_len, int32_t* accept_stat, int32_t k_min,
                                        void* stream) {
  if (!blk_len || !accept_stat) return ORTHRUS_ERR_NULL_PTR;
  if (d && (k_min < 1 || k_min > d->block_k)) return ORTHRUS_ERR_BAD_SHAPE;
  return run_commit(d, k_cache, v_cache, k_blk, v_blk, cache_len, accept_len, correction, cand, next_anchor,
                    tokens, n_tokens, blk_len, accept_stat, k_min, stream);
}

size_t orthrus_kl_workspace_size(int32_t rows, int32_t vocab, int32_t dtype) {
  if (check_kl_sizes(rows, vocab, dtype) != ORTHRUS_OK) return 0;
  return make_kl_plan(rows, vocab, dtype).ws_bytes;
}

orthrus_status orthrus_forward_kl(int32_t rows, int32_t vocab, int32_t dtype, const void* target_logits,
                                  const void* draft_logits, float* kl, void* grad, float grad_scale,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  const orthrus_status st = check_kl_sizes(rows, vocab, dtype);
  if (st != ORTHRUS_OK) return st;
  if (!target_logits || !draft_logits || !kl || !workspace) return ORTHRUS_ERR_NULL_PTR;
  if (!isfinite(grad_scale)) return ORTHRUS_ERR_BAD_SHAPE;
  if (!aligned16(target_logits) || !aligned16(draft_logits) || !aligned4(kl) || (grad && !aligned16(grad)) ||
      !aligned16(workspace))
    return ORTHRUS_ERR_MISALIGNED;
  const KlPlan plan = make_kl_plan(rows, vocab, dtype);
  if (workspace_bytes < plan.ws_bytes) return ORTHRUS_ERR_WORKSPACE_TOO_SMALL;
  const int cus = device_cus();
  if (cus < 1) return ORTHRUS_ERR_HIP;
  const hipError_t e = launch_forward_kl(rows, vocab, plan.esize, plan.vec, target_logits, draft_logits, kl, grad,
                                         grad_scale, cus, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_HIP;
}

orthrus_status orthrus_train_attn_fwd(const orthrus_train_attn_desc* d, const uint16_t* q_ar,
                                      const uint16_t* k_ar, const uint16_t* v_ar, const uint16_t* q_diff,
                                      const uint16_t* k_diff, const uint16_t* v_diff, const int32_t* anchors,
                                      uint16_t* out_ar, float* lse_ar, uint16_t* out_diff, float* lse_diff,
                                      void* stream) {
  const orthrus_status st = check_train_desc(d);
  if (st != ORTHRUS_OK) return st;
  const bool ar = q_ar != nullptr || out_ar != nullptr;
  const bool diff = d->n_blocks > 0;
  if (!k_ar || !v_ar) return ORTHRUS_ERR_NULL_PTR;
  if (ar && (!q_ar || !out_ar)) return ORTHRUS_ERR_NULL_PTR;
  if (diff && (!q_diff || !k_diff || !v_diff || !anchors || !out_diff)) return ORTHRUS_ERR_NULL_PTR;
  if (!aligned16(k_ar) || !aligned16(v_ar) || (ar && (!aligned16(q_ar) || !aligned16(out_ar))) ||
      (lse_ar && !aligned4(lse_ar)) ||
      (diff && (!aligned16(q_diff) || !aligned16(k_diff) || !aligned16(v_diff) || !aligned4(anchors) ||
                !aligned16(out_diff) || (lse_diff && !aligned4(lse_diff)))))
    return ORTHRUS_ERR_MISALIGNED;
  if (device_cus() < 1) return ORTHRUS_ERR_HIP;
  const long long D = d->head_dim, L = d->seq_len, K = d->block_k, NK = (long long)d->n_blocks * d->block_k;
  if (ar) {  // clean rows: groups of 32 causal rows over the clean prefix before the group
    AttnArgs a{};
    a.q = q_ar;
    a.k_blk = k_ar;
    a.v_blk = v_ar;
    a.k_cache = k_ar;
    a.v_cache = v_ar;
    a.cache_len = nullptr;
    a.out = out_ar;
    a.lse = lse_ar;
    a.q_bs = a.o_bs = kTrainArGroup * D;
    a.q_hs = a.o_hs = L * D;
    a.l_bs = kTrainArGroup;
    a.l_hs = L;
    a.blk_bs = kTrainArGroup * D;
    a.blk_gs = L * D;
    a.c_bs = 0;
    a.c_gs = L * D;
    a.len_step = kTrainArGroup;
    const orthrus_status r = run_train_part(d, (int)(L / kTrainArGroup), kTrainArGroup, 1, a, stream);
    if (r != ORTHRUS_OK) return r;
  }
  if (diff) {  // block n: clean prefix [0, anchors[n]) shared by all blocks, plus its own K keys
    AttnArgs a{};
    a.q = q_diff;
    a.k_blk = k_diff;
    a.v_blk = v_diff;
    a.k_cache = k_ar;
    a.v_cache = v_ar;
    a.cache_len = anchors;
    a.out = out_diff;
    a.lse = lse_diff;
    a.q_bs = a.o_bs = K * D;
    a.q_hs = a.o_hs = NK * D;
    a.l_bs = K;
    a.l_hs = NK;
    a.blk_bs = K * D;
    a.blk_gs = NK * D;
    a.c_bs = 0;
    a.c_gs = L * D;
    a.len_step = 0;
    a.rank_blocks = 1;  // the longest prefixes first
    const orthrus_status r = run_train_part(d, d->n_blocks, (int)K, 0, a, stream);
    if (r != ORTHRUS_OK) return r;
  }
  return ORTHRUS_OK;
}

orthrus_status orthrus_train_attn_bwd(const orthrus_train_attn_desc* d, const uint16_t* k_ar,
                                      const uint16_t* v_ar, const uint16_t* q_diff, const uint16_t* k_diff,
                                      const uint16_t* v_diff, const int32_t* anchors, const uint16_t* out_diff,
                                      const float* lse_diff, const uint16_t* d_out_diff, uint16_t* dq_diff,
                                      uint16_t* dk_diff, uint16_t* dv_diff, void* stream) {
  const orthrus_status st = check_train_desc(d);
  if (st != ORTHRUS_OK) return st;
  if ((long long)(d->n_q_heads / d->n_kv_heads) * d->block_k > 128) return ORTHRUS_ERR_UNSUPPORTED;
  if (d->n_blocks == 0) return ORTHRUS_OK;
  if (!k_ar || !v_ar || !q_diff || !k_diff || !v_diff || !anchors || !out_diff || !lse_diff || !d_out_diff ||
      !dq_diff || !dk_diff || !dv_diff)
    return ORTHRUS_ERR_NULL_PTR;
  if (!aligned16(k_ar) || !aligned16(v_ar) || !aligned16(q_diff) || !aligned16(k_diff) || !aligned16(v_diff) ||
      !aligned4(anchors) || !aligned16(out_diff) || !aligned4(lse_diff) || !aligned16(d_out_diff) ||
      !aligned16(dq_diff) || !aligned16(dk_diff) || !aligned16(dv_diff))
    return ORTHRUS_ERR_MISALIGNED;
  if (device_cus() < 1) return ORTHRUS_ERR_HIP;
  TrainBwdArgs a{};
  a.k_ar = k_ar;
  a.v_ar = v_ar;
  a.q_diff = q_diff;
  a.k_diff = k_diff;
  a.v_diff = v_diff;
  a.anchors = anchors;
  a.out_diff = out_diff;
  a.lse_diff = lse_diff;
  a.d_out = d_out_diff;
  a.dq = dq_diff;
  a.dk = dk_diff;
  a.dv = dv_diff;
  a.seq_len = d->seq_len;
  a.n_blocks = d->n_blocks;
  a.block_k = d->block_k;
  a.group = d->n_q_heads / d->n_kv_heads;
  a.n_kv_heads = d->n_kv_heads;
  a.head_dim = d->head_dim;
  a.scale = d->softmax_scale > 0.0f ? d->softmax_scale : 1.0f / sqrtf((float)d->head_dim);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  const hipError_t e = launch_train_bwd(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_HIP;
}

orthrus_status orthrus_tree_masks(int32_t batch, int32_t block_k, const int32_t* parent, uint64_t* mask,
                                  void* stream) {
  if (batch < 1 || block_k < 1) return ORTHRUS_ERR_BAD_SHAPE;
  if (block_k > 64) return ORTHRUS_ERR_UNSUPPORTED;
  if ((long long)batch * block_k > 0x7fffffffLL) return ORTHRUS_ERR_BAD_SHAPE;
  if (!parent || !mask) return ORTHRUS_ERR_NULL_PTR;
  if (!aligned4(parent) || (reinterpret_cast<uintptr_t>(mask) & 7u)) return ORTHRUS_ERR_MISALIGNED;
  const hipError_t e = launch_tree_masks(batch, block_k, parent, mask, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_HIP;
}

orthrus_status orthrus_consensus_tree_greedy(int32_t batch, int32_t block_k, int32_t vocab, const float* logits,
                                             const int32_t* tokens, const int32_t* parent, int32_t* accept_len,
                                             int32_t* path, int32_t* correction, int32_t* row_argmax,
                                             void* workspace, size_t workspace_bytes, void* stream) {
  const orthrus_status st = check_consensus_sizes(batch, block_k, vocab);
  if (st != ORTHRUS_OK) return st;
  if (!logits || !tokens || !parent || !accept_len || !path || !correction || !workspace)
    return ORTHRUS_ERR_NULL_PTR;
  if (!aligned16(logits) || !aligned4(tokens) || !aligned4(parent) || !aligned4(accept_len) || !aligned4(path) ||
      !aligned4(correction) || (row_argmax && !aligned4(row_argmax)) || !aligned16(workspace))
    return ORTHRUS_ERR_MISALIGNED;
  const ConsensusPlan plan = make_consensus_plan(batch, block_k, vocab);
  if (workspace_bytes < plan.ws_bytes) return ORTHRUS_ERR_WORKSPACE_TOO_SMALL;
  const hipError_t e = launch_consensus_tree_greedy(batch, block_k, vocab, logits, tokens, parent, accept_len, path,
                                                    correction, row_argmax, workspace, plan,
                                                    reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_HIP;
}

orthrus_status orthrus_cache_commit_path(const orthrus_commit_desc* d, uint16_t* k_cache, uint16_t* v_cache,
                                         const uint16_t* k_blk, const uint16_t* v_blk, int32_t* cache_len,
                                         const int32_t* accept_len, const int32_t* path, const int32_t* node_tokens,
                                         const int32_t* correction, int32_t* next_anchor, int32_t* tokens,
                                         int32_t* n_tokens, void* stream) {
  const orthrus_status st = check_commit_desc(d);
  if (st != ORTHRUS_OK) return st;
  if (!k_cache || !v_cache || !k_blk || !v_blk || !cache_len || !accept_len || !path || !node_tokens ||
      !correction || !next_anchor || !tokens || !n_tokens)
    return ORTHRUS_ERR_NULL_PTR;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_blk) || !aligned16(v_blk) ||
      !aligned4(cache_len) || !aligned4(accept_len) || !aligned4(path) || !aligned4(node_tokens) ||
      !aligned4(correction) || !aligned4(next_anchor) || !aligned4(tokens) || !aligned4(n_tokens))
    return ORTHRUS_ERR_MISALIGNED;
  const size_t planes = (size_t)d->n_layers * d->batch * d->n_kv_heads;
  const size_t cache_bytes = planes * d->max_len * d->head_dim * sizeof(uint16_t);
  const size_t blk_bytes = planes * d->block_k * d->head_dim * sizeof(uint16_t);
  if (overlaps(k_cache, cache_bytes, k_blk, blk_bytes) || overlaps(k_cache, cache_bytes, v_blk, blk_bytes) ||
      overlaps(v_cache, cache_bytes, k_blk, blk_bytes) || overlaps(v_cache, cache_bytes, v_blk, blk_bytes) ||
      overlaps(k_cache, cache_bytes, v_cache, cache_bytes))
    return ORTHRUS_ERR_BAD_SHAPE;
  const hipError_t e = launch_cache_commit_path(d->n_layers, d->batch, d->n_kv_heads, d->head_dim, d->block_k,
                                                d->max_len, k_cache, v_cache, k_blk, v_blk, cache_len, accept_len,
                                                path, node_tokens, correction, next_anchor, tokens, n_tokens,
                                                reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_HIP;
}

size_t orthrus_topk_workspace_size(int32_t rows, int32_t vocab, int32_t m) {
  if (rows < 1 || vocab < 1 || m < 1 || m > 32 || m > vocab || rows > 65535 || vocab > kMaxVocab) return 0;
  const size_t chunks = (size_t)topk_chunks(vocab);
  return round_up((size_t)rows * chunks * ((size_t)m * 8 + 8), kAlign);
}

orthrus_status orthrus_topk_logprobs(int32_t rows, int32_t vocab, int32_t m, const float* logits, float* logp,
                                     int32_t* idx, void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 1 || vocab < 1 || m < 1 || m > vocab) return ORTHRUS_ERR_BAD_SHAPE;
  if (m > 32 || rows > 65535 || vocab > kMaxVocab) return ORTHRUS_ERR_UNSUPPORTED;
  if (!logits || !logp || !idx || !workspace) return ORTHRUS_ERR_NULL_PTR;
  if (!aligned4(logits) || !aligned4(logp) || !aligned4(idx) || !aligned16(workspace))
    return ORTHRUS_ERR_MISALIGNED;
  if (workspace_bytes < orthrus_topk_workspace_size(rows, vocab, m)) return ORTHRUS_ERR_WORKSPACE_TOO_SMALL;
  const hipError_t e = launch_topk_logprobs(rows, vocab, m, logits, logp, idx, workspace,
                                            reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_HIP;
}

orthrus_status orthrus_tree_build(int32_t batch, int32_t depth, int32_t m, int32_t n_nodes, const float* logp,
                                  const int32_t* tok, const int32_t* anchor, int32_t* parent, int32_t* tokens,
                                  int32_t* node_depth, void* stream) {
  if (batch < 1 || depth < 0 || m < 1 || n_nodes < 1) return ORTHRUS_ERR_BAD_SHAPE;
  if (n_nodes > 64 || m > 1024 || depth > 65535) return ORTHRUS_ERR_UNSUPPORTED;
  if ((depth > 0 && (!logp || !tok)) || !anchor || !parent || !tokens || !node_depth) return ORTHRUS_ERR_NULL_PTR;
  if ((logp && !aligned4(logp)) || (tok && !aligned4(tok)) || !aligned4(anchor) || !aligned4(parent) ||
      !aligned4(tokens) || !aligned4(node_depth))
    return ORTHRUS_ERR_MISALIGNED;
  const hipError_t e = launch_tree_build(batch, depth, m, n_nodes, logp, tok, anchor, parent, tokens, node_depth,
                                         reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_HIP;
}

const char* orthrus_status_string(int32_t status) {
  switch (status) {
    case ORTHRUS_OK: return "ORTHRUS_OK";
    case ORTHRUS_ERR_NULL_PTR: return "ORTHRUS_ERR_NULL_PTR: a required pointer is NULL";
    case ORTHRUS_ERR_BAD_SHAPE: return "ORTHRUS_ERR_BAD_SHAPE: a size is out of range or inconsistent";
    case ORTHRUS_ERR_UNSUPPORTED: return "ORTHRUS_ERR_UNSUPPORTED: valid size that this build does not support";
    case ORTHRUS_ERR_MISALIGNED: return "ORTHRUS_ERR_MISALIGNED: a device pointer is not 16-byte aligned";
    case ORTHRUS_ERR_WORKSPACE_TOO_SMALL: return "ORTHRUS_ERR_WORKSPACE_TOO_SMALL: workspace below the size query";
    case ORTHRUS_ERR_HIP: return "ORTHRUS_ERR_HIP: the HIP runtime refused the launch";
  }
  return "ORTHRUS_ERR_UNKNOWN";
}

}  // extern "C"
