// Closing a decode cycle on the device: the verified rows of the AR verify
// block go into the shared KV cache, and the per-sequence state (length,
// emitted tokens, next anchor) advances -- all stream-ordered, with no host
// synchronisation (Orthrus paper notes §4.1 step 3: keep the matching
// candidates, emit the correction, cut the cache back to t+j; §2.2: only the
// AR path writes the cache).
//
// The unverified rows are simply never written, so the cut-back costs
// nothing.  For one sequence with length t and a accepted candidates, verify
// rows 0..r-1 (r = a + [a < K]: the anchor and the accepted candidates) are
// one contiguous run of r*D bf16 in the block and land as one contiguous run
// at row t of the same (layer, KV head) plane of the cache, so each plane is a
// plain 16-byte-vector copy of at most K*D*2 bytes.
//
// Two launches: the row copies (every work-group reads the old length) and
// then the state update, which rewrites the length in place.  Stream order
// keeps the second behind the first.
#include "common.h"

namespace orthrus {
namespace {

struct CommitArgs {
  uint16_t* k_cache;
  uint16_t* v_cache;
  const uint16_t* k_blk;
  const uint16_t* v_blk;
  int32_t* cache_len;
  const int32_t* accept_len;
  const int32_t* correction;
  const int32_t* cand;
  int32_t* next_anchor;
  int32_t* tokens;
  int32_t* n_tokens;
  // dynamic block sizes: NULL, or the live block length per sequence
  // (clamped to [1, block_k]), rewritten in place with the next cycle's, and
  // each sequence's packed acceptance statistics (see next_block_len)
  int32_t* blk_len;
  int32_t* accept_stat;
  int k_min;       // floor of the block-length rule
  int planes;      // n_layers * B * Hkv
  int batch, n_kv_heads, head_dim, block_k, max_len;
};

constexpr int kCommitThreads = 256;

// Rows a sequence commits, or -1 if the commit is refused (length or accept
// count out of range, or not enough room left in the cache).
__device__ __forceinline__ int commit_rows(int t, int a, int K, int max_len) {
  if (t < 0 || a < 0 || a > K) return -1;
  const int r = a < K ? a + 1 : K;
  return t <= max_len - r ? r : -1;
}

// Block length of sequence b in this cycle: its first k_b positions.
__device__ __forceinline__ int live_k(const CommitArgs& a, int b) {
  if (a.blk_len == nullptr) return a.block_k;
  const int k = a.blk_len[b];
  return k < 1 ? 1 : (k > a.block_k ? a.block_k : k);
}

// The block-length rule (Orthrus paper notes §7.4, §9.6: a large block where
// acceptance is high, a small one where it is low).  Each sequence's
// statistic packs A (high 16 bits) and N (low 16 bits): accepted and tested
// draft candidates, in units of 1/16, decayed by 7/8 per committed cycle --
// A / N estimates the probability p that a candidate matches once the ones
// before it did.  The next block is the smallest power of two k with
// p^k <= 1/8 (p in Q16, powers by squaring with the floor), clamped to
// [k_min, cap]; cap while nothing has been seen (N = 0).  Integers only, so
// every implementation takes the same decision.
__device__ __forceinline__ uint32_t next_accept_stat(uint32_t stat, int a, int k) {
  uint32_t A = stat >> 16, N = stat & 0xFFFFu;
  if (A > N) A = N;
  const uint32_t tested = (uint32_t)(a + (a < k ? 1 : 0));
  N = min(N - N / 8 + 16u * tested, 0xFFFFu);  // both fields saturate
  A = min(A - A / 8 + 16u * (uint32_t)a, N);
  return (A << 16) | N;
}

__device__ __forceinline__ int next_block_len(uint32_t stat, int cap, int k_min) {
  const uint32_t A = min(stat >> 16, stat & 0xFFFFu), N = stat & 0xFFFFu;
  int k = cap;
  if (N != 0) {
    unsigned long long x = ((unsigned long long)A << 16) / N;  // p in Q16
    k = 1;
    while (k < cap && x > 8192ull) {  // 8192: 1/8
      x = (x * x) >> 16;
      k *= 2;
    }
  }
  return min(max(min(k, cap), k_min), cap);
}

// grid.x = planes, grid.y = 2 (keys, values)
__global__ __launch_bounds__(kCommitThreads) void commit_rows_kernel(const CommitArgs a) {
  const int plane = blockIdx.x;
  const int b = (plane / a.n_kv_heads) % a.batch;
  const int t = a.cache_len[b];
  const int r = commit_rows(t, a.accept_len[b], live_k(a, b), a.max_len);
  if (r <= 0) return;
  const bool vals = blockIdx.y != 0;
  const uint16_t* src = (vals ? a.v_blk : a.k_blk) + (size_t)plane * a.block_k * a.head_dim;
  uint16_t* dst = (vals ? a.v_cache : a.k_cache) + ((size_t)plane * a.max_len + t) * a.head_dim;
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  const int n = r * (a.head_dim / 8);  // 16-byte vectors in the run
  for (int i = threadIdx.x; i < n; i += kCommitThreads) d4[i] = s4[i];
}

// one thread per sequence
__global__ __launch_bounds__(kCommitThreads) void commit_state_kernel(const CommitArgs a) {
  const int b = blockIdx.x * kCommitThreads + threadIdx.x;
  if (b >= a.batch) return;
  const int K = a.block_k;  // row stride of cand and tokens
  const int kb = live_k(a, b);
  const int t = a.cache_len[b];
  const int acc = a.accept_len[b];
  const int r = commit_rows(t, acc, kb, a.max_len);
  int32_t* tok = a.tokens + (size_t)b * K;
  if (r < 0) {
    for (int i = 0; i < K; ++i) tok[i] = -1;
    a.n_tokens[b] = 0;
    a.next_anchor[b] = -1;
    if (a.blk_len != nullptr) a.blk_len[b] = kb;  // the statistics stay
    return;
  }
  const int32_t* cd = a.cand + (size_t)b * K;
  for (int i = 0; i < acc; ++i) tok[i] = cd[i];
  int last = acc > 0 ? cd[acc - 1] : -1;
  int n = acc;
  if (acc < kb) {
    last = a.correction[b];
    tok[n++] = last;
  }
  for (int i = n; i < K; ++i) tok[i] = -1;
  a.n_tokens[b] = n;
  a.next_anchor[b] = last;
  a.cache_len[b] = t + r;
  if (a.blk_len != nullptr) {
    const uint32_t st = next_accept_stat((uint32_t)a.accept_stat[b], acc, kb);
    a.accept_stat[b] = (int32_t)st;
    a.blk_len[b] = next_block_len(st, K, a.k_min);
  }
}

// ---- commit of an accepted tree path: rows path[0..a] (root first) of the
// verify block go to cache rows t..t+a; the correction is always emitted and
// becomes the next anchor.  A commit is refused (nothing written, length
// kept, n_tokens 0) if t < 0, a outside [0, K-1], t + a + 1 > max_len, or a
// path node outside [0, K).
struct PathArgs {
  CommitArgs c;
  const int32_t* path;
  const int32_t* node_tokens;
};

__device__ __forceinline__ int path_rows(const PathArgs& p, int b) {
  const int t = p.c.cache_len[b], a = p.c.accept_len[b], K = p.c.block_k;
  if (t < 0 || a < 0 || a > K - 1 || t > p.c.max_len - (a + 1)) return -1;
  const int32_t* pth = p.path + (size_t)b * K;
  for (int i = 0; i <= a; ++i)
    if (pth[i] < 0 || pth[i] >= K) return -1;
  return a + 1;
}

// grid.x = planes, grid.y = 2 (keys, values)
__global__ __launch_bounds__(kCommitThreads) void commit_path_rows_kernel(const PathArgs p) {
  const CommitArgs& a = p.c;
  const int plane = blockIdx.x;
  const int b = (plane / a.n_kv_heads) % a.batch;
  const int r = path_rows(p, b);
  if (r <= 0) return;
  const int t = a.cache_len[b];
  const bool vals = blockIdx.y != 0;
  const uint16_t* src = (vals ? a.v_blk : a.k_blk) + (size_t)plane * a.block_k * a.head_dim;
  uint16_t* dst = (vals ? a.v_cache : a.k_cache) + ((size_t)plane * a.max_len + t) * a.head_dim;
  const int32_t* pth = p.path + (size_t)b * a.block_k;
  const int vpr = a.head_dim / 8;  // 16-byte vectors per row
  for (int n = threadIdx.x; n < r * vpr; n += kCommitThreads) {
    const int i = n / vpr, c = n % vpr;
    reinterpret_cast<uint4*>(dst + (size_t)i * a.head_dim)[c] =
        reinterpret_cast<const uint4*>(src + (size_t)pth[i] * a.head_dim)[c];
  }
}

__global__ __launch_bounds__(kCommitThreads) void commit_path_state_kernel(const PathArgs p) {
  const CommitArgs& a = p.c;
  const int b = blockIdx.x * kCommitThreads + threadIdx.x;
  if (b >= a.batch) return;
  const int K = a.block_k;
  const int r = path_rows(p, b);
  int32_t* tok = a.tokens + (size_t)b * K;
  if (r < 0) {
    for (int i = 0; i < K; ++i) tok[i] = -1;
    a.n_tokens[b] = 0;
    a.next_anchor[b] = -1;
    return;
  }
  const int32_t* pth = p.path + (size_t)b * K;
  const int32_t* nt = p.node_tokens + (size_t)b * K;
  const int acc = r - 1;
  for (int i = 0; i < acc; ++i) tok[i] = nt[pth[i + 1]];
  const int corr = a.correction[b];
  tok[acc] = corr;
  for (int i = acc + 1; i < K; ++i) tok[i] = -1;
  a.n_tokens[b] = r;
  a.next_anchor[b] = corr;
  a.cache_len[b] = a.cache_len[b] + r;
}

}  // namespace

hipError_t launch_cache_commit_path(int n_layers, int batch, int n_kv_heads, int head_dim, int block_k,
                                    int max_len, uint16_t* k_cache, uint16_t* v_cache, const uint16_t* k_blk,
                                    const uint16_t* v_blk, int32_t* cache_len, const int32_t* accept_len,
                                    const int32_t* path, const int32_t* node_tokens, const int32_t* correction,
                                    int32_t* next_anchor, int32_t* tokens, int32_t* n_tokens, hipStream_t stream) {
  PathArgs p{};
  CommitArgs& a = p.c;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_blk = k_blk;
  a.v_blk = v_blk;
  a.cache_len = cache_len;
  a.accept_len = accept_len;
  a.correction = correction;
  a.cand = nullptr;
  a.next_anchor = next_anchor;
  a.tokens = tokens;
  a.n_tokens = n_tokens;
  a.planes = n_layers * batch * n_kv_heads;
  a.batch = batch;
  a.n_kv_heads = n_kv_heads;
  a.head_dim = head_dim;
  a.block_k = block_k;
  a.max_len = max_len;
  p.path = path;
  p.node_tokens = node_tokens;
  hipLaunchKernelGGL(commit_path_rows_kernel, dim3(a.planes, 2), dim3(kCommitThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(commit_path_state_kernel, dim3((batch + kCommitThreads - 1) / kCommitThreads),
                     dim3(kCommitThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_cache_commit(int n_layers, int batch, int n_kv_heads, int head_dim, int block_k,
                               int max_len, uint16_t* k_cache, uint16_t* v_cache, const uint16_t* k_blk,
                               const uint16_t* v_blk, int32_t* cache_len, const int32_t* accept_len,
                               const int32_t* correction, const int32_t* cand, int32_t* next_anchor,
                               int32_t* tokens, int32_t* n_tokens, int32_t* blk_len, int32_t* accept_stat,
                               int k_min, hipStream_t stream) {
  CommitArgs a{};
  a.blk_len = blk_len;
  a.accept_stat = accept_stat;
  a.k_min = k_min;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_blk = k_blk;
  a.v_blk = v_blk;
  a.cache_len = cache_len;
  a.accept_len = accept_len;
  a.correction = correction;
  a.cand = cand;
  a.next_anchor = next_anchor;
  a.tokens = tokens;
  a.n_tokens = n_tokens;
  a.planes = n_layers * batch * n_kv_heads;
  a.batch = batch;
  a.n_kv_heads = n_kv_heads;
  a.head_dim = head_dim;
  a.block_k = block_k;
  a.max_len = max_len;
  hipLaunchKernelGGL(commit_rows_kernel, dim3(a.planes, 2), dim3(kCommitThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(commit_state_kernel, dim3((batch + kCommitThreads - 1) / kCommitThreads),
                     dim3(kCommitThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace orthrus
