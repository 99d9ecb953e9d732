// Draft trees for tree verification (Orthrus paper notes §7.4-7.5: verify a
// tree of candidate prefixes built from the K diffusion marginals, DDTree
// style, instead of one chain):
//  * topk_*: the m largest logits of every row (ties: lower index first) and
//    their log-probabilities logit - logsumexp(row) -- the per-position
//    marginals a tree is built from;
//  * tree_build_kernel: best-first trees, one wave per sequence: every
//    candidate child (parent node, rank) sits in one lane with its float32
//    score = score(parent) + logp[depth(parent)][rank]; each step takes the
//    best candidate (score, then lower parent, then lower rank, as one
//    order-preserving 64-bit key), makes it a node, and replaces it by the
//    parent's next rank and the new node's first child;
//  * tree_mask_kernel: the ancestor-or-self bitmask of every node, the block
//    mask of the tree-verify attention.
#include "common.h"
#include "order_keys.h"

#include <math.h>

namespace orthrus {
namespace {

using namespace keys;

constexpr int kTreeThreads = 256;
constexpr int kTreeMaxNodes = 64;  // nodes per tree (one wave holds them all)
constexpr int kTopkPerThread = 16;
constexpr int kTopkChunk = kTopkPerThread * kTreeThreads;
constexpr float kLog2eT = 1.4426950408889634f;

__global__ __launch_bounds__(kTreeThreads) void tree_mask_kernel(int batch, int K, const int32_t* parent,
                                                                 uint64_t* mask) {
  const int n = blockIdx.x * kTreeThreads + threadIdx.x;
  if (n >= batch * K) return;
  const int b = n / K, i = n % K;
  const int32_t* par = parent + (size_t)b * K;
  uint64_t m = 0;
  int j = i;
  for (int step = 0; step < K; ++step) {  // at most K links
    m |= 1ull << j;
    if (j == 0) break;
    const int p = par[j];
    if (p < 0 || p >= j) break;  // an unused node or a malformed link ends the walk
    j = p;
  }
  mask[n] = m;
}

// Wave reductions in registers, the result in every lane, without LDS: the
// partners at the six levels are lane ^ 1 and lane ^ 2 (quad permutes), the
// mirrored quad of the 8-lane half and the mirrored half of the 16-lane row
// (DPP), then lane ^ 16 and lane ^ 32 (permlane swaps).  Each lane combines
// its value with its partner's, so after six levels every lane holds the
// result; for sums both lanes of a pair add the same two values, so every
// lane ends with the same bits.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_partner(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t partner16(uint32_t x) {  // lane ^ 16
  const auto sw = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return ((threadIdx.x >> 4) & 1) ? sw[0] : sw[1];
}
__device__ __forceinline__ uint32_t partner32(uint32_t x) {  // lane ^ 32
  const auto sw = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return ((threadIdx.x >> 5) & 1) ? sw[0] : sw[1];
}
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce32(uint32_t v, Op op) {
  v = op(v, dpp_partner<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = op(v, dpp_partner<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = op(v, dpp_partner<0x141>(v));  // row_half_mirror
  v = op(v, dpp_partner<0x140>(v));  // row_mirror
  v = op(v, partner16(v));
  v = op(v, partner32(v));
  return v;
}
__device__ __forceinline__ float wave_max_f_regs(float v) {
  return __uint_as_float(wave_reduce32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_sum_f_regs(float v) {
  return __uint_as_float(wave_reduce32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}
__device__ __forceinline__ unsigned long long pick_max(unsigned long long v, uint32_t ohi, uint32_t olo) {
  const unsigned long long o = ((unsigned long long)ohi << 32) | olo;
  return o > v ? o : v;
}
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_max_step(unsigned long long v) {
  return pick_max(v, dpp_partner<CTRL>((uint32_t)(v >> 32)), dpp_partner<CTRL>((uint32_t)v));
}
__device__ __forceinline__ unsigned long long wave_max64_regs(unsigned long long v) {
  v = dpp_max_step<0xB1>(v);
  v = dpp_max_step<0x4E>(v);
  v = dpp_max_step<0x141>(v);
  v = dpp_max_step<0x140>(v);
  v = pick_max(v, partner16((uint32_t)(v >> 32)), partner16((uint32_t)v));
  v = pick_max(v, partner32((uint32_t)(v >> 32)), partner32((uint32_t)v));
  return v;
}

__device__ __forceinline__ float block_max_f(float v, float* red) {
  v = wave_max_f_regs(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_sum_f(float v, float* red) {
  v = wave_sum_f_regs(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}
__device__ __forceinline__ unsigned long long block_max_k(unsigned long long v, unsigned long long* red) {
  v = wave_max64_regs(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return umax64(umax64(red[0], red[1]), umax64(red[2], red[3]));
}

// grid (chunks, rows): chunk maximum, exponential sum and top-m keys
__global__ __launch_bounds__(kTreeThreads) void topk_partial_kernel(const float* __restrict__ logits, int vocab,
                                                                    int m, float* __restrict__ part_ml,
                                                                    unsigned long long* __restrict__ part_keys) {
  __shared__ float redf[4];
  __shared__ unsigned long long redk[4];
  const int c = blockIdx.x;
  const size_t row = blockIdx.y;
  const int chunks = gridDim.x;
  const float* rp = logits + row * (size_t)vocab;
  float x[kTopkPerThread];
  unsigned long long key[kTopkPerThread];
  float mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < kTopkPerThread; ++i) {
    const int e = c * kTopkChunk + i * kTreeThreads + (int)threadIdx.x;
    const bool ok = e < vocab;
    x[i] = ok ? rp[e] : -__builtin_inff();
    key[i] = ok ? pack_key(x[i], (uint32_t)e) : 0ull;
    mx = fmaxf(mx, x[i]);
  }
  const float M = block_max_f(mx, redf);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kTopkPerThread; ++i)
    if (key[i] != 0ull) s += __builtin_amdgcn_exp2f((x[i] - M) * kLog2eT);
  const float S = block_sum_f(s, redf);
  const size_t slot = row * chunks + c;
  unsigned long long last = ~0ull;
  for (int r = 0; r < m; ++r) {
    unsigned long long best = 0ull;
#pragma unroll
    for (int i = 0; i < kTopkPerThread; ++i) best = umax64(best, key[i] < last ? key[i] : 0ull);
    last = block_max_k(best, redk);
    if (threadIdx.x == 0) part_keys[slot * m + r] = last;
  }
  if (threadIdx.x == 0) {
    part_ml[slot * 2] = M;
    part_ml[slot * 2 + 1] = S;
  }
}

// one wave per row: log-sum-exp over the chunks and the merged top-m
__global__ __launch_bounds__(kTreeThreads) void topk_finalize_kernel(int rows, int chunks, int m,
                                                                     const float* __restrict__ part_ml,
                                                                     const unsigned long long* __restrict__ part_keys,
                                                                     float* __restrict__ logp,
                                                                     int32_t* __restrict__ idx) {
  const int row = blockIdx.x * (kTreeThreads / 64) + (int)(threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const float* ml = part_ml + (size_t)row * chunks * 2;
  float M = -__builtin_inff();
  for (int c = lane; c < chunks; c += 64) M = fmaxf(M, ml[2 * c]);
  M = wave_max_f_regs(M);
  float S = 0.0f;
  for (int c = lane; c < chunks; c += 64) S = fmaf(ml[2 * c + 1], __builtin_amdgcn_exp2f((ml[2 * c] - M) * kLog2eT), S);
  S = wave_sum_f_regs(S);
  const float lse = M + logf(S);
  const unsigned long long* ks = part_keys + (size_t)row * chunks * m;
  unsigned long long last = ~0ull;
  for (int r = 0; r < m; ++r) {
    unsigned long long best = 0ull;
    for (int c = lane; c < chunks; c += 64)
      for (int j = 0; j < m; ++j) {
        const unsigned long long k = ks[(size_t)c * m + j];
        best = umax64(best, k < last ? k : 0ull);
      }
    last = wave_max64_regs(best);
    if (lane == 0) {
      logp[(size_t)row * m + r] = key_value((uint32_t)(last >> 32)) - lse;
      idx[(size_t)row * m + r] = (int32_t)(0xFFFFFFFFu - (uint32_t)(last & 0xFFFFFFFFull));
    }
  }
}

__device__ __forceinline__ unsigned long long cand_key(float score, int parent, int rank) {
  return ((unsigned long long)order_key(score) << 32) | ((unsigned long long)(0xFFFF - parent) << 16) |
         (unsigned long long)(0xFFFF - rank);
}

// one wave per sequence; n <= 64 nodes, so every live candidate has a lane
__global__ __launch_bounds__(64) void tree_build_kernel(int Dd, int m, int n, const float* __restrict__ logp,
                                                        const int32_t* __restrict__ tok,
                                                        const int32_t* __restrict__ anchor, int32_t* parent,
                                                        int32_t* tokens, int32_t* node_depth) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const float* lp = logp + (size_t)b * Dd * m;
  const int32_t* tk = tok + (size_t)b * Dd * m;
  int32_t* po = parent + (size_t)b * n;
  int32_t* to = tokens + (size_t)b * n;
  int32_t* dout = node_depth + (size_t)b * n;
  if (lane < n) {
    po[lane] = -1;
    to[lane] = lane == 0 ? anchor[b] : -1;
    dout[lane] = 0;
  }
  // The reachable part of this sequence's marginals, staged in LDS once: a
  // tree of n <= 64 nodes reaches depth n - 1 <= 63 at most, and a parent's
  // rank r at most n - 2, so depths < 64 and ranks < 64 cover every step.
  // Each step then reads LDS instead of waiting on a global load.
  __shared__ float slp[kTreeMaxNodes * kTreeMaxNodes];
  __shared__ int32_t stk[kTreeMaxNodes * kTreeMaxNodes];
  const int dd = Dd < kTreeMaxNodes ? Dd : kTreeMaxNodes;
  const int mm = m < kTreeMaxNodes ? m : kTreeMaxNodes;
  for (int e = lane; e < dd * mm; e += 64) {
    const int d = e / mm, r = e % mm;
    slp[e] = lp[(size_t)d * m + r];
    stk[e] = tk[(size_t)d * m + r];
  }
  __syncthreads();
  float nscore = 0.0f;  // lane j: score of node j
  int ndep = 0;         // lane j: depth of node j
  bool cv = false;      // this lane's candidate slot
  float cs = 0.0f;
  int cp = 0, cr = 0;
  if (lane == 0 && Dd > 0 && m > 0) {
    cv = true;
    cs = 0.0f + slp[0];
  }
  for (int made = 1; made < n; ++made) {
    const unsigned long long key = cv ? cand_key(cs, cp, cr) : 0ull;
    const unsigned long long best = wave_max64_regs(key);
    if (best == 0ull) break;
    // winner and p are the same in every lane: read the values straight from
    // their lanes (readlane) rather than through an LDS shuffle
    const int winner = __builtin_ctzll(__ballot(key == best));
    const int p = __builtin_amdgcn_readlane(cp, winner), r = __builtin_amdgcn_readlane(cr, winner);
    const float s = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(cs), winner));
    const int d = __builtin_amdgcn_readlane(ndep, p);
    const float ps = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(nscore), p));
    if (lane == made) {
      nscore = s;
      ndep = d + 1;
    }
    if (lane == 0) {
      po[made] = p;
      to[made] = stk[d * mm + r];
      dout[made] = d + 1;
    }
    if (lane == winner) {  // the parent's next-ranked child takes the slot
      if (r + 1 < m) {
        cs = ps + slp[d * mm + r + 1];
        cr = r + 1;
      } else {
        cv = false;
      }
    }
    if (d + 1 < Dd) {  // the new node's first child goes to a free lane
      const int slot = __builtin_ctzll(__ballot(!cv));
      if (lane == slot) {
        cv = true;
        cs = s + slp[(d + 1) * mm];
        cp = made;
        cr = 0;
      }
    }
  }
}

}  // namespace

hipError_t launch_tree_masks(int batch, int block_k, const int32_t* parent, uint64_t* mask, hipStream_t stream) {
  const int total = batch * block_k;
  hipLaunchKernelGGL(tree_mask_kernel, dim3((total + kTreeThreads - 1) / kTreeThreads), dim3(kTreeThreads), 0,
                     stream, batch, block_k, parent, mask);
  return hipGetLastError();
}

int topk_chunks(int vocab) { return (vocab + kTopkChunk - 1) / kTopkChunk; }

hipError_t launch_topk_logprobs(int rows, int vocab, int m, const float* logits, float* logp, int32_t* idx,
                                void* workspace, hipStream_t stream) {
  const int chunks = topk_chunks(vocab);
  auto* keys_ws = reinterpret_cast<unsigned long long*>(workspace);
  auto* ml = reinterpret_cast<float*>(keys_ws + (size_t)rows * chunks * m);
  hipLaunchKernelGGL(topk_partial_kernel, dim3(chunks, rows), dim3(kTreeThreads), 0, stream, logits, vocab, m, ml,
                     keys_ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int per = kTreeThreads / 64;
  hipLaunchKernelGGL(topk_finalize_kernel, dim3((rows + per - 1) / per), dim3(kTreeThreads), 0, stream, rows,
                     chunks, m, ml, keys_ws, logp, idx);
  return hipGetLastError();
}

hipError_t launch_tree_build(int batch, int depth, int m, int n_nodes, const float* logp, const int32_t* tok,
                             const int32_t* anchor, int32_t* parent, int32_t* tokens, int32_t* node_depth,
                             hipStream_t stream) {
  hipLaunchKernelGGL(tree_build_kernel, dim3(batch), dim3(64), 0, stream, depth, m, n_nodes, logp, tok, anchor,
                     parent, tokens, node_depth);
  return hipGetLastError();
}

}  // namespace orthrus
