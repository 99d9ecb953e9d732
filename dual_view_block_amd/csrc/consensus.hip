// In-model consensus for gfx950: greedy argmax matching and exact
// rejection sampling (Orthrus paper notes, zhangshuibai.github.io, §4.1 step
// 3, §4.2, §4.3 and §7.2).
//
// Greedy: the verify logits [B, K, V] are scanned once.  A row's argmax is the
// maximum of a 64-bit key (order-preserving float bits << 32 | ~index), so the
// lowest index wins ties, NaN (canonical key 0xFFFFFFFF) beats every number,
// and -0 is folded onto +0.  Reduction order cannot change a max, so the
// result is bit-exact.  Stage 1: one work-group per (row, vocab chunk) with
// 128-bit loads and wave-shuffle reductions; stage 2: one wave per sequence
// reduces the chunks, compares candidates with a ballot and takes the first
// mismatch.
//
// Sampling: one wave per sequence evaluates the accept tests u*q < p exactly
// in fp64 and takes the first rejection a.  If a < K, the residual of row a is
// drawn by an integer inverse CDF: w_v = max(0, F(p) - F(q)) with
// F(x) = floor(clamp(x,0,1) * 2^60) in uint64, chunk sums per work-group,
// then one work-group scans the chunk sums, finds the chunk holding the
// target T = floor(m*S/2^24) (128-bit product) and scans inside it.  Integer
// sums make the pick independent of reduction order.
#include "common.h"
#include "order_keys.h"

namespace orthrus {
namespace {

using namespace keys;

constexpr int kThreads = 256;

// Live block length of sequence b: blk_len[b] clamped to [1, block_k], or
// block_k when no per-sequence lengths are given.
__device__ __forceinline__ int live_k(const int32_t* blk_len, int b, int block_k) {
  if (blk_len == nullptr) return block_k;
  const int k = blk_len[b];
  return k < 1 ? 1 : (k > block_k ? block_k : k);
}

// ---------------------------------------------------------------- greedy --
__global__ __launch_bounds__(kThreads) void argmax_partial_kernel(const float* __restrict__ logits,
                                                                  int vocab, int chunk_len,
                                                                  unsigned long long* part, int block_k,
                                                                  const int32_t* blk_len) {
  const int c = blockIdx.x;
  const size_t row = blockIdx.y;
  // rows past the sequence's live block length are not needed
  if (blk_len != nullptr && (int)(row % block_k) >= live_k(blk_len, (int)(row / block_k), block_k)) return;
  const int begin = c * chunk_len;
  const int end = min(vocab, begin + chunk_len);
  const float* rp = logits + row * (size_t)vocab;
  unsigned long long best = 0;  // below every packed key of a real element
  // kUnroll loads in flight per thread before any is reduced.  Positions past
  // the chunk end are clamped to its last vector (or element): a repeated
  // element repeats its key, which cannot change a maximum.
  constexpr int kUnroll = 8;
  if ((vocab & 3) == 0) {
    // chunk_len is a multiple of 4, so begin is 16-byte aligned within the row
    for (int v0 = begin + 4 * threadIdx.x; v0 < end; v0 += 4 * kThreads * kUnroll) {
      float4 x[kUnroll];
      int vv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        vv[u] = min(v0 + 4 * kThreads * u, end - 4);
        x[u] = *reinterpret_cast<const float4*>(rp + vv[u]);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        best = umax64(best, pack_key(x[u].x, vv[u]));
        best = umax64(best, pack_key(x[u].y, vv[u] + 1));
        best = umax64(best, pack_key(x[u].z, vv[u] + 2));
        best = umax64(best, pack_key(x[u].w, vv[u] + 3));
      }
    }
  } else {
    for (int v0 = begin + threadIdx.x; v0 < end; v0 += kThreads * kUnroll) {
      float x[kUnroll];
      int vv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        vv[u] = min(v0 + kThreads * u, end - 1);
        x[u] = rp[vv[u]];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) best = umax64(best, pack_key(x[u], vv[u]));
    }
  }
  __shared__ unsigned long long red[kThreads / 64];
  best = wave_max64(best);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long m = red[0];
    for (int w = 1; w < kThreads / 64; ++w) m = umax64(m, red[w]);
    part[row * gridDim.x + c] = m;
  }
}

// Maximum of a row's chunk keys, eight loads in flight at a time (indices
// past the last chunk repeat it).
__device__ __forceinline__ unsigned long long chunks_max(const unsigned long long* pp, int chunks) {
  unsigned long long m = 0;
  for (int c0 = 0; c0 < chunks; c0 += 8) {
    unsigned long long k[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) k[u] = pp[min(c0 + u, chunks - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) m = umax64(m, k[u]);
  }
  return m;
}

__global__ __launch_bounds__(64) void greedy_finalize_kernel(int block_k, int chunks,
                                                             const unsigned long long* part,
                                                             const int32_t* cand, const int32_t* blk_len,
                                                             int32_t* accept_len, int32_t* row_argmax,
                                                             int32_t* correction) {
  const int b = blockIdx.x;
  const int kb = live_k(blk_len, b, block_k);  // rows [0, kb) are the block
  // rows in groups of 64 (one per lane); the first group with a mismatch ends the scan
  int a = kb, am_a = -1;
  for (int base = 0; base < block_k; base += 64) {
    const int i = base + (int)threadIdx.x;
    int am = -1;
    bool mismatch = false;
    if (i >= kb && i < block_k && row_argmax != nullptr) row_argmax[(size_t)b * block_k + i] = -1;
    if (i < kb) {
      const unsigned long long m = chunks_max(part + ((size_t)b * block_k + i) * chunks, chunks);
      am = (int)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFull));
      mismatch = cand[(size_t)b * block_k + i] != am;
      if (row_argmax != nullptr) row_argmax[(size_t)b * block_k + i] = am;
    }
    const unsigned long long mm = __ballot(mismatch);
    if (mm && a == kb) {
      const int lane = __builtin_ctzll(mm);
      a = base + lane;
      am_a = __shfl(am, lane);
    }
  }
  if (threadIdx.x == 0) {
    accept_len[b] = a;
    correction[b] = a < kb ? am_a : -1;
  }
}

// ------------------------------------------------------------ tree greedy --
// One wave per sequence: the argmax of every node's row (nodes lane and
// lane + 64), then the walk from the root: at node cur the next node is the
// lowest-index node c > cur with parent[c] == cur and token[c] equal to the
// argmax of row cur (one ballot per step); the correction is the argmax of the
// last node's row.
__global__ __launch_bounds__(64) void tree_finalize_kernel(int K, int chunks, const unsigned long long* part,
                                                           const int32_t* tokens, const int32_t* parent,
                                                           int32_t* accept_len, int32_t* path, int32_t* correction,
                                                           int32_t* row_argmax) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  int am[2] = {-1, -1}, par[2] = {-2, -2}, tok[2] = {-1, -1};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = lane + 64 * h;
    if (i < K) {
      const unsigned long long m = chunks_max(part + ((size_t)b * K + i) * chunks, chunks);
      am[h] = (int)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFull));
      par[h] = parent[(size_t)b * K + i];
      tok[h] = tokens[(size_t)b * K + i];
      if (row_argmax != nullptr) row_argmax[(size_t)b * K + i] = am[h];
    }
  }
  int32_t* pth = path + (size_t)b * K;
  if (lane == 0) pth[0] = 0;
  int cur = 0, a = 0;
  for (int step = 1; step < K; ++step) {
    const int want = cur < 64 ? __shfl(am[0], cur) : __shfl(am[1], cur - 64);
    const bool c0 = lane > cur && lane < K && par[0] == cur && tok[0] == want;
    const bool c1 = lane + 64 > cur && lane + 64 < K && par[1] == cur && tok[1] == want;
    const unsigned long long m0 = __ballot(c0), m1 = __ballot(c1);
    if (!m0 && !m1) break;
    cur = m0 ? __builtin_ctzll(m0) : 64 + __builtin_ctzll(m1);
    ++a;
    if (lane == 0) pth[a] = cur;
  }
  const int last_am = cur < 64 ? __shfl(am[0], cur) : __shfl(am[1], cur - 64);
  for (int i = a + 1 + lane; i < K; i += 64) pth[i] = -1;
  if (lane == 0) {
    accept_len[b] = a;
    correction[b] = last_am;
  }
}

// -------------------------------------------------------------- sampling --
__device__ __forceinline__ unsigned long long fixed_point(float x) {
  const float c = (x > 0.0f) ? fminf(x, 1.0f) : 0.0f;  // NaN and negatives -> 0
  return (unsigned long long)((double)c * 1152921504606846976.0);  // 2^60, exact
}

__global__ __launch_bounds__(64) void sample_accept_kernel(int block_k, int vocab,
                                                           const float* __restrict__ p,
                                                           const float* __restrict__ q,
                                                           const int32_t* __restrict__ cand,
                                                           const float* __restrict__ uniforms,
                                                           const int32_t* blk_len,
                                                           int32_t* accept_len, int32_t* correction,
                                                           int32_t* ws_a) {
  const int b = blockIdx.x;
  const int kb = live_k(blk_len, b, block_k);  // rows [0, kb) are the block
  int a = kb;
  for (int base = 0; base < kb && a == kb; base += 64) {  // groups of 64 rows
    const int i = base + (int)threadIdx.x;
    bool reject = false;
    if (i < kb) {
      const size_t row = (size_t)b * block_k + i;
      const int c = cand[row];
      const bool valid = c >= 0 && c < vocab;
      const float pv = valid ? p[row * vocab + c] : 0.0f;
      const float qv = valid ? q[row * vocab + c] : 0.0f;
      const float u = uniforms[(size_t)b * (block_k + 1) + i];
      const bool acc = valid && (__dmul_rn((double)u, (double)qv) < (double)pv);
      reject = !acc;
    }
    const unsigned long long mm = __ballot(reject);
    if (mm) a = base + __builtin_ctzll(mm);
  }
  if (threadIdx.x == 0) {
    accept_len[b] = a;
    ws_a[b] = a < kb ? a : block_k;  // block_k: no residual draw
    if (a >= kb) correction[b] = -1;
  }
}

constexpr int kChunkEpt = 16;  // elements per thread and pass in the residual chunk sums

__global__ __launch_bounds__(kThreads) void residual_chunks_kernel(int block_k, int vocab, int chunk_len,
                                                                   const float* __restrict__ p,
                                                                   const float* __restrict__ q,
                                                                   const int32_t* ws_a,
                                                                   unsigned long long* sums) {
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  const int a = ws_a[b];
  if (a >= block_k) return;
  const size_t row = ((size_t)b * block_k + a) * vocab;
  const int begin = c * chunk_len;
  const int end = min(vocab, begin + chunk_len);
  unsigned long long sw = 0, sp = 0;
  // Each pass issues all of a thread's loads (elements t + 256 i, coalesced
  // across the wave) before any arithmetic: one memory round trip per pass.
  // Integer sums, so the order does not matter.
  for (int base = begin; base < end; base += kThreads * kChunkEpt) {
    float pv[kChunkEpt], qv[kChunkEpt];
#pragma unroll
    for (int i = 0; i < kChunkEpt; ++i) {
      const int v = base + (int)threadIdx.x + i * kThreads;
      pv[i] = v < end ? p[row + v] : 0.0f;
      qv[i] = v < end ? q[row + v] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kChunkEpt; ++i) {
      const unsigned long long fp = fixed_point(pv[i]);
      const unsigned long long fq = fixed_point(qv[i]);
      sw += fp > fq ? fp - fq : 0ull;
      sp += fp;
    }
  }
  __shared__ unsigned long long red[2][kThreads / 64];
  sw = wave_sum64(sw);
  sp = wave_sum64(sp);
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = sw;
    red[1][threadIdx.x >> 6] = sp;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long tw = 0, tp = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      tw += red[0][w];
      tp += red[1][w];
    }
    sums[((size_t)b * gridDim.x + c) * 2 + 0] = tw;
    sums[((size_t)b * gridDim.x + c) * 2 + 1] = tp;
  }
}

// Inclusive block-wide scan of one uint64 per thread; also returns the total.
__device__ unsigned long long block_scan64(unsigned long long v, unsigned long long* total,
                                           unsigned long long* scratch) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long n = __shfl_up(v, o);
    if (lane >= o) v += n;
  }
  if (lane == 63) scratch[w] = v;
  __syncthreads();
  unsigned long long off = 0, tot = 0;
  for (int k = 0; k < kThreads / 64; ++k) {
    if (k < w) off += scratch[k];
    tot += scratch[k];
  }
  __syncthreads();
  *total = tot;
  return v + off;
}

constexpr int kSelectEpt = 16;  // consecutive elements per thread in the in-chunk scan

__global__ __launch_bounds__(kThreads) void residual_select_kernel(int block_k, int vocab, int chunk_len,
                                                                   int chunks,
                                                                   const float* __restrict__ p,
                                                                   const float* __restrict__ q,
                                                                   const float* __restrict__ uniforms,
                                                                   const int32_t* ws_a,
                                                                   const unsigned long long* sums,
                                                                   int32_t* correction) {
  const int b = blockIdx.x;
  const int a = ws_a[b];
  if (a >= block_k) return;
  __shared__ unsigned long long scratch[kThreads / 64];
  __shared__ int found;
  // ---- totals of both weight families (chunks <= kThreads by construction)
  const int c = threadIdx.x;
  const unsigned long long cw = c < chunks ? sums[((size_t)b * chunks + c) * 2 + 0] : 0ull;
  const unsigned long long cp = c < chunks ? sums[((size_t)b * chunks + c) * 2 + 1] : 0ull;
  unsigned long long Sw, Sp;
  const unsigned long long incw = block_scan64(cw, &Sw, scratch);
  const unsigned long long incp = block_scan64(cp, &Sp, scratch);
  const bool use_p = (Sw == 0);
  const unsigned long long S = use_p ? Sp : Sw;
  if (S == 0) {  // no probability mass at all: token 0
    if (threadIdx.x == 0) correction[b] = 0;
    return;
  }
  // ---- target T = floor(m * S / 2^24), m = floor(u_K * 2^24) in [0, 2^24)
  const float u = uniforms[(size_t)b * (block_k + 1) + block_k];
  float mf = (u > 0.0f) ? u * 16777216.0f : 0.0f;
  unsigned long long m = (unsigned long long)mf;
  if (m > 16777215ull) m = 16777215ull;
  const unsigned long long lo = m * S;
  const unsigned long long hi = __umul64hi(m, S);
  const unsigned long long T = (hi << 40) | (lo >> 24);
  // ---- chunk holding T: exclusive prefix <= T < inclusive prefix
  const unsigned long long inc = use_p ? incp : incw;
  const unsigned long long mine = use_p ? cp : cw;
  if (threadIdx.x == 0) found = chunks - 1;
  __syncthreads();
  if (c < chunks && mine > 0 && inc - mine <= T && T < inc) found = c;
  __syncthreads();
  const int cs = found;
  // exclusive prefix of the chosen chunk, straight from the scan above
  __shared__ unsigned long long run_sh;
  if (c == cs) run_sh = inc - mine;
  __syncthreads();
  unsigned long long run = run_sh;
  // ---- scan inside the chunk: each thread takes kSelectEpt consecutive
  // elements (all their loads in flight at once), one block scan of the
  // per-thread sums finds the thread whose elements hold T, and that thread
  // walks its own elements; chunks longer than kThreads * kSelectEpt take
  // several passes
  const size_t row = ((size_t)b * block_k + a) * vocab;
  const int begin = cs * chunk_len;
  const int end = min(vocab, begin + chunk_len);
  __shared__ int pick;
  if (threadIdx.x == 0) pick = -1;
  __syncthreads();
  for (int base = begin; base < end; base += kThreads * kSelectEpt) {
    const int v0 = base + (int)threadIdx.x * kSelectEpt;
    unsigned long long w[kSelectEpt];
    unsigned long long tw = 0;
#pragma unroll
    for (int i = 0; i < kSelectEpt; ++i) {
      const int v = v0 + i;
      unsigned long long wi = 0;
      if (v < end) {
        const unsigned long long fp = fixed_point(p[row + v]);
        if (use_p) {
          wi = fp;
        } else {
          const unsigned long long fq = fixed_point(q[row + v]);
          wi = fp > fq ? fp - fq : 0ull;
        }
      }
      w[i] = wi;
      tw += wi;
    }
    unsigned long long tot;
    const unsigned long long incl = block_scan64(tw, &tot, scratch) + run;
    const unsigned long long excl = incl - tw;
    if (tw > 0 && excl <= T && T < incl) {  // exactly one thread holds T
      unsigned long long acc = excl;
#pragma unroll
      for (int i = 0; i < kSelectEpt; ++i) {
        acc += w[i];
        if (acc > T) {
          pick = v0 + i;
          break;
        }
      }
    }
    __syncthreads();
    if (pick >= 0) break;
    run += tot;
  }
  if (threadIdx.x == 0) correction[b] = pick >= 0 ? pick : end - 1;
}

}  // namespace

hipError_t launch_consensus_greedy(int batch, int block_k, int vocab, const float* logits,
                                   const int32_t* cand, const int32_t* blk_len, int32_t* accept_len,
                                   int32_t* row_argmax, int32_t* correction, void* workspace,
                                   const ConsensusPlan& plan, hipStream_t stream) {
  auto* part = reinterpret_cast<unsigned long long*>(workspace);
  const int chunks = plan.greedy_chunks;
  int chunk_len = (vocab + chunks - 1) / chunks;
  chunk_len = (chunk_len + 3) & ~3;
  hipLaunchKernelGGL(argmax_partial_kernel, dim3(chunks, batch * block_k), dim3(kThreads), 0, stream,
                     logits, vocab, chunk_len, part, block_k, blk_len);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(greedy_finalize_kernel, dim3(batch), dim3(64), 0, stream, block_k, chunks, part,
                     cand, blk_len, accept_len, row_argmax, correction);
  return hipGetLastError();
}

hipError_t launch_consensus_tree_greedy(int batch, int block_k, int vocab, const float* logits,
                                        const int32_t* tokens, const int32_t* parent, int32_t* accept_len,
                                        int32_t* path, int32_t* correction, int32_t* row_argmax, void* workspace,
                                        const ConsensusPlan& plan, hipStream_t stream) {
  const int chunks = plan.greedy_chunks;
  int chunk_len = (vocab + chunks - 1) / chunks;
  chunk_len = (chunk_len + 3) & ~3;  // as for the greedy rule: whole 16-byte groups per chunk
  auto* part = reinterpret_cast<unsigned long long*>(workspace);
  hipLaunchKernelGGL(argmax_partial_kernel, dim3(chunks, batch * block_k), dim3(kThreads), 0, stream, logits,
                     vocab, chunk_len, part, block_k, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tree_finalize_kernel, dim3(batch), dim3(64), 0, stream, block_k, chunks, part, tokens, parent,
                     accept_len, path, correction, row_argmax);
  return hipGetLastError();
}

hipError_t launch_consensus_sample(int batch, int block_k, int vocab, const float* p_target,
                                   const float* q_draft, const int32_t* cand, const float* uniforms,
                                   const int32_t* blk_len, int32_t* accept_len, int32_t* correction,
                                   void* workspace, const ConsensusPlan& plan, hipStream_t stream) {
  auto* ws = reinterpret_cast<uint8_t*>(workspace);
  auto* sums = reinterpret_cast<unsigned long long*>(ws);
  auto* ws_a = reinterpret_cast<int32_t*>(ws + (size_t)batch * plan.sample_chunks * 2 * 8);
  const int chunks = plan.sample_chunks;
  const int chunk_len = (vocab + chunks - 1) / chunks;
  hipLaunchKernelGGL(sample_accept_kernel, dim3(batch), dim3(64), 0, stream, block_k, vocab, p_target,
                     q_draft, cand, uniforms, blk_len, accept_len, correction, ws_a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(residual_chunks_kernel, dim3(chunks, batch), dim3(kThreads), 0, stream, block_k,
                     vocab, chunk_len, p_target, q_draft, ws_a, sums);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(residual_select_kernel, dim3(batch), dim3(kThreads), 0, stream, block_k, vocab,
                     chunk_len, chunks, p_target, q_draft, uniforms, ws_a, sums, correction);
  return hipGetLastError();
}

}  // namespace orthrus
