// Forward KL over the vocabulary for distilling the diffusion view against the
// frozen AR model (Orthrus paper notes §3.1, §3.3): for every position n,
//   KL_n = sum_v p_v (ln p_v - ln q_v),  p = softmax(target row), q = softmax(draft row)
// and, optionally, its gradient with respect to the draft logits,
//   grad[n, v] = scale * (q_v - p_v).
//
// With A = ln sum_v e^{a_v} and B = ln sum_v e^{b_v} (a = target row, b = draft
// row) the loss is KL = sum_v p_v (a_v - b_v) - A + B, so one pass over both
// rows gives it: per chunk of the vocabulary the running maxima, the two
// exponential sums and sum_v e^{a_v - m_a} (a_v - b_v).
//
// Kernels (HBM-bound; every element is read once per pass, with coalesced
// 16-byte loads when the row length allows it):
//  1. kl_partial_kernel: a persistent grid (8 work-groups per CU) strides over
//     the (row, vocabulary chunk) items and reduces each to
//     (m_a, s_a, t, m_b, s_b) in the workspace.
//  2. kl_finalize_kernel: one wave per row combines the chunk partials in a
//     fixed order, writes KL and keeps (A, B) for the gradient pass.
//  3. kl_grad_kernel (only if a gradient is wanted): grid (chunks, rows),
//     re-reads both rows and writes scale * (e^{b-B} - e^{a-A}).
#include "common.h"

#include <math.h>

namespace orthrus {
namespace {

constexpr int kKlThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInfKl = -__builtin_inff();

typedef unsigned kl_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Elements per 16-byte vector and the per-thread element count of a chunk.
template <typename T> struct KlTraits;
template <> struct KlTraits<float> { static constexpr int kVec = 4; };
template <> struct KlTraits<uint16_t> { static constexpr int kVec = 8; };

// Unpack one 16-byte vector into floats.
__device__ __forceinline__ void unpack(const kl_u32x4& v, float (&x)[4]) {
  x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
  x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack(const kl_u32x4& v, float (&x)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ float load_one(const float* p) { return *p; }
__device__ __forceinline__ float load_one(const uint16_t* p) { return bf16_to_f32(*p); }


// Elements of one chunk held per thread: EPT = VPT vectors of kVec elements.
template <typename T, bool VEC> struct KlChunk {
  static constexpr int kVecEl = VEC ? KlTraits<T>::kVec : 1;
  static constexpr int kVpt = VEC ? 4 : 16;  // vectors (or scalars) per thread
  static constexpr int kEpt = kVecEl * kVpt;
  static constexpr int kChunk = kEpt * kKlThreads;
};

// Load this thread's elements of a row chunk (coalesced: vector i of thread
// tid sits at (i * threads + tid) * kVecEl).  Elements past `vocab` read as
// -inf.
template <typename T, bool VEC>
__device__ __forceinline__ void load_chunk(const T* row, long long base, int vocab,
                                           float (&x)[KlChunk<T, VEC>::kEpt]) {
  using C = KlChunk<T, VEC>;
#pragma unroll
  for (int i = 0; i < C::kVpt; ++i) {
    const long long e0 = base + (long long)(i * kKlThreads + (int)threadIdx.x) * C::kVecEl;
    if constexpr (VEC) {
      float v[C::kVecEl];
      if (e0 < vocab) {
        const kl_u32x4 raw = __builtin_nontemporal_load(reinterpret_cast<const kl_u32x4*>(row + e0));
        unpack(raw, v);
      } else {
#pragma unroll
        for (int j = 0; j < C::kVecEl; ++j) v[j] = kNegInfKl;
      }
#pragma unroll
      for (int j = 0; j < C::kVecEl; ++j) x[i * C::kVecEl + j] = v[j];
    } else {
      x[i] = e0 < vocab ? load_one(row + e0) : kNegInfKl;
    }
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Work-group reductions over the 4 waves (fixed order: deterministic).
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// e^(x - m) as 2^((x - m) * log2 e).  The difference is taken first, so the
// terms near the maximum, which dominate every sum, carry almost no argument
// error; 0 for x = -inf (m finite).
__device__ __forceinline__ float exp_shift(float x, float m) {
  return __builtin_amdgcn_exp2f((x - m) * kLog2e);
}

// One wave per row: KL and the two log-sum-exps.
__global__ __launch_bounds__(kKlThreads) void kl_finalize_kernel(const float* __restrict__ part, int chunks,
                                                                  int rows, float* __restrict__ kl,
                                                                  float* __restrict__ lse) {
  const int row = blockIdx.x * (kKlThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const float* p = part + (size_t)row * chunks * 8;
  float ma = kNegInfKl, mb = kNegInfKl;
  for (int c = lane; c < chunks; c += 64) {
    ma = fmaxf(ma, p[c * 8 + 0]);
    mb = fmaxf(mb, p[c * 8 + 3]);
  }
  ma = wave_max(ma);
  mb = wave_max(mb);
  float sa = 0.0f, t = 0.0f, sb = 0.0f;
  for (int c = lane; c < chunks; c += 64) {
    const float wa = exp_shift(p[c * 8 + 0], ma);
    const float wb = exp_shift(p[c * 8 + 3], mb);
    sa = fmaf(p[c * 8 + 1], wa, sa);
    t = fmaf(p[c * 8 + 2], wa, t);
    sb = fmaf(p[c * 8 + 4], wb, sb);
  }
  sa = wave_sum(sa);
  t = wave_sum(t);
  sb = wave_sum(sb);
  if (lane == 0) {
    // KL = t/s_a - (A - B) with A - B = (m_a - m_b) + ln(s_a / s_b): no
    // cancellation between the two (possibly large) log-sum-exps
    kl[row] = t / sa - ((ma - mb) + logf(sa / sb));
    if (lse) {
      lse[2 * (size_t)row] = ma + logf(sa);
      lse[2 * (size_t)row + 1] = mb + logf(sb);
    }
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kKlThreads) void kl_grad_kernel(const T* __restrict__ target,
                                                              const T* __restrict__ draft, int vocab,
                                                              const float* __restrict__ lse, float scale,
                                                              T* __restrict__ grad) {
  using C = KlChunk<T, VEC>;
  const long long row = blockIdx.y;
  const long long base = (long long)blockIdx.x * C::kChunk;
  const float A = lse[2 * row], B = lse[2 * row + 1];
  float a[C::kEpt], b[C::kEpt];
  load_chunk<T, VEC>(target + row * vocab, base, vocab, a);
  load_chunk<T, VEC>(draft + row * vocab, base, vocab, b);
  T* g = grad + row * vocab;
#pragma unroll
  for (int i = 0; i < C::kVpt; ++i) {
    const long long e0 = base + (long long)(i * kKlThreads + (int)threadIdx.x) * C::kVecEl;
    if (e0 >= vocab) continue;
    float r[C::kVecEl];
#pragma unroll
    for (int j = 0; j < C::kVecEl; ++j) {
      const int k = i * C::kVecEl + j;
      r[j] = scale * (exp_shift(b[k], B) - exp_shift(a[k], A));
    }
    if constexpr (VEC) {
      kl_u32x4 w;
      if constexpr (sizeof(T) == 4) {
        w = kl_u32x4{__float_as_uint(r[0]), __float_as_uint(r[1]), __float_as_uint(r[2]), __float_as_uint(r[3])};
      } else {
        uint32_t u[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) u[q] = (uint32_t)f32_to_bf16(r[2 * q]) | ((uint32_t)f32_to_bf16(r[2 * q + 1]) << 16);
        w = kl_u32x4{u[0], u[1], u[2], u[3]};
      }
      __builtin_nontemporal_store(w, reinterpret_cast<kl_u32x4*>(g + e0));
    } else {
      if constexpr (sizeof(T) == 4) g[e0] = r[0];
      else g[e0] = f32_to_bf16(r[0]);
    }
  }
}

// Rows [r0, r0 + n) through the partial, finalize and (with grad) gradient kernels.
// ---- the partial pass is persistent: a grid of a few work-groups per CU
// strides over the (row, chunk) items, issuing the next item's loads before
// it reduces the current one, so every work-group keeps a chunk of both rows
// in flight while it computes (measured 12-15 % faster than one short
// work-group per item).
template <typename T, bool VEC> struct RawChunk {
  using C = KlChunk<T, VEC>;
  kl_u32x4 v[VEC ? C::kVpt : 1];
  float s[VEC ? 1 : C::kVpt];
  __device__ __forceinline__ void load(const T* row, long long base, int vocab) {
#pragma unroll
    for (int i = 0; i < C::kVpt; ++i) {
      const long long e0 = base + (long long)(i * kKlThreads + (int)threadIdx.x) * C::kVecEl;
      if constexpr (VEC) {
        if (e0 < vocab) {
          v[i] = __builtin_nontemporal_load(reinterpret_cast<const kl_u32x4*>(row + e0));
        } else {  // -inf in every lane of the vector
          const uint32_t ninf = sizeof(T) == 4 ? 0xff800000u : 0xff80ff80u;
          v[i] = kl_u32x4{ninf, ninf, ninf, ninf};
        }
      } else {
        s[i] = e0 < vocab ? load_one(row + e0) : kNegInfKl;
      }
    }
  }
  // element k of this thread's EPT elements
  __device__ __forceinline__ float get(int k) const {
    if constexpr (!VEC) {
      return s[k];
    } else if constexpr (sizeof(T) == 4) {
      return __uint_as_float(v[k >> 2][k & 3]);
    } else {
      const uint32_t w = v[k >> 3][(k & 7) >> 1];
      return __uint_as_float((k & 1) ? (w & 0xffff0000u) : (w << 16));
    }
  }
};

// Partial per (row, chunk) item: {m_a, s_a, t, m_b, s_b} (8 floats reserved).
template <typename T, bool VEC>
__global__ __launch_bounds__(kKlThreads) void kl_partial_kernel(const T* __restrict__ target,
                                                                     const T* __restrict__ draft, int vocab,
                                                                     int chunks, long long items,
                                                                     float* __restrict__ part) {
  using C = KlChunk<T, VEC>;
  __shared__ float red[4];
  long long it = blockIdx.x;
  RawChunk<T, VEC> ra, rb;
  if (it < items) {
    const long long row = it / chunks, base = (it % chunks) * (long long)C::kChunk;
    ra.load(target + row * vocab, base, vocab);
    rb.load(draft + row * vocab, base, vocab);
  }
  while (it < items) {
    const long long nx = it + gridDim.x;
    RawChunk<T, VEC> na, nb;
    if (nx < items) {
      const long long row = nx / chunks, base = (nx % chunks) * (long long)C::kChunk;
      na.load(target + row * vocab, base, vocab);
      nb.load(draft + row * vocab, base, vocab);
    }
    float ma = kNegInfKl, mb = kNegInfKl;
#pragma unroll
    for (int k = 0; k < C::kEpt; ++k) {
      ma = fmaxf(ma, ra.get(k));
      mb = fmaxf(mb, rb.get(k));
    }
    ma = block_max(ma, red);
    mb = block_max(mb, red);
    float sa = 0.0f, t = 0.0f, sb = 0.0f;
#pragma unroll
    for (int k = 0; k < C::kEpt; ++k) {
      const float x = ra.get(k), y = rb.get(k);
      if (x != kNegInfKl) {  // padding past the row end
        const float ea = exp_shift(x, ma);
        sa += ea;
        t = fmaf(ea, x - y, t);
        sb += exp_shift(y, mb);
      }
    }
    sa = block_sum(sa, red);
    t = block_sum(t, red);
    sb = block_sum(sb, red);
    if (threadIdx.x == 0) {
      float4* o = reinterpret_cast<float4*>(part + it * 8);
      o[0] = make_float4(ma, sa, t, mb);
      o[1] = make_float4(sb, 0.0f, 0.0f, 0.0f);
    }
    ra = na;
    rb = nb;
    it = nx;
  }
}

template <typename T, bool VEC>
hipError_t launch_kl_t(int rows, int vocab, const void* target, const void* draft, float* kl, void* grad,
                       float scale, float* part, float* lse, int groups, hipStream_t stream) {
  using C = KlChunk<T, VEC>;
  const int chunks = (vocab + C::kChunk - 1) / C::kChunk;
  const T* a = reinterpret_cast<const T*>(target);
  const T* b = reinterpret_cast<const T*>(draft);
  const long long items = (long long)rows * chunks;
  const int pgrid = (int)(items < groups ? items : groups);
  hipLaunchKernelGGL((kl_partial_kernel<T, VEC>), dim3(pgrid), dim3(kKlThreads), 0, stream, a, b, vocab, chunks,
                     items, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int per = kKlThreads / 64;
  hipLaunchKernelGGL(kl_finalize_kernel, dim3((rows + per - 1) / per), dim3(kKlThreads), 0, stream, part, chunks,
                     rows, kl, grad ? lse : nullptr);
  e = hipGetLastError();
  if (e != hipSuccess || !grad) return e;
  hipLaunchKernelGGL((kl_grad_kernel<T, VEC>), dim3(chunks, rows), dim3(kKlThreads), 0, stream, a, b, vocab, lse,
                     scale, reinterpret_cast<T*>(grad));
  return hipGetLastError();
}

}  // namespace

int kl_chunks(int vocab, int dtype_bytes, bool vec) {
  int chunk;
  if (dtype_bytes == 4) chunk = vec ? KlChunk<float, true>::kChunk : KlChunk<float, false>::kChunk;
  else chunk = vec ? KlChunk<uint16_t, true>::kChunk : KlChunk<uint16_t, false>::kChunk;
  return (vocab + chunk - 1) / chunk;
}

hipError_t launch_forward_kl(int rows, int vocab, int dtype_bytes, bool vec, const void* target,
                             const void* draft, float* kl, void* grad, float scale, float* part, float* lse,
                             int groups, hipStream_t stream) {
  if (dtype_bytes == 4) {
    return vec ? launch_kl_t<float, true>(rows, vocab, target, draft, kl, grad, scale, part, lse, groups, stream)
               : launch_kl_t<float, false>(rows, vocab, target, draft, kl, grad, scale, part, lse, groups, stream);
  }
  return vec ? launch_kl_t<uint16_t, true>(rows, vocab, target, draft, kl, grad, scale, part, lse, groups, stream)
             : launch_kl_t<uint16_t, false>(rows, vocab, target, draft, kl, grad, scale, part, lse, groups, stream);
}

}  // namespace orthrus
