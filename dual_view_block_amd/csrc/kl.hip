// Forward KL over the vocabulary for distilling the diffusion view against the
// frozen AR model (Orthrus paper notes §3.1, §3.3): for every position n,
//   KL_n = sum_v p_v (ln p_v - ln q_v),  p = softmax(target row), q = softmax(draft row)
// and, optionally, its gradient with respect to the draft logits,
//   grad[n, v] = scale * (q_v - p_v).
//
// With A = ln sum_v e^{a_v} and B = ln sum_v e^{b_v} (a = target row, b = draft
// row) the loss is KL = sum_v p_v (a_v - b_v) - A + B, so one pass over both
// rows gives it: per thread the running maxima, the two exponential sums and
// sum_v e^{a_v - m_a} (a_v - b_v), combined over the work-group at the row end.
// The gradient needs A and B, hence a second pass over the same row, written
// as e^{b-B} - e^{a-A}.
//
// One kernel, kl_rowwise_kernel: a persistent grid whose work-groups each take
// whole rows.  Pass 1 streams both rows once with ordinary loads, so the
// 256 MiB memory-side cache keeps them; pass 2 walks the row backwards -- the
// chunks read last first, the likeliest still to be cached -- and writes the
// gradient with streaming stores.  With a gradient the grid holds one
// work-group per CU (256 rows of both arrays in flight: about 152 MB at
// V = 151936 in bf16), so the re-read stays off HBM.
//
// The inner loops have no branches around memory operations: loads past the
// row end are clamped to the row's last vector (masked out of the sums in the
// row's last chunk; in pass 2 they recompute and store that vector's own
// values again), and the chunk after the last is the last chunk again.  A
// branch around a load makes the compiler wait for every load in flight at the
// join, which would serialise the two register buffers that overlap one
// chunk's loads with the previous chunk's arithmetic.
#include "common.h"

#include <math.h>

namespace orthrus {
namespace {

constexpr int kKlThreads = 512;  // 8 waves per work-group
constexpr int kKlWaves = kKlThreads / 64;
constexpr int kKlGroupsPerCuGrad = 1, kKlGroupsPerCuLoss = 2;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInfKl = -__builtin_inff();

typedef unsigned kl_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Elements per 16-byte vector.
template <typename T> struct KlTraits;
template <> struct KlTraits<float> { static constexpr int kVec = 4; };
template <> struct KlTraits<uint16_t> { static constexpr int kVec = 8; };

__device__ __forceinline__ float load_one(const float* p) { return *p; }
__device__ __forceinline__ float load_one(const uint16_t* p) { return bf16_to_f32(*p); }

// Elements of one chunk held per thread: EPT = VPT vectors of kVecEl elements
// (16-byte vectors when every row starts 16-byte aligned, else scalars).
template <typename T, bool VEC> struct KlChunk {
  static constexpr int kVecEl = VEC ? KlTraits<T>::kVec : 1;
  static constexpr int kVpt = VEC ? 4 : 16;  // vectors (or scalars) per thread
  static constexpr int kEpt = kVecEl * kVpt;
  static constexpr int kChunk = kEpt * kKlThreads;
};

// This thread's part of one row chunk, raw, in registers.  Vector i of the
// chunk at `base` holds elements elem(base, i) .. + kVecEl - 1 (coalesced:
// consecutive threads, consecutive vectors).
template <typename T, bool VEC> struct RawChunk {
  using C = KlChunk<T, VEC>;
  kl_u32x4 v[VEC ? C::kVpt : 1];
  float s[VEC ? 1 : C::kVpt];
  static __device__ __forceinline__ long long elem(long long base, int i) {
    return base + (long long)(i * kKlThreads + (int)threadIdx.x) * C::kVecEl;
  }
  // NTL: streaming (nontemporal) loads, else ordinary ones that the caches
  // keep.  Vectors past the row end read the row's last vector.
  template <bool NTL>
  __device__ __forceinline__ void load(const T* row, long long base, int vocab) {
    const long long last = (long long)vocab - C::kVecEl;
#pragma unroll
    for (int i = 0; i < C::kVpt; ++i) {
      const long long e0 = elem(base, i);
      const long long e = e0 < last ? e0 : last;
      if constexpr (VEC) {
        const kl_u32x4* p = reinterpret_cast<const kl_u32x4*>(row + e);
        v[i] = NTL ? __builtin_nontemporal_load(p) : *p;
      } else {
        s[i] = load_one(row + e);
      }
    }
  }
  // element k of this thread's EPT elements (in vector k / kVecEl)
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

// Work-group reductions over the waves (fixed order: deterministic).
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kKlWaves; ++i) r = fmaxf(r, red[i]);
  return r;
}
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kKlWaves; ++i) r += red[i];
  return r;
}

// e^(x - m) as 2^((x - m) * log2 e).  The difference is taken first, so the
// terms near the maximum, which dominate every sum, carry almost no argument
// error; 0 for x = -inf (m finite).
__device__ __forceinline__ float exp_shift(float x, float m) {
  return __builtin_amdgcn_exp2f((x - m) * kLog2e);
}

// One thread's running statistics of a row pair: maxima m_a, m_b and, relative
// to them, s_a = sum e^{a - m_a}, s_b = sum e^{b - m_b}, t = sum e^{a - m_a} (a - b).
struct KlStats {
  float ma = kNegInfKl, mb = kNegInfKl, sa = 0.0f, t = 0.0f, sb = 0.0f;
};

// Fold one chunk into the statistics.  TAIL (the row's last chunk): only the
// elements inside the row count.  Logits are finite, so away from the tail
// every element does.
template <bool TAIL, typename T, bool VEC>
__device__ __forceinline__ void fold(KlStats& st, const RawChunk<T, VEC>& xa, const RawChunk<T, VEC>& xb,
                                     long long base, int vocab) {
  using C = KlChunk<T, VEC>;
  bool ok[C::kVpt];
#pragma unroll
  for (int i = 0; i < C::kVpt; ++i) ok[i] = !TAIL || RawChunk<T, VEC>::elem(base, i) < vocab;
  float ca = kNegInfKl, cb = kNegInfKl;
#pragma unroll
  for (int k = 0; k < C::kEpt; ++k) {
    const bool in = ok[k / C::kVecEl];
    ca = fmaxf(ca, in ? xa.get(k) : kNegInfKl);
    cb = fmaxf(cb, in ? xb.get(k) : kNegInfKl);
  }
  const float nma = fmaxf(st.ma, ca), nmb = fmaxf(st.mb, cb);
  // rescale the running sums (which are 0 while the maxima are still -inf)
  const float fa = st.ma == kNegInfKl ? 0.0f : exp_shift(st.ma, nma);
  const float fb = st.mb == kNegInfKl ? 0.0f : exp_shift(st.mb, nmb);
  float sa = st.sa * fa, t = st.t * fa, sb = st.sb * fb;
#pragma unroll
  for (int k = 0; k < C::kEpt; ++k) {
    const float x = xa.get(k), y = xb.get(k);
    float ea = exp_shift(x, nma), eb = exp_shift(y, nmb), d = x - y;
    if (TAIL && !ok[k / C::kVecEl]) ea = eb = d = 0.0f;
    sa += ea;
    t = fmaf(ea, d, t);
    sb += eb;
  }
  st = KlStats{nma, nmb, sa, t, sb};
}

// Gradient of one chunk: scale * (e^{b - B} - e^{a - A}) for every vector,
// stored at the (clamped) place it was loaded from.
template <typename T, bool VEC>
__device__ __forceinline__ void write_grad(T* g, const RawChunk<T, VEC>& xa, const RawChunk<T, VEC>& xb,
                                           long long base, int vocab, float A, float B, float scale) {
  using C = KlChunk<T, VEC>;
  const long long last = (long long)vocab - C::kVecEl;
#pragma unroll
  for (int i = 0; i < C::kVpt; ++i) {
    const long long e0 = RawChunk<T, VEC>::elem(base, i);
    const long long e = e0 < last ? e0 : last;
    float r[C::kVecEl];
#pragma unroll
    for (int j = 0; j < C::kVecEl; ++j) {
      const int k = i * C::kVecEl + j;
      r[j] = scale * (exp_shift(xb.get(k), B) - exp_shift(xa.get(k), A));
    }
    if constexpr (VEC) {
      kl_u32x4 w;
      if constexpr (sizeof(T) == 4) {
        w = kl_u32x4{__float_as_uint(r[0]), __float_as_uint(r[1]), __float_as_uint(r[2]), __float_as_uint(r[3])};
      } else {
        uint32_t u[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          u[q] = (uint32_t)f32_to_bf16(r[2 * q]) | ((uint32_t)f32_to_bf16(r[2 * q + 1]) << 16);
        w = kl_u32x4{u[0], u[1], u[2], u[3]};
      }
      __builtin_nontemporal_store(w, reinterpret_cast<kl_u32x4*>(g + e));
    } else {
      if constexpr (sizeof(T) == 4) g[e] = r[0];
      else g[e] = f32_to_bf16(r[0]);
    }
  }
}

// Loss (and gradient) row by row.  Two register buffers per row array are used
// in turn (chunk c in buffer c & 1): the next chunk's loads are in flight
// while this one is folded, and no buffer is ever copied (a copy would wait
// for the loads it moves).  Every sum runs in a fixed order.
template <typename T, bool VEC>
__global__ __launch_bounds__(kKlThreads) void kl_rowwise_kernel(const T* __restrict__ target,
                                                                const T* __restrict__ draft, int rows, int vocab,
                                                                int chunks, float* __restrict__ kl, float scale,
                                                                T* __restrict__ grad) {
  using C = KlChunk<T, VEC>;
  __shared__ float red[kKlWaves];
  RawChunk<T, VEC> ra[2], rb[2];
  const int last = chunks - 1;
  for (int row = blockIdx.x; row < rows; row += gridDim.x) {
    const T* ar = target + (long long)row * vocab;
    const T* br = draft + (long long)row * vocab;
    // ---- pass 1: statistics; past the last chunk the loads repeat it (cached)
    KlStats st;
    auto fold_any = [&](const RawChunk<T, VEC>& xa, const RawChunk<T, VEC>& xb, int c) __attribute__((always_inline)) {
      if (c == last) fold<true>(st, xa, xb, (long long)c * C::kChunk, vocab);
      else fold<false>(st, xa, xb, (long long)c * C::kChunk, vocab);
    };
    ra[0].template load<false>(ar, 0, vocab);
    rb[0].template load<false>(br, 0, vocab);
    for (int c = 0; c < chunks; c += 2) {
      const long long n1 = (long long)(c + 1 < chunks ? c + 1 : last) * C::kChunk;
      ra[1].template load<false>(ar, n1, vocab);
      rb[1].template load<false>(br, n1, vocab);
      __builtin_amdgcn_sched_barrier(0);
      fold_any(ra[0], rb[0], c);
      __builtin_amdgcn_sched_barrier(0);
      const long long n2 = (long long)(c + 2 < chunks ? c + 2 : last) * C::kChunk;
      ra[0].template load<false>(ar, n2, vocab);
      rb[0].template load<false>(br, n2, vocab);
      __builtin_amdgcn_sched_barrier(0);
      if (c + 1 < chunks) fold_any(ra[1], rb[1], c + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // row totals, in a fixed order
    const float Ma = block_max(st.ma, red), Mb = block_max(st.mb, red);
    const float wa = st.ma == kNegInfKl ? 0.0f : exp_shift(st.ma, Ma);
    const float wb = st.mb == kNegInfKl ? 0.0f : exp_shift(st.mb, Mb);
    const float Sa = block_sum(st.sa * wa, red);
    const float Tt = block_sum(st.t * wa, red);
    const float Sb = block_sum(st.sb * wb, red);
    // KL = t/s_a - (A - B) with A - B = (m_a - m_b) + ln(s_a / s_b): no
    // cancellation between the two (possibly large) log-sum-exps
    if (threadIdx.x == 0) kl[row] = Tt / Sa - ((Ma - Mb) + logf(Sa / Sb));
    if (grad == nullptr) continue;  // the loss only
    const float A = Ma + logf(Sa), B = Mb + logf(Sb);
    // ---- pass 2: the gradient, chunks in reverse order; past chunk 0 the loads repeat it
    T* g = grad + (long long)row * vocab;
    ra[0].template load<true>(ar, (long long)last * C::kChunk, vocab);
    rb[0].template load<true>(br, (long long)last * C::kChunk, vocab);
    // Chunk last - i in buffer 0, last - i - 1 in buffer 1.  With an odd
    // chunk count the last step writes chunk 0 a second time, with the same
    // values, so the loop body has no branch.  The scheduling barriers keep
    // each buffer's loads ahead of the other buffer's arithmetic.
    for (int i = 0; i < chunks; i += 2) {
      const int c = last - i;
      const long long c1 = (long long)(c >= 1 ? c - 1 : 0) * C::kChunk;
      ra[1].template load<true>(ar, c1, vocab);
      rb[1].template load<true>(br, c1, vocab);
      __builtin_amdgcn_sched_barrier(0);
      write_grad(g, ra[0], rb[0], (long long)c * C::kChunk, vocab, A, B, scale);
      __builtin_amdgcn_sched_barrier(0);
      const long long c2 = (long long)(c >= 2 ? c - 2 : 0) * C::kChunk;
      ra[0].template load<true>(ar, c2, vocab);
      rb[0].template load<true>(br, c2, vocab);
      __builtin_amdgcn_sched_barrier(0);
      write_grad(g, ra[1], rb[1], c1, vocab, A, B, scale);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <typename T, bool VEC>
hipError_t launch_kl_t(int rows, int vocab, const void* target, const void* draft, float* kl, void* grad,
                       float scale, int groups, hipStream_t stream) {
  using C = KlChunk<T, VEC>;
  const int chunks = (vocab + C::kChunk - 1) / C::kChunk;
  const int grid = rows < groups ? rows : groups;
  hipLaunchKernelGGL((kl_rowwise_kernel<T, VEC>), dim3(grid), dim3(kKlThreads), 0, stream,
                     reinterpret_cast<const T*>(target), reinterpret_cast<const T*>(draft), rows, vocab, chunks, kl,
                     scale, reinterpret_cast<T*>(grad));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_kl(int rows, int vocab, int dtype_bytes, bool vec, const void* target,
                             const void* draft, float* kl, void* grad, float scale, int cus, hipStream_t stream) {
  // with a gradient one work-group per CU (the rows in flight stay cached for
  // the second pass); the loss alone takes two per CU
  const int groups = (grad ? kKlGroupsPerCuGrad : kKlGroupsPerCuLoss) * cus;
  if (dtype_bytes == 4) {
    return vec ? launch_kl_t<float, true>(rows, vocab, target, draft, kl, grad, scale, groups, stream)
               : launch_kl_t<float, false>(rows, vocab, target, draft, kl, grad, scale, groups, stream);
  }
  return vec ? launch_kl_t<uint16_t, true>(rows, vocab, target, draft, kl, grad, scale, groups, stream)
             : launch_kl_t<uint16_t, false>(rows, vocab, target, draft, kl, grad, scale, groups, stream);
}

}  // namespace orthrus
