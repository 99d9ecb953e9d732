// Dual-view block attention for gfx950 (MI355X): split-L cache streaming with
// bf16 MFMA, online softmax in fp32, and a cross-split log-sum-exp merge.
//
// What is computed (Orthrus paper notes, zhangshuibai.github.io, §2.1, §3.2,
// §4.1): for every (sequence b, KV head g), the G*K query rows of the q heads
// that share g attend to the cached keys [0, L_b) and to the K block keys in
// one softmax; block key j is visible to block row i always (diffusion view)
// or iff j <= i (AR verify view).
//
// Layout of the work (one work-group = 4 waves, 256 threads):
//   grid = (splits, row groups, B * Hkv).  A work-group owns one contiguous
//   chunk of the (b, g) cache rows plus up to 128 query rows.  Split 0 also
//   takes the block keys, as one extra masked tile.
//   The cache chunk is streamed in tiles of 64 keys: every thread issues
//   128-bit global loads for the next tile into registers while the waves
//   compute on the current tile in LDS (two LDS stages).  Rows are stored in
//   LDS with the 16-byte chunks of row r XOR-swizzled by 2*(r mod 8), which
//   keeps both read patterns below free of bank conflicts.
//   Per wave: S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (32 keys x 32 query
//   rows; K rows from LDS, Q rows held in registers), so each lane owns one
//   query row -- softmax row statistics are per-lane plus one exchange with
//   lane^32.  Then O^T += V^T P^T on the same MFMA: P^T comes straight from
//   the S^T accumulator registers, and V^T is read from the row-major V tile
//   with ds_read_b64_tr_b16 (the transposing LDS read), key order matched to
//   the accumulator's register order.
//   Each work-group writes an unnormalised partial (max, sum, acc) per row;
//   a second kernel merges the splits: out = sum_s 2^(m_s-M) acc_s /
//   sum_s 2^(m_s-M) l_s, lse = (M + log2 sum) * ln 2.
#include "common.h"

#include <math.h>

namespace orthrus {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kThreads = 256;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ int swizzle_chunk(int row, int chunk, int chunks_per_row) {
  return chunk ^ ((2 * row) & (chunks_per_row - 2));
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D, int NQB>
__global__ __launch_bounds__(kThreads, 2) void attn_split_kernel(AttnArgs a, AttnPlan plan) {
  constexpr int KS = (NQB <= 2) ? 2 : 1;  // waves sharing one query block (key subsets)
  constexpr int KPW = kTileKeys / KS;     // keys per wave per tile
  constexpr int NKB = KPW / 32;           // 32-key MFMA blocks per wave per tile
  constexpr int DCH = D / 8;              // 16-byte chunks per row
  constexpr int ROWB = D * 2;             // bytes per row
  constexpr int TILEB = kTileKeys * ROWB; // bytes of one K or V tile
  constexpr int NDS = D / 16;             // MFMA steps over head_dim for S^T
  constexpr int NMB = D / 32;             // 32-wide head_dim blocks of O^T
  constexpr int NCH = kTileKeys * DCH / kThreads;  // 16-byte chunks per thread per tile
  static_assert(NCH >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) uint8_t smem[2][2][TILEB];

  const int split = blockIdx.x;
  const int rg = blockIdx.y;
  const int bg = blockIdx.z;
  const int b = bg / a.n_kv_heads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const bool active = wave < NQB * KS;
  const int qb = wave % NQB;
  const int ks = wave / NQB;
  const int R = plan.rows;
  const int S = plan.splits;
  const int K = a.block_k;

  int L = a.cache_len[b];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  int chunk = (L + S - 1) / S;
  chunk = (chunk + kTileKeys - 1) / kTileKeys * kTileKeys;
  const int kstart = split * chunk;
  const int kend = min(kstart + chunk, L);
  const int ncache = kstart < kend ? (kend - kstart + kTileKeys - 1) / kTileKeys : 0;
  const int has_block = split == 0 ? 1 : 0;
  const int ntiles = ncache + has_block;

  // ---- this lane's query row (the N index of every MFMA it joins)
  const int qrow = rg * plan.rows_per_wg + qb * 32 + (lane & 31);
  const int qrow_i = qrow % K;  // block position of the row (row = head_in_group * K + i)
  const size_t row_base = ((size_t)b * a.n_q_heads + (size_t)(bg % a.n_kv_heads) * a.group) * K;
  bf16x8 qf[NDS];
  {
    const bool ok = active && qrow < R;
    const uint16_t* qp = a.q + (row_base + (ok ? qrow : 0)) * D + 8 * half;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      if (ok) {
        qf[ds] = *reinterpret_cast<const bf16x8*>(qp + 16 * ds);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ds][e] = (__bf16)0.0f;
      }
    }
  }

  // ---- tile loader: registers <- global (rows beyond the valid count are zero)
  uint4 kreg[NCH], vreg[NCH];
  int tile_valid = 0;  // valid rows of the tile held in registers
  auto load_tile = [&](int t) {
    const uint16_t* kp;
    const uint16_t* vp;
    int nvalid;
    if (has_block && t == 0) {
      kp = a.k_blk + (size_t)bg * K * D;
      vp = a.v_blk + (size_t)bg * K * D;
      nvalid = K;
    } else {
      const int r0 = kstart + (t - has_block) * kTileKeys;
      kp = a.k_cache + ((size_t)bg * a.max_len + r0) * D;
      vp = a.v_cache + ((size_t)bg * a.max_len + r0) * D;
      nvalid = min(kTileKeys, kend - r0);
    }
    tile_valid = nvalid;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int n = tid + kThreads * c;
      const int row = n / DCH;
      const int ch = n % DCH;
      if (row < nvalid) {
        kreg[c] = *reinterpret_cast<const uint4*>(kp + (size_t)row * D + ch * 8);
        vreg[c] = *reinterpret_cast<const uint4*>(vp + (size_t)row * D + ch * 8);
      } else {
        kreg[c] = make_uint4(0, 0, 0, 0);
        vreg[c] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int stage) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int n = tid + kThreads * c;
      const int row = n / DCH;
      const int ch = n % DCH;
      const int off = row * ROWB + swizzle_chunk(row, ch, DCH) * 16;
      *reinterpret_cast<uint4*>(&smem[stage][0][off]) = kreg[c];
      *reinterpret_cast<uint4*>(&smem[stage][1][off]) = vreg[c];
    }
  };

  // ---- running softmax state (per lane = per query row; l is this lane's half)
  float m_run = kNegInf;
  float l_run = 0.0f;
  f32x16 oacc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[mb][r] = 0.0f;

  const float c2 = a.scale_log2;

  int stage_valid[2] = {0, 0};
  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
    stage_valid[0] = tile_valid;
    if (ntiles > 1) load_tile(1);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    const bool block_tile = has_block && t == 0;
    const int nvalid = stage_valid[stage];
    if (active) {
      const uint8_t* Ks = smem[stage][0];
      const uint8_t* Vs = smem[stage][1];
      f32x16 sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
        const int krow = ks * KPW + kb * 32 + (lane & 31);
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
          const int ch = 2 * ds + half;
          const bf16x8 kf =
              *reinterpret_cast<const bf16x8*>(Ks + krow * ROWB + swizzle_chunk(krow, ch, DCH) * 16);
          sacc[kb] = mfma32(kf, qf[ds], sacc[kb]);
        }
      }
      // ---- mask: padded / out-of-range keys, and the causal block for verify
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = ks * KPW + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          bool ok = kk < nvalid;
          if (block_tile && a.causal) ok = ok && kk <= qrow_i;
          const float s = ok ? sacc[kb][r] : kNegInf;
          sacc[kb][r] = s;
          mx = fmaxf(mx, s);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float mc = (m_new == kNegInf) ? 0.0f : m_new * c2;
      const float alpha = fast_exp2(m_run * c2 - mc);
      m_run = m_new;
      float lsum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = fast_exp2(fmaf(sacc[kb][r], c2, -mc));
          sacc[kb][r] = pv;
          lsum += pv;
        }
      l_run = l_run * alpha + lsum;
      if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;
      }
      // ---- O^T += V^T P^T
      const int grp = lane >> 4;
      const int jj = (lane & 15) >> 2;
      const int qq = lane & 3;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          bf16x8 pb;
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sacc[kb][8 * tt + e];
          const int keyA = ks * KPW + kb * 32 + 16 * tt + 4 * half + jj;
          const int keyB = keyA + 8;
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
            const int d0 = 32 * mb + 16 * (grp & 1) + 4 * qq;
            const int ch = d0 >> 3;
            const int hb = (d0 & 7) * 2;
            const uint8_t* pa = Vs + keyA * ROWB + swizzle_chunk(keyA, ch, DCH) * 16 + hb;
            const uint8_t* pbp = Vs + keyB * ROWB + swizzle_chunk(keyB, ch, DCH) * 16 + hb;
            // whole-vector bit casts: element-wise inserts of the i16 lanes into
            // the bf16 operand were lowered incorrectly by the compiler
            const bf16x4 va = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa)));
            const bf16x4 vb = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pbp)));
            const bf16x8 vf = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[mb] = mfma32(vf, pb, oacc[mb]);
          }
        }
      }
    }
    // ---- advance the pipeline: registers -> other LDS stage, next loads in flight
    if (t + 1 < ntiles) {
      store_tile(stage ^ 1);
      stage_valid[stage ^ 1] = tile_valid;
      if (t + 2 < ntiles) load_tile(t + 2);
    }
    __syncthreads();
  }

  // ---- per-row totals: this lane holds half of the keys of its row
  float l_row = l_run + __shfl_xor(l_run, 32);
  float m_out = (m_run == kNegInf) ? kNegInf : m_run * c2;

  // ---- combine the key subsets of one query block inside the work-group
  if (KS > 1) {
    float* red = reinterpret_cast<float*>(&smem[0][0][0]);
    constexpr int WSTRIDE = NMB * 16 * 64 + 2 * 64;  // floats per donor wave
    if (active && ks > 0) {
      float* dst = red + (size_t)(wave - NQB) * WSTRIDE;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[(mb * 16 + r) * 64 + lane] = oacc[mb][r];
      dst[NMB * 16 * 64 + lane] = m_out;
      dst[NMB * 16 * 64 + 64 + lane] = l_row;
    }
    __syncthreads();
    if (active && ks == 0) {
      const float* src = red + (size_t)qb * WSTRIDE;
      const float m2 = src[NMB * 16 * 64 + lane];
      const float l2 = src[NMB * 16 * 64 + 64 + lane];
      const float M = fmaxf(m_out, m2);
      const float w1 = (M == kNegInf) ? 0.0f : fast_exp2(m_out - M);
      const float w2 = (M == kNegInf) ? 0.0f : fast_exp2(m2 - M);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          oacc[mb][r] = oacc[mb][r] * w1 + src[(mb * 16 + r) * 64 + lane] * w2;
      l_row = l_row * w1 + l2 * w2;
      m_out = M;
    }
  }

  // ---- write this split's partial for the query block
  if (active && ks == 0) {
    const size_t slot = ((size_t)bg * plan.row_groups + rg) * S + split;
    const int wrow = qb * 32 + (lane & 31);
    float* acc = a.ws_acc + (slot * plan.rows_per_wg + wrow) * D;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 v;
        v[0] = oacc[mb][4 * q4 + 0];
        v[1] = oacc[mb][4 * q4 + 1];
        v[2] = oacc[mb][4 * q4 + 2];
        v[3] = oacc[mb][4 * q4 + 3];
        *reinterpret_cast<f32x4*>(acc + 32 * mb + 8 * q4 + 4 * half) = v;
      }
    if (half == 0) {
      float2 ml;
      ml.x = m_out;
      ml.y = l_row;
      *reinterpret_cast<float2*>(a.ws_ml + (slot * plan.rows_per_wg + wrow) * 2) = ml;
    }
  }
}

// Merge the splits of every query row: one row per D/4 threads, 4 head_dim
// values per thread.
template <int D>
__global__ __launch_bounds__(128) void attn_merge_kernel(AttnArgs a, AttnPlan plan) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 128 / TPR;
  const int tid = threadIdx.x;
  const long long total_rows = (long long)a.batch * a.n_kv_heads * plan.rows;
  const long long gr = (long long)blockIdx.x * RPB + tid / TPR;
  if (gr >= total_rows) return;
  const int sub = tid % TPR;
  const long long bg = gr / plan.rows;
  const int r = (int)(gr % plan.rows);
  const int rg = r / plan.rows_per_wg;
  const int rr = r % plan.rows_per_wg;
  const int S = plan.splits;
  const size_t slot0 = ((size_t)bg * plan.row_groups + rg) * S;

  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, a.ws_ml[((slot0 + s) * plan.rows_per_wg + rr) * 2]);
  float lsum = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < S; ++s) {
    const size_t idx = (slot0 + s) * plan.rows_per_wg + rr;
    const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + idx * 2);
    const float w = (ml.x == kNegInf) ? 0.0f : fast_exp2(ml.x - M);
    lsum += w * ml.y;
    const f32x4 v = *reinterpret_cast<const f32x4*>(a.ws_acc + idx * D + 4 * sub);
    acc += w * v;
  }
  const float inv = 1.0f / lsum;
  // out row index: ((b*Hq + g*G)*K + r) == bg*R + r because Hq = Hkv*G
  uint16_t* op = a.out + (size_t)gr * D + 4 * sub;
  ushort4 o;
  o.x = __builtin_bit_cast(uint16_t, (__bf16)(acc[0] * inv));
  o.y = __builtin_bit_cast(uint16_t, (__bf16)(acc[1] * inv));
  o.z = __builtin_bit_cast(uint16_t, (__bf16)(acc[2] * inv));
  o.w = __builtin_bit_cast(uint16_t, (__bf16)(acc[3] * inv));
  *reinterpret_cast<ushort4*>(op) = o;
  if (a.lse != nullptr && sub == 0) a.lse[gr] = (M + log2f(lsum)) * 0.69314718055994531f;
}

template <int D, int NQB>
hipError_t launch_split(const AttnArgs& a, const AttnPlan& p, hipStream_t stream) {
  dim3 grid(p.splits, p.row_groups, a.batch * a.n_kv_heads);
  hipLaunchKernelGGL((attn_split_kernel<D, NQB>), grid, dim3(kThreads), 0, stream, a, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& p, int phases, hipStream_t stream) {
  if (phases & 1) {
    hipError_t e;
    switch (p.qblocks) {
      case 1: e = launch_split<D, 1>(a, p, stream); break;
      case 2: e = launch_split<D, 2>(a, p, stream); break;
      default: e = launch_split<D, 4>(a, p, stream); break;
    }
    if (e != hipSuccess) return e;
  }
  if (!(phases & 2)) return hipSuccess;
  constexpr int RPB = 128 / (D / 4);
  const long long total_rows = (long long)a.batch * a.n_kv_heads * p.rows;
  const unsigned blocks = (unsigned)((total_rows + RPB - 1) / RPB);
  hipLaunchKernelGGL((attn_merge_kernel<D>), dim3(blocks), dim3(128), 0, stream, a, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_attention(const AttnArgs& a, const AttnPlan& plan, int phases,
                                  hipStream_t stream) {
  if (a.head_dim == 64) return launch_d<64>(a, plan, phases, stream);
  return launch_d<128>(a, plan, phases, stream);
}

}  // namespace orthrus
