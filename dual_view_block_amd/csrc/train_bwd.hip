// Backward of the training dual-pass block-mask attention for the diffusion
// rows (Orthrus paper notes §3.1-3.2; the AR backbone is frozen, so only the
// diffusion queries, keys and values get gradients).
//
// For every anchor block n and KV head g, the G*K diffusion rows of the q
// heads that share g attend to the clean keys [0, a_n) and to the K keys of
// block n.  With the forward's log-sum-exp per row, P = exp(scale*QK^T - lse)
// is recomputed exactly, and
//   dP = dO V^T,  D_i = rowsum(dO * O),  dS = P * (dP - D),
//   dQ = scale * dS K          (over every key of the row)
//   dV_blk = P_blk^T dO,  dK_blk = scale * dS_blk^T Q   (block keys; the sum
//                                                          over rows covers all G heads)
//
// One work-group of 8 waves (512 threads, two per SIMD) per (block, KV head),
// numbered so that each XCD serves one KV head and its L2 keeps that head's
// clean K/V, which every block of the head re-reads.  Wave w owns rows 32*(w>>1) .. +31 (each lane one row, as in the streaming
// kernel) against key half w & 1 (32 keys) of every 64-key tile.  Per tile,
// with the tile in LDS:
//   S^T  = K Q^T      (A = K rows, B = Q fragments in registers)
//   dP^T = V dO^T     (A = V rows, B = dO fragments in registers)
//   dS^T = P^T * (dP^T - D) elementwise, rounded to bf16 in place
//   dQ^T += K^T dS^T  (A = K^T through the transposing LDS read)
// all on v_mfma_f32_32x32x16_bf16, 8 of each per wave and tile.  K is kept in
// LDS twice, once in the layout the row reads want and once in the layout
// the transposing read wants, and V once in the row-read layout, so no read
// conflicts.  Tiles come in through registers one tile ahead into a 2-stage
// LDS ring (one barrier per tile; each wave computes a tile before writing
// the next).  The two key halves of a row block add their dQ partials
// through LDS, each wave finishing half of head_dim.  After the last (block)
// tile the waves put P_blk, dS_blk, Q and dO in LDS and wave w forms dV_blk
// (w even) or dK_blk (w odd) for head_dim block w >> 1, with the row sum as
// the MFMA contraction.
#include "attn_frag.h"
#include "common.h"
#include "block_order.h"

#include <math.h>

namespace orthrus {
namespace {

using namespace frag;

constexpr int kBwdThreads = 512;
constexpr int kBwdTile = 64;

template <int D>
__global__ __launch_bounds__(kBwdThreads) void train_bwd_kernel(const TrainBwdArgs a) {
  constexpr int DCH = D / 8;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = kBwdTile * ROWB;
  constexpr int SLOT_KK = 0, SLOT_KV = TILEB, SLOT_VK = 2 * TILEB;  // K row layout, K^T layout, V row layout
  constexpr int STAGEB = 3 * TILEB;
  constexpr int HALFB = 32 * ROWB;
  constexpr int NDS = D / 16;
  constexpr int NMB = D / 32;
  constexpr int HMB = NMB / 2;  // head_dim blocks each wave of a pair finishes
  constexpr int CPT = kBwdTile * DCH / kBwdThreads;
  constexpr int OPITCH = ROWB + 16;
  static_assert(CPT >= 1 && HMB >= 1, "tile and head_dim fit the work-group");
  static_assert(8 * HMB * 16 * 64 * 4 <= 2 * STAGEB && 128 * OPITCH <= 2 * STAGEB, "epilogue fits the ring");

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGEB];

  // Work-group lin takes KV head lin % Hkv.  Work-groups go to the 8 XCDs
  // round robin, so with Hkv = 8 every XCD serves one KV head and its L2
  // holds that head's whole clean K/V (the prefix all the head's blocks
  // re-read); with blockIdx.x as the block, every XCD would touch every head.
  // 441 -> 385 us at L 2048, 256 blocks of 32, 32/8 heads.
  const int lin = (int)blockIdx.x + (int)gridDim.x * (int)blockIdx.y;
  const int g = lin % (int)gridDim.y;  // KV head
  // anchor block: longest prefix first (see block_order.h)
  const int n = a.n_blocks <= kRankMaxBlocks ? block_by_rank(a.anchors, a.n_blocks, a.seq_len, lin / (int)gridDim.y)
                                             : lin / (int)gridDim.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qb = w >> 1;  // row block
  const int kh = w & 1;   // key half of every tile
  const int half = lane >> 5;
  const int K = a.block_k;
  const int R = a.group * K;
  const bool wave_active = qb * 32 < R;
  const int wrow = qb * 32 + (lane & 31);  // this lane's row: head_in_group * K + i
  const bool active = wrow < R;
  const int hh = active ? wrow / K : 0, ii = active ? wrow % K : 0;
  const long long NK = (long long)a.n_blocks * K;
  // element offset of this lane's row in the [Hq, N*K, D] arrays
  const long long row_off = ((long long)(g * a.group + hh) * NK + (long long)n * K + ii) * D;
  int La = a.anchors[n];
  La = La < 0 ? 0 : (La > a.seq_len ? a.seq_len : La);
  const int ncache = (La + kBwdTile - 1) / kBwdTile;
  const int ntiles = ncache + 1;  // + the block tile

  // ---- tile copies through registers (thread tid moves chunks tid + c*512)
  int crow[CPT];
  uint32_t cchunk[CPT], dkk[CPT], dkv[CPT], dvk[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int m = tid + c * kBwdThreads;
    crow[c] = m / DCH;
    const int ch = m % DCH;
    cchunk[c] = (uint32_t)ch * 16;
    dkk[c] = (uint32_t)(SLOT_KK + crow[c] * ROWB + swz_k<DCH>(crow[c], ch) * 16);
    dkv[c] = (uint32_t)(SLOT_KV + crow[c] * ROWB + swz_v<DCH>(crow[c], ch) * 16);
    dvk[c] = (uint32_t)(SLOT_VK + crow[c] * ROWB + swz_k<DCH>(crow[c], ch) * 16);
  }
  const uint8_t* kc0 = reinterpret_cast<const uint8_t*>(a.k_ar + (long long)g * a.seq_len * D);
  const uint8_t* vc0 = reinterpret_cast<const uint8_t*>(a.v_ar + (long long)g * a.seq_len * D);
  const long long blk_off = ((long long)g * NK + (long long)n * K) * D;
  const uint8_t* kb0 = reinterpret_cast<const uint8_t*>(a.k_diff + blk_off);
  const uint8_t* vb0 = reinterpret_cast<const uint8_t*>(a.v_diff + blk_off);
  typedef u32x4 Stage[2 * CPT];
  // Rows past the valid count re-read the last valid row (finite data; their
  // scores are masked to -inf, so P = 0 exactly).
  auto load_tile = [&](int t, Stage& r) __attribute__((always_inline)) {
    const bool blk = t == ncache;
    const int last = blk ? K - 1 : min(kBwdTile, La - t * kBwdTile) - 1;
    const uint8_t* kp = blk ? kb0 : kc0 + (size_t)t * TILEB;
    const uint8_t* vp = blk ? vb0 : vc0 + (size_t)t * TILEB;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const uint32_t off = (uint32_t)(min(crow[c], last) * ROWB) + cchunk[c];
      r[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + off));
      r[CPT + c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + off));
    }
  };
  auto store_tile = [&](int stage, const Stage& r) __attribute__((always_inline)) {
    uint8_t* sb = smem + stage * STAGEB;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      *reinterpret_cast<u32x4*>(sb + dkk[c]) = r[c];
      *reinterpret_cast<u32x4*>(sb + dkv[c]) = r[c];
      *reinterpret_cast<u32x4*>(sb + dvk[c]) = r[CPT + c];
    }
  };

  // ---- this lane's row: Q and dO fragments (B operands), O, lse, D_i
  bf16x8 qf[NDS], df[NDS];
  float di = 0.0f;
  {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(a.q_diff + row_off);
    const bf16x8* gp = reinterpret_cast<const bf16x8*>(a.d_out + row_off);
    const bf16x8* op = reinterpret_cast<const bf16x8*>(a.out_diff + row_off);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      qf[ds] = active ? qp[2 * ds + half] : bf16x8{};
      df[ds] = active ? gp[2 * ds + half] : bf16x8{};
      const bf16x8 o = active ? op[2 * ds + half] : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) di = fmaf((float)df[ds][e], (float)o[e], di);
    }
    di += __shfl_xor(di, 32);
  }
  // P = 2^(s*c2 - m2) with m2 = lse * log2(e); inactive rows get P = 0
  const float c2 = a.scale_log2;
  const float m2 = active ? a.lse_diff[((long long)(g * a.group + hh) * NK + (long long)n * K + ii)] *
                                1.4426950408889634f
                          : __builtin_inff();

  const int grp16 = lane >> 4;
  const int jj = (lane & 15) >> 2;
  const int qq = lane & 3;
  const int krow = lane & 31;
  // row-layout reads (K and V as A operands) of this wave's 32-key half
  const uint32_t rbase = (uint32_t)(kh * HALFB + krow * ROWB) + 16u * (uint32_t)swz_k<DCH>(krow, half);
  auto load_rows = [&](int base_slot, int stage, bf16x8 (&f)[NDS]) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(stage * STAGEB + base_slot) + rbase;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) f[ds] = *reinterpret_cast<const bf16x8*>(smem + (base ^ (32u * ds)));
  };
  // transposed reads of the K^T layout: keys in the S^T accumulator order
  uint32_t tbase[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int key0 = 4 * half + jj;
    const int d0 = 32 * mb + 16 * (grp16 & 1) + 4 * qq;
    tbase[mb] = (uint32_t)(SLOT_KV + kh * HALFB + key0 * ROWB + swz_v<DCH>(key0, d0 >> 3) * 16 + (d0 & 7) * 2);
  }
  typedef bf16x8 TFrag[2][NMB];
  auto load_kt = [&](int stage, TFrag& tf) __attribute__((always_inline)) {
    uint32_t tb[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      tb[mb] = (uint32_t)(stage * STAGEB) + tbase[mb];
      asm("" : "+v"(tb[mb]));
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const uint8_t* pa = smem + tb[mb] + (16 * tt) * ROWB;
        const bf16x4 x0 = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa)));
        const bf16x4 x1 =
            __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa + 8 * ROWB)));
        tf[tt][mb] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
  };

  f32x16 dq[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[mb][r] = 0.0f;
  bf16x8 pblk[2], dsblk[2];  // block tile, keys 0..31 (key half 0): P^T and dS^T in bf16
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) pblk[ks] = dsblk[ks] = bf16x8{};

  // One tile of this wave's key half.
  auto compute = [&](int st, int t) __attribute__((always_inline)) {
    const bool blk = t == ncache;
    const int nvalid = blk ? K : min(kBwdTile, La - t * kBwdTile);
    if (!wave_active || nvalid <= 32 * kh) return;  // no real key in this half
    f32x16 s, dp;
    {
      bf16x8 kf[NDS];
      load_rows(SLOT_KK, st, kf);
      // all K fragment reads in flight before the first MFMA (doing the same
      // for the V rows below costs spills)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) s = mfma32(kf[ds], qf[ds], s);
    }
    {
      bf16x8 vf[NDS];
      load_rows(SLOT_VK, st, vf);
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = 0.0f;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) dp = mfma32(vf[ds], df[ds], dp);
    }
    // register r holds key 32*kh + 8*(r/4) + 4*half + r%4 of the tile
    int rel = nvalid - 4 * half - 32 * kh;
    asm volatile("" : "+v"(rel));
    bf16x8 dsb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool ok = (8 * (r >> 2) + (r & 3)) < rel;
      const float p = ok ? fast_exp2(fmaf(s[r], c2, -m2)) : 0.0f;
      s[r] = p;
      dp[r] = p * (dp[r] - di);
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 8; ++e) dsb[tt][e] = (__bf16)dp[8 * tt + e];
    if (blk) {  // the block keys (K <= 32) lie in key half 0
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        dsblk[tt] = dsb[tt];
#pragma unroll
        for (int e = 0; e < 8; ++e) pblk[tt][e] = (__bf16)s[8 * tt + e];
      }
    }
    TFrag tf;
    load_kt(st, tf);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) dq[mb] = mfma32(tf[tt][mb], dsb[tt], dq[mb]);
  };

  Stage stg;
  load_tile(0, stg);
  store_tile(0, stg);
  if (ntiles > 1) load_tile(1, stg);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    compute(t & 1, t);
    if (t + 1 < ntiles) {
      store_tile((t + 1) & 1, stg);  // readers of that stage finished before the last barrier
      if (t + 2 < ntiles) load_tile(t + 2, stg);
    }
    __syncthreads();
  }

  // ---- dQ: the two key halves of a row block add their partials (wave w
  // hands the head_dim blocks its partner w ^ 1 finishes, a raw register dump,
  // lane-major); then bf16 rows via LDS and coalesced stores.
  float* xch = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int j = 0; j < HMB; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) xch[((w * HMB + j) * 16 + r) * 64 + lane] = kh ? dq[j][r] : dq[HMB + j][r];
  __syncthreads();
  f32x16 own[HMB];
  {
    const int pw = w ^ 1;
#pragma unroll
    for (int j = 0; j < HMB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        own[j][r] = (kh ? dq[HMB + j][r] : dq[j][r]) + xch[((pw * HMB + j) * 16 + r) * 64 + lane];
  }
  __syncthreads();  // the exchange is consumed: the staging rows reuse it
  {
    uint8_t* orow = smem + wrow * OPITCH;
    const float sc = a.scale;
#pragma unroll
    for (int j = 0; j < HMB; ++j) {
      const int mb = kh * HMB + j;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        ushort4 o;
        o.x = to_bf16_bits(own[j][4 * q4 + 0] * sc);
        o.y = to_bf16_bits(own[j][4 * q4 + 1] * sc);
        o.z = to_bf16_bits(own[j][4 * q4 + 2] * sc);
        o.w = to_bf16_bits(own[j][4 * q4 + 3] * sc);
        *reinterpret_cast<ushort4*>(orow + 2 * (32 * mb + 8 * q4 + 4 * half)) = o;
      }
    }
  }
  __syncthreads();
  for (int m = tid; m < 128 * DCH; m += kBwdThreads) {
    const int r = m / DCH, ch = m % DCH;
    if (r < R) {
      const long long off = ((long long)(g * a.group + r / K) * NK + (long long)n * K + r % K) * D + ch * 8;
      *reinterpret_cast<u32x4*>(a.dq + off) = *reinterpret_cast<const u32x4*>(smem + r * OPITCH + ch * 16);
    }
  }
  __syncthreads();

  // ---- block keys: dV_blk^T = dO^T P_blk, dK_blk^T = scale * Q^T dS_blk,
  // contracted over all 128 rows.  LDS: P and dS as [key][row] bf16 (row
  // pitch 128 rows), Q and dO as [row][D] in the transposing-read layout,
  // written by the key-half-0 waves (which hold the block's P and dS and
  // between them every row).
  constexpr int PB = 0;                       // P_blk   [32][128] bf16
  constexpr int DSB = 32 * 128 * 2;           // dS_blk  [32][128] bf16
  constexpr int QB = 2 * DSB;                 // Q       [128][D]
  constexpr int GB = QB + 128 * ROWB;         // dO      [128][D]
  static_assert(GB + 128 * ROWB <= 2 * STAGEB, "block operands fit the ring");
  if (kh == 0) {
    const int key_lo = 4 * half;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // register 8*ks + e holds key 8*((8*ks + e)/4) + 4*half + e%4
        const int key = 8 * ((8 * ks + e) >> 2) + key_lo + (e & 3);
        *reinterpret_cast<__bf16*>(smem + PB + (key * 128 + wrow) * 2) = pblk[ks][e];
        *reinterpret_cast<__bf16*>(smem + DSB + (key * 128 + wrow) * 2) = dsblk[ks][e];
      }
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const int ch = 2 * ds + half;
      *reinterpret_cast<bf16x8*>(smem + QB + wrow * ROWB + swz_v<DCH>(wrow, ch) * 16) = qf[ds];
      *reinterpret_cast<bf16x8*>(smem + GB + wrow * ROWB + swz_v<DCH>(wrow, ch) * 16) = df[ds];
    }
  }
  __syncthreads();
  const int mb = w >> 1;     // head_dim block of this wave
  const bool want_dk = w & 1;  // dK_blk (odd waves) or dV_blk (even waves)
  if (mb < NMB) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const int row0 = 4 * half + jj;
    const int d0 = 32 * mb + 16 * (grp16 & 1) + 4 * qq;
    // A operand: Q^T (dK) or dO^T (dV); B operand: dS_blk (dK) or P_blk (dV)
    const uint32_t aoff = (uint32_t)((want_dk ? QB : GB) + row0 * ROWB + swz_v<DCH>(row0, d0 >> 3) * 16 +
                                     (d0 & 7) * 2);
    const int boff = want_dk ? DSB : PB;
    // B operand rows for k-step (h, tt): the same two runs of 4 rows the
    // transposing read returns, rows 32h + 16tt + 4*half + {0..3} and + 8
    const int key = lane & 31;
#pragma unroll
    for (int h = 0; h < 4; ++h)  // 4 x 32 rows
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int rb = 32 * h + 16 * tt;
        const uint8_t* pa = smem + aoff + rb * ROWB;
        const bf16x4 x0 = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa)));
        const bf16x4 x1 =
            __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa + 8 * ROWB)));
        const int r0 = rb + 4 * half;
        const bf16x4 b0 = *reinterpret_cast<const bf16x4*>(smem + boff + (key * 128 + r0) * 2);
        const bf16x4 b1 = *reinterpret_cast<const bf16x4*>(smem + boff + (key * 128 + r0 + 8) * 2);
        acc = mfma32(__builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7),
                     __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7), acc);
      }
    // lane: key = lane % 32, head_dim 32*mb + 8i + 4*half + j in register 4i + j
    if (key < K) {
      const long long off = blk_off + (long long)key * D + 32 * mb + 4 * half;
      const float sc = want_dk ? a.scale : 1.0f;
      uint16_t* dst = want_dk ? a.dk : a.dv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ushort4 o;
        o.x = to_bf16_bits(acc[4 * i + 0] * sc);
        o.y = to_bf16_bits(acc[4 * i + 1] * sc);
        o.z = to_bf16_bits(acc[4 * i + 2] * sc);
        o.w = to_bf16_bits(acc[4 * i + 3] * sc);
        *reinterpret_cast<ushort4*>(dst + off + 8 * i) = o;
      }
    }
  }
}

}  // namespace

hipError_t launch_train_bwd(const TrainBwdArgs& a, hipStream_t stream) {
  dim3 grid(a.n_blocks, a.n_kv_heads);
  if (a.head_dim == 64)
    hipLaunchKernelGGL(train_bwd_kernel<64>, grid, dim3(kBwdThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(train_bwd_kernel<128>, grid, dim3(kBwdThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace orthrus
