// Dual-view block attention for gfx950 (MI355X): split-L cache streaming with
// bf16 MFMA, online softmax in fp32, and a cross-split log-sum-exp merge that
// runs inside the same launch.
//
// What is computed (Orthrus paper notes, zhangshuibai.github.io, §2.1, §3.2,
// §4.1): for every (sequence b, KV head g), the G*K query rows of the q heads
// that share g attend to the cached keys [0, L_b) and to the K block keys in
// one softmax; block key j is visible to block row i always (diffusion view)
// or iff j <= i (AR verify view).
//
// Work layout.  grid = (S splits, row groups, B * Hkv); one work-group of 8
// waves (512 threads) per CU.  A work-group owns one contiguous chunk of the
// (b, g) cache rows and up to 128 query rows (4 blocks of 32); the last split
// also takes the K block keys as one extra masked tile.
//  * Streaming: the chunk is read in tiles of 64 keys.  Each thread keeps the
//    next three tiles' 128-bit loads in flight in registers (the compiler
//    tracks each with its own vmcnt) and writes the oldest into one of two
//    LDS stages per tile, with the 16-byte chunks of row r XOR-swizzled by
//    2*(r mod 8) so that both read patterns below are conflict-free.
//  * Compute: wave w takes query block w%4 against key half w/4 of every
//    tile.  S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (32 keys x 32 query rows;
//    Q held in registers), so each lane owns one query row and its softmax
//    statistics need one exchange with lane^32.  O^T += V^T P^T on the same
//    MFMA: P^T is the S^T accumulator converted to bf16 in place; V^T comes
//    from the row-major V tile through ds_read_b64_tr_b16, the transposing LDS
//    read, with the key order matched to the accumulator's register order.
//  * The two key halves of a query block are combined through LDS.  With one
//    split the work-group normalises and writes the rows itself.  Otherwise
//    it stores an unnormalised partial (max, sum, weighted value sum) per row,
//    counts itself in at the split group's arrival counter, waits (bounded)
//    until all S splits have arrived, and merges its share of the group's
//    rows: out = sum_s 2^(m_s-M) acc_s / sum_s 2^(m_s-M) l_s,
//    lse = (M + log2 sum) * ln 2.  The last work-group to leave resets the
//    counters, so the workspace is ready for the next call.
#include "common.h"

#include <math.h>

namespace orthrus {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // plain vector: stays in registers
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kThreads = kAttnThreads;
constexpr int kStages = 4;  // LDS ring stages (kStages - 1 tiles in flight)
constexpr float kLazy = 8.0f;  // base-2 headroom before the softmax reference is raised
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994531f;
constexpr unsigned kSpinLimit = 1u << 20;  // arrival wait bound (about a second)
constexpr int kCounterStride = 32;           // uint32 per split group: one 128-byte line each

// LDS layouts of the K and V tiles (and of q): the 16-byte chunks of a row are
// permuted by an XOR with a row-dependent value so that the read patterns hit
// distinct banks.  K (and q) rows are read 16 lanes per row index apart, so
// 16 consecutive rows get 16 different chunk offsets.  V is read through the
// transposing LDS read, where 16 lanes take 4 consecutive rows x 2 adjacent
// chunks; XOR with 4 * (row mod 4) gives those 4 rows disjoint chunk quads.
template <int DCH>
__device__ __forceinline__ int swz_k(int row, int chunk) {
  if constexpr (DCH == 16) return chunk ^ (row & 15);
  else return chunk ^ ((row >> 1) & 7);
}
template <int DCH>
__device__ __forceinline__ int swz_v(int row, int chunk) {
  if constexpr (DCH == 16) return chunk ^ (4 * (row & 3));
  else return chunk ^ (2 * (row & 3));
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte global -> LDS copies (global_load_lds_dwordx4): for each copy, lane
// l of the wave writes LDS bytes [lds + 16 l, lds + 16 l + 16) from its own
// global address.  The LDS address goes through M0 and must be the same for
// the whole wave; M0 is saved and restored around the batch (the compiler does
// not otherwise use M0 in these kernels).  The copies are invisible to the
// compiler's wait-count tracking: callers wait for them with wait_vmcnt()
// before reading the LDS they fill.
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ void dma16x2(const void* s0, uint32_t l0, const void* s1, uint32_t l1) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(s0), "v"(s1), "s"(uniform(l0)), "s"(uniform(l1))
      : "memory");
}

__device__ __forceinline__ void dma16x4(const void* s0, uint32_t l0, const void* s1, uint32_t l1,
                                        const void* s2, uint32_t l2, const void* s3, uint32_t l3) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %5\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %6\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %7\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, off\n\t"
      "s_mov_b32 m0, %8\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %4, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(s0), "v"(s1), "v"(s2), "v"(s3), "s"(uniform(l0)), "s"(uniform(l1)), "s"(uniform(l2)),
        "s"(uniform(l3))
      : "memory");
}

// s_waitcnt vmcnt(N) (N < 64), leaving the other counters unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Cache range of one split of sequence b: [kstart, kend).
struct SplitRange {
  int kstart, kend, ncache, has_block, ntiles;
};

__device__ __forceinline__ SplitRange split_range(const AttnArgs& a, int b, int split) {
  SplitRange r;
  int L = a.cache_len[b];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  const int S = a.splits;
  int chunk = (L + S - 1) / S;
  chunk = (chunk + kTileKeys - 1) / kTileKeys * kTileKeys;
  r.kstart = split * chunk;
  r.kend = min(r.kstart + chunk, L);
  r.ncache = r.kstart < r.kend ? (r.kend - r.kstart + kTileKeys - 1) / kTileKeys : 0;
  r.has_block = split == S - 1 ? 1 : 0;
  r.ntiles = r.ncache + r.has_block;
  return r;
}

// Merge rows [r0, r1) (indices inside the work-group row block) of split group
// `grp` from its S partials.  Each row is handled by D/4 threads x 4 split
// lanes: thread (row, d4, sg) folds splits sg, sg+4, sg+8, ... of four head_dim
// values with a running (max, sum) -- its loads are independent of each other,
// so they are all in flight at once -- and the four split lanes are then
// combined with two butterfly exchanges in a fixed order.  Shared by the fused
// path and the stand-alone merge kernel, so both give identical bits.
template <int D>
__device__ void merge_rows(const AttnArgs& a, const AttnPlan& p, int grp, int r0, int r1) {
  constexpr int TPR = (D / 4) * 4;        // threads per row: 4 head_dim values x 4 split lanes
  constexpr int RPP = kThreads / TPR;     // rows per pass
  static_assert(RPP >= 1, "work-group too small for one merged row");
  const int S = a.splits;
  const int tid = threadIdx.x;
  const int sg = tid & 3;                 // split lane (adjacent lanes: cheap exchanges)
  const int d4 = (tid >> 2) % (D / 4);
  const int bg = grp / p.row_groups;
  const int rg = grp % p.row_groups;
  const size_t slot0 = (size_t)grp * S;
  for (int base = r0; base < r1; base += RPP) {
    const int row = base + tid / TPR;
    const int r = rg * p.rows_per_wg + row;  // row inside the (b, g) group
    const bool ok = row < r1 && r < p.rows;
    float M = kNegInf, lsum = 0.0f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (ok) {
#pragma unroll 4
      for (int s = sg; s < S; s += 4) {
        const size_t idx = (slot0 + s) * p.rows_per_wg + row;
        const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + idx * 2);
        const ushort4 vb = *reinterpret_cast<const ushort4*>(a.ws_acc + idx * D + 4 * d4);
        if (ml.x == kNegInf) continue;  // empty split: contributes nothing
        f32x4 v;
        v[0] = bf16_bits_to_f32(vb.x);
        v[1] = bf16_bits_to_f32(vb.y);
        v[2] = bf16_bits_to_f32(vb.z);
        v[3] = bf16_bits_to_f32(vb.w);
        const float Mn = fmaxf(M, ml.x);
        const float wo = (M == kNegInf) ? 0.0f : fast_exp2(M - Mn);
        const float wn = fast_exp2(ml.x - Mn) * ml.y;  // the partial is normalised by its sum
        lsum = lsum * wo + wn;
        acc = acc * wo + v * wn;
        M = Mn;
      }
    }
    // combine the four split lanes: (0,1), (2,3), then (01, 23)
#pragma unroll
    for (int o = 1; o <= 2; o <<= 1) {
      const float Mo = __shfl_xor(M, o);
      const float lo = __shfl_xor(lsum, o);
      f32x4 ao;
      ao[0] = __shfl_xor(acc[0], o);
      ao[1] = __shfl_xor(acc[1], o);
      ao[2] = __shfl_xor(acc[2], o);
      ao[3] = __shfl_xor(acc[3], o);
      // order-independent pairing: the lower split lane's values come first
      const bool low = (sg & o) == 0;
      const float Ma = low ? M : Mo, Mb = low ? Mo : M;
      const float la = low ? lsum : lo, lb = low ? lo : lsum;
      const f32x4 aa = low ? acc : ao, ab = low ? ao : acc;
      const float Mn = fmaxf(Ma, Mb);
      const float wa = (Ma == kNegInf) ? 0.0f : fast_exp2(Ma - Mn);
      const float wb = (Mb == kNegInf) ? 0.0f : fast_exp2(Mb - Mn);
      lsum = la * wa + lb * wb;
      acc = aa * wa + ab * wb;
      M = Mn;
    }
    if (ok && sg == 0) {
      const size_t orow = (size_t)bg * p.rows + r;  // == (b*Hq + g*G)*K + r since Hq = Hkv*G
      const float inv = 1.0f / lsum;
      ushort4 o;
      o.x = to_bf16_bits(acc[0] * inv);
      o.y = to_bf16_bits(acc[1] * inv);
      o.z = to_bf16_bits(acc[2] * inv);
      o.w = to_bf16_bits(acc[3] * inv);
      *reinterpret_cast<ushort4*>(a.out + orow * D + 4 * d4) = o;
      if (a.lse != nullptr && d4 == 0) a.lse[orow] = (M + log2f(lsum)) * kLn2;
    }
  }
}

template <int D, int NQB>
__global__ __launch_bounds__(kThreads, 1) void attn_stream_kernel(AttnArgs a, AttnPlan plan, int fuse) {
  constexpr int DCH = D / 8;               // 16-byte chunks per row
  constexpr int ROWB = D * 2;              // bytes per row
  constexpr int TILEB = kTileKeys * ROWB;  // bytes of one K or V tile
  constexpr int NDS = D / 16;              // MFMA steps over head_dim for S^T
  constexpr int NMB = D / 32;              // 32-wide head_dim blocks of O^T
  constexpr int NWAVES = kThreads / 64;
  constexpr int CPT = kTileKeys * DCH / kThreads;     // 16-byte copies per thread per array per tile
  constexpr int RED_FLOATS = NMB * 16 * 64 + 2 * 64;  // one donor wave's state
  constexpr int RING_BYTES = kStages * 2 * TILEB;
  constexpr int RED_BYTES = 4 * RED_FLOATS * 4;
  constexpr int QROWS = 32 * NQB;                      // query rows of the work-group block
  constexpr int QCH_BLOCKS = QROWS * DCH / 64;         // 64-chunk blocks of q
  constexpr int SMEM = (RING_BYTES > RED_BYTES ? RING_BYTES : RED_BYTES) + QROWS * ROWB;
  static_assert(NWAVES == 8, "eight waves: four query blocks x two key halves");
  static_assert(RED_BYTES <= RING_BYTES, "the key-half exchange reuses the ring");
  static_assert(CPT >= 1, "tile too small for the work-group");

  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];

  const int split = blockIdx.x;
  const int rg = blockIdx.y;
  const int bg = blockIdx.z;
  const int grp = bg * plan.row_groups + rg;
  const int b = bg / a.n_kv_heads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int qb = wave & 3;   // query block of this wave
  const int kh = wave >> 2;  // which 32-key half of every tile this wave takes
  const bool active = qb < NQB;
  const int R = plan.rows;
  const int K = a.block_k;
  const SplitRange sr = split_range(a, b, split);
  const size_t row_base = (size_t)bg * R;  // first output row of the (b, g) group

  // ---- this lane's query row (the N index of every MFMA it joins)
  const int wrow = qb * 32 + (lane & 31);         // row inside the work-group block
  const int qrow = rg * plan.rows_per_wg + wrow;  // row inside the (b, g) group
  const int qrow_i = qrow % K;                    // its block position (row = head_in_group*K + i)
  // q rows of the block go to LDS (after the ring) with the same copies and
  // swizzle as the K tiles; every wave reads its fragments from there after
  // the first tile's barrier.  Rows past R re-read row R-1 (their outputs are
  // never written).
  const uint32_t q_lds = (uint32_t)(uintptr_t)(smem + (RING_BYTES > RED_BYTES ? RING_BYTES : RED_BYTES));
  for (int cb = wave; cb < QCH_BLOCKS; cb += 2 * NWAVES) {
    // two copies per batch; a wave's second block may lie past the end, then
    // it repeats the first (same data to the same place)
    const int cb2 = cb + NWAVES < QCH_BLOCKS ? cb + NWAVES : cb;
    const int n1 = cb * 64 + lane, n2 = cb2 * 64 + lane;
    const int row1 = n1 / DCH, row2 = n2 / DCH;
    const int src1 = min(rg * plan.rows_per_wg + row1, R - 1);
    const int src2 = min(rg * plan.rows_per_wg + row2, R - 1);
    dma16x2(a.q + (row_base + src1) * D + swz_k<DCH>(row1, n1 % DCH) * 8, q_lds + cb * 1024,
            a.q + (row_base + src2) * D + swz_k<DCH>(row2, n2 % DCH) * 8, q_lds + cb2 * 1024);
  }
  bf16x8 qf[NDS];

  // ---- tile t -> LDS stage t % kStages by direct-to-LDS copies.  Wave w
  // fills 64-chunk blocks w, w + 8, ... of the K tile and of the V tile in the
  // swizzled layout: LDS chunk n = row * DCH + pc holds the row's logical
  // chunk pc ^ swizzle(row).  Rows past the valid count re-read the last valid
  // row (finite data; their scores are masked to -inf, so P = 0 exactly).
  // Tiles past the end copy the first block-key row (one 256-byte row: no
  // HBM traffic to speak of) into a stage nobody reads any more, so every wave
  // always has the same number of copies in flight and the waits are constants.
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  int src_row[CPT], src_ck[CPT], src_cv[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int n = (wave + NWAVES * c) * 64 + lane;
    src_row[c] = n / DCH;
    src_ck[c] = swz_k<DCH>(src_row[c], n % DCH);  // logical chunk stored at this slot of the K tile
    src_cv[c] = swz_v<DCH>(src_row[c], n % DCH);  // ... of the V tile
  }
  auto issue_tile = [&](int t) __attribute__((always_inline)) {
    const bool real = t < sr.ntiles;
    const bool blk = sr.has_block && t == sr.ncache;
    const int r0 = sr.kstart + t * kTileKeys;
    const size_t cache_off = ((size_t)bg * a.max_len + r0) * D;
    const size_t blk_off = (size_t)bg * K * D;
    const uint16_t* kp = !real ? a.k_blk : (blk ? a.k_blk + blk_off : a.k_cache + cache_off);
    const uint16_t* vp = !real ? a.k_blk : (blk ? a.v_blk + blk_off : a.v_cache + cache_off);
    const int last = (!real ? 1 : (blk ? K : min(kTileKeys, sr.kend - r0))) - 1;
    const uint32_t stage = lds_base + (uint32_t)((t % kStages) * 2 * TILEB);
    const int rk0 = min(src_row[0], last) * D;
    if constexpr (CPT == 1) {
      dma16x2(kp + rk0 + src_ck[0] * 8, stage + wave * 1024, vp + rk0 + src_cv[0] * 8,
              stage + TILEB + wave * 1024);
    } else {
      static_assert(CPT == 2, "copy batches are written for one or two blocks per wave");
      const int rk1 = min(src_row[1], last) * D;
      dma16x4(kp + rk0 + src_ck[0] * 8, stage + wave * 1024, vp + rk0 + src_cv[0] * 8,
              stage + TILEB + wave * 1024, kp + rk1 + src_ck[1] * 8, stage + (wave + NWAVES) * 1024,
              vp + rk1 + src_cv[1] * 8, stage + TILEB + (wave + NWAVES) * 1024);
    }
  };

  // ---- running softmax state of this lane's row.  `mref` is a reference
  // maximum in base-2 units (score * scale * log2 e): P = 2^(s*c2 - mref).  It
  // is only raised when a score exceeds it by more than 2^kLazy, so P <= 2^8
  // (exact in bf16 and fp32) and the accumulator rescale runs on a handful of
  // tiles only; normalisation by the sum makes the reference cancel exactly.
  float mref = kNegInf, neg_mref = 0.0f;
  float l_run = 0.0f;  // this lane's half of the keys of each 32-key block
  f32x16 oacc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[mb][r] = 0.0f;
  const float c2 = a.scale_log2;
  const int kbase = kh * 32;  // first key of this wave's half
  const int grp16 = lane >> 4;
  const int jj = (lane & 15) >> 2;
  const int qq = lane & 3;

  auto compute_tile = [&](int stage, int nvalid, bool block_tile) __attribute__((always_inline)) {
    if (!active || nvalid <= kbase) return;  // wave-uniform
    const uint8_t* Ks = smem + stage * 2 * TILEB;
    const uint8_t* Vs = Ks + TILEB;
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
    const int krow = kbase + (lane & 31);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const int ch = 2 * ds + half;
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + krow * ROWB + swz_k<DCH>(krow, ch) * 16);
      sacc = mfma32(kf, qf[ds], sacc);
    }
    // mask padded keys and, for the verify view, block keys after the row
    if (block_tile || nvalid < kbase + 32) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = kbase + 8 * (r >> 2) + 4 * half + (r & 3);
        bool ok = kk < nvalid;
        if (block_tile && a.causal) ok = ok && kk <= qrow_i;
        sacc[r] = ok ? sacc[r] : kNegInf;
      }
    }
    float mx = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
#pragma unroll
    for (int r = 4; r < 16; r += 4)
      mx = fmaxf(mx, fmaxf(fmaxf(sacc[r], sacc[r + 1]), fmaxf(sacc[r + 2], sacc[r + 3])));
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
    if (__ballot(mx > mref + kLazy)) {  // rare: raise the reference, rescale
      const float mnew = fmaxf(mref, mx);
      const float alpha = (mref == kNegInf) ? 0.0f : fast_exp2(mref - mnew);
      mref = mnew;
      neg_mref = (mnew == kNegInf) ? 0.0f : -mnew;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) oacc[mb] *= alpha;
    }
    float lsum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pv = fast_exp2(fmaf(sacc[r], c2, neg_mref));
      sacc[r] = pv;
      lsum += pv;
    }
    l_run += lsum;
    // O^T += V^T P^T over the 32 keys, two MFMA k-steps of 16
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sacc[8 * tt + e];
      const int keyA = kbase + 16 * tt + 4 * half + jj;
      const int keyB = keyA + 8;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const int d0 = 32 * mb + 16 * (grp16 & 1) + 4 * qq;
        const int ch = d0 >> 3;
        const int hb = (d0 & 7) * 2;
        const uint8_t* pa = Vs + keyA * ROWB + swz_v<DCH>(keyA, ch) * 16 + hb;
        const uint8_t* pbp = Vs + keyB * ROWB + swz_v<DCH>(keyB, ch) * 16 + hb;
        // whole-vector bit casts: element-wise inserts of the i16 lanes into
        // the bf16 operand were lowered incorrectly by the compiler
        const bf16x4 va = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa)));
        const bf16x4 vb = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pbp)));
        const bf16x8 vf = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[mb] = mfma32(vf, pb, oacc[mb]);
      }
    }
  };

  // ---- pipeline: kStages-stage LDS ring, kStages-1 tiles in flight.  The
  // only loads are the copies, so the waits below count them exactly.
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t) issue_tile(t);
  for (int t = 0; t < sr.ntiles; ++t) {
    wait_vmcnt<2 * CPT * (kStages - 2)>();  // this wave's copies of tile t (and of q) have landed
    __syncthreads();                          // everyone's have; stage (t-1) % kStages is free
    if (t == 0) {
      const int row = qb * 32 + (lane & 31);
      const uint8_t* qs = smem + (RING_BYTES > RED_BYTES ? RING_BYTES : RED_BYTES) + row * ROWB;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds)
        qf[ds] = *reinterpret_cast<const bf16x8*>(qs + swz_k<DCH>(row, 2 * ds + half) * 16);
    }
    issue_tile(t + kStages - 1);
    const bool blk = sr.has_block && t == sr.ncache;
    compute_tile(t % kStages, blk ? K : min(kTileKeys, sr.kend - (sr.kstart + t * kTileKeys)), blk);
  }
  wait_vmcnt<0>();  // trailing copies land before the ring is reused below

  // ---- per-row totals: this lane holds half of the keys of its 32-key blocks
  float l_row = l_run + __shfl_xor(l_run, 32);
  float m_out = mref;  // base-2 reference of acc and l

  // ---- combine the two key halves of every query block through LDS
  __syncthreads();
  {
    float* slot = reinterpret_cast<float*>(smem) + (size_t)qb * RED_FLOATS;
    if (active && kh == 1) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) slot[(mb * 16 + r) * 64 + lane] = oacc[mb][r];
      slot[NMB * 16 * 64 + lane] = m_out;
      slot[NMB * 16 * 64 + 64 + lane] = l_row;
    }
    __syncthreads();
    if (active && kh == 0) {
      const float m2 = slot[NMB * 16 * 64 + lane];
      const float l2 = slot[NMB * 16 * 64 + 64 + lane];
      const float M = fmaxf(m_out, m2);
      const float w1 = (m_out == kNegInf) ? 0.0f : fast_exp2(m_out - M);
      const float w2 = (m2 == kNegInf) ? 0.0f : fast_exp2(m2 - M);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[mb][r] = oacc[mb][r] * w1 + slot[(mb * 16 + r) * 64 + lane] * w2;
      l_row = l_row * w1 + l2 * w2;
      m_out = M;
    }
  }
  const bool owner = active && kh == 0;

  if (a.splits == 1 && fuse) {
    // ---- one split: this work-group holds the final softmax of its rows
    if (owner && qrow < R) {
      const float inv = 1.0f / l_row;
      uint16_t* op = a.out + (row_base + qrow) * D;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          ushort4 o;
          o.x = to_bf16_bits(oacc[mb][4 * q4 + 0] * inv);
          o.y = to_bf16_bits(oacc[mb][4 * q4 + 1] * inv);
          o.z = to_bf16_bits(oacc[mb][4 * q4 + 2] * inv);
          o.w = to_bf16_bits(oacc[mb][4 * q4 + 3] * inv);
          *reinterpret_cast<ushort4*>(op + 32 * mb + 8 * q4 + 4 * half) = o;
        }
      if (a.lse != nullptr && half == 0) a.lse[row_base + qrow] = (m_out + log2f(l_row)) * kLn2;
    }
    return;
  }

  // ---- store this split's partial: (reference max, sum) in fp32 and the
  // normalised output acc / sum in bf16
  {
    const size_t slot = (size_t)grp * a.splits + split;
    if (owner) {
      const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
      uint16_t* acc = a.ws_acc + (slot * plan.rows_per_wg + wrow) * D;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          ushort4 o;
          o.x = to_bf16_bits(oacc[mb][4 * q4 + 0] * inv);
          o.y = to_bf16_bits(oacc[mb][4 * q4 + 1] * inv);
          o.z = to_bf16_bits(oacc[mb][4 * q4 + 2] * inv);
          o.w = to_bf16_bits(oacc[mb][4 * q4 + 3] * inv);
          *reinterpret_cast<ushort4*>(acc + 32 * mb + 8 * q4 + 4 * half) = o;
        }
      if (half == 0) {
        float2 ml;
        ml.x = m_out;
        ml.y = l_row;
        *reinterpret_cast<float2*>(a.ws_ml + (slot * plan.rows_per_wg + wrow) * 2) = ml;
      }
    }
  }
  if (!fuse) return;

  // ---- arrive, wait for the whole split group, merge a share of its rows.
  // The work-group barrier makes every wave's partial stores visible to thread
  // 0; its release RMW at agent scope then publishes them (one L2 write-back
  // per work-group).  Polling is relaxed (no cache maintenance per poll); one
  // acquire fence after the wait makes the other splits' partials visible.
  uint32_t* cnt = a.counters + kCounterStride * (size_t)grp;
  const unsigned S = (unsigned)a.splits;
  __syncthreads();
  if (tid == 0) {
    __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    for (unsigned n = 0; n < kSpinLimit; ++n) {
      if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= S) break;
      __builtin_amdgcn_s_sleep(8);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  const int share = (plan.rows_per_wg + a.splits - 1) / a.splits;
  const int r0 = split * share;
  const int r1 = min(plan.rows_per_wg, r0 + share);
  merge_rows<D>(a, plan, grp, r0, r1);
  __syncthreads();
  if (tid == 0) {
    const unsigned d = __hip_atomic_fetch_add(cnt + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == S - 1) {
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(cnt + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Stand-alone merge of the partials left by a streaming launch with fuse = 0:
// one work-group per (split group, chunk of rows).
template <int D>
__global__ __launch_bounds__(kThreads) void attn_merge_kernel(AttnArgs a, AttnPlan plan, int rows_per_block) {
  const int grp = blockIdx.y;
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(plan.rows_per_wg, r0 + rows_per_block);
  merge_rows<D>(a, plan, grp, r0, r1);
}

template <int D, int NQB>
hipError_t launch_stream(const AttnArgs& a, const AttnPlan& p, int fuse, hipStream_t stream) {
  dim3 grid(a.splits, p.row_groups, a.batch * a.n_kv_heads);
  hipLaunchKernelGGL((attn_stream_kernel<D, NQB>), grid, dim3(kThreads), 0, stream, a, p, fuse);
  return hipGetLastError();
}

template <int D>
hipError_t launch_merge(const AttnArgs& a, const AttnPlan& p, hipStream_t stream) {
  constexpr int rows_per_block = kThreads / D;  // one merged row per D threads
  const int groups = a.batch * a.n_kv_heads * p.row_groups;
  dim3 grid((p.rows_per_wg + rows_per_block - 1) / rows_per_block, groups);
  hipLaunchKernelGGL((attn_merge_kernel<D>), grid, dim3(kThreads), 0, stream, a, p, rows_per_block);
  return hipGetLastError();
}

template <int D>
hipError_t launch_stream_any(const AttnArgs& a, const AttnPlan& p, int fuse, hipStream_t stream) {
  switch (p.qblocks) {
    case 1: return launch_stream<D, 1>(a, p, fuse, stream);
    case 2: return launch_stream<D, 2>(a, p, fuse, stream);
    default: return launch_stream<D, 4>(a, p, fuse, stream);
  }
}

// phases 1: streaming kernel only (partials); 2: merge kernel only; 3: the
// whole call -- one launch when there is a single split (the work-group
// writes the output) or when the in-kernel merge is selected, otherwise the
// streaming kernel followed by the merge kernel.
template <int D>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& p, int phases, bool fused_merge, hipStream_t stream) {
  if (phases == 1) return launch_stream_any<D>(a, p, 0, stream);
  if (phases == 2) return launch_merge<D>(a, p, stream);
  if (a.splits == 1 || fused_merge) return launch_stream_any<D>(a, p, 1, stream);
  const hipError_t e = launch_stream_any<D>(a, p, 0, stream);
  if (e != hipSuccess) return e;
  return launch_merge<D>(a, p, stream);
}

}  // namespace

int attn_launch_splits(const AttnPlan& plan, int batch, int n_kv_heads, int max_len, int cus) {
  const long long groups = (long long)batch * n_kv_heads * plan.row_groups;
  long long s = cus / groups;  // at most one work-group per CU when splitting
  const long long tiles = (max_len + kTileKeys - 1) / kTileKeys;
  if (s > tiles) s = tiles;
  if (s > plan.splits) s = plan.splits;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_block_attention(const AttnArgs& a, const AttnPlan& plan, int phases, bool fused_merge,
                                  hipStream_t stream) {
  if (a.head_dim == 64) return launch_d<64>(a, plan, phases, fused_merge, stream);
  return launch_d<128>(a, plan, phases, fused_merge, stream);
}

}  // namespace orthrus
