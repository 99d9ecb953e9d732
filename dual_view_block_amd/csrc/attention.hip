// Dual-view block attention for gfx950 (MI355X): split-L cache streaming with
// bf16 MFMA, online softmax in fp32, and a cross-split log-sum-exp merge.
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
//  * Streaming: the chunk is read in tiles of 64 keys straight into a 5-stage
//    LDS ring with global_load_lds (16 bytes per lane, no register staging);
//    four tiles are in flight while one is computed.  The 16-byte chunks of
//    every K and V row are XOR-permuted per row so that both read patterns
//    below hit distinct LDS banks.  q is staged through the last ring stage
//    before the first tile needs it.
//  * Compute: wave w takes query block w%4 against key half w/4 of every
//    tile.  S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (32 keys x 32 query rows;
//    Q held in registers), so each lane owns one query row and its softmax
//    statistics need one exchange with lane^32.  O^T += V^T P^T on the same
//    MFMA: P^T is the S^T accumulator converted to bf16 in place; V^T comes
//    from the row-major V tile through ds_read_b64_tr_b16, the transposing LDS
//    read, with the key order matched to the accumulator's register order.
//    The loop is software-pipelined: while the vector ALU exponentiates S(t),
//    the same wave's matrix-core instructions compute S(t+1).
//  * Softmax: P = 2^(s*scale*log2(e) - m_ref) with a lazily raised reference
//    m_ref (raised only when a score exceeds it by more than 2^8), so the
//    accumulator rescale is rare; the sum cancels the reference exactly.
//  * The two key halves of a query block are combined through LDS.  With one
//    split the work-group normalises and writes the rows itself.  Otherwise it
//    stores a partial per row -- fp32 (m_ref, sum) and the bf16 value sum
//    normalised by that sum -- and a second kernel merges the S partials:
//    out = sum_s 2^(m_s-M) l_s o_s / sum_s 2^(m_s-M) l_s,
//    lse = (M + log2 sum_s 2^(m_s-M) l_s) * ln 2, with one wave per row.
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
constexpr int kStages = 5;  // LDS ring stages (kStages - 1 tiles in flight; q uses the last one first)
constexpr float kLazy = 8.0f;  // base-2 headroom before the softmax reference is raised
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994531f;

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

// lane `src`'s value of x, for the whole wave (the builtin moves 32-bit ints)
__device__ __forceinline__ float readlane_f(float x, int src) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(x), src));
}

// 16-byte global -> LDS copies (global_load_lds_dwordx4, scalar-base form):
// for each copy, lane l of the wave writes LDS bytes [lds + 16 l, lds + 16 l
// + 16) from global address base + off_l, with `base` uniform across the wave
// (an SGPR pair) and `off_l` a 32-bit per-lane byte offset.  The LDS address
// goes through M0 and must be the same for the whole wave; M0 is saved and
// restored around the batch (the compiler does not otherwise use M0 in these
// kernels).  The copies are invisible to the compiler's wait-count tracking:
// callers wait for them with wait_vmcnt() before reading the LDS they fill.
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ void dma16x2(const void* b0, uint32_t o0, uint32_t l0, const void* b1, uint32_t o1,
                                        uint32_t l1) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %5\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %6\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %4\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(o0), "s"(b0), "v"(o1), "s"(b1), "s"(uniform(l0)), "s"(uniform(l1))
      : "memory");
}

__device__ __forceinline__ void dma16x4(const void* b0, uint32_t o0, uint32_t l0, const void* b1, uint32_t o1,
                                        uint32_t l1, uint32_t o2, uint32_t l2, uint32_t o3, uint32_t l3) {
  // copies 0 and 2 read from b0, copies 1 and 3 from b1
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %7\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %8\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %4\n\t"
      "s_mov_b32 m0, %9\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %5, %2\n\t"
      "s_mov_b32 m0, %10\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %6, %4\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(o0), "s"(b0), "v"(o1), "s"(b1), "v"(o2), "v"(o3), "s"(uniform(l0)), "s"(uniform(l1)),
        "s"(uniform(l2)), "s"(uniform(l3))
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

// Merge of the S split partials of one output row: with per-split reference
// maxima m_s (base 2), sums l_s and normalised outputs o_s,
//   M = max_s m_s,  w_s = 2^(m_s - M) l_s,  out = sum_s w_s o_s / sum_s w_s,
//   lse = (M + log2 sum_s w_s) ln 2;  an empty split (m_s = -inf) has w_s = 0.
// One wave merges one row (D = 128) or two rows (D = 64, one per half-wave):
// lane j of a row owns head_dim values 2j and 2j + 1, and lane j also holds
// the statistics of splits j, j + D/2, ...  All SMAX partial loads are issued
// before any arithmetic (one memory round trip); splits past S re-read split
// S-1 and get weight 0.  Every sum runs in a fixed order, so all callers get
// identical bits.  `row` is inside the work-group row block; rows at or past
// `row_end` are read (clamped) but not written.
template <int D, int SMAX>
__device__ __forceinline__ void merge_wave(const AttnArgs& a, const AttnPlan& p, int grp, int row, int row_end) {
  constexpr int LPR = D / 2;                  // lanes per row
  constexpr int NW = (SMAX + LPR - 1) / LPR;  // split statistics per lane
  static_assert(LPR == 32 || LPR == 64, "head_dim 64 or 128");
  const int lane = threadIdx.x & 63;
  const int j = lane & (LPR - 1);
  const int hw = LPR == 32 ? (lane >> 5) : 0;  // which row of the wave
  const int myrow = row + hw;
  const int rrow = min(myrow, p.rows_per_wg - 1);
  const int S = a.splits;
  const size_t slot0 = (size_t)grp * S;
  uint32_t v[SMAX];
#pragma unroll
  for (int s = 0; s < SMAX; ++s) {
    const size_t idx = (slot0 + min(s, S - 1)) * p.rows_per_wg + rrow;
    v[s] = *reinterpret_cast<const uint32_t*>(a.ws_acc + idx * D + 2 * j);
  }
  float m[NW], l[NW];
#pragma unroll
  for (int c = 0; c < NW; ++c) {
    const int sp = min(c * LPR + j, S - 1);
    const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + ((slot0 + sp) * p.rows_per_wg + rrow) * 2);
    const bool real = c * LPR + j < S;
    m[c] = real ? ml.x : kNegInf;
    l[c] = real ? ml.y : 0.0f;
  }
  // M over the row's lanes
  float M = m[0];
#pragma unroll
  for (int c = 1; c < NW; ++c) M = fmaxf(M, m[c]);
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
  float wt[NW];
  float L = 0.0f;
#pragma unroll
  for (int c = 0; c < NW; ++c) {
    wt[c] = (m[c] == kNegInf) ? 0.0f : fast_exp2(m[c] - M) * l[c];
    L += wt[c];
  }
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) L += __shfl_xor(L, o);
  // out = sum_s w_s o_s in split order; w_s is read from the lane holding it
  float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
  for (int s = 0; s < SMAX; ++s) {
    const int c = s / LPR, src = s % LPR;
    float ws;
    if constexpr (LPR == 64) {
      ws = readlane_f(wt[c], src);
    } else {
      const float w0 = readlane_f(wt[c], src);
      const float w1 = readlane_f(wt[c], src + 32);
      ws = hw ? w1 : w0;
    }
    ws = s < S ? ws : 0.0f;
    acc0 = fmaf(ws, __uint_as_float(v[s] << 16), acc0);
    acc1 = fmaf(ws, __uint_as_float(v[s] & 0xFFFF0000u), acc1);
  }
  if (myrow < row_end) {
    const int rg = grp % p.row_groups;
    const int r = rg * p.rows_per_wg + myrow;  // row inside the (b, g) group
    if (r < p.rows) {
      const size_t orow = (size_t)(grp / p.row_groups) * p.rows + r;  // == (b*Hq + g*G)*K + r
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      const uint32_t o = (uint32_t)to_bf16_bits(acc0 * inv) | ((uint32_t)to_bf16_bits(acc1 * inv) << 16);
      *reinterpret_cast<uint32_t*>(a.out + orow * D + 2 * j) = o;
      if (a.lse != nullptr && j == 0) a.lse[orow] = (M + log2f(L)) * kLn2;
    }
  }
}

template <int D, int NQB>
__global__ __launch_bounds__(kThreads, 1) void attn_stream_kernel(AttnArgs a, AttnPlan plan, int direct) {
  constexpr int DCH = D / 8;               // 16-byte chunks per row
  constexpr int ROWB = D * 2;              // bytes per row
  constexpr int TILEB = kTileKeys * ROWB;  // bytes of one K or V tile
  constexpr int NDS = D / 16;              // MFMA steps over head_dim for S^T
  constexpr int NMB = D / 32;              // 32-wide head_dim blocks of O^T
  constexpr int NWAVES = kThreads / 64;
  constexpr int CPT = kTileKeys * DCH / kThreads;     // 16-byte copies per thread per array per tile
  constexpr int RED_FLOATS = NMB * 16 * 64 + 2 * 64;  // one donor wave's state
  constexpr int STAGEB = 2 * TILEB;                    // one ring stage: a K tile and a V tile
  constexpr int SMEM = kStages * STAGEB;
  constexpr int RED_BYTES = 4 * RED_FLOATS * 4;
  constexpr int QROWS = 32 * NQB;                      // query rows of the work-group block
  constexpr int QCH_BLOCKS = QROWS * DCH / 64;         // 64-chunk blocks of q
  constexpr int QSTAGE = kStages - 1;                  // q is staged where tile kStages-1 goes
  static_assert(NWAVES == 8, "eight waves: four query blocks x two key halves");
  static_assert(RED_BYTES <= SMEM, "the key-half exchange reuses the ring");
  static_assert(QROWS * ROWB <= STAGEB, "q fits one ring stage");
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
  // q rows of the block go to ring stage QSTAGE with the same copies and
  // swizzle as the K tiles; every wave reads its fragments from there after
  // the first tile's barrier, before the stage is handed to tile QSTAGE.  Rows
  // past R re-read row R-1 (their outputs are never written).
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  const uint32_t q_lds = lds_base + QSTAGE * STAGEB;
  for (int cb = wave; cb < QCH_BLOCKS; cb += 2 * NWAVES) {
    // two copies per batch; a wave's second block may lie past the end, then
    // it repeats the first (same data to the same place)
    const int cb2 = cb + NWAVES < QCH_BLOCKS ? cb + NWAVES : cb;
    const int n1 = cb * 64 + lane, n2 = cb2 * 64 + lane;
    const int row1 = n1 / DCH, row2 = n2 / DCH;
    const int src1 = min(rg * plan.rows_per_wg + row1, R - 1);
    const int src2 = min(rg * plan.rows_per_wg + row2, R - 1);
    const uint16_t* qbase = a.q + row_base * D;
    dma16x2(qbase, (uint32_t)(src1 * ROWB + swz_k<DCH>(row1, n1 % DCH) * 16), q_lds + cb * 1024, qbase,
            (uint32_t)(src2 * ROWB + swz_k<DCH>(row2, n2 % DCH) * 16), q_lds + cb2 * 1024);
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
  int src_row[CPT];
  uint32_t src_ck[CPT], src_cv[CPT];
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
    const uint32_t stage = lds_base + (uint32_t)((t % kStages) * STAGEB);
    const uint32_t rk0 = (uint32_t)(min(src_row[0], last) * ROWB);
    if constexpr (CPT == 1) {
      dma16x2(kp, rk0 + src_ck[0] * 16, stage + wave * 1024, vp, rk0 + src_cv[0] * 16, stage + TILEB + wave * 1024);
    } else {
      static_assert(CPT == 2, "copy batches are written for one or two blocks per wave");
      const uint32_t rk1 = (uint32_t)(min(src_row[1], last) * ROWB);
      dma16x4(kp, rk0 + src_ck[0] * 16, stage + wave * 1024, vp, rk0 + src_cv[0] * 16, stage + TILEB + wave * 1024,
              rk1 + src_ck[1] * 16, stage + (wave + NWAVES) * 1024, rk1 + src_cv[1] * 16,
              stage + TILEB + (wave + NWAVES) * 1024);
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
  const int krow = kbase + (lane & 31);

  // Keys of tile t: nvalid(t) of them are real; the block tile is the last.
  auto tile_valid = [&](int t) __attribute__((always_inline)) {
    return (sr.has_block && t == sr.ncache) ? K : min(kTileKeys, sr.kend - (sr.kstart + t * kTileKeys));
  };

  // K fragments of this wave's 32 keys of the tile in `stage`.  Logical chunk
  // 2*ds + half of row krow sits at byte 16 * (chunk ^ f(krow)) of the row,
  // i.e. at (32*ds) ^ kswz with kswz = 16 * (half ^ f(krow)) < ROWB, so one
  // per-lane base and an XOR per read address all NDS fragments.
  const uint32_t kswz = 16u * (uint32_t)swz_k<DCH>(krow, half);
  auto load_k = [&](int stage, bf16x8 (&kf)[NDS]) __attribute__((always_inline)) {
    const uint32_t rowb = (uint32_t)(stage * STAGEB + krow * ROWB);  // multiple of ROWB
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      kf[ds] = *reinterpret_cast<const bf16x8*>(smem + ((rowb + kswz) ^ (32u * ds)));
  };
  // V^T fragments of the tile in `stage`, in the key order of the S^T
  // accumulator registers (two MFMA k-steps of 16 keys x NMB head_dim blocks).
  // The lane reads keys kA = kbase + 4*half + jj + 16*tt and kA + 8; all four
  // are congruent mod 4, and the V swizzle depends on the row mod 4 only, so
  // one base per head_dim block plus constant row offsets address them all.
  uint32_t vbase[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int key0 = kbase + 4 * half + jj;
    const int d0 = 32 * mb + 16 * (grp16 & 1) + 4 * qq;
    vbase[mb] = (uint32_t)(TILEB + key0 * ROWB + swz_v<DCH>(key0, d0 >> 3) * 16 + (d0 & 7) * 2);
  }
  auto load_v = [&](int stage, bf16x8 (&vf)[2][NMB]) __attribute__((always_inline)) {
    // per-tile bases, opaque to the optimiser so that the constant row
    // offsets below fold into the LDS instructions instead of being
    // precomputed per read and held in registers
    uint32_t vb[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      vb[mb] = (uint32_t)(stage * STAGEB) + vbase[mb];
      asm("" : "+v"(vb[mb]));
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const uint8_t* pa = smem + vb[mb] + (16 * tt) * ROWB;
        const uint8_t* pbp = pa + 8 * ROWB;
        // whole-vector bit casts: element-wise inserts of the i16 lanes into
        // the bf16 operand were lowered incorrectly by the compiler
        const bf16x4 va = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa)));
        const bf16x4 vb = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pbp)));
        vf[tt][mb] = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
  };
  // Padded keys and, in the verify view, block keys after the row: -inf.
  auto mask_scores = [&](f32x16& s, int nvalid, bool block_tile) __attribute__((always_inline)) {
    int lim = nvalid;
    if (block_tile && a.causal) lim = min(lim, qrow_i + 1);
    // register r holds key kbase + 4*half + 8*(r/4) + r%4; compare the
    // constant part against an opaque per-lane bound (keeps the 16 key
    // indices from being precomputed and held in registers)
    int rel = lim - (kbase + 4 * half);
    asm volatile("" : "+v"(rel));
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = (8 * (r >> 2) + (r & 3)) < rel ? s[r] : kNegInf;
  };
  // Row maximum of the tile; raise the reference (rare) if it is exceeded by
  // more than 2^kLazy, rescaling the running sum and accumulator.
  auto update_ref = [&](const f32x16& s) __attribute__((always_inline)) {
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
#pragma unroll
    for (int r = 4; r < 16; r += 4) mx = fmaxf(mx, fmaxf(fmaxf(s[r], s[r + 1]), fmaxf(s[r + 2], s[r + 3])));
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
    if (__ballot(mx > mref + kLazy)) {
      const float mnew = fmaxf(mref, mx);
      const float alpha = (mref == kNegInf) ? 0.0f : fast_exp2(mref - mnew);
      mref = mnew;
      neg_mref = (mnew == kNegInf) ? 0.0f : -mnew;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) oacc[mb] *= alpha;
    }
  };
  // O^T += V^T P^T with P the exponentiated scores in bf16.
  auto pv = [&](const bf16x8 (&pb)[2], const bf16x8 (&vf)[2][NMB]) __attribute__((always_inline)) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) oacc[mb] = mfma32(vf[tt][mb], pb[tt], oacc[mb]);
  };
  auto s_mfma = [&](const bf16x8 (&kf)[NDS]) __attribute__((always_inline)) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) acc = mfma32(kf[ds], qf[ds], acc);
    return acc;
  };
  // exp2 of one score in the base-2 frame of the reference
  auto expo = [&](float s) __attribute__((always_inline)) { return fast_exp2(fmaf(s, c2, neg_mref)); };

  // ---- software pipeline over an LDS ring of kStages stages with kStages-1
  // tiles in flight.  Iteration t holds the scores S(t) in registers, waits for
  // tile t+1 and, on the same wave, issues the S(t+1) MFMAs interleaved with
  // the exponentials of S(t) (the matrix core and the vector ALU overlap),
  // then accumulates P(t) V(t).  The only loads are the copies, so the waits
  // below count them exactly: q plus tiles 0..kStages-2 are in flight at the
  // first wait.  Waves whose query block lies past the work-group's rows run
  // the same code on zero queries (no branches in the loop) and write nothing.
  auto stage_of = [](int t) __attribute__((always_inline)) { return (int)((unsigned)t % (unsigned)kStages); };
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t) issue_tile(t);
  f32x16 sa, sb;
  if (sr.ntiles > 0) {  // work-group uniform
    wait_vmcnt<2 * CPT * (kStages - 2)>();  // q and tile 0 have landed for this wave
    __syncthreads();                          // ... and for every wave
    const int row = qb * 32 + (lane & 31);
    const uint8_t* qs = smem + QSTAGE * STAGEB + row * ROWB;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      qf[ds] = *reinterpret_cast<const bf16x8*>(qs + swz_k<DCH>(row, 2 * ds + half) * 16);
      if (!active) qf[ds] = bf16x8{};
    }
    if (tile_valid(0) > kbase) {
      bf16x8 kf[NDS];
      load_k(0, kf);
      sa = s_mfma(kf);
    }
  }
  // tiles [0, nfull) are whole cache tiles: no masking, every wave computes them
  const int nfull = min((sr.kend - sr.kstart) / kTileKeys, sr.ncache);
  const int nmain = nfull > 0 ? nfull - 1 : 0;  // iterations whose next tile is whole too

  // One steady-state iteration: cur = S(t) -> P(t) V(t), nxt = S(t+1).
  auto steady = [&](int t, f32x16& cur, f32x16& nxt) __attribute__((always_inline)) {
    update_ref(cur);
    wait_vmcnt<2 * CPT * (kStages - 3)>();  // this wave's copies of tile t+1 have landed
    __syncthreads();  // everyone's have; all waves are past iteration t-1 (and the q reads)
    issue_tile(t + kStages - 1);  // into the stage tile t-1 used
    bf16x8 kf[NDS];
    load_k(stage_of(t + 1), kf);
#pragma unroll
    for (int r = 0; r < 16; ++r) nxt[r] = 0.0f;
    constexpr int EPS = 16 / NDS;  // exponentials per MFMA step
    float lsum = 0.0f;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      nxt = mfma32(kf[ds], qf[ds], nxt);
#pragma unroll
      for (int e = 0; e < EPS; ++e) {
        const float p_ = expo(cur[EPS * ds + e]);
        cur[EPS * ds + e] = p_;
        lsum += p_;
      }
    }
    l_run += lsum;
    bf16x8 pb[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[tt][e] = (__bf16)cur[8 * tt + e];
    bf16x8 vf[2][NMB];
    load_v(stage_of(t), vf);
    pv(pb, vf);
  };
  int t = 0;
  for (; t + 2 <= nmain; t += 2) {  // unrolled by two: the score registers alternate
    steady(t, sa, sb);
    steady(t + 1, sb, sa);
  }
  if (t < nmain) {
    steady(t, sa, sb);
    sa = sb;
    ++t;
  }
  // ---- the remaining (at most three) tiles: the last whole tile, a partial
  // tile, the block tile
  for (; t < sr.ntiles; ++t) {
    const int nv = tile_valid(t);
    const bool blk = sr.has_block && t == sr.ncache;
    const bool does = nv > kbase;
    if (does) {
      if (blk || nv < kbase + 32) mask_scores(sa, nv, blk);
      update_ref(sa);
      float lsum = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p_ = expo(sa[r]);
        sa[r] = p_;
        lsum += p_;
      }
      l_run += lsum;
    }
    if (t + 1 < sr.ntiles) {
      wait_vmcnt<2 * CPT * (kStages - 3)>();
      __syncthreads();
      issue_tile(t + kStages - 1);
    }
    if (does) {
      bf16x8 pb[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[tt][e] = (__bf16)sa[8 * tt + e];
      bf16x8 vf[2][NMB];
      load_v(stage_of(t), vf);
      pv(pb, vf);
    }
    if (t + 1 < sr.ntiles && tile_valid(t + 1) > kbase) {
      bf16x8 kf[NDS];
      load_k(stage_of(t + 1), kf);
      sa = s_mfma(kf);
    }
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

  if (a.splits == 1 && direct) {
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
}

// Stand-alone merge of the partials left by a streaming launch with fuse = 0:
// 256 threads, one wave per row (D = 128) or per two rows (D = 64) over all
// split groups.
constexpr int kMergeThreads = 256;
template <int D, int SMAX>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(AttnArgs a, AttnPlan plan, int total_rows) {
  constexpr int RPW = 128 / D;
  const int gw = blockIdx.x * (kMergeThreads / 64) + (int)(threadIdx.x >> 6);
  const int first = gw * RPW;  // rows_per_wg is a multiple of 32: a wave's rows share a group
  if (first >= total_rows) return;
  const int grp = first / plan.rows_per_wg;
  merge_wave<D, SMAX>(a, plan, grp, first % plan.rows_per_wg, plan.rows_per_wg);
}

template <int D, int NQB>
hipError_t launch_stream(const AttnArgs& a, const AttnPlan& p, int direct, hipStream_t stream) {
  dim3 grid(a.splits, p.row_groups, a.batch * a.n_kv_heads);
  hipLaunchKernelGGL((attn_stream_kernel<D, NQB>), grid, dim3(kThreads), 0, stream, a, p, direct);
  return hipGetLastError();
}

template <int D, int SMAX>
hipError_t launch_merge_s(const AttnArgs& a, const AttnPlan& p, hipStream_t stream) {
  constexpr int rows_per_block = (kMergeThreads / 64) * (128 / D);
  const int total = a.batch * a.n_kv_heads * p.row_groups * p.rows_per_wg;
  dim3 grid((total + rows_per_block - 1) / rows_per_block);
  hipLaunchKernelGGL((attn_merge_kernel<D, SMAX>), grid, dim3(kMergeThreads), 0, stream, a, p, total);
  return hipGetLastError();
}

template <int D>
hipError_t launch_merge(const AttnArgs& a, const AttnPlan& p, hipStream_t stream) {
  if (a.splits <= 8) return launch_merge_s<D, 8>(a, p, stream);
  if (a.splits <= 16) return launch_merge_s<D, 16>(a, p, stream);
  if (a.splits <= 32) return launch_merge_s<D, 32>(a, p, stream);
  return launch_merge_s<D, kMaxSplits>(a, p, stream);
}

template <int D>
hipError_t launch_stream_any(const AttnArgs& a, const AttnPlan& p, int direct, hipStream_t stream) {
  switch (p.qblocks) {
    case 1: return launch_stream<D, 1>(a, p, direct, stream);
    case 2: return launch_stream<D, 2>(a, p, direct, stream);
    default: return launch_stream<D, 4>(a, p, direct, stream);
  }
}

// phases 1: streaming kernel only (partials); 2: merge kernel only; 3: the
// whole call -- one launch when there is a single split (the work-group
// writes the output), otherwise the streaming kernel followed by the merge
// kernel on the same stream.
template <int D>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& p, int phases, hipStream_t stream) {
  if (phases == 1) return launch_stream_any<D>(a, p, 0, stream);
  if (phases == 2) return launch_merge<D>(a, p, stream);
  if (a.splits == 1) return launch_stream_any<D>(a, p, 1, stream);
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

hipError_t launch_block_attention(const AttnArgs& a, const AttnPlan& plan, int phases, hipStream_t stream) {
  if (a.head_dim == 64) return launch_d<64>(a, plan, phases, stream);
  return launch_d<128>(a, plan, phases, stream);
}

}  // namespace orthrus
