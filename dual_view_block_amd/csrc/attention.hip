// Dual-view block attention for gfx950 (MI355X): split-L cache streaming with
// bf16 MFMA, online softmax in fp32, and a cross-split log-sum-exp merge.
//
// What is computed (Orthrus paper notes, zhangshuibai.github.io, §2.1, §3.2,
// §4.1): for every (sequence b, KV head g), the G*K query rows of the q heads
// that share g attend to the cached keys [0, L_b) and to the K block keys in
// one softmax; block key j is visible to block row i always (diffusion view)
// or iff j <= i (AR verify view).
//
// Work layout.  grid = (S splits, row groups, B * Hkv); one work-group of 4
// waves (256 threads, one wave per SIMD) per CU.  A work-group owns one
// contiguous chunk of the (b, g) cache rows and up to 128 query rows (4
// blocks of 32, one per wave); the last split also takes the K block keys as
// one extra masked tile.
//  * Streaming: the chunk is read in tiles of 64 keys (16 KiB of K and 16 KiB
//    of V at D = 128).  Every thread issues coalesced 16-byte nontemporal
//    loads into registers two tiles ahead of use, then writes them into a
//    4-stage LDS ring (tiles t-1 .. t+2, 128 KiB) at the row's permuted chunk
//    position; one barrier per tile orders writes and reads.  The 16-byte
//    chunks of every K and V row are XOR-permuted per row so that both read
//    patterns below hit distinct LDS banks.
//  * Compute: each wave takes its query block against both 32-key halves of
//    every tile.  S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (32 keys x 32 query
//    rows; Q held in registers), so each lane owns one query row and its
//    softmax statistics need one exchange with lane^32 (a permlane32 swap).
//    O^T += V^T P^T on the same MFMA: P^T is the S^T accumulator converted to
//    bf16 in place; V^T comes from the row-major V tile through
//    ds_read_b64_tr_b16, the transposing LDS read, with the key order matched
//    to the accumulator's register order.  The loop is software-pipelined
//    with P V delayed by one tile: iteration t interleaves the S(t+1) MFMAs,
//    the P(t-1) V(t-1) MFMAs and the exponentials of S(t).
//  * Softmax: P = 2^(s*scale*log2(e) - m_ref) with a lazily raised reference
//    m_ref (raised only when a shifted score exceeds it by more than 2^8; a
//    raise first flushes the pending P V), so the accumulator rescale is
//    rare; the sum cancels the reference exactly.
//  * Epilogue: with one split the work-group normalises and writes the rows
//    itself.  Otherwise it stores a partial per row -- fp32 (m_ref, sum) and
//    the bf16 value sum normalised by that sum, staged through LDS and written
//    as whole coalesced rows -- and a second kernel merges the S partials:
//    out = sum_s 2^(m_s-M) l_s o_s / sum_s 2^(m_s-M) l_s,
//    lse = (M + log2 sum_s 2^(m_s-M) l_s) * ln 2, with one wave per row.
#include "attn_frag.h"
#include "common.h"

#include <math.h>

namespace orthrus {
namespace {

using namespace frag;

constexpr int kThreads = kAttnThreads;
constexpr int kStages = 4;  // LDS ring stages: tiles t-1 .. t+2
constexpr float kLazy = 8.0f;  // base-2 headroom before the softmax reference is raised
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994531f;

// Cache range of one split of sequence b: [kstart, kend).
struct SplitRange {
  int kstart, kend, ncache, has_block, ntiles;  // block tiles: ncache .. ntiles-1 when has_block
};

__device__ __forceinline__ SplitRange split_range(const AttnArgs& a, int b, int split) {
  SplitRange r;
  int L = a.len_step > 0 ? b * a.len_step : a.cache_len[b];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  const int S = a.splits;
  int chunk = (L + S - 1) / S;
  chunk = (chunk + kTileKeys - 1) / kTileKeys * kTileKeys;
  r.kstart = split * chunk;
  r.kend = min(r.kstart + chunk, L);
  r.ncache = r.kstart < r.kend ? (r.kend - r.kstart + kTileKeys - 1) / kTileKeys : 0;
  r.has_block = split == S - 1 ? 1 : 0;
  r.ntiles = r.ncache + (r.has_block ? (a.block_k + kTileKeys - 1) / kTileKeys : 0);
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
    const int r = rg * p.rows_per_wg + myrow;  // row inside the (b, g) group: head_in_group*K + i
    if (r < p.rows) {
      const int bg = grp / p.row_groups;
      const int b = bg / a.n_kv_heads, h = (bg % a.n_kv_heads) * a.group + r / a.block_k, i = r % a.block_k;
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      const uint32_t o = (uint32_t)to_bf16_bits(acc0 * inv) | ((uint32_t)to_bf16_bits(acc1 * inv) << 16);
      *reinterpret_cast<uint32_t*>(a.out + b * a.o_bs + h * a.o_hs + (long long)i * D + 2 * j) = o;
      if (a.lse != nullptr && j == 0) a.lse[b * a.l_bs + h * a.l_hs + i] = (M + log2f(L)) * kLn2;
    }
  }
}

// EXPL: the block tile takes the explicit per-row masks of a.blk_mask (a
// separate instantiation, so the mode-masked launches keep their registers).
template <int D, int NQB, bool EXPL>
__global__ __launch_bounds__(kThreads, 1) void attn_stream_kernel(AttnArgs a, AttnPlan plan, int direct) {
  constexpr int DCH = D / 8;               // 16-byte chunks per row
  constexpr int ROWB = D * 2;              // bytes per row
  constexpr int TILEB = kTileKeys * ROWB;  // bytes of one K or V tile
  constexpr int STAGEB = 2 * TILEB;        // one ring stage: a K tile and a V tile
  constexpr int HALFB = 32 * ROWB;         // offset of a tile's second 32-key half
  constexpr int NDS = D / 16;              // MFMA steps over head_dim for S^T
  constexpr int NMB = D / 32;              // 32-wide head_dim blocks of O^T
  constexpr int NWAVES = kThreads / 64;
  constexpr int CPT = kTileKeys * DCH / kThreads;  // 16-byte chunks per thread per array per tile
  static_assert(NWAVES == 4, "four waves, one 32-row query block each");
  static_assert(CPT >= 1, "tile too small for the work-group");
  static_assert(4 * NMB == 2 * NDS, "two PV MFMAs per S step");

  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * STAGEB];

  const int split = blockIdx.x;
  const int rg = blockIdx.y;
  const int bg = blockIdx.z;
  const int grp = bg * plan.row_groups + rg;
  const int b = bg / a.n_kv_heads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int qb = __builtin_amdgcn_readfirstlane(tid >> 6);  // this wave's query block
  const int half = lane >> 5;
  const bool active = qb < NQB;
  const int R = plan.rows;
  const int K = a.block_k;
  const SplitRange sr = split_range(a, b, split);
  const int g = bg % a.n_kv_heads;
  // q / out / lse element offset of row r (= head_in_group * K + i) of the (b, g) group
  const long long q_grp = b * a.q_bs + (long long)g * a.group * a.q_hs;
  const long long o_grp = b * a.o_bs + (long long)g * a.group * a.o_hs;
  const long long l_grp = b * a.l_bs + (long long)g * a.group * a.l_hs;

  // ---- this lane's query row (the N index of every MFMA it joins)
  const int wrow = qb * 32 + (lane & 31);         // row inside the work-group block
  const int qrow = rg * plan.rows_per_wg + wrow;  // row inside the (b, g) group
  const int qrow_i = qrow % K;                    // its block position (row = head_in_group*K + i)

  // ---- tile copies: thread tid moves 16-byte chunks n = tid + c*kThreads of
  // the K tile and of the V tile (row n / DCH, chunk n % DCH, so consecutive
  // lanes read consecutive 16 bytes of the head-major cache) with
  // nontemporal loads into registers, two tiles ahead, and later writes them
  // into the LDS ring at the row's permuted chunk position.  Rows past the
  // valid count re-read the last valid row (finite data; their scores are
  // masked to -inf, so P = 0 exactly).  Tiles past the end re-read the first
  // block-key row (no HBM traffic to speak of) into a stage nobody reads.
  int crow[CPT];
  uint32_t cchunk[CPT], dk[CPT], dv[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int n = tid + c * kThreads;
    crow[c] = n / DCH;
    cchunk[c] = (uint32_t)(n % DCH) * 16;
    dk[c] = (uint32_t)(crow[c] * ROWB + swz_k<DCH>(crow[c], n % DCH) * 16);
    dv[c] = (uint32_t)(TILEB + crow[c] * ROWB + swz_v<DCH>(crow[c], n % DCH) * 16);
  }
  // tiles [0, nfull) are whole cache tiles: no masking, no row clamping
  const int nfull = min((sr.kend - sr.kstart) / kTileKeys, sr.ncache);
  const long long split_off = b * a.c_bs + g * a.c_gs + (long long)sr.kstart * D;
  const uint8_t* kc0 = reinterpret_cast<const uint8_t*>(a.k_cache + split_off);  // tile 0 of this split
  const uint8_t* vc0 = reinterpret_cast<const uint8_t*>(a.v_cache + split_off);
  const long long blk_off = b * a.blk_bs + g * a.blk_gs;
  const uint8_t* kblk = reinterpret_cast<const uint8_t*>(a.k_blk + blk_off);
  const uint8_t* vblk = reinterpret_cast<const uint8_t*>(a.v_blk + blk_off);
  typedef u32x4 Stage[2 * CPT];  // K chunks, then V chunks
  auto load_tile = [&](int t, Stage& r) __attribute__((always_inline)) {
    const bool whole = t < nfull;
    const bool real = t < sr.ntiles;
    const bool blk = sr.has_block && t >= sr.ncache;  // block tile t - ncache
    const int bt = t - sr.ncache;
    const int last = whole ? kTileKeys - 1
                           : (!real ? 0 : (blk ? min(kTileKeys, K - bt * kTileKeys)
                                               : min(kTileKeys, sr.kend - (sr.kstart + t * kTileKeys))) - 1);
    const size_t toff = (size_t)t * TILEB;
    const size_t boff = blk && real ? (size_t)bt * TILEB : 0;
    const uint8_t* kp = (whole || (real && !blk)) ? kc0 + toff : kblk + boff;
    const uint8_t* vp = (whole || (real && !blk)) ? vc0 + toff : (real ? vblk + boff : kblk);
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
      *reinterpret_cast<u32x4*>(sb + dk[c]) = r[c];
      *reinterpret_cast<u32x4*>(sb + dv[c]) = r[CPT + c];
    }
  };

  // ---- running softmax state of this lane's row.  `mref` is a reference
  // maximum in base-2 units (score * scale * log2 e): P = 2^(s*c2 - mref).  It
  // is only raised when a score exceeds it by more than 2^kLazy, so P <= 2^8
  // (exact in bf16 and fp32) and the accumulator rescale runs on a handful of
  // tiles only; normalisation by the sum makes the reference cancel exactly.
  float mref = kNegInf, neg_mref = 0.0f;
  float l_run = 0.0f;  // this lane's half of the keys of each 8-key group
  f32x16 oacc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[mb][r] = 0.0f;
  const float c2 = a.scale_log2;
  const int grp16 = lane >> 4;
  const int jj = (lane & 15) >> 2;
  const int qq = lane & 3;
  const int krow = lane & 31;  // key inside a 32-key half

  // Keys of tile t: nvalid(t) of them are real; the block tile is the last.
  auto tile_valid = [&](int t) __attribute__((always_inline)) {
    return (sr.has_block && t >= sr.ncache) ? min(kTileKeys, K - (t - sr.ncache) * kTileKeys)
                                            : min(kTileKeys, sr.kend - (sr.kstart + t * kTileKeys));
  };

  // K fragments of both 32-key halves of the tile in `stage`.  Logical chunk
  // 2*ds + half of row krow sits at byte 16 * (chunk ^ f(krow)) of the row,
  // i.e. at (32*ds) ^ kswz with kswz = 16 * (half ^ f(krow)) < ROWB; f is the
  // same for row krow + 32, so the second half is a constant offset away.
  const uint32_t kswz = 16u * (uint32_t)swz_k<DCH>(krow, half);
  auto load_k = [&](int stage, bf16x8 (&kf)[2][NDS]) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(stage * STAGEB + krow * ROWB) + kswz;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const uint8_t* p = smem + (base ^ (32u * ds));
      kf[0][ds] = *reinterpret_cast<const bf16x8*>(p);
      kf[1][ds] = *reinterpret_cast<const bf16x8*>(p + HALFB);
    }
  };
  // V^T fragments of the tile in `stage`, in the key order of the S^T
  // accumulator registers: key half h, MFMA k-step tt of 16 keys, head_dim
  // block mb.  The lane reads keys 32h + 16tt + 4*half + jj and that + 8; all
  // are congruent mod 4 and the V swizzle depends on the row mod 4 only, so
  // one base per head_dim block plus constant offsets address them all.
  uint32_t vbase[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int key0 = 4 * half + jj;
    const int d0 = 32 * mb + 16 * (grp16 & 1) + 4 * qq;
    vbase[mb] = (uint32_t)(TILEB + key0 * ROWB + swz_v<DCH>(key0, d0 >> 3) * 16 + (d0 & 7) * 2);
  }
  typedef bf16x8 VFrag[2][2][NMB];
  auto load_v = [&](int stage, VFrag& vf) __attribute__((always_inline)) {
    // per-tile bases, opaque to the optimiser so that the constant offsets
    // below fold into the LDS instructions
    uint32_t vb[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      vb[mb] = (uint32_t)(stage * STAGEB) + vbase[mb];
      asm("" : "+v"(vb[mb]));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          const uint8_t* pa = smem + vb[mb] + h * HALFB + (16 * tt) * ROWB;
          const uint8_t* pbp = pa + 8 * ROWB;
          // whole-vector bit casts: element-wise inserts of the i16 lanes into
          // the bf16 operand were lowered incorrectly by the compiler
          const bf16x4 va = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa)));
          const bf16x4 vb2 = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pbp)));
          vf[h][tt][mb] = __builtin_shufflevector(va, vb2, 0, 1, 2, 3, 4, 5, 6, 7);
        }
  };
  // Padded keys and, in the verify view, block keys after the row: -inf.
  // Explicit masks: the visible block keys of this lane's row, shifted so
  // that register r of half h tests bit 32h + 8*(r/4) + r%4 of the word.

  auto mask_scores = [&](f32x16 (&s)[2], int nvalid, bool block_tile, int key0) __attribute__((always_inline)) {
    int lim = nvalid;
    if (block_tile && a.causal) lim = min(lim, qrow_i + 1 - key0);
    // register r of half h holds key 32h + 8*(r/4) + 4*half + r%4; compare the
    // constant part against an opaque per-lane bound
    int rel = lim - 4 * half;
    asm volatile("" : "+v"(rel));
    if (EXPL && block_tile) {
      // the row's mask word is read here, once, rather than kept live through the loop
      const int mrow = min(rg * plan.rows_per_wg + wrow, R - 1) % K;
      const uint64_t m = a.blk_mask[(size_t)b * K + mrow] >> (4 * half);
      const uint32_t emask_lo = (uint32_t)m, emask_hi = (uint32_t)(m >> 32);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 32 * h + 8 * (r >> 2) + (r & 3);
          const uint32_t bit = (h ? emask_hi : emask_lo) & (1u << (kk & 31));
          s[h][r] = (kk < rel && bit) ? s[h][r] : kNegInf;
        }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[h][r] = (32 * h + 8 * (r >> 2) + (r & 3)) < rel ? s[h][r] : kNegInf;
    }
  };
  bf16x8 qf[NDS];
  // O^T += V^T P^T over the 64 keys of a tile (k-step 2h + tt).
  auto pv = [&](const bf16x8 (&pb)[4], const VFrag& vf) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) oacc[mb] = mfma32(vf[ks >> 1][ks & 1][mb], pb[ks], oacc[mb]);
  };
  // Scores -> base-2 exponents relative to the reference, x = s*c2 - mref,
  // in place; then the reference is raised (rare) if some x exceeds 2^kLazy
  // or the row has none yet.  The raise first adds the previous tile's P V,
  // still pending (it belongs to the old reference), then shifts x and
  // rescales the accumulator and the running sum.  The maximum is taken over
  // the x values (finite or -inf, never NaN) and across the lane pair that
  // shares a row with one permlane32 swap.
  auto update_ref = [&](f32x16 (&s)[2], bf16x8 (&pprev)[4], const VFrag& vprev) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[h][r] = fmaf(s[h][r], c2, neg_mref);
    float mx = fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[1][0], s[1][1]));
#pragma unroll
    for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(fmaxf(s[0][r], s[0][r + 1]), fmaxf(s[1][r], s[1][r + 1])));
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    if (__ballot(mx > kLazy || mref == kNegInf)) {
      pv(pprev, vprev);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) pprev[ks] = bf16x8{};
      // raise by mx where that helps (mx is relative to the current frame)
      const bool raise = mx != kNegInf && (mx > kLazy || mref == kNegInf);
      const float shift = raise ? mx : 0.0f;
      const float alpha = (mref == kNegInf || !raise) ? (mref == kNegInf ? 0.0f : 1.0f) : fast_exp2(-mx);
      mref = raise ? (mref == kNegInf ? mx : mref + mx) : mref;
      neg_mref = (mref == kNegInf) ? 0.0f : -mref;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[h][r] -= shift;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) oacc[mb] *= alpha;
    }
  };
  // exp2 of one score in the base-2 frame of the reference
  auto expo = [&](float x) __attribute__((always_inline)) { return fast_exp2(x); };
  auto next_stage = [](int s) __attribute__((always_inline)) { return s == kStages - 1 ? 0 : s + 1; };
  auto prev_stage = [](int s) __attribute__((always_inline)) { return s == 0 ? kStages - 1 : s - 1; };

  // ---- software pipeline.  LDS holds four tiles: t-1 (its V for the pending
  // P(t-1) V(t-1)), t (V next), t+1 (K for S(t+1)) and t+2 (being written);
  // registers hold the next two.  Iteration t issues three independent pieces
  // of work on one wave: the S(t+1) MFMAs, the P(t-1) V(t-1) MFMAs and the
  // exponentials of S(t), so the matrix core and the vector ALU overlap.  One
  // barrier per tile: after it every wave is past iteration t-1, so the
  // stage of tile t-2 can take tile t+2, and tile t+1 (written in iteration
  // t-1) is visible.  Waves whose query block lies past the work-group's rows
  // run the same code on zero queries and write nothing.
  Stage stg0, stg1;  // at iteration t: tiles t+2 and t+3 (in flight or landed)
  {
    const int row = min(rg * plan.rows_per_wg + wrow, R - 1);
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(a.q + q_grp + (row / K) * a.q_hs + (long long)(row % K) * D);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qf[ds] = active ? qp[2 * ds + half] : bf16x8{};
  }
  {
    Stage t0, t1;
    load_tile(0, t0);
    load_tile(1, t1);
    store_tile(0, t0);
    load_tile(2, stg0);
    store_tile(1, t1);
    load_tile(3, stg1);
  }
  __syncthreads();
  f32x16 sa[2], sb[2];
  bf16x8 pprev[4];  // P(t-1) in bf16, the pending product's left operand
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) pprev[ks] = bf16x8{};
  auto s_mfma = [&](const bf16x8 (&kf)[2][NDS], f32x16 (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[h][r] = 0.0f;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) s[h] = mfma32(kf[h][ds], qf[ds], s[h]);
    }
  };
  if (sr.ntiles > 0) {
    bf16x8 kf[2][NDS];
    load_k(0, kf);
    s_mfma(kf, sa);
  }
  const int nmain = nfull > 0 ? nfull - 1 : 0;  // iterations whose next tile is whole too

  // One iteration: cur = S(t) -> P(t); pending P(t-1) V(t-1) is added;
  // nxt = S(t+1) if there is a next tile.  Tile t sits in stage st, the
  // pending V in stage vst; `refill` holds tile t+2 and takes tile t+4.
  auto iteration = [&](int t, int st, int vst, f32x16 (&cur)[2], f32x16 (&nxt)[2], Stage& refill, bool masked,
                       bool has_next) __attribute__((always_inline)) {
    const int st1 = next_stage(st);   // tile t+1
    const int st2 = next_stage(st1);  // tile t+2 (the stage tile t-2 used)
    VFrag vf;
    load_v(vst, vf);
    if (masked) {
      const bool blk = sr.has_block && t >= sr.ncache;
      if (blk || tile_valid(t) < kTileKeys) mask_scores(cur, tile_valid(t), blk, (t - sr.ncache) * kTileKeys);
    }
    update_ref(cur, pprev, vf);
    float lsum = 0.0f;
    bf16x8 pnew[4];
    if (has_next) {
      __syncthreads();
      store_tile(st2, refill);
      load_tile(t + 4, refill);
      bf16x8 kf[2][NDS];
      load_k(st1, kf);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) nxt[h][r] = 0.0f;
      // per S step: two S MFMAs, four exponentials, two pending PV MFMAs
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        nxt[0] = mfma32(kf[0][ds], qf[ds], nxt[0]);
#pragma unroll
        for (int e = 0; e < 32 / NDS; ++e) {
          const int i = ds * (32 / NDS) + e;  // score i of the 32 this lane holds
          const float p_ = expo(cur[i >> 4][i & 15]);
          cur[i >> 4][i & 15] = p_;
          lsum += p_;
        }
        nxt[1] = mfma32(kf[1][ds], qf[ds], nxt[1]);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int j = 2 * ds + u;  // pending PV MFMA j of 4 * NMB
          const int ks = j / NMB, mb = j % NMB;
          oacc[mb] = mfma32(vf[ks >> 1][ks & 1][mb], pprev[ks], oacc[mb]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float p_ = expo(cur[i >> 4][i & 15]);
        cur[i >> 4][i & 15] = p_;
        lsum += p_;
      }
      pv(pprev, vf);
    }
    l_run += lsum;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) pnew[ks][e] = (__bf16)cur[ks >> 1][8 * (ks & 1) + e];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pprev[ks] = pnew[ks];
  };
  int t = 0, st = 0;
  for (; t + 2 <= nmain; t += 2) {  // unrolled by two: scores and staging registers alternate
    iteration(t, st, t == 0 ? st : prev_stage(st), sa, sb, stg0, false, true);
    st = next_stage(st);
    iteration(t + 1, st, prev_stage(st), sb, sa, stg1, false, true);
    st = next_stage(st);
  }
  // ---- the remaining tiles (the last whole tile, a partial tile, the block
  // tile; all of them if there are fewer than two whole tiles)
  for (; t < sr.ntiles; ++t) {
    const bool has_next = t + 1 < sr.ntiles;
    iteration(t, st, t == 0 ? st : prev_stage(st), sa, sb, stg0, true, has_next);
    if (has_next) {
#pragma unroll
      for (int h = 0; h < 2; ++h) sa[h] = sb[h];
#pragma unroll
      for (int c = 0; c < 2 * CPT; ++c) {  // keep "stg0 holds tile t+2"
        const u32x4 x = stg0[c];
        stg0[c] = stg1[c];
        stg1[c] = x;
      }
    }
    st = has_next ? next_stage(st) : st;
  }
  if (sr.ntiles > 0) {  // the last tile's P V
    VFrag vf;
    load_v(st, vf);
    pv(pprev, vf);
  }

  // ---- per-row totals: this lane holds half of the keys of every 8-key group
  const float l_row = l_run + __shfl_xor(l_run, 32);
  const float m_out = mref;  // base-2 reference of acc and l

  // ---- normalised rows in bf16 -> LDS (row pitch ROWB + 16 spreads the 32
  // rows a store instruction touches over the banks) -> coalesced 16-byte
  // global stores of whole rows.  The ring is free once every wave is past
  // its last P V.
  constexpr int OPITCH = ROWB + 16;
  static_assert(128 * OPITCH <= kStages * STAGEB, "output rows fit the ring");
  __syncthreads();
  if (active) {
    const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
    uint8_t* orow = smem + wrow * OPITCH;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        ushort4 o;
        o.x = to_bf16_bits(oacc[mb][4 * q4 + 0] * inv);
        o.y = to_bf16_bits(oacc[mb][4 * q4 + 1] * inv);
        o.z = to_bf16_bits(oacc[mb][4 * q4 + 2] * inv);
        o.w = to_bf16_bits(oacc[mb][4 * q4 + 3] * inv);
        *reinterpret_cast<ushort4*>(orow + 2 * (32 * mb + 8 * q4 + 4 * half)) = o;
      }
  }
  __syncthreads();
  const int nrows = plan.rows_per_wg;  // the rows of the active query blocks
  const bool one_split = a.splits == 1 && direct;
  // destination of row r: the output (one split) or this split's partial slot
  const size_t slot = (size_t)grp * a.splits + split;
  for (int n = tid; n < nrows * DCH; n += kThreads) {
    const int r = n / DCH, ch = n % DCH;
    const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * OPITCH + ch * 16);
    if (one_split) {
      const int gr = rg * plan.rows_per_wg + r;  // row inside the (b, g) group
      if (gr < R)
        *reinterpret_cast<u32x4*>(a.out + o_grp + (gr / K) * a.o_hs + (long long)(gr % K) * D + ch * 8) = v;
    } else {
      *reinterpret_cast<u32x4*>(a.ws_acc + (slot * plan.rows_per_wg + r) * D + ch * 8) = v;
    }
  }
  if (active && half == 0) {
    if (one_split) {
      if (a.lse != nullptr && qrow < R) a.lse[l_grp + (qrow / K) * a.l_hs + qrow % K] = (m_out + log2f(l_row)) * kLn2;
    } else {
      float2 ml;
      ml.x = m_out;
      ml.y = l_row;
      *reinterpret_cast<float2*>(a.ws_ml + (slot * plan.rows_per_wg + wrow) * 2) = ml;
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
  if (a.blk_mask != nullptr)
    hipLaunchKernelGGL((attn_stream_kernel<D, NQB, true>), grid, dim3(kThreads), 0, stream, a, p, direct);
  else
    hipLaunchKernelGGL((attn_stream_kernel<D, NQB, false>), grid, dim3(kThreads), 0, stream, a, p, direct);
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
