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
// waves (512 threads, two waves per SIMD) per CU.  A work-group owns one
// contiguous chunk of the (b, g) cache rows and up to 128 query rows (4
// blocks of 32), or 256 (8 blocks, one per wave over whole tiles) when a KV
// head has more than 128; split 0 also takes the K block keys as one extra masked
// tile, before its cache tiles, so that the block is computed while the first
// cache tile is on its way from HBM.  Work-groups are numbered so that the
// (b, g) groups interleave and the block-carrying splits are dispatched
// first: the dispatcher starts the work-groups over a couple of
// microseconds, and the heaviest ones should not start last.
//  * Streaming: the chunk is read in tiles of 64 keys (16 KiB of K and 16 KiB
//    of V at D = 128).  Every thread issues coalesced 16-byte nontemporal
//    loads of the next tile into registers (32 KiB in flight per CU: more
//    than that measured slower on MI355X), then writes them into a 2-stage
//    LDS ring at the row's permuted chunk position; one barrier per tile
//    orders writes and reads.  The 16-byte chunks of every K and V row are
//    XOR-permuted per row so that both read patterns below hit distinct LDS
//    banks.
//  * Compute: wave w takes query block w >> 1 against key half w & 1 (32
//    keys) of every tile, so each SIMD runs two waves whose matrix and vector
//    work interleave (one wave per SIMD issues MFMAs at half the SIMD's
//    rate).  S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (32 keys x 32 query
//    rows; Q held in registers), so each lane owns one query row and its
//    softmax statistics need one exchange with lane^32 (a permlane32 swap).
//    O^T += V^T P^T on the same MFMA: P^T is the S^T accumulator converted to
//    bf16 in place; V^T comes from the row-major V tile through
//    ds_read_b64_tr_b16, the transposing LDS read, with the key order matched
//    to the accumulator's register order.
//  * Softmax: P = 2^(s*scale*log2(e) - m_ref) with a lazily raised reference
//    m_ref (raised only when a shifted score exceeds it by more than 8, so
//    P <= 2^8), so the accumulator rescale is rare; the sum cancels the
//    reference exactly.
//    Each key half keeps its own reference, sum and accumulator; at the end
//    the two waves of a query block combine theirs through LDS, each
//    finishing half of head_dim.
//  * Epilogue: with one split the work-group normalises and writes the rows
//    itself.  Otherwise it stores a partial per row -- fp32 (m_ref, sum) and
//    the bf16 value sum normalised by that sum, staged through LDS and written
//    as whole coalesced rows with nontemporal stores -- and a second kernel
//    merges the S partials:
//    out = sum_s 2^(m_s-M) l_s o_s / sum_s 2^(m_s-M) l_s,
//    lse = (M + log2 sum_s 2^(m_s-M) l_s) * ln 2, with one wave per row and
//    each XCD merging the rows whose partials its own streaming work-groups
//    wrote.
#include "attn_frag.h"
#include "common.h"
#include "block_order.h"

#include <math.h>

namespace orthrus {
namespace {

using namespace frag;

constexpr float kLazy = 8.0f;  // base-2 headroom before the softmax reference is raised
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994531f;

// Cache range of one split of sequence b: [kstart, kend).
struct SplitRange {
  // tiles 0 .. nblk-1: block-key tiles blk0 .. blk0+nblk-1; then ncache cache tiles
  int kstart, kend, ncache, nblk, ntiles, blk0;
};

__device__ __forceinline__ int seq_len(const AttnArgs& a, int b) {
  const int L = a.len_step > 0 ? b * a.len_step : a.cache_len[b];
  return L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
}

// Live block length of sequence b (dynamic block size): its first k_b block
// positions are the block; block_k when no per-sequence length is given.
__device__ __forceinline__ int live_k(const AttnArgs& a, int b) {
  if (a.blk_len == nullptr) return a.block_k;
  const int k = a.blk_len[b];
  return k < 1 ? 1 : (k > a.block_k ? a.block_k : k);
}

// Row groups of sequence b that hold a live row: ceil(G k_b / rows_per_wg).
__device__ __forceinline__ int live_row_groups(const AttnArgs& a, const AttnPlan& p, int b) {
  const int R = a.group * live_k(a, b);
  return min(p.row_groups, (R + p.rows_per_wg - 1) / p.rows_per_wg);
}

// A block length that leaves row groups without a live row: the n = RG * S
// work-groups of a (sequence, KV head) are dealt round robin over its lrg live
// row groups -- work-group j takes split j / lrg of live row group j % lrg, its
// partial in slot j of the head's n -- so the whole launch keeps streaming.
// Live row group rg then has this many splits (at most kMaxSplits; work-groups
// past that stay idle).
__device__ __forceinline__ int dealt_splits(int n, int lrg, int rg) {
  return min((n - 1 - rg) / lrg + 1, kMaxSplits);
}

__device__ __forceinline__ SplitRange split_range(const AttnArgs& a, int b, int split, int S) {
  SplitRange r;
  const int L = seq_len(a, b);
  // as even as the key count allows: a length that is not a multiple of S
  // tiles leaves every split a short last tile rather than some splits a whole
  // extra one (splits need not start on a tile boundary)
  const int chunk = (L + S - 1) / S;
  r.kstart = split * chunk;
  r.kend = min(r.kstart + chunk, L);
  r.ncache = r.kstart < r.kend ? (r.kend - r.kstart + kTileKeys - 1) / kTileKeys : 0;
  // split 0 streams the (live) block keys first: their tile is computed while
  // the first cache tile is still on its way from HBM
  r.nblk = split == 0 ? (live_k(a, b) + kTileKeys - 1) / kTileKeys : 0;
  r.ntiles = r.nblk + r.ncache;
  r.blk0 = 0;
  return r;
}

// ---- balanced placement for batches of several sequences
//
// With several sequences of different lengths the launch's N work-groups
// share one list of work: for every sequence b and every one of its
// H = Hkv * row_groups groups h (b-major), a segment of kPieceCost cost units
// followed by S_b tiles -- the nblk = ceil(K / 64) block-key tiles, then the
// ceil(L_b / 64) cache tiles.  With W units in all and n = min(N, W),
// work-group w < n takes units [w W / n, (w+1) W / n): every work-group gets
// the same amount of work (to within one unit), whatever the lengths.  A
// work-group's range can cross segments; it computes one partial per segment
// whose tiles it touches, in slot w + seg (seg = b H + h): the pieces of one
// segment come from consecutive work-groups, so their slots are consecutive,
// and no two pieces share a slot (slots stay below N + B H).  The work-group
// holding a segment's first tile records the first slot, the one holding its
// last tile the last slot, for the merge.  The lengths are read on the device
// (no host sync).

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
// Tiles of one segment of sequence b: (live) block-key tiles, then cache tiles.
__device__ __forceinline__ int seg_tiles(const AttnArgs& a, int b) {
  return (live_k(a, b) + kTileKeys - 1) / kTileKeys + (seq_len(a, b) + kTileKeys - 1) / kTileKeys;
}
// The fixed cost of one piece (its q and first tiles' latency, the closing
// combine and partial write: about 7.7 us against 1.2 us per tile, fitted
// over the work-groups of a 16-sequence launch), counted as this many tiles
// of work at the head of every segment when the list is divided, so that
// work-groups whose ranges cross many short segments get fewer tiles.
constexpr int kPieceCost = 6;

// Up to kRaggedMaxSeqs sequences: lane l of a wave holds the segment tile
// counts of sequences l, l + 64, ... in registers, read once.
constexpr int kRaggedSlots = kRaggedMaxSeqs / 64;

struct RaggedTiles {
  // units per KV head of sequence lane + 64*k (0 past the batch): its row
  // groups with a live row (all of them unless the block is short), each a
  // segment of kPieceCost + tiles units
  int su[kRaggedSlots];
};

__device__ __forceinline__ RaggedTiles ragged_tiles(const AttnArgs& a, const AttnPlan& p) {
  const int lane = threadIdx.x & 63;
  RaggedTiles r;
#pragma unroll
  for (int k = 0; k < kRaggedSlots; ++k) {
    const int b = lane + 64 * k;
    r.su[k] = b < a.batch ? live_row_groups(a, p, b) * (kPieceCost + seg_tiles(a, b)) : 0;
  }
  return r;
}

// Units of the whole list: every sequence's live segments, for every KV head.
__device__ __forceinline__ long long ragged_total(const AttnArgs& a, const RaggedTiles& rt) {
  int t = 0;
#pragma unroll
  for (int k = 0; k < kRaggedSlots; ++k) t += rt.su[k];
  return (long long)wave_sum(t) * a.n_kv_heads;
}

struct SeqAt {
  int b;           // the sequence
  long long base;  // index of its first unit (segment h = 0) in the list
};

// The sequence whose segments hold list unit T < W (a whole wave calls it).
__device__ SeqAt seq_at(const AttnArgs& a, const RaggedTiles& rt, long long T) {
  const int lane = threadIdx.x & 63;
  long long base = 0;
#pragma unroll
  for (int k = 0; k < kRaggedSlots; ++k) {
    const int bb = 64 * k + lane;
    const long long sz = (long long)rt.su[k] * a.n_kv_heads;  // this lane's sequence: its live segments
    long long incl = sz;                          // inclusive scan over the lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const long long excl = incl - sz;
    const unsigned long long m = __ballot(bb < a.batch && T >= base + excl && T < base + incl);
    if (m) {
      const int src = __builtin_ctzll(m);
      return {64 * k + src, base + __shfl(excl, src)};
    }
    base += __shfl(incl, 63);
  }
  return {-1, base};
}

// Key range of tiles [p0, p1) of a segment of sequence b.
__device__ __forceinline__ SplitRange piece_range(const AttnArgs& a, int b, int p0, int p1) {
  SplitRange r;
  const int L = seq_len(a, b);
  const int nb = (live_k(a, b) + kTileKeys - 1) / kTileKeys;  // as in seg_tiles
  r.blk0 = min(p0, nb);
  r.nblk = min(p1, nb) - r.blk0;
  const int c0 = max(p0, nb) - nb, c1 = max(p1, nb) - nb;  // cache tiles [c0, c1)
  r.kstart = c0 * kTileKeys;
  r.kend = min(c1 * kTileKeys, L);
  r.ncache = c1 - c0;
  r.ntiles = r.nblk + r.ncache;
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
// Reductions over the LPR lanes of a merge row, in registers (no LDS): the
// partners at each level are lane ^ 1 and lane ^ 2 (quad permutes), the
// mirrored quad of the 8-lane half and the mirrored half of the 16-lane row
// (DPP), lane ^ 16 and, for 64-lane rows, lane ^ 32 (permlane swaps).  Both
// lanes of a pair combine the same two values, so every lane of the row ends
// with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_partner_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float partner16_f(float x) {  // lane ^ 16
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(((threadIdx.x >> 4) & 1) ? sw[0] : sw[1]);
}
__device__ __forceinline__ float partner32_f(float x) {  // lane ^ 32
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(((threadIdx.x >> 5) & 1) ? sw[0] : sw[1]);
}
template <int LPR, typename Op>
__device__ __forceinline__ float row_reduce(float v, Op op) {
  v = op(v, dpp_partner_f<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = op(v, dpp_partner_f<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = op(v, dpp_partner_f<0x141>(v));  // row_half_mirror
  v = op(v, dpp_partner_f<0x140>(v));  // row_mirror
  v = op(v, partner16_f(v));
  if constexpr (LPR == 64) v = op(v, partner32_f(v));
  return v;
}

// The merge itself (described above the lane reductions).
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
  // partial s of the group sits in slot slot0 + s * stride
  int S = a.splits, stride = 1;
  size_t slot0 = (size_t)grp * S;
  if (a.blk_len != nullptr && p.row_groups > 1) {
    const int bg = grp / p.row_groups, rg = grp % p.row_groups;
    const int lrg = __builtin_amdgcn_readfirstlane(live_row_groups(a, p, bg / a.n_kv_heads));
    if (lrg < p.row_groups) {  // the streaming launch dealt the head's work-groups over lrg row groups
      if (rg >= lrg) return;   // a row group with no live row: nothing to merge
      const int n = p.row_groups * a.splits;
      S = dealt_splits(n, lrg, rg);
      stride = lrg;
      slot0 = (size_t)bg * n + rg;
    }
  }
  uint32_t v[SMAX];
#pragma unroll
  for (int s = 0; s < SMAX; ++s) {
    const size_t idx = (slot0 + (size_t)min(s, S - 1) * stride) * p.rows_per_wg + rrow;
    v[s] = *reinterpret_cast<const uint32_t*>(a.ws_acc + idx * D + 2 * j);
  }
  float m[NW], l[NW];
#pragma unroll
  for (int c = 0; c < NW; ++c) {
    const int sp = min(c * LPR + j, S - 1);
    const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + ((slot0 + (size_t)sp * stride) * p.rows_per_wg + rrow) * 2);
    const bool real = c * LPR + j < S;
    m[c] = real ? ml.x : kNegInf;
    l[c] = real ? ml.y : 0.0f;
  }
  // M over the row's lanes
  float M = m[0];
#pragma unroll
  for (int c = 1; c < NW; ++c) M = fmaxf(M, m[c]);
  M = row_reduce<LPR>(M, [](float a, float b) { return fmaxf(a, b); });
  float wt[NW];
  float L = 0.0f;
#pragma unroll
  for (int c = 0; c < NW; ++c) {
    wt[c] = (m[c] == kNegInf) ? 0.0f : fast_exp2(m[c] - M) * l[c];
    L += wt[c];
  }
  L = row_reduce<LPR>(L, [](float a, float b) { return a + b; });
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
  // rows past the live block length (a block shorter than block_k) were read
  // but are not written
  const int bg = grp / p.row_groups, rg = grp % p.row_groups;
  const int kb = __builtin_amdgcn_readfirstlane(live_k(a, bg / a.n_kv_heads));  // one group per wave
  const int r = rg * p.rows_per_wg + myrow;  // row inside the (b, g) group: head_in_group*kb + i
  if (myrow < row_end && r < a.group * kb) {
    {
      const int b = bg / a.n_kv_heads, h = (bg % a.n_kv_heads) * a.group + r / kb, i = r % kb;
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      const uint32_t o = (uint32_t)to_bf16_bits(acc0 * inv) | ((uint32_t)to_bf16_bits(acc1 * inv) << 16);
      *reinterpret_cast<uint32_t*>(a.out + b * a.o_bs + h * a.o_hs + (long long)i * D + 2 * j) = o;
      if (a.lse != nullptr && j == 0) a.lse[b * a.l_bs + h * a.l_hs + i] = (M + log2f(L)) * kLn2;
    }
  }
}

// The streaming kernel (see the top of the file).  Per wave and tile at D 128:
// 8 S^T MFMAs, 16 exponentials per lane, 8 O^T MFMAs.
constexpr int kStreamThreads = kAttnThreads;

template <int D, int NQB, bool EXPL, bool RAGGED>
__global__ __launch_bounds__(kStreamThreads) void attn_stream_kernel(AttnArgs a, AttnPlan plan, int direct) {
  constexpr int DCH = D / 8;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = kTileKeys * ROWB;
  constexpr int STAGEB = 2 * TILEB;
  constexpr int HALFB = 32 * ROWB;
  constexpr int NDS = D / 16;
  constexpr int NMB = D / 32;
  constexpr int HMB = NMB / 2;  // head_dim blocks each wave of a pair finishes
  constexpr int CPT = kTileKeys * DCH / kStreamThreads;
  constexpr int RINGB = 2 * STAGEB;
  constexpr int XCHB = 8 * HMB * 16 * 64 * 4;  // accumulator blocks handed to the partner wave
  constexpr int REGION0 = RINGB > XCHB ? RINGB : XCHB;
  constexpr int OPITCH = ROWB + 16;
  static_assert(CPT >= 1 && HMB >= 1, "tile and head_dim fit the work-group");

  // NQB 8 (256 rows): every wave takes its own query block over the whole
  // tile, both key halves one after the other, so no two waves share a row
  // and the key halves need no combine at the end
  constexpr bool WT = NQB == 8;
  constexpr int STG_ROWS = NQB > 4 ? 32 * NQB : 128;
  __shared__ __attribute__((aligned(16))) uint8_t smem[REGION0 + STG_ROWS * OPITCH];
  __shared__ float2 xstat[8][32];

  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  // One piece of work: the key range `sr` of group (bg, rg), its partial
  // written to `slot` (or, with a single split, the output itself).
  auto piece = [&](const int bg, const int rg, const SplitRange sr, const size_t slot) __attribute__((always_inline)) {
  const int b = bg / a.n_kv_heads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qb = WT ? w : w >> 1;  // query block
  const int kh = WT ? 0 : w & 1;   // key half of every tile (both halves with WT)
  const int half = lane >> 5;
  // block_k rows per q head in memory; kb of them live (the rows are packed
  // h * kb + i), R live rows per (sequence, KV head)
  const int K = a.block_k;
  const int kb = __builtin_amdgcn_readfirstlane(live_k(a, b));  // b is the work-group's sequence
  const int R = a.group * kb;
  if (rg * plan.rows_per_wg >= R) return;  // no live row in this row group
  const bool active = qb < NQB && rg * plan.rows_per_wg + qb * 32 < R;
  const int g = bg % a.n_kv_heads;
  const long long q_grp = b * a.q_bs + (long long)g * a.group * a.q_hs;
  const long long o_grp = b * a.o_bs + (long long)g * a.group * a.o_hs;
  const long long l_grp = b * a.l_bs + (long long)g * a.group * a.l_hs;
  const int wrow = qb * 32 + (lane & 31);
  const int qrow = rg * plan.rows_per_wg + wrow;
  const int qrow_i = qrow % kb;

  // ---- tile copies: thread tid moves 16-byte chunks n = tid + c*512 of the K
  // tile and of the V tile (row n / DCH, chunk n % DCH, so consecutive lanes
  // read consecutive 16 bytes of the head-major cache) with nontemporal loads
  // into registers, and writes them into the LDS ring at the row's permuted
  // chunk position one iteration later.  Rows past the valid count re-read the
  // last valid row (finite data; their scores are masked to -inf, so P = 0
  // exactly).  A tile past the end re-reads the first block-key row into
  // registers that are never stored.
  int crow[CPT];
  uint32_t cchunk[CPT], dk[CPT], dv[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int n = tid + c * kStreamThreads;
    crow[c] = n / DCH;
    cchunk[c] = (uint32_t)(n % DCH) * 16;
    dk[c] = (uint32_t)(crow[c] * ROWB + swz_k<DCH>(crow[c], n % DCH) * 16);
    dv[c] = (uint32_t)(TILEB + crow[c] * ROWB + swz_v<DCH>(crow[c], n % DCH) * 16);
  }
  const int nfull = min((sr.kend - sr.kstart) / kTileKeys, sr.ncache);
  const long long split_off = b * a.c_bs + g * a.c_gs + (long long)sr.kstart * D;
  const uint8_t* kc0 = reinterpret_cast<const uint8_t*>(a.k_cache + split_off);
  const uint8_t* vc0 = reinterpret_cast<const uint8_t*>(a.v_cache + split_off);
  const long long blk_off = b * a.blk_bs + g * a.blk_gs;
  const uint8_t* kblk = reinterpret_cast<const uint8_t*>(a.k_blk + blk_off);
  const uint8_t* vblk = reinterpret_cast<const uint8_t*>(a.v_blk + blk_off);
  typedef u32x4 Stage[2 * CPT];
  auto load_tile = [&](int t, Stage& r) __attribute__((always_inline)) {
    const bool real = t < sr.ntiles;
    const bool blk = real && t < sr.nblk;
    const int ct = t - sr.nblk;  // cache tile index
    const bool cache = real && !blk;
    const bool whole = cache && ct < nfull;
    const int bt = sr.blk0 + t;  // block tile index
    const int last = whole ? kTileKeys - 1
                           : (!real ? 0 : (blk ? min(kTileKeys, K - bt * kTileKeys)
                                               : min(kTileKeys, sr.kend - (sr.kstart + ct * kTileKeys))) - 1);
    const size_t toff = (size_t)ct * TILEB;
    const size_t boff = blk ? (size_t)bt * TILEB : 0;
    const uint8_t* kp = cache ? kc0 + toff : kblk + boff;
    const uint8_t* vp = cache ? vc0 + toff : (real ? vblk + boff : kblk);
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
  // valid keys of tile t (block tiles: the live block keys; <= 0 for a block
  // tile wholly past them, whose loads still stay inside the block buffer)
  auto tile_valid = [&](int t) __attribute__((always_inline)) {
    return t < sr.nblk ? min(kTileKeys, kb - (sr.blk0 + t) * kTileKeys)
                       : min(kTileKeys, sr.kend - (sr.kstart + (t - sr.nblk) * kTileKeys));
  };

  // ---- running softmax state of this lane's row over this wave's key half
  float mref = kNegInf, neg_mref = 0.0f;
  float l_run = 0.0f;
  f32x16 oacc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[mb][r] = 0.0f;
  const float c2 = a.scale_log2;
  const int grp16 = lane >> 4;
  const int jj = (lane & 15) >> 2;
  const int qq = lane & 3;
  const int krow = lane & 31;

  // K fragments of this wave's 32-key half.  Logical chunk 2*ds + half of row
  // krow sits at byte 16 * (chunk ^ f(krow)) of the row, i.e. at (32*ds) ^
  // kswz with kswz = 16 * (half ^ f(krow)) < ROWB.
  const uint32_t kbase = (uint32_t)(kh * HALFB + krow * ROWB) + 16u * (uint32_t)swz_k<DCH>(krow, half);
  auto load_k = [&](int stage, int khx, bf16x8 (&kf)[NDS]) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(stage * STAGEB + (khx - kh) * HALFB) + kbase;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) kf[ds] = *reinterpret_cast<const bf16x8*>(smem + (base ^ (32u * ds)));
  };
  // V^T fragments of the half in the key order of the S^T accumulator: k-step
  // tt of 16 keys, head_dim block mb.  The lane reads keys 32*kh + 16*tt +
  // 4*half + jj and that + 8; all are congruent mod 4 and the V swizzle
  // depends on the row mod 4 only, so one base per head_dim block plus
  // constant offsets address them all.  The per-tile bases are opaque to the
  // optimiser so that those offsets fold into the LDS instructions, and the
  // fragments are assembled with whole-vector bit casts (element-wise inserts
  // of the i16 lanes into the bf16 operand were lowered incorrectly).
  uint32_t vbase[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int key0 = 4 * half + jj;
    const int d0 = 32 * mb + 16 * (grp16 & 1) + 4 * qq;
    vbase[mb] = (uint32_t)(TILEB + kh * HALFB + key0 * ROWB + swz_v<DCH>(key0, d0 >> 3) * 16 + (d0 & 7) * 2);
  }
  auto load_v = [&](int stage, int khx, bf16x8 (&vf)[2][NMB]) __attribute__((always_inline)) {
    uint32_t vb[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      vb[mb] = (uint32_t)(stage * STAGEB + (khx - kh) * HALFB) + vbase[mb];
      asm("" : "+v"(vb[mb]));
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const uint8_t* pa = smem + vb[mb] + (16 * tt) * ROWB;
        const uint8_t* pbp = pa + 8 * ROWB;
        const bf16x4 va = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa)));
        const bf16x4 vb2 = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pbp)));
        vf[tt][mb] = __builtin_shufflevector(va, vb2, 0, 1, 2, 3, 4, 5, 6, 7);
      }
  };
  // register r holds key 32*kh + 8*(r/4) + 4*half + r%4 of the tile
  auto mask_scores = [&](f32x16& s, int khx, int nvalid, bool block_tile, int key0) __attribute__((always_inline)) {
    int lim = nvalid;
    if (block_tile && a.causal) lim = min(lim, qrow_i + 1 - key0);
    int rel = lim - 4 * half - 32 * khx;
    asm volatile("" : "+v"(rel));
    if (EXPL && block_tile) {
      const int mrow = min(qrow, R - 1) % kb;
      const uint32_t em = (uint32_t)(a.blk_mask[(size_t)b * K + mrow] >> (4 * half + 32 * khx));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 8 * (r >> 2) + (r & 3);
        s[r] = (kk < rel && (em & (1u << kk))) ? s[r] : kNegInf;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = (8 * (r >> 2) + (r & 3)) < rel ? s[r] : kNegInf;
    }
  };
  // shifted base-2 exponents and the lazy reference raise (no pending P V here)
  auto update_ref = [&](f32x16& s) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = fmaf(s[r], c2, neg_mref);
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
#pragma unroll
    for (int r = 4; r < 16; r += 4) mx = fmaxf(mx, fmaxf(fmaxf(s[r], s[r + 1]), fmaxf(s[r + 2], s[r + 3])));
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    if (__ballot(mx > kLazy || mref == kNegInf)) {
      const bool raise = mx != kNegInf && (mx > kLazy || mref == kNegInf);
      const float shift = raise ? mx : 0.0f;
      const float alpha = (mref == kNegInf || !raise) ? (mref == kNegInf ? 0.0f : 1.0f) : fast_exp2(-mx);
      mref = raise ? (mref == kNegInf ? mx : mref + mx) : mref;
      neg_mref = (mref == kNegInf) ? 0.0f : -mref;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] -= shift;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) oacc[mb] *= alpha;
    }
  };
  bf16x8 qf[NDS];
  {
    const int row = min(qrow, R - 1);
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(a.q + q_grp + (row / kb) * a.q_hs + (long long)(row % kb) * D);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qf[ds] = active ? qp[2 * ds + half] : bf16x8{};
  }
  // One tile of this wave's half (both halves in turn with WT): S^T, mask,
  // softmax, O^T += V^T P^T.
  auto compute = [&](int st, int t) __attribute__((always_inline)) {
    const int nval = tile_valid(t);
    if (!active) return;
#pragma unroll
    for (int hk = 0; hk < (WT ? 2 : 1); ++hk) {
    const int khx = WT ? hk : kh;
    if (nval <= 32 * khx) break;  // no real key in this half (or past it)
    bf16x8 kf[NDS];
    load_k(st, khx, kf);
    // all K fragment reads in flight before the first MFMA (left alone, the
    // scheduler keeps two or three and each MFMA waits on its own read)
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) s = mfma32(kf[ds], qf[ds], s);
    bf16x8 vf[2][NMB];
    load_v(st, khx, vf);
    if (t < sr.nblk || t - sr.nblk >= nfull) {
      const bool blk = t < sr.nblk;
      mask_scores(s, khx, nval, blk, (sr.blk0 + t) * kTileKeys);
    }
    update_ref(s);
    float lsum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p_ = fast_exp2(s[r]);
      s[r] = p_;
      lsum += p_;
    }
    l_run += lsum;
    bf16x8 pb[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[tt][e] = (__bf16)s[8 * tt + e];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) oacc[mb] = mfma32(vf[tt][mb], pb[tt], oacc[mb]);
    }
  };

  // ---- pipeline: at the top of iteration t, tile t sits in LDS stage t & 1
  // (written before the last barrier) and the registers hold tile t+1 (landed
  // or landing).  Each wave computes tile t, then writes tile t+1 into the
  // other stage -- every wave finished reading it before the last barrier --
  // and loads tile t+2 into the registers; the barrier then publishes tile
  // t+1.  Computing first keeps the stage writes off the path of this wave's
  // LDS reads.
  // The first two tiles are requested together: the first one's latency is
  // the longest of the launch, and the second one's hides under it.
  Stage stg, stg0;
  load_tile(0, stg0);
  load_tile(1, stg);
  store_tile(0, stg0);
  __syncthreads();
  for (int t = 0; t < sr.ntiles; ++t) {
    compute(t & 1, t);
    if (t + 1 < sr.ntiles) {
      store_tile((t + 1) & 1, stg);
      load_tile(t + 2, stg);
    }
    __syncthreads();
  }

  // ---- combine the two key halves of each query block through LDS: wave w
  // hands the head_dim blocks its partner finishes (a raw register dump,
  // lane-major) and its row statistics to the partner wave w ^ 1.
  const float l_row = l_run + __shfl_xor(l_run, 32);
  float* xch = reinterpret_cast<float*>(smem);
  // every wave is past its last tile (the loop ends on a barrier): the ring is free
  if (!WT && active) {
#pragma unroll
    for (int j = 0; j < HMB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) xch[((w * HMB + j) * 16 + r) * 64 + lane] = kh ? oacc[j][r] : oacc[HMB + j][r];
    if (half == 0) xstat[w][lane] = make_float2(mref, l_row);
  }
  __syncthreads();
  float m_out = kNegInf, l_out = 0.0f;
  if (WT && active) {  // this wave saw every key of its rows: normalise and stage them
    m_out = mref;
    l_out = l_row;
    const float inv = l_out > 0.0f ? 1.0f / l_out : 0.0f;
    uint8_t* orow = smem + REGION0 + wrow * OPITCH;
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
  } else if (active) {
    const int pw = w ^ 1;
    const float2 po = xstat[pw][lane & 31];
    m_out = fmaxf(mref, po.x);
    const float a_s = mref == kNegInf ? 0.0f : fast_exp2(mref - m_out);
    const float a_o = po.x == kNegInf ? 0.0f : fast_exp2(po.x - m_out);
    l_out = a_s * l_row + a_o * po.y;
    const float inv = l_out > 0.0f ? 1.0f / l_out : 0.0f;
    const float ws = a_s * inv, wo = a_o * inv;
    uint8_t* orow = smem + REGION0 + wrow * OPITCH;
#pragma unroll
    for (int j = 0; j < HMB; ++j) {
      const int mb = kh * HMB + j;
      const float* xp = xch + (size_t)((pw * HMB + j) * 16) * 64 + lane;
      f32x16 own;  // register selects: a runtime index would put the accumulators in scratch
#pragma unroll
      for (int r = 0; r < 16; ++r) own[r] = kh ? oacc[HMB + j][r] : oacc[j][r];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        ushort4 o;
        o.x = to_bf16_bits(own[4 * q4 + 0] * ws + xp[(4 * q4 + 0) * 64] * wo);
        o.y = to_bf16_bits(own[4 * q4 + 1] * ws + xp[(4 * q4 + 1) * 64] * wo);
        o.z = to_bf16_bits(own[4 * q4 + 2] * ws + xp[(4 * q4 + 2) * 64] * wo);
        o.w = to_bf16_bits(own[4 * q4 + 3] * ws + xp[(4 * q4 + 3) * 64] * wo);
        *reinterpret_cast<ushort4*>(orow + 2 * (32 * mb + 8 * q4 + 4 * half)) = o;
      }
    }
  }
  __syncthreads();
  const int nrows = plan.rows_per_wg;
  const bool one_split = !a.ragged && a.splits == 1 && direct;
  for (int n = tid; n < nrows * DCH; n += kStreamThreads) {
    const int r = n / DCH, ch = n % DCH;
    const u32x4 v = *reinterpret_cast<const u32x4*>(smem + REGION0 + r * OPITCH + ch * 16);
    if (one_split) {
      const int gr = rg * plan.rows_per_wg + r;
      if (gr < R)
        *reinterpret_cast<u32x4*>(a.out + o_grp + (gr / kb) * a.o_hs + (long long)(gr % kb) * D + ch * 8) = v;
    } else {
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(a.ws_acc + (slot * plan.rows_per_wg + r) * D + ch * 8));
    }
  }
  if (active && kh == 0 && half == 0) {
    if (one_split) {
      if (a.lse != nullptr && qrow < R) a.lse[l_grp + (qrow / kb) * a.l_hs + qrow % kb] = (m_out + log2f(l_out)) * kLn2;
    } else {
      __builtin_nontemporal_store(m_out, a.ws_ml + (slot * plan.rows_per_wg + wrow) * 2);
      __builtin_nontemporal_store(l_out, a.ws_ml + (slot * plan.rows_per_wg + wrow) * 2 + 1);
    }
  }
  };

  if constexpr (RAGGED) {
    // Balanced placement (several sequences): this work-group's units
    // [T, T1) of the launch's list, one piece per group whose tiles they touch.
    const int H = a.n_kv_heads * plan.row_groups;
    long long T, T1;
    {
      const long long W = ragged_total(a, ragged_tiles(a, plan));
      // with fewer units than work-groups, one unit each: no used
      // work-group's range is empty, so the slots of every group stay
      // consecutive
      const long long n = min((long long)a.nwg, W);
      if (lin >= n) return;
      T1 = W * (lin + 1) / n;
      T = W * lin / n;
    }
    bool first = true;
    while (T < T1) {  // uniform: every wave walks the same pieces
      const SeqAt sq = seq_at(a, ragged_tiles(a, plan), T);
      if (sq.b < 0) break;  // not reached: T < W lies in some sequence
      const int stiles = kPieceCost + seg_tiles(a, sq.b);  // units of each of its segments
      const int lrg = live_row_groups(a, plan, sq.b);
      const long long off = T - sq.base;
      const int h = (int)(off / stiles);
      const int u0 = (int)(off % stiles);  // units [u0, u1) of the segment
      const int u1 = (int)min((long long)stiles, T1 - (sq.base + (long long)h * stiles));
      T += u1 - u0;
      const int p0 = max(u0 - kPieceCost, 0), p1 = max(u1 - kPieceCost, 0);  // its tiles
      if (p0 == p1) continue;  // only the segment's cost units: no piece here
      // live segment h: KV head h / lrg, row group h % lrg (all row groups
      // are live unless the block is short)
      const int g = h / lrg, rg = h % lrg;
      const int seg = sq.b * H + g * plan.row_groups + rg;
      const size_t slot = (size_t)lin + seg;
      if (threadIdx.x == 0) {  // the group's first and last slots, for the merge
        if (p0 == 0) a.ws_tab[seg].x = (int)slot;
        if (p1 == stiles - kPieceCost) a.ws_tab[seg].y = (int)slot;
      }
      if (!first) __syncthreads();  // this piece reuses the LDS of the last one
      first = false;
      piece(sq.b * a.n_kv_heads + g, rg, piece_range(a, sq.b, p0, p1), slot);
    }
  } else {
    // one piece: dispatch order (b, g) groups interleaved, split 0 (the block
    // keys) first.  With lengths growing with b (the training clean rows:
    // sequence b sees b * len_step keys) the longest groups go first, so the
    // short ones fill in behind them rather than the long ones starting last.
    int bg = a.len_step > 0 ? (int)gridDim.z - 1 - lin % (int)gridDim.z : lin % (int)gridDim.z;
    // anchor blocks of a training sequence, or a decode batch without splits:
    // likewise longest first, ranked on the device
    if (a.rank_blocks && a.batch <= kRankMaxBlocks)
      bg = block_by_rank(a.cache_len, a.batch, a.max_len, bg / a.n_kv_heads) * a.n_kv_heads + bg % a.n_kv_heads;
    int rg = (lin / (int)gridDim.z) % (int)gridDim.y;
    int split = lin / ((int)gridDim.z * (int)gridDim.y);
    int S = a.splits;
    size_t slot = (size_t)(bg * plan.row_groups + rg) * a.splits + split;
    if (a.blk_len != nullptr && plan.row_groups > 1) {
      const int lrg = live_row_groups(a, plan, bg / a.n_kv_heads);
      if (lrg < plan.row_groups) {  // short block: deal the head's work-groups over its live row groups
        const int n = plan.row_groups * a.splits, j = rg * a.splits + split;
        rg = j % lrg;
        split = j / lrg;
        S = dealt_splits(n, lrg, rg);
        if (split >= S) return;
        slot = (size_t)bg * n + j;
      }
    }
    piece(bg, rg, split_range(a, bg / a.n_kv_heads, split, S), slot);
  }
}

// Stand-alone merge of the partials left by a streaming launch with fuse = 0:
// 256 threads, one wave per row (D = 128) or per two rows (D = 64) over all
// split groups.
constexpr int kMergeThreads = 256;
template <int D, int SMAX>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(AttnArgs a, AttnPlan plan, int total_rows) {
  constexpr int RPW = 128 / D;
  // Work-group x takes row chunk (x % 8) * (n / 8) + x / 8 of the n chunks.
  // Work-groups are placed on the 8 XCDs round robin, so each XCD merges a
  // contiguous eighth of the rows; with 8 (b, g) groups that is the group
  // whose partials the same XCD's streaming work-groups wrote (the streaming
  // kernel numbers its groups lin % groups), and the reads stay near that
  // XCD's L2.  About 1 us faster per call at L 32768, K 32.
  const int nwg = (int)gridDim.x;
  const int bx = nwg % 8 == 0 ? ((int)blockIdx.x % 8) * (nwg / 8) + (int)blockIdx.x / 8 : (int)blockIdx.x;
  const int gw = bx * (kMergeThreads / 64) + (int)(threadIdx.x >> 6);
  const int first = gw * RPW;  // rows_per_wg is a multiple of 32: a wave's rows share a group
  if (first >= total_rows) return;
  const int grp = first / plan.rows_per_wg;
  merge_wave<D, SMAX>(a, plan, grp, first % plan.rows_per_wg, plan.rows_per_wg);
}

// Merge after a balanced streaming launch: a group's partials sit in
// consecutive slots, whose first and last the streaming launch left in the
// workspace table; there are usually few.  A row takes D / 8 lanes, each
// owning 8 head_dim values (one 16-byte load per partial), and every lane
// reads each partial's (m, l) itself, so no lane exchange is needed.  Partials
// are folded four at a time with an online maximum, in slot order.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_ragged_kernel(AttnArgs a, AttnPlan plan, int total_rows) {
  constexpr int LPR = D / 8;
  constexpr int NB = 4;
  const int mrow = (int)blockIdx.x * (kMergeThreads / LPR) + (int)threadIdx.x / LPR;
  if (mrow >= total_rows) return;
  const int j = (int)threadIdx.x % LPR;
  const int grp = mrow / plan.rows_per_wg;
  const int row = mrow % plan.rows_per_wg;
  // a row group with no live row had no segment, so its table entry is stale
  if (a.blk_len != nullptr && grp % plan.row_groups >= live_row_groups(a, plan, grp / plan.row_groups / a.n_kv_heads))
    return;
  const int2 sl = a.ws_tab[grp];  // first and last slot of the group's partials
  const int S = sl.y - sl.x + 1;
  float M = kNegInf, L = 0.0f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int s0 = 0; s0 < S; s0 += NB) {
    u32x4 v[NB];
    float2 ml[NB];
#pragma unroll
    for (int t = 0; t < NB; ++t) {  // past the last partial: re-read it, weight 0
      const size_t idx = ((size_t)sl.x + min(s0 + t, S - 1)) * plan.rows_per_wg + row;
      v[t] = *reinterpret_cast<const u32x4*>(a.ws_acc + idx * D + 8 * j);
      ml[t] = *reinterpret_cast<const float2*>(a.ws_ml + idx * 2);
    }
    float m[NB];
    float Mn = M;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      m[t] = s0 + t < S ? ml[t].x : kNegInf;
      Mn = fmaxf(Mn, m[t]);
    }
    const float sc = M == kNegInf ? 0.0f : fast_exp2(M - Mn);
    L *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= sc;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const float w = m[t] == kNegInf ? 0.0f : fast_exp2(m[t] - Mn) * ml[t].y;
      L += w;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(w, __uint_as_float(v[t][q] << 16), acc[2 * q]);
        acc[2 * q + 1] = fmaf(w, __uint_as_float(v[t][q] & 0xFFFF0000u), acc[2 * q + 1]);
      }
    }
    M = Mn;
  }
  // rows past the live block length (a block shorter than block_k) were
  // folded from unwritten partials and are not written
  const int rg = grp % plan.row_groups;
  const int bg = grp / plan.row_groups;
  const int kb = live_k(a, bg / a.n_kv_heads);
  const int r = rg * plan.rows_per_wg + row;
  if (r >= a.group * kb) return;
  const int b = bg / a.n_kv_heads, h = (bg % a.n_kv_heads) * a.group + r / kb, i = r % kb;
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = (uint32_t)to_bf16_bits(acc[2 * q] * inv) | ((uint32_t)to_bf16_bits(acc[2 * q + 1] * inv) << 16);
  *reinterpret_cast<u32x4*>(a.out + b * a.o_bs + h * a.o_hs + (long long)i * D + 8 * j) = o;
  if (a.lse != nullptr && j == 0) a.lse[b * a.l_bs + h * a.l_hs + i] = (M + log2f(L)) * kLn2;
}

template <int D, int NQB>
hipError_t launch_stream(const AttnArgs& a, const AttnPlan& p, int direct, hipStream_t stream) {
  dim3 grid(a.splits, p.row_groups, a.batch * a.n_kv_heads);
  if (a.ragged) {
    if (a.blk_mask != nullptr)
      hipLaunchKernelGGL((attn_stream_kernel<D, NQB, true, true>), grid, dim3(kStreamThreads), 0, stream, a, p, direct);
    else
      hipLaunchKernelGGL((attn_stream_kernel<D, NQB, false, true>), grid, dim3(kStreamThreads), 0, stream, a, p, direct);
  } else if (a.blk_mask != nullptr) {
    hipLaunchKernelGGL((attn_stream_kernel<D, NQB, true, false>), grid, dim3(kStreamThreads), 0, stream, a, p, direct);
  } else {
    hipLaunchKernelGGL((attn_stream_kernel<D, NQB, false, false>), grid, dim3(kStreamThreads), 0, stream, a, p, direct);
  }
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
  if (a.ragged) {
    constexpr int rows_per_block = kMergeThreads / (D / 8);
    const int total = a.batch * a.n_kv_heads * p.row_groups * p.rows_per_wg;
    dim3 grid((total + rows_per_block - 1) / rows_per_block);
    hipLaunchKernelGGL((attn_merge_ragged_kernel<D>), grid, dim3(kMergeThreads), 0, stream, a, p, total);
    return hipGetLastError();
  }
  // with a per-sequence block length a live row group can hold the splits of
  // every row group of its head (dealt), up to kMaxSplits
  const int smax = (a.blk_len != nullptr && p.row_groups > 1) ? min(a.splits * p.row_groups, kMaxSplits) : a.splits;
  if (smax <= 8) return launch_merge_s<D, 8>(a, p, stream);
  if (smax <= 16) return launch_merge_s<D, 16>(a, p, stream);
  if (smax <= 32) return launch_merge_s<D, 32>(a, p, stream);
  return launch_merge_s<D, kMaxSplits>(a, p, stream);
}

template <int D>
hipError_t launch_stream_any(const AttnArgs& a, const AttnPlan& p, int direct, hipStream_t stream) {
  switch (p.qblocks) {
    case 1: return launch_stream<D, 1>(a, p, direct, stream);
    case 2: return launch_stream<D, 2>(a, p, direct, stream);
    case 4: return launch_stream<D, 4>(a, p, direct, stream);
    default: return launch_stream<D, 8>(a, p, direct, stream);
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
  // one split writes the rows directly -- unless short blocks may deal several
  // splits to one row group
  if (a.splits == 1 && !a.ragged && !(a.blk_len != nullptr && p.row_groups > 1))
    return launch_stream_any<D>(a, p, 1, stream);
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
