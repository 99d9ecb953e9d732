/*
 * orthrus.h -- C ABI of the MI355X (gfx950) dual-view decode-step library.
 *
 * One Orthrus decode cycle over a frozen AR model's shared KV cache runs, per
 * layer, a diffusion-view block attention and an AR verify attention, then one
 * consensus over the verify distributions.  Sources for what each call
 * computes (the Orthrus pages):
 *   - Paper notes on Orthrus (zhangshuibai.github.io paper-notes,
 *     "Orthrus: Memory-Efficient Parallel Token Generation via Dual-View
 *     Diffusion"): §2.1-2.2 (two views share one KV cache; the diffusion K/V
 *     of the block are transient), §3.2 (block mask), §4.1-4.3 (the cycle:
 *     parallel projection, AR verification, consensus; greedy and T>0).
 *   - hotdry.top blog post on Orthrus dual-view diffusion decoding, sections
 *     on the dual-view attention architecture and on in-model consensus.
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers to contiguous row-major arrays with
 *     the shapes given below; bf16 values travel as uint16_t bit patterns.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream).  No call synchronises, allocates or frees,
 *     and the library keeps no pointer after it returns: buffers must stay
 *     alive until the stream has passed the call.
 *   - All argument checks run on the host before anything is enqueued; on a
 *     non-OK status nothing was enqueued.  No exception crosses the ABI.
 *   - Calls are reentrant and thread-safe (the library has no mutable state).
 *   - Device buffers must be 16-byte aligned (128-bit loads and stores).
 *
 * Environment (read by the block-attention calls on every call; for tuning
 * and diagnosis only, results stay within the documented tolerances):
 *   ORTHRUS_MAX_SPLITS=n   caps the cache splits per (sequence, KV head) at n
 *                          (it can only lower them); it must not change
 *                          between an orthrus_block_attn_partial call and the
 *                          orthrus_block_attn_merge of its partials.
 *   ORTHRUS_ROWS128=1      caps a work-group at 128 query rows (more rows per
 *                          KV head then take several row groups, each
 *                          streaming the cache); it changes the workspace
 *                          size, so it must be set alike for the size query
 *                          and the calls.
 *   ORTHRUS_EVEN_SPLITS=1  gives batches of several sequences equal splits
 *                          per group instead of the balanced placement.
 *   ORTHRUS_DEBUG          prints each attention launch plan to stderr.
 */
#ifndef ORTHRUS_H
#define ORTHRUS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ORTHRUS_OK = 0,
  ORTHRUS_ERR_NULL_PTR = 1,            /* a required pointer is NULL */
  ORTHRUS_ERR_BAD_SHAPE = 2,           /* a size is out of range or inconsistent */
  ORTHRUS_ERR_UNSUPPORTED = 3,         /* valid but not built (e.g. head_dim 96) */
  ORTHRUS_ERR_MISALIGNED = 4,          /* a device pointer is not 16-byte aligned */
  ORTHRUS_ERR_WORKSPACE_TOO_SMALL = 5, /* workspace_bytes below the size query */
  ORTHRUS_ERR_HIP = 6                  /* the HIP runtime refused the launch */
} orthrus_status;

/* Which block keys a block row may see (paper notes §3.2 and §4.1):
 * DIFF_BIDIR   -- diffusion view: every block row sees all K block keys
 *                 (anchor + K-1 mask positions attend to each other);
 * VERIFY_CAUSAL -- AR verify pass: block row i sees block keys j <= i;
 * EXPLICIT     -- a given set per row (orthrus_block_attn_masked only): tree
 *                 verification (ancestors and self) and ragged blocks.
 * In every mode every row sees all cached positions [0, cache_len[b]). */
typedef enum {
  ORTHRUS_MASK_DIFF_BIDIR = 0,
  ORTHRUS_MASK_VERIFY_CAUSAL = 1,
  ORTHRUS_MASK_EXPLICIT = 2
} orthrus_mask_mode;

typedef struct {
  int32_t batch;         /* B >= 1 sequences */
  int32_t n_q_heads;     /* Hq >= 1, a multiple of n_kv_heads */
  int32_t n_kv_heads;    /* Hkv >= 1; q head h reads KV head h / (Hq / Hkv) */
  int32_t head_dim;      /* D, 64 or 128 (other values: ORTHRUS_ERR_UNSUPPORTED) */
  int32_t block_k;       /* K, 1..128 block positions (anchor + K-1 masks) */
  int32_t max_len;       /* cache capacity per sequence = row stride of the cache,
                            0..2^30 (more: ORTHRUS_ERR_UNSUPPORTED) */
  float softmax_scale;   /* 0 -> 1/sqrt(D) */
} orthrus_attn_desc;

/* Workspace bytes that orthrus_block_attn* needs for `d` (0 if `d` is invalid).
 * Depends only on the descriptor's shapes -- never on the cached lengths --
 * so one buffer serves every decode step of a sequence batch. */
size_t orthrus_attn_workspace_size(const orthrus_attn_desc* d);

/* Largest number of cache splits one (sequence, KV head) is streamed in
 * (diagnostic; -1 if `d` is invalid).  Fixed by the descriptor alone; a
 * device with fewer than 256 compute units uses fewer. */
int32_t orthrus_attn_num_splits(const orthrus_attn_desc* d);

/* Dual-view block attention of one layer (paper notes §2.1, §3.2, §4.1).
 *
 * For every sequence b, q head h (KV head g = h / (Hq/Hkv)) and block row i,
 * with L = clamp(cache_len[b], 0, max_len):
 *   keys   = k_cache[b, g, 0:L] ++ k_blk[b, g, 0:K]   (values likewise)
 *   s_j    = softmax_scale * <q[b, h, i], key_j>, over the keys `mode` allows
 *   out    = sum_j softmax(s)_j * value_j              (one joint softmax)
 *   lse    = ln sum_j exp(s_j)
 *
 *   q        bf16 [B, Hq, K, D]
 *   k_blk    bf16 [B, Hkv, K, D]  diffusion view: the transient K_diff of the
 *                                 block; verify: the AR keys of the block tokens
 *   v_blk    bf16 [B, Hkv, K, D]
 *   k_cache  bf16 [B, Hkv, max_len, D]  shared AR cache; read-only, rows >= L
 *                                        are never read
 *   v_cache  bf16 [B, Hkv, max_len, D]
 *   cache_len int32 [B] on the device (positions before the anchor)
 *   out      bf16 [B, Hq, K, D]  (written)
 *   lse      fp32 [B, Hq, K]     natural-log LSE (written; may be NULL)
 *   workspace  device scratch of at least orthrus_attn_workspace_size(d)
 *              bytes, owned by the caller; no initialisation is needed (each
 *              call writes every byte it later reads).  Calls that share a
 *              workspace must not overlap in time (use one workspace per
 *              stream).
 * Neither k_blk/v_blk nor anything else is ever written into the cache. */
orthrus_status orthrus_block_attn(const orthrus_attn_desc* d, int32_t mode,
                                  const uint16_t* q, const uint16_t* k_blk,
                                  const uint16_t* v_blk, const uint16_t* k_cache,
                                  const uint16_t* v_cache, const int32_t* cache_len,
                                  uint16_t* out, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* orthrus_block_attn with mode = ORTHRUS_MASK_DIFF_BIDIR: the diffusion view's
 * block attention (anchor + K-1 masks, bidirectional within the block). */
orthrus_status orthrus_block_attn_diff(const orthrus_attn_desc* d, const uint16_t* q,
                                       const uint16_t* k_blk, const uint16_t* v_blk,
                                       const uint16_t* k_cache, const uint16_t* v_cache,
                                       const int32_t* cache_len, uint16_t* out, float* lse,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* orthrus_block_attn with mode = ORTHRUS_MASK_VERIFY_CAUSAL: the AR verify
 * pass over the K candidate tokens (causal within the block, paper notes
 * §4.1 step 2). */
orthrus_status orthrus_block_attn_verify(const orthrus_attn_desc* d, const uint16_t* q,
                                         const uint16_t* k_blk, const uint16_t* v_blk,
                                         const uint16_t* k_cache, const uint16_t* v_cache,
                                         const int32_t* cache_len, uint16_t* out, float* lse,
                                         void* workspace, size_t workspace_bytes,
                                         void* stream);

/* Block attention with an explicit per-row block mask (tree verification,
 * paper notes §7.4-7.5; ragged blocks): block key j is visible to block row i
 * of sequence b iff bit j of block_mask[b*K + i] is set (uint64 [B, K] on the
 * device; K <= 64, else ORTHRUS_ERR_UNSUPPORTED).  Every row also sees the
 * whole cache [0, cache_len[b]); a row that sees no key at all gets out = 0
 * and lse = -inf.  Everything else is orthrus_block_attn. */
orthrus_status orthrus_block_attn_masked(const orthrus_attn_desc* d, const uint16_t* q,
                                         const uint16_t* k_blk, const uint16_t* v_blk,
                                         const uint16_t* k_cache, const uint16_t* v_cache,
                                         const int32_t* cache_len, const uint64_t* block_mask,
                                         uint16_t* out, float* lse, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* Block attention with a block length per sequence (dynamic block sizes,
 * paper notes §7.4 and §9.6: the block size chosen per sequence from
 * acceptance).  blk_len int32 [B] on the device: sequence b's block in this
 * call is its first k_b = clamp(blk_len[b], 1, K) positions.  Its block rows
 * i < k_b attend to the cache [0, cache_len[b]) and to block keys j < k_b --
 * all of them (ORTHRUS_MASK_DIFF_BIDIR) or j <= i (ORTHRUS_MASK_VERIFY_CAUSAL;
 * other modes: ORTHRUS_ERR_BAD_SHAPE) -- exactly as orthrus_block_attn with
 * K = k_b.  Block keys j >= k_b are invisible, and rows i >= k_b of out and
 * lse are not written.  The buffers keep their [.., K, ..] layouts, so one
 * descriptor and one workspace serve every length; rows past k_b are not
 * computed, so a short block costs less matrix work.  blk_len NULL:
 * ORTHRUS_ERR_NULL_PTR.  Everything else is orthrus_block_attn. */
orthrus_status orthrus_block_attn_dyn(const orthrus_attn_desc* d, int32_t mode,
                                      const uint16_t* q, const uint16_t* k_blk,
                                      const uint16_t* v_blk, const uint16_t* k_cache,
                                      const uint16_t* v_cache, const int32_t* cache_len,
                                      const int32_t* blk_len, uint16_t* out, float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the device scratch behind orthrus_block_attn_noalloc (32 MiB per
 * device, held from library load until the process ends): enough for one
 * sequence of 8 KV heads at any block up to K = 128 (GQA 4). */
#define ORTHRUS_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* orthrus_block_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the call allocates nothing and uses a
 * scratch array the library keeps in device memory, one per device, of
 * ORTHRUS_NOALLOC_SCRATCH_BYTES.  The caller still passes every input and
 * output.  mode is ORTHRUS_MASK_DIFF_BIDIR or ORTHRUS_MASK_VERIFY_CAUSAL.
 * Results are those of orthrus_block_attn with the same arguments, bit for
 * bit.  A descriptor whose orthrus_attn_workspace_size exceeds the scratch
 * returns ORTHRUS_ERR_UNSUPPORTED (nothing enqueued); other errors as
 * orthrus_block_attn.  Every call on one device shares that device's scratch,
 * which keeps the last call's contents: calls that overlap in time on one
 * device (several streams, several host threads) race and give wrong
 * results; calls in one stream's order are safe. */
orthrus_status orthrus_block_attn_noalloc(const orthrus_attn_desc* d, int32_t mode,
                                          const uint16_t* q, const uint16_t* k_blk,
                                          const uint16_t* v_blk, const uint16_t* k_cache,
                                          const uint16_t* v_cache, const int32_t* cache_len,
                                          uint16_t* out, float* lse, void* stream);

/* The two halves of orthrus_block_attn, for callers that schedule or time
 * them separately (or, later, combine partials from several cache shards).
 * orthrus_block_attn_partial streams the cache and the block and leaves one
 * partial softmax state per query row and cache split in `workspace` (fp32
 * reference max and sum, and the bf16 value sum normalised by that sum);
 * orthrus_block_attn_merge combines the splits into `out` and `lse` exactly as
 * orthrus_block_attn does (the pair gives bit-identical results).  Both calls
 * must get the same descriptor and workspace, in this order on one stream;
 * arguments, layouts and errors are those of orthrus_block_attn. */
orthrus_status orthrus_block_attn_partial(const orthrus_attn_desc* d, int32_t mode,
                                          const uint16_t* q, const uint16_t* k_blk,
                                          const uint16_t* v_blk, const uint16_t* k_cache,
                                          const uint16_t* v_cache, const int32_t* cache_len,
                                          void* workspace, size_t workspace_bytes, void* stream);
orthrus_status orthrus_block_attn_merge(const orthrus_attn_desc* d, uint16_t* out, float* lse,
                                        const void* workspace, size_t workspace_bytes,
                                        void* stream);

/* Workspace bytes for either consensus call (0 if the sizes are invalid). */
size_t orthrus_consensus_workspace_size(int32_t batch, int32_t block_k, int32_t vocab);

/* Greedy consensus (paper notes §4.1 step 3 and §4.2).
 *   logits     fp32 [B, K, V]  AR verify logits; row i is checked against cand[i]
 *   cand       int32 [B, K]    diffusion candidates
 *   accept_len int32 [B]       a = leading rows with cand[i] == argmax(row i)
 *   row_argmax int32 [B, K]    argmax of every row (may be NULL)
 *   correction int32 [B]       argmax of row a if a < K, else -1 (no bonus)
 * argmax: lowest index among equal maxima; NaN ranks above every number (first
 * NaN wins); -0 equals +0.  Results are bit-exact (comparisons only).
 * Sizes: 1 <= B, 1 <= K <= 128, B * K <= 65535, 1 <= V <= 2^30 (larger K or
 * V: ORTHRUS_ERR_UNSUPPORTED; larger B * K: ORTHRUS_ERR_BAD_SHAPE). */
orthrus_status orthrus_consensus_greedy(int32_t batch, int32_t block_k, int32_t vocab,
                                        const float* logits, const int32_t* cand,
                                        int32_t* accept_len, int32_t* row_argmax,
                                        int32_t* correction, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* Greedy consensus over a block length per sequence (dynamic block sizes,
 * paper notes §7.4 and §9.6).  blk_len int32 [B] on the device, k_b =
 * clamp(blk_len[b], 1, K): orthrus_consensus_greedy over rows [0, k_b) of
 * sequence b -- accept_len a <= k_b, correction = argmax of row a if a < k_b,
 * else -1 -- with row_argmax (if not NULL) -1 for rows i >= k_b.  Rows past
 * k_b of logits and cand are never read.  blk_len NULL: ORTHRUS_ERR_NULL_PTR.
 * Sizes, workspace and everything else as orthrus_consensus_greedy. */
orthrus_status orthrus_consensus_greedy_dyn(int32_t batch, int32_t block_k, int32_t vocab,
                                            const float* logits, const int32_t* cand,
                                            const int32_t* blk_len, int32_t* accept_len,
                                            int32_t* row_argmax, int32_t* correction,
                                            void* workspace, size_t workspace_bytes, void* stream);

/* T>0 consensus by exact rejection sampling (paper notes §4.3 and §7.2,
 * Leviathan/Chen rule).
 *   p_target  fp32 [B, K, V]  AR probabilities at the sampling temperature
 *   q_draft   fp32 [B, K, V]  diffusion probabilities; cand[b, i] ~ q_draft[b, i]
 *   cand      int32 [B, K]    values in [0, V)
 *   uniforms  fp32 [B, K+1]   on the 2^-24 grid in [0, 1): [0, K) accept tests,
 *                             [K] the residual draw
 *   accept_len int32 [B]      first i with NOT(u_i * q_i(cand_i) < p_i(cand_i)),
 *                             evaluated exactly in fp64; K if none
 *   correction int32 [B]      -1 if a == K; else the token picked from the residual
 *                             w_v = max(0, F(p_a[v]) - F(q_a[v])),
 *                             F(x) = floor(clamp(x, 0, 1) * 2^60) (w = F(p_a) if
 *                             all w are 0; token 0 if that is 0 too):
 *                             smallest v with prefix_sum(w)_v > floor(m * S / 2^24),
 *                             S = sum w, m = floor(u_K * 2^24).
 * Integer arithmetic makes the result bit-exact and independent of reduction
 * order.  Rows must be probability vectors (each summing to at most 8);
 * a cand outside [0, V) counts as a rejection.  Sizes as for
 * orthrus_consensus_greedy. */
orthrus_status orthrus_consensus_sample(int32_t batch, int32_t block_k, int32_t vocab,
                                        const float* p_target, const float* q_draft,
                                        const int32_t* cand, const float* uniforms,
                                        int32_t* accept_len, int32_t* correction,
                                        void* workspace, size_t workspace_bytes,
                                        void* stream);

/* T>0 consensus over a block length per sequence (dynamic block sizes,
 * paper notes §7.4 and §9.6).  blk_len int32 [B] on the device, k_b =
 * clamp(blk_len[b], 1, K): orthrus_consensus_sample over rows [0, k_b) of
 * sequence b -- accept tests with u_0 .. u_{k_b-1}, a <= k_b, correction -1
 * if a == k_b, else drawn from row a's residual with u_K (the uniforms keep
 * their [B, K+1] layout).  Rows past k_b of p_target, q_draft and cand are
 * never read.  blk_len NULL: ORTHRUS_ERR_NULL_PTR.  Everything else as
 * orthrus_consensus_sample. */
orthrus_status orthrus_consensus_sample_dyn(int32_t batch, int32_t block_k, int32_t vocab,
                                            const float* p_target, const float* q_draft,
                                            const int32_t* cand, const float* uniforms,
                                            const int32_t* blk_len, int32_t* accept_len,
                                            int32_t* correction, void* workspace,
                                            size_t workspace_bytes, void* stream);

/* Shapes of one cycle commit.  The cache and block arrays of all n_layers
 * layers are laid out layer-major, one after the other (a caller with
 * separate per-layer buffers commits one layer per call, n_layers = 1). */
typedef struct {
  int32_t n_layers;    /* >= 1 layers committed by one call */
  int32_t batch;       /* B >= 1 */
  int32_t n_kv_heads;  /* Hkv >= 1 */
  int32_t head_dim;    /* D, a multiple of 8, at most 1024 */
  int32_t block_k;     /* K, 1..1024 */
  int32_t max_len;     /* cache capacity per sequence = row stride of the cache,
                          0..2^30 (more: ORTHRUS_ERR_UNSUPPORTED) */
} orthrus_commit_desc;

/* Close one decode cycle on the device: write the verified rows of the AR
 * verify block into the shared cache and advance every sequence's state
 * (paper notes §4.1 step 3: keep the matching candidates, emit the correction
 * drawn at the first mismatch, cut the cache back to just past the kept
 * prefix; §2.2: only the AR path writes the cache).
 *
 * For sequence b with t = cache_len[b] (positions before the anchor) and
 * a = accept_len[b] (from orthrus_consensus_greedy / _sample), let
 * r = a + [a < K].  Verify block rows 0..r-1 -- the anchor and the a accepted
 * candidates, the tokens at positions t..t+r-1 -- are copied, byte for byte,
 * into cache rows t..t+r-1 of every layer and KV head; no other cache row is
 * touched (the unverified rows are never written, which is the cut-back).
 *   k_cache, v_cache  bf16 [n_layers, B, Hkv, max_len, D]   (updated)
 *   k_blk, v_blk      bf16 [n_layers, B, Hkv, K, D]  the AR K/V of the verify
 *                     block (the k_blk/v_blk of orthrus_block_attn_verify);
 *                     must not overlap the cache
 *   cache_len   int32 [B]  read, then advanced IN PLACE to t + r
 *   accept_len  int32 [B]
 *   correction  int32 [B]  used when a < K
 *   cand        int32 [B, K]  the diffusion candidates y1..yK
 *   next_anchor int32 [B]  (written) correction if a < K, else cand[b, K-1]
 *                          (all K accepted, no bonus token)
 *   tokens      int32 [B, K] (written) the tokens the cycle emits:
 *                          cand[b, 0..a-1], then the correction if a < K; -1 after
 *   n_tokens    int32 [B]  (written) r, the number of emitted tokens (1..K)
 * A sequence whose commit cannot be done -- t < 0, a outside [0, K], or
 * t + r > max_len -- is left alone: no cache row is written, cache_len[b]
 * stays, n_tokens[b] = 0 and next_anchor[b] and its tokens row are -1 (the
 * caller checks n_tokens; a full cache is the usual cause).  Everything runs
 * on `stream` without synchronising; the int32 arrays must not overlap one
 * another.  Returns ORTHRUS_ERR_BAD_SHAPE if the block overlaps the cache or
 * the K and V caches overlap. */
orthrus_status orthrus_cache_commit(const orthrus_commit_desc* d, uint16_t* k_cache, uint16_t* v_cache,
                                    const uint16_t* k_blk, const uint16_t* v_blk, int32_t* cache_len,
                                    const int32_t* accept_len, const int32_t* correction,
                                    const int32_t* cand, int32_t* next_anchor, int32_t* tokens,
                                    int32_t* n_tokens, void* stream);

/* orthrus_cache_commit with a block length per sequence (dynamic block
 * sizes, paper notes §7.4 and §9.6), which it also advances.
 *   blk_len      int32 [B] on the device: read as k_b = clamp(blk_len[b], 1, K),
 *                then rewritten IN PLACE with the next cycle's block length.
 *   accept_stat  int32 [B] on the device, the caller's per-sequence state
 *                (0 when a sequence starts: no evidence), updated IN PLACE.
 *   k_min        floor of the block length, 1 <= k_min <= K (else
 *                ORTHRUS_ERR_BAD_SHAPE).
 * The commit is orthrus_cache_commit with K = k_b for sequence b: with
 * r = a + [a < k_b], verify rows 0..r-1 go to cache rows t..t+r-1, the
 * correction is emitted when a < k_b, and a = k_b makes cand[b, k_b-1] the
 * next anchor; a commit is refused when t < 0, a outside [0, k_b] or
 * t + r > max_len.  cand and tokens keep their [B, K] layout.
 * The next length.  accept_stat packs A (bits 31..16) and N (bits 15..0), the
 * accepted and the tested draft candidates in units of 1/16, decayed by 7/8
 * per committed cycle: with t = a + [a < k_b] candidates tested,
 *   N <- min(N - floor(N/8) + 16 t, 65535),  A <- min(A - floor(A/8) + 16 a, N)
 * (an A above N is read as N).  P = floor(65536 A / N) estimates, in Q16, the
 * probability that a candidate matches once the ones before it did; the next
 * block length is the smallest power of two k with P^k <= 8192 (1/8; the
 * powers by repeated squaring, x <- floor(x^2 / 65536)), or K when N = 0,
 * clamped to [k_min, K].  A refused commit writes k_b back and leaves
 * accept_stat alone.  blk_len or accept_stat NULL: ORTHRUS_ERR_NULL_PTR; other
 * errors as orthrus_cache_commit. */
orthrus_status orthrus_cache_commit_dyn(const orthrus_commit_desc* d, uint16_t* k_cache,
                                        uint16_t* v_cache, const uint16_t* k_blk,
                                        const uint16_t* v_blk, int32_t* cache_len,
                                        const int32_t* accept_len, const int32_t* correction,
                                        const int32_t* cand, int32_t* next_anchor,
                                        int32_t* tokens, int32_t* n_tokens, int32_t* blk_len,
                                        int32_t* accept_stat, int32_t k_min, void* stream);

/* Element type of logits for orthrus_forward_kl. */
typedef enum {
  ORTHRUS_DTYPE_F32 = 0,
  ORTHRUS_DTYPE_BF16 = 1
} orthrus_dtype;

/* Workspace bytes orthrus_forward_kl needs (0 if the sizes are invalid). */
size_t orthrus_kl_workspace_size(int32_t rows, int32_t vocab, int32_t dtype);

/* Forward KL of the diffusion view against the frozen AR model over the whole
 * vocabulary -- the distillation loss of paper notes §3.1 and §3.3,
 * KL(P_AR || P_Diff) at every trained position -- and optionally its gradient
 * with respect to the draft (diffusion) logits.
 *   target_logits  [rows, V] (dtype)  AR logits; p = softmax(row)
 *   draft_logits   [rows, V] (dtype)  diffusion logits; q = softmax(row)
 *   kl    fp32 [rows]       (written) sum_v p_v (ln p_v - ln q_v)
 *   grad  [rows, V] (dtype) (written; may be NULL) grad_scale * (q_v - p_v),
 *                           the derivative of kl[n] * grad_scale with respect to
 *                           draft_logits[n, v]; the AR side is frozen
 *   workspace  device scratch of at least orthrus_kl_workspace_size bytes
 *              (one 256-byte unit: the kernel keeps its row statistics in
 *              registers), owned by the caller; no initialisation needed.
 * Logits must be finite; no temperature is applied (the caller scales the
 * logits for one).  Sums run in fp32 in a fixed order, so results are
 * deterministic.  Rows are contiguous with stride V; rows up to 65535 and
 * V up to 2^30 (more: ORTHRUS_ERR_UNSUPPORTED).  grad may alias neither input. */
orthrus_status orthrus_forward_kl(int32_t rows, int32_t vocab, int32_t dtype,
                                  const void* target_logits, const void* draft_logits, float* kl,
                                  void* grad, float grad_scale, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Shapes of the training-time dual-pass attention of one packed sequence. */
typedef struct {
  int32_t seq_len;      /* L clean positions; a multiple of 32 */
  int32_t n_blocks;     /* N anchor blocks (0: AR rows only) */
  int32_t block_k;      /* K positions per block, 1..32 */
  int32_t n_q_heads;    /* Hq, a multiple of n_kv_heads */
  int32_t n_kv_heads;   /* Hkv; q head h reads KV head h / (Hq / Hkv) */
  int32_t head_dim;     /* D, 64 or 128 */
  float softmax_scale;  /* 0 -> 1/sqrt(D) */
} orthrus_train_attn_desc;

/* Forward of the dual-pass block-mask attention used to train the diffusion
 * view (paper notes §3.1-3.2): one packed sequence of L clean tokens carries
 * N anchor blocks of K positions.  In one softmax per row:
 *   AR row i (clean position i) attends to clean keys 0..i (causal);
 *   diffusion row p of block n attends to the clean keys before the block's
 *   anchor, [0, anchors[n]), and to the K diffusion keys of block n
 *   (bidirectionally); blocks never see each other.
 * Layouts are head-major, bf16:
 *   q_ar [Hq, L, D], k_ar / v_ar [Hkv, L, D]      the AR path's q and the
 *                                                 clean keys/values
 *   q_diff [Hq, N*K, D], k_diff / v_diff [Hkv, N*K, D]   block n holds rows
 *                                                 n*K .. n*K+K-1
 *   anchors int32 [N] on the device (clamped to [0, L])
 *   out_ar [Hq, L, D], lse_ar fp32 [Hq, L] (may be NULL)
 *   out_diff [Hq, N*K, D], lse_diff fp32 [Hq, N*K] (may be NULL; the
 *   backward needs it)
 * lse is the natural-log normaliser of each row.  q_ar and out_ar may both be
 * NULL to skip the AR rows.  No workspace: every work-group streams its
 * row's whole prefix.  Asynchronous on `stream`. */
orthrus_status orthrus_train_attn_fwd(const orthrus_train_attn_desc* d, const uint16_t* q_ar,
                                      const uint16_t* k_ar, const uint16_t* v_ar,
                                      const uint16_t* q_diff, const uint16_t* k_diff,
                                      const uint16_t* v_diff, const int32_t* anchors,
                                      uint16_t* out_ar, float* lse_ar, uint16_t* out_diff,
                                      float* lse_diff, void* stream);

/* Backward of the training dual-pass attention for the diffusion rows (the
 * AR backbone is frozen, paper notes §2.1-2.2, so only the diffusion queries,
 * keys and values get gradients).  With P the forward's softmax of a
 * diffusion row (recomputed from lse_diff), O its output and dO the upstream
 * gradient:  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
 *   dq_diff = scale * dS K        over all keys of the row,
 *   dk_diff = scale * dS^T Q,  dv_diff = P^T dO   for the block's own keys,
 * summed over the q heads that share a KV head.
 *   k_ar, v_ar, q_diff, k_diff, v_diff, anchors   as orthrus_train_attn_fwd
 *   out_diff [Hq, N*K, D], lse_diff fp32 [Hq, N*K]   from the forward
 *   d_out_diff [Hq, N*K, D] bf16   upstream gradient of out_diff
 *   dq_diff [Hq, N*K, D], dk_diff / dv_diff [Hkv, N*K, D]   bf16 (written;
 *   every element, no accumulation into existing values)
 * Needs (Hq / Hkv) * K <= 128 (else ORTHRUS_ERR_UNSUPPORTED): one work-group
 * holds every row that reads a block's keys.  No workspace; asynchronous on
 * `stream`. */
orthrus_status orthrus_train_attn_bwd(const orthrus_train_attn_desc* d, const uint16_t* k_ar,
                                      const uint16_t* v_ar, const uint16_t* q_diff,
                                      const uint16_t* k_diff, const uint16_t* v_diff,
                                      const int32_t* anchors, const uint16_t* out_diff,
                                      const float* lse_diff, const uint16_t* d_out_diff,
                                      uint16_t* dq_diff, uint16_t* dk_diff, uint16_t* dv_diff,
                                      void* stream);

/* ------------------------------------------------------------------------
 * Tree verification (paper notes §7.4-7.5 and §9.6: verify a tree of
 * candidate prefixes built from the K diffusion marginals, DDTree style; a
 * tree with unused nodes also carries a shorter block, and the *_dyn entry
 * points above give every sequence its own block length).  A draft tree
 * has K nodes: node 0 is the anchor, node i > 0 has parent[b*K + i] < i and a
 * token; parent -1 marks an unused node.  Verify row i is the AR distribution
 * after the path root..i, so the verify attention lets row i see the block
 * keys of its ancestors and itself (orthrus_tree_masks +
 * orthrus_block_attn_masked).
 * ------------------------------------------------------------------------ */

/* Top-m logits of every row and their log-probabilities (the per-position
 * marginals a draft tree is built from): idx = the m largest logits (ties:
 * lower index first), logp = logit - ln sum_v exp(logit_v), descending.
 *   logits fp32 [rows, V];  logp fp32 [rows, m];  idx int32 [rows, m]
 * 1 <= m <= min(32, V); rows <= 65535; V <= 2^30.  Workspace: orthrus_topk_workspace_size
 * (0 if the sizes are invalid). */
size_t orthrus_topk_workspace_size(int32_t rows, int32_t vocab, int32_t m);
orthrus_status orthrus_topk_logprobs(int32_t rows, int32_t vocab, int32_t m, const float* logits,
                                     float* logp, int32_t* idx, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Best-first draft trees of n_nodes (<= 64) nodes from per-depth marginals:
 *   logp fp32 [B, depth, m] (descending per depth), tok int32 [B, depth, m]:
 *   the top-m tokens of block positions 1..depth;  anchor int32 [B]
 *   parent, tokens, node_depth int32 [B, n_nodes] (written)
 * score(child of node p with rank r) = score(p) + logp[depth(p)][r] in fp32,
 * score(root) = 0; the tree takes the best candidates one at a time (higher
 * score, then lower parent index, then lower rank) -- the n_nodes-1
 * highest-scoring prefixes.  Nodes that cannot be made (too few candidates)
 * get parent -1 and token -1. */
orthrus_status orthrus_tree_build(int32_t batch, int32_t depth, int32_t m, int32_t n_nodes,
                                  const float* logp, const int32_t* tok, const int32_t* anchor,
                                  int32_t* parent, int32_t* tokens, int32_t* node_depth, void* stream);

/* Ancestor-or-self bitmask of every node (bit j of mask[b*K + i] set iff node
 * j lies on the path root..i), the block_mask of the tree-verify attention.
 * parent int32 [B, K], mask uint64 [B, K] (8-byte aligned); K <= 64. */
orthrus_status orthrus_tree_masks(int32_t batch, int32_t block_k, const int32_t* parent,
                                  uint64_t* mask, void* stream);

/* Greedy consensus along a draft tree: from the root, move to the child
 * (lowest node index first, children after their parent) whose token equals
 * the AR argmax of the current node's row; stop when none does.
 *   logits fp32 [B, K, V] (row i: AR logits after the path to node i)
 *   tokens, parent int32 [B, K]
 *   accept_len int32 [B]   a = accepted nodes after the root
 *   path int32 [B, K]      root, n_1, .., n_a, then -1
 *   correction int32 [B]   argmax of the last accepted node's row (always
 *                          emitted: a cycle emits a + 1 tokens)
 *   row_argmax int32 [B, K] (may be NULL)
 * Argmax ties as orthrus_consensus_greedy.  K <= 128.  Workspace:
 * orthrus_consensus_workspace_size. */
orthrus_status orthrus_consensus_tree_greedy(int32_t batch, int32_t block_k, int32_t vocab,
                                             const float* logits, const int32_t* tokens,
                                             const int32_t* parent, int32_t* accept_len,
                                             int32_t* path, int32_t* correction, int32_t* row_argmax,
                                             void* workspace, size_t workspace_bytes, void* stream);

/* Commit an accepted tree path: verify rows path[b, 0..a] (root first) of
 * every layer and KV head go to cache rows t..t+a (t = cache_len[b]); the
 * length grows by a + 1 in place; tokens[b] = the tokens of nodes
 * path[1..a], then the correction (-1 after); n_tokens = a + 1; the
 * correction becomes next_anchor.  Refused per sequence (nothing written,
 * n_tokens 0, -1 outputs) if t < 0, a outside [0, K-1], t + a + 1 > max_len or
 * a path node outside [0, K).  Layouts, aliasing rules and errors as
 * orthrus_cache_commit. */
orthrus_status orthrus_cache_commit_path(const orthrus_commit_desc* d, uint16_t* k_cache,
                                         uint16_t* v_cache, const uint16_t* k_blk,
                                         const uint16_t* v_blk, int32_t* cache_len,
                                         const int32_t* accept_len, const int32_t* path,
                                         const int32_t* node_tokens, const int32_t* correction,
                                         int32_t* next_anchor, int32_t* tokens, int32_t* n_tokens,
                                         void* stream);

/* Static, human-readable name of a status code (any value: unknown codes
 * give "ORTHRUS_ERR_UNKNOWN").  Enumerations travel as int32_t across this
 * interface, so out-of-range values are well defined and are rejected. */
const char* orthrus_status_string(int32_t status);

#ifdef __cplusplus
}
#endif
#endif /* ORTHRUS_H */
