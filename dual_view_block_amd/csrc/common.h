// Internal declarations shared by the host layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace orthrus {

// ---------------------------------------------------------------- attention
// Keys per LDS tile.  Every (sequence, KV head) range of cache rows is cut
// into `splits` contiguous chunks of ceil(L / splits) keys, each streamed in
// tiles of this many keys (the last one of a chunk possibly short).
constexpr int kTileKeys = 64;
// The streaming kernel runs one 512-thread work-group (two waves per SIMD)
// per CU; with more than one split per (sequence, KV head) the launch never
// exceeds the device's CU count.
constexpr int kAttnThreads = 512;
// CU count the workspace is sized for (MI355X).  A device with fewer CUs runs
// fewer splits inside the same workspace.
constexpr int kPlanCUs = 256;
constexpr int kMaxSplits = 64;
// Largest batch whose work-groups are shared out by cache length.
constexpr int kRaggedMaxSeqs = 256;

struct AttnPlan {
  int rows;          // R = G * K query rows per (sequence, KV head)
  int qblocks;       // 32-row query blocks per work-group: 1, 2, 4 or 8
  int rows_per_wg;   // 32 * qblocks
  int row_groups;    // ceil(R / rows_per_wg)
  int splits;        // most splits per (sequence, KV head, row group) the workspace holds
  size_t ml_bytes;       // fp32 (max, sum) per row and split
  size_t acc_bytes;      // bf16 normalised partial outputs per row and split
  size_t tab_bytes;      // int2 per group: first and last partial slot (balanced launches)
  size_t ws_bytes;       // total workspace
};

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k_blk;
  const uint16_t* v_blk;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* cache_len;
  uint16_t* out;
  float* lse;
  float* ws_ml;       // fp32 (reference max, sum) per row and split
  uint16_t* ws_acc;   // bf16 normalised partial output per row and split
  int2* ws_tab;       // per group: first and last partial slot (balanced launches)
  int batch, n_q_heads, n_kv_heads, group, block_k, head_dim, max_len;
  int causal;
  int splits;        // splits of this launch (<= plan.splits)
  int ragged;        // 1: several sequences, the work-groups share one list of tiles (balanced)
  int nwg;           // work-groups of the streaming launch (balanced placement)
  float scale_log2;  // softmax scale * log2(e)
  // Element strides.  Block row i of q head h in sequence b is at
  // q + b*q_bs + h*q_hs + i*head_dim (out likewise with o_*, lse with l_*, in
  // elements of lse); block key j of KV head g at k_blk + b*blk_bs + g*blk_gs
  // + j*head_dim; cache row r at k_cache + b*c_bs + g*c_gs + r*head_dim.
  // The decode layouts are the contiguous ones; c_bs = 0 shares one cache
  // between all sequences.
  long long q_bs, q_hs, o_bs, o_hs, l_bs, l_hs, blk_bs, blk_gs, c_bs, c_gs;
  // > 0: sequence b attends to cache rows [0, b*len_step) and cache_len is
  // not read (causal rows processed in groups of block_k)
  int len_step;
  // 1: the sequences (anchor blocks of a training sequence, or a decode batch
  // with one work-group per group) are taken longest first: work-group j of a
  // KV head takes the sequence of rank j by ceil(cache_len / 64) (see
  // block_order.h); 0: in index order
  int rank_blocks;
  // Explicit block masks (block_k <= 64): bit j of blk_mask[b*block_k + i]
  // set = block key j visible to block row i; NULL = the mode's mask.
  const uint64_t* blk_mask;
  // Live block length per sequence (device, [batch]): sequence b's block is
  // its first k_b = clamp(blk_len[b], 1, block_k) positions; its rows are
  // packed h*k_b + i and rows i >= k_b are neither computed nor written.
  // NULL = block_k for every sequence.
  const int32_t* blk_len;
};

// Contiguous decode layouts: q/out [B,Hq,K,D], lse [B,Hq,K], blocks
// [B,Hkv,K,D], caches [B,Hkv,max_len,D].
inline void set_decode_strides(AttnArgs& a) {
  const long long D = a.head_dim, K = a.block_k;
  a.q_hs = a.o_hs = K * D;
  a.q_bs = a.o_bs = (long long)a.n_q_heads * K * D;
  a.l_hs = K;
  a.l_bs = (long long)a.n_q_heads * K;
  a.blk_gs = K * D;
  a.blk_bs = (long long)a.n_kv_heads * K * D;
  a.c_gs = (long long)a.max_len * D;
  a.c_bs = (long long)a.n_kv_heads * a.max_len * D;
  a.len_step = 0;
  a.rank_blocks = 0;
  a.blk_mask = nullptr;
  a.blk_len = nullptr;
}

// Splits a launch uses on a device with `cus` compute units.
int attn_launch_splits(const AttnPlan& plan, int batch, int n_kv_heads, int max_len, int cus);

// phases: 1 = stream the cache into split partials, 2 = merge the splits,
// 3 = the whole call (a single split writes the output directly; otherwise
// the merge runs as a second kernel on the same stream)
hipError_t launch_block_attention(const AttnArgs& a, const AttnPlan& plan, int phases, hipStream_t stream);

// ---------------------------------------------------------------- consensus
struct ConsensusPlan {
  int greedy_chunks;   // vocab chunks per row for the argmax scan
  int sample_chunks;   // vocab chunks for the residual sums
  size_t greedy_bytes;
  size_t sample_bytes;
  size_t ws_bytes;
};

// blk_len: NULL, or the live block length per sequence (device, [batch]):
// rows i >= clamp(blk_len[b], 1, block_k) are not part of sequence b's block.
hipError_t launch_consensus_greedy(int batch, int block_k, int vocab, const float* logits,
                                   const int32_t* cand, const int32_t* blk_len, int32_t* accept_len,
                                   int32_t* row_argmax, int32_t* correction, void* workspace,
                                   const ConsensusPlan& plan, hipStream_t stream);

hipError_t launch_consensus_sample(int batch, int block_k, int vocab, const float* p_target,
                                   const float* q_draft, const int32_t* cand,
                                   const float* uniforms, const int32_t* blk_len, int32_t* accept_len,
                                   int32_t* correction, void* workspace,
                                   const ConsensusPlan& plan, hipStream_t stream);

// ---------------------------------------------------------------- training backward
// Diffusion-row backward of the dual-pass training attention, head-major
// layouts: q/out/d_out/dq [Hq, N*K, D], k/v/dk/dv_diff [Hkv, N*K, D],
// k/v_ar [Hkv, L, D], lse_diff [Hq, N*K] (natural log), anchors [N].
struct TrainBwdArgs {
  const uint16_t* k_ar;
  const uint16_t* v_ar;
  const uint16_t* q_diff;
  const uint16_t* k_diff;
  const uint16_t* v_diff;
  const int32_t* anchors;
  const uint16_t* out_diff;
  const float* lse_diff;
  const uint16_t* d_out;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int seq_len, n_blocks, block_k, group, n_kv_heads, head_dim;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
};
hipError_t launch_train_bwd(const TrainBwdArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- commit
// Row copies of the verified block into the cache, then the in-place state
// update (two launches on `stream`).  blk_len: NULL, or the live block length
// per sequence, which the state update replaces with the next cycle's
// (floor k_min) from the acceptance statistics accept_stat (updated too).
hipError_t launch_cache_commit(int n_layers, int batch, int n_kv_heads, int head_dim, int block_k,
                               int max_len, uint16_t* k_cache, uint16_t* v_cache, const uint16_t* k_blk,
                               const uint16_t* v_blk, int32_t* cache_len, const int32_t* accept_len,
                               const int32_t* correction, const int32_t* cand, int32_t* next_anchor,
                               int32_t* tokens, int32_t* n_tokens, int32_t* blk_len, int32_t* accept_stat,
                               int k_min, hipStream_t stream);

// ---------------------------------------------------------------- forward KL
// Forward KL (and, if grad != NULL, its gradient) of `rows` logit rows: one
// row-wise launch on `stream` sized from the device's CU count.  vec: every
// row starts 16-byte aligned (16-byte loads).
hipError_t launch_forward_kl(int rows, int vocab, int dtype_bytes, bool vec, const void* target,
                             const void* draft, float* kl, void* grad, float scale, int cus, hipStream_t stream);

// Commit of an accepted tree path (rows path[0..a]); the same two-launch shape.
hipError_t launch_cache_commit_path(int n_layers, int batch, int n_kv_heads, int head_dim, int block_k,
                                    int max_len, uint16_t* k_cache, uint16_t* v_cache, const uint16_t* k_blk,
                                    const uint16_t* v_blk, int32_t* cache_len, const int32_t* accept_len,
                                    const int32_t* path, const int32_t* node_tokens, const int32_t* correction,
                                    int32_t* next_anchor, int32_t* tokens, int32_t* n_tokens, hipStream_t stream);

// Greedy consensus along a draft tree (argmax partials, then one wave per
// sequence walks the tree); the greedy workspace.
hipError_t launch_consensus_tree_greedy(int batch, int block_k, int vocab, const float* logits,
                                        const int32_t* tokens, const int32_t* parent, int32_t* accept_len,
                                        int32_t* path, int32_t* correction, int32_t* row_argmax, void* workspace,
                                        const ConsensusPlan& plan, hipStream_t stream);

// ---------------------------------------------------------------- tree drafting
// Ancestor-or-self masks (uint64 per node) of draft trees, K <= 64.
hipError_t launch_tree_masks(int batch, int block_k, const int32_t* parent, uint64_t* mask, hipStream_t stream);
// Top-m logits and their log-probabilities per row.
int topk_chunks(int vocab);
hipError_t launch_topk_logprobs(int rows, int vocab, int m, const float* logits, float* logp, int32_t* idx,
                                void* workspace, hipStream_t stream);
// Best-first draft trees (one wave per sequence), n_nodes <= 64.
hipError_t launch_tree_build(int batch, int depth, int m, int n_nodes, const float* logp, const int32_t* tok,
                             const int32_t* anchor, int32_t* parent, int32_t* tokens, int32_t* node_depth,
                             hipStream_t stream);

}  // namespace orthrus
