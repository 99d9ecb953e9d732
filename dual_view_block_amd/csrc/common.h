// Internal declarations shared by the host layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace orthrus {

// ---------------------------------------------------------------- attention
// Keys per LDS tile.  Every (sequence, KV head) range of cache rows is cut
// into `splits` contiguous chunks that are whole multiples of this.
constexpr int kTileKeys = 64;
// Work-groups one attention launch aims for: two per CU on a 256-CU MI355X.
constexpr int kTargetAttnGroups = 512;
constexpr int kMaxSplits = 64;

struct AttnPlan {
  int rows;         // R = G * K query rows per (sequence, KV head)
  int qblocks;      // 32-row query blocks per work-group: 1, 2 or 4
  int rows_per_wg;  // 32 * qblocks
  int row_groups;   // ceil(R / rows_per_wg)
  int splits;       // S cache chunks per (sequence, KV head, row group)
  size_t acc_bytes; // fp32 partial outputs
  size_t ml_bytes;  // fp32 (max, sum) pairs
  size_t ws_bytes;  // total workspace
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
  float* ws_acc;
  float* ws_ml;
  int batch, n_q_heads, n_kv_heads, group, block_k, head_dim, max_len;
  int causal;
  float scale_log2;  // softmax scale * log2(e)
};

// phases: 1 = stream the cache into split partials, 2 = merge the splits, 3 = both
hipError_t launch_block_attention(const AttnArgs& a, const AttnPlan& plan, int phases,
                                  hipStream_t stream);

// ---------------------------------------------------------------- consensus
struct ConsensusPlan {
  int greedy_chunks;   // vocab chunks per row for the argmax scan
  int sample_chunks;   // vocab chunks for the residual sums
  size_t greedy_bytes;
  size_t sample_bytes;
  size_t ws_bytes;
};

hipError_t launch_consensus_greedy(int batch, int block_k, int vocab, const float* logits,
                                   const int32_t* cand, int32_t* accept_len,
                                   int32_t* row_argmax, int32_t* correction, void* workspace,
                                   const ConsensusPlan& plan, hipStream_t stream);

hipError_t launch_consensus_sample(int batch, int block_k, int vocab, const float* p_target,
                                   const float* q_draft, const int32_t* cand,
                                   const float* uniforms, int32_t* accept_len,
                                   int32_t* correction, void* workspace,
                                   const ConsensusPlan& plan, hipStream_t stream);

}  // namespace orthrus
