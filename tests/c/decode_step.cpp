// One dual-view decode step of one layer through the C ABI alone, with no
// Python in the call path: the diffusion-view and the verify block attention
// over a shared bf16 cache, then the greedy consensus over given verify
// logits (Orthrus paper notes, zhangshuibai.github.io, §4.1 steps 1-3).
//
// usage: decode_step DIR
//   DIR/meta.txt   B Hq Hkv D K max_len V, then the B cache lengths
//   DIR/q_diff.bin, q_verify.bin   bf16 [B, Hq, K, D]
//   DIR/k_blk_diff.bin, v_blk_diff.bin, k_blk_verify.bin, v_blk_verify.bin   bf16 [B, Hkv, K, D]
//   DIR/k_cache.bin, v_cache.bin   bf16 [B, Hkv, max_len, D]
//   DIR/logits.bin  fp32 [B, K, V];  DIR/cand.bin  int32 [B, K]
// writes DIR/out_diff.bin, out_verify.bin (bf16 [B, Hq, K, D]), lse_diff.bin,
// lse_verify.bin (fp32 [B, Hq, K]), accept_len.bin, correction.bin (int32 [B])
// and row_argmax.bin (int32 [B, K]).
// Exit status: 0 done, 2 no GPU (after printing the host-side workspace
// sizes), 1 any other failure.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "orthrus.h"

namespace {

std::string dir;

bool read_file(const char* name, void* dst, size_t bytes) {
  FILE* f = std::fopen((dir + "/" + name).c_str(), "rb");
  if (!f) return false;
  const size_t got = std::fread(dst, 1, bytes, f);
  std::fclose(f);
  return got == bytes;
}

bool write_file(const char* name, const void* src, size_t bytes) {
  FILE* f = std::fopen((dir + "/" + name).c_str(), "wb");
  if (!f) return false;
  const size_t put = std::fwrite(src, 1, bytes, f);
  std::fclose(f);
  return put == bytes;
}

#define HIP_OK(call)                                                              \
  do {                                                                            \
    const hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));      \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

#define ORTHRUS_OK(call)                                                          \
  do {                                                                            \
    const orthrus_status s_ = (call);                                             \
    if (s_ != ORTHRUS_OK) {                                                       \
      std::fprintf(stderr, "%s: %s\n", #call, orthrus_status_string(s_));        \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

struct Buf {
  std::vector<uint8_t> host;
  void* dev = nullptr;
};

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 1;
  }
  dir = argv[1];
  int B, Hq, Hkv, D, K, max_len, V;
  FILE* mf = std::fopen((dir + "/meta.txt").c_str(), "r");
  if (!mf || std::fscanf(mf, "%d %d %d %d %d %d %d", &B, &Hq, &Hkv, &D, &K, &max_len, &V) != 7) {
    std::fprintf(stderr, "cannot read %s/meta.txt\n", dir.c_str());
    return 1;
  }
  std::vector<int32_t> lens(B);
  for (int b = 0; b < B; ++b)
    if (std::fscanf(mf, "%d", &lens[b]) != 1) {
      std::fprintf(stderr, "meta.txt holds fewer than %d cache lengths\n", B);
      return 1;
    }
  std::fclose(mf);

  const orthrus_attn_desc desc = {B, Hq, Hkv, D, K, max_len, 0.0f};
  const size_t attn_ws = orthrus_attn_workspace_size(&desc);
  const size_t cons_ws = orthrus_consensus_workspace_size(B, K, V);
  std::printf("attn_workspace_bytes %zu\nconsensus_workspace_bytes %zu\n", attn_ws, cons_ws);
  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) != hipSuccess || n_dev < 1) {
    std::printf("no GPU\n");
    return 2;
  }

  const size_t nq = (size_t)B * Hq * K * D, nb = (size_t)B * Hkv * K * D;
  const size_t nc = (size_t)B * Hkv * max_len * D, nl = (size_t)B * K * V;
  struct In { const char* name; size_t bytes; };
  const In ins[] = {{"q_diff.bin", nq * 2},      {"q_verify.bin", nq * 2},     {"k_blk_diff.bin", nb * 2},
                    {"v_blk_diff.bin", nb * 2},  {"k_blk_verify.bin", nb * 2}, {"v_blk_verify.bin", nb * 2},
                    {"k_cache.bin", nc * 2},     {"v_cache.bin", nc * 2},      {"logits.bin", nl * 4},
                    {"cand.bin", (size_t)B * K * 4}};
  Buf in[10];
  for (int i = 0; i < 10; ++i) {
    in[i].host.resize(ins[i].bytes);
    if (!read_file(ins[i].name, in[i].host.data(), ins[i].bytes)) {
      std::fprintf(stderr, "cannot read %s (%zu bytes)\n", ins[i].name, ins[i].bytes);
      return 1;
    }
    HIP_OK(hipMalloc(&in[i].dev, ins[i].bytes));
    HIP_OK(hipMemcpy(in[i].dev, in[i].host.data(), ins[i].bytes, hipMemcpyHostToDevice));
  }
  int32_t* d_len = nullptr;
  HIP_OK(hipMalloc((void**)&d_len, (size_t)B * 4));
  HIP_OK(hipMemcpy(d_len, lens.data(), (size_t)B * 4, hipMemcpyHostToDevice));
  void *d_out_diff, *d_out_verify, *d_lse_diff, *d_lse_verify, *d_acc, *d_corr, *d_am, *d_ws;
  HIP_OK(hipMalloc(&d_out_diff, nq * 2));
  HIP_OK(hipMalloc(&d_out_verify, nq * 2));
  HIP_OK(hipMalloc(&d_lse_diff, (size_t)B * Hq * K * 4));
  HIP_OK(hipMalloc(&d_lse_verify, (size_t)B * Hq * K * 4));
  HIP_OK(hipMalloc(&d_acc, (size_t)B * 4));
  HIP_OK(hipMalloc(&d_corr, (size_t)B * 4));
  HIP_OK(hipMalloc(&d_am, (size_t)B * K * 4));
  const size_t ws_bytes = attn_ws > cons_ws ? attn_ws : cons_ws;
  HIP_OK(hipMalloc(&d_ws, ws_bytes > 0 ? ws_bytes : 16));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));

  auto u16 = [&](int i) { return static_cast<const uint16_t*>(in[i].dev); };
  // step 1: the diffusion view; step 2: the verify view; step 3: consensus.
  // The calls share one workspace: they run in order on one stream.
  ORTHRUS_OK(orthrus_block_attn_diff(&desc, u16(0), u16(2), u16(3), u16(6), u16(7), d_len,
                                     static_cast<uint16_t*>(d_out_diff), static_cast<float*>(d_lse_diff), d_ws,
                                     ws_bytes, stream));
  ORTHRUS_OK(orthrus_block_attn_verify(&desc, u16(1), u16(4), u16(5), u16(6), u16(7), d_len,
                                       static_cast<uint16_t*>(d_out_verify), static_cast<float*>(d_lse_verify),
                                       d_ws, ws_bytes, stream));
  ORTHRUS_OK(orthrus_consensus_greedy(B, K, V, static_cast<const float*>(in[8].dev),
                                      static_cast<const int32_t*>(in[9].dev), static_cast<int32_t*>(d_acc),
                                      static_cast<int32_t*>(d_am), static_cast<int32_t*>(d_corr), d_ws, ws_bytes,
                                      stream));
  HIP_OK(hipStreamSynchronize(stream));

  struct Out { const char* name; void* dev; size_t bytes; };
  const Out outs[] = {{"out_diff.bin", d_out_diff, nq * 2},
                      {"out_verify.bin", d_out_verify, nq * 2},
                      {"lse_diff.bin", d_lse_diff, (size_t)B * Hq * K * 4},
                      {"lse_verify.bin", d_lse_verify, (size_t)B * Hq * K * 4},
                      {"accept_len.bin", d_acc, (size_t)B * 4},
                      {"correction.bin", d_corr, (size_t)B * 4},
                      {"row_argmax.bin", d_am, (size_t)B * K * 4}};
  for (const Out& o : outs) {
    std::vector<uint8_t> h(o.bytes);
    HIP_OK(hipMemcpy(h.data(), o.dev, o.bytes, hipMemcpyDeviceToHost));
    if (!write_file(o.name, h.data(), o.bytes)) {
      std::fprintf(stderr, "cannot write %s\n", o.name);
      return 1;
    }
  }
  HIP_OK(hipStreamDestroy(stream));
  for (Buf& b : in) HIP_OK(hipFree(b.dev));
  for (void* p : {(void*)d_len, d_out_diff, d_out_verify, d_lse_diff, d_lse_verify, d_acc, d_corr, d_am, d_ws})
    HIP_OK(hipFree(p));
  std::printf("done\n");
  return 0;
}
