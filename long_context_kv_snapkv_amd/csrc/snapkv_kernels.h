// Internal interface between the host API (snapkv_api.cpp) and the gfx950
// kernels of the SnapKV compression path. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace snapkv {

constexpr int kMaxBatch = 256;
constexpr int kMaxRows = 512;      // G * W scored rows per KV head
constexpr int kMaxKernel = 2049;   // pooling kernel
constexpr int kKeyTile = 64;       // keys staged in LDS per step
constexpr int kPoolTile = 1024;    // pooled outputs per workgroup
constexpr int kTopkThreads = 1024;
constexpr int kTopkLdsKeys = 32768;  // prefix lengths kept in LDS by topk
constexpr int kGatherRows = 32;    // compressed rows per gather workgroup

// Per-prompt table passed by value in the kernel arguments (2 KiB).
struct PromptTable {
  int32_t off[kMaxBatch];  // first packed token of prompt b
  int32_t len[kMaxBatch];  // L_b
};

// Both passes of the window scoring (snapkv_score).
struct ScoreParams {
  const uint16_t* q;  // bf16 [batch, Hq, W, D]
  const uint16_t* k;  // bf16 [T, Hkv, D]
  float2* part;       // [batch, Hkv, nchunk, rows_pad] per-chunk (max, sum) in log2 units
  float* raw;         // [batch, Hkv, p_stride] window vote s_h[j]
  int32_t hq, hkv, window, group;
  int32_t rows, rows_pad;  // G*W and its round-up to 32
  int32_t nwr;             // waves that split the row tiles (power of two)
  int32_t chunk;           // keys per workgroup, multiple of kKeyTile
  int32_t nchunk;          // chunk slots per (prompt, head) in part
  int32_t p_stride;
  int32_t budget, skip_fitting;  // skip prompts with L <= budget when set
  float scale_log2;              // log2(e) / sqrt(D)
  PromptTable tab;
};

struct PoolParams {
  const float* raw;  // [batch, Hkv, p_stride]
  float* out;        // [batch, Hkv, out_stride]
  int32_t hkv, window, kernel, mode;
  int32_t p_stride, out_stride;
  int32_t budget, skip_fitting;
  PromptTable tab;
};

struct TopkParams {
  const float* pooled;  // [batch, Hkv, p_stride]
  int32_t* out_idx;     // [batch, Hkv, budget]
  int32_t hkv, window, budget, p_stride;
  PromptTable tab;
};

struct GatherParams {
  const uint16_t* k;  // bf16 [T, Hkv, D]
  const uint16_t* v;
  uint16_t* out_k;    // bf16 [batch, Hkv, budget, D]
  uint16_t* out_v;
  int32_t* out_idx;   // [batch, Hkv, budget]
  int32_t hkv, budget;
  PromptTable tab;
};

hipError_t launch_score_stats(const ScoreParams& p, int head_dim, int waves,
                              dim3 grid, hipStream_t stream);
hipError_t launch_score_vote(const ScoreParams& p, int head_dim, int waves,
                             dim3 grid, hipStream_t stream);
hipError_t launch_pool(const PoolParams& p, dim3 grid, hipStream_t stream);
hipError_t launch_topk(const TopkParams& p, dim3 grid, hipStream_t stream);
hipError_t launch_gather(const GatherParams& p, int head_dim, dim3 grid,
                         hipStream_t stream);

}  // namespace snapkv
