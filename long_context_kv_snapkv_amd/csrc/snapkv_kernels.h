// Internal interface between the host API (snapkv_api.cpp) and the gfx950
// kernels of the SnapKV compression path. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace snapkv {

constexpr int kMaxBatch = 256;
constexpr int kMaxRows = 512;      // G * W scored rows per KV head
constexpr int kMaxKernel = 2049;   // pooling kernel
constexpr int kThreads = 512;      // workgroup size of every kernel
constexpr int kKeyTile = 64;       // keys per LDS tile
constexpr int kMaxChunk = 4096;    // keys per scoring work item
constexpr int kPoolTile = 2048;    // pooled outputs per standalone pool workgroup
constexpr int kSelectLdsKeys = 32768;  // prefixes up to this stay in LDS during selection
constexpr int kGatherRows = 64;    // compressed rows per gather work item

// Per-prompt table passed by value in the kernel arguments.
struct PromptTable {
  int32_t off[kMaxBatch];  // first packed token of prompt b
  int32_t len[kMaxBatch];  // L_b
};

// Everything the stages read, for one call. Passed by value (< 4 KiB).
struct PathParams {
  const uint16_t* q;  // bf16 [batch, Hq, W, D]
  const uint16_t* k;  // bf16 [T, Hkv, D]
  const uint16_t* v;  // bf16 [T, Hkv, D]
  uint16_t* out_k;    // bf16 [batch, Hkv, budget, D]
  uint16_t* out_v;
  int32_t* out_idx;   // [batch, Hkv, budget]
  float2* part;       // [batch, Hkv, nchunk, rows_pad] per-chunk (max, sum) in log2 units
  float* raw;         // [batch, Hkv, p_stride] window vote s_h[j]
  float* pooled;      // [batch, Hkv, pooled_stride] pooled scores (export, or spill of
                      // selections whose prefix exceeds kSelectLdsKeys)
  uint32_t* sync;     // persistent-kernel counters (see snapkv_api.cpp)
  int32_t batch, hq, hkv, window, group;
  int32_t rows, rows_pad;  // G*W and its round-up to 32
  int32_t nwr;             // waves that split the row tiles (power of two)
  int32_t chunk;           // keys per scoring item, multiple of kKeyTile
  int32_t nchunk;          // chunk slots per (prompt, head) in part
  int32_t p_stride, pooled_stride;
  int32_t budget, kernel, pool_mode;
  int32_t score_all;       // 1: score every prompt with P >= 1 (export); 0: only L > budget
  int32_t n_score_items;   // scoring items (persistent kernel)
  int32_t n_gather_blocks; // gather items per (prompt, head)
  int32_t n_tickets;       // all items of the persistent kernel
  float scale_log2;        // log2(e) / sqrt(D)
  PromptTable tab;
  int32_t item_start[kMaxBatch + 1];  // first scoring item of prompt b
};

// Layout of PathParams::sync (uint32 words); zero between calls.
enum SyncWord { kSyncTicket = 0, kSyncExit = 1, kSyncError = 2, kSyncHeads = 4 };
// then done_stats[batch*Hkv], done_vote[batch*Hkv], done_select[batch*Hkv]

// Standalone stage kernels (grids of work items) and the persistent kernel.
hipError_t launch_score_stats(const PathParams& p, int head_dim, hipStream_t stream);
hipError_t launch_score_vote(const PathParams& p, int head_dim, hipStream_t stream);
hipError_t launch_pool(const PathParams& p, hipStream_t stream);
hipError_t launch_topk(const PathParams& p, hipStream_t stream);
hipError_t launch_gather(const PathParams& p, int head_dim, hipStream_t stream);
hipError_t launch_persistent(const PathParams& p, int head_dim, int workgroups,
                             hipStream_t stream);
hipError_t persistent_blocks_per_cu(int head_dim, int row_tiles_per_wave, int* blocks);

}  // namespace snapkv
