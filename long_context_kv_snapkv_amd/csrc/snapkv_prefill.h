// Internal interface of the prefill attention kernel (snapkv_prefill.hip):
// causal attention of every prompt row, with each row's log-sum-exp, whose
// window rows feed snapkv_compress_from_lse. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "snapkv_kernels.h"

namespace snapkv {

constexpr int kPrefillRows = 128;    // query rows per work item (32 per wave)
constexpr int kPrefillKeys = 64;     // keys per LDS tile
constexpr int kPrefillThreads = 256; // four waves

struct PrefillParams {
  const uint16_t* q;  // bf16 [T, Hq, D]
  const uint16_t* k;  // bf16 [T, Hkv, D]
  const uint16_t* v;  // bf16 [T, Hkv, D]
  uint16_t* out;      // bf16 [T, Hq, D]
  float* window_lse;  // [batch, Hq, W] natural-log normalisers of the last W rows, or null
  uint16_t* q_win;    // bf16 [batch, Hq, W, D] copies of the last W query rows, or null
  int32_t batch, hq, hkv, group, window;
  int32_t nqb;        // query blocks per prompt (of the longest prompt)
  float scale_log2;   // log2(e) / sqrt(D)
  PromptTable tab;
};

hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t stream);

}  // namespace snapkv
