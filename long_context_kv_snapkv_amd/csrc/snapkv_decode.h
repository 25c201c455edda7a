// Internal interface of the decode-step attention kernels (host API in
// snapkv_api.cpp). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "snapkv_kernels.h"

namespace snapkv {

constexpr int kDecodeThreads = 256;  // 4 wave64s per workgroup
constexpr int kDecodeMaxGroup = 8;   // query heads per KV head
constexpr int kDecodeRowQuantum = 128;  // chunk sizes are multiples of this
constexpr int kDecodeMergeThreads = 1024;
// at most this many chunks per (prompt, KV head): one launch, a chunk item
// that finds every chunk of its head done merges them
constexpr int kDecodeFusedMaxChunks = 16;

// One decode step over a cache. Rows of (prompt b, KV head h) start at
//   compressed: k + ((b * hkv + h) * capacity) * D, consecutive rows D apart;
//   packed:     k + (off[b] * hkv + h) * D,          rows hkv * D apart.
struct DecodeParams {
  const uint16_t* q;  // bf16 [batch, hq, D]
  const uint16_t* k;  // bf16 cache
  const uint16_t* v;
  float* out;         // float32 [batch, hq, D]
  float* part;        // [batch * hkv, nchunk, group, D + 2]: per chunk and query
                      // head (max in log2 units, sum of weights, weighted V sum)
  uint64_t* flags;    // [batch * hkv, kDecodeFusedMaxChunks] one-launch form: chunk done marks
  uint64_t epoch;     // this call's mark (new per call)
  int32_t fused;      // one launch (every prompt has at most kDecodeFusedMaxChunks chunks)
  int32_t batch, hq, hkv, group;
  int32_t chunk;      // cache rows per work item (a multiple of kDecodeRowQuantum)
  int32_t nchunk;     // chunk slots per (prompt, head) in part
  int32_t layout;     // 0 compressed, 1 packed
  int32_t capacity;   // rows per (prompt, head) slot in the compressed layout
  float scale_log2;   // log2(e) / sqrt(D)
  int32_t off[kMaxBatch];  // packed layout: first row of prompt b
  int32_t len[kMaxBatch];  // cached rows of prompt b
};

// Partial attention per chunk of rows, then the per-(prompt, head) merge
// that writes out: in one launch when p.fused, else two. The events, if not
// null, are recorded by the dispatches at the first kernel's start and the
// last kernel's end.
hipError_t launch_decode(const DecodeParams& p, int head_dim, hipStream_t stream,
                         hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

}  // namespace snapkv
