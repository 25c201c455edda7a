// snapkv_gather: assemble the compressed cache from the kept indices, as work
// items of 64 output rows.
//
// out_k[b,h,t,:] = k[off_b + idx[t], h, :] and likewise for V, for the first
// n = min(L, B) entries; the remaining entries are zero rows with index -1
// (glossary page "SnapKV(スナップケーブイ)", section "SnapKVの仕組み", steps
// 3-4: the kept pairs form the cache that decode then reads). A prompt with
// L <= B is copied whole (indices 0 .. L-1) and its index list is written
// here; for longer prompts the list comes from the selection.
//
// Each lane moves one 16-byte piece of a row, so a wave moves whole rows:
// reads are row-granular gathers from the packed [T, H_kv, D] cache, writes
// are contiguous. All of a thread's loads are issued before its stores.
// Rows are bit copies.
#pragma once

#include "snapkv_device.h"

namespace snapkv {

template <int D>
__device__ __forceinline__ void snapkv_gather_item(const PathParams& p, int b, int h, int rb) {
  constexpr int PIECES = D / 8;
  constexpr int ROWS_PER_PASS = kThreads / PIECES;
  constexpr int PASSES = kGatherRows / ROWS_PER_PASS;
  static_assert(PASSES >= 1 && kGatherRows % ROWS_PER_PASS == 0, "row split");
  const int t0 = rb * kGatherRows;
  const int L = p.tab.len[b];
  const int B = p.budget;
  const bool whole = L <= B;
  const int tid = threadIdx.x;
  int32_t* idx = p.out_idx + (size_t)(b * p.hkv + h) * B;
  const size_t tstride = (size_t)p.hkv * D;
  const uint16_t* ksrc = p.k + ((size_t)p.tab.off[b] * p.hkv + h) * D;
  const uint16_t* vsrc = p.v + ((size_t)p.tab.off[b] * p.hkv + h) * D;
  const size_t obase = (size_t)(b * p.hkv + h) * B * D;
  const int piece = tid % PIECES;
  u32x4 kx[PASSES], vx[PASSES];
  int tt[PASSES];
#pragma unroll
  for (int q = 0; q < PASSES; ++q) {
    const int t = t0 + tid / PIECES + q * ROWS_PER_PASS;
    tt[q] = t;
    kx[q] = vx[q] = u32x4{0u, 0u, 0u, 0u};
    if (t >= B) continue;
    const int j = whole ? (t < L ? t : -1) : idx[t];
    if (j >= 0 && j < L) {  // the bound also keeps a bad index list in range
      kx[q] = *reinterpret_cast<const u32x4*>(ksrc + (size_t)j * tstride + piece * 8);
      vx[q] = *reinterpret_cast<const u32x4*>(vsrc + (size_t)j * tstride + piece * 8);
    }
  }
#pragma unroll
  for (int q = 0; q < PASSES; ++q) {
    const int t = tt[q];
    if (t >= B) continue;
    *reinterpret_cast<u32x4*>(p.out_k + obase + (size_t)t * D + piece * 8) = kx[q];
    *reinterpret_cast<u32x4*>(p.out_v + obase + (size_t)t * D + piece * 8) = vx[q];
    if (whole && piece == 0) idx[t] = t < L ? t : -1;
  }
}

}  // namespace snapkv
