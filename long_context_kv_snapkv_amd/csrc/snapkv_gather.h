// snapkv_gather: assemble the compressed cache, as work items of 64 output
// slots.
//
// out_k[b,h,t,:] = k[off_b + idx[t], h, :] and likewise for V, for the first
// n = min(L, B) slots; the remaining slots are zero rows with index -1
// (glossary page "SnapKV(スナップケーブイ)", section "SnapKVの仕組み", steps
// 3-4: the kept pairs form the cache that decode then reads). A prompt with
// L <= B is copied whole (indices 0 .. L-1). For longer prompts slots
// 0 .. m-1 (m = B - W) hold the kept prefix positions in ascending order and
// slots m .. B-1 the window positions P .. L-1; the item finds the kept
// positions of its slots from the selection's count table: only the
// segments whose kept keys fall into its slots are rescanned (at most one
// per slot), and each kept key's slot follows from the counts before it.
//
// Each lane moves one 16-byte piece of a row, so a wave moves whole rows:
// reads are row-granular gathers from the packed [T, H_kv, D] cache, writes
// are contiguous. All of a thread's loads are issued before its stores.
// Rows are bit copies; out_idx is written here for every slot. The 4-bit
// and 8-bit instances store each row instead as codes and a scale
// (quantize_piece_int4, quantize_piece_fp8).
#pragma once

#include "snapkv_device.h"

namespace snapkv {

struct GatherSmem {
  int32_t pos[kGatherRows];     // kept position of each of the item's slots
  int32_t seg[kGatherRows];     // segments holding them
  uint32_t above[kGatherRows];  // keys above the threshold before each such segment
  uint32_t equal[kGatherRows];  // keys equal to it before each such segment
  uint32_t wa[kWaves], we[kWaves];  // per-wave totals of one round of the scan
  uint32_t nseg;
};

// s.pos[t - lo] = the kept prefix position in slot t, for lo <= t < hi <= m,
// of prompt b / head h with L > B, from the selection's count table `tab`
// and threshold `thr` (global memory, or LDS when the selection ran in this
// workgroup).
__device__ __forceinline__ void locate_kept(const PathParams& p, GatherSmem& s, int b, int h,
                                            int lo, int hi, const uint32_t* tab,
                                            const uint32_t* thr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = p.tab.len[b] - p.window;
  const size_t head = (size_t)(b * p.hkv + h);
  const uint32_t tau = thr[0], need = thr[1];
  const bool settled = thr[2] != 0u;
  const int nseg = (P + kSegment - 1) / kSegment;
  if (tid < kGatherRows) s.pos[tid] = -1;
  if (tid == 0) s.nseg = 0u;
  __syncthreads();
  // running sums of the per-segment counts (kThreads segments per round),
  // then the segments whose kept slots [before, before next) meet [lo, hi):
  // each holds at least one of the item's slots, so there are at most
  // kGatherRows of them (empty segments are skipped). After the last
  // segment the kept count is m.
  uint32_t carry_a = 0u, carry_e = 0u;
  for (int base = 0; base < nseg; base += kThreads) {
    const int e = base + tid;
    const uint32_t a = e < nseg ? tab[2 * e] : 0u, q = e < nseg ? tab[2 * e + 1] : 0u;
    const uint32_t ia = wave_incl_scan(a), iq = wave_incl_scan(q);
    if (lane == 63) {
      s.wa[wave] = ia;
      s.we[wave] = iq;
    }
    __syncthreads();
    uint32_t ba = carry_a + ia - a, bq = carry_e + iq - q;  // before segment e
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t ta = s.wa[w], tq = s.we[w];
      if (w < wave) {
        ba += ta;
        bq += tq;
      }
      carry_a += ta;
      carry_e += tq;
    }
    const uint32_t kb = ba + min(bq, need);
    const uint32_t ka = ba + a + min(bq + q, need);
    if (e < nseg && kb < ka && kb < (uint32_t)hi && ka > (uint32_t)lo) {
      const uint32_t slot = atomicAdd(&s.nseg, 1u);
      if (slot < (uint32_t)kGatherRows) {
        s.seg[slot] = e;
        s.above[slot] = ba;
        s.equal[slot] = bq;
      }
    }
    __syncthreads();  // wa / we are rewritten by the next round
  }
  const int nneed = min((int)s.nseg, kGatherRows);
  const float* src = p.pooled + head * p.pooled_stride;
  const int last = (P - 1) & ~3;
  for (int q = wave; q < nneed; q += kWaves) {
    const int e = s.seg[q];
    const int j0 = e * kSegment + 4 * lane;
    const float4 v = *reinterpret_cast<const float4*>(src + min(j0, last));
    uint32_t key[4] = {j0 < P ? order_key(v.x) : 0u, j0 + 1 < P ? order_key(v.y) : 0u,
                       j0 + 2 < P ? order_key(v.z) : 0u, j0 + 3 < P ? order_key(v.w) : 0u};
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c += (settled ? key[k] >= tau : key[k] > tau) ? 1u : 0u;
      c += (!settled && key[k] == tau) ? 0x10000u : 0u;
    }
    const uint32_t ex = wave_incl_scan(c) - c;
    uint32_t above = s.above[q] + (ex & 0xFFFFu);
    uint32_t equal = s.equal[q] + (ex >> 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t slot = 0xFFFFFFFFu;
      if (settled ? key[k] >= tau : key[k] > tau) {
        slot = above + min(equal, need);
        ++above;
      } else if (!settled && key[k] == tau) {
        if (equal < need) slot = above + equal;
        ++equal;
      }
      if (slot >= (uint32_t)lo && slot < (uint32_t)hi) s.pos[slot - lo] = j0 + k;
    }
  }
  __syncthreads();
}

// Largest magnitude of a row spread over PIECES consecutive lanes, each
// holding one 16-byte piece (8 bf16 values): bf16 magnitude bits order
// finite values, so an integer maximum over the lanes finds it. Every lane
// of the group must call it (the reduction reads the other lanes).
template <int PIECES>
__device__ __forceinline__ float row_amax(const u32x4& w) {
  uint32_t mx = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) mx = max(mx, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
#pragma unroll
  for (int o = 1; o < PIECES; o <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  return __uint_as_float(mx << 16);
}

__device__ __forceinline__ float piece_elem(const u32x4& w, int e) {
  const uint32_t word = w[e >> 1];
  return __uint_as_float((e & 1) ? (word & 0xFFFF0000u) : (word << 16));
}

// 4-bit form of one piece: scale = amax / 7 and codes rint(x * (7 / amax))
// in [-7, 7], in float32 with IEEE rounding; the 8 codes as nibbles,
// element e at bits 4e.
template <int PIECES>
__device__ __forceinline__ uint32_t quantize_piece_int4(const u32x4& w, float& scale) {
  const float amax = row_amax<PIECES>(w);
  scale = amax / 7.0f;
  const float inv = amax > 0.f ? 7.0f / amax : 0.f;
  uint32_t out = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = min(max((int)rintf(piece_elem(w, e) * inv), -7), 7);
    out |= ((uint32_t)c & 0xFu) << (4 * e);
  }
  return out;
}

// 8-bit form of one piece in OCP FP8 E4M3: scale = amax / 448 and codes
// E4M3(x * (448 / amax)) (float32 product, the conversion instruction
// rounding to nearest even); byte e holds element e.
template <int PIECES>
__device__ __forceinline__ uint2 quantize_piece_fp8(const u32x4& w, float& scale) {
  const float amax = row_amax<PIECES>(w);
  scale = amax / 448.0f;
  const float inv = amax > 0.f ? 448.0f / amax : 0.f;
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(piece_elem(w, 0) * inv, piece_elem(w, 1) * inv, 0,
                                           false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(piece_elem(w, 2) * inv, piece_elem(w, 3) * inv, lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(piece_elem(w, 4) * inv, piece_elem(w, 5) * inv, 0,
                                           false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(piece_elem(w, 6) * inv, piece_elem(w, 7) * inv, hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// Storage forms of the kept rows.
constexpr int kStoreBf16 = 0, kStoreInt4 = 1, kStoreFp8 = 2;

// The rows of the item's slots t0 .. t0 + RW - 1, once gs.pos holds the kept
// positions of its slots below m (prompts with L > B).
template <int D, int FORM, int RW>
__device__ __forceinline__ void gather_rows(const PathParams& p, const GatherSmem& gs, int b,
                                            int h, int rb) {
  constexpr int PIECES = D / 8;
  constexpr int ROWS_PER_PASS = kThreads / PIECES;
  constexpr int PASSES = RW / ROWS_PER_PASS;  // RW: rows of this item
  static_assert(PASSES >= 1 && RW % ROWS_PER_PASS == 0, "row split");
  const int t0 = rb * RW;
  const int L = p.tab.len[b];
  const int B = p.budget;
  const bool whole = L <= B;
  const int P = L - p.window, m = B - p.window;
  const int tid = threadIdx.x;
  int32_t* idx = p.out_idx + (size_t)(b * p.hkv + h) * B;
  const size_t tstride = (size_t)p.hkv * D;
  const uint16_t* ksrc = p.k + ((size_t)p.tab.off[b] * p.hkv + h) * D;
  const uint16_t* vsrc = p.v + ((size_t)p.tab.off[b] * p.hkv + h) * D;
  const size_t obase = (size_t)(b * p.hkv + h) * B * D;
  const int piece = tid % PIECES;
  u32x4 kx[PASSES], vx[PASSES];
  int tt[PASSES], jj[PASSES];
#pragma unroll
  for (int q = 0; q < PASSES; ++q) {
    const int t = t0 + tid / PIECES + q * ROWS_PER_PASS;
    tt[q] = t;
    kx[q] = vx[q] = u32x4{0u, 0u, 0u, 0u};
    int j = -1;
    if (t < B) j = whole ? (t < L ? t : -1) : (t < m ? gs.pos[t - t0] : P + (t - m));
    jj[q] = j;
    if (j >= 0 && j < L) {  // the bound also keeps an inconsistent table in range
      kx[q] = *reinterpret_cast<const u32x4*>(ksrc + (size_t)j * tstride + piece * 8);
      vx[q] = *reinterpret_cast<const u32x4*>(vsrc + (size_t)j * tstride + piece * 8);
    }
  }
  if constexpr (FORM == kStoreInt4) {
    // rows of slots >= B and padding rows are zero and quantise to zero
    const size_t hrow = (size_t)(b * p.hkv + h) * B;
#pragma unroll
    for (int q = 0; q < PASSES; ++q) {
      float ks, vs;
      const uint32_t kc = quantize_piece_int4<PIECES>(kx[q], ks);
      const uint32_t vc = quantize_piece_int4<PIECES>(vx[q], vs);
      const int t = tt[q];
      if (t >= B) continue;
      *reinterpret_cast<uint32_t*>(p.out_kq + (hrow + t) * (D / 2) + piece * 4) = kc;
      *reinterpret_cast<uint32_t*>(p.out_vq + (hrow + t) * (D / 2) + piece * 4) = vc;
      if (piece == 0) {
        idx[t] = jj[q];
        p.out_ks[hrow + t] = ks;
        p.out_vs[hrow + t] = vs;
      }
    }
  } else if constexpr (FORM == kStoreFp8) {
    const size_t hrow = (size_t)(b * p.hkv + h) * B;
#pragma unroll
    for (int q = 0; q < PASSES; ++q) {
      float ks, vs;
      const uint2 kc = quantize_piece_fp8<PIECES>(kx[q], ks);
      const uint2 vc = quantize_piece_fp8<PIECES>(vx[q], vs);
      const int t = tt[q];
      if (t >= B) continue;
      *reinterpret_cast<uint2*>(p.out_kq + (hrow + t) * D + piece * 8) = kc;
      *reinterpret_cast<uint2*>(p.out_vq + (hrow + t) * D + piece * 8) = vc;
      if (piece == 0) {
        idx[t] = jj[q];
        p.out_ks[hrow + t] = ks;
        p.out_vs[hrow + t] = vs;
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < PASSES; ++q) {
      const int t = tt[q];
      if (t >= B) continue;
      *reinterpret_cast<u32x4*>(p.out_k + obase + (size_t)t * D + piece * 8) = kx[q];
      *reinterpret_cast<u32x4*>(p.out_v + obase + (size_t)t * D + piece * 8) = vx[q];
      if (piece == 0) idx[t] = jj[q];
    }
  }
}

template <int D, int FORM, int RW>
__device__ __forceinline__ void snapkv_gather_item(const PathParams& p, GatherSmem& gs, int b,
                                                   int h, int rb) {
  const int t0 = rb * RW;
  const int L = p.tab.len[b];
  const int m = p.budget - p.window;
  if (L > p.budget && t0 < m) {
    const size_t head = (size_t)(b * p.hkv + h);
    locate_kept(p, gs, b, h, t0, min(t0 + RW, m), p.sel_table + head * (size_t)p.table_stride * 2,
                p.sel_meta + head * 4);
  }
  gather_rows<D, FORM, RW>(p, gs, b, h, rb);
}

}  // namespace snapkv
