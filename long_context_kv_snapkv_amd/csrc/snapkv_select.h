// snapkv_pool and snapkv_topk: smoothing of a head's vote vector and the
// per-head selection of the m = B - W best prefix positions, as work items.
//
// Pooling (glossary page "SnapKV(スナップケーブイ)", section "SnapKVの仕組み",
// paragraph "Pooling for Robustness"; paper page "SnapKV: LLM Knows What You
// are Looking for Before Generation", section "기술적 접근법": max or average
// pooling, kernel 5-13; kernel 1 leaves the scores as they are):
//   avg: c[j] = (1/k) * sum_{|u-j| <= r} s[u]      (u outside [0, P) adds 0)
//   max: c[j] = max_{|u-j| <= r, 0 <= u < P} s[u]
// with r = k / 2. pool_value() fixes the operation order, so every kernel
// that pools produces identical bits.
//
// Selection (glossary page, same section, step 3: keep the top-budget pairs;
// paper page, abstract: per attention head): the m largest pooled scores,
// ties going to the lower position, in ascending order, followed by the
// window positions P .. L-1. One workgroup per (prompt, head):
//   * the raw votes are staged in LDS and pooled in place; the pooled values
//     become order-preserving 32-bit keys (sign flipped for non-negatives,
//     all bits flipped for negatives); prefixes longer than the LDS cache
//     spill to global memory;
//   * a radix select over three digits (11, 11 and 10 bits) finds the m-th
//     largest key tau and how many keys equal to tau are taken: the first
//     digit over all keys (LDS atomics merged per wave: lanes sharing a bin
//     add once), the last two on the keys of the threshold bin only;
//   * each wave then owns a contiguous segment of positions: per-wave counts
//     of keys above and equal to tau decide which ties are kept (lowest
//     positions first) and where each wave writes; within a wave, ballots
//     and mbcnt prefixes place the kept positions in ascending order.
// Integer-only decisions on the fp32 bits: exact given the scores.
#pragma once

#include "snapkv_device.h"

namespace snapkv {

constexpr int kBins = 2048;
constexpr int kCandCap = 4096;

struct alignas(16) SelectSmem {
  uint32_t keys[kSelectLdsKeys];
  uint32_t hist[kBins];
  uint32_t cand[kCandCap];
  uint32_t wsum[2][kWaves];
  uint32_t sh_bin, sh_need, sh_ncand;
};

// Pooled value at position j from an accessor get(u) for 0 <= u < P.
template <typename Get>
__device__ __forceinline__ float pool_value(Get get, int j, int P, int kernel, int mode) {
  const int r = kernel >> 1;
  if (mode == 1) {
    float v = -kInf;
    for (int e = 0; e < kernel; ++e) {
      const int u = j - r + e;
      if (u >= 0 && u < P) v = fmaxf(v, get(u));
    }
    return v;
  }
  float acc = 0.f;
  for (int e = 0; e < kernel; ++e) {
    const int u = j - r + e;
    if (u >= 0 && u < P) acc += get(u);
  }
  return kernel == 1 ? acc : acc * (1.0f / (float)kernel);
}

// dst[i] = src[i] for i < n (dst in LDS): each thread issues 16 independent
// global loads before storing any, so the copy costs few memory round trips.
__device__ __forceinline__ void load_floats(float* dst, const float* src, int n) {
  constexpr int kBatch = 16;
  for (int base = 0; base < n; base += kThreads * kBatch) {
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base + threadIdx.x + u * kThreads;
      v[u] = src[min(i, n - 1)];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base + threadIdx.x + u * kThreads;
      if (i < n) dst[i] = v[u];
    }
  }
}

// Visit keys j = 0 .. n-1, thread tid taking j = base + tid + u * kThreads:
// kKeyBatch keys are fetched (from LDS, or from the global spill) before any
// is processed. f(j, valid, key) runs on every thread for every slot, so it
// may use wave-wide primitives.
constexpr int kKeyBatch = 8;
template <typename Get, typename F>
__device__ __forceinline__ void for_each_key(int n, Get&& get, F&& f) {
  for (int base = 0; base < n; base += kThreads * kKeyBatch) {
    uint32_t key[kKeyBatch];
#pragma unroll
    for (int u = 0; u < kKeyBatch; ++u) key[u] = get(min(base + (int)threadIdx.x + u * kThreads, n - 1));
#pragma unroll
    for (int u = 0; u < kKeyBatch; ++u) {
      const int j = base + (int)threadIdx.x + u * kThreads;
      f(j, j < n, key[u]);
    }
  }
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Add 1 to hist[bin] for every active lane; lanes sharing a bin are merged
// into one atomic by their lowest lane (up to 4 rounds, then plain atomics).
__device__ __forceinline__ void hist_add(uint32_t* hist, bool active, uint32_t bin) {
  uint64_t pending = __ballot(active);
  const int lane = threadIdx.x & 63;
#pragma unroll 1
  for (int round = 0; round < 4 && pending; ++round) {
    const int leader = __builtin_ctzll(pending);
    const uint32_t lbin = __shfl(bin, leader);
    const uint64_t same = __ballot(active && bin == lbin) & pending;
    if (lane == leader) atomicAdd(&hist[lbin], (uint32_t)__popcll(same));
    pending &= ~same;
  }
  if ((pending >> lane) & 1ull) atomicAdd(&hist[bin], 1u);
}

// Wave 0: the bin holding the need-th largest key among 64*PER bins (bins
// ordered by value), and the count still needed inside it. Each lane holds
// PER contiguous bins in registers.
template <int PER>
__device__ __forceinline__ void find_bin(const uint32_t* hist, uint32_t need, uint32_t* sh_bin,
                                         uint32_t* sh_need) {
  const int lane = threadIdx.x & 63;
  uint32_t c[PER];
  const uint4* h4 = reinterpret_cast<const uint4*>(hist + lane * PER);
#pragma unroll
  for (int i = 0; i < PER / 4; ++i) {
    const uint4 q = h4[i];
    c[4 * i] = q.x;
    c[4 * i + 1] = q.y;
    c[4 * i + 2] = q.z;
    c[4 * i + 3] = q.w;
  }
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) local += c[i];
  uint32_t incl = local;  // sum over lanes >= this lane
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(incl, off);
    if (lane + off < 64) incl += y;
  }
  const uint32_t above = incl - local;
  if (above < need && need <= incl) {
    uint32_t a = above;
    int bin = 0;
    bool found = false;
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      if (!found && (a + c[i] >= need || i == 0)) {
        bin = i;
        found = true;
      } else if (!found) {
        a += c[i];
      }
    }
    *sh_bin = (uint32_t)(lane * PER + bin);
    *sh_need = need - a;
  }
}

// Pool, select and write out_idx for one (prompt, head) with L > budget.
__device__ void snapkv_topk_item(const PathParams& p, SelectSmem& sm, int b, int h) {
  const int L = p.tab.len[b];
  const int P = L - p.window;
  const uint32_t m = (uint32_t)(p.budget - p.window);  // 1 <= m < P
  const float* raw = p.raw + (size_t)(b * p.hkv + h) * p.p_stride;
  float* spill = p.pooled + (size_t)(b * p.hkv + h) * p.pooled_stride;
  int32_t* out = p.out_idx + (size_t)(b * p.hkv + h) * p.budget;
  const int tid = threadIdx.x, lane = tid & 63;
  const bool in_lds = P <= kSelectLdsKeys;

  // ---- pooled keys. Cached prefixes are pooled in place, kCandCap
  // positions at a time: a chunk's pooled values are staged in `cand`, the
  // raw values of its last r positions (the next chunk's left halo) are saved
  // in `hist`, then the chunk is overwritten with its keys.
  if (in_lds) {
    float* vals = reinterpret_cast<float*>(sm.keys);
    float* staged = reinterpret_cast<float*>(sm.cand);
    float* halo = reinterpret_cast<float*>(sm.hist);  // r <= kBins raw values
    const int r = p.kernel >> 1;
    load_floats(vals, raw, P);
    __syncthreads();
    for (int a = 0; a < P; a += kCandCap) {
      const int e = min(P, a + kCandCap);
      for (int j = a + tid; j < e; j += kThreads)
        staged[j - a] = pool_value([&](int u) { return u >= a ? vals[u] : halo[u - (a - r)]; },
                                   j, P, p.kernel, p.pool_mode);
      __syncthreads();
      for (int i = tid; i < r; i += kThreads)
        if (e - r + i >= 0) halo[i] = vals[e - r + i];
      __syncthreads();
      for (int j = a + tid; j < e; j += kThreads) sm.keys[j] = order_key(staged[j - a]);
      __syncthreads();
    }
  } else {
    // long prefix: pool tile by tile through LDS, keys spill to global
    float* vals = reinterpret_cast<float*>(sm.keys);
    const int r = p.kernel >> 1;
    const int span = kSelectLdsKeys - 2 * r;  // positions pooled per tile
    for (int a = 0; a < P; a += span) {
      const int lo = max(0, a - r), hi = min(P, a + span + r);
      load_floats(vals, raw + lo, hi - lo);
      __syncthreads();
      for (int j = a + tid; j < min(P, a + span); j += kThreads)
        spill[j] = pool_value([&](int u) { return vals[u - lo]; }, j, P, p.kernel, p.pool_mode);
      __syncthreads();
    }
  }
  for (int i = tid; i < kBins; i += kThreads) sm.hist[i] = 0u;
  if (tid == 0) sm.sh_ncand = 0u;
  __syncthreads();
  auto key_at = [&](int j) -> uint32_t { return in_lds ? sm.keys[j] : order_key(spill[j]); };

  // ---- digit 1: bits 31..21 over all keys
  for_each_key(P, key_at, [&](int, bool valid, uint32_t u) { hist_add(sm.hist, valid, u >> 21); });
  __syncthreads();
  if (tid < 64) find_bin<kBins / 64>(sm.hist, m, &sm.sh_bin, &sm.sh_need);
  __syncthreads();
  uint32_t prefix = sm.sh_bin << 21;
  uint32_t need = sm.sh_need;
  const uint32_t in_bin = sm.hist[sm.sh_bin];
  const bool use_cand = in_bin <= (uint32_t)kCandCap;
  __syncthreads();

  // ---- the threshold bin's keys (their order is irrelevant for tau)
  if (use_cand) {
    for_each_key(P, key_at, [&](int, bool valid, uint32_t u) {
      const bool hit = valid && (u >> 21) == (prefix >> 21);
      const uint64_t bal = __ballot(hit);
      uint32_t base = 0;
      if (lane == 0 && bal) base = atomicAdd(&sm.sh_ncand, (uint32_t)__popcll(bal));
      base = __shfl(base, 0);
      if (hit) sm.cand[base + lanes_below(bal)] = u;
    });
  }

  // ---- digits 2 (bits 20..10) and 3 (bits 9..0)
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    const uint32_t dmask = pass == 0 ? 0x7FFu : 0x3FFu;
    const uint32_t pmask = pass == 0 ? 0xFFE00000u : 0xFFFFFC00u;
    for (int i = tid; i < kBins; i += kThreads) sm.hist[i] = 0u;
    __syncthreads();
    auto visit = [&](int, bool valid, uint32_t u) {
      hist_add(sm.hist, valid && (u & pmask) == prefix, (u >> shift) & dmask);
    };
    if (use_cand)
      for_each_key((int)in_bin, [&](int j) { return sm.cand[j]; }, visit);
    else
      for_each_key(P, key_at, visit);
    __syncthreads();
    if (tid < 64) {
      if (pass == 0)
        find_bin<2048 / 64>(sm.hist, need, &sm.sh_bin, &sm.sh_need);
      else
        find_bin<1024 / 64>(sm.hist, need, &sm.sh_bin, &sm.sh_need);
    }
    __syncthreads();
    prefix |= sm.sh_bin << shift;
    need = sm.sh_need;
    __syncthreads();  // sh_* and hist are rewritten next pass
  }
  const uint32_t tau = prefix;  // the m-th largest key; `need` keys equal to it are kept

  // ---- compaction: wave w owns one contiguous segment of positions and
  // walks it 64 at a time (coalesced, conflict-free); ballots count in order
  const int wave = tid >> 6;
  const int seg = (P + kWaves * 64 - 1) / (kWaves * 64) * 64;
  const int s0 = min(P, wave * seg), s1 = min(P, s0 + seg);
  // each wave visits its segment 64 keys at a time, kKeyBatch steps per fetch
  auto for_segment = [&](auto&& f) {
    for (int base = s0; base < s1; base += 64 * kKeyBatch) {
      uint32_t key[kKeyBatch];
#pragma unroll
      for (int u = 0; u < kKeyBatch; ++u) key[u] = key_at(min(base + u * 64 + lane, s1 - 1));
#pragma unroll
      for (int u = 0; u < kKeyBatch; ++u) {
        const int j = base + u * 64 + lane;
        f(j, j < s1, key[u]);
      }
    }
  };
  uint32_t w_gt = 0, w_eq = 0;
  if (s0 < s1) {
    for_segment([&](int, bool valid, uint32_t u) {
      w_gt += (uint32_t)__popcll(__ballot(valid && u > tau));
      w_eq += (uint32_t)__popcll(__ballot(valid && u == tau));
    });
  }
  if (lane == 0) {
    sm.wsum[0][wave] = w_gt;
    sm.wsum[1][wave] = w_eq;
  }
  __syncthreads();
  uint32_t eq_before = 0, pos_base = 0;
  for (int w = 0; w < wave; ++w) {
    const uint32_t gt_w = sm.wsum[0][w], eq_w = sm.wsum[1][w];
    const uint32_t take_w = eq_before >= need ? 0u : min(eq_w, need - eq_before);
    pos_base += gt_w + take_w;
    eq_before += eq_w;
  }
  uint32_t eq_seen = 0, sel_seen = 0;
  if (s0 < s1) for_segment([&](int j, bool valid, uint32_t u) {
    const bool gt = valid && u > tau;
    const bool eq = valid && u == tau;
    const uint64_t beq = __ballot(eq);
    const uint32_t eq_rank = eq_before + eq_seen + lanes_below(beq);
    const bool sel = gt || (eq && eq_rank < need);
    const uint64_t bsel = __ballot(sel);
    const uint32_t pos = pos_base + sel_seen + lanes_below(bsel);
    if (sel && pos < m) out[pos] = j;
    eq_seen += (uint32_t)__popcll(beq);
    sel_seen += (uint32_t)__popcll(bsel);
  });
  for (int i = tid; i < p.window; i += kThreads) out[m + i] = P + i;
  __syncthreads();  // LDS is reused by the next item
}

}  // namespace snapkv
