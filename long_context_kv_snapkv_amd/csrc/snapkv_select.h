// snapkv_select: per-head selection of the m = B - W best prefix positions
// (glossary page "SnapKV(スナップケーブイ)", section "SnapKVの仕組み", step 3:
// the top-budget positions by pooled score are kept; paper page "SnapKV: LLM
// Knows What You are Looking for Before Generation", abstract: selection is
// per attention head). Output: the m positions with the largest pooled
// scores, ties going to the lower position, in ascending order, followed by
// the window positions P .. L-1.
//
// One workgroup per (prompt, head), integer decisions only (exact given the
// fp32 pooled scores):
//   * pooled scores become order-preserving 32-bit keys (sign bit set for
//     non-negatives, all bits flipped for negatives);
//   * positions are read in slabs of 4 * kThreads: thread t holds positions
//     4t .. 4t+3 of every slab (one coalesced 16-byte load per slab). Up to
//     kMaxSlabsHeld slabs (64 keys per thread) stay in registers for the
//     whole selection; longer prefixes are re-read in batches of that size;
//   * a radix select over digits of 11, 11 and 10 bits finds tau, the m-th
//     largest key, and `need`, how many keys equal to tau are kept (the
//     lowest-positioned ones). Histograms are LDS atomics into kReplicas
//     copies (lane l adds to copy l % kReplicas, copies 4 banks apart):
//     scores concentrate in few bins, and lanes that hit the same address
//     serialise, so the copies bound that to 64 / kReplicas lanes. One wave
//     sums the copies and finds the bin holding the threshold (row totals,
//     then a suffix scan over lanes) while the others clear the second
//     histogram buffer for the next digit;
//   * ordered compaction: per (slab, wave) counts of keys above and equal to
//     tau, one exclusive scan of those counts in position order, then within
//     a wave ballots and mbcnt give every kept position its output slot.
#pragma once

#include <type_traits>

#include "snapkv_device.h"

namespace snapkv {

constexpr int kSlab = 4 * kThreads;  // positions per slab
constexpr int kMaxSlabsHeld = 16;    // slabs per thread batch: 64 keys in VGPRs
constexpr int kBins = 2048;          // digits: key bits 31..21, 20..10, 9..0
constexpr int kReplicas = 8;         // histogram copies
constexpr int kRepStride = kBins + 4;  // words between copies: 16-byte aligned, 4 banks apart
constexpr int kHistWords = kReplicas * kRepStride;

struct alignas(16) SelectSmem {
  uint32_t rep[2][kHistWords];  // two replicated histograms, used by alternate digits
  uint32_t cnt[kMaxSlabsHeld * kWaves][2];   // per (slab, wave): keys > tau, keys == tau
  uint32_t base[kMaxSlabsHeld * kWaves][2];  // exclusive prefix of cnt in position order
  uint32_t sh_bin, sh_need, sh_gt_carry, sh_eq_carry;
};

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Keys of slabs slab0 .. slab0+NS-1 for this thread. Loads are unconditional
// (clamped to the float4 group holding position P-1, inside the row since
// rows are padded to 64 floats) so they all issue before the first use.
template <int NS>
__device__ __forceinline__ void load_keys(uint32_t (&key)[NS][4], const float* src, int P,
                                          int slab0) {
  const int last = (P - 1) & ~3;
  float4 v[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j = (slab0 + s) * kSlab + 4 * (int)threadIdx.x;
    v[s] = *reinterpret_cast<const float4*>(src + min(j, last));
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    key[s][0] = order_key(v[s].x);
    key[s][1] = order_key(v[s].y);
    key[s][2] = order_key(v[s].z);
    key[s][3] = order_key(v[s].w);
  }
}

// Zero histogram buffer h with 16-byte stores, threads first .. kThreads-1.
__device__ __forceinline__ void clear_hist(uint32_t* h, int first) {
  u32x4* h4 = reinterpret_cast<u32x4*>(h);
  for (int i = (int)threadIdx.x - first; i < kHistWords / 4; i += kThreads - first)
    h4[i] = u32x4{0u, 0u, 0u, 0u};
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Wave 0 only: the bin of replicated histogram h holding the need-th largest
// key (bins ordered by value, the largest last) -> *sh_bin, and how many keys
// of that bin are still needed -> *sh_need. Requires 1 <= need <= total.
// Lane l sums the copies of bins 256 i + 4 l .. +3 for rows i = 0..7 (reads
// of consecutive 16-byte words, conflict-free); the row holding the
// threshold comes from the wave-wide row totals, then a suffix scan over
// the lanes of that row finds the bin.
__device__ __forceinline__ void find_bin_wave(const uint32_t* h, uint32_t need, uint32_t* sh_bin,
                                              uint32_t* sh_need) {
  const int lane = threadIdx.x & 63;
  uint32_t c[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) c[i][e] = 0u;
#pragma unroll
  for (int r = 0; r < kReplicas; ++r) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(h + r * kRepStride + 256 * i + 4 * lane);
      c[i][0] += x[0];
      c[i][1] += x[1];
      c[i][2] += x[2];
      c[i][3] += x[3];
    }
  }
  uint32_t rs[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) rs[i] = wave_sum(c[i][0] + c[i][1] + c[i][2] + c[i][3]);
  // the row from the top whose keys reach `need` (uniform over the wave)
  uint32_t above = 0, cr[4] = {0u, 0u, 0u, 0u};
  int row = 0;
  bool found = false;
#pragma unroll
  for (int i = 7; i >= 0; --i) {
    if (!found && (above + rs[i] >= need || i == 0)) {
      found = true;
      row = i;
#pragma unroll
      for (int e = 0; e < 4; ++e) cr[e] = c[i][e];
    } else if (!found) {
      above += rs[i];
    }
  }
  const uint32_t local = cr[0] + cr[1] + cr[2] + cr[3];
  uint32_t incl = local;  // sum over lanes >= lane
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(incl, off);
    if (lane + off < 64) incl += y;
  }
  const uint32_t ex = above + incl - local;  // keys in bins above this lane's four
  if (ex < need && need <= ex + local) {
    uint32_t a = ex;
    int e_hit = 0;
    bool hit = false;
#pragma unroll
    for (int e = 3; e >= 0; --e) {
      if (!hit && (a + cr[e] >= need || e == 0)) {
        hit = true;
        e_hit = e;
      } else if (!hit) {
        a += cr[e];
      }
    }
    *sh_bin = (uint32_t)(256 * row + 4 * lane + e_hit);
    *sh_need = need - a;
  }
}

// Select for one (prompt, head) with L > budget. NS slabs per batch; with
// RESIDENT the prefix fits in one batch and is loaded once.
template <int NS, bool RESIDENT>
__device__ __forceinline__ void select_head(const PathParams& p, SelectSmem& sm, int b, int h) {
  const int L = p.tab.len[b];
  const int P = L - p.window;
  const uint32_t m = (uint32_t)(p.budget - p.window);  // 1 <= m < P
  const size_t head = (size_t)(b * p.hkv + h);
  const float* src = p.pooled + head * p.pooled_stride;
  int32_t* out = p.out_idx + head * p.budget;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nbatch = RESIDENT ? 1 : (P + NS * kSlab - 1) / (NS * kSlab);

  uint32_t key[NS][4];
  if (RESIDENT) load_keys<NS>(key, src, P, 0);
  clear_hist(sm.rep[0], 0);
  clear_hist(sm.rep[1], 0);
  if (tid == 0) {
    sm.sh_gt_carry = 0u;
    sm.sh_eq_carry = 0u;
  }
  __syncthreads();

  // f(jb, keys) over every float4 group of every batch, in batch order:
  // keys[e] is position jb + e
  auto visit_groups = [&](auto&& f) {
    for (int bt = 0; bt < nbatch; ++bt) {
      if (!RESIDENT) load_keys<NS>(key, src, P, bt * NS);
#pragma unroll
      for (int s = 0; s < NS; ++s) f((bt * NS + s) * kSlab + 4 * tid, key[s]);
    }
  };
  // One digit: keys matching the known prefix are counted into histogram
  // buffer `buf` (copy tid % kReplicas; equal bins within a float4 group add
  // once), then wave 0 finds the threshold bin while the other waves clear
  // the other buffer for the next digit.
  uint32_t prefix = 0u, need = m;
  auto digit = [&](int buf, int shift, uint32_t dmask, uint32_t pmask, bool clear_other) {
    uint32_t* h = sm.rep[buf] + (tid % kReplicas) * kRepStride;
    visit_groups([&](int jb, const uint32_t(&k4)[4]) {
      uint32_t bin[4];
      bool ok[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ok[e] = jb + e < P && (k4[e] & pmask) == prefix;
        bin[e] = (k4[e] >> shift) & dmask;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bool first = ok[e];
        uint32_t c = 0;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const bool same = ok[f] && bin[f] == bin[e];
          if (f < e && same) first = false;
          if (f >= e && same) ++c;
        }
        if (first) atomicAdd(&h[bin[e]], c);
      }
    });
    __syncthreads();
    if (wave == 0)
      find_bin_wave(sm.rep[buf], need, &sm.sh_bin, &sm.sh_need);
    else if (clear_other)
      clear_hist(sm.rep[buf ^ 1], 64);
    __syncthreads();
    prefix |= sm.sh_bin << shift;
    need = sm.sh_need;
  };

  // ---- radix select: digits of 11, 11 and 10 bits
  digit(0, 21, 0x7FFu, 0x00000000u, false);
  digit(1, 10, 0x7FFu, 0xFFE00000u, true);
  digit(0, 0, 0x3FFu, 0xFFFFFC00u, false);
  const uint32_t tau = prefix;  // the m-th largest key
  // `need`: keys equal to tau that are kept

  // ---- ordered compaction, one batch at a time
  const int nent = NS * kWaves;
  for (int bt = 0; bt < nbatch; ++bt) {
    if (!RESIDENT) load_keys<NS>(key, src, P, bt * NS);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int jb = (bt * NS + s) * kSlab + 4 * tid;
      uint32_t gt = 0, eq = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool valid = jb + e < P;
        gt += (uint32_t)__popcll(__ballot(valid && key[s][e] > tau));
        eq += (uint32_t)__popcll(__ballot(valid && key[s][e] == tau));
      }
      if (lane == 0) {
        sm.cnt[s * kWaves + wave][0] = gt;
        sm.cnt[s * kWaves + wave][1] = eq;
      }
    }
    __syncthreads();
    if (wave == 0) {  // exclusive scan of (gt, eq) over entries (slab-major)
      const uint32_t cg = sm.sh_gt_carry, cq = sm.sh_eq_carry;
      const int e0 = 2 * lane, e1 = 2 * lane + 1;
      const uint32_t g0 = e0 < nent ? sm.cnt[e0][0] : 0u, q0 = e0 < nent ? sm.cnt[e0][1] : 0u;
      const uint32_t g1 = e1 < nent ? sm.cnt[e1][0] : 0u, q1 = e1 < nent ? sm.cnt[e1][1] : 0u;
      uint32_t gi = g0 + g1, qi = q0 + q1;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t yg = __shfl_up(gi, off), yq = __shfl_up(qi, off);
        if (lane >= off) {
          gi += yg;
          qi += yq;
        }
      }
      const uint32_t gx = cg + gi - (g0 + g1), qx = cq + qi - (q0 + q1);
      if (e0 < nent) {
        sm.base[e0][0] = gx;
        sm.base[e0][1] = qx;
      }
      if (e1 < nent) {
        sm.base[e1][0] = gx + g0;
        sm.base[e1][1] = qx + q0;
      }
      if (lane == 63) {
        sm.sh_gt_carry = cg + gi;
        sm.sh_eq_carry = cq + qi;
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int jb = (bt * NS + s) * kSlab + 4 * tid;
      const uint32_t gt_before = sm.base[s * kWaves + wave][0];
      const uint32_t eq_before = sm.base[s * kWaves + wave][1];
      bool gt[4], eq[4];
      uint64_t beq[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool valid = jb + e < P;
        gt[e] = valid && key[s][e] > tau;
        eq[e] = valid && key[s][e] == tau;
        beq[e] = __ballot(eq[e]);
      }
      uint32_t eq_rank = eq_before;
#pragma unroll
      for (int e = 0; e < 4; ++e) eq_rank += lanes_below(beq[e]);
      bool sel[4];
      uint64_t bsel[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sel[e] = gt[e] || (eq[e] && eq_rank < need);
        eq_rank += eq[e] ? 1u : 0u;
        bsel[e] = __ballot(sel[e]);
      }
      uint32_t pos = gt_before + min(eq_before, need);
#pragma unroll
      for (int e = 0; e < 4; ++e) pos += lanes_below(bsel[e]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (sel[e] && pos < m) out[pos] = jb + e;
        pos += sel[e] ? 1u : 0u;
      }
    }
    __syncthreads();  // cnt / base are rewritten by the next batch
  }
  for (int i = tid; i < p.window; i += kThreads) out[m + i] = P + i;
}

// Selection of one (prompt, head): the smallest register batch that holds
// the prefix, or batches of kMaxSlabsHeld slabs re-read for longer prefixes.
__device__ __forceinline__ void snapkv_select_item(const PathParams& p, SelectSmem& sm, int b,
                                                   int h) {
  const int P = p.tab.len[b] - p.window;
  const int slabs = (P + kSlab - 1) / kSlab;
  if (slabs <= 1)
    select_head<1, true>(p, sm, b, h);
  else if (slabs <= 2)
    select_head<2, true>(p, sm, b, h);
  else if (slabs <= 4)
    select_head<4, true>(p, sm, b, h);
  else if (slabs <= 8)
    select_head<8, true>(p, sm, b, h);
  else if (slabs <= kMaxSlabsHeld)
    select_head<kMaxSlabsHeld, true>(p, sm, b, h);
  else
    select_head<kMaxSlabsHeld, false>(p, sm, b, h);
}

}  // namespace snapkv
