// snapkv_select: per-head selection of the m = B - W best prefix positions
// (glossary page "SnapKV(スナップケーブイ)", section "SnapKVの仕組み", step 3:
// the top-budget positions by pooled score are kept; paper page "SnapKV: LLM
// Knows What You are Looking for Before Generation", abstract: selection is
// per attention head): the m positions with the largest pooled scores, ties
// going to the lower position, in ascending order. This kernel finds the
// threshold and a table of counts from which the gather places every kept
// position in its output slot (the window positions P .. L-1 follow).
//
// One workgroup per (prompt, head), integer decisions only (exact given the
// fp32 pooled scores):
//   * pooled scores are compared as order-preserving 32-bit keys
//     (order_key); positions past P get key 0, below every score's key, so
//     they never count;
//   * positions are read in slabs of 4 * kThreads: thread t holds positions
//     4t .. 4t+3 of every slab (one coalesced 16-byte load per slab). Up to
//     kMaxSlabsHeld slabs (64 keys per thread) stay in registers for the
//     whole selection; longer prefixes are re-read in batches of that size;
//   * radix select, digits of 11, 11 and 10 bits, most significant first.
//     The first digit's histogram was accumulated by the vote kernel. Each
//     later digit counts the keys that match the known prefix into kReplicas
//     LDS copies (lane l adds to copy l % kReplicas, copies 4 banks apart):
//     scores concentrate in few bins and lanes that hit one address
//     serialise, so the copies bound that to 64 / kReplicas lanes. Each wave
//     sums the copies of one histogram row and the bin holding the m-th
//     largest key is found from the row totals. When every key of that bin
//     is needed the threshold is settled at that digit: the kept keys are
//     exactly those >= the bin's lowest key;
//   * count table: for every kSegment positions, how many keys before them
//     lie above the threshold and how many equal it (per-slab wave scans of
//     packed counts, one exclusive scan of the per-(slab, wave) totals).
//     Only if the last digit leaves a bin of equal keys of which some are
//     kept are the lowest-positioned ones of them taken.
#pragma once

#include "snapkv_device.h"

namespace snapkv {

constexpr int kSlab = 4 * kThreads;  // positions per slab
constexpr int kMaxSlabsHeld = 16;    // slabs per thread batch: 64 keys in VGPRs
constexpr int kBins = kTopBins;      // bins per digit (the last digit uses 1024)
constexpr int kReplicas = 8;         // histogram copies
constexpr int kRepStride = kBins + 4;  // words between copies: 16-byte aligned, 4 banks apart
constexpr int kHistWords = kReplicas * kRepStride;

struct alignas(16) SelectSmem {
  uint32_t rep[2][kHistWords];  // replicated histograms of digits 2 and 3
  uint32_t cnt[kMaxSlabsHeld * kWaves];      // per (slab, wave): above | equal << 16
  uint32_t rowtot[kWaves];                   // histogram row totals (find)
  uint32_t sh_bin, sh_need, sh_count, sh_carry0, sh_carry1;
};

// Keys of slabs slab0 .. slab0+NS-1 for this thread; 0 past P. Loads are
// unconditional (clamped to the float4 group holding position P-1, inside
// the row since rows are padded to 64 floats) so they all issue before the
// first use.
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
    const int j = (slab0 + s) * kSlab + 4 * (int)threadIdx.x;
    key[s][0] = j < P ? order_key(v[s].x) : 0u;
    key[s][1] = j + 1 < P ? order_key(v[s].y) : 0u;
    key[s][2] = j + 2 < P ? order_key(v[s].z) : 0u;
    key[s][3] = j + 3 < P ? order_key(v[s].w) : 0u;
  }
}

// Zero histogram buffer h with 16-byte stores, threads first .. kThreads-1.
__device__ __forceinline__ void clear_hist(uint32_t* h, int first) {
  u32x4* h4 = reinterpret_cast<u32x4*>(h);
  for (int i = (int)threadIdx.x - first; i < kHistWords / 4; i += kThreads - first)
    h4[i] = u32x4{0u, 0u, 0u, 0u};
}

// All waves: the bin holding the need-th largest key (bins ordered by value,
// the largest last) -> sm.sh_bin, the keys of that bin still needed ->
// sm.sh_need, and the bin's count -> sm.sh_count. Wave w takes row w (bins
// 256 w .. 256 w + 255); counts() gives this lane's four bins 256 w + 4 lane
// .. +3. Row totals are exchanged through LDS; the wave holding the
// threshold then finds it with its lane scan. Requires 1 <= need <= total.
// Contains two barriers; the result is valid after the second.
template <typename Counts>
__device__ __forceinline__ void find_bin(Counts&& counts, uint32_t need, SelectSmem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  static_assert(kWaves * 256 == kBins, "one histogram row per wave");
  const u32x4 c = counts();
  const uint32_t local = c[0] + c[1] + c[2] + c[3];
  const uint32_t incl = wave_incl_scan(local);  // lanes <= lane of this row
  const uint32_t total = wave_total(incl);
  if (lane == 0) sm.rowtot[wave] = total;
  __syncthreads();
  uint32_t above = 0;  // keys in the rows above this one
  for (int w = kWaves - 1; w > wave; --w) above += sm.rowtot[w];
  if (above < need && need <= above + total) {  // the threshold is in this row
    const uint32_t ex = above + total - incl;   // keys in the lanes above this one
    if (ex < need && need <= ex + local) {
      uint32_t a = ex;
      int e_hit = 0;
      bool hit = false;
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        if (!hit && (a + c[e] >= need || e == 0)) {
          hit = true;
          e_hit = e;
        } else if (!hit) {
          a += c[e];
        }
      }
      sm.sh_bin = (uint32_t)(256 * wave + 4 * lane + e_hit);
      sm.sh_need = need - a;
      sm.sh_count = c[e_hit];
    }
  }
  __syncthreads();
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
  const uint32_t* top = p.top_hist + head * kTopBins;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nbatch = RESIDENT ? 1 : (P + NS * kSlab - 1) / (NS * kSlab);

  uint32_t key[NS][4];
  if (RESIDENT) load_keys<NS>(key, src, P, 0);
  clear_hist(sm.rep[0], 0);
  if (tid == 0) {
    sm.sh_carry0 = 0u;
    sm.sh_carry1 = 0u;
  }
  // digit 1: the histogram the vote kernel accumulated
  find_bin([&] { return *reinterpret_cast<const u32x4*>(top + 256 * wave + 4 * lane); }, m, sm);
  uint32_t prefix = sm.sh_bin << kTopShift;  // resolved high bits of tau
  uint32_t need = sm.sh_need;
  bool settled = need == sm.sh_count;  // the whole threshold bin is kept
  int low = kTopShift;                 // bits below the resolved prefix

  // f(jb, keys) over every float4 group of every batch, in batch order:
  // keys[e] is position jb + e
  auto visit_groups = [&](auto&& f) {
    for (int bt = 0; bt < nbatch; ++bt) {
      if (!RESIDENT) load_keys<NS>(key, src, P, bt * NS);
#pragma unroll
      for (int s = 0; s < NS; ++s) f((bt * NS + s) * kSlab + 4 * tid, key[s]);
    }
  };
  // one more digit of `bits` bits below the resolved prefix, counted into
  // histogram buffer `buf`; the threshold bin is found, then the other
  // buffer is cleared for the next digit
  auto digit = [&](int buf, int bits) {
    const int shift = low - bits;
    const uint32_t dmask = (1u << bits) - 1u;
    uint32_t* hrep = sm.rep[buf] + (tid % kReplicas) * kRepStride;
    visit_groups([&](int, const uint32_t(&k4)[4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((k4[e] >> low) == (prefix >> low)) atomicAdd(&hrep[(k4[e] >> shift) & dmask], 1u);
    });
    __syncthreads();
    const uint32_t* hb = sm.rep[buf];
    find_bin(
        [&] {
          u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int r = 0; r < kReplicas; ++r)
            acc += *reinterpret_cast<const u32x4*>(hb + r * kRepStride + 256 * wave + 4 * lane);
          return acc;
        },
        need, sm);
    clear_hist(sm.rep[buf ^ 1], 0);  // the other buffer, for the next digit
    lds_barrier();
    prefix |= sm.sh_bin << shift;
    need = sm.sh_need;
    settled = need == sm.sh_count;
    low = shift;
  };
  if (!settled) digit(0, 11);
  if (!settled) digit(1, 10);
  // settled: keep every key >= prefix (low bits zero). Otherwise low == 0,
  // tau = prefix exactly, and `need` of the keys equal to tau are kept.
  const uint32_t tau = prefix;

  // ---- count table, one batch at a time. Per slab, each thread counts its
  // keys above the threshold (settled: >= prefix; otherwise > tau) and equal
  // to tau, packed as above | equal << 16 (a wave sums at most 256 of each);
  // the wave totals go through LDS and wave 0 turns them into the counts
  // before every kSegment positions (one (slab, wave) unit), in position
  // order. The gather turns these into output slots: a key above the
  // threshold lands at (above before it) + min(equal before it, need), a key
  // equal to tau is kept while (equal before it) < need and lands at
  // (above before it) + (equal before it).
  static_assert(kSegment == 4 * 64, "a segment is one wave's share of a slab");
  const int nent = NS * kWaves;
  uint32_t* table = p.sel_table + head * (size_t)p.table_stride * 2;
  for (int bt = 0; bt < nbatch; ++bt) {
    if (!RESIDENT) load_keys<NS>(key, src, P, bt * NS);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = key[s][e];
        c += (settled ? u >= tau : u > tau) ? 1u : 0u;
        c += (!settled && u == tau) ? 0x10000u : 0u;
      }
      const uint32_t incl = wave_incl_scan(c);
      if (lane == 63) sm.cnt[s * kWaves + wave] = incl;
    }
    __syncthreads();
    if (wave == 0) {  // exclusive prefix of the (above, equal) totals, slab-major
      const int e0 = 2 * lane, e1 = 2 * lane + 1;
      const uint32_t c0 = e0 < nent ? sm.cnt[e0] : 0u, c1 = e1 < nent ? sm.cnt[e1] : 0u;
      const uint32_t a0 = c0 & 0xFFFFu, b0 = c0 >> 16, a1 = c1 & 0xFFFFu, b1 = c1 >> 16;
      const uint32_t ia = wave_incl_scan(a0 + a1), ib = wave_incl_scan(b0 + b1);
      const uint32_t ca = sm.sh_carry0, cb = sm.sh_carry1;
      const uint32_t xa = ca + ia - (a0 + a1), xb = cb + ib - (b0 + b1);
      const int g0 = bt * nent + e0, g1 = bt * nent + e1;  // segment index in the prefix
      if (e0 < nent && g0 < p.table_stride) {
        table[2 * g0] = xa;
        table[2 * g0 + 1] = xb;
      }
      if (e1 < nent && g1 < p.table_stride) {
        table[2 * g1] = xa + a0;
        table[2 * g1 + 1] = xb + b0;
      }
      if (lane == 63) {
        sm.sh_carry0 = ca + ia;
        sm.sh_carry1 = cb + ib;
      }
    }
    __syncthreads();  // cnt is rewritten by the next batch
  }
  if (tid == 0) {
    uint32_t* meta = p.sel_meta + head * 4;
    meta[0] = tau;
    meta[1] = need;
    meta[2] = settled ? 1u : 0u;
  }
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
