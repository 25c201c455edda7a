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
//     later digit counts the keys that match the known prefix into an LDS
//     histogram with atomic adds (kReplicas copies are supported, lane l
//     adding to copy l % kReplicas, copies 4 banks apart, to spread lanes
//     that hit one address; one copy measured fastest: only the keys of the
//     threshold bin are counted, and clearing and summing copies costs more
//     than the adds they spread). Each wave sums the copies of one histogram
//     row and the bin holding the m-th largest key is found from the row
//     totals. When every key of that bin
//     is needed the threshold is settled at that digit: the kept keys are
//     exactly those >= the bin's lowest key;
//   * count table: for every kSegment positions, how many of its keys lie
//     above the threshold and how many equal it (one wave sum of packed
//     counts per segment). Only if the last digit leaves a bin of equal keys
//     of which some are kept are the lowest-positioned ones of them taken.
//
// Long prefixes (sel_slices > 0) spread each head over workgroups of
// kSliceKeys positions instead, in three kernels (digit 2's histogram,
// digit 3's histogram and the count table) or in one launch that passes
// the histograms between its workgroups (below). Each workgroup re-derives the
// threshold digits known so far from the head's global histograms (the same
// integer search in every workgroup, so all agree), counts its slice into
// LDS and adds the non-zero bins to the head's next histogram with global
// atomics; the kernel boundaries order the passes. Integer sums do not
// depend on the order of the atomics, so the result is the same.
#pragma once

#include "snapkv_device.h"

namespace snapkv {

constexpr int kSlab = 4 * kThreads;  // positions per slab
constexpr int kMaxSlabsHeld = 16;    // slabs per thread batch: 64 keys in VGPRs
static_assert(kMaxSlabsHeld * kSlab == kSelectHeldKeys, "resident prefix length");
constexpr int kBins = kTopBins;      // bins per digit (the last digit uses 1024)
constexpr int kReplicas = 1;         // histogram copies
constexpr int kRepStride = kBins + 4;  // words between copies: 16-byte aligned, 4 banks apart
constexpr int kHistWords = kReplicas * kRepStride;

struct alignas(16) SelectSmem {
  uint32_t rep[2][kHistWords];  // replicated histograms of digits 2 and 3
  uint32_t rowtot[kWaves];                   // histogram row totals (find)
  uint32_t sh_bin, sh_need, sh_count;
  uint32_t sh_lost;  // a search found no bin holding the threshold
};

// Where a selection puts its result: the global count table and threshold
// (the gather reads them after the kernel boundary), or, for a selection
// that runs inside a gather item, a count table in LDS and the threshold
// in `thr` (tau, need, settled, lost: 1 when a radix search found no bin
// holding the threshold, which a consistent histogram never causes).
struct SelectOut {
  uint32_t* table;  // [nseg][2]
  uint32_t* thr;    // [4]
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
// When no bin holds it (need outside [1, total]: an inconsistent histogram)
// the result is bin 0 with need 1 and count 0, and sm.sh_lost is set; a
// consistent histogram leaves sm.sh_lost as it was.
template <typename Counts, typename Smem>
__device__ __forceinline__ void find_bin(Counts&& counts, uint32_t need, Smem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  static_assert(kWaves * 256 == kBins, "one histogram row per wave");
  const u32x4 c = counts();
  const uint32_t local = c[0] + c[1] + c[2] + c[3];
  const uint32_t incl = wave_incl_scan(local);  // lanes <= lane of this row
  const uint32_t total = wave_total(incl);
  if (lane == 0) sm.rowtot[wave] = total;
  if (threadIdx.x == 0) {  // overwritten below by the thread that finds the bin
    sm.sh_bin = 0u;
    sm.sh_need = 1u;
    sm.sh_count = 0u;
  }
  __syncthreads();
  {
    uint32_t all = 0;
    for (int w = 0; w < kWaves; ++w) all += sm.rowtot[w];
    if (threadIdx.x == 0 && (need < 1u || need > all)) sm.sh_lost = 1u;
  }
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
__device__ __forceinline__ void select_head(const PathParams& p, SelectSmem& sm, int b, int h,
                                            const SelectOut& out) {
  const int L = p.tab.len[b];
  const int P = L - p.window;
  const uint32_t m = (uint32_t)(p.budget - p.window);  // 1 <= m < P
  const size_t head = (size_t)(b * p.hkv + h);
  const float* src = p.pooled + head * p.pooled_stride;
  const uint32_t* top = p.top_hist + head * kSelHistWords;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nbatch = RESIDENT ? 1 : (P + NS * kSlab - 1) / (NS * kSlab);

  // digit 1: the histogram the vote kernel accumulated. Its row is loaded
  // before the keys, so the first search waits for it alone while the keys
  // are still in flight. When the score kernel marked it untrustworthy for
  // this call (hist_bad), the digit is recounted here from the keys.
  const bool recount = p.hist_bad[head] == p.epoch;
  u32x4 top4 = u32x4{0u, 0u, 0u, 0u};
  if (!recount) top4 = *reinterpret_cast<const u32x4*>(top + 256 * wave + 4 * lane);
  asm volatile("" ::: "memory");  // the histogram loads stay older than the keys'
  uint32_t key[NS][4];
  if (RESIDENT) load_keys<NS>(key, src, P, 0);
  // both digit histograms are cleared now, while the keys are in flight
  // (the search's barriers order the clearing before the counting)
  clear_hist(sm.rep[0], 0);
  clear_hist(sm.rep[1], 0);
  if (tid == 0) sm.sh_lost = 0u;

  // f(jb, keys) over every float4 group of every batch, in batch order:
  // keys[e] is position jb + e
  auto visit_groups = [&](auto&& f) {
    for (int bt = 0; bt < nbatch; ++bt) {
      if (!RESIDENT) load_keys<NS>(key, src, P, bt * NS);
#pragma unroll
      for (int s = 0; s < NS; ++s) f((bt * NS + s) * kSlab + 4 * tid, key[s]);
    }
  };
  if (recount) {
    __syncthreads();  // the clearing is done
    visit_groups([&](int jb, const uint32_t(&k4)[4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (jb + e < P) lds_count(sm.rep[1], k4[e] >> kTopShift);
    });
    __syncthreads();
    top4 = *reinterpret_cast<const u32x4*>(sm.rep[1] + 256 * wave + 4 * lane);
    __syncthreads();  // every row is read before the buffer is cleared again
    clear_hist(sm.rep[1], 0);  // for digit 3; ordered by the search's barriers
  }
  find_bin([&] { return top4; }, m, sm);
  uint32_t prefix = sm.sh_bin << kTopShift;  // resolved high bits of tau
  uint32_t need = sm.sh_need;
  bool settled = need == sm.sh_count;  // the whole threshold bin is kept
  int low = kTopShift;                 // bits below the resolved prefix
  // one more digit of `bits` bits below the resolved prefix, counted into
  // histogram buffer `buf` (cleared at the start); the threshold bin is found
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

  // ---- count table: per kSegment positions (one wave's share of a slab),
  // the keys above the threshold (settled: >= prefix; otherwise > tau) and
  // the keys equal to tau. The gather turns the running sums of these into
  // output slots: a key above the threshold lands at (above before it) +
  // min(equal before it, need), a key equal to tau is kept while (equal
  // before it) < need and lands at (above before it) + (equal before it).
  static_assert(kSegment == 4 * 64, "a segment is one wave's share of a slab");
  const int nseg = (P + kSegment - 1) / kSegment;
  uint32_t* table = out.table;
  // `settled` is the same in every thread (read from LDS after a barrier);
  // taken as a scalar, each key costs one or two compares, not both forms
  const bool settled_s = __builtin_amdgcn_readfirstlane(settled ? 1 : 0) != 0;
  for (int bt = 0; bt < nbatch; ++bt) {
    if (!RESIDENT) load_keys<NS>(key, src, P, bt * NS);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      // the wave's counts from ballots of its 64 lanes (scalar popcounts)
      uint32_t above = 0, equal = 0;
      if (settled_s) {
#pragma unroll
        for (int e = 0; e < 4; ++e) above += (uint32_t)__popcll(__ballot(key[s][e] >= tau));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          above += (uint32_t)__popcll(__ballot(key[s][e] > tau));
          equal += (uint32_t)__popcll(__ballot(key[s][e] == tau));
        }
      }
      const int g = (bt * NS + s) * kWaves + wave;  // segment index in the prefix
      if (lane == 0 && g < nseg) {
        table[2 * g] = above;
        table[2 * g + 1] = equal;
      }
    }
  }
  if (tid == 0) {
    out.thr[0] = tau;
    out.thr[1] = need;
    out.thr[2] = settled ? 1u : 0u;
    out.thr[3] = sm.sh_lost;
  }
}

// ------------------------------------------------------ sliced selection ---
constexpr int kSliceReplicas = 1;  // histogram copies (one measured fastest, as for kReplicas)
static_assert(kSliceKeys == 2 * kSlab, "a slice is two slabs: 8 keys per thread");

struct alignas(16) SliceSmem {
  uint32_t rep[kSliceReplicas * kRepStride];
  uint32_t rowtot[kWaves];
  uint32_t sh_bin, sh_need, sh_count;
  uint32_t sh_lost;
};

// The threshold as far as `digits` radix digits, from the head's global
// histograms hist (digit 1: 2048 bins, digit 2: 2048 bins at +2048, digit
// 3: 1024 bins at +4096): the resolved high bits `prefix`, the number of
// bits below them `low`, the keys of the final bin still needed, and whether
// every key of that bin is kept. Uniform over the workgroup.
struct Threshold {
  uint32_t prefix, need;
  int low;
  bool settled;
};

// `d1` is the first digit's histogram (the head's, in global memory or LDS).
template <typename Smem>
__device__ __forceinline__ Threshold resolve_digits(const uint32_t* hist, const uint32_t* d1,
                                                    int digits, uint32_t m, Smem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  Threshold t{0u, m, 32, false};
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    if (d >= digits || t.settled) break;
    const int shift = d == 0 ? kTopShift : (d == 1 ? 10 : 0);
    const int nbins = d == 2 ? 1024 : 2048;
    const uint32_t* hd = d == 0 ? d1 : hist + (d == 1 ? kHistD2 : kHistD3);
    find_bin(
        [&] {
          const int i = 256 * wave + 4 * lane;
          return i < nbins ? *reinterpret_cast<const u32x4*>(hd + i) : u32x4{0u, 0u, 0u, 0u};
        },
        t.need, sm);
    t.prefix |= sm.sh_bin << shift;
    t.need = sm.sh_need;
    t.settled = t.need == sm.sh_count;
    t.low = shift;
  }
  return t;
}

// Keys of positions s0 .. s0 + kSliceKeys - 1 for this thread: slab g holds
// s0 + g * kSlab + 4t .. +3; 0 past P.
__device__ __forceinline__ void load_slice_keys(uint32_t (&key)[2][4], const float* src, int P,
                                                int s0) {
  const int last = (P - 1) & ~3;
  float4 v[2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
    v[g] = *reinterpret_cast<const float4*>(src + min(s0 + g * kSlab + 4 * (int)threadIdx.x, last));
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int j = s0 + g * kSlab + 4 * (int)threadIdx.x;
    key[g][0] = j < P ? order_key(v[g].x) : 0u;
    key[g][1] = j + 1 < P ? order_key(v[g].y) : 0u;
    key[g][2] = j + 2 < P ? order_key(v[g].z) : 0u;
    key[g][3] = j + 3 < P ? order_key(v[g].w) : 0u;
  }
}

// Digit DIGIT (2: 11 bits at bit 10, 3: 10 bits at bit 0) of the slice's
// keys that match the threshold's resolved prefix, added to the head's
// histogram of that digit. Nothing to do once the threshold is settled.
template <int DIGIT>
__device__ __forceinline__ void select_digit_slice(const PathParams& p, SliceSmem& sm, int b,
                                                   int h, int sl) {
  static_assert(DIGIT == 2 || DIGIT == 3, "digits 2 and 3");
  constexpr int kShift = DIGIT == 2 ? 10 : 0;
  constexpr int kBinsHere = DIGIT == 2 ? 2048 : 1024;
  const int P = p.tab.len[b] - p.window;
  const int s0 = sl * kSliceKeys;
  if (s0 >= P) return;
  const size_t head = (size_t)(b * p.hkv + h);
  uint32_t* hist = p.top_hist + head * kSelHistWords;
  const int tid = threadIdx.x;
  const float* src = p.pooled + head * p.pooled_stride;
  const bool recount = p.hist_bad[head] == p.epoch;
  uint32_t key[2][4];
  load_slice_keys(key, src, P, s0);
  u32x4* r4 = reinterpret_cast<u32x4*>(sm.rep);
  auto clear = [&] {
    for (int i = tid; i < kSliceReplicas * kRepStride / 4; i += kThreads)
      r4[i] = u32x4{0u, 0u, 0u, 0u};
  };
  clear();
  if (tid == 0) sm.sh_lost = 0u;
  const uint32_t* d1 = hist + (recount && DIGIT == 3 ? kHistFix : kHistD1);
  if (DIGIT == 2 && recount) {
    // the score kernel's first-digit counts are not to be trusted for this
    // call: every slice recounts that digit over the whole prefix, and
    // slice 0 leaves it for the later passes
    __syncthreads();
    for (int a = 0; a < P; a += kSliceKeys) {
      uint32_t k2[2][4];
      load_slice_keys(k2, src, P, a);
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (a + g * kSlab + 4 * tid + e < P) lds_count(sm.rep, k2[g][e] >> kTopShift);
    }
    __syncthreads();
    if (sl == 0)
      for (int i = tid; i < kTopBins; i += kThreads) hist[kHistFix + i] = sm.rep[i];
    d1 = sm.rep;
  }
  // (the search's barriers also order the clearing before the counting)
  const Threshold t = resolve_digits(hist, d1, DIGIT - 1, (uint32_t)(p.budget - p.window), sm);
  if (t.settled) return;
  if (DIGIT == 2 && recount) {
    clear();  // after the search's reads of the recount; its barrier orders this
    __syncthreads();
  }
  uint32_t* hrep = sm.rep + (tid % kSliceReplicas) * kRepStride;
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((key[g][e] >> t.low) == (t.prefix >> t.low))
        atomicAdd(&hrep[(key[g][e] >> kShift) & (kBinsHere - 1)], 1u);
  __syncthreads();
  uint32_t* dst = hist + (DIGIT == 2 ? 2048 : 4096);
  for (int i = tid; i < kBinsHere; i += kThreads) {
    uint32_t n = 0;
#pragma unroll
    for (int r = 0; r < kSliceReplicas; ++r) n += sm.rep[r * kRepStride + i];
    if (n != 0u) atomicAdd(&dst[i], n);
  }
}

// Count table entries of the slice's segments (the same counts as the
// one-workgroup selection writes) and, from the first slice, the threshold.
__device__ __forceinline__ void select_count_slice(const PathParams& p, SliceSmem& sm, int b,
                                                   int h, int sl) {
  const int P = p.tab.len[b] - p.window;
  const int s0 = sl * kSliceKeys;
  if (s0 >= P) return;
  const size_t head = (size_t)(b * p.hkv + h);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t key[2][4];
  load_slice_keys(key, p.pooled + head * p.pooled_stride, P, s0);
  const uint32_t* hist = p.top_hist + head * kSelHistWords;
  const bool recount = p.hist_bad[head] == p.epoch;
  if (tid == 0) sm.sh_lost = 0u;
  const Threshold t = resolve_digits(hist, hist + (recount ? kHistFix : kHistD1), 3,
                                     (uint32_t)(p.budget - p.window), sm);
  const uint32_t tau = t.prefix;  // settled: keep keys >= prefix; else > tau, and `need` == tau
  const int nseg = (P + kSegment - 1) / kSegment;
  uint32_t* table = p.sel_table + head * (size_t)p.table_stride * 2;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    // the wave's counts from ballots of its 64 lanes (scalar popcounts)
    uint32_t above = 0, equal = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = key[g][e];
      above += (uint32_t)__popcll(__ballot(t.settled ? u >= tau : u > tau));
      equal += (uint32_t)__popcll(__ballot(!t.settled && u == tau));
    }
    const int seg = (s0 + g * kSlab) / kSegment + wave;
    if (lane == 0 && seg < nseg) {
      table[2 * seg] = above;
      table[2 * seg + 1] = equal;
    }
  }
  if (sl == 0 && tid == 0) {
    uint32_t* meta = p.sel_meta + head * 4;
    meta[0] = tau;
    meta[1] = t.need;
    meta[2] = t.settled ? 1u : 0u;
    meta[3] = sm.sh_lost;
  }
}

// ---------------------------------------------- one-launch sliced selection ---
// The three sliced passes as one launch (sel_one_launch, when every slice
// workgroup of the call fits the device at once). Each slice workgroup loads
// its keys once and keeps them in registers for every pass. A pass's digit
// histogram is complete once every slice of the head has added its counts
// (agent-scope atomics, performed at the device's coherence point) and
// published that with its flag (publish_item: its atomics acknowledged, a
// barrier, then the flag = the call's epoch). The workgroup then waits for
// the flags of the head's slices (wait_head: bounded) and reads the
// histogram with device-coherent loads. If the wait gives up, the workgroup
// counts that digit over the head's whole prefix itself, in LDS: integer
// counts, so the same histogram and the same threshold. The threshold
// search, the counting and the count table are those of the three kernels.
struct alignas(16) SliceOneSmem {
  uint32_t rep[kRepStride];  // this slice's counts of the digit being counted
  uint32_t own[kRepStride];  // a digit counted over the whole prefix here
  uint32_t rowtot[kWaves];
  uint32_t sh_bin, sh_need, sh_count;
  uint32_t sh_lost;
};

// Four histogram words with device-coherent loads (16-byte aligned).
__device__ __forceinline__ u32x4 load_coherent4(const uint32_t* a) {
  uint64_t* w = const_cast<uint64_t*>(reinterpret_cast<const uint64_t*>(a));
  const uint64_t lo = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(w + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
}

// One more radix digit (bits shift .. of nbins bins) of threshold t from
// that digit's histogram, row(i) giving bins i .. i + 3: the step
// resolve_digits takes for each digit.
template <typename Row, typename Smem>
__device__ __forceinline__ void next_digit(Threshold& t, int shift, int nbins, Row&& row,
                                           Smem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  find_bin(
      [&] {
        const int i = 256 * wave + 4 * lane;
        return i < nbins ? row(i) : u32x4{0u, 0u, 0u, 0u};
      },
      t.need, sm);
  t.prefix |= sm.sh_bin << shift;
  t.need = sm.sh_need;
  t.settled = t.need == sm.sh_count;
  t.low = shift;
}

__device__ __forceinline__ void select_slices_one_launch(const PathParams& p, SliceOneSmem& sm,
                                                         int b, int h, int sl) {
  const int P = p.tab.len[b] - p.window;
  const int s0 = sl * kSliceKeys;
  if (s0 >= P) return;
  const int nsl = (P + kSliceKeys - 1) / kSliceKeys;  // slices of this head that publish
  const size_t head = (size_t)(b * p.hkv + h);
  uint32_t* hist = p.top_hist + head * kSelHistWords;
  const float* src = p.pooled + head * p.pooled_stride;
  uint64_t* flags = p.sel_flags + head * 2 * (size_t)p.sel_slices;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool recount = p.hist_bad[head] == p.epoch;
  uint32_t key[2][4];
  load_slice_keys(key, src, P, s0);
  if (tid == 0) sm.sh_lost = 0u;
  auto clear = [&](uint32_t* h4) {
    for (int i = tid; i < kRepStride / 4; i += kThreads)
      reinterpret_cast<u32x4*>(h4)[i] = u32x4{0u, 0u, 0u, 0u};
  };
  Threshold t{0u, (uint32_t)(p.budget - p.window), 32, false};

  // digit 1: the score kernel's histogram (complete before this launch), or
  // recounted here when that kernel marked it untrustworthy for this call
  if (recount) {
    clear(sm.own);
    __syncthreads();
    for (int a = 0; a < P; a += kSliceKeys) {
      uint32_t k2[2][4];
      load_slice_keys(k2, src, P, a);
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (a + g * kSlab + 4 * tid + e < P) lds_count(sm.own, k2[g][e] >> kTopShift);
    }
    __syncthreads();
    next_digit(t, kTopShift, kBins,
               [&](int i) { return *reinterpret_cast<const u32x4*>(sm.own + i); }, sm);
  } else {
    next_digit(t, kTopShift, kBins,
               [&](int i) { return *reinterpret_cast<const u32x4*>(hist + kHistD1 + i); }, sm);
  }

  // digits 2 and 3 (every workgroup of the head reaches the same `settled`)
#pragma unroll
  for (int d = 2; d <= 3; ++d) {
    if (t.settled) break;
    const int shift = d == 2 ? 10 : 0;
    const int nbins = d == 2 ? 2048 : 1024;
    const uint32_t mask = (uint32_t)nbins - 1u;
    uint32_t* dst = hist + (d == 2 ? kHistD2 : kHistD3);
    clear(sm.rep);
    __syncthreads();
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((key[g][e] >> t.low) == (t.prefix >> t.low))
          atomicAdd(&sm.rep[(key[g][e] >> shift) & mask], 1u);
    __syncthreads();
    for (int i = tid; i < nbins; i += kThreads) {
      const uint32_t n = sm.rep[i];
      if (n != 0u) atomicAdd(&dst[i], n);
    }
    uint64_t* pass_flags = flags + (d - 2) * (size_t)p.sel_slices;
    publish_item(p, pass_flags, sl);
    if (wait_head(p, pass_flags, nsl)) {
      // not every slice has published: this digit over the whole prefix here
      clear(sm.own);
      __syncthreads();
      for (int a = 0; a < P; a += kSliceKeys) {
        uint32_t k2[2][4];
        load_slice_keys(k2, src, P, a);
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if ((k2[g][e] >> t.low) == (t.prefix >> t.low))
              atomicAdd(&sm.own[(k2[g][e] >> shift) & mask], 1u);
      }
      __syncthreads();
      next_digit(t, shift, nbins,
                 [&](int i) { return *reinterpret_cast<const u32x4*>(sm.own + i); }, sm);
    } else {
      next_digit(t, shift, nbins, [&](int i) { return load_coherent4(dst + i); }, sm);
    }
  }

  // count table of this slice's segments, as select_count_slice writes it
  const uint32_t tau = t.prefix;  // settled: keep keys >= prefix; else > tau, and `need` == tau
  const int nseg = (P + kSegment - 1) / kSegment;
  uint32_t* table = p.sel_table + head * (size_t)p.table_stride * 2;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    // the wave's counts from ballots of its 64 lanes (scalar popcounts)
    uint32_t above = 0, equal = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = key[g][e];
      above += (uint32_t)__popcll(__ballot(t.settled ? u >= tau : u > tau));
      equal += (uint32_t)__popcll(__ballot(!t.settled && u == tau));
    }
    const int seg = (s0 + g * kSlab) / kSegment + wave;
    if (lane == 0 && seg < nseg) {
      table[2 * seg] = above;
      table[2 * seg + 1] = equal;
    }
  }
  if (sl == 0 && tid == 0) {
    uint32_t* meta = p.sel_meta + head * 4;
    meta[0] = tau;
    meta[1] = t.need;
    meta[2] = t.settled ? 1u : 0u;
    meta[3] = sm.sh_lost;
  }
}

// Selection of one (prompt, head): the smallest register batch that holds
// the prefix, or batches of kMaxSlabsHeld slabs re-read for longer prefixes.
__device__ __forceinline__ void select_dispatch(const PathParams& p, SelectSmem& sm, int b, int h,
                                                const SelectOut& out) {
  const int P = p.tab.len[b] - p.window;
  const int slabs = (P + kSlab - 1) / kSlab;
  if (slabs <= 1)
    select_head<1, true>(p, sm, b, h, out);
  else if (slabs <= 2)
    select_head<2, true>(p, sm, b, h, out);
  else if (slabs <= 4)
    select_head<4, true>(p, sm, b, h, out);
  else if (slabs <= 8)
    select_head<8, true>(p, sm, b, h, out);
  else if (slabs <= kMaxSlabsHeld)
    select_head<kMaxSlabsHeld, true>(p, sm, b, h, out);
  else
    select_head<kMaxSlabsHeld, false>(p, sm, b, h, out);
}

__device__ __forceinline__ void snapkv_select_item(const PathParams& p, SelectSmem& sm, int b,
                                                   int h) {
  const size_t head = (size_t)(b * p.hkv + h);
  select_dispatch(p, sm, b, h,
                  SelectOut{p.sel_table + head * (size_t)p.table_stride * 2, p.sel_meta + head * 4});
}

}  // namespace snapkv
