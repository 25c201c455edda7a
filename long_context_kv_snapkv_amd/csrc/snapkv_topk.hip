// snapkv_topk: per-head selection of the m = B - W best prefix positions.
//
// The kept set is the m largest pooled scores c_h[j], j < P, ties going to
// the lower position, written in ascending position order and followed by
// the window positions P .. L-1 (glossary page "SnapKV(スナップケーブイ)",
// section "SnapKVの仕組み", step 3: keep the top-budget pairs; paper page
// "SnapKV: LLM Knows What You are Looking for Before Generation", abstract:
// selection is made for each attention head).
//
// One 1024-thread workgroup per (prompt, head). Scores become order-preserving
// 32-bit keys (sign flipped for non-negatives, all bits flipped for
// negatives) and are cached in LDS when the prefix fits (<= 32768). A radix
// select over four 8-bit digits, most significant first, finds the m-th
// largest key tau and how many keys equal to tau are needed; LDS histograms
// use wave-level peeling (lanes sharing a bin add once) because scores pile
// up in few bins. A final ascending pass keeps every key > tau and the first
// `need` keys == tau, compacting positions with wave ballots and mbcnt
// prefixes plus per-wave totals in LDS. Integer-only decisions on the fp32
// bits: the selection is exact given the scores.
#include "snapkv_kernels.h"

namespace snapkv {
namespace {

constexpr int kWaves = kTopkThreads / 64;

__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
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

__global__ void __launch_bounds__(kTopkThreads) snapkv_topk(const TopkParams p) {
  __shared__ uint32_t keys[kTopkLdsKeys];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wtot[2][kWaves];
  __shared__ uint32_t sh_digit, sh_need;

  const int h = blockIdx.x, b = blockIdx.y;
  const int L = p.tab.len[b];
  if (L <= p.budget) return;  // kept whole by the gather
  const int P = L - p.window;
  const int m = p.budget - p.window;  // 1 <= m < P here
  const float* cs = p.pooled + (size_t)(b * p.hkv + h) * p.p_stride;
  int32_t* out = p.out_idx + (size_t)(b * p.hkv + h) * p.budget;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool in_lds = P <= kTopkLdsKeys;

  if (in_lds) {
    for (int j = tid; j < P; j += kTopkThreads) keys[j] = order_key(cs[j]);
  }
  __syncthreads();
  auto key_at = [&](int j) -> uint32_t { return in_lds ? keys[j] : order_key(cs[j]); };

  uint32_t prefix = 0, pmask = 0;
  uint32_t need = (uint32_t)m;  // still to take among keys matching prefix
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (int j0 = 0; j0 < P; j0 += kTopkThreads) {
      const int j = j0 + tid;
      uint32_t u = 0;
      bool act = false;
      if (j < P) {
        u = key_at(j);
        act = (u & pmask) == prefix;
      }
      hist_add(hist, act, (u >> shift) & 255u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns bins 4l .. 4l+3; suffix sums from the top bin down
      const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1];
      const uint32_t c2 = hist[4 * lane + 2], c3 = hist[4 * lane + 3];
      const uint32_t local = c0 + c1 + c2 + c3;
      uint32_t incl = local;  // sum over lanes >= this lane
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_down(incl, off);
        if (lane + off < 64) incl += y;
      }
      const uint32_t above = incl - local;  // keys in higher bins
      if (above < need && need <= incl) {
        uint32_t a = above;
        const uint32_t cnt[4] = {c0, c1, c2, c3};
        int d = 3;
        for (; d > 0; --d) {
          if (a + cnt[d] >= need) break;
          a += cnt[d];
        }
        sh_digit = 4u * lane + d;
        sh_need = need - a;
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    pmask |= 255u << shift;
    need = sh_need;
    __syncthreads();  // sh_* reused next pass
  }
  const uint32_t tau = prefix;  // m-th largest key; `need` keys equal to it are kept

  uint32_t base_eq = 0, base_sel = 0;
  for (int j0 = 0; j0 < P; j0 += kTopkThreads) {
    const int j = j0 + tid;
    uint32_t u = 0;
    const bool valid = j < P;
    if (valid) u = key_at(j);
    const bool gt = valid && u > tau;
    const bool eq = valid && u == tau;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) wtot[0][wave] = (uint32_t)__popcll(beq);
    __syncthreads();
    uint32_t eq_before = 0, eq_all = 0;
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t x = wtot[0][w];
      eq_before += w < wave ? x : 0u;
      eq_all += x;
    }
    const uint32_t eq_rank = base_eq + eq_before + lanes_below(beq);
    const bool sel = gt || (eq && eq_rank < need);
    const uint64_t bsel = __ballot(sel);
    if (lane == 0) wtot[1][wave] = (uint32_t)__popcll(bsel);
    __syncthreads();
    uint32_t sel_before = 0, sel_all = 0;
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t x = wtot[1][w];
      sel_before += w < wave ? x : 0u;
      sel_all += x;
    }
    const uint32_t pos = base_sel + sel_before + lanes_below(bsel);
    if (sel && pos < (uint32_t)m) out[pos] = j;
    base_eq += eq_all;
    base_sel += sel_all;
    __syncthreads();  // wtot reused next block
  }
  for (int i = tid; i < p.window; i += kTopkThreads) out[m + i] = P + i;
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL(snapkv_topk, grid, dim3(kTopkThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace snapkv
