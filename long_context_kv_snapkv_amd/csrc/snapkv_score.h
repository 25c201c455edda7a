// snapkv_score: the observation-window vote of SnapKV, as work items.
//
// For KV head h of prompt b (length L, prefix P = L - W) the R = G*W window
// rows (query head h*G + g, window row i, absolute position P + i) are scored
// against the prompt's keys with a causal softmax at scale 1/sqrt(D), and the
// probabilities of each prefix key are summed over all R rows:
//   s_h[j] = sum_r exp(l_rj - lse_r),  l_rj = q_r . k_j / sqrt(D),  j < P,
//   lse_r  = log sum_{j' <= P + i(r)} exp(l_rj').
// (Glossary page "SnapKV(スナップケーブイ)", section "SnapKVの仕組み": the
// window tokens' per-head attention scores are aggregated; FAQ Q1: GQA.)
//
// Every row's normaliser must be known before a column can be summed, so the
// keys are visited twice, each time as a bf16 MFMA contraction Q_win . K^T
// with fp32 accumulation (v_mfma_f32_32x32x16_bf16):
//   stats item (chunk c): per row, the maximum and the sum of 2^(x - max)
//        over the chunk's visible keys, x = l * log2(e); C = K . Q^T so a lane
//        owns one row and the statistics are in-lane online reductions;
//   vote item (chunk c): combines the partials of all chunks of the head into
//        lse_r, recomputes its logits as C = Q . K^T so a lane owns one key,
//        and column-sums 2^(x - lse) over the rows (in-lane over 16 rows, then
//        across the two lane halves and the row-tile waves through LDS).
// Keys stream through two 128-key LDS tiles with two more tiles in flight in
// registers; the group's query rows stay in VGPRs as MFMA operands.
//
// snapkv_pool is fused into the vote item: the item also computes the votes
// of the r = k/2 keys beyond each end of its chunk (the same values the
// neighbouring items compute: same keys, same operation order), pools its
// own positions from LDS and writes only pooled scores. It also counts its
// pooled keys' top 11 bits (the selection's first radix digit) into the
// head's histogram.
// All reductions run in a fixed order, so results are bitwise reproducible
// and independent of which workgroup runs an item.
#pragma once

#include "snapkv_device.h"

namespace snapkv {

template <int D>
struct alignas(16) StatsSmem {
  unsigned char ring[2][KTile<D>::BYTES];
  float2 wstats[kWaves][kMaxRowTilesPerWave * 32];
};

template <int D>
struct alignas(16) VoteSmem {
  unsigned char ring[2][KTile<D>::BYTES];
  float lse[kMaxRows];
  float vred[2][kWaves][KTile<D>::KEYS];
  float s_chunk[kMaxChunk + kMaxKernel];  // the chunk plus its pooling halo
  uint32_t top[kTopBins];                 // top-digit histogram of this chunk's pooled keys
};

// Which row tiles and key blocks a wave owns: waves split the row tiles
// (nwr of them, a power of two), and the key blocks of a tile when there
// are fewer row tiles than waves.
struct WaveRole {
  int nwr, nwk, wr, wk, my_nrt;
};

__device__ __forceinline__ WaveRole wave_role(const PathParams& p, int wave) {
  WaveRole r;
  const int nrt = p.rows_pad >> 5;
  r.nwr = p.nwr;
  r.nwk = kWaves / p.nwr;
  r.wr = wave % r.nwr;
  r.wk = wave / r.nwr;
  r.my_nrt = (nrt - r.wr + r.nwr - 1) / r.nwr;
  return r;
}

// Pooled value at position j from an accessor get(u), 0 <= u < P:
//   avg: (1/k) * sum_{|u-j| <= r} s[u]   (u outside [0, P) adds 0)
//   max: max_{|u-j| <= r, 0 <= u < P} s[u]
// with r = k / 2 (glossary page "SnapKV(スナップケーブイ)", section
// "SnapKVの仕組み", paragraph "Pooling for Robustness"; paper page "SnapKV:
// LLM Knows What You are Looking for Before Generation", section
// "기술적 접근법": max or average pooling, kernel 5-13; kernel 1 leaves the
// scores as they are). The operation order is fixed here, so every kernel
// that pools produces identical bits.
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

// ---------------------------------------------------------------- stats ---
template <int D, int RTW>
__device__ __forceinline__ void snapkv_score_stats_item(const PathParams& p, StatsSmem<D>& sm, int b, int h,
                                        int c) {
  const int L = p.tab.len[b];
  const int P = L - p.window;
  const int key0 = c * p.chunk;
  const int kend = min(key0 + p.chunk, L);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const WaveRole role = wave_role(p, wave);

  bf16x8 qf[RTW][D / 16];
  const uint16_t* qbase = p.q + (size_t)(b * p.hq + h * p.group) * p.window * D;
  load_query_frags<D, RTW>(qf, qbase, p.rows, role.wr, role.nwr, role.my_nrt, lane);
  asm volatile("" ::: "memory");  // query loads stay older than the key-tile loads

  int lim[RTW];  // last key visible to this lane's row
  float mrun[RTW], srun[RTW];
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    const int r = (role.wr + role.nwr * t) * 32 + (lane & 31);
    lim[t] = (t < role.my_nrt && r < p.rows) ? P + r % p.window : -1;
    mrun[t] = -kInf;
    srun[t] = 0.f;
  }
  const float scale = p.scale_log2;
  const int full_end = min(P, kend);  // keys below this are visible to every row

  const size_t tstride = (size_t)p.hkv * D;
  const uint16_t* kbase = p.k + ((size_t)p.tab.off[b] * p.hkv + h) * D;
  auto compute = [&](const unsigned char* tile, int i) {
    const int tk0 = key0 + i * KTile<D>::KEYS;
    for (int kb = role.wk; kb < KTile<D>::KEYS / 32; kb += role.nwk) {
      const int bk0 = tk0 + kb * 32;
      if (bk0 >= kend) break;
      bf16x8 kf[D / 16];
      read_key_frags<D>(kf, tile, kb, lane);
      const bool full = bk0 + 32 <= full_end;
#pragma unroll
      for (int t = 0; t < RTW; ++t) {
        if (t >= role.my_nrt) break;
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[t][s], acc, 0, 0, 0);
        // acc[v]: logit of key bk0 + acc_row(v, lane) for this lane's row
        if (!full) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int j = bk0 + acc_row(v, lane);
            if (j > lim[t] || j >= kend) acc[v] = -kInf;
          }
        }
        float mx = -kInf;
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, acc[v]);
        const float mnew = fmaxf(mrun[t], mx * scale);
        if (mnew != -kInf) {
          float sum = 0.f;
#pragma unroll
          for (int v = 0; v < 16; ++v) sum += exp2_fast(fmaf(acc[v], scale, -mnew));
          srun[t] = srun[t] * exp2_fast(mrun[t] - mnew) + sum;
          mrun[t] = mnew;
        }
      }
    }
  };
  stream_key_tiles<D>(kbase, tstride, key0, kend, sm.ring, compute, [](int) {});

  // lanes l and l^32 hold the same row over different keys
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    const float mo = __shfl_xor(mrun[t], 32);
    const float so = __shfl_xor(srun[t], 32);
    lse_merge(mrun[t], srun[t], mo, so);
    if (lane < 32 && t < role.my_nrt) sm.wstats[wave][t * 32 + lane] = make_float2(mrun[t], srun[t]);
  }
  __syncthreads();
  float2* dst = p.part + ((size_t)(b * p.hkv + h) * p.nchunk + c) * p.rows_pad;
  if (c == 0) {  // the vote items of this head accumulate into it next
    uint32_t* top = p.top_hist + (size_t)(b * p.hkv + h) * kTopBins;
    for (int i = tid; i < kTopBins; i += kThreads) top[i] = 0u;
  }
  for (int r = tid; r < p.rows; r += kThreads) {
    const int rt = r >> 5, owner = rt % role.nwr, t = rt / role.nwr;
    float m = -kInf, s = 0.f;
    for (int q = 0; q < role.nwk; ++q) {
      const float2 e = sm.wstats[owner + role.nwr * q][t * 32 + (r & 31)];
      lse_merge(m, s, e.x, e.y);
    }
    dst[r] = make_float2(m, s);
  }
  __syncthreads();  // LDS is reused by the next item
}

// ----------------------------------------------------------------- vote ---
template <int D, int RTW>
__device__ __forceinline__ void snapkv_score_vote_item(const PathParams& p, VoteSmem<D>& sm, int b, int h,
                                       int c) {
  const int L = p.tab.len[b];
  const int P = L - p.window;
  const int key0 = c * p.chunk;
  const int kend = min(key0 + p.chunk, P);
  // the votes of r keys on each side are recomputed so this item can pool
  // its own positions (identical values: same keys, same operation order)
  const int r = p.kernel >> 1;
  const int kv0 = max(0, key0 - r), kv1 = min(P, kend + r);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const WaveRole role = wave_role(p, wave);

  for (int i = tid; i < kTopBins; i += kThreads) sm.top[i] = 0u;

  // lse of every row from the per-chunk statistics: `tpr` threads share a
  // row, each merging every tpr-th chunk, then a fixed-order fold in LDS
  {
    const int nch = (L + p.chunk - 1) / p.chunk;
    const float2* part = p.part + (size_t)(b * p.hkv + h) * p.nchunk * p.rows_pad;
    float2* scratch = reinterpret_cast<float2*>(&sm.vred[0][0][0]);  // kThreads float2
    int tpr = 1;
    while (tpr * 2 * p.rows_pad <= kThreads) tpr *= 2;
    const int span = kThreads / tpr;  // rows per round (>= rows_pad)
    const int r = tid % span, sub = tid / span;
    float m = -kInf, s = 0.f;
    if (r < p.rows) {
#pragma unroll 4
      for (int cc = sub; cc < nch; cc += tpr) m = fmaxf(m, part[(size_t)cc * p.rows_pad + r].x);
      if (m != -kInf) {  // a chunk subset may see none of this row's keys
#pragma unroll 4
        for (int cc = sub; cc < nch; cc += tpr) {
          const float2 e = part[(size_t)cc * p.rows_pad + r];
          s += e.y * exp2_fast(e.x - m);
        }
      }
    }
    scratch[tid] = make_float2(m, s);
    __syncthreads();
    if (tid < p.rows_pad) {
      float mm = -kInf, ss = 0.f;
      for (int q = 0; q < tpr; ++q) {
        const float2 e = scratch[q * span + tid];
        lse_merge(mm, ss, e.x, e.y);
      }
      sm.lse[tid] = tid < p.rows ? mm + log2f(ss) : kInf;  // padded rows add 0
    }
    __syncthreads();
  }

  bf16x8 qf[RTW][D / 16];
  const uint16_t* qbase = p.q + (size_t)(b * p.hq + h * p.group) * p.window * D;
  load_query_frags<D, RTW>(qf, qbase, p.rows, role.wr, role.nwr, role.my_nrt, lane);
  asm volatile("" ::: "memory");  // query loads stay older than the key-tile loads
  float lr[RTW][16];
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    const int rt = role.wr + role.nwr * t;
#pragma unroll
    for (int v = 0; v < 16; ++v)
      lr[t][v] = t < role.my_nrt ? sm.lse[min(rt * 32 + acc_row(v, lane), kMaxRows - 1)] : kInf;
  }
  const float scale = p.scale_log2;

  constexpr int KEYS = KTile<D>::KEYS;
  const size_t tstride = (size_t)p.hkv * D;
  const uint16_t* kbase = p.k + ((size_t)p.tab.off[b] * p.hkv + h) * D;
  const int ntiles = (kv1 - kv0 + KEYS - 1) / KEYS;
  // fold tile i's row-tile partials (written before the barrier that
  // precedes tile i + 1) in a fixed order
  auto fold = [&](int i) {
    for (int kk = tid; kk < KEYS; kk += kThreads) {
      float s = 0.f;
      for (int q = 0; q < role.nwr; ++q) s += sm.vred[i & 1][q][kk];
      sm.s_chunk[i * KEYS + kk] = s;
    }
  };
  auto compute = [&](const unsigned char* tile, int i) {
    const int tk0 = kv0 + i * KEYS;
    for (int kb = role.wk; kb < KEYS / 32; kb += role.nwk) {
      if (tk0 + kb * 32 >= kv1) break;
      bf16x8 kf[D / 16];
      read_key_frags<D>(kf, tile, kb, lane);
      float cs = 0.f;
#pragma unroll
      for (int t = 0; t < RTW; ++t) {
        if (t >= role.my_nrt) break;
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[t][s], kf[s], acc, 0, 0, 0);
        // acc[v]: logit of row acc_row(v, lane) for key tk0 + kb*32 + (lane & 31)
#pragma unroll
        for (int v = 0; v < 16; ++v) cs += exp2_fast(fmaf(acc[v], scale, -lr[t][v]));
      }
      cs += __shfl_xor(cs, 32);
      if (lane < 32) sm.vred[i & 1][role.wr][kb * 32 + lane] = cs;
    }
  };
  stream_key_tiles<D>(kbase, tstride, kv0, kv1, sm.ring, compute, [&](int i) {
    if (i > 0) fold(i - 1);
  });
  __syncthreads();
  fold(ntiles - 1);
  __syncthreads();
  // snapkv_pool, staged in LDS: pooled scores of this item's positions
  const size_t head = (size_t)(b * p.hkv + h);
  float* pooled = p.pooled + head * p.pooled_stride;
  for (int j = key0 + tid; j < kend; j += kThreads) {
    const float c_j = pool_value([&](int u) { return sm.s_chunk[u - kv0]; }, j, P, p.kernel,
                                 p.pool_mode);
    pooled[j] = c_j;
    if (!p.export_scores) atomicAdd(&sm.top[order_key(c_j) >> kTopShift], 1u);
  }
  if (!p.export_scores) {
    // the selection's first radix digit: this chunk's counts join the head's
    // histogram (few distinct bins per chunk, so few global atomics)
    __syncthreads();
    uint32_t* top = p.top_hist + head * kTopBins;
    for (int i = tid; i < kTopBins; i += kThreads) {
      const uint32_t n = sm.top[i];
      if (n != 0u) atomicAdd(&top[i], n);
    }
  }
  __syncthreads();  // LDS is reused next
}

}  // namespace snapkv
