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
//   stats item (chunk c): per row, a reference m (a block maximum, moved up
//        only when a later logit exceeds it by more than 64) and the sum of
//        2^(x - m) over the chunk's visible keys, x = l * log2(e); C = K . Q^T
//        so a lane owns one row and the statistics are in-lane reductions;
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
  // column partials per (row-tile wave, lane half), three tiles deep: a
  // tile's last block may be summed while the next tile is processed
  float vred[3][2 * kWaves][KTile<D>::KEYS];
  float vdummy[kThreads];  // destination of the pipeline's empty first slot
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

// The MFMA chains of a group are all issued before the softmax arithmetic
// that consumes them, so the matrix core works on the later chains while
// the VALU works on the first: with one row tile per wave a group is two of
// the wave's key blocks, with two row tiles it is one key block (two chains
// either way, within the register budget).
template <int RTW>
struct KeyGroup {
  static constexpr int G = RTW == 1 ? 2 : 1;  // key blocks per group
  int kb[G];
  bool has[G];
  __device__ __forceinline__ KeyGroup(int kb0, int nwk, int tk0, int kend, int keys) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      kb[g] = kb0 + g * nwk;
      has[g] = g == 0 || (kb[g] < keys / 32 && tk0 + kb[g] * 32 < kend);
    }
  }
};

// ---------------------------------------------------------------- stats ---
// The statistics pass of one item. `qbuf` (one tile of LDS) stages the query
// rows, `wstats` collects the waves' row statistics, and run(ks, compute)
// streams the chunk's key tiles (through a ring, or into resident slots for
// the fused kernel). The query fragments are left in `qf`. With COHERENT the
// statistics and the histogram clearing are written with device-coherent
// stores (another workgroup of the same kernel reads them). Item 0 of a head
// clears the head's selection histograms unless CLEAR is false (an item
// recomputing another item's statistics leaves that to the owner).
template <int D, int RTW, bool COHERENT, bool DEEP = false, bool CLEAR = true, bool PIPE = true,
          typename Run>
__device__ __forceinline__ void score_stats_body(const PathParams& p, unsigned char* qbuf,
                                                 float2 (*wstats)[kMaxRowTilesPerWave * 32],
                                                 bf16x8 (&qf)[RTW][D / 16], Run&& run, int b,
                                                 int h, int c) {
  const int L = p.tab.len[b];
  const int P = L - p.window;
  const int key0 = c * p.chunk;
  const int kend = min(key0 + p.chunk, L);
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const WaveRole role = wave_role(p, wave);

  // last tile first: the vote item of the same chunk (same workgroup index,
  // so the same XCD) starts with the tiles this item read last, which are
  // then the most likely to still be in that XCD's L2
  KeyStream<D> ks{{}, {}, p.k + ((size_t)p.tab.off[b] * p.hkv + h) * D, (size_t)p.hkv * D,
                  key0, kend, true, DEEP};
  stage_query_frags<D, RTW>(qf, p.q + (size_t)(b * p.hq + h * p.group) * p.window * D, p.rows,
                            p.rows_pad, role.wr, role.nwr, role.my_nrt, qbuf,
                            [&] { ks.prefetch(); });

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

  // online (max, sum) update of row tile t with block logits acc (keys bk0 + m)
  auto update = [&](f32x16 acc, int t, int bk0) {
    if (bk0 + 32 > full_end) {
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
  };
  // A block every row sees in full. The first block of a row sets its
  // reference to the block maximum; later blocks are summed against the
  // reference directly, without a maximum: the pair (m, s) stands for
  // m + log2(s) whichever m it holds, and a term 2^(x - m) stays finite and
  // exact to rounding as long as x - m <= 64 (checked on the block sum, which
  // bounds every term). Terms far below the reference are at most what the
  // first block's own term (exactly 1) leaves below rounding. A block with a
  // logit more than 64 above the reference, or the first block, takes the
  // maximum path, which moves the reference up.
  auto update_max = [&](const f32x16& acc, int t) {
    float mx0 = fmaxf(acc[0], acc[1]), mx1 = fmaxf(acc[2], acc[3]);
#pragma unroll
    for (int v = 4; v < 16; v += 4) {
      mx0 = fmaxf(mx0, fmaxf(acc[v], acc[v + 1]));
      mx1 = fmaxf(mx1, fmaxf(acc[v + 2], acc[v + 3]));
    }
    const float mnew = fmaxf(mrun[t], fmaxf(mx0, mx1) * scale);
    const float mref = mnew == -kInf ? 0.f : mnew;  // an all -inf block changes nothing
    // the first terms start the sums (0 + e is e exactly for every value
    // exp2 returns, so no add of zero is issued)
    float s0 = exp2_fast(fmaf(acc[0], scale, -mref)), s1 = exp2_fast(fmaf(acc[1], scale, -mref));
#pragma unroll
    for (int v = 2; v < 16; v += 2) {
      s0 += exp2_fast(fmaf(acc[v], scale, -mref));
      s1 += exp2_fast(fmaf(acc[v + 1], scale, -mref));
    }
    srun[t] = fmaf(srun[t], exp2_fast(mrun[t] - mref), s0 + s1);
    mrun[t] = mnew;
  };
  constexpr float kBlockSumCap = 0x1p64f;
  // The direct sum is computed unconditionally, so it can interleave with
  // the MFMA chain of the next block; with no reference yet (m = -inf) it is
  // +inf or NaN and the block falls to the maximum path.
  auto direct_sum = [&](const f32x16& acc, int t) {
    const float m = mrun[t];
    float s4[4];  // short dependent add chains, started by their first terms
#pragma unroll
    for (int v = 0; v < 4; ++v) s4[v] = exp2_fast(fmaf(acc[v], scale, -m));
#pragma unroll
    for (int v = 4; v < 16; ++v) s4[v & 3] += exp2_fast(fmaf(acc[v], scale, -m));
    return (s4[0] + s4[1]) + (s4[2] + s4[3]);
  };
  auto retire = [&](const f32x16& acc, int t, float sb) {
    const bool ok = sb <= kBlockSumCap;  // false for +inf and NaN too
    srun[t] = ok ? srun[t] + sb : srun[t];
    if (!ok) update_max(acc, t);
  };
  auto update_full = [&](const f32x16& acc, int t) { retire(acc, t, direct_sum(acc, t)); };
  // the MFMA chains of one key block for every row tile of this wave; the
  // row tiles' chains alternate, k-step by k-step, so each key fragment is
  // dead after its RTW uses (each chain sums its k-steps in the same order)
  auto chain_block = [&](f32x16 (&acc)[RTW], const bf16x8 (&kf)[D / 16]) {
#pragma unroll
    for (int t = 0; t < RTW; ++t) acc[t] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int t = 0; t < RTW; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[t][s], acc[t], 0, 0, 0);
  };
  // Software pipeline over this wave's key blocks: the MFMA chains of block
  // n are issued, then the update of block n - 1 runs while they execute.
  // Blocks go in pairs whose accumulators take turns as the pending one, so
  // nothing is copied between them. Tiles whose keys are all visible to
  // every row take this path; the tile that reaches the window or the chunk
  // end flushes the pending block and is processed with masking.
  f32x16 pacc[RTW];  // pending block (all -inf: nothing pending)
#pragma unroll
  for (int t = 0; t < RTW; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) pacc[t][v] = -kInf;
  auto compute = [&](const unsigned char* tile, int i) {
    const int tk0 = ks.tile_key(i);
    if (RTW > 1 && !PIPE && tk0 + KTile<D>::KEYS <= full_end) {
      // the same blocks in the same order, each retired right after its
      // chains (fewer registers: for the rarely taken recomputation)
#pragma unroll
      for (int t = 0; t < RTW; ++t) update_full(pacc[t], t);
      for (int kb = role.wk; kb < KTile<D>::KEYS / 32; kb += role.nwk) {
        f32x16 acc[RTW];
        bf16x8 kf[D / 16];
        read_key_frags<D>(kf, tile, kb, lane);
        chain_block(acc, kf);
#pragma unroll
        for (int t = 0; t < RTW; ++t) update_full(acc[t], t);
      }
#pragma unroll
      for (int t = 0; t < RTW; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) pacc[t][v] = -kInf;
    } else if (RTW > 1 && role.nwk == 1 && tk0 + KTile<D>::KEYS <= full_end) {
      // Two row tiles, and every wave visits every key block (nwk == 1).
      // The chains of block kb are issued interleaved with the direct sums
      // of the pending block (kb - 1, across tiles too), so one wave keeps
      // both the matrix core and the VALU busy; the pending block is retired
      // (its rare maximum path included) once the chains are issued. The
      // pairs' accumulators take turns as the pending one.
#pragma unroll
      for (int kb = 0; kb < KTile<D>::KEYS / 32; kb += 2) {
        f32x16 acc[RTW];
        float sb[RTW];
        {
          pin_here(pacc);
          bf16x8 kf[D / 16];
          read_key_frags<D, false>(kf, tile, kb, lane);
          chain_block(acc, kf);
#pragma unroll
          for (int t = 0; t < RTW; ++t) sb[t] = direct_sum(pacc[t], t);
          interleave_mfma_valu<D / 16, RTW>();
          pin_here(sb);
        }
#pragma unroll
        for (int t = 0; t < RTW; ++t) retire(pacc[t], t, sb[t]);
        {
          pin_here(acc);
          bf16x8 kf[D / 16];
          read_key_frags<D, false>(kf, tile, kb + 1, lane);
          chain_block(pacc, kf);
#pragma unroll
          for (int t = 0; t < RTW; ++t) sb[t] = direct_sum(acc[t], t);
          interleave_mfma_valu<D / 16, RTW>();
          pin_here(sb);
        }
#pragma unroll
        for (int t = 0; t < RTW; ++t) retire(acc[t], t, sb[t]);
      }
    } else if (tk0 + KTile<D>::KEYS <= full_end) {
      for (int kb = role.wk; kb < KTile<D>::KEYS / 32; kb += 2 * role.nwk) {
        f32x16 acc[RTW];
        {
          bf16x8 kf[D / 16];
          read_key_frags<D>(kf, tile, kb, lane);
          chain_block(acc, kf);
        }
#pragma unroll
        for (int t = 0; t < RTW; ++t) update_full(pacc[t], t);
        if (kb + role.nwk < KTile<D>::KEYS / 32) {
          bf16x8 kf[D / 16];
          read_key_frags<D>(kf, tile, kb + role.nwk, lane);
          chain_block(pacc, kf);
#pragma unroll
          for (int t = 0; t < RTW; ++t) update_full(acc[t], t);
        } else {
#pragma unroll
          for (int t = 0; t < RTW; ++t) pacc[t] = acc[t];
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < RTW; ++t) {
        update_full(pacc[t], t);
#pragma unroll
        for (int v = 0; v < 16; ++v) pacc[t][v] = -kInf;
      }
      for (int kb = role.wk; kb < KTile<D>::KEYS / 32; kb += role.nwk) {
        const int bk0 = tk0 + kb * 32;
        if (bk0 >= kend) break;
        bf16x8 kf[D / 16];
        read_key_frags<D>(kf, tile, kb, lane);
#pragma unroll
        for (int t = 0; t < RTW; ++t) {
          f32x16 acc = {};
#pragma unroll
          for (int s = 0; s < D / 16; ++s)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[t][s], acc, 0, 0, 0);
          update(acc, t, bk0);
        }
      }
    }
  };
  run(ks, compute);
#pragma unroll
  for (int t = 0; t < RTW; ++t) update_full(pacc[t], t);

  // lanes l and l^32 hold the same row over different keys: the lower
  // half's pair merged with the upper half's
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    const float2 mh = halves32(mrun[t]), sh = halves32(srun[t]);
    float mm = mh.x, ss = sh.x;
    lse_merge(mm, ss, mh.y, sh.y);
    if (lane < 32 && t < role.my_nrt) wstats[wave][t * 32 + lane] = make_float2(mm, ss);
  }
  __syncthreads();
  float2* dst = p.part + ((size_t)(b * p.hkv + h) * p.nchunk + c) * p.rows_pad;
  if (CLEAR && c == 0) {  // the vote items (digit 1) and a sliced selection (digits 2, 3) add to these
    uint32_t* top = p.top_hist + (size_t)(b * p.hkv + h) * kSelHistWords;
    for (int i = tid; i < kHistCleared; i += kThreads) {
      if constexpr (COHERENT)
        __hip_atomic_store(&top[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        top[i] = 0u;
    }
  }
  for (int r = tid; r < p.rows; r += kThreads) {
    const int rt = r >> 5, owner = rt % role.nwr, t = rt / role.nwr;
    float m = -kInf, s = 0.f;
    for (int q = 0; q < role.nwk; ++q) {
      const float2 e = wstats[owner + role.nwr * q][t * 32 + (r & 31)];
      lse_merge(m, s, e.x, e.y);
    }
    if constexpr (COHERENT)
      __hip_atomic_store(reinterpret_cast<uint64_t*>(&dst[r]),
                         __builtin_bit_cast(uint64_t, make_float2(m, s)), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    else
      dst[r] = make_float2(m, s);
  }
}

template <int D, int RTW>
__device__ __forceinline__ void snapkv_score_stats_item(const PathParams& p, StatsSmem<D>& sm,
                                                        int b, int h, int c) {
  bf16x8 qf[RTW][D / 16];
  score_stats_body<D, RTW, false, true>(
      p, sm.ring[1], sm.wstats, qf,
      [&](KeyStream<D>& ks, auto&& compute) { ks.run(sm.ring, compute, [](int) {}); }, b, h, c);
}

// ----------------------------------------------------------------- vote ---
// Loads are issued in the order the item needs them to be complete: first
// the row normalisers' inputs (the first kPartBatch per-chunk statistics per
// thread, or with EXT_LSE the caller's log-sum-exp of each row), then the
// query rows and the first key tile. The lse computation then waits only
// for its own inputs while the rest is still in flight.
constexpr int kPartBatch = 8;

// The head's first-digit histogram may hold counts added before item 0 of
// the head cleared it (an item gave up waiting for item 0's flag): the
// selection of this call recounts that digit itself (plain store; the
// selection runs after a kernel boundary).
__device__ __forceinline__ void mark_hist_bad(const PathParams& p, size_t head) {
  if (threadIdx.x == 0) p.hist_bad[head] = p.epoch;
}

// Per-chunk statistics of one row, with a device-coherent load when another
// workgroup of the same kernel wrote them (COHERENT).
template <bool COHERENT>
__device__ __forceinline__ float2 load_part(const float2* a) {
  if constexpr (COHERENT)
    return __builtin_bit_cast(
        float2, __hip_atomic_load(const_cast<uint64_t*>(reinterpret_cast<const uint64_t*>(a)),
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  else
    return *a;
}

// With ZERO_FIRST (normalisers from the caller, every item resident at
// once) the item also stands in for the histogram clearing: item 0 of a head
// clears the head's selection histograms with device-coherent stores and
// publishes its flag, and every item checks that flag (bounded wait) before
// adding its counts.
template <int D, int RTW, bool EXT_LSE, bool COHERENT = false, bool ZERO_FIRST = false>
__device__ __forceinline__ void snapkv_score_vote_item(const PathParams& p, VoteSmem<D>& sm,
                                                       int b, int h, int c) {
  const int L = p.tab.len[b];
  const int P = L - p.window;
  const int key0 = c * p.chunk;
  const int kend = min(key0 + p.chunk, P);
  // the votes of r keys on each side are recomputed so this item can pool
  // its own positions (identical values: same keys, same operation order)
  const int r = p.kernel >> 1;
  const int kv0 = max(0, key0 - r), kv1 = min(P, kend + r);
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const WaveRole role = wave_role(p, wave);

  // statistics of row `row`, chunks sub, sub + tpr, ...: the first batch
  const int nch = (L + p.chunk - 1) / p.chunk;
  const float2* part = p.part + (size_t)(b * p.hkv + h) * p.nchunk * p.rows_pad;
  int tpr = 1;
  while (tpr * 2 * p.rows_pad <= kThreads) tpr *= 2;
  const int span = kThreads / tpr;  // rows per round (>= rows_pad)
  const int row = tid % span, sub = tid / span;
  const bool row_ok = row < p.rows;
  const int row_c = min(row, p.rows - 1);
  float2 pe[EXT_LSE ? 1 : kPartBatch];
  float ext = 0.f;
  if (EXT_LSE) {
    // the group's rows are consecutive in [batch, H_q, W]
    ext = p.window_lse[(size_t)(b * p.hq + h * p.group) * p.window + min(tid, p.rows - 1)];
  } else {
#pragma unroll
    for (int u = 0; u < kPartBatch; ++u)
      pe[u] = load_part<COHERENT>(&part[(size_t)min(sub + u * tpr, nch - 1) * p.rows_pad + row_c]);
  }
  asm volatile("" ::: "memory");  // these loads stay older than the rest

  bf16x8 qf[RTW][D / 16];
  KeyStream<D> ks{{}, {}, p.k + ((size_t)p.tab.off[b] * p.hkv + h) * D, (size_t)p.hkv * D,
                  kv0, kv1};
  stage_query_frags<D, RTW>(qf, p.q + (size_t)(b * p.hq + h * p.group) * p.window * D, p.rows,
                            p.rows_pad, role.wr, role.nwr, role.my_nrt, sm.ring[1],
                            [&] { ks.prefetch(); });

  for (int i = tid; i < kTopBins; i += kThreads) sm.top[i] = 0u;
  if constexpr (ZERO_FIRST) {
    if (c == 0) {
      const size_t head0 = (size_t)(b * p.hkv + h);
      uint32_t* top = p.top_hist + head0 * kSelHistWords;
      for (int i = tid; i < kHistCleared; i += kThreads)
        __hip_atomic_store(&top[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      publish_item(p, p.flags + head0 * p.nchunk, 0);
    }
  }
  if (EXT_LSE) {
    // natural-log normaliser -> log2 units of the scaled logits
    if (tid < p.rows_pad) sm.lse[tid] = tid < p.rows ? ext * 1.4426950408889634f : kInf;
    lds_barrier();
  } else {
    // lse of every row: `tpr` threads share a row, each merging every tpr-th
    // chunk (max first, then the rescaled sum), then a fixed-order fold in LDS
    float m = -kInf, s = 0.f;
#pragma unroll
    for (int u = 0; u < kPartBatch; ++u)
      if (sub + u * tpr < nch) m = fmaxf(m, pe[u].x);
    if (m != -kInf) {  // a chunk subset may see none of this row's keys
#pragma unroll
      for (int u = 0; u < kPartBatch; ++u)
        if (sub + u * tpr < nch) s += pe[u].y * exp2_fast(pe[u].x - m);
    }
    // more chunks (long prompts): merged one by one in chunk order, their
    // loads issued kPartBatch at a time
    for (int c0 = sub + kPartBatch * tpr; c0 < nch; c0 += kPartBatch * tpr) {
      float2 e[kPartBatch];
#pragma unroll
      for (int u = 0; u < kPartBatch; ++u)
        e[u] = load_part<COHERENT>(&part[(size_t)min(c0 + u * tpr, nch - 1) * p.rows_pad + row_c]);
#pragma unroll
      for (int u = 0; u < kPartBatch; ++u)
        if (c0 + u * tpr < nch) lse_merge(m, s, e[u].x, e[u].y);
    }
    float2* scratch = reinterpret_cast<float2*>(&sm.vred[0][0][0]);  // kThreads float2
    scratch[tid] = row_ok ? make_float2(m, s) : make_float2(-kInf, 0.f);
    lds_barrier();
    if (tid < p.rows_pad) {
      float mm = -kInf, ss = 0.f;
      for (int q = 0; q < tpr; ++q) {
        const float2 e = scratch[q * span + tid];
        lse_merge(mm, ss, e.x, e.y);
      }
      sm.lse[tid] = tid < p.rows ? mm + log2f(ss) : kInf;  // padded rows add 0
    }
    lds_barrier();
  }
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
  const int ntiles = (kv1 - kv0 + KEYS - 1) / KEYS;
  const int nparts = 2 * role.nwr;  // (row-tile wave, lane half) partial sums per key
  // fold tile i's partials in a fixed order; they are complete once the
  // barrier that precedes tile i + 2 has passed (a tile's last block may be
  // summed during the next tile)
  auto fold = [&](int i) {
    for (int kk = tid; kk < KEYS; kk += kThreads) {
      float s = 0.f;
      for (int q = 0; q < nparts; ++q) s += sm.vred[i % 3][q][kk];
      sm.s_chunk[i * KEYS + kk] = s;
    }
  };
  // column sums over this wave's rows of block kb (keys tk0 + kb*32 + lane%32):
  // lanes l and l + 32 hold different rows of the same key, so each half
  // writes its own partial. Four partial sums keep the dependent add chains
  // short; every key of a wave is summed in this same order on every path,
  // so equal columns give equal votes.
  // The first four terms start the partial sums: 0 + e is e exactly for
  // every value exp2 returns, so this equals summing into zeros.
  auto colsum = [&](const f32x16(&acc)[RTW]) {
    if (role.my_nrt < 1) return 0.f;
    float c4[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) c4[v] = exp2_fast(fmaf(acc[0][v], scale, -lr[0][v]));
#pragma unroll
    for (int v = 4; v < 16; ++v) c4[v & 3] += exp2_fast(fmaf(acc[0][v], scale, -lr[0][v]));
#pragma unroll
    for (int t = 1; t < RTW; ++t) {
      if (t >= role.my_nrt) break;
#pragma unroll
      for (int v = 0; v < 16; ++v) c4[v & 3] += exp2_fast(fmaf(acc[t][v], scale, -lr[t][v]));
    }
    return (c4[0] + c4[1]) + (c4[2] + c4[3]);
  };
  // Two row tiles per wave, every wave visiting every key block: the
  // chains of block kb are issued interleaved with the column sums of the
  // pending block (kb - 1, across tiles too), whose partial is stored once
  // they are done. vacc holds the pending block's logits, vdst where its
  // partial goes (at first a dummy slot, with -inf logits that sum to 0).
  f32x16 vacc[RTW];
#pragma unroll
  for (int t = 0; t < RTW; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) vacc[t][v] = -kInf;
  float* vdst = &sm.vdummy[tid];
  auto flush_pending = [&] {
    if constexpr (RTW > 1) {
      *vdst = colsum(vacc);
#pragma unroll
      for (int t = 0; t < RTW; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) vacc[t][v] = -kInf;
      vdst = &sm.vdummy[tid];
    }
  };
  auto compute = [&](const unsigned char* tile, int i) {
    const int tk0 = kv0 + i * KEYS;
    float* vr = &sm.vred[i % 3][2 * role.wr + (lane >> 5)][lane & 31];
    constexpr int GB = KeyGroup<RTW>::G;
    if (RTW > 1 && role.nwk == 1 && tk0 + KEYS <= kv1 && role.my_nrt == RTW) {
      auto chain = [&](f32x16 (&acc)[RTW], const bf16x8 (&kf)[D / 16]) {
#pragma unroll
        for (int t = 0; t < RTW; ++t) acc[t] = f32x16{};
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
#pragma unroll
          for (int t = 0; t < RTW; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[t][s], kf[s], acc[t], 0, 0, 0);
      };
#pragma unroll
      for (int kb = 0; kb < KEYS / 32; kb += 2) {
        f32x16 acc[RTW];
        float c;
        {
          pin_here(vacc);
          bf16x8 kf[D / 16];
          read_key_frags<D, false>(kf, tile, kb, lane);
          chain(acc, kf);
          c = colsum(vacc);
          interleave_mfma_valu<D / 16, RTW>();
        }
        *vdst = c;
        vdst = vr + kb * 32;
        {
          pin_here(acc);
          bf16x8 kf[D / 16];
          read_key_frags<D, false>(kf, tile, kb + 1, lane);
          chain(vacc, kf);
          c = colsum(acc);
          interleave_mfma_valu<D / 16, RTW>();
        }
        *vdst = c;
        vdst = vr + (kb + 1) * 32;
      }
      return;
    }
    flush_pending();
    // A tile inside the voted range, with every row tile of this wave present
    // and every group whole, takes a path without per-chain conditions (no
    // accumulators to define for chains that are not run).
    if (tk0 + KEYS <= kv1 && role.my_nrt == RTW && GB * role.nwk <= KEYS / 32) {
      for (int kb = role.wk; kb < KEYS / 32; kb += GB * role.nwk) {
        bf16x8 kf[GB][D / 16];
        f32x16 acc[GB][RTW];
#pragma unroll
        for (int g = 0; g < GB; ++g) read_key_frags<D>(kf[g], tile, kb + g * role.nwk, lane);
        mfma_phase_begin();
#pragma unroll
        for (int g = 0; g < GB; ++g) {
#pragma unroll
          for (int t = 0; t < RTW; ++t) {
            acc[g][t] = f32x16{};
#pragma unroll
            for (int s = 0; s < D / 16; ++s)
              acc[g][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[t][s], kf[g][s], acc[g][t], 0, 0, 0);
          }
        }
        mfma_phase_end();
#pragma unroll
        for (int g = 0; g < GB; ++g) {
          // the order of colsum below
          float c4[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) c4[v] = exp2_fast(fmaf(acc[g][0][v], scale, -lr[0][v]));
#pragma unroll
          for (int v = 4; v < 16; ++v) c4[v & 3] += exp2_fast(fmaf(acc[g][0][v], scale, -lr[0][v]));
#pragma unroll
          for (int t = 1; t < RTW; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) c4[v & 3] += exp2_fast(fmaf(acc[g][t][v], scale, -lr[t][v]));
          vr[(kb + g * role.nwk) * 32] = (c4[0] + c4[1]) + (c4[2] + c4[3]);
        }
      }
      return;
    }
    for (int kb = role.wk; kb < KEYS / 32; kb += KeyGroup<RTW>::G * role.nwk) {
      if (tk0 + kb * 32 >= kv1) break;
      KeyGroup<RTW> grp(kb, role.nwk, tk0, kv1, KEYS);
      bf16x8 kf[KeyGroup<RTW>::G][D / 16];
      f32x16 acc[KeyGroup<RTW>::G][RTW];
#pragma unroll
      for (int g = 0; g < KeyGroup<RTW>::G; ++g)
        if (grp.has[g]) read_key_frags<D>(kf[g], tile, grp.kb[g], lane);
#pragma unroll
      for (int g = 0; g < KeyGroup<RTW>::G; ++g) {
#pragma unroll
        for (int t = 0; t < RTW; ++t) {
          acc[g][t] = f32x16{};
          if (grp.has[g] && t < role.my_nrt) {
#pragma unroll
            for (int s = 0; s < D / 16; ++s)
              acc[g][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[t][s], kf[g][s], acc[g][t], 0, 0, 0);
          }
        }
      }
      // acc[g][t][v]: logit of row acc_row(v, lane) of row tile t for this lane's key
#pragma unroll
      for (int g = 0; g < KeyGroup<RTW>::G; ++g)
        if (grp.has[g]) vr[grp.kb[g] * 32] = colsum(acc[g]);
    }
  };
  ks.run(sm.ring, compute, [&](int i) {
    if (i > 1) fold(i - 2);
  });
  flush_pending();
  __syncthreads();
  if (ntiles > 1) fold(ntiles - 2);
  fold(ntiles - 1);
  __syncthreads();
  // snapkv_pool, staged in LDS: pooled scores of this item's positions
  const size_t head = (size_t)(b * p.hkv + h);
  float* pooled = p.pooled + head * p.pooled_stride;
  for (int j = key0 + tid; j < kend; j += kThreads) {
    const float c_j = pool_value([&](int u) { return sm.s_chunk[u - kv0]; }, j, P, p.kernel,
                                 p.pool_mode);
    pooled[j] = c_j;
    if (!p.export_scores) lds_count(sm.top, order_key(c_j) >> kTopShift);
  }
  if (!p.export_scores) {
    // the selection's first radix digit: this chunk's counts join the head's
    // histogram (few distinct bins per chunk, so few global atomics); the
    // barrier covers LDS only, the pooled stores need not have landed
    lds_barrier();
    if constexpr (ZERO_FIRST) {
      if (wait_head(p, p.flags + head * p.nchunk, 1)) {
        // item 0 has not published that it cleared the histograms: adding
        // now could be undone by its clearing, so this item adds nothing and
        // the selection recounts the first digit from the pooled scores
        mark_hist_bad(p, head);
        return;
      }
    }
    uint32_t* top = p.top_hist + head * kSelHistWords;
    for (int i = tid; i < kTopBins; i += kThreads) {
      const uint32_t n = sm.top[i];
      if (n != 0u) atomicAdd(&top[i], n);
    }
  }
}

// ---------------------------------------------------------------- fused ---
// Statistics and vote of one chunk in a single launch, for shapes where every
// item can be resident at once and a chunk's keys fit in LDS. Phase 1 is the
// statistics pass with the chunk's key tiles kept in LDS; the item publishes
// its row statistics with device-coherent stores and then a per-item flag
// (this call's `epoch`). Phase 2 waits for the flags of every chunk of its
// head, merges the statistics into each row's normaliser, and votes from the
// resident tiles plus a block of the r halo keys on each side (loaded while
// it waits), then pools and counts as the vote item does. The arithmetic of
// every vote, normaliser and pooled value is the vote item's, in the same
// order, so both paths give identical bits. Every wait is bounded: after
// p.spin_limit polls (kSpinLimit unless the caller lowers it) the item stops
// waiting and computes the statistics of the chunks whose flags were still
// unset itself, with the same code (so the same bits as their own items
// write); the result does not depend on whether a wait gave up. The host
// takes this path only when the grid fits the device one workgroup per CU,
// so normally no wait gives up; when other work holds CUs the items still
// finish, more slowly.

template <int D>
struct alignas(16) FusedSmem {
  unsigned char k[kFusedTiles][KTile<D>::BYTES];  // the chunk's key tiles
  unsigned char halo[32 * KTile<D>::ROWB];       // r keys on each side of the voted range
  union {
    float2 wstats[kWaves][kMaxRowTilesPerWave * 32];
    float2 scratch[kThreads];
  } u;
  float lse[kFusedMaxRows];
  float s_chunk[kFusedChunk + 2 * kFusedMaxHalo];  // votes of keys kv0 ..
  uint8_t missing[kThreads];                       // chunks whose flags a wait gave up on
};
static_assert(sizeof(FusedSmem<128>) <= 160 * 1024, "fused item LDS");

// After a wait gave up: the statistics of every chunk in `missing` (LDS,
// read after a barrier, so the same in every thread), computed with the
// statistics pass's own code and written to that chunk's words with
// device-coherent stores (identical bits to what the chunk's item writes,
// so it does not matter which store lands last). `run` streams the keys
// through two LDS tiles and `qbuf` stages the query rows. Ends when every
// thread's stores are acknowledged and a barrier has passed, so the merge
// that follows reads them.
template <int D, int RTW, typename Run>
__device__ __forceinline__ void recompute_missing_stats(const PathParams& p, const uint8_t* missing,
                                                        int nch, unsigned char* qbuf,
                                                        float2 (*wstats)[kMaxRowTilesPerWave * 32],
                                                        Run&& run, int b, int h) {
  for (int cc = 0; cc < nch; ++cc) {
    // the same value in every thread: taken as a scalar, so the statistics
    // code below keeps its uniform values in scalar registers
    if (__builtin_amdgcn_readfirstlane((int)missing[cc]) == 0) continue;
    // opaque copies of the indices, renewed every iteration: nothing derived
    // from them is hoisted out of the loop or shared with the item's own
    // statistics pass (either would keep registers live across the body)
    int bb = b, hh = h;
    asm volatile("" : "+s"(bb), "+s"(hh));
    bf16x8 qf[RTW][D / 16];
    score_stats_body<D, RTW, true, true, false, false>(p, qbuf, wstats, qf, run, bb, hh, cc);
    __syncthreads();  // the tiles and wstats are reused by the next chunk
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}
static_assert(kTopBins * 4 <= KTile<128>::BYTES, "histogram in a key slot");

template <int D>
__device__ __forceinline__ void snapkv_score_fused_item(const PathParams& p, FusedSmem<D>& sm,
                                                        int b, int h, int c) {
  constexpr int RTW = 1;
  constexpr int KEYS = KTile<D>::KEYS;
  const int L = p.tab.len[b];
  const int P = L - p.window;
  const int key0 = c * p.chunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const WaveRole role = wave_role(p, wave);
  const int nch = (L + p.chunk - 1) / p.chunk;
  const size_t head = (size_t)(b * p.hkv + h);
  const uint16_t* kbase = p.k + ((size_t)p.tab.off[b] * p.hkv + h) * D;
  const size_t tstride = (size_t)p.hkv * D;

  // phase 1: statistics; the query rows are staged through the last slot,
  // which the stream fills last
  bf16x8 qf[RTW][D / 16];
  int nst = 0;  // tiles of the chunk, stored to the slots last tile first
  score_stats_body<D, RTW, true, true>(
      p, sm.k[kFusedTiles - 1], sm.u.wstats, qf,
      [&](KeyStream<D>& ks, auto&& compute) {
        nst = ks.ntiles();
        ks.run_resident(sm.k, compute);
      },
      b, h, c);
  uint64_t* flags = p.flags + head * p.nchunk;
  publish_item(p, flags, c);
  if (key0 >= P) return;  // a chunk of window keys only: nothing to vote

  // phase 2: the voted positions [key0, kend) and their pooling halo
  const int kend = min(key0 + p.chunk, P);
  const int r = p.kernel >> 1;
  const int kv0 = max(0, key0 - r), kv1 = min(P, kend + r);
  const int rl = key0 - kv0, rr = kv1 - kend;  // halo keys before and after
  {
    // halo row i: key kv0 + i (i < rl), kend + i - rl (i < rl + rr); other
    // rows repeat key0 and are never folded
    constexpr int PIECES = KTile<D>::PIECES;
    for (int pc = tid; pc < 32 * PIECES; pc += kThreads) {
      const int row = pc / PIECES, col = pc % PIECES;
      const int j = row < rl ? kv0 + row : (row < rl + rr ? kend + row - rl : key0);
      const u32x4 x = *reinterpret_cast<const u32x4*>(kbase + (size_t)j * tstride + col * 8);
      *reinterpret_cast<u32x4*>(sm.halo + row * KTile<D>::ROWB + col * 16) = x;
    }
  }
  // wait for the statistics of every chunk of this head (bounded)
  if (wait_head(p, flags, nch, sm.missing)) {
    // Some items have not published: their statistics are computed here.
    // The stream needs two tile slots and the query slot, so this chunk's
    // own tiles are reloaded into their slots afterwards (the halo block
    // and the query fragments are unaffected).
    if (__builtin_amdgcn_readfirstlane((int)sm.missing[0])) mark_hist_bad(p, head);
    recompute_missing_stats<D, RTW>(
        p, sm.missing, nch, sm.k[kFusedTiles - 1], sm.u.wstats,
        [&](KeyStream<D>& ks, auto&& compute) {
          ks.run(reinterpret_cast<unsigned char(*)[KTile<D>::BYTES]>(&sm.k[0][0]), compute,
                 [](int) {});
        },
        b, h);
    KeyStream<D> own{{}, {}, kbase, tstride, key0, min(key0 + p.chunk, L), true, true};
    own.prefetch();
    own.run_resident(sm.k, [](const unsigned char*, int) {});
    __syncthreads();
  }

  // lse of every row, exactly as the vote item merges it, from coherent loads
  const float2* part = p.part + head * p.nchunk * p.rows_pad;
  int tpr = 1;
  while (tpr * 2 * p.rows_pad <= kThreads) tpr *= 2;
  const int span = kThreads / tpr;  // rows per round (>= rows_pad)
  const int row = tid % span, sub = tid / span;
  const bool row_ok = row < p.rows;
  const int row_c = min(row, p.rows - 1);
  auto part_of = [&](int cc) { return load_part<true>(&part[(size_t)cc * p.rows_pad + row_c]); };
  float2 pe[kPartBatch];
#pragma unroll
  for (int u = 0; u < kPartBatch; ++u) pe[u] = part_of(min(sub + u * tpr, nch - 1));
  {
    float m = -kInf, s = 0.f;
#pragma unroll
    for (int u = 0; u < kPartBatch; ++u)
      if (sub + u * tpr < nch) m = fmaxf(m, pe[u].x);
    if (m != -kInf) {
#pragma unroll
      for (int u = 0; u < kPartBatch; ++u)
        if (sub + u * tpr < nch) s += pe[u].y * exp2_fast(pe[u].x - m);
    }
    for (int cc = sub + kPartBatch * tpr; cc < nch; cc += tpr) {
      const float2 e = part_of(cc);
      lse_merge(m, s, e.x, e.y);
    }
    sm.u.scratch[tid] = row_ok ? make_float2(m, s) : make_float2(-kInf, 0.f);
    lds_barrier();
    if (tid < p.rows_pad) {
      float mm = -kInf, ss = 0.f;
      for (int q = 0; q < tpr; ++q) {
        const float2 e = sm.u.scratch[q * span + tid];
        lse_merge(mm, ss, e.x, e.y);
      }
      sm.lse[tid] = tid < p.rows ? mm + log2f(ss) : kInf;  // padded rows add 0
    }
    __syncthreads();
  }
  float lr[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) lr[v] = sm.lse[min(role.wr * 32 + acc_row(v, lane), kFusedMaxRows - 1)];
  const float scale = p.scale_log2;

  // the vote item's per-key arithmetic: the block's logits by one MFMA
  // chain, then the column sum over this wave's rows in colsum's order
  auto chain = [&](const unsigned char* tile, int kb) {
    bf16x8 kf[D / 16];
    read_key_frags<D, false>(kf, tile, kb, lane);
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[0][s], kf[s], acc, 0, 0, 0);
    return acc;
  };
  auto colsum = [&](const f32x16& acc) {
    float c4[4];  // started by the first terms, as in the vote item
#pragma unroll
    for (int v = 0; v < 4; ++v) c4[v] = exp2_fast(fmaf(acc[v], scale, -lr[v]));
#pragma unroll
    for (int v = 4; v < 16; ++v) c4[v & 3] += exp2_fast(fmaf(acc[v], scale, -lr[v]));
    return (c4[0] + c4[1]) + (c4[2] + c4[3]);
  };
  const int nparts = 2 * role.nwr;  // (row-tile wave, lane half) partial sums per key
  // Every block this wave votes (its blocks of each resident tile, and the
  // halo block for the waves of key group 0) is computed first, with the
  // column sums kept in registers, so the waves run through the MFMA and
  // exp work without meeting at barriers. The key tiles are then dead: the
  // partial sums of every voted key go to an array in their place and are
  // folded in one pass, in the fixed order of the vote item.
  const int nvt = (kend - key0 + KEYS - 1) / KEYS;  // tiles holding voted keys
  auto has = [&](int tt, int q) {
    const int kb = role.wk + q * role.nwk;
    return tt < nvt && kb < KEYS / 32 && key0 + tt * KEYS + kb * 32 < kend;
  };
  const bool halo = rl + rr > 0;
  float ph = 0.f;
  if (halo && role.wk == 0) ph = colsum(chain(sm.halo, 0));
  float pv[kFusedTiles][4] = {};
#pragma unroll
  for (int tt = 0; tt < kFusedTiles; ++tt) {
    const unsigned char* tile = sm.k[max(nst - 1 - tt, 0)];
#pragma unroll
    for (int q = 0; q < 4; q += 2) {
      const int kb0 = role.wk + q * role.nwk, kb1 = kb0 + role.nwk;
      if (has(tt, q + 1)) {  // two chains in flight before either column sum
        bf16x8 k0[D / 16], k1[D / 16];
        read_key_frags<D, false>(k0, tile, kb0, lane);
        read_key_frags<D, true>(k1, tile, kb1, lane);
        f32x16 a0 = {}, a1 = {};
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
          a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[0][s], k0[s], a0, 0, 0, 0);
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
          a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[0][s], k1[s], a1, 0, 0, 0);
        pv[tt][q] = colsum(a0);
        pv[tt][q + 1] = colsum(a1);
      } else if (has(tt, q)) {
        pv[tt][q] = colsum(chain(tile, kb0));
      }
    }
  }
  constexpr int kVotedMax = kFusedChunk + 2 * kFusedMaxHalo;
  static_assert(2 * kWaves * kVotedMax * 4 <= 2 * KTile<D>::BYTES, "partials in two key slots");
  float (*vall)[kVotedMax] = reinterpret_cast<float (*)[kVotedMax]>(&sm.k[0][0]);
  __syncthreads();  // every wave is done with the key tiles
  // the first digit's histogram lives in a key slot no longer read; cleared
  // here, it is ordered before the counting below by the fold's barriers
  uint32_t* top = reinterpret_cast<uint32_t*>(sm.k[2]);
  for (int i = tid; i < kTopBins; i += kThreads) top[i] = 0u;
  {
    const int col = lane & 31;
    float* mine = vall[2 * role.wr + (lane >> 5)];  // this (row-tile wave, lane half)
    if (halo && role.wk == 0 && col < rl + rr)
      mine[col < rl ? col : kend - kv0 + col - rl] = ph;
#pragma unroll
    for (int tt = 0; tt < kFusedTiles; ++tt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int key = key0 + tt * KEYS + (role.wk + q * role.nwk) * 32 + col;
        if (has(tt, q) && key < kend) mine[key - kv0] = pv[tt][q];
      }
  }
  __syncthreads();
  for (int kk = tid; kk < kv1 - kv0; kk += kThreads) {
    float s = 0.f;
    for (int q = 0; q < nparts; ++q) s += vall[q][kk];
    sm.s_chunk[kk] = s;
  }
  __syncthreads();

  // snapkv_pool and the first radix digit, as in the vote item
  float* pooled = p.pooled + head * p.pooled_stride;
  for (int j = key0 + tid; j < kend; j += kThreads) {
    const float c_j = pool_value([&](int u) { return sm.s_chunk[u - kv0]; }, j, P, p.kernel,
                                 p.pool_mode);
    pooled[j] = c_j;
    lds_count(top, order_key(c_j) >> kTopShift);
  }
  lds_barrier();
  uint32_t* gtop = p.top_hist + head * kSelHistWords;
  for (int i = tid; i < kTopBins; i += kThreads) {
    const uint32_t n = top[i];
    if (n != 0u) atomicAdd(&gtop[i], n);
  }
}

// Statistics and vote in one launch for chunks too long to keep in LDS: the
// statistics item as in snapkv_score_stats (statistics written with
// device-coherent stores), the same publication and bounded wait as the
// fused item, then the vote item as in snapkv_score_vote with coherent loads
// of the statistics; its keys stream through the ring again (this CU read
// them moments before, so mostly from the caches). The same code in the same
// order as the two kernels, so identical bits. When the wait gives up, the
// item computes the missing chunks' statistics itself, as the fused item does.
template <int D, int RTW>
struct FusedStreamSmem {
  union {
    StatsSmem<D> st;
    VoteSmem<D> vt;
  };
  uint8_t missing[kThreads];  // chunks whose flags the wait gave up on
};

template <int D, int RTW>
__device__ __forceinline__ void snapkv_score_fused_stream_item(const PathParams& p,
                                                               FusedStreamSmem<D, RTW>& sm,
                                                               int b, int h, int c) {
  const int L = p.tab.len[b];
  const int P = L - p.window;
  const int nch = (L + p.chunk - 1) / p.chunk;
  const size_t head = (size_t)(b * p.hkv + h);
  {
    bf16x8 qf[RTW][D / 16];
    score_stats_body<D, RTW, true, true>(
        p, sm.st.ring[1], sm.st.wstats, qf,
        [&](KeyStream<D>& ks, auto&& compute) { ks.run(sm.st.ring, compute, [](int) {}); }, b,
        h, c);
  }
  uint64_t* flags = p.flags + head * p.nchunk;
  publish_item(p, flags, c);
  if (c * p.chunk >= P) return;  // a chunk of window keys only: nothing to vote
  if (wait_head(p, flags, nch, sm.missing)) {  // its barrier also frees the LDS
    if (__builtin_amdgcn_readfirstlane((int)sm.missing[0])) mark_hist_bad(p, head);
    recompute_missing_stats<D, RTW>(
        p, sm.missing, nch, sm.st.ring[1], sm.st.wstats,
        [&](KeyStream<D>& ks, auto&& compute) { ks.run(sm.st.ring, compute, [](int) {}); }, b,
        h);
  }
  // opaque copies of the indices: the vote recomputes what it derives from
  // them instead of holding the statistics pass's values through it
  asm volatile("" : "+s"(b), "+s"(h), "+s"(c));
  snapkv_score_vote_item<D, RTW, false, true>(p, sm.vt, b, h, c);
}

}  // namespace snapkv
