// snapkv_score: the observation-window vote of SnapKV on gfx950.
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
// Because every row's normaliser must be known before any column can be
// summed, the work is two passes over the keys, each a bf16 MFMA contraction
// Q_win . K^T with fp32 accumulation:
//   pass 1 (snapkv_score_stats): per key chunk, per row, the running maximum
//          and sum of 2^(x - max) with x = l * log2(e); written as partials;
//   pass 2 (snapkv_score_vote):  every chunk combines the partials of all
//          chunks into lse_r, recomputes its logits and column-sums
//          2^(x - lse) over the rows into s_h[j].
//
// Work decomposition: one workgroup per (key chunk, KV head, prompt). Keys are
// staged through LDS in tiles of 64 (padded rows, conflict-free fragment
// reads); the group's query rows stay in VGPRs as MFMA operands for the whole
// chunk. Waves split the 32-row tiles (and the 32-key blocks when there are
// fewer row tiles than waves). MFMA v_mfma_f32_32x32x16_bf16:
//   pass 1 computes C[key][row] so a lane owns one row -> row statistics are
//          in-lane reductions over 16 keys;
//   pass 2 computes C[row][key] so a lane owns one key -> column sums are
//          in-lane reductions over 16 rows.
// Both use the same D-to-k-slot map for Q and K (lane half hf supplies
// elements 16*s + 8*hf .. +7 of k-step s), so any consistent map is exact.
// All reductions run in a fixed order: results are bitwise reproducible.
#include "snapkv_kernels.h"

namespace snapkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxRowTilesPerWave = 2;
constexpr float kInf = __builtin_inff();

__device__ __forceinline__ float exp2_fast(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32
}

// Row (M index) of accumulator element v held by `lane` in a 32x32 tile.
__device__ __forceinline__ int acc_row(int v, int lane) {
  return ((v >> 2) << 3) + ((lane >> 5) << 2) + (v & 3);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) {
  return __builtin_bit_cast(bf16x8, x);
}

__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mx = fmaxf(m, m2);
  if (mx == -kInf) return;
  s = s * exp2_fast(m - mx) + s2 * exp2_fast(m2 - mx);
  m = mx;
}

template <int D, int NW>
struct Tiles {
  static constexpr int KS = D / 16;               // MFMA k-steps over D
  static constexpr int ROWB = D * 2 + 16;          // padded LDS key row (bytes)
  static constexpr int PIECES = D / 8;             // 16-byte pieces per key row
  static constexpr int NT = NW * 64;
  static constexpr int LOADS = kKeyTile * PIECES / NT;  // 16-byte loads per thread per tile
  static_assert(LOADS >= 1 && kKeyTile * PIECES % NT == 0, "tile split");
  typedef u32x4 Regs[LOADS];  // one key tile's share of a thread
};

// Global -> registers: this thread's pieces of keys [tk0, tk0 + 64); keys at
// or beyond kend read as zero.
template <int D, int NW>
__device__ __forceinline__ void load_key_tile(typename Tiles<D, NW>::Regs& r,
                                              const uint16_t* kb, size_t tstride,
                                              int tk0, int kend, int tid) {
  using T = Tiles<D, NW>;
#pragma unroll
  for (int u = 0; u < T::LOADS; ++u) {
    const int pc = tid + u * T::NT;
    const int key = pc / T::PIECES, col = pc % T::PIECES;
    const int j = tk0 + key;
    if (j < kend) {
      r[u] = *reinterpret_cast<const u32x4*>(kb + (size_t)j * tstride + col * 8);
    } else {
      r[u] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <int D, int NW>
__device__ __forceinline__ void store_key_tile(const typename Tiles<D, NW>::Regs& r,
                                               unsigned char* lds, int tid) {
  using T = Tiles<D, NW>;
#pragma unroll
  for (int u = 0; u < T::LOADS; ++u) {
    const int pc = tid + u * T::NT;
    const int key = pc / T::PIECES, col = pc % T::PIECES;
    *reinterpret_cast<u32x4*>(lds + key * T::ROWB + col * 16) = r[u];
  }
}

// K fragments of key block kb (32 keys) for this lane: key kb*32 + (lane&31).
template <int D, int NW>
__device__ __forceinline__ void read_key_frag(bf16x8 (&kf)[D / 16], const unsigned char* lds,
                                              int kb, int lane) {
  using T = Tiles<D, NW>;
  const unsigned char* row = lds + (kb * 32 + (lane & 31)) * T::ROWB + (lane >> 5) * 16;
#pragma unroll
  for (int s = 0; s < T::KS; ++s) {
    kf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(row + s * 32));
  }
}

// Query fragments of this wave's row tiles; rows at or beyond `rows` are zero.
template <int D>
__device__ __forceinline__ void load_query_frags(bf16x8 (&qf)[kMaxRowTilesPerWave][D / 16],
                                                 const uint16_t* qbase, int rows, int wr,
                                                 int nwr, int my_nrt, int lane) {
#pragma unroll
  for (int t = 0; t < kMaxRowTilesPerWave; ++t) {
    const int r = (wr + nwr * t) * 32 + (lane & 31);
    const bool ok = t < my_nrt && r < rows;
    const uint16_t* src = qbase + (size_t)r * D + (lane >> 5) * 8;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 x = u32x4{0u, 0u, 0u, 0u};
      if (ok) x = *reinterpret_cast<const u32x4*>(src + s * 16);
      qf[t][s] = as_bf16x8(x);
    }
  }
}

// ------------------------------------------------------------ pass 1 ------
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64)
snapkv_score_stats(const ScoreParams p) {
  using T = Tiles<D, NW>;
  __shared__ __attribute__((aligned(16))) unsigned char klds[2][kKeyTile * T::ROWB];
  __shared__ float2 wstats[NW][kMaxRowTilesPerWave * 32];

  const int b = blockIdx.z, h = blockIdx.y, c = blockIdx.x;
  const int L = p.tab.len[b];
  const int P = L - p.window;
  if (P < 1 || (p.skip_fitting && L <= p.budget)) return;
  const int key0 = c * p.chunk;
  if (key0 >= L) return;
  const int kend = min(key0 + p.chunk, L);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nrt = p.rows_pad >> 5;
  const int nwr = p.nwr, nwk = NW / nwr;
  const int wr = wave % nwr, wk = wave / nwr;
  const int my_nrt = (nrt - wr + nwr - 1) / nwr;

  bf16x8 qf[kMaxRowTilesPerWave][D / 16];
  const uint16_t* qbase = p.q + (size_t)(b * p.hq + h * p.group) * p.window * D;
  load_query_frags<D>(qf, qbase, p.rows, wr, nwr, my_nrt, lane);

  // last key visible to this lane's row in each row tile (causal window row)
  int lim[kMaxRowTilesPerWave];
  float mrun[kMaxRowTilesPerWave], srun[kMaxRowTilesPerWave];
#pragma unroll
  for (int t = 0; t < kMaxRowTilesPerWave; ++t) {
    const int r = (wr + nwr * t) * 32 + (lane & 31);
    lim[t] = (t < my_nrt && r < p.rows) ? P + r % p.window : -1;
    mrun[t] = -kInf;
    srun[t] = 0.f;
  }
  const float scale = p.scale_log2;
  const int full_end = min(P, kend);  // keys below this are visible to every row

  const size_t tstride = (size_t)p.hkv * D;
  const uint16_t* kbase = p.k + ((size_t)p.tab.off[b] * p.hkv + h) * D;
  const int ntiles = (kend - key0 + kKeyTile - 1) / kKeyTile;

  typename T::Regs pre;
  load_key_tile<D, NW>(pre, kbase, tstride, key0, kend, tid);
  for (int i = 0; i < ntiles; ++i) {
    const int buf = i & 1;
    const int tk0 = key0 + i * kKeyTile;
    store_key_tile<D, NW>(pre, klds[buf], tid);
    __syncthreads();
    if (i + 1 < ntiles) load_key_tile<D, NW>(pre, kbase, tstride, tk0 + kKeyTile, kend, tid);
    for (int kb = wk; kb < kKeyTile / 32; kb += nwk) {
      const int bk0 = tk0 + kb * 32;
      if (bk0 >= kend) break;
      bf16x8 kf[D / 16];
      read_key_frag<D, NW>(kf, klds[buf], kb, lane);
      const bool full = bk0 + 32 <= full_end;
#pragma unroll
      for (int t = 0; t < kMaxRowTilesPerWave; ++t) {
        if (t >= my_nrt) break;
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[t][s], acc, 0, 0, 0);
        }
        // acc[v]: logit of key bk0 + acc_row(v, lane) for this lane's row
        float mx = -kInf;
        if (!full) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int j = bk0 + acc_row(v, lane);
            if (j > lim[t] || j >= kend) acc[v] = -kInf;
          }
        }
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
  }

  // lanes l and l^32 hold the same row over different keys
#pragma unroll
  for (int t = 0; t < kMaxRowTilesPerWave; ++t) {
    const float mo = __shfl_xor(mrun[t], 32);
    const float so = __shfl_xor(srun[t], 32);
    lse_merge(mrun[t], srun[t], mo, so);
    if (lane < 32 && t < my_nrt) wstats[wave][t * 32 + lane] = make_float2(mrun[t], srun[t]);
  }
  __syncthreads();
  float2* dst = p.part + ((size_t)(b * p.hkv + h) * p.nchunk + c) * p.rows_pad;
  for (int r = tid; r < p.rows; r += T::NT) {
    const int rt = r >> 5, owner = rt % nwr, t = rt / nwr;
    float m = -kInf, s = 0.f;
    for (int q = 0; q < nwk; ++q) {
      const float2 e = wstats[owner + nwr * q][t * 32 + (r & 31)];
      lse_merge(m, s, e.x, e.y);
    }
    dst[r] = make_float2(m, s);
  }
}

// ------------------------------------------------------------ pass 2 ------
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64)
snapkv_score_vote(const ScoreParams p) {
  using T = Tiles<D, NW>;
  __shared__ __attribute__((aligned(16))) unsigned char klds[2][kKeyTile * T::ROWB];
  __shared__ float lse_s[kMaxRows];
  __shared__ float vred[2][NW][kKeyTile];

  const int b = blockIdx.z, h = blockIdx.y, c = blockIdx.x;
  const int L = p.tab.len[b];
  const int P = L - p.window;
  if (P < 1 || (p.skip_fitting && L <= p.budget)) return;
  const int key0 = c * p.chunk;
  if (key0 >= P) return;
  const int kend = min(key0 + p.chunk, P);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nrt = p.rows_pad >> 5;
  const int nwr = p.nwr, nwk = NW / nwr;
  const int wr = wave % nwr, wk = wave / nwr;
  const int my_nrt = (nrt - wr + nwr - 1) / nwr;

  // combine the per-chunk statistics of every row into lse (log2 units)
  {
    const int nch = (L + p.chunk - 1) / p.chunk;
    const float2* part = p.part + (size_t)(b * p.hkv + h) * p.nchunk * p.rows_pad;
    for (int r = tid; r < p.rows_pad; r += T::NT) {
      float lse = kInf;  // padded rows contribute exp2(-inf) = 0
      if (r < p.rows) {
        float m = -kInf;
        for (int cc = 0; cc < nch; ++cc) m = fmaxf(m, part[(size_t)cc * p.rows_pad + r].x);
        float s = 0.f;
        for (int cc = 0; cc < nch; ++cc) {
          const float2 e = part[(size_t)cc * p.rows_pad + r];
          s += e.y * exp2_fast(e.x - m);
        }
        lse = m + log2f(s);
      }
      lse_s[r] = lse;
    }
  }

  bf16x8 qf[kMaxRowTilesPerWave][D / 16];
  const uint16_t* qbase = p.q + (size_t)(b * p.hq + h * p.group) * p.window * D;
  load_query_frags<D>(qf, qbase, p.rows, wr, nwr, my_nrt, lane);
  __syncthreads();
  float lr[kMaxRowTilesPerWave][16];
#pragma unroll
  for (int t = 0; t < kMaxRowTilesPerWave; ++t) {
    const int rt = wr + nwr * t;
#pragma unroll
    for (int v = 0; v < 16; ++v)
      lr[t][v] = t < my_nrt ? lse_s[min(rt * 32 + acc_row(v, lane), kMaxRows - 1)] : kInf;
  }
  const float scale = p.scale_log2;

  const size_t tstride = (size_t)p.hkv * D;
  const uint16_t* kbase = p.k + ((size_t)p.tab.off[b] * p.hkv + h) * D;
  float* out = p.raw + (size_t)(b * p.hkv + h) * p.p_stride;
  const int ntiles = (kend - key0 + kKeyTile - 1) / kKeyTile;

  typename T::Regs pre;
  load_key_tile<D, NW>(pre, kbase, tstride, key0, kend, tid);
  for (int i = 0; i < ntiles; ++i) {
    const int buf = i & 1;
    const int tk0 = key0 + i * kKeyTile;
    store_key_tile<D, NW>(pre, klds[buf], tid);
    __syncthreads();
    if (i > 0) {  // finish the previous tile: sum the waves' row-tile partials
      const int pk0 = tk0 - kKeyTile;
      for (int kk = tid; kk < kKeyTile; kk += T::NT) {
        if (pk0 + kk < kend) {
          float s = 0.f;
          for (int q = 0; q < nwr; ++q) s += vred[buf ^ 1][q][kk];
          out[pk0 + kk] = s;
        }
      }
    }
    if (i + 1 < ntiles) load_key_tile<D, NW>(pre, kbase, tstride, tk0 + kKeyTile, kend, tid);
    for (int kb = wk; kb < kKeyTile / 32; kb += nwk) {
      const int bk0 = tk0 + kb * 32;
      if (bk0 >= kend) break;
      bf16x8 kf[D / 16];
      read_key_frag<D, NW>(kf, klds[buf], kb, lane);
      float cs = 0.f;
#pragma unroll
      for (int t = 0; t < kMaxRowTilesPerWave; ++t) {
        if (t >= my_nrt) break;
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[t][s], kf[s], acc, 0, 0, 0);
        }
        // acc[v]: logit of row acc_row(v, lane) for key bk0 + (lane & 31)
#pragma unroll
        for (int v = 0; v < 16; ++v) cs += exp2_fast(fmaf(acc[v], scale, -lr[t][v]));
      }
      cs += __shfl_xor(cs, 32);
      if (lane < 32) vred[buf][wr][kb * 32 + lane] = cs;
    }
  }
  __syncthreads();
  {
    const int buf = (ntiles - 1) & 1;
    const int pk0 = key0 + (ntiles - 1) * kKeyTile;
    for (int kk = tid; kk < kKeyTile; kk += T::NT) {
      if (pk0 + kk < kend) {
        float s = 0.f;
        for (int q = 0; q < nwr; ++q) s += vred[buf][q][kk];
        out[pk0 + kk] = s;
      }
    }
  }
}

}  // namespace

hipError_t launch_score_stats(const ScoreParams& p, int head_dim, int waves, dim3 grid,
                              hipStream_t stream) {
  if (head_dim == 128 && waves == 4)
    hipLaunchKernelGGL((snapkv_score_stats<128, 4>), grid, dim3(256), 0, stream, p);
  else if (head_dim == 128 && waves == 8)
    hipLaunchKernelGGL((snapkv_score_stats<128, 8>), grid, dim3(512), 0, stream, p);
  else if (head_dim == 64 && waves == 4)
    hipLaunchKernelGGL((snapkv_score_stats<64, 4>), grid, dim3(256), 0, stream, p);
  else if (head_dim == 64 && waves == 8)
    hipLaunchKernelGGL((snapkv_score_stats<64, 8>), grid, dim3(512), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_score_vote(const ScoreParams& p, int head_dim, int waves, dim3 grid,
                             hipStream_t stream) {
  if (head_dim == 128 && waves == 4)
    hipLaunchKernelGGL((snapkv_score_vote<128, 4>), grid, dim3(256), 0, stream, p);
  else if (head_dim == 128 && waves == 8)
    hipLaunchKernelGGL((snapkv_score_vote<128, 8>), grid, dim3(512), 0, stream, p);
  else if (head_dim == 64 && waves == 4)
    hipLaunchKernelGGL((snapkv_score_vote<64, 4>), grid, dim3(256), 0, stream, p);
  else if (head_dim == 64 && waves == 8)
    hipLaunchKernelGGL((snapkv_score_vote<64, 8>), grid, dim3(512), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace snapkv
