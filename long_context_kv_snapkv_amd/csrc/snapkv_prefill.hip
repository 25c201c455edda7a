// snapkv_prefill: causal prefill attention of every prompt row on gfx950,
// with each row's log-sum-exp (glossary page "SnapKV(スナップケーブイ)", FAQ
// Q3: the window scores come out of the ordinary prefill attention at
// almost no extra cost; the normalisers of the observation window's rows
// are what the window vote needs, and snapkv_compress_from_lse takes them).
//
// Per prompt b, query head q (KV head h = q / G) and row i (position i):
//   lse[i] = log sum_{j <= i} exp(q_i . k_j / sqrt(D))
//   out[i] = sum_{j <= i} exp(q_i . k_j / sqrt(D) - lse[i]) v_j
//
// Work item: 128 query rows of one (prompt, query head), four waves of 32
// rows. Keys and values go through LDS 64 at a time (K row-major, V
// row-major); the item visits the keys up to its last row. Per 32-key block
// a wave computes S^T = K . Q^T with bf16 MFMAs (v_mfma_f32_32x32x16_bf16),
// so a lane holds 16 keys of one row: the running maximum and sum of that
// row are in-lane (plus the other lane half). P = 2^(s - m) goes, rounded to
// bf16, straight into the A operand of the P . V MFMAs: its 16 keys per lane
// are taken as the k-slots in the order the S^T layout holds them, and the V
// operand is read from the transposed tile in the same key order. The
// output accumulates in float32 and is rescaled only when some row's maximum
// moved. V stays row-major in LDS, as K does; the P . V operand (four keys
// of one column per lane and step half) comes from the transposing LDS read
// of gfx950 (ds_read_b64_tr_b16). At the end each row is divided by its sum
// and written as bf16; the
// rows of each prompt's observation window also report their natural-log
// normaliser and a copy of their query, in the layouts snapkv_compress_from_lse
// reads.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "snapkv_device.h"
#include "snapkv_prefill.h"

namespace snapkv {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// ds_read_b64_tr_b16 at an 8-byte aligned LDS address (a generic pointer
// into a __shared__ array)
__device__ __forceinline__ uint2 read_tr16(const unsigned char* a) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(a)));
}

constexpr int BM = kPrefillRows;
constexpr int BN = kPrefillKeys;

template <int D>
struct alignas(16) PrefillSmem {
  static constexpr int ROWB = D * 2 + 16;   // padded row (bytes): MFMA fragment reads hit distinct banks
  // V row (bytes): a transposing read takes 8 bytes from each of 4
  // consecutive rows per 16-lane group, and the two groups of a lane half
  // read columns 16 apart; a row stride of 16 banks (mod 64) keeps all 32
  // lanes on distinct banks
  static constexpr int VROWB = D * 2 + 64;
  unsigned char qo[BM * ROWB];              // the item's query rows, later its output rows
  unsigned char kt[BN * ROWB];              // K tile [key][d]
  unsigned char vt[BN * VROWB];             // V tile [key][d]
};

template <int D>
__global__ void __launch_bounds__(kPrefillThreads, 2) snapkv_prefill(const PrefillParams p) {
  using S = PrefillSmem<D>;
  constexpr int ROWB = S::ROWB;
  constexpr int PIECES = D / 8;  // 16-byte pieces per row
  constexpr int NDS = D / 32;    // 32-wide column slices of the output
  __shared__ S sm;
  const int b = blockIdx.z, hq = blockIdx.y;
  const int L = p.tab.len[b];
  const int nqb = (L + BM - 1) / BM;
  if ((int)blockIdx.x >= nqb) return;
  const int qb = nqb - 1 - (int)blockIdx.x;  // the longest items (last rows) first
  const int r0 = qb * BM;
  const int h = hq / p.group;
  const size_t off = (size_t)p.tab.off[b];
  const size_t qstride = (size_t)p.hq * D, kstride = (size_t)p.hkv * D;
  const uint16_t* qbase = p.q + off * qstride + (size_t)hq * D;
  const uint16_t* kbase = p.k + off * kstride + (size_t)h * D;
  const uint16_t* vbase = p.v + off * kstride + (size_t)h * D;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();

  // the item's query rows (rows past the prompt are zero)
  for (int pc = tid; pc < BM * PIECES; pc += kPrefillThreads) {
    const int row = pc / PIECES, col = pc % PIECES;
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
    if (r0 + row < L) x = *reinterpret_cast<const u32x4*>(qbase + (size_t)(r0 + row) * qstride + col * 8);
    *reinterpret_cast<u32x4*>(sm.qo + row * ROWB + col * 16) = x;
  }
  __syncthreads();
  bf16x8 qf[D / 16];  // this wave's 32 rows as the B operand of S^T = K . Q^T
  {
    const unsigned char* qrow = sm.qo + (32 * wave + (lane & 31)) * ROWB + (lane >> 5) * 16;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + s * 32));
  }
  const int wr0 = r0 + 32 * wave;          // first row of this wave
  const int my_row = wr0 + (lane & 31);    // the row of this lane's S^T column
  const float scale = p.scale_log2;
  float m = -kInf;  // the row's reference (scaled log2 units, within 8 of its maximum so far), same in lanes l and l^32
  float lsum = 0.f; // this lane's part of the row's sum of 2^(x - m)
  f32x16 o[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) o[ds] = f32x16{};

  const int kend = min(r0 + BM, L);  // keys up to the item's last row
  const int ntiles = (kend + BN - 1) / BN;
  // a thread moves the same 16-byte pieces of K and of V
  constexpr int LOADS = BN * PIECES / kPrefillThreads;
  static_assert(LOADS >= 1 && BN * PIECES % kPrefillThreads == 0, "tile split");
  u32x4 kx[LOADS], vx[LOADS];
  // tile k0's loads into the registers (rows past the prompt: a valid row,
  // masked in the logits)
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int pc = tid + u * kPrefillThreads;
      const int j = min(k0 + pc / PIECES, L - 1);
      kx[u] = *reinterpret_cast<const u32x4*>(kbase + (size_t)j * kstride + (pc % PIECES) * 8);
      vx[u] = *reinterpret_cast<const u32x4*>(vbase + (size_t)j * kstride + (pc % PIECES) * 8);
    }
  };
  load_tile(0);
  for (int it = 0; it < ntiles; ++it) {
    const int k0 = it * BN;
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int pc = tid + u * kPrefillThreads;
      *reinterpret_cast<u32x4*>(sm.kt + (pc / PIECES) * ROWB + (pc % PIECES) * 16) = kx[u];
      *reinterpret_cast<u32x4*>(sm.vt + (pc / PIECES) * S::VROWB + (pc % PIECES) * 16) = vx[u];
    }
    // the next tile's loads fly while this one is computed
    if (it + 1 < ntiles) load_tile(k0 + BN);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      const int bk0 = k0 + 32 * kb;
      if (bk0 > wr0 + 31) break;  // every row of this wave is before these keys
      f32x16 s = f32x16{};
      {
        const unsigned char* krow = sm.kt + (32 * kb + (lane & 31)) * ROWB + (lane >> 5) * 16;
        bf16x8 kf[D / 16];
#pragma unroll
        for (int st = 0; st < D / 16; ++st)
          kf[st] = as_bf16x8(*reinterpret_cast<const u32x4*>(krow + st * 32));
#pragma unroll
        for (int st = 0; st < D / 16; ++st)
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[st], s, 0, 0, 0);
      }
      // s[v]: logit of row my_row with key bk0 + acc_row(v, lane)
      // masked keys get -inf logits; the scale enters each term's exponent
      // through an fma, and the block maximum is scaled once (scale > 0 and
      // rounding is monotonic, so that is the maximum of the scaled logits)
      f32x16 x = s;
      const bool edge = bk0 + 31 > wr0 || bk0 + 31 >= L;  // the diagonal or the prompt's end
      if (edge) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = bk0 + acc_row(v, lane);
          if (key > my_row || key >= L) x[v] = -kInf;
        }
      }
      float bm = x[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) bm = fmaxf(bm, x[v]);
      const float2 bh = halves32(bm);
      bm = fmaxf(bh.x, bh.y) * scale;
      // the row's reference moves only when the block's maximum exceeds it
      // by more than 8 (log2 units): the terms 2^(x - m) then stay below 2^8,
      // and the output rows are rescaled rarely (m + log2(sum) is the row's
      // normaliser whichever reference m holds)
      const float mn = bm > m + 8.f ? bm : m;  // finite: every row sees key 0 in the first block
      const float alpha = exp2_fast(m - mn);
      float pv[16];
      float ps = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        pv[v] = exp2_fast(fmaf(x[v], scale, -mn));
        ps += pv[v];
      }
      lsum = lsum * alpha + ps;
      m = mn;
      if (__ballot(alpha != 1.f) != 0) {
        // rescale the output rows whose maximum moved: output lane l holds
        // rows acc_row(v, l), whose factors sit in lanes acc_row(v, l)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float a = __shfl(alpha, acc_row(v, lane));
#pragma unroll
          for (int ds = 0; ds < NDS; ++ds) o[ds][v] *= a;
        }
      }
      bf16x8 pa[2];  // P as the A operand: k-slot i of step t is this lane's element 8t + i
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 8; ++i) pa[t][i] = (__bf16)pv[8 * t + i];
      // The V operand in the same key order: step t, lane half hh holds keys
      // 16t + 4hh + {0..3} and 16t + 8 + 4hh + {0..3} of column 32ds + lane%32.
      // Within each 16-lane group the transposing read hands lane j, slot c,
      // bytes 2j % 8 .. +1 of the 8 that lane 4c + j/4 points at; so lane
      // i = 4c + q of a group points at key (base + c), columns n0 + 4q .. +3,
      // and lane j receives column n0 + j of keys base .. base + 3.
      const int gi = lane & 15;
      const unsigned char* vgrp = sm.vt + (32 * kb + 4 * (lane >> 5) + (gi >> 2)) * S::VROWB +
                                  (16 * ((lane >> 4) & 1) + 4 * (gi & 3)) * 2;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
          const unsigned char* a = vgrp + 16 * t * S::VROWB + 32 * ds * 2;
          const uint2 l2 = read_tr16(a), h2 = read_tr16(a + 8 * S::VROWB);
          const bf16x8 vb = as_bf16x8(u32x4{l2.x, l2.y, h2.x, h2.y});
          o[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[t], vb, o[ds], 0, 0, 0);
        }
      }
    }
  }

  // the row's sum (both lane halves), its normaliser, and the output rows
  const float2 lh = halves32(lsum);
  const float ltot = lh.x + lh.y;
  const float inv = 1.f / ltot;
  __syncthreads();  // every wave is done with the query rows in LDS
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = acc_row(v, lane);
    const float f = __shfl(inv, row);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const __bf16 y = (__bf16)(o[ds][v] * f);
      *reinterpret_cast<__bf16*>(sm.qo + (32 * wave + row) * ROWB + (32 * ds + (lane & 31)) * 2) = y;
    }
  }
  __syncthreads();
  uint16_t* obase = p.out + off * qstride + (size_t)hq * D;
  for (int pc = tid; pc < BM * PIECES; pc += kPrefillThreads) {
    const int row = pc / PIECES, col = pc % PIECES;
    if (r0 + row < L)
      *reinterpret_cast<u32x4*>(obase + (size_t)(r0 + row) * qstride + col * 8) =
          *reinterpret_cast<const u32x4*>(sm.qo + row * ROWB + col * 16);
  }
  // the observation window's rows: normaliser and query copy
  const int w0 = L - p.window;  // position of window row 0
  if (p.window_lse != nullptr && lane < 32 && my_row < L && my_row >= w0) {
    const float lse2 = m + log2f(ltot);
    p.window_lse[((size_t)b * p.hq + hq) * p.window + (my_row - w0)] = lse2 * 0.6931471805599453f;
  }
  if (p.q_win != nullptr) {
    uint16_t* qw = p.q_win + ((size_t)b * p.hq + hq) * p.window * D;
    for (int pc = tid; pc < BM * PIECES; pc += kPrefillThreads) {
      const int row = pc / PIECES, col = pc % PIECES;
      const int t = r0 + row;
      if (t < L && t >= w0)
        *reinterpret_cast<u32x4*>(qw + (size_t)(t - w0) * D + col * 8) =
            *reinterpret_cast<const u32x4*>(qbase + (size_t)t * qstride + col * 8);
    }
  }
  if (qb == 0 && w0 < 0) {  // a prompt shorter than the window: rows before its start
    for (int i = tid; i < -w0; i += kPrefillThreads)
      if (p.window_lse != nullptr)
        p.window_lse[((size_t)b * p.hq + hq) * p.window + i] = __builtin_nanf("");
    if (p.q_win != nullptr) {
      uint16_t* qw = p.q_win + ((size_t)b * p.hq + hq) * p.window * D;
      for (int pc = tid; pc < -w0 * PIECES; pc += kPrefillThreads)
        *reinterpret_cast<u32x4*>(qw + (size_t)(pc / PIECES) * D + (pc % PIECES) * 8) =
            u32x4{0u, 0u, 0u, 0u};
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid(p.nqb, p.hq, p.batch);
  if (head_dim == 128)
    hipLaunchKernelGGL(snapkv_prefill<128>, grid, dim3(kPrefillThreads), 0, stream, p);
  else if (head_dim == 64)
    hipLaunchKernelGGL(snapkv_prefill<64>, grid, dim3(kPrefillThreads), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace snapkv
