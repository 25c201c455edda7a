// Decode-step attention over a KV cache on gfx950: after compression the
// decode phase attends over the kept rows only (glossary page
// "SnapKV(スナップケーブイ)", section "SnapKVの仕組み", step 4; the paper
// page reports the generation speed-up at 16K tokens that follows). For
// prompt b and query head q of KV head h:
//
//   out[b, q] = sum_t softmax_t(q_dec . k_t / sqrt(D)) v_t  over the cached rows
//
// The step streams each row of K and V once, so it is bound by HBM. Two
// kernels:
//
//   snapkv_decode_partial  (chunk, KV head, prompt)  one chunk of rows for all
//                          G query heads of the KV head: each row is read by
//                          D/8 lanes (16 bytes each, so a wave reads whole
//                          rows), the G dot products are reduced over those
//                          lanes with DPP row exchanges, and an online
//                          softmax keeps (max, sum of weights, weighted V)
//                          per lane group while the next rows load; the lane
//                          groups merge through LDS in a fixed order and the
//                          chunk's partial goes to the workspace;
//   snapkv_decode_merge    (query head of the group, KV head, prompt)
//                          merges the chunks in a fixed order and writes out.
//
// Logits are taken in log2 units (q pre-scaled by log2(e)/sqrt(D)); every
// sum has a fixed order, so results are bit-reproducible.
#include "snapkv_decode.h"
#include "snapkv_device.h"

namespace snapkv {
namespace {

__device__ __forceinline__ float bf16_elem(const u32x4& w, int e) {
  const uint32_t x = w[e >> 1];
  return __uint_as_float((e & 1) ? (x & 0xFFFF0000u) : (x << 16));
}

// Sum over aligned groups of W = 8, 16 or 32 lanes, left in every lane of
// the group: DPP exchanges within quads (lane ^ 1, lane ^ 2), then across
// the halves of 8 (half mirror) and of 16 (mirror), then one lane shuffle
// across two rows. Each step adds a value and its partner's, so all lanes of
// a group hold the same bits.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false));
  if (W >= 16)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xf, 0xf, false));
  if (W == 32) x += __shfl_xor(x, 16);
  return x;
}

// Maximum over aligned groups of W = 16 or 32 lanes, in every lane (DPP
// within rows of 16, one lane shuffle across two rows).
template <int W>
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf,
                                                          false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf,
                                                          false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf,
                                                          false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xf, 0xf,
                                                          false)));
  if (W == 32) x = fmaxf(x, __shfl_xor(x, 16));
  return x;
}

template <int D, int GM>
__global__ void __launch_bounds__(kDecodeThreads) snapkv_decode_partial(const DecodeParams p) {
  constexpr int PIECES = D / 8;                 // lanes per row
  constexpr int GROUPS = 64 / PIECES;           // rows per wave per step
  constexpr int NW = kDecodeThreads / 64;
  constexpr int NG = GROUPS * NW;               // lane groups (rows per workgroup step)
  constexpr int NB = GM >= 8 ? 2 : 4;           // steps whose rows load together
  __shared__ float sm_ml[NG][GM][2];
  __shared__ float sm_acc[NG][GM][D];
  __shared__ float sm_f[NG][GM];
  static_assert(NG == 16 || NG == 32, "lane groups per workgroup");

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n = p.len[b];
  const int r0 = c * p.chunk;
  if (r0 >= n) return;
  const int r1 = min(r0 + p.chunk, n);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int piece = lane % PIECES, gi = wave * GROUPS + lane / PIECES;
  size_t base, rs;
  if (p.layout == 0) {
    base = (size_t)(b * p.hkv + h) * p.capacity * D;
    rs = D;
  } else {
    base = ((size_t)p.off[b] * p.hkv + h) * D;
    rs = (size_t)p.hkv * D;
  }
  const uint16_t* kb = p.k + base + piece * 8;
  const uint16_t* vb = p.v + base + piece * 8;

  // rows of this lane group: r0 + gi, r0 + gi + NG, ...; two register sets
  // alternate so that one set's rows load while the other's are used. Row
  // indices past the chunk are clamped to its last row (a cached re-read)
  // and masked, so every load is unconditional.
  constexpr int STEP = NG * NB;
  // the query slice first (query heads past the group re-read the last one
  // and are zeroed), so that waiting for it leaves the rows in flight
  u32x4 qw[GM];
#pragma unroll
  for (int g = 0; g < GM; ++g)
    qw[g] = *reinterpret_cast<const u32x4*>(
        p.q + (size_t)(b * p.hq + h * p.group + min(g, p.group - 1)) * D + piece * 8);
  u32x4 ka[NB], va[NB], kb2[NB], vb2[NB];
  auto load = [&](u32x4 (&kd)[NB], u32x4 (&vd)[NB], int rb) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const size_t r = (size_t)min(rb + u * NG + gi, r1 - 1);
      kd[u] = *reinterpret_cast<const u32x4*>(kb + r * rs);
      vd[u] = *reinterpret_cast<const u32x4*>(vb + r * rs);
    }
    // issued before the work that follows (neither memory operations nor
    // arithmetic move across)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  load(ka, va, r0);
  load(kb2, vb2, r0 + STEP);

  float qv[GM][8];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    const float sc = g < p.group ? p.scale_log2 : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[g][e] = bf16_elem(qw[g], e) * sc;
  }
  float m[GM], l[GM], acc[GM][8];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    m[g] = -kInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }

  auto process = [&](const u32x4 (&kd)[NB], const u32x4 (&vd)[NB], int rb) {
    float s[NB][GM];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const bool ok = rb + u * NG + gi < r1;
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) dot = fmaf(qv[g][e], bf16_elem(kd[u], e), dot);
        dot = group_sum<PIECES>(dot);
        s[u][g] = ok ? dot : -kInf;
      }
    }
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      float mx = m[g];
#pragma unroll
      for (int u = 0; u < NB; ++u) mx = fmaxf(mx, s[u][g]);
      if (mx == -kInf) continue;  // no row of this lane group yet
      const float cs = exp2_fast(m[g] - mx);
      l[g] *= cs;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= cs;
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const float pw = exp2_fast(s[u][g] - mx);
        l[g] += pw;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pw, bf16_elem(vd[u], e), acc[g][e]);
      }
      m[g] = mx;
    }
  };

  // rounds of two register sets: both sets' loads are in flight before the
  // first is used (a chunk is a whole number of rounds, 2 * STEP rows)
  process(ka, va, r0);
  process(kb2, vb2, r0 + STEP);
  for (int rb = r0 + 2 * STEP; rb < r1; rb += 2 * STEP) {
    load(ka, va, rb);
    load(kb2, vb2, rb + STEP);
    process(ka, va, rb);
    process(kb2, vb2, rb + STEP);
  }

  // every lane group's state to LDS; then, per query head, the groups'
  // weights 2^(m_w - max) and the sum of weights by DPP reductions over NG
  // lanes, and each output element as a fixed-order sum over the groups
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    if (piece == 0) {
      sm_ml[gi][g][0] = m[g];
      sm_ml[gi][g][1] = l[g];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_acc[gi][g][piece * 8 + e] = acc[g][e];
  }
  __syncthreads();
  float* dst = p.part + ((size_t)(b * p.hkv + h) * p.nchunk + c) * p.group * (D + 2);
  if (tid < NG * GM) {  // whole waves: NG * GM is a multiple of 16, and of 64 or below it
    const int w = tid % NG, g = tid / NG;
    const float mw = sm_ml[w][g][0];
    const float mx = group_max<NG>(mw);  // finite: every chunk holds a row
    const float f = exp2_fast(mw - mx);  // 0 for a group without rows
    sm_f[w][g] = f;
    const float lsum = group_sum<NG>(f * sm_ml[w][g][1]);
    if (w == 0 && g < p.group) {
      dst[g * (D + 2)] = mx;
      dst[g * (D + 2) + 1] = lsum;
    }
  }
  __syncthreads();
  for (int i = tid; i < p.group * D; i += kDecodeThreads) {
    const int g = i / D, d = i % D;
    float sa = 0.f;
#pragma unroll
    for (int w = 0; w < NG; ++w) sa = fmaf(sm_f[w][g], sm_acc[w][g][d], sa);
    dst[g * (D + 2) + 2 + d] = sa;
  }
}

// One workgroup per (query head, KV head, prompt); kDecodeMergeThreads / D
// slices of threads each fold every S-th chunk into a running (max, sum,
// weighted sum) with eight chunks' loads in flight, then the slices are
// combined in a fixed order.
template <int D>
__global__ void __launch_bounds__(kDecodeMergeThreads) snapkv_decode_merge(const DecodeParams p) {
  constexpr int S = kDecodeMergeThreads / D;
  constexpr int U = 8;
  __shared__ float red_m[kDecodeMergeThreads], red_l[kDecodeMergeThreads],
      red_a[kDecodeMergeThreads];
  const int g = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nch = (p.len[b] + p.chunk - 1) / p.chunk;
  const size_t cstride = (size_t)p.group * (D + 2);
  const float* col = p.part + (size_t)(b * p.hkv + h) * p.nchunk * cstride + g * (D + 2);
  const int tid = threadIdx.x, d = tid % D, sl = tid / D;
  float rm = -kInf, rl = 0.f, ra = 0.f;
  auto fold = [&](float mc, float lc, float ac) {
    const float mx = fmaxf(rm, mc);
    const float fr = exp2_fast(rm - mx), fc = exp2_fast(mc - mx);
    rl = rl * fr + lc * fc;
    ra = ra * fr + ac * fc;
    rm = mx;
  };
  int c = sl;
  for (; c + (U - 1) * S < nch; c += U * S) {
    float mc[U], lc[U], ac[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float* e = col + (size_t)(c + u * S) * cstride;
      mc[u] = e[0];
      lc[u] = e[1];
      ac[u] = e[2 + d];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) fold(mc[u], lc[u], ac[u]);
  }
  for (; c < nch; c += S) {
    const float* e = col + (size_t)c * cstride;
    fold(e[0], e[1], e[2 + d]);
  }
  red_m[tid] = rm;
  red_l[tid] = rl;
  red_a[tid] = ra;
  __syncthreads();
  if (sl == 0) {
    float mx = -kInf;
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) mx = fmaxf(mx, red_m[s2 * D + d]);
    float a = 0.f, l = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) {
      const float ms = red_m[s2 * D + d];
      if (ms == -kInf) continue;  // a slice without chunks
      const float f = exp2_fast(ms - mx);
      a = fmaf(red_a[s2 * D + d], f, a);
      l = fmaf(red_l[s2 * D + d], f, l);
    }
    p.out[(size_t)(b * p.hq + h * p.group + g) * D + d] = a / l;
  }
}

template <int D, int GM>
hipError_t launch_decode_dg(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((snapkv_decode_partial<D, GM>), dim3(p.nchunk, p.hkv, p.batch),
                     dim3(kDecodeThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((snapkv_decode_merge<D>), dim3(p.group, p.hkv, p.batch),
                     dim3(kDecodeMergeThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, hipStream_t stream) {
  if (p.group <= 1) return launch_decode_dg<D, 1>(p, stream);
  if (p.group <= 2) return launch_decode_dg<D, 2>(p, stream);
  if (p.group <= 4) return launch_decode_dg<D, 4>(p, stream);
  if (p.group <= kDecodeMaxGroup) return launch_decode_dg<D, 8>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int head_dim, hipStream_t stream) {
  if (head_dim == 128) return launch_decode_d<128>(p, stream);
  if (head_dim == 64) return launch_decode_d<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace snapkv
