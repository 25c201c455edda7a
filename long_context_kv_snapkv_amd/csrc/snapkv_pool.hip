// snapkv_pool: same-length stride-1 pooling of each head's vote vector.
//
// c_h[j] = (1/k) * sum_{|u-j| <= r} s_h[u]          (average; u outside [0,P) is 0)
// c_h[j] = max_{|u-j| <= r, 0 <= u < P} s_h[u]      (maximum)
// with r = k / 2 (glossary page "SnapKV(スナップケーブイ)", section
// "SnapKVの仕組み", paragraph "Pooling for Robustness"; paper page "SnapKV:
// LLM Knows What You are Looking for Before Generation", section
// "기술적 접근법": max or average pooling, kernel 5-13; k = 1 leaves s as is).
//
// One workgroup per 1024 outputs of one (prompt, head): the tile and its
// r-wide halo are staged in LDS once, then every thread pools from LDS. The
// halo is filled with 0 (average: padding counts as zero) or -inf (maximum:
// only in-range positions compete). Outputs past P are written as 0, so an
// exported score buffer is fully defined.
#include "snapkv_kernels.h"

namespace snapkv {
namespace {

__global__ void __launch_bounds__(256) snapkv_pool(const PoolParams p) {
  __shared__ float tile[kPoolTile + kMaxKernel];
  const int b = blockIdx.z, h = blockIdx.y;
  const int j0 = blockIdx.x * kPoolTile;
  const int L = p.tab.len[b];
  const int P = L - p.window;
  if (p.skip_fitting && L <= p.budget) return;
  if (j0 >= p.out_stride) return;
  float* out = p.out + (size_t)(b * p.hkv + h) * p.out_stride;
  const int tid = threadIdx.x;
  const int jend = min(j0 + kPoolTile, p.out_stride);
  if (P < 1) {
    for (int j = j0 + tid; j < jend; j += 256) out[j] = 0.f;
    return;
  }
  const int r = p.kernel >> 1;
  const bool is_max = p.mode == 1;
  const float fill = is_max ? -__builtin_inff() : 0.f;
  const float* src = p.raw + (size_t)(b * p.hkv + h) * p.p_stride;
  const int span = kPoolTile + 2 * r;
  for (int u = tid; u < span; u += 256) {
    const int j = j0 - r + u;
    tile[u] = (j >= 0 && j < P) ? src[j] : fill;
  }
  __syncthreads();
  const float inv_k = 1.0f / (float)p.kernel;
  for (int u = tid; u < kPoolTile; u += 256) {
    const int j = j0 + u;
    if (j >= jend) break;
    float val = 0.f;
    if (j < P) {
      if (is_max) {
        val = tile[u];
        for (int e = 1; e < p.kernel; ++e) val = fmaxf(val, tile[u + e]);
      } else {
        float acc = 0.f;
        for (int e = 0; e < p.kernel; ++e) acc += tile[u + e];
        val = p.kernel == 1 ? acc : acc * inv_k;
      }
    }
    out[j] = val;
  }
}

}  // namespace

hipError_t launch_pool(const PoolParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL(snapkv_pool, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace snapkv
