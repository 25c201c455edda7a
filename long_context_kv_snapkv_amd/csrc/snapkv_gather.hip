// snapkv_gather: assemble the compressed cache from the kept indices.
//
// out_k[b,h,t,:] = k[off_b + idx[t], h, :] and likewise for V, for the first
// n = min(L, B) entries; the remaining entries are zero rows with index -1
// (glossary page "SnapKV(スナップケーブイ)", section "SnapKVの仕組み", steps
// 3-4: the kept pairs form the cache that decode then reads). A prompt with
// L <= B is copied whole (indices 0 .. L-1) and this kernel writes its index
// list too; for longer prompts the list comes from snapkv_topk.
//
// Each 16-byte piece of a row is one lane's load and store, so a wave moves
// whole 128/256-byte rows: reads are row-granular gathers from the packed
// [T, H_kv, D] cache, writes are fully contiguous. Rows are bit copies.
#include "snapkv_kernels.h"

namespace snapkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ void __launch_bounds__(256) snapkv_gather(const GatherParams p) {
  constexpr int PIECES = D / 8;
  constexpr int ROWS_PER_PASS = 256 / PIECES;
  const int b = blockIdx.z, h = blockIdx.y;
  const int t0 = blockIdx.x * kGatherRows;
  const int L = p.tab.len[b];
  const int B = p.budget;
  const bool whole = L <= B;
  const int tid = threadIdx.x;
  int32_t* idx = p.out_idx + (size_t)(b * p.hkv + h) * B;
  if (whole) {
    for (int tt = tid; tt < kGatherRows; tt += 256) {
      const int t = t0 + tt;
      if (t < B) idx[t] = t < L ? t : -1;
    }
  }
  const size_t tstride = (size_t)p.hkv * D;
  const uint16_t* ksrc = p.k + ((size_t)p.tab.off[b] * p.hkv + h) * D;
  const uint16_t* vsrc = p.v + ((size_t)p.tab.off[b] * p.hkv + h) * D;
  const size_t obase = (size_t)(b * p.hkv + h) * B * D;
  const int piece = tid % PIECES;
  for (int tt = tid / PIECES; tt < kGatherRows; tt += ROWS_PER_PASS) {
    const int t = t0 + tt;
    if (t >= B) break;
    const int j = whole ? (t < L ? t : -1) : idx[t];
    u32x4 kx = u32x4{0u, 0u, 0u, 0u}, vx = u32x4{0u, 0u, 0u, 0u};
    if (j >= 0 && j < L) {  // the bound also keeps a bad index list in range
      kx = *reinterpret_cast<const u32x4*>(ksrc + (size_t)j * tstride + piece * 8);
      vx = *reinterpret_cast<const u32x4*>(vsrc + (size_t)j * tstride + piece * 8);
    }
    *reinterpret_cast<u32x4*>(p.out_k + obase + (size_t)t * D + piece * 8) = kx;
    *reinterpret_cast<u32x4*>(p.out_v + obase + (size_t)t * D + piece * 8) = vx;
  }
}

}  // namespace

hipError_t launch_gather(const GatherParams& p, int head_dim, dim3 grid, hipStream_t stream) {
  if (head_dim == 128)
    hipLaunchKernelGGL(snapkv_gather<128>, grid, dim3(256), 0, stream, p);
  else if (head_dim == 64)
    hipLaunchKernelGGL(snapkv_gather<64>, grid, dim3(256), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace snapkv
