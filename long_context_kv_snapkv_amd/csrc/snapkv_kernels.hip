// Kernels of the SnapKV compression path on gfx950, as grids of work items:
//
//   snapkv_score_stats  (chunk, head, prompt)   per-row softmax statistics
//   snapkv_score_vote   (chunk, head, prompt)   window vote + pooling
//     or, when every item fits the device at once, both in one launch:
//   snapkv_score_fused  (chunk, head, prompt)   keys kept in LDS between them
//   snapkv_score_fused_stream (chunk, head, prompt)  keys streamed twice
//   snapkv_select       (head, prompt)          threshold of the top-(B - W)
//                                               and its count table
//     or, for long prefixes, snapkv_select_digit<2>, snapkv_select_digit<3>
//     and snapkv_select_count over (slice, head, prompt)
//   snapkv_gather       (row block, head, prompt)  slots -> positions, rows
//     or, when the prefixes fit one workgroup's registers and the grid fits
//     the device at once, snapkv_gather_select (row block, head, prompt):
//     each item runs its head's selection, then places and moves its rows
//
//   snapkv_clear_hist   (head, prompt)          zeroes the vote's digit
//                                               histogram when the caller
//                                               supplies the normalisers
//
// A compress call runs the four in stream order; the kernel boundaries carry
// every hand-off between stages, except inside the fused score kernels,
// whose items wait (bounded) for per-item flags of the other items of their
// head.
// The score export runs stats and vote only, with the caller's buffer as the
// pooled rows.
#include <hip/hip_ext.h>

#include <type_traits>

#include "snapkv_gather.h"
#include "snapkv_score.h"
#include "snapkv_select.h"

namespace snapkv {
namespace {

// The kernel arguments an item's first decisions and address computations
// read, requested at entry in one batch: each scalar load from the argument
// block is a round trip of a few hundred nanoseconds, and without this the
// compiler issues them one branch at a time.
__device__ __forceinline__ void prefetch_score_args(const PathParams& p, int b) {
  asm volatile("" ::"s"(p.tab.len[b]), "s"(p.tab.off[b]), "s"(p.window), "s"(p.budget),
               "s"(p.score_all), "s"(p.chunk), "s"(p.nchunk), "s"(p.rows), "s"(p.rows_pad),
               "s"(p.nwr), "s"(p.hkv), "s"(p.hq), "s"(p.group), "s"(p.q), "s"(p.k));
  asm volatile("" ::"s"(p.export_scores), "s"(p.pooled_stride), "s"(p.kernel), "s"(p.pooled),
               "s"(p.part));
}

__device__ __forceinline__ void prefetch_gather_args(const PathParams& p, int b) {
  asm volatile("" ::"s"(p.tab.len[b]), "s"(p.tab.off[b]), "s"(p.window), "s"(p.budget),
               "s"(p.hkv), "s"(p.pooled_stride), "s"(p.table_stride), "s"(p.pooled),
               "s"(p.k), "s"(p.v), "s"(p.out_k), "s"(p.out_v), "s"(p.out_idx));
  asm volatile("" ::"s"(p.hist_bad), "s"(p.epoch));
}

// The (prompt, KV head, chunk) of a scoring workgroup, from the compact
// grid's pair table or the full grid's coordinates.
struct ScoreItem {
  int b, h, c;
};
__device__ __forceinline__ ScoreItem score_item(const PathParams& p) {
  if (p.npairs > 0) {
    const uint32_t e = p.pair[blockIdx.x];
    return ScoreItem{(int)(e >> 8), (int)blockIdx.y, (int)(e & 255u)};
  }
  return ScoreItem{(int)blockIdx.z, (int)blockIdx.y, (int)blockIdx.x};
}

// The grid of the score kernels.
dim3 score_grid(const PathParams& p) {
  return p.npairs > 0 ? dim3(p.npairs, p.hkv, 1) : dim3(p.nchunk, p.hkv, p.batch);
}

__device__ __forceinline__ bool is_scored(const PathParams& p, int b) {
  const int L = p.tab.len[b];
  return L - p.window >= 1 && (p.score_all || L > p.budget);
}

__device__ __forceinline__ int num_chunks(const PathParams& p, int b) {
  return (p.tab.len[b] + p.chunk - 1) / p.chunk;
}

template <int D, int RTW>
__global__ void __launch_bounds__(kThreads) snapkv_score_stats(const PathParams p) {
  __shared__ StatsSmem<D> sm;
  const ScoreItem it = score_item(p);
  const int b = it.b, h = it.h, c = it.c;
  prefetch_score_args(p, b);
  if (!is_scored(p, b) || c >= num_chunks(p, b)) return;
  snapkv_score_stats_item<D, RTW>(p, sm, b, h, c);
}

template <int D, int RTW, bool EXT_LSE, bool ZERO_FIRST = false>
__global__ void __launch_bounds__(kThreads) snapkv_score_vote(const PathParams p) {
  __shared__ VoteSmem<D> sm;
  const ScoreItem it = score_item(p);
  const int b = it.b, h = it.h, c = it.c;
  prefetch_score_args(p, b);
  const int P = p.tab.len[b] - p.window;
  const int nvote = P >= 1 ? (P + p.chunk - 1) / p.chunk : 0;
  if (p.export_scores && c == (nvote > 0 ? nvote - 1 : 0)) {
    // exported rows are zero past P (the whole row when nothing is scored)
    float* row = p.pooled + (size_t)(b * p.hkv + h) * p.pooled_stride;
    for (int j = max(P, 0) + (int)threadIdx.x; j < p.pooled_stride; j += kThreads) row[j] = 0.f;
  }
  if (!is_scored(p, b) || c >= nvote) return;
  snapkv_score_vote_item<D, RTW, EXT_LSE, false, ZERO_FIRST>(p, sm, b, h, c);
}

// Statistics and vote in one launch (every item resident at once; the host
// checks the grid against the device's CUs).
template <int D>
__global__ void __launch_bounds__(kThreads) snapkv_score_fused(const PathParams p) {
  __shared__ FusedSmem<D> sm;
  const ScoreItem it = score_item(p);
  const int b = it.b, h = it.h, c = it.c;
  prefetch_score_args(p, b);
  if (!is_scored(p, b) || c >= num_chunks(p, b)) return;
  snapkv_score_fused_item<D>(p, sm, b, h, c);
}

// Statistics and vote in one launch with the keys streamed twice (every item
// resident at once; the host checks the grid against the device's CUs).
template <int D, int RTW>
__global__ void __launch_bounds__(kThreads) snapkv_score_fused_stream(const PathParams p) {
  __shared__ FusedStreamSmem<D, RTW> sm;
  const ScoreItem it = score_item(p);
  const int b = it.b, h = it.h, c = it.c;
  prefetch_score_args(p, b);
  if (!is_scored(p, b) || c >= num_chunks(p, b)) return;
  snapkv_score_fused_stream_item<D, RTW>(p, sm, b, h, c);
}

// With the caller's row normalisers there is no statistics pass to clear the
// selection's radix histograms: one workgroup per head does it.
__global__ void __launch_bounds__(kThreads) snapkv_clear_hist(const PathParams p) {
  const int h = blockIdx.x, b = blockIdx.y;
  if (!is_scored(p, b)) return;
  uint4* top = reinterpret_cast<uint4*>(p.top_hist + (size_t)(b * p.hkv + h) * kSelHistWords);
  for (int i = threadIdx.x; i < kHistCleared / 4; i += kThreads) top[i] = make_uint4(0u, 0u, 0u, 0u);
}

__global__ void __launch_bounds__(kThreads) snapkv_select(const PathParams p) {
  __shared__ SelectSmem sm;
  const int h = blockIdx.x, b = blockIdx.y;
  if (p.tab.len[b] <= p.budget) return;  // kept whole by the gather
  snapkv_select_item(p, sm, b, h);
}

// sliced selection of long prefixes: grid (slice, head, prompt)
template <int DIGIT>
__global__ void __launch_bounds__(kThreads) snapkv_select_digit(const PathParams p) {
  __shared__ SliceSmem sm;
  const int sl = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (p.tab.len[b] <= p.budget) return;
  select_digit_slice<DIGIT>(p, sm, b, h, sl);
}

__global__ void __launch_bounds__(kThreads) snapkv_select_count(const PathParams p) {
  __shared__ SliceSmem sm;
  const int sl = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (p.tab.len[b] <= p.budget) return;
  select_count_slice(p, sm, b, h, sl);
}

// the sliced selection as one launch: grid (slice, head, prompt), every
// workgroup resident at once
__global__ void __launch_bounds__(kThreads) snapkv_select_slices(const PathParams p) {
  __shared__ SliceOneSmem sm;
  const int sl = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (p.tab.len[b] <= p.budget) return;
  select_slices_one_launch(p, sm, b, h, sl);
}

template <int D, int FORM, int RW>
__global__ void __launch_bounds__(kThreads) snapkv_gather(const PathParams p) {
  __shared__ GatherSmem sm;
  prefetch_gather_args(p, blockIdx.z);
  snapkv_gather_item<D, FORM, RW>(p, sm, blockIdx.z, blockIdx.y, blockIdx.x);
}

// The gather with the selection inside: every item whose slots hold kept
// prefix positions runs its head's whole selection (the same integer
// decisions as snapkv_select, so all items of a head agree) with the count
// table in LDS, then places and moves its rows. Taken when the prefixes fit
// one workgroup's registers and the grid fits the device at once, so the
// repeated selections run side by side instead of after each other; it
// saves the selection's launch and the table's round trip through memory.
struct alignas(16) GatherSelectSmem {
  SelectSmem sel;
  GatherSmem gs;
  uint32_t table[2 * (kSelectHeldKeys / kSegment)];
  uint32_t thr[4];
};

template <int D, int FORM, int RW>
__global__ void __launch_bounds__(kThreads) snapkv_gather_select(const PathParams p) {
  __shared__ GatherSelectSmem sm;
  // Every item of a head on one XCD: workgroups are dealt to the 8 XCDs in
  // turn, so workgroup w goes to XCD w mod 8, and item (head, rb) is given to
  // w = 8 * ((head / 8) * nb + rb) + head mod 8. Each item reads its head's
  // whole pooled row, which then comes into one L2 instead of eight (HBM
  // traffic 1.50 -> 1.04x the algorithmic bytes on the 16K layer). Any other
  // placement of workgroups still gives every item exactly once.
  int b = blockIdx.z, h = blockIdx.y, rb = blockIdx.x;
  {
    const int nb = gridDim.x, heads = gridDim.y * gridDim.z;
    if (heads % 8 == 0) {
      const int w = blockIdx.x + nb * (blockIdx.y + gridDim.y * blockIdx.z);
      const int slot = w / 8, head = (slot / nb) * 8 + w % 8;
      rb = slot % nb;
      h = head % gridDim.y;
      b = head / gridDim.y;
    }
  }
  prefetch_gather_args(p, b);
  const int t0 = rb * RW;
  const int L = p.tab.len[b];
  const int m = p.budget - p.window;
  if (L > p.budget && t0 < m) {
    select_dispatch(p, sm.sel, b, h, SelectOut{sm.table, sm.thr});
    __syncthreads();
    locate_kept(p, sm.gs, b, h, t0, min(t0 + RW, m), sm.table, sm.thr);
  }
  gather_rows<D, FORM, RW>(p, sm.gs, b, h, rb);
}

// The pooled rows a compress call selected from, copied out of the
// workspace after the call's own kernels (stream order): entry j < P of each
// compressed prompt (L > budget), zero everywhere else.
__global__ void __launch_bounds__(kThreads) snapkv_export_pooled(const PathParams p) {
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t head = (size_t)(b * p.hkv + h);
  const int L = p.tab.len[b];
  const int P = L > p.budget ? L - p.window : 0;
  const float* src = p.pooled + head * p.pooled_stride;
  float* dst = p.scores_out + head * p.scores_len;
  for (int j = threadIdx.x; j < p.scores_len; j += kThreads) dst[j] = j < P ? src[j] : 0.f;
}

// Launch with one PathParams argument; with events, through the extended
// launch that records them at the kernel's own start and end.
template <typename K>
hipError_t launch(K kernel, dim3 grid, hipStream_t stream, const StageEvents& ev,
                  const PathParams& p, bool cooperative = false) {
  if (cooperative) {
    // the runtime makes every workgroup resident at once (or fails the
    // launch); events, if any, are recorded on the stream around it
    void* args[] = {const_cast<PathParams*>(&p)};
    hipError_t e = hipSuccess;
    if (ev.start != nullptr) e = hipEventRecord(ev.start, stream);
    if (e == hipSuccess)
      e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kernel), grid, dim3(kThreads),
                                     args, 0, stream);
    if (e == hipSuccess && ev.stop != nullptr) e = hipEventRecord(ev.stop, stream);
    return e;
  }
  if (ev.start != nullptr || ev.stop != nullptr) {
    void* args[] = {const_cast<PathParams*>(&p)};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, dim3(kThreads), args,
                              0, stream, ev.start, ev.stop, 0);
  }
  hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <typename F>
hipError_t dispatch_dim(int head_dim, F&& f) {
  if (head_dim == 128) return f(std::integral_constant<int, 128>());
  if (head_dim == 64) return f(std::integral_constant<int, 64>());
  return hipErrorInvalidValue;
}

// (head_dim, row tiles per wave) -> template instance
template <typename F>
hipError_t dispatch_dim_rtw(int head_dim, int rtw, F&& f) {
  using I = std::integral_constant<int, 1>;
  using II = std::integral_constant<int, 2>;
  if (head_dim == 128 && rtw == 1) return f(std::integral_constant<int, 128>(), I());
  if (head_dim == 128 && rtw == 2) return f(std::integral_constant<int, 128>(), II());
  if (head_dim == 64 && rtw == 1) return f(std::integral_constant<int, 64>(), I());
  if (head_dim == 64 && rtw == 2) return f(std::integral_constant<int, 64>(), II());
  return hipErrorInvalidValue;
}

int row_tiles_per_wave(const PathParams& p) {
  const int nrt = p.rows_pad / 32;
  return (nrt + p.nwr - 1) / p.nwr;
}

}  // namespace

hipError_t launch_score_stats(const PathParams& p, int head_dim, hipStream_t stream,
                              StageEvents ev) {
  return dispatch_dim_rtw(head_dim, row_tiles_per_wave(p), [&](auto d, auto rtw) {
    return launch(snapkv_score_stats<decltype(d)::value, decltype(rtw)::value>, score_grid(p),
                  stream, ev, p);
  });
}

hipError_t launch_score_vote(const PathParams& p, int head_dim, hipStream_t stream,
                             StageEvents ev, bool ext_lse, bool zero_first) {
  if (zero_first && (!ext_lse || p.nchunk > kThreads)) return hipErrorInvalidValue;
  return dispatch_dim_rtw(head_dim, row_tiles_per_wave(p), [&](auto d, auto rtw) {
    const dim3 grid = score_grid(p);
    if (zero_first)
      return launch(snapkv_score_vote<decltype(d)::value, decltype(rtw)::value, true, true>, grid,
                    stream, ev, p);
    if (ext_lse)
      return launch(snapkv_score_vote<decltype(d)::value, decltype(rtw)::value, true>, grid,
                    stream, ev, p);
    return launch(snapkv_score_vote<decltype(d)::value, decltype(rtw)::value, false>, grid,
                  stream, ev, p);
  });
}

hipError_t launch_score_fused(const PathParams& p, int head_dim, hipStream_t stream,
                              StageEvents ev) {
  if (head_dim != 128 || p.rows_pad > kFusedMaxRows || row_tiles_per_wave(p) != 1 ||
      p.chunk > kFusedChunk || p.kernel / 2 > kFusedMaxHalo || p.nchunk > kThreads)
    return hipErrorInvalidValue;
  return launch(snapkv_score_fused<128>, score_grid(p), stream, ev, p, p.cooperative != 0);
}

hipError_t launch_score_fused_stream(const PathParams& p, int head_dim, hipStream_t stream,
                                     StageEvents ev) {
  if (p.nchunk > kThreads) return hipErrorInvalidValue;
  return dispatch_dim_rtw(head_dim, row_tiles_per_wave(p), [&](auto d, auto rtw) {
    return launch(snapkv_score_fused_stream<decltype(d)::value, decltype(rtw)::value>,
                  score_grid(p), stream, ev, p, p.cooperative != 0);
  });
}

hipError_t launch_export_pooled(const PathParams& p, hipStream_t stream) {
  return launch(snapkv_export_pooled, dim3(p.hkv, p.batch), stream, StageEvents{}, p);
}

hipError_t launch_clear_hist(const PathParams& p, hipStream_t stream, StageEvents ev) {
  return launch(snapkv_clear_hist, dim3(p.hkv, p.batch), stream, ev, p);
}

hipError_t launch_select(const PathParams& p, hipStream_t stream, StageEvents ev) {
  if (p.sel_slices == 0) return launch(snapkv_select, dim3(p.hkv, p.batch), stream, ev, p);
  const dim3 grid(p.sel_slices, p.hkv, p.batch);
  if (p.sel_one_launch) {
    if (p.sel_slices > kThreads) return hipErrorInvalidValue;  // one flag poll per thread
    return launch(snapkv_select_slices, grid, stream, ev, p);
  }
  // the stage's events bracket the three kernels
  StageEvents first, last;
  first.start = ev.start;
  last.stop = ev.stop;
  hipError_t e = launch(snapkv_select_digit<2>, grid, stream, first, p);
  if (e == hipSuccess) e = launch(snapkv_select_digit<3>, grid, stream, StageEvents{}, p);
  if (e == hipSuccess) e = launch(snapkv_select_count, grid, stream, last, p);
  return e;
}

hipError_t launch_gather(const PathParams& p, int head_dim, hipStream_t stream,
                         StageEvents ev, int form) {
  return dispatch_dim(head_dim, [&](auto d) {
    constexpr int D = decltype(d)::value;
    const dim3 grid(p.n_gather_blocks, p.hkv, p.batch);
    auto go = [&](auto rw) {
      constexpr int RW = decltype(rw)::value;
      if (form == kStoreInt4) return launch(snapkv_gather<D, kStoreInt4, RW>, grid, stream, ev, p);
      if (form == kStoreFp8) return launch(snapkv_gather<D, kStoreFp8, RW>, grid, stream, ev, p);
      return launch(snapkv_gather<D, kStoreBf16, RW>, grid, stream, ev, p);
    };
    if constexpr (D == 128) {
      if (p.gather_rows == kGatherRows / 2)
        return go(std::integral_constant<int, kGatherRows / 2>());
    }
    return go(std::integral_constant<int, kGatherRows>());
  });
}

hipError_t launch_gather_select(const PathParams& p, int head_dim, hipStream_t stream,
                                StageEvents ev, int form) {
  if (p.sel_slices != 0) return hipErrorInvalidValue;  // prefixes must fit the registers
  return dispatch_dim(head_dim, [&](auto d) {
    constexpr int D = decltype(d)::value;
    const dim3 grid(p.n_gather_blocks, p.hkv, p.batch);
    auto go = [&](auto rw) {
      constexpr int RW = decltype(rw)::value;
      if (form == kStoreInt4)
        return launch(snapkv_gather_select<D, kStoreInt4, RW>, grid, stream, ev, p);
      if (form == kStoreFp8)
        return launch(snapkv_gather_select<D, kStoreFp8, RW>, grid, stream, ev, p);
      return launch(snapkv_gather_select<D, kStoreBf16, RW>, grid, stream, ev, p);
    };
    if constexpr (D == 128) {
      if (p.gather_rows == kGatherRows / 2)
        return go(std::integral_constant<int, kGatherRows / 2>());
    }
    return go(std::integral_constant<int, kGatherRows>());
  });
}

}  // namespace snapkv
