// Device-side building blocks shared by every kernel of the SnapKV path on
// gfx950 (CDNA4): vector types, MFMA fragment helpers, key tiles staged
// through LDS, and barriers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "snapkv_kernels.h"

namespace snapkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kInf = __builtin_inff();
constexpr int kWaves = kThreads / 64;
constexpr int kMaxRowTilesPerWave = 2;  // row tiles of 32 window rows per wave

// Index of this thread's wave in the workgroup, as a wave-uniform (scalar)
// value, so branches on it and on roles derived from it stay scalar.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

__device__ __forceinline__ float exp2_fast(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Row (M index) of accumulator element v held by `lane` in a 32x32 MFMA tile
// (the N index is lane & 31).
__device__ __forceinline__ int acc_row(int v, int lane) {
  return ((v >> 2) << 3) + ((lane >> 5) << 2) + (v & 3);
}

// The values x of lanes l & ~32 and l | 32 (the wave's two halves), in every
// lane, from one v_permlane32_swap: a VALU exchange, in place of an LDS
// crossbar round trip. A commutative combine of .x and .y gives every lane
// the same bits as combining its own x with lane l ^ 32's.
__device__ __forceinline__ float2 halves32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Likewise lanes l & ~16 and l | 16 (the even and odd 16-lane rows of each
// pair), from one v_permlane16_swap.
__device__ __forceinline__ float2 rows16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Merge two (reference m, sum of 2^(x - m)) pairs (the reference need not be
// the maximum; the result takes the larger one).
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mx = fmaxf(m, m2);
  if (mx == -kInf) return;
  s = s * exp2_fast(m - mx) + s2 * exp2_fast(m2 - mx);
  m = mx;
}

// ------------------------------------------------------- selection keys ---
// Order-preserving 32-bit key of an fp32 score: unsigned comparison of keys
// orders the scores (sign bit set for non-negatives, all bits flipped for
// negatives). The top 11 bits are the first radix digit of the selection.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
constexpr int kTopShift = 21;
constexpr int kTopBins = kTopHistBins;
static_assert(kTopBins == 1 << (32 - kTopShift), "top digit");

// hist[bin] += 1 for every active lane, one LDS atomic per distinct bin in
// the wave (lanes with the bin of the lowest pending lane add together): the
// pooled scores of a chunk fall into very few bins, and same-address LDS
// atomics serialise.
__device__ __forceinline__ void lds_count(uint32_t* hist, uint32_t bin) {
  const int lane = (int)(threadIdx.x & 63);
  uint64_t todo = __ballot(1);
  while (todo != 0) {
    const int leader = __builtin_ctzll(todo);
    const uint32_t lb = (uint32_t)__shfl((int)bin, leader);
    const uint64_t same = __ballot(bin == lb) & todo;
    if (lane == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(same));
    todo &= ~same;
  }
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive prefix sum over the lanes of a wave64: DPP row shifts within each
// 16-lane row, then the row totals (read from lanes 15, 31, 47) are added to
// the rows above them.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
  const int row = (int)(threadIdx.x & 63) >> 4;
  x += (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
  return x;
}

// Sum over the lanes of a wave64, in the lane-63 order of wave_incl_scan's
// total (integer, so any order gives the same value): DPP row shifts, then
// the four row totals.
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 15) +
         (uint32_t)__builtin_amdgcn_readlane((int)x, 31) +
         (uint32_t)__builtin_amdgcn_readlane((int)x, 47) +
         (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ uint32_t wave_total(uint32_t incl_scan) {
  return (uint32_t)__builtin_amdgcn_readlane((int)incl_scan, 63);
}

// ---------------------------------------------------------------- waits ----
// Workgroup barrier for LDS hand-offs that leaves this wave's outstanding
// global loads (into registers) in flight; this wave's LDS reads and writes
// are complete before it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Issue priority of this wave around its MFMA chains. Of the waves sharing a
// SIMD, one that is about to issue matrix work goes ahead of one doing its
// exp work, so the waves settle into alternating phases (one on the matrix
// core while the other uses the VALU) instead of meeting at the matrix core
// together after each barrier.
__device__ __forceinline__ void mfma_phase_begin() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(2);
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void mfma_phase_end() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
}

// Scheduling hint for a region holding the MFMA chains of one key block (KS
// k-steps, each a fragment read followed by RTW MFMAs, one per row tile) and
// independent VALU work (the exp2 sums of another key block): the fragment
// reads run four k-steps ahead of the MFMAs that use them, and every MFMA is
// followed by a share of the VALU work, so the wave keeps the matrix core
// fed while its VALU works and holds only a few fragments at a time.
template <int KS, int RTW>
__device__ __forceinline__ void interleave_mfma_valu() {
  constexpr int kAhead = 4;
  __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);  // fragment reads
#pragma unroll
  for (int s = 0; s < KS; ++s) {
#pragma unroll
    for (int t = 0; t < RTW; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
    }
    if (s + kAhead < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // next read
  }
}

// Marks the accumulators as rewritten here (an empty asm that takes and
// returns their registers): work on them stays below this point, so it is
// not hoisted out of the region that interleaves it with MFMAs.
template <int N>
__device__ __forceinline__ void pin_here(f32x16 (&a)[N]) {
#pragma unroll
  for (int t = 0; t < N; ++t) asm volatile("" : "+v"(a[t]));
}
template <int N>
__device__ __forceinline__ void pin_here(float (&a)[N]) {
#pragma unroll
  for (int t = 0; t < N; ++t) asm volatile("" : "+v"(a[t]));
}

// ------------------------------------------------------------- exchange ---
// Publish what this workgroup wrote for other workgroups of the same launch
// (device-coherent stores or atomics already issued by every thread): each
// thread's writes complete, then flags[c] = the call's epoch.
__device__ __forceinline__ void publish_item(const PathParams& p, uint64_t* flags, int c) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(&flags[c], p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until the flags of chunks 0 .. nch-1 of a head carry this call's
// epoch, at most p.spin_limit polls each; returns non-zero (in every thread)
// if any poll gave up, and with `missing` (LDS, nch entries) records which
// chunks' flags were still unset. Ends with a workgroup barrier.
//
// Ordering: the publishing item writes its words with device-coherent stores
// (agent-scope relaxed atomics: performed at the device's coherence point,
// not held in one XCD's L2), waits until every one of its threads has had
// them acknowledged (s_waitcnt vmcnt(0), then a workgroup barrier), and only
// then stores its flag the same way. A waiting thread polls the flag with
// device-coherent loads and issues the loads of the published words only
// after it has seen the flag (the loop exit depends on the loaded value),
// again device-coherent, so they are served from the coherence point, which
// already holds the words. No cache write-back or invalidation is needed
// for these words. The same holds for counts added with agent-scope atomics
// (the one-launch sliced selection's histograms): those are performed at the
// coherence point too. Requires nch <= kThreads.
__device__ __forceinline__ int wait_head(const PathParams& p, const uint64_t* flags, int nch,
                                         uint8_t* missing = nullptr) {
  int timed_out = 0;
  if ((int)threadIdx.x < nch) {
    int spins = 0;
    uint64_t* f = const_cast<uint64_t*>(&flags[threadIdx.x]);
    while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != p.epoch) {
      if (++spins > p.spin_limit) {
        timed_out = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (missing != nullptr) missing[threadIdx.x] = (uint8_t)timed_out;
  }
  // the same in every thread; returned as a scalar
  return __builtin_amdgcn_readfirstlane(__syncthreads_or(timed_out));
}

// ------------------------------------------------------------ key tiles ---
// A tile is 128 keys x D bf16 of one KV head. Threads load it from global
// memory into registers (16-byte pieces, consecutive threads on consecutive
// pieces of a key row) and store it to LDS with rows padded by 16 bytes, so
// the MFMA fragment reads (32 rows at one column offset) hit distinct banks.
// Two register stages keep two tiles in flight while one is consumed.
template <int D>
struct KTile {
  static constexpr int ROWB = D * 2 + 16;          // padded LDS row (bytes)
  static constexpr int KEYS = 128;                 // keys per tile
  static constexpr int BYTES = KEYS * ROWB;
  static constexpr int PIECES = D / 8;             // 16-byte pieces per row
  static constexpr int LOADS = KEYS * PIECES / kThreads;  // per thread per tile
  static_assert(LOADS >= 1 && KEYS * PIECES % kThreads == 0, "tile split");
  typedef u32x4 Regs[LOADS];
};

// This thread's pieces of keys [tk0, tk0 + 128) into registers. Rows at or
// beyond kend repeat key kend - 1 (every consumer masks them): the loads stay
// unconditional, so the compiler can count them and wait only for the tile
// it stores while the next one is still in flight.
template <int D>
__device__ __forceinline__ void load_key_tile(typename KTile<D>::Regs& r, const uint16_t* kb,
                                              size_t tstride, int tk0, int kend, int tid) {
  using T = KTile<D>;
#pragma unroll
  for (int u = 0; u < T::LOADS; ++u) {
    const int pc = tid + u * kThreads;
    const int key = pc / T::PIECES, col = pc % T::PIECES;
    const int j = min(tk0 + key, kend - 1);
    r[u] = *reinterpret_cast<const u32x4*>(kb + (size_t)j * tstride + col * 8);
  }
}

template <int D>
__device__ __forceinline__ void store_key_tile(const typename KTile<D>::Regs& r,
                                               unsigned char* tile, int tid) {
  using T = KTile<D>;
#pragma unroll
  for (int u = 0; u < T::LOADS; ++u) {
    const int pc = tid + u * kThreads;
    const int key = pc / T::PIECES, col = pc % T::PIECES;
    *reinterpret_cast<u32x4*>(tile + key * T::ROWB + col * 16) = r[u];
  }
}

// MFMA fragments of key block kb (32 keys) of a staged tile: lane holds key
// kb*32 + (lane & 31), D elements 16*s + 8*(lane >> 5) .. +7 for k-step s.
template <int D, bool FENCE = true>
__device__ __forceinline__ void read_key_frags(bf16x8 (&kf)[D / 16], const unsigned char* tile,
                                               int kb, int lane) {
  using T = KTile<D>;
  const unsigned char* row = tile + (kb * 32 + (lane & 31)) * T::ROWB + (lane >> 5) * 16;
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    kf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(row + s * 32));
  // issue every fragment read before the MFMAs that consume them, instead of
  // one LDS round trip per MFMA (without FENCE the compiler schedules them
  // freely, e.g. under the previous block's exp2 work)
  if constexpr (FENCE) __builtin_amdgcn_sched_barrier(0);
}

// Stream the keys [key0, kend) of one head through two LDS tile buffers,
// with two more tiles in flight in registers. KeyStream::prefetch issues the
// loads of tile 0, and of tile 1 when deep (the caller may do other work
// while they fly, as long as it does not wait on global loads issued after
// them); run() then stores
// tile i to LDS, loads tile i + 2 into the freed registers, and after
// a barrier that makes tile i visible (and guarantees every wave is done with
// tile i - 1) calls after_barrier(i) and compute(tile, i). Global loads stay
// in flight across the barriers. The loads are unconditional (past the end
// they re-read key kend - 1) and the loop starts with compute, so every store
// waits only for its own registers.
template <int D>
struct KeyStream {
  using T = KTile<D>;
  typename T::Regs ra, rb;
  const uint16_t* kb;
  size_t tstride;
  int key0, kend;
  bool reverse = false;  // visit the tiles last to first
  bool deep = false;     // prefetch() requests the first two tiles

  __device__ __forceinline__ int ntiles() const { return (kend - key0 + T::KEYS - 1) / T::KEYS; }
  // first key of the i-th tile visited
  __device__ __forceinline__ int tile_key(int i) const {
    return key0 + (reverse ? ntiles() - 1 - i : i) * T::KEYS;
  }

  // The vote item requests only tile 0 up front (two measured slower
  // there). Every statistics pass (deep) requests tiles 0 and 1 while its
  // query rows are staged, which measured faster: the 128K layer's
  // streaming kernel and the ragged batch's statistics kernel by about 1%.
  __device__ __forceinline__ void prefetch() {
    load_key_tile<D>(ra, kb, tstride, tile_key(0), kend, threadIdx.x);
    if (deep) {
      asm volatile("" ::: "memory");  // tile 0's loads stay older than tile 1's
      load_key_tile<D>(rb, kb, tstride, tile_key(min(1, ntiles() - 1)), kend, threadIdx.x);
    }
  }

  template <typename Compute>
  __device__ __forceinline__ void run_resident(unsigned char (*slots)[T::BYTES],
                                               Compute&& compute);

  template <typename Compute, typename After>
  __device__ __forceinline__ void run(unsigned char (*ring)[T::BYTES], Compute&& compute,
                                      After&& after_barrier) {
    const int tid = threadIdx.x;
    const int ntiles = this->ntiles();
    // tiles past the end (visited indices >= ntiles) re-read a valid tile
    auto start = [&](int i) { return tile_key(min(i, ntiles - 1)); };
    store_key_tile<D>(ra, ring[0], tid);
    if (!deep) {  // else tile 1 is already in flight
      load_key_tile<D>(rb, kb, tstride, start(1), kend, tid);
      asm volatile("" ::: "memory");  // keep tile 1's loads older than tile 2's
    }
    load_key_tile<D>(ra, kb, tstride, start(2), kend, tid);
    lds_barrier();
    after_barrier(0);
    for (int i = 0;; i += 2) {
      compute(ring[0], i);
      if (i + 1 >= ntiles) break;
      store_key_tile<D>(rb, ring[1], tid);
      load_key_tile<D>(rb, kb, tstride, start(i + 3), kend, tid);
      lds_barrier();
      after_barrier(i + 1);
      compute(ring[1], i + 1);
      if (i + 2 >= ntiles) break;
      store_key_tile<D>(ra, ring[0], tid);
      load_key_tile<D>(ra, kb, tstride, start(i + 4), kend, tid);
      lds_barrier();
      after_barrier(i + 2);
    }
  }
};

// The same stream with every tile kept: tile i (in visit order) is stored
// to slots[i] and stays there after compute(slots[i], i) returns, so a later
// pass can read the chunk's keys from LDS. The caller provides one slot per
// tile.
template <int D>
template <typename Compute>
__device__ __forceinline__ void KeyStream<D>::run_resident(unsigned char (*slots)[T::BYTES],
                                                           Compute&& compute) {
  const int tid = threadIdx.x;
  const int ntiles = this->ntiles();
  auto start = [&](int i) { return tile_key(min(i, ntiles - 1)); };
  store_key_tile<D>(ra, slots[0], tid);
  if (!deep) {
    load_key_tile<D>(rb, kb, tstride, start(1), kend, tid);
    asm volatile("" ::: "memory");  // keep tile 1's loads older than tile 2's
  }
  load_key_tile<D>(ra, kb, tstride, start(2), kend, tid);
  lds_barrier();
  for (int i = 0;; i += 2) {
    compute(slots[i], i);
    if (i + 1 >= ntiles) break;
    store_key_tile<D>(rb, slots[i + 1], tid);
    load_key_tile<D>(rb, kb, tstride, start(i + 3), kend, tid);
    lds_barrier();
    compute(slots[i + 1], i + 1);
    if (i + 2 >= ntiles) break;
    store_key_tile<D>(ra, slots[i + 2], tid);
    load_key_tile<D>(ra, kb, tstride, start(i + 4), kend, tid);
    lds_barrier();
  }
}

// Query fragments of this wave's row tiles (same D-to-k-slot map as the
// keys), staged through LDS: the group's rows (contiguous in q_win) are read
// with whole-row coalesced loads, 128 rows per round, into `buf` laid out
// like a key tile, and each wave reads its row tiles' fragments from there.
// Rows at or beyond `rows` are zero. issue_next() runs right after the first
// round's loads are issued (the caller starts its key prefetch there: those
// loads are younger, so waiting for the query rows does not wait for them).
// Ends with a barrier after which `buf` may be reused.
template <int D, int RTW, typename Next>
__device__ __forceinline__ void stage_query_frags(bf16x8 (&qf)[RTW][D / 16], const uint16_t* qbase,
                                                  int rows, int rows_pad, int wr, int nwr,
                                                  int my_nrt, unsigned char* buf, Next&& issue_next) {
  using T = KTile<D>;
  constexpr int PIECES = T::PIECES;                 // 16-byte pieces per row
  constexpr int PER = T::KEYS * PIECES / kThreads;  // pieces per thread per round
  const int tid = threadIdx.x, lane = tid & 63;
#pragma unroll
  for (int t = 0; t < RTW; ++t)
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[t][s] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  for (int r0 = 0; r0 < rows_pad; r0 += T::KEYS) {
    u32x4 x[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int piece = tid + u * kThreads;
      const int row = r0 + piece / PIECES;
      x[u] = *reinterpret_cast<const u32x4*>(qbase + (size_t)min(row, rows - 1) * D +
                                             (piece % PIECES) * 8);
    }
    if (r0 == 0) {
      asm volatile("" ::: "memory");  // the query loads stay older than the caller's
      issue_next();
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int piece = tid + u * kThreads;
      const int row = piece / PIECES;
      const uint32_t keep = r0 + row < rows ? 0xFFFFFFFFu : 0u;
      *reinterpret_cast<u32x4*>(buf + row * T::ROWB + (piece % PIECES) * 16) =
          x[u] & u32x4{keep, keep, keep, keep};
    }
    lds_barrier();
#pragma unroll
    for (int t = 0; t < RTW; ++t) {
      const int rt = wr + nwr * t;  // row tile of this wave
      const int local = rt - r0 / 32;
      if (t < my_nrt && local >= 0 && local < T::KEYS / 32) read_key_frags<D>(qf[t], buf, local, lane);
    }
    lds_barrier();
  }
}

}  // namespace snapkv
