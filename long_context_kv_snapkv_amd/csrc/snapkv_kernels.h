// Internal interface between the host API (snapkv_api.cpp) and the gfx950
// kernels of the SnapKV compression path. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace snapkv {

constexpr int kMaxBatch = 256;
constexpr int kMaxRows = 512;      // G * W scored rows per KV head
constexpr int kMaxKernel = 2049;   // pooling kernel
constexpr int kThreads = 512;      // workgroup size of every kernel
constexpr int kKeyTile = 64;       // keys per LDS tile
constexpr int kMaxChunk = 8192;    // keys per scoring work item
constexpr int kTargetItems = 256;  // scoring items per call the chunk length aims at
constexpr int kMaxPairs = 512;     // (prompt, chunk) pairs of a compact scoring grid
constexpr int kGatherRows = 64;    // compressed rows per gather work item (at most)
constexpr int kTopHistBins = 2048; // bins of the selection's first radix digit
constexpr int kSegment = 256;      // positions per selection count-table entry
// per head: the selection's radix histograms of digits 1, 2 and 3 (2048,
// 2048 and 1024 bins), adjacent, then a first-digit histogram that the sliced
// selection recounts from the pooled scores when the score kernel's counts
// are not to be trusted (see PathParams::hist_bad)
constexpr int kHistD1 = 0, kHistD2 = 2048, kHistD3 = 4096, kHistFix = 5120;
constexpr int kHistCleared = kHistFix;  // words zeroed before each call's counting
constexpr int kSelHistWords = kHistFix + 2048;
constexpr int kSliceKeys = 4096;   // prefix positions per sliced-selection work item
constexpr int kSelectHeldKeys = 64 * kThreads;  // prefix positions one selection workgroup
                                                // keeps in registers (longer: sliced)
// fused score kernel (statistics and vote in one launch, key chunk resident
// in LDS): limits of the shapes it takes
constexpr int kFusedTiles = 4;                  // resident 128-key tiles per item
constexpr int kFusedChunk = kFusedTiles * 128;  // keys per item (at most)
constexpr int kFusedMaxHalo = 16;               // kernel / 2 (at most)
constexpr int kFusedMaxRows = 256;              // G * W rounded up to 32 (one row tile per wave)
constexpr int kSpinLimit = 1 << 20;             // polls of a fused item's bounded wait (~1 s)

// Size of the library's fixed scratch area (snapkv_compress_static).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
// Device address of that area on the current device (looked up on the first
// call for each device, then kept).
hipError_t static_scratch(void** ptr);

// Per-prompt table passed by value in the kernel arguments.
struct PromptTable {
  int32_t off[kMaxBatch];  // first packed token of prompt b
  int32_t len[kMaxBatch];  // L_b
};

// Everything the stages read, for one call. Passed by value (< 4 KiB).
struct PathParams {
  const uint16_t* q;  // bf16 [batch, Hq, W, D]
  const uint16_t* k;  // bf16 [T, Hkv, D]
  const uint16_t* v;  // bf16 [T, Hkv, D]
  uint16_t* out_k;    // bf16 [batch, Hkv, budget, D]
  uint16_t* out_v;
  int32_t* out_idx;   // [batch, Hkv, budget]
  // 4-bit or 8-bit storage (snapkv_compress_int4 / _fp8), else null: codes
  // [batch, Hkv, budget, D/2] (two's-complement nibbles, even element low) or
  // [batch, Hkv, budget, D] (FP8 E4M3 bytes), and per-row scales [batch, Hkv,
  // budget]
  uint8_t* out_kq;
  float* out_ks;
  uint8_t* out_vq;
  float* out_vs;
  float2* part;       // [batch, Hkv, nchunk, rows_pad] per-chunk (reference m, sum of
                      // 2^(x - m)) in log2 units
  float* pooled;      // [batch, Hkv, pooled_stride] pooled scores c_h[j], j < P
  const float* window_lse;  // [batch, Hq, W] caller's natural-log normaliser of each window
                            // row (snapkv_compress_from_lse), or null
  uint32_t* top_hist;   // [batch * Hkv, kSelHistWords] histograms of the pooled keys' radix
                        // digits: top 11 bits, next 11 bits, low 10 bits
  uint32_t* sel_table;  // [batch * Hkv, table_stride, 2] per kSegment positions: keys in the
                        // segment above / equal to the threshold
  uint32_t* sel_meta;   // [batch * Hkv, 4]: threshold key, keys equal to it kept, settled
  uint64_t* flags;      // [batch, Hkv, nchunk] fused score kernel: `epoch` once an item's
                        // row statistics are published
  uint64_t* hist_bad;   // [batch * Hkv] `epoch` when an item of the head added its counts to
                        // the first-digit histogram without having seen it cleared (a bounded
                        // wait gave up): the selection then recounts that digit itself
  uint64_t epoch;       // this call's mark (unique per call in the process)
  int32_t cooperative;  // launch the fused score kernels as cooperative launches
  int32_t spin_limit;   // polls before a fused score item stops waiting (kSpinLimit)
  int32_t batch, hq, hkv, window, group;
  int32_t rows, rows_pad;  // G*W and its round-up to 32
  int32_t nwr;             // waves that split the row tiles (power of two)
  int32_t chunk;           // keys per scoring item, multiple of kKeyTile
  int32_t nchunk;          // chunk slots per (prompt, head) in part
  int32_t pooled_stride;   // floats per pooled row (>= max P; a multiple of 64 in the workspace)
  int32_t table_stride;    // segments per head in sel_table (>= ceil(max P / kSegment))
  int32_t budget, kernel, pool_mode;
  int32_t score_all;       // 1: score every prompt with P >= 1; 0: only L > budget
  int32_t export_scores;   // 1: pooled rows are the caller's, zero past P
  int32_t n_gather_blocks; // gather items per (prompt, head)
  int32_t gather_rows;     // rows per gather item: kGatherRows, or half of it when
                           // there are few items (D = 128 only)
  int32_t sel_slices;      // 0: one selection workgroup per head; else kSliceKeys-position
                           // slices per head of the sliced selection
  int32_t sel_one_launch;  // sliced selection as one launch exchanging its histograms
  uint64_t* sel_flags;     // [batch * Hkv, 2, sel_slices] that launch: `epoch` once a slice's
                           // digit-2 (then digit-3) counts are added
  float* scores_out;       // snapkv_compress_with_scores: [batch, Hkv, scores_len] copy of
  int32_t scores_len;      // the pooled rows the selection read (0 where not compressed)
  float scale_log2;        // log2(e) / sqrt(D)
  // Compact scoring grid (npairs > 0): the score kernels run over (pair,
  // KV head), pair i being prompt pair[i] >> 8 and chunk pair[i] & 255, only
  // for the prompts the call scores; otherwise over (chunk, KV head, prompt)
  // with nchunk chunk slots for every prompt.
  int32_t npairs;
  uint16_t pair[kMaxPairs];
  PromptTable tab;
};
static_assert(sizeof(PathParams) <= 4096, "kernel arguments");

// Optional events recorded by the dispatch itself at the kernel's start and
// end (so they time the kernel alone, as a profiler's kernel trace does).
struct StageEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Stage kernels: grids of work items.
hipError_t launch_score_stats(const PathParams& p, int head_dim, hipStream_t stream,
                              StageEvents ev = {});
// with ext_lse the row normalisers come from PathParams::window_lse; with
// zero_first (ext_lse only, every item resident at once) the kernel also
// clears the selection histograms that snapkv_clear_hist would
hipError_t launch_score_vote(const PathParams& p, int head_dim, hipStream_t stream,
                             StageEvents ev = {}, bool ext_lse = false, bool zero_first = false);
// zeroes top_hist of the scored heads (stands in for the statistics pass,
// which does it otherwise)
hipError_t launch_clear_hist(const PathParams& p, hipStream_t stream, StageEvents ev = {});
// statistics and vote in one launch (head_dim 128 and the kFused* limits;
// every item of the grid must be able to be resident at once)
hipError_t launch_score_fused(const PathParams& p, int head_dim, hipStream_t stream,
                              StageEvents ev = {});
// statistics and vote in one launch with the keys streamed twice (any
// head_dim and row tiling; every item of the grid resident at once)
hipError_t launch_score_fused_stream(const PathParams& p, int head_dim, hipStream_t stream,
                                     StageEvents ev = {});
// one workgroup per head, or (sel_slices > 0) the sliced selection: one
// launch when every slice workgroup fits the device at once
// (sel_one_launch), else three kernels
hipError_t launch_select(const PathParams& p, hipStream_t stream, StageEvents ev = {});
// form 0: bf16 rows; 1: 4-bit, 2: FP8 E4M3 codes with per-row scales, through
// out_kq/out_ks/out_vq/out_vs
hipError_t launch_gather(const PathParams& p, int head_dim, hipStream_t stream,
                         StageEvents ev = {}, int form = 0);
// the gather with the selection inside each item (sel_slices == 0 only)
hipError_t launch_gather_select(const PathParams& p, int head_dim, hipStream_t stream,
                                StageEvents ev = {}, int form = 0);
// copy of the pooled rows of compressed prompts to p.scores_out (zeros elsewhere)
hipError_t launch_export_pooled(const PathParams& p, hipStream_t stream);

}  // namespace snapkv
