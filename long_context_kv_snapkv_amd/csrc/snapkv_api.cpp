// Host side of the SnapKV compression library: argument validation, the
// workspace plan, and the launches on the caller's stream. Every check runs
// before the first HIP call, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>

#include "snapkv.h"
#include "snapkv_decode.h"
#include "snapkv_kernels.h"
#include "snapkv_prefill.h"

static_assert(SNAPKV_STATIC_SCRATCH_BYTES == snapkv::kStaticScratchBytes,
              "static scratch size in the header and the library");

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

const char* const kStageNames[SNAPKV_NUM_STAGES] = {"snapkv_score_stats", "snapkv_score_vote",
                                                    "snapkv_select", "snapkv_gather"};

int largest_pow2_at_most(int x) {
  int p = 1;
  while (p * 2 <= x) p *= 2;
  return p;
}

// Everything a call needs, derived from shapes alone, so the workspace size
// computed ahead of a call matches the call. Workspace layout:
//   top_hist  uint32[batch * H_kv, 5120]            radix-digit histograms per head
//   sel_table uint32[batch * H_kv, t_stride, 2]     per-segment counts
//   sel_meta  uint32[batch * H_kv, 4]               threshold of each head
//   part      float2[batch, H_kv, nchunk, rows_pad]  per-chunk row statistics
//   flags     uint64[batch, H_kv, nchunk]       fused score kernel: published items
//   sflags    uint64[batch * H_kv, 2, slices]   one-launch sliced selection: published
//                                                digit counts (slices = 0 for short prefixes)
//   hist_bad  uint64[batch * H_kv]               call whose first-digit counts are untrusted
//   pooled    float [batch, H_kv, p_stride]      pooled scores, p_stride =
//                                                max P rounded up to 64
// Every word is written by a call before that call reads it, except flags,
// sflags and hist_bad, which only count when they hold the call's own epoch.
struct Plan {
  int batch, hq, hkv, d, window, group, rows, rows_pad, nrt, nwr;
  int chunk, nchunk, l_max, p_max, p_stride;
  int scored_pairs;  // (prompt, chunk) pairs of the prompts longer than the window
  bool compact;      // the score kernels can run over a compact (pair, head) grid
  size_t off_top, off_table, off_meta, off_part, off_flags, off_sflags, off_bad, off_pooled, bytes;
  int t_stride;
  snapkv::PromptTable tab;
};

int32_t make_plan(int32_t batch, int32_t hq, int32_t hkv, int32_t d, const int32_t* seq_lens,
                  int32_t window, Plan* pl) {
  if (seq_lens == nullptr) return fail(SNAPKV_ERR_INVALID_ARGUMENT, "seq_lens is NULL");
  if (batch < 1 || batch > SNAPKV_MAX_BATCH)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT,
                "batch must be in [1, " + std::to_string(SNAPKV_MAX_BATCH) + "], got " +
                    std::to_string(batch));
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT,
                "num_q_heads must be a positive multiple of num_kv_heads (" +
                    std::to_string(hq) + " vs " + std::to_string(hkv) + ")");
  if (window < 1) return fail(SNAPKV_ERR_INVALID_ARGUMENT, "window must be >= 1");
  if (d != 64 && d != 128)
    return fail(SNAPKV_ERR_UNSUPPORTED, "head_dim must be 64 or 128, got " + std::to_string(d));
  const int64_t group = hq / hkv;
  if (group * window > SNAPKV_MAX_ROWS)
    return fail(SNAPKV_ERR_UNSUPPORTED, "num_q_heads / num_kv_heads * window must be <= " +
                                            std::to_string(SNAPKV_MAX_ROWS));
  if ((int64_t)batch * hkv > (1 << 20))
    return fail(SNAPKV_ERR_UNSUPPORTED, "batch * num_kv_heads must be <= 2^20");
  int64_t total = 0, key_sum = 0;
  int l_max = 0;
  for (int b = 0; b < batch; ++b) {
    const int32_t L = seq_lens[b];
    if (L < 1)
      return fail(SNAPKV_ERR_INVALID_ARGUMENT,
                  "seq_lens[" + std::to_string(b) + "] must be >= 1, got " + std::to_string(L));
    pl->tab.off[b] = (int32_t)total;
    pl->tab.len[b] = L;
    total += L;
    if (total > INT32_MAX) return fail(SNAPKV_ERR_INVALID_ARGUMENT, "more than 2^31-1 tokens");
    if (L > window) key_sum += L;
    l_max = L > l_max ? L : l_max;
  }
  for (int b = batch; b < snapkv::kMaxBatch; ++b) pl->tab.off[b] = pl->tab.len[b] = 0;
  pl->batch = batch;
  pl->hq = hq;
  pl->hkv = hkv;
  pl->d = d;
  pl->window = window;
  pl->group = (int)group;
  pl->rows = (int)(group * window);
  pl->rows_pad = (pl->rows + 31) / 32 * 32;
  pl->nrt = pl->rows_pad / 32;
  pl->nwr = largest_pow2_at_most(pl->nrt < 8 ? pl->nrt : 8);
  // keys per scoring item: about kTargetItems items over the whole call (one
  // per CU and phase), 64-key granularity, 256 .. kMaxChunk keys: the
  // shortest chunk with which the prompts longer than the window form at
  // most kTargetItems (prompt, chunk, KV head) items, so that a ragged
  // batch's items run in one round rather than spilling into a second
  auto pairs_for = [&](int64_t c) {
    int64_t n = 0;
    for (int b = 0; b < batch; ++b)
      if (seq_lens[b] > window) n += (seq_lens[b] + c - 1) / c;
    return n;
  };
  int64_t chunk = (key_sum * hkv + snapkv::kTargetItems - 1) / snapkv::kTargetItems;
  chunk = (chunk + snapkv::kKeyTile - 1) / snapkv::kKeyTile * snapkv::kKeyTile;
  if (chunk < 256) chunk = 256;
  while (chunk < snapkv::kMaxChunk && pairs_for(chunk) * hkv > snapkv::kTargetItems)
    chunk += snapkv::kKeyTile;
  if (chunk > snapkv::kMaxChunk) chunk = snapkv::kMaxChunk;
  pl->chunk = (int)chunk;
  pl->nchunk = (int)((l_max + chunk - 1) / chunk);
  pl->scored_pairs = (int)pairs_for(chunk);
  // pair entries hold the chunk in 8 bits; an export adds one entry for each
  // prompt not longer than the window (it zeroes that prompt's row)
  pl->compact = pl->nchunk <= 256 && pl->scored_pairs + batch <= snapkv::kMaxPairs;
  pl->l_max = l_max;
  pl->p_max = l_max - window > 1 ? l_max - window : 1;
  pl->p_stride = (int)align_up((size_t)pl->p_max, 64);
  const size_t heads = (size_t)batch * hkv;
  size_t off = 0;
  pl->off_top = off;
  off = align_up(off + heads * snapkv::kSelHistWords * sizeof(uint32_t), 256);
  pl->t_stride = (pl->p_stride + snapkv::kSegment - 1) / snapkv::kSegment;
  pl->off_table = off;
  off = align_up(off + heads * pl->t_stride * 2 * sizeof(uint32_t), 256);
  pl->off_meta = off;
  off = align_up(off + heads * 4 * sizeof(uint32_t), 256);
  pl->off_part = off;
  off = align_up(off + heads * pl->nchunk * pl->rows_pad * sizeof(float2), 256);
  pl->off_flags = off;
  off = align_up(off + heads * pl->nchunk * sizeof(uint64_t), 256);
  pl->off_sflags = off;
  const int64_t slices = pl->p_max > snapkv::kSelectHeldKeys
                             ? (pl->p_max + snapkv::kSliceKeys - 1) / snapkv::kSliceKeys
                             : 0;
  off = align_up(off + heads * 2 * slices * sizeof(uint64_t), 256);
  pl->off_bad = off;
  off = align_up(off + heads * sizeof(uint64_t), 256);
  pl->off_pooled = off;
  off = align_up(off + heads * pl->p_stride * sizeof(float), 256);
  pl->bytes = off;
  return SNAPKV_OK;
}

int32_t check_pool(int32_t kernel, int32_t pool_mode) {
  if (kernel < 1 || kernel % 2 == 0)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT,
                "kernel_size must be odd and >= 1, got " + std::to_string(kernel));
  if (kernel > SNAPKV_MAX_KERNEL)
    return fail(SNAPKV_ERR_UNSUPPORTED,
                "kernel_size must be <= " + std::to_string(SNAPKV_MAX_KERNEL));
  if (pool_mode != SNAPKV_POOL_AVG && pool_mode != SNAPKV_POOL_MAX)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "unknown pool_mode " + std::to_string(pool_mode));
  return SNAPKV_OK;
}

// Gather items and the selection's layout for a budget: half-size gather
// items (D = 128) when full ones would leave CUs idle (fewer than about two
// per CU over the call); prefixes longer than one selection workgroup holds
// in registers are spread over workgroups of kSliceKeys positions.
void gather_plan(const Plan& pl, int32_t budget, snapkv::PathParams* p) {
  p->budget = budget;
  const int full_items =
      budget > 0 ? pl.batch * pl.hkv * ((budget + snapkv::kGatherRows - 1) / snapkv::kGatherRows)
                 : 0;
  p->gather_rows =
      pl.d == 128 && full_items < 512 ? snapkv::kGatherRows / 2 : snapkv::kGatherRows;
  p->n_gather_blocks = budget > 0 ? (budget + p->gather_rows - 1) / p->gather_rows : 0;
  p->sel_slices = pl.p_max > snapkv::kSelectHeldKeys
                      ? (pl.p_max + snapkv::kSliceKeys - 1) / snapkv::kSliceKeys
                      : 0;
}

snapkv::PathParams path_params(const Plan& pl, const void* q, const void* k, const void* v,
                               void* ws, int32_t budget, int32_t kernel, int32_t pool_mode,
                               bool score_all) {
  snapkv::PathParams p{};
  std::memset(&p, 0, sizeof(p));
  char* w = static_cast<char*>(ws);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.top_hist = reinterpret_cast<uint32_t*>(w + pl.off_top);
  p.sel_table = reinterpret_cast<uint32_t*>(w + pl.off_table);
  p.sel_meta = reinterpret_cast<uint32_t*>(w + pl.off_meta);
  p.table_stride = pl.t_stride;
  p.part = reinterpret_cast<float2*>(w + pl.off_part);
  p.flags = reinterpret_cast<uint64_t*>(w + pl.off_flags);
  p.sel_flags = reinterpret_cast<uint64_t*>(w + pl.off_sflags);
  p.hist_bad = reinterpret_cast<uint64_t*>(w + pl.off_bad);
  p.pooled = reinterpret_cast<float*>(w + pl.off_pooled);
  p.pooled_stride = pl.p_stride;
  p.batch = pl.batch;
  p.hq = pl.hq;
  p.hkv = pl.hkv;
  p.window = pl.window;
  p.group = pl.group;
  p.rows = pl.rows;
  p.rows_pad = pl.rows_pad;
  p.nwr = pl.nwr;
  p.chunk = pl.chunk;
  p.nchunk = pl.nchunk;
  p.budget = budget;
  p.kernel = kernel;
  p.pool_mode = pool_mode;
  p.score_all = score_all ? 1 : 0;
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)pl.d));
  p.tab = pl.tab;
  // the compact scoring grid: every chunk of each prompt this call scores
  // (with score_all, an export, also chunk 0 of the other prompts, whose
  // rows the vote kernel zeroes)
  p.npairs = 0;
  if (pl.compact) {
    int n = 0;
    for (int b = 0; b < pl.batch; ++b) {
      const int L = pl.tab.len[b];
      if (L - pl.window >= 1 && (score_all || L > budget)) {
        for (int c = 0; c * pl.chunk < L; ++c) p.pair[n++] = (uint16_t)(b << 8 | c);
      } else if (score_all) {
        p.pair[n++] = (uint16_t)(b << 8);
      }
    }
    p.npairs = n;
  }
  gather_plan(pl, budget, &p);
  return p;
}

// Compute units of the current device (0 if unknown), cached per device.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Marks of a call (the fused score kernels' publication flags, the
// untrusted-histogram word): unique per call in this process and started at
// a random odd value, so neither an earlier call's marks nor stale memory in
// a fresh workspace can match.
uint64_t next_epoch() {
  static std::atomic<uint64_t> counter{[] {
    std::random_device rd;
    const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    return ((((uint64_t)rd() << 32) ^ (uint64_t)rd() ^ (t * 0x9E3779B97F4A7C15ull)) | 1ull);
  }()};
  return counter.fetch_add(2, std::memory_order_relaxed);
}

// SNAPKV_NO_FUSED_SCORE set to a non-empty value other than "0" at the call
// turns the one-launch forms off (two kernels); SNAPKV_COOPERATIVE launches
// them as cooperative kernels (the runtime then guarantees co-residency even
// with other work on the device, at a cost of about 19 us per call).
// Whether environment variable `name` is set to a non-empty value other
// than "0" (read at every call, so a process can compare both paths).
bool env_flag(const char* name) {
  const char* e = std::getenv(name);
  return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
}

// How the statistics and the vote run: two kernels, or one launch whose
// items exchange the statistics (every item of the grid resident at once,
// one workgroup per CU), keeping a chunk's keys in LDS when they fit
// (head_dim 128, one row tile per wave, at most 512 keys, a halo of at most
// 16 keys) and streaming them twice otherwise. One row tile per wave needs
// the window rows to form a power-of-two number of row tiles (at most 8):
// 3, 5, 6 or 7 tiles give some waves two, which the streaming form handles.
enum class Scoring { kTwoKernels, kFusedResident, kFusedStream };

// Workgroups of the score kernels' grid (an upper bound for a call that
// scores fewer prompts: the compact grid then has fewer pairs).
int64_t score_items(const Plan& pl) {
  return pl.compact ? (int64_t)pl.scored_pairs * pl.hkv : (int64_t)pl.nchunk * pl.hkv * pl.batch;
}

Scoring scoring_plan(const Plan& pl, int32_t kernel) {
  if (env_flag("SNAPKV_NO_FUSED_SCORE") || pl.nchunk > snapkv::kThreads)
    return Scoring::kTwoKernels;
  const int64_t items = score_items(pl);
  const int cus = device_cus();
  if (cus <= 0 || items > cus) return Scoring::kTwoKernels;
  if (pl.d == 128 && pl.rows_pad <= snapkv::kFusedMaxRows && pl.nrt == pl.nwr &&
      pl.chunk <= snapkv::kFusedChunk && kernel / 2 <= snapkv::kFusedMaxHalo)
    return Scoring::kFusedResident;
  return Scoring::kFusedStream;
}

// The selection inside the gather (snapkv_gather_select): every prefix fits
// one workgroup's registers and the whole gather grid fits the device at
// once, with 64-row items if 32-row ones would not. Sets p->gather_rows and
// p->n_gather_blocks for the chosen items. SNAPKV_NO_FUSED_SELECT set to a
// non-empty value other than "0" turns it off.
// Polls before a fused score item stops waiting for its head: kSpinLimit
// (about a second), or SNAPKV_SPIN_LIMIT (read at every call, 0 .. the
// default) to exercise the give-up path.
int32_t spin_limit() {
  const char* e = std::getenv("SNAPKV_SPIN_LIMIT");
  if (e == nullptr || e[0] == '\0') return snapkv::kSpinLimit;
  char* end = nullptr;
  const long v = std::strtol(e, &end, 10);
  if (end == e || v < 0 || v > snapkv::kSpinLimit) return snapkv::kSpinLimit;
  return (int32_t)v;
}

// The sliced selection in one launch (its slice workgroups exchange the
// digit histograms through flags, with a bounded wait): when every slice
// workgroup of the call fits the device at once. SNAPKV_NO_FUSED_SELECT
// turns it off too (three kernels).
bool use_one_launch_slices(const Plan& pl, const snapkv::PathParams& p) {
  if (p.sel_slices == 0 || p.sel_slices > snapkv::kThreads || env_flag("SNAPKV_NO_FUSED_SELECT"))
    return false;
  const int cus = device_cus();
  return cus > 0 && (int64_t)p.sel_slices * pl.hkv * pl.batch <= cus;
}

bool use_select_in_gather(const Plan& pl, snapkv::PathParams* p) {
  const bool disabled = env_flag("SNAPKV_NO_FUSED_SELECT");
  if (disabled || p->sel_slices != 0 || p->budget <= 0) return false;
  const int cus = device_cus();
  if (cus <= 0) return false;
  for (int rows : {p->gather_rows, snapkv::kGatherRows}) {
    const int64_t blocks = (p->budget + rows - 1) / rows;
    if (blocks * pl.hkv * pl.batch <= cus) {
      p->gather_rows = rows;
      p->n_gather_blocks = (int)blocks;
      return true;
    }
  }
  return false;
}

// Every scoring item of the call fits the device one workgroup per CU (the
// vote kernel with the caller's normalisers then clears the histograms
// itself); SNAPKV_NO_FUSED_SCORE turns that off too.
bool votes_resident(const Plan& pl) {
  if (env_flag("SNAPKV_NO_FUSED_SCORE") || pl.nchunk > snapkv::kThreads) return false;
  const int cus = device_cus();
  return cus > 0 && score_items(pl) <= cus;
}

bool any_scored(const Plan& pl, int32_t budget, bool score_all) {
  for (int b = 0; b < pl.batch; ++b) {
    const int L = pl.tab.len[b];
    if (L - pl.window >= 1 && (score_all || L > budget)) return true;
  }
  return false;
}

int32_t hip_fail(hipError_t e, const char* what) {
  return fail(SNAPKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int32_t check_tensors(const void* q_win, const void* k, const void* v, const void* out_k,
                      const void* out_v, const void* out_idx) {
  if (!q_win || !k || !v || !out_k || !out_v || !out_idx)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "a tensor pointer is NULL");
  if (misaligned(q_win) || misaligned(k) || misaligned(v) || misaligned(out_k) ||
      misaligned(out_v) || misaligned(out_idx))
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
  return SNAPKV_OK;
}

// Output buffers of the 4-bit and 8-bit forms (snapkv_compress_int4 / _fp8).
struct QuantOut {
  uint8_t* kq;
  float* ks;
  uint8_t* vq;
  float* vs;
  int form;  // 1: 4-bit, 2: FP8 E4M3
};

// Export of the pooled rows the selection read (snapkv_compress_with_scores).
struct ScoresOut {
  float* scores;
  int32_t len;
};

int32_t compress_impl(int32_t batch, int32_t hq, int32_t hkv, int32_t d, const void* q_win,
                      const void* k, const void* v, const int32_t* seq_lens, int32_t window,
                      int32_t kernel, int32_t pool_mode, int32_t budget, void* out_k,
                      void* out_v, int32_t* out_idx, void* workspace, size_t workspace_bytes,
                      void* stream, void* const* stage_events, const float* window_lse,
                      const QuantOut* q4 = nullptr, const ScoresOut* so = nullptr) {
  int32_t st = q4 ? check_tensors(q_win, k, v, q4->kq, q4->vq, out_idx)
                  : check_tensors(q_win, k, v, out_k, out_v, out_idx);
  if (st != SNAPKV_OK) return st;
  if (q4 && (!q4->ks || !q4->vs || misaligned(q4->ks) || misaligned(q4->vs)))
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "scale buffers must be non-null and 16-byte aligned");
  Plan pl;
  st = make_plan(batch, hq, hkv, d, seq_lens, window, &pl);
  if (st != SNAPKV_OK) return st;
  if (budget <= window)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "budget must exceed window (it includes the window)");
  st = check_pool(kernel, pool_mode);
  if (st != SNAPKV_OK) return st;
  if (so != nullptr) {
    if (so->scores == nullptr || misaligned(so->scores))
      return fail(SNAPKV_ERR_INVALID_ARGUMENT, "out_scores must be non-null and 16-byte aligned");
    if (so->len < pl.p_max)
      return fail(SNAPKV_ERR_INVALID_ARGUMENT,
                  "scores_len must be >= max(seq_len) - window = " + std::to_string(pl.p_max));
  }
  if (workspace == nullptr || workspace_bytes < pl.bytes || misaligned(workspace))
    return fail(SNAPKV_ERR_WORKSPACE, "workspace must be 16-byte aligned and hold " +
                                          std::to_string(pl.bytes) + " bytes");
  hipStream_t s = static_cast<hipStream_t>(stream);
  snapkv::PathParams p =
      path_params(pl, q_win, k, v, workspace, budget, kernel, pool_mode, /*score_all=*/false);
  p.out_k = static_cast<uint16_t*>(out_k);
  p.out_v = static_cast<uint16_t*>(out_v);
  if (q4) {
    p.out_kq = q4->kq;
    p.out_ks = q4->ks;
    p.out_vq = q4->vq;
    p.out_vs = q4->vs;
  }
  p.out_idx = out_idx;
  p.window_lse = window_lse;
  p.epoch = next_epoch();
  p.spin_limit = spin_limit();
  const bool ext_lse = window_lse != nullptr;
  hipError_t e;
  // optional caller events, recorded by each stage's dispatch at the
  // kernel's start and end (snapkv_compress_staged); a stage that has no
  // work records both events back to back
  hipEvent_t const* ev = reinterpret_cast<hipEvent_t const*>(stage_events);
  auto events = [&](int stage) {
    snapkv::StageEvents e;
    if (ev) {
      e.start = ev[2 * stage];
      e.stop = ev[2 * stage + 1];
    }
    return e;
  };
  auto skip = [&](int stage) {
    if (ev) {
      (void)hipEventRecord(ev[2 * stage], s);
      (void)hipEventRecord(ev[2 * stage + 1], s);
    }
  };
  const bool scored = any_scored(pl, budget, false);
  if (!scored) {
    skip(0);
    skip(1);
    skip(2);
  } else {
    const Scoring sc = ext_lse ? Scoring::kTwoKernels : scoring_plan(pl, kernel);
    if (sc != Scoring::kTwoKernels) {
      // statistics and vote in one launch (stage 0); stage 1 is empty
      p.cooperative = env_flag("SNAPKV_COOPERATIVE") ? 1 : 0;
      if (sc == Scoring::kFusedResident) {
        if ((e = snapkv::launch_score_fused(p, d, s, events(0))) != hipSuccess)
          return hip_fail(e, "snapkv_score_fused launch");
      } else if ((e = snapkv::launch_score_fused_stream(p, d, s, events(0))) != hipSuccess) {
        return hip_fail(e, "snapkv_score_fused_stream launch");
      }
      skip(1);
    } else {
      // the caller's normalisers replace the statistics pass, which would
      // also have cleared the vote's digit histograms: a clearing kernel, or
      // (every vote item resident at once) the vote kernel's item 0 per head
      const bool zero_first = ext_lse && votes_resident(pl);
      if (zero_first) {
        skip(0);
      } else if (ext_lse) {
        if ((e = snapkv::launch_clear_hist(p, s, events(0))) != hipSuccess)
          return hip_fail(e, "snapkv_clear_hist launch");
      } else if ((e = snapkv::launch_score_stats(p, d, s, events(0))) != hipSuccess) {
        return hip_fail(e, "snapkv_score_stats launch");
      }
      if ((e = snapkv::launch_score_vote(p, d, s, events(1), ext_lse, zero_first)) != hipSuccess)
        return hip_fail(e, "snapkv_score_vote launch");
    }
  }
  // the selection inside the gather (stage 2 then has no work), or its own
  // kernel before the gather
  const bool sel_in_gather = scored && use_select_in_gather(pl, &p);
  if (scored && !sel_in_gather) {
    p.sel_one_launch = use_one_launch_slices(pl, p) ? 1 : 0;
    if ((e = snapkv::launch_select(p, s, events(2))) != hipSuccess)
      return hip_fail(e, "snapkv_select launch");
  } else if (scored) {
    skip(2);
  }
  if (sel_in_gather) {
    if ((e = snapkv::launch_gather_select(p, d, s, events(3), q4 ? q4->form : 0)) != hipSuccess)
      return hip_fail(e, "snapkv_gather_select launch");
  } else if ((e = snapkv::launch_gather(p, d, s, events(3), q4 ? q4->form : 0)) != hipSuccess) {
    return hip_fail(e, "snapkv_gather launch");
  }
  if (so != nullptr) {
    p.scores_out = so->scores;
    p.scores_len = so->len;
    if ((e = snapkv::launch_export_pooled(p, s)) != hipSuccess)
      return hip_fail(e, "snapkv_export_pooled launch");
  }
  return SNAPKV_OK;
}

// Decode step: rows per prompt, chunking and workspace, from shapes alone.
//   part     float[batch * H_kv, nchunk, G, D + 2]  per-chunk partial softmax
//   flags    uint64[batch * H_kv, 16]              one-launch form's chunk marks
// The one-launch form is taken when no prompt has more than
// kDecodeFusedMaxChunks chunks (SNAPKV_NO_FUSED_DECODE turns it off).
struct DecodePlan {
  int batch, hq, hkv, d, group, layout, capacity, chunk, nchunk, fused;
  size_t off_flags, bytes;
  int32_t off[snapkv::kMaxBatch], len[snapkv::kMaxBatch];
};

int32_t make_decode_plan(int32_t batch, int32_t hq, int32_t hkv, int32_t d, int32_t layout,
                         int32_t capacity, const int32_t* cache_lens, DecodePlan* pl) {
  if (cache_lens == nullptr) return fail(SNAPKV_ERR_INVALID_ARGUMENT, "cache_lens is NULL");
  if (batch < 1 || batch > SNAPKV_MAX_BATCH)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT,
                "batch must be in [1, " + std::to_string(SNAPKV_MAX_BATCH) + "]");
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT,
                "num_q_heads must be a positive multiple of num_kv_heads");
  if (layout != SNAPKV_CACHE_COMPRESSED && layout != SNAPKV_CACHE_PACKED)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "unknown cache layout " + std::to_string(layout));
  if (layout == SNAPKV_CACHE_COMPRESSED && capacity < 1)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "capacity must be >= 1");
  if (d != 64 && d != 128)
    return fail(SNAPKV_ERR_UNSUPPORTED, "head_dim must be 64 or 128, got " + std::to_string(d));
  if (hq / hkv > snapkv::kDecodeMaxGroup)
    return fail(SNAPKV_ERR_UNSUPPORTED, "num_q_heads / num_kv_heads must be <= " +
                                            std::to_string(snapkv::kDecodeMaxGroup));
  if ((int64_t)batch * hkv > (1 << 20))
    return fail(SNAPKV_ERR_UNSUPPORTED, "batch * num_kv_heads must be <= 2^20");
  int64_t total = 0, rows = 0;
  int n_max = 0;
  for (int b = 0; b < batch; ++b) {
    const int32_t n = cache_lens[b];
    if (n < 1)
      return fail(SNAPKV_ERR_INVALID_ARGUMENT,
                  "cache_lens[" + std::to_string(b) + "] must be >= 1, got " + std::to_string(n));
    if (layout == SNAPKV_CACHE_COMPRESSED && n > capacity)
      return fail(SNAPKV_ERR_INVALID_ARGUMENT,
                  "cache_lens[" + std::to_string(b) + "] exceeds the capacity");
    pl->off[b] = (int32_t)total;
    pl->len[b] = n;
    total += n;
    if (total > INT32_MAX) return fail(SNAPKV_ERR_INVALID_ARGUMENT, "more than 2^31-1 rows");
    rows += n;
    n_max = n > n_max ? n : n_max;
  }
  for (int b = batch; b < snapkv::kMaxBatch; ++b) pl->off[b] = pl->len[b] = 0;
  pl->batch = batch;
  pl->hq = hq;
  pl->hkv = hkv;
  pl->d = d;
  pl->group = hq / hkv;
  pl->layout = layout;
  pl->capacity = layout == SNAPKV_CACHE_COMPRESSED ? capacity : 0;
  // rows per work item: about 1024 items over the call (four per CU), in
  // multiples of 128 rows, 128 .. 8192
  const int64_t q = snapkv::kDecodeRowQuantum;
  int64_t chunk = (rows * hkv + 1023) / 1024;
  chunk = (chunk + q - 1) / q * q;
  if (chunk < q) chunk = q;
  if (chunk > 8192) chunk = 8192;
  pl->chunk = (int)chunk;
  pl->nchunk = (int)((n_max + chunk - 1) / chunk);
  pl->fused = pl->nchunk <= snapkv::kDecodeFusedMaxChunks && !env_flag("SNAPKV_NO_FUSED_DECODE");
  pl->off_flags = align_up(
      (size_t)batch * hkv * pl->nchunk * pl->group * (d + 2) * sizeof(float), 256);
  pl->bytes = align_up(pl->off_flags + (size_t)batch * hkv * snapkv::kDecodeFusedMaxChunks *
                                           sizeof(uint64_t),
                       256);
  return SNAPKV_OK;
}

}  // namespace

extern "C" {

int32_t snapkv_score_kernels(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, const int32_t* seq_lens, int32_t window,
                             int32_t kernel_size, int32_t* kernels) {
  if (kernels == nullptr) return fail(SNAPKV_ERR_INVALID_ARGUMENT, "kernels is NULL");
  Plan pl;
  int32_t st = make_plan(batch, num_q_heads, num_kv_heads, head_dim, seq_lens, window, &pl);
  if (st != SNAPKV_OK) return st;
  st = check_pool(kernel_size, SNAPKV_POOL_AVG);
  if (st != SNAPKV_OK) return st;
  const Scoring sc = scoring_plan(pl, kernel_size);
  *kernels = sc == Scoring::kTwoKernels ? 2 : (sc == Scoring::kFusedResident ? 1 : 3);
  return SNAPKV_OK;
}

int32_t snapkv_gather_selects(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, const int32_t* seq_lens, int32_t window,
                              int32_t budget, int32_t* fused) {
  if (fused == nullptr) return fail(SNAPKV_ERR_INVALID_ARGUMENT, "fused is NULL");
  Plan pl;
  const int32_t st = make_plan(batch, num_q_heads, num_kv_heads, head_dim, seq_lens, window, &pl);
  if (st != SNAPKV_OK) return st;
  if (budget <= window)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "budget must exceed window (it includes the window)");
  snapkv::PathParams p{};
  gather_plan(pl, budget, &p);
  *fused = any_scored(pl, budget, false) && use_select_in_gather(pl, &p) ? 1 : 0;
  return SNAPKV_OK;
}

int32_t snapkv_select_kernels(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, const int32_t* seq_lens, int32_t window,
                              int32_t budget, int32_t* kernels) {
  if (kernels == nullptr) return fail(SNAPKV_ERR_INVALID_ARGUMENT, "kernels is NULL");
  Plan pl;
  const int32_t st = make_plan(batch, num_q_heads, num_kv_heads, head_dim, seq_lens, window, &pl);
  if (st != SNAPKV_OK) return st;
  if (budget <= window)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "budget must exceed window (it includes the window)");
  snapkv::PathParams p{};
  gather_plan(pl, budget, &p);
  if (!any_scored(pl, budget, false) || use_select_in_gather(pl, &p))
    *kernels = 0;
  else if (p.sel_slices == 0)
    *kernels = 1;
  else
    *kernels = use_one_launch_slices(pl, p) ? 2 : 3;
  return SNAPKV_OK;
}

int32_t snapkv_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, const int32_t* seq_lens, int32_t window,
                              size_t* bytes) {
  if (bytes == nullptr) return fail(SNAPKV_ERR_INVALID_ARGUMENT, "bytes is NULL");
  Plan pl;
  const int32_t st = make_plan(batch, num_q_heads, num_kv_heads, head_dim, seq_lens, window, &pl);
  if (st != SNAPKV_OK) return st;
  *bytes = pl.bytes;
  return SNAPKV_OK;
}

int32_t snapkv_compress(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, const void* q_win, const void* k, const void* v,
                        const int32_t* seq_lens, int32_t window, int32_t kernel_size,
                        int32_t pool_mode, int32_t budget, void* out_k, void* out_v,
                        int32_t* out_idx, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return compress_impl(batch, num_q_heads, num_kv_heads, head_dim, q_win, k, v, seq_lens, window,
                       kernel_size, pool_mode, budget, out_k, out_v, out_idx, workspace,
                       workspace_bytes, stream, nullptr, nullptr);
}

int32_t snapkv_compress_from_lse(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, const void* q_win, const void* k,
                                 const void* v, const int32_t* seq_lens, int32_t window,
                                 const float* window_lse, int32_t kernel_size,
                                 int32_t pool_mode, int32_t budget, void* out_k, void* out_v,
                                 int32_t* out_idx, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (window_lse == nullptr) return fail(SNAPKV_ERR_INVALID_ARGUMENT, "window_lse is NULL");
  if ((reinterpret_cast<uintptr_t>(window_lse) & 3u) != 0)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "window_lse must be 4-byte aligned");
  return compress_impl(batch, num_q_heads, num_kv_heads, head_dim, q_win, k, v, seq_lens, window,
                       kernel_size, pool_mode, budget, out_k, out_v, out_idx, workspace,
                       workspace_bytes, stream, nullptr, window_lse);
}

int32_t snapkv_compress_static(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, const void* q_win, const void* k, const void* v,
                               const int32_t* seq_lens, int32_t window, int32_t kernel_size,
                               int32_t pool_mode, int32_t budget, void* out_k, void* out_v,
                               int32_t* out_idx, void* stream) {
  // host checks first: a call the fixed area cannot serve enqueues nothing
  int32_t st = check_tensors(q_win, k, v, out_k, out_v, out_idx);
  if (st != SNAPKV_OK) return st;
  Plan pl;
  st = make_plan(batch, num_q_heads, num_kv_heads, head_dim, seq_lens, window, &pl);
  if (st != SNAPKV_OK) return st;
  if (budget <= window)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "budget must exceed window (it includes the window)");
  st = check_pool(kernel_size, pool_mode);
  if (st != SNAPKV_OK) return st;
  if (pl.bytes > snapkv::kStaticScratchBytes)
    return fail(SNAPKV_ERR_WORKSPACE, "this shape needs " + std::to_string(pl.bytes) +
                                          " bytes of scratch; the static area holds " +
                                          std::to_string(snapkv::kStaticScratchBytes));
  void* ws = nullptr;
  const hipError_t e = snapkv::static_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "static scratch lookup");
  return compress_impl(batch, num_q_heads, num_kv_heads, head_dim, q_win, k, v, seq_lens, window,
                       kernel_size, pool_mode, budget, out_k, out_v, out_idx, ws,
                       snapkv::kStaticScratchBytes, stream, nullptr, nullptr);
}

int32_t snapkv_compress_with_scores(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, const void* q_win, const void* k,
                                    const void* v, const int32_t* seq_lens, int32_t window,
                                    const float* window_lse, int32_t kernel_size,
                                    int32_t pool_mode, int32_t budget, void* out_k, void* out_v,
                                    int32_t* out_idx, float* out_scores, int32_t scores_len,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (window_lse != nullptr && (reinterpret_cast<uintptr_t>(window_lse) & 3u) != 0)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "window_lse must be 4-byte aligned");
  const ScoresOut so{out_scores, scores_len};
  return compress_impl(batch, num_q_heads, num_kv_heads, head_dim, q_win, k, v, seq_lens, window,
                       kernel_size, pool_mode, budget, out_k, out_v, out_idx, workspace,
                       workspace_bytes, stream, nullptr, window_lse, nullptr, &so);
}

int32_t snapkv_compress_staged(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, const void* q_win, const void* k,
                               const void* v, const int32_t* seq_lens, int32_t window,
                               int32_t kernel_size, int32_t pool_mode, int32_t budget,
                               void* out_k, void* out_v, int32_t* out_idx, void* workspace,
                               size_t workspace_bytes, void* stream,
                               void* const* stage_events) {
  return compress_impl(batch, num_q_heads, num_kv_heads, head_dim, q_win, k, v, seq_lens, window,
                       kernel_size, pool_mode, budget, out_k, out_v, out_idx, workspace,
                       workspace_bytes, stream, stage_events, nullptr);
}

int32_t snapkv_compress_int4(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, const void* q_win, const void* k, const void* v,
                             const int32_t* seq_lens, int32_t window, const float* window_lse,
                             int32_t kernel_size, int32_t pool_mode, int32_t budget,
                             uint8_t* out_kq, float* out_ks, uint8_t* out_vq, float* out_vs,
                             int32_t* out_idx, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (window_lse != nullptr && (reinterpret_cast<uintptr_t>(window_lse) & 3u) != 0)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "window_lse must be 4-byte aligned");
  const QuantOut q4{out_kq, out_ks, out_vq, out_vs, 1};
  return compress_impl(batch, num_q_heads, num_kv_heads, head_dim, q_win, k, v, seq_lens, window,
                       kernel_size, pool_mode, budget, nullptr, nullptr, out_idx, workspace,
                       workspace_bytes, stream, nullptr, window_lse, &q4);
}

int32_t snapkv_compress_fp8(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, const void* q_win, const void* k, const void* v,
                            const int32_t* seq_lens, int32_t window, const float* window_lse,
                            int32_t kernel_size, int32_t pool_mode, int32_t budget,
                            uint8_t* out_kq, float* out_ks, uint8_t* out_vq, float* out_vs,
                            int32_t* out_idx, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (window_lse != nullptr && (reinterpret_cast<uintptr_t>(window_lse) & 3u) != 0)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "window_lse must be 4-byte aligned");
  const QuantOut q8{out_kq, out_ks, out_vq, out_vs, 2};
  return compress_impl(batch, num_q_heads, num_kv_heads, head_dim, q_win, k, v, seq_lens, window,
                       kernel_size, pool_mode, budget, nullptr, nullptr, out_idx, workspace,
                       workspace_bytes, stream, nullptr, window_lse, &q8);
}

int32_t snapkv_window_scores(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, const void* q_win, const void* k,
                             const int32_t* seq_lens, int32_t window, int32_t kernel_size,
                             int32_t pool_mode, float* out_scores, int32_t scores_len,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!q_win || !k || !out_scores)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "a tensor pointer is NULL");
  if (misaligned(q_win) || misaligned(k) || misaligned(out_scores))
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
  Plan pl;
  int32_t st = make_plan(batch, num_q_heads, num_kv_heads, head_dim, seq_lens, window, &pl);
  if (st != SNAPKV_OK) return st;
  st = check_pool(kernel_size, pool_mode);
  if (st != SNAPKV_OK) return st;
  if (scores_len < pl.p_max)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT,
                "scores_len must be >= max(seq_len) - window = " + std::to_string(pl.p_max));
  if (workspace == nullptr || workspace_bytes < pl.bytes || misaligned(workspace))
    return fail(SNAPKV_ERR_WORKSPACE, "workspace must be 16-byte aligned and hold " +
                                          std::to_string(pl.bytes) + " bytes");
  hipStream_t s = static_cast<hipStream_t>(stream);
  snapkv::PathParams p = path_params(pl, q_win, k, nullptr, workspace, /*budget=*/0, kernel_size,
                                     pool_mode, /*score_all=*/true);
  p.pooled = out_scores;
  p.pooled_stride = scores_len;
  p.export_scores = 1;
  hipError_t e;
  // stats only where something is scored; the vote grid always runs, as it
  // also zeroes the exported rows past P
  if (any_scored(pl, 0, true) && (e = snapkv::launch_score_stats(p, head_dim, s)) != hipSuccess)
    return hip_fail(e, "snapkv_score_stats launch");
  if ((e = snapkv::launch_score_vote(p, head_dim, s)) != hipSuccess)
    return hip_fail(e, "snapkv_score_vote launch");
  return SNAPKV_OK;
}

int32_t snapkv_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t layout, int32_t capacity,
                                     const int32_t* cache_lens, size_t* bytes) {
  if (bytes == nullptr) return fail(SNAPKV_ERR_INVALID_ARGUMENT, "bytes is NULL");
  DecodePlan pl;
  const int32_t st = make_decode_plan(batch, num_q_heads, num_kv_heads, head_dim, layout,
                                      capacity, cache_lens, &pl);
  if (st != SNAPKV_OK) return st;
  *bytes = pl.bytes;
  return SNAPKV_OK;
}

int32_t snapkv_decode_kernels(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t layout, int32_t capacity,
                              const int32_t* cache_lens, int32_t* kernels) {
  if (kernels == nullptr) return fail(SNAPKV_ERR_INVALID_ARGUMENT, "kernels is NULL");
  DecodePlan pl;
  const int32_t st = make_decode_plan(batch, num_q_heads, num_kv_heads, head_dim, layout,
                                      capacity, cache_lens, &pl);
  if (st != SNAPKV_OK) return st;
  *kernels = pl.fused ? 1 : 2;
  return SNAPKV_OK;
}

int32_t snapkv_decode_attention_timed(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, const void* q, const void* k_cache,
                                      const void* v_cache, int32_t layout, int32_t capacity,
                                      const int32_t* cache_lens, float* out, void* workspace,
                                      size_t workspace_bytes, void* stream, void* start_event,
                                      void* stop_event) {
  if (!q || !k_cache || !v_cache || !out)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "a tensor pointer is NULL");
  if (misaligned(q) || misaligned(k_cache) || misaligned(v_cache) || misaligned(out))
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
  DecodePlan pl;
  int32_t st = make_decode_plan(batch, num_q_heads, num_kv_heads, head_dim, layout, capacity,
                                cache_lens, &pl);
  if (st != SNAPKV_OK) return st;
  if (workspace == nullptr || workspace_bytes < pl.bytes || misaligned(workspace))
    return fail(SNAPKV_ERR_WORKSPACE, "workspace must be 16-byte aligned and hold " +
                                          std::to_string(pl.bytes) + " bytes");
  snapkv::DecodeParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k_cache);
  p.v = static_cast<const uint16_t*>(v_cache);
  p.out = out;
  p.part = static_cast<float*>(workspace);
  p.batch = pl.batch;
  p.hq = pl.hq;
  p.hkv = pl.hkv;
  p.group = pl.group;
  p.chunk = pl.chunk;
  p.nchunk = pl.nchunk;
  p.layout = pl.layout;
  p.capacity = pl.capacity;
  p.fused = pl.fused;
  p.flags = reinterpret_cast<uint64_t*>(static_cast<unsigned char*>(workspace) + pl.off_flags);
  p.epoch = next_epoch();
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
  std::memcpy(p.off, pl.off, sizeof(p.off));
  std::memcpy(p.len, pl.len, sizeof(p.len));
  const hipError_t e =
      snapkv::launch_decode(p, head_dim, static_cast<hipStream_t>(stream),
                            static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
  if (e != hipSuccess) return hip_fail(e, "snapkv_decode launch");
  return SNAPKV_OK;
}

int32_t snapkv_decode_attention(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, const void* q, const void* k_cache,
                                const void* v_cache, int32_t layout, int32_t capacity,
                                const int32_t* cache_lens, float* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return snapkv_decode_attention_timed(batch, num_q_heads, num_kv_heads, head_dim, q, k_cache,
                                       v_cache, layout, capacity, cache_lens, out, workspace,
                                       workspace_bytes, stream, nullptr, nullptr);
}

int32_t snapkv_prefill_attention(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, const void* q, const void* k, const void* v,
                                 const int32_t* seq_lens, int32_t window, void* out,
                                 float* window_lse, void* q_win, void* stream) {
  if (!q || !k || !v || !out) return fail(SNAPKV_ERR_INVALID_ARGUMENT, "a tensor pointer is NULL");
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) ||
      (q_win != nullptr && misaligned(q_win)))
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
  if (window_lse != nullptr && (reinterpret_cast<uintptr_t>(window_lse) & 3u) != 0)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "window_lse must be 4-byte aligned");
  if (seq_lens == nullptr) return fail(SNAPKV_ERR_INVALID_ARGUMENT, "seq_lens is NULL");
  if (batch < 1 || batch > SNAPKV_MAX_BATCH)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT,
                "batch must be in [1, " + std::to_string(SNAPKV_MAX_BATCH) + "]");
  if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT,
                "num_q_heads must be a positive multiple of num_kv_heads");
  if ((window_lse != nullptr || q_win != nullptr) && window < 1)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "window must be >= 1 when its outputs are asked for");
  if (head_dim != 64 && head_dim != 128)
    return fail(SNAPKV_ERR_UNSUPPORTED, "head_dim must be 64 or 128, got " +
                                            std::to_string(head_dim));
  if ((int64_t)batch * num_q_heads > 65535)
    return fail(SNAPKV_ERR_UNSUPPORTED, "batch * num_q_heads must be <= 65535");
  snapkv::PrefillParams p{};
  int64_t total = 0;
  int l_max = 0;
  for (int b = 0; b < batch; ++b) {
    const int32_t L = seq_lens[b];
    if (L < 1)
      return fail(SNAPKV_ERR_INVALID_ARGUMENT,
                  "seq_lens[" + std::to_string(b) + "] must be >= 1, got " + std::to_string(L));
    p.tab.off[b] = (int32_t)total;
    p.tab.len[b] = L;
    total += L;
    if (total > INT32_MAX) return fail(SNAPKV_ERR_INVALID_ARGUMENT, "more than 2^31-1 tokens");
    l_max = L > l_max ? L : l_max;
  }
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.out = static_cast<uint16_t*>(out);
  p.window_lse = window_lse;
  p.q_win = static_cast<uint16_t*>(q_win);
  p.batch = batch;
  p.hq = num_q_heads;
  p.hkv = num_kv_heads;
  p.group = num_q_heads / num_kv_heads;
  p.window = window_lse != nullptr || q_win != nullptr ? window : 0;
  p.nqb = (l_max + snapkv::kPrefillRows - 1) / snapkv::kPrefillRows;
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
  const hipError_t e = snapkv::launch_prefill(p, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "snapkv_prefill launch");
  return SNAPKV_OK;
}

const char* snapkv_status_string(int32_t status) {
  switch (status) {
    case SNAPKV_OK: return "ok";
    case SNAPKV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SNAPKV_ERR_UNSUPPORTED: return "unsupported";
    case SNAPKV_ERR_WORKSPACE: return "workspace too small";
    case SNAPKV_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* snapkv_last_error(void) { return g_last_error.c_str(); }

const char* snapkv_stage_name(int32_t stage) {
  if (stage < 0 || stage >= SNAPKV_NUM_STAGES) return nullptr;
  return kStageNames[stage];
}

}  // extern "C"
