// Host side of the SnapKV compression library: argument validation, the
// workspace plan, and the launch sequence on the caller's stream. Every check
// runs before the first HIP call, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>

#include "snapkv.h"
#include "snapkv_kernels.h"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

const char* const kStageNames[SNAPKV_NUM_STAGES] = {
    "snapkv_score_stats", "snapkv_score_vote", "snapkv_pool", "snapkv_topk", "snapkv_gather"};

// Everything a call needs, derived from shapes alone (so the workspace size
// computed ahead of a call matches the call).
struct Plan {
  int batch, hq, hkv, d, window, group, rows, rows_pad, nrt;
  int waves, nwr;
  int chunk, nchunk;
  int l_max, p_max, p_stride;
  size_t off_part, off_raw, off_pooled, bytes;
  snapkv::PromptTable tab;
};

int largest_pow2_at_most(int x) {
  int p = 1;
  while (p * 2 <= x) p *= 2;
  return p;
}

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
  pl->waves = pl->nrt <= 8 ? 4 : 8;
  pl->nwr = largest_pow2_at_most(pl->nrt < pl->waves ? pl->nrt : pl->waves);
  // keys per scoring workgroup: about 512 workgroups over the whole call,
  // 64-key granularity, at most 8192 keys
  int64_t chunk = (key_sum * hkv + 511) / 512;
  chunk = (chunk + snapkv::kKeyTile - 1) / snapkv::kKeyTile * snapkv::kKeyTile;
  if (chunk < 256) chunk = 256;
  if (chunk > 8192) chunk = 8192;
  pl->chunk = (int)chunk;
  pl->nchunk = (int)((l_max + chunk - 1) / chunk);
  pl->l_max = l_max;
  pl->p_max = l_max - window > 1 ? l_max - window : 1;
  pl->p_stride = (int)align_up((size_t)pl->p_max, 64);
  size_t off = 0;
  pl->off_part = off;
  off = align_up(off + (size_t)batch * hkv * pl->nchunk * pl->rows_pad * sizeof(float2), 256);
  pl->off_raw = off;
  off = align_up(off + (size_t)batch * hkv * pl->p_stride * sizeof(float), 256);
  pl->off_pooled = off;
  off = align_up(off + (size_t)batch * hkv * pl->p_stride * sizeof(float), 256);
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

snapkv::ScoreParams score_params(const Plan& pl, const void* q, const void* k, void* ws,
                                 int32_t budget, bool skip_fitting) {
  snapkv::ScoreParams sp;
  sp.q = static_cast<const uint16_t*>(q);
  sp.k = static_cast<const uint16_t*>(k);
  sp.part = reinterpret_cast<float2*>(static_cast<char*>(ws) + pl.off_part);
  sp.raw = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.off_raw);
  sp.hq = pl.hq;
  sp.hkv = pl.hkv;
  sp.window = pl.window;
  sp.group = pl.group;
  sp.rows = pl.rows;
  sp.rows_pad = pl.rows_pad;
  sp.nwr = pl.nwr;
  sp.chunk = pl.chunk;
  sp.nchunk = pl.nchunk;
  sp.p_stride = pl.p_stride;
  sp.budget = budget;
  sp.skip_fitting = skip_fitting ? 1 : 0;
  sp.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)pl.d));
  sp.tab = pl.tab;
  return sp;
}

int32_t hip_fail(hipError_t e, const char* what) {
  return fail(SNAPKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Stages 1-2 (scoring and pooling) into `pooled` with row stride out_stride.
int32_t run_scores(const Plan& pl, const snapkv::ScoreParams& sp, int32_t kernel,
                   int32_t pool_mode, float* pooled, int out_stride, hipStream_t stream,
                   hipEvent_t const* ev) {
  const dim3 sgrid(pl.nchunk, pl.hkv, pl.batch);
  if (ev) (void)hipEventRecord(ev[0], stream);
  hipError_t e = snapkv::launch_score_stats(sp, pl.d, pl.waves, sgrid, stream);
  if (e != hipSuccess) return hip_fail(e, "snapkv_score_stats launch");
  if (ev) (void)hipEventRecord(ev[1], stream);
  if (ev) (void)hipEventRecord(ev[2], stream);
  e = snapkv::launch_score_vote(sp, pl.d, pl.waves, sgrid, stream);
  if (e != hipSuccess) return hip_fail(e, "snapkv_score_vote launch");
  if (ev) (void)hipEventRecord(ev[3], stream);

  snapkv::PoolParams pp;
  pp.raw = sp.raw;
  pp.out = pooled;
  pp.hkv = pl.hkv;
  pp.window = pl.window;
  pp.kernel = kernel;
  pp.mode = pool_mode;
  pp.p_stride = pl.p_stride;
  pp.out_stride = out_stride;
  pp.budget = sp.budget;
  pp.skip_fitting = sp.skip_fitting;
  pp.tab = pl.tab;
  const dim3 pgrid((out_stride + snapkv::kPoolTile - 1) / snapkv::kPoolTile, pl.hkv, pl.batch);
  if (ev) (void)hipEventRecord(ev[4], stream);
  e = snapkv::launch_pool(pp, pgrid, stream);
  if (e != hipSuccess) return hip_fail(e, "snapkv_pool launch");
  if (ev) (void)hipEventRecord(ev[5], stream);
  return SNAPKV_OK;
}

int32_t compress_impl(int32_t batch, int32_t hq, int32_t hkv, int32_t d, const void* q_win,
                      const void* k, const void* v, const int32_t* seq_lens, int32_t window,
                      int32_t kernel, int32_t pool_mode, int32_t budget, void* out_k,
                      void* out_v, int32_t* out_idx, void* workspace, size_t workspace_bytes,
                      void* stream, void* const* stage_events) {
  if (!q_win || !k || !v || !out_k || !out_v || !out_idx)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "a tensor pointer is NULL");
  if (misaligned(q_win) || misaligned(k) || misaligned(v) || misaligned(out_k) ||
      misaligned(out_v) || misaligned(out_idx))
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
  Plan pl;
  int32_t st = make_plan(batch, hq, hkv, d, seq_lens, window, &pl);
  if (st != SNAPKV_OK) return st;
  if (budget <= window)
    return fail(SNAPKV_ERR_INVALID_ARGUMENT, "budget must exceed window (it includes the window)");
  st = check_pool(kernel, pool_mode);
  if (st != SNAPKV_OK) return st;
  if (workspace == nullptr || workspace_bytes < pl.bytes || misaligned(workspace))
    return fail(SNAPKV_ERR_WORKSPACE, "workspace must be 16-byte aligned and hold " +
                                          std::to_string(pl.bytes) + " bytes");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t const* ev = reinterpret_cast<hipEvent_t const*>(stage_events);
  bool any_scored = false;
  for (int b = 0; b < batch; ++b) any_scored |= seq_lens[b] > budget;

  const snapkv::ScoreParams sp = score_params(pl, q_win, k, workspace, budget, true);
  float* pooled = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.off_pooled);
  if (any_scored) {
    st = run_scores(pl, sp, kernel, pool_mode, pooled, pl.p_stride, s, ev);
    if (st != SNAPKV_OK) return st;
    snapkv::TopkParams tp;
    tp.pooled = pooled;
    tp.out_idx = out_idx;
    tp.hkv = hkv;
    tp.window = window;
    tp.budget = budget;
    tp.p_stride = pl.p_stride;
    tp.tab = pl.tab;
    if (ev) (void)hipEventRecord(ev[6], s);
    hipError_t e = snapkv::launch_topk(tp, dim3(hkv, batch), s);
    if (e != hipSuccess) return hip_fail(e, "snapkv_topk launch");
    if (ev) (void)hipEventRecord(ev[7], s);
  } else if (ev) {
    for (int i = 0; i < 8; ++i) (void)hipEventRecord(ev[i], s);
  }
  snapkv::GatherParams gp;
  gp.k = static_cast<const uint16_t*>(k);
  gp.v = static_cast<const uint16_t*>(v);
  gp.out_k = static_cast<uint16_t*>(out_k);
  gp.out_v = static_cast<uint16_t*>(out_v);
  gp.out_idx = out_idx;
  gp.hkv = hkv;
  gp.budget = budget;
  gp.tab = pl.tab;
  if (ev) (void)hipEventRecord(ev[8], s);
  hipError_t e = snapkv::launch_gather(
      gp, d, dim3((budget + snapkv::kGatherRows - 1) / snapkv::kGatherRows, hkv, batch), s);
  if (e != hipSuccess) return hip_fail(e, "snapkv_gather launch");
  if (ev) (void)hipEventRecord(ev[9], s);
  return SNAPKV_OK;
}

}  // namespace

extern "C" {

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
                       workspace_bytes, stream, nullptr);
}

int32_t snapkv_compress_profiled(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, const void* q_win, const void* k,
                                 const void* v, const int32_t* seq_lens, int32_t window,
                                 int32_t kernel_size, int32_t pool_mode, int32_t budget,
                                 void* out_k, void* out_v, int32_t* out_idx, void* workspace,
                                 size_t workspace_bytes, void* stream,
                                 void* const* stage_events) {
  return compress_impl(batch, num_q_heads, num_kv_heads, head_dim, q_win, k, v, seq_lens, window,
                       kernel_size, pool_mode, budget, out_k, out_v, out_idx, workspace,
                       workspace_bytes, stream, stage_events);
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
  const snapkv::ScoreParams sp = score_params(pl, q_win, k, workspace, 0, false);
  return run_scores(pl, sp, kernel_size, pool_mode, out_scores, scores_len,
                    static_cast<hipStream_t>(stream), nullptr);
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
