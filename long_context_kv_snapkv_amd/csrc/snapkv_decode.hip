// Decode-step attention over a KV cache on gfx950: after compression the
// decode phase attends over the kept rows only (glossary page
// "SnapKV(スナップケーブイ)", section "SnapKVの仕組み", step 4; the paper
// page reports the generation speed-up at 16K tokens that follows). For
// prompt b and query head q of KV head h:
//
//   out[b, q] = sum_t softmax_t(q_dec . k_t / sqrt(D)) v_t  over the cached rows
//
// The step streams each row of K and V once, so it is bound by HBM. Two
// kernels, or the first alone when every prompt's rows form few chunks (a
// compressed cache):
//
//   snapkv_decode_partial  (chunk, KV head, prompt)  one chunk of rows for all
//                          G query heads of the KV head, in tiles of 16 rows
//                          per wave: the scores of a tile for all G queries
//                          come from v_mfma_f32_16x16x32_bf16 (K rows as the
//                          A operand, the queries as B); the online softmax
//                          (running max, weights, rescale factor) runs in
//                          that layout, one lane per (row, query), and the
//                          weights pass through a per-wave LDS tile to the
//                          row layout (D/8 lanes per V row, 16 bytes each)
//                          that accumulates the weighted V; the waves merge
//                          through LDS in a fixed order and the chunk's
//                          partial goes to the workspace;
//   snapkv_decode_merge    (query head of the group, KV head, prompt)
//                          merges the chunks in a fixed order and writes out.
//
// In the one-launch form a prompt of one chunk writes out directly. For
// more chunks each chunk item stores its partial with device-coherent
// stores and waits until they are acknowledged, then stores its chunk's
// done mark (this call's epoch) the same way, waits for that too, and reads
// the marks of all chunks of its head. An item that finds every mark merges
// the head's chunks (device-coherent loads) in the merge kernel's order, so
// both forms give the same bits; the others end. Since every item's mark is
// at the coherence point before it reads the others', the item whose reads
// come last finds them all: at least one item merges (two that finish
// together may both merge, writing the same bits). Nothing waits, and the
// marks carry the call's epoch, so they need no clearing between calls.
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
// the halves of 8 (half mirror) and of 16 (mirror), then a permlane swap
// across two rows. Each step adds a value and its partner's, so all lanes of
// a group hold the same bits.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false));
  if (W >= 16)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xf, 0xf, false));
  if (W == 32) {
    const float2 r = rows16(x);
    x = r.x + r.y;
  }
  return x;
}

// Maximum over aligned groups of W = 16 or 32 lanes, in every lane (DPP
// within rows of 16, a permlane swap across two rows).
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
  if (W == 32) {
    const float2 r = rows16(x);
    x = fmaxf(r.x, r.y);
  }
  return x;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store_coherent(float* a, float x) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(a), __float_as_uint(x), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_coherent(const float* a) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(a)),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// One chunk's (max, sum of weights, weighted sum) folded into a running
// triple with a finite max: the merge's arithmetic, shared by both forms.
__device__ __forceinline__ void fold_step(float& rm, float& rl, float& ra, float mc, float lc,
                                          float ac) {
  const float mx = fmaxf(rm, mc);
  const float fr = exp2_fast(rm - mx), fc = exp2_fast(mc - mx);
  rl = fmaf(rl, fr, lc * fc);
  ra = fmaf(ra, fr, ac * fc);
  rm = mx;
}

// The same from any running triple: the first chunk (running max -inf) is
// taken as it is, which is what the general step gives for it, exactly.
__device__ __forceinline__ void fold_chunk(float& rm, float& rl, float& ra, float mc, float lc,
                                           float ac) {
  if (rm == -kInf) {
    rm = mc;
    rl = lc;
    ra = ac;
    return;
  }
  fold_step(rm, rl, ra, mc, lc, ac);
}

// The slices' running triples combined in order, and the output element.
template <int S>
__device__ __forceinline__ float combine_slices(const float (&sm)[S], const float (&sl)[S],
                                                const float (&sa)[S]) {
  float mx = -kInf;
#pragma unroll
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, sm[s]);
  float a = 0.f, l = 0.f;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (sm[s] == -kInf) continue;  // a slice without chunks
    const float f = exp2_fast(sm[s] - mx);
    a = fmaf(sa[s], f, a);
    l = fmaf(sl[s], f, l);
  }
  return a / l;
}

// The merge of one output element of query head g over nch <= C chunk
// partials, in the merge kernel's order: slice s folds chunks s, s + S, ...,
// then the slices combine in order. (max, sum) pairs come from LDS, the
// weighted sums from registers (all loaded before this runs).
template <int D, int C, int GM>
__device__ __forceinline__ float merge_loaded(const float2 (*mlc)[GM], int g, const float (&a)[C],
                                              int nch) {
  constexpr int S = kDecodeMergeThreads / D;
  static_assert(S <= C, "slices");
  float2 e[C];  // every slot read at once (slots past nch are not used)
#pragma unroll
  for (int c = 0; c < C; ++c) e[c] = mlc[c][g];
  float sm[S], sl[S], sa[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const bool live = s < nch;  // the slice's first chunk, taken as it is
    float rm = live ? e[s].x : -kInf, rl = live ? e[s].y : 0.f, ra = live ? a[s] : 0.f;
#pragma unroll
    for (int c = s + S; c < C; c += S)
      if (c < nch) fold_step(rm, rl, ra, e[c].x, e[c].y, a[c]);
    sm[s] = rm;
    sl[s] = rl;
    sa[s] = ra;
  }
  return combine_slices<S>(sm, sl, sa);
}

template <int D, int GM, bool FUSED>
__global__ void __launch_bounds__(kDecodeThreads) snapkv_decode_partial(const DecodeParams p) {
  constexpr int PIECES = D / 8;         // lanes per row in the row layout
  constexpr int RPI = 64 / PIECES;      // rows per wave instruction in the row layout
  constexpr int TILE = 16;              // rows per score tile (one MFMA row block)
  constexpr int STEPS = TILE / RPI;     // row-layout steps per tile
  constexpr int KB = D / 32;            // MFMA k blocks
  constexpr int NW = kDecodeThreads / 64;
  constexpr int NG = NW * RPI;          // lane groups of the row layout per workgroup
  constexpr int SP = 20;                // LDS pitch of a score-tile row (floats)
  constexpr int ROUND = 2 * NW * TILE;  // rows per workgroup round (two tiles per wave)
  static_assert(ROUND == kDecodeRowQuantum, "chunk quantum");
  __shared__ float sm_s[NW][(TILE + 1) * SP];
  __shared__ float sm_ml[NG][GM][2];
  __shared__ float sm_acc[NG][GM][D];
  __shared__ float sm_f[NG][GM];
  __shared__ float sm_l[GM];  // one-chunk prompts of the one-launch form: sum of weights
  __shared__ float2 sm_mlc[FUSED ? kDecodeFusedMaxChunks : 1][GM];  // the merging item's (max, sum)
  static_assert(NG == 16 || NG == 32, "lane groups per workgroup");

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  // the kernel arguments the item starts with, requested together: one
  // scalar round trip instead of one per branch that depends on them
  const int n = p.len[b], off_b = p.off[b], chunk = p.chunk, layout = p.layout;
  const int capacity = p.capacity, hkv = p.hkv, hq = p.hq, group = p.group;
  const uint16_t *pq = p.q, *pk = p.k, *pv = p.v;
  asm volatile("" ::"s"(n), "s"(off_b), "s"(chunk), "s"(layout), "s"(capacity), "s"(hkv), "s"(hq),
               "s"(group), "s"(pq), "s"(pk), "s"(pv));
  const int r0 = c * chunk;
  if (r0 >= n) return;
  const int r1 = min(r0 + chunk, n);
  const int nch = (n + chunk - 1) / chunk;
  // the one-launch form writes out directly when the prompt has one chunk
  const bool direct = FUSED && nch == 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int piece = lane % PIECES, grp = lane / PIECES, gi = wave * RPI + grp;
  const int mrow = lane % 16, mk = lane / 16;  // MFMA operand layout
  size_t base, rs;
  if (layout == 0) {
    base = (size_t)(b * hkv + h) * capacity * D;
    rs = D;
  } else {
    base = ((size_t)off_b * hkv + h) * D;
    rs = (size_t)hkv * D;
  }
  const uint16_t* kbase = pk + base + mk * 8;
  const uint16_t* vbase = pv + base + piece * 8;

  // Q^T as the MFMA B operand: query mrow, elements kb * 32 + 8 * mk + e
  // (slots past the group repeat its last query; their results are unused)
  u32x4 qop[KB];
  const uint16_t* qrow = pq + (size_t)(b * hq + h * group + min(mrow, group - 1)) * D;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) qop[kb] = *reinterpret_cast<const u32x4*>(qrow + kb * 32 + mk * 8);

  // a tile of 16 rows t0 .. t0 + 15: K in the MFMA A layout (row t0 + mrow),
  // V in the row layout (row t0 + RPI * s + grp for step s). Rows past the
  // chunk are clamped to its last row (a cached re-read) and masked, so every
  // load is unconditional.
  struct Tile {
    u32x4 k[KB];
    u32x4 v[STEPS];
  };
  auto load_tile = [&](Tile& T, int t0) {
    const size_t rk = (size_t)min(t0 + mrow, r1 - 1);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      T.k[kb] = *reinterpret_cast<const u32x4*>(kbase + rk * rs + kb * 32);
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const size_t rv = (size_t)min(t0 + st * RPI + grp, r1 - 1);
      T.v[st] = *reinterpret_cast<const u32x4*>(vbase + rv * rs);
    }
    // issued before the work that follows (neither memory operations nor
    // arithmetic move across)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // softmax state: the running max and (partial) sum of weights of query
  // mrow over the wave's rows live in the MFMA layout (the four lanes mk of
  // a query share the max; each sums its own rows), the weighted V sums in
  // the row layout
  float m_run = -kInf, l_run = 0.f;
  float acc[GM][8];
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  float* stile = sm_s[wave];

  auto process = [&](const Tile& T, int t0) {
    // scores of the tile's rows 4 * mk + r for query mrow on the MFMA
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(T.k[kb]), as_bf16x8(qop[kb]), sc,
                                                   0, 0, 0);
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = t0 + 4 * mk + r < r1 ? sc[r] * p.scale_log2 : -kInf;
    float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    const float2 t16 = rows16(tmax);
    const float2 t32 = halves32(fmaxf(t16.x, t16.y));
    tmax = fmaxf(t32.x, t32.y);
    const float mnew = fmaxf(m_run, tmax);
    float cs = 1.f, pr[4] = {0.f, 0.f, 0.f, 0.f};
    if (mnew != -kInf) {  // some row of the wave seen so far
      cs = exp2_fast(m_run - mnew);
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = exp2_fast(x[r] - mnew);
    }
    l_run = l_run * cs + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m_run = mnew;
    // weights and rescale factors through this wave's LDS tile to the row
    // layout (one wave writes and reads it, in order)
#pragma unroll
    for (int r = 0; r < 4; ++r) stile[(4 * mk + r) * SP + mrow] = pr[r];
    if (mk == 0) stile[TILE * SP + mrow] = cs;
    __builtin_amdgcn_wave_barrier();
    float csv[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g) csv[g] = stile[TILE * SP + g];
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      // the same word for every lane: a scalar test skips the common cs == 1
      const float csg = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(csv[g])));
      if (csg != 1.f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] *= csg;
      }
    }
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const float* prow = stile + (st * RPI + grp) * SP;
      float pg[GM];
#pragma unroll
      for (int g = 0; g < GM; ++g) pg[g] = prow[g];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ve = bf16_elem(T.v[st], e);
#pragma unroll
        for (int g = 0; g < GM; ++g) acc[g][e] = fmaf(pg[g], ve, acc[g][e]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // rounds: each wave loads two tiles (rows t0 and t0 + 64 of the round)
  // before using the first
  Tile ta, tb;
  const int w0 = wave * TILE;
  load_tile(ta, r0 + w0);
  load_tile(tb, r0 + w0 + NW * TILE);
  process(ta, r0 + w0);
  process(tb, r0 + w0 + NW * TILE);
  for (int rb = r0 + ROUND; rb < r1; rb += ROUND) {
    load_tile(ta, rb + w0);
    load_tile(tb, rb + w0 + NW * TILE);
    process(ta, rb + w0);
    process(tb, rb + w0 + NW * TILE);
  }

  // every lane group's state to LDS; then, per query head, the groups'
  // weights 2^(m_w - max) and the sum of weights by DPP reductions over NG
  // lanes, and each output element as a fixed-order sum over the groups
  // the wave's sum of weights per query (fixed-order butterfly over mk); its
  // lane groups share the wave's max, and the sum is carried by group 0
  const float2 l16 = rows16(l_run);
  const float2 l32 = halves32(l16.x + l16.y);
  l_run = l32.x + l32.y;
  if (mk == 0 && mrow < GM) {
#pragma unroll
    for (int j = 0; j < RPI; ++j) {
      sm_ml[wave * RPI + j][mrow][0] = m_run;
      sm_ml[wave * RPI + j][mrow][1] = j == 0 ? l_run : 0.f;
    }
  }
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_acc[gi][g][piece * 8 + e] = acc[g][e];
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
      if (direct) {
        sm_l[g] = lsum;
      } else if (FUSED) {
        store_coherent(&dst[g * (D + 2)], mx);
        store_coherent(&dst[g * (D + 2) + 1], lsum);
      } else {
        dst[g * (D + 2)] = mx;
        dst[g * (D + 2) + 1] = lsum;
      }
    }
  }
  __syncthreads();
  float* out = p.out + (size_t)(b * p.hq + h * p.group) * D;
  for (int i = tid; i < p.group * D; i += kDecodeThreads) {
    const int g = i / D, d = i % D;
    float sa = 0.f;
#pragma unroll
    for (int w = 0; w < NG; ++w) sa = fmaf(sm_f[w][g], sm_acc[w][g][d], sa);
    if (direct)
      out[i] = sa / sm_l[g];  // the merge of a single chunk, exactly
    else if (FUSED)
      store_coherent(&dst[g * (D + 2) + 2 + d], sa);
    else
      dst[g * (D + 2) + 2 + d] = sa;
  }
  if constexpr (FUSED) {
    if (direct) return;
    // this item's partial is at the coherence point before its mark, and its
    // mark before it reads the others' (wave 0 does both)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    uint64_t* marks = p.flags + (size_t)(b * p.hkv + h) * kDecodeFusedMaxChunks;
    if (tid == 0) __hip_atomic_store(&marks[c], p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    int missing = 0;
    if (tid < nch)
      missing = __hip_atomic_load(&marks[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != p.epoch;
    if (__syncthreads_or(missing)) return;
    // every chunk's partial was acknowledged before its mark, and these
    // loads are issued after the marks were read. All of them are in flight
    // at once: each thread's weighted sums into registers, the (max, sum)
    // pairs of every (chunk, query head) into LDS.
    constexpr int C = kDecodeFusedMaxChunks;
    constexpr int KO = (GM * D + kDecodeThreads - 1) / kDecodeThreads;
    const size_t cstride = (size_t)p.group * (D + 2);
    const float* col0 = p.part + (size_t)(b * p.hkv + h) * p.nchunk * cstride;
    float av[KO][C];
#pragma unroll
    for (int o = 0; o < KO; ++o) {
      const int i = tid + o * kDecodeThreads;
      const int g = min(i / D, p.group - 1), d = i % D;  // past the group: an unused in-range load
#pragma unroll
      for (int c = 0; c < C; ++c)
        av[o][c] = c < nch ? load_coherent(col0 + c * cstride + g * (D + 2) + 2 + d) : 0.f;
    }
    for (int j = tid; j < nch * p.group; j += kDecodeThreads) {
      const float* e = col0 + (j / p.group) * cstride + (j % p.group) * (D + 2);
      sm_mlc[j / p.group][j % p.group] = make_float2(load_coherent(e), load_coherent(e + 1));
    }
    __syncthreads();
#pragma unroll
    for (int o = 0; o < KO; ++o) {
      const int i = tid + o * kDecodeThreads;
      if (i < p.group * D) out[i] = merge_loaded<D, C, GM>(sm_mlc, i / D, av[o], nch);
    }
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
  auto fold = [&](float mc, float lc, float ac) { fold_chunk(rm, rl, ra, mc, lc, ac); };
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
    float ms[S], ls[S], as[S];
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) {
      ms[s2] = red_m[s2 * D + d];
      ls[s2] = red_l[s2 * D + d];
      as[s2] = red_a[s2 * D + d];
    }
    p.out[(size_t)(b * p.hq + h * p.group + g) * D + d] = combine_slices<S>(ms, ls, as);
  }
}

// With events, through the extended launch that has the dispatch record
// them at the kernel's own start and end.
template <typename K>
hipError_t launch_ev(K kernel, dim3 grid, int threads, hipStream_t stream, hipEvent_t start,
                     hipEvent_t stop, const DecodeParams& p) {
  if (start != nullptr || stop != nullptr) {
    void* args[] = {const_cast<DecodeParams*>(&p)};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, dim3(threads), args,
                              0, stream, start, stop, 0);
  }
  hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, stream, p);
  return hipGetLastError();
}

template <int D, int GM>
hipError_t launch_decode_dg(const DecodeParams& p, hipStream_t stream, hipEvent_t start,
                            hipEvent_t stop) {
  const dim3 grid(p.nchunk, p.hkv, p.batch);
  if (p.fused) return launch_ev(snapkv_decode_partial<D, GM, true>, grid, kDecodeThreads, stream,
                                start, stop, p);
  hipError_t e = launch_ev(snapkv_decode_partial<D, GM, false>, grid, kDecodeThreads, stream,
                           start, nullptr, p);
  if (e != hipSuccess) return e;
  return launch_ev(snapkv_decode_merge<D>, dim3(p.group, p.hkv, p.batch), kDecodeMergeThreads,
                   stream, nullptr, stop, p);
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, hipStream_t stream, hipEvent_t start,
                           hipEvent_t stop) {
  if (p.group <= 1) return launch_decode_dg<D, 1>(p, stream, start, stop);
  if (p.group <= 2) return launch_decode_dg<D, 2>(p, stream, start, stop);
  if (p.group <= 4) return launch_decode_dg<D, 4>(p, stream, start, stop);
  if (p.group <= kDecodeMaxGroup) return launch_decode_dg<D, 8>(p, stream, start, stop);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int head_dim, hipStream_t stream,
                         hipEvent_t start, hipEvent_t stop) {
  if (head_dim == 128) return launch_decode_d<128>(p, stream, start, stop);
  if (head_dim == 64) return launch_decode_d<64>(p, stream, start, stop);
  return hipErrorInvalidValue;
}

}  // namespace snapkv
