// Internal helpers shared by the dfx HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dfx.h"

namespace dfx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// e^x as 2^(x log2 e) on the hardware exponential (v_exp_f32), for the softmax statistics
// and the mixture of the output head: the product adds one rounding of the argument (about
// |x| 2^-24 relative in the result, the size of the rounding of x itself) and results below
// 2^-126 flush to zero; a few instructions instead of the library's range-reduced expf.
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// ---- bf16 <-> fp32 on raw bit patterns ----------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN -> quiet NaN with the sign kept.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Splits x into NT bf16 terms t[0] + t[1] + ... : every term but the last is the remainder
// so far truncated to bf16, the last is the remainder rounded to nearest even. Each
// truncation keeps the next 8 significant bits, so the terms carry 8 NT bits of x: NT = 2
// leaves |error| <= 2^-16 |x|, and NT = 3 holds every bit of an fp32 x exactly (the
// last remainder has at most 8 significant bits), so NT bf16 MFMA passes multiply an fp32
// value at fp32 precision.
// (With NT >= 3 the last remainder is already a bf16 value -- its low 16 bits are zero for
// every x from 2^-110 up -- so it is taken by truncation, which is then exact.)
template <int NT>
__device__ __forceinline__ void split_terms(float x, uint32_t *t) {
  float r = x;
#pragma unroll
  for (int i = 0; i < NT - 1; ++i) {
    const uint32_t h = __float_as_uint(r) & 0xffff0000u;
    t[i] = h >> 16;
    r -= __uint_as_float(h);
  }
  t[NT - 1] = NT >= 3 ? __float_as_uint(r) >> 16 : f32_to_bf16_rne(r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// silu(g) = g * sigmoid(g), the gate of SwiGLU
__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Element offset of row r of flow f, column k, in the fragment-ordered activations that the
// grouped linear reads directly: [groups][K/32][4 blocks][64 lanes][8]. Row group r / (64/F)
// holds row q = f (64/F) + r % (64/F); lane (q % 16) + 16 ((k % 32) / 8) of block q / 16
// holds columns 8 ((k % 32) / 8) .. +7 of k-step k / 32, i.e. exactly one B operand of the
// 16x16x32 MFMA. A buffer of F rows of B sequences holds ceil(B / (64/F)) * 64 * K elements.
__device__ __forceinline__ int64_t xpack_offset(int F, int f, int r, int k, int K) {
  const int rpg = 64 / F, grp = r / rpg, q = f * rpg + r % rpg;
  return ((((int64_t)grp * (K >> 5) + (k >> 5)) * 4 + (q >> 4)) * 64 + (q & 15) + 16 * ((k & 31) >> 3)) * 8 +
         (k & 7);
}

// Sum of the K-split fp32 tiles [ksplit][groups][64 rows][N] at one (group, row q, col),
// added in split order. The loads of each group of 8 splits are all issued before the first
// add (indices past the last split re-read it and are not added), so the sum costs one
// memory round trip per 8 splits instead of one per split.
__device__ __forceinline__ f32x4 sum_split_tiles(const float *tiles, int ksplit, int groups, int N,
                                                 int grp, int q, int col) {
  constexpr int U = 8;
  f32x4 s{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < ksplit; k0 += U) {
    f32x4 t[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = min(k0 + u, ksplit - 1);
      t[u] = *(const f32x4 *)(tiles + (((int64_t)k * groups + grp) * 64 + q) * N + col);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (k0 + u < ksplit) s += t[u];
  }
  return s;
}

// RMSNorm of one row by a 1024-thread work-group: thread t owns the float4 slices
// t + 1024 u (u < kNormSlices; zero past the row, dim <= 16384). The reduction order is fixed
// (each thread's slices in order, the wave butterfly, then the 16 waves in order), so every
// kernel that normalizes a row through these helpers rounds identical rows identically.
constexpr int kNormSlices = 4;

__device__ __forceinline__ float norm_scale(const f32x4 *v, int dim, float eps, float *red) {
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < kNormSlices; ++u) ss += v[u][0] * v[u][0] + v[u][1] * v[u][1] + v[u][2] * v[u][2] + v[u][3] * v[u][3];
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < 16; ++w) tot += red[w];
  return 1.0f / sqrtf(tot / (float)dim + eps);
}

// y = bf16(v * r * gain) for this thread's slices of row (f, b) (row index `row` when
// row-major); packed_flows > 0 writes the fragment order of xpack_offset.
__device__ __forceinline__ void norm_store(const f32x4 *v, const f32x4 *gg, float r, int dim, uint16_t *y,
                                           int packed_flows, int f, int b, int64_t row) {
#pragma unroll
  for (int u = 0; u < kNormSlices; ++u) {
    const int i = threadIdx.x + 1024 * u;
    if (4 * i >= dim) continue;
    const u32x2 o{pack_bf16x2(v[u][0] * r * gg[u][0], v[u][1] * r * gg[u][1]),
                  pack_bf16x2(v[u][2] * r * gg[u][2], v[u][3] * r * gg[u][3])};
    const int64_t at = packed_flows ? xpack_offset(packed_flows, f, b, 4 * i, dim) : row * dim + 4 * i;
    *(u32x2 *)(y + at) = o;
  }
}

// ---- launch-time parameter blocks --------------------------------------------------

struct AttnArgs {
  const void *k, *v;
  const int32_t *table;
  int64_t num_blocks;
  int32_t max_blocks, block_size, block_shift;  // block_shift < 0: contiguous layout
  int32_t num_kv_heads, head_dim, group, num_q_heads, n_flows, batch;
  const int32_t *ctx;
  int32_t max_context;
  const void *q1, *q2;
  int64_t q_bstride;
  int32_t q_bf16, kv_bf16;
  const float *a;
  int32_t a_hstride;
  float scale_log2;  // softmax scale * log2(e)
  float *o1, *o2, *lse;
  int32_t o_bf16;  // o1/o2 hold bf16 (uint16) rows instead of fp32
  int32_t o_packed;  // bf16 rows in the grouped linear's fragment order, both flows in o1
  float *part_o, *part_lse;  // [S][F][B][Hq][D], [S][F][B][Hq] (log2 domain)
  int32_t num_splits, chunk;
  int32_t k_rows;  // matrix-core decode: stage K tiles through LDS as whole rows
  // prefill (primary only): T query positions per sequence, ctx[b] = position of the first;
  // q1 rows are (b, t) with row stride q_bstride
  int32_t prefill_T;
};

struct GemmArgs {
  int32_t n_flows, rows, K, N;
  int32_t x_f32;
  int32_t x_packed;  // bf16 rows in the fragment order of xpack_offset instead of row-major
  const void *x;
  const uint16_t *w;
  int32_t w_packed;  // DFX_W_PACKED fragment order instead of row-major
  int32_t y_bf16;
  void *y;
  const float *couple, *residual;
  int32_t ksplit;      // work-groups along K per feature tile
  int32_t kper;        // k-steps of 32 per split (the last split may have fewer)
  float *partial;      // [ksplit][groups][64 rows][N] fp32 when ksplit > 1 or tiles_only
  int32_t tiles_only;  // write the fp32 tiles even for one split (a finish kernel follows)
  // gate/up mode (one split): N = 2 I with the gate rows of W first; a wave pairs gate
  // features c.. c+15 with up features I + c..; y receives bf16 silu(gate) * up, flow 1
  // plus couple * flow 0, in the fragment order of xpack_offset with K = I
  int32_t swiglu;
  // expert mode (blockIdx.z = expert e): the rows of expert e are expert_rows[e] (read on the
  // device, so an expert with no rows reads none of its weights), at most max_groups groups;
  // x, w, y and partial of expert e start e * x_estride, w_estride, y_estride, p_estride
  // elements in, and the partial tiles of an expert use max_groups as their group count
  // (x bf16 in fragment order; gate/up mode or tiles_only); grid z = experts
  const int32_t *expert_rows;
  int32_t experts, max_groups;
  int64_t x_estride, w_estride, y_estride, p_estride;
  // many row groups (prefill), one split: grid z = group_split slices of the row groups, each
  // work-group streams its weight columns once per group of its slice
  int32_t group_split;
  // output-head mode (one split, plain outputs, packed X and W): softmax statistics of every
  // (128-feature tile, row) of the fp32 outputs, from the accumulators: record
  // [row][tile][kMixStat] = tile max and sum of e^(l - max) of each flow, and for the primary
  // the sum of e^(2 (l - max)) (the layout the mixture's apply pass reads)
  float *mix_stats;
};
// per (sequence, statistics chunk): m0, s0, q0, m1, s1, 3 unused
constexpr int kMixStat = 8;
constexpr int kHeadTile = 128;  // output features per grouped-linear work-group (plain mode)

// Destination of attention output (flow f, sequence b, column c = head * D + d): rows
// [B][Hq * D] of o1 / o2, or, with o_packed, both flows in o1 in the fragment order of
// xpack_offset (K = Hq * D). Returns the row base pointer; *off receives the element offset.
__device__ __forceinline__ float *attn_out(const AttnArgs &p, int f, int b, int c, int64_t *off) {
  const int K = p.num_q_heads * p.head_dim;
  if (p.o_packed) {
    *off = xpack_offset(p.n_flows, f, b, c, K);
    return p.o1;
  }
  *off = (int64_t)b * K + c;
  return f == 0 ? p.o1 : p.o2;
}

// Arguments of the kernels that finish a projection of the decode layer.
enum { kGlueQkv = 0, kGlueONorm = 1, kGlueDown = 3, kGlueDownNorm = 4 };
struct LayerGlueArgs {
  int32_t n_flows, batch, N, ksplit;
  const float *tiles;  // [ksplit][groups][64][N]
  float *out;          // qkv: Q columns [F][B][N] fp32
  float *x;            // residual rows [F][B][N] fp32 (in place)
  uint16_t *h;         // bf16 rows for the next projection (fragment order, xpack_offset)
  const float *gain;   // RMSNorm gain
  float eps;
  const float *couple; // c coupling vector of the down projection, or NULL
  dfx_kv_cache kv;     // cache written by the Q/K/V finish (primary rows only)
  const int32_t *ctx;  // context lengths after the step, clamped to [1, max_context] as the
                       // attention clamps them (append position = clamped length - 1)
  int32_t max_context;
  int32_t num_q_heads, head_dim;
};

// Kernel launchers (defined next to their kernels). They assume validated arguments.
hipError_t launch_attn_mfma(const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_valu(const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_merge(const AttnArgs &a, hipStream_t s);
hipError_t launch_kv_append(const dfx_kv_cache &kv, int32_t batch, const int32_t *positions,
                            int32_t pos_minus_one, int32_t src_f32, const void *k_new,
                            const void *v_new, int64_t src_stride, hipStream_t s);
hipError_t launch_grouped_linear(const GemmArgs &g, hipStream_t s);
hipError_t launch_pack_weight(int32_t N, int32_t K, const uint16_t *w, uint16_t *packed,
                              hipStream_t s);
hipError_t launch_layer_glue(int which, const LayerGlueArgs &a, hipStream_t s);

// Mixture-of-experts block (router replay). Selections are stored kMoeMaxK per (flow,
// sequence), ranks past the flow's fan-out hold id -1 and weight 0.
constexpr int kMoeMaxK = 16;
constexpr int kMoeMaxExperts = 256;
enum { kMoeRoute = 0, kMoeLists = 1, kMoeGather = 2, kMoeCombine = 3 };
struct MoeArgs {
  int32_t F, B, H, E, k1, k2, max_groups, ksplit;
  const uint16_t *h;         // bf16 [F][B][H] normed rows, row-major
  const uint16_t *w_router;  // bf16 [E][H]
  float *logits;             // [F][B][E]
  int32_t *ids;              // [F][B][kMoeMaxK]
  float *wts;                // [F][B][kMoeMaxK]
  int32_t *pos;              // [F][B][kMoeMaxK]: row of the sequence in its expert's list
  int32_t *counts;           // [E]
  int32_t *seqs;             // [E][B]
  uint16_t *xg;              // [E][max_groups * 64 * H] bf16, fragment order
  const float *tiles;        // [E][ksplit][max_groups][64][H]
  const float *couple_c;     // [H] or NULL
  float *x;                  // [F][B][H] residual rows, updated in place
  const float *gain;         // [H] norm gain
  float eps;
};
hipError_t launch_moe(int which, const MoeArgs &a, hipStream_t s);

// Prefill (primary only): causal attention of T new positions per sequence over the cache,
// and the Q/K/V finish that appends the chunk's keys and values.
hipError_t launch_prefill_attn(const AttnArgs &a, hipStream_t s);
struct PrefillGlueArgs {
  int32_t B, T, N, num_q_heads, head_dim;
  const float *qkv;        // [B * T][N] fp32 projection rows
  dfx_kv_cache kv;
  const int32_t *start;    // [B] position of each sequence's first new token
};
hipError_t launch_prefill_append(const PrefillGlueArgs &a, hipStream_t s);

// Dense projection of many rows (prefill, one flow); packed operands as the grouped linear's.
struct PrefillGemmArgs {
  int32_t M, K, N;          // rows, in features, out features (gate/up mode: N = 2 I)
  const uint16_t *x;        // packed rows [ceil(M / 64)][K / 32][4][64][8]
  const uint16_t *w;        // packed [K / 32][N / 16][64][8]
  void *y;                  // fp32 [M][N], or gate/up mode: bf16 packed rows with K = N / 2
  const float *residual;    // [M][N] or NULL (may alias y)
};
bool prefill_gemm_fits(int32_t K, int32_t N, bool swiglu);
hipError_t launch_prefill_gemm(const PrefillGemmArgs &a, bool swiglu, hipStream_t s);
// packed_flows > 0: y in the fragment order of xpack_offset for that many flows (rows =
// flows x batch); 0: row-major.
hipError_t launch_rmsnorm(int32_t rows, int32_t dim, const float *x, const float *gain, float eps,
                          uint16_t *y, hipStream_t s, int packed_flows = 0);
// The same norm for many rows (one wave per row; its own reduction order), y in the fragment
// order of xpack_offset for one flow.
hipError_t launch_rmsnorm_rows(int32_t rows, int32_t dim, const float *x, const float *gain, float eps,
                               uint16_t *y, hipStream_t s);
// x[f][b] = widen(embed_f[tokens[b]]) (token ids clamped to the table) and h1 = bf16(rmsnorm
// (x) * gain) in the fragment order of xpack_offset, for flows f < n_flows.
hipError_t launch_embed_norm(int32_t n_flows, int32_t batch, int32_t dim, const int32_t *tokens,
                             int32_t vocab, const uint16_t *embed0, const uint16_t *embed1,
                             const float *gain, float eps, float *x, uint16_t *h1, hipStream_t s);
// Mixture workspace: per-sequence statistics records (enough for either chunking) and the
// apply pass's per-chunk results.
size_t mixture_stats_bytes(int32_t batch, int32_t vocab);
// stats_per_tile: the projection already wrote one statistics record per 128-logit tile
// (output-head mode of the grouped linear); otherwise a statistics pass runs first.
hipError_t launch_mixture(int32_t n_flows, int32_t batch, int32_t vocab, const float *logits, const float *noise,
                          float *stats, int32_t *token, float *alpha, float *p_mix, bool stats_per_tile,
                          hipStream_t s);
hipError_t launch_swiglu(int32_t n_flows, int32_t rows, int32_t dim, const float *gu,
                         const float *b, uint16_t *out, hipStream_t s);
hipError_t launch_copy(void *dst, const void *src, size_t bytes, hipStream_t s);
// Work-groups of the read helper (its sink holds 4096 x 256 words). Over 4 GiB: 256 -> 6.92,
// 512 -> 7.07, 768 -> 6.92, 1024 -> 6.84, 4096 -> 6.75 TB/s.
constexpr int kReadBlocks = 512;
hipError_t launch_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t s);
hipError_t launch_fill(void *dst, size_t bytes, uint32_t pattern, hipStream_t s);

}  // namespace dfx
