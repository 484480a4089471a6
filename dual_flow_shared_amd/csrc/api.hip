// C ABI of libdfx.so: argument validation (before any HIP call), split planning,
// workspace carving and kernel dispatch. No device memory is allocated here and
// nothing synchronizes; every launch goes to the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "common.h"

using namespace dfx;

namespace {

thread_local char g_err[512];

dfx_status fail(dfx_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

dfx_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return DFX_OK;
  return fail(DFX_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int kMaxGridRows = 65535;  // the y and z extents of a launch grid
constexpr int kChunkQuantum = 128;  // tokens: 4 waves x 32-token tiles
constexpr int kMinChunk = 1024;   // tokens: shorter splits cost more in merge than they gain
// The vector-ALU kernel walks its split one 32-token tile after another, loading the next
// tile while it multiplies the current one, so it takes splits of two tiles or more: at batch
// 1 x 512 fp32 tokens (8 KV heads), 8 splits of 64 tokens 17.7 us against 16 of 32 tokens
// 18.2 us (4 splits 26 us, 1 split 75 us).
constexpr int kValuQuantum = 32;
constexpr int kValuMinChunk = 64;
constexpr int kMaxChunk = 8192;   // tokens: longer splits leave CUs idle when lengths differ
                                  // (doubled for small batches, see attn_plan)
constexpr int kMaxChunkLargeBatch = 3072;  // tokens, at >= 2 (sequence, KV head) pairs per CU
// Launch-shape defaults (compile-time so that alternatives can be measured).
#ifndef DFX_ATTN_TARGET
#define DFX_ATTN_TARGET 256
#endif
#ifndef DFX_GEMM_TARGET
#define DFX_GEMM_TARGET 256
#endif
#ifndef DFX_GEMM_MIN_STEPS
#define DFX_GEMM_MIN_STEPS 8
#endif
constexpr int kTargetAttnGroups = DFX_ATTN_TARGET;
constexpr int kTargetGemmGroups = DFX_GEMM_TARGET;
constexpr int kMinGemmSteps = DFX_GEMM_MIN_STEPS;  // k-steps of 32 per split, at least

dfx_status check_kv(const dfx_kv_cache *kv, int32_t batch) {
  if (!kv) return fail(DFX_EINVAL, "kv is NULL");
  if (kv->dtype != DFX_F32 && kv->dtype != DFX_BF16) return fail(DFX_EINVAL, "kv.dtype %d", kv->dtype);
  if (kv->head_dim != 64 && kv->head_dim != 128)
    return fail(DFX_EUNSUPPORTED, "head_dim %d (64 or 128 supported)", kv->head_dim);
  if (kv->num_kv_heads < 1) return fail(DFX_EINVAL, "num_kv_heads %d", kv->num_kv_heads);
  if (kv->block_size < 1) return fail(DFX_EINVAL, "block_size %d", kv->block_size);
  if (kv->num_blocks < 1) return fail(DFX_EINVAL, "num_blocks %lld", (long long)kv->num_blocks);
  if (!kv->k || !kv->v) return fail(DFX_EINVAL, "kv.k / kv.v is NULL");
  if (!aligned16(kv->k) || !aligned16(kv->v)) return fail(DFX_EINVAL, "kv.k / kv.v not 16-byte aligned");
  if (kv->reserved != 0) return fail(DFX_EINVAL, "kv.reserved must be 0");
  if (kv->block_table) {
    if (!pow2(kv->block_size)) return fail(DFX_EINVAL, "paged block_size %d is not a power of two", kv->block_size);
    if (kv->max_blocks_per_seq < 1) return fail(DFX_EINVAL, "max_blocks_per_seq %d", kv->max_blocks_per_seq);
  } else if (kv->num_blocks < batch) {
    return fail(DFX_EINVAL, "contiguous cache has %lld sequences < batch %d", (long long)kv->num_blocks, batch);
  }
  return DFX_OK;
}

int64_t capacity(const dfx_kv_cache *kv) {
  return kv->block_table ? (int64_t)kv->max_blocks_per_seq * kv->block_size : kv->block_size;
}

// block_size: paged block size, 0 for a contiguous cache. A paged split must span at
// most kMaxChunkBlocks - 1 whole blocks (the kernel holds the split's block ids in LDS).
constexpr int kMaxChunkBlocks = 1024;

// The matrix-core kernel serves bf16 caches with at most 16 query rows per KV head and paged
// blocks of >= 16 tokens (a 16-token half tile then lies in one block); the rest runs on the
// vector-ALU kernel.
bool attn_mfma_path(const dfx_kv_cache *kv, int n_flows, int group) {
  return kv->dtype == DFX_BF16 && n_flows * group <= 16 && (!kv->block_table || kv->block_size >= 16);
}

void attn_plan(int batch, int hkv, int max_ctx, int requested, int block_size, bool mfma,
               int *splits, int *chunk) {
  const int quantum = mfma ? kChunkQuantum : kValuQuantum;
  const int min_chunk = mfma ? kMinChunk : kValuMinChunk;
  const int max_s = max_ctx > 0 ? (max_ctx + quantum - 1) / quantum : 1;
  // Splits start at multiples of the quantum. The matrix-core kernel stages a split's block
  // ids in LDS: with blocks of at most a quantum a split covers whole blocks and may span
  // all kMaxChunkBlocks of them. The vector-ALU kernel reads the table directly.
  const int64_t cap = block_size <= 0 || !mfma ? (int64_t)1 << 30
      : block_size <= quantum ? (int64_t)kMaxChunkBlocks * block_size
      : ((int64_t)(kMaxChunkBlocks - 1) * block_size) / quantum * quantum;
  int s;
  if (requested > 0) {
    s = requested < max_s ? requested : max_s;
  } else {
    // Enough work-groups to fill the CUs, and splits short enough to balance the load:
    // large batches are where context lengths differ, and the more (sequence, KV head)
    // pairs per CU, the shorter the splits (the dispatcher then evens out the tails).
    // Small batches with long contexts take longer splits: there every split is full and
    // fewer, longer ones stream better. (Measured: B64 ragged 1k-16k, 456 -> 413 us with
    // 2816-token splits; B8 x 131072 with 16384-token splits, 690 -> 660 us.)
    const int pairs = batch * hkv > 0 ? batch * hkv : 1;
    s = (kTargetAttnGroups + pairs - 1) / pairs;
    const int max_chunk = pairs >= 2 * kTargetAttnGroups ? kMaxChunkLargeBatch
                          : pairs >= kTargetAttnGroups ? kMaxChunk : 2 * kMaxChunk;
    const int by_max = (max_ctx + max_chunk - 1) / max_chunk;
    if (s < by_max) s = by_max;
    const int by_min = max_ctx > min_chunk ? (max_ctx + min_chunk - 1) / min_chunk : 1;
    if (s > by_min) s = by_min;
    if (s > max_s) s = max_s;
    if (s < 1) s = 1;
  }
  int64_t c = max_ctx > 0 ? (max_ctx + s - 1) / s : quantum;
  c = (c + quantum - 1) / quantum * quantum;
  if (c > cap) c = cap;
  *chunk = (int)c;
  *splits = max_ctx > 0 ? (int)((max_ctx + c - 1) / c) : 1;
}

int paged_bs(const dfx_kv_cache *kv) { return kv->block_table ? kv->block_size : 0; }

size_t attn_ws_bytes(int splits, int n_flows, int batch, int hq, int d) {
  if (splits <= 1) return 0;
  const size_t rows = (size_t)splits * n_flows * batch * hq;
  return round_up(rows * d * sizeof(float), 256) + round_up(rows * sizeof(float), 256);
}

// The linear kernel tiles 128 output features per work-group (32 per wave) and may split K
// over ksplit work-groups of kper k-steps each, whose fp32 tiles a second kernel (or the
// layer's finish kernel) sums in split order. Splits are whole multiples of the kernel's
// 4-step unroll where K allows, so no split streams padding steps.
struct GemmPlan {
  int ksplit, kper, tiles, groups;
  size_t partial_bytes;
  size_t total() const { return partial_bytes; }
};

GemmPlan gemm_plan(int n_flows, int rows, int K, int N) {
  GemmPlan g{};
  g.tiles = (N + 127) / 128;
  const int nks = K / 32;
  // about kTargetGemmGroups work-groups (one per CU): more would add split-K partial
  // traffic faster than they add bandwidth
  int ks = kTargetGemmGroups / g.tiles;
  const int max_ks = nks / kMinGemmSteps > 1 ? nks / kMinGemmSteps : 1;
  if (ks > max_ks) ks = max_ks;
  if (ks > 16) ks = 16;
  if (ks < 1) ks = 1;
  int per = (nks + ks - 1) / ks;
  if (ks > 1) per = (per + 3) / 4 * 4;
  g.kper = per;
  g.ksplit = (nks + per - 1) / per;
  const int rpg = 64 / n_flows;
  g.groups = rows > 0 ? (rows + rpg - 1) / rpg : 0;
  if (g.ksplit > 1) g.partial_bytes = round_up((size_t)g.ksplit * g.groups * 64 * N * sizeof(float), 256);
  return g;
}

dfx_status check_linear(int32_t n_flows, int32_t rows, int32_t K, int32_t N) {
  if (n_flows != 1 && n_flows != 2) return fail(DFX_EINVAL, "n_flows %d (1 or 2)", n_flows);
  if (rows < 0) return fail(DFX_EINVAL, "rows %d", rows);
  if (K < 32 || K % 32) return fail(DFX_EUNSUPPORTED, "in_features %d is not a positive multiple of 32", K);
  if (N < 16 || N % 16) return fail(DFX_EUNSUPPORTED, "out_features %d is not a positive multiple of 16", N);
  return DFX_OK;
}

// partial: >= plan.partial_bytes of scratch (unused when the plan has one K split).
// x_f32: 0 bf16 row-major, 1 fp32 row-major, 2 bf16 in the fragment order of xpack_offset.
dfx_status run_linear_parts(int32_t n_flows, int32_t rows, int32_t K, int32_t N, int x_f32,
                            const void *x, const uint16_t *w, int w_packed, int y_bf16, void *y,
                            const float *couple, const float *residual, float *partial,
                            hipStream_t s, int tiles_only = 0, float *mix_stats = nullptr) {
  if (rows == 0) return DFX_OK;
  const GemmPlan g = gemm_plan(n_flows, rows, K, N);
  GemmArgs a{};
  a.mix_stats = g.ksplit == 1 ? mix_stats : nullptr;
  a.n_flows = n_flows; a.rows = rows; a.K = K; a.N = N;
  a.x_f32 = x_f32 == 1; a.x_packed = x_f32 == 2;
  a.x = x; a.w = w; a.w_packed = w_packed; a.y_bf16 = y_bf16; a.y = y;
  a.couple = couple; a.residual = residual; a.ksplit = g.ksplit; a.kper = g.kper;
  a.partial = g.ksplit > 1 || tiles_only ? partial : nullptr;
  a.tiles_only = tiles_only;
  return hip_status(launch_grouped_linear(a, s), "grouped_linear launch");
}

// Gate/up projection fused with SwiGLU and the b coupling (one split, no tiles): bf16 rows of
// the intermediate, in the down projection's fragment order, straight from the accumulators.
dfx_status run_gate_up_swiglu(int32_t n_flows, int32_t rows, int32_t H, int32_t I, const void *x_packed,
                              const uint16_t *w_packed, const float *b, uint16_t *inter, hipStream_t s) {
  if (rows == 0) return DFX_OK;
  GemmArgs a{};
  a.n_flows = n_flows; a.rows = rows; a.K = H; a.N = 2 * I;
  a.x_packed = 1; a.x = x_packed; a.w = w_packed; a.w_packed = 1; a.y = inter;
  a.couple = n_flows == 2 ? b : nullptr; a.ksplit = 1; a.kper = H / 32; a.swiglu = 1;
  return hip_status(launch_grouped_linear(a, s), "gate/up launch");
}

dfx_status run_linear(int32_t n_flows, int32_t rows, int32_t K, int32_t N, int x_f32, const void *x,
                      const uint16_t *w, int w_packed, int y_bf16, void *y, const float *couple,
                      const float *residual, void *ws, size_t ws_bytes, hipStream_t s) {
  if (rows == 0) return DFX_OK;
  const GemmPlan g = gemm_plan(n_flows, rows, K, N);
  if (g.total() > 0 && (!ws || ws_bytes < g.total()))
    return fail(DFX_EWORKSPACE, "grouped_linear needs %zu workspace bytes, got %zu", g.total(), ws_bytes);
  return run_linear_parts(n_flows, rows, K, N, x_f32, x, w, w_packed, y_bf16, y, couple,
                          residual, (float *)ws, s);
}

struct AttnCall {
  const dfx_kv_cache *kv;
  const int32_t *ctx;
  int32_t batch, max_context, hq, q_dtype;
  const void *q1, *q2;
  int64_t q_bstride;
  const float *a;
  int32_t a_stride;
  float scale;
  float *o1, *o2, *lse;
  int32_t splits;
  void *ws;
  size_t ws_bytes;
  int32_t o_bf16;  // layer-internal: 1 = outputs rounded to bf16 (the rows entering W_o),
                   // 2 = bf16 in the grouped linear's fragment order, both flows from o1
};

dfx_status validate_attn(const AttnCall &c) {
  dfx_status st = check_kv(c.kv, c.batch);
  if (st) return st;
  const dfx_kv_cache *kv = c.kv;
  if (c.batch < 0) return fail(DFX_EINVAL, "batch %d", c.batch);
  if (c.hq < 1 || c.hq % kv->num_kv_heads)
    return fail(DFX_EINVAL, "num_q_heads %d is not a positive multiple of num_kv_heads %d", c.hq, kv->num_kv_heads);
  if (c.q_dtype != DFX_F32 && c.q_dtype != DFX_BF16) return fail(DFX_EINVAL, "q_dtype %d", c.q_dtype);
  if (c.max_context < 0 || c.max_context > capacity(kv))
    return fail(DFX_EINVAL, "max_context %d outside [0, capacity %lld]", c.max_context, (long long)capacity(kv));
  if (c.batch > kMaxGridRows) return fail(DFX_EUNSUPPORTED, "batch %d above %d", c.batch, kMaxGridRows);
  if (c.batch > 0 && !c.ctx) return fail(DFX_EINVAL, "context_lens is NULL");
  if (c.batch > 0 && kv->block_table == nullptr && kv->num_blocks < c.batch)
    return fail(DFX_EINVAL, "contiguous cache smaller than batch");
  if (!c.q1 || !c.o1) return fail(DFX_EINVAL, "q1 / o1 is NULL");
  if ((c.q2 == nullptr) != (c.o2 == nullptr)) return fail(DFX_EINVAL, "q2_raw and o2 must be both NULL or both set");
  if (c.a && !c.q2) return fail(DFX_EINVAL, "coupling vector a given without q2_raw");
  if (c.a_stride != 0 && c.a_stride != kv->head_dim)
    return fail(DFX_EINVAL, "a_head_stride %d (0 or head_dim)", c.a_stride);
  const int64_t row = (int64_t)c.hq * kv->head_dim;
  if (c.q_bstride < 0 || (c.q_bstride != 0 && (c.q_bstride < row || c.q_bstride % 8)))
    return fail(DFX_EINVAL, "q_batch_stride %lld", (long long)c.q_bstride);
  if (!aligned16(c.q1) || (c.q2 && !aligned16(c.q2)) || !aligned16(c.o1) || (c.o2 && !aligned16(c.o2)))
    return fail(DFX_EINVAL, "q / o pointers must be 16-byte aligned");
  if (c.a && ((uintptr_t)c.a & 3)) return fail(DFX_EINVAL, "a not 4-byte aligned");
  if (c.splits < 0) return fail(DFX_EINVAL, "num_splits %d", c.splits);
  const int G = c.hq / kv->num_kv_heads, F = c.q2 ? 2 : 1;
  if (F * G > 32) return fail(DFX_EUNSUPPORTED, "%d query rows per KV head (at most 32)", F * G);
  return DFX_OK;
}

dfx_status run_attn(const AttnCall &c, hipStream_t s) {
  dfx_status st = validate_attn(c);
  if (st) return st;
  const dfx_kv_cache *kv = c.kv;
  const int F = c.q2 ? 2 : 1, G = c.hq / kv->num_kv_heads;
  int splits, chunk;
  const bool mfma = attn_mfma_path(kv, F, G);
  attn_plan(c.batch, kv->num_kv_heads, c.max_context, c.splits, paged_bs(kv), mfma, &splits, &chunk);
  if (splits > kMaxGridRows) return fail(DFX_EUNSUPPORTED, "%d context splits above %d", splits, kMaxGridRows);
  const size_t need = attn_ws_bytes(splits, F, c.batch, c.hq, kv->head_dim);
  if (need && (!c.ws || c.ws_bytes < need))
    return fail(DFX_EWORKSPACE, "decode_attn needs %zu workspace bytes for %d splits, got %zu", need, splits, c.ws_bytes);
  if (c.batch == 0) return DFX_OK;
  AttnArgs a{};
  a.k = kv->k; a.v = kv->v; a.table = kv->block_table; a.num_blocks = kv->num_blocks;
  a.max_blocks = kv->max_blocks_per_seq; a.block_size = kv->block_size;
  a.block_shift = kv->block_table ? (int)__builtin_ctz((unsigned)kv->block_size) : -1;
  a.num_kv_heads = kv->num_kv_heads; a.head_dim = kv->head_dim; a.group = G;
  a.num_q_heads = c.hq; a.n_flows = F; a.batch = c.batch; a.ctx = c.ctx; a.max_context = c.max_context;
  a.q1 = c.q1; a.q2 = c.q2; a.q_bstride = c.q_bstride ? c.q_bstride : (int64_t)c.hq * kv->head_dim;
  a.q_bf16 = c.q_dtype == DFX_BF16; a.kv_bf16 = kv->dtype == DFX_BF16;
  a.a = c.a; a.a_hstride = c.a_stride;
  const float scale = c.scale > 0.f ? c.scale : 1.0f / sqrtf((float)kv->head_dim);
  a.scale_log2 = scale * kLog2e;
  a.o1 = c.o1; a.o2 = c.o2; a.lse = c.lse; a.o_bf16 = c.o_bf16 != 0; a.o_packed = c.o_bf16 == 2;
  a.num_splits = splits; a.chunk = chunk;
  // K tiles through LDS as whole rows at >= 2 (sequence, KV head) pairs per CU, where the
  // whole-row loads stream faster (measured: B64 ragged 1k-16k paged, 412 -> 388 us); with
  // fewer pairs the direct A-operand loads are as fast or slightly faster (B32 x 8192 paged
  // 165 vs 167 us, B16 x 4096 contiguous 49.6 vs 50.5 us, B8 x 131072 the same).
  a.k_rows = c.batch * kv->num_kv_heads >= 2 * kTargetAttnGroups;
  if (splits > 1) {
    const size_t rows = (size_t)splits * F * c.batch * c.hq;
    a.part_o = (float *)c.ws;
    a.part_lse = (float *)((char *)c.ws + round_up(rows * kv->head_dim * sizeof(float), 256));
  }
  hipError_t e = mfma ? launch_attn_mfma(a, s) : launch_attn_valu(a, s);
  if (e != hipSuccess) return hip_status(e, "decode_attn launch");
  if (splits > 1) return hip_status(launch_attn_merge(a, s), "decode_attn merge launch");
  return DFX_OK;
}

}  // namespace

extern "C" {

int dfx_version(void) { return DFX_VERSION; }

const char *dfx_last_error(void) { return g_err; }

#define DFX_BEGIN g_err[0] = 0; try {
#define DFX_END } catch (...) { return fail(DFX_EINVAL, "internal error"); }

dfx_status dfx_decode_attn_plan(const dfx_kv_cache *kv, int32_t batch, int32_t num_q_heads,
                                int32_t n_flows, int32_t max_context, int32_t num_splits,
                                int32_t *splits_out, size_t *workspace_bytes) {
  DFX_BEGIN
  dfx_status st = check_kv(kv, batch < 0 ? 0 : batch);
  if (st) return st;
  if (batch < 0 || num_q_heads < 1 || (n_flows != 1 && n_flows != 2) || max_context < 0 || num_splits < 0)
    return fail(DFX_EINVAL, "bad plan arguments");
  if (max_context > capacity(kv)) return fail(DFX_EINVAL, "max_context above cache capacity");
  int s, c;
  const int G = num_q_heads % kv->num_kv_heads == 0 ? num_q_heads / kv->num_kv_heads : 32;
  attn_plan(batch, kv->num_kv_heads, max_context, num_splits, paged_bs(kv), attn_mfma_path(kv, n_flows, G),
            &s, &c);
  if (splits_out) *splits_out = s;
  if (workspace_bytes) *workspace_bytes = attn_ws_bytes(s, n_flows, batch, num_q_heads, kv->head_dim);
  return DFX_OK;
  DFX_END
}

dfx_status dfx_decode_attn_workspace_size(int32_t batch, int32_t num_q_heads, int32_t n_flows,
                                          const dfx_kv_cache *kv, int32_t max_context, int32_t num_splits,
                                          size_t *bytes) {
  DFX_BEGIN
  if (!bytes) return fail(DFX_EINVAL, "bytes is NULL");
  return dfx_decode_attn_plan(kv, batch, num_q_heads, n_flows, max_context, num_splits, nullptr, bytes);
  DFX_END
}

dfx_status dfx_decode_attn(const dfx_kv_cache *kv, const int32_t *context_lens, int32_t batch,
                           int32_t max_context, int32_t num_q_heads, int32_t q_dtype,
                           const void *q1, const void *q2_raw, int64_t q_batch_stride,
                           const float *a, int32_t a_head_stride, float softmax_scale,
                           float *o1, float *o2, float *lse, int32_t num_splits,
                           void *workspace, size_t workspace_bytes, void *stream) {
  DFX_BEGIN
  AttnCall c{kv, context_lens, batch, max_context, num_q_heads, q_dtype, q1, q2_raw, q_batch_stride,
             a, a_head_stride, softmax_scale, o1, o2, lse, num_splits, workspace, workspace_bytes, 0};
  return run_attn(c, (hipStream_t)stream);
  DFX_END
}

dfx_status dfx_kv_append_primary(const dfx_kv_cache *kv, int32_t batch, const int32_t *positions,
                                 int32_t src_dtype, const void *k_new, const void *v_new,
                                 int64_t src_row_stride, void *stream) {
  DFX_BEGIN
  dfx_status st = check_kv(kv, batch < 0 ? 0 : batch);
  if (st) return st;
  if (batch < 0) return fail(DFX_EINVAL, "batch %d", batch);
  if (src_dtype != DFX_F32 && src_dtype != DFX_BF16) return fail(DFX_EINVAL, "src_dtype %d", src_dtype);
  if (batch > 0 && (!positions || !k_new || !v_new)) return fail(DFX_EINVAL, "positions / k_new / v_new is NULL");
  const int64_t row = (int64_t)kv->num_kv_heads * kv->head_dim;
  if (src_row_stride < 0 || (src_row_stride != 0 && (src_row_stride < row || src_row_stride % 8)))
    return fail(DFX_EINVAL, "src_row_stride %lld", (long long)src_row_stride);
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(DFX_EINVAL, "k_new / v_new not 16-byte aligned");
  if (batch == 0) return DFX_OK;
  return hip_status(launch_kv_append(*kv, batch, positions, 0, src_dtype == DFX_F32, k_new, v_new,
                                     src_row_stride ? src_row_stride : row, (hipStream_t)stream),
                    "kv_append launch");
  DFX_END
}

dfx_status dfx_grouped_linear_workspace_size(int32_t n_flows, int32_t rows, int32_t in_features,
                                             int32_t out_features, size_t *bytes) {
  DFX_BEGIN
  dfx_status st = check_linear(n_flows, rows, in_features, out_features);
  if (st) return st;
  if (!bytes) return fail(DFX_EINVAL, "bytes is NULL");
  *bytes = rows > 0 ? gemm_plan(n_flows, rows, in_features, out_features).total() : 0;
  return DFX_OK;
  DFX_END
}

dfx_status dfx_grouped_linear(int32_t n_flows, int32_t rows, int32_t in_features,
                              int32_t out_features, int32_t x_dtype, const void *x,
                              const uint16_t *w, int32_t w_layout, int32_t y_dtype, void *y,
                              const float *couple, const float *residual, void *workspace,
                              size_t workspace_bytes, void *stream) {
  DFX_BEGIN
  dfx_status st = check_linear(n_flows, rows, in_features, out_features);
  if (st) return st;
  if (x_dtype != DFX_F32 && x_dtype != DFX_BF16) return fail(DFX_EINVAL, "x_dtype %d", x_dtype);
  if (y_dtype != DFX_F32 && y_dtype != DFX_BF16) return fail(DFX_EINVAL, "y_dtype %d", y_dtype);
  if (w_layout != DFX_W_ROW_MAJOR && w_layout != DFX_W_PACKED) return fail(DFX_EINVAL, "w_layout %d", w_layout);
  if (rows > 0 && (!x || !w || !y)) return fail(DFX_EINVAL, "x / w / y is NULL");
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (residual && !aligned16(residual)))
    return fail(DFX_EINVAL, "x / w / y / residual not 16-byte aligned");
  if (couple && ((uintptr_t)couple & 3)) return fail(DFX_EINVAL, "couple not 4-byte aligned");
  return run_linear(n_flows, rows, in_features, out_features, x_dtype == DFX_F32, x, w,
                    w_layout == DFX_W_PACKED, y_dtype == DFX_BF16, y, couple, residual, workspace,
                    workspace_bytes, (hipStream_t)stream);
  DFX_END
}

dfx_status dfx_pack_weight(int32_t out_features, int32_t in_features, const uint16_t *w,
                           uint16_t *packed, void *stream) {
  DFX_BEGIN
  if (out_features < 16 || out_features % 16 || in_features < 32 || in_features % 32)
    return fail(DFX_EINVAL, "pack_weight needs N %% 16 == 0 and K %% 32 == 0 (got %d x %d)", out_features, in_features);
  if (!w || !packed || !aligned16(w) || !aligned16(packed)) return fail(DFX_EINVAL, "w / packed NULL or misaligned");
  const size_t bytes = (size_t)out_features * in_features * 2;
  if ((const char *)w < (const char *)packed + bytes && (const char *)packed < (const char *)w + bytes)
    return fail(DFX_EINVAL, "w and packed overlap");
  return hip_status(launch_pack_weight(out_features, in_features, w, packed, (hipStream_t)stream),
                    "pack_weight launch");
  DFX_END
}

dfx_status dfx_rmsnorm(int32_t rows, int32_t dim, const float *x, const float *gain, float eps,
                       uint16_t *y, void *stream) {
  DFX_BEGIN
  if (rows < 0 || dim < 4 || dim % 4 || dim > 16384) return fail(DFX_EINVAL, "rows %d dim %d", rows, dim);
  if (rows > 0 && (!x || !gain || !y)) return fail(DFX_EINVAL, "x / gain / y is NULL");
  if (!aligned16(x) || !aligned16(gain) || ((uintptr_t)y & 7)) return fail(DFX_EINVAL, "misaligned pointer");
  if (!(eps >= 0.f)) return fail(DFX_EINVAL, "eps");
  return hip_status(launch_rmsnorm(rows, dim, x, gain, eps, y, (hipStream_t)stream), "rmsnorm launch");
  DFX_END
}

dfx_status dfx_swiglu_couple(int32_t rows, int32_t n_flows, int32_t dim, const float *gate_up,
                             const float *b, uint16_t *out, void *stream) {
  DFX_BEGIN
  if ((n_flows != 1 && n_flows != 2) || rows < 0 || dim < 4 || dim % 4)
    return fail(DFX_EINVAL, "n_flows %d rows %d dim %d", n_flows, rows, dim);
  if (rows > 0 && (!gate_up || !out)) return fail(DFX_EINVAL, "gate_up / out is NULL");
  if (!aligned16(gate_up) || (b && !aligned16(b)) || ((uintptr_t)out & 7)) return fail(DFX_EINVAL, "misaligned pointer");
  return hip_status(launch_swiglu(n_flows, rows, dim, gate_up, b, out, (hipStream_t)stream), "swiglu launch");
  DFX_END
}

// ---- one dual-flow decode layer ---------------------------------------------------

namespace {

// Workspace regions of one layer call, in this order: the projections' split-K tiles, then
// every intermediate the step rounds to bf16 or hands on, each in a region of its own so
// that it can be inspected after the call (dfx_dual_flow_decode_layer_taps), then the
// attention's split partials.
struct LayerPlan {
  size_t tiles, h1, qkv, o, h2, inter, attn_ws, total;
  int splits;
};

dfx_status layer_plan(const dfx_layer_weights *w, const dfx_kv_cache *kv, int32_t batch,
                      int32_t n_flows, int32_t max_context, LayerPlan *pl) {
  if (!w) return fail(DFX_EINVAL, "weights is NULL");
  dfx_status st = check_kv(kv, batch < 0 ? 0 : batch);
  if (st) return st;
  if (batch < 0 || (n_flows != 1 && n_flows != 2)) return fail(DFX_EINVAL, "batch %d n_flows %d", batch, n_flows);
  if (batch > kMaxGridRows) return fail(DFX_EUNSUPPORTED, "batch %d above %d", batch, kMaxGridRows);
  if (kv->dtype != DFX_BF16) return fail(DFX_EUNSUPPORTED, "layer needs a bf16 cache");
  if (w->head_dim != kv->head_dim || w->num_kv_heads != kv->num_kv_heads)
    return fail(DFX_EINVAL, "weights and cache disagree on head_dim / num_kv_heads");
  if (w->num_q_heads < 1 || w->num_q_heads % w->num_kv_heads) return fail(DFX_EINVAL, "num_q_heads %d", w->num_q_heads);
  if (w->hidden < 32 || w->hidden % 32 || w->hidden > 16384) return fail(DFX_EUNSUPPORTED, "hidden %d", w->hidden);
  if (w->intermediate < 32 || w->intermediate % 32) return fail(DFX_EUNSUPPORTED, "intermediate %d", w->intermediate);
  if (!(w->rms_eps >= 0.f)) return fail(DFX_EINVAL, "rms_eps");
  if (!w->attn_norm_gain || !w->w_qkv || !w->w_o || !w->mlp_norm_gain || !w->w_gate_up || !w->w_down)
    return fail(DFX_EINVAL, "a weight pointer is NULL");
  if (max_context < 1 || max_context > capacity(kv)) return fail(DFX_EINVAL, "max_context %d", max_context);
  const int F = n_flows, B = batch, H = w->hidden, D = w->head_dim, Hq = w->num_q_heads;
  const int Nqkv = (Hq + 2 * w->num_kv_heads) * D, I = w->intermediate;
  LayerPlan p{};
  auto a256 = [](size_t x) { return round_up(x, 256); };
  // bf16 rows entering a projection are stored in its fragment order: 64 rows per group
  const size_t prow = (size_t)(B + 64 / F - 1) / (64 / F) * 64;
  p.h1 = a256(prow * H * 2);               // normed rows entering W_qkv
  p.qkv = a256((size_t)F * B * Nqkv * 4);  // Q columns (row stride Nqkv)
  p.o = a256(prow * Hq * D * 2);           // attention rows entering W_o
  p.h2 = a256(prow * H * 2);               // normed rows entering W_gate_up
  p.inter = a256(prow * I * 2);            // SwiGLU rows entering W_down
  int chunk;
  attn_plan(B, kv->num_kv_heads, max_context, 0, paged_bs(kv), attn_mfma_path(kv, F, Hq / kv->num_kv_heads),
            &p.splits, &chunk);
  if (p.splits > kMaxGridRows) return fail(DFX_EUNSUPPORTED, "%d context splits above %d", p.splits, kMaxGridRows);
  p.attn_ws = a256(attn_ws_bytes(p.splits, F, B, Hq, D));
  // the projections followed by a finish kernel write their fp32 tiles
  // [ksplit][groups][64][N]; they run in stream order, so one region serves them all
  const int shapes[3][2] = {{H, Nqkv}, {Hq * D, H}, {I, H}};  // the gate/up pass writes no tiles
  for (auto &sh : shapes) {
    const GemmPlan g = gemm_plan(F, B, sh[0], sh[1]);
    const size_t t = (size_t)g.ksplit * g.groups * 64 * sh[1] * sizeof(float);
    p.tiles = t > p.tiles ? t : p.tiles;
  }
  p.tiles = a256(p.tiles);
  p.total = p.tiles + p.h1 + p.qkv + p.o + p.h2 + p.inter + p.attn_ws;
  *pl = p;
  return DFX_OK;
}


// Workspace regions large enough for every layer of a stack (same hidden size): each region
// the largest any layer needs, so all layers share one layout.
dfx_status step_plan(const dfx_layer_weights *layers, const dfx_kv_cache *caches, int32_t n_layers,
                     int32_t batch, int32_t n_flows, int32_t max_context, LayerPlan *pl) {
  if (n_layers < 1 || !layers || !caches) return fail(DFX_EINVAL, "n_layers %d / layers / caches", n_layers);
  LayerPlan m{};
  for (int l = 0; l < n_layers; ++l) {
    LayerPlan q;
    dfx_status st = layer_plan(&layers[l], &caches[l], batch, n_flows, max_context, &q);
    if (st) return st;
    if (layers[l].hidden != layers[0].hidden) return fail(DFX_EINVAL, "layer %d hidden %d != %d", l, layers[l].hidden, layers[0].hidden);
    m.tiles = std::max(m.tiles, q.tiles); m.h1 = std::max(m.h1, q.h1); m.qkv = std::max(m.qkv, q.qkv);
    m.o = std::max(m.o, q.o); m.h2 = std::max(m.h2, q.h2); m.inter = std::max(m.inter, q.inter);
    m.attn_ws = std::max(m.attn_ws, q.attn_ws);
  }
  m.total = m.tiles + m.h1 + m.qkv + m.o + m.h2 + m.inter + m.attn_ws;
  *pl = m;
  return DFX_OK;
}

// One layer on a workspace laid out by the region sizes of `p`. norm_in: normalize x into h1
// first (else h1 already holds this layer's normed rows). next: finish the down projection
// into the next layer's normed rows (in h1) instead of a plain residual update.
dfx_status run_layer(const dfx_layer_weights *w, const dfx_kv_cache *kv, const int32_t *context_lens, int B,
                     int max_context, int F, float *x, const LayerPlan &p, char *base, hipStream_t s,
                     bool norm_in, const dfx_layer_weights *next) {
  const int H = w->hidden, D = w->head_dim, Hq = w->num_q_heads;
  const int Hkv = w->num_kv_heads, Nqkv = (Hq + 2 * Hkv) * D, I = w->intermediate;
  float *tiles = (float *)base;
  uint16_t *h1 = (uint16_t *)(base + p.tiles);
  float *qkv = (float *)((char *)h1 + p.h1);
  uint16_t *ob = (uint16_t *)((char *)qkv + p.qkv);
  uint16_t *h2 = (uint16_t *)((char *)ob + p.o);
  uint16_t *inter = (uint16_t *)((char *)h2 + p.h2);
  void *aws = (char *)inter + p.inter;
  dfx_status r;
  LayerGlueArgs g{};
  g.n_flows = F; g.batch = B; g.tiles = tiles; g.x = x; g.eps = w->rms_eps;
  g.kv = *kv; g.ctx = context_lens; g.max_context = max_context; g.num_q_heads = Hq; g.head_dim = D;
  auto ksplit = [&](int K, int N) { return gemm_plan(F, B, K, N).ksplit; };
  // attention block: norm, shared Q/K/V projection, primary-only append, dual attention
  if (norm_in && (r = hip_status(launch_rmsnorm(F * B, H, x, w->attn_norm_gain, w->rms_eps, h1, s, F), "rmsnorm launch")))
    return r;
  if ((r = run_linear_parts(F, B, H, Nqkv, 2, h1, w->w_qkv, 1, 0, nullptr, nullptr, nullptr, tiles, s, 1))) return r;
  g.N = Nqkv; g.ksplit = ksplit(H, Nqkv); g.out = qkv;
  if ((r = hip_status(launch_layer_glue(kGlueQkv, g, s), "qkv finish launch"))) return r;
  // attention writes its rows already rounded to bf16, in W_o's fragment order
  AttnCall c{kv, context_lens, B, max_context, Hq, DFX_F32, qkv, F == 2 ? qkv + (size_t)B * Nqkv : nullptr,
             Nqkv, F == 2 ? w->couple_a : nullptr, 0, 0.f, (float *)ob,
             F == 2 ? (float *)ob : nullptr, nullptr, 0, aws, p.attn_ws, 2};
  if ((r = run_attn(c, s))) return r;
  // output projection + residual, then the MLP norm
  if ((r = run_linear_parts(F, B, Hq * D, H, 2, ob, w->w_o, 1, 0, nullptr, nullptr, nullptr, tiles, s, 1))) return r;
  g.N = H; g.ksplit = ksplit(Hq * D, H); g.gain = w->mlp_norm_gain; g.h = h2;
  if ((r = hip_status(launch_layer_glue(kGlueONorm, g, s), "o finish launch"))) return r;
  // MLP: shared gate/up projection, SwiGLU with b coupling, shared down projection with
  // c coupling and the residual (and the next layer's norm)
  if ((r = run_gate_up_swiglu(F, B, H, I, h2, w->w_gate_up, w->couple_b, inter, s))) return r;
  if ((r = run_linear_parts(F, B, I, H, 2, inter, w->w_down, 1, 0, nullptr, nullptr, nullptr, tiles, s, 1))) return r;
  g.N = H; g.ksplit = ksplit(I, H); g.couple = F == 2 ? w->couple_c : nullptr;
  if (!next) return hip_status(launch_layer_glue(kGlueDown, g, s), "down finish launch");
  g.gain = next->attn_norm_gain; g.eps = next->rms_eps; g.h = h1;
  return hip_status(launch_layer_glue(kGlueDownNorm, g, s), "down finish + norm launch");
}

}  // namespace

dfx_status dfx_dual_flow_decode_layer_workspace_size(const dfx_layer_weights *w,
                                                     const dfx_kv_cache *kv, int32_t batch,
                                                     int32_t n_flows, int32_t max_context,
                                                     size_t *bytes) {
  DFX_BEGIN
  LayerPlan p;
  dfx_status st = layer_plan(w, kv, batch, n_flows, max_context, &p);
  if (st) return st;
  if (!bytes) return fail(DFX_EINVAL, "bytes is NULL");
  *bytes = p.total;
  return DFX_OK;
  DFX_END
}

dfx_status dfx_dual_flow_decode_layer(const dfx_layer_weights *w, const dfx_kv_cache *kv,
                                      const int32_t *context_lens, int32_t batch,
                                      int32_t max_context, int32_t n_flows, float *x,
                                      void *workspace, size_t workspace_bytes, void *stream) {
  DFX_BEGIN
  LayerPlan p;
  dfx_status st = layer_plan(w, kv, batch, n_flows, max_context, &p);
  if (st) return st;
  if (batch > 0 && (!context_lens || !x)) return fail(DFX_EINVAL, "context_lens / x is NULL");
  if (!aligned16(x)) return fail(DFX_EINVAL, "x not 16-byte aligned");
  if (!workspace || workspace_bytes < p.total)
    return fail(DFX_EWORKSPACE, "layer needs %zu workspace bytes, got %zu", p.total, workspace_bytes);
  if (batch == 0) return DFX_OK;
  return run_layer(w, kv, context_lens, batch, max_context, n_flows, x, p, (char *)workspace,
                   (hipStream_t)stream, true, nullptr);
  DFX_END
}

dfx_status dfx_dual_flow_decode_step_workspace_size(const dfx_layer_weights *layers,
                                                    const dfx_kv_cache *caches, int32_t n_layers,
                                                    int32_t batch, int32_t n_flows,
                                                    int32_t max_context, size_t *bytes) {
  DFX_BEGIN
  LayerPlan p;
  dfx_status st = step_plan(layers, caches, n_layers, batch, n_flows, max_context, &p);
  if (st) return st;
  if (!bytes) return fail(DFX_EINVAL, "bytes is NULL");
  *bytes = p.total;
  return DFX_OK;
  DFX_END
}

dfx_status dfx_dual_flow_decode_step(const dfx_layer_weights *layers, const dfx_kv_cache *caches,
                                     int32_t n_layers, const int32_t *tokens, int32_t vocab,
                                     const uint16_t *embed_primary, const uint16_t *embed_aux,
                                     const int32_t *context_lens, int32_t batch, int32_t max_context,
                                     int32_t n_flows, float *x, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  DFX_BEGIN
  LayerPlan p;
  dfx_status st = step_plan(layers, caches, n_layers, batch, n_flows, max_context, &p);
  if (st) return st;
  if (vocab < 1) return fail(DFX_EINVAL, "vocab %d", vocab);
  if (!embed_primary || (n_flows == 2 && !embed_aux))
    return fail(DFX_EINVAL, "embedding table is NULL (the auxiliary flow has its own)");
  if (((uintptr_t)embed_primary & 7) || (embed_aux && ((uintptr_t)embed_aux & 7)))
    return fail(DFX_EINVAL, "embedding tables must be 8-byte aligned");
  if (batch > 0 && (!context_lens || !x || !tokens)) return fail(DFX_EINVAL, "tokens / context_lens / x is NULL");
  if (!aligned16(x)) return fail(DFX_EINVAL, "x not 16-byte aligned");
  if (!workspace || workspace_bytes < p.total)
    return fail(DFX_EWORKSPACE, "decode step needs %zu workspace bytes, got %zu", p.total, workspace_bytes);
  if (batch == 0) return DFX_OK;
  hipStream_t s = (hipStream_t)stream;
  const dfx_layer_weights &w0 = layers[0];
  // both flows' embedding rows and layer 0's normed rows, in one kernel
  dfx_status r = hip_status(launch_embed_norm(n_flows, batch, w0.hidden, tokens, vocab, embed_primary, embed_aux,
                                              w0.attn_norm_gain, w0.rms_eps, x,
                                              (uint16_t *)((char *)workspace + p.tiles), s),
                            "embedding launch");
  if (r) return r;
  // each layer but the last finishes its down projection into the next layer's normed rows
  for (int l = 0; l < n_layers; ++l) {
    r = run_layer(&layers[l], &caches[l], context_lens, batch, max_context, n_flows, x, p, (char *)workspace, s,
                  false, l + 1 < n_layers ? &layers[l + 1] : nullptr);
    if (r) return r;
  }
  return DFX_OK;
  DFX_END
}

dfx_status dfx_dual_flow_decode_layer_taps(const dfx_layer_weights *w, const dfx_kv_cache *kv,
                                           int32_t batch, int32_t n_flows, int32_t max_context,
                                           dfx_layer_taps *taps) {
  DFX_BEGIN
  LayerPlan p;
  dfx_status st = layer_plan(w, kv, batch, n_flows, max_context, &p);
  if (st) return st;
  if (!taps) return fail(DFX_EINVAL, "taps is NULL");
  taps->h1 = p.tiles;
  taps->q = taps->h1 + p.h1;
  taps->o = taps->q + p.qkv;
  taps->h2 = taps->o + p.o;
  taps->inter = taps->h2 + p.h2;
  return DFX_OK;
  DFX_END
}

namespace {

// Workspace of the output head: normed rows (bf16, the projection's fragment order), fp32
// logits [F][B][V], the projection's split-K partials, the mixture's per-chunk statistics.
struct HeadPlan {
  size_t h, logits, partial, stats, total;
};

dfx_status head_plan(int32_t F, int32_t B, int32_t H, int32_t V, HeadPlan *hp) {
  if ((F != 1 && F != 2) || B < 0 || B > 65535) return fail(DFX_EINVAL, "n_flows %d batch %d", F, B);
  if (H < 32 || H % 32 || H > 16384) return fail(DFX_EUNSUPPORTED, "hidden %d (a multiple of 32, at most 16384)", H);
  if (V < 16 || V % 16) return fail(DFX_EUNSUPPORTED, "vocab %d is not a positive multiple of 16", V);
  auto a256 = [](size_t x) { return round_up(x, 256); };
  HeadPlan p{};
  const size_t prow = (size_t)(B + 64 / F - 1) / (64 / F) * 64;
  p.h = a256(prow * H * 2);
  p.logits = a256((size_t)F * B * V * 4);
  p.partial = B > 0 ? a256(gemm_plan(F, B, H, V).total()) : 0;
  p.stats = a256(mixture_stats_bytes(B, V));
  p.total = p.h + p.logits + p.partial + p.stats;
  *hp = p;
  return DFX_OK;
}

}  // namespace

dfx_status dfx_dual_flow_output_head_workspace_size(int32_t n_flows, int32_t batch, int32_t hidden,
                                                    int32_t vocab, size_t *bytes) {
  DFX_BEGIN
  HeadPlan p;
  dfx_status st = head_plan(n_flows, batch, hidden, vocab, &p);
  if (st) return st;
  if (!bytes) return fail(DFX_EINVAL, "bytes is NULL");
  *bytes = p.total;
  return DFX_OK;
  DFX_END
}

dfx_status dfx_dual_flow_output_head_taps(int32_t n_flows, int32_t batch, int32_t hidden, int32_t vocab,
                                          size_t *h_offset, size_t *logits_offset) {
  DFX_BEGIN
  HeadPlan p;
  dfx_status st = head_plan(n_flows, batch, hidden, vocab, &p);
  if (st) return st;
  if (!h_offset || !logits_offset) return fail(DFX_EINVAL, "offset pointer is NULL");
  *h_offset = 0;
  *logits_offset = p.h;
  return DFX_OK;
  DFX_END
}

dfx_status dfx_dual_flow_output_head(int32_t n_flows, int32_t batch, int32_t hidden, int32_t vocab,
                                     const float *x, const float *norm_gain, float eps,
                                     const uint16_t *w_out, const float *uniform_noise,
                                     int32_t *next_token, float *alpha, float *p_mix, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  DFX_BEGIN
  HeadPlan p;
  dfx_status st = head_plan(n_flows, batch, hidden, vocab, &p);
  if (st) return st;
  if (!(eps >= 0.f)) return fail(DFX_EINVAL, "eps");
  if (batch > 0 && (!x || !norm_gain || !w_out || !next_token))
    return fail(DFX_EINVAL, "x / norm_gain / w_out / next_token is NULL");
  if (!aligned16(x) || !aligned16(norm_gain) || !aligned16(w_out) || !aligned16(uniform_noise) || !aligned16(p_mix) ||
      ((uintptr_t)next_token & 3) || ((uintptr_t)alpha & 3))
    return fail(DFX_EINVAL, "misaligned pointer");
  if (batch == 0) return DFX_OK;
  if (!workspace || workspace_bytes < p.total)
    return fail(DFX_EWORKSPACE, "output head needs %zu workspace bytes, got %zu", p.total, workspace_bytes);
  hipStream_t s = (hipStream_t)stream;
  char *base = (char *)workspace;
  uint16_t *h = (uint16_t *)base;
  float *logits = (float *)(base + p.h);
  float *partial = (float *)(base + p.h + p.logits);
  float *stats = (float *)(base + p.h + p.logits + p.partial);
  dfx_status r = hip_status(launch_rmsnorm(n_flows * batch, hidden, x, norm_gain, eps, h, s, n_flows), "rmsnorm launch");
  if (r) return r;
  // one pass over the shared vocabulary matrix for both flows' rows; in one K split the
  // projection also writes the softmax statistics of each 128-logit tile
  const bool tile_stats = gemm_plan(n_flows, batch, hidden, vocab).ksplit == 1;
  if ((r = run_linear_parts(n_flows, batch, hidden, vocab, 2, h, w_out, 1, 0, logits, nullptr, nullptr, partial, s,
                            0, stats)))
    return r;
  return hip_status(launch_mixture(n_flows, batch, vocab, logits, uniform_noise, stats, next_token, alpha, p_mix,
                                   tile_stats, s),
                    "mixture launch");
  DFX_END
}

namespace {

// Workspace of the MoE block, in this order: normed rows, router logits, selections, expert
// lists, gathered rows, intermediates, the down projection's tiles.
struct MoePlan {
  size_t h, logits, ids, wts, pos, counts, seqs, xg, inter, tiles, total;
  int max_groups, ksplit, kper;
};

dfx_status moe_plan(const dfx_moe_weights *w, int32_t B, int32_t F, MoePlan *mp) {
  if (!w) return fail(DFX_EINVAL, "weights is NULL");
  if ((F != 1 && F != 2) || B < 0 || B > 65535) return fail(DFX_EINVAL, "n_flows %d batch %d", F, B);
  const int H = w->hidden, E = w->num_experts, I = w->intermediate;
  if (H < 32 || H % 32 || H > 16384) return fail(DFX_EUNSUPPORTED, "hidden %d (a multiple of 32, at most 16384)", H);
  if (E < 1 || E > kMoeMaxExperts) return fail(DFX_EUNSUPPORTED, "num_experts %d (1 .. %d)", E, kMoeMaxExperts);
  if (I < 32 || I % 32) return fail(DFX_EUNSUPPORTED, "intermediate %d is not a positive multiple of 32", I);
  const int kcap = E < kMoeMaxK ? E : kMoeMaxK;
  if (w->top_k_primary < 1 || w->top_k_primary > kcap) return fail(DFX_EINVAL, "top_k_primary %d", w->top_k_primary);
  if (F == 2 && (w->top_k_aux < 1 || w->top_k_aux > kcap)) return fail(DFX_EINVAL, "top_k_aux %d", w->top_k_aux);
  if ((size_t)E * ((B + 31) / 32) > 16384) return fail(DFX_EUNSUPPORTED, "num_experts * ceil(batch / 32) above 16384");
  if (!(w->rms_eps >= 0.f)) return fail(DFX_EINVAL, "rms_eps");
  if (!w->norm_gain || !w->w_router || !w->w_gate_up || !w->w_down) return fail(DFX_EINVAL, "a weight pointer is NULL");
  if (!aligned16(w->norm_gain) || !aligned16(w->w_router) || !aligned16(w->w_gate_up) || !aligned16(w->w_down) ||
      !aligned16(w->couple_b) || !aligned16(w->couple_c))
    return fail(DFX_EINVAL, "misaligned weight pointer");
  auto a256 = [](size_t x) { return round_up(x, 256); };
  MoePlan p{};
  const int rpg = 64 / F;
  p.max_groups = B > 0 ? (B + rpg - 1) / rpg : 0;
  // down projection: about 256 work-groups over all experts
  const int nks = I / 32, tiles = (H + 127) / 128;
  int ks = kTargetGemmGroups / (tiles * E);
  const int max_ks = nks / kMinGemmSteps > 1 ? nks / kMinGemmSteps : 1;
  ks = std::max(1, std::min(std::min(ks, max_ks), 16));
  int per = (nks + ks - 1) / ks;
  if (ks > 1) per = (per + 3) / 4 * 4;
  p.kper = per;
  p.ksplit = (nks + per - 1) / per;
  const size_t rows64 = (size_t)p.max_groups * 64;
  p.h = a256((size_t)F * B * H * 2);
  p.logits = a256((size_t)F * B * E * 4);
  p.ids = p.wts = p.pos = a256((size_t)F * B * kMoeMaxK * 4);
  p.counts = a256((size_t)E * 4);
  p.seqs = a256((size_t)E * B * 4);
  p.xg = a256((size_t)E * rows64 * H * 2);
  p.inter = a256((size_t)E * rows64 * I * 2);
  p.tiles = a256((size_t)E * p.ksplit * rows64 * H * 4);
  p.total = p.h + p.logits + p.ids + p.wts + p.pos + p.counts + p.seqs + p.xg + p.inter + p.tiles;
  *mp = p;
  return DFX_OK;
}

}  // namespace

dfx_status dfx_dual_flow_moe_mlp_workspace_size(const dfx_moe_weights *w, int32_t batch, int32_t n_flows,
                                                size_t *bytes) {
  DFX_BEGIN
  MoePlan p;
  dfx_status st = moe_plan(w, batch, n_flows, &p);
  if (st) return st;
  if (!bytes) return fail(DFX_EINVAL, "bytes is NULL");
  *bytes = p.total;
  return DFX_OK;
  DFX_END
}

dfx_status dfx_dual_flow_moe_mlp_taps(const dfx_moe_weights *w, int32_t batch, int32_t n_flows,
                                      dfx_moe_taps *taps) {
  DFX_BEGIN
  MoePlan p;
  dfx_status st = moe_plan(w, batch, n_flows, &p);
  if (st) return st;
  if (!taps) return fail(DFX_EINVAL, "taps is NULL");
  taps->h = 0;
  taps->logits = p.h;
  taps->ids = taps->logits + p.logits;
  taps->weights = taps->ids + p.ids;
  taps->counts = taps->weights + p.wts + p.pos;
  taps->seqs = taps->counts + p.counts;
  taps->inter = taps->seqs + p.seqs + p.xg;
  taps->inter_stride = (size_t)p.max_groups * 64 * w->intermediate;
  return DFX_OK;
  DFX_END
}

dfx_status dfx_dual_flow_moe_mlp(const dfx_moe_weights *w, int32_t batch, int32_t n_flows, float *x,
                                 void *workspace, size_t workspace_bytes, void *stream) {
  DFX_BEGIN
  MoePlan p;
  dfx_status st = moe_plan(w, batch, n_flows, &p);
  if (st) return st;
  if (batch == 0) return DFX_OK;
  if (!x) return fail(DFX_EINVAL, "x is NULL");
  if (!aligned16(x)) return fail(DFX_EINVAL, "x not 16-byte aligned");
  if (!workspace || workspace_bytes < p.total)
    return fail(DFX_EWORKSPACE, "MoE block needs %zu workspace bytes, got %zu", p.total, workspace_bytes);
  hipStream_t s = (hipStream_t)stream;
  const int F = n_flows, B = batch, H = w->hidden, E = w->num_experts, I = w->intermediate;
  char *c = (char *)workspace;
  MoeArgs a{};
  a.F = F; a.B = B; a.H = H; a.E = E; a.k1 = w->top_k_primary; a.k2 = F == 2 ? w->top_k_aux : 0;
  a.max_groups = p.max_groups; a.ksplit = p.ksplit;
  a.h = (const uint16_t *)c;                     c += p.h;
  a.w_router = w->w_router;
  a.logits = (float *)c;                          c += p.logits;
  a.ids = (int32_t *)c;                           c += p.ids;
  a.wts = (float *)c;                             c += p.wts;
  a.pos = (int32_t *)c;                           c += p.pos;
  a.counts = (int32_t *)c;                        c += p.counts;
  a.seqs = (int32_t *)c;                          c += p.seqs;
  a.xg = (uint16_t *)c;                           c += p.xg;
  uint16_t *inter = (uint16_t *)c;                c += p.inter;
  float *tiles = (float *)c;
  a.tiles = tiles; a.couple_c = F == 2 ? w->couple_c : nullptr; a.x = x;
  a.gain = w->norm_gain; a.eps = w->rms_eps;
  dfx_status r = hip_status(launch_moe(kMoeRoute, a, s), "norm + route launch");
  if (r) return r;
  if ((r = hip_status(launch_moe(kMoeLists, a, s), "expert lists launch"))) return r;
  if ((r = hip_status(launch_moe(kMoeGather, a, s), "gather launch"))) return r;
  const size_t rows64 = (size_t)p.max_groups * 64;
  GemmArgs g{};
  g.n_flows = F; g.rows = B; g.x_packed = 1; g.w_packed = 1;
  g.expert_rows = a.counts; g.experts = E; g.max_groups = p.max_groups;
  // gate/up with SwiGLU and the b coupling, per expert
  g.K = H; g.N = 2 * I; g.x = a.xg; g.w = w->w_gate_up; g.y = inter;
  g.couple = F == 2 ? w->couple_b : nullptr; g.ksplit = 1; g.kper = H / 32; g.swiglu = 1;
  g.x_estride = (int64_t)rows64 * H; g.w_estride = (int64_t)2 * I * H; g.y_estride = (int64_t)rows64 * I;
  if ((r = hip_status(launch_grouped_linear(g, s), "expert gate/up launch"))) return r;
  // down projection tiles, per expert
  g.K = I; g.N = H; g.x = inter; g.w = w->w_down; g.y = nullptr; g.couple = nullptr; g.swiglu = 0;
  g.ksplit = p.ksplit; g.kper = p.kper; g.partial = tiles; g.tiles_only = 1;
  g.x_estride = (int64_t)rows64 * I; g.w_estride = (int64_t)H * I; g.y_estride = 0;
  g.p_estride = (int64_t)p.ksplit * rows64 * H;
  if ((r = hip_status(launch_grouped_linear(g, s), "expert down launch"))) return r;
  return hip_status(launch_moe(kMoeCombine, a, s), "combine launch");
  DFX_END
}

namespace {

// ---- prefill (primary only)

dfx_status check_prefill(const dfx_kv_cache *kv, int32_t B, int32_t T, int32_t max_context, int32_t hq) {
  dfx_status st = check_kv(kv, B < 0 ? 0 : B);
  if (st) return st;
  if (B < 0 || B > 65535 || T < 0) return fail(DFX_EINVAL, "batch %d chunk %d", B, T);
  if ((int64_t)B * T > (int64_t)1 << 22) return fail(DFX_EUNSUPPORTED, "batch * chunk above 2^22 rows");
  if (T > 65535 * 16) return fail(DFX_EUNSUPPORTED, "chunk %d above %d positions (16 per grid row)", T, 65535 * 16);
  if (kv->dtype != DFX_BF16) return fail(DFX_EUNSUPPORTED, "prefill needs a bf16 cache");
  if (kv->block_table && kv->block_size < 16)
    return fail(DFX_EUNSUPPORTED, "prefill needs paged blocks of >= 16 tokens (got %d)", kv->block_size);
  if (hq < 4 || hq % 4 || hq % kv->num_kv_heads)
    return fail(DFX_EUNSUPPORTED, "num_q_heads %d (a multiple of 4 and of num_kv_heads)", hq);
  if (max_context < 1 || max_context > capacity(kv))
    return fail(DFX_EINVAL, "max_context %d outside [1, capacity %lld]", max_context, (long long)capacity(kv));
  return DFX_OK;
}

AttnArgs prefill_attn_args(const dfx_kv_cache *kv, const int32_t *start, int32_t B, int32_t T, int32_t max_context,
                           int32_t hq, const float *q, int64_t q_stride, float *o, int o_packed, float *lse) {
  AttnArgs a{};
  a.k = kv->k; a.v = kv->v; a.table = kv->block_table; a.num_blocks = kv->num_blocks;
  a.max_blocks = kv->max_blocks_per_seq; a.block_size = kv->block_size;
  a.block_shift = kv->block_table ? (int)__builtin_ctz((unsigned)kv->block_size) : -1;
  a.num_kv_heads = kv->num_kv_heads; a.head_dim = kv->head_dim; a.group = hq / kv->num_kv_heads;
  a.num_q_heads = hq; a.n_flows = 1; a.batch = B; a.ctx = start; a.max_context = max_context;
  a.q1 = q; a.q_bstride = q_stride; a.kv_bf16 = 1;
  a.scale_log2 = kLog2e / sqrtf((float)kv->head_dim);
  a.o1 = o; a.o_packed = o_packed; a.o_bf16 = o_packed; a.lse = lse; a.num_splits = 1;
  a.prefill_T = T;
  return a;
}

struct PrefillPlan {
  size_t h1, qkv, o, h2, inter, total;
};

dfx_status prefill_plan(const dfx_layer_weights *w, const dfx_kv_cache *kv, int32_t B, int32_t T,
                        int32_t max_context, PrefillPlan *pp) {
  if (!w) return fail(DFX_EINVAL, "weights is NULL");
  dfx_status st = check_prefill(kv, B, T, max_context, w->num_q_heads);
  if (st) return st;
  if (w->head_dim != kv->head_dim || w->num_kv_heads != kv->num_kv_heads)
    return fail(DFX_EINVAL, "weights and cache disagree on head_dim / num_kv_heads");
  if (w->hidden < 32 || w->hidden % 32 || w->hidden > 16384) return fail(DFX_EUNSUPPORTED, "hidden %d", w->hidden);
  if (w->intermediate < 32 || w->intermediate % 32) return fail(DFX_EUNSUPPORTED, "intermediate %d", w->intermediate);
  if (!(w->rms_eps >= 0.f)) return fail(DFX_EINVAL, "rms_eps");
  if (!w->attn_norm_gain || !w->w_qkv || !w->w_o || !w->mlp_norm_gain || !w->w_gate_up || !w->w_down)
    return fail(DFX_EINVAL, "a weight pointer is NULL");
  const int H = w->hidden, D = w->head_dim, Hq = w->num_q_heads, I = w->intermediate;
  const size_t rows = (size_t)B * T, prow = (rows + 63) / 64 * 64;
  auto a256 = [](size_t x) { return round_up(x, 256); };
  PrefillPlan p{};
  p.h1 = a256(prow * H * 2);
  p.qkv = a256(rows * (Hq + 2 * w->num_kv_heads) * D * 4);
  p.o = a256(prow * Hq * D * 2);
  p.h2 = a256(prow * H * 2);
  p.inter = a256(prow * I * 2);
  p.total = p.h1 + p.qkv + p.o + p.h2 + p.inter;
  *pp = p;
  return DFX_OK;
}

// One projection of the prefill rows (one flow): the LDS-staged dense kernel when there is more
// than one row group (K a multiple of 32), else the grouped linear with every 64-row group
// its own work-group slice. fp32 out (optionally plus residual, in place), or SwiGLU bf16 rows.
dfx_status prefill_linear(int32_t rows, int32_t K, int32_t N, const uint16_t *x_packed, const uint16_t *w,
                          void *y, const float *residual, int swiglu, hipStream_t s) {
  if (rows > 64 && prefill_gemm_fits(K, N, swiglu)) {
    PrefillGemmArgs a{rows, K, N, x_packed, w, y, residual};
    return hip_status(launch_prefill_gemm(a, swiglu, s), "prefill projection launch");
  }
  GemmArgs g{};
  g.n_flows = 1; g.rows = rows; g.K = K; g.N = N; g.x_packed = 1; g.x = x_packed; g.w = w; g.w_packed = 1;
  g.y = y; g.residual = residual; g.ksplit = 1; g.kper = K / 32; g.swiglu = swiglu;
  g.group_split = (rows + 63) / 64;
  return hip_status(launch_grouped_linear(g, s), "prefill projection launch");
}

dfx_status run_prefill_layer(const dfx_layer_weights *w, const dfx_kv_cache *kv, const int32_t *start, int B, int T,
                             int max_context, float *x, const PrefillPlan &p, char *base, hipStream_t s,
                             bool norm_in) {
  const int H = w->hidden, D = w->head_dim, Hq = w->num_q_heads;
  const int Nqkv = (Hq + 2 * w->num_kv_heads) * D, I = w->intermediate, rows = B * T;
  uint16_t *h1 = (uint16_t *)base;
  float *qkv = (float *)(base + p.h1);
  uint16_t *ob = (uint16_t *)((char *)qkv + p.qkv);
  uint16_t *h2 = (uint16_t *)((char *)ob + p.o);
  uint16_t *inter = (uint16_t *)((char *)h2 + p.h2);
  dfx_status r;
  if (norm_in && (r = hip_status(launch_rmsnorm_rows(rows, H, x, w->attn_norm_gain, w->rms_eps, h1, s), "rmsnorm launch")))
    return r;
  if ((r = prefill_linear(rows, H, Nqkv, h1, w->w_qkv, qkv, nullptr, 0, s))) return r;
  PrefillGlueArgs ga{B, T, Nqkv, Hq, D, qkv, *kv, start};
  if ((r = hip_status(launch_prefill_append(ga, s), "prefill append launch"))) return r;
  AttnArgs a = prefill_attn_args(kv, start, B, T, max_context, Hq, qkv, Nqkv, (float *)ob, 1, nullptr);
  if ((r = hip_status(launch_prefill_attn(a, s), "prefill attention launch"))) return r;
  if ((r = prefill_linear(rows, Hq * D, H, ob, w->w_o, x, x, 0, s))) return r;
  if ((r = hip_status(launch_rmsnorm_rows(rows, H, x, w->mlp_norm_gain, w->rms_eps, h2, s), "rmsnorm launch")))
    return r;
  if ((r = prefill_linear(rows, H, 2 * I, h2, w->w_gate_up, inter, nullptr, 1, s))) return r;
  return prefill_linear(rows, I, H, inter, w->w_down, x, x, 0, s);
}

}  // namespace

dfx_status dfx_prefill_attn(const dfx_kv_cache *kv, const int32_t *start_pos, int32_t batch, int32_t chunk,
                            int32_t max_context, int32_t num_q_heads, const float *q, int64_t q_row_stride,
                            float *o, float *lse, void *stream) {
  DFX_BEGIN
  dfx_status st = check_prefill(kv, batch, chunk, max_context, num_q_heads);
  if (st) return st;
  const int64_t row = (int64_t)num_q_heads * kv->head_dim;
  if (q_row_stride == 0) q_row_stride = row;
  if (q_row_stride < row || q_row_stride % 4) return fail(DFX_EINVAL, "q_row_stride %lld", (long long)q_row_stride);
  if (batch == 0 || chunk == 0) return DFX_OK;
  if (!start_pos || !q || !o) return fail(DFX_EINVAL, "start_pos / q / o is NULL");
  if (!aligned16(q) || !aligned16(o) || ((uintptr_t)lse & 3)) return fail(DFX_EINVAL, "misaligned pointer");
  AttnArgs a = prefill_attn_args(kv, start_pos, batch, chunk, max_context, num_q_heads, q, q_row_stride, o, 0, lse);
  return hip_status(launch_prefill_attn(a, (hipStream_t)stream), "prefill attention launch");
  DFX_END
}

dfx_status dfx_prefill_dual_attn(const dfx_kv_cache *kv, const int32_t *start_pos, int32_t batch, int32_t chunk,
                                 int32_t max_context, int32_t num_q_heads, const float *q1, const float *q2_raw,
                                 const float *a, int32_t a_head_stride, int64_t q_row_stride, float *o1, float *o2,
                                 float *lse, void *stream) {
  DFX_BEGIN
  dfx_status st = check_prefill(kv, batch, chunk, max_context, num_q_heads);
  if (st) return st;
  const int64_t row = (int64_t)num_q_heads * kv->head_dim;
  if (q_row_stride == 0) q_row_stride = row;
  if (q_row_stride < row || q_row_stride % 4) return fail(DFX_EINVAL, "q_row_stride %lld", (long long)q_row_stride);
  if (a_head_stride != 0 && a_head_stride != kv->head_dim)
    return fail(DFX_EINVAL, "a_head_stride %d (0 or head_dim)", a_head_stride);
  if (batch == 0 || chunk == 0) return DFX_OK;
  if (!start_pos || !q1 || !q2_raw || !o1 || !o2) return fail(DFX_EINVAL, "start_pos / q1 / q2_raw / o1 / o2 is NULL");
  if (!aligned16(q1) || !aligned16(q2_raw) || !aligned16(o1) || !aligned16(o2) || ((uintptr_t)lse & 3) ||
      ((uintptr_t)a & 3))
    return fail(DFX_EINVAL, "misaligned pointer");
  AttnArgs at = prefill_attn_args(kv, start_pos, batch, chunk, max_context, num_q_heads, q1, q_row_stride, o1, 0, lse);
  at.n_flows = 2;
  at.q2 = q2_raw;
  at.a = a;
  at.a_hstride = a_head_stride;
  at.o2 = o2;
  return hip_status(launch_prefill_attn(at, (hipStream_t)stream), "prefill dual attention launch");
  DFX_END
}

dfx_status dfx_prefill_layer_workspace_size(const dfx_layer_weights *w, const dfx_kv_cache *kv, int32_t batch,
                                            int32_t chunk, int32_t max_context, size_t *bytes) {
  DFX_BEGIN
  PrefillPlan p;
  dfx_status st = prefill_plan(w, kv, batch, chunk, max_context, &p);
  if (st) return st;
  if (!bytes) return fail(DFX_EINVAL, "bytes is NULL");
  *bytes = p.total;
  return DFX_OK;
  DFX_END
}

dfx_status dfx_prefill_layer_taps(const dfx_layer_weights *w, const dfx_kv_cache *kv, int32_t batch,
                                  int32_t chunk, int32_t max_context, dfx_layer_taps *taps) {
  DFX_BEGIN
  PrefillPlan p;
  dfx_status st = prefill_plan(w, kv, batch, chunk, max_context, &p);
  if (st) return st;
  if (!taps) return fail(DFX_EINVAL, "taps is NULL");
  taps->h1 = 0;
  taps->q = p.h1;
  taps->o = taps->q + p.qkv;
  taps->h2 = taps->o + p.o;
  taps->inter = taps->h2 + p.h2;
  return DFX_OK;
  DFX_END
}

dfx_status dfx_prefill_layer(const dfx_layer_weights *w, const dfx_kv_cache *kv, const int32_t *start_pos,
                             int32_t batch, int32_t chunk, int32_t max_context, float *x, void *workspace,
                             size_t workspace_bytes, void *stream) {
  DFX_BEGIN
  PrefillPlan p;
  dfx_status st = prefill_plan(w, kv, batch, chunk, max_context, &p);
  if (st) return st;
  if (batch == 0 || chunk == 0) return DFX_OK;
  if (!start_pos || !x) return fail(DFX_EINVAL, "start_pos / x is NULL");
  if (!aligned16(x)) return fail(DFX_EINVAL, "x not 16-byte aligned");
  if (!workspace || workspace_bytes < p.total)
    return fail(DFX_EWORKSPACE, "prefill layer needs %zu workspace bytes, got %zu", p.total, workspace_bytes);
  return run_prefill_layer(w, kv, start_pos, batch, chunk, max_context, x, p, (char *)workspace,
                           (hipStream_t)stream, true);
  DFX_END
}

dfx_status dfx_prefill_step_workspace_size(const dfx_layer_weights *layers, const dfx_kv_cache *caches,
                                           int32_t n_layers, int32_t batch, int32_t chunk, int32_t max_context,
                                           size_t *bytes) {
  DFX_BEGIN
  if (n_layers < 1 || !layers || !caches) return fail(DFX_EINVAL, "n_layers %d / layers / caches", n_layers);
  if (!bytes) return fail(DFX_EINVAL, "bytes is NULL");
  size_t m = 0;
  for (int l = 0; l < n_layers; ++l) {
    PrefillPlan p;
    dfx_status st = prefill_plan(&layers[l], &caches[l], batch, chunk, max_context, &p);
    if (st) return st;
    if (layers[l].hidden != layers[0].hidden) return fail(DFX_EINVAL, "layer %d hidden differs", l);
    m = std::max(m, p.total);
  }
  *bytes = m;
  return DFX_OK;
  DFX_END
}

dfx_status dfx_prefill_step(const dfx_layer_weights *layers, const dfx_kv_cache *caches, int32_t n_layers,
                            const int32_t *tokens, int32_t vocab, const uint16_t *embed_primary,
                            const int32_t *start_pos, int32_t batch, int32_t chunk, int32_t max_context, float *x,
                            void *workspace, size_t workspace_bytes, void *stream) {
  DFX_BEGIN
  size_t need = 0;
  dfx_status st = dfx_prefill_step_workspace_size(layers, caches, n_layers, batch, chunk, max_context, &need);
  if (st) return st;
  if (vocab < 1 || !embed_primary) return fail(DFX_EINVAL, "vocab %d / embed_primary", vocab);
  if ((uintptr_t)embed_primary & 7) return fail(DFX_EINVAL, "embed_primary must be 8-byte aligned");
  if (batch == 0 || chunk == 0) return DFX_OK;
  if (!tokens || !start_pos || !x) return fail(DFX_EINVAL, "tokens / start_pos / x is NULL");
  if (!aligned16(x)) return fail(DFX_EINVAL, "x not 16-byte aligned");
  if (!workspace || workspace_bytes < need)
    return fail(DFX_EWORKSPACE, "prefill step needs %zu workspace bytes, got %zu", need, workspace_bytes);
  hipStream_t s = (hipStream_t)stream;
  const dfx_layer_weights &w0 = layers[0];
  // the primary's embedding rows and layer 0's normed rows, in one kernel
  dfx_status r = hip_status(launch_embed_norm(1, batch * chunk, w0.hidden, tokens, vocab, embed_primary, nullptr,
                                              w0.attn_norm_gain, w0.rms_eps, x, (uint16_t *)workspace, s),
                            "embedding launch");
  if (r) return r;
  for (int l = 0; l < n_layers; ++l) {
    PrefillPlan p;
    prefill_plan(&layers[l], &caches[l], batch, chunk, max_context, &p);
    if ((r = run_prefill_layer(&layers[l], &caches[l], start_pos, batch, chunk, max_context, x, p, (char *)workspace,
                               s, l > 0)))
      return r;
  }
  return DFX_OK;
  DFX_END
}

dfx_status dfx_copy_bytes(void *dst, const void *src, size_t bytes, void *stream) {
  DFX_BEGIN
  if (bytes % 16 || !aligned16(dst) || !aligned16(src) || (bytes && (!dst || !src)))
    return fail(DFX_EINVAL, "copy needs 16-byte aligned pointers and a multiple of 16 bytes");
  return hip_status(launch_copy(dst, src, bytes, (hipStream_t)stream), "copy launch");
  DFX_END
}

dfx_status dfx_read_bytes(const void *src, size_t bytes, uint32_t *sink, void *stream) {
  DFX_BEGIN
  if (bytes % 16 || !aligned16(src) || (bytes && (!src || !sink)))
    return fail(DFX_EINVAL, "read needs a 16-byte aligned source, a multiple of 16 bytes and a sink");
  return hip_status(launch_read(src, bytes, sink, (hipStream_t)stream), "read launch");
  DFX_END
}

dfx_status dfx_fill_bytes(void *dst, size_t bytes, uint32_t pattern, void *stream) {
  DFX_BEGIN
  if (bytes % 16 || !aligned16(dst) || (bytes && !dst))
    return fail(DFX_EINVAL, "fill needs a 16-byte aligned pointer and a multiple of 16 bytes");
  return hip_status(launch_fill(dst, bytes, pattern, (hipStream_t)stream), "fill launch");
  DFX_END
}

}  // extern "C"

// ---- allocation-free decode attention -------------------------------------------------

namespace {

// Scratch of dfx_decode_attn_noalloc: the split partials live in this file-scope device array
// (each device holds its own copy, from module load to process end). Host code never uses the
// array's name as an address: its device address is looked up once per device.
constexpr size_t kNoallocScratch = (size_t)DFX_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratch];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (hipGetSymbolAddress once per device,
// with that device current).
dfx_status scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DFX_EUNSUPPORTED, "device %d (at most %d devices)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(DFX_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DFX_OK;
}

}  // namespace

extern "C" dfx_status dfx_decode_attn_noalloc(const dfx_kv_cache *kv, const int32_t *context_lens, int32_t batch,
                                              int32_t max_context, int32_t num_q_heads, int32_t q_dtype,
                                              const void *q1, const void *q2_raw, int64_t q_batch_stride,
                                              const float *a, int32_t a_head_stride, float softmax_scale,
                                              float *o1, float *o2, float *lse, int32_t num_splits,
                                              void *stream) {
  DFX_BEGIN
  AttnCall c{kv, context_lens, batch, max_context, num_q_heads, q_dtype, q1, q2_raw, q_batch_stride,
             a, a_head_stride, softmax_scale, o1, o2, lse, num_splits, nullptr, 0, 0};
  dfx_status st = validate_attn(c);
  if (st) return st;
  // the plan's scratch, checked against the array before any HIP call
  const int F = q2_raw ? 2 : 1, G = num_q_heads / kv->num_kv_heads;
  int splits, chunk;
  attn_plan(batch, kv->num_kv_heads, max_context, num_splits, paged_bs(kv), attn_mfma_path(kv, F, G), &splits,
            &chunk);
  const size_t need = attn_ws_bytes(splits, F, batch, num_q_heads, kv->head_dim);
  if (need > kNoallocScratch)
    return fail(DFX_EWORKSPACE, "decode_attn_noalloc needs %zu bytes of scratch for %d splits; the library's "
                "array holds %zu (DFX_NOALLOC_SCRATCH_BYTES)", need, splits, kNoallocScratch);
  if (batch == 0) return DFX_OK;
  if (need > 0) {
    if ((st = scratch_address(&c.ws))) return st;
    c.ws_bytes = kNoallocScratch;
  }
  return run_attn(c, (hipStream_t)stream);
  DFX_END
}
