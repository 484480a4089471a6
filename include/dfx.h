/*
 * dfx.h -- C ABI of the dual-flow decode library (libdfx.so), MI355X / gfx950.
 *
 * The Dual-Flow Transformer runs two residual rows per generated position: a
 * primary flow, which is a complete causal Transformer and the only writer of
 * the persistent K/V cache, and an auxiliary flow, which reads the primary's
 * cache and never writes it (Sintesi Tecnica: Dual-Flow Transformers,
 * section "Architettura Core"). The auxiliary query Q2 is coupled to the
 * primary query Q1 through a learned vector a and attends to the primary keys
 * and values, so one pass over the cache and one pass over the shared weights
 * serve both flows (same page, section "Meccanismi Chiave"; the cost claim --
 * no larger cache, no extra unique weights read in decode -- is in section
 * "Costi di Inferenza vs. Addestramento").
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates no device memory, keeps no per-call state and never
 *    synchronizes. Every call is asynchronous on `stream` (a hipStream_t;
 *    NULL = the null stream). Calls on one stream run in issue order.
 *  - Flow 0 is the primary flow, flow 1 the auxiliary flow. Arrays with a
 *    flow axis put it first: [n_flows][rows][...], flows back to back.
 *  - bf16 values are stored as uint16 bit patterns; every bf16 rounding in
 *    the library is round-to-nearest-even. Accumulation is fp32.
 *  - Arguments are validated on the host before any HIP call. On failure a
 *    call returns a non-zero dfx_status, launches nothing and leaves a message
 *    for dfx_last_error(). A failed launch returns DFX_EHIP. No C++ exception
 *    crosses this interface.
 *  - Device-resident indices (context lengths, positions, block-table
 *    entries) are clamped inside the kernels to the sizes given here, so a
 *    bad value yields wrong numbers, never an out-of-bounds access.
 */
#ifndef DFX_H
#define DFX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFX_VERSION 100

typedef enum {
  DFX_OK = 0,
  DFX_EINVAL = 1,       /* a null pointer, bad size, bad stride or misaligned pointer */
  DFX_EUNSUPPORTED = 2, /* a valid request outside what the kernels implement */
  DFX_EWORKSPACE = 3,   /* workspace missing or smaller than the *_workspace_size result */
  DFX_EHIP = 4          /* a HIP call or kernel launch failed */
} dfx_status;

typedef enum { DFX_F32 = 0, DFX_BF16 = 1 } dfx_dtype;

/* Layout of a bf16 weight matrix W with N output and K input features.
 *  DFX_W_ROW_MAJOR: W[n][k] at n*K + k.
 *  DFX_W_PACKED:    matrix-core fragment order (see dfx_pack_weight): each 16-row x
 *                   32-column block is 1 KiB contiguous and the blocks of one
 *                   32-column slice of all rows are adjacent, so the grouped linear's
 *                   work-groups read neighbouring KiB runs at full HBM burst length. */
typedef enum { DFX_W_ROW_MAJOR = 0, DFX_W_PACKED = 1 } dfx_weight_layout;

/*
 * The single persistent K/V cache of the primary flow (same page, section
 * "Architettura Core": only the primary writes it, the auxiliary flow reads it).
 *
 * Layout of k and v: [num_blocks][num_kv_heads][block_size][head_dim], elements
 * of `dtype`, each pointer 16-byte aligned.
 *  - Paged (block_table != NULL): position p of sequence b, KV head g is
 *    element row [block_table[b*max_blocks_per_seq + p/block_size]][g][p % block_size].
 *    block_size must be a power of two; block_table is device int32
 *    [batch][max_blocks_per_seq].
 *  - Contiguous (block_table == NULL): sequence b owns block b, block_size is
 *    the per-sequence capacity (any value >= 1) and num_blocks >= batch.
 */
typedef struct dfx_kv_cache {
  int32_t dtype;              /* dfx_dtype of the pool: DFX_BF16 or DFX_F32 */
  int32_t num_kv_heads;       /* >= 1 */
  int32_t head_dim;           /* 64 or 128 */
  int32_t block_size;         /* tokens per block (paged) or capacity (contiguous) */
  int64_t num_blocks;         /* blocks in the pool (block ids are clamped to it) */
  void *k;                    /* device [num_blocks][num_kv_heads][block_size][head_dim] */
  void *v;                    /* same layout as k */
  const int32_t *block_table; /* device [batch][max_blocks_per_seq], or NULL (contiguous) */
  int32_t max_blocks_per_seq; /* row length of block_table (ignored when contiguous) */
  int32_t reserved;           /* must be 0 */
} dfx_kv_cache;

/* Library version (the DFX_VERSION it was compiled with). */
int dfx_version(void);

/* Message of the last failing call on this thread ("" if none). The pointer is
 * valid until the next dfx_* call on the same thread. */
const char *dfx_last_error(void);

/*
 * Split plan of dfx_decode_attn. Attention over one sequence's context is cut into
 * context splits whose partial softmax states are merged by a log-sum-exp combine; the
 * auxiliary flow reads the same cache positions as the primary (Sintesi Tecnica:
 * Dual-Flow Transformers, section "Meccanismi Chiave"), so both flows share every split.
 * Reports the number of context splits dfx_decode_attn will use for these arguments
 * (num_splits = 0 asks for the automatic plan) and the workspace it needs in bytes (0
 * when the plan has a single split). Pure host arithmetic; splits_out and
 * workspace_bytes may each be NULL. Errors: DFX_EINVAL for an invalid cache descriptor,
 * batch < 0, num_q_heads < 1, n_flows not 1 or 2, max_context outside [0, capacity] or
 * num_splits < 0.
 */
dfx_status dfx_decode_attn_plan(const dfx_kv_cache *kv, int32_t batch, int32_t num_q_heads,
                                int32_t n_flows, int32_t max_context, int32_t num_splits,
                                int32_t *splits_out, size_t *workspace_bytes);

/*
 * Workspace bytes dfx_decode_attn needs for these arguments: the fp32 partial outputs
 * and log-sum-exp values of every context split ([splits][n_flows][batch][num_q_heads]
 * x (head_dim + 1) floats, 256-byte aligned regions), 0 when the plan has one split.
 * The same plan as dfx_decode_attn_plan (same page and section). *bytes receives the
 * size; bytes == NULL is DFX_EINVAL, and so is every argument dfx_decode_attn_plan
 * rejects. Pure host arithmetic.
 */
dfx_status dfx_decode_attn_workspace_size(int32_t batch, int32_t num_q_heads, int32_t n_flows,
                                          const dfx_kv_cache *kv, int32_t max_context,
                                          int32_t num_splits, size_t *bytes);

/*
 * Dual-query decode attention over the primary cache (same page, section
 * "Meccanismi Chiave": the auxiliary query Q2 is coupled to Q1 through the
 * learned vector a and attends to the primary K1, V1; the cache is read once
 * and serves both flows).
 *
 * For each sequence b < batch, query head h (KV head g = h / (num_q_heads /
 * num_kv_heads)) and flow f:
 *   Q1 = q1[b][h]                       Q2 = q2_raw[b][h] + a_h * Q1 (elementwise)
 *   s_p = scale * <Q_f, K[b][g][p]>     for 0 <= p < n_b = min(context_lens[b], max_context)
 *   o_f[b][h] = sum_p softmax(s)_p V[b][g][p],   lse[f][b][h] = log sum_p exp(s_p)
 * a_h = a[h * a_head_stride + d] (a_head_stride 0: one vector of head_dim for
 * all heads; head_dim: one vector per head). a == NULL means Q2 = q2_raw.
 * n_b = 0 gives o = 0 and lse = -inf. Positions >= n_b are never read as data.
 *
 *  q1, q2_raw   device [batch][num_q_heads][head_dim] of q_dtype, rows of
 *               consecutive sequences q_batch_stride elements apart (0 =
 *               num_q_heads*head_dim; must be a multiple of 8); 16-byte aligned.
 *               q2_raw == NULL runs the primary flow only (n_flows = 1).
 *  a            device fp32, NULL, or [head_dim] / [num_q_heads][head_dim].
 *  softmax_scale  <= 0 selects 1/sqrt(head_dim).
 *  o1, o2       device fp32 [batch][num_q_heads][head_dim]; o2 NULL iff q2_raw NULL.
 *  lse          device fp32 [n_flows][batch][num_q_heads] (natural log) or NULL.
 *  max_context  host upper bound of context_lens (used for split planning and
 *               clamping; <= the cache capacity).
 *  num_splits   0 = automatic; otherwise the requested number of context splits,
 *               merged in a fixed order by a log-sum-exp combine (deterministic). With
 *               a paged cache one split spans at most 1023 blocks, so the plan may use
 *               more splits than requested; dfx_decode_attn_plan reports the count.
 *  workspace    device scratch of >= the dfx_decode_attn_plan size (may be NULL
 *               when that size is 0); owned by the caller, not kept after the call.
 *  Limits: batch and the plan's split count at most 65535 each (DFX_EUNSUPPORTED).
 * The pool is only read. Results for one (b, h, f) do not depend on the other
 * flow, heads or sequences: o1 is bit-identical with and without q2_raw.
 */
dfx_status dfx_decode_attn(const dfx_kv_cache *kv, const int32_t *context_lens, int32_t batch,
                           int32_t max_context, int32_t num_q_heads, int32_t q_dtype,
                           const void *q1, const void *q2_raw, int64_t q_batch_stride,
                           const float *a, int32_t a_head_stride, float softmax_scale,
                           float *o1, float *o2, float *lse, int32_t num_splits,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * dfx_decode_attn without a workspace argument, for callers that cannot allocate device
 * memory around the call: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. Same arguments (minus workspace / workspace_bytes), same plan, same
 * kernels and the same results bit for bit. The split partials go to a file-scope device
 * array of DFX_NOALLOC_SCRATCH_BYTES inside the library (one per device, held from the
 * library's load until the process ends); the call itself allocates nothing. The first
 * call on a device looks the array's address up (hipGetSymbolAddress) with that device
 * current. Nothing in the array needs initial contents: every split the merge reads is
 * written by the same call. All calls on one device share that device's array, so calls
 * that overlap in time on one device (different streams, or host threads) race on it:
 * serialize them. Errors: as dfx_decode_attn, plus DFX_EWORKSPACE (before any HIP call)
 * when the plan's partials exceed DFX_NOALLOC_SCRATCH_BYTES (dfx_decode_attn_workspace_size
 * gives that size), DFX_EUNSUPPORTED for a device index above 63, DFX_EHIP if the address
 * lookup fails.
 */
#define DFX_NOALLOC_SCRATCH_BYTES (16u << 20)

dfx_status dfx_decode_attn_noalloc(const dfx_kv_cache *kv, const int32_t *context_lens, int32_t batch,
                                   int32_t max_context, int32_t num_q_heads, int32_t q_dtype,
                                   const void *q1, const void *q2_raw, int64_t q_batch_stride,
                                   const float *a, int32_t a_head_stride, float softmax_scale,
                                   float *o1, float *o2, float *lse, int32_t num_splits, void *stream);

/*
 * Append the primary flow's new key and value rows to the cache (same page,
 * section "Architettura Core": the primary flow writes the persistent cache,
 * the auxiliary flow never does -- this call has no flow argument, so no
 * auxiliary row can reach the cache).
 *
 * For each b < batch: row positions[b] of sequence b, every KV head g, gets
 * k_new[b*src_row_stride + g*head_dim + d] (and v likewise), converted to the
 * pool dtype (fp32 -> bf16 round to nearest even). positions is device int32
 * [batch], each clamped to [0, capacity). src_dtype is the element type of
 * k_new / v_new; src_row_stride (elements, 0 = num_kv_heads*head_dim) lets the
 * rows come straight from a fused QKV projection output. Re-running the call
 * rewrites the same bytes (idempotent).
 */
dfx_status dfx_kv_append_primary(const dfx_kv_cache *kv, int32_t batch, const int32_t *positions,
                                 int32_t src_dtype, const void *k_new, const void *v_new,
                                 int64_t src_row_stride, void *stream);

/*
 * Grouped shared-weight linear: one pass over W for the rows of every flow
 * (same page, section "Architettura Core": both flows share the attention,
 * MLP and output matrices; section "Costi di Inferenza vs. Addestramento":
 * the flows are grouped so decode reads no extra unique weights).
 *
 *   Y[f][r][n] = sum_k bf16(X[f][r][k]) * W[n][k]          (fp32 accumulate)
 *   if couple && n_flows == 2:  Y[1][r][n] += couple[n] * Y[0][r][n]
 *   if residual:                Y[f][r][n] += residual[f][r][n]
 *   y = Y (fp32) or bf16(Y)
 *
 *  x        device [n_flows][rows][in_features], x_dtype (fp32 rows are rounded
 *           to bf16 on load), 16-byte aligned, in_features a multiple of 32.
 *  w        device bf16 weights of out_features x in_features (out_features a multiple
 *           of 16) in w_layout (DFX_W_PACKED streams at full bandwidth).
 *  y        device [n_flows][rows][out_features] of y_dtype; may alias residual
 *           (in-place residual update), must not overlap x or w.
 *  couple   device fp32 [out_features] or NULL; residual device fp32 or NULL.
 *  workspace  device scratch of >= dfx_grouped_linear_workspace_size bytes (may be
 *           NULL when that is 0): the fp32 partial tiles of the K splits, fully
 *           written by each call before they are read (no initial contents needed).
 *           Calls sharing one workspace must not overlap in time.
 * The K-reduction order of every output element is fixed by (in_features,
 * out_features) alone: flow-0 outputs are bit-identical for n_flows 1 and 2
 * and for any row count.
 */
dfx_status dfx_grouped_linear_workspace_size(int32_t n_flows, int32_t rows, int32_t in_features,
                                             int32_t out_features, size_t *bytes);

dfx_status dfx_grouped_linear(int32_t n_flows, int32_t rows, int32_t in_features,
                              int32_t out_features, int32_t x_dtype, const void *x,
                              const uint16_t *w, int32_t w_layout, int32_t y_dtype, void *y,
                              const float *couple, const float *residual, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * Reorder a row-major bf16 weight matrix into DFX_W_PACKED (a pure permutation, done once
 * per static weight): packed[((s * N/16 + t) * 64 + l) * 8 + v] = w[16 t + l % 16][32 s +
 * 8 (l / 16) + v] for t < N/16, s < K/32, l < 64, v < 8. N must be a multiple of 16 and K
 * of 32; w and packed are device buffers of N*K elements that must not overlap.
 */
dfx_status dfx_pack_weight(int32_t out_features, int32_t in_features, const uint16_t *w,
                           uint16_t *packed, void *stream);

/*
 * RMSNorm with one gain vector shared by all rows (the flows add no
 * parameters besides embeddings and coupling vectors: same page, section
 * "Costi di Inferenza vs. Addestramento"):
 *   y[r][i] = bf16( x[r][i] / sqrt(mean_j x[r][j]^2 + eps) * gain[i] )
 *  x device fp32 [rows][dim], gain device fp32 [dim], y device bf16 [rows][dim];
 *  dim a multiple of 4, at most 16384.
 */
dfx_status dfx_rmsnorm(int32_t rows, int32_t dim, const float *x, const float *gain, float eps,
                       uint16_t *y, void *stream);

/*
 * SwiGLU activation with the MLP-intermediate coupling b (same page, section
 * "Meccanismi Chiave": one-way primary -> auxiliary vectors at the
 * MLP-intermediate level; the formula is this library's reading):
 *   inter[f][r][i] = silu(gu[f][r][i]) * gu[f][r][dim + i]     (r < rows, rows per flow)
 *   if b && n_flows == 2:  inter[1][r][i] += b[i] * inter[0][r][i]
 *   out = bf16(inter)
 *  gate_up device fp32 [n_flows][rows][2*dim] ([gate | up] per row),
 *  b device fp32 [dim] or NULL, out device bf16 [n_flows][rows][dim]; dim % 4 == 0.
 */
dfx_status dfx_swiglu_couple(int32_t rows, int32_t n_flows, int32_t dim, const float *gate_up,
                             const float *b, uint16_t *out, void *stream);

/*
 * Weights of one dual-flow decoder layer. Every matrix is shared by the two
 * flows; a, b, c are the coupling vectors at the query, MLP-intermediate and
 * MLP-output levels (same page, sections "Architettura Core" and "Meccanismi
 * Chiave"). NULL coupling vectors give the minimal two-flow form (separate
 * rows, shared cache, no coupling; section "Risultati" reports this variant).
 * All pointers are device pointers; the four matrices are bf16 [out][in] in
 * DFX_W_PACKED layout (dfx_pack_weight).
 */
typedef struct dfx_layer_weights {
  int32_t hidden;             /* model width; a multiple of 32, at most 16384 */
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;           /* 64 or 128; num_q_heads * head_dim may differ from hidden */
  int32_t intermediate;       /* MLP width; a multiple of 32 */
  float rms_eps;
  const float *attn_norm_gain;     /* [hidden] */
  const uint16_t *w_qkv;           /* packed [(num_q_heads + 2*num_kv_heads)*head_dim][hidden]: Q, K, V rows */
  const uint16_t *w_o;             /* packed [hidden][num_q_heads*head_dim] */
  const float *mlp_norm_gain;      /* [hidden] */
  const uint16_t *w_gate_up;       /* packed [2*intermediate][hidden]: gate rows, then up rows */
  const uint16_t *w_down;          /* packed [hidden][intermediate] */
  const float *couple_a;           /* [head_dim] (one vector for all heads) or NULL */
  const float *couple_b;           /* [intermediate] or NULL */
  const float *couple_c;           /* [hidden] or NULL */
} dfx_layer_weights;

/* Byte offsets of a layer call's intermediates in its workspace (see below). */
typedef struct dfx_layer_taps {
  size_t h1, q, o, h2, inter;
} dfx_layer_taps;

/* Workspace bytes dfx_dual_flow_decode_layer needs for these sizes. */
dfx_status dfx_dual_flow_decode_layer_workspace_size(const dfx_layer_weights *w,
                                                     const dfx_kv_cache *kv, int32_t batch,
                                                     int32_t n_flows, int32_t max_context,
                                                     size_t *bytes);

/*
 * One decode step of one layer for both flows (n_flows = 2) or the primary
 * alone (n_flows = 1), in place on the fp32 residual rows x [n_flows][batch][hidden]:
 *   h1 = rmsnorm(x, attn_norm_gain)                               (bf16)
 *   qkv = h1 W_qkv^T                                              (one weight pass, both flows)
 *   append K, V columns of the flow-0 rows at position context_lens[b] - 1   (bf16)
 *   o  = dfx_decode_attn(Q1 = flow-0 Q columns, q2_raw = flow-1 Q columns, a)   (bf16)
 *   x += o W_o^T
 *   h2 = rmsnorm(x, mlp_norm_gain)                                (bf16)
 *   inter = swiglu_couple(h2 W_gate_up^T, b)                      (bf16)
 *   m  = inter W_down^T;  m[1] += c * m[0];  x += m
 * context_lens (device int32 [batch]) counts the positions attended in this
 * step, the new one included (>= 1). The flow-1 K, V columns are computed by
 * the shared projection and discarded. workspace: >= the size above, no initial
 * contents needed; after the call it holds the step's intermediates
 * (dfx_dual_flow_decode_layer_taps). Calls sharing a workspace must not overlap.
 * batch at most 65535 (DFX_EUNSUPPORTED), as for dfx_decode_attn.
 */
dfx_status dfx_dual_flow_decode_layer(const dfx_layer_weights *w, const dfx_kv_cache *kv,
                                      const int32_t *context_lens, int32_t batch,
                                      int32_t max_context, int32_t n_flows, float *x,
                                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step of a stack of dual-flow layers, from token ids to the residual rows
 * after the last layer (Sintesi Tecnica: Dual-Flow Transformers, "Architettura Core": at
 * every generated position the auxiliary flow runs beside the primary; the two flows use
 * separate token embeddings and share every layer's matrices; only the primary writes each
 * layer's cache):
 *   x[0][b] = embed_primary[tokens[b]],  x[1][b] = embed_aux[tokens[b]]   (bf16 rows, widened)
 *   for l < n_layers:  x = layer_l(x)   (exactly dfx_dual_flow_decode_layer with layers[l],
 *                                        caches[l], the same context_lens and max_context)
 *  layers, caches  host arrays of n_layers structs (device pointers inside); every layer has
 *                  the same hidden size; layer l appends to caches[l] only.
 *  tokens          device int32 [batch]: the token at the generated position (ids are
 *                  clamped to [0, vocab)).
 *  embed_primary, embed_aux  device bf16 [vocab][hidden], 8-byte aligned; embed_aux is the
 *                  auxiliary flow's own table (may be NULL when n_flows = 1).
 *  x               device fp32 [n_flows][batch][hidden], output.
 *  workspace       >= dfx_dual_flow_decode_step_workspace_size bytes, no initial contents.
 * Results equal n_layers dfx_dual_flow_decode_layer calls on the embedded rows bit for bit
 * (each layer's down projection finishes straight into the next layer's norm, with the same
 * arithmetic). The call allocates nothing and never synchronizes, so a caller may capture it
 * in a graph (max_context then fixes the attention plan for every replay).
 */
dfx_status dfx_dual_flow_decode_step_workspace_size(const dfx_layer_weights *layers,
                                                    const dfx_kv_cache *caches, int32_t n_layers,
                                                    int32_t batch, int32_t n_flows,
                                                    int32_t max_context, size_t *bytes);

dfx_status dfx_dual_flow_decode_step(const dfx_layer_weights *layers, const dfx_kv_cache *caches,
                                     int32_t n_layers, const int32_t *tokens, int32_t vocab,
                                     const uint16_t *embed_primary, const uint16_t *embed_aux,
                                     const int32_t *context_lens, int32_t batch, int32_t max_context,
                                     int32_t n_flows, float *x, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * Where a completed dfx_dual_flow_decode_layer call with the same sizes leaves its
 * intermediates in the workspace: byte offsets of
 *   h1     bf16 normed rows entering W_qkv            [hidden columns]
 *   q      fp32 rows [n_flows][batch][(Hq + 2 Hkv) * D]; columns < Hq * D hold the
 *          flows' queries (q2_raw for flow 1), the rest is unspecified
 *   o      bf16 attention rows entering W_o             [Hq * D columns]
 *   h2     bf16 normed rows entering W_gate_up          [hidden columns]
 *   inter  bf16 SwiGLU rows entering W_down            [intermediate columns]
 * The bf16 regions use the activation fragment order of the grouped linear: element
 * (flow f, sequence b, column k) of a K-column region sits at
 *   ((((g * K/32 + k/32) * 4 + q/16) * 64 + q%16 + 16 ((k%32)/8)) * 8 + k%8)
 * with R = 64 / n_flows, g = b / R, q = f R + b % R (64-row groups; rows past the batch
 * are unspecified). The appended K/V rows are in the cache. Host-only: no GPU work.
 */
dfx_status dfx_dual_flow_decode_layer_taps(const dfx_layer_weights *w, const dfx_kv_cache *kv,
                                           int32_t batch, int32_t n_flows, int32_t max_context,
                                           struct dfx_layer_taps *taps);

/*
 * The shared output head and the mixture of the two flows' predictions (Sintesi Tecnica:
 * Dual-Flow Transformers, "Architettura Core": both flows share the output matrix;
 * "Meccanismi Chiave", mixture objective: the prediction mixes the flows' distributions with
 * a weight alpha_t on the primary that follows the primary's collision probability and is
 * never below one half):
 *   h_f       = bf16(rmsnorm(x_f) * norm_gain)               (one gain for both flows)
 *   logits_f  = h_f W_out^T                                   (one pass over W_out, both rows)
 *   p_f       = softmax(logits_f)
 *   c         = sum_i p_0,i^2                                 (collision probability)
 *   alpha     = (1 + c) / 2          -- the pages give no formula; this is the reading taken:
 *                                       monotone in c, 1/2 only as c -> 0, 1 for a certain primary
 *   p_mix     = alpha p_0 + (1 - alpha) p_1                   (n_flows = 1: alpha = 1, p_mix = p_0)
 *   token     = argmax_i p_mix,i                              (uniform_noise NULL: greedy)
 *             = argmax_i log p_mix,i - log(-log u_i)          (u = uniform_noise: a Gumbel-max
 *                                                              draw from p_mix)
 * Ties go to the lowest index. Softmax, mixture and argmax run in fp32.
 *  x             device fp32 [n_flows][batch][hidden]: the residual rows after the last layer.
 *  norm_gain     device fp32 [hidden]. hidden: a multiple of 32, at most 16384.
 *  w_out         device bf16 [vocab][hidden] in DFX_W_PACKED layout; vocab a multiple of 16.
 *  uniform_noise device fp32 [batch][vocab] with values in (0, 1), or NULL (greedy). The
 *                library draws no random numbers.
 *  next_token    device int32 [batch], output.
 *  alpha         device fp32 [batch], output, or NULL.
 *  p_mix         device fp32 [batch][vocab], output, or NULL.
 *  workspace     >= dfx_dual_flow_output_head_workspace_size bytes, no initial contents; after
 *                the call it holds h at byte h_offset (the activation fragment order of
 *                dfx_dual_flow_decode_layer_taps, hidden columns) and the fp32 logits
 *                [n_flows][batch][vocab] at logits_offset (dfx_dual_flow_output_head_taps,
 *                host-only). Calls sharing a workspace must not overlap.
 * x, norm_gain, w_out, uniform_noise and p_mix are 16-byte aligned. The call allocates
 * nothing and never synchronizes.
 */
dfx_status dfx_dual_flow_output_head_workspace_size(int32_t n_flows, int32_t batch, int32_t hidden,
                                                    int32_t vocab, size_t *bytes);

dfx_status dfx_dual_flow_output_head_taps(int32_t n_flows, int32_t batch, int32_t hidden, int32_t vocab,
                                          size_t *h_offset, size_t *logits_offset);

dfx_status dfx_dual_flow_output_head(int32_t n_flows, int32_t batch, int32_t hidden, int32_t vocab,
                                     const float *x, const float *norm_gain, float eps,
                                     const uint16_t *w_out, const float *uniform_noise,
                                     int32_t *next_token, float *alpha, float *p_mix, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * Mixture-of-experts MLP block with router replay (Sintesi Tecnica: Dual-Flow Transformers,
 * "Meccanismi Chiave", router replay: the auxiliary flow uses the experts chosen by the
 * primary's router with mixture weights of its own; "Contributi Chiave" item 3: the two
 * flows' expert fan-outs are set independently). In place on the residual rows x:
 *   h_f      = bf16(rmsnorm(x_f) * norm_gain)
 *   l_f      = h_f W_router^T                     (fp32; one shared router for both flows)
 *   ranking  = experts by descending l_0, the lower id first on equal logits
 *   S_0      = first top_k_primary of the ranking; S_1 = first top_k_aux of the SAME ranking
 *   w_f,e    = softmax over S_f of l_f            (each flow its own weights)
 *   i_f,e    = silu(h_f Wg_e^T) * (h_f Wu_e^T);  i_1,e += b * i_0,e  (i_0,e = 0 if e not in S_0);
 *              rounded to bf16
 *   m_f      = sum over e in S_f, in ranking order, of w_f,e * (i_f,e Wd_e^T)
 *   m_1     += c * m_0;   x_f += m_f
 * (the readings where the pages give no formula: the shared router, the auxiliary's experts as
 * the head of the primary's ranking, the softmax over the selected experts, b on experts both
 * flows ran, c on the block output). Every expert used by at least one row is read once for
 * all rows of both flows that use it; an expert no row uses is not read.
 */
typedef struct dfx_moe_weights {
  int32_t hidden;          /* a multiple of 32, at most 16384 */
  int32_t num_experts;     /* 1 .. 256 */
  int32_t intermediate;    /* per expert; a multiple of 32 */
  int32_t top_k_primary;   /* 1 .. min(num_experts, 16) */
  int32_t top_k_aux;       /* 1 .. min(num_experts, 16); ignored when n_flows = 1 */
  float rms_eps;
  const float *norm_gain;      /* [hidden] */
  const uint16_t *w_router;    /* bf16 [num_experts][hidden], row-major */
  const uint16_t *w_gate_up;   /* num_experts packed [2*intermediate][hidden] matrices, back to back */
  const uint16_t *w_down;      /* num_experts packed [hidden][intermediate] matrices, back to back */
  const float *couple_b;       /* [intermediate] or NULL */
  const float *couple_c;       /* [hidden] or NULL */
} dfx_moe_weights;

/* Byte offsets in the workspace of a completed dfx_dual_flow_moe_mlp call:
 *   h       bf16 [n_flows][batch][hidden] normed rows, row-major
 *   logits  fp32 [n_flows][batch][num_experts] router logits
 *   ids     int32 [n_flows][batch][16] expert ids in ranking order (-1 past the fan-out)
 *   weights fp32 [n_flows][batch][16] mixture weights (0 past the fan-out)
 *   counts  int32 [num_experts] sequences using each expert (by either flow)
 *   seqs    int32 [num_experts][batch] those sequences, ascending
 *   inter   bf16 intermediates per expert: expert e's row r (flow f, sequence seqs[e][r]) at
 *           e * inter_stride elements plus the fragment-order offset of
 *           dfx_dual_flow_decode_layer_taps with K = intermediate (inter_stride in elements).
 * Host-only: no GPU work. */
typedef struct dfx_moe_taps {
  size_t h, logits, ids, weights, counts, seqs, inter, inter_stride;
} dfx_moe_taps;

dfx_status dfx_dual_flow_moe_mlp_workspace_size(const dfx_moe_weights *w, int32_t batch, int32_t n_flows,
                                                size_t *bytes);

dfx_status dfx_dual_flow_moe_mlp_taps(const dfx_moe_weights *w, int32_t batch, int32_t n_flows,
                                      dfx_moe_taps *taps);

/*
 *  x          device fp32 [n_flows][batch][hidden], 16-byte aligned, updated in place.
 *  batch      0 .. 65535, with num_experts * ceil(batch / 32) <= 16384.
 *  workspace  >= dfx_dual_flow_moe_mlp_workspace_size bytes, no initial contents.
 * All vectors and matrices 16-byte aligned. The call allocates nothing and never synchronizes;
 * calls sharing a workspace must not overlap.
 */
dfx_status dfx_dual_flow_moe_mlp(const dfx_moe_weights *w, int32_t batch, int32_t n_flows, float *x,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * Prefill by the primary flow alone (Sintesi Tecnica: Dual-Flow Transformers, "Costi di
 * Inferenza vs. Addestramento": prefill costs what a standard Transformer's does, the
 * auxiliary flow being skipped entirely; "Architettura Core": the auxiliary flow starts at the
 * last prompt position). A prompt of n tokens is a prefill of tokens 0 .. n-2 with these calls,
 * then dfx_dual_flow_decode_step at position n-1 with both flows. A chunk holds `chunk` new
 * positions of every sequence; start_pos[b] (device int32 [batch]) is the position of
 * sequence b's first new token, and start_pos[b] + chunk <= max_context <= the cache's capacity.
 * The cache must be bf16, paged blocks >= 16 tokens; num_q_heads a multiple of 4; batch * chunk
 * at most 2^22 rows and chunk at most 1048560 positions. Positions and block ids are clamped on
 * the device like the decode calls'.
 *
 * dfx_prefill_attn: causal attention of the new positions, whose keys and values are already
 * in the cache: query t of sequence b attends to positions [0, start_pos[b] + t].
 *   q    device fp32 rows (b, t) of num_q_heads * head_dim values, row (b * chunk + t) at
 *        q + row * q_row_stride (0: num_q_heads * head_dim); 16-byte aligned, stride % 4 == 0.
 *   o    device fp32 [batch][chunk][num_q_heads][head_dim], output.
 *   lse  device fp32 [batch][chunk][num_q_heads] natural-log sums, output, or NULL.
 * No workspace.
 */
dfx_status dfx_prefill_attn(const dfx_kv_cache *kv, const int32_t *start_pos, int32_t batch, int32_t chunk,
                            int32_t max_context, int32_t num_q_heads, const float *q, int64_t q_row_stride,
                            float *o, float *lse, void *stream);

/*
 * dfx_prefill_dual_attn: the same causal attention with both flows at every new position, the
 * training-time forward of the attention (Sintesi Tecnica: Dual-Flow Transformers, "Costi di
 * Inferenza vs. Addestramento": training runs both flows over the whole sequence; "Meccanismi
 * Chiave": the auxiliary's query is coupled to the primary's and attends to the primary's keys
 * and values). Query t of sequence b, flow f, attends to positions [0, start_pos[b] + t] of the
 * cache, which holds the primary's keys and values; each K/V tile is loaded once for both
 * flows.
 *   q1, q2_raw     device fp32 rows laid out as dfx_prefill_attn's q (same q_row_stride); the
 *                  auxiliary's query is Q2 = q2_raw + a (.) Q1 (fp32 fma).
 *   a              device fp32 [head_dim] (a_head_stride 0) or [num_q_heads][head_dim]
 *                  (a_head_stride head_dim), 4-byte aligned; NULL: Q2 = q2_raw.
 *   o1, o2         device fp32 [batch][chunk][num_q_heads][head_dim], outputs.
 *   lse            device fp32 [2][batch][chunk][num_q_heads] natural-log sums, or NULL.
 * The limits and errors of dfx_prefill_attn. No workspace; the cache is only read.
 */
dfx_status dfx_prefill_dual_attn(const dfx_kv_cache *kv, const int32_t *start_pos, int32_t batch, int32_t chunk,
                                 int32_t max_context, int32_t num_q_heads, const float *q1, const float *q2_raw,
                                 const float *a, int32_t a_head_stride, int64_t q_row_stride, float *o1, float *o2,
                                 float *lse, void *stream);

/*
 * dfx_prefill_layer: one layer for the new positions of the primary, in place on x (device
 * fp32 [batch][chunk][hidden]): the decode layer's steps with one flow and every position a
 * row -- norm, shared Q/K/V projection, the chunk's keys and values appended at start_pos[b] + t
 * (bf16, nearest even), causal attention (rows rounded to bf16), W_o + residual, norm, gate/up
 * with SwiGLU (no coupling: the auxiliary is off), W_down + residual. The same bf16 rounding
 * points as the decode layer. workspace: >= dfx_prefill_layer_workspace_size bytes.
 */
dfx_status dfx_prefill_layer_workspace_size(const dfx_layer_weights *w, const dfx_kv_cache *kv, int32_t batch,
                                            int32_t chunk, int32_t max_context, size_t *bytes);

dfx_status dfx_prefill_layer(const dfx_layer_weights *w, const dfx_kv_cache *kv, const int32_t *start_pos,
                             int32_t batch, int32_t chunk, int32_t max_context, float *x, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * Where a completed dfx_prefill_layer call with the same sizes leaves its intermediates in the
 * workspace (the same rounding points as the decode layer; Sintesi Tecnica: Dual-Flow
 * Transformers, section "Architettura Core": during prefill the primary runs alone), byte
 * offsets of, for the batch * chunk rows r = b * chunk + t:
 *   h1     bf16 normed rows entering W_qkv, in the activation fragment order of
 *          dfx_dual_flow_decode_layer_taps with one flow (64-row groups of r)  [hidden columns]
 *   q      fp32 rows [batch * chunk][(Hq + 2 Hkv) * D]: the whole Q/K/V projection
 *   o      bf16 attention rows entering W_o, fragment order                     [Hq * D]
 *   h2     bf16 normed rows entering W_gate_up, fragment order                  [hidden]
 *   inter  bf16 SwiGLU rows entering W_down, fragment order                     [intermediate]
 * Pure host arithmetic; the arguments dfx_prefill_layer_workspace_size rejects are rejected.
 */
dfx_status dfx_prefill_layer_taps(const dfx_layer_weights *w, const dfx_kv_cache *kv, int32_t batch,
                                  int32_t chunk, int32_t max_context, dfx_layer_taps *taps);

/*
 * dfx_prefill_step: tokens (device int32 [batch][chunk], clamped to [0, vocab)) through the
 * primary's embedding table (bf16 [vocab][hidden], 8-byte aligned) and every layer
 * (dfx_prefill_layer with layers[l], caches[l]); x (device fp32 [batch][chunk][hidden]) is
 * the output. The call allocates nothing and never synchronizes.
 */
dfx_status dfx_prefill_step_workspace_size(const dfx_layer_weights *layers, const dfx_kv_cache *caches,
                                           int32_t n_layers, int32_t batch, int32_t chunk, int32_t max_context,
                                           size_t *bytes);

dfx_status dfx_prefill_step(const dfx_layer_weights *layers, const dfx_kv_cache *caches, int32_t n_layers,
                            const int32_t *tokens, int32_t vocab, const uint16_t *embed_primary,
                            const int32_t *start_pos, int32_t batch, int32_t chunk, int32_t max_context, float *x,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Measurement helpers (not part of the method): a plain device copy of
 * `bytes` (multiple of 16, both pointers 16-byte aligned) used to calibrate
 * hardware traffic counters, a read of `bytes` (achievable read bandwidth;
 * sink: device uint32 [4096 * 256] receiving per-thread XORs of the data),
 * and a write of `bytes` used to evict caches between timed iterations.
 */
dfx_status dfx_copy_bytes(void *dst, const void *src, size_t bytes, void *stream);
dfx_status dfx_read_bytes(const void *src, size_t bytes, uint32_t *sink, void *stream);
dfx_status dfx_fill_bytes(void *dst, size_t bytes, uint32_t pattern, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DFX_H */
