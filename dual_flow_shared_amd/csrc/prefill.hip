// Prefill by the primary flow alone (Sintesi Tecnica: Dual-Flow Transformers, "Costi di
// Inferenza vs. Addestramento": the auxiliary flow is skipped during prefill and the primary
// is an ordinary causal Transformer writing the cache; the auxiliary starts at the last prompt
// position, which is a decode step).
//
// prefill_append_kernel: the chunk's key and value columns of the fused projection rows go to
// the cache at positions start_b + t (bf16, nearest even), the query columns stay in place.
// prefill_attn_kernel: causal attention of every new position over the cache. A work-group is
// 4 waves; wave w takes query head 4x + w and 16 consecutive positions of one sequence, and
// streams all keys up to the tile's last position in 32-token tiles with the decode kernel's
// MFMA tile code (attn_tiles.h); each lane masks its own row at the row's position. The waves
// of a group of heads read the same K/V lines at about the same time, so the cache is fetched
// from HBM about once per work-group and re-read from the CU's caches by the other waves.
//
// The same kernels with both flows at every position are the training-time forward of the
// attention (the summary's cost section: training runs both flows over the whole sequence):
// a work-group then holds 2 query heads x 2 flows, the auxiliary's query coupled to the
// primary's (Q2 = q2_raw + a (.) Q1), both attending to the primary's keys and values.
#include "attn_tiles.h"

namespace dfx {

// One thread per 4 key or value columns of one (sequence, position) row.
__global__ void __launch_bounds__(256) prefill_append_kernel(PrefillGlueArgs a) {
  const dfx_kv_cache &kv = a.kv;
  const int kvcols = kv.num_kv_heads * kv.head_dim;
  const int n4 = 2 * kvcols / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.B * a.T * n4) return;
  const int c = (int)(idx % n4) * 4;
  const int64_t row = idx / n4;
  const int b = (int)(row / a.T), t = (int)(row % a.T);
  const bool is_v = c >= kvcols;
  const int cc = is_v ? c - kvcols : c;
  const int g = cc / kv.head_dim, d = cc % kv.head_dim;
  const f32x4 v = *(const f32x4 *)(a.qkv + row * a.N + a.num_q_heads * a.head_dim + c);
  const bool paged = kv.block_table != nullptr;
  const int64_t cap = paged ? (int64_t)kv.max_blocks_per_seq * kv.block_size : kv.block_size;
  int64_t pos = (int64_t)a.start[b] + t;
  pos = pos < 0 ? 0 : (pos >= cap ? cap - 1 : pos);
  int64_t blk, slot;
  if (paged) {
    const uint32_t e = (uint32_t)kv.block_table[(int64_t)b * kv.max_blocks_per_seq + pos / kv.block_size];
    blk = (uint64_t)e < (uint64_t)kv.num_blocks ? (int64_t)e : kv.num_blocks - 1;
    slot = pos % kv.block_size;
  } else {
    blk = b;
    slot = pos;
  }
  uint16_t *pool = (uint16_t *)(is_v ? kv.v : kv.k);
  const int64_t dst = ((blk * kv.num_kv_heads + g) * kv.block_size + slot) * kv.head_dim + d;
  *(u32x2 *)(pool + dst) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

hipError_t launch_prefill_append(const PrefillGlueArgs &a, hipStream_t s) {
  const int64_t threads = (int64_t)a.B * a.T * (2 * a.kv.num_kv_heads * a.kv.head_dim / 4);
  if (threads == 0) return hipSuccess;
  prefill_append_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

// bf16 terms of the queries and of P in the causal attention: three, every bit of the fp32
// values (the attention rows are rounded to bf16 before W_o; with fp32-exact operands the
// rounding decisions are those of an fp32 evaluation).
constexpr int kPrefillTerms = 3;

// Per-flow state of a wave's 16 query rows: the queries split into bf16 terms, O^T
// accumulators and the online-softmax statistics of the lane's row.
template <int D>
struct FlowAcc {
  u32x4 q[kPrefillTerms][D / 32];
  f32x4 oacc[D / 16];
  float m_run, l_run;
};

// Query row n of the wave (position t0 + n of head h) for flow f. The auxiliary's query is
// q2_raw + a (.) q1 in fp32 (the decode kernels' formula); rows past the chunk are zero.
template <int D>
__device__ __forceinline__ void prefill_query(const AttnArgs &p, int f, int b, int t0, int n, int j, int rows,
                                              int h, FlowAcc<D> &fa) {
  constexpr int KS = D / 32;
  const bool valid = n < rows;
  const int64_t qoff = ((int64_t)b * p.prefill_T + t0 + (valid ? n : 0)) * p.q_bstride + (int64_t)h * D;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int d0 = 8 * (4 * s + j);
    float q[8];
    load8<false>(p.q1, qoff + d0, q);
    if (f == 1) {
      float q2[8];
      load8<false>(p.q2, qoff + d0, q2);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        q[i] = p.a ? fmaf(p.a[(int64_t)h * p.a_hstride + d0 + i], q[i], q2[i]) : q2[i];
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t t0[kPrefillTerms], t1[kPrefillTerms];
      split_terms<kPrefillTerms>(valid ? q[2 * w] : 0.f, t0);
      split_terms<kPrefillTerms>(valid ? q[2 * w + 1] : 0.f, t1);
#pragma unroll
      for (int t = 0; t < kPrefillTerms; ++t) fa.q[t][s][w] = t0[t] | (t1[t] << 16);
    }
  }
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) fa.oacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  fa.m_run = -INFINITY;
  fa.l_run = 0.f;
}

// Row n's result for flow f: its sum over the four lanes that hold it, then 32 consecutive
// head-dim values per lane -- fp32 rows of o1 / o2, or (one flow) bf16 rows of W_o's input in
// the grouped linear's fragment order -- and the natural-log sum, [F][batch * chunk][Hq].
template <int D>
__device__ __forceinline__ void prefill_store(const AttnArgs &p, int f, int b, int t0, int n, int j, int rows,
                                              int h, const FlowAcc<D> &fa) {
  constexpr int VEC = D / 16;
  float l_tot = fa.l_run + __shfl_xor(fa.l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (n >= rows) return;
  const float inv = 1.0f / l_tot;
  const int64_t r = (int64_t)b * p.prefill_T + t0 + n;
  const int Hq = p.num_q_heads;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float o[VEC];
#pragma unroll
    for (int mb = 0; mb < VEC; ++mb) o[mb] = fa.oacc[mb][i] * inv;
    const int d0 = VEC * (4 * j + i);
    if (p.o_packed) {
      uint16_t *dst = (uint16_t *)p.o1 + xpack_offset(1, 0, (int)r, h * D + d0, Hq * D);
      if constexpr (VEC == 8)
        *(u32x4 *)dst = u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                              pack_bf16x2(o[6], o[7])};
      else
        *(u32x2 *)dst = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    } else {
      float *dst = (f == 0 ? p.o1 : p.o2) + (r * Hq + h) * D + d0;
#pragma unroll
      for (int v = 0; v < VEC; v += 4) *(f32x4 *)(dst + v) = f32x4{o[v], o[v + 1], o[v + 2], o[v + 3]};
    }
  }
  if (j == 0 && p.lse)
    p.lse[((int64_t)f * p.batch * p.prefill_T + r) * Hq + h] = (fa.m_run + __log2f(l_tot)) * kLn2;
}

// F flows: wave w takes flow w % F of query head (4 / F) x + w / F, so with both flows the two
// waves of a head read the same K/V lines at the same time.
template <int D, bool PAGED, int F>
__global__ void __launch_bounds__(256) prefill_attn_kernel(AttnArgs p) {
  __shared__ int32_t s_tbl[kMaxChunkBlocks];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;  // a scalar
  const int n = lane & 15, j = lane >> 4;
  const int h = blockIdx.x * (4 / F) + wave / F, f = wave % F, b = blockIdx.y;
  const int tile = gridDim.z - 1 - blockIdx.z;  // the longest tiles are dispatched first
  const int T = p.prefill_T, t0 = 16 * tile;
  const int g = h / p.group;
  const int cap = p.max_context;
  const int start = min(max(p.ctx[b], 0), cap);
  const int rows = min(16, T - t0);
  // keys [0, kend): up to this tile's last position; each lane's row stops at its own
  const int kend = max(min(start + t0 + rows, cap), 1);
  const int my_end = n < rows ? min(start + t0 + n + 1, kend) : 1;

  FlowAcc<D> fa;
  prefill_query<D>(p, f, b, t0, n, j, rows, h, fa);

  const uint16_t *kp = (const uint16_t *)p.k;
  const uint16_t *vp = (const uint16_t *)p.v;

  // keys in chunks of at most kMaxChunkBlocks staged block ids
  const int chunk_tok = PAGED ? (kMaxChunkBlocks << p.block_shift) : kend;
  for (int cs = 0; cs < kend; cs += chunk_tok) {
    const int ce = min(cs + chunk_tok, kend);
    const int first_blk = PAGED ? (cs >> p.block_shift) : 0;
    if constexpr (PAGED) {
      __syncthreads();  // every wave is done with the previous chunk's ids
      const int nblk = ((ce - 1) >> p.block_shift) - first_blk + 1;
      for (int i = threadIdx.x; i < nblk; i += 256) {
        const uint32_t e = (uint32_t)p.table[(int64_t)b * p.max_blocks + first_blk + i];
        s_tbl[i] = (uint64_t)e < (uint64_t)p.num_blocks ? (int32_t)e : (int32_t)(p.num_blocks - 1);
      }
      __syncthreads();
    }
    TileRegs<D> tr;
    int64_t hb[2];
    int lx[2];
    f32x4 sacc[2];
    int t = cs;
    half_bases<PAGED>(p, s_tbl, first_blk, b, g, t, ce, hb, lx);
    load_k<D>(kp, hb, lx, n, j, tr);
    load_v<D>(vp, hb, lx, n, j, tr);
    for (; t + 32 < ce; t += 32) {
      half_bases<PAGED>(p, s_tbl, first_blk, b, g, t + 32, ce, hb, lx);
      tile_scores<D, kPrefillTerms>(tr, fa.q, sacc);
      load_k<D>(kp, hb, lx, n, j, tr);
      tile_softmax_pv<D, kPrefillTerms, true>(p, tr, sacc, t, my_end, j, fa.m_run, fa.l_run, fa.oacc);
      load_v<D>(vp, hb, lx, n, j, tr);
    }
    tile_scores<D, kPrefillTerms>(tr, fa.q, sacc);
    tile_softmax_pv<D, kPrefillTerms, true>(p, tr, sacc, t, my_end, j, fa.m_run, fa.l_run, fa.oacc);
  }

  prefill_store<D>(p, f, b, t0, n, j, rows, h, fa);
}

// The same attention with the four waves' K/V tiles shared through LDS (head_dim 128, the
// four heads of a work-group in one KV group). A tile's register image -- what load_k and
// load_v leave in each lane: 8 K fragments and 8 V rows of 16 bytes -- is 16 components of 64
// lanes; wave w loads components 4w .. 4w + 3 of the next tile from memory while all waves
// multiply the current one from LDS, so each K/V byte is fetched once per work-group.
__device__ __forceinline__ u32x4 tile_component(const uint16_t *kp, const uint16_t *vp, const int64_t *hb,
                                                const int *lx, int n, int j, int c) {
  constexpr int D = 128;
  if (c < 8) {  // K fragment: 16-token half c / 4, head-dim chunk 4 (c % 4) + j of row n
    const int mb = c >> 2, s = c & 3;
    return kv_load<u32x4>(kp + hb[mb] + (int64_t)min(n, lx[mb]) * D + 8 * (4 * s + j));
  }
  const int v = c - 8, h = v >> 2, x = 4 * j + (v & 3);  // V row tau(j, v), elements 8n .. 8n + 7
  return kv_load<u32x4>(vp + hb[h] + (int64_t)min(x, lx[h]) * D + 8 * n);
}

template <bool PAGED, int F>
__global__ void __launch_bounds__(256) prefill_attn_shared_kernel(AttnArgs p) {
  constexpr int D = 128;
  __shared__ int32_t s_tbl[kMaxChunkBlocks];
  __shared__ u32x4 s_img[2][16][64];
  // the wave index in a scalar register: the head, the flow and every address base derived
  // from it are then the wave's scalars, and their arithmetic runs on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;
  // wave w: flow w % F of query head (4 / F) x + w / F
  const int h = blockIdx.x * (4 / F) + wave / F, f = wave % F, b = blockIdx.y;
  const int tile = gridDim.z - 1 - blockIdx.z;  // the longest tiles are dispatched first
  const int T = p.prefill_T, t0 = 16 * tile;
  const int g = h / p.group;  // the same for the four waves (group % 4 == 0)
  const int cap = p.max_context;
  const int start = min(max(p.ctx[b], 0), cap);
  const int rows = min(16, T - t0);
  const int kend = max(min(start + t0 + rows, cap), 1);
  const int my_end = n < rows ? min(start + t0 + n + 1, kend) : 1;

  FlowAcc<D> fa;
  prefill_query<D>(p, f, b, t0, n, j, rows, h, fa);
  const uint16_t *kp = (const uint16_t *)p.k;
  const uint16_t *vp = (const uint16_t *)p.v;

  const int chunk_tok = PAGED ? (kMaxChunkBlocks << p.block_shift) : kend;
  for (int cs = 0; cs < kend; cs += chunk_tok) {
    const int ce = min(cs + chunk_tok, kend);
    const int first_blk = PAGED ? (cs >> p.block_shift) : 0;
    __syncthreads();  // the previous chunk's ids and images are no longer read
    if constexpr (PAGED) {
      const int nblk = ((ce - 1) >> p.block_shift) - first_blk + 1;
      for (int i = threadIdx.x; i < nblk; i += 256) {
        const uint32_t e = (uint32_t)p.table[(int64_t)b * p.max_blocks + first_blk + i];
        s_tbl[i] = (uint64_t)e < (uint64_t)p.num_blocks ? (int32_t)e : (int32_t)(p.num_blocks - 1);
      }
      __syncthreads();
    }
    int64_t hb[2];
    int lx[2];
    u32x4 st[4];
    half_bases<PAGED>(p, s_tbl, first_blk, b, g, cs, ce, hb, lx);
#pragma unroll
    for (int i = 0; i < 4; ++i) st[i] = tile_component(kp, vp, hb, lx, n, j, 4 * wave + i);
#pragma unroll
    for (int i = 0; i < 4; ++i) s_img[0][4 * wave + i][lane] = st[i];
    __syncthreads();
    int slot = 0;
    for (int t = cs; t < ce; t += 32) {
      // the next tile's components (the current tile again after the last: never read)
      const int tn = t + 32 < ce ? t + 32 : t;
      half_bases<PAGED>(p, s_tbl, first_blk, b, g, tn, ce, hb, lx);
#pragma unroll
      for (int i = 0; i < 4; ++i) st[i] = tile_component(kp, vp, hb, lx, n, j, 4 * wave + i);
      TileRegs<D> tr;
#pragma unroll
      for (int c = 0; c < 8; ++c) tr.kf[c >> 2][c & 3] = s_img[slot][c][lane];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const u32x4 y = s_img[slot][8 + v][lane];
        tr.vr[v][0] = y[0]; tr.vr[v][1] = y[1]; tr.vr[v][2] = y[2]; tr.vr[v][3] = y[3];
      }
      f32x4 sacc[2];
      tile_scores<D, kPrefillTerms>(tr, fa.q, sacc);
      tile_softmax_pv<D, kPrefillTerms, true>(p, tr, sacc, t, my_end, j, fa.m_run, fa.l_run, fa.oacc);
#pragma unroll
      for (int i = 0; i < 4; ++i) s_img[slot ^ 1][4 * wave + i][lane] = st[i];
      __syncthreads();
      slot ^= 1;
    }
  }

  prefill_store<D>(p, f, b, t0, n, j, rows, h, fa);
}

template <int F>
void launch_prefill_attn_flows(const AttnArgs &a, dim3 grid, dim3 block, hipStream_t s) {
  const bool paged = a.block_shift >= 0;
  if (a.head_dim == 128 && a.group % 4 == 0) {
    if (paged) prefill_attn_shared_kernel<true, F><<<grid, block, 0, s>>>(a);
    else prefill_attn_shared_kernel<false, F><<<grid, block, 0, s>>>(a);
  } else if (a.head_dim == 128) {
    if (paged) prefill_attn_kernel<128, true, F><<<grid, block, 0, s>>>(a);
    else prefill_attn_kernel<128, false, F><<<grid, block, 0, s>>>(a);
  } else {
    if (paged) prefill_attn_kernel<64, true, F><<<grid, block, 0, s>>>(a);
    else prefill_attn_kernel<64, false, F><<<grid, block, 0, s>>>(a);
  }
}

hipError_t launch_prefill_attn(const AttnArgs &a, hipStream_t s) {
  if (a.batch == 0 || a.prefill_T == 0) return hipSuccess;
  const dim3 grid(a.num_q_heads * a.n_flows / 4, a.batch, (a.prefill_T + 15) / 16), block(256);
  if (a.n_flows == 2) launch_prefill_attn_flows<2>(a, grid, block, s);
  else launch_prefill_attn_flows<1>(a, grid, block, s);
  return hipGetLastError();
}

}  // namespace dfx
