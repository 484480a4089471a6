// Dual-query flash-decoding over a bf16 K/V cache on gfx950 matrix cores.
//
// The auxiliary query attends to the primary's keys and values, so one pass over the
// cache serves both flows (Sintesi Tecnica: Dual-Flow Transformers, "Meccanismi
// Chiave"). One work-group owns (sequence b, KV head g, context split); its query
// tile holds every query row that reads KV head g: n_flows x (Hq / Hkv) rows, at most
// 16 -- both flows and all grouped-query heads share each K/V byte fetched from HBM.
//
// Per 32-token tile a wave computes
//   S^T[tok][row] = K[tok][:] . Q[row][:]       (16x16x32 bf16 MFMA, two 16-token blocks)
//   O^T[d][row]  += V^T[d][tok] . P^T[tok][row] (one MFMA per 16 head-dim rows)
// with fp32 accumulation. Q and P are fp32 values; each is split into bf16 terms and
// multiplied once per term (K and V are exact bf16 already): three terms for fp32 queries
// carry every bit of Q and P, two for bf16 queries about 16 significant bits. The softmax is online (running max m, sum l) in the
// log2 domain; a row's statistics live in the same lane as its O^T column, so the
// per-tile rescale needs no cross-lane traffic.
//
// Lane layouts (64 lanes, n = lane % 16, j = lane / 16):
//   A operand 16 x 32: lane holds row n, k = 8j .. 8j+7;  B operand 32 x 16: column n,
//   k = 8j .. 8j+7;  C 16 x 16: column n, rows 4j .. 4j+3.
// The k order of a contraction is free as long as both operands use it, which fixes the
// loads: score k-step s uses head-dim chunk c = 4s + j (so one load instruction reads a
// 64-byte run of 16 token rows); the P.V contraction orders tokens as
// tau(j, v) = 4j + v (v < 4), 16 + 4j + v - 4 (v >= 4), which is exactly where the
// score MFMA left them, and its M rows are head-dim d = VEC * m + mb, so one lane loads
// VEC contiguous elements of 8 token rows (4 full rows per load instruction) and a
// register transpose yields the V^T operand.
#include "attn_tiles.h"

namespace dfx {

// Writes one finished (row, d) value: final output when there is a single split,
// otherwise the split's normalized partial and its log2-domain LSE.
__device__ __forceinline__ void store_result(const AttnArgs &p, int split, int b, int g, int r,
                                             int d, float M, float L, float O) {
  const int G = p.group;
  const int f = r / G, h = g * G + r % G;
  const int Hq = p.num_q_heads, D = p.head_dim;
  const float o = L > 0.f ? O / L : 0.f;
  const float lse2 = L > 0.f ? M + __log2f(L) : -INFINITY;
  if (p.num_splits == 1) {
    int64_t oi;
    float *out = attn_out(p, f, b, h * D + d, &oi);
    if (p.o_bf16) ((uint16_t *)out)[oi] = (uint16_t)f32_to_bf16_rne(o);
    else out[oi] = o;
    if (d == 0 && p.lse) p.lse[((int64_t)f * p.batch + b) * Hq + h] = lse2 * kLn2;
  } else {
    const int64_t row = (((int64_t)split * p.n_flows + f) * p.batch + b) * Hq + h;
    p.part_o[row * D + d] = o;
    if (d == 0) p.part_lse[row] = lse2;
  }
}

#ifndef DFX_ATTN_WAVES
#define DFX_ATTN_WAVES 4
#endif

// K through LDS (AttnArgs::k_rows): a wave loads its tile's K rows with whole-row accesses (one
// load instruction covers 64 x 16 contiguous bytes, D / 8 lanes per row), writes them to a padded
// row-major LDS area of its own, and reads them back in the MFMA A-operand order (row n, head-dim
// chunk 4 s + j). The direct path reads the A operand straight from memory, 16 rows x 64 bytes per
// instruction. Which one streams faster depends on the launch; the planner picks.
template <int D>
struct KRows {
  static constexpr int CPR = D / 8;         // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;      // rows per load instruction
  static constexpr int NI = 2 * 16 / RPI;   // load instructions per 32-token tile
};

template <int D>
__device__ __forceinline__ void load_k_rows(const uint16_t *kp, const int64_t *hb, const int *lastx, int lane,
                                            u32x4 *kr) {
  using R = KRows<D>;
#pragma unroll
  for (int i = 0; i < R::NI; ++i) {
    const int mb = i / (R::NI / 2), tok = (i % (R::NI / 2)) * R::RPI + lane / R::CPR;
    kr[i] = kv_load<u32x4>(kp + hb[mb] + (int64_t)min(tok, lastx[mb]) * D + 8 * (lane % R::CPR));
  }
}

template <int D>
__device__ __forceinline__ void store_k_rows(u32x4 (*sk)[KRows<D>::CPR + 1], int lane, const u32x4 *kr) {
  using R = KRows<D>;
#pragma unroll
  for (int i = 0; i < R::NI; ++i) {
    const int mb = i / (R::NI / 2), tok = (i % (R::NI / 2)) * R::RPI + lane / R::CPR;
    sk[16 * mb + tok][lane % R::CPR] = kr[i];
  }
}

template <int D>
__device__ __forceinline__ void read_k_frags(u32x4 (*sk)[KRows<D>::CPR + 1], int n, int j, TileRegs<D> &r) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int s = 0; s < D / 32; ++s) r.kf[mb][s] = sk[16 * mb + n][4 * s + j];
}
constexpr int kAttnWaves = DFX_ATTN_WAVES;  // waves per work-group, interleaved over the tiles

template <int D, bool QBF16, bool PAGED, bool KROWS>
__device__ __forceinline__ void attn_mfma_body(const AttnArgs &p) {
  constexpr int KS = D / 32;  // k-steps of the score contraction
  constexpr int VEC = D / 16; // head-dim elements one lane loads per V row; also O^T blocks
  constexpr int W = kAttnWaves, NTH = 64 * kAttnWaves;
  // bf16 terms of Q and P per MFMA operand: three for fp32 queries (every fp32 bit, so the
  // scores and the P.V products carry fp32 precision), two for bf16 queries (whose
  // auxiliary query is fp32 only through the coupling; about 16 significant bits)
  constexpr int NT = QBF16 ? 2 : 3;
  __shared__ float s_o[W][16][D];
  __shared__ float s_m[W][16], s_l[W][16];
  __shared__ int32_t s_tbl[kMaxChunkBlocks];
  __shared__ u32x4 s_k[KROWS ? W : 1][32][KRows<D>::CPR + 1];  // each wave's K rows of its tile

  const int g = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;
  const int ctx = min(max(p.ctx[b], 0), p.max_context);
  const int start = split * p.chunk;
  if (split > 0 && start >= ctx) return;  // uniform for the whole work-group
  const int end = min(start + p.chunk, ctx);
  const int G = p.group, R = p.n_flows * G;

  // ---- query tile: lane holds query row n, head-dim chunks 4s + j; Q2 coupled here.
  u32x4 q3[NT][KS];
  {
    const bool valid = n < R;
    const int f = valid ? n / G : 0;
    const int h = g * G + (valid ? n % G : 0);
    const int64_t qoff = (int64_t)b * p.q_bstride + (int64_t)h * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int d0 = 8 * (4 * s + j);
      float q[8];
      load8<QBF16>(p.q1, qoff + d0, q);
      if (f == 1) {
        float q2[8];
        load8<QBF16>(p.q2, qoff + d0, q2);
        if (p.a) {
          const float *av = p.a + (int64_t)h * p.a_hstride + d0;
#pragma unroll
          for (int v = 0; v < 8; ++v) q[v] = fmaf(av[v], q[v], q2[v]);
        } else {
#pragma unroll
          for (int v = 0; v < 8; ++v) q[v] = q2[v];
        }
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t t0[NT], t1[NT];
        split_terms<NT>(valid ? q[2 * w] : 0.f, t0);
        split_terms<NT>(valid ? q[2 * w + 1] : 0.f, t1);
#pragma unroll
        for (int t = 0; t < NT; ++t) q3[t][s][w] = t0[t] | (t1[t] << 16);
      }
    }
  }

  const uint16_t *kp = (const uint16_t *)p.k;
  const uint16_t *vp = (const uint16_t *)p.v;
  f32x4 oacc[VEC];
#pragma unroll
  for (int mb = 0; mb < VEC; ++mb) oacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Block ids of this chunk go to LDS once, so no K/V load waits on a table load.
  const int first_blk = PAGED ? (start >> p.block_shift) : 0;
  if constexpr (PAGED) {
    const int nblk = end > start ? ((end - 1) >> p.block_shift) - first_blk + 1 : 0;
    for (int i = threadIdx.x; i < nblk; i += NTH) {
      const uint32_t e = (uint32_t)p.table[(int64_t)b * p.max_blocks + first_blk + i];
      s_tbl[i] = (uint64_t)e < (uint64_t)p.num_blocks ? (int32_t)e : (int32_t)(p.num_blocks - 1);
    }
  }
  __syncthreads();

  // Tiles of a wave are 32 W tokens apart (the W waves interleave). The next tile's K
  // loads are issued as soon as this tile's scores have consumed the K registers, and
  // its V loads as soon as P.V has consumed the V registers. The steady-state loop has
  // no conditional loads, so the compiler can wait for exactly the loads it needs.
  TileRegs<D> tr;
  int t0 = start + 32 * wave;
  if (t0 < end) {
    int64_t hb[2];
    int lx[2];
    half_bases<PAGED>(p, s_tbl, first_blk, b, g, t0, end, hb, lx);
    f32x4 sacc[2];
    if constexpr (KROWS) {
      u32x4 kr[KRows<D>::NI];
      load_k_rows<D>(kp, hb, lx, lane, kr);
      load_v<D>(vp, hb, lx, n, j, tr);
      store_k_rows<D>(s_k[wave], lane, kr);
      for (; t0 + 32 * W < end; t0 += 32 * W) {
        half_bases<PAGED>(p, s_tbl, first_blk, b, g, t0 + 32 * W, end, hb, lx);
        read_k_frags<D>(s_k[wave], n, j, tr);
        tile_scores<D, NT>(tr, q3, sacc);
        load_k_rows<D>(kp, hb, lx, lane, kr);
        tile_softmax_pv<D, NT>(p, tr, sacc, t0, end, j, m_run, l_run, oacc);
        load_v<D>(vp, hb, lx, n, j, tr);
        store_k_rows<D>(s_k[wave], lane, kr);  // after this wave's reads of the current rows
      }
      read_k_frags<D>(s_k[wave], n, j, tr);
    } else {
      load_k<D>(kp, hb, lx, n, j, tr);
      load_v<D>(vp, hb, lx, n, j, tr);
      for (; t0 + 32 * W < end; t0 += 32 * W) {
        half_bases<PAGED>(p, s_tbl, first_blk, b, g, t0 + 32 * W, end, hb, lx);
        tile_scores<D, NT>(tr, q3, sacc);
        load_k<D>(kp, hb, lx, n, j, tr);
        tile_softmax_pv<D, NT>(p, tr, sacc, t0, end, j, m_run, l_run, oacc);
        load_v<D>(vp, hb, lx, n, j, tr);
      }
    }
    tile_scores<D, NT>(tr, q3, sacc);
    tile_softmax_pv<D, NT>(p, tr, sacc, t0, end, j, m_run, l_run, oacc);
  }

  // ---- combine the W waves (fixed order), then store output or split partial
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (j == 0) {
    s_m[wave][n] = m_run;
    s_l[wave][n] = l_tot;
  }
#pragma unroll
  for (int mb = 0; mb < VEC; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[wave][n][VEC * (4 * j + i) + mb] = oacc[mb][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < R * D; idx += NTH) {
    const int r = idx / D, d = idx % D;
    float M = s_m[0][r];
#pragma unroll
    for (int w = 1; w < W; ++w) M = fmaxf(M, s_m[w][r]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float c = exp2f(s_m[w][r] - M);
        L += c * s_l[w][r];
        O += c * s_o[w][r][d];
      }
    }
    store_result(p, split, b, g, r, d, M, L, O);
  }
}

// bf16 queries (two bf16 terms of Q and P)
template <int D, bool PAGED, bool KROWS>
__global__ void __launch_bounds__(64 * kAttnWaves) attn_mfma_kernel(AttnArgs p) {
  attn_mfma_body<D, true, PAGED, KROWS>(p);
}

// fp32 queries (three terms): the bound keeps two waves per SIMD, which the register allocator
// gives up for the third term's registers on some variants otherwise.
template <int D, bool PAGED, bool KROWS>
__global__ void __launch_bounds__(64 * kAttnWaves, 2) attn_mfma_f32q_kernel(AttnArgs p) {
  attn_mfma_body<D, false, PAGED, KROWS>(p);
}

hipError_t launch_attn_mfma(const AttnArgs &a, hipStream_t s) {
  // The hardware hands work-group i to XCD i % 8. With the KV head fastest, XCD k serves
  // head k of every sequence (an equal share whatever the context lengths), and each XCD
  // dispatches all first splits (the longest pieces of ragged batches) before the later ones.
  const dim3 grid(a.num_kv_heads, a.batch, a.num_splits), block(64 * kAttnWaves);
  const bool paged = a.block_shift >= 0;
#define DFX_ATTN_LAUNCH(KERNEL, D, PG)                                 \
  do {                                                                 \
    if (a.k_rows) KERNEL<D, PG, true><<<grid, block, 0, s>>>(a);        \
    else KERNEL<D, PG, false><<<grid, block, 0, s>>>(a);                \
  } while (0)
  if (a.head_dim == 128) {
    if (a.q_bf16) { if (paged) DFX_ATTN_LAUNCH(attn_mfma_kernel, 128, true); else DFX_ATTN_LAUNCH(attn_mfma_kernel, 128, false); }
    else { if (paged) DFX_ATTN_LAUNCH(attn_mfma_f32q_kernel, 128, true); else DFX_ATTN_LAUNCH(attn_mfma_f32q_kernel, 128, false); }
  } else {
    if (a.q_bf16) { if (paged) DFX_ATTN_LAUNCH(attn_mfma_kernel, 64, true); else DFX_ATTN_LAUNCH(attn_mfma_kernel, 64, false); }
    else { if (paged) DFX_ATTN_LAUNCH(attn_mfma_f32q_kernel, 64, true); else DFX_ATTN_LAUNCH(attn_mfma_f32q_kernel, 64, false); }
  }
#undef DFX_ATTN_LAUNCH
  return hipGetLastError();
}

// ---- split merge: O = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M), lse = M + log2 sum
// One wave per output row. With up to kMergeBatch splits every partial of the row is loaded
// in one round trip (indices past the last split re-read it and are masked), together with
// the context length that decides how many splits hold data; more splits take the same sums
// in two passes. Either way M is the max over the valid splits and the sums run in split
// order, so the arithmetic does not depend on the path taken.
constexpr int kMergeBatch = 8;

template <int D>
__global__ void __launch_bounds__(256) attn_merge_kernel(AttnArgs p) {
  constexpr int PER = D / 64;
  const int rows = p.n_flows * p.batch * p.num_q_heads;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int Hq = p.num_q_heads;
  const int h = row % Hq, b = (row / Hq) % p.batch, f = row / (Hq * p.batch);
  const int64_t stride = (int64_t)p.n_flows * p.batch * Hq;  // rows per split
  const int S = p.num_splits;
  float M = -INFINITY, L = 0.f, O[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) O[k] = 0.f;
  int nvalid;
  if (S <= kMergeBatch) {
    float lse[kMergeBatch], po[kMergeBatch][PER];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int64_t r = (int64_t)min(u, S - 1) * stride + row;
      lse[u] = p.part_lse[r];
#pragma unroll
      for (int k = 0; k < PER; ++k) po[u][k] = p.part_o[r * D + lane + 64 * k];
    }
    const int ctx = min(max(p.ctx[b], 0), p.max_context);
    nvalid = min((ctx + p.chunk - 1) / p.chunk, S);
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      if (u < nvalid) M = fmaxf(M, lse[u]);
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      if (u < nvalid) {
        const float c = exp2f(lse[u] - M);
        L += c;
#pragma unroll
        for (int k = 0; k < PER; ++k) O[k] += c * po[u][k];
      }
  } else {
    const int ctx = min(max(p.ctx[b], 0), p.max_context);
    nvalid = min((ctx + p.chunk - 1) / p.chunk, S);
    for (int s = 0; s < nvalid; ++s) M = fmaxf(M, p.part_lse[s * stride + row]);
    for (int s = 0; s < nvalid; ++s) {
      const float c = exp2f(p.part_lse[s * stride + row] - M);
      L += c;
      const float *po = p.part_o + (s * stride + row) * D;
#pragma unroll
      for (int k = 0; k < PER; ++k) O[k] += c * po[lane + 64 * k];
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const float o = nvalid ? O[k] / L : 0.f;
    int64_t oi;
    float *out = attn_out(p, f, b, h * D + lane + 64 * k, &oi);
    if (p.o_bf16) ((uint16_t *)out)[oi] = (uint16_t)f32_to_bf16_rne(o);
    else out[oi] = o;
  }
  if (lane == 0 && p.lse)
    p.lse[((int64_t)f * p.batch + b) * Hq + h] = nvalid ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

hipError_t launch_attn_merge(const AttnArgs &a, hipStream_t s) {
  const int rows = a.n_flows * a.batch * a.num_q_heads;
  const dim3 grid((rows + 3) / 4), block(256);
  if (a.head_dim == 128) attn_merge_kernel<128><<<grid, block, 0, s>>>(a);
  else attn_merge_kernel<64><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dfx
