// Grouped shared-weight linear on gfx950 matrix cores: Y[f] = bf16(X[f]) W^T for every
// flow in one pass over W.
//
// Both flows apply the same matrices (Sintesi Tecnica: Dual-Flow Transformers,
// "Architettura Core"), so every weight fragment fetched from HBM is multiplied into
// the rows of both flows before it is dropped; the decode step reads no extra unique
// weights ("Costi di Inferenza vs. Addestramento").
//
// Decode rows are few (64 per group: 64 / n_flows rows of each flow), so the kernel is a
// weight stream. A work-group owns 128 output features (32 per wave) over one K range; per
// k-step of 32 a wave computes C[32 features][64 rows] += W[32][32] . X^T[32][64] with
// eight 16x16x32 bf16 MFMAs (A = W rows, B = X rows, fp32 accumulate). The 4 KiB of X of a
// k-step is fetched once per work-group (one KiB per wave), staged in LDS in B-operand
// order and read by all four waves; weight fragments stream into registers kPipeW k-steps
// ahead with non-temporal loads, so the weight stream does not evict the shared X from
// L2. Rows are taken in groups of 64 so that a flow-1 row and its flow-0 partner are 32
// rows apart and sit in the same lane for the coupling epilogue.
//
// When K is split over several work-groups each writes its fp32 tile to a workspace and a
// second kernel (or the layer's finish kernel) sums the splits in split order; either way
// the reduction order of an output element depends only on (K, N), never on rows or flows.
//
// Output-head mode (one split, fp32 logits): after storing its tile a work-group also writes
// the softmax statistics of every row over its 128 outputs (max, sum of e^(l - max), and for
// the primary sum of e^(2 (l - max))), which the mixture's apply pass combines; the logits are
// stored non-temporally. Its work-groups hold two 128-output tiles on 8 waves (TW below).
#include "common.h"

namespace dfx {

#ifndef DFX_GEMM_PIPE
#define DFX_GEMM_PIPE 4
#endif
#ifndef DFX_GEMM_PIPE_X
#define DFX_GEMM_PIPE_X 4
#endif
constexpr int kPipeW = DFX_GEMM_PIPE;    // k-steps of weight fragments in flight per wave
constexpr int kPipeX = DFX_GEMM_PIPE_X;  // k-steps of row fragments in flight per wave
constexpr int kUnroll = kPipeW > kPipeX ? kPipeW : kPipeX;
static_assert(kUnroll % 2 == 0 && kUnroll % kPipeW == 0 && kUnroll % kPipeX == 0, "ring sizes");

// One B-operand fragment of 8 row elements: bf16 rows are used as loaded; fp32 rows are
// kept raw in flight and rounded to bf16 (nearest even) when the MFMA consumes them.
template <bool XF32>
struct XFrag;

template <>
struct XFrag<false> {
  u32x4 v;
  __device__ __forceinline__ void load(const void *x, int64_t off) {
    v = *(const u32x4 *)((const uint16_t *)x + off);
  }
  __device__ __forceinline__ void zero() { v = u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ u32x4 bf16() const { return v; }
};

template <>
struct XFrag<true> {
  f32x4 a, c;
  __device__ __forceinline__ void load(const void *x, int64_t off) {
    a = *(const f32x4 *)((const float *)x + off);
    c = *(const f32x4 *)((const float *)x + off + 4);
  }
  __device__ __forceinline__ void zero() { a = c = f32x4{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ u32x4 bf16() const {
    return u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(c[0], c[1]),
                 pack_bf16x2(c[2], c[3])};
  }
};

__device__ __forceinline__ void epilogue4(const GemmArgs &p, int f, int rr, int col, float *v,
                                          const float *prim) {
  if (f == 1 && p.couple) {
    const f32x4 c = *(const f32x4 *)(p.couple + col);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = fmaf(c[i], prim[i], v[i]);
  }
  const int64_t o = ((int64_t)f * p.rows + rr) * p.N + col;
  if (p.residual) {
    const f32x4 r = *(const f32x4 *)(p.residual + o);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += r[i];
  }
  if (p.y_bf16) *(u32x2 *)((uint16_t *)p.y + o) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  else *(f32x4 *)((float *)p.y + o) = f32x4{v[0], v[1], v[2], v[3]};
}

// One k-step of X for a 64-row group, as the B fragments of the 16x16x32 MFMA: block nb,
// lane (n, j) holds row 16 nb + n, columns 8 j .. 8 j + 7 of the step. Reads and writes
// are 16 B per lane at consecutive addresses, so no LDS bank conflicts.
constexpr int kXSlot = 4 * 64;  // u32x4 per slot

// XPACKED: X in the fragment order of xpack_offset (bf16 only). WPACKED: DFX_W_PACKED.
// STATS: output-head mode, the softmax statistics of every (tile, row) after the outputs.
// TW: feature tiles per work-group, each on its own four waves with its own staging ring; the
// tiles of one work-group are dispatched together and share its barriers, so they stream at
// the same pace (two work-groups sharing a CU do not: the one dispatched first takes most of
// the CU's loads and finishes far earlier, measured 64 against 90 us at vocabulary 128256).
template <bool XF32, bool XPACKED, bool WPACKED, bool STATS, int TW = 1>
__global__ void __launch_bounds__(256 * TW) grouped_linear_kernel(GemmArgs p) {
  __shared__ u32x4 xs_all[TW][2][kXSlot];
  int sub = 0;  // this wave's tile of the work-group
  if constexpr (TW > 1) sub = (int)(threadIdx.x >> 8);
  u32x4 (*xs)[kXSlot] = xs_all[TW > 1 ? sub : 0];
  const int wave = TW > 1 ? (int)((threadIdx.x >> 6) & 3) : (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;
  const int F = p.n_flows, K = p.K, N = p.N;
  const int ks = blockIdx.y;
  int tile = TW > 1 ? blockIdx.x * TW + sub : blockIdx.x, gslice = blockIdx.z;
  if (!p.expert_rows && p.group_split > 1) {
    // one-dimensional grid, XCD-grouped: work-group i runs on XCD i % 8, and every group slice
    // of a feature tile goes to the same XCD back to back, so the tile's weights stay in that
    // XCD's L2 while the row groups pass over them
    const int tiles = p.swiglu ? (N / 2 + 63) / 64 : (N + 127) / 128;
    const int xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
    tile = xcd + 8 * (idx / p.group_split);
    gslice = idx % p.group_split;
    if (tile >= tiles) return;
  }
  const int rpg = 64 / F;  // rows of each flow in one group
  int rows = p.rows;
  const void *px = p.x;
  const uint16_t *pw = p.w;
  void *py = p.y;
  float *ppart = p.partial;
  if (p.expert_rows) {
    const int e = blockIdx.z;
    rows = min(p.expert_rows[e], p.max_groups * rpg);
    px = (const uint16_t *)p.x + e * p.x_estride;
    pw = p.w + e * p.w_estride;
    py = (uint16_t *)p.y + e * p.y_estride;
    ppart = p.partial ? p.partial + e * p.p_estride : nullptr;
  }
  const int groups = (rows + rpg - 1) / rpg;
  const int tgroups = p.expert_rows ? p.max_groups : groups;  // group count of the tile layout
  int g_begin = 0, g_end = groups;
  if (!p.expert_rows && p.group_split > 1) {
    const int per = (groups + p.group_split - 1) / p.group_split;
    g_begin = gslice * per;
    g_end = min(groups, g_begin + per);
  }
  const int nks = K / 32, ng = N / 16;
  const int kbeg = ks * p.kper;
  const int nk = min(p.kper, nks - kbeg);  // >= 1: the plan leaves no split empty
  // this wave's two 16-feature groups: cg and cg + 1, or in gate/up mode gate group cg and
  // the matching up group cg + ngh (a dead group streams a live one and stores nothing)
  const int ngh = ng / 2;
  const int cg = p.swiglu ? tile * 4 + wave : 2 * (tile * 4 + wave);
  const int cga = p.swiglu ? min(cg, ngh - 1) : min(cg, ng - 1);
  const int cgb = p.swiglu ? cga + ngh : min(cg + 1, ng - 1);
  // weight fragments of k-step kk of this split: wa + kk * wstep and wb + kk * wstep
  const uint16_t *wa, *wb;
  int64_t wstep;
  if constexpr (WPACKED) {  // [K/32][N/16][64][8]: the column groups of a k-step are adjacent
    wa = pw + (((int64_t)kbeg * ng + cga) * 64 + lane) * 8;
    wb = wa + (int64_t)(cgb - cga) * 512;
    wstep = (int64_t)ng * 512;
  } else {                  // row-major: 64 B of each of 16 rows per k-step
    wa = pw + (int64_t)(16 * cga + n) * K + 8 * j + 32 * kbeg;
    wb = wa + (int64_t)16 * (cgb - cga) * K;
    wstep = 32;
  }

  for (int grp = g_begin; grp < g_end; ++grp) {
    // the row fragment this lane stages: block nb = wave of the k-step, i.e. row
    // q = 16 wave + n of the group (a row past the batch reads row 0 in row-major X; its
    // outputs are never stored)
    int64_t xoff, xstep;
    if constexpr (XPACKED) {
      xoff = (((int64_t)grp * nks + kbeg) * 4 + wave) * 512 + lane * 8;
      xstep = 2048;
    } else {
      const int q = 16 * wave + n, f = q / rpg, rr = grp * rpg + q % rpg;
      xoff = (f < F && rr < rows ? ((int64_t)f * rows + rr) * K : 0) + 8 * j + 32 * kbeg;
      xstep = 32;
    }
    f32x4 acc[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[h][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Rings: weight fragments kPipeW k-steps ahead, raw row fragments kPipeX ahead. Every
    // load is issued unconditionally; a k-step past the split re-reads the split's last
    // one, so no branch guards a load and the compiler's waits stay exact.
    u32x4 wfa[kPipeW], wfb[kPipeW];
    XFrag<XF32> xr[kPipeX];
    u32x4 xf[4];
    auto wload = [&](int kk, u32x4 &da, u32x4 &db) {
      const int64_t o = (int64_t)min(kk, nk - 1) * wstep;
      da = __builtin_nontemporal_load((const u32x4 *)(wa + o));
      db = __builtin_nontemporal_load((const u32x4 *)(wb + o));
    };
    auto xload = [&](int kk, XFrag<XF32> &d) { d.load(px, xoff + (int64_t)min(kk, nk - 1) * xstep); };
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u < kPipeX) xload(u, xr[u]);
      if (u < kPipeW) wload(u, wfa[u], wfb[u]);
    }
    xs[0][wave * 64 + lane] = xr[0].bf16();
    xload(kPipeX, xr[0]);
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) xf[nb] = xs[0][nb * 64 + lane];

    // k-step s = base + u: xf holds X(s), xr[(u + 1) % kPipeX] X(s + 1), wf*[u % kPipeW] W(s)
    for (int base = 0; base < nk; base += kUnroll) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int s = base + u;
        xs[(u + 1) & 1][wave * 64 + lane] = xr[(u + 1) % kPipeX].bf16();
        xload(s + 1 + kPipeX, xr[(u + 1) % kPipeX]);
        // a k-step past the split multiplies zero weights (adds exact zeros)
        const bool live = s < nk;
        const u32x4 z{0u, 0u, 0u, 0u};
        const u32x4 a0 = live ? wfa[u % kPipeW] : z, a1 = live ? wfb[u % kPipeW] : z;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          acc[0][nb] = mfma16x16x32(as_bf16x8(a0), as_bf16x8(xf[nb]), acc[0][nb]);
          acc[1][nb] = mfma16x16x32(as_bf16x8(a1), as_bf16x8(xf[nb]), acc[1][nb]);
        }
        wload(s + kPipeW, wfa[u % kPipeW], wfb[u % kPipeW]);
        __syncthreads();
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) xf[nb] = xs[(u + 1) & 1][nb * 64 + lane];
      }
    }
    __syncthreads();  // the staging slots are reused by the next row group

    // C layout: lane holds row q = 16 nb + n and features 16 (cg + h) + 4 j + i (gate/up
    // mode: gate feature 16 cg + 4 j + i in acc[0], its up feature in acc[1])
    if (p.swiglu) {
      if (cg >= ngh) continue;
      const int I = N / 2, col = 16 * cg + 4 * j;
      f32x4 inter[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) inter[nb][i] = silu(acc[0][nb][i]) * acc[1][nb][i];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int q = 16 * nb + n, f = q / rpg, rr = grp * rpg + q % rpg;
        if (f >= F || rr >= rows) continue;
        f32x4 v = inter[nb];
        if (f == 1 && p.couple) {
          // the flow-0 partner row q - 32 is block nb - 2 in this same lane
          const f32x4 c = *(const f32x4 *)(p.couple + col), pr = inter[nb >= 2 ? nb - 2 : 0];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = fmaf(c[i], pr[i], v[i]);
        }
        *(u32x2 *)((uint16_t *)py + xpack_offset(F, f, rr, col, I)) =
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
      continue;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (cg + h >= ng) continue;
      const int col = 16 * (cg + h) + 4 * j;
      if (p.ksplit > 1 || p.tiles_only) {
        // partial tile [ks][grp][64 rows][N]
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          float *dst = ppart + (((int64_t)ks * tgroups + grp) * 64 + 16 * nb + n) * N + col;
          *(f32x4 *)dst = acc[h][nb];
        }
        continue;
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int q = 16 * nb + n, f = q / rpg, rr = grp * rpg + q % rpg;
        if (f >= F || rr >= rows) continue;
        float v[4] = {acc[h][nb][0], acc[h][nb][1], acc[h][nb][2], acc[h][nb][3]};
        float prim[4] = {0.f, 0.f, 0.f, 0.f};
        if (f == 1) {
          // the flow-0 partner row q - 32 is block nb - 2 in this same lane
#pragma unroll
          for (int i = 0; i < 4; ++i) prim[i] = acc[h][nb >= 2 ? nb - 2 : 0][i];
        }
        if constexpr (STATS) {
          // output-head logits (plain fp32, no coupling or residual): stored non-temporally,
          // so that the ~33 MB of a large vocabulary does not sit dirty in L2 until the
          // kernel ends (measured: 3 us less per head call at vocabulary 128256)
          const int64_t o = ((int64_t)f * rows + rr) * N + col;
          __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, (f32x4 *)((float *)py + o));
        } else {
          epilogue4(p, f, rr, col, v, prim);
        }
      }
    }
    if constexpr (STATS) {
      // Softmax statistics of this tile's outputs, per row: the lane holds 8 of row
      // q = 16 nb + n (features 16 (cg + h) + 4 j + i); a feature group past N is absent.
      // The row's max over the tile, then sum e^(l - max) and sum e^(2 (l - max)): lane
      // values in (h, i) order, then the four lanes j, then the four waves in wave order.
      float *red = (float *)&xs[0][0];  // [3][4 waves][64 rows]; the staging ring is idle here
      float mt[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        float m = -INFINITY;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (cg + h < ng)
#pragma unroll
            for (int i = 0; i < 4; ++i) m = fmaxf(m, acc[h][nb][i]);
        m = fmaxf(m, __shfl_xor(m, 16));
        mt[nb] = fmaxf(m, __shfl_xor(m, 32));
      }
      if (j == 0)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) red[wave * 64 + 16 * nb + n] = mt[nb];
      __syncthreads();
      float sw[4], qw[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int q = 16 * nb + n;
        mt[nb] = fmaxf(fmaxf(red[q], red[64 + q]), fmaxf(red[128 + q], red[192 + q]));
        float sum = 0.f, sq = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (cg + h < ng)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float e = exp_hw(acc[h][nb][i] - mt[nb]);
              sum += e;
              sq = fmaf(e, e, sq);
            }
        sum += __shfl_xor(sum, 16);
        sw[nb] = sum + __shfl_xor(sum, 32);
        sq += __shfl_xor(sq, 16);
        qw[nb] = sq + __shfl_xor(sq, 32);
      }
      if (j == 0)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          red[256 + wave * 64 + 16 * nb + n] = sw[nb];
          red[512 + wave * 64 + 16 * nb + n] = qw[nb];
        }
      __syncthreads();
      if (wave == 0 && j == 0 && tile * kHeadTile < N) {  // a tile past N (TW > 1) has no record
        const int tiles = (N + kHeadTile - 1) / kHeadTile;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int q = 16 * nb + n, f = q / rpg, rr = grp * rpg + q % rpg;
          if (f >= F || rr >= rows) continue;
          float *rec = p.mix_stats + ((int64_t)rr * tiles + tile) * kMixStat + 3 * f;
          rec[0] = mt[nb];
          rec[1] = ((red[256 + q] + red[320 + q]) + red[384 + q]) + red[448 + q];
          if (f == 0) rec[2] = ((red[512 + q] + red[576 + q]) + red[640 + q]) + red[704 + q];
        }
      }
      __syncthreads();  // the ring is staged again by the next row group
    }
  }
}

// Sums the K-split partial tiles in split order, then applies the epilogue. One thread per
// 4 consecutive features of one row index of one group (both flows).
__global__ void __launch_bounds__(256) grouped_linear_reduce_kernel(GemmArgs p) {
  const int F = p.n_flows, rows = p.rows, N = p.N;
  const int rpg = 64 / F;
  const int groups = (rows + rpg - 1) / rpg;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int n4 = N / 4;
  if (idx >= (int64_t)groups * rpg * n4) return;
  const int col = (int)(idx % n4) * 4;
  const int64_t rest = idx / n4;
  const int qr = (int)(rest % rpg), grp = (int)(rest / rpg);
  const int rr = grp * rpg + qr;
  if (rr >= rows) return;
  // rows q = qr (flow 0) and q = qr + 32 (flow 1) of this group, summed in split order
  float v[2][4];
  for (int f = 0; f < F; ++f) {
    const f32x4 s = sum_split_tiles(p.partial, p.ksplit, groups, N, grp, f * rpg + qr, col);
    v[f][0] = s[0]; v[f][1] = s[1]; v[f][2] = s[2]; v[f][3] = s[3];
  }
  for (int f = 0; f < F; ++f) {
    float out[4] = {v[f][0], v[f][1], v[f][2], v[f][3]};
    epilogue4(p, f, rr, col, out, v[0]);
  }
}

hipError_t launch_grouped_linear(const GemmArgs &g, hipStream_t s) {
  const int tiles = g.swiglu ? (g.N / 2 + 63) / 64 : (g.N + 127) / 128;
  const bool gsplit = !g.expert_rows && g.group_split > 1;  // one split, XCD-grouped 1-D grid
  const dim3 grid(gsplit ? 8 * ((tiles + 7) / 8) * g.group_split : tiles, gsplit ? 1 : g.ksplit,
                  g.expert_rows ? g.experts : 1),
      block(256);
#define DFX_GL(XF, XP, WP) grouped_linear_kernel<XF, XP, WP, false><<<grid, block, 0, s>>>(g)
  if (g.mix_stats) {
    // output-head mode: one split, plain fp32 outputs, packed rows and weights
    if (!g.x_packed || !g.w_packed || g.ksplit != 1 || g.tiles_only || g.swiglu || g.expert_rows || g.y_bf16 ||
        g.couple || g.residual)
      return hipErrorInvalidValue;
    // two tiles per work-group: one work-group per CU at a time, both tiles at one pace
    if (gsplit) grouped_linear_kernel<false, true, true, true><<<grid, block, 0, s>>>(g);
    else grouped_linear_kernel<false, true, true, true, 2><<<dim3((tiles + 1) / 2, 1, 1), dim3(512), 0, s>>>(g);
    return hipGetLastError();
  }
  if (g.x_packed) {
    if (g.w_packed) DFX_GL(false, true, true); else DFX_GL(false, true, false);
  } else if (g.x_f32) {
    if (g.w_packed) DFX_GL(true, false, true); else DFX_GL(true, false, false);
  } else {
    if (g.w_packed) DFX_GL(false, false, true); else DFX_GL(false, false, false);
  }
#undef DFX_GL
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.ksplit == 1 || g.tiles_only || g.swiglu || g.expert_rows) return e;
  const int rpg = 64 / g.n_flows;
  const int groups = (g.rows + rpg - 1) / rpg;
  const int64_t threads = (int64_t)groups * rpg * (g.N / 4);
  grouped_linear_reduce_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(g);
  return hipGetLastError();
}

// DFX_W_PACKED reorder: one thread moves one 16-byte fragment (8 consecutive k of a row).
// Destination fragment ((s * N/16 + t) * 64 + l) holds w[16 t + l % 16][32 s + 8 (l / 16) ..].
__global__ void __launch_bounds__(256) pack_weight_kernel(int32_t N, int32_t K, const uint16_t *w,
                                                          uint16_t *packed) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // destination fragment
  const int64_t total = (int64_t)N * K / 8;
  if (idx >= total) return;
  const int lane = (int)(idx % 64);
  const int64_t rest = idx / 64;
  const int ng = N / 16;
  const int t = (int)(rest % ng);
  const int64_t s = rest / ng;
  const int64_t row = 16 * (int64_t)t + lane % 16;
  const int64_t col = 32 * s + 8 * (lane / 16);
  *(u32x4 *)(packed + idx * 8) = *(const u32x4 *)(w + row * K + col);
}

hipError_t launch_pack_weight(int32_t N, int32_t K, const uint16_t *w, uint16_t *packed,
                              hipStream_t s) {
  const int64_t total = (int64_t)N * K / 8;
  if (total == 0) return hipSuccess;
  pack_weight_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(N, K, w, packed);
  return hipGetLastError();
}

}  // namespace dfx
