// Grouped shared-weight linear on gfx950 matrix cores: Y[f] = bf16(X[f]) W^T for every
// flow in one pass over W.
//
// Both flows apply the same matrices (Sintesi Tecnica: Dual-Flow Transformers,
// "Architettura Core"), so every weight fragment fetched from HBM is multiplied into
// the rows of both flows before it is dropped; the decode step reads no extra unique
// weights ("Costi di Inferenza vs. Addestramento").
//
// Each wave owns 16 output features and streams their weight rows over its K range with a
// ring of kPipeW k-steps of 32 in flight; the four waves of a work-group cover 64
// adjacent features and read the same X fragments (served by the CU's L1 after the first
// wave). Per k-step a wave computes C[16 features][64 rows] += W[16][32] . X^T[32][64]
// with four 16x16x32 bf16 MFMAs (A = W rows, B = X rows, fp32 accumulate). Rows are taken
// in groups of 64: 64 / n_flows consecutive rows of each flow, so a flow-1 row and its
// flow-0 partner are 32 rows apart and sit in the same lane for the coupling epilogue.
//
// When K is split over several work-groups each writes its fp32 tile to a workspace and a
// second kernel sums the splits in split order before the epilogue; either way the
// reduction order of an output element depends only on (K, N), never on rows or flows.
#include "common.h"

namespace dfx {

#ifndef DFX_GEMM_PIPE
#define DFX_GEMM_PIPE 8
#endif
constexpr int kPipeW = DFX_GEMM_PIPE;  // k-steps of weight fragments in flight per wave
// Experiment switch for measuring what limits the kernel (0 in the library):
// 1 = X rows padded to K + 64 elements, 2 = every X row read from row 0, 3 = no X loads.
#ifndef DFX_GEMM_XMODE
#define DFX_GEMM_XMODE 0
#endif
#ifndef DFX_GEMM_PIPE_X
#define DFX_GEMM_PIPE_X 4
#endif
constexpr int kPipeX = DFX_GEMM_PIPE_X;  // k-steps of row fragments in flight per wave

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
  __device__ __forceinline__ u32x4 bf16() const { return v; }
};

template <>
struct XFrag<true> {
  f32x4 a, c;
  __device__ __forceinline__ void load(const void *x, int64_t off) {
    a = *(const f32x4 *)((const float *)x + off);
    c = *(const f32x4 *)((const float *)x + off + 4);
  }
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

template <bool XF32, bool PACKED>
__global__ void __launch_bounds__(256) grouped_linear_kernel(GemmArgs p) {
  const int tile = blockIdx.x, ks = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;
  const int F = p.n_flows, rows = p.rows, K = p.K, N = p.N;
  const int rpg = 64 / F;  // rows of each flow in one group
  const int groups = (rows + rpg - 1) / rpg;
  const int nks = K / 32;
  const int kbeg = (int)((int64_t)ks * nks / p.ksplit), kend = (int)((int64_t)(ks + 1) * nks / p.ksplit);
  const int col0 = tile * 64 + wave * 16;  // this wave's features
  if (col0 >= N) return;                   // N is a multiple of 16, not always of 64
  // weight fragment of k-step kk for this lane: wrow + kk * wstep
  const uint16_t *wrow;
  int64_t wstep;
  if constexpr (PACKED) {  // [N/16][K/32][64 lanes][8]: one contiguous KiB per k-step
    wrow = p.w + ((int64_t)(col0 / 16) * nks * 64 + lane) * 8;
    wstep = 512;
  } else {                 // row-major: 64 B of each of 16 rows per k-step
    wrow = p.w + (int64_t)(col0 + n) * K + 8 * j;
    wstep = 32;
  }

  for (int grp = 0; grp < groups; ++grp) {
    // B operand rows q = 16 nb + n of this group; a row past the batch reads row 0 instead
    // (its output columns are never stored), so no load is conditional
    int64_t xoff[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int q = 16 * nb + n, f = q / rpg, rr = grp * rpg + q % rpg;
      const bool ok = f < F && rr < rows;
      const int64_t xs = DFX_GEMM_XMODE == 1 ? K + 64 : K;
      xoff[nb] = (ok && DFX_GEMM_XMODE != 2 ? ((int64_t)f * rows + rr) * xs : 0) + 8 * j;
    }
    f32x4 acc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // rings: weight fragments kPipeW k-steps ahead, row fragments kPipeX ahead (fp32 rows
    // are kept raw and rounded to bf16 when used)
    u32x4 wf[kPipeW];
    XFrag<XF32> xf[kPipeX][4];
    auto load_x = [&](int kk, XFrag<XF32> *bx) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        if constexpr (DFX_GEMM_XMODE == 3) bx[nb] = XFrag<XF32>{};
        else bx[nb].load(p.x, xoff[nb] + kk * 32);
      }
    };
    auto step = [&](const u32x4 &w, const XFrag<XF32> *bx) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[nb] = mfma16x16x32(as_bf16x8(w), as_bf16x8(bx[nb].bf16()), acc[nb]);
    };
    const int nk = kend - kbeg;
#pragma unroll
    for (int u = 0; u < kPipeW; ++u)
      if (u < nk) wf[u] = *(const u32x4 *)(wrow + (kbeg + u) * wstep);
#pragma unroll
    for (int u = 0; u < kPipeX; ++u)
      if (u < nk) load_x(kbeg + u, xf[u]);
    int base = kbeg;
    // steady state: every refill lands inside [kbeg, kend), no conditional loads
    for (; base + 2 * kPipeW <= kend; base += kPipeW) {
#pragma unroll
      for (int u = 0; u < kPipeW; ++u) {
        step(wf[u], xf[u % kPipeX]);
        wf[u] = *(const u32x4 *)(wrow + (base + u + kPipeW) * wstep);
        load_x(base + u + kPipeX, xf[u % kPipeX]);
      }
    }
    // tail: fewer than 2 * kPipeW k-steps remain; slot u % kPipeW holds k-step base + u
#pragma unroll
    for (int u = 0; u < 2 * kPipeW; ++u) {
      const int kk = base + u;
      if (kk < kend) {
        step(wf[u % kPipeW], xf[u % kPipeX]);
        if (kk + kPipeW < kend) wf[u % kPipeW] = *(const u32x4 *)(wrow + (kk + kPipeW) * wstep);
        if (kk + kPipeX < kend) load_x(kk + kPipeX, xf[u % kPipeX]);
      }
    }

    // C layout: lane holds row q = 16 nb + n and features col0 + 4 j + i
    const int col = col0 + 4 * j;
    if (p.ksplit > 1 || p.tiles_only) {
      // partial tile [ks][grp][64 rows][N]
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        float *dst = p.partial + (((int64_t)ks * groups + grp) * 64 + 16 * nb + n) * N + col;
        *(f32x4 *)dst = acc[nb];
      }
      continue;
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int q = 16 * nb + n, f = q / rpg, rr = grp * rpg + q % rpg;
      if (f >= F || rr >= rows) continue;
      float v[4] = {acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]};
      float prim[4] = {0.f, 0.f, 0.f, 0.f};
      if (f == 1) {
        // the flow-0 partner row q - 32 is block nb - 2 in this same lane
#pragma unroll
        for (int i = 0; i < 4; ++i) prim[i] = acc[nb >= 2 ? nb - 2 : 0][i];
      }
      epilogue4(p, f, rr, col, v, prim);
    }
  }
}

// Fast path for K-slices that are whole 256-column chunks. The 64 rows x 256 columns of X
// for a chunk are staged in LDS once per work-group (each load instruction reads 512
// contiguous bytes of a row) and shared by the four waves; weight fragments stream
// straight into registers one chunk ahead (two register sets ping-pong), so the weight
// loads and the LDS reads wait on separate counters and the steady state has no
// conditional load.
constexpr int kChunkK = 256;              // columns of X per LDS chunk (8 k-steps)
constexpr int kXPitch = kChunkK + 8;      // bf16 elements per staged row (16 B pad)

template <bool XF32, bool PACKED>
__device__ __forceinline__ void chunk_load_x(const GemmArgs &p, const int64_t *xrow, int c0,
                                             int lane, u32x4 *xr) {
  // instruction i: lanes 0-31 read row 2i, lanes 32-63 row 2i + 1 of this wave's 16 rows
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t off = xrow[i] + c0 + 8 * (lane & 31);
    if constexpr (XF32) {
      const f32x4 a = *(const f32x4 *)((const float *)p.x + off);
      const f32x4 b = *(const f32x4 *)((const float *)p.x + off + 4);
      xr[i] = u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                    pack_bf16x2(b[2], b[3])};
    } else {
      xr[i] = *(const u32x4 *)((const uint16_t *)p.x + off);
    }
  }
}

__device__ __forceinline__ void chunk_stage_x(uint16_t *buf, int wave, int lane, const u32x4 *xr) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 16 * wave + 2 * i + (lane >> 5);
    *(u32x4 *)(buf + row * kXPitch + 8 * (lane & 31)) = xr[i];
  }
}

template <bool PACKED>
__device__ __forceinline__ void chunk_load_w(const uint16_t *wrow, int64_t wstep, int k0, u32x4 *wr) {
#pragma unroll
  for (int s = 0; s < 8; ++s) wr[s] = *(const u32x4 *)(wrow + (int64_t)(k0 + s) * wstep);
}

__device__ __forceinline__ void chunk_compute(const uint16_t *buf, int n, int j, const u32x4 *wr,
                                              f32x4 *acc) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const u32x4 xf = *(const u32x4 *)(buf + (16 * nb + n) * kXPitch + 32 * s + 8 * j);
      acc[nb] = mfma16x16x32(as_bf16x8(wr[s]), as_bf16x8(xf), acc[nb]);
    }
  }
}

template <bool XF32, bool PACKED>
__global__ void __launch_bounds__(256) grouped_linear_chunked_kernel(GemmArgs p) {
  __shared__ uint16_t xs[2][64 * kXPitch];
  const int tile = blockIdx.x, ks = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;
  const int F = p.n_flows, rows = p.rows, K = p.K, N = p.N;
  const int rpg = 64 / F;
  const int groups = (rows + rpg - 1) / rpg;
  const int nks = K / 32;
  // this split's k-steps: whole chunks of 8
  const int nch_all = nks / 8;
  const int per = (nch_all + p.ksplit - 1) / p.ksplit;
  const int kbeg = ks * per * 8;
  const int nch = min(per, nch_all - ks * per);
  const int col0 = tile * 64 + wave * 16;
  const bool wave_live = col0 < N;  // N is a multiple of 16, not always of 64
  const uint16_t *wrow;
  int64_t wstep;
  if constexpr (PACKED) {
    wrow = p.w + ((int64_t)(min(col0, N - 16) / 16) * nks * 64 + lane) * 8;
    wstep = 512;
  } else {
    wrow = p.w + (int64_t)(min(col0, N - 16) + n) * K + 8 * j;
    wstep = 32;
  }

  for (int grp = 0; grp < groups; ++grp) {
    // element offset of the row this lane stages in load instruction i (rows past the batch
    // read row 0: their output columns are never stored)
    int64_t xrow[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = 16 * wave + 2 * i + (lane >> 5);
      const int f = q / rpg, rr = grp * rpg + q % rpg;
      xrow[i] = (f < F && rr < rows) ? ((int64_t)f * rows + rr) * K : 0;
    }
    f32x4 acc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 xr[8], wa[8], wb[8];
    if (nch > 0) {
      chunk_load_x<XF32, PACKED>(p, xrow, kbeg * 32, lane, xr);
      chunk_load_w<PACKED>(wrow, wstep, kbeg, wa);
    }
    int c = 0;
    for (; c + 2 < nch; c += 2) {
      chunk_stage_x(xs[0], wave, lane, xr);
      __syncthreads();
      chunk_load_x<XF32, PACKED>(p, xrow, (kbeg + 8 * (c + 1)) * 32, lane, xr);
      chunk_load_w<PACKED>(wrow, wstep, kbeg + 8 * (c + 1), wb);
      chunk_compute(xs[0], n, j, wa, acc);
      chunk_stage_x(xs[1], wave, lane, xr);
      __syncthreads();
      chunk_load_x<XF32, PACKED>(p, xrow, (kbeg + 8 * (c + 2)) * 32, lane, xr);
      chunk_load_w<PACKED>(wrow, wstep, kbeg + 8 * (c + 2), wa);
      chunk_compute(xs[1], n, j, wb, acc);
    }
    if (c + 1 < nch) {  // two chunks left
      chunk_stage_x(xs[0], wave, lane, xr);
      __syncthreads();
      chunk_load_x<XF32, PACKED>(p, xrow, (kbeg + 8 * (c + 1)) * 32, lane, xr);
      chunk_load_w<PACKED>(wrow, wstep, kbeg + 8 * (c + 1), wb);
      chunk_compute(xs[0], n, j, wa, acc);
      chunk_stage_x(xs[1], wave, lane, xr);
      __syncthreads();
      chunk_compute(xs[1], n, j, wb, acc);
    } else if (c < nch) {  // one chunk left
      chunk_stage_x(xs[0], wave, lane, xr);
      __syncthreads();
      chunk_compute(xs[0], n, j, wa, acc);
    }
    __syncthreads();  // the staging buffers are reused by the next row group

    const int col = col0 + 4 * j;
    if (!wave_live) continue;
    if (p.ksplit > 1 || p.tiles_only) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        float *dst = p.partial + (((int64_t)ks * groups + grp) * 64 + 16 * nb + n) * N + col;
        *(f32x4 *)dst = acc[nb];
      }
      continue;
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int q = 16 * nb + n, f = q / rpg, rr = grp * rpg + q % rpg;
      if (f >= F || rr >= rows) continue;
      float v[4] = {acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]};
      float prim[4] = {0.f, 0.f, 0.f, 0.f};
      if (f == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) prim[i] = acc[nb >= 2 ? nb - 2 : 0][i];
      }
      epilogue4(p, f, rr, col, v, prim);
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
    const int q = f * rpg + qr;
    f32x4 s{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < p.ksplit; ++k)
      s += *(const f32x4 *)(p.partial + (((int64_t)k * groups + grp) * 64 + q) * N + col);
    v[f][0] = s[0]; v[f][1] = s[1]; v[f][2] = s[2]; v[f][3] = s[3];
  }
  for (int f = 0; f < F; ++f) {
    float out[4] = {v[f][0], v[f][1], v[f][2], v[f][3]};
    epilogue4(p, f, rr, col, out, v[0]);
  }
}

hipError_t launch_grouped_linear(const GemmArgs &g, hipStream_t s) {
  const dim3 grid((g.N + 63) / 64, g.ksplit), block(256);
  if (g.K % kChunkK == 0) {
#define DFX_GL_CHUNKED(XF, PK) grouped_linear_chunked_kernel<XF, PK><<<grid, block, 0, s>>>(g)
    if (g.w_packed) { if (g.x_f32) DFX_GL_CHUNKED(true, true); else DFX_GL_CHUNKED(false, true); }
    else { if (g.x_f32) DFX_GL_CHUNKED(true, false); else DFX_GL_CHUNKED(false, false); }
#undef DFX_GL_CHUNKED
  } else if (g.w_packed) {
    if (g.x_f32) grouped_linear_kernel<true, true><<<grid, block, 0, s>>>(g);
    else grouped_linear_kernel<false, true><<<grid, block, 0, s>>>(g);
  } else {
    if (g.x_f32) grouped_linear_kernel<true, false><<<grid, block, 0, s>>>(g);
    else grouped_linear_kernel<false, false><<<grid, block, 0, s>>>(g);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.ksplit == 1 || g.tiles_only) return e;
  const int rpg = 64 / g.n_flows;
  const int groups = (g.rows + rpg - 1) / rpg;
  const int64_t threads = (int64_t)groups * rpg * (g.N / 4);
  grouped_linear_reduce_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(g);
  return hipGetLastError();
}

// DFX_W_PACKED reorder: one thread moves one 16-byte fragment (8 consecutive k of a row).
__global__ void __launch_bounds__(256) pack_weight_kernel(int32_t N, int32_t K, const uint16_t *w,
                                                          uint16_t *packed) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // destination fragment
  const int64_t total = (int64_t)N * K / 8;
  if (idx >= total) return;
  const int lane = (int)(idx % 64);
  const int64_t rest = idx / 64;
  const int nks = K / 32;
  const int s = (int)(rest % nks);
  const int64_t t = rest / nks;
  const int64_t row = 16 * t + lane % 16;
  const int64_t col = 32 * (int64_t)s + 8 * (lane / 16);
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
