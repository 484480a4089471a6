// Grouped shared-weight linear on gfx950 matrix cores: Y[f] = bf16(X[f]) W^T for every
// flow in one pass over W.
//
// Both flows apply the same matrices (Sintesi Tecnica: Dual-Flow Transformers,
// "Architettura Core"), so every weight fragment fetched from HBM is multiplied into
// the rows of both flows before it is dropped; the decode step reads no extra unique
// weights ("Costi di Inferenza vs. Addestramento").
//
// A work-group owns NT output features and a K range; it computes the tile
// C = W[NT][K] . X^T[K][64 rows] with 16x16x32 bf16 MFMAs (A = W rows, B = X rows, fp32
// accumulate). Its four waves take interleaved 32-wide k-steps and their partial tiles
// are summed in LDS in wave order. When the grid splits K over several work-groups the
// tiles go to a workspace and the last work-group to arrive (per-tile counter) sums them
// in split order and runs the epilogue, so every output's reduction order is fixed and
// does not depend on how many rows or flows share the call. Rows are taken in groups of
// 64: 64 / n_flows consecutive rows of each flow, so a flow-1 row and its flow-0 partner
// (for the coupling epilogue) always sit in the same group.
#include "common.h"

namespace dfx {

template <int NT, bool XF32>
__global__ void __launch_bounds__(256) grouped_linear_kernel(GemmArgs p) {
  constexpr int MB = NT / 16;
  __shared__ float red[4][NT][65];
  __shared__ uint32_t s_last;

  const int tile = blockIdx.x, ks = blockIdx.y;
  const int tiles = gridDim.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;
  const int F = p.n_flows, rows = p.rows, K = p.K, N = p.N;
  const int rpg = 64 / F;  // rows of each flow in one group
  const int groups = (rows + rpg - 1) / rpg;
  const int nks = K / 32;
  const int kbeg = (int)((int64_t)ks * nks / p.ksplit), kend = (int)((int64_t)(ks + 1) * nks / p.ksplit);
  const int n0 = tile * NT;

  for (int grp = 0; grp < groups; ++grp) {
    // B operand rows q = 16 nb + n of this group
    int64_t xoff[4];
    bool xok[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int q = 16 * nb + n, f = q / rpg, rr = grp * rpg + q % rpg;
      xok[nb] = f < F && rr < rows;
      xoff[nb] = xok[nb] ? ((int64_t)f * rows + rr) * K : 0;
    }
    f32x4 acc[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};


    for (int kk = kbeg + wave; kk < kend; kk += 4) {
      const int k0 = kk * 32 + 8 * j;
      u32x4 af[MB], bfr[4];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        af[mb] = *(const u32x4 *)(p.w + (int64_t)(n0 + 16 * mb + n) * K + k0);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        if (!xok[nb]) {
          bfr[nb] = u32x4{0u, 0u, 0u, 0u};
        } else if constexpr (XF32) {
          const float *xs = (const float *)p.x + xoff[nb] + k0;
          const f32x4 a = *(const f32x4 *)xs, c = *(const f32x4 *)(xs + 4);
          bfr[nb] = u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                          pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3])};
        } else {
          bfr[nb] = *(const u32x4 *)((const uint16_t *)p.x + xoff[nb] + k0);
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = mfma16x16x32(as_bf16x8(af[mb]), as_bf16x8(bfr[nb]), acc[mb][nb]);
    }

    // C layout: lane holds row q = 16 nb + n, features 16 mb + 4 j + i
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][16 * mb + 4 * j + i][16 * nb + n] = acc[mb][nb][i];
    __syncthreads();
    for (int e = threadIdx.x; e < NT * 64; e += 256) {
      const int fl = e / 64, q = e % 64;
      red[0][fl][q] = ((red[0][fl][q] + red[1][fl][q]) + red[2][fl][q]) + red[3][fl][q];
    }
    __syncthreads();

    if (p.ksplit > 1) {
      float *mine = p.partial + (((int64_t)ks * groups + grp) * tiles + tile) * (64 * NT);
      for (int e = threadIdx.x; e < NT * 64; e += 256) mine[e] = red[0][e / 64][e % 64];
      __threadfence();
      __syncthreads();
      if (threadIdx.x == 0) s_last = atomicAdd(&p.counters[grp * tiles + tile], 1u);
      __syncthreads();
      if (s_last != (uint32_t)(p.ksplit - 1)) continue;  // uniform: another work-group finishes
      __threadfence();
      for (int e = threadIdx.x; e < NT * 64; e += 256) {
        float s = 0.f;
        for (int k2 = 0; k2 < p.ksplit; ++k2)
          s += __hip_atomic_load(p.partial + (((int64_t)k2 * groups + grp) * tiles + tile) * (64 * NT) + e,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        red[0][e / 64][e % 64] = s;
      }
      if (threadIdx.x == 0) p.counters[grp * tiles + tile] = 0u;  // ready for the next call
      __syncthreads();
    }

    // epilogue: coupling (aux row += couple * primary row), residual, store
    for (int e = threadIdx.x; e < 64 * (NT / 4); e += 256) {
      const int q = e / (NT / 4), c4 = (e % (NT / 4)) * 4;
      const int f = q / rpg, rr = grp * rpg + q % rpg;
      if (f >= F || rr >= rows) continue;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = red[0][c4 + i][q];
      if (f == 1 && p.couple) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = fmaf(p.couple[n0 + c4 + i], red[0][c4 + i][q - rpg], v[i]);
      }
      const int64_t o = ((int64_t)f * rows + rr) * N + n0 + c4;
      if (p.residual) {
        const f32x4 r = *(const f32x4 *)(p.residual + o);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += r[i];
      }
      if (p.y_bf16) *(u32x2 *)((uint16_t *)p.y + o) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      else *(f32x4 *)((float *)p.y + o) = f32x4{v[0], v[1], v[2], v[3]};
    }
    __syncthreads();
  }
}

hipError_t launch_grouped_linear(const GemmArgs &g, int nt, hipStream_t s) {
  const dim3 grid(g.N / nt, g.ksplit), block(256);
  if (nt == 64) {
    if (g.x_f32) grouped_linear_kernel<64, true><<<grid, block, 0, s>>>(g);
    else grouped_linear_kernel<64, false><<<grid, block, 0, s>>>(g);
  } else if (nt == 32) {
    if (g.x_f32) grouped_linear_kernel<32, true><<<grid, block, 0, s>>>(g);
    else grouped_linear_kernel<32, false><<<grid, block, 0, s>>>(g);
  } else {
    if (g.x_f32) grouped_linear_kernel<16, true><<<grid, block, 0, s>>>(g);
    else grouped_linear_kernel<16, false><<<grid, block, 0, s>>>(g);
  }
  return hipGetLastError();
}

}  // namespace dfx
