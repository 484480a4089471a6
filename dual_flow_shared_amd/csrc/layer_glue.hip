// Layer-internal kernels that finish the K-split projections of the decode layer (Q/K/V,
// output, down; the gate/up projection finishes in its own epilogue): they
// sum the K-split fp32 tiles of the projection in split order and apply the glue that
// follows it, so no separate reduction pass, norm or activation pass touches HBM.
//
// Tiles are [ksplit][groups][64 rows][N]; row q of a group is flow q / (64 / F), batch
// row grp * (64 / F) + q % (64 / F) (the layout the grouped linear writes).
#include "common.h"

namespace dfx {

__device__ __forceinline__ f32x4 sum_tiles(const float *tiles, int ksplit, int groups, int N,
                                           int f, int rr, int rpg, int col) {
  return sum_split_tiles(tiles, ksplit, groups, N, rr / rpg, f * rpg + rr % rpg, col);
}

// Q columns of both flows -> qkv rows (fp32); K and V columns of flow 0 -> the cache at
// position min(max(context_lens[b], 1), max_context) - 1 as bf16 (the auxiliary flow's K/V columns are dropped: only
// the primary flow writes the cache). One thread per 4 columns of one (flow, row).
__global__ void __launch_bounds__(256) qkv_finish_kernel(LayerGlueArgs a) {
  const int F = a.n_flows, B = a.batch, N = a.N;
  const int rpg = 64 / F, groups = (B + rpg - 1) / rpg;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int n4 = N / 4;
  if (idx >= (int64_t)F * B * n4) return;
  const int col = (int)(idx % n4) * 4;
  const int row = (int)(idx / n4);
  const int f = row / B, b = row % B;
  const int qcols = a.num_q_heads * a.head_dim;
  if (col >= qcols && f != 0) return;
  const f32x4 v = sum_tiles(a.tiles, a.ksplit, groups, N, f, b, rpg, col);
  if (col < qcols) {
    *(f32x4 *)(a.out + ((int64_t)f * B + b) * N + col) = v;
    return;
  }
  const dfx_kv_cache &kv = a.kv;
  const int kvcols = kv.num_kv_heads * kv.head_dim;
  const int c = col - qcols;
  const bool is_v = c >= kvcols;
  const int cc = is_v ? c - kvcols : c;
  const int g = cc / kv.head_dim, d = cc % kv.head_dim;
  const bool paged = kv.block_table != nullptr;
  // the attention of this step reads positions [0, min(max(ctx, 0), max_context)); the new
  // row goes to the last of them (max_context <= capacity, checked on the host)
  const int64_t pos = (int64_t)min(max(a.ctx[b], 1), a.max_context) - 1;
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

// x += sum of the W_o tiles (in place), then h = bf16(rmsnorm(x) * gain) in the fragment
// order of the next projection (xpack_offset). One work-group of 1024 threads per
// (flow, row); its slices (norm_scale) are held in registers, and every load (tiles,
// residual, gain) is issued before the reduction.
__global__ void __launch_bounds__(1024) o_finish_norm_kernel(LayerGlueArgs a) {
  __shared__ float red[16];
  const int F = a.n_flows, B = a.batch, N = a.N;
  const int rpg = 64 / F, groups = (B + rpg - 1) / rpg;
  const int row = blockIdx.x, f = row / B, b = row % B;
  float *xr = a.x + (int64_t)row * N;
  const int n4 = N / 4;
  f32x4 v[kNormSlices], gg[kNormSlices];
#pragma unroll
  for (int u = 0; u < kNormSlices; ++u) {
    const int i = threadIdx.x + 1024 * u;
    v[u] = gg[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < n4) {
      v[u] = sum_tiles(a.tiles, a.ksplit, groups, N, f, b, rpg, 4 * i) + *(const f32x4 *)(xr + 4 * i);
      gg[u] = *(const f32x4 *)(a.gain + 4 * i);
      *(f32x4 *)(xr + 4 * i) = v[u];
    }
  }
  const float r = norm_scale(v, N, a.eps, red);
  norm_store(v, gg, r, N, a.h, F, f, b, row);
}

// The last projection of a layer finishing into the next layer: m = summed W_down tiles,
// flow 1 += c * flow 0, x += m (in place), then the next layer's h1 = bf16(rmsnorm(x) *
// gain) in W_qkv's fragment order. The same arithmetic, in the same order, as down_finish
// followed by the RMSNorm kernel. One work-group of 1024 threads per (flow, row).
__global__ void __launch_bounds__(1024) down_finish_norm_kernel(LayerGlueArgs a) {
  __shared__ float red[16];
  const int F = a.n_flows, B = a.batch, N = a.N;
  const int rpg = 64 / F, groups = (B + rpg - 1) / rpg;
  const int row = blockIdx.x, f = row / B, b = row % B;
  float *xr = a.x + (int64_t)row * N;
  const int n4 = N / 4;
  f32x4 v[kNormSlices], gg[kNormSlices];
#pragma unroll
  for (int u = 0; u < kNormSlices; ++u) {
    const int i = threadIdx.x + 1024 * u;
    v[u] = gg[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < n4) {
      const int col = 4 * i;
      f32x4 m = sum_tiles(a.tiles, a.ksplit, groups, N, f, b, rpg, col);
      if (f == 1 && a.couple) {
        const f32x4 prim = sum_tiles(a.tiles, a.ksplit, groups, N, 0, b, rpg, col);
        const f32x4 c = *(const f32x4 *)(a.couple + col);
        m = f32x4{fmaf(c[0], prim[0], m[0]), fmaf(c[1], prim[1], m[1]), fmaf(c[2], prim[2], m[2]),
                  fmaf(c[3], prim[3], m[3])};
      }
      v[u] = *(const f32x4 *)(xr + col) + m;
      gg[u] = *(const f32x4 *)(a.gain + col);
      *(f32x4 *)(xr + col) = v[u];
    }
  }
  const float r = norm_scale(v, N, a.eps, red);
  norm_store(v, gg, r, N, a.h, F, f, b, row);
}

// m = summed W_down tiles; flow 1 += c * flow 0; x += m (in place). One thread per 4
// columns of one row index (both flows).
__global__ void __launch_bounds__(256) down_finish_kernel(LayerGlueArgs a) {
  const int F = a.n_flows, B = a.batch, N = a.N;
  const int rpg = 64 / F, groups = (B + rpg - 1) / rpg;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int n4 = N / 4;
  if (idx >= (int64_t)B * n4) return;
  const int col = (int)(idx % n4) * 4, b = (int)(idx / n4);
  f32x4 prim;
  for (int f = 0; f < F; ++f) {
    f32x4 m = sum_tiles(a.tiles, a.ksplit, groups, N, f, b, rpg, col);
    if (f == 0) prim = m;
    else if (a.couple) {
      const f32x4 c = *(const f32x4 *)(a.couple + col);
      m = f32x4{fmaf(c[0], prim[0], m[0]), fmaf(c[1], prim[1], m[1]), fmaf(c[2], prim[2], m[2]),
                fmaf(c[3], prim[3], m[3])};
    }
    float *xr = a.x + ((int64_t)f * B + b) * N + col;
    *(f32x4 *)xr = *(const f32x4 *)xr + m;
  }
}

hipError_t launch_layer_glue(int which, const LayerGlueArgs &a, hipStream_t s) {
  const int F = a.n_flows, B = a.batch;
  int64_t threads = 0;
  switch (which) {
    case kGlueQkv:
      threads = (int64_t)F * B * (a.N / 4);
      qkv_finish_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(a);
      break;
    case kGlueONorm:
      o_finish_norm_kernel<<<F * B, 1024, 0, s>>>(a);
      break;
    case kGlueDownNorm:
      down_finish_norm_kernel<<<F * B, 1024, 0, s>>>(a);
      break;
    default:
      threads = (int64_t)B * (a.N / 4);
      down_finish_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(a);
      break;
  }
  return hipGetLastError();
}

}  // namespace dfx
