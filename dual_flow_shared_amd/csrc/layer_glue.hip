// Layer-internal kernels that finish the K-split projections of the decode layer (Q/K/V,
// output, down; the gate/up projection finishes in its own epilogue): they
// sum the K-split fp32 tiles of the projection in split order and apply the glue that
// follows it, so no separate reduction pass, norm or activation pass touches HBM.
//
// Tiles are [ksplit][groups][64 rows][N]; row q of a group is flow q / (64 / F), batch
// row grp * (64 / F) + q % (64 / F) (the layout the grouped linear writes).
#include "common.h"

namespace dfx {

// The split tiles of one (flow, row, 4 columns), in two phases so that a kernel can issue all
// of its loads before the first one is waited for: load_tiles issues U loads (indices past
// the last split re-read it), add_tiles sums the first ksplit in split order, starting from
// zero: the arithmetic of sum_split_tiles, so the results are the same bits.
template <int U>
__device__ __forceinline__ void load_tiles(f32x4 (&t)[U], const LayerGlueArgs &a, int groups, int N, int f,
                                           int b, int rpg, int col) {
  const int grp = b / rpg, q = f * rpg + b % rpg;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = min(u, a.ksplit - 1);
    t[u] = *(const f32x4 *)(a.tiles + (((int64_t)k * groups + grp) * 64 + q) * N + col);
  }
}

template <int U>
__device__ __forceinline__ f32x4 add_tiles(const f32x4 (&t)[U], int ksplit) {
  f32x4 s{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (u < ksplit) s += t[u];
  return s;
}

// Q columns of both flows -> qkv rows (fp32); K and V columns of flow 0 -> the cache at
// position min(max(context_lens[b], 1), max_context) - 1 as bf16 (the auxiliary flow's K/V
// columns are dropped: only the primary flow writes the cache). One thread per 4 columns of
// one (flow, row). Two memory round trips: the context length, then the block id of the
// append position together with every split tile.
template <int U>
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
  const dfx_kv_cache &kv = a.kv;
  const bool paged = kv.block_table != nullptr;
  // the attention of this step reads positions [0, min(max(ctx, 0), max_context)); the new
  // row goes to the last of them (max_context <= capacity, checked on the host). Its block
  // id is loaded by every thread of the row (a Q column discards it; a contiguous cache
  // re-reads the length) together with the tiles, so that no branch holds the loads back.
  const int64_t pos = (int64_t)min(max(a.ctx[b], 1), a.max_context) - 1;
  // (a relaxed atomic load: the compiler keeps it here instead of sinking it to its only use)
  const int32_t *ep = paged ? kv.block_table + (int64_t)b * kv.max_blocks_per_seq + pos / kv.block_size : a.ctx + b;
  const uint32_t e = (uint32_t)__hip_atomic_load(ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  f32x4 t[U];
  load_tiles<U>(t, a, groups, N, f, b, rpg, col);
  const f32x4 v = add_tiles<U>(t, a.ksplit);
  if (col < qcols) {
    *(f32x4 *)(a.out + ((int64_t)f * B + b) * N + col) = v;
    return;
  }
  const int kvcols = kv.num_kv_heads * kv.head_dim;
  const int c = col - qcols;
  const bool is_v = c >= kvcols;
  const int cc = is_v ? c - kvcols : c;
  const int g = cc / kv.head_dim, d = cc % kv.head_dim;
  int64_t blk, slot;
  if (paged) {
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
// (flow, row); its slices (norm_scale) are held in registers. A slice's residual, gain and
// split tiles are all loaded before the first wait (one memory round trip per slice).
template <int U>
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
      const f32x4 xv = *(const f32x4 *)(xr + 4 * i);
      gg[u] = *(const f32x4 *)(a.gain + 4 * i);
      f32x4 t[U];
      load_tiles<U>(t, a, groups, N, f, b, rpg, 4 * i);
      v[u] = add_tiles<U>(t, a.ksplit) + xv;
      *(f32x4 *)(xr + 4 * i) = v[u];
    }
  }
  const float r = norm_scale(v, N, a.eps, red);
  norm_store(v, gg, r, N, a.h, F, f, b, row);
}

// The last projection of a layer finishing into the next layer: m = summed W_down tiles,
// flow 1 += c * flow 0, x += m (in place), then the next layer's h1 = bf16(rmsnorm(x) *
// gain) in W_qkv's fragment order. The same arithmetic, in the same order, as down_finish
// followed by the RMSNorm kernel. One work-group of 1024 threads per (flow, row); a slice's
// loads (residual, gain, coupling, both flows' tiles) are all issued before the first wait.
template <int U>
__global__ void __launch_bounds__(1024) down_finish_norm_kernel(LayerGlueArgs a) {
  __shared__ float red[16];
  const int F = a.n_flows, B = a.batch, N = a.N;
  const int rpg = 64 / F, groups = (B + rpg - 1) / rpg;
  const int row = blockIdx.x, f = row / B, b = row % B;
  const bool coupled = f == 1 && a.couple;
  float *xr = a.x + (int64_t)row * N;
  const int n4 = N / 4;
  f32x4 v[kNormSlices], gg[kNormSlices];
#pragma unroll
  for (int u = 0; u < kNormSlices; ++u) {
    const int i = threadIdx.x + 1024 * u;
    v[u] = gg[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < n4) {
      const int col = 4 * i;
      const f32x4 xv = *(const f32x4 *)(xr + col);
      gg[u] = *(const f32x4 *)(a.gain + col);
      f32x4 t[U], tp[U], c{0.f, 0.f, 0.f, 0.f};
      load_tiles<U>(t, a, groups, N, f, b, rpg, col);
      if (coupled) {
        c = *(const f32x4 *)(a.couple + col);
        // both flows' tiles in one round trip up to 8 splits; beyond, two (registers)
        if constexpr (U <= 8) load_tiles<U>(tp, a, groups, N, 0, b, rpg, col);
      }
      f32x4 m = add_tiles<U>(t, a.ksplit);
      if (coupled) {
        if constexpr (U > 8) load_tiles<U>(tp, a, groups, N, 0, b, rpg, col);
        const f32x4 prim = add_tiles<U>(tp, a.ksplit);
        m = f32x4{fmaf(c[0], prim[0], m[0]), fmaf(c[1], prim[1], m[1]), fmaf(c[2], prim[2], m[2]),
                  fmaf(c[3], prim[3], m[3])};
      }
      v[u] = xv + m;
      *(f32x4 *)(xr + col) = v[u];
    }
  }
  const float r = norm_scale(v, N, a.eps, red);
  norm_store(v, gg, r, N, a.h, F, f, b, row);
}

// m = summed W_down tiles; flow 1 += c * flow 0; x += m (in place). One thread per 4
// columns of one row index (both flows); every load (both flows' tiles and residuals, the
// coupling) is issued before the first wait.
template <int U>
__global__ void __launch_bounds__(256) down_finish_kernel(LayerGlueArgs a) {
  const int F = a.n_flows, B = a.batch, N = a.N;
  const int rpg = 64 / F, groups = (B + rpg - 1) / rpg;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int n4 = N / 4;
  if (idx >= (int64_t)B * n4) return;
  const int col = (int)(idx % n4) * 4, b = (int)(idx / n4);
  float *x0 = a.x + (int64_t)b * N + col, *x1 = a.x + ((int64_t)B + b) * N + col;
  const f32x4 xv0 = *(const f32x4 *)x0;
  f32x4 t0[U], t1[U], xv1{0.f, 0.f, 0.f, 0.f}, c{0.f, 0.f, 0.f, 0.f};
  load_tiles<U>(t0, a, groups, N, 0, b, rpg, col);
  if (F == 2) {
    xv1 = *(const f32x4 *)x1;
    // read unconditionally (any valid row when there is no coupling, then unused), so that no
    // branch makes the compiler wait for the loads before it
    c = *(const f32x4 *)((a.couple ? a.couple : a.tiles) + col);
    load_tiles<U>(t1, a, groups, N, 1, b, rpg, col);
  }
  const f32x4 prim = add_tiles<U>(t0, a.ksplit);
  *(f32x4 *)x0 = xv0 + prim;
  if (F == 2) {
    f32x4 m = add_tiles<U>(t1, a.ksplit);
    if (a.couple)
      m = f32x4{fmaf(c[0], prim[0], m[0]), fmaf(c[1], prim[1], m[1]), fmaf(c[2], prim[2], m[2]),
                fmaf(c[3], prim[3], m[3])};
    *(f32x4 *)x1 = xv1 + m;
  }
}

template <int U>
static void launch_glue(int which, const LayerGlueArgs &a, hipStream_t s) {
  const int F = a.n_flows, B = a.batch;
  int64_t threads = 0;
  switch (which) {
    case kGlueQkv:
      threads = (int64_t)F * B * (a.N / 4);
      qkv_finish_kernel<U><<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(a);
      break;
    case kGlueONorm:
      o_finish_norm_kernel<U><<<F * B, 1024, 0, s>>>(a);
      break;
    case kGlueDownNorm:
      down_finish_norm_kernel<U><<<F * B, 1024, 0, s>>>(a);
      break;
    default:
      threads = (int64_t)B * (a.N / 4);
      down_finish_kernel<U><<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(a);
      break;
  }
}

hipError_t launch_layer_glue(int which, const LayerGlueArgs &a, hipStream_t s) {
  // one round of tile loads covers the split count (the projection plans at most 16 splits)
  if (a.ksplit < 1 || a.ksplit > 16) return hipErrorInvalidValue;
  if (a.ksplit <= 8) launch_glue<8>(which, a, s);
  else launch_glue<16>(which, a, s);
  return hipGetLastError();
}

}  // namespace dfx
