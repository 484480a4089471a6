// Layer glue: RMSNorm (shared gain, bf16 out), SwiGLU with the MLP-intermediate coupling
// b (bf16 out), and two measurement helpers (plain copy, fill).
#include "common.h"

namespace dfx {

// One work-group of 1024 threads per row; thread t owns float4 slices t, t + 1024, ... of the
// row (norm_scale), held in registers, and its gain slices are loaded up front, so the kernel
// makes one round trip to memory before the reduction.
// packed_flows > 0: row r = f * batch + b is written in the fragment order of xpack_offset.
__global__ void __launch_bounds__(1024) rmsnorm_kernel(int32_t dim, const float *x,
                                                       const float *gain, float eps, uint16_t *y,
                                                       int packed_flows, int batch) {
  __shared__ float red[16];
  const int64_t row = blockIdx.x;
  const f32x4 *xr = (const f32x4 *)(x + row * dim);
  const f32x4 *g4 = (const f32x4 *)gain;
  const int n4 = dim / 4;
  f32x4 v[kNormSlices], gg[kNormSlices];
#pragma unroll
  for (int u = 0; u < kNormSlices; ++u) {
    const int i = threadIdx.x + 1024 * u;
    v[u] = i < n4 ? xr[i] : f32x4{0.f, 0.f, 0.f, 0.f};
    gg[u] = i < n4 ? g4[i] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float r = norm_scale(v, dim, eps, red);
  const int f = packed_flows ? (int)(row / batch) : 0, b = packed_flows ? (int)(row % batch) : 0;
  norm_store(v, gg, r, dim, y, packed_flows, f, b, row);
}

// Embedding gather of both flows (each from its own table) plus the first layer's RMSNorm:
// one work-group of 1024 threads per (flow, sequence) row.
__global__ void __launch_bounds__(1024) embed_norm_kernel(int32_t F, int32_t B, int32_t dim,
                                                          const int32_t *tokens, int32_t vocab,
                                                          const uint16_t *e0, const uint16_t *e1,
                                                          const float *gain, float eps, float *x,
                                                          uint16_t *h1) {
  __shared__ float red[16];
  const int row = blockIdx.x, f = row / B, b = row % B;
  const int tok = min(max(tokens[b], 0), vocab - 1);
  const uint16_t *er = (f == 0 ? e0 : e1) + (int64_t)tok * dim;
  float *xr = x + (int64_t)row * dim;
  const int n4 = dim / 4;
  f32x4 v[kNormSlices], gg[kNormSlices];
#pragma unroll
  for (int u = 0; u < kNormSlices; ++u) {
    const int i = threadIdx.x + 1024 * u;
    v[u] = gg[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < n4) {
      const u32x2 w = *(const u32x2 *)(er + 4 * i);
      v[u] = f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
      gg[u] = *(const f32x4 *)(gain + 4 * i);
      *(f32x4 *)(xr + 4 * i) = v[u];
    }
  }
  const float r = norm_scale(v, dim, eps, red);
  norm_store(v, gg, r, dim, h1, F, f, b, row);
}

hipError_t launch_embed_norm(int32_t n_flows, int32_t batch, int32_t dim, const int32_t *tokens,
                             int32_t vocab, const uint16_t *embed0, const uint16_t *embed1,
                             const float *gain, float eps, float *x, uint16_t *h1, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  embed_norm_kernel<<<n_flows * batch, 1024, 0, s>>>(n_flows, batch, dim, tokens, vocab, embed0, embed1,
                                                     gain, eps, x, h1);
  return hipGetLastError();
}

// RMSNorm of many rows (a prefill chunk): one wave per row, four rows per work-group. Lane l
// holds the float4 slices l, l + 64, ... of the row (the first kRowSlices in registers; a
// longer row's remaining slices are read twice), sums their squares in slice order, then the
// wave butterfly; y = bf16(x * r * gain) in the fragment order of xpack_offset (one flow).
// Every load of the resident slices is issued before the first wait; the gains (the same
// small vector for every row, cached) are read after the reduction.
constexpr int kRowSlices = 16;  // rows up to 4096 wide held in registers

__global__ void __launch_bounds__(256) rmsnorm_rows_kernel(int32_t rows, int32_t dim, const float *x,
                                                           const float *gain, float eps, uint16_t *y) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const f32x4 *xr = (const f32x4 *)(x + (int64_t)row * dim);
  const f32x4 *g4 = (const f32x4 *)gain;
  const int n4 = dim / 4;
  f32x4 v[kRowSlices];
#pragma unroll
  for (int u = 0; u < kRowSlices; ++u)  // a slice past the row re-reads slice 0 (masked below)
    v[u] = xr[lane + 64 * u < n4 ? lane + 64 * u : 0];
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < kRowSlices; ++u)
    if (lane + 64 * u < n4) ss += v[u][0] * v[u][0] + v[u][1] * v[u][1] + v[u][2] * v[u][2] + v[u][3] * v[u][3];
  for (int i = lane + 64 * kRowSlices; i < n4; i += 64) {
    const f32x4 w = xr[i];
    ss += w[0] * w[0] + w[1] * w[1] + w[2] * w[2] + w[3] * w[3];
  }
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float r = 1.0f / sqrtf(ss / (float)dim + eps);
  auto store = [&](int i, const f32x4 &a, const f32x4 &g) {
    *(u32x2 *)(y + xpack_offset(1, 0, row, 4 * i, dim)) =
        u32x2{pack_bf16x2(a[0] * r * g[0], a[1] * r * g[1]), pack_bf16x2(a[2] * r * g[2], a[3] * r * g[3])};
  };
#pragma unroll
  for (int u = 0; u < kRowSlices; ++u)
    if (lane + 64 * u < n4) store(lane + 64 * u, v[u], g4[lane + 64 * u]);
  for (int i = lane + 64 * kRowSlices; i < n4; i += 64) store(i, xr[i], g4[i]);
}

hipError_t launch_rmsnorm_rows(int32_t rows, int32_t dim, const float *x, const float *gain, float eps,
                               uint16_t *y, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  rmsnorm_rows_kernel<<<(rows + 3) / 4, 256, 0, s>>>(rows, dim, x, gain, eps, y);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int32_t rows, int32_t dim, const float *x, const float *gain, float eps,
                          uint16_t *y, hipStream_t s, int packed_flows) {
  if (rows == 0) return hipSuccess;
  rmsnorm_kernel<<<rows, 1024, 0, s>>>(dim, x, gain, eps, y, packed_flows,
                                       packed_flows ? rows / packed_flows : rows);
  return hipGetLastError();
}

// One thread per 4 intermediate elements of one row index, covering both flows.
__global__ void __launch_bounds__(256) swiglu_kernel(int32_t n_flows, int32_t rows, int32_t dim,
                                                     const float *gu, const float *bvec,
                                                     uint16_t *out) {
  const int q = dim / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)rows * q) return;
  const int64_t r = idx / q;
  const int i4 = (int)(idx % q) * 4;
  f32x4 prim;
  for (int f = 0; f < n_flows; ++f) {
    const float *row = gu + ((int64_t)f * rows + r) * 2 * dim;
    const f32x4 g = *(const f32x4 *)(row + i4), u = *(const f32x4 *)(row + dim + i4);
    f32x4 v{silu(g[0]) * u[0], silu(g[1]) * u[1], silu(g[2]) * u[2], silu(g[3]) * u[3]};
    if (f == 0) prim = v;
    else if (bvec) {
      const f32x4 bb = *(const f32x4 *)(bvec + i4);
      v = f32x4{fmaf(bb[0], prim[0], v[0]), fmaf(bb[1], prim[1], v[1]),
                fmaf(bb[2], prim[2], v[2]), fmaf(bb[3], prim[3], v[3])};
    }
    *(u32x2 *)(out + ((int64_t)f * rows + r) * dim + i4) =
        u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
}

hipError_t launch_swiglu(int32_t n_flows, int32_t rows, int32_t dim, const float *gu,
                         const float *b, uint16_t *out, hipStream_t s) {
  const int64_t t = (int64_t)rows * (dim / 4);
  if (t == 0) return hipSuccess;
  swiglu_kernel<<<(unsigned)((t + 255) / 256), 256, 0, s>>>(n_flows, rows, dim, gu, b, out);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) copy_kernel(u32x4 *dst, const u32x4 *src, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = src[i];
}

__global__ void __launch_bounds__(256) fill_kernel(u32x4 *dst, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = u32x4{v, v, v, v};
}

// Reads every 16-byte word once (a measurement of achievable read bandwidth); the XOR of
// what each thread read goes to sink[thread] so the loads cannot be dropped. The source is
// cut into 4 KiB tiles; each wave streams a contiguous run of them, two tiles (8 loads of 16
// bytes per lane, each instruction covering 1 KiB) in flight, non-temporal -- the fastest read
// pattern measured on this GPU. Words past the last whole tile are read grid-stride.
__global__ void __launch_bounds__(256) read_kernel(const u32x4 *src, int64_t n, uint32_t *sink) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * 4, w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t tiles = n / 256, per = (tiles + waves - 1) / waves;
  const int64_t t_end = min(min(w * per, tiles) + per, tiles);
  int64_t t = min(w * per, tiles);
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  for (; t + 1 < t_end; t += 2) {
    u32x4 v[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) v[s] = __builtin_nontemporal_load(src + t * 256 + 64 * s + lane);
#pragma unroll
    for (int s = 0; s < 8; ++s) acc ^= v[s];
  }
  if (t < t_end) {
    u32x4 v[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) v[s] = __builtin_nontemporal_load(src + t * 256 + 64 * s + lane);
#pragma unroll
    for (int s = 0; s < 4; ++s) acc ^= v[s];
  }
  for (int64_t i = tiles * 256 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    acc ^= src[i];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

hipError_t launch_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  read_kernel<<<kReadBlocks, 256, 0, s>>>((const u32x4 *)src, n, sink);
  return hipGetLastError();
}

hipError_t launch_copy(void *dst, const void *src, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  const int64_t blocks = n / 256 < 4096 ? (n + 255) / 256 : 4096;
  copy_kernel<<<(unsigned)blocks, 256, 0, s>>>((u32x4 *)dst, (const u32x4 *)src, n);
  return hipGetLastError();
}

hipError_t launch_fill(void *dst, size_t bytes, uint32_t pattern, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  const int64_t blocks = n / 256 < 4096 ? (n + 255) / 256 : 4096;
  fill_kernel<<<(unsigned)blocks, 256, 0, s>>>((u32x4 *)dst, n, pattern);
  return hipGetLastError();
}

}  // namespace dfx
