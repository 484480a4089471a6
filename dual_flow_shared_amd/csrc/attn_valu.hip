// Dual-query decode attention on the vector ALUs, all in fp32.
//
// Serves fp32 caches (where a bf16 matrix-core pass would not keep fp32 accuracy) and
// shapes outside the matrix-core tile (more than 16 query rows per KV head). Same
// contract as the MFMA kernel: one work-group per (sequence, KV head, split), every
// query row of both flows for that KV head reads each staged K/V tile from LDS, online
// softmax in the log2 domain, fixed-order reductions (deterministic).
#include "common.h"

namespace dfx {

__device__ __forceinline__ int64_t kv_row_v(const AttnArgs &p, int b, int g, int pos) {
  int64_t blk;
  int slot;
  if (p.block_shift >= 0) {
    const uint32_t e = (uint32_t)p.table[(int64_t)b * p.max_blocks + (pos >> p.block_shift)];
    blk = (uint64_t)e < (uint64_t)p.num_blocks ? (int64_t)e : p.num_blocks - 1;
    slot = pos & (p.block_size - 1);
  } else {
    blk = b;
    slot = pos;
  }
  return ((blk * p.num_kv_heads + g) * (int64_t)p.block_size + slot) * p.head_dim;
}

template <bool BF16>
__device__ __forceinline__ float ld(const void *base, int64_t i) {
  if constexpr (BF16) return __uint_as_float((uint32_t)((const uint16_t *)base)[i] << 16);
  else return ((const float *)base)[i];
}

constexpr int kT = 32;     // tokens per tile
constexpr int kMaxR = 32;  // query rows per KV head
constexpr int kMaxD = 128;

template <bool KVBF16, bool QBF16>
__global__ void __launch_bounds__(256) attn_valu_kernel(AttnArgs p) {
  __shared__ float q_s[kMaxR][kMaxD];
  __shared__ float k_s[kT][kMaxD + 1];
  __shared__ float v_s[kT][kMaxD];
  __shared__ float p_s[kMaxR][kT];
  __shared__ float m_s[kMaxR], l_s[kMaxR], a_s[kMaxR];

  const int g = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ctx = min(max(p.ctx[b], 0), p.max_context);
  const int start = split * p.chunk;
  if (split > 0 && start >= ctx) return;
  const int end = min(start + p.chunk, ctx);
  const int D = p.head_dim, G = p.group, R = p.n_flows * G;

  for (int idx = tid; idx < R * D; idx += 256) {
    const int r = idx / D, d = idx % D;
    const int f = r / G, h = g * G + r % G;
    const int64_t off = (int64_t)b * p.q_bstride + (int64_t)h * D + d;
    float q = ld<QBF16>(p.q1, off);
    if (f == 1) {
      const float q2 = ld<QBF16>(p.q2, off);
      q = p.a ? fmaf(p.a[(int64_t)h * p.a_hstride + d], q, q2) : q2;
    }
    q_s[r][d] = q * p.scale_log2;
  }
  if (tid < R) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;

  // The next tile's K/V elements are loaded into registers while the current tile is
  // multiplied. Thread tid holds elements tid + 256 i of the [kT][D] tile; tokens past the
  // split re-read its last token and are zeroed when stored.
  constexpr int kPer = kT * kMaxD / 256;
  float kn[kPer], vn[kPer];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + 256 * i;
      if (idx < kT * D) {
        const int t = idx / D, d = idx % D;
        const int64_t row = kv_row_v(p, b, g, min(t0 + t, end - 1));
        kn[i] = ld<KVBF16>(p.k, row + d);
        vn[i] = ld<KVBF16>(p.v, row + d);
      }
    }
  };
  if (start < end) load_tile(start);
  for (int t0 = start; t0 < end; t0 += kT) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + 256 * i;
      if (idx < kT * D) {
        const int t = idx / D, d = idx % D;
        const bool ok = t0 + t < end;
        k_s[t][d] = ok ? kn[i] : 0.f;
        v_s[t][d] = ok ? vn[i] : 0.f;
      }
    }
    if (t0 + kT < end) load_tile(t0 + kT);
    __syncthreads();
    for (int idx = tid; idx < R * kT; idx += 256) {
      const int r = idx / kT, t = idx % kT;
      float s = 0.f;
      for (int d = 0; d < D; ++d) s = fmaf(q_s[r][d], k_s[t][d], s);
      p_s[r][t] = t0 + t < end ? s : -INFINITY;
    }
    __syncthreads();
    for (int r = wave; r < R; r += 4) {
      const float x = lane < kT ? p_s[r][lane] : -INFINITY;
      float mx = x;
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float m_old = m_s[r];
      const float m_new = fmaxf(m_old, mx);
      const float pv = lane < kT ? exp2f(x - m_new) : 0.f;
      float sum = pv;
      for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      if (lane < kT) p_s[r][lane] = pv;
      if (lane == 0) {
        const float alpha = exp2f(m_old - m_new);
        a_s[r] = alpha;
        l_s[r] = l_s[r] * alpha + sum;
        m_s[r] = m_new;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int idx = tid + 256 * i;
      if (idx < R * D) {
        const int r = idx / D, d = idx % D;
        float o = acc[i] * a_s[r];
        for (int t = 0; t < kT; ++t) o = fmaf(p_s[r][t], v_s[t][d], o);
        acc[i] = o;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int idx = tid + 256 * i;
    if (idx < R * D) {
      const int r = idx / D, d = idx % D;
      const int f = r / G, h = g * G + r % G;
      const float L = l_s[r], M = m_s[r];
      const float o = L > 0.f ? acc[i] / L : 0.f;
      const float lse2 = L > 0.f ? M + __log2f(L) : -INFINITY;
      if (p.num_splits == 1) {
        int64_t oi;
        float *out = attn_out(p, f, b, h * D + d, &oi);
        if (p.o_bf16) ((uint16_t *)out)[oi] = (uint16_t)f32_to_bf16_rne(o);
        else out[oi] = o;
        if (d == 0 && p.lse) p.lse[((int64_t)f * p.batch + b) * p.num_q_heads + h] = lse2 * kLn2;
      } else {
        const int64_t row = (((int64_t)split * p.n_flows + f) * p.batch + b) * p.num_q_heads + h;
        p.part_o[row * D + d] = o;
        if (d == 0) p.part_lse[row] = lse2;
      }
    }
  }
}

hipError_t launch_attn_valu(const AttnArgs &a, hipStream_t s) {
  if (a.head_dim > kMaxD || a.n_flows * a.group > kMaxR) return hipErrorInvalidValue;
  // The hardware hands work-group i to XCD i % 8. With the KV head fastest, XCD k serves
  // head k of every sequence (an equal share whatever the context lengths), and each XCD
  // dispatches all first splits (the longest pieces of ragged batches) before the later ones.
  const dim3 grid(a.num_kv_heads, a.batch, a.num_splits), block(256);
  if (a.kv_bf16) {
    if (a.q_bf16) attn_valu_kernel<true, true><<<grid, block, 0, s>>>(a);
    else attn_valu_kernel<true, false><<<grid, block, 0, s>>>(a);
  } else {
    if (a.q_bf16) attn_valu_kernel<false, true><<<grid, block, 0, s>>>(a);
    else attn_valu_kernel<false, false><<<grid, block, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace dfx
