// Mixture of the two flows' next-token distributions and the next token (Sintesi Tecnica:
// Dual-Flow Transformers, "Meccanismi Chiave", mixture objective): p_f = softmax(logits_f),
// c = sum_i p_0,i^2 (the primary's collision probability), alpha = (1 + c) / 2 (a reading: the
// pages fix only that alpha follows c and never drops below 1/2), p_mix = alpha p_0 +
// (1 - alpha) p_1. The token is argmax_i p_mix,i, or with uniform noise u argmax_i
// log p_mix,i - log(-log u_i) (a Gumbel-max draw); ties go to the lowest index.
//
// The vocabulary is cut into chunks (whole load rounds of kMixVec logits) so that a batch of
// a few sequences still fills the chip. Three passes, each one launch:
//   stats: per (chunk, sequence) the chunk's max m, sum e^(l - m) and, for the primary,
//          sum e^(2 (l - m)), from the chunk's logits held in registers;
//   mix:   per (chunk, sequence) the sequence's stats combined from all chunks in chunk order
//          (every work-group of a sequence combines the same numbers in the same order, so
//          all agree bit for bit), alpha, p_mix of the chunk, and the chunk's best score;
//   pick:  per sequence the best over the chunks (lowest index on ties), and alpha.
#include "common.h"

namespace dfx {

constexpr int kMixThreads = 256;
constexpr int kMixVec = 4 * kMixThreads;  // logits per work-group and load round
constexpr int kMixRounds = 8;             // rounds held in registers: chunks up to 8192 logits

// per (sequence, chunk): m0, s0, q0, m1, s1, alpha (written by the mix pass), best value,
// best index (as bits)
constexpr int kMixStat = 8;

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Block-wide reductions over the 4 waves, in wave order.
__device__ __forceinline__ float block_max(float v, float *red) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

__device__ __forceinline__ void better(float &bv, int32_t &bi, float ov, int32_t oi) {
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}

struct MixArgs {
  int32_t F, B, V, chunk, nchunks;
  const float *logits;  // [F][B][V]
  const float *noise;   // [B][V] or NULL
  float *stats;         // [B][nchunks][kMixStat]
  float *p_mix;         // [B][V] or NULL
  int32_t *token;       // [B]
  float *alpha;         // [B] or NULL
};

__global__ void __launch_bounds__(kMixThreads) mix_stats_kernel(MixArgs a) {
  __shared__ float red[4];
  const int c = blockIdx.x, b = blockIdx.y;
  const int64_t lo = (int64_t)c * a.chunk;
  const int64_t n = min((int64_t)a.chunk, (int64_t)a.V - lo);
  float *st = a.stats + ((int64_t)b * a.nchunks + c) * kMixStat;
  for (int f = 0; f < a.F; ++f) {
    const float *l = a.logits + ((int64_t)f * a.B + b) * a.V + lo;
    f32x4 v[kMixRounds];
    float m = -INFINITY;
#pragma unroll
    for (int r = 0; r < kMixRounds; ++r) {
      const int i = r * kMixVec + 4 * threadIdx.x;
      v[r] = i < n ? *(const f32x4 *)(l + i) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      m = fmaxf(m, fmaxf(fmaxf(v[r][0], v[r][1]), fmaxf(v[r][2], v[r][3])));
    }
    m = block_max(m, red);
    float s = 0.f, q = 0.f;
#pragma unroll
    for (int r = 0; r < kMixRounds; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = expf(v[r][j] - m);
        s += e;
        q = fmaf(e, e, q);
      }
    s = block_sum(s, red);
    if (f == 0) q = block_sum(q, red);
    if (threadIdx.x == 0) {
      st[3 * f] = m;
      st[3 * f + 1] = s;
      if (f == 0) st[2] = q;
    }
  }
}

__global__ void __launch_bounds__(kMixThreads) mix_apply_kernel(MixArgs a) {
  __shared__ float red[4];
  __shared__ float best_v[4];
  __shared__ int32_t best_i[4];
  const int c = blockIdx.x, b = blockIdx.y;
  const float *sb = a.stats + (int64_t)b * a.nchunks * kMixStat;
  // the sequence's max per flow, then the sums rescaled to it, chunk order within a thread
  float m0 = -INFINITY, m1 = -INFINITY;
  for (int k = threadIdx.x; k < a.nchunks; k += kMixThreads) {
    m0 = fmaxf(m0, sb[k * kMixStat]);
    if (a.F == 2) m1 = fmaxf(m1, sb[k * kMixStat + 3]);
  }
  m0 = block_max(m0, red);
  if (a.F == 2) m1 = block_max(m1, red);
  float s0 = 0.f, q0 = 0.f, s1 = 0.f;
  for (int k = threadIdx.x; k < a.nchunks; k += kMixThreads) {
    const float *st = sb + k * kMixStat;
    const float r0 = expf(st[0] - m0);
    s0 = fmaf(st[1], r0, s0);
    q0 = fmaf(st[2], r0 * r0, q0);
    if (a.F == 2) s1 = fmaf(st[4], expf(st[3] - m1), s1);
  }
  s0 = block_sum(s0, red);
  q0 = block_sum(q0, red);
  if (a.F == 2) s1 = block_sum(s1, red);
  const float coll = q0 / (s0 * s0);
  const float alpha = a.F == 2 ? 0.5f * (1.0f + coll) : 1.0f;
  const float w0 = alpha / s0, w1 = a.F == 2 ? (1.0f - alpha) / s1 : 0.f;
  const int64_t lo = (int64_t)c * a.chunk;
  const int64_t n = min((int64_t)a.chunk, (int64_t)a.V - lo);
  const float *l0 = a.logits + (int64_t)b * a.V + lo;
  const float *l1 = a.logits + ((int64_t)a.B + b) * a.V + lo;
  float bv = -INFINITY;
  int32_t bi = INT32_MAX;
  for (int r = 0; r < kMixRounds; ++r) {
    const int i = r * kMixVec + 4 * threadIdx.x;
    if (i >= n) break;
    const f32x4 x0 = *(const f32x4 *)(l0 + i);
    f32x4 p;
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = w0 * expf(x0[j] - m0);
    if (a.F == 2) {
      const f32x4 x1 = *(const f32x4 *)(l1 + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = fmaf(w1, expf(x1[j] - m1), p[j]);
    }
    if (a.p_mix) *(f32x4 *)(a.p_mix + (int64_t)b * a.V + lo + i) = p;
    f32x4 score = p;
    if (a.noise) {
      const f32x4 u = *(const f32x4 *)(a.noise + (int64_t)b * a.V + lo + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) score[j] = logf(p[j]) - logf(-logf(u[j]));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) better(bv, bi, score[j], (int32_t)(lo + i + j));
  }
  for (int o = 32; o > 0; o >>= 1) better(bv, bi, __shfl_xor(bv, o), __shfl_xor(bi, o));
  if ((threadIdx.x & 63) == 0) {
    best_v[threadIdx.x >> 6] = bv;
    best_i[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) better(bv, bi, best_v[w], best_i[w]);
    float *st = a.stats + ((int64_t)b * a.nchunks + c) * kMixStat;
    st[5] = alpha;
    st[6] = bv;
    st[7] = __int_as_float(bi);
  }
}

// One wave per sequence.
__global__ void __launch_bounds__(64) mix_pick_kernel(MixArgs a) {
  const int b = blockIdx.x;
  const float *sb = a.stats + (int64_t)b * a.nchunks * kMixStat;
  float bv = -INFINITY;
  int32_t bi = INT32_MAX;
  for (int k = threadIdx.x; k < a.nchunks; k += 64) better(bv, bi, sb[k * kMixStat + 6], __float_as_int(sb[k * kMixStat + 7]));
  for (int o = 32; o > 0; o >>= 1) better(bv, bi, __shfl_xor(bv, o), __shfl_xor(bi, o));
  if (threadIdx.x == 0) {
    // every score NaN (or -inf): no candidate won; fall back to index 0 rather than an
    // out-of-range token
    a.token[b] = bi < a.V ? bi : 0;
    if (a.alpha) a.alpha[b] = sb[5];
  }
}

int mixture_chunk(int32_t batch, int32_t vocab) {
  // about 512 work-groups per pass, chunks of whole load rounds, at most kMixRounds rounds
  const int per_seq = batch > 0 ? (512 + batch - 1) / batch : 512;
  int chunk = (int)((vocab + per_seq - 1) / per_seq);
  chunk = (chunk + kMixVec - 1) / kMixVec * kMixVec;
  return chunk < kMixVec ? kMixVec : (chunk > kMixRounds * kMixVec ? kMixRounds * kMixVec : chunk);
}

size_t mixture_stats_bytes(int32_t batch, int32_t vocab) {
  const int chunk = mixture_chunk(batch, vocab);
  return (size_t)batch * ((vocab + chunk - 1) / chunk) * kMixStat * sizeof(float);
}

hipError_t launch_mixture(int32_t n_flows, int32_t batch, int32_t vocab, const float *logits, const float *noise,
                          float *stats, int32_t *token, float *alpha, float *p_mix, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  MixArgs a{};
  a.F = n_flows; a.B = batch; a.V = vocab;
  a.chunk = mixture_chunk(batch, vocab);
  a.nchunks = (vocab + a.chunk - 1) / a.chunk;
  a.logits = logits; a.noise = noise; a.stats = stats; a.p_mix = p_mix; a.token = token; a.alpha = alpha;
  const dim3 grid(a.nchunks, batch);
  mix_stats_kernel<<<grid, kMixThreads, 0, s>>>(a);
  mix_apply_kernel<<<grid, kMixThreads, 0, s>>>(a);
  mix_pick_kernel<<<batch, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dfx
