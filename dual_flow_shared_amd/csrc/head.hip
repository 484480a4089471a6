// Mixture of the two flows' next-token distributions and the next token (Sintesi Tecnica:
// Dual-Flow Transformers, "Meccanismi Chiave", mixture objective): p_f = softmax(logits_f),
// c = sum_i p_0,i^2 (the primary's collision probability), alpha = (1 + c) / 2 (a reading: the
// pages fix only that alpha follows c and never drops below 1/2), p_mix = alpha p_0 +
// (1 - alpha) p_1. The token is argmax_i p_mix,i, or with uniform noise u argmax_i
// log p_mix,i - log(-log u_i) (a Gumbel-max draw); ties go to the lowest index.
//
// The vocabulary is cut into chunks (whole load rounds of kMixVec logits) so that a batch of
// a few sequences still fills the chip. Three passes, each one launch:
//   stats: per (statistics chunk, sequence) the chunk's max m, sum e^(l - m) and, for the
//          primary, sum e^(2 (l - m)). When the projection runs in one K split it writes these
//          itself, per 128-logit tile, from its accumulators, and this pass is skipped;
//          otherwise this kernel computes them per mixture chunk from the logits;
//   mix:   per (chunk, sequence) the sequence's stats combined from all statistics records in
//          record order (every work-group of a sequence combines the same numbers in the same
//          order, so all agree bit for bit), alpha, p_mix of the chunk, and the chunk's best
//          score;
//   pick:  per sequence the best over the chunks (lowest index on ties), and alpha.
#include "common.h"

namespace dfx {

constexpr int kMixThreads = 256;
constexpr int kMixVec = 4 * kMixThreads;  // logits per work-group and load round
constexpr int kMixRounds = 8;             // rounds held in registers: chunks up to 8192 logits

// per (sequence, chunk), written by the mix pass: alpha, best value, best index (as bits)
constexpr int kMixBest = 4;

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

constexpr int kFoldBatch = 8;  // statistics records per thread loaded together

__device__ __forceinline__ void better(float &bv, int32_t &bi, float ov, int32_t oi) {
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}

struct MixArgs {
  int32_t F, B, V, chunk, nchunks;
  int32_t nstat;        // statistics records per sequence
  const float *logits;  // [F][B][V]
  const float *noise;   // [B][V] or NULL
  float *stats;         // [B][nstat][kMixStat]
  float *best;          // [B][nchunks][kMixBest]
  float *p_mix;         // [B][V] or NULL
  int32_t *token;       // [B]
  float *alpha;         // [B] or NULL
};

__global__ void __launch_bounds__(kMixThreads) mix_stats_kernel(MixArgs a) {
  __shared__ float red[4];
  const int c = blockIdx.x, b = blockIdx.y;
  const int64_t lo = (int64_t)c * a.chunk;
  const int64_t n = min((int64_t)a.chunk, (int64_t)a.V - lo);
  float *st = a.stats + ((int64_t)b * a.nstat + c) * kMixStat;
  for (int f = 0; f < a.F; ++f) {
    const float *l = a.logits + ((int64_t)f * a.B + b) * a.V + lo;
    f32x4 v[kMixRounds];
    float m = -INFINITY;
    // every load is issued (a lane past the chunk re-reads its last 4 logits), so none waits
    // for another; the lanes past the chunk are masked afterwards
#pragma unroll
    for (int r = 0; r < kMixRounds; ++r) v[r] = *(const f32x4 *)(l + min((int64_t)(r * kMixVec + 4 * threadIdx.x), n - 4));
#pragma unroll
    for (int r = 0; r < kMixRounds; ++r) {
      if (r * kMixVec + 4 * (int)threadIdx.x >= n) v[r] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      m = fmaxf(m, fmaxf(fmaxf(v[r][0], v[r][1]), fmaxf(v[r][2], v[r][3])));
    }
    m = block_max(m, red);
    float s = 0.f, q = 0.f;
#pragma unroll
    for (int r = 0; r < kMixRounds; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = exp_hw(v[r][j] - m);
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
  __shared__ float best_v[4];
  __shared__ int32_t best_i[4];
  const int c = blockIdx.x, b = blockIdx.y;
  const int64_t lo = (int64_t)c * a.chunk;
  const int64_t n = min((int64_t)a.chunk, (int64_t)a.V - lo);
  const float *l0 = a.logits + (int64_t)b * a.V + lo;
  const float *l1 = a.logits + ((int64_t)a.B + b) * a.V + lo;
  const float *sb = a.stats + (int64_t)b * a.nstat * kMixStat;
  // The sequence's statistics records (the first kFoldBatch per thread), then the chunk's
  // logits (and noise), are all loaded before anything waits: the logits do not depend on
  // the statistics, so their round trip overlaps the combination below. Every load is issued
  // (a lane past the end re-reads the last record or the last 4 logits and is skipped
  // later), so none waits for another.
  f32x4 r[kFoldBatch];
  float rs1[kFoldBatch];
  auto load_records = [&](int k0) {
#pragma unroll
    for (int t = 0; t < kFoldBatch; ++t) {
      const int64_t k = min(k0 + t * kMixThreads + (int)threadIdx.x, a.nstat - 1);
      r[t] = *(const f32x4 *)(sb + k * kMixStat);
      rs1[t] = sb[k * kMixStat + 4];
    }
  };
  load_records(0);
  f32x4 x0[kMixRounds], x1[kMixRounds], u[kMixRounds];
#pragma unroll
  for (int q = 0; q < kMixRounds; ++q) x0[q] = *(const f32x4 *)(l0 + min((int64_t)(q * kMixVec + 4 * threadIdx.x), n - 4));
  if (a.F == 2) {
#pragma unroll
    for (int q = 0; q < kMixRounds; ++q) x1[q] = *(const f32x4 *)(l1 + min((int64_t)(q * kMixVec + 4 * threadIdx.x), n - 4));
  }
  if (a.noise) {
    const float *nz = a.noise + (int64_t)b * a.V + lo;
#pragma unroll
    for (int q = 0; q < kMixRounds; ++q) u[q] = *(const f32x4 *)(nz + min((int64_t)(q * kMixVec + 4 * threadIdx.x), n - 4));
  }
  // the sequence's max per flow, then the sums rescaled to it (record order within a
  // thread, then the lanes and the four waves in a fixed order)
  const int batch_recs = kFoldBatch * kMixThreads;
  auto live = [&](int k0, int t) { return k0 + t * kMixThreads + (int)threadIdx.x < a.nstat; };
  float m0 = -INFINITY, m1 = -INFINITY;
  auto max_records = [&](int k0) {
#pragma unroll
    for (int t = 0; t < kFoldBatch; ++t)
      if (live(k0, t)) {
        m0 = fmaxf(m0, r[t][0]);
        m1 = fmaxf(m1, r[t][3]);
      }
  };
  max_records(0);
  for (int k0 = batch_recs; k0 < a.nstat; k0 += batch_recs) {  // more than one batch of records
    load_records(k0);
    max_records(k0);
  }
  m0 = wave_max(m0);
  m1 = wave_max(m1);
  __shared__ float red[3][4];
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = m0;
    red[1][threadIdx.x >> 6] = m1;
  }
  __syncthreads();
  m0 = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  m1 = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  float s0 = 0.f, q0 = 0.f, s1 = 0.f;
  auto sum_records = [&](int k0) {
#pragma unroll
    for (int t = 0; t < kFoldBatch; ++t)
      if (live(k0, t)) {
        const float e = exp_hw(r[t][0] - m0);
        s0 = fmaf(r[t][1], e, s0);
        q0 = fmaf(r[t][2], e * e, q0);
        if (a.F == 2) s1 = fmaf(rs1[t], exp_hw(r[t][3] - m1), s1);
      }
  };
  if (a.nstat <= batch_recs) {
    sum_records(0);  // the records are still in registers
  } else {
    for (int k0 = 0; k0 < a.nstat; k0 += batch_recs) {
      load_records(k0);
      sum_records(k0);
    }
  }
  s0 = wave_sum(s0);
  q0 = wave_sum(q0);
  s1 = wave_sum(s1);
  __syncthreads();  // the maxima have been read
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = s0;
    red[1][threadIdx.x >> 6] = q0;
    red[2][threadIdx.x >> 6] = s1;
  }
  __syncthreads();
  s0 = ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3];
  q0 = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
  s1 = ((red[2][0] + red[2][1]) + red[2][2]) + red[2][3];
  const float coll = q0 / (s0 * s0);
  const float alpha = a.F == 2 ? 0.5f * (1.0f + coll) : 1.0f;
  const float w0 = alpha / s0, w1 = a.F == 2 ? (1.0f - alpha) / s1 : 0.f;
  float bv = -INFINITY;
  int32_t bi = INT32_MAX;
#pragma unroll
  for (int q = 0; q < kMixRounds; ++q) {
    const int i = q * kMixVec + 4 * threadIdx.x;
    if (i >= n) continue;
    f32x4 p;
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = w0 * exp_hw(x0[q][j] - m0);
    if (a.F == 2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = fmaf(w1, exp_hw(x1[q][j] - m1), p[j]);
    }
    if (a.p_mix) *(f32x4 *)(a.p_mix + (int64_t)b * a.V + lo + i) = p;
    f32x4 score = p;
    if (a.noise) {
#pragma unroll
      for (int j = 0; j < 4; ++j) score[j] = logf(p[j]) - logf(-logf(u[q][j]));
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
    float *bs = a.best + ((int64_t)b * a.nchunks + c) * kMixBest;
    bs[0] = alpha;
    bs[1] = bv;
    bs[2] = __int_as_float(bi);
  }
}

// One wave per sequence.
__global__ void __launch_bounds__(64) mix_pick_kernel(MixArgs a) {
  const int b = blockIdx.x;
  const float *sb = a.best + (int64_t)b * a.nchunks * kMixBest;
  float bv = -INFINITY;
  int32_t bi = INT32_MAX;
  for (int k = threadIdx.x; k < a.nchunks; k += 64) better(bv, bi, sb[k * kMixBest + 1], __float_as_int(sb[k * kMixBest + 2]));
  for (int o = 32; o > 0; o >>= 1) better(bv, bi, __shfl_xor(bv, o), __shfl_xor(bi, o));
  if (threadIdx.x == 0) {
    // every score NaN (or -inf): no candidate won; fall back to index 0 rather than an
    // out-of-range token
    a.token[b] = bi < a.V ? bi : 0;
    if (a.alpha) a.alpha[b] = sb[0];
  }
}

int mixture_chunk(int32_t batch, int32_t vocab) {
  // about 512 work-groups per pass, chunks of whole load rounds, at most kMixRounds rounds
  const int per_seq = batch > 0 ? (512 + batch - 1) / batch : 512;
  int chunk = (int)((vocab + per_seq - 1) / per_seq);
  chunk = (chunk + kMixVec - 1) / kMixVec * kMixVec;
  return chunk < kMixVec ? kMixVec : (chunk > kMixRounds * kMixVec ? kMixRounds * kMixVec : chunk);
}

// statistics records per sequence: one per 128-logit tile when the projection writes them,
// else one per mixture chunk (never more than the tiles)
static int mixture_records(int32_t vocab) { return (vocab + kHeadTile - 1) / kHeadTile; }

static size_t mixture_record_bytes(int32_t batch, int32_t vocab) {
  return ((size_t)batch * mixture_records(vocab) * kMixStat * sizeof(float) + 255) / 256 * 256;
}

size_t mixture_stats_bytes(int32_t batch, int32_t vocab) {
  const int chunk = mixture_chunk(batch, vocab);
  return mixture_record_bytes(batch, vocab) +
         (size_t)batch * ((vocab + chunk - 1) / chunk) * kMixBest * sizeof(float);
}

hipError_t launch_mixture(int32_t n_flows, int32_t batch, int32_t vocab, const float *logits, const float *noise,
                          float *stats, int32_t *token, float *alpha, float *p_mix, bool stats_per_tile,
                          hipStream_t s) {
  if (batch == 0) return hipSuccess;
  MixArgs a{};
  a.F = n_flows; a.B = batch; a.V = vocab;
  a.chunk = mixture_chunk(batch, vocab);
  a.nchunks = (vocab + a.chunk - 1) / a.chunk;
  a.nstat = stats_per_tile ? mixture_records(vocab) : a.nchunks;
  a.logits = logits; a.noise = noise; a.stats = stats; a.p_mix = p_mix; a.token = token; a.alpha = alpha;
  a.best = stats + mixture_record_bytes(batch, vocab) / sizeof(float);
  const dim3 grid(a.nchunks, batch);
  if (!stats_per_tile) mix_stats_kernel<<<grid, kMixThreads, 0, s>>>(a);
  mix_apply_kernel<<<grid, kMixThreads, 0, s>>>(a);
  mix_pick_kernel<<<batch, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dfx
