// Tile helpers of the matrix-core attention kernels (decode and prefill): loads of a 32-token
// K/V tile into registers in the lane layouts of the 16x16x32 bf16 MFMA, the score MFMAs, and
// the online-softmax update with the P.V MFMAs. The layouts are described at the top of
// attn_mfma.hip.
#pragma once
#include "common.h"

namespace dfx {

template <bool BF16>
__device__ __forceinline__ void load8(const void *base, int64_t off, float *out) {
  if constexpr (BF16) {
    const u32x4 w = *(const u32x4 *)((const uint16_t *)base + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16_lo(w[i]);
      out[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    const f32x4 a = *(const f32x4 *)((const float *)base + off);
    const f32x4 c = *(const f32x4 *)((const float *)base + off + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[i] = a[i];
      out[4 + i] = c[i];
    }
  }
}

constexpr int kMaxChunkBlocks = 1024;  // block ids of one split held in LDS

template <int D>
struct TileRegs {
  u32x4 kf[2][D / 32];            // K rows of two 16-token blocks (A operand)
  uint32_t vr[8][D / 32];         // V: D/16 elements of the 8 token rows tau(j, v)
};

// Element offsets of the first row of each 16-token half of the tile at t0 and the
// largest in-half index that is still inside [t0, end). A half lies in one block (paged
// blocks hold >= 16 tokens and halves start 16-aligned); a half entirely past `end`
// reuses the first half, and rows past `end` are clamped to the last valid one (their
// scores are masked), so every address stays inside this split's staged blocks.
template <bool PAGED>
__device__ __forceinline__ void half_bases(const AttnArgs &p, const int32_t *tbl, int first_blk,
                                           int b, int g, int t0, int end, int64_t *hb, int *lastx) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int hs = t0 + 16 * h < end ? t0 + 16 * h : t0;
    int64_t blk;
    int slot;
    if constexpr (PAGED) {
      // the same block id for the whole wave (t0 is the wave's): moved into a scalar register
      // (an asm operand, which the compiler cannot fold back into the vector value), so that
      // the address arithmetic of the tile runs on the scalar unit
      const int bv = tbl[(hs >> p.block_shift) - first_blk];
      int bs_;
      asm("v_readfirstlane_b32 %0, %1" : "=s"(bs_) : "v"(bv));
      blk = bs_;
      slot = hs & (p.block_size - 1);
    } else {
      blk = b;
      slot = hs;
    }
    hb[h] = ((blk * p.num_kv_heads + g) * (int64_t)p.block_size + slot) * p.head_dim;
    lastx[h] = end - 1 - hs;
  }
}

#ifndef DFX_ATTN_NT
#define DFX_ATTN_NT 1
#endif
// K/V loads: non-temporal by default (each line is read once per call, and the hint keeps
// the stream from displacing the rest of L2); 0 gives plain loads for comparison.
template <typename T>
__device__ __forceinline__ T kv_load(const uint16_t *p) {
  if constexpr (DFX_ATTN_NT) return __builtin_nontemporal_load((const T *)p);
  else return *(const T *)p;
}

// Issue the K (resp. V) loads of the tile described by (hb, lastx).
template <int D>
__device__ __forceinline__ void load_k(const uint16_t *kp, const int64_t *hb, const int *lastx,
                                       int n, int j, TileRegs<D> &r) {
  constexpr int KS = D / 32;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const uint16_t *row = kp + hb[mb] + (int64_t)min(n, lastx[mb]) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) r.kf[mb][s] = kv_load<u32x4>(row + 8 * (4 * s + j));
  }
}

template <int D>
__device__ __forceinline__ void load_v(const uint16_t *vp, const int64_t *hb, const int *lastx,
                                       int n, int j, TileRegs<D> &r) {
  constexpr int VEC = D / 16;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int h = v >> 2, x = 4 * j + (v & 3);  // token tau(j, v) = t0 + 16 h + x
    const uint16_t *src = vp + hb[h] + (int64_t)min(x, lastx[h]) * D + VEC * n;
    if constexpr (VEC == 8) {
      const u32x4 y = kv_load<u32x4>(src);
      r.vr[v][0] = y[0]; r.vr[v][1] = y[1]; r.vr[v][2] = y[2]; r.vr[v][3] = y[3];
    } else {
      const u32x2 y = kv_load<u32x2>(src);
      r.vr[v][0] = y[0]; r.vr[v][1] = y[1];
    }
  }
}

// Scores of one loaded tile (S^T blocks for its two 16-token halves); the query rows are the
// sum of NT bf16 terms q[0..NT-1] (split_terms), one MFMA pass per term.
template <int D, int NT>
__device__ __forceinline__ void tile_scores(const TileRegs<D> &r, const u32x4 (&q)[NT][D / 32], f32x4 *sacc) {
  constexpr int KS = D / 32;
  sacc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  sacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t) sacc[mb] = mfma16x16x32(as_bf16x8(r.kf[mb][s]), as_bf16x8(q[t][s]), sacc[mb]);
}

// Lazy running max (prefill): a row keeps its running max m until a tile's max exceeds it by
// more than kLazyMax (log2 units), so that P = 2^(s - m) stays below 2^kLazyMax -- exact in
// fp32 and in the bf16 terms, and far from overflow -- and most tiles need no rescale of O.
constexpr float kLazyMax = 8.f;

// Online-softmax update for query row n (the lane holds 8 of the tile's 32 tokens) and
// P.V accumulation into O^T, with P split into NT bf16 terms (one MFMA pass per term).
// Both forms skip the rescale of O when no row of the wave moved its max (the factor is then
// exactly 1 for every row, so skipping it changes no bit) and the per-token test on a tile
// inside every row's range. LAZY (prefill, where the vector instructions bound the kernel):
// the running max moves only by more than kLazyMax, so that most tiles need no rescale, and P
// is 2^x from the hardware exponential (P below 2^-126, flushed to zero, is below the fp32
// resolution of the row sum, which is >= 1). Decode, a memory stream, keeps the eager max:
// the lazy one saved 1% of the decode layer step, and its different rounding of the rows left
// the small decode layer's median error at the edge of the ensemble parity bar.
template <int D, int NT, bool LAZY = false>
__device__ __forceinline__ void tile_softmax_pv(const AttnArgs &p, const TileRegs<D> &r,
                                                const f32x4 *sacc, int t0, int end, int j,
                                                float &m_run, float &l_run, f32x4 *oacc) {
  constexpr int VEC = D / 16;
  float sv[8];
  float mx = -INFINITY;
  const bool whole = __all(t0 + 32 <= end);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = t0 + 16 * mb + 4 * j + i;
      const float x = whole || tok < end ? sacc[mb][i] * p.scale_log2 : -INFINITY;
      sv[4 * mb + i] = x;
      mx = fmaxf(mx, x);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float m_new, alpha;
  if constexpr (LAZY) {
    m_new = mx > m_run + kLazyMax ? mx : m_run;
    alpha = m_new == m_run ? 1.f : exp2f(m_run - m_new);
  } else {
    m_new = fmaxf(m_run, mx);
    alpha = exp2f(m_run - m_new);
  }
  float psum = 0.f;
  u32x4 pk[NT];
  if constexpr (NT >= 3) {
    // every term a truncation (split_terms: exact with three terms); the bf16 halves of two
    // tokens' remainders go into one word by a byte permute
    uint32_t rem[8][NT];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const float pv = LAZY ? __builtin_amdgcn_exp2f(sv[v] - m_new) : exp2f(sv[v] - m_new);
      psum += pv;
      float r = pv;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        rem[v][t] = __float_as_uint(r);
        if (t + 1 < NT) r -= __uint_as_float(rem[v][t] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int w = 0; w < 4; ++w) pk[t][w] = __builtin_amdgcn_perm(rem[2 * w + 1][t], rem[2 * w][t], 0x07060302u);
  } else {
    uint32_t pt[8][NT];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const float pv = LAZY ? __builtin_amdgcn_exp2f(sv[v] - m_new) : exp2f(sv[v] - m_new);
      psum += pv;
      split_terms<NT>(pv, pt[v]);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int w = 0; w < 4; ++w) pk[t][w] = pt[2 * w][t] | (pt[2 * w + 1][t] << 16);
  }
  l_run = l_run * alpha + psum;
  m_run = m_new;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int mb = 0; mb < VEC; ++mb) oacc[mb] *= alpha;
  }
#pragma unroll
  for (int mb = 0; mb < VEC; ++mb) {
    // V^T rows d = VEC*n + mb over tokens tau(j, 0..7): element mb of each loaded row, two
    // tokens' halves per word (one byte permute: the low halves for even mb, the high halves
    // for odd mb)
    u32x4 af;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x0 = r.vr[2 * w][mb >> 1], x1 = r.vr[2 * w + 1][mb >> 1];
      af[w] = __builtin_amdgcn_perm(x1, x0, (mb & 1) ? 0x07060302u : 0x05040100u);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) oacc[mb] = mfma16x16x32(as_bf16x8(af), as_bf16x8(pk[t]), oacc[mb]);
  }
}

}  // namespace dfx
