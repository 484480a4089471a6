// Mixture-of-experts MLP block with router replay (Sintesi Tecnica: Dual-Flow Transformers,
// "Meccanismi Chiave", router replay: the auxiliary flow uses the experts that the primary's
// router selected, with mixture weights of its own; "Contributi Chiave" item 3: the flows'
// expert fan-outs are independent settings).
//
// Readings: one shared router matrix scores both flows' normed rows; the primary's logits
// rank the experts (lower id first on ties); the primary takes the first k1, the auxiliary the
// first k2 of that ranking; each flow weights its experts by the softmax of its own logits
// over them; b couples each expert's intermediate where the primary also ran the expert, c the
// block output.
//
// Launches: norm + route (per sequence: both flows' normed rows, their router logits, the
// ranking, weights) -> lists (per expert: the sequences that use it, in ascending order) -> gather
// (each expert's rows in the grouped linear's fragment order; a flow that did not select the
// expert gets a zero row, so its intermediate is exactly zero) -> gate/up and down as the
// grouped linear in expert mode (an expert's weights are read once for every row of both
// flows that uses it, and not at all when no row does) -> combine (weighted sum of each row's
// experts in ranking order, c coupling, residual).
#include "common.h"

namespace dfx {

// One work-group of 16 waves per sequence: first both flows' rows are normalized (the shared
// norm helpers, so the rounding is the RMSNorm kernel's) into h; then wave w computes the
// router dot products d = w, w + 16, ... of the F * E (flow, expert) pairs (lane slices of 8,
// fixed order, wave butterfly); then wave 0 ranks the primary's logits by kmax rounds of a
// wave arg max and lane 0 forms each flow's weights. NaN logits rank last.
__global__ void __launch_bounds__(1024) moe_route_kernel(MoeArgs a) {
  __shared__ float red[2][16];
  __shared__ float lg[2][kMoeMaxExperts];
  __shared__ int32_t sel[kMoeMaxK];
  extern __shared__ u32x2 s_h[];  // the normed bf16 rows of both flows, 4 values per entry
  const int b = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int F = a.F, E = a.E, H = a.H;
  // This wave's first (flow, expert) router row does not depend on the norm: it is loaded
  // now, together with both flows' rows and the gain (one memory round trip), and each row is
  // then normed.
  constexpr int kPre = 8;  // router values per lane held: rows up to 512 kPre = 4096 wide
  const bool pre = wave < F * E && H <= 512 * kPre;
  u32x4 wpre[kPre];
  {
    const uint16_t *wr = a.w_router + (int64_t)(wave < F * E ? wave % E : 0) * H;
#pragma unroll
    for (int i = 0; i < kPre; ++i) wpre[i] = *(const u32x4 *)(wr + min(lane * 8 + 512 * i, H - 8));
  }
  f32x4 v[2][kNormSlices], gg[kNormSlices];
#pragma unroll
  for (int u = 0; u < kNormSlices; ++u) {
    const int i = threadIdx.x + 1024 * u;
    v[0][u] = v[1][u] = gg[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (4 * i < H) {
      gg[u] = *(const f32x4 *)(a.gain + 4 * i);
#pragma unroll
      for (int f = 0; f < 2; ++f)
        if (f < F) v[f][u] = *(const f32x4 *)(a.x + ((int64_t)f * a.B + b) * H + 4 * i);
    }
  }
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    if (f >= F) break;
    const int64_t row = (int64_t)f * a.B + b;
    const float r = norm_scale(v[f], H, a.eps, red[f]);
    // h = bf16(v * r * gain), to the workspace (the experts' rows are gathered from it) and
    // to LDS for the router's dot products
#pragma unroll
    for (int u = 0; u < kNormSlices; ++u) {
      const int i = threadIdx.x + 1024 * u;
      if (4 * i >= H) continue;
      const u32x2 o{pack_bf16x2(v[f][u][0] * r * gg[u][0], v[f][u][1] * r * gg[u][1]),
                    pack_bf16x2(v[f][u][2] * r * gg[u][2], v[f][u][3] * r * gg[u][3])};
      *(u32x2 *)(a.h + row * H + 4 * i) = o;
      s_h[f * (H / 4) + i] = o;
    }
  }
  __syncthreads();  // the normed rows are in LDS
  for (int d = wave; d < F * E; d += 16) {
    const int f = d / E, e = d % E;
    const u32x2 *hr = s_h + f * (H / 4);
    const uint16_t *wr = a.w_router + (int64_t)e * H;
    float acc = 0.f;
    auto dot8 = [&](int k, const u32x4 &wv) {
      const u32x2 h0 = hr[k / 4], h1 = hr[k / 4 + 1];
      const uint32_t hv[4] = {h0[0], h0[1], h1[0], h1[1]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = fmaf(bf16_lo(hv[i]), bf16_lo(wv[i]), acc);
        acc = fmaf(bf16_hi(hv[i]), bf16_hi(wv[i]), acc);
      }
    };
    if (d == wave && pre) {  // the prefetched row, in the same k order
#pragma unroll
      for (int i = 0; i < kPre; ++i)
        if (lane * 8 + 512 * i < H) dot8(lane * 8 + 512 * i, wpre[i]);
    } else {
#pragma unroll 8
      for (int k = lane * 8; k < H; k += 512) dot8(k, *(const u32x4 *)(wr + k));
    }
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) lg[f][e] = acc;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < F * E; i += 1024)
    a.logits[((int64_t)(i / E) * a.B + b) * E + i % E] = lg[i / E][i % E];
  if (wave != 0) return;
  const int kmax = F == 2 ? max(a.k1, a.k2) : a.k1;
  uint32_t taken = 0;  // bit t: expert lane + 64 t is already ranked
  for (int r = 0; r < kmax; ++r) {
    float bv = -INFINITY;
    int32_t bi = INT32_MAX;
    for (int t = 0; t < kMoeMaxExperts / 64; ++t) {
      const int e = lane + 64 * t;
      if (e >= E || ((taken >> t) & 1u)) continue;
      float v = lg[0][e];
      v = v == v ? v : -INFINITY;
      if (v > bv || (v == bv && e < bi)) {
        bv = v;
        bi = e;
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int32_t oi = __shfl_xor(bi, o);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == 0) sel[r] = bi;
  }
  if (lane != 0) return;
  for (int f = 0; f < F; ++f) {
    const int k = f == 0 ? a.k1 : a.k2;
    float m = -INFINITY;
    for (int j = 0; j < k; ++j) m = fmaxf(m, lg[f][sel[j]]);
    float s = 0.f;
    for (int j = 0; j < k; ++j) s += expf(lg[f][sel[j]] - m);
    const int64_t o = ((int64_t)f * a.B + b) * kMoeMaxK;
    for (int j = 0; j < kMoeMaxK; ++j) {
      a.ids[o + j] = j < k ? sel[j] : -1;
      a.wts[o + j] = j < k ? expf(lg[f][sel[j]] - m) / s : 0.f;
    }
  }
}

// One work-group: a bitmap [E][ceil(B / 32)] in LDS of the sequences using each expert (by
// either flow), then per expert the ascending list of those sequences and its length, and
// per (flow, sequence, rank) the row of that sequence in its expert's list.
__global__ void __launch_bounds__(1024) moe_lists_kernel(MoeArgs a) {
  extern __shared__ uint32_t bm[];
  const int W = (a.B + 31) / 32, E = a.E;
  for (int i = threadIdx.x; i < E * W; i += 1024) bm[i] = 0u;
  __syncthreads();
  const int n = a.F * a.B * kMoeMaxK;
  for (int t = threadIdx.x; t < n; t += 1024) {
    const int f = t / (a.B * kMoeMaxK), b = (t / kMoeMaxK) % a.B, j = t % kMoeMaxK;
    if (j >= (f == 0 ? a.k1 : a.k2)) continue;
    const int e = min(max(a.ids[t], 0), E - 1);
    atomicOr(&bm[e * W + b / 32], 1u << (b % 32));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 1024) {
    int c = 0;
    for (int w = 0; w < W; ++w) {
      uint32_t m = bm[e * W + w];
      while (m) {
        a.seqs[(int64_t)e * a.B + c++] = 32 * w + __ffs(m) - 1;
        m &= m - 1u;
      }
    }
    a.counts[e] = c;
  }
  for (int t = threadIdx.x; t < n; t += 1024) {
    const int f = t / (a.B * kMoeMaxK), b = (t / kMoeMaxK) % a.B, j = t % kMoeMaxK;
    if (j >= (f == 0 ? a.k1 : a.k2)) {
      a.pos[t] = -1;
      continue;
    }
    const int e = min(max(a.ids[t], 0), E - 1);
    int p = __popc(bm[e * W + b / 32] & ((1u << (b % 32)) - 1u));
    for (int w = 0; w < b / 32; ++w) p += __popc(bm[e * W + w]);
    a.pos[t] = p;
  }
}

__device__ __forceinline__ bool selects(const MoeArgs &a, int f, int b, int e) {
  const int k = f == 0 ? a.k1 : a.k2;
  const int32_t *ids = a.ids + ((int64_t)f * a.B + b) * kMoeMaxK;
  for (int j = 0; j < k; ++j)
    if (ids[j] == e) return true;
  return false;
}

// One thread per 8 columns of one row slot of one expert: the row of sequence seqs[e][r] of
// flow f if that flow selected e, else zeros, at its fragment-order position. Slots past the
// expert's count are left as they are (their outputs are never read).
__global__ void __launch_bounds__(256) moe_gather_kernel(MoeArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int k8 = a.H / 8;
  const int64_t total = (int64_t)a.E * a.max_groups * 64 * k8;
  if (t >= total) return;
  const int kc = (int)(t % k8);
  int64_t rest = t / k8;
  const int q = (int)(rest % 64);
  rest /= 64;
  const int grp = (int)(rest % a.max_groups), e = (int)(rest / a.max_groups);
  const int rpg = 64 / a.F, f = q / rpg, r = grp * rpg + q % rpg;
  if (f >= a.F || r >= a.counts[e]) return;
  const int b = min(max(a.seqs[(int64_t)e * a.B + r], 0), a.B - 1);
  u32x4 v{0u, 0u, 0u, 0u};
  if (selects(a, f, b, e)) v = *(const u32x4 *)(a.h + ((int64_t)f * a.B + b) * a.H + 8 * kc);
  *(u32x4 *)(a.xg + (int64_t)e * a.max_groups * 64 * a.H + xpack_offset(a.F, f, r, 8 * kc, a.H)) = v;
}

// One thread per 4 columns of one sequence (both flows): each flow's experts in ranking
// order, weight times the expert's output (its K-split tiles summed in split order), then the
// auxiliary's c coupling and the residual add, in place. The experts are taken kCombineJ at a
// time per flow: their ids, positions and weights in one round trip, then (one K split) their
// output tiles and the residual rows in another.
constexpr int kCombineJ = 4;

__global__ void __launch_bounds__(256) moe_combine_kernel(MoeArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int n4 = a.H / 4;
  if (t >= (int64_t)a.B * n4) return;
  const int col = (int)(t % n4) * 4, b = (int)(t / n4);
  const int rpg = 64 / a.F;
  const int kf[2] = {a.k1, a.F == 2 ? a.k2 : 0};
  const int kmax = max(kf[0], kf[1]);
  f32x4 m[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  for (int j0 = 0; j0 < kmax; j0 += kCombineJ) {
    int e[2][kCombineJ], r[2][kCombineJ];
    float w[2][kCombineJ];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int u = 0; u < kCombineJ; ++u) {  // entries past a flow's fan-out re-read its first
        const int64_t o = ((int64_t)min(f, a.F - 1) * a.B + b) * kMoeMaxK + (j0 + u < kf[f] ? j0 + u : 0);
        e[f][u] = min(max(a.ids[o], 0), a.E - 1);
        r[f][u] = min(max(a.pos[o], 0), a.B - 1);
        w[f][u] = a.wts[o];
      }
    f32x4 y[2][kCombineJ];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int u = 0; u < kCombineJ; ++u) {
        const float *tiles = a.tiles + (int64_t)e[f][u] * a.ksplit * a.max_groups * 64 * a.H;
        const int ff = min(f, a.F - 1), grp = r[f][u] / rpg, q = ff * rpg + r[f][u] % rpg;
        y[f][u] = a.ksplit == 1 ? *(const f32x4 *)(tiles + ((int64_t)grp * 64 + q) * a.H + col)
                                : sum_split_tiles(tiles, a.ksplit, a.max_groups, a.H, grp, q, col);
      }
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int u = 0; u < kCombineJ; ++u)
        if (j0 + u < kf[f])
#pragma unroll
          for (int i = 0; i < 4; ++i) m[f][i] = fmaf(w[f][u], y[f][u][i], m[f][i]);
  }
  if (a.F == 2 && a.couple_c) {
    const f32x4 c = *(const f32x4 *)(a.couple_c + col);
#pragma unroll
    for (int i = 0; i < 4; ++i) m[1][i] = fmaf(c[i], m[0][i], m[1][i]);
  }
  for (int f = 0; f < a.F; ++f) {
    float *xr = a.x + ((int64_t)f * a.B + b) * a.H + col;
    *(f32x4 *)xr = *(const f32x4 *)xr + m[f];
  }
}

hipError_t launch_moe(int which, const MoeArgs &a, hipStream_t s) {
  switch (which) {
    case kMoeRoute:
      moe_route_kernel<<<a.B, 1024, (size_t)a.F * a.H * sizeof(uint16_t), s>>>(a);
      break;
    case kMoeLists:
      moe_lists_kernel<<<1, 1024, (size_t)a.E * ((a.B + 31) / 32) * sizeof(uint32_t), s>>>(a);
      break;
    case kMoeGather: {
      const int64_t total = (int64_t)a.E * a.max_groups * 64 * (a.H / 8);
      moe_gather_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(a);
      break;
    }
    default: {
      const int64_t total = (int64_t)a.B * (a.H / 4);
      moe_combine_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(a);
      break;
    }
  }
  return hipGetLastError();
}

}  // namespace dfx
