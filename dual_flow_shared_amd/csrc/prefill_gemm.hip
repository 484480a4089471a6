// Shared-weight projections of a prompt chunk (prefill, one flow): Y = bf16(X) W^T over many
// rows, a dense contraction on the matrix cores.
//
// Operands are the grouped linear's packed layouts: W [K/32][N/16][64 lanes][8] (the A
// fragment of a 16x16x32 bf16 MFMA for 16 output features and one 32-wide k-step, 1 KiB
// contiguous) and X [M/64][K/32][4][64 lanes][8] (the B fragment of 16 rows likewise).
// A work-group owns 256 output features x 128 rows as 2 x 4 waves of 64 features x 64 rows
// (two waves per SIMD, so one can issue MFMAs while the other waits). Per k-step it stages the 24
// fragments it needs (16 of W, 8 of X; 24 KiB) in LDS, each loaded once from global memory
// straight into LDS (global_load_lds, no register staging) two k-steps ahead; every wave reads
// its 8 fragments from LDS and issues 16 MFMAs. LDS holds three k-steps: the one being read and
// the two in flight (one barrier per k-step).
//
// Work-group i runs on XCD i % 8; all row tiles of one feature tile go to one XCD back to back,
// so the tile's weights are fetched from HBM about once and re-read from that XCD's L2.
//
// Epilogues: fp32 rows [M][N] (plus a residual that may alias them), or, in gate/up mode, the
// work-group's 256 features are 128 gate features and their 128 up features (the gate rows of
// W come first; a wave holds 32 gate features and their up features) and it writes bf16
// silu(gate) * up rows in the packed X layout of the next projection (K = N / 2).
#include "common.h"

namespace dfx {

constexpr int kDenseAhead = 2;  // k-steps of fragments in flight (LDS slots: kDenseAhead + 1)
// feature waves (64 features each) per work-group; 2 (128 x 128 per work-group, 4 waves) ran
// the prefill layer in 2.59 ms against 2.10
constexpr int kFeatWaves = 4;
constexpr int kWFrags = 4 * kFeatWaves;    // W fragments per k-step (16 features each)
constexpr int kDenseFrags = kWFrags + 8;   // plus 8 X fragments (2 row groups of 64)

constexpr int kDenseWaves = 2 * kFeatWaves;  // 2 row waves x kFeatWaves feature waves
constexpr int kDenseStage = kDenseFrags * 64 / (64 * kDenseWaves);  // fragments a thread stages
static_assert(kDenseFrags % kDenseWaves == 0, "staging");

template <bool SWIGLU>
__global__ void __launch_bounds__(64 * kDenseWaves) prefill_gemm_kernel(PrefillGemmArgs p) {
  __shared__ u32x4 lds[kDenseAhead + 1][kDenseFrags][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;
  const int wr = wave / kFeatWaves, wc = wave % kFeatWaves;  // row group of the tile, feature wave
  const int M = p.M, K = p.K, N = p.N;
  const int nks = K / 32, ng = N / 16, ngh = ng / 2, groups = (M + 63) / 64;
  const int RT = (groups + 1) / 2;
  const int CT = SWIGLU ? (N / 2 + 32 * kFeatWaves - 1) / (32 * kFeatWaves)
                        : (N + 64 * kFeatWaves - 1) / (64 * kFeatWaves);
  const int xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
  const int ct = xcd + 8 * (idx / RT), rt = idx % RT;
  if (ct >= CT) return;  // uniform for the work-group, before any barrier

  // global feature group of the work-group's feature group fg (0 .. kWFrags - 1)
  auto wgroup = [&](int fg) {
    if (SWIGLU) {
      const int g = min(ct * (kWFrags / 2) + fg % (kWFrags / 2), ngh - 1);
      return fg < kWFrags / 2 ? g : g + ngh;
    }
    return min(ct * kWFrags + fg, ng - 1);
  };
  // this thread stages fragments f = wave + kDenseWaves r, lane `lane` of each
  const uint16_t *src[kDenseStage];
  int64_t sstep[kDenseStage];
#pragma unroll
  for (int r = 0; r < kDenseStage; ++r) {
    const int f = wave + kDenseWaves * r;
    if (f < kWFrags) {
      src[r] = p.w + ((int64_t)wgroup(f) * 64 + lane) * 8;
      sstep[r] = (int64_t)ng * 512;
    } else {
      const int grp = min(2 * rt + (f - kWFrags) / 4, groups - 1), nb = (f - kWFrags) % 4;
      src[r] = p.x + (((int64_t)grp * nks * 4 + nb) * 64 + lane) * 8;
      sstep[r] = 4 * 512;
    }
  }
  // this wave's weight fragments in LDS (gate/up mode: 2 gate groups and their 2 up groups)
  int wfrag[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    wfrag[c] = SWIGLU ? (c < 2 ? 2 * wc + c : kWFrags / 2 + 2 * wc + c - 2) : 4 * wc + c;

  f32x4 acc[4][4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[c][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Fragments go from global memory straight to LDS (16 bytes per lane; a fragment's 64 lanes
  // are 1 KiB contiguous in LDS) kDenseAhead k-steps ahead. Waits are explicit: this thread's
  // loads of k-step s are done once at most kDenseStage loads (those of s + 1) are outstanding;
  // the barrier then makes k-step s's slot complete for every wave, and every wave has finished
  // reading the slot that the loads of s + 2 overwrite. Those loads are issued after this
  // wave's LDS reads of k-step s (measured: 2% faster than before them).
  static_assert(kDenseAhead == 2 && kDenseStage < 16, "one k-step of loads outstanding at each wait");
  typedef __attribute__((address_space(3))) void lds_void;
  auto dma = [&](int st, int slot) {
    const int sc = min(st, nks - 1);  // past the last k-step: re-read it (never used)
#pragma unroll
    for (int r = 0; r < kDenseStage; ++r)
      __builtin_amdgcn_global_load_lds((const void *)(src[r] + sc * sstep[r]),
                                       (lds_void *)&lds[slot][wave + kDenseWaves * r][0], 16, 0, 0);
  };
  // s_waitcnt immediates (vmcnt in bits 3:0, expcnt and lgkmcnt fields at their no-wait maxima)
  constexpr int kWaitNext = kDenseStage | (0x7 << 4) | (0xF << 8);
  constexpr int kWaitAll = 0 | (0x7 << 4) | (0xF << 8);
  dma(0, 0);
  dma(1, 1);
  int slot = 0;
  for (int s = 0; s < nks; ++s) {
    __builtin_amdgcn_s_waitcnt(kWaitNext);
    __builtin_amdgcn_s_barrier();
    u32x4 wf[4], xf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) wf[c] = lds[slot][wfrag[c]][lane];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) xf[nb] = lds[slot][kWFrags + 4 * wr + nb][lane];
    dma(s + 2, slot == 0 ? 2 : slot - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[c][nb] = mfma16x16x32(as_bf16x8(wf[c]), as_bf16x8(xf[nb]), acc[c][nb]);
    slot = slot == 2 ? 0 : slot + 1;
  }
  __builtin_amdgcn_s_waitcnt(kWaitAll);  // no load into LDS in flight when the work-group ends

  // C layout: lane holds row 16 nb + n of its group and features 16 cg + 4 j .. + 3
  const int grp = 2 * rt + wr;
  if (grp >= groups) return;
  if constexpr (SWIGLU) {
    const int I = N / 2;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int g = ct * (kWFrags / 2) + 2 * wc + c;
      if (g >= ngh) continue;
      const int col = 16 * g + 4 * j;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int row = 64 * grp + 16 * nb + n;
        if (row >= M) continue;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = silu(acc[c][nb][i]) * acc[c + 2][nb][i];
        *(u32x2 *)((uint16_t *)p.y + xpack_offset(1, 0, row, col, I)) =
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int g = ct * kWFrags + 4 * wc + c;
      if (g >= ng) continue;
      const int col = 16 * g + 4 * j;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int row = 64 * grp + 16 * nb + n;
        if (row >= M) continue;
        const int64_t o = (int64_t)row * N + col;
        f32x4 v = acc[c][nb];
        if (p.residual) v += *(const f32x4 *)(p.residual + o);
        *(f32x4 *)((float *)p.y + o) = v;
      }
    }
  }
}

bool prefill_gemm_fits(int32_t K, int32_t N, bool swiglu) {
  return K % 32 == 0 && N % (swiglu ? 32 : 16) == 0;
}

hipError_t launch_prefill_gemm(const PrefillGemmArgs &a, bool swiglu, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  const int groups = (a.M + 63) / 64, RT = (groups + 1) / 2;
  const int CT = swiglu ? (a.N / 2 + 32 * kFeatWaves - 1) / (32 * kFeatWaves)
                        : (a.N + 64 * kFeatWaves - 1) / (64 * kFeatWaves);
  const int64_t per_xcd = (int64_t)((CT + 7) / 8) * RT;  // work-groups of the busiest XCD
  const dim3 grid((unsigned)(8 * per_xcd)), block(64 * kDenseWaves);
  if (swiglu) prefill_gemm_kernel<true><<<grid, block, 0, s>>>(a);
  else prefill_gemm_kernel<false><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dfx
