// Shared-weight projections of a prompt chunk (prefill, one flow): Y = bf16(X) W^T over many
// rows, a dense contraction on the matrix cores.
//
// Operands are the grouped linear's packed layouts: W [K/32][N/16][64 lanes][8] (the A
// fragment of a 16x16x32 bf16 MFMA for 16 output features and one 32-wide k-step, 1 KiB
// contiguous) and X [M/64][K/32][4][64 lanes][8] (the B fragment of 16 rows likewise).
// Two work-group tiles, each putting two waves on every SIMD (one can issue MFMAs while the
// other waits): 256 output features x 128 rows as 4 x 2 waves of 64 features x 64 rows (two
// work-groups per CU), and 256 x 256 as 2 x 4 waves of 128 x 64 (one per CU). Per k-step a
// work-group stages the fragments it needs (16 of W and 8 or 16 of X, 1 KiB each) in LDS,
// each loaded once from global memory straight into LDS (global_load_lds, no register
// staging) two k-steps ahead; every wave reads its fragments from LDS and issues 16 or 32
// MFMAs. LDS holds three k-steps: the one being read and the two in flight (one barrier per
// k-step).
//
// Work-group i runs on XCD i % 8; all row tiles of one feature tile go to one XCD back to back,
// so the tile's weights are fetched from HBM about once and re-read from that XCD's L2.
//
// Epilogues: fp32 rows [M][N] (plus a residual that may alias them), or, in gate/up mode, the
// work-group's 256 features are 128 gate features and their 128 up features (the gate rows of
// W come first; a wave holds 32 or 64 gate features and their up features) and it writes bf16
// silu(gate) * up rows in the packed X layout of the next projection (K = N / 2).
#include "common.h"

namespace dfx {

// Work-group tile: FWAVES x RWAVES waves, each owning FW feature fragments (16 features each)
// x RW row fragments (16 rows each; a multiple of 4, i.e. whole 64-row groups), with the
// fragments of AHEAD k-steps in flight (LDS slots: AHEAD + 1).
template <int FW_, int RW_, int FWAVES_, int RWAVES_, int AHEAD_ = 2>
struct DenseTile {
  static constexpr int FW = FW_, RW = RW_, FWAVES = FWAVES_, RWAVES = RWAVES_, Ahead = AHEAD_;
  static constexpr int Slots = Ahead + 1;
  static constexpr int WFrags = FW * FWAVES;          // W fragments per k-step
  static constexpr int XFrags = RW * RWAVES;          // X fragments per k-step
  static constexpr int Frags = WFrags + XFrags;
  static constexpr int Waves = FWAVES * RWAVES;
  static constexpr int Stage = Frags / Waves;         // fragments a thread stages per k-step
  static constexpr int Groups = XFrags / 4;           // 64-row groups per row tile
  static constexpr int Features = 16 * WFrags;        // output features per tile (gate/up: half gate)
  static_assert(Frags % Waves == 0 && RW % 4 == 0 && FW % 2 == 0, "tile shape");
  static_assert(Ahead >= 2 && (Ahead - 1) * Stage < 16, "loads outstanding at each wait (vmcnt bits 3:0)");
};
// 256 features x 128 rows over 8 waves of 64 x 64 (two work-groups per CU)
using TileNarrow = DenseTile<4, 4, 4, 2>;
// 256 features x 256 rows over 8 waves of 128 x 64 (one work-group per CU, 96 KiB of LDS):
// 1.5x the flops per byte staged through LDS, 1.37x per byte read from LDS
using TileWide = DenseTile<8, 4, 2, 4>;

template <class T>
__device__ __forceinline__ int dense_col_tiles(int N, bool swiglu) {
  return swiglu ? (N / 2 + T::Features / 2 - 1) / (T::Features / 2) : (N + T::Features - 1) / T::Features;
}

template <class T, bool SWIGLU>
__global__ void __launch_bounds__(64 * T::Waves) __attribute__((amdgpu_waves_per_eu(2)))
prefill_gemm_kernel(PrefillGemmArgs p) {
  constexpr int FW = T::FW, RW = T::RW, kWFrags = T::WFrags, kStage = T::Stage;
  __shared__ u32x4 lds[T::Slots][T::Frags][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;
  const int wr = wave / T::FWAVES, wc = wave % T::FWAVES;  // row wave, feature wave
  const int M = p.M, K = p.K, N = p.N;
  const int nks = K / 32, ng = N / 16, ngh = ng / 2, groups = (M + 63) / 64;
  const int RT = (groups + T::Groups - 1) / T::Groups;
  const int CT = dense_col_tiles<T>(N, SWIGLU);
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
  // this thread stages fragments f = wave + Waves r, lane `lane` of each
  const uint16_t *src[kStage];
  int64_t sstep[kStage];
#pragma unroll
  for (int r = 0; r < kStage; ++r) {
    const int f = wave + T::Waves * r;
    if (f < kWFrags) {
      src[r] = p.w + ((int64_t)wgroup(f) * 64 + lane) * 8;
      sstep[r] = (int64_t)ng * 512;
    } else {
      const int xf = f - kWFrags;
      const int grp = min(T::Groups * rt + xf / 4, groups - 1), nb = xf % 4;
      src[r] = p.x + (((int64_t)grp * nks * 4 + nb) * 64 + lane) * 8;
      sstep[r] = 4 * 512;
    }
  }
  // this wave's weight fragments in LDS (gate/up mode: FW/2 gate groups, then their up groups)
  int wfrag[FW];
#pragma unroll
  for (int c = 0; c < FW; ++c)
    wfrag[c] = SWIGLU ? (c < FW / 2 ? (FW / 2) * wc + c : kWFrags / 2 + (FW / 2) * wc + c - FW / 2)
                      : FW * wc + c;

  f32x4 acc[FW][RW];
#pragma unroll
  for (int c = 0; c < FW; ++c)
#pragma unroll
    for (int nb = 0; nb < RW; ++nb) acc[c][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Fragments go from global memory straight to LDS (16 bytes per lane; a fragment's 64 lanes
  // are 1 KiB contiguous in LDS) Ahead k-steps ahead. Waits are explicit: this thread's loads
  // of k-step s are done once at most (Ahead - 1) kStage loads (those of s + 1 ..) are
  // outstanding; the barrier then makes k-step s's slot complete for every wave, and every
  // wave has finished reading the slot that the loads of s + Ahead overwrite. Those loads are
  // issued after this wave's LDS reads of k-step s (measured: 2% faster than before them).
  typedef __attribute__((address_space(3))) void lds_void;
  auto dma = [&](int st, int slot) {
    const int sc = min(st, nks - 1);  // past the last k-step: re-read it (never used)
#pragma unroll
    for (int r = 0; r < kStage; ++r)
      __builtin_amdgcn_global_load_lds((const void *)(src[r] + sc * sstep[r]),
                                       (lds_void *)&lds[slot][wave + T::Waves * r][0], 16, 0, 0);
  };
  // s_waitcnt immediates (vmcnt in bits 3:0, expcnt and lgkmcnt fields at their no-wait maxima)
  constexpr int kWaitNext = (T::Ahead - 1) * kStage | (0x7 << 4) | (0xF << 8);
  constexpr int kWaitAll = 0 | (0x7 << 4) | (0xF << 8);
#pragma unroll
  for (int st = 0; st < T::Ahead; ++st) dma(st, st);
  int slot = 0;
  for (int s = 0; s < nks; ++s) {
    __builtin_amdgcn_s_waitcnt(kWaitNext);
    __builtin_amdgcn_s_barrier();
    u32x4 wf[FW], xf[RW];
#pragma unroll
    for (int c = 0; c < FW; ++c) wf[c] = lds[slot][wfrag[c]][lane];
#pragma unroll
    for (int nb = 0; nb < RW; ++nb) xf[nb] = lds[slot][kWFrags + RW * wr + nb][lane];
    dma(s + T::Ahead, slot == 0 ? T::Slots - 1 : slot - 1);
#pragma unroll
    for (int c = 0; c < FW; ++c)
#pragma unroll
      for (int nb = 0; nb < RW; ++nb)
        acc[c][nb] = mfma16x16x32(as_bf16x8(wf[c]), as_bf16x8(xf[nb]), acc[c][nb]);
    slot = slot == T::Slots - 1 ? 0 : slot + 1;
  }
  __builtin_amdgcn_s_waitcnt(kWaitAll);  // no load into LDS in flight when the work-group ends

  // C layout: lane holds row 16 q + n of the tile's row fragment q = RW wr + nb and features
  // 16 g + 4 j .. + 3
  const int row0 = 16 * (T::XFrags * rt + RW * wr) + n;
  if constexpr (SWIGLU) {
    const int I = N / 2;
#pragma unroll
    for (int c = 0; c < FW / 2; ++c) {
      const int g = ct * (kWFrags / 2) + (FW / 2) * wc + c;
      if (g >= ngh) continue;
      const int col = 16 * g + 4 * j;
#pragma unroll
      for (int nb = 0; nb < RW; ++nb) {
        const int row = row0 + 16 * nb;
        if (row >= M) continue;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = silu(acc[c][nb][i]) * acc[c + FW / 2][nb][i];
        *(u32x2 *)((uint16_t *)p.y + xpack_offset(1, 0, row, col, I)) =
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < FW; ++c) {
      const int g = ct * kWFrags + FW * wc + c;
      if (g >= ng) continue;
      const int col = 16 * g + 4 * j;
#pragma unroll
      for (int nb = 0; nb < RW; ++nb) {
        const int row = row0 + 16 * nb;
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

template <class T>
static int64_t dense_grid(const PrefillGemmArgs &a, bool swiglu);

template <class T>
static hipError_t launch_dense(const PrefillGemmArgs &a, bool swiglu, hipStream_t s) {
  const dim3 grid((unsigned)dense_grid<T>(a, swiglu)), block(64 * T::Waves);
  if (swiglu) prefill_gemm_kernel<T, true><<<grid, block, 0, s>>>(a);
  else prefill_gemm_kernel<T, false><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

template <class T>
static int64_t dense_grid(const PrefillGemmArgs &a, bool swiglu) {
  const int groups = (a.M + 63) / 64, RT = (groups + T::Groups - 1) / T::Groups;
  const int CT = swiglu ? (a.N / 2 + T::Features / 2 - 1) / (T::Features / 2)
                        : (a.N + T::Features - 1) / T::Features;
  return 8 * (int64_t)((CT + 7) / 8) * RT;  // 8 x the work-groups of the busiest XCD
}

hipError_t launch_prefill_gemm(const PrefillGemmArgs &a, bool swiglu, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  // The wide tile runs one work-group per CU. Where its grid ends in a partly filled round of
  // 256 work-groups (Q/K/V at 4096 rows: 384), the narrow tile was measured faster (231 vs
  // 243 us); on whole rounds the wide one is (gate/up 876 vs 886 us, W_o and W_down 392 vs
  // 422 us on average, 4096 rows).
  if (dense_grid<TileWide>(a, swiglu) % 256 == 0) return launch_dense<TileWide>(a, swiglu, s);
  return launch_dense<TileNarrow>(a, swiglu, s);
}

}  // namespace dfx
