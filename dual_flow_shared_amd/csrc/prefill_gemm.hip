// Shared-weight projections of a prompt chunk (prefill, one flow): Y = bf16(X) W^T over many
// rows, a dense contraction on the matrix cores.
//
// Operands are the grouped linear's packed layouts: W [K/32][N/16][64 lanes][8] (the A
// fragment of a 16x16x32 bf16 MFMA for 16 output features and one 32-wide k-step, 1 KiB
// contiguous) and X [M/64][K/32][4][64 lanes][8] (the B fragment of 16 rows likewise).
// Per k-step a work-group stages the fragments it needs (1 KiB each) in LDS, each loaded once
// from global memory straight into LDS (global_load_lds, no register staging) k-steps ahead;
// every wave reads its fragments from LDS and issues its MFMAs; one barrier per k-step.
// Work-group tiles:
// - 256 output features x 256 rows as 2 x 2 waves of 128 x 128 (and 192 x 256 as 2 x 2 waves of
//   96 x 128), one wave per SIMD. Per k-step a wave reads 16 (14) fragments from LDS for 64 (48)
//   MFMAs: a third fewer LDS reads per MFMA than 8 waves of 128 x 64, which matters because the
//   chip runs at a power-limited clock under matrix load. The accumulators fill (three quarters
//   of) the 256 matrix registers; the k-loop is register-buffered (fragments of k-step s + 1 are
//   read while the MFMAs of s run) with the loads spread between the MFMAs, since no second wave
//   on the SIMD covers them.
// - 256 x 128 as 4 x 2 waves of 64 x 64, two work-groups per CU, for grids that would end in a
//   partly filled round of the larger tiles.
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
// REGBUF: fragments are read from LDS one k-step ahead into a second register set (AHEAD >= 3).
template <int FW_, int RW_, int FWAVES_, int RWAVES_, int AHEAD_ = 2, bool REGBUF_ = false>
struct DenseTile {
  static constexpr int FW = FW_, RW = RW_, FWAVES = FWAVES_, RWAVES = RWAVES_, Ahead = AHEAD_;
  static constexpr bool RegBuf = REGBUF_;
  // waves of the work-group per SIMD: the register budget (512 per lane over this count)
  static constexpr int WavesPerSimd = (FWAVES_ * RWAVES_ + 3) / 4;
  static constexpr int Slots = Ahead + 1;
  static constexpr int WFrags = FW * FWAVES;          // W fragments per k-step
  static constexpr int XFrags = RW * RWAVES;          // X fragments per k-step
  static constexpr int Frags = WFrags + XFrags;
  static constexpr int Waves = FWAVES * RWAVES;
  static constexpr int Stage = Frags / Waves;         // fragments a thread stages per k-step
  static constexpr int Groups = XFrags / 4;           // 64-row groups per row tile
  static constexpr int Features = 16 * WFrags;        // output features per tile (gate/up: half gate)
  static_assert(Frags % Waves == 0 && RW % 4 == 0 && FW % 2 == 0, "tile shape");
  static_assert(Ahead >= 2 && (Ahead - 1) * Stage < 64, "loads outstanding at each wait (6-bit vmcnt)");
  static_assert(!RegBuf || Ahead >= 3, "a register-buffered k-loop reads LDS one step ahead of the MFMAs");
  static_assert(!RegBuf || WavesPerSimd == 1, "the register-buffered k-loop keeps its accumulators in place by asm");
};
// 256 features x 128 rows over 8 waves of 64 x 64 (two work-groups per CU)
using TileNarrow = DenseTile<4, 4, 4, 2>;
// 256 (192) features x 256 rows over 4 waves of 128 (96) x 128: one wave per SIMD, four LDS
// slots (128 / 112 KiB)
using TileQuad = DenseTile<8, 8, 2, 2, 3, true>;
using TileQuad6 = DenseTile<6, 8, 2, 2, 3, true>;

// s_waitcnt immediate on gfx9: vmcnt bits 3:0 and 15:14, expcnt and lgkmcnt at their no-wait maxima
constexpr int waitcnt_vm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// acc += W.X^T with the accumulator tied in place to one matrix-register quadruple (with 256
// accumulator registers the compiler's own allocation rotates them through copies). Only for
// k-loops whose operands come straight from LDS loads: the compiler does not see the asm as a
// matrix instruction, so the caller waits out its latency before anything reads the accumulators.
__device__ __forceinline__ void mfma_agpr(f32x4 &acc, const u32x4 &a, const u32x4 &b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

template <class T>
__device__ __forceinline__ int dense_col_tiles(int N, bool swiglu) {
  return swiglu ? (N / 2 + T::Features / 2 - 1) / (T::Features / 2) : (N + T::Features - 1) / T::Features;
}

template <class T, bool SWIGLU>
__global__ void __launch_bounds__(64 * T::Waves) __attribute__((amdgpu_waves_per_eu(T::WavesPerSimd)))
prefill_gemm_kernel(PrefillGemmArgs p) {
  constexpr int FW = T::FW, RW = T::RW, kWFrags = T::WFrags, kStage = T::Stage;
  __shared__ u32x4 lds[T::Slots][T::Frags][64];
  // the wave index in a scalar register, so that the per-wave fragment strides and offsets are too
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
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
  constexpr int kWaitNext = waitcnt_vm((T::Ahead - 1) * kStage);
  constexpr int kWaitAll = waitcnt_vm(0);
#pragma unroll
  for (int st = 0; st < T::Ahead; ++st) dma(st, st);
  if constexpr (T::RegBuf) {
    // Fragments of k-step s + 1 are read from LDS while the MFMAs of k-step s run from the
    // other register set. LDS holds four k-steps: s + 1 (being read), s + 2 and s + 3 (in
    // flight), and the slot of s (already in registers), which the loads of s + 4 overwrite
    // one step later. At the top of step s this thread's loads of s + 1 are done (those of
    // s + 2 may be outstanding); the barrier makes s + 1 complete for every wave and shows
    // that every wave has read k-step s's slot into registers.
    // One wave per SIMD: nothing else covers this wave's loads, so they are spread over its
    // MFMAs (an LDS read of k-step s + 1 after every 3, a global-to-LDS load of k-step s + Ahead
    // after every 8 or 6), each held in place between empty asm memory fences.
    constexpr int kWaitRead = waitcnt_vm((T::Ahead - 2) * kStage);
    constexpr int kReadEvery = 3, kDmaEvery = FW * RW / kStage;
    static_assert(kReadEvery * (FW + RW) <= FW * RW && kDmaEvery >= 1, "interleave pattern");
    u32x4 wa[FW], xa[RW], wb[FW], xb[RW];
    auto step = [&](int s, const u32x4 (&wc)[FW], const u32x4 (&xc)[RW], u32x4 (&wn)[FW], u32x4 (&xn)[RW]) {
      __builtin_amdgcn_s_waitcnt(kWaitRead);
      __builtin_amdgcn_s_barrier();
      const int sl = (s + 1) % T::Slots;  // past the last k-step: the re-read copy of it (never used)
      const int sc = min(s + T::Ahead, nks - 1), dslot = (s + T::Ahead) % T::Slots;
#pragma unroll
      for (int c = 0; c < FW; ++c)
#pragma unroll
        for (int nb = 0; nb < RW; ++nb) {
          mfma_agpr(acc[c][nb], wc[c], xc[nb]);
          const int i = c * RW + nb;
          if (i % kReadEvery == kReadEvery - 1 && i / kReadEvery < FW + RW) {
            const int q = i / kReadEvery;
            asm volatile("" ::: "memory");
            if (q < FW) wn[q] = lds[sl][wfrag[q]][lane];
            else xn[q - FW] = lds[sl][kWFrags + RW * wr + q - FW][lane];
            asm volatile("" ::: "memory");
          }
          if (i % kDmaEvery == kDmaEvery - 1 && i / kDmaEvery < kStage) {
            const int r = i / kDmaEvery;
            asm volatile("" ::: "memory");
            __builtin_amdgcn_global_load_lds((const void *)(src[r] + sc * sstep[r]),
                                             (lds_void *)&lds[dslot][wave + T::Waves * r][0], 16, 0, 0);
            asm volatile("" ::: "memory");
          }
        }
    };
    __builtin_amdgcn_s_waitcnt(kWaitNext);  // k-step 0 is in LDS
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int c = 0; c < FW; ++c) wa[c] = lds[0][wfrag[c]][lane];
#pragma unroll
    for (int nb = 0; nb < RW; ++nb) xa[nb] = lds[0][kWFrags + RW * wr + nb][lane];
    int s = 0;
    for (; s + 1 < nks; s += 2) {
      step(s, wa, xa, wb, xb);
      step(s + 1, wb, xb, wa, xa);
    }
    if (s < nks) step(s, wa, xa, wb, xb);
    // the last MFMAs' results are ready 24 wait states later (a 16-pass one needs 19); every
    // accumulator then passes through an empty asm ordered after the wait, so that no read of
    // it can be scheduled earlier
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int c = 0; c < FW; ++c)
#pragma unroll
      for (int nb = 0; nb < RW; ++nb) asm volatile("" : "+a"(acc[c][nb]));
  } else {
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
    // The residual may alias the output, so the compiler keeps each residual load after every
    // earlier store; loaded one tile at a time, every load is a memory round trip of its own.
    // Every element is read and written by its lane alone, so the residual tiles of two feature
    // fragments are loaded together (rows past M clamped: loaded, never stored), then stored.
    constexpr int kBatch = 2;
    const bool rows_full = 16 * (T::XFrags * rt + RW * wr + RW) <= M;  // uniform for the wave
#pragma unroll
    for (int c0 = 0; c0 < FW; c0 += kBatch) {
      f32x4 res[kBatch][RW];
      if (p.residual) {
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const int g = min(ct * kWFrags + FW * wc + c0 + b, ng - 1);
#pragma unroll
          for (int nb = 0; nb < RW; ++nb)
            res[b][nb] = *(const f32x4 *)(p.residual + (int64_t)min(row0 + 16 * nb, M - 1) * N + 16 * g + 4 * j);
        }
      }
      // a wave whose rows are all below M stores without per-row branches (the compiler waits
      // for every load at each divergent store otherwise); only the last row tile checks rows
      auto store = [&](bool check_rows) {
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const int g = ct * kWFrags + FW * wc + c0 + b;
          if (g >= ng) continue;
          const int col = 16 * g + 4 * j;
#pragma unroll
          for (int nb = 0; nb < RW; ++nb) {
            const int row = row0 + 16 * nb;
            if (check_rows && row >= M) continue;
            f32x4 v = acc[c0 + b][nb];
            if (p.residual) v += res[b][nb];
            *(f32x4 *)((float *)p.y + (int64_t)row * N + col) = v;
          }
        }
      };
      if (rows_full) store(false);
      else store(true);
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
  // The four-wave tiles run one work-group per CU, so they are taken where their grid fills
  // whole rounds of 256 work-groups (at 4096 rows: gate/up, W_o and W_down on 256 features,
  // Q/K/V's 6144 on 192); elsewhere the narrow tile, two work-groups per CU.
  if (dense_grid<TileQuad>(a, swiglu) % 256 == 0) return launch_dense<TileQuad>(a, swiglu, s);
  if (!swiglu && dense_grid<TileQuad6>(a, swiglu) % 256 == 0) return launch_dense<TileQuad6>(a, swiglu, s);
  return launch_dense<TileNarrow>(a, swiglu, s);
}

}  // namespace dfx
