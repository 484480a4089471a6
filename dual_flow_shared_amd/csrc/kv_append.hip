// Primary-only K/V append into the persistent cache.
//
// Only the primary flow writes the cache (Sintesi Tecnica: Dual-Flow Transformers,
// "Architettura Core"); the launcher takes no flow argument. One thread moves 8
// consecutive head-dim elements of one (sequence, KV head) row: a 16-byte bf16 store
// (after round-to-nearest-even from fp32 sources) or a 32-byte fp32 store.
#include "common.h"

namespace dfx {

template <bool POOL_BF16, bool SRC_F32>
__global__ void __launch_bounds__(256) kv_append_kernel(dfx_kv_cache kv, int32_t batch,
                                                        const int32_t *positions, int32_t minus_one,
                                                        const void *k_new, const void *v_new,
                                                        int64_t stride) {
  const int D = kv.head_dim, Hkv = kv.num_kv_heads, chunks = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)batch * Hkv * chunks * 2) return;
  const int which = (int)(idx & 1);  // 0: key row, 1: value row
  const int64_t rest = idx >> 1;
  const int c = (int)(rest % chunks), g = (int)((rest / chunks) % Hkv), b = (int)(rest / (chunks * Hkv));
  const bool paged = kv.block_table != nullptr;
  const int64_t cap = paged ? (int64_t)kv.max_blocks_per_seq * kv.block_size : kv.block_size;
  int64_t pos = (int64_t)positions[b] - minus_one;
  pos = pos < 0 ? 0 : (pos >= cap ? cap - 1 : pos);
  int64_t blk, slot;
  if (paged) {
    const uint32_t e = (uint32_t)kv.block_table[(int64_t)b * kv.max_blocks_per_seq + pos / kv.block_size];
    blk = (uint64_t)e < (uint64_t)kv.num_blocks ? (int64_t)e : kv.num_blocks - 1;
    slot = pos % kv.block_size;
  } else {
    blk = b;
    slot = pos;
  }
  const int64_t dst = ((blk * Hkv + g) * kv.block_size + slot) * D + 8 * c;
  const int64_t src = (int64_t)b * stride + (int64_t)g * D + 8 * c;
  const void *s = which ? v_new : k_new;
  void *pool = which ? kv.v : kv.k;
  float x[8];
  if constexpr (SRC_F32) {
    const f32x4 a = *(const f32x4 *)((const float *)s + src);
    const f32x4 bb = *(const f32x4 *)((const float *)s + src + 4);
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = bb[i]; }
  } else {
    const u32x4 w = *(const u32x4 *)((const uint16_t *)s + src);
    if constexpr (POOL_BF16) {
      *(u32x4 *)((uint16_t *)pool + dst) = w;
      return;
    }
    for (int i = 0; i < 4; ++i) { x[2 * i] = bf16_lo(w[i]); x[2 * i + 1] = bf16_hi(w[i]); }
  }
  if constexpr (POOL_BF16) {
    u32x4 w;
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    *(u32x4 *)((uint16_t *)pool + dst) = w;
  } else {
    *(f32x4 *)((float *)pool + dst) = f32x4{x[0], x[1], x[2], x[3]};
    *(f32x4 *)((float *)pool + dst + 4) = f32x4{x[4], x[5], x[6], x[7]};
  }
}

hipError_t launch_kv_append(const dfx_kv_cache &kv, int32_t batch, const int32_t *positions,
                            int32_t minus_one, int32_t src_f32, const void *k_new,
                            const void *v_new, int64_t stride, hipStream_t s) {
  const int64_t threads = (int64_t)batch * kv.num_kv_heads * (kv.head_dim / 8) * 2;
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  const bool pb = kv.dtype == DFX_BF16;
  if (pb && src_f32) kv_append_kernel<true, true><<<grid, block, 0, s>>>(kv, batch, positions, minus_one, k_new, v_new, stride);
  else if (pb) kv_append_kernel<true, false><<<grid, block, 0, s>>>(kv, batch, positions, minus_one, k_new, v_new, stride);
  else if (src_f32) kv_append_kernel<false, true><<<grid, block, 0, s>>>(kv, batch, positions, minus_one, k_new, v_new, stride);
  else kv_append_kernel<false, false><<<grid, block, 0, s>>>(kv, batch, positions, minus_one, k_new, v_new, stride);
  return hipGetLastError();
}

}  // namespace dfx
