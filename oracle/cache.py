"""Primary-only K/V append into the persistent cache (oracle).

Only the primary flow writes the cache; the auxiliary flow reads it and never
writes (Sintesi Tecnica: Dual-Flow Transformers, "Architettura Core"). The
new key and value rows of sequence b go to logical position positions[b]:
pool[blk][g][p % block_size] with blk = block_table[b][p // block_size]
(sequence b's own block b without a table). Stored as bf16 by round to
nearest even when the pool is bf16.
"""
import numpy as np

from .numerics import bf16_bits, widen


def kv_append(k_pool, v_pool, block_table, positions, k_new, v_new):
    """Return copies of the pools with row positions[b] of every sequence written.

    k_new, v_new: [B][Hkv*D] (float32/float64 values or uint16 bf16 bits).
    """
    kp, vp = k_pool.copy(), v_pool.copy()
    nb, Hkv, bs, D = kp.shape
    for b, p in enumerate(np.asarray(positions)):
        p = int(p)
        if block_table is None:
            blk, slot = b, p
        else:
            blk, slot = int(block_table[b][p // bs]), p % bs
        for pool, src in ((kp, k_new), (vp, v_new)):
            row = np.asarray(src[b])
            if pool.dtype == np.uint16:
                bits = row if row.dtype == np.uint16 else bf16_bits(widen(row))
                pool[blk, :, slot, :] = bits.reshape(Hkv, D)
            else:
                pool[blk, :, slot, :] = widen(row).reshape(Hkv, D).astype(np.float32)
    return kp, vp
