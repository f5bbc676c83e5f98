"""Byte image of the paged K/V pools (oracle; test infrastructure only).

The pages fix only that each block holds the keys and values of a handful of
tokens and that blocks may sit anywhere in memory ("Paged Attention: Virtual
Memory for the KV Cache", §The fix borrowed from operating systems;
"Paged Attention as a Memory Manager", §Virtual Memory as the Blueprint).  The
layout inside a block is the library's own published contract (head-major,
so each (block, kv head) tile is one contiguous run of BS*D elements):

    K pool  [num_blocks][Hkv][D / X][BS][X]    X = 16 bytes / element size
    V pool  [num_blocks][Hkv][D][BS]

slot s = block * BS + offset.  Token t of a write lands in block s // BS at
offset s % BS; a negative slot is skipped.  Copying a block copies the whole
K and V tile of every head, padding included.

Storage holds raw bit patterns (uint16 for f16/bf16, uint32 for f32) so pool
images compare bit for bit; unwritten storage holds a quiet-NaN poison.
"""
from __future__ import annotations

import numpy as np

__all__ = ["PagedCacheModel", "POISON", "encode", "decode"]

POISON = {"bf16": 0x7FC0, "f16": 0x7E00, "f32": 0x7FC00000}
_BITS = {"bf16": np.uint16, "f16": np.uint16, "f32": np.uint32}
_ESIZE = {"bf16": 2, "f16": 2, "f32": 4}


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values exactly representable in dtype -> raw bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.view(np.uint32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        bits = x.view(np.uint32)
        if np.any(bits & np.uint32(0xFFFF)):
            raise ValueError("value not representable in bf16")
        return (bits >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dtype)


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """raw bits -> float64 values (exact)."""
    if dtype == "f32":
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


class PagedCacheModel:
    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int,
                 dtype: str):
        self.N, self.H, self.D, self.BS, self.dtype = num_blocks, num_kv_heads, head_dim, block_size, dtype
        self.X = 16 // _ESIZE[dtype]
        if head_dim % self.X:
            raise ValueError("head_dim must be a multiple of 16 bytes")
        bt = _BITS[dtype]
        self.k = np.full((num_blocks, num_kv_heads, head_dim // self.X, block_size, self.X),
                         POISON[dtype], dtype=bt)
        self.v = np.full((num_blocks, num_kv_heads, head_dim, block_size), POISON[dtype], dtype=bt)

    def write(self, slots, k_new, v_new) -> None:
        """k_new/v_new [T, Hkv, D] float32 (exact in dtype); slots [T]."""
        slots = np.asarray(slots, dtype=np.int64)
        keep = slots >= 0
        s = slots[keep]
        if s.size == 0:
            return
        if np.unique(s).size != s.size:
            raise ValueError("duplicate slots in one write")
        if s.max() >= self.N * self.BS:
            raise ValueError("slot out of range")
        kb = encode(np.asarray(k_new)[keep], self.dtype)          # [T, H, D]
        vb = encode(np.asarray(v_new)[keep], self.dtype)
        blk, off = s // self.BS, s % self.BS
        T = s.size
        # K[b, h, d // X, o, d % X] = k[t, h, d]
        kx = kb.reshape(T, self.H, self.D // self.X, self.X)
        self.k[blk, :, :, off, :] = kx
        # V[b, h, d, o] = v[t, h, d]
        self.v[blk, :, :, off] = vb

    def copy_blocks(self, pairs) -> None:
        """Whole-block copies (src, dst), applied in order."""
        for src, dst in pairs:
            self.k[dst] = self.k[src]
            self.v[dst] = self.v[src]

    def gather(self, table, n: int):
        """Logical K, V [n, Hkv, D] float64 of a sequence of length n whose
        block table is ``table`` (entries past ceil(n/BS) are ignored)."""
        nb = -(-n // self.BS)
        tab = np.asarray(table[:nb], dtype=np.int64)
        if nb and (tab.min() < 0 or tab.max() >= self.N):
            raise ValueError("table entry out of range")
        t = np.arange(n)
        blk, off = tab[t // self.BS], t % self.BS
        kbits = self.k[blk, :, :, off, :].reshape(n, self.H, self.D)   # [n, H, D/X, X]
        vbits = self.v[blk, :, :, off]                                  # [n, H, D]
        return decode(kbits, self.dtype), decode(vbits, self.dtype)

    def pool_bits(self):
        return self.k, self.v
