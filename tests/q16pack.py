"""Test-side packer/unpacker of the PG_Q16 activation layout documented in
include/pingala.h (digits, per-block scale, per-half-block sums).  Written
from that description, independently of the library's kernels."""
from __future__ import annotations

import numpy as np


def row_bytes(k: int) -> int:
    raw = 2 * k + k // 32 + k // 16
    return (raw + 63) & ~63


def pack(q: np.ndarray, sx: np.ndarray) -> np.ndarray:
    """q int32 [rows][k] with |q| <= 32512, sx f32 [rows][k/128] -> u8
    [rows][row_bytes(k)]."""
    rows, k = q.shape
    out = np.zeros((rows, row_bytes(k)), dtype=np.uint8)
    hi = (q + 128) >> 8
    lo = q - 256 * hi
    assert np.all((lo >= -128) & (lo <= 127)) and np.all(np.abs(hi) <= 127)
    i = np.arange(k)
    off = (i // 16) * 32 + 4 * (i % 4) + (i // 4) % 4
    out[:, off] = hi.astype(np.int8).view(np.uint8)
    out[:, off + 16] = lo.astype(np.int8).view(np.uint8)
    out[:, 2 * k:2 * k + k // 32] = np.ascontiguousarray(sx, dtype=np.float32).view(np.uint8).reshape(rows, -1)
    sums = q.reshape(rows, k // 64, 64).sum(axis=2).astype(np.int32)
    out[:, 2 * k + k // 32:2 * k + k // 32 + k // 16] = sums.view(np.uint8).reshape(rows, -1)
    return out


def unpack(buf: np.ndarray, k: int):
    """-> (q int32 [rows][k], sx f32 [rows][k/128], half-block sums int32)."""
    rows = buf.shape[0]
    i = np.arange(k)
    off = (i // 16) * 32 + 4 * (i % 4) + (i // 4) % 4
    hi = buf[:, off].view(np.int8).astype(np.int32)
    lo = buf[:, off + 16].view(np.int8).astype(np.int32)
    q = 256 * hi + lo
    sx = np.ascontiguousarray(buf[:, 2 * k:2 * k + k // 32]).view(np.float32).reshape(rows, k // 128)
    sums = np.ascontiguousarray(buf[:, 2 * k + k // 32:2 * k + k // 32 + k // 16]).view(np.int32).reshape(rows, k // 64)
    return q, sx, sums


def dequant(q: np.ndarray, sx: np.ndarray) -> np.ndarray:
    rows, k = q.shape
    return (q.reshape(rows, k // 128, 128).astype(np.float64) * sx.astype(np.float64)[..., None]).reshape(rows, k)


def random_q16(rows: int, k: int, seed: int):
    """Seeded Q16 activations: q uniform in [-32512, 32512] with one value per
    block at the bound, sx = |N(0,1)| / 32512-ish per block."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-32512, 32513, (rows, k), dtype=np.int64).astype(np.int32)
    q.reshape(rows, k // 128, 128)[:, :, 0] = 32512
    sx = (np.abs(rng.standard_normal((rows, k // 128))) * 3.0 / 32512).astype(np.float32)
    return q, sx
