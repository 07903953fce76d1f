"""Counter-based and stream-based generators (no step of the method lives here)."""

from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

MASTER_SEED = 20261026
MASK32 = 0xFFFFFFFF
_M1 = 0x7FEB352D
_M2 = 0x846CA68B


@dataclass(frozen=True)
class StreamKey:
    """Two 32-bit words that select one counter-based stream."""

    k1: int
    k2: int

    @property
    def seed64(self) -> int:
        return (self.k1 << 32) | self.k2


def stream_key(*names) -> StreamKey:
    """Derive an independent stream from the master seed and a tuple of names."""
    text = repr((MASTER_SEED,) + tuple(names)).encode()
    d = hashlib.blake2b(text, digest_size=8).digest()
    return StreamKey(int.from_bytes(d[:4], "little"), int.from_bytes(d[4:], "little"))


def rng_np(key: StreamKey) -> np.random.Generator:
    """A NumPy PCG64 stream for small host-side draws."""
    return np.random.Generator(np.random.PCG64(key.seed64))


# ---------------------------------------------------------------- mixer (NumPy)
def _mix32_np(x: np.ndarray) -> np.ndarray:
    x = x & MASK32
    x ^= x >> np.uint64(16)
    x = (x * np.uint64(_M1)) & MASK32
    x ^= x >> np.uint64(15)
    x = (x * np.uint64(_M2)) & MASK32
    x ^= x >> np.uint64(16)
    return x


def _hash_np(key: StreamKey, idx: np.ndarray) -> np.ndarray:
    x = (idx.astype(np.uint64) + np.uint64(key.k1)) & np.uint64(MASK32)
    x = _mix32_np(x)
    x ^= np.uint64(key.k2)
    return _mix32_np(x)


# ---------------------------------------------------------------- mixer (torch)
def _mulmod32_t(x, c: int):
    # (x * c) mod 2^32 for 0 <= x < 2^32 without leaving the int64 range.
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & MASK32


def _mix32_t(x):
    x = x ^ (x >> 16)
    x = _mulmod32_t(x, _M1)
    x = x ^ (x >> 15)
    x = _mulmod32_t(x, _M2)
    x = x ^ (x >> 16)
    return x


def _hash_t(key: StreamKey, idx):
    x = (idx + key.k1) & MASK32
    x = _mix32_t(x)
    x = x ^ key.k2
    return _mix32_t(x)


# ---------------------------------------------------------------- normal table
_TABLE: np.ndarray | None = None


def _f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def normal_bf16_table() -> np.ndarray:
    """BF16 bit patterns of the 65536 standard-normal quantiles (midpoint rule)."""
    global _TABLE
    if _TABLE is None:
        from scipy.special import ndtri

        j = np.arange(65536, dtype=np.float64)
        q = ndtri((j + 0.5) / 65536.0).astype(np.float32)
        _TABLE = _f32_to_bf16_bits_rne(q)
        _TABLE.setflags(write=False)
    return _TABLE


def normal_bf16_np(key: StreamKey, count: int, start: int = 0) -> np.ndarray:
    """Elements ``start .. start+count-1`` of a BF16 N(0,1) stream, as uint16 bits."""
    assert 0 <= start and start + count <= (1 << 32)
    idx = np.arange(start, start + count, dtype=np.uint64)
    h = _hash_np(key, idx)
    return normal_bf16_table()[(h >> np.uint64(16)).astype(np.int64)]


def normal_bf16_at_np(key: StreamKey, idx: np.ndarray) -> np.ndarray:
    """The stream's elements at arbitrary flat indices ``idx`` (uint16 BF16 bits)."""
    idx = np.asarray(idx, dtype=np.uint64)
    assert idx.size == 0 or int(idx.max()) < (1 << 32)
    h = _hash_np(key, idx)
    return normal_bf16_table()[(h >> np.uint64(16)).astype(np.int64)]


def normal_bf16_torch_(out, key: StreamKey, start: int = 0, chunk: int = 1 << 26) -> None:
    """Fill the contiguous 16-bit tensor ``out`` with the same stream, on out's device.

    ``out`` may have dtype int16, uint16 or bfloat16; its bits receive the draw
    for flat indices ``start .. start+out.numel()-1``.
    """
    import torch

    n = out.numel()
    assert out.is_contiguous() and out.element_size() == 2
    assert 0 <= start and start + n <= (1 << 32)
    flat = out.view(torch.int16).view(-1)
    table = torch.from_numpy(normal_bf16_table().view(np.int16).copy()).to(out.device)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        idx = torch.arange(start + c0, start + c1, dtype=torch.int64, device=out.device)
        h = _hash_t(key, idx)
        flat[c0:c1] = table[h >> 16]
        del idx, h


def normal_f32_np(key: StreamKey, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """FP32 draws of N(mean, std^2) from a PCG64 stream (host)."""
    z = rng_np(key).standard_normal(size=shape)
    return (mean + std * z).astype(np.float32)


def distinct_ints_np(key: StreamKey, count: int, lo: int, hi: int) -> np.ndarray:
    """``count`` distinct integers drawn uniformly from [lo, hi) (a uniform random subset)."""
    assert hi - lo >= count
    return (rng_np(key).choice(hi - lo, size=count, replace=False) + lo).astype(np.int32)


def bf16_bits_to_f32_np(bits: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns to float32 (used only to summarise drawn inputs)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- FP8 (E4M3) codes
_E4M3_TABLE: np.ndarray | None = None
E4M3_SPREAD = 128.0  # a N(0,1) quantile q is stored as the code nearest to 128 * q


def normal_e4m3_table() -> np.ndarray:
    """OCP E4M3 codes of the 65536 standard-normal quantiles times 128, clipped to
    the format's largest finite magnitude 448 (torch's float8_e4m3fn cast, nearest
    even).  Stored with a row scale near 1/128, a code decodes to about N(0,1)."""
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        import torch
        from scipy.special import ndtri

        j = np.arange(65536, dtype=np.float64)
        q = np.clip(ndtri((j + 0.5) / 65536.0) * E4M3_SPREAD, -448.0, 448.0).astype(np.float32)
        t = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
        assert not np.any((t & 0x7F) == 0x7F)  # no NaN code
        _E4M3_TABLE = t
        _E4M3_TABLE.setflags(write=False)
    return _E4M3_TABLE


def normal_e4m3_np(key: StreamKey, count: int, start: int = 0) -> np.ndarray:
    """Elements ``start .. start+count-1`` of an E4M3 code stream (uint8)."""
    assert 0 <= start and start + count <= (1 << 32)
    idx = np.arange(start, start + count, dtype=np.uint64)
    return normal_e4m3_table()[(_hash_np(key, idx) >> np.uint64(16)).astype(np.int64)]


def normal_e4m3_torch_(out, key: StreamKey, start: int = 0, chunk: int = 1 << 26) -> None:
    """Fill the contiguous 8-bit tensor ``out`` with the same code stream."""
    import torch

    n = out.numel()
    assert out.is_contiguous() and out.element_size() == 1
    assert 0 <= start and start + n <= (1 << 32)
    flat = out.view(torch.uint8).view(-1)
    table = torch.from_numpy(normal_e4m3_table().copy()).to(out.device)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        idx = torch.arange(start + c0, start + c1, dtype=torch.int64, device=out.device)
        flat[c0:c1] = table[_hash_t(key, idx) >> 16]
        del idx


def row_scale_np(key: StreamKey, count: int, start: int = 0, denom: int = 512) -> np.ndarray:
    """FP32 row scales in [3/denom, 4/denom) (denom a power of two): (3 + u) / denom with
    u = (hash >> 10) / 2^22, every operation exact in FP32 (so host and device streams
    agree bit for bit)."""
    assert 0 <= start and start + count <= (1 << 32) and denom & (denom - 1) == 0
    idx = np.arange(start, start + count, dtype=np.uint64)
    u = (_hash_np(key, idx) >> np.uint64(10)).astype(np.float32) * np.float32(2.0 ** -22)
    return ((np.float32(3.0) + u) * np.float32(1.0 / denom)).astype(np.float32)


def row_scale_torch_(out, key: StreamKey, start: int = 0, chunk: int = 1 << 24,
                     denom: int = 512) -> None:
    """Fill the contiguous FP32 tensor ``out`` with the same scale stream."""
    import torch

    n = out.numel()
    assert out.is_contiguous() and out.dtype == torch.float32
    assert 0 <= start and start + n <= (1 << 32) and denom & (denom - 1) == 0
    flat = out.view(-1)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        idx = torch.arange(start + c0, start + c1, dtype=torch.int64, device=out.device)
        u = (_hash_t(key, idx) >> 10).to(torch.float32) * (2.0 ** -22)
        flat[c0:c1] = (u + 3.0) * (1.0 / denom)
        del idx, u


# ---------------------------------------------------------------- INT8 code streams
I8_SPREAD = 36.0  # codes ~ N(0, 36^2), clipped at 127 (3.5 sigma)
_I8_TABLE = None


def normal_i8_table() -> np.ndarray:
    """Signed 8-bit codes (as uint8 bytes) of the 65536 standard-normal quantiles times
    36, rounded to nearest and clipped to [-127, 127].  With a row scale near 1/36 (the
    scale stream with denom 128) a code stands for about N(0,1)."""
    global _I8_TABLE
    if _I8_TABLE is None:
        from scipy.special import ndtri

        j = np.arange(65536, dtype=np.float64)
        q = np.clip(np.rint(ndtri((j + 0.5) / 65536.0) * I8_SPREAD), -127, 127)
        _I8_TABLE = q.astype(np.int8).view(np.uint8).copy()
        _I8_TABLE.setflags(write=False)
    return _I8_TABLE


def normal_i8_np(key: StreamKey, count: int, start: int = 0) -> np.ndarray:
    """Elements ``start .. start+count-1`` of an INT8 code stream (uint8 bytes)."""
    assert 0 <= start and start + count <= (1 << 32)
    idx = np.arange(start, start + count, dtype=np.uint64)
    return normal_i8_table()[(_hash_np(key, idx) >> np.uint64(16)).astype(np.int64)]


def normal_i8_torch_(out, key: StreamKey, start: int = 0, chunk: int = 1 << 26) -> None:
    """Fill the contiguous 8-bit tensor ``out`` with the same code stream."""
    import torch

    n = out.numel()
    assert out.is_contiguous() and out.element_size() == 1
    assert 0 <= start and start + n <= (1 << 32)
    flat = out.view(torch.uint8).view(-1)
    table = torch.from_numpy(normal_i8_table().copy()).to(out.device)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        idx = torch.arange(start + c0, start + c1, dtype=torch.int64, device=out.device)
        flat[c0:c1] = table[_hash_t(key, idx) >> 16]
        del idx


# ---------------------------------------------------------------- FP16 / FP32 state streams
def scaled_normal_np(key: StreamKey, count: int, start: int = 0, scale: float = 0.125,
                     dtype=np.float16) -> np.ndarray:
    """BF16 N(0,1) stream values times a power of two, stored as float16 (nearest
    even) or float32 (exact)."""
    x = bf16_bits_to_f32_np(normal_bf16_np(key, count, start)) * np.float32(scale)
    return x.astype(dtype)


def scaled_normal_torch_(out, key: StreamKey, scale: float = 0.125, chunk: int = 1 << 26) -> None:
    """Fill the contiguous float16/float32 tensor ``out`` with the same values."""
    import torch

    n = out.numel()
    assert out.is_contiguous() and out.dtype in (torch.float16, torch.float32)
    flat = out.view(-1)
    tmp = torch.empty(min(n, chunk), dtype=torch.bfloat16, device=out.device)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        t = tmp[:c1 - c0]
        normal_bf16_torch_(t, key, start=c0)
        flat[c0:c1] = (t.float() * scale).to(out.dtype)
