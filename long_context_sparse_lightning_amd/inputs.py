"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds no LSA arithmetic: it only turns (seed, tensor tag, flat element index)
into values.  The generator is counter based, so any element (or any set of rows) can be
produced on its own, on the host or on the GPU, and both give identical bits.

Definition (the numpy functions below are the normative version; the native fills in
``csrc/lsa_gen.hip`` must match them bit for bit, which ``tests/test_inputs.py`` checks):

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014; finaliser constants as published by Vigna):
  ``mix(z) = z ^= z>>30; z *= 0xBF58476D1CE4E5B9; z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31``
  and the i-th output of a stream with state ``base`` is ``mix(base + (i+1)*GAMMA)``,
  ``GAMMA = 0x9E3779B97F4A7C15`` (all arithmetic mod 2**64).
* Stream of a tensor: ``base = mix(seed*256 + tag)``; element ``i`` of the row-major flattened
  tensor uses output ``i``.
* Kinds:
  - ``DYADIC`` (bf16): ``((h mod 7) - 3) / 4``, i.e. one of {-0.75, ..., 0.75}; exact in bf16.
    Products and sums of these are exact in fp32 at the indexer's sizes, so indexer scores
    are bit-reproducible in any summation order.
  - ``WEIGHT`` (fp32): ``(1 + h mod 4) / 8``, i.e. one of {0.125, 0.25, 0.375, 0.5}.
  - ``NORMAL`` (bf16): unit-variance stand-in for N(0,1): the sum ``s`` of the four 16-bit
    fields of ``h`` (Irwin-Hall with n = 4) centred and scaled, ``z = (s - 131070) * C`` in
    fp64 with ``C = 1/sqrt(4*(65536**2 - 1)/12)``, rounded to fp32 and then to bf16 (both round
    to nearest even).  Only correctly rounded IEEE operations are involved, so host and GPU
    agree exactly (Box-Muller would need log/cos, whose last bit differs between libraries).
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MUL1 = 0xBF58476D1CE4E5B9
MUL2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

DYADIC, WEIGHT, NORMAL = 0, 1, 2
KIND_NAMES = {"dyadic": DYADIC, "weight": WEIGHT, "normal": NORMAL}

# tensor tags
TAGS = {"qidx": 1, "w": 2, "kidx": 3, "q": 4, "kv0": 5, "kv1": 6, "q1": 7, "scores": 8,
        # indexer front end: q-LoRA representation, hidden state, projections, key-norm gain
        "cq": 9, "hid": 10, "wq_b": 11, "wk": 12, "w_proj": 13, "k_gain": 14,
        # third multi-token-prediction draft query
        "q2": 15}

NORMAL_SCALE = 1.0 / math.sqrt(4.0 * (65536.0 * 65536.0 - 1.0) / 12.0)


def _mix_int(z: int) -> int:
    z &= MASK64
    z ^= z >> 30
    z = (z * MUL1) & MASK64
    z ^= z >> 27
    z = (z * MUL2) & MASK64
    z ^= z >> 31
    return z


def stream_base(seed: int, tag: int) -> int:
    """State of the SplitMix64 stream that generates tensor ``tag`` under ``seed``."""
    return _mix_int((seed * 256 + tag) & MASK64)


def _mix_np(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * np.uint64(MUL1)
    z = z ^ (z >> np.uint64(27))
    z = z * np.uint64(MUL2)
    return z ^ (z >> np.uint64(31))


def hashes(seed: int, tag: int, flat_idx: np.ndarray) -> np.ndarray:
    """64-bit outputs for the given flat element indices (numpy reference version)."""
    base = np.uint64(stream_base(seed, tag))
    idx = np.asarray(flat_idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix_np(base + (idx + np.uint64(1)) * np.uint64(GAMMA))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def values_from_hashes(h: np.ndarray, kind: int) -> np.ndarray:
    """Map hashes to values: uint16 bf16 bits for DYADIC/NORMAL, float32 for WEIGHT."""
    if kind == DYADIC:
        v = (h % np.uint64(7)).astype(np.int64) - 3
        return f32_to_bf16_bits(v.astype(np.float32) * np.float32(0.25))
    if kind == WEIGHT:
        v = (h % np.uint64(4)).astype(np.int64) + 1
        return v.astype(np.float32) * np.float32(0.125)
    if kind == NORMAL:
        m = np.uint64(0xFFFF)
        s = (h & m) + ((h >> np.uint64(16)) & m) + ((h >> np.uint64(32)) & m) + (h >> np.uint64(48))
        z = (s.astype(np.int64) - 131070).astype(np.float64) * NORMAL_SCALE
        return f32_to_bf16_bits(z.astype(np.float32))
    raise ValueError(f"unknown kind {kind}")


def ref_tensor(seed: int, tag: int, shape, kind: int) -> np.ndarray:
    """Whole tensor through the numpy reference path (small tensors only)."""
    n = int(np.prod(shape))
    return values_from_hashes(hashes(seed, tag, np.arange(n, dtype=np.uint64)), kind).reshape(shape)


# ---------------------------------------------------------------- native fills (fast paths)
_gen = None


def _lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblsa_gen.so")


def gen_lib():
    global _gen
    if _gen is None:
        path = _lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        lib.lsa_gen_fill_host.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double]
        lib.lsa_gen_fill_host.restype = ctypes.c_int
        lib.lsa_gen_fill_host_rows.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                               ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                               ctypes.c_double]
        lib.lsa_gen_fill_host_rows.restype = ctypes.c_int
        lib.lsa_gen_fill_device.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                            ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double,
                                            ctypes.c_void_p]
        lib.lsa_gen_fill_device.restype = ctypes.c_int
        _gen = lib
    return _gen


def _np_dtype(kind: int):
    return np.float32 if kind == WEIGHT else np.uint16


def host_tensor(seed: int, tag: int, shape, kind: int, start: int = 0) -> np.ndarray:
    """Tensor of ``shape`` whose element j is stream output ``start + j`` (native host loop)."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=_np_dtype(kind))
    if out.size:
        rc = gen_lib().lsa_gen_fill_host(out.ctypes.data, kind, stream_base(seed, tag), start,
                                         out.size, NORMAL_SCALE)
        if rc != 0:
            raise RuntimeError(f"lsa_gen_fill_host failed ({rc})")
    return out


def host_rows(seed: int, tag: int, row_ids, row_len: int, kind: int) -> np.ndarray:
    """Rows ``row_ids`` (indices into the tensor viewed as [-1, row_len]) -> [len(row_ids), row_len]."""
    rows = np.ascontiguousarray(np.asarray(row_ids, dtype=np.uint64))
    out = np.empty((rows.size, int(row_len)), dtype=_np_dtype(kind))
    if out.size:
        rc = gen_lib().lsa_gen_fill_host_rows(out.ctypes.data, kind, stream_base(seed, tag),
                                              rows.ctypes.data, rows.size, int(row_len),
                                              NORMAL_SCALE)
        if rc != 0:
            raise RuntimeError(f"lsa_gen_fill_host_rows failed ({rc})")
    return out


def device_tensor(seed: int, tag: int, shape, kind: int, device="cuda"):
    """Tensor generated directly in device memory (torch is used for the allocation only)."""
    import torch

    dtype = torch.float32 if kind == WEIGHT else torch.bfloat16
    t = torch.empty(tuple(int(s) for s in shape), dtype=dtype, device=device)
    if t.numel():
        stream = torch.cuda.current_stream(t.device).cuda_stream
        rc = gen_lib().lsa_gen_fill_device(t.data_ptr(), kind, stream_base(seed, tag), 0,
                                           t.numel(), NORMAL_SCALE, ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"lsa_gen_fill_device failed ({rc})")
    return t


def as_bf16_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact)."""
    return bf16_bits_to_f32(bits).astype(np.float64)
