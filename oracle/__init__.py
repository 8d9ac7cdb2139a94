"""CPU oracle for the paged KV write and paged varlen attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package; the product path (``paged_kv_attention_05_amd``) never
does, and shares no code with it.

The arithmetic lives in ``paged_oracle.c`` (plain float64 loops, written from the pages'
``write_kv`` and ``ReferenceBackend.forward`` in "Engine v2: one core for every request",
section "Attention over the pool"); this module only marshals numpy arrays into it.

Arrays: float32 data is ``np.float32``; bfloat16 data is carried as its 16-bit patterns in
``np.uint16`` and flagged with ``dtype="bf16"``.

Every function here has a pin in ``tests/test_oracle_*.py`` that does not reuse this code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "paged_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_LIB = None

DTYPES = {"f32": 0, "bf16": 1}


def build(force: bool = False) -> str:
    """Compile paged_oracle.c into liboracle.so with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load_library(path: str):
    """Load a compiled oracle library and declare its entry points."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.oracle_kv_write.restype = ctypes.c_int
    lib.oracle_kv_write.argtypes = [P, P, P, P, P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    lib.oracle_gather_context.restype = None
    lib.oracle_gather_context.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, P]
    lib.oracle_paged_attention.restype = ctypes.c_int
    lib.oracle_paged_attention.argtypes = [P, P, P, P, P, P, ctypes.c_int32, ctypes.c_double, P, P,
                                           ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int64, ctypes.c_int32, P, ctypes.c_int32, ctypes.c_int32, P, P]
    lib.oracle_kv_write_fp8.restype = ctypes.c_int
    lib.oracle_kv_write_fp8.argtypes = [P, P, P, P, P, P, P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int64, ctypes.c_int32]
    lib.oracle_fp8_e4m3_decode.restype = ctypes.c_double
    lib.oracle_fp8_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_fp8_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_fp8_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_copy_blocks.restype = ctypes.c_int
    lib.oracle_copy_blocks.argtypes = [P, P, P, P, ctypes.c_int64, ctypes.c_int64]
    lib.oracle_round_to_bf16.restype = ctypes.c_uint16
    lib.oracle_round_to_bf16.argtypes = [ctypes.c_double]
    return lib


def _lib():
    global _LIB
    if _LIB is None:
        build()
        _LIB = load_library(_LIB_PATH)
    return _LIB


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _check_data(a: np.ndarray, dtype: str, name: str) -> None:
    want = np.float32 if dtype == "f32" else np.uint16
    if a.dtype != want or not a.flags.c_contiguous:
        raise TypeError(f"{name}: expected C-contiguous {np.dtype(want).name} for dtype {dtype}")


def round_to_bf16(x: float) -> int:
    """bfloat16 bit pattern of a float64 value, round-to-nearest-even."""
    return int(_lib().oracle_round_to_bf16(float(x)))


def kv_write(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray, k_cache: np.ndarray,
             v_cache: np.ndarray, in_dtype: str, cache_dtype: str) -> None:
    """write_kv: copy k, v [N, Hkv, D] into the pools [NB+1, bs, Hkv, D] at the flat slots.

    A negative slot goes to the pool's last slot.  Mutates k_cache and v_cache in place.
    """
    _check_data(k, in_dtype, "k")
    _check_data(v, in_dtype, "v")
    _check_data(k_cache, cache_dtype, "k_cache")
    _check_data(v_cache, cache_dtype, "v_cache")
    slot_mapping = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    n, hkv, d = k.shape
    num_slots = k_cache.shape[0] * k_cache.shape[1]
    rc = _lib().oracle_kv_write(_ptr(k), _ptr(v), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache),
                                n, hkv, d, num_slots, DTYPES[in_dtype], DTYPES[cache_dtype])
    if rc != 0:
        raise ValueError("oracle kv_write: slot out of range")


def fp8_e4m3_encode(y: float) -> int:
    """Nearest fp8 E4M3 (OCP FN) code of a float32 value, ties to even, saturating at 448."""
    return int(_lib().oracle_fp8_e4m3_encode(float(np.float32(y))))


def fp8_e4m3_decode(code: int) -> float:
    return float(_lib().oracle_fp8_e4m3_decode(int(code)))


def kv_write_fp8(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                 k_scale: np.ndarray, v_scale: np.ndarray, in_dtype: str) -> None:
    """write_kv into quantized pools: codes into k_cache / v_cache ([NB+1, bs, Hkv, D] uint8),
    scales into k_scale / v_scale ([NB+1, bs, Hkv] float32); negative slots go to the last."""
    _check_data(k, in_dtype, "k")
    _check_data(v, in_dtype, "v")
    for name, a, dt in (("k_cache", k_cache, np.uint8), ("v_cache", v_cache, np.uint8),
                        ("k_scale", k_scale, np.float32), ("v_scale", v_scale, np.float32)):
        if a.dtype != dt or not a.flags.c_contiguous:
            raise TypeError(f"{name}: expected C-contiguous {np.dtype(dt).name}")
    slot_mapping = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    n, hkv, d = k.shape
    num_slots = k_cache.shape[0] * k_cache.shape[1]
    rc = _lib().oracle_kv_write_fp8(_ptr(k), _ptr(v), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(k_scale), _ptr(v_scale), n, hkv, d, num_slots, DTYPES[in_dtype])
    if rc != 0:
        raise ValueError("oracle kv_write_fp8: slot out of range")


def copy_blocks(src: np.ndarray, dst: np.ndarray, src_block: np.ndarray, dst_block: np.ndarray) -> None:
    """swap_out / swap_in / copy-on-write: block dst_block[i] of dst becomes block src_block[i]
    of src, pairs in order.  src and dst are C-contiguous arrays whose first axis is the block
    (they may be the same array); dst is modified in place."""
    if not (src.flags.c_contiguous and dst.flags.c_contiguous):
        raise ValueError("src and dst must be C-contiguous")
    bb = src.nbytes // src.shape[0]
    if dst.nbytes // dst.shape[0] != bb:
        raise ValueError("src and dst blocks differ in size")
    sb = np.ascontiguousarray(src_block, dtype=np.int64)
    db = np.ascontiguousarray(dst_block, dtype=np.int64)
    if sb.shape != db.shape:
        raise ValueError("src_block and dst_block differ in length")
    if sb.size and (sb.max() >= src.shape[0] or db.max() >= dst.shape[0]):
        raise ValueError("block id out of range")
    if _lib().oracle_copy_blocks(_ptr(src), _ptr(dst), _ptr(sb), _ptr(db), sb.size, bb) != 0:
        raise ValueError("negative block id")


def gather_context(cache: np.ndarray, table_row: np.ndarray, length: int, dtype: str) -> np.ndarray:
    """First `length` rows of one request's context in logical order, float64 [length, Hkv, D]."""
    _check_data(cache, dtype, "cache")
    table_row = np.ascontiguousarray(table_row, dtype=np.int32)
    bs, hkv, d = cache.shape[1], cache.shape[2], cache.shape[3]
    out = np.empty((length, hkv, d), dtype=np.float64)
    _lib().oracle_gather_context(_ptr(cache), _ptr(table_row), length, bs, hkv, d, DTYPES[dtype], _ptr(out))
    return out


def paged_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                    query_start_loc: np.ndarray, seq_lens: np.ndarray, block_table: np.ndarray,
                    scale: float, dtype: str, row_mask: Optional[np.ndarray] = None,
                    want_f64: bool = False, window: int = 0, k_scale: Optional[np.ndarray] = None,
                    v_scale: Optional[np.ndarray] = None):
    """ReferenceBackend.forward over the pool.

    q [N, H, D]; caches [NB+1, bs, Hkv, D]; query_start_loc [R+1]; seq_lens [R];
    block_table [R, W].  Returns out [N, H, D] in `dtype` (and the float64 result if
    want_f64).  With row_mask, only the selected flattened rows are computed; the others
    are left at zero (and NaN in the float64 result) so they cannot pass for results.
    window > 0: a row at position p sees only keys p - window + 1 .. p (the sliding window
    of ReferenceBackend.forward); 0 sees every key up to p.
    With k_scale / v_scale ([NB+1, bs, Hkv] float32) the caches are fp8 E4M3 codes (uint8)
    and every gathered row is its codes' values times its scale (ReferenceBackend.dequantize).
    """
    _check_data(q, dtype, "q")
    fp8 = k_scale is not None
    if fp8:
        for name, a in (("k_cache", k_cache), ("v_cache", v_cache)):
            if a.dtype != np.uint8 or not a.flags.c_contiguous:
                raise TypeError(f"{name}: expected C-contiguous uint8 fp8 codes")
        k_scale = np.ascontiguousarray(k_scale, dtype=np.float32)
        v_scale = np.ascontiguousarray(v_scale, dtype=np.float32)
        if k_scale.shape != k_cache.shape[:3] or v_scale.shape != v_cache.shape[:3]:
            raise ValueError("scales must be [NB+1, bs, Hkv]")
    else:
        _check_data(k_cache, dtype, "k_cache")
        _check_data(v_cache, dtype, "v_cache")
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    table = np.ascontiguousarray(block_table, dtype=np.int32)
    n, h, d = q.shape
    hkv, bs = k_cache.shape[2], k_cache.shape[1]
    num_slots = k_cache.shape[0] * bs
    out = np.zeros_like(q)
    out64 = np.full(q.shape, np.nan, dtype=np.float64) if want_f64 else None
    mask = None if row_mask is None else np.ascontiguousarray(row_mask, dtype=np.uint8)
    rc = _lib().oracle_paged_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(qsl), _ptr(lens),
                                       _ptr(table), bs, float(scale), _ptr(out), _ptr(out64),
                                       len(lens), n, h, hkv, d, table.shape[1], num_slots,
                                       DTYPES[dtype], _ptr(mask), int(window), 2 if fp8 else DTYPES[dtype],
                                       _ptr(k_scale), _ptr(v_scale))
    if rc == -1:
        raise ValueError("oracle paged_attention: inconsistent batch metadata")
    if rc != 0:
        raise MemoryError("oracle paged_attention: allocation failed")
    return (out, out64) if want_f64 else out
