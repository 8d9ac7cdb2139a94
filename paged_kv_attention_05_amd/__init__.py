"""Paged KV write and paged varlen attention for MI355X (gfx950), behind a C ABI.

This module only marshals torch tensors into ``libpagedattn.so`` (built in place by
``build.py``); every step of the computation runs in its HIP kernels.  Torch supplies
device memory and the current stream.  If the library is missing, every call raises:
there is no fallback.

Names follow the C ABI in ``include/paged_attn.h``:
    paged_kv_write(k, v, slot_mapping, k_cache, v_cache)
    paged_attention_varlen(q, k_cache, v_cache, query_start_loc, seq_lens, block_table,
                           block_size, scale, out, query_start_loc_host=..., seq_lens_host=...,
                           sliding_window=0)     (calls paged_attention_varlen_ex)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")

PA_DTYPE = {torch.float32: 0, torch.bfloat16: 1}
PA_DTYPE_FP8_E4M3 = 2
NOALLOC_SCRATCH_BYTES = 64 << 20     # PA_NOALLOC_SCRATCH_BYTES of the C ABI
ERRORS = {-1: "PA_ERR_NULL", -2: "PA_ERR_SHAPE", -3: "PA_ERR_DTYPE", -4: "PA_ERR_METADATA",
          -5: "PA_ERR_WORKSPACE", -6: "PA_ERR_LAUNCH", -7: "PA_ERR_RANGE"}
EXPORTS = ["paged_kv_write", "paged_kv_write_fp8", "paged_copy_blocks", "paged_attention_varlen", "paged_attention_workspace_bytes",
           "paged_attention_varlen_ex", "paged_attention_workspace_bytes_ex", "paged_attention_varlen_noalloc",
           "paged_attn_last_error", "paged_attn_set_debug_checks", "paged_attn_set_path",
           "paged_attn_set_timing", "paged_attn_timing_report", "paged_hbm_read_probe", "paged_mfma_probe"]
KINDS = ["kv_write", "plan", "prefill", "small", "merge"]

_lib = None


class AttentionOptions(ctypes.Structure):
    """pa_attention_options of the C ABI."""
    _fields_ = [("sliding_window", ctypes.c_int32), ("graph_max_seq_len", ctypes.c_int32),
                ("kv_cache_dtype", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p), ("reserved", ctypes.c_int64 * 4)]


class PagedAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERRORS.get(code, code)}: {message}")
        self.code = code


def load_library(path: str = LIB_PATH):
    """Load libpagedattn.so and declare its entry points (raises if it is not built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.paged_kv_write.restype = ctypes.c_int
    lib.paged_kv_write.argtypes = [P, P, P, P, P, I64, I32, I32, I64, I32, I32, P]
    lib.paged_kv_write_fp8.restype = ctypes.c_int
    lib.paged_kv_write_fp8.argtypes = [P, P, P, P, P, P, P, I64, I32, I32, I64, I32, P]
    lib.paged_hbm_read_probe.restype = ctypes.c_int
    lib.paged_hbm_read_probe.argtypes = [P, I64, P, I32, P]
    lib.paged_mfma_probe.restype = ctypes.c_int
    lib.paged_mfma_probe.argtypes = [I32, I32, I32, P, P, P]
    lib.paged_copy_blocks.restype = ctypes.c_int
    lib.paged_copy_blocks.argtypes = [P, P, P, P, I64, I64, I64, I64, P]
    lib.paged_attention_workspace_bytes.restype = SZ
    lib.paged_attention_workspace_bytes.argtypes = [I32, I64, I32, I32, I32, I32, P, P, I32]
    lib.paged_attention_varlen.restype = ctypes.c_int
    lib.paged_attention_varlen.argtypes = [P, P, P, P, P, P, I32, ctypes.c_float, P, I32, I64, I32, I32,
                                           I32, I32, I64, P, P, I32, I32, P, SZ, I32, P]
    OPT = ctypes.POINTER(AttentionOptions)
    lib.paged_attention_workspace_bytes_ex.restype = SZ
    lib.paged_attention_workspace_bytes_ex.argtypes = [I32, I64, I32, I32, I32, I32, P, P, I32, OPT]
    lib.paged_attention_varlen_ex.restype = ctypes.c_int
    lib.paged_attention_varlen_ex.argtypes = [P, P, P, P, P, P, I32, ctypes.c_float, P, I32, I64, I32, I32,
                                              I32, I32, I64, P, P, I32, I32, P, SZ, I32, P, OPT]
    lib.paged_attention_varlen_noalloc.restype = ctypes.c_int
    lib.paged_attention_varlen_noalloc.argtypes = [P, P, P, P, P, P, I32, ctypes.c_float, P, I32, I64, I32, I32,
                                                   I32, I32, I64, P, P, I32, I32, I32, P, OPT]
    lib.paged_attn_last_error.restype = ctypes.c_char_p
    lib.paged_attn_last_error.argtypes = []
    lib.paged_attn_set_debug_checks.restype = None
    lib.paged_attn_set_debug_checks.argtypes = [I32]
    lib.paged_attn_set_path.restype = None
    lib.paged_attn_set_path.argtypes = [I32]
    lib.paged_attn_set_timing.restype = None
    lib.paged_attn_set_timing.argtypes = [I32]
    lib.paged_attn_timing_report.restype = ctypes.c_int
    lib.paged_attn_timing_report.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32), I32]
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != 0:
        raise PagedAttnError(rc, load_library().paged_attn_last_error().decode())


def _dptr(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _host_i32(x: Sequence[int]):
    arr = (ctypes.c_int32 * len(x))(*[int(v) for v in x])
    return arr


def set_debug_checks(enable: bool) -> None:
    load_library().paged_attn_set_debug_checks(1 if enable else 0)


def set_path(path: int) -> None:
    """0: automatic kernel choice; 1: vector-ALU tile kernel for every request."""
    load_library().paged_attn_set_path(int(path))


def hbm_read_probe(buf: torch.Tensor, sink: torch.Tensor, grid: int, stream=None) -> None:
    """Read all of the device tensor buf once (measurement of the achievable HBM read rate)."""
    lib = load_library()
    _check(lib.paged_hbm_read_probe(_dptr(buf, "buf"), buf.numel() * buf.element_size(), _dptr(sink, "sink"),
                                    int(grid), _stream(stream)))


def mfma_probe(iters: int, grid: int, sink: torch.Tensor, stream=None, random_operands: bool = False) -> int:
    """Run back-to-back bf16 matrix products (measurement of the sustained matrix-core rate),
    on small-integer or random operands; returns the launch's floating-point operation count."""
    lib = load_library()
    flops = ctypes.c_int64(0)
    _check(lib.paged_mfma_probe(int(iters), int(grid), 1 if random_operands else 0, _dptr(sink, "sink"),
                                ctypes.byref(flops), _stream(stream)))
    return flops.value


def set_timing(enable: bool) -> None:
    """Bracket every library launch on this thread with HIP events (measurement only)."""
    load_library().paged_attn_set_timing(1 if enable else 0)


def timing_report() -> dict:
    """{kind: (total_ms, launches)} over the launches recorded since timing was enabled."""
    lib = load_library()
    tot = (ctypes.c_double * len(KINDS))()
    cnt = (ctypes.c_int32 * len(KINDS))()
    rc = lib.paged_attn_timing_report(tot, cnt, len(KINDS))
    if rc < 0:
        _check(rc)
    return {KINDS[i]: (float(tot[i]), int(cnt[i])) for i in range(len(KINDS))}


def paged_kv_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                   v_cache: torch.Tensor, stream=None) -> None:
    """Scatter k, v [N, Hkv, D] into the pools [NB+1, bs, Hkv, D] at slot_mapping (int64)."""
    lib = load_library()
    if slot_mapping.dtype != torch.int64:
        raise ValueError("slot_mapping must be int64")
    n, hkv, d = k.shape
    if v.shape != k.shape or k_cache.shape != v_cache.shape or tuple(k_cache.shape[2:]) != (hkv, d):
        raise ValueError("shape mismatch between k, v and the caches")
    if k.dtype != v.dtype or k_cache.dtype != v_cache.dtype:
        raise ValueError("k and v (and the two caches) must share a dtype")
    num_slots = k_cache.shape[0] * k_cache.shape[1]
    _check(lib.paged_kv_write(_dptr(k, "k"), _dptr(v, "v"), _dptr(slot_mapping, "slot_mapping"),
                              _dptr(k_cache, "k_cache"), _dptr(v_cache, "v_cache"), n, hkv, d, num_slots,
                              PA_DTYPE[k.dtype], PA_DTYPE[k_cache.dtype], _stream(stream)))


def _options(sliding_window: int, graph_max_seq_len: int = 0, k_scale=None, v_scale=None, fp8: bool = False):
    opts = AttentionOptions()
    opts.sliding_window = int(sliding_window)
    opts.graph_max_seq_len = int(graph_max_seq_len)
    if k_scale is not None or fp8:
        opts.kv_cache_dtype = PA_DTYPE_FP8_E4M3
    if k_scale is not None:
        opts.k_scale = k_scale.data_ptr()
        opts.v_scale = v_scale.data_ptr()
    return ctypes.byref(opts), opts


def paged_kv_write_fp8(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                       v_cache: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor, stream=None) -> None:
    """Quantize k, v [N, Hkv, D] (f32 or bf16) into fp8 E4M3 pools k_cache / v_cache
    ([NB+1, bs, Hkv, D] uint8) and their per-(slot, KV head) scales k_scale / v_scale
    ([NB+1, bs, Hkv] float32) at slot_mapping (int64; negative: the scratch slot)."""
    lib = load_library()
    if slot_mapping.dtype != torch.int64:
        raise ValueError("slot_mapping must be int64")
    n, hkv, d = k.shape
    if v.shape != k.shape or k_cache.shape != v_cache.shape or tuple(k_cache.shape[2:]) != (hkv, d):
        raise ValueError("shape mismatch between k, v and the caches")
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("fp8 pools are uint8 tensors of codes")
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        if t.dtype != torch.float32 or tuple(t.shape) != tuple(k_cache.shape[:3]):
            raise ValueError(f"{name} must be float32 [NB+1, bs, Hkv]")
    num_slots = k_cache.shape[0] * k_cache.shape[1]
    _check(lib.paged_kv_write_fp8(_dptr(k, "k"), _dptr(v, "v"), _dptr(slot_mapping, "slot_mapping"),
                                  _dptr(k_cache, "k_cache"), _dptr(v_cache, "v_cache"), _dptr(k_scale, "k_scale"),
                                  _dptr(v_scale, "v_scale"), n, hkv, d, num_slots, PA_DTYPE[k.dtype], _stream(stream)))


def paged_copy_blocks(src: torch.Tensor, dst: torch.Tensor, src_block: torch.Tensor, dst_block: torch.Tensor,
                      stream=None) -> None:
    """Block dst_block[i] of dst becomes block src_block[i] of src (first axis = block).
    swap_out: src = pool, dst = (pinned host or device) staging; swap_in: the reverse;
    copy-on-write: src is dst.  src_block / dst_block are int64 device tensors."""
    lib = load_library()
    for name, t in (("src", src), ("dst", dst)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be device memory or pinned host memory")
    if src.dtype != dst.dtype or src.shape[1:] != dst.shape[1:]:
        raise ValueError("src and dst blocks differ")
    if src_block.dtype != torch.int64 or dst_block.dtype != torch.int64 or src_block.shape != dst_block.shape:
        raise ValueError("src_block and dst_block must be int64 tensors of one length")
    if src_block.numel() == 0:
        return
    block_bytes = src[0].numel() * src.element_size()
    _check(lib.paged_copy_blocks(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                 _dptr(src_block, "src_block"), _dptr(dst_block, "dst_block"), src_block.numel(),
                                 block_bytes, src.shape[0], dst.shape[0], _stream(stream)))


def paged_attention_workspace_bytes(num_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                                    query_start_loc_host: Sequence[int], seq_lens_host: Sequence[int],
                                    dtype: torch.dtype, sliding_window: int = 0, graph_max_seq_len: int = 0,
                                    kv_fp8: bool = False) -> int:
    lib = load_library()
    r = len(query_start_loc_host) - 1
    n = int(query_start_loc_host[-1]) if r > 0 else 0
    ref, _keep = _options(sliding_window, graph_max_seq_len, fp8=kv_fp8)
    lens = _host_i32(seq_lens_host) if seq_lens_host is not None else None
    return int(lib.paged_attention_workspace_bytes_ex(r, n, num_heads, num_kv_heads, head_dim, block_size,
                                                      _host_i32(query_start_loc_host), lens, PA_DTYPE[dtype], ref))


def paged_attention_varlen(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           query_start_loc: torch.Tensor, seq_lens: torch.Tensor, block_table: torch.Tensor,
                           block_size: int, scale: float, out: Optional[torch.Tensor] = None, *,
                           query_start_loc_host: Sequence[int], seq_lens_host: Sequence[int],
                           max_query_len: int = 0, max_seq_len: int = 0,
                           workspace: Optional[torch.Tensor] = None, stream=None,
                           sliding_window: int = 0, graph_max_seq_len: int = 0,
                           k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                           noalloc: bool = False) -> torch.Tensor:
    """Causal attention of the flattened batch over the pool; returns out [N, H, D].
    sliding_window > 0 limits the row at position p to keys p - sliding_window + 1 .. p.
    graph_max_seq_len > 0 sizes the launches for any device seq_lens up to it (for a call
    captured in a graph and replayed as the contexts grow); seq_lens_host may be None.
    With k_scale / v_scale ([NB+1, bs, Hkv] float32) the caches are fp8 E4M3 pools (uint8
    codes written by paged_kv_write_fp8) and q / out are bf16.
    noalloc=True calls paged_attention_varlen_noalloc: the library's fixed per-GPU scratch
    array serves as the workspace (workspace must then be None; out must be given)."""
    lib = load_library()
    n, h, d = q.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[1] != block_size or k_cache.shape[3] != d:
        raise ValueError("cache shape must be [num_blocks + 1, block_size, Hkv, D]")
    fp8 = k_scale is not None
    if fp8:
        if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8 or v_scale is None:
            raise ValueError("fp8 pools: uint8 caches with k_scale and v_scale")
        for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
            if t.dtype != torch.float32 or tuple(t.shape) != tuple(k_cache.shape[:3]) or not t.is_cuda:
                raise ValueError(f"{name} must be a float32 device tensor [NB+1, bs, Hkv]")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
    elif q.dtype != k_cache.dtype or q.dtype != v_cache.dtype:
        raise ValueError("q and the caches must share a dtype")
    for name, t in (("query_start_loc", query_start_loc), ("seq_lens", seq_lens), ("block_table", block_table)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    if noalloc and (workspace is not None or out is None):
        raise ValueError("noalloc: pass out and no workspace")
    if out is None:
        out = torch.empty_like(q)
    hkv = k_cache.shape[2]
    r = len(query_start_loc_host) - 1
    qh = _host_i32(query_start_loc_host)
    sh = _host_i32(seq_lens_host) if seq_lens_host is not None else None
    ref, _keep = _options(sliding_window, graph_max_seq_len, k_scale, v_scale)
    stride = block_table.shape[1] if block_table.dim() == 2 else 0
    num_slots = k_cache.shape[0] * k_cache.shape[1]
    if noalloc:
        _check(lib.paged_attention_varlen_noalloc(
            _dptr(q, "q"), _dptr(k_cache, "k_cache"), _dptr(v_cache, "v_cache"),
            _dptr(query_start_loc, "query_start_loc"), _dptr(seq_lens, "seq_lens"),
            _dptr(block_table, "block_table"), block_size, float(scale), _dptr(out, "out"), r, n, h, hkv, d, stride,
            num_slots, qh, sh, int(max_query_len), int(max_seq_len), PA_DTYPE[q.dtype], _stream(stream), ref))
        return out
    need = lib.paged_attention_workspace_bytes_ex(r, n, h, hkv, d, block_size, qh, sh, PA_DTYPE[q.dtype], ref)
    if workspace is None:
        workspace = torch.empty(max(int(need), 256), dtype=torch.uint8, device=q.device)
    _check(lib.paged_attention_varlen_ex(
        _dptr(q, "q"), _dptr(k_cache, "k_cache"), _dptr(v_cache, "v_cache"),
        _dptr(query_start_loc, "query_start_loc"), _dptr(seq_lens, "seq_lens"), _dptr(block_table, "block_table"),
        block_size, float(scale), _dptr(out, "out"), r, n, h, hkv, d, stride, num_slots, qh, sh,
        int(max_query_len), int(max_seq_len), _dptr(workspace, "workspace"), workspace.numel(),
        PA_DTYPE[q.dtype], _stream(stream), ref))
    return out
