"""The C ABI without a GPU: the library loads, exports every declared symbol, and rejects
malformed metadata from the host copies alone (no device pointer is touched)."""
import ctypes
import os
import re

import pytest

import paged_kv_attention_05_amd as pk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "paged_attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert set(pk.EXPORTS) == set(names), names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(pk.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def _host(x):
    return (ctypes.c_int32 * len(x))(*x)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def call_attention(qsl, lens, H=8, Hkv=2, D=128, bs=16, stride=4, dtype=1, ws_bytes=1 << 30, N=None, null=False):
    lib = pk.load_library()
    R = len(lens)
    N = qsl[-1] if N is None else N
    p = None if null else FAKE
    return lib.paged_attention_varlen(p, FAKE, FAKE, FAKE, FAKE, FAKE, bs, 0.1, FAKE, R, N, H, Hkv, D, stride,
                                      1024, _host(qsl), _host(lens), 0, 0, FAKE, ws_bytes, dtype, None)


@pytest.mark.parametrize("qsl,lens,kw,code", [
    ([0, 3, 2], [5, 5], {}, -4),                  # non-monotone query_start_loc
    ([1, 3], [5], {}, -4),                        # query_start_loc[0] != 0
    ([0, 3], [5], {"N": 4}, -4),                  # query_start_loc[R] != N
    ([0, 6], [5], {}, -4),                        # more rows than seq_len
    ([0, 1], [100], {}, -4),                      # table too narrow (7 blocks > 4)
    ([0, 1], [-1], {}, -4),                       # negative seq_len
    ([0, 1], [5], {"H": 7}, -2),                  # H not a multiple of Hkv
    ([0, 1], [5], {"D": 40}, -2),                 # unsupported head_dim
    ([0, 1], [5], {"bs": 0}, -2),                 # block size
    ([0, 1], [5], {"dtype": 7}, -3),              # dtype code
    ([0, 1], [5], {"ws_bytes": 16}, -5),          # workspace too small
    ([0, 1], [5], {"null": True}, -1),            # null q
])
def test_attention_rejects_bad_arguments(qsl, lens, kw, code):
    assert call_attention(qsl, lens, **kw) == code
    assert pk.load_library().paged_attn_last_error()


def test_workspace_query_and_padding_rows():
    lib = pk.load_library()
    n = lib.paged_attention_workspace_bytes(3, 4, 8, 2, 128, 16, _host([0, 1, 3, 4]), _host([10, 0, 300]), 1)
    assert n > 0
    assert lib.paged_attention_workspace_bytes(1, 4, 8, 2, 40, 16, _host([0, 4]), _host([10]), 1) == 0


def test_kv_write_rejects_bad_arguments():
    lib = pk.load_library()
    assert lib.paged_kv_write(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 8, 64, 9, 0, None) == -3
    assert lib.paged_kv_write(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0, 8, 64, 0, 0, None) == -2
    assert lib.paged_kv_write(None, FAKE, FAKE, FAKE, FAKE, 4, 2, 8, 64, 0, 0, None) == -1
    assert lib.paged_kv_write(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 8, 0, 0, 0, None) == -2
    assert lib.paged_kv_write(None, None, None, None, None, 0, 2, 8, 64, 0, 0, None) == 0


def test_binding_requires_the_library(tmp_path):
    with pytest.raises(RuntimeError):
        pk.load_library(str(tmp_path / "missing.so"))


def _call_ex(opts, lens=(5,), qsl=(0, 1)):
    lib = pk.load_library()
    return lib.paged_attention_varlen_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 0.1, FAKE, len(lens), qsl[-1], 8, 2,
                                         128, 4, 1024, _host(list(qsl)), _host(list(lens)), 0, 0, FAKE, 16, 1, None,
                                         ctypes.byref(opts) if opts is not None else None)


def test_options_are_validated():
    bad = pk.AttentionOptions()
    bad.sliding_window = -3
    assert _call_ex(bad) == -2 and "sliding_window" in pk.load_library().paged_attn_last_error().decode()
    bad = pk.AttentionOptions()
    bad.reserved[2] = 1
    assert _call_ex(bad) == -2 and "reserved" in pk.load_library().paged_attn_last_error().decode()
    # valid options (or none) get as far as the workspace check
    assert _call_ex(pk.AttentionOptions()) == -5
    assert _call_ex(None) == -5


def test_window_shrinks_the_split_workspace():
    """Long decodes split their keys over workgroups; a short window needs fewer splits."""
    lib = pk.load_library()
    qsl, lens = _host([0, 1, 2]), _host([30000, 20000])
    full = lib.paged_attention_workspace_bytes(2, 2, 8, 2, 128, 16, qsl, lens, 1)
    opts = pk.AttentionOptions()
    opts.sliding_window = 256
    windowed = lib.paged_attention_workspace_bytes_ex(2, 2, 8, 2, 128, 16, qsl, lens, 1, ctypes.byref(opts))
    assert 0 < windowed < full
    opts.sliding_window = 0
    assert lib.paged_attention_workspace_bytes_ex(2, 2, 8, 2, 128, 16, qsl, lens, 1, ctypes.byref(opts)) == full


def test_copy_blocks_rejects_bad_arguments():
    lib = pk.load_library()
    assert lib.paged_copy_blocks(FAKE, FAKE, FAKE, FAKE, 3, 100, 8, 8, None) == -2     # not a multiple of 16
    assert lib.paged_copy_blocks(FAKE, FAKE, FAKE, FAKE, -1, 64, 8, 8, None) == -2     # negative count
    assert lib.paged_copy_blocks(None, FAKE, FAKE, FAKE, 3, 64, 8, 8, None) == -1
    assert lib.paged_copy_blocks(ctypes.c_void_p(0x1008), FAKE, FAKE, FAKE, 3, 64, 8, 8, None) == -2   # misaligned
    assert lib.paged_copy_blocks(None, None, None, None, 0, 64, 0, 0, None) == 0        # nothing to copy


def test_graph_sizing():
    """Sized for capacity: host seq_lens may be absent; chunks over 64 query columns are
    refused (their routing could change with the device lengths)."""
    lib = pk.load_library()
    opts = pk.AttentionOptions()
    opts.graph_max_seq_len = 4096
    ok = lib.paged_attention_workspace_bytes_ex(3, 3, 32, 8, 128, 16, _host([0, 1, 2, 3]), None, 1, ctypes.byref(opts))
    assert ok > 0
    long_chunk = lib.paged_attention_workspace_bytes_ex(2, 40, 32, 8, 128, 16, _host([0, 1, 40]), None, 1,
                                                        ctypes.byref(opts))
    assert long_chunk == 0
    opts.graph_max_seq_len = -1
    assert lib.paged_attention_workspace_bytes_ex(3, 3, 32, 8, 128, 16, _host([0, 1, 2, 3]), None, 1,
                                                  ctypes.byref(opts)) == 0


def test_read_probe_rejects_bad_arguments():
    lib = pk.load_library()
    sink = ctypes.c_void_p(0x2000)                 # never dereferenced: validation fails first
    assert lib.paged_hbm_read_probe(None, 1024, sink, 64, None) == -1
    assert lib.paged_hbm_read_probe(FAKE, 1024, None, 64, None) == -1
    assert lib.paged_hbm_read_probe(FAKE, 1000, sink, 64, None) == -2                 # not a multiple of 16
    assert lib.paged_hbm_read_probe(FAKE, 0, sink, 64, None) == -2
    assert lib.paged_hbm_read_probe(ctypes.c_void_p(0x1008), 1024, sink, 64, None) == -2   # misaligned
    assert lib.paged_hbm_read_probe(FAKE, 1024, sink, 0, None) == -2
    assert lib.paged_hbm_read_probe(FAKE, 1024, sink, 70000, None) == -2


def test_mfma_probe_rejects_bad_arguments():
    lib = pk.load_library()
    sink = ctypes.c_void_p(0x2000)                 # never dereferenced: validation fails first
    assert lib.paged_mfma_probe(16, 64, 0, None, None, None) == -1
    assert lib.paged_mfma_probe(0, 64, 0, sink, None, None) == -2
    assert lib.paged_mfma_probe(1 << 21, 64, 0, sink, None, None) == -2
    assert lib.paged_mfma_probe(16, 0, 0, sink, None, None) == -2
    assert lib.paged_mfma_probe(16, 70000, 0, sink, None, None) == -2
    assert lib.paged_mfma_probe(16, 64, 2, sink, None, None) == -2


def test_no_kernel_spills_registers():
    """The build records the compiler's resource report for every kernel and refuses a
    kernel that spills to scratch. The report covers each kernel family of the library, and
    every kernel fits one compute unit's LDS (160 KiB)."""
    from paged_kv_attention_05_amd import build as B
    if not os.path.exists(B.RESOURCES):
        B.build(verbose=False)
    with open(B.RESOURCES) as f:
        head, *rows = [line.rstrip("\n").split("\t") for line in f]
    kernels = [dict(zip(head, r)) for r in rows]
    names = " ".join(k["name"] for k in kernels)
    for family in ("kv_copy16", "kv_quant_fp8", "copy_blocks16", "plan_kernel", "small_tile_valu",
                   "merge_splits", "small_tile_mfma", "prefill_tile_mfma", "stage_fp8", "stage_v16"):
        assert family in names, family
    for k in kernels:
        assert int(k["scratch"]) == 0 and int(k["vgpr_spill"]) == 0, k["name"]
        assert int(k["lds"]) <= 160 * 1024, k["name"]


def test_noalloc_refuses_batches_beyond_its_scratch():
    """The no-alloc entry point sizes the batch from the host metadata before it looks up its
    scratch array: 2000 decodes of 32768 tokens need far more than PA_NOALLOC_SCRATCH_BYTES of
    split partials and are refused with PA_ERR_WORKSPACE (no device is touched)."""
    lib = pk.load_library()
    R, L = 2000, 32768
    qsl = list(range(R + 1))
    lens = [L] * R
    need = lib.paged_attention_workspace_bytes(R, R, 64, 8, 128, 16, _host(qsl), _host(lens), 1)
    assert need > pk.NOALLOC_SCRATCH_BYTES
    rc = lib.paged_attention_varlen_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 0.1, FAKE, R, R, 64, 8, 128,
                                            L // 16, (L // 16 + 1) * 16, _host(qsl), _host(lens), 1, L, 1, None,
                                            None)
    assert rc == -5
    msg = lib.paged_attn_last_error().decode()
    assert "no-alloc maximum" in msg and str(pk.NOALLOC_SCRATCH_BYTES) in msg
    # malformed metadata is refused the same way as by the workspace entry points
    assert lib.paged_attention_varlen_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 0.1, FAKE, 1, 6, 8, 2, 128, 4,
                                              1024, _host([0, 6]), _host([5]), 0, 0, 1, None, None) == -4


def test_noalloc_scratch_size_matches_the_header():
    text = open(os.path.join(ROOT, "include", "paged_attn.h")).read()
    m = re.search(r"#define PA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == pk.NOALLOC_SCRATCH_BYTES
