"""The prefill path's global and LDS addresses, recomputed on the host for every workgroup
and lane of every launch that the GPU parity batches make, checked against the buffers they
point into (tests/host/prefill_addr.cpp).  No GPU: the batches are built without values.

Covers every bf16 and fp8 parity batch whose chunks take the prefill kernels: the workload
configurations at full size (the shared-prefix and long-context ones included), the edge,
window and fp8 cases, every piece of the chunking test, and the full-size fp8 runs."""
import math
import os
import shutil
import subprocess
import zlib

import pytest
import torch

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _record(name, b, window=0, f8=0):
    t = b.block_table
    head = (f"batch {name} {b.num_reqs} {b.num_heads} {b.num_kv_heads} {b.head_dim} {b.block_size} {window} {f8} "
            f"{b.num_blocks} {t.shape[1]} {b.num_tokens}")
    return "\n".join([head, " ".join(map(str, b.query_start_loc_host)), " ".join(map(str, b.seq_lens_host)),
                      " ".join(map(str, t.reshape(-1).tolist()))])


def _meta_only(r, h, hkv, d, table, nb, bs=16):
    """A one-request batch record from its rows, length and table."""
    class _B:
        pass
    b = _B()
    b.num_reqs, b.num_heads, b.num_kv_heads, b.head_dim, b.block_size, b.num_blocks = 1, h, hkv, d, bs, nb
    b.block_table = table[None, :]
    b.query_start_loc_host = [0, r[1]]
    b.seq_lens_host = [r[0]]
    b.num_tokens = r[1]
    return b


def _parity_records():
    from tests import test_gpu_parity as P
    recs = []
    small = lambda specs, h, hkv, d, bs=16, name="", **kw: workloads.small_batch(
        specs, dtype="bf16", num_heads=h, num_kv_heads=hkv, head_dim=d, block_size=bs,
        seed=zlib.crc32(name.encode()) % 1000, values=False, **kw)
    # the workload configurations at full size
    for name, make in workloads.CONFIGS.items():
        b = make(values=False)
        if b.dtype == "bf16":
            recs.append(_record(name, b))
            recs.append(_record(name + "_fp8", b, f8=1))
    b = workloads.long_context(values=False)
    recs.append(_record("long_context_window_4096", b, window=4096))
    for name, specs, h, hkv, d, bs, dtype in P.EDGE:
        if dtype == "bf16":
            recs.append(_record(name, small(specs, h, hkv, d, bs, name)))
    for name, specs, h, hkv, d, bs, dtype, windows in P.WINDOW:
        if dtype == "bf16":
            b = small(specs, h, hkv, d, bs, name)
            recs += [_record(f"{name}_w{w}", b, window=w) for w in windows]
    for name, specs, h, hkv, d, window in P.FP8:
        recs.append(_record("fp8_" + name, small(specs, h, hkv, d, 16, name), window=window, f8=1))
    b = small([(700, 150), (90, 1), (3000, 1)], 32, 8, 128, name="window_cover")
    recs += [_record(f"window_cover_{w}", b, window=w) for w in (3001, 1 << 30)]
    recs.append(_record("wide_v", small([(500, 200), (300, 150)], 32, 8, 128, name="wide_v")))
    recs.append(_record("relabel", small([(300, 1), (40, 8), (1000, 1), (77, 3), (0, 40), (12, 1), (600, 2), (5, 1)],
                                          16, 4, 128, name="relabel")))
    # every piece of the chunking test (one request, the full table, rows a .. e of L)
    for L in (300, 5000):
        gen = torch.Generator().manual_seed(31 + L)
        nb = L // 16 + 3
        table = torch.randperm(nb, generator=gen)[: -(-L // 16)].to(torch.int32)
        for chunk in (L, 8, 33, 64, 4096):
            for a in range(0, L, chunk):
                e = min(L, a + chunk)
                recs.append(_record(f"chunking_L{L}_c{chunk}_{a}", _meta_only((e, e - a), 8, 2, 128, table, nb)))
    return recs


@pytest.fixture(scope="module")
def prefill_addr_exe(tmp_path_factory):
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    exe = str(tmp_path_factory.mktemp("prefill_addr") / "prefill_addr")
    src = os.path.join(ROOT, "tests", "host", "prefill_addr.cpp")
    inc = os.path.join(ROOT, "paged_kv_attention_05_amd", "csrc")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-x", "hip", "-I", inc, src, "-o", exe],
                   check=True, capture_output=True, text=True)
    return exe


def test_every_prefill_access_of_the_parity_batches_is_in_bounds(prefill_addr_exe):
    recs = _parity_records()
    res = subprocess.run([prefill_addr_exe], input="\n".join(recs) + "\n", capture_output=True, text=True,
                         timeout=600)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-2000:]
    assert f"checked {len(recs)} batches" in res.stdout, res.stdout


def test_the_replica_catches_a_table_read_past_the_request(prefill_addr_exe):
    """A table one entry short of the last full tile's blocks: the replica must flag the
    full-tile read of the missing entry (the check is not vacuous)."""
    L = 256                                          # four full 64-key tiles, sixteen blocks
    table = torch.arange(16, dtype=torch.int32)
    rec = _record("short", _meta_only((L, 200), 8, 2, 128, table, 20))
    # claim one more key than the table holds: the last tile reads entries up to 16
    rec = rec.replace(f"\n0 200\n{L}\n", f"\n0 200\n{L + 64}\n")
    res = subprocess.run([prefill_addr_exe], input=rec + "\n", capture_output=True, text=True, timeout=60)
    assert res.returncode == 1 and "table entry" in res.stdout, res.stdout
