"""paged_attention_varlen_noalloc (the workspace is the library's fixed scratch array) against
paged_attention_varlen_ex with a caller workspace, through the C ABI on the GPU: two calls in
a row on one GPU, the second on a smaller batch, each bit-identical to the workspace entry
point and within the bound of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from tests import gpu_harness as H
from tests._util import attention_error

pytestmark = pytest.mark.gpu

# (computed, new) per request: a prefill chunk, long decodes (split partials and the merge),
# verification rows (grouped tiles), a zero-row request; then a smaller decode batch
CALLS = [
    ([(700, 150), (9000, 1), (4000, 1), (300, 5), (57, 3), (20, 0), (2049, 9)], None),
    ([(33, 1), (1000, 1), (5, 2)], 5),
]


def _noalloc(lib, b, t, out):
    P = lambda x: ctypes.c_void_p(x.data_ptr())
    host = lambda xs: (ctypes.c_int32 * len(xs))(*xs)
    return lib.paged_attention_varlen_noalloc(
        P(t["q"]), P(t["k_cache"]), P(t["v_cache"]), P(t["query_start_loc"]), P(t["seq_lens"]),
        P(t["block_table"]), b.block_size, ctypes.c_float(b.scale), P(out), b.num_reqs, b.num_tokens, b.num_heads,
        b.num_kv_heads, b.head_dim, t["block_table"].shape[1], b.num_slots, host(b.query_start_loc_host),
        host(b.seq_lens_host), b.max_query_len, b.max_seq_len, 1, None, None)


def test_noalloc_matches_the_workspace_entry_point():
    import paged_kv_attention_05_amd as pk
    lib = pk.load_library()
    dev = torch.device("cuda:0")
    for i, (specs, pad) in enumerate(CALLS):
        H.log(f"[noalloc] call {i}: {len(specs)} requests, pad_to={pad}")
        b = workloads.small_batch(specs, dtype="bf16", num_heads=32, num_kv_heads=8, head_dim=128, pad_to=pad,
                                  seed=71 + i)
        t = {n: getattr(b, n).to(dev).contiguous() for n in ("q", "k", "v", "k_cache", "v_cache", "slot_mapping",
                                                              "query_start_loc", "seq_lens", "block_table")}
        pk.paged_kv_write(t["k"], t["v"], t["slot_mapping"], t["k_cache"], t["v_cache"])
        ref = pk.paged_attention_varlen(t["q"], t["k_cache"], t["v_cache"], t["query_start_loc"], t["seq_lens"],
                                        t["block_table"], b.block_size, b.scale,
                                        query_start_loc_host=b.query_start_loc_host, seq_lens_host=b.seq_lens_host)
        out = torch.full_like(t["q"], float("nan"))
        rc = _noalloc(lib, b, t, out)
        assert rc == 0, lib.paged_attn_last_error()
        torch.cuda.synchronize()
        assert torch.equal(out.cpu().view(torch.int16), ref.cpu().view(torch.int16)), i
        ref64, _, _ = H.oracle_step(b)
        err = attention_error(out.float().cpu().numpy(), ref64, "bf16")
        H.log(f"[noalloc] call {i}: bit-identical to the workspace entry point; error {err:.3g} x bound")
        assert err <= 1.0, (i, err)
