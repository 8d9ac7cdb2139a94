"""HIP path against the CPU oracle on the same seeded inputs (needs the GPU).

Pools must match bit for bit after the KV write (except the scratch slot); attention must be
within 1e-5 of the row's max |value| (float32) or 2e-2 + half a bf16 ulp (bfloat16) of the
float64 oracle run on the same data.  Dead slots are NaN in every case.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import workloads
from tests import gpu_harness as H
from tests._util import attention_error, to_np

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------------------ KV write
@pytest.mark.parametrize("in_dt,cache_dt", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("hkv,d", [(4, 48), (8, 128), (1, 8), (3, 16)])
def test_kv_write_bit_exact(in_dt, cache_dt, hkv, d):
    import oracle
    import paged_kv_attention_05_amd as pk
    H.log(f"[kv_write] {in_dt}->{cache_dt} hkv={hkv} d={d}")
    gen = torch.Generator().manual_seed(hkv * 1000 + d)
    n, bs, nb = 333, 16, 40
    tin, tc = workloads.TORCH_DTYPES[in_dt], workloads.TORCH_DTYPES[cache_dt]
    k = (torch.randn((n, hkv, d), generator=gen) * 4).to(tin)
    v = (torch.randn((n, hkv, d), generator=gen) * 4).to(tin)
    kc = torch.randn((nb + 1, bs, hkv, d), generator=gen).to(tc)
    vc = torch.randn((nb + 1, bs, hkv, d), generator=gen).to(tc)
    slots = torch.randperm(nb * bs, generator=gen)[:n].to(torch.int64)
    slots[::17] = -1
    okc, ovc = to_np(kc).copy(), to_np(vc).copy()
    oracle.kv_write(to_np(k), to_np(v), slots.numpy(), okc, ovc, in_dt, cache_dt)
    dkc, dvc = kc.cuda(), vc.cuda()
    pk.paged_kv_write(k.cuda(), v.cuda(), slots.cuda(), dkc, dvc)
    torch.cuda.synchronize()
    H.assert_pools_equal(dkc.cpu(), okc)
    H.assert_pools_equal(dvc.cpu(), ovc)


def test_kv_write_empty_and_all_padding():
    import paged_kv_attention_05_amd as pk
    kc = torch.zeros((3, 4, 2, 8), device="cuda")
    vc = torch.zeros_like(kc)
    e = torch.zeros((0, 2, 8), device="cuda")
    pk.paged_kv_write(e, e, torch.zeros(0, dtype=torch.int64, device="cuda"), kc, vc)
    k = torch.arange(5 * 16, dtype=torch.float32, device="cuda").view(5, 2, 8) + 1
    pk.paged_kv_write(k, k, torch.full((5,), -1, dtype=torch.int64, device="cuda"), kc, vc)
    torch.cuda.synchronize()
    flat = kc.view(-1, 2, 8).cpu()
    assert torch.all(flat[:-1] == 0)
    assert any(torch.equal(flat[-1], k[i].cpu()) for i in range(5))


# ------------------------------------------------------------------------------ configs
def test_worked_batch():
    H.check_batch(workloads.worked_batch())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mixed_step(dtype):
    H.check_batch(workloads.mixed_step(dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mixed_step_vector_path(dtype):
    H.check_batch(workloads.mixed_step(dtype), path=1, label=f"mixed_step_{dtype}_vector")


def test_decode_only_full_size():
    H.check_batch(workloads.decode_only())


def _sample_rows(batch, seed, n_random=256, edge=64):
    """All decode rows, the first and last `edge` rows of every chunk, and random chunk rows."""
    mask = np.zeros(batch.num_tokens, np.uint8)
    rng = np.random.default_rng(seed)
    for r, req in enumerate(batch.requests):
        b, e = batch.query_start_loc_host[r], batch.query_start_loc_host[r + 1]
        if e - b <= 2 * edge:
            mask[b:e] = 1
        else:
            mask[b:b + edge] = 1
            mask[e - edge:e] = 1
            mask[rng.choice(np.arange(b + edge, e - edge), size=min(n_random, e - b - 2 * edge), replace=False)] = 1
    return mask


def test_shared_prefix_full_size():
    b = workloads.shared_prefix()
    H.check_batch(b, row_mask=_sample_rows(b, 4))


def test_spec_verify_full_size():
    """128 verifications of 1 + k rows (k = 1, 2, 4, 8) over contexts of 512..8192 tokens."""
    H.check_batch(workloads.spec_verify())


def test_long_context_full_size():
    b = workloads.long_context()
    H.check_batch(b, row_mask=_sample_rows(b, 5))


# ------------------------------------------------------------------------------ edge cases
EDGE = [
    # (name, specs (computed, new), H, Hkv, D, bs, dtype)
    ("fresh_prompt_g1", [(0, 37)], 4, 4, 64, 16, "bf16"),
    ("single_key", [(0, 1), (0, 1)], 8, 2, 128, 16, "bf16"),
    ("spec_verify_rows", [(100, 2), (57, 3), (300, 4), (16, 5)], 8, 2, 128, 16, "bf16"),
    ("g8_decodes", [(1000, 1), (15, 1), (16, 1), (17, 1)], 64, 8, 128, 16, "bf16"),
    ("g16", [(40, 1), (20, 20)], 32, 2, 64, 16, "bf16"),
    ("g32_mqa", [(70, 1), (5, 9)], 32, 1, 64, 16, "f32"),
    ("block_size_1", [(19, 3), (0, 6)], 4, 2, 48, 1, "f32"),
    ("block_size_4", [(19, 3), (0, 6), (33, 1)], 4, 2, 16, 4, "bf16"),
    ("block_size_64", [(130, 2), (0, 70)], 8, 4, 64, 64, "bf16"),
    ("head_dim_8", [(12, 4), (0, 2)], 4, 2, 8, 16, "f32"),
    ("head_dim_256", [(77, 1), (3, 20)], 4, 2, 256, 16, "bf16"),
    ("head_dim_96", [(77, 1), (3, 20)], 6, 2, 96, 16, "f32"),
    ("long_decode_many_splits", [(20000, 1), (9000, 1)], 8, 1, 128, 16, "bf16"),
    ("long_decode_f32", [(5000, 1)], 4, 2, 64, 16, "f32"),
    # 9 and 17 key splits of 2048: the merge folds a full batch of 8 splits, then a partial one
    ("merge_batches_9_17", [(16500, 1), (34000, 1), (4000, 3)], 8, 2, 128, 16, "bf16"),
    ("merge_batches_f32", [(16500, 1), (2, 1)], 4, 1, 64, 16, "f32"),
    ("block_boundaries", [(15, 1), (16, 1), (31, 2), (32, 16), (47, 17)], 8, 2, 128, 16, "bf16"),
    ("chunk_ragged_tail", [(1000, 131), (0, 200)], 16, 4, 128, 16, "bf16"),
    ("prefill_g8_d64", [(500, 300), (0, 77), (2, 1)], 64, 8, 64, 16, "bf16"),
    ("prefill_g2", [(33, 200), (64, 64)], 8, 4, 128, 16, "bf16"),
    ("prefill_g1_long_context", [(3000, 129)], 8, 8, 128, 16, "bf16"),
    ("prefill_g16_d64", [(100, 9), (0, 3)], 32, 2, 64, 16, "bf16"),
    ("prefill_outliers", [(700, 150), (90, 1)], 32, 8, 128, 16, "bf16"),
    # grouped small tiles with two head subsets per token (g = 32): groups cross tokens
    ("groups_two_head_subsets", [(70, 1), (5, 9), (300, 4), (2100, 2)], 32, 1, 64, 16, "bf16"),
    ("groups_g4_spec_splits", [(5000, 9), (2047, 5), (2049, 9), (100, 3)], 16, 4, 128, 16, "bf16"),
    # g = 3 and g = 6 do not divide the prefill tile's 256 rows: long chunks take the small tiles
    ("g3_chunks_on_small_tiles", [(300, 150), (10, 1), (0, 70), (2100, 33)], 12, 4, 128, 16, "bf16"),
    ("g6_chunks_on_small_tiles", [(40, 120), (999, 1), (0, 17)], 12, 2, 128, 16, "bf16"),
    # g = 4: 17 rows (68 columns) is the shortest chunk on the prefill tiles, 16 rows (64) the
    # longest on the small tiles
    ("prefill_threshold", [(100, 17), (5, 16), (0, 17), (3000, 16)], 32, 8, 128, 16, "bf16"),
    # head_dim 48 on the matrix-core small tiles (padded to 64): decodes, grouped tiles of a
    # chunk, a request with no context, speculative rows, key splits merged, g = 8 and g = 1
    ("head_dim_48_mfma", [(1000, 1), (17, 1), (40, 30), (0, 64), (300, 5), (15, 1)], 8, 4, 48, 16, "bf16"),
    ("head_dim_48_splits_g8", [(5000, 1), (9000, 1), (33, 3), (0, 1)], 32, 4, 48, 16, "bf16"),
    ("head_dim_48_g1", [(70, 1), (5, 40), (2100, 2)], 4, 4, 48, 16, "bf16"),
]


@pytest.mark.parametrize("name,specs,h,hkv,d,bs,dtype", EDGE, ids=[e[0] for e in EDGE])
def test_edge_case(name, specs, h, hkv, d, bs, dtype):
    b = workloads.small_batch(specs, dtype=dtype, num_heads=h, num_kv_heads=hkv, head_dim=d, block_size=bs,
                              seed=zlib.crc32(name.encode()) % 1000,
                              outlier_p=0.01 if "outliers" in name else 0.0)
    H.check_batch(b, label=name)


# ------------------------------------------------------------------- items without a planner
INLINE = [
    # (name, specs (computed, new), H, Hkv, D, window, pad_to)
    ("decodes_splits", [(1000, 1), (15, 1), (300, 1), (5000, 1), (0, 1), (2100, 1)], 32, 8, 128, 0, None),
    ("spec_rows_groups", [(100, 2), (57, 3), (300, 4), (16, 5), (2049, 9), (5000, 9)], 16, 4, 128, 0, None),
    ("d64_window", [(20000, 1), (9000, 1), (70, 3)], 8, 1, 64, 300, None),
    ("sixty_four_requests_d48", [(17 + (31 * i) % 900, 1 + i % 3) for i in range(64)], 8, 4, 48, 0, None),
    ("padding_rows", [(700, 1), (90, 1), (2000, 1)], 32, 8, 128, 0, 8),
]


@pytest.mark.parametrize("name,specs,h,hkv,d,window,pad_to", INLINE, ids=[c[0] for c in INLINE])
def test_inline_items_match_the_planner(name, specs, h, hkv, d, window, pad_to):
    """A batch of at most 64 requests on the matrix-core small tiles runs without the planner
    kernel: every workgroup of the small kernels and of the merge derives its own item.  The
    outputs are bit-identical to those of the same call with the planner launched (path 2),
    the planner really is skipped (no planner launch recorded), and both match the oracle."""
    import paged_kv_attention_05_amd as pk
    b = workloads.small_batch(specs, dtype="bf16", num_heads=h, num_kv_heads=hkv, head_dim=d,
                              seed=zlib.crc32(name.encode()) % 1000, pad_to=pad_to)
    assert b.num_reqs <= 64
    launches = {}
    outs = {}
    for path in (0, 2):
        pk.set_timing(True)
        try:
            outs[path], _, _ = H.gpu_step(b, path=path, window=window)
            launches[path] = pk.timing_report()
        finally:
            pk.set_timing(False)
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))
    assert launches[0]["plan"][1] == 0 and launches[2]["plan"][1] == 1, launches
    ref64, _, _ = H.oracle_step(b, window=window)
    err = attention_error(outs[0].float().numpy(), ref64, "bf16")
    H.log(f"[parity] inline items {name}: error {err:.3g} x bound")
    assert err <= 1.0, err


# ------------------------------------------------------------------------- fp8 pools
def _fp8_pools(b):
    """The batch's context pool quantized slot by slot with the oracle's write: codes and scales."""
    import oracle
    from tests._util import to_np
    shape = tuple(b.k_cache.shape)
    kc = np.zeros(shape, np.uint8)
    vc = np.zeros(shape, np.uint8)
    ks = np.zeros(shape[:3], np.float32)
    vs = np.zeros(shape[:3], np.float32)
    flat = lambda t: np.ascontiguousarray(to_np(t).reshape(-1, shape[2], shape[3]))
    oracle.kv_write_fp8(flat(b.k_cache), flat(b.v_cache), np.arange(shape[0] * shape[1], dtype=np.int64),
                        kc, vc, ks, vs, b.dtype)
    return kc, vc, ks, vs


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_kv_write_fp8_parity(in_dtype):
    """Codes and scales bit for bit as the oracle's write (both divide in float32)."""
    import oracle
    import paged_kv_attention_05_amd as pk
    from tests._util import to_np
    dev = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(71)
    n, hkv, d, nb, bs = 300, 8, 128, 40, 16
    k = torch.randn((n, hkv, d), generator=gen) * torch.tensor([1e-4, 1.0, 30.0, 1e3])[torch.arange(n) % 4][:, None, None]
    v = torch.randn((n, hkv, d), generator=gen) * 2
    k[5, 3] = 0.0
    k, v = k.to(workloads.TORCH_DTYPES[in_dtype]), v.to(workloads.TORCH_DTYPES[in_dtype])
    slots = torch.randperm(nb * bs, generator=gen)[:n].to(torch.int64)
    slots[[7, 100]] = -1
    kc = torch.zeros((nb + 1, bs, hkv, d), dtype=torch.uint8)
    vc, ks, vs = kc.clone(), torch.zeros((nb + 1, bs, hkv)), torch.zeros((nb + 1, bs, hkv))
    okc, ovc, oks, ovs = kc.numpy().copy(), vc.numpy().copy(), ks.numpy().copy(), vs.numpy().copy()
    oracle.kv_write_fp8(to_np(k), to_np(v), slots.numpy(), okc, ovc, oks, ovs, in_dtype)
    g = [t.to(dev) for t in (kc, vc, ks, vs)]
    pk.paged_kv_write_fp8(k.to(dev), v.to(dev), slots.to(dev), *g)
    torch.cuda.synchronize()
    live = np.ones((nb + 1) * bs, bool)
    live[-1] = False                                   # padding rows race for the scratch slot
    for got, want in zip(g, (okc, ovc, oks, ovs)):
        got = got.cpu().numpy().reshape((nb + 1) * bs, -1)[live]
        assert np.array_equal(got.view(np.uint8), want.reshape((nb + 1) * bs, -1)[live].view(np.uint8))


FP8 = [
    # (name, specs, H, Hkv, D, window); chunks over 64 query columns at D=128 take the
    # prefill kernel on the staged copy, everything else the small tiles
    ("decodes", [(1000, 1), (15, 1), (300, 1), (5000, 1), (0, 1)], 32, 8, 128, 0),
    ("chunks", [(700, 150), (90, 1), (0, 300)], 32, 8, 128, 0),
    ("spec_rows_d64", [(100, 2), (57, 3), (300, 4), (16, 5)], 8, 2, 64, 0),
    ("window", [(3000, 1), (200, 40), (9, 1)], 32, 8, 128, 100),
    ("long_chunk_g8", [(3000, 600), (37, 1), (0, 70)], 64, 8, 128, 0),
    ("chunk_window", [(2000, 400), (5, 1), (100, 33)], 32, 8, 128, 300),
    ("chunk_g2_tail", [(33, 200), (64, 64), (1000, 131)], 8, 4, 128, 0),
    ("chunk_d64_small_tiles", [(500, 300), (0, 77)], 64, 8, 64, 0),
]


@pytest.mark.parametrize("name,specs,h,hkv,d,window", FP8, ids=[f[0] for f in FP8])
def test_fp8_attention_parity(name, specs, h, hkv, d, window):
    """The step on fp8 pools: the write of the new tokens bit-exact, attention within the
    bf16 bound of the oracle's attention over the dequantized pools."""
    import oracle
    import paged_kv_attention_05_amd as pk
    from tests._util import to_np
    dev = torch.device("cuda:0")
    b = workloads.small_batch(specs, dtype="bf16", num_heads=h, num_kv_heads=hkv, head_dim=d,
                              seed=zlib.crc32(name.encode()) % 1000)
    kc, vc, ks, vs = _fp8_pools(b)
    g = [torch.from_numpy(x.copy()).to(dev) for x in (kc, vc, ks, vs)]
    pk.paged_kv_write_fp8(b.k.to(dev), b.v.to(dev), b.slot_mapping.to(dev), *g)
    out = pk.paged_attention_varlen(b.q.to(dev), g[0], g[1], b.query_start_loc.to(dev), b.seq_lens.to(dev),
                                    b.block_table.to(dev), b.block_size, b.scale,
                                    query_start_loc_host=b.query_start_loc_host, seq_lens_host=b.seq_lens_host,
                                    sliding_window=window, k_scale=g[2], v_scale=g[3])
    torch.cuda.synchronize()
    oracle.kv_write_fp8(to_np(b.k), to_np(b.v), b.slot_mapping.numpy(), kc, vc, ks, vs, "bf16")
    n = kc.shape[0] * kc.shape[1]
    for got, want in zip(g, (kc, vc, ks, vs)):
        assert np.array_equal(got.cpu().numpy().reshape(n, -1)[:-1].view(np.uint8),
                              want.reshape(n, -1)[:-1].view(np.uint8))
    _, ref64 = oracle.paged_attention(to_np(b.q), kc, vc, b.query_start_loc.numpy(), b.seq_lens.numpy(),
                                      b.block_table.numpy(), b.scale, "bf16", want_f64=True, window=window,
                                      k_scale=ks, v_scale=vs)
    err = attention_error(out.float().cpu().numpy(), ref64, "bf16")
    H.log(f"[parity] fp8_{name}: error {err:.3g} x bound")
    H.record({"case": f"fp8_{name}", "dtype": "bf16", "kv": "fp8_e4m3", "window": window, "error_x_bound": err})
    assert err <= 1.0, err


def _fp8_step(b, window=0):
    """KV write + attention on fp8 pools (the oracle's quantization of the batch's context
    pool); returns (GPU out, float64 oracle out) for every row."""
    import oracle
    import paged_kv_attention_05_amd as pk
    from tests._util import to_np
    dev = torch.device("cuda:0")
    kc, vc, ks, vs = _fp8_pools(b)
    g = [torch.from_numpy(x.copy()).to(dev) for x in (kc, vc, ks, vs)]
    pk.paged_kv_write_fp8(b.k.to(dev), b.v.to(dev), b.slot_mapping.to(dev), *g)
    out = pk.paged_attention_varlen(b.q.to(dev), g[0], g[1], b.query_start_loc.to(dev), b.seq_lens.to(dev),
                                    b.block_table.to(dev), b.block_size, b.scale,
                                    query_start_loc_host=b.query_start_loc_host, seq_lens_host=b.seq_lens_host,
                                    sliding_window=window, k_scale=g[2], v_scale=g[3])
    torch.cuda.synchronize()
    oracle.kv_write_fp8(to_np(b.k), to_np(b.v), b.slot_mapping.numpy(), kc, vc, ks, vs, "bf16")
    _, ref64 = oracle.paged_attention(to_np(b.q), kc, vc, b.query_start_loc.numpy(), b.seq_lens.numpy(),
                                      b.block_table.numpy(), b.scale, "bf16", want_f64=True, window=window,
                                      k_scale=ks, v_scale=vs)
    return out.float().cpu().numpy(), ref64


def test_fp8_inline_items_match_the_planner():
    """fp8 pools, a batch of decodes and speculative rows with key splits: the call without a
    planner launch gives the same bits as the one with it (path 2)."""
    import paged_kv_attention_05_amd as pk
    b = workloads.small_batch([(1000, 1), (15, 1), (5000, 1), (300, 3), (2100, 5), (0, 1)], dtype="bf16",
                              num_heads=32, num_kv_heads=8, head_dim=128, seed=91)
    outs = []
    for path in (0, 2):
        pk.set_path(path)
        try:
            outs.append(torch.from_numpy(_fp8_step(b)[0]))
        finally:
            pk.set_path(0)
    assert torch.equal(outs[0], outs[1])


def test_fp8_prefill_v_beyond_fp16_range():
    """fp8 pools whose dequantized V passes fp16's largest finite value (65504) in a few
    slots of one request (context and new tokens): that request's prefill items are redone
    by the bf16 kernel, the other request's stay on the fp16 kernel; both within the bound."""
    b = _plant_wide_v(workloads.small_batch([(500, 200), (300, 150)], dtype="bf16", num_heads=32,
                                            num_kv_heads=8, head_dim=128, seed=37))
    got, ref64 = _fp8_step(b)
    err = attention_error(got, ref64, "bf16")
    H.log(f"[parity] fp8 prefill with V beyond fp16: error {err:.3g} x bound")
    H.record({"case": "fp8_prefill_wide_v", "dtype": "bf16", "kv": "fp8_e4m3", "error_x_bound": err})
    assert err <= 1.0, err


def test_fp8_prefill_k_beyond_fp16_range():
    """fp8 pools whose dequantized K passes fp16's largest finite value (65504) in a few slots
    of one request (context and a new token): the prefill kernels keep K as exact codes and
    apply the float32 scales per score, so nothing overflows.  Those keys take (almost) all of
    the weight of the rows whose scores they dominate, so the rows stay of ordinary size."""
    b = workloads.small_batch([(500, 200), (300, 150)], dtype="bf16", num_heads=32, num_kv_heads=8,
                              head_dim=128, seed=38)
    r0 = b.requests[0]
    pool_k = b.k_cache.view(-1, b.num_kv_heads, b.head_dim)
    for pos, hk, d, val in [(9, 1, 17, 1.2e5), (333, 6, 90, -8.0e4)]:
        pool_k[workloads.slot_of(r0.blocks, pos, b.block_size), hk, d] = val
    b.k[5, 3, 40] = 9.5e4                # new token 5 of request 0
    got, ref64 = _fp8_step(b)
    err = attention_error(got, ref64, "bf16")
    H.log(f"[parity] fp8 prefill with K beyond fp16: error {err:.3g} x bound")
    H.record({"case": "fp8_prefill_wide_k", "dtype": "bf16", "kv": "fp8_e4m3", "error_x_bound": err})
    assert err <= 1.0, err


def test_fp8_prefill_q_beyond_fp16_range():
    """Finite query values past 65504 (bf16 holds them, fp16 does not) in prefill rows on fp8
    pools: the QK^T product stays in bf16 on the exact codes, so the rows come out right."""
    b = workloads.small_batch([(500, 200), (300, 150)], dtype="bf16", num_heads=32, num_kv_heads=8,
                              head_dim=128, seed=39)
    b.q[57, 9, 3] = 1.5e5                # request 0, row 57, query head 9 (KV head 2)
    b.q[260, 30, 100] = -7.0e4           # request 1, row 60
    got, ref64 = _fp8_step(b)
    err = attention_error(got, ref64, "bf16")
    H.log(f"[parity] fp8 prefill with q beyond fp16: error {err:.3g} x bound")
    H.record({"case": "fp8_prefill_wide_q", "dtype": "bf16", "kv": "fp8_e4m3", "error_x_bound": err})
    assert err <= 1.0, err


@pytest.mark.parametrize("scale", [-0.11, 0.0])
def test_negative_and_zero_scale_every_path(scale):
    """A negative softmax scale (applied as |scale| on -q) and a zero scale (uniform weights
    over the visible keys), through the prefill kernel, single and grouped small tiles, and
    both on fp8 pools (the staged K scales carry |scale| log2 e)."""
    specs = [(700, 150), (90, 1), (300, 9), (2000, 5), (0, 1)]
    b = workloads.small_batch(specs, dtype="bf16", num_heads=32, num_kv_heads=8, head_dim=128, seed=83)
    b.scale = scale
    H.check_batch(b, label=f"scale_{scale}")
    b8 = workloads.small_batch(specs, dtype="bf16", num_heads=32, num_kv_heads=8, head_dim=128, seed=84)
    b8.scale = scale
    got, ref64 = _fp8_step(b8)
    err = attention_error(got, ref64, "bf16")
    H.log(f"[parity] fp8 scale {scale}: error {err:.3g} x bound")
    assert err <= 1.0, err


def test_fp8_long_context_full_size():
    """The long-context batch (16 decodes at 32768 + a 4096-token chunk at 28672, 64/8
    heads) on fp8 pools: sampled rows, the chunk through the staged prefill kernel."""
    import oracle
    import paged_kv_attention_05_amd as pk
    from tests._util import to_np
    dev = torch.device("cuda:0")
    b = workloads.long_context()
    kc, vc, ks, vs = _fp8_pools(b)
    g = [torch.from_numpy(x.copy()).to(dev) for x in (kc, vc, ks, vs)]
    pk.paged_kv_write_fp8(b.k.to(dev), b.v.to(dev), b.slot_mapping.to(dev), *g)
    out = pk.paged_attention_varlen(b.q.to(dev), g[0], g[1], b.query_start_loc.to(dev), b.seq_lens.to(dev),
                                    b.block_table.to(dev), b.block_size, b.scale,
                                    query_start_loc_host=b.query_start_loc_host, seq_lens_host=b.seq_lens_host,
                                    k_scale=g[2], v_scale=g[3])
    torch.cuda.synchronize()
    oracle.kv_write_fp8(to_np(b.k), to_np(b.v), b.slot_mapping.numpy(), kc, vc, ks, vs, "bf16")
    mask = _sample_rows(b, 9)
    _, ref64 = oracle.paged_attention(to_np(b.q), kc, vc, b.query_start_loc.numpy(), b.seq_lens.numpy(),
                                      b.block_table.numpy(), b.scale, "bf16", want_f64=True, row_mask=mask,
                                      k_scale=ks, v_scale=vs)
    rows = np.nonzero(mask)[0]
    err = attention_error(out.float().cpu().numpy()[rows], ref64[rows], "bf16")
    H.log(f"[parity] fp8_long_context: error {err:.3g} x bound over {len(rows)} rows")
    H.record({"case": "fp8_long_context", "dtype": "bf16", "kv": "fp8_e4m3", "rows": int(len(rows)),
              "error_x_bound": err})
    assert err <= 1.0, err


def test_fp8_decode_only_full_size():
    """The 256-decode batch (seq_len 512..8192) on fp8 pools, every row."""
    import oracle
    import paged_kv_attention_05_amd as pk
    from tests._util import to_np
    dev = torch.device("cuda:0")
    b = workloads.decode_only()
    kc, vc, ks, vs = _fp8_pools(b)
    g = [torch.from_numpy(x.copy()).to(dev) for x in (kc, vc, ks, vs)]
    pk.paged_kv_write_fp8(b.k.to(dev), b.v.to(dev), b.slot_mapping.to(dev), *g)
    out = pk.paged_attention_varlen(b.q.to(dev), g[0], g[1], b.query_start_loc.to(dev), b.seq_lens.to(dev),
                                    b.block_table.to(dev), b.block_size, b.scale,
                                    query_start_loc_host=b.query_start_loc_host, seq_lens_host=b.seq_lens_host,
                                    k_scale=g[2], v_scale=g[3])
    torch.cuda.synchronize()
    oracle.kv_write_fp8(to_np(b.k), to_np(b.v), b.slot_mapping.numpy(), kc, vc, ks, vs, "bf16")
    _, ref64 = oracle.paged_attention(to_np(b.q), kc, vc, b.query_start_loc.numpy(), b.seq_lens.numpy(),
                                      b.block_table.numpy(), b.scale, "bf16", want_f64=True, k_scale=ks, v_scale=vs)
    err = attention_error(out.float().cpu().numpy(), ref64, "bf16")
    H.record({"case": "fp8_decode_only", "dtype": "bf16", "kv": "fp8_e4m3", "error_x_bound": err})
    assert err <= 1.0, err


# ------------------------------------------------------------------------- block copies
@pytest.mark.parametrize("dtype,shape", [("bf16", (41, 16, 8, 128)), ("f32", (23, 16, 4, 48)), ("bf16", (25, 1, 1, 8))],
                         ids=["bf16_d128", "f32_d48", "bf16_tiny_block"])
def test_copy_blocks_parity(dtype, shape):
    """swap_out to device and to pinned host staging, swap_in from pinned host, and
    copy-on-write inside the pool: every byte as the oracle's copy."""
    import oracle
    import paged_kv_attention_05_amd as pk
    from tests._util import to_np
    dev = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(51)
    pool = torch.randn(shape, generator=gen).to(workloads.TORCH_DTYPES[dtype])
    nb = shape[0]
    perm = torch.randperm(nb, generator=gen)
    out_ids, in_ids = perm[:7].to(torch.int64), perm[7:14].to(torch.int64)
    cow_src, cow_dst = perm[14:17].to(torch.int64), perm[17:20].to(torch.int64)
    n = len(out_ids)
    ref = to_np(pool).copy()
    gpu = pool.to(dev)
    # swap_out: pool -> device staging and pool -> pinned host staging
    st_dev = torch.zeros((n,) + shape[1:], dtype=pool.dtype, device=dev)
    st_host = torch.zeros((n,) + shape[1:], dtype=pool.dtype).pin_memory()
    seq = torch.arange(n, dtype=torch.int64)
    pk.paged_copy_blocks(gpu, st_dev, out_ids.to(dev), seq.to(dev))
    pk.paged_copy_blocks(gpu, st_host, out_ids.to(dev), seq.to(dev))
    torch.cuda.synchronize()
    want_st = np.zeros((n,) + ref.shape[1:], ref.dtype)
    oracle.copy_blocks(ref, want_st, out_ids.numpy(), seq.numpy())
    assert np.array_equal(to_np(st_dev.cpu()).view(np.uint8), want_st.view(np.uint8))
    assert np.array_equal(to_np(st_host).view(np.uint8), want_st.view(np.uint8))
    # swap_in: pinned host staging -> other blocks of the pool; then copy-on-write pairs
    pk.paged_copy_blocks(st_host, gpu, seq.to(dev), in_ids.to(dev))
    pk.paged_copy_blocks(gpu, gpu, cow_src.to(dev), cow_dst.to(dev))
    torch.cuda.synchronize()
    oracle.copy_blocks(want_st, ref, seq.numpy(), in_ids.numpy())
    oracle.copy_blocks(ref, ref, cow_src.numpy(), cow_dst.numpy())
    assert np.array_equal(to_np(gpu.cpu()).view(np.uint8), ref.view(np.uint8))


def test_swap_round_trip_keeps_attention():
    """Swap a prefill request's and a decode's blocks out to pinned host memory, poison them,
    swap them into free blocks and remap the tables: the GPU output is bit-identical."""
    import paged_kv_attention_05_amd as pk
    dev = torch.device("cuda:0")
    b = workloads.small_batch([(700, 150), (3000, 1), (40, 1)], dtype="bf16", num_heads=32, num_kv_heads=8,
                              head_dim=128, seed=52, num_blocks=600)
    ref, kc, vc = H.gpu_step(b)
    used = {x for r in b.requests for x in r.blocks}
    free = [x for x in range(b.num_blocks) if x not in used]
    table = b.block_table.clone()
    kc, vc = kc.to(dev), vc.to(dev)
    for r in (0, 1):
        blocks = torch.tensor(b.requests[r].blocks, dtype=torch.int64)
        n = len(blocks)
        new = torch.tensor(free[:n], dtype=torch.int64)
        free = free[n:]
        seq = torch.arange(n, dtype=torch.int64, device=dev)
        for pool in (kc, vc):
            host = torch.empty((n,) + tuple(pool.shape[1:]), dtype=pool.dtype).pin_memory()
            pk.paged_copy_blocks(pool, host, blocks.to(dev), seq)
            torch.cuda.synchronize()
            pool[blocks.to(dev)] = float("nan")
            pk.paged_copy_blocks(host, pool, seq, new.to(dev))
        table[r, :n] = new.to(torch.int32)
    out = pk.paged_attention_varlen(b.q.to(dev), kc, vc, b.query_start_loc.to(dev), b.seq_lens.to(dev),
                                    table.to(dev), b.block_size, b.scale,
                                    query_start_loc_host=b.query_start_loc_host, seq_lens_host=b.seq_lens_host)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu().view(torch.int16), ref.view(torch.int16))


def test_copy_blocks_debug_checks():
    import paged_kv_attention_05_amd as pk
    dev = torch.device("cuda:0")
    pool = torch.zeros((8, 16, 2, 64), dtype=torch.bfloat16, device=dev)
    pk.set_debug_checks(True)
    try:
        with pytest.raises(pk.PagedAttnError) as e:
            pk.paged_copy_blocks(pool, pool, torch.tensor([1, 2], device=dev), torch.tensor([3, 3], device=dev))
        assert e.value.code == -7
        with pytest.raises(pk.PagedAttnError):
            pk.paged_copy_blocks(pool, pool, torch.tensor([1], device=dev), torch.tensor([8], device=dev))
        with pytest.raises(pk.PagedAttnError):      # 2 is a destination and another pair's source
            pk.paged_copy_blocks(pool, pool, torch.tensor([1, 2], device=dev), torch.tensor([2, 5], device=dev))
    finally:
        pk.set_debug_checks(False)


# ------------------------------------------------------------------------- graph capture
GRAPH = [
    # (name, query rows of the 13 requests, padded request count: padding requests have one
    # row, slot -1 and seq_len 0, query heads, KV heads)
    ("decodes", [1] * 13, 16, 32, 8),
    ("spec_rows", [2, 3, 5, 9] * 3 + [2], 16, 32, 8),     # 1 + k rows: single and grouped tiles
    # g = 32 and 64: a token's heads fill two or four 16-column tiles, so every request (the
    # padding rows too) takes the grouped tiles
    ("decodes_g32", [1] * 13, 16, 32, 1),
    ("rows_g32", [2, 1, 2, 1] * 3 + [2], 16, 32, 1),
    ("decodes_g64", [1] * 13, 16, 64, 1),
]


@pytest.mark.parametrize("name,rows,pad,nh,nkv", GRAPH, ids=[g_[0] for g_ in GRAPH])
def test_graph_captured_decode_step_replays(name, rows, pad, nh, nkv):
    """A padded batch of 13 requests (pad_to of "Flattened ragged batches") captured once in
    a HIP graph as KV write + attention sized for seq_len <= 2048, then replayed on four
    batches with other lengths, tables and values copied into the captured buffers.  Every
    replay matches the oracle, and the same call made eagerly with the same sizing gives the
    same bits; eager work and synchronisations run between replays."""
    import paged_kv_attention_05_amd as pk
    dev = torch.device("cuda:0")
    MAX, NB, W = 2048, 2100, 2048 // 16
    R = pad
    rng = np.random.default_rng(61)

    def batch(seed):
        lens = [int(rng.integers(t, MAX)) for t in rows]
        return workloads.small_batch([(L - t, t) for L, t in zip(lens, rows)], dtype="bf16", num_heads=nh,
                                     num_kv_heads=nkv, head_dim=128, num_blocks=NB, seed=seed, pad_to=pad)

    def table_of(b):
        t = torch.zeros((R, W), dtype=torch.int32)
        t[:, :b.block_table.shape[1]] = b.block_table
        return t

    b0 = batch(100)
    st = {"q": b0.q.to(dev), "k": b0.k.to(dev), "v": b0.v.to(dev), "slots": b0.slot_mapping.to(dev),
          "qsl": b0.query_start_loc.to(dev), "lens": b0.seq_lens.to(dev), "table": table_of(b0).to(dev),
          "kc": b0.k_cache.to(dev), "vc": b0.v_cache.to(dev)}
    out = torch.empty_like(st["q"])
    qsl_host = b0.query_start_loc_host
    need = pk.paged_attention_workspace_bytes(nh, nkv, 128, 16, qsl_host, None, torch.bfloat16, graph_max_seq_len=MAX)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def step(o, kc, vc, wsp):
        pk.paged_kv_write(st["k"], st["v"], st["slots"], kc, vc)
        pk.paged_attention_varlen(st["q"], kc, vc, st["qsl"], st["lens"], st["table"], 16, b0.scale, o,
                                  query_start_loc_host=qsl_host, seq_lens_host=None, workspace=wsp,
                                  graph_max_seq_len=MAX)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out, st["kc"], st["vc"], ws)            # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out, st["kc"], st["vc"], ws)

    for i in range(4):
        b = batch(200 + i)
        assert b.query_start_loc_host == qsl_host
        for key, src in (("q", b.q), ("k", b.k), ("v", b.v), ("slots", b.slot_mapping), ("qsl", b.query_start_loc),
                         ("lens", b.seq_lens), ("table", table_of(b)), ("kc", b.k_cache), ("vc", b.v_cache)):
            st[key].copy_(src.to(dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu()
        # eager: the same sizing on fresh caches and workspace, then the oracle
        kc2, vc2 = b.k_cache.to(dev), b.v_cache.to(dev)
        out2 = torch.empty_like(st["q"])
        ws2 = torch.empty_like(ws)
        step(out2, kc2, vc2, ws2)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), out2.cpu().view(torch.int16)), i
        assert torch.equal(st["kc"].cpu().view(torch.int16)[:-1], kc2.cpu().view(torch.int16)[:-1])
        ref64, _, _ = H.oracle_step(b)
        err = attention_error(got.float().numpy(), ref64, "bf16")
        H.log(f"[parity] graph {name} replay {i}: error {err:.3g} x bound")
        assert err <= 1.0, (i, err)


# ------------------------------------------------------------------------- sliding window
WINDOW = [
    # (name, specs (computed, new), H, Hkv, D, bs, dtype, windows)
    ("decodes_bf16", [(1000, 1), (15, 1), (300, 1), (5000, 1), (0, 1)], 32, 8, 128, 16, "bf16", (1, 16, 100, 4096)),
    ("prefill_bf16", [(700, 150), (90, 1), (0, 300)], 32, 8, 128, 16, "bf16", (1, 63, 64, 65, 200, 1000)),
    ("spec_rows_bf16", [(100, 2), (57, 3), (300, 4), (16, 5)], 8, 2, 128, 16, "bf16", (2, 7)),
    ("vector_f32", [(60, 10), (1, 1), (0, 23), (3000, 1)], 8, 2, 48, 4, "f32", (1, 5, 64, 1000)),
    ("decodes_d64_long", [(20000, 1), (9000, 1)], 8, 1, 64, 16, "bf16", (300, 5000)),
    ("mixed_d48_bf16", [(1000, 1), (300, 3), (0, 20), (60, 40)], 8, 4, 48, 16, "bf16", (1, 100)),
]


@pytest.mark.parametrize("name,specs,h,hkv,d,bs,dtype,windows", WINDOW, ids=[w[0] for w in WINDOW])
def test_sliding_window(name, specs, h, hkv, d, bs, dtype, windows):
    b = workloads.small_batch(specs, dtype=dtype, num_heads=h, num_kv_heads=hkv, head_dim=d, block_size=bs,
                              seed=zlib.crc32(name.encode()) % 1000)
    for w in windows:
        H.check_batch(b, label=f"window_{name}_{w}", window=w)


def test_window_covering_every_context_changes_nothing():
    b = workloads.small_batch([(700, 150), (90, 1), (3000, 1)], dtype="bf16", num_heads=32, num_kv_heads=8,
                              head_dim=128, seed=41)
    ref, _, _ = H.gpu_step(b)
    for w in (3001, 1 << 30):
        got, _, _ = H.gpu_step(b, window=w)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), w


def test_long_context_full_size_window():
    b = workloads.long_context()
    H.check_batch(b, row_mask=_sample_rows(b, 6), label="long_context_window_4096", window=4096)


def _plant_wide_v(b):
    """Request 0 of b gets V values past fp16's largest finite value (65504) in three context
    slots and in one of its new tokens.  The K rows of those (slot, KV head) pairs are zeroed,
    so every row gives them a small weight: the outputs stay of ordinary size, where the bf16
    bound measures the arithmetic rather than the rounding of a 10^5-sized output, while the
    whole request still has to take the redo path (an fp16 V would hold infinities)."""
    r0 = b.requests[0]
    pool_k = b.k_cache.view(-1, b.num_kv_heads, b.head_dim)
    pool_v = b.v_cache.view(-1, b.num_kv_heads, b.head_dim)
    for pos, hk, d, val in [(7, 0, 3, 1.0e5), (260, 5, 100, -2.5e5), (431, 7, 64, 7.0e4)]:
        slot = workloads.slot_of(r0.blocks, pos, b.block_size)
        pool_v[slot, hk, d] = val
        pool_k[slot, hk, :] = 0.0
    b.v[3, 2, 5] = 9.0e4                 # row 3 of request 0 (position 503)
    b.k[3, 2, :] = 0.0
    return b


def _wide_v_batch():
    """Two prefill chunks, request 0 with V beyond fp16's range (_plant_wide_v)."""
    return _plant_wide_v(workloads.small_batch([(500, 200), (300, 150)], dtype="bf16", num_heads=32,
                                               num_kv_heads=8, head_dim=128, seed=31))


def test_prefill_v_beyond_fp16_range():
    """Such a request takes the bf16 prefill kernel; the other one stays on the fp16 kernel."""
    H.check_batch(_wide_v_batch(), label="prefill_wide_v")


def test_prefill_range_flags_cleared_between_calls():
    """An ordinary batch gives the same bits before and after a wide-V call that used the same
    workspace: the per-item redo flags start cleared on every call."""
    import paged_kv_attention_05_amd as pk
    dev = torch.device("cuda:0")
    plain = workloads.small_batch([(500, 200), (300, 150)], dtype="bf16", num_heads=32, num_kv_heads=8,
                                  head_dim=128, seed=32)
    wide = _wide_v_batch()

    def run(b, ws):
        kc, vc = b.k_cache.to(dev), b.v_cache.to(dev)
        pk.paged_kv_write(b.k.to(dev), b.v.to(dev), b.slot_mapping.to(dev), kc, vc)
        return pk.paged_attention_varlen(b.q.to(dev), kc, vc, b.query_start_loc.to(dev), b.seq_lens.to(dev),
                                         b.block_table.to(dev), b.block_size, b.scale,
                                         query_start_loc_host=b.query_start_loc_host, seq_lens_host=b.seq_lens_host,
                                         workspace=ws)

    need = max(pk.paged_attention_workspace_bytes(32, 8, 128, 16, x.query_start_loc_host, x.seq_lens_host,
                                                  torch.bfloat16) for x in (plain, wide))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    before = run(plain, ws).cpu()
    run(wide, ws)
    after = run(plain, ws).cpu()
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int16), after.view(torch.int16))


def test_padding_rows_and_zero_length():
    b = workloads.small_batch([(10, 2), (0, 5), (30, 1)], dtype="bf16", num_heads=8, num_kv_heads=2,
                              head_dim=128, pad_to=7, seed=21)
    assert b.seq_lens_host[-4:] == [0, 0, 0, 0]
    H.check_batch(b, label="padding_rows")


def test_empty_batch():
    import paged_kv_attention_05_amd as pk
    kc = torch.zeros((2, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = pk.paged_attention_varlen(q, kc, kc, z, z[:0], torch.zeros((0, 1), dtype=torch.int32, device="cuda"), 16,
                                    0.125, query_start_loc_host=[0], seq_lens_host=[])
    torch.cuda.synchronize()
    assert out.shape == (0, 4, 64)


def test_request_with_no_rows():
    b = workloads.small_batch([(10, 2), (20, 0), (5, 1)], dtype="bf16", num_heads=8, num_kv_heads=2,
                              head_dim=128, seed=22)
    H.check_batch(b, label="request_with_no_rows")


def test_plain_entry_points_through_ctypes():
    """paged_kv_write and the plain paged_attention_varlen (no options struct) called through
    the C ABI with device buffers, a workspace sized by the plain
    paged_attention_workspace_bytes, and the default stream: a chunk, decodes, verification
    rows and a padding row, against the oracle."""
    import ctypes
    import paged_kv_attention_05_amd as pk
    lib = pk.load_library()
    b = workloads.small_batch([(300, 150), (1000, 1), (57, 3), (0, 20)], dtype="bf16", num_heads=32, num_kv_heads=8,
                              head_dim=128, pad_to=5, seed=23)
    dev = torch.device("cuda:0")
    t = {n: getattr(b, n).to(dev).contiguous() for n in ("q", "k", "v", "k_cache", "v_cache", "slot_mapping",
                                                          "query_start_loc", "seq_lens", "block_table")}
    out = torch.full_like(t["q"], float("nan"))
    P = lambda x: ctypes.c_void_p(x.data_ptr())
    host = lambda xs: (ctypes.c_int32 * len(xs))(*xs)
    R, N, Hq, Hkv, D = b.num_reqs, b.num_tokens, b.num_heads, b.num_kv_heads, b.head_dim
    num_slots = b.num_slots
    need = lib.paged_attention_workspace_bytes(R, N, Hq, Hkv, D, b.block_size, host(b.query_start_loc_host),
                                               host(b.seq_lens_host), 1)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    assert lib.paged_kv_write(P(t["k"]), P(t["v"]), P(t["slot_mapping"]), P(t["k_cache"]), P(t["v_cache"]), N, Hkv,
                              D, num_slots, 1, 1, None) == 0
    rc = lib.paged_attention_varlen(P(t["q"]), P(t["k_cache"]), P(t["v_cache"]), P(t["query_start_loc"]),
                                    P(t["seq_lens"]), P(t["block_table"]), b.block_size, ctypes.c_float(b.scale),
                                    P(out), R, N, Hq, Hkv, D, t["block_table"].shape[1], num_slots,
                                    host(b.query_start_loc_host), host(b.seq_lens_host), b.max_query_len,
                                    b.max_seq_len, P(ws), need, 1, None)
    assert rc == 0, lib.paged_attn_last_error()
    torch.cuda.synchronize()
    ref64, okc, ovc = H.oracle_step(b)
    H.assert_pools_equal(t["k_cache"].cpu(), okc)
    H.assert_pools_equal(t["v_cache"].cpu(), ovc)
    err = attention_error(out.float().cpu().numpy(), ref64, "bf16")
    H.log(f"[parity] plain entry points: error {err:.3g} x bound")
    assert err <= 1.0, err


# ------------------------------------------------------------------------------ invariants on the GPU
def _gpu_out(batch, path=0):
    out, _, _ = H.gpu_step(batch, path=path)
    return out.float().numpy()


@pytest.mark.parametrize("dtype,d,L", [("bf16", 128, 300), ("bf16", 128, 5000), ("bf16", 48, 300), ("f32", 48, 300),
                                       ("f32", 48, 5000)])
def test_gpu_chunking_invariance(dtype, d, L):
    """A prompt prefilled in one piece or in chunks of 8, 33, 64 or 4096 tokens (each step
    writes its chunk, then attends) matches the oracle's one-shot output within the bound,
    every run on its own; the report says whether a chunked run is bit-exact with the
    one-piece run.  At L = 5000 the 4096-token chunk really splits the prompt."""
    import oracle
    import paged_kv_attention_05_amd as pk
    from tests._util import to_np
    hq, hkv, bs = 8, 2, 16
    H.log(f"[invariance] chunking {dtype} d={d} L={L}")
    gen = torch.Generator().manual_seed(31 + L)
    tdt = workloads.TORCH_DTYPES[dtype]
    q_c = torch.randn((L, hq, d), generator=gen).to(tdt)
    k_c = torch.randn((L, hkv, d), generator=gen).to(tdt)
    v_c = torch.randn((L, hkv, d), generator=gen).to(tdt)
    nb = L // bs + 3
    table = torch.randperm(nb, generator=gen)[: -(-L // bs)].to(torch.int32)
    pos = torch.arange(L)
    slots = table[pos // bs].to(torch.int64) * bs + pos % bs
    # the oracle's one-shot step: write every token, then attend with all L rows
    okc = np.full((nb + 1, bs, hkv, d), np.nan, np.float32)
    okc = to_np(torch.from_numpy(okc).to(tdt)).copy()
    ovc = okc.copy()
    oracle.kv_write(to_np(k_c), to_np(v_c), slots.numpy(), okc, ovc, dtype, dtype)
    _, ref64 = oracle.paged_attention(to_np(q_c), okc, ovc, np.array([0, L], np.int32), np.array([L], np.int32),
                                      table[None, :].numpy(), 1 / math.sqrt(d), dtype, want_f64=True)
    q, k, v = q_c.cuda(), k_c.cuda(), v_c.cuda()
    outs = {}
    for chunk in (L, 8, 33, 64, 4096):
        kc = torch.full((nb + 1, bs, hkv, d), float("nan"), dtype=tdt, device="cuda")
        vc = kc.clone()
        pieces = []
        for a in range(0, L, chunk):
            e = min(L, a + chunk)
            pk.paged_kv_write(k[a:e], v[a:e], slots[a:e].cuda(), kc, vc)
            pieces.append(pk.paged_attention_varlen(
                q[a:e].contiguous(), kc, vc, torch.tensor([0, e - a], dtype=torch.int32, device="cuda"),
                torch.tensor([e], dtype=torch.int32, device="cuda"), table[None, :].cuda().contiguous(), bs,
                1 / math.sqrt(d), query_start_loc_host=[0, e - a], seq_lens_host=[e]))
        outs[chunk] = torch.cat(pieces).float().cpu().numpy()
        err = attention_error(outs[chunk], ref64, dtype)
        exact = chunk != L and np.array_equal(outs[chunk], outs[L])
        H.log(f"[invariance] L={L} chunk {chunk}: error {err:.3g} x bound"
              f"{' (bit-exact with one piece)' if exact else ''}")
        H.record({"case": f"chunking_{dtype}_L{L}_{chunk}", "error_x_bound": err, "bit_exact": bool(exact)})
        assert err <= 1.0, (chunk, err)


def test_gpu_block_relabelling_and_batch_composition():
    b = workloads.small_batch([(300, 1), (40, 8), (1000, 1), (77, 3), (0, 40), (12, 1), (600, 2), (5, 1)],
                              dtype="bf16", num_heads=16, num_kv_heads=4, head_dim=128, seed=41)
    ref = _gpu_out(b)
    # relabel: move every block to a new id and remap the tables
    pi = torch.randperm(b.num_blocks, generator=torch.Generator().manual_seed(42))
    for name in ("k_cache", "v_cache"):
        old = getattr(b, name)
        new = old.clone()
        new[pi] = old[: b.num_blocks]
        setattr(b, name, new)
    b.block_table = torch.where(torch.arange(b.block_table.shape[1])[None, :] <
                                torch.tensor([len(r.blocks) for r in b.requests])[:, None],
                                pi[b.block_table.long()].to(torch.int32), b.block_table)
    for r in b.requests:
        r.blocks = [int(pi[x]) for x in r.blocks]
    b.slot_mapping = torch.tensor([workloads.slot_of(r.blocks, p, b.block_size)
                                   for r in b.requests for p in range(r.computed, r.seq_len)], dtype=torch.int64)
    relabelled = _gpu_out(b)
    H.log(f"[invariance] relabelling: {'bit-exact' if np.array_equal(relabelled, ref) else 'differs'}")
    H.record({"case": "relabelling", "bit_exact": bool(np.array_equal(relabelled, ref))})
    assert np.array_equal(relabelled, ref)
    # the first request alone
    alone = workloads.small_batch([(300, 1)], dtype="bf16", num_heads=16, num_kv_heads=4, head_dim=128, seed=41)
    alone.k_cache, alone.v_cache = b.k_cache, b.v_cache
    alone.block_table = b.block_table[:1].contiguous()
    alone.requests = b.requests[:1]
    alone.slot_mapping = b.slot_mapping[:1]
    alone.q, alone.k, alone.v = b.q[:1], b.k[:1], b.v[:1]
    got = _gpu_out(alone)
    H.log(f"[invariance] alone vs batched: {'bit-exact' if np.array_equal(got, ref[:1]) else 'differs'}")
    H.record({"case": "alone_vs_batched", "bit_exact": bool(np.array_equal(got, ref[:1]))})
    assert attention_error(got, ref[:1].astype(np.float64), "bf16") <= 1.0


def test_gpu_aliasing():
    """Requests whose tables share prefix blocks (written in this very step by the first
    request) match the oracle."""
    b = workloads.small_batch([(0, 64), (64, 1), (100, 1), (64, 30)], dtype="bf16", num_heads=8, num_kv_heads=2,
                              head_dim=128, shared_prefix_blocks=4, seed=51)
    H.check_batch(b, label="aliased_prefix")


def test_many_requests_cross_planner_chunks():
    """More requests than the planner kernel takes in one chunk (512): the per-request
    offsets carry across chunks, and each chunk boundary sits between requests of different
    kinds (decodes, verification rows, prefill chunks, zero-row and zero-length requests).
    Both item lists are checked: the matrix-core kernels' and the vector kernel's."""
    rng = np.random.default_rng(91)
    specs = []
    for r in range(2600):
        if r in (511, 1022, 1023, 1535, 2047, 2049):        # prefill chunks at the chunk edges
            specs.append((int(rng.integers(0, 300)), int(rng.integers(65, 200))))
        elif r in (512, 1024, 2048):
            specs.append((int(rng.integers(1, 50)), 0))     # a request with no rows this step
        elif r % 97 == 5:
            specs.append((int(rng.integers(1, 400)), int(rng.integers(2, 10))))   # verification rows
        elif r % 211 == 7:
            specs.append((0, 1))                            # a first token
        else:
            specs.append((int(rng.integers(1, 300)), 1))    # decodes
    b = workloads.small_batch(specs, dtype="bf16", num_heads=8, num_kv_heads=2, head_dim=128, seed=92)
    assert b.num_reqs > 2048
    H.check_batch(b, label="many_requests")
    H.check_batch(b, path=1, label="many_requests_vector")


def test_mfma_probe_runs():
    """The matrix-core probe runs and reports its launch's operation count: grid x 8 waves x
    iters x 8 products x 2*32*32*16."""
    import paged_kv_attention_05_amd as pk
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for iters, grid in ((1, 1), (64, 256), (16, 2048)):
        for rnd in (False, True):
            assert pk.mfma_probe(iters, grid, sink, random_operands=rnd) == grid * 8 * iters * 8 * 2 * 32 * 32 * 16
    torch.cuda.synchronize()


def test_hbm_read_probe_runs():
    """The measurement probe reads a buffer end to end (it writes its sink only for one
    unlikely xor value) without an error."""
    import paged_kv_attention_05_amd as pk
    buf = torch.ones(16 << 20, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for grid in (1, 256, 4096):
        pk.hbm_read_probe(buf, sink, grid)
    torch.cuda.synchronize()
