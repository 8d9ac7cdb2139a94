"""Pins for the CPU oracle: checks against what the pages and the mathematics fix, none of
which reuses the oracle's own code.

Each ``check_*`` function takes the oracle module and raises AssertionError on a mismatch.
``test_oracle_pins.py`` runs them against the oracle; ``test_oracle_mutants.py`` runs them
against copies of the oracle with a planted mistake and requires that each mistake trips
at least one of them.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

import workloads
from tests._util import as_f64, dense_fold_attention, from_np, sdpa_attention, to_np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------------------------------
# scenario: contiguous per-request K/V/Q drawn here, scattered into a permuted pool here
# ------------------------------------------------------------------------------------------

class Scenario:
    """Requests given as (computed, new) with contiguous K, V [L, Hkv, D] and Q [t, H, D],
    scattered into a pool through tables taken from a random permutation of block ids."""

    def __init__(self, specs, H, Hkv, D, bs, dtype="f32", seed=0, num_blocks=None, shared=None,
                 qzero=False, vconst=None):
        rng = np.random.default_rng(seed)
        self.specs, self.H, self.Hkv, self.D, self.bs, self.dtype = list(specs), H, Hkv, D, bs, dtype
        self.ctx_k, self.ctx_v, self.q = [], [], []
        for c, t in self.specs:
            L = c + t
            k = rng.standard_normal((L, Hkv, D)).astype(np.float32)
            v = rng.standard_normal((L, Hkv, D)).astype(np.float32)
            q = rng.standard_normal((t, H, D)).astype(np.float32)
            if qzero:
                q[:] = 0
            if vconst is not None:
                v[:] = np.float32(vconst)
            self.ctx_k.append(self._store(k))
            self.ctx_v.append(self._store(v))
            self.q.append(self._store(q))
        need = sum(-(-(c + t) // bs) for c, t in self.specs)
        self.num_blocks = num_blocks or need + 3
        perm = rng.permutation(self.num_blocks)
        self.tables, nxt = [], 0
        for c, t in self.specs:
            nb = -(-(c + t) // bs)
            self.tables.append([int(b) for b in perm[nxt:nxt + nb]])
            nxt += nb
        self.build_pool()

    def _store(self, x):
        """Round float32 draws to the storage dtype; keep oracle-format arrays."""
        if self.dtype == "f32":
            return x
        return to_np(torch.from_numpy(x).to(torch.bfloat16))

    def build_pool(self):
        hkv, d, bs = self.Hkv, self.D, self.bs
        shape = ((self.num_blocks + 1) * bs, hkv, d)
        if self.dtype == "f32":
            kp = np.full(shape, np.nan, dtype=np.float32)
        else:
            kp = np.full(shape, 0x7FC0, dtype=np.uint16)
        vp = kp.copy()
        for r, (c, t) in enumerate(self.specs):
            for p in range(c + t):
                s = workloads.slot_of(self.tables[r], p, bs)
                kp[s] = self.ctx_k[r][p]
                vp[s] = self.ctx_v[r][p]
        self.k_pool = kp.reshape(self.num_blocks + 1, bs, hkv, d)
        self.v_pool = vp.reshape(self.num_blocks + 1, bs, hkv, d)

    def meta(self):
        qsl = [0]
        for c, t in self.specs:
            qsl.append(qsl[-1] + t)
        lens = [c + t for c, t in self.specs]
        width = max(1, max(len(t) for t in self.tables))
        table = np.zeros((len(self.specs), width), dtype=np.int32)
        for r, tb in enumerate(self.tables):
            table[r, :len(tb)] = tb
        return np.array(qsl, np.int32), np.array(lens, np.int32), table

    def run_oracle(self, orc, scale=None, want_f64=True, window=0):
        qsl, lens, table = self.meta()
        q = np.concatenate(self.q, axis=0) if self.q else np.zeros((0, self.H, self.D), np.float32)
        scale = 1.0 / math.sqrt(self.D) if scale is None else scale
        kw = {"window": window} if window else {}
        return orc.paged_attention(np.ascontiguousarray(q), self.k_pool, self.v_pool, qsl, lens, table,
                                   scale, self.dtype, want_f64=want_f64, **kw)

    def dense(self, r, scale=None, ref=dense_fold_attention, window=0):
        c, t = self.specs[r]
        scale = 1.0 / math.sqrt(self.D) if scale is None else scale
        return ref(as_f64(self.q[r], self.dtype), as_f64(self.ctx_k[r], self.dtype),
                   as_f64(self.ctx_v[r], self.dtype), scale, c, window=window)


def _rel_err(a, b):
    """max |a - b| relative to the max |b| of each (row, head)."""
    den = np.maximum(np.abs(b).max(axis=-1, keepdims=True), 1e-300)
    return float((np.abs(a - b) / den).max()) if a.size else 0.0


# ------------------------------------------------------------------------------------------
# integer pins from the pages' worked examples
# ------------------------------------------------------------------------------------------

def check_slot_formula_page_example(orc=None):
    g = _golden("p3_block_table_example.json")
    got = [workloads.slot_of(g["table"], p, g["block_size"]) for p in g["positions"]]
    assert got == g["slots"], got


def check_worked_batch_layout(orc=None):
    g = _golden("worked_batch_layout.json")
    b = workloads.worked_batch()
    assert b.positions.tolist() == g["positions"]
    assert b.query_start_loc_host == g["query_start_loc"]
    assert b.seq_lens_host == g["seq_lens"]
    assert [len(r.blocks) for r in b.requests] == g["blocks_per_request"]
    assert [(r.computed, r.new) for r in b.requests] == [tuple(x) for x in g["requests"]]


def check_gather_follows_page_example(orc):
    """A pool whose every element holds its own slot number, gathered through the page's
    table [4, 9, 2, 6]: the gathered rows must carry the slots the page's example gives."""
    g = _golden("p3_block_table_example.json")
    bs, nb = g["block_size"], 10
    pool = np.repeat(np.arange((nb + 1) * bs, dtype=np.float32), 2 * 3).reshape(nb + 1, bs, 2, 3)
    ctx = orc.gather_context(pool, np.array(g["table"], np.int32), 64, "f32")
    assert ctx.shape == (64, 2, 3)
    got = [int(ctx[p, 0, 0]) for p in g["positions"]]
    assert got == g["slots"], got
    assert np.all(ctx == ctx[:, :1, :1])


# ------------------------------------------------------------------------------------------
# the write: index_copy_ semantics of the page's write_kv, bit for bit
# ------------------------------------------------------------------------------------------

def _write_case(orc, in_dtype, cache_dtype, seed):
    gen = torch.Generator().manual_seed(seed)
    n, hkv, d, bs, nb = 37, 3, 8, 4, 20
    tin, tc = workloads.TORCH_DTYPES[in_dtype], workloads.TORCH_DTYPES[cache_dtype]
    k = (torch.randn((n, hkv, d), generator=gen) * 3).to(tin)
    v = (torch.randn((n, hkv, d), generator=gen) * 3).to(tin)
    pool_k = torch.randn(((nb + 1) * bs, hkv, d), generator=gen).to(tc)
    pool_v = torch.randn(((nb + 1) * bs, hkv, d), generator=gen).to(tc)
    slots = torch.randperm(nb * bs, generator=gen)[:n].to(torch.int64)
    slots[[3, 11, 30]] = -1
    slots[17] = -5
    # expected: torch's index_copy_ on the flat pool, negative slots redirected to the last slot
    exp_k, exp_v = pool_k.clone(), pool_v.clone()
    idx = torch.where(slots >= 0, slots, torch.full_like(slots, (nb + 1) * bs - 1))
    exp_k.index_copy_(0, idx, k.to(tc))
    exp_v.index_copy_(0, idx, v.to(tc))
    got_k, got_v = to_np(pool_k).copy(), to_np(pool_v).copy()
    orc.kv_write(to_np(k), to_np(v), slots.numpy(), got_k.reshape(nb + 1, bs, hkv, d),
                 got_v.reshape(nb + 1, bs, hkv, d), in_dtype, cache_dtype)
    scratch = (nb + 1) * bs - 1
    live = np.ones((nb + 1) * bs, bool)
    live[scratch] = False                      # many rows race for the scratch slot
    assert np.array_equal(got_k[live], to_np(exp_k)[live])
    assert np.array_equal(got_v[live], to_np(exp_v)[live])


def check_kv_write_index_copy(orc):
    for i, (a, b) in enumerate([("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"), ("bf16", "f32")]):
        _write_case(orc, a, b, seed=10 + i)


def check_kv_write_scratch_gets_a_padding_row(orc):
    """All rows padding: the scratch slot holds one of them and nothing else changes."""
    n, hkv, d, bs, nb = 4, 1, 2, 2, 3
    k = np.arange(n * hkv * d, dtype=np.float32).reshape(n, hkv, d) + 1
    pool = np.zeros((nb + 1, bs, hkv, d), np.float32)
    pool2 = pool.copy()
    orc.kv_write(k, k.copy(), np.full(n, -1, np.int64), pool, pool2, "f32", "f32")
    flat = pool.reshape(-1, hkv, d)
    assert np.all(flat[:-1] == 0)
    assert any(np.array_equal(flat[-1], k[i]) for i in range(n))


def check_bf16_rounding(orc):
    """Round-to-nearest-even to bfloat16: against torch's conversion of float32 values,
    and against exact rational rounding for float64 values that are not float32."""
    rng = np.random.default_rng(7)
    f = rng.standard_normal(20000).astype(np.float32) * np.float32(1e3)
    bits = f.view(np.uint32)
    ties = ((bits & ~np.uint32(0xFFFF)) | np.uint32(0x8000)).view(np.float32)        # exact halfway
    tiny = (rng.integers(1, 1 << 23, 2000).astype(np.uint32)).view(np.float32)       # subnormals
    vals = np.concatenate([f, ties, tiny, np.array([0.0, -0.0, 1.0, -2.5, 3.3895e38, 3.4e38,
                                                    np.inf, -np.inf], np.float32)])
    want = to_np(torch.from_numpy(vals).to(torch.bfloat16))
    got = np.array([orc.round_to_bf16(float(x)) for x in vals], np.uint16)
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:5]
    # doubles just above and below a bfloat16 tie: no double rounding through float32
    for m in range(129, 255, 3):
        base = Fraction(m, 128) + Fraction(1, 256)           # halfway between m/128 and (m+1)/128
        for delta, up in ((Fraction(1, 2 ** 40), True), (-Fraction(1, 2 ** 40), False)):
            x = float(base + delta)
            want_val = Fraction(m + 1, 128) if up else Fraction(m, 128)
            got_bits = orc.round_to_bf16(x)
            got_val = Fraction(float(np.array([got_bits << 16], np.uint32).view(np.float32)[0]))
            assert got_val == want_val, (m, delta, got_val, want_val)
    assert orc.round_to_bf16(float("nan")) & 0x7FFF > 0x7F80


# ------------------------------------------------------------------------------------------
# attention: dense brute force, closed forms
# ------------------------------------------------------------------------------------------

DENSE_CASES = [
    # specs (computed, new), H, Hkv, D, bs
    ([(6, 3), (41, 1), (9, 1), (0, 4)], 8, 4, 48, 16),
    ([(0, 5), (13, 2), (30, 40)], 4, 4, 8, 16),
    ([(5, 1), (0, 17), (16, 16), (47, 1), (2, 7)], 8, 1, 8, 16),
    ([(60, 10), (1, 1)], 8, 2, 48, 4),
    ([(3, 3)], 16, 2, 8, 1),
]


def check_dense_fold(orc):
    for i, (specs, H, Hkv, D, bs) in enumerate(DENSE_CASES):
        sc = Scenario(specs, H, Hkv, D, bs, seed=100 + i)
        _, got = sc.run_oracle(orc)
        row = 0
        for r, (c, t) in enumerate(specs):
            want = sc.dense(r)
            err = _rel_err(got[row:row + t], want)
            assert err < 1e-12, (i, r, err)
            row += t


def check_dense_sdpa_bf16(orc):
    sc = Scenario([(20, 5), (0, 9), (33, 1)], 8, 2, 48, 16, dtype="bf16", seed=5)
    out, got = sc.run_oracle(orc)
    row = 0
    for r, (c, t) in enumerate(sc.specs):
        want = sc.dense(r, ref=sdpa_attention)
        assert _rel_err(got[row:row + t], want) < 1e-12
        # the stored output is the float64 result rounded once to bfloat16
        exp_bits = to_np(torch.from_numpy(want.astype(np.float32)).to(torch.bfloat16))
        diff = np.abs(as_f64(out[row:row + t], "bf16") - want)
        ulp = np.abs(as_f64(exp_bits, "bf16")) * 2.0 ** -7 + 1e-38
        assert np.all(diff <= 0.5 * ulp * (1 + 1e-6)), float((diff / ulp).max())
        row += t


def check_position_zero_is_v0(orc):
    """A row at position 0 sees only key 0, so its output is v_0 exactly."""
    sc = Scenario([(0, 6), (0, 1), (12, 3)], 8, 4, 48, 16, seed=3)
    out, _ = sc.run_oracle(orc)
    g = sc.H // sc.Hkv
    for h in range(sc.H):
        assert np.array_equal(out[0, h], sc.ctx_v[0][0, h // g])
        assert np.array_equal(out[6, h], sc.ctx_v[1][0, h // g])


def check_zero_query_gives_prefix_mean(orc):
    """q = 0: every allowed score is 0, so row i outputs the mean of v_0 .. v_pos."""
    sc = Scenario([(10, 5), (0, 8), (29, 1)], 4, 2, 8, 4, seed=4, qzero=True)
    _, got = sc.run_oracle(orc)
    row = 0
    for r, (c, t) in enumerate(sc.specs):
        v = as_f64(sc.ctx_v[r], "f32")
        csum = np.cumsum(v, axis=0)
        for i in range(t):
            pos = c + i
            mean = csum[pos] / (pos + 1)                           # [Hkv, D]
            want = np.repeat(mean, sc.H // sc.Hkv, axis=0)
            assert np.allclose(got[row + i], want, rtol=1e-12, atol=1e-13)
        row += t


def check_constant_values(orc):
    sc = Scenario([(7, 2), (0, 3)], 4, 2, 8, 4, seed=6, vconst=1.75)
    _, got = sc.run_oracle(orc)
    assert np.allclose(got, 1.75, rtol=0, atol=1e-14)


def check_dominant_key(orc):
    """One key aligned with the query and scaled up: the output tends to that key's value."""
    sc = Scenario([(19, 1)], 2, 1, 8, 4, seed=8)
    j = 11
    q = as_f64(sc.q[0], "f32")[0, 0]
    sc.ctx_k[0][j, 0] = (q * 400.0 / np.dot(q, q)).astype(np.float32)    # score ~ 400 / sqrt(D)
    sc.q[0][0, 1] = sc.q[0][0, 0]
    sc.build_pool()
    _, got = sc.run_oracle(orc)
    assert np.allclose(got[0, 0], sc.ctx_v[0][j, 0], rtol=0, atol=1e-12)
    assert np.allclose(got[0, 1], sc.ctx_v[0][j, 0], rtol=0, atol=1e-12)


def check_large_scores(orc):
    """Scores in the thousands: softmax is shift-invariant, so the result stays finite and
    equal to the dense reference (which subtracts the row maximum itself)."""
    sc = Scenario([(9, 3), (0, 4)], 4, 2, 8, 4, seed=17)
    for r in range(2):
        sc.q[r] *= np.float32(40.0)
        sc.ctx_k[r] *= np.float32(40.0)
    sc.build_pool()
    _, got = sc.run_oracle(orc)
    assert np.all(np.isfinite(got))
    row = 0
    for r, (c, t) in enumerate(sc.specs):
        assert _rel_err(got[row:row + t], sc.dense(r)) < 1e-9
        row += t


# ------------------------------------------------------------------------------------------
# sliding window ("Attention over the pool": allowed = k_pos > q_pos - window)
# ------------------------------------------------------------------------------------------

WINDOW_CASES = [
    # specs, H, Hkv, D, bs, windows
    ([(6, 3), (41, 1), (9, 1), (0, 4)], 8, 4, 48, 16, (1, 2, 5, 16, 40)),
    ([(60, 10), (1, 1), (0, 23)], 8, 2, 8, 4, (3, 7, 64)),
]


def check_window_dense(orc):
    for i, (specs, H, Hkv, D, bs, windows) in enumerate(WINDOW_CASES):
        sc = Scenario(specs, H, Hkv, D, bs, seed=200 + i)
        for w in windows:
            _, got = sc.run_oracle(orc, window=w)
            row = 0
            for r, (c, t) in enumerate(specs):
                err = _rel_err(got[row:row + t], sc.dense(r, window=w))
                assert err < 1e-12, (i, w, r, err)
                row += t


def check_window_sdpa_bf16(orc):
    sc = Scenario([(20, 5), (0, 9), (33, 1)], 8, 2, 48, 16, dtype="bf16", seed=25)
    _, got = sc.run_oracle(orc, window=6)
    row = 0
    for r, (c, t) in enumerate(sc.specs):
        assert _rel_err(got[row:row + t], sc.dense(r, ref=sdpa_attention, window=6)) < 1e-12
        row += t


def check_window_one_is_own_v(orc):
    """A window of one token leaves each row only its own key: the output is its own V row."""
    sc = Scenario([(12, 4), (0, 3)], 8, 2, 16, 4, seed=26)
    out, _ = sc.run_oracle(orc, window=1)
    g, row = sc.H // sc.Hkv, 0
    for r, (c, t) in enumerate(sc.specs):
        for i in range(t):
            for h in range(sc.H):
                assert np.array_equal(out[row + i, h], sc.ctx_v[r][c + i, h // g]), (r, i, h)
        row += t


def check_window_zero_query_gives_window_mean(orc):
    """q = 0: every visible score is 0, so row i outputs the mean of its last w values."""
    sc = Scenario([(10, 5), (0, 8), (29, 1)], 4, 2, 8, 4, seed=27, qzero=True)
    for w in (2, 3, 11):
        _, got = sc.run_oracle(orc, window=w)
        row = 0
        for r, (c, t) in enumerate(sc.specs):
            v = as_f64(sc.ctx_v[r], "f32")
            csum = np.concatenate([np.zeros((1,) + v.shape[1:]), np.cumsum(v, axis=0)])
            for i in range(t):
                pos = c + i
                lo = max(0, pos - w + 1)
                mean = (csum[pos + 1] - csum[lo]) / (pos + 1 - lo)
                want = np.repeat(mean, sc.H // sc.Hkv, axis=0)
                assert np.allclose(got[row + i], want, rtol=1e-12, atol=1e-13), (w, r, i)
            row += t


def check_window_covering_context(orc):
    """A window at least as long as the context changes nothing, bit for bit."""
    sc = Scenario([(30, 4), (0, 9), (64, 1)], 8, 2, 8, 4, seed=28)
    ref = sc.run_oracle(orc, want_f64=False)
    for w in (65, 66, 1000):
        assert np.array_equal(sc.run_oracle(orc, want_f64=False, window=w), ref), w


# ------------------------------------------------------------------------------------------
# block copies (swap out / swap in, copy-on-write), pinned through the attention they serve
# ------------------------------------------------------------------------------------------

def check_swap_roundtrip_preserves_attention(orc):
    """Swap a request's blocks out to a staging buffer, poison them, swap the copy into other
    free blocks and point the table there: the attention output must not move, bit for bit
    (a wrong block, a partial block or a reversed copy changes it or turns it NaN)."""
    sc = Scenario([(30, 4), (0, 9), (50, 2)], 8, 2, 8, 4, seed=31, num_blocks=60)
    ref = sc.run_oracle(orc, want_f64=False)
    used = {b for tb in sc.tables for b in tb}
    free = [b for b in range(sc.num_blocks) if b not in used]
    for r in (0, 2):
        blocks = np.array(sc.tables[r], np.int64)
        n = len(blocks)
        for pool in (sc.k_pool, sc.v_pool):
            staging = np.zeros((n,) + pool.shape[1:], pool.dtype)
            orc.copy_blocks(pool, staging, blocks, np.arange(n))
            pool[blocks] = np.nan
            new = np.array(free[:n], np.int64)
            orc.copy_blocks(staging, pool, np.arange(n), new)
        sc.tables[r] = [int(b) for b in free[:n]]
        free = free[n:]
    assert np.array_equal(sc.run_oracle(orc, want_f64=False), ref)


def check_copy_on_write(orc):
    """Two requests alias a prefix block; copy-on-write gives request 1 a private copy and
    the next write goes there: request 0 still sees the old contents, request 1 the new."""
    bs = 4
    sc = Scenario([(10, 1), (7, 1)], 4, 2, 8, bs, seed=32, num_blocks=12)
    sc.ctx_k[1][:4] = sc.ctx_k[0][:4]
    sc.ctx_v[1][:4] = sc.ctx_v[0][:4]
    sc.build_pool()
    shared = sc.tables[0][0]
    sc.tables[1][0] = shared
    before = sc.run_oracle(orc, want_f64=False)
    used = {b for tb in sc.tables for b in tb}
    private = next(b for b in range(sc.num_blocks) if b not in used)
    for pool in (sc.k_pool, sc.v_pool):
        orc.copy_blocks(pool, pool, np.array([shared]), np.array([private]))
    sc.tables[1][0] = private
    assert np.array_equal(sc.run_oracle(orc, want_f64=False), before)      # the copy is exact
    # request 1 overwrites position 2 of its private block
    rng = np.random.default_rng(33)
    kn = rng.standard_normal((1, sc.Hkv, sc.D)).astype(np.float32)
    vn = rng.standard_normal((1, sc.Hkv, sc.D)).astype(np.float32)
    orc.kv_write(kn, vn, np.array([private * bs + 2], np.int64), sc.k_pool, sc.v_pool, "f32", "f32")
    after = sc.run_oracle(orc, want_f64=False)
    assert np.array_equal(after[0], before[0])                              # the sharer is untouched
    sc.ctx_k[1][2] = kn[0]
    sc.ctx_v[1][2] = vn[0]
    assert _rel_err(after[1:2], sc.dense(1)) < 1e-6 and not np.array_equal(after[1], before[1])


# ------------------------------------------------------------------------------------------
# fp8 E4M3 pools with per-(slot, KV head) scales (ReferenceBackend.dequantize)
# ------------------------------------------------------------------------------------------

def _torch_fp8_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def check_fp8_codec_vs_torch(orc):
    """Every code decodes as torch's float8_e4m3fn does; float32 values round to the code
    torch picks (nearest, ties to even) up to the overflow midpoint 464, and saturate past it."""
    codes = np.arange(256)
    want = _torch_fp8_decode(codes)
    got = np.array([orc.fp8_e4m3_decode(c) for c in codes])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)])
    rng = np.random.default_rng(41)
    finite = want[~np.isnan(want)]
    grid = np.unique(np.abs(finite))
    mids = (grid[:-1] + grid[1:]) / 2                                    # exact ties
    vals = np.concatenate([rng.standard_normal(3000) * 30, rng.standard_normal(1000) * 2e-3, mids, -mids,
                           np.nextafter(mids.astype(np.float32), np.float32(0)), grid, [463.99, -463.99, 0.0, -0.0]])
    vals = vals.astype(np.float32)
    vals = vals[np.abs(vals) < 464]
    want_codes = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got_codes = np.array([orc.fp8_e4m3_encode(float(x)) for x in vals], np.uint8)
    assert np.array_equal(got_codes, want_codes), vals[got_codes != want_codes][:5]
    for big in (464.0, 1e6, 3e38):
        assert orc.fp8_e4m3_encode(big) == 0x7E and orc.fp8_e4m3_encode(-big) == 0xFE


def _fp8_case(orc, seed, n=23, hkv=3, d=40, nb=9, bs=4):
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((n, hkv, d)) * rng.choice([1e-3, 1.0, 50.0], size=(n, hkv, 1))).astype(np.float32)
    v = (rng.standard_normal((n, hkv, d)) * 3).astype(np.float32)
    k[4, 1] = 0.0                                                        # an all-zero row: scale 1
    kc = np.zeros((nb + 1, bs, hkv, d), np.uint8)
    vc = kc.copy()
    ks = np.zeros((nb + 1, bs, hkv), np.float32)
    vs = ks.copy()
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    orc.kv_write_fp8(k, v, slots, kc, vc, ks, vs, "f32")
    return k, v, slots, kc, vc, ks, vs


def check_fp8_write_quantizes_each_row(orc):
    """Each row's largest magnitude maps to code +-448 with scale max|x| / 448, and every
    element dequantizes to within half an fp8 step (at its magnitude) of its value."""
    k, v, slots, kc, vc, ks, vs = _fp8_case(orc, 42)
    hkv, d = k.shape[1], k.shape[2]
    for x, cache, sc in ((k, kc, ks), (v, vc, vs)):
        codes = cache.reshape(-1, hkv, d)[slots]
        scale = sc.reshape(-1, hkv)[slots].astype(np.float64)
        deq = _torch_fp8_decode(codes) * scale[..., None]
        amax = np.abs(x).max(axis=2)
        nz = amax > 0
        assert np.allclose(scale[nz], (amax[nz].astype(np.float32) / np.float32(448)).astype(np.float64), rtol=0)
        assert np.all(scale[~nz] == 1.0) and np.all(codes[~nz] == 0)
        assert np.all(np.abs(_torch_fp8_decode(codes)).max(axis=2)[nz] == 448.0)
        y = np.abs(x / np.where(nz, scale, 1.0)[..., None])
        step = np.where(y < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3))
        assert np.all(np.abs(deq - x) <= 0.5 * step * scale[..., None] * (1 + 1e-6) + 1e-30)


def check_fp8_attention_dequantizes(orc):
    """Attention over fp8 pools equals dense attention over the dequantized rows (codes
    decoded by torch, times their own (slot, KV head) scale)."""
    sc = Scenario([(20, 3), (0, 6), (37, 1)], 6, 3, 40, 4, seed=43)
    qsl, lens, table = sc.meta()
    q = np.concatenate(sc.q, axis=0)
    n_slots = (sc.num_blocks + 1) * sc.bs
    kc = np.zeros((sc.num_blocks + 1, sc.bs, sc.Hkv, sc.D), np.uint8)
    vc = kc.copy()
    ks = np.zeros((sc.num_blocks + 1, sc.bs, sc.Hkv), np.float32)
    vs = ks.copy()
    for r, (c, t) in enumerate(sc.specs):
        slots = np.array([workloads.slot_of(sc.tables[r], p, sc.bs) for p in range(c + t)], np.int64)
        orc.kv_write_fp8(np.ascontiguousarray(sc.ctx_k[r]), np.ascontiguousarray(sc.ctx_v[r]), slots, kc, vc, ks, vs,
                         "f32")
    _, got = orc.paged_attention(q, kc, vc, qsl, lens, table, 1.0 / math.sqrt(sc.D), "f32", want_f64=True,
                                 k_scale=ks, v_scale=vs)
    row = 0
    for r, (c, t) in enumerate(sc.specs):
        slots = np.array([workloads.slot_of(sc.tables[r], p, sc.bs) for p in range(c + t)], np.int64)
        dk = _torch_fp8_decode(kc.reshape(n_slots, sc.Hkv, sc.D)[slots]) * ks.reshape(n_slots, sc.Hkv)[slots][..., None]
        dv = _torch_fp8_decode(vc.reshape(n_slots, sc.Hkv, sc.D)[slots]) * vs.reshape(n_slots, sc.Hkv)[slots][..., None]
        want = dense_fold_attention(as_f64(sc.q[r], "f32"), dk, dv, 1.0 / math.sqrt(sc.D), c)
        assert _rel_err(got[row:row + t], want) < 1e-12, r
        row += t


def check_padding_rows_zero(orc):
    """Padding rows (seq_len 0, one query row, slot -1) produce zeros, not 0/0."""
    b = workloads.small_batch([(5, 2), (0, 3)], pad_to=5, seed=9)
    assert b.seq_lens_host[-3:] == [0, 0, 0]
    out, f64 = orc.paged_attention(to_np(b.q), to_np(b.k_cache), to_np(b.v_cache),
                                   b.query_start_loc.numpy(), b.seq_lens.numpy(), b.block_table.numpy(),
                                   b.scale, "f32", want_f64=True)
    assert np.all(out[5:] == 0) and np.all(f64[5:] == 0)


# ------------------------------------------------------------------------------------------
# invariants the pages' test suites assert: outputs must not move, bit for bit
# ------------------------------------------------------------------------------------------

def _prompt(seed, L, H, Hkv, D, dtype="f32"):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((L, H, D)).astype(np.float32)
    return q, k, v


def _run_chunked(orc, q, k, v, chunk, bs, nb, seed):
    """Prefill one prompt in steps of `chunk` tokens: each step writes the chunk's K/V into
    the pool at its slots, then attends the chunk's queries over the pool."""
    L, H, D = q.shape
    Hkv = k.shape[1]
    rng = np.random.default_rng(seed)
    table = [int(x) for x in rng.permutation(nb)[: -(-L // bs)]]
    kp = np.full(((nb + 1) * bs, Hkv, D), np.nan, np.float32)
    vp = kp.copy()
    outs = []
    for a in range(0, L, chunk):
        b = min(L, a + chunk)
        slots = np.array([workloads.slot_of(table, p, bs) for p in range(a, b)], np.int64)
        orc.kv_write(np.ascontiguousarray(k[a:b]), np.ascontiguousarray(v[a:b]), slots,
                     kp.reshape(nb + 1, bs, Hkv, D), vp.reshape(nb + 1, bs, Hkv, D), "f32", "f32")
        tb = np.zeros((1, max(1, -(-b // bs))), np.int32)
        tb[0, :] = table[: tb.shape[1]]
        outs.append(orc.paged_attention(np.ascontiguousarray(q[a:b]), kp.reshape(nb + 1, bs, Hkv, D),
                                        vp.reshape(nb + 1, bs, Hkv, D), np.array([0, b - a], np.int32),
                                        np.array([b], np.int32), tb, 1.0 / math.sqrt(D), "f32"))
    return np.concatenate(outs, axis=0)


def check_chunking_invariance(orc, long_prompt=True):
    cases = [(300, 4, 2, 16, 16)]
    if long_prompt:
        cases.append((5000, 2, 1, 8, 16))
    for L, H, Hkv, D, bs in cases:
        q, k, v = _prompt(L, L, H, Hkv, D)
        nb = -(-L // bs) + 5
        ref = _run_chunked(orc, q, k, v, L, bs, nb, seed=1)
        for chunk in (8, 33, 64, 4096):
            got = _run_chunked(orc, q, k, v, chunk, bs, nb, seed=1)
            assert np.array_equal(got, ref), (L, chunk)


def check_block_relabelling(orc):
    sc = Scenario([(30, 4), (0, 9), (64, 1), (17, 17)], 8, 2, 8, 4, seed=11)
    ref = sc.run_oracle(orc, want_f64=False)
    rng = np.random.default_rng(12)
    pi = rng.permutation(sc.num_blocks)
    kp, vp = sc.k_pool.copy(), sc.v_pool.copy()
    sc.k_pool[pi] = kp[:sc.num_blocks]          # block b moves to pi[b]; the scratch block stays
    sc.v_pool[pi] = vp[:sc.num_blocks]
    sc.tables = [[int(pi[b]) for b in tb] for tb in sc.tables]
    got = sc.run_oracle(orc, want_f64=False)
    assert np.array_equal(got, ref)


def check_aliasing(orc):
    """Two requests sharing a 2-block prefix through aliased blocks give the same output as
    with private copies of the prefix."""
    bs = 4
    sc = Scenario([(13, 2), (9, 3)], 4, 2, 8, bs, seed=13, num_blocks=20)
    # make request 1's first 8 positions equal to request 0's, then alias its first 2 blocks
    sc.ctx_k[1][:8] = sc.ctx_k[0][:8]
    sc.ctx_v[1][:8] = sc.ctx_v[0][:8]
    sc.build_pool()
    private = sc.run_oracle(orc, want_f64=False)
    freed = sc.tables[1][:2]
    sc.tables[1][:2] = sc.tables[0][:2]
    for b in freed:                       # poison the now-unused private copies
        sc.k_pool[b] = np.nan
        sc.v_pool[b] = np.nan
    shared = sc.run_oracle(orc, want_f64=False)
    assert np.array_equal(shared, private)


def check_batch_composition(orc):
    specs = [(40, 3), (0, 12), (7, 1), (90, 1), (15, 15), (3, 2), (60, 6), (1, 1)]
    sc = Scenario(specs, 8, 4, 8, 16, seed=14)
    batched = sc.run_oracle(orc, want_f64=False)
    alone = Scenario(specs, 8, 4, 8, 16, seed=14)
    alone.specs, alone.q = [specs[0]], [alone.q[0]]
    alone.ctx_k, alone.ctx_v, alone.tables = [alone.ctx_k[0]], [alone.ctx_v[0]], [alone.tables[0]]
    got = alone.run_oracle(orc, want_f64=False)
    assert np.array_equal(got, batched[:3])


def check_block_size_invariance(orc):
    specs = [(70, 5), (0, 20), (129, 1)]
    ref = None
    for bs in (1, 4, 16, 64):
        sc = Scenario(specs, 4, 2, 8, bs, seed=15)
        got = sc.run_oracle(orc, want_f64=False)
        if ref is None:
            ref = got
        assert np.array_equal(got, ref), bs


def check_rejects_bad_metadata(orc):
    sc = Scenario([(4, 2)], 4, 2, 8, 4, seed=16)
    qsl, lens, table = sc.meta()
    q = np.ascontiguousarray(sc.q[0])
    bad = [
        (np.array([0, 3], np.int32), lens, table),            # qsl[R] != N
        (qsl, np.array([1], np.int32), table),                # t > seq_len
        (qsl, np.array([40], np.int32), table),               # table too narrow for seq_len
    ]
    for a, b, c in bad:
        try:
            orc.paged_attention(q, sc.k_pool, sc.v_pool, a, b, c, 0.5, "f32")
        except ValueError:
            continue
        raise AssertionError("inconsistent metadata accepted")


ALL_CHECKS = [
    check_gather_follows_page_example, check_kv_write_index_copy, check_kv_write_scratch_gets_a_padding_row,
    check_bf16_rounding, check_dense_fold, check_dense_sdpa_bf16, check_position_zero_is_v0,
    check_zero_query_gives_prefix_mean, check_constant_values, check_dominant_key, check_large_scores,
    check_padding_rows_zero, check_block_relabelling, check_aliasing, check_batch_composition,
    check_block_size_invariance, check_rejects_bad_metadata, check_window_dense, check_window_sdpa_bf16,
    check_window_one_is_own_v, check_window_zero_query_gives_window_mean, check_window_covering_context,
    check_swap_roundtrip_preserves_attention, check_copy_on_write, check_fp8_codec_vs_torch,
    check_fp8_write_quantizes_each_row, check_fp8_attention_dequantizes,
]
