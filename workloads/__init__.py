"""Seeded synthetic batches for the paged KV write and paged varlen attention.

This module serves both the oracle and the HIP path and holds none of the attention
arithmetic: it only draws random values and lays out the batch metadata that an engine's
batch builder hands to the attention backend ("Engine v2: one core for every request",
section "Flattened ragged batches": BatchMeta and build_batch).

A batch is a list of requests.  Request r has c_r tokens already in the pool
(num_computed_tokens) and t_r new tokens this step, so seq_len_r = c_r + t_r and its new
tokens sit at positions c_r .. c_r + t_r - 1.  Position p of request r lives at flat slot
table_r[p // block_size] * block_size + p % block_size.

Draw order, all from one CPU torch.Generator seeded with the config's seed:
  1. lengths (config-specific),
  2. a permutation of the pool's physical block ids (tables take consecutive ids from it;
     shared-prefix blocks come first and are reused by every sharer),
  3. pool contents: K then V, N(0, 1) float32, one draw covering every slot that holds a
     context position (< c_r) and is not written by this step, in increasing slot order,
  4. the new q [N, H, D], then k, v [N, Hkv, D], N(0, 1) float32.
Each drawn tensor is followed, when the config has outliers, by a U(0, 1) draw of the same
shape; elements whose draw is below the outlier probability are multiplied by 10.
bfloat16 data is the float32 draw rounded to nearest-even.  Every slot not drawn in step 3
(dead slots, the tails of last blocks, the scratch block, slots this step writes) holds NaN
when ``poison`` is set (correctness runs) and 0 otherwise (timing runs).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class Request:
    computed: int                  # c: tokens whose K/V are already in the pool
    new: int                       # t: tokens computed this step
    blocks: List[int] = field(default_factory=list)   # physical block ids in logical order

    @property
    def seq_len(self) -> int:
        return self.computed + self.new


@dataclass
class Batch:
    name: str
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int                # blocks handed out; the pool has num_blocks + 1 (scratch last)
    requests: List[Request]
    scale: float
    # tensors (CPU)
    q: torch.Tensor                # [N, H, D]
    k: torch.Tensor                # [N, Hkv, D]
    v: torch.Tensor                # [N, Hkv, D]
    k_cache: torch.Tensor          # [NB+1, bs, Hkv, D], contents before this step's write
    v_cache: torch.Tensor
    query_start_loc: torch.Tensor  # [R+1] int32
    seq_lens: torch.Tensor         # [R] int32
    block_table: torch.Tensor      # [R, W] int32, zero-padded
    slot_mapping: torch.Tensor     # [N] int64, -1 for padding rows
    positions: torch.Tensor        # [N] int64
    query_start_loc_host: List[int]
    seq_lens_host: List[int]
    max_query_len: int
    max_seq_len: int
    description: str = ""

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc_host[-1])

    @property
    def num_reqs(self) -> int:
        return len(self.seq_lens_host)

    @property
    def num_slots(self) -> int:
        return (self.num_blocks + 1) * self.block_size


def slot_of(table: Sequence[int], position: int, block_size: int) -> int:
    """Flat pool slot of a token position: the page's slot formula."""
    return int(table[position // block_size]) * block_size + position % block_size


def batch_metadata(requests: Sequence[Request], block_size: int, pad_to: Optional[int] = None):
    """The BatchMeta arrays of a flattened batch ("Flattened ragged batches"): per-row
    positions and pool slots, query_start_loc, seq_lens and a zero-padded block table.
    pad_to > len(requests) appends padding requests of one row each, with seq_len 0, no
    blocks and slot -1 (the scratch slot).

    Built from per-request arrays: query_start_loc is the running sum of the row counts, each
    row finds its request by a search over it, and its position and slot follow from the
    request's first computed position and its table row."""
    real = len(requests)
    n_pad = max(0, (pad_to or 0) - real)
    computed = np.array([r.computed for r in requests] + [0] * n_pad, dtype=np.int64)
    rows = np.array([r.new for r in requests] + [1] * n_pad, dtype=np.int64)
    ctx = computed + rows
    ctx[real:] = 0                                        # padding: nothing to attend to
    counts = np.array([len(r.blocks) for r in requests] + [0] * n_pad, dtype=np.int64)
    short = np.nonzero(counts[:real] * block_size < ctx[:real])[0]
    if len(short):
        raise ValueError(f"request {int(short[0])} has too few blocks for its sequence")
    qsl = np.zeros(real + n_pad + 1, dtype=np.int64)
    np.cumsum(rows, out=qsl[1:])
    # block table: every request's ids laid out along its row, zeros after them
    table = np.zeros((real + n_pad, max(1, int(counts.max(initial=0)))), dtype=np.int32)
    if counts.sum():
        ids = np.concatenate([np.asarray(r.blocks, dtype=np.int64) for r in requests])
        owner = np.repeat(np.arange(real + n_pad), counts)
        col = np.arange(len(ids)) - np.repeat(np.cumsum(counts) - counts, counts)
        table[owner, col] = ids
    # rows: owning request, position, slot (padding rows: position 0, slot -1)
    n = int(qsl[-1])
    owner = np.searchsorted(qsl, np.arange(n), side="right") - 1
    pos = computed[owner] + (np.arange(n) - qsl[owner])
    pad_row = owner >= real
    pos[pad_row] = 0
    slot = table[owner, pos // block_size].astype(np.int64) * block_size + pos % block_size
    slot[pad_row] = -1
    qsl_list = [int(x) for x in qsl]
    lens_list = [int(x) for x in ctx]
    return dict(
        positions=torch.from_numpy(pos.astype(np.int64)),
        slot_mapping=torch.from_numpy(slot.astype(np.int64)),
        query_start_loc=torch.tensor(qsl_list, dtype=torch.int32),
        seq_lens=torch.tensor(lens_list, dtype=torch.int32),
        block_table=torch.from_numpy(table),
        query_start_loc_host=qsl_list,
        seq_lens_host=lens_list,
        max_query_len=int(rows.max(initial=0)),
        max_seq_len=int(ctx.max(initial=0)),
    )


def _draw(gen: torch.Generator, shape, outlier_p: float) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if outlier_p > 0:
        u = torch.rand(shape, generator=gen, dtype=torch.float32)
        x = torch.where(u < outlier_p, x * 10.0, x)
    return x


def assign_blocks(gen: torch.Generator, requests: Sequence[Request], num_blocks: int,
                  block_size: int, shared_prefix_blocks: int = 0) -> None:
    """Give each request the physical blocks it needs, drawn from one random permutation of
    the pool's ids.  The first `shared_prefix_blocks` ids head every request's table."""
    perm = torch.randperm(num_blocks, generator=gen).tolist()
    shared = perm[:shared_prefix_blocks]
    nxt = shared_prefix_blocks
    for req in requests:
        need = -(-req.seq_len // block_size)
        own = need - len(shared)
        if own < 0:
            raise ValueError("request shorter than the shared prefix")
        req.blocks = list(shared) + perm[nxt:nxt + own]
        nxt += own
        if nxt > num_blocks:
            raise ValueError("pool too small for the batch")


def make_batch(name: str, requests: List[Request], *, dtype: str, num_heads: int, num_kv_heads: int,
               head_dim: int, block_size: int, num_blocks: int, gen: torch.Generator,
               poison: bool = True, outlier_p: float = 0.0, pad_to: Optional[int] = None,
               scale: Optional[float] = None, description: str = "", values: bool = True) -> Batch:
    """Draw the pool contents and the new q, k, v for requests whose blocks are assigned.
    values=False lays out the metadata only: the data tensors are then empty (for checks of
    the batch's shape and indexing that need no values)."""
    meta = batch_metadata(requests, block_size, pad_to)
    hkv, d, bs = num_kv_heads, head_dim, block_size
    n = len(meta["positions"])
    if not values:
        e = torch.empty(0)
        return Batch(name=name, dtype=dtype, num_heads=num_heads, num_kv_heads=hkv, head_dim=d,
                     block_size=bs, num_blocks=num_blocks, requests=list(requests),
                     scale=(1.0 / math.sqrt(d)) if scale is None else scale,
                     q=e, k=e, v=e, k_cache=e, v_cache=e, description=description, **meta)
    written = set(s for s in meta["slot_mapping"].tolist() if s >= 0)
    context = set()
    for req in requests:
        for p in range(req.computed):
            context.add(slot_of(req.blocks, p, bs))
    prefilled = torch.tensor(sorted(context - written), dtype=torch.int64)
    fill = float("nan") if poison else 0.0
    tdt = TORCH_DTYPES[dtype]
    caches = []
    for _ in range(2):
        pool = torch.full(((num_blocks + 1) * bs, hkv, d), fill, dtype=tdt)
        if len(prefilled):
            pool[prefilled] = _draw(gen, (len(prefilled), hkv, d), outlier_p).to(tdt)
        caches.append(pool.view(num_blocks + 1, bs, hkv, d))
    q = _draw(gen, (n, num_heads, d), outlier_p).to(tdt)
    k = _draw(gen, (n, hkv, d), outlier_p).to(tdt)
    v = _draw(gen, (n, hkv, d), outlier_p).to(tdt)
    return Batch(name=name, dtype=dtype, num_heads=num_heads, num_kv_heads=hkv, head_dim=d,
                 block_size=bs, num_blocks=num_blocks, requests=list(requests),
                 scale=(1.0 / math.sqrt(d)) if scale is None else scale,
                 q=q, k=k, v=v, k_cache=caches[0], v_cache=caches[1], description=description, **meta)


# ----------------------------------------------------------------------------------------
# The five workload shapes.  Sizes follow the configurations the benchmarks quote; the
# length distributions stand in for the pages' lognormal request mix and shared prompts.
# ----------------------------------------------------------------------------------------

def worked_batch(poison: bool = True, seed: int = 1, values: bool = True) -> Batch:
    """The 9-token batch of "Flattened ragged batches": a chunk of 3 at positions 6-8,
    decodes at 41 and 9, and a new request of 4 tokens.  fp32, 8/4 heads, D=48, bs=16,
    a 64-block pool whose tables are the first ids of a random permutation."""
    gen = torch.Generator().manual_seed(seed)
    reqs = [Request(6, 3), Request(41, 1), Request(9, 1), Request(0, 4)]
    assign_blocks(gen, reqs, 64, 16)
    return make_batch("worked_batch", reqs, dtype="f32", num_heads=8, num_kv_heads=4, head_dim=48,
                      block_size=16, num_blocks=64, gen=gen, poison=poison, values=values,
                      description="9 tokens / 4 requests, fp32, H=8 Hkv=4 D=48 bs=16, 64-block pool")


def mixed_step(dtype: str = "f32", poison: bool = True, seed: int = 2, values: bool = True) -> Batch:
    """48 requests: seq_len ~ lognormal(4.463, 0.701) clipped to [17, 443]; the first 8 are
    prefill chunks of min(64, seq_len) tokens, the other 40 decode one token.  A budget of
    512 tokens is applied decodes first, then chunks in order, each capped by what is left."""
    gen = torch.Generator().manual_seed(seed)
    z = torch.randn(48, generator=gen, dtype=torch.float64)
    lens = torch.exp(4.463 + 0.701 * z).round().clamp(17, 443).to(torch.int64).tolist()
    budget = 512 - 40
    prefill, decode = [], []
    for i, L in enumerate(lens):
        if i < 8:
            t = min(64, L)
            c = L - t
            t = min(t, budget)
            budget -= t
            if t > 0:
                prefill.append(Request(c, t))
        else:
            decode.append(Request(L - 1, 1))
    reqs = decode + prefill
    need = sum(-(-r.seq_len // 16) for r in reqs)
    nb = math.ceil(1.2 * need)
    assign_blocks(gen, reqs, nb, 16)
    return make_batch(f"mixed_step_{dtype}", reqs, dtype=dtype, num_heads=8, num_kv_heads=4, head_dim=48,
                      block_size=16, num_blocks=nb, gen=gen, poison=poison, values=values,
                      description="48 requests (40 decodes + 8 chunks <= 64), budget 512, H=8 Hkv=4 D=48")


def decode_only(poison: bool = True, seed: int = 3, num_reqs: int = 256, min_len: int = 512,
                max_len: int = 8192, values: bool = True) -> Batch:
    """256 single-token decodes, seq_len ~ U{512..8192}, bf16, 32/8 heads, D=128, bs=16,
    pool 1.2x the blocks needed, tables scattered by a random permutation."""
    gen = torch.Generator().manual_seed(seed)
    lens = torch.randint(min_len, max_len + 1, (num_reqs,), generator=gen).tolist()
    reqs = [Request(L - 1, 1) for L in lens]
    need = sum(-(-L // 16) for L in lens)
    nb = math.ceil(1.2 * need)
    assign_blocks(gen, reqs, nb, 16)
    return make_batch("decode_only", reqs, dtype="bf16", num_heads=32, num_kv_heads=8, head_dim=128,
                      block_size=16, num_blocks=nb, gen=gen, poison=poison, values=values,
                      description=f"{num_reqs} decodes, seq_len U{{{min_len}..{max_len}}}, bf16 H=32 Hkv=8 D=128")


def shared_prefix(poison: bool = True, seed: int = 4, values: bool = True) -> Batch:
    """64 requests whose tables start with the same 16 blocks (a 256-token shared prefix):
    60 decodes with seq_len ~ U{300..4000} and 4 prefill chunks of 2048 tokens at
    num_computed_tokens (0, 2048, 4096, 2048).  Budget 8192, decodes first, then the chunks
    in order (the last is cut to 1988).  The chunk at position 0 writes the prefix blocks in
    this very step; every request reads them afterwards.  bf16, 32/8 heads, D=128."""
    gen = torch.Generator().manual_seed(seed)
    lens = torch.randint(300, 4001, (60,), generator=gen).tolist()
    reqs = [Request(L - 1, 1) for L in lens]
    budget = 8192 - 60
    for c in (0, 2048, 4096, 2048):
        t = min(2048, budget)
        budget -= t
        reqs.append(Request(c, t))
    need = 16 + sum(-(-r.seq_len // 16) - 16 for r in reqs)
    nb = math.ceil(1.2 * need)
    assign_blocks(gen, reqs, nb, 16, shared_prefix_blocks=16)
    return make_batch("shared_prefix", reqs, dtype="bf16", num_heads=32, num_kv_heads=8, head_dim=128,
                      block_size=16, num_blocks=nb, gen=gen, poison=poison, values=values,
                      description="60 decodes + 4 chunks (2048,2048,2048,1988), 256-token shared prefix")


def long_context(poison: bool = True, seed: int = 5, values: bool = True) -> Batch:
    """16 decodes at seq_len 32768 plus one prefill chunk of 4096 tokens at position 28672,
    bf16, 64/8 heads, D=128, a 40000-block pool, every value N(0,1) with 1% scaled by 10."""
    gen = torch.Generator().manual_seed(seed)
    reqs = [Request(32767, 1) for _ in range(16)] + [Request(28672, 4096)]
    assign_blocks(gen, reqs, 40000, 16)
    return make_batch("long_context", reqs, dtype="bf16", num_heads=64, num_kv_heads=8, head_dim=128,
                      block_size=16, num_blocks=40000, gen=gen, poison=poison, values=values, outlier_p=0.01,
                      description="16 decodes at 32768 + 1 chunk of 4096 at 28672, H=64 Hkv=8 D=128")


def spec_verify(poison: bool = True, seed: int = 6, num_reqs: int = 128, min_len: int = 512,
                max_len: int = 8192, values: bool = True) -> Batch:
    """Speculative verification: every request scores 1 + k new rows (its last accepted
    token and k draft tokens), k cycling over 1, 2, 4, 8, at seq_len ~ U{512..8192} that
    includes those rows; bf16, 32/8 heads, D=128, bs=16, pool 1.2x the blocks needed.
    The verifier's rows are the last t positions of the context like any chunk's."""
    gen = torch.Generator().manual_seed(seed)
    lens = torch.randint(min_len, max_len + 1, (num_reqs,), generator=gen).tolist()
    ks = [(1, 2, 4, 8)[i % 4] for i in range(num_reqs)]
    reqs = [Request(L - (1 + k), 1 + k) for L, k in zip(lens, ks)]
    need = sum(-(-L // 16) for L in lens)
    nb = math.ceil(1.2 * need)
    assign_blocks(gen, reqs, nb, 16)
    return make_batch("spec_verify", reqs, dtype="bf16", num_heads=32, num_kv_heads=8, head_dim=128,
                      block_size=16, num_blocks=nb, gen=gen, poison=poison, values=values,
                      description=f"{num_reqs} verifications of 1+k rows, k in (1,2,4,8), seq_len "
                                  f"U{{{min_len}..{max_len}}}, bf16 H=32 Hkv=8 D=128")


def small_decode(poison: bool = True, seed: int = 7, values: bool = True) -> Batch:
    """A decode batch of 13 requests padded to 16 rows (pad_to of "Flattened ragged
    batches": three rows with slot -1 and seq_len 0, the shape a captured graph serves),
    seq_len ~ U{256..2048}, bf16, 32/8 heads, D=128, bs=16, pool 1.2x the blocks needed."""
    gen = torch.Generator().manual_seed(seed)
    lens = torch.randint(256, 2049, (13,), generator=gen).tolist()
    reqs = [Request(L - 1, 1) for L in lens]
    need = sum(-(-L // 16) for L in lens)
    nb = math.ceil(1.2 * need)
    assign_blocks(gen, reqs, nb, 16)
    return make_batch("small_decode", reqs, dtype="bf16", num_heads=32, num_kv_heads=8, head_dim=128,
                      block_size=16, num_blocks=nb, gen=gen, poison=poison, values=values, pad_to=16,
                      description="13 decodes padded to 16 rows, seq_len U{256..2048}, bf16 H=32 Hkv=8 D=128")


CONFIGS = {
    "worked_batch": worked_batch,
    "mixed_step_f32": lambda poison=True, values=True: mixed_step("f32", poison, values=values),
    "mixed_step_bf16": lambda poison=True, values=True: mixed_step("bf16", poison, values=values),
    "decode_only": decode_only,
    "shared_prefix": shared_prefix,
    "long_context": long_context,
    "spec_verify": spec_verify,
    "small_decode": small_decode,
}


def small_batch(specs: Sequence[Tuple[int, int]], *, dtype: str = "f32", num_heads: int = 4,
                num_kv_heads: int = 2, head_dim: int = 16, block_size: int = 16,
                num_blocks: Optional[int] = None, seed: int = 0, poison: bool = True,
                shared_prefix_blocks: int = 0, outlier_p: float = 0.0,
                pad_to: Optional[int] = None, values: bool = True) -> Batch:
    """A batch of requests given as (computed, new) pairs, for tests."""
    gen = torch.Generator().manual_seed(seed)
    reqs = [Request(c, t) for c, t in specs]
    need = shared_prefix_blocks + sum(-(-r.seq_len // block_size) - shared_prefix_blocks for r in reqs)
    nb = num_blocks if num_blocks is not None else max(1, math.ceil(1.5 * need) + 2)
    assign_blocks(gen, reqs, nb, block_size, shared_prefix_blocks)
    return make_batch("small", reqs, dtype=dtype, num_heads=num_heads, num_kv_heads=num_kv_heads,
                      head_dim=head_dim, block_size=block_size, num_blocks=nb, gen=gen, poison=poison, values=values,
                      outlier_p=outlier_p, pad_to=pad_to)
