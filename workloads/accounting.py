"""Algorithmic work of one step: the bytes the method must move and the flops it must do.

No attention arithmetic here, only counting.  Conventions:
  * KV bytes count every live (slot, KV head) row a step reads once, K and V, whatever the
    number of query heads that share it (grouped-query attention reads a KV head once per
    group) and however many requests alias the block; plus q, out and the metadata.
  * flops count QK^T and PV over unmasked scores only: 4 * D per (query row, head, key)
    with key position <= the row's position (and, with a sliding window of w tokens, >
    the row's position - w); softmax work is not counted.
  * With a window, the live rows are those some query row of the request can see.
  * Per-token KV size follows the page's M_token = 2 * L * H_KV * d_head * B.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional

ELEM_BYTES = {"f32": 4, "bf16": 2}


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V bytes one token occupies across all layers."""
    return 2 * layers * kv_heads * head_dim * elem_bytes


def _first_visible(req, window: int) -> int:
    """First key position any query row of the request sees (its first row's window start)."""
    if window <= 0 or req.new == 0:
        return 0
    return max(0, req.computed - window + 1)


def _live_slots(batch, req_ids: Iterable[int], window: int = 0) -> int:
    bs = batch.block_size
    slots = set()
    for r in req_ids:
        req = batch.requests[r]
        for p in range(_first_visible(req, window), req.seq_len):
            slots.add(req.blocks[p // bs] * bs + p % bs)
    return len(slots)


def attention_work(batch, req_ids: Optional[Iterable[int]] = None, window: int = 0,
                   kv_fp8: bool = False) -> Dict[str, float]:
    """Algorithmic bytes and flops of paged attention over the given requests (default: all),
    with a sliding window of `window` tokens (0: none).  kv_fp8: the pools hold one-byte E4M3
    codes plus a float32 scale per (slot, KV head) and tensor; q and out keep the batch dtype."""
    ids = list(range(len(batch.requests))) if req_ids is None else list(req_ids)
    e = ELEM_BYTES[batch.dtype]
    H, Hkv, D = batch.num_heads, batch.num_kv_heads, batch.head_dim
    rows = sum(batch.requests[r].new for r in ids)
    slot_bytes = Hkv * (D + 4) if kv_fp8 else Hkv * D * e
    kv = _live_slots(batch, ids, window) * slot_bytes * 2
    qo = rows * H * D * e * 2
    meta = sum(4 * (len(batch.requests[r].blocks) + 2) for r in ids)
    scores = 0
    for r in ids:
        req = batch.requests[r]
        c, t = req.computed, req.new
        if window <= 0:
            scores += t * c + t * (t + 1) // 2        # sum over rows i of (c + i + 1)
        else:
            scores += sum(min(c + i + 1, window) for i in range(t))
    flops = 4.0 * H * D * scores
    return {"kv_bytes": float(kv), "qo_bytes": float(qo), "meta_bytes": float(meta),
            "bytes": float(kv + qo + meta), "flops": flops, "rows": rows, "scores_per_head": scores}


def write_work(batch, kv_fp8: bool = False) -> Dict[str, float]:
    """Bytes the KV write must move: read k and v, write them into the pool, read the slots.
    kv_fp8: the pool row is one code byte per element plus a float32 scale per KV head."""
    e = ELEM_BYTES[batch.dtype]
    n = batch.num_tokens
    row = batch.num_kv_heads * batch.head_dim * e
    stored = batch.num_kv_heads * (batch.head_dim + 4) if kv_fp8 else row
    return {"bytes": float(2 * n * (row + stored) + 8 * n)}
