"""Runs a batch through the HIP library and through the CPU oracle, for the parity tests."""
from __future__ import annotations

import json
import os
import sys
from typing import Optional

import numpy as np
import torch

import oracle
import paged_kv_attention_05_amd as pk
from tests._util import attention_error, rounding_excess, to_np


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def record(entry: dict) -> None:
    """Append one result line to $PA_PARITY_LOG (if set): a record of each parity check."""
    path = os.environ.get("PA_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(entry) + "\n")


def gpu_step(batch, path: int = 0, write: bool = True, out_dtype=None, window: int = 0):
    """KV write then attention on cuda:0; returns (out, k_cache, v_cache) on the CPU."""
    dev = torch.device("cuda:0")
    pk.set_path(path)
    try:
        kc, vc = batch.k_cache.to(dev), batch.v_cache.to(dev)
        if write:
            pk.paged_kv_write(batch.k.to(dev), batch.v.to(dev), batch.slot_mapping.to(dev), kc, vc)
        out = torch.full(batch.q.shape, float("nan"), dtype=batch.q.dtype, device=dev)
        pk.paged_attention_varlen(batch.q.to(dev), kc, vc, batch.query_start_loc.to(dev), batch.seq_lens.to(dev),
                                  batch.block_table.to(dev), batch.block_size, batch.scale, out,
                                  query_start_loc_host=batch.query_start_loc_host,
                                  seq_lens_host=batch.seq_lens_host, max_query_len=batch.max_query_len,
                                  max_seq_len=batch.max_seq_len, sliding_window=window)
        torch.cuda.synchronize()
        return out.cpu(), kc.cpu(), vc.cpu()
    finally:
        pk.set_path(0)


def oracle_step(batch, row_mask: Optional[np.ndarray] = None, write: bool = True, window: int = 0):
    """The oracle's KV write then attention; returns (float64 out, k_cache, v_cache) as numpy."""
    kc, vc = to_np(batch.k_cache).copy(), to_np(batch.v_cache).copy()
    if write:
        oracle.kv_write(to_np(batch.k), to_np(batch.v), batch.slot_mapping.numpy(), kc, vc, batch.dtype, batch.dtype)
    _, out64 = oracle.paged_attention(to_np(batch.q), kc, vc, batch.query_start_loc.numpy(), batch.seq_lens.numpy(),
                                      batch.block_table.numpy(), batch.scale, batch.dtype, row_mask=row_mask,
                                      want_f64=True, window=window)
    return out64, kc, vc


def assert_pools_equal(gpu_cache: torch.Tensor, oracle_cache: np.ndarray) -> None:
    """Bit-exact on every slot except the scratch slot (padding rows race for it)."""
    g = to_np(gpu_cache).reshape(-1, gpu_cache.shape[2] * gpu_cache.shape[3])
    o = oracle_cache.reshape(g.shape)
    assert np.array_equal(g[:-1].view(np.uint8), o[:-1].view(np.uint8)), "pool differs from the oracle's"


def check_batch(batch, path: int = 0, row_mask: Optional[np.ndarray] = None, label: str = "",
                window: int = 0) -> float:
    """Full parity of one step: pools bit-exact, attention within the bound on every row
    (or the rows of row_mask).  Returns the error as a multiple of the bound."""
    log(f"[parity] {label or batch.name}: N={batch.num_tokens} R={batch.num_reqs} dtype={batch.dtype} path={path}"
        f" window={window}")
    out, kc, vc = gpu_step(batch, path=path, window=window)
    ref64, okc, ovc = oracle_step(batch, row_mask=row_mask, window=window)
    assert_pools_equal(kc, okc)
    assert_pools_equal(vc, ovc)
    got = out.float().numpy()
    rows = slice(None) if row_mask is None else np.nonzero(row_mask)[0]
    err = attention_error(got[rows], ref64[rows], batch.dtype)
    log(f"[parity] {label or batch.name}: error {err:.3g} x bound")
    entry = {"case": label or batch.name, "dtype": batch.dtype, "path": path, "window": window, "error_x_bound": err,
             "rows_checked": int(len(got) if row_mask is None else row_mask.sum())}
    if batch.dtype == "bf16":
        entry["excess_over_rounding_x_2e-2"] = rounding_excess(got[rows], ref64[rows])
    record(entry)
    assert err <= 1.0, f"{label or batch.name}: error {err:.3g} x the bound"
    return err
