"""Test helpers: tensor <-> numpy marshalling and independent dense references.

Nothing here is shared with the HIP path; the dense references below do not call the
oracle and do not go through a block pool.
"""
from __future__ import annotations

import numpy as np
import torch


def to_np(t: torch.Tensor) -> np.ndarray:
    """CPU tensor -> numpy for the oracle (bfloat16 as its uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


def from_np(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    return torch.from_numpy(a.copy())


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of an oracle-format array."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def dense_fold_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, computed: int,
                         window: int = 0) -> np.ndarray:
    """Causal attention of t query rows at positions computed .. computed + t - 1 over
    contiguous keys 0 .. L-1, written with the grouped-query fold the vllm-lite README prints
    (query heads folded into the row dimension of their KV head, no repeated K), a full
    score matrix and an explicit bottom-right mask; window > 0 also masks keys at or before
    position - window (a band).  q [t,H,D], k/v [L,Hkv,D], float64."""
    t, H, D = q.shape
    L, Hkv, _ = k.shape
    rep = H // Hkv
    qg = q.transpose(1, 0, 2).reshape(Hkv, rep * t, D)
    scores = scale * (qg @ k.transpose(1, 2, 0))                 # [Hkv, rep*t, L]
    row_pos = computed + (np.arange(rep * t) % t)                 # query row of each folded row
    allowed = np.arange(L)[None, :] <= row_pos[:, None]
    if window > 0:
        allowed &= np.arange(L)[None, :] > row_pos[:, None] - window
    scores = np.where(allowed[None], scores, -np.inf)
    scores = scores - scores.max(axis=2, keepdims=True)
    p = np.exp(scores)
    p = p / p.sum(axis=2, keepdims=True)
    og = p @ v.transpose(1, 0, 2)                                 # [Hkv, rep*t, D]
    return og.reshape(H, t, D).transpose(1, 0, 2)


def sdpa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, computed: int,
                   window: int = 0) -> np.ndarray:
    """The same attention through torch's scaled_dot_product_attention in float64 on the
    CPU, with an explicit bottom-right boolean mask (is_causal aligns top-left; with a
    window, a band) and torch's own grouped-query expansion."""
    t, H, D = q.shape
    L = k.shape[0]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2)[None]
    pos = (computed + torch.arange(t))[:, None]
    mask = torch.arange(L)[None, :] <= pos
    if window > 0:
        mask &= torch.arange(L)[None, :] > pos - window
    y = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale,
                                                         enable_gqa=True)
    return y[0].permute(1, 0, 2).numpy()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def attention_error(got: np.ndarray, ref64: np.ndarray, dtype: str) -> float:
    """Error of a GPU attention output against the float64 oracle, as a multiple of the bound.

    float32: |got - ref| <= 1e-5 * max|ref| over the (row, head) vector, since outputs are
    convex combinations of V rows and may cross zero.
    bfloat16: |got - ref| <= 2e-2 + half a bfloat16 ulp of ref (the rounding of the stored
    output alone can exceed 2e-2 once |ref| >= 8).
    Returns max(error / bound); <= 1 passes.  NaN anywhere returns inf.
    """
    got = np.asarray(got, dtype=np.float64)
    if got.size == 0:
        return 0.0
    if not np.all(np.isfinite(got)) or not np.all(np.isfinite(ref64)):
        return float("inf")
    diff = np.abs(got - ref64)
    if dtype == "f32":
        bound = 1e-5 * np.maximum(np.abs(ref64).max(axis=-1, keepdims=True), 1e-30)
    else:
        bound = 2e-2 + 0.5 * bf16_ulp(ref64)
    return float((diff / bound).max())


def rounding_excess(got: np.ndarray, ref64: np.ndarray) -> float:
    """bfloat16 outputs: the largest error beyond half a bf16 ulp of the reference (the part
    the output rounding cannot explain), as a fraction of 2e-2.  Shows how much of the
    absolute budget the kernel's arithmetic itself uses."""
    got = np.asarray(got, dtype=np.float64)
    if got.size == 0:
        return 0.0
    ex = np.abs(got - ref64) - 0.5 * bf16_ulp(ref64)
    return float(max(0.0, ex.max()) / 2e-2)
