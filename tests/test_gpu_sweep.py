"""Seeded random batches through the GPU path: each checked against the oracle at the bf16 bound,
and the call without a planner launch (batches of at most 64 requests on the small tiles)
checked bit for bit against the same call with the planner launched (path 2).

The shapes cover what the fixed cases cover one at a time, in combination: 1, 2, 4 or 8 KV
heads with 1 to 16 query heads each, head_dim 48 (small tiles only), 64 and 128, fp8 pools,
sliding windows, decodes, speculative rows and chunks on both the small and the prefill tiles,
contexts at block and tile boundaries, pad_to rows, and batches just over 64 requests."""
import random

import numpy as np
import pytest

import workloads
from tests import gpu_harness as H
from tests import test_gpu_parity as T
from tests._util import attention_error

N_CASES = 60


def _case(rng):
    hkv = rng.choice([1, 2, 4, 8])
    g = rng.choice([1, 2, 3, 4, 6, 8, 16])
    if g * hkv > 64:
        g = max(1, 64 // hkv)
    d = rng.choice([48, 64, 128])
    fp8 = d != 48 and rng.random() < 0.25
    window = rng.choice([0, 0, 0, 1, 17, 64, 300, 2000])
    nreq = rng.choice([1, 2, 3, 5, 9, 17, 40, 64, 65])
    specs = []
    for _ in range(nreq):
        kind = rng.random()
        c = rng.choice([0, 1, 15, 16, 17, 63, 64, 100, 500, 2047, 2049, 5000])
        if kind < 0.6:
            t = 1
        elif kind < 0.85:
            t = rng.choice([2, 3, 5, 9])
        else:
            t = rng.choice([10, 31, 64, 129, 300])
        specs.append((c, t))
    pad = rng.choice([None, None, nreq + 3])
    return dict(hkv=hkv, g=g, d=d, fp8=fp8, window=window, specs=specs, pad=pad, seed=rng.randrange(1000))


CASES = []
_rng = random.Random(7)
for _i in range(N_CASES):
    CASES.append(_case(_rng))


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(N_CASES)])
def test_random_batch(case):
    import paged_kv_attention_05_amd as pk
    b = workloads.small_batch(case["specs"], dtype="bf16", num_heads=case["g"] * case["hkv"],
                              num_kv_heads=case["hkv"], head_dim=case["d"], seed=case["seed"], pad_to=case["pad"])
    H.log(f"[sweep] hkv={case['hkv']} g={case['g']} d={case['d']} fp8={case['fp8']} window={case['window']} "
          f"requests={len(case['specs'])} pad_to={case['pad']} seed={case['seed']}")
    outs = []
    ref64 = None
    for path in (0, 2):
        pk.set_path(path)
        try:
            if case["fp8"]:
                got, ref64 = T._fp8_step(b, window=case["window"])
                outs.append(got)
            else:
                got, _, _ = H.gpu_step(b, path=path, window=case["window"])
                outs.append(got.float().numpy())
        finally:
            pk.set_path(0)
    if not case["fp8"]:
        ref64, _, _ = H.oracle_step(b, window=case["window"])
    err = attention_error(outs[0], ref64, "bf16")
    assert err <= 1.0, err
    assert np.array_equal(outs[0], outs[1], equal_nan=True)
