"""Helpers shared by the GPU parity tests (comparison and oracle drivers)."""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np
import torch

import oracle


def f64(t):
    return t.detach().cpu().double().numpy()


def maxabs(a, b):
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))


def ulp16(x, dtype):
    """Spacing of the 16-bit format at |x|."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    mant = 10 if dtype == torch.float16 else 7
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -14)))
    return 2.0 ** (e - mant)


def threads():
    return max(1, min(16, os.cpu_count() or 1))


def oracle_core_heads(q, k, v, S0, head_map, heads, **kw):
    """oracle.core for one sequence, restricted to the listed v-heads, with the
    heads spread over host threads (each call covers one head; the oracle is
    sequential within it). Returns (y, S) with untouched heads left at 0 / S0."""
    Hv = v.shape[1]
    T, dv = v.shape[0], v.shape[2]
    y = np.zeros((T, Hv, dv))
    S = np.array(S0, dtype=np.float64, copy=True)

    def one(hh):
        return hh, oracle.core(q, k, v, S0, head_map, heads=(hh, hh + 1), **kw)

    with ThreadPoolExecutor(max_workers=threads()) as ex:
        for hh, (yh, Sh) in ex.map(one, list(heads)):
            y[:, hh] = yh[:, hh]
            S[hh] = Sh[hh]
    return y, S
