"""Shared helpers for the GPU parity tests (inputs from synth, expectations
from the oracle only)."""
import functools
import sys

import numpy as np

import synth

U = {synth.F16: 2.0 ** -11, synth.BF16: 2.0 ** -8, synth.F32: 0.0}  # unit roundoff
ROT_TOL = 1e-3   # rotated activations: max |dX_r| <= 1e-3 * row max |X_r|
LIN_TOL = 5e-3   # outputs: max |dY| <= 5e-3 * max |Y_ref|


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=16)
def workload(cfg: int, li: int = 0):
    spec = synth.WORKLOADS[cfg]
    lname, I, O = spec["layers"][li]
    L = synth.make_layer(cfg, li, I, O)
    x = synth.make_x(cfg, li, spec["tokens"], I, spec["act"])
    return lname, L, x, spec["act"]


def torch_dtype(dt):
    import torch
    return {synth.F16: torch.float16, synth.BF16: torch.bfloat16, synth.F32: torch.float32}[dt]


def x_to_device(x, dt):
    import torch
    if dt == synth.F32:
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch_dtype(dt))


def to_host_bits(t):
    """Device tensor -> numpy (uint16 bit patterns for 16-bit types, float32 else)."""
    import torch
    t = t.detach().cpu()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def sample_rows(M, n=48, seed=0):
    """A seeded sample of row indices that always includes the first and last."""
    if M <= n:
        return np.arange(M)
    r = np.random.default_rng(seed).choice(np.arange(1, M - 1), size=n - 2, replace=False)
    return np.unique(np.concatenate([[0, M - 1], r]))


def stratified_rows(M, per_tile=3, seed=0, tile=256):
    """Rows that cover every `tile`-row block of M (the prefill GEMM's M tile)
    with `per_tile` rows each, whose residues mod 16 (the row inside an MFMA
    fragment) run through 0..15 in turn across the sample, plus rows 0 and
    M - 1.  Each row sits in a seeded random 16-row block of its tile."""
    rng = np.random.default_rng(seed)
    rows = {0, M - 1}
    n = 0
    for t0 in range(0, M, tile):
        span = min(tile, M - t0)
        for _ in range(per_tile):
            res = n % 16
            n += 1
            blocks = [b for b in range((span + 15) // 16) if t0 + 16 * b + res < M]
            if blocks:
                rows.add(t0 + 16 * int(rng.choice(blocks)) + res)
    return np.array(sorted(rows))


def bits_to_f64(bits, dt):
    if dt == synth.F16:
        return np.asarray(bits).view(np.float16).astype(np.float64)
    if dt == synth.BF16:
        return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(bits, dtype=np.float64)
