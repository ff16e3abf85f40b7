"""Runs the oracle's quantiser over a whole tensor in row slices, in parallel
worker processes (spawned: they import numpy and the oracle only, never the
GPU).  Test infrastructure for the full-size parity checks."""
import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np

from oracle import nvfp4_oracle as orc


TIMEOUT_S = 900        # a stuck worker pool fails the test instead of hanging it


def _slice(args):
    bits, alpha = args
    _, scales, codes = orc.quantize(bits, alpha=alpha)
    return scales, codes


def worker_count():
    return max(1, min(16, os.cpu_count() or 1))


def new_pool():
    return cf.ProcessPoolExecutor(max_workers=worker_count(), mp_context=mp.get_context("spawn"))


def quantize_all_rows(pool, bits: np.ndarray, alpha):
    """The oracle's scale bytes and codes of every row of bits, with the
    tensor's alpha given (rows quantised in slices share it)."""
    rows, k = bits.shape
    step = max(1, (1 << 22) // k)                 # about 4 M elements a slice
    parts = list(pool.map(_slice, [(bits[r:r + step], alpha) for r in range(0, rows, step)],
                          timeout=TIMEOUT_S))
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))


def quantize_many(pool, tensors):
    """quantize_all_rows over several (bits, alpha) tensors at once."""
    jobs, owner = [], []
    for t, (bits, alpha) in enumerate(tensors):
        step = max(1, (1 << 22) // bits.shape[1])
        for r in range(0, bits.shape[0], step):
            jobs.append((bits[r:r + step], alpha))
            owner.append(t)
    parts = list(pool.map(_slice, jobs, timeout=TIMEOUT_S))
    out = []
    for t in range(len(tensors)):
        mine = [p for p, o in zip(parts, owner) if o == t]
        out.append((np.concatenate([p[0] for p in mine]), np.concatenate([p[1] for p in mine])))
    return out


def _rms_slice(args):
    bits, gamma_bits, eps = args
    return orc.rmsnorm(bits, gamma_bits, eps)[1]


def rmsnorm_all_rows(pool, bits: np.ndarray, gamma_bits: np.ndarray, eps):
    """The oracle's RMSNorm (BF16 bits) of every row of bits, in row slices."""
    rows, k = bits.shape
    step = max(1, (1 << 20) // k)
    parts = pool.map(_rms_slice, [(bits[r:r + step], gamma_bits, eps) for r in range(0, rows, step)],
                     timeout=TIMEOUT_S)
    return np.concatenate(list(parts))
