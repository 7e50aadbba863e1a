"""Helpers for the GPU parity tests: device transfer of fp16 bit arrays and
the acceptance checks against the oracle."""
import sys

import numpy as np
import torch

import oracle

DEV = "cuda:0"
ORACLE_THREADS = min(16, oracle.threads())


def say(*msg):
    """Name the case on stdout before each GPU step, so a crash is attributable."""
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def to_dev(bits):
    """numpy uint16 (fp16 bits) -> torch.float16 on the GPU, same shape."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(DEV).view(torch.float16)


def to_host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def val(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def tolerance_violations(gpu_bits, ref_bits):
    """Elementwise check of |C_gpu - C_oracle| <= 1e-2 + 2e-3 |C_oracle| with
    C_oracle the oracle's fp16 output; NaN anywhere is a violation.  Returns
    (number of violations, worst excess, index of the worst)."""
    g, r = val(gpu_bits), val(ref_bits)
    err = np.abs(g - r)
    bound = 1e-2 + 2e-3 * np.abs(r)
    bad = ~(err <= bound)                       # NaN counts as bad
    if not bad.any():
        return 0, 0.0, None
    excess = np.where(np.isnan(err), np.inf, err - bound)
    idx = np.unravel_index(np.argmax(excess), excess.shape)
    return int(bad.sum()), float(excess[idx]), idx


def assert_close(gpu_bits, ref_bits, what=""):
    n, worst, idx = tolerance_violations(gpu_bits, ref_bits)
    assert n == 0, (f"{what}: {n} outputs outside 1e-2 + 2e-3|C| (worst excess {worst} at {idx}: "
                    f"gpu {val(gpu_bits)[idx]} oracle {val(ref_bits)[idx]})")


def assert_bits_equal(gpu_bits, ref_bits, what=""):
    if not np.array_equal(gpu_bits, ref_bits):
        diff = np.argwhere(gpu_bits != ref_bits)
        i = tuple(diff[0])
        raise AssertionError(f"{what}: {len(diff)} outputs differ in bits; first at {i}: "
                             f"gpu {gpu_bits[i]:#06x} ({val(gpu_bits)[i]}) oracle "
                             f"{ref_bits[i]:#06x} ({val(ref_bits)[i]})")


def ulp_histogram(gpu_bits, ref_bits):
    """Distance in units in the last place between two fp16 arrays (finite)."""
    def ordered(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)
    d = np.abs(ordered(gpu_bits) - ordered(ref_bits))
    return {int(k): int(v) for k, v in zip(*np.unique(d, return_counts=True))}
