"""Seeded randomized parity: random shapes (1..700 on each axis), strides
(padded rows, transposed views, leading offsets) and every forced plan
family and tile, in fp16 and bfloat16, against the oracle.  Integer inputs
in [-4, 4] keep every fp32 sum exact (|sum| <= 16 K < 2^24), so each output
is the correctly rounded exact sum on both sides and must agree bit for bit.
Plans that the library declines for a case (GEMM_ERR_OPTS, e.g. the skinny
family for M > 64) are skipped; each case must run at least the automatic
plan and four forced ones.
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_fp16_amd as g
import oracle
import synth
from gpu_util import ORACLE_THREADS, Out, assert_bits_equal, place, say

pytestmark = pytest.mark.gpu

PLANS = [dict(variant="auto"), dict(variant="main"), dict(variant="main", tile=14),
         dict(variant="main", tile=13), dict(variant="main", tile=1), dict(variant="main", tile=6),
         dict(variant="tile64x32"), dict(variant="splitk"),
         dict(variant="splitk", tile=14, split_k=3), dict(variant="splitk", tile=1, split_k=5),
         dict(variant="streamk"), dict(variant="streamk", split_k=2), dict(variant="skinny"),
         dict(variant="skinny", split_k=3), dict(variant="main", panel=-1),
         dict(variant="main", panel=3)]


def _case(seed):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(1, 65)) if rng.random() < 0.3 else int(rng.integers(65, 701))
    N, K = int(rng.integers(1, 701)), int(rng.integers(1, 701))
    a_layout = "col" if rng.random() < 0.25 else "row"
    b_layout = "col" if rng.random() < 0.4 else "row"
    # Row padding 0 (contiguous), 8 (aligned rows) or odd (unaligned rows);
    # a leading offset of whole NaN rows.
    pa = (int(rng.integers(0, 3)), int(rng.choice([0, 8, 3, 13])))
    pb = (int(rng.integers(0, 3)), int(rng.choice([0, 8, 5])))
    fmt = "bf16" if rng.random() < 0.3 else "f16"
    return M, N, K, a_layout, b_layout, pa, pb, fmt


@pytest.mark.parametrize("seed", range(18000, 18024))
def test_random_case_all_plans(seed):
    M, N, K, al, bl, pa, pb, fmt = _case(seed)
    A = synth.matrix(M, K, seed, 0, "int", fmt=fmt)
    B = synth.matrix(K, N, seed, 1, "int", fmt=fmt)
    ref = oracle.gemm(A, (K, 1), B, (N, 1), M, N, K, nthreads=ORACLE_THREADS,
                      dtype="bf16" if fmt == "bf16" else "f16")
    a, b = place(A, al, pa), place(B, bl, pb)
    if fmt == "bf16":
        a, b = a.view(torch.bfloat16), b.view(torch.bfloat16)
    ran = 0
    for kw in PLANS:
        out = Out(M, N, ldc=N + (seed % 3) * 8)
        if fmt == "bf16":
            out.view = out.view.view(torch.bfloat16)
        try:
            p = g.plan(a, b, out=out.view, **kw)
        except g.GemmError as e:
            if e.status != -7:             # only a declined option combination may skip
                raise
            continue
        say(f"fuzz seed={seed} {fmt} {M}x{N}x{K} A={al}{pa} B={bl}{pb} {kw} -> "
            f"{p['variant']} tile {p['tile_id']} split {p['split_k']} sk {p['sk_tiles']}")
        g.gemm(a, b, out=out.view, **kw)
        torch.cuda.synchronize()
        assert_bits_equal(out.result(), ref, f"seed {seed} {kw} plan {p}")
        ran += 1
    assert ran >= 5, f"seed {seed}: only {ran} plans ran"
