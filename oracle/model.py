"""Pure-Python model of the tiled GEMM method, for small cases only.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

It follows the Triton article ("Triton GEMM: from one output tile to
addresses, bounds and data reuse"):
  - section "parallelise over outputs, keep K in the accumulator": a grid of
    G_M x G_N programs; program p owns rows p_m*B_M.. and columns p_n*B_N..
    with p_m = p // G_N and p_n = p % G_N, clears an accumulator, walks K in
    rounds of B_K and stores once;
  - section "three dimensions that do not divide": the A load is masked by
    (row < M and k < K), the B load by (k < K and col < N), the C store by
    (row < M and col < N), and masked positions contribute zero.  A modulo
    policy is modelled too, because the article's worked K = 3 example shows
    what it does wrong on K (and why it is harmless on M and N);
and the read ledger of the tiling tutorial ("Matrix multiplication and
memory-access optimisation", sections 02-03), which counts every indexed
element read and models no cache.

Numbers are Python ints or Fractions, so sums are exact.
"""
from fractions import Fraction


def cdiv(a, b):
    return -(-a // b)


class TiledRun:
    """Result and counters of one modelled tiled GEMM."""

    def __init__(self):
        self.C = None
        self.grid = (0, 0)
        self.k_rounds = 0
        self.reads_a = 0
        self.reads_b = 0
        self.writes = 0
        self.block_flops = 0
        self.valid_outputs = {}     # program id -> number of outputs it stores
        self.last_round_valid_k = 0

    @property
    def reads(self):
        return self.reads_a + self.reads_b


def tiled_gemm(A, B, BM, BN, BK, k_policy="mask", mn_policy="mask"):
    """Model C = A.B computed tile by tile.

    A is a list of M rows of K numbers, B a list of K rows of N numbers.
    k_policy / mn_policy: "mask" (zero fill of out-of-range positions) or
    "modulo" (out-of-range indices wrapped back into range).
    """
    M, K = len(A), len(A[0])
    N = len(B[0])
    assert len(B) == K
    run = TiledRun()
    GM, GN = cdiv(M, BM), cdiv(N, BN)
    rounds = cdiv(K, BK)
    run.grid, run.k_rounds = (GM, GN), rounds
    C = [[None] * N for _ in range(M)]
    for p in range(GM * GN):
        pm, pn = p // GN, p % GN
        rm = [pm * BM + i for i in range(BM)]
        rn = [pn * BN + j for j in range(BN)]
        acc = [[0] * BN for _ in range(BM)]
        for q in range(rounds):
            rk = [q * BK + t for t in range(BK)]
            a_tile = [[0] * BK for _ in range(BM)]
            b_tile = [[0] * BN for _ in range(BK)]
            for i, r in enumerate(rm):
                for t, k in enumerate(rk):
                    rr, kk = r, k
                    if mn_policy == "modulo":
                        rr = r % M
                    if k_policy == "modulo":
                        kk = k % K
                    if rr < M and kk < K:
                        a_tile[i][t] = A[rr][kk]
                        run.reads_a += 1
            for t, k in enumerate(rk):
                for j, c in enumerate(rn):
                    kk, cc = k, c
                    if k_policy == "modulo":
                        kk = k % K
                    if mn_policy == "modulo":
                        cc = c % N
                    if kk < K and cc < N:
                        b_tile[t][j] = B[kk][cc]
                        run.reads_b += 1
            for i in range(BM):
                for j in range(BN):
                    s = acc[i][j]
                    for t in range(BK):
                        s += a_tile[i][t] * b_tile[t][j]
                    acc[i][j] = s
            run.block_flops += 2 * BM * BN * BK
            if q == rounds - 1:
                run.last_round_valid_k = sum(1 for k in rk if k < K)
        stored = 0
        for i, r in enumerate(rm):
            for j, c in enumerate(rn):
                if r < M and c < N:
                    assert C[r][c] is None, "two programs wrote one output"
                    C[r][c] = acc[i][j]
                    stored += 1
                    run.writes += 1
        run.valid_outputs[p] = stored
    run.C = C
    return run


def naive_reads(M, N, K):
    """Reads of the straightforward triple loop: each output reads K elements
    of its A row and K elements of its B column."""
    reads = 0
    for _i in range(M):
        for _j in range(N):
            for _k in range(K):
                reads += 2
    return reads


# ---- closed forms of the TileLang tutorial's GEMM ledger (ch. 14, section 1)
# and of the Triton article's per-stage intensity (section "bigger tiles").

def flops(M, N, K):
    """Multiply-adds counted as 2 FLOP each: 2MNK, independent of tiling."""
    return 2 * M * N * K


def min_bytes(M, N, K, b):
    """A and B read once, C written once: b(MK + KN + MN)."""
    return b * (M * K + K * N + M * N)


def intensity(M, N, K, b):
    return Fraction(flops(M, N, K), min_bytes(M, N, K, b))


def tile_reread_bytes(M, N, K, m1, n1, b):
    """Operand reads when output tiles are m1 x n1 and nothing is cached:
    b * M*N*K * (1/m1 + 1/n1)."""
    return Fraction(b * M * N * K) * (Fraction(1, m1) + Fraction(1, n1))


def stage_bytes(BM, BN, BK, b, stages=1):
    """On-chip bytes for `stages` copies of the A (BM x BK) and B (BK x BN) tiles."""
    return stages * (BM * BK + BK * BN) * b


def stage_intensity(BM, BN, b):
    """FLOP per loaded byte in one K round of one tile; B_K cancels."""
    return Fraction(2 * BM * BN, b * (BM + BN))


def accumulator_bytes(BM, BN):
    return 4 * BM * BN
