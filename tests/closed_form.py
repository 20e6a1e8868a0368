"""Hand-built inputs whose attention output is known in closed form (shared by
the oracle pins and the GPU parity tests; numpy only).

Online rescale case.  One query row sees two 128-key blocks whose scores are
constant inside each block and differ by exactly `jump` ExpCast code units
(jump = 8 is one factor of two in probability, the slope of the byte relation in
the ExpCast-FP8 section of the noticiai.com.br VC-Attention article).  Every
value is a power of two times a small integer, so the block scales (amax/448),
the E4M3 codes (256 -> byte 0x78), the raw score (2^16) and the code gain
(softmax scale chosen so that 8*log2(e)*scale rounds to exactly 1 in fp32) are
all exact:

  block 0 scores t0 = -jump/2, block 1 scores t1 = +jump/2 (code units)
  after block 0:  M = t0, every code = 56+8k, l = 128 * p(code)
  block 1:        M moves to t1, r = 2^((t0 - t1)/8) = 2^(-jump/8), every
                  code = 56+8k again, l = l*r + 128 * p(code)
  V constant inside each block (rows mu0, mu1) and one cluster, so V-Smooth's
  block means carry all of V (residual codes 0) and Restore returns them:
  O = (r * mu0 + mu1) / (r + 1).

With mu0 = (1 + 2^(jump/8)) u and mu1 = (1 + 2^(-jump/8)) w the output is
u + w exactly; exact softmax attention gives the same weights 1 : 2^(jump/8).
"""
from __future__ import annotations

import numpy as np

LOG2E = 1.4426950408889634


def unit_gain_scale() -> float:
    """An fp32 softmax scale s with fp32(8 * log2(e) * s) == 1 exactly, the
    product taken in double as the library and the oracle form it."""
    s0 = np.float32(1.0 / (8.0 * LOG2E))
    for cand in (s0, np.nextafter(s0, np.float32(1)), np.nextafter(s0, np.float32(0))):
        if np.float32(8.0 * LOG2E * float(cand)) == np.float32(1.0):
            return float(cand)
    raise AssertionError("no fp32 scale gives a unit code gain")


def rescale_case(jump: int, seed: int = 0):
    """bf16-exact float32 arrays q, k, v [1, 1, 256, 128], the checked query row,
    and its expected output row.  jump in {8, 16} code units."""
    assert jump in (8, 16)
    N, d = 256, 128
    a = -7
    b = (-14 if jump == 8 else -13) - a          # 2^16 * 2^(a+b) = jump / 2
    q = np.zeros((N, d), np.float32)
    k = np.zeros((N, d), np.float32)
    row = 5
    q[row, 0] = 256.0 * 2.0 ** a                 # code 256 after the scale 2^a
    q[7, 1] = 448.0 * 2.0 ** a                   # sets the block maximum: scale 2^a
    k[:128, 0] = -256.0 * 2.0 ** b
    k[128:, 0] = 256.0 * 2.0 ** b
    for j0 in (10, 140):                         # block maxima 448 * 2^b, channel mean 0
        k[j0, 1] = 448.0 * 2.0 ** b
        k[j0 + 1, 1] = -448.0 * 2.0 ** b
    rng = np.random.default_rng(seed)
    u = rng.integers(-4, 5, d).astype(np.float32)
    w = rng.integers(-4, 5, d).astype(np.float32)
    g = 2.0 ** (jump / 8)
    v = np.zeros((N, d), np.float32)
    v[:128] = (1 + g) * u
    v[128:] = (1 + 1 / g) * w
    want = (u + w).astype(np.float64)
    shp = (1, 1, N, d)
    return q.reshape(shp), k.reshape(shp), v.reshape(shp), row, want


def lazy_max_case(seed: int = 0):
    """The online case with a jump of 4 code units, below a lazy-maximum slack
    tau = 6 (R11: M moves only when a block maximum exceeds it by more than
    tau).  M stays at block 0's maximum, so block 0's codes are 56+8k = 120
    (E4M3 256) and block 1's are 124 (E4M3 384), with no rescale:
    O = (256 mu0 + 384 mu1) / 640 = 0.4 mu0 + 0.6 mu1.  Without the slack M
    would move and the weights would be 1 : 2^(-1/2) instead.  Returns bf16-exact
    float32 q, k, v [1, 1, 256, 128], the row and its expected output (k = 8)."""
    N, d = 256, 128
    a = -7
    b = -15 - a                                  # 2^16 * 2^(a+b) = 2 = jump / 2
    q = np.zeros((N, d), np.float32)
    k = np.zeros((N, d), np.float32)
    row = 5
    q[row, 0] = 256.0 * 2.0 ** a
    q[7, 1] = 448.0 * 2.0 ** a
    k[:128, 0] = -256.0 * 2.0 ** b
    k[128:, 0] = 256.0 * 2.0 ** b
    for j0 in (10, 140):
        k[j0, 1] = 448.0 * 2.0 ** b
        k[j0 + 1, 1] = -448.0 * 2.0 ** b
    rng = np.random.default_rng(seed)
    mu0 = rng.integers(-4, 5, d).astype(np.float32)
    mu1 = rng.integers(-4, 5, d).astype(np.float32)
    v = np.zeros((N, d), np.float32)
    v[:128] = mu0
    v[128:] = mu1
    want = (256.0 * mu0.astype(np.float64) + 384.0 * mu1.astype(np.float64)) / 640.0
    shp = (1, 1, N, d)
    return q.reshape(shp), k.reshape(shp), v.reshape(shp), row, want


def block_constant_values(N: int, seed: int = 0) -> np.ndarray:
    """float32 V [N, 128] constant inside every 128-token block (rows of small
    multiples of 1/4, exact in bf16)."""
    rng = np.random.default_rng(seed)
    nb = (N + 127) // 128
    rows = rng.integers(-16, 17, (nb, 128)).astype(np.float32) / 4
    return np.repeat(rows, 128, axis=0)[:N]
