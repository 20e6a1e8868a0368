"""Pins of the oracle's query smoothing (the SageAttention2-style Q smoothing
the pages name as prior art): per 128-position query block the channel mean is
subtracted before the Q codes are formed and returns as a per-key score term.
Checked against numpy's fp64 means and dot products, an exact invariance of the
codes, error bounds against exact scores, and accuracy on queries with a mean
offset.  CPU only."""
import numpy as np
import pytest

from oracle import oracle as orc
from synthetic import inputs

F32 = np.float32


def _f(bits):
    return inputs.bf16_bits_to_f32(bits).astype(np.float64)


def _qoffset_case(N=300, H=2, off=4.0, seed=3):
    """Queries with a per-channel mean offset (bf16), the regime smoothing is for."""
    q, k, v = inputs.make_custom(1, H, N, seed=seed, rate=0.01, sigma=20.0)
    rng = np.random.default_rng(seed)
    qf = inputs.bf16_bits_to_f32(q) + F32(off) * rng.standard_normal((1, H, 1, 128)).astype(F32)
    return inputs.to_bf16_bits(qf), k, v


@pytest.fixture(scope="module")
def sq_case():
    q, k, v = _qoffset_case()
    P = orc.make_params(1, 2, 300, C_=4, T=3, rho=0.02, flags=orc.DEFAULT_FLAGS | orc.SMOOTH_Q)
    return P, q, k, v, orc.prepare(P, q, k, v)


def test_block_means_are_the_query_block_means(sq_case):
    P, q, k, v, pr = sq_case
    N = P.N
    for s in range(2):
        rows = pr["perm"][s]  # PERMUTE_Q: query blocks in cluster order
        qq = _f(q[0, s])[rows]
        for b in range((N + 127) // 128):
            want = qq[b * 128:min(N, b * 128 + 128)].mean(0)
            got = pr["qbar"][s][b].astype(np.float64)
            # exact sum on the 2^-24 grid, one division, one fp32 rounding
            assert np.all(np.abs(got - want) <= 2.0 ** -25 + np.abs(want) * 2.0 ** -24 + 1e-12)


def test_codes_come_from_the_centred_queries(sq_case):
    P, q, k, v, pr = sq_case
    N = P.N
    for s in range(2):
        qq = _f(q[0, s])[pr["perm"][s]]
        for b in range((N + 127) // 128):
            r = slice(b * 128, min(N, b * 128 + 128))
            xc = qq[r] - pr["qbar"][s][b].astype(np.float64)
            deq = orc.e4m3_decode(pr["q8"][s][r]) * pr["sq"][s][b]
            # E4M3 keeps 3 mantissa bits: error at most half a step, 2^-4 relative
            # (absolute 2^-10 * scale below the normal range)
            tol = np.maximum(np.abs(xc) * 2.0 ** -4, pr["sq"][s][b] * 2.0 ** -10) * (1 + 1e-6) + 1e-30
            assert np.all(np.abs(deq - xc) <= tol)
            # the block scale is set by the centred block's maximum
            assert pr["sq"][s][b] == pytest.approx(np.abs(xc).max() / 448.0, rel=1e-6)


def test_score_term_is_the_mean_query_dot_smoothed_key(sq_case):
    P, q, k, v, pr = sq_case
    N, npad = P.N, ((P.N + 127) // 128) * 128
    c0 = 8.0 * np.log2(np.e) / np.sqrt(128.0)
    for s in range(2):
        kt = _f(k[0, s])[pr["perm"][s]] - pr["kbar"][s].astype(np.float64)
        for b in range((N + 127) // 128):
            qm = pr["qbar"][s][b].astype(np.float64)
            exact = kt @ qm * c0
            got = pr["qbias"][s][b][:N].astype(np.float64)
            # fp32 chain of 128 fma plus the fp32 rounding of k - kbar and of c0 * delta
            bound = c0 * (np.abs(kt) @ np.abs(qm)) * 130 * 2.0 ** -24 + np.abs(exact) * 2.0 ** -23
            assert np.all(np.abs(got - exact) <= bound + 1e-30)
            assert not pr["qbias"][s][b][N:npad].any()


def test_shifting_a_block_leaves_its_codes_unchanged():
    """Adding a constant vector to every query of the sequence changes only the
    block means: codes and scales are those of the centred queries.  Inputs on
    a 2^-4 grid keep every sum exact, so the invariance is bit-exact."""
    N = 256
    q, k, v = inputs.make_custom(1, 1, N, seed=11)
    rng = np.random.default_rng(1)
    qg = (np.round(rng.standard_normal((1, 1, N, 128)) * 16) / 16).clip(-3.875, 3.875).astype(F32)
    qg = qg + F32(0.0)  # no negative zeros: -0 - 0 codes as E4M3 -0, (-0 + u) - u as +0
    u = rng.integers(-3, 4, (1, 1, 1, 128)).astype(F32)
    P = orc.make_params(1, 1, N, C_=3, T=3, flags=orc.VSMOOTH | orc.PERMUTE_Q | orc.SMOOTH_Q)
    assert np.array_equal(inputs.bf16_bits_to_f32(inputs.to_bf16_bits(qg + u)), qg + u)  # exact in bf16
    a = orc.prepare(P, inputs.to_bf16_bits(qg), k, v)
    b = orc.prepare(P, inputs.to_bf16_bits(qg + u), k, v)
    assert np.array_equal(a["q8"], b["q8"]) and np.array_equal(a["sq"], b["sq"])
    assert np.allclose(b["qbar"] - a["qbar"], np.broadcast_to(u.reshape(1, 1, 128), a["qbar"].shape))
    # without smoothing the shift does change the codes
    P0 = orc.make_params(1, 1, N, C_=3, T=3, flags=orc.VSMOOTH | orc.PERMUTE_Q)
    assert not np.array_equal(orc.prepare(P0, inputs.to_bf16_bits(qg), k, v)["q8"],
                              orc.prepare(P0, inputs.to_bf16_bits(qg + u), k, v)["q8"])


def test_smoothing_brings_outputs_closer_to_exact_attention():
    q, k, v = _qoffset_case(N=512, H=2, off=4.0, seed=5)
    rows = np.arange(0, 512, 5, dtype=np.int32)
    slot = np.repeat(np.arange(2), len(rows)).astype(np.int32)
    idx = np.tile(rows, 2).astype(np.int32)
    err = {}
    for name, flags in (("plain", orc.DEFAULT_FLAGS), ("smooth", orc.DEFAULT_FLAGS | orc.SMOOTH_Q)):
        P = orc.make_params(1, 2, 512, C_=4, flags=flags)
        pr = orc.prepare(P, q, k, v)
        sim = orc.forward_rows(P, pr, slot, idx)
        ex = orc.exact_rows(P, q, k, v, slot, idx)
        err[name] = np.linalg.norm(sim - ex) / np.linalg.norm(ex)
    assert err["smooth"] < 0.7 * err["plain"], err


def test_zero_mean_queries_lose_nothing_to_smoothing():
    """On zero-mean queries the block means are small: the two paths carry
    independent quantisation errors of the same size, and smoothing does not
    move the simulation further from exact attention (within 20%)."""
    q, k, v = inputs.make_inputs(0)
    rows = np.arange(0, 1024, 9, dtype=np.int32)
    slot = np.repeat(np.arange(2), len(rows)).astype(np.int32)
    idx = np.tile(rows, 2).astype(np.int32)
    err = []
    for flags in (orc.DEFAULT_FLAGS, orc.DEFAULT_FLAGS | orc.SMOOTH_Q):
        P = orc.make_params(1, 2, 1024, C_=8, flags=flags)
        sim = orc.forward_rows(P, orc.prepare(P, q, k, v), slot, idx)
        ex = orc.exact_rows(P, q, k, v, slot, idx)
        err.append(np.linalg.norm(sim - ex) / np.linalg.norm(ex))
    assert err[1] < 1.2 * err[0], err
