"""Pins of the CPU oracle against facts fixed outside it: the OCP E4M3 definition
(checked through torch's independent float8_e4m3fn codec), the ExpCast byte
relation the VC-Attention article states, closed forms, special cases that
reduce to plain means, invariances of non-causal attention, brute force on tiny
inputs and torch's fp64 attention.  CPU only."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from synthetic import inputs

import closed_form  # noqa: E402  (tests/ is on sys.path under pytest)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _page_facts():
    facts, ms = {}, {}
    for line in open(os.path.join(GOLD, "page_facts.txt")):
        line = line.split("#")[0].split()
        if not line:
            continue
        if line[0] == "repair_m":
            ms[int(line[1])] = int(line[2])
        else:
            facts[line[0]] = float(line[1])
    return facts, ms


def _torch_e4m3_encode(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _torch_e4m3_decode(c: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(c, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


# --------------------------------------------------------------------------- codec

def test_e4m3_decode_ocp_points():
    for line in open(os.path.join(GOLD, "e4m3_ocp_points.txt")):
        line = line.split("#")[0].split()
        if not line:
            continue
        code, val = int(line[0], 16), float(line[1])
        got = orc.e4m3_decode([code])[0]
        if math.isnan(val):
            assert math.isnan(got)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val)


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = orc.e4m3_decode(codes), _torch_e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(np.diff(ours[:127]) > 0)  # strictly increasing over 0x00..0x7e


def test_e4m3_encode_vs_torch_sweep():
    rng = np.random.default_rng(0)
    # every bf16-representable value in [-448, 448], random fp32 in several scales,
    # and the exact midpoints between neighbouring codes (ties go to even codes)
    bf = (np.arange(0, 1 << 16, dtype=np.uint32) << 16).view(np.float32)
    bf = bf[np.isfinite(bf) & (np.abs(bf) <= 448)]
    rnd = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.05, 1, 30, 200)])
    vals = orc.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([bf, rnd.astype(np.float32), mids, -mids]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    assert np.array_equal(orc.e4m3_encode(x), _torch_e4m3_encode(x))
    # ties: midpoint between codes c and c+1 rounds to the even code
    mc = orc.e4m3_encode(mids.astype(np.float32))
    assert np.all(mc % 2 == 0)


def test_e4m3_encode_saturates_and_keeps_sign():
    out = orc.e4m3_encode(np.array([448, 449, 470, 1e6, -1e6, -0.0, -1e-9, 1e-9], np.float32))
    assert list(out) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x80, 0x00]


def test_byte_is_about_8log2_plus_56():
    """The page's reading of an E4M3 byte as 8*log2(v)+56 holds within 0.7 over
    every positive normal code (and exactly on powers of two); a decoder with the
    wrong exponent bias is off by a multiple of 8."""
    facts, _ = _page_facts()
    codes = np.arange(8, 127, dtype=np.uint8)
    v = orc.e4m3_decode(codes)
    dev = codes - (facts["expcast_slope"] * np.log2(v) + facts["expcast_offset"])
    assert np.max(np.abs(dev)) < 0.7
    pw = codes[codes % 8 == 0]
    assert np.all(pw == facts["expcast_slope"] * np.log2(orc.e4m3_decode(pw)) + facts["expcast_offset"])


# --------------------------------------------------------------------------- ExpCast

@pytest.mark.parametrize("k", [0, 8])
def test_expcast_within_one_code_of_rne_exp2(k):
    """code = rne(8*u + 56 + 8k) for u = log2(p); over the normal range of E4M3 it
    is within one code of the round-to-nearest E4M3 encoding of p*2^k; below it
    (the subnormal band) the value error stays under 2^-6 in the shifted domain."""
    u = np.linspace(-25.0, 0.0, 400001).astype(np.float32)  # log2 of the probability
    s_raw = (u * np.float32(8.0)).astype(np.float32)  # alpha = 1: raw score in code units
    bias = np.float32(56 + 8 * k)
    codes = orc.expcast(s_raw, 1.0, float(bias))  # row maximum M = 0
    target = np.exp2(u.astype(np.float64) + k)
    rne = _torch_e4m3_encode(target)
    normal = target >= 2.0 ** -6
    assert np.max(np.abs(codes[normal].astype(int) - rne[normal].astype(int))) <= 1
    val = orc.e4m3_decode(codes)
    assert np.max(np.abs(val[~normal] - target[~normal])) <= 2.0 ** -6
    assert np.all(np.diff(codes.astype(int)) >= 0)  # monotone in the score
    assert codes[-1] == 56 + 8 * k  # p = 1 maps to 56 + 8k


def test_expcast_clamps():
    c = orc.expcast(np.array([-np.inf, -1e30, 1e30, 0.4, 0.5, 1.5, 2.5], np.float32), 1.0, 0.0)
    assert list(c) == [0, 0, 126, 0, 0, 2, 2]  # rne: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2


# --------------------------------------------------------------------------- generator

def test_splitmix64_reference_value_and_counter_form():
    # first output for state 0 of Vigna's reference splitmix64
    assert int(orc.splitmix64(0, 1)[0]) == 0xE220A8397B1DCDAF
    seq = orc.splitmix64(12345, 1000)
    assert np.array_equal(seq, inputs.stream(12345, 1000))


def test_kmeans_init_indices_distinct():
    for N, C_ in [(10, 3), (1024, 8), (16544, 32), (75600, 64)]:
        idx = orc.kmeans_init_indices(0, 5, N, C_)
        assert len(set(idx.tolist())) == C_ and idx.min() >= 0 and idx.max() < N


# --------------------------------------------------------------------------- k-means

def _lloyd_fp64(v, init_idx, T):
    cent = v[init_idx].astype(np.float64)
    lab = None
    for _ in range(T):
        d2 = ((v[:, None, :] - cent[None, :, :]) ** 2).sum(-1)
        lab = np.argmin(d2, axis=1)
        srt = np.sort(d2, axis=1)
        margin = (srt[:, 1] - srt[:, 0]).min() if d2.shape[1] > 1 else np.inf
        for kk in range(cent.shape[0]):
            if np.any(lab == kk):
                cent[kk] = v[lab == kk].mean(0)
        if margin < 1e-2 * max(1.0, np.abs(v).max() ** 2):
            return None, None
    return lab, cent


def _lloyd_fixed_numpy(v, init_idx, T):
    """Independent integer Lloyd: values scaled by the largest power of two
    keeping max|v| below 2^13, exact int64 distances, ties to the lowest id,
    rounded (half to even) integer means."""
    a = np.abs(v).max()
    sh = 13 - int(np.frexp(a)[1]) if a > 0 else 0
    u = np.rint(v * 2.0 ** sh).astype(np.int64)
    c = u[init_idx].copy()
    lab = None
    for _ in range(T):
        d = (c * c).sum(1)[None, :] - 2 * (u @ c.T)
        lab = np.argmin(d, axis=1)  # first minimum = lowest id
        for kk in range(c.shape[0]):
            sel = lab == kk
            if sel.any():
                c[kk] = np.rint(u[sel].sum(0) / sel.sum()).astype(np.int64)
    return lab, c.astype(np.float64) * 2.0 ** -sh


def test_kmeans_tiny_brute_force():
    """Labels and centroids equal an independent integer Lloyd from the same
    initial indices; where no assignment is near a tie they also equal the
    real-valued fp64 Lloyd (the fixed-point grid is 2^-13 of max|v|)."""
    checked = 0
    for seed in range(40):
        N = 4 + seed % 7
        C_ = 1 + seed % 3
        T = 1 + seed % 3
        q, k, v = inputs.make_custom(1, 1, N, seed=seed, rate=0.0)
        P = orc.make_params(1, 1, N, C_=C_, T=T, seed=seed, rho=0.0)
        pr = orc.prepare(P, q, k, v)
        vf = inputs.bf16_bits_to_f32(v[0, 0]).astype(np.float64)
        init = orc.kmeans_init_indices(seed, 0, N, C_)
        lab_i, cent_i = _lloyd_fixed_numpy(vf, init, T)
        assert np.array_equal(pr["labels"][0], lab_i)
        assert np.array_equal(pr["centroids"][0].astype(np.float64), cent_i)
        lab, cent = _lloyd_fp64(vf, init, T)
        if lab is None:
            continue
        checked += 1
        assert np.array_equal(pr["labels"][0], lab)
        np.testing.assert_allclose(pr["centroids"][0], cent, rtol=0, atol=2.0 ** -12 * np.abs(vf).max())
    assert checked >= 20


def test_kmeans_fixed_point_larger_head():
    """Exact agreement with the independent integer Lloyd on a head with
    outliers (many clusters, several iterations)."""
    q, k, v = inputs.make_custom(1, 1, 900, seed=31, rate=0.02, sigma=30.0)
    P = orc.make_params(1, 1, 900, C_=12, T=6, seed=4, rho=0.0)
    pr = orc.prepare(P, q, k, v)
    vf = inputs.bf16_bits_to_f32(v[0, 0]).astype(np.float64)
    lab, cent = _lloyd_fixed_numpy(vf, orc.kmeans_init_indices(4, 0, 900, 12), 6)
    assert np.array_equal(pr["labels"][0], lab)
    assert np.array_equal(pr["centroids"][0].astype(np.float64), cent)


def test_kmeans_fixed_point_quality_matches_real_valued_lloyd():
    """At head sizes like the workloads', the fixed-point Lloyd (R1) clusters as
    well as a real-valued fp64 Lloyd from the same initial centroids: the
    within-cluster sum of squares after ten rounds is within 2% of it (the
    labels themselves drift apart from ties on the 2^-13 max|v| grid)."""
    for (N, C_, T, seed) in [(2048, 32, 10, 3), (1024, 8, 10, 0)]:
        q, k, v = inputs.make_custom(1, 1, N, seed=seed, rate=0.01, sigma=20.0)
        P = orc.make_params(1, 1, N, C_=C_, T=T, seed=seed, rho=0.0)
        pr = orc.prepare(P, q, k, v)
        vf = inputs.bf16_bits_to_f32(v[0, 0]).astype(np.float64)
        cent = vf[orc.kmeans_init_indices(seed, 0, N, C_)].copy()
        for _ in range(T):
            d2 = (vf * vf).sum(1)[:, None] + (cent * cent).sum(1)[None, :] - 2 * vf @ cent.T
            lab = np.argmin(d2, axis=1)
            for kk in range(C_):
                if np.any(lab == kk):
                    cent[kk] = vf[lab == kk].mean(0)
        sse_real = ((vf - cent[lab]) ** 2).sum()
        cf = pr["centroids"][0].astype(np.float64)
        sse_fixed = ((vf - cf[pr["labels"][0]]) ** 2).sum()
        assert abs(sse_fixed - sse_real) <= 0.02 * sse_real, (N, C_, sse_fixed, sse_real)


def _one_channel_head(vals, N_extra=0):
    """bf16 bits [1, 1, N, 128] whose channel 0 holds vals (fixed-point units of
    2^-12: the first value 1.0 sets max|v| = 1, so sh = 12) and the rest 0."""
    v = np.zeros((len(vals), 128), np.float64)
    v[:, 0] = np.asarray(vals, np.float64) / 4096.0
    return inputs.to_bf16_bits(v)[None, None]


def test_kmeans_ties_go_to_the_lowest_id():
    """R1: a token at the same integer distance from two centroids joins the
    one with the lower id.  Tokens 4096, -8, 8, 0 (fixed-point units, sh = 12);
    a seed whose Forgy draw picks tokens -8 and 8 leaves token 0 exactly between
    them, and after one assignment it carries the smaller of their ids."""
    vb = _one_channel_head([4096, -8, 8, 0])
    z = np.zeros_like(vb)
    for seed in range(200):
        init = orc.kmeans_init_indices(seed, 0, 4, 2)
        if sorted(init.tolist()) == [1, 2]:
            break
    else:
        raise AssertionError("no seed draws tokens 1 and 2")
    P = orc.make_params(1, 1, 4, C_=2, T=1, seed=seed, rho=0.0)
    lab = orc.prepare(P, z, z, vb)["labels"][0]
    id_of = {int(init[0]): 0, int(init[1]): 1}
    assert lab[1] == id_of[1] and lab[2] == id_of[2]
    assert lab[3] == 0            # the tie: the lower id
    assert lab[0] == id_of[2]     # 4096 is nearer to 8


def test_empty_cluster_keeps_its_centroid():
    """R1: a cluster left without members keeps its centroid.  Tokens 4096,
    100, 100, 50 (fixed-point units); a Forgy draw of the two tokens at 100
    puts both centroids there, every token ties and joins the lower id, so
    cluster 1 is empty: it stays at 100 while cluster 0 moves to the rounded
    mean 1086 (4346 / 4 = 1086.5, ties to even)."""
    vb = _one_channel_head([4096, 100, 100, 50])
    z = np.zeros_like(vb)
    for seed in range(400):
        if sorted(orc.kmeans_init_indices(seed, 0, 4, 2).tolist()) == [1, 2]:
            break
    else:
        raise AssertionError("no seed draws tokens 1 and 2")
    P = orc.make_params(1, 1, 4, C_=2, T=1, seed=seed, rho=0.0)
    pr = orc.prepare(P, z, z, vb)
    assert pr["labels"][0].tolist() == [0, 0, 0, 0]
    cent = pr["centroids"][0][:, 0].astype(np.float64) * 4096.0
    assert cent.tolist() == [1086.0, 100.0]


def test_repair_ties_go_to_lower_positions():
    """R14: among equal errors the lower position is repaired first.  Every V
    row is the same, so every token has the same error (0 after demeaning, or the
    same quantisation error without V-Smooth): the repair set is the first m
    positions."""
    N = 300
    rng = np.random.default_rng(2)
    q = inputs.to_bf16_bits(rng.standard_normal((N, 128)))[None, None]
    k = inputs.to_bf16_bits(rng.standard_normal((N, 128)))[None, None]
    row = rng.standard_normal(128) * 3.0
    v = inputs.to_bf16_bits(np.tile(row, (N, 1)))[None, None]
    for flags in (orc.DEFAULT_FLAGS, orc.REPAIR | orc.PERMUTE_Q):
        P = orc.make_params(1, 1, N, C_=1, T=1, rho=0.02)
        P.flags = flags
        pr = orc.prepare(P, q, k, v)
        m = pr["m"]
        assert m == 6
        assert pr["rep_pos"][0][:m].tolist() == list(range(m))


def test_warm_start_rounds_centroids_to_nearest():
    """R17: warm-start centroids are scaled to the current fixed point and
    rounded to the nearest integer.  Centroids 2.6 and 7.6 (units of 2^-12)
    become 3 and 8, so token 5 (distance 2 against 3) joins the first and token
    4096 the second; truncation (2 and 7) would send token 5 to the second."""
    vb = _one_channel_head([4096, 5, 0])
    z = np.zeros_like(vb)
    cent = np.zeros((1, 2, 128), np.float32)
    cent[0, 0, 0] = 2.6 / 4096.0
    cent[0, 1, 0] = 7.6 / 4096.0
    P = orc.make_params(1, 1, 3, C_=2, T=1, rho=0.0)
    P.flags |= orc.WARM_START
    lab = orc.prepare(P, z, z, vb, init_centroids=cent)["labels"][0]
    assert lab.tolist() == [1, 0, 0]


def test_warm_start_clamp_decides_the_labels():
    """R17: scaled warm-start centroids are clamped to [-2^13, 2^13 - 1].
    Tokens 7936 and 4512 (fixed-point units; max|v| = 1.9375 gives sh = 12).  The
    warm centroid 2.5 scales to 10240 and is clamped to 8191; the other sits at
    1000.  Token 7936 joins the first (255 against 6936), token 4512 the second
    (3512 against 3679).  A clamp at 4095 would pull token 4512 to the first
    (417 against 3512)."""
    vb = _one_channel_head([7936, 4512])
    z = np.zeros_like(vb)
    cent = np.zeros((1, 2, 128), np.float32)
    cent[0, 0, 0] = 2.5
    cent[0, 1, 0] = 1000.0 / 4096.0
    P = orc.make_params(1, 1, 2, C_=2, T=1, rho=0.0)
    P.flags |= orc.WARM_START
    assert orc.prepare(P, z, z, vb, init_centroids=cent)["labels"][0].tolist() == [0, 1]


def test_fixed_point_means_round_to_nearest():
    """R8: means are exact sums of values rounded to the 2^-24 grid.  Every K
    (and V) value of channel 0 is +-1.5 * 2^-25, i.e. +-0.75 grid steps, which
    rounds to +-1 step: the K channel mean and the V block means are then
    exactly +-2^-24 (truncation would give 0)."""
    N = 256
    for sgn in (1.0, -1.0):
        x = np.zeros((N, 128), np.float64)
        x[:, 0] = sgn * 1.5 * 2.0 ** -25
        x[:, 1] = np.linspace(-1, 1, N)            # a nonzero head, ordinary values elsewhere
        xb = inputs.to_bf16_bits(x)[None, None]
        P = orc.make_params(1, 1, N, C_=1, T=1, rho=0.0)
        pr = orc.prepare(P, xb, xb, xb)
        assert pr["kbar"][0][0] == np.float32(sgn * 2.0 ** -24)
        assert np.all(pr["mu"][0][:, 0] == np.float32(sgn * 2.0 ** -24))


def test_kmeans_recovers_planted_blobs():
    rng = np.random.default_rng(3)
    N, C_ = 600, 4
    centers = rng.standard_normal((C_, 128)) * 6.0
    truth = rng.integers(0, C_, N)
    v = centers[truth] + 0.3 * rng.standard_normal((N, 128))
    vb = inputs.to_bf16_bits(v)[None, None]
    z = np.zeros_like(vb)
    # Forgy init may put two seeds in one blob; enough rounds and a seed that
    # draws one per blob make the recovery exact
    for seed in range(20):
        init = orc.kmeans_init_indices(seed, 0, N, C_)
        if len(set(truth[init].tolist())) == C_:
            break
    P = orc.make_params(1, 1, N, C_=C_, T=5, seed=seed, rho=0.0)
    lab = orc.prepare(P, z, z, vb)["labels"][0]
    # identical partition up to relabelling
    pairs = set(zip(truth.tolist(), lab.tolist()))
    assert len(pairs) == C_ and len({a for a, _ in pairs}) == C_ and len({b for _, b in pairs}) == C_


def test_kmeans_sse_non_increasing():
    q, k, v = inputs.make_custom(1, 1, 700, seed=7)
    vf = inputs.bf16_bits_to_f32(v[0, 0]).astype(np.float64)
    sse = []
    for T in range(1, 8):
        P = orc.make_params(1, 1, 700, C_=6, T=T, seed=1, rho=0.0)
        pr = orc.prepare(P, q, k, v)
        cent = pr["centroids"][0].astype(np.float64)
        sse.append(((vf - cent[pr["labels"][0]]) ** 2).sum())
    assert all(b <= a * (1 + 1e-6) for a, b in zip(sse, sse[1:]))


# --------------------------------------------------------------------------- prepare

@pytest.fixture(scope="module")
def ragged():
    """Two heads, N = 300 (two full blocks and a 44-token tail), outliers."""
    B, H, N = 1, 2, 300
    q, k, v = inputs.make_custom(B, H, N, seed=11, rate=0.03, sigma=25.0, vmean=0.3)
    P = orc.make_params(B, H, N, C_=5, T=6, seed=2, rho=0.05)
    return P, q, k, v, orc.prepare(P, q, k, v)


def test_permutation_is_stable_sort_by_label(ragged):
    P, q, k, v, pr = ragged
    for s in range(2):
        lab, perm, iperm = pr["labels"][s], pr["perm"][s], pr["iperm"][s]
        assert np.array_equal(perm, np.argsort(lab, kind="stable"))
        assert np.array_equal(iperm[perm], np.arange(P.N))


def test_k_smoothing_and_qk_codes(ragged):
    P, q, k, v, pr = ragged
    N = P.N
    for s in range(2):
        kf = inputs.bf16_bits_to_f32(k[0, s]).astype(np.float64)
        qf = inputs.bf16_bits_to_f32(q[0, s]).astype(np.float64)
        # fixed-point grid (2^-25 per term) plus one fp32 rounding of the mean
        km = kf.mean(0)
        assert np.all(np.abs(pr["kbar"][s] - km) <= np.abs(km) * 2.0 ** -24 + 2.0 ** -24)
        perm = pr["perm"][s]
        kt = (kf - pr["kbar"][s].astype(np.float64))[perm]
        qt = qf[perm]
        for name, x, sc in (("k8", kt, pr["sk"][s]), ("q8", qt, pr["sq"][s])):
            codes = pr[name][s]
            assert np.all(codes[N:] == 0)
            for b in range((N + 127) // 128):
                blk = x[b * 128:min(N, b * 128 + 128)]
                amax = np.abs(blk).max()
                assert abs(sc[b] - amax / 448) <= 1e-6 * amax / 448
                deq = orc.e4m3_decode(codes[b * 128:b * 128 + len(blk)]) * sc[b]
                # half an E4M3 ulp in the normal range, 2^-10 (code units) below it
                bound = np.abs(blk) * 2.0 ** -4 * 1.0001 + sc[b] * 2.0 ** -10 + 1e-7 * amax
                assert np.all(np.abs(deq - blk) <= bound)
                assert np.abs(orc.e4m3_decode(codes[b * 128:b * 128 + len(blk)])).max() == 448


def test_v_demean_residual_codes(ragged):
    P, q, k, v, pr = ragged
    N = P.N
    for s in range(2):
        vf = inputs.bf16_bits_to_f32(v[0, s]).astype(np.float64)[pr["perm"][s]]
        mu, sv = pr["mu"][s].astype(np.float64), pr["sv"][s].astype(np.float64)
        for b in range((N + 127) // 128):
            blk = vf[b * 128:min(N, b * 128 + 128)]
            bm = blk.mean(0)
            assert np.all(np.abs(mu[b] - bm) <= np.abs(bm) * 2.0 ** -24 + 2.0 ** -24)
            deq = mu[b] + sv * orc.e4m3_decode(pr["v8"][s][b * 128:b * 128 + len(blk)])
            bound = np.abs(blk - mu[b]) * 2.0 ** -4 * 1.001 + sv * 2.0 ** -10 + 1e-6
            assert np.all(np.abs(deq - blk) <= bound)
        resid = vf - mu[np.arange(N) // 128]
        np.testing.assert_allclose(sv, np.abs(resid).max(0) / 448, rtol=1e-6)
        np.testing.assert_allclose(pr["mup"][s], pr["mu"][s] * pr["inv"][s][None, :], rtol=1e-6)


def test_demean_removes_more_energy_after_clustering():
    """The pages report that block demeaning removes a larger share of block energy
    once tokens are sorted by cluster than in sequence order."""
    q, k, v = inputs.make_inputs(0)
    P = orc.make_params(1, 2, 1024, C_=8)
    pr = orc.prepare(P, q, k, v)
    for s in range(2):
        vf = inputs.bf16_bits_to_f32(v[0, s]).astype(np.float64)

        def removed(x):
            blocks = x.reshape(-1, 128, 128)
            return 1 - ((blocks - blocks.mean(1, keepdims=True)) ** 2).sum() / (blocks ** 2).sum()

        assert removed(vf[pr["perm"][s]]) > 2 * removed(vf)


def test_repair_set_is_topm_of_error(ragged):
    P, q, k, v, pr = ragged
    m = pr["m"]
    assert m == math.ceil(float(np.float32(P.rho)) * P.N)
    for s in range(2):
        err = pr["err"][s]
        order = np.lexsort((np.arange(P.N), -err.astype(np.float64)))
        assert np.array_equal(pr["rep_pos"][s][:m], np.sort(order[:m]))
        # criterion recomputed in fp64 from the codes
        vf = inputs.bf16_bits_to_f32(v[0, s]).astype(np.float64)[pr["perm"][s]]
        x = (vf - pr["mu"][s].astype(np.float64)[np.arange(P.N) // 128]) * pr["inv"][s]
        dl = x - orc.e4m3_decode(pr["v8"][s][:P.N])
        e64 = ((pr["sv"][s] * dl) ** 2).sum(1)
        np.testing.assert_allclose(err, e64, rtol=1e-4, atol=1e-12)
        sel = pr["rep_pos"][s][:m]
        d16 = inputs.bf16_bits_to_f32(pr["rep_delta"][s][:m]).astype(np.float64)
        # bf16 rounding, plus fp32 rounding of x = (v - mu) * inv (|x| <= 448)
        np.testing.assert_allclose(d16, dl[sel], rtol=2.0 ** -8, atol=448 * 2.0 ** -22)


def test_repair_counts_match_page_budget():
    facts, ms = _page_facts()
    for N, m in ms.items():
        P = orc.make_params(1, 1, N, rho=facts["rho"])
        assert orc.repair_count(P) == m
    assert orc.repair_count(orc.make_params(1, 1, 100, rho=0.0)) == 0
    assert orc.repair_count(orc.make_params(1, 1, 100, rho=1.0)) == 100


# --------------------------------------------------------------------------- forward

def _sim(P, q, k, v, rows=None, pcodes=False):
    pr = orc.prepare(P, q, k, v)
    BH = P.B * P.H
    rows = np.arange(P.N) if rows is None else np.asarray(rows)
    slot = np.repeat(np.arange(BH), len(rows)).astype(np.int32)
    idx = np.tile(rows, BH).astype(np.int32)
    res = orc.forward_rows(P, pr, slot, idx, want_pcodes=pcodes)
    return res, pr, slot, idx


def _dequant_v(pr, s, N, with_repair=True):
    """V in real units as the method represents it: sV * (mu' + code [+ delta]),
    mu' being the fp32 block mean in V code units."""
    mup = pr["mup"][s].astype(np.float64)[np.arange(N) // 128]
    codes = orc.e4m3_decode(pr["v8"][s][:N])
    if with_repair:
        m = pr["m"]
        codes[pr["rep_pos"][s][:m]] += inputs.bf16_bits_to_f32(pr["rep_delta"][s][:m])
    return pr["sv"][s].astype(np.float64) * (mup + codes)


@pytest.mark.parametrize("N", [300, 128, 1])
def test_zero_query_gives_mean_of_dequantised_v(N):
    """Q = 0 makes every score 0, so every code is 56+8k and the output is the plain
    mean of the dequantised V (block means restored through the row sum, tail keys
    excluded, repaired residuals included)."""
    q, k, v = inputs.make_custom(1, 2, N, seed=5, rate=0.05, vmean=0.7)
    q[:] = 0
    P = orc.make_params(1, 2, N, C_=min(4, N), T=3, rho=0.05)
    out, pr, slot, idx = _sim(P, q, k, v)
    out = out.reshape(2, N, 128)
    for s in range(2):
        want = _dequant_v(pr, s, N).mean(0)
        np.testing.assert_allclose(out[s], np.broadcast_to(want, (N, 128)), rtol=1e-12, atol=1e-12)
        vf = inputs.bf16_bits_to_f32(v[0, s]).astype(np.float64)
        assert np.abs(want - vf.mean(0)).max() < 0.02 * np.abs(vf).max()


def test_constant_keys_are_smoothed_away():
    """K rows all equal: the channel mean removes K entirely, so scores vanish and
    the output is the mean of the dequantised V whatever Q is."""
    N = 260
    q, k, v = inputs.make_custom(1, 1, N, seed=9)
    k[0, 0] = k[0, 0, 17][None, :]
    P = orc.make_params(1, 1, N, C_=3, T=2, rho=0.01)
    out, pr, _, _ = _sim(P, q, k, v)
    assert np.all(pr["k8"][0] & 0x7F == 0)
    np.testing.assert_allclose(out, np.broadcast_to(_dequant_v(pr, 0, N).mean(0), out.shape),
                               rtol=1e-12, atol=1e-12)


def test_shifting_every_key_by_one_vector_changes_nothing():
    """Softmax ignores a per-channel constant added to every key, and the method
    removes it exactly by the K channel mean.  Integer keys in [-60, 60], a
    shift of +-64 per channel (exact in bf16) and N a power of two keep the
    sums, means and K - kbar exact in fp32, so the simulated output and every
    code are bit-identical with and without the shift.  A dropped smoothing
    term, a wrong sign or a mean over the wrong axis fails it."""
    N = 256
    q, _, v = inputs.make_custom(1, 2, N, seed=14)
    rng = np.random.default_rng(15)
    kf = rng.integers(-60, 61, (1, 2, N, 128)).astype(np.float32)
    shift = rng.choice([-64.0, 64.0], (1, 2, 1, 128)).astype(np.float32)
    to_bits = lambda x: (x.view(np.uint32) >> 16).astype(np.uint16)  # noqa: E731 (exact values)
    k0, k1 = to_bits(kf), to_bits(kf + shift)
    assert np.array_equal(inputs.bf16_bits_to_f32(k1), kf + shift)
    P = orc.make_params(1, 2, N, C_=4, T=3, rho=0.02, sm_scale=0.01)
    (o0, pc0), pr0, _, _ = _sim(P, q, k0, v, pcodes=True)
    (o1, pc1), pr1, _, _ = _sim(P, q, k1, v, pcodes=True)
    assert not np.array_equal(pr0["kbar"], pr1["kbar"])
    assert np.array_equal(pr0["k8"], pr1["k8"]) and np.array_equal(pr0["sk"], pr1["sk"])
    assert np.array_equal(pc0, pc1)
    assert np.array_equal(o0, o1)


def test_zero_repair_budget_equals_repair_off():
    """rho = 0 leaves no token to repair: the same output as the repair flag off,
    bit for bit, and an empty repair set."""
    q, k, v = inputs.make_custom(1, 2, 300, seed=16, rate=0.02, sigma=20.0)
    Pa = orc.make_params(1, 2, 300, C_=4, T=3, rho=0.0)
    Pb = orc.make_params(1, 2, 300, C_=4, T=3, rho=0.3, flags=orc.VSMOOTH | orc.PERMUTE_Q)
    oa, pra, _, _ = _sim(Pa, q, k, v)
    ob, prb, _, _ = _sim(Pb, q, k, v)
    assert pra["m"] == 0 and prb["m"] == 0
    assert np.array_equal(oa, ob)


def test_row_max_code_is_bias():
    q, k, v = inputs.make_custom(1, 1, 400, seed=4)
    for tau, lo, hi in ((0.0, 120, 120), (6.0, 120, 126)):
        P = orc.make_params(1, 1, 400, C_=4, T=2, tau=tau)
        (out, pc), pr, _, _ = _sim(P, q, k, v, pcodes=True)
        mx = pc[:, :400].max(1)
        assert mx.min() >= lo and mx.max() <= hi
        assert np.all(pc[:, 400:] == 0)


def _rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


def test_simulation_tracks_exact_attention_with_uneven_block_scales():
    """With V-Smooth off (identity order) and Q/K blocks scaled by very different
    powers of two, a wrong block scale, a dropped rescale or restore, or a
    transposed operand would move the output far from exact attention."""
    B, H, N = 1, 2, 520
    q, k, v = inputs.make_custom(B, H, N, seed=21, vmean=1.5)
    qf = inputs.bf16_bits_to_f32(q).astype(np.float64)
    kf = inputs.bf16_bits_to_f32(k).astype(np.float64)
    blk = np.arange(N) // 128
    # per-block Q and K magnitudes differ by up to 4x each (alpha by up to 16x
    # between block pairs) while logits keep a std between 1/8 and 2
    mq = 2.0 ** np.array([-1, 1, 0, 1, -1])[blk]
    mk = 2.0 ** np.array([1, -1, 0, 1, -1])[blk]
    q = inputs.to_bf16_bits(qf * mq[None, None, :, None] * 0.5)
    k = inputs.to_bf16_bits(kf * mk[None, None, :, None] + 2.0)
    for flags in (orc.REPAIR, orc.DEFAULT_FLAGS):
        P = orc.make_params(B, H, N, C_=4, T=3, rho=0.01, flags=flags)
        out, pr, slot, idx = _sim(P, q, k, v)
        ex = orc.exact_rows(P, q, k, v, slot, idx)
        assert _rel(out, ex) < 0.08


def test_vsmooth_and_tau_variants_agree_with_exact():
    q, k, v = inputs.make_inputs(0)
    rows = np.arange(0, 1024, 3)
    res = {}
    for name, kw in dict(full={}, tau6=dict(tau=6.0), k0=dict(expcast_k=0),
                         off=dict(flags=0), noq=dict(flags=orc.VSMOOTH | orc.REPAIR)).items():
        P = orc.make_params(1, 2, 1024, C_=8, **kw)
        out, pr, slot, idx = _sim(P, q, k, v, rows=rows)
        res[name] = out
    ex = orc.exact_rows(P, q, k, v, slot, idx)
    for name, out in res.items():
        assert _rel(out, ex) < 0.08, name
    # tau only changes the P codes (same Q/K/V codes), so the two stay close
    assert _rel(res["tau6"], res["full"]) < 0.03


def test_repair_moves_output_toward_unquantised_v():
    """Raising rho corrects more residual error: with rho = 1 the V used by the
    simulation equals the bf16-rounded residual, so its distance to exact V-side
    arithmetic shrinks."""
    q, k, v = inputs.make_custom(1, 1, 384, seed=8, rate=0.05, sigma=40)
    errs = []
    for rho in (0.0, 0.05, 1.0):
        P = orc.make_params(1, 1, 384, C_=4, T=3, rho=rho)
        pr = orc.prepare(P, q, k, v)
        vf = inputs.bf16_bits_to_f32(v[0, 0]).astype(np.float64)[pr["perm"][0]]
        errs.append(np.linalg.norm(_dequant_v(pr, 0, 384) - vf))
    assert errs[0] > errs[1] > errs[2] and errs[2] < 1e-2 * errs[0]


# --------------------------------------------------------------------------- exact

def test_exact_matches_torch_sdpa_fp64():
    q, k, v = inputs.make_custom(1, 2, 150, seed=13)
    P = orc.make_params(1, 2, 150)
    slot = np.repeat([0, 1], 150)
    idx = np.tile(np.arange(150), 2)
    ours = orc.exact_rows(P, q, k, v, slot, idx).reshape(1, 2, 150, 128)
    t = [torch.from_numpy(inputs.bf16_bits_to_f32(x).astype(np.float64)) for x in (q, k, v)]
    # the oracle's scale is the fp32 parameter 1/sqrt(128) rounded to fp32
    scale = float(np.float32(1.0 / math.sqrt(128)))
    ref = torch.nn.functional.scaled_dot_product_attention(*t, scale=scale).numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-10, atol=1e-12)


def test_exact_invariant_to_joint_kv_permutation():
    """Permuting K and V together leaves non-causal attention unchanged; permuting Q
    as well permutes the output rows."""
    q, k, v = inputs.make_custom(1, 1, 200, seed=17)
    perm = np.random.default_rng(1).permutation(200)
    P = orc.make_params(1, 1, 200)
    rows = np.arange(200)
    base = orc.exact_rows(P, q, k, v, np.zeros(200), rows)
    kp, vp, qp = (np.ascontiguousarray(t[:, :, perm]) for t in (k, v, q))
    np.testing.assert_allclose(orc.exact_rows(P, q, kp, vp, np.zeros(200), rows), base,
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(orc.exact_rows(P, qp, kp, vp, np.zeros(200), rows), base[perm],
                               rtol=1e-12, atol=1e-14)


def test_restore_returns_block_means_through_row_sums():
    """V-Smooth's Restore (noticiai.com.br article, section V-Smooth: the block
    mean comes back through the row sum online softmax already keeps), checked
    against the P.V path of the same simulation.  With one cluster the order is
    the identity, so V-Smooth on and off give the same Q/K codes and the same
    ExpCast weights.  V = block indicator (channel c is 1 on the tokens of block
    c): with V-Smooth off its E4M3 codes are exact and P.V returns the weight
    w_b of each block (ragged tail included); with V-Smooth on every residual
    code is 0 and only Restore (row sum times block mean) can return it.  The
    two must agree, sum to 1, and any other block-constant V must give
    sum_b w_b mu_b.  A dropped restore term, a mean added without its row sum,
    or a rescale missing from the restore accumulator breaks the agreement."""
    N = 300
    nb = 3
    q, k, _ = inputs.make_custom(1, 1, N, seed=12)
    blk = np.arange(N) // 128
    ind = np.zeros((N, 128), np.float32)
    ind[np.arange(N), blk] = 1.75  # 448 * 2^-8: scale 2^-8, code 448, both exact
    rows = np.arange(N, dtype=np.int32)

    def run(vf, flags):
        v = inputs.to_bf16_bits(vf).reshape(1, 1, N, 128)
        P = orc.make_params(1, 1, N, C_=1, T=2, flags=flags)
        (out, pc), pr, _, _ = _sim(P, q, k, v, rows=rows, pcodes=True)
        return out, pc, pr

    w_pv, pc_off, pr_off = run(ind, orc.PERMUTE_Q)
    w_rs, pc_on, pr_on = run(ind, orc.VSMOOTH | orc.PERMUTE_Q)
    w_pv, w_rs = w_pv / 1.75, w_rs / 1.75
    np.testing.assert_array_equal(pc_on, pc_off)
    assert np.all(pr_on["v8"] == 0) and np.array_equal(pr_on["perm"][0], np.arange(N))
    np.testing.assert_allclose(pr_off["sv"][0][:nb] * orc.e4m3_decode(pr_off["v8"][0][:N, :nb]),
                               ind[:, :nb], rtol=0, atol=0)  # indicator codes are exact
    np.testing.assert_allclose(w_rs, w_pv, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(w_pv[:, :nb].sum(1), 1.0, rtol=1e-12)
    assert np.all(w_pv[:, nb:] == 0) and np.all(w_pv[:, :nb] > 0)
    vf = closed_form.block_constant_values(N, seed=3)
    out, _, _ = run(vf, orc.VSMOOTH | orc.PERMUTE_Q)
    mu = vf[[0, 128, 256]].astype(np.float64)
    np.testing.assert_allclose(out, w_pv[:, :nb] @ mu, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("jump,tau", [(8, 0.0), (16, 0.0), (8, 6.0)])
def test_online_rescale_closed_form(jump, tau):
    """Two key blocks, the second raising the row maximum by exactly `jump` code
    units: the running sums are rescaled by 2^(-jump/8) and every code stays at
    56 + 8k, so the output is (r mu0 + mu1)/(r + 1) = u + w exactly (worked out
    in tests/closed_form.py).  A wrong base or divisor in the rescale, a missing
    rescale of l or of the accumulator, or M moved after the block's codes
    changes the result."""
    q, k, v, row, want = closed_form.rescale_case(jump, seed=jump)
    q, k, v = (inputs.to_bf16_bits(x) for x in (q, k, v))
    P = orc.make_params(1, 1, 256, C_=1, T=2, tau=tau, sm_scale=closed_form.unit_gain_scale())
    (out, pc), pr, _, _ = _sim(P, q, k, v, rows=[row], pcodes=True)
    assert np.all(pc[0] == 120)
    np.testing.assert_array_equal(out[0], want)
    ex = orc.exact_rows(P, q, k, v, np.zeros(1), np.array([row]))
    np.testing.assert_allclose(ex[0], want, rtol=1e-6, atol=1e-6)


def test_repair_restores_coherent_residuals_with_their_own_block_scales():
    """R14: repaired keys are coded with their own block's scale.  V is 17/32
    everywhere but one token at 1 (which sets each channel's scale), so every
    other value lands 2 code units from its E4M3 code, the same error on every
    key; K's second block is 8x larger, so its keys dominate the softmax.
    Without repair the output is off by 0.8%; repairing every key (rho = 1)
    restores V and the output equals exact attention to 1e-5.  A repaired key
    coded with another block's scale would weight its correction wrongly."""
    N = 384
    rng = np.random.default_rng(5)
    q = rng.standard_normal((N, 128))
    k = rng.standard_normal((N, 128))
    k[128:256] *= 8.0
    k[256:] /= 8.0
    v = np.full((N, 128), 17.0 / 32.0)
    v[17, :] = 1.0
    rows = np.arange(0, N, 3).astype(np.int32)
    # plain, and with smoothed queries around a query mean offset of 2 (R20:
    # repaired keys then carry the per-key score term too)
    for extra, qoff in ((0, 0.0), (orc.SMOOTH_Q, 2.0)):
        qb, kb, vb = (inputs.to_bf16_bits(x)[None, None] for x in (q + qoff, k, v))
        rel = {}
        for rho in (0.0, 1.0):
            P = orc.make_params(1, 1, N, C_=1, T=1, rho=rho, sm_scale=0.2)
            P.flags = orc.REPAIR | orc.PERMUTE_Q | extra  # V-Smooth off: the residual codes carry V
            pr = orc.prepare(P, qb, kb, vb)
            out = orc.forward_rows(P, pr, np.zeros(len(rows), np.int32), rows)
            ex = orc.exact_rows(P, qb, kb, vb, np.zeros(len(rows), np.int32), rows)
            rel[rho] = np.linalg.norm(out - ex) / np.linalg.norm(ex)
        assert rel[0.0] > 5e-3 and rel[1.0] < 1e-5, (extra, rel)


def test_lazy_maximum_closed_form():
    """R11 with tau = 6: block 1's maximum exceeds block 0's by 4 code units,
    within the slack, so M stays, block 1's codes are 124 and the output is
    0.4 mu0 + 0.6 mu1 (tests/closed_form.py).  With tau = 0 the same inputs move
    M and give codes of 120 in both blocks."""
    q, k, v, row, want = closed_form.lazy_max_case(seed=3)
    q, k, v = (inputs.to_bf16_bits(x) for x in (q, k, v))
    P = orc.make_params(1, 1, 256, C_=1, T=2, tau=6.0, sm_scale=closed_form.unit_gain_scale())
    (out, pc), pr, _, _ = _sim(P, q, k, v, rows=[row], pcodes=True)
    assert np.all(pc[0][:128] == 120) and np.all(pc[0][128:] == 124)
    np.testing.assert_allclose(out[0], want, rtol=1e-12, atol=1e-12)
    P0 = orc.make_params(1, 1, 256, C_=1, T=2, tau=0.0, sm_scale=closed_form.unit_gain_scale())
    (out0, pc0), _, _, _ = _sim(P0, q, k, v, rows=[row], pcodes=True)
    assert np.all(pc0[0] == 120)


def test_online_equals_two_pass_when_the_maximum_never_moves():
    """Rows whose largest score lies in the first key block never move M after
    that block, so the online loop must give the codes of the two-pass
    softmax: the row maximum over all keys first, then every code from it."""
    N = 700
    q, k, v = inputs.make_custom(1, 1, N, seed=19)
    P = orc.make_params(1, 1, N, C_=4, T=3)
    (out, pc), pr, _, _ = _sim(P, q, k, v, pcodes=True)
    c0 = orc.code_gain(0.0)
    k8 = pr["k8"][0][:N]
    checked = 0
    blk = np.arange(N) // 128
    nb = blk[-1] + 1
    for row in range(0, N, 3):
        pos = pr["iperm"][0][row]
        s = orc.scores(np.repeat(pr["q8"][0][pos][None], N, 0), k8, exact=True)
        alpha = (pr["sq"][0][pos // 128] * pr["sk"][0][blk]).astype(np.float32) * c0
        # block maxima in code units as the loop forms them: max raw score times
        # the block's alpha (alpha > 0), one fp32 product
        tb = np.array([np.float32(s[blk == b].max() * alpha[blk == b][0]) for b in range(nb)])
        if np.any(tb[1:] > tb[0]):
            continue
        beta = np.float32(np.float32(120.0) - tb[0])
        two_pass = np.concatenate([orc.expcast(s[blk == b], float(alpha[blk == b][0]), float(beta))
                                   for b in range(nb)])
        np.testing.assert_array_equal(pc[row][:N], two_pass)
        checked += 1
    assert checked >= 10


# ------------------------------------------------------------------ warm start

def _cold(P, q, k, v):
    pr = orc.prepare(P, q, k, v)
    return pr["labels"].copy(), pr["centroids"].copy()


def test_warm_start_from_forgy_centroids_equals_cold_start():
    """Starting the Lloyd rounds from the seeded Forgy draw (given as centroids)
    reproduces the cold start exactly."""
    q, k, v = inputs.make_custom(1, 2, 300, seed=11)
    Pc = orc.make_params(1, 2, 300, C_=5, T=4)
    lab, cen = _cold(Pc, q, k, v)
    vf = inputs.bf16_bits_to_f32(v).reshape(2, 300, 128)
    init = np.stack([vf[h][orc.kmeans_init_indices(0, h, 300, 5)] for h in range(2)])
    sh = [orc.kmeans_shift(vf[h]) for h in range(2)]
    # centroids as the oracle stores them: integers at 2^-sh
    init = np.stack([np.ldexp(np.rint(np.ldexp(init[h].astype(np.float64), sh[h])), -sh[h])
                     for h in range(2)]).astype(np.float32)
    Pw = orc.make_params(1, 2, 300, C_=5, T=4, flags=orc.DEFAULT_FLAGS | orc.WARM_START)
    pr = orc.prepare(Pw, q, k, v, init_centroids=init)
    np.testing.assert_array_equal(pr["labels"], lab)
    np.testing.assert_array_equal(pr["centroids"], cen)


def test_converged_centroids_are_a_fixed_point_of_warm_start():
    """Lloyd's fixed point: from converged centroids one more round changes
    neither labels nor centroids."""
    q, k, v = inputs.make_custom(1, 1, 400, seed=12)
    lab60, cen60 = _cold(orc.make_params(1, 1, 400, C_=4, T=60), q, k, v)
    lab61, cen61 = _cold(orc.make_params(1, 1, 400, C_=4, T=61), q, k, v)
    np.testing.assert_array_equal(lab60, lab61)   # converged
    Pw = orc.make_params(1, 1, 400, C_=4, T=1, flags=orc.DEFAULT_FLAGS | orc.WARM_START)
    pr = orc.prepare(Pw, q, k, v, init_centroids=cen60)
    np.testing.assert_array_equal(pr["labels"], lab60)
    np.testing.assert_array_equal(pr["centroids"], cen60)


def test_warm_start_after_drift_keeps_sse_low():
    """After a small drift, three warm rounds reach a within-cluster energy no
    worse than ten cold rounds from the seeded draw (within 2%)."""
    q, k, v = inputs.make_custom(1, 1, 600, seed=13)
    _, cen = _cold(orc.make_params(1, 1, 600, C_=6, T=10), q, k, v)
    v1 = inputs.drift(v, step=1, seed=13)
    Pw = orc.make_params(1, 1, 600, C_=6, T=3, flags=orc.DEFAULT_FLAGS | orc.WARM_START)
    prw = orc.prepare(Pw, q, k, v1, init_centroids=cen)
    prc = orc.prepare(orc.make_params(1, 1, 600, C_=6, T=10), q, k, v1)
    vf = inputs.bf16_bits_to_f32(v1).reshape(600, 128).astype(np.float64)

    def sse(pr):
        c = pr["centroids"][0].astype(np.float64)
        return float(np.sum((vf - c[pr["labels"][0]]) ** 2))
    assert sse(prw) <= 1.02 * sse(prc), (sse(prw), sse(prc))


def test_warm_start_clamps_to_fourteen_bits():
    """Centroids far outside the current value range are clamped to the 14-bit
    fixed-point range instead of wrapping."""
    q, k, v = inputs.make_custom(1, 1, 200, seed=14)
    init = np.full((1, 3, 128), 1.0e6, np.float32)
    init[0, 1] = -1.0e6
    init[0, 2] = 0.0
    Pw = orc.make_params(1, 1, 200, C_=3, T=1, flags=orc.DEFAULT_FLAGS | orc.WARM_START)
    pr = orc.prepare(Pw, q, k, v, init_centroids=init)
    vf = inputs.bf16_bits_to_f32(v).reshape(200, 128)
    sh = orc.kmeans_shift(vf)
    # every token is nearest to the zero centroid or to a clamped corner; the
    # clamped corners sit at +-(2^13 - 1) or -2^13 in fixed point
    assert set(np.unique(pr["labels"])) <= {0, 1, 2}
    assert np.all(np.isfinite(pr["centroids"]))
    assert np.max(np.abs(np.ldexp(pr["centroids"].astype(np.float64), sh))) <= 8192
