"""Shared helpers of the GPU parity tests: run the library through its C ABI and
read the prepared workspace back in the oracle's natural layouts."""
from __future__ import annotations

import math
import sys

import numpy as np

import precision_fp8_attention_amd as vc
from oracle import oracle as orc

ATOL = 1e-2   # max-abs bound on O against the oracle's simulation
RTOL_L2 = 5e-3  # relative-L2 bound on O against the oracle's simulation


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def lib_params(B, H, N, C_, T=10, seed=0, rho=0.005, expcast_k=8, tau=0.0, flags=vc.DEFAULT_FLAGS,
               sm_scale=0.0):
    return vc.default_params(B, H, N, n_clusters=C_, kmeans_iters=T, seed=seed, rho=rho,
                             expcast_k=expcast_k, tau=tau, flags=flags, sm_scale=sm_scale)


def exact_mode(p) -> bool:
    """Whether the library computes this call's scores exactly (bf16 MFMA) or on
    the FP8 MFMA: the score flag, else the token count."""
    if p.flags & vc.EXACT_SCORES:
        return True
    if p.flags & vc.FP8_SCORES:
        return False
    return p.N < vc.FP8_SCORES_MIN_TOKENS


def oracle_params(p, diagnostic_rule=False) -> orc.Params:
    """The oracle's parameters for a library call.  The reference scores are
    always the exact dot product; diagnostic_rule selects the probe-fitted FP8
    instruction model instead (only to explain code differences)."""
    flags = p.flags & (vc.VSMOOTH | vc.REPAIR | vc.PERMUTE_Q | vc.WARM_START | vc.V4 | vc.SMOOTH_Q)
    return orc.make_params(p.B, p.H, p.N, C_=p.n_clusters, T=p.kmeans_iters, seed=p.seed,
                           rho=p.rho, sm_scale=p.sm_scale, expcast_k=p.expcast_k, tau=p.tau,
                           flags=flags | (orc.MFMA_RULE if diagnostic_rule else 0))


def to_device(q, k, v):
    import torch
    return [torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() for x in (q, k, v)]


def run(p, qd, kd, vd, ws=None):
    """prepare + forward on the current stream; returns (workspace, output)."""
    import torch
    if ws is None:
        ws = vc.alloc_workspace(p)
    o = torch.empty_like(qd)
    vc.prepare(p, qd, kd, vd, ws)
    vc.forward(p, ws, o)
    torch.cuda.synchronize()
    return ws, o


def out_f64(o) -> np.ndarray:
    import torch
    return o.float().cpu().numpy().astype(np.float64)


def _v_col(r):
    return 32 * ((r & 15) >> 2) + 4 * (r >> 4) + (r & 3)


def _v4_byte(k):
    """Byte of key k's E2M1 code in its block's 64-byte channel row (low nibble
    for even k): key order."""
    return k >> 1


def v4_krow(r):
    """With the 4-bit residual, row r of a block's K codes holds the key at block
    position v4_krow(r) (bits 2-3 and 4-5 of r swapped; its own inverse)."""
    return (r & 0x43) | ((r >> 2) & 0x0C) | ((r << 2) & 0x30)


def _rep_col(s):
    return 32 * (s >> 5) + 8 * ((s >> 2) & 3) + 4 * ((s >> 4) & 1) + (s & 3)


def read_prepared(p, ws, heads) -> dict:
    """Workspace arrays of the given global heads, in the oracle's layouts."""
    L = vc.workspace_layout(p)
    host = ws.cpu().numpy()
    BH, N = p.B * p.H, p.N
    nblk = (N + 127) // 128
    npad = nblk * 128
    m = orc.repair_count(oracle_params(p))
    mpad = ((m + 127) // 128) * 128
    C_ = p.n_clusters
    heads = np.asarray(heads)

    def arr(name, dtype, shape):
        n = int(np.prod(shape)) * np.dtype(dtype).itemsize
        return host[L[name]:L[name] + n].view(dtype).reshape(shape)[heads]

    out = dict(
        labels=arr("labels", np.int32, (BH, N)), perm=arr("perm", np.int32, (BH, N)),
        iperm=arr("iperm", np.int32, (BH, N)), centroids=arr("centroids", np.float32, (BH, C_, 128)),
        kbar=arr("kbar", np.float32, (BH, 128)), q8=arr("q8", np.uint8, (BH, npad, 128)),
        k8=arr("k8", np.uint8, (BH, npad, 128)), sq=arr("sq", np.float32, (BH, nblk)),
        sk=arr("sk", np.float32, (BH, nblk)), mu=arr("mu", np.float32, (BH, nblk, 128)),
        mup=arr("mup", np.float32, (BH, nblk, 128)), sv=arr("sv", np.float32, (BH, 128)),
        inv=arr("inv", np.float32, (BH, 128)), err=arr("err", np.float32, (BH, N)))
    if p.flags & vc.V4:
        # K code rows back in position order
        rows = (np.arange(npad) // 128) * 128 + v4_krow(np.arange(npad) % 128)
        out["k8"] = np.ascontiguousarray(out["k8"][:, rows])
        # codes as one byte per (position, channel), exponents [nblk][4][128]
        t = arr("v4t", np.uint8, (BH, nblk, 128, 64))
        k = np.arange(128)
        by = t[:, :, :, _v4_byte(k)]                      # [h][b][c][k]
        codes = (by >> (4 * (k & 1)).astype(np.uint8)) & 15
        out["v8"] = np.ascontiguousarray(codes.transpose(0, 1, 3, 2).reshape(len(heads), npad, 128))
        rec = host[L["v4s"]:L["v4s"] + BH * nblk * 512].reshape(BH, nblk, 4, 16, 8)[heads]
        c = np.arange(128)
        out["vexp"] = (rec[:, :, :, c & 15, c >> 4].astype(np.int16) - 127).astype(np.int8)
    else:
        v8t = arr("v8t", np.uint8, (BH, 128, npad))
        cols = (np.arange(npad) // 128) * 128 + _v_col(np.arange(npad) % 128)
        out["v8"] = np.ascontiguousarray(v8t[:, :, cols].transpose(0, 2, 1))
    if p.flags & vc.SMOOTH_Q:
        out["qbar"] = arr("qbar", np.float32, (BH, nblk, 128))
        out["qbias"] = arr("qbias", np.float32, (BH, nblk, npad))
    if m > 0:
        out["rep_pos"] = arr("rep_pos", np.int32, (BH, mpad))[:, :m]
        dt = arr("rep_dt", np.uint16, (BH, 128, mpad))
        s = np.arange(m)
        rc = (s // 128) * 128 + _rep_col(s % 128)
        out["rep_delta"] = np.ascontiguousarray(dt[:, :, rc].transpose(0, 2, 1))
    out["m"] = m
    return out


EXACT_KEYS = ("labels", "perm", "iperm", "centroids", "kbar", "q8", "k8", "sq", "sk", "mu", "mup",
              "sv", "inv", "v8", "err", "rep_pos", "rep_delta")


def compare_prepared(gpu: dict, ora: dict, vsmooth: bool) -> list[str]:
    """Names of arrays that are not bit-identical (with mismatch counts)."""
    bad = []
    m = gpu["m"]
    keys = EXACT_KEYS + tuple(k for k in ("vexp", "qbar", "qbias") if k in gpu)
    for key in keys:
        if key in ("labels", "centroids") and not vsmooth:
            continue
        if key in ("rep_pos", "rep_delta"):
            if m == 0:
                continue
            a, b = gpu[key], ora[key][:, :m]
        else:
            a, b = gpu[key], ora[key]
        a = np.ascontiguousarray(a)
        b = np.ascontiguousarray(b)
        if a.dtype.kind == "f":
            a, b = a.view(np.uint32), b.view(np.uint32)
        if a.shape != b.shape:
            bad.append(f"{key}: shape {a.shape} vs {b.shape}")
        elif not np.array_equal(a, b):
            bad.append(f"{key}: {int(np.sum(a != b))} of {a.size} differ")
    return bad


def rel_l2(a, b) -> float:
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def sample_rows(N: int, n: int, seed: int = 0) -> np.ndarray:
    """n rows spread over [0, N), always including the first and last row."""
    if n >= N:
        return np.arange(N, dtype=np.int32)
    rng = np.random.default_rng(seed)
    r = np.unique(np.concatenate([[0, N - 1], rng.choice(N, n - 2, replace=False)]))
    return r.astype(np.int32)


BF16_HALF_STEP = 2.0 ** -8  # bf16 rounding of x moves it by at most 2^-8 |x|


def check_output(p, q, k, v, o_gpu, heads, rows, prep_oracle=None, label="", bf16_step=False):
    """Compare GPU output rows with the oracle's simulation (exact scores) and
    report the distance to exact fp64 attention.

    Bar: max-abs 1e-2 and relative L2 5e-3.  O is returned in bf16, whose
    rounding alone moves it by up to 2^-8 |O|: above |O| ~ 2.5 that exceeds the
    max-abs bar by itself, so with bf16_step the max-abs bar applies to what lies
    beyond that rounding.  With FP8 scores on fewer than FP8_SCORES_MIN_TOKENS
    keys (only when forced) one ExpCast code one step off the exact score's code
    can move a row by more than the max-abs bar (1/8 of the key's share of the
    row sum times |V|), so there only the relative-L2 bar is asserted and
    max-abs is reported."""
    P = oracle_params(p)
    if prep_oracle is None:
        prep_oracle = orc.prepare(P, q, k, v, heads=heads)
    slots = np.repeat(np.arange(len(heads)), len(rows)).astype(np.int32)
    idx = np.tile(rows, len(heads)).astype(np.int32)
    sim = orc.forward_rows(P, prep_oracle, slots, idx)
    ghead = np.asarray(heads)[slots]
    og = out_f64(o_gpu).reshape(p.B * p.H, p.N, 128)[ghead, idx]
    ex = orc.exact_rows(P, q, k, v, ghead, idx)
    exact = exact_mode(p)
    res = dict(scores="exact" if exact else "fp8", max_abs=float(np.max(np.abs(og - sim))),
               rel_l2=rel_l2(og, sim), rel_l2_exact=rel_l2(og, ex), sim_rel_l2_exact=rel_l2(sim, ex),
               max_abs_beyond_bf16=float(np.max(np.abs(og - sim) - BF16_HALF_STEP * np.abs(sim))))
    log(f"{label} output vs oracle: {res}")
    assert np.all(np.isfinite(og))
    if exact or p.N >= vc.FP8_SCORES_MIN_TOKENS:
        assert (res["max_abs_beyond_bf16"] if bf16_step else res["max_abs"]) <= ATOL, res
    assert res["rel_l2"] <= RTOL_L2, res
    return res


CODE_EPS = 0.01  # code units: FP8-score codes may differ only this close to a rounding boundary


def compare_pcodes(got, ref, pvals, label, exact, min_agree=0.999):
    """GPU ExpCast bytes against the exact-score oracle's codes for the same
    (query, key).  Exact scores: bit-exact.  FP8 scores: the FP8 MFMA's sum
    differs from the exact one in the low bits only (under 2.5e-3 code units on
    the workloads in the diagnostic model of the instruction), so a code may
    differ only by one step and only where the exact fp32 value lies within
    CODE_EPS of the rounding boundary between the two codes; at most 1 - min_agree
    of the codes differ.  Returns (differing, total)."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    bad = got != ref
    nbad, total = int(bad.sum()), got.size
    log(f"pcodes {label}: {nbad} of {total} codes differ from the exact-score oracle "
        f"(agreement {1 - nbad / max(total, 1):.6f})")
    if exact:
        assert nbad == 0, f"{label}: {nbad} of {total} P codes differ from the oracle"
        return nbad, total
    assert nbad <= (1 - min_agree) * total, (label, nbad, total)
    if nbad:
        g, r = got[bad].astype(int), ref[bad].astype(int)
        assert np.all(np.abs(g - r) == 1), (label, g[:8], r[:8])
        boundary = np.minimum(g, r) + 0.5
        dist = np.abs(pvals[bad].astype(np.float64) - boundary)
        log(f"pcodes {label}: largest distance of a differing code's exact value to its "
            f"rounding boundary {dist.max():.2e} code units")
        assert np.all(dist <= CODE_EPS), (label, dist.max())
    return nbad, total
