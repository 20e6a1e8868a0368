"""ctypes front end of the CPU oracle for VC-Attention FP8.

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product library never does, and
this module never touches the product library.

The arithmetic lives in vc_oracle.c (plain C, fp64 accumulation, explicit fp32
fma where the method's decisions are taken in fp32).  This file only marshals
numpy arrays and builds the shared object with gcc when it is missing.
"""
from __future__ import annotations

import ctypes as C
import math
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "vc_oracle.c")
LIB = os.path.join(HERE, "libvcoracle.so")
# Test hook: a prebuilt variant of the oracle to load instead (the mutation
# test plants one mistake per build and checks that the pins catch it).
LIB_OVERRIDE = os.environ.get("VC_ORACLE_LIB")

# Flag bits of the oracle's own parameter block (the same meaning as the
# library's public flags, defined here independently).
VSMOOTH = 1
REPAIR = 2
PERMUTE_Q = 4
WARM_START = 32
V4 = 64
SMOOTH_Q = 128
# Diagnostic only: raw scores by the probe-fitted model of gfx950's FP8 matrix
# instruction instead of the exact dot product (the reference reading).
MFMA_RULE = 256
DEFAULT_FLAGS = VSMOOTH | REPAIR | PERMUTE_Q


def build(force: bool = True) -> str:
    """Compile vc_oracle.c into libvcoracle.so (gcc, OpenMP, no fp contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-mfma", "-fPIC", "-shared",
               "-Wall", SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


class Params(C.Structure):
    _fields_ = [("B", C.c_int32), ("H", C.c_int32), ("N", C.c_int32), ("d", C.c_int32),
                ("C", C.c_int32), ("T", C.c_int32), ("seed", C.c_uint64), ("rho", C.c_float),
                ("sm_scale", C.c_float), ("expcast_k", C.c_int32), ("tau", C.c_float),
                ("flags", C.c_uint32)]


class _Prep(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "labels", "perm", "iperm", "centroids", "kbar", "q8", "k8", "sq", "sk", "mu", "mup",
        "v8", "sv", "inv", "err", "rep_pos", "rep_delta", "vexp", "qbar", "qbias")] + [("mcap", C.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if LIB_OVERRIDE:
            L = C.CDLL(LIB_OVERRIDE)
        else:
            build(force=False)
            L = C.CDLL(LIB)
        vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        L.oc_prepare.argtypes = [C.POINTER(Params), vp, vp, vp, vp, i32, C.POINTER(_Prep)]
        L.oc_forward_rows.argtypes = [C.POINTER(Params), C.POINTER(_Prep), vp, vp, i32, vp, vp, vp]
        L.oc_exact_rows.argtypes = [C.POINTER(Params), vp, vp, vp, vp, vp, i32, vp]
        L.oc_e4m3_decode_array.argtypes = [vp, vp, i64]
        L.oc_e4m3_encode_array.argtypes = [vp, vp, i64]
        L.oc_expcast_array.argtypes = [vp, C.c_float, C.c_float, vp, i64]
        L.oc_splitmix64_array.argtypes = [C.c_uint64, vp, i64]
        L.oc_e2m1_decode_array.argtypes = [vp, vp, i64]
        L.oc_e2m1_encode_array.argtypes = [vp, vp, i64]
        L.oc_mx_exponent_array.argtypes = [vp, vp, i64]
        L.oc_score_array.argtypes = [vp, vp, i64, i32, i32, vp]
        L.oc_kmeans_init_indices.argtypes = [C.c_uint64, i64, i32, i32, vp]
        L.oc_kmeans_shift.argtypes = [vp, i64]
        L.oc_kmeans_shift.restype = C.c_int
        L.oc_repair_count.argtypes = [C.POINTER(Params)]
        L.oc_repair_count.restype = i32
        for f in (L.oc_prepare, L.oc_forward_rows, L.oc_exact_rows):
            f.restype = C.c_int
        _lib = L
    return _lib


def make_params(B, H, N, C_=8, T=10, seed=0, rho=0.005, sm_scale=0.0, expcast_k=8, tau=0.0,
                flags=DEFAULT_FLAGS, d=128) -> Params:
    return Params(B, H, N, d, C_, T, seed, rho, sm_scale, expcast_k, tau, flags)


def _ptr(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(C.c_void_p)


def repair_count(P: Params) -> int:
    return int(lib().oc_repair_count(C.byref(P)))


def prepare(P: Params, q, k, v, heads=None, init_centroids=None) -> dict:
    """Run the prepare stage on the listed global heads (default: all).

    q, k, v are uint16 bf16 bit arrays [B, H, N, 128].  Returns a dict of numpy
    arrays whose first axis is the slot (position in `heads`).  init_centroids
    (fp32 [nheads, C, 128]) are the starting centroids when P has WARM_START."""
    B, H, N, d = P.B, P.H, P.N, P.d
    heads = np.arange(B * H, dtype=np.int32) if heads is None else np.asarray(heads, np.int32)
    if heads.ndim != 1 or np.any(heads < 0) or np.any(heads >= B * H):
        raise ValueError(f"heads must be global head indices in [0, {B * H})")
    for t in (q, k, v):
        if tuple(np.shape(t)) != (B, H, N, d):
            raise ValueError(f"inputs must have shape {(B, H, N, d)}, got {np.shape(t)}")
    nh = len(heads)
    nblk = (N + 127) // 128
    npad = nblk * 128
    m = repair_count(P)
    mcap = max(m, 1)
    out = dict(
        labels=np.zeros((nh, N), np.int32), perm=np.zeros((nh, N), np.int32),
        iperm=np.zeros((nh, N), np.int32), centroids=np.zeros((nh, P.C, d), np.float32),
        kbar=np.zeros((nh, d), np.float32), q8=np.zeros((nh, npad, d), np.uint8),
        k8=np.zeros((nh, npad, d), np.uint8), sq=np.zeros((nh, nblk), np.float32),
        sk=np.zeros((nh, nblk), np.float32), mu=np.zeros((nh, nblk, d), np.float32),
        mup=np.zeros((nh, nblk, d), np.float32), v8=np.zeros((nh, npad, d), np.uint8),
        sv=np.zeros((nh, d), np.float32), inv=np.zeros((nh, d), np.float32),
        err=np.zeros((nh, N), np.float32), rep_pos=np.zeros((nh, mcap), np.int32),
        rep_delta=np.zeros((nh, mcap, d), np.uint16), vexp=np.zeros((nh, nblk, 4, d), np.int8),
        qbar=np.zeros((nh, nblk, d), np.float32),
        qbias=np.zeros((nh, nblk, npad) if P.flags & SMOOTH_Q else (nh, 1, 1), np.float32))
    if P.flags & WARM_START:
        if init_centroids is None:
            raise ValueError("WARM_START needs init_centroids")
        out["centroids"][...] = np.asarray(init_centroids, np.float32).reshape(nh, P.C, d)
    pr = _Prep(*[out[n].ctypes.data for n, _ in _Prep._fields_[:-1]], mcap)
    q, k, v = (np.ascontiguousarray(t) for t in (q, k, v))
    rc = lib().oc_prepare(C.byref(P), _ptr(q), _ptr(k), _ptr(v), _ptr(heads), nh, C.byref(pr))
    if rc != 0:
        raise ValueError(f"oracle prepare rejected the parameters (code {rc})")
    out["heads"] = heads
    out["m"] = m
    out["_struct"] = pr
    return out


def forward_rows(P: Params, prep: dict, row_slot, row_index, want_pcodes=False, want_pvals=False):
    """Simulated outputs (fp64 [n, 128]) of query rows given in ORIGINAL order.

    want_pcodes adds the rows' ExpCast codes (uint8 [n, Npad], key position
    order); want_pvals adds the fp32 values those codes round (-inf past N).
    Returns out, or a tuple (out, pcodes?, pvals?) in that order."""
    row_slot = np.ascontiguousarray(row_slot, np.int32)
    row_index = np.ascontiguousarray(row_index, np.int32)
    n = len(row_index)
    out = np.zeros((n, P.d), np.float64)
    npad = ((P.N + 127) // 128) * 128
    pc = np.zeros((n, npad), np.uint8) if want_pcodes else None
    pv = np.zeros((n, npad), np.float32) if want_pvals else None
    rc = lib().oc_forward_rows(C.byref(P), C.byref(prep["_struct"]), _ptr(row_slot),
                               _ptr(row_index), n, _ptr(out), _ptr(pc) if want_pcodes else None,
                               _ptr(pv) if want_pvals else None)
    if rc != 0:
        raise ValueError("oracle forward rejected the parameters")
    extra = tuple(x for x in (pc, pv) if x is not None)
    return (out, *extra) if extra else out


def exact_rows(P: Params, q, k, v, row_head, row_index):
    """Exact fp64 softmax attention rows (row_head = global head index b*H+h)."""
    row_head = np.ascontiguousarray(row_head, np.int32)
    row_index = np.ascontiguousarray(row_index, np.int32)
    n = len(row_index)
    out = np.zeros((n, P.d), np.float64)
    q, k, v = (np.ascontiguousarray(t) for t in (q, k, v))
    rc = lib().oc_exact_rows(C.byref(P), _ptr(q), _ptr(k), _ptr(v), _ptr(row_head),
                             _ptr(row_index), n, _ptr(out))
    if rc != 0:
        raise ValueError("oracle exact rejected the parameters")
    return out


def e4m3_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, np.uint8)
    out = np.zeros(c.shape, np.float64)
    lib().oc_e4m3_decode_array(_ptr(c), _ptr(out), c.size)
    return out


def e4m3_encode(x) -> np.ndarray:
    xf = np.ascontiguousarray(x, np.float32)
    out = np.zeros(xf.shape, np.uint8)
    lib().oc_e4m3_encode_array(_ptr(xf), _ptr(out), xf.size)
    return out


def e2m1_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, np.uint8)
    out = np.zeros(c.shape, np.float64)
    lib().oc_e2m1_decode_array(_ptr(c), _ptr(out), c.size)
    return out


def e2m1_encode(x) -> np.ndarray:
    xf = np.ascontiguousarray(x, np.float32)
    out = np.zeros(xf.shape, np.uint8)
    lib().oc_e2m1_encode_array(_ptr(xf), _ptr(out), xf.size)
    return out


def mx_exponent(a) -> np.ndarray:
    af = np.ascontiguousarray(a, np.float32)
    out = np.zeros(af.shape, np.int32)
    lib().oc_mx_exponent_array(_ptr(af), _ptr(out), af.size)
    return out


def v4_group(k):
    """32-key group of key k (0..127) of a block for the 4-bit residual: 32
    consecutive positions."""
    k = np.asarray(k)
    return k >> 5


def expcast(s, alpha: float, beta: float) -> np.ndarray:
    sf = np.ascontiguousarray(s, np.float32)
    out = np.zeros(sf.shape, np.uint8)
    lib().oc_expcast_array(_ptr(sf), float(alpha), float(beta), _ptr(out), sf.size)
    return out


def scores(a, b, exact: bool = False) -> np.ndarray:
    """Raw scores of code rows a[i] . b[i] (uint8 [n, d]): the exact dot product
    rounded to fp32 (exact=True), or the diagnostic FP8 matrix-instruction
    model."""
    a = np.ascontiguousarray(a, np.uint8)
    b = np.ascontiguousarray(b, np.uint8)
    assert a.shape == b.shape and a.ndim == 2 and a.shape[1] % 8 == 0
    out = np.zeros(a.shape[0], np.float32)
    lib().oc_score_array(_ptr(a), _ptr(b), a.shape[0], a.shape[1], int(exact), _ptr(out))
    return out


def splitmix64(state: int, n: int) -> np.ndarray:
    out = np.zeros(n, np.uint64)
    lib().oc_splitmix64_array(state, _ptr(out), n)
    return out


def kmeans_init_indices(seed: int, head: int, N: int, C_: int) -> np.ndarray:
    out = np.zeros(C_, np.int32)
    lib().oc_kmeans_init_indices(seed, head, N, C_, _ptr(out))
    return out


def kmeans_shift(v) -> int:
    """Fixed-point exponent sh of a head's values (max|v| * 2^sh < 2^13)."""
    vf = np.ascontiguousarray(v, np.float32)
    return int(lib().oc_kmeans_shift(_ptr(vf), vf.size))


def code_gain(sm_scale: float, d: int = 128) -> np.float32:
    """fp32 factor from raw scores to ExpCast code units: 8*log2(e)*scale."""
    s = np.float32(sm_scale) if sm_scale > 0 else np.float32(1.0 / math.sqrt(d))
    return np.float32(8.0 * 1.4426950408889634 * float(s))
