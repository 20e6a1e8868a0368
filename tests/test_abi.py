"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/vc_attn.h, validates parameters and pointers before any
device call, and lays the workspace out without overlaps."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import precision_fp8_attention_amd as vc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "vc_attn.h")).read()
    return sorted(set(re.findall(r"\b(vc_attn_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = vc.lib()
    names = _declared()
    assert set(names) == set(vc.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_defaults_and_version():
    p = vc.default_params(1, 2, 1024)
    assert (p.d, p.block, p.n_clusters, p.kmeans_iters, p.expcast_k) == (128, 128, 16, 10, 8)
    assert abs(p.rho - 0.005) < 1e-9 and p.flags == vc.DEFAULT_FLAGS and p.tau == 0.0
    assert vc.check_params(p) == vc.OK
    assert vc.version() >= 100
    assert vc.status_string(vc.ERR_WORKSPACE).startswith("workspace")


BAD = [
    (dict(d=64), vc.ERR_UNSUPPORTED),
    (dict(block=64), vc.ERR_UNSUPPORTED),
    (dict(B=0), vc.ERR_INVALID_ARG),
    (dict(N=0), vc.ERR_INVALID_ARG),
    (dict(N=(1 << 20) + 1), vc.ERR_INVALID_ARG),
    (dict(n_clusters=0), vc.ERR_INVALID_ARG),
    (dict(n_clusters=65), vc.ERR_INVALID_ARG),
    (dict(N=10, n_clusters=11), vc.ERR_INVALID_ARG),
    (dict(kmeans_iters=0), vc.ERR_INVALID_ARG),
    (dict(expcast_k=9), vc.ERR_INVALID_ARG),
    (dict(rho=-0.1), vc.ERR_INVALID_ARG),
    (dict(rho=1.5), vc.ERR_INVALID_ARG),
    (dict(rho=float("nan")), vc.ERR_INVALID_ARG),
    (dict(tau=-1.0), vc.ERR_INVALID_ARG),
    (dict(tau=7.0), vc.ERR_INVALID_ARG),
    (dict(expcast_k=0, tau=71.0), vc.ERR_INVALID_ARG),
    (dict(sm_scale=float("inf")), vc.ERR_INVALID_ARG),
    (dict(flags=512), vc.ERR_INVALID_ARG),
    (dict(flags=vc.DEFAULT_FLAGS | vc.EXACT_SCORES | vc.FP8_SCORES), vc.ERR_INVALID_ARG),
    # the smoothed-query score terms grow as N^2: refused above the documented bound
    (dict(N=vc.SMOOTH_Q_MAX_TOKENS + 1, flags=vc.DEFAULT_FLAGS | vc.SMOOTH_Q), vc.ERR_UNSUPPORTED),
    (dict(N=1 << 20, flags=vc.DEFAULT_FLAGS | vc.SMOOTH_Q), vc.ERR_UNSUPPORTED),
    (dict(flags=vc.WARM_START | vc.REPAIR), vc.ERR_INVALID_ARG),  # warm start needs V-Smooth
    (dict(flags=vc.DEFAULT_FLAGS | vc.WARM_START | vc.REUSE_CLUSTERS), vc.ERR_INVALID_ARG),
]


@pytest.mark.parametrize("kw,status", BAD)
def test_parameter_validation(kw, status):
    base = dict(B=1, H=2, N=1024)
    base.update(kw)
    B, H, N = base.pop("B"), base.pop("H"), base.pop("N")
    p = vc.default_params(B, H, N, **base)
    assert vc.check_params(p) == status
    assert vc.workspace_size(p) == 0
    with pytest.raises(vc.VCError):
        vc.workspace_layout(p)


def test_pointer_and_workspace_errors_before_device_work():
    L = vc.lib()
    p = vc.default_params(1, 2, 1024)
    need = vc.workspace_size(p)
    fake = C.c_void_p(0x10000)  # never dereferenced: checks fail first
    mis = C.c_void_p(0x10008)
    P = C.byref(p)
    assert L.vc_attn_prepare(P, None, fake, fake, fake, need, None) == vc.ERR_INVALID_ARG
    assert L.vc_attn_prepare(P, mis, fake, fake, fake, need, None) == vc.ERR_INVALID_ARG
    assert L.vc_attn_prepare(P, fake, fake, fake, None, need, None) == vc.ERR_WORKSPACE
    assert L.vc_attn_prepare(P, fake, fake, fake, fake, need - 1, None) == vc.ERR_WORKSPACE
    assert L.vc_attn_prepare(P, fake, fake, fake, C.c_void_p(0x10080), need, None) == vc.ERR_WORKSPACE
    assert L.vc_attn_forward(P, fake, need, None, None) == vc.ERR_INVALID_ARG
    assert L.vc_attn_forward(P, fake, need - 1, fake, None) == vc.ERR_WORKSPACE
    assert L.vc_attn_forward(None, fake, need, fake, None) == vc.ERR_INVALID_ARG
    bad = vc.default_params(1, 2, 1024, d=64)
    assert L.vc_attn_forward(C.byref(bad), fake, need, fake, None) == vc.ERR_UNSUPPORTED
    assert L.vc_attn_forward_pcodes(P, fake, need, fake, None, None) == vc.ERR_INVALID_ARG
    assert L.vc_attn_forward_pcodes(P, fake, need, fake, mis, None) == vc.ERR_INVALID_ARG
    assert L.vc_attn_forward_pcodes(P, fake, need - 1, fake, fake, None) == vc.ERR_WORKSPACE
    assert L.vc_attn_forward_pcodes(C.byref(bad), fake, need, fake, None, None) == vc.ERR_UNSUPPORTED
    assert L.vc_attn_run_noalloc(P, fake, fake, None, fake, None) == vc.ERR_INVALID_ARG
    assert L.vc_attn_run_noalloc(P, fake, fake, fake, mis, None) == vc.ERR_INVALID_ARG
    assert L.vc_attn_run_noalloc(C.byref(bad), fake, fake, fake, fake, None) == vc.ERR_UNSUPPORTED
    # more than the static workspace: refused before any device work
    big = vc.default_params(2, 24, 16544, n_clusters=32)
    assert vc.workspace_size(big) > vc.NOALLOC_WORKSPACE_BYTES
    assert L.vc_attn_run_noalloc(C.byref(big), fake, fake, fake, fake, None) == vc.ERR_WORKSPACE


def test_smooth_q_accepted_up_to_its_bound():
    p = vc.default_params(1, 1, vc.SMOOTH_Q_MAX_TOKENS, flags=vc.DEFAULT_FLAGS | vc.SMOOTH_Q)
    assert vc.check_params(p) == vc.OK
    L = vc.workspace_layout(p)
    nblk = vc.SMOOTH_Q_MAX_TOKENS // 128
    assert L["total"] >= nblk * vc.SMOOTH_Q_MAX_TOKENS * 4  # the score terms, 512 MiB


@pytest.mark.parametrize("N,flags,exact", [
    (1024, 0, True), (vc.FP8_SCORES_MIN_TOKENS - 1, 0, True), (vc.FP8_SCORES_MIN_TOKENS, 0, False),
    (16544, 0, False), (1024, vc.FP8_SCORES, False), (16544, vc.EXACT_SCORES, True)])
def test_score_mode_by_flags_and_token_count(N, flags, exact):
    """Exact scores (bf16 copy of the K codes in the workspace) below the token
    count where the default turns to FP8 scores, or when asked for."""
    p = vc.default_params(1, 1, N, flags=vc.DEFAULT_FLAGS | flags)
    L = vc.workspace_layout(p)
    npad = -(-N // 128) * 128
    k16 = L["sq"] - L["k16"]  # k16 is followed by sq; 0 bytes (next offset) when unused
    assert (k16 >= npad * 256) == exact and (k16 < 256) == (not exact)


def test_binding_refuses_tensors_the_abi_would_misread():
    """The binding checks dtype, shape, layout and device before it passes
    bare pointers (here on CPU tensors, so no library call is made)."""
    import torch
    p = vc.default_params(1, 2, 64)
    good = torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16)
    ws = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="bfloat16"):
        vc.prepare(p, good.float(), good, good, ws)
    with pytest.raises(ValueError, match="shape"):
        vc.prepare(p, good[:, :1], good, good, ws)
    with pytest.raises(ValueError, match="contiguous"):
        vc.prepare(p, good.transpose(1, 2).contiguous().transpose(1, 2), good, good, ws)
    with pytest.raises(ValueError, match="GPU"):
        vc.prepare(p, good, good, good, ws)
    with pytest.raises(ValueError, match="GPU"):
        vc.forward(p, ws, good)


@pytest.mark.parametrize("v4,sq", [(False, False), (True, False), (False, True), (True, True)],
                         ids=["e4m3_v", "v4", "smooth_q", "v4_smooth_q"])
@pytest.mark.parametrize("B,H,N,C_,rho", [(1, 2, 1024, 8, 0.005), (2, 24, 16544, 32, 0.005),
                                          (1, 40, 75600, 64, 0.005), (1, 1, 1, 1, 1.0),
                                          (1, 3, 300, 5, 0.0)])
def test_layout_aligned_and_disjoint(B, H, N, C_, rho, v4, sq):
    p = vc.default_params(B, H, N, n_clusters=C_, rho=rho,
                          flags=vc.DEFAULT_FLAGS | (vc.V4 if v4 else 0) | (vc.SMOOTH_Q if sq else 0))
    L = vc.workspace_layout(p)
    BH, nblk = B * H, (N + 127) // 128
    npad = nblk * 128
    m = 0 if rho == 0 else min(N, int(-(-float(C.c_float(rho).value) * N // 1)))
    mpad = -(-m // 128) * 128
    sizes = dict(header=256, kbar=BH * 512, ksum=BH * (-(-N // 512)) * 1024, init_idx=BH * C_ * 4,
                 centroids=BH * C_ * 512, labels=BH * N * 4, perm=BH * N * 4, iperm=BH * N * 4,
                 q8=BH * npad * 128, k8=BH * npad * 128,
                 k16=BH * npad * 256 if N < vc.FP8_SCORES_MIN_TOKENS else 0, sq=BH * nblk * 4, sk=BH * nblk * 4,
                 mu=BH * nblk * 512, bamax=BH * nblk * 512, mup=BH * nblk * 512,
                 mupt=BH * (-(-nblk // 16)) * 8192, sv=BH * 512,
                 inv=BH * 512, v8t=0 if v4 else BH * 128 * npad, err=BH * N * 4, rep_pos=BH * mpad * 4,
                 rep_dt=BH * 128 * mpad * 2, v4t=BH * nblk * 8192 if v4 else 0,
                 v4s=(BH * nblk + 1) * 512 if v4 else 0, qbar=BH * nblk * 512 if sq else 0,
                 qbias=BH * nblk * npad * 4 if sq else 0)
    spans = sorted((L[k], L[k] + n, k) for k, n in sizes.items())
    for (a0, a1, ka), (b0, b1, kb) in zip(spans, spans[1:]):
        assert a1 <= b0, (ka, kb)
    for k in sizes:
        assert L[k] % 256 == 0
    assert spans[-1][1] <= L["total"] == vc.workspace_size(p)


# Operand layout of v_mfma_scale_f32_16x16x128_f8f6f4 with an FP4 A operand, as
# measured on gfx950 by an in-bounds probe: lane group g's dword d, nibble n
# multiplies the B operand's K index FP4_K[g][d] + n (n = 0..7).
FP4_K = [[0, 8, 32, 40], [64, 72, 96, 104], [16, 24, 48, 56], [80, 88, 112, 120]]


def test_v4_code_bytes_meet_their_own_p_bytes():
    """The 4-bit tile stores key k's code where the FP4 operand multiplies it
    with key k's ExpCast byte.  Lane group g of the B operand holds, in byte
    4t + v (K index 32g + 4t + v), the key of K row 16t + 4g + v, and with the
    4-bit residual that row holds block position v4_krow(16t + 4g + v).  The
    tile keeps key k in byte k/2 (low nibble for even k), so lane group G of A
    (one E8M0 scale) covers positions 32G .. 32G+31: 32 consecutive keys."""
    sys_path = os.path.join(ROOT, "tests")
    import sys
    sys.path.insert(0, sys_path)
    import gpu_common as G
    assert sorted(G.v4_krow(np.arange(128))) == list(range(128))
    assert np.array_equal(G.v4_krow(G.v4_krow(np.arange(128))), np.arange(128))
    seen = set()
    for k in range(128):
        b = int(G._v4_byte(np.int64(k)))
        g, within = divmod(b, 16)
        d, half = divmod(within, 4)
        n = 2 * half + (k & 1)
        assert g == k // 32
        kappa = FP4_K[g][d] + n                  # B operand K index
        bg, byte = divmod(kappa, 32)             # its lane group and byte
        t, vv = divmod(byte, 4)
        assert int(G.v4_krow(16 * t + 4 * bg + vv)) == k, k
        seen.add((b, k & 1))
    assert len(seen) == 128


def test_library_binds_to_torchs_hip_runtime():
    """Loading the library through the binding before torch is imported must not
    bring a second HIP runtime into the process (torch's libraries request the
    runtime under another file name; two runtimes leave the library with no
    device and fail every launch).  Checked in a fresh process, no GPU needed."""
    import subprocess
    import sys
    code = ("import precision_fp8_attention_amd as vc; vc.lib(); import torch; "
            "print(len({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "1", r.stdout
