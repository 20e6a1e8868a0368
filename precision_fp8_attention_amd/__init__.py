"""Python binding of libvcattn.so, the VC-Attention FP8 library for MI355X.

Argument marshalling only: every step of the method runs in the library's HIP
kernels.  torch supplies device memory and the current HIP stream.  The names
mirror the C ABI in include/vc_attn.h (without the vc_attn_ prefix).
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libvcattn.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_NOT_PREPARED, ERR_HIP, ERR_INTERNAL = range(7)
VSMOOTH, REPAIR, PERMUTE_Q, REUSE_CLUSTERS, EXACT_SCORES, WARM_START, V4, SMOOTH_Q = 1, 2, 4, 8, 16, 32, 64, 128
FP8_SCORES = 256
DEFAULT_FLAGS = VSMOOTH | REPAIR | PERMUTE_Q
FP8_SCORES_MIN_TOKENS = 4096   # without a score flag: FP8 scores from this N on
SMOOTH_Q_MAX_TOKENS = 131072   # largest N accepted with SMOOTH_Q

EXPORTS = ("vc_attn_default_params", "vc_attn_workspace_size", "vc_attn_workspace_layout",
           "vc_attn_check_params", "vc_attn_prepare", "vc_attn_forward", "vc_attn_forward_pcodes",
           "vc_attn_status_string", "vc_attn_version", "vc_attn_run_noalloc")
NOALLOC_WORKSPACE_BYTES = 256 << 20  # static workspace of run_noalloc, per GPU


class Params(C.Structure):
    _fields_ = [("B", C.c_int32), ("H", C.c_int32), ("N", C.c_int32), ("d", C.c_int32),
                ("block", C.c_int32), ("n_clusters", C.c_int32), ("kmeans_iters", C.c_int32),
                ("expcast_k", C.c_int32), ("seed", C.c_uint64), ("rho", C.c_float),
                ("sm_scale", C.c_float), ("tau", C.c_float), ("flags", C.c_uint32)]


LAYOUT_FIELDS = ("total", "header", "kbar", "ksum", "init_idx", "centroids", "labels", "perm",
                 "iperm", "q8", "k8", "k16", "sq", "sk", "mu", "bamax", "mup", "mupt", "sv", "inv", "v8t", "err",
                 "rep_pos", "rep_dt", "v4t", "v4s", "qbar", "qbias")


class Layout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in LAYOUT_FIELDS]


class VCError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> C.CDLL:
    """Load the HIP library; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m precision_fp8_attention_amd.build`")
        # torch ships its own HIP runtime, which its libraries request as
        # libamdhip64.so; the library asks for the SONAME libamdhip64.so.7 and binds
        # to torch's copy only if that is loaded first.  Loaded the other way round
        # the process holds two runtimes, and the library's own (which does not own
        # torch's streams or allocations) fails every launch.
        import torch  # noqa: F401
        L = C.CDLL(LIB_PATH)
        P = C.POINTER(Params)
        L.vc_attn_default_params.argtypes = [P]
        L.vc_attn_default_params.restype = None
        L.vc_attn_workspace_size.argtypes = [P]
        L.vc_attn_workspace_size.restype = C.c_size_t
        L.vc_attn_workspace_layout.argtypes = [P, C.POINTER(Layout)]
        L.vc_attn_check_params.argtypes = [P]
        L.vc_attn_prepare.argtypes = [P, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                      C.c_size_t, C.c_void_p]
        L.vc_attn_forward.argtypes = [P, C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p]
        L.vc_attn_forward_pcodes.argtypes = [P, C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p,
                                             C.c_void_p]
        L.vc_attn_run_noalloc.argtypes = [P, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                          C.c_void_p]
        L.vc_attn_status_string.argtypes = [C.c_int]
        L.vc_attn_status_string.restype = C.c_char_p
        L.vc_attn_version.restype = C.c_int32
        for f in ("vc_attn_workspace_layout", "vc_attn_check_params", "vc_attn_prepare",
                  "vc_attn_forward", "vc_attn_forward_pcodes", "vc_attn_run_noalloc"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def default_params(B=0, H=0, N=0, **kw) -> Params:
    p = Params()
    lib().vc_attn_default_params(C.byref(p))
    p.B, p.H, p.N = B, H, N
    for k, v in kw.items():
        if not hasattr(p, k):
            raise AttributeError(k)
        setattr(p, k, v)
    return p


def status_string(s: int) -> str:
    return lib().vc_attn_status_string(s).decode()


def version() -> int:
    return int(lib().vc_attn_version())


def check_params(p: Params) -> int:
    return int(lib().vc_attn_check_params(C.byref(p)))


def workspace_size(p: Params) -> int:
    return int(lib().vc_attn_workspace_size(C.byref(p)))


def workspace_layout(p: Params) -> dict:
    out = Layout()
    st = lib().vc_attn_workspace_layout(C.byref(p), C.byref(out))
    if st != OK:
        raise VCError(st, "workspace_layout")
    return {n: int(getattr(out, n)) for n in LAYOUT_FIELDS}


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _check(what: str, p: Params, tensors: dict, workspace=None) -> None:
    """The C ABI takes bare pointers: refuse tensors it would misread (wrong
    dtype, shape or layout, host memory, mixed devices) before passing them."""
    import torch
    dev = None
    for name, t in tensors.items():
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{what}: {name} must be bfloat16, got {t.dtype}")
        if tuple(t.shape) != (p.B, p.H, p.N, p.d):
            raise ValueError(f"{what}: {name} must have shape {(p.B, p.H, p.N, p.d)}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{what}: {name} must be contiguous [B, H, N, d]")
        if t.device.type != "cuda":
            raise ValueError(f"{what}: {name} must be a GPU tensor")
        if dev is not None and t.device != dev:
            raise ValueError(f"{what}: {name} is on {t.device}, expected {dev}")
        dev = t.device
    if workspace is not None:
        if workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_contiguous():
            raise ValueError(f"{what}: the workspace must be a contiguous 1-D uint8 tensor")
        if dev is not None and workspace.device != dev:
            raise ValueError(f"{what}: the workspace is on {workspace.device}, expected {dev}")


def _stream(stream, device) -> int | None:
    """The given stream, else the current stream of the tensors' device."""
    if stream is not None:
        return int(stream)
    import torch
    return int(torch.cuda.current_stream(device).cuda_stream)


def prepare(p: Params, q, k, v, workspace, stream=None) -> None:
    """vc_attn_prepare on torch device tensors (bf16 [B,H,N,128], uint8 workspace)."""
    _check("prepare", p, dict(q=q, k=k, v=v), workspace)
    st = lib().vc_attn_prepare(C.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    if st != OK:
        raise VCError(st, "vc_attn_prepare")


def forward(p: Params, workspace, o, stream=None) -> None:
    """vc_attn_forward: writes o (bf16 [B,H,N,128], original token order)."""
    _check("forward", p, dict(o=o), workspace)
    st = lib().vc_attn_forward(C.byref(p), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _ptr(o),
                               _stream(stream, o.device))
    if st != OK:
        raise VCError(st, "vc_attn_forward")


def forward_pcodes(p: Params, workspace, o, pcodes, stream=None) -> None:
    """vc_attn_forward_pcodes: forward plus every ExpCast byte of the main loop in
    pcodes (uint8 [B*H, Npad, Npad], processing order)."""
    import torch
    _check("forward_pcodes", p, dict(o=o), workspace)
    npad = ((p.N + 127) // 128) * 128
    if (pcodes.dtype != torch.uint8 or not pcodes.is_contiguous() or pcodes.device != o.device
            or pcodes.numel() < p.B * p.H * npad * npad):
        raise ValueError("forward_pcodes: pcodes must be a contiguous uint8 GPU tensor of "
                         f"at least B*H*Npad*Npad = {p.B * p.H * npad * npad} bytes on {o.device}")
    st = lib().vc_attn_forward_pcodes(C.byref(p), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _ptr(o),
                                      _ptr(pcodes), _stream(stream, o.device))
    if st != OK:
        raise VCError(st, "vc_attn_forward_pcodes")


def run_noalloc(p: Params, q, k, v, o, stream=None) -> None:
    """vc_attn_run_noalloc: prepare + forward with the library's static
    per-GPU workspace (no allocation); o receives the output."""
    _check("run_noalloc", p, dict(q=q, k=k, v=v, o=o))
    st = lib().vc_attn_run_noalloc(C.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                   _stream(stream, q.device))
    if st != OK:
        raise VCError(st, "vc_attn_run_noalloc")


def alloc_workspace(p: Params, device="cuda"):
    import torch
    n = workspace_size(p)
    if n == 0:
        raise VCError(check_params(p), "workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def attention(q, k, v, **kw):
    """One-shot VC-Attention FP8: allocates the workspace and output with torch,
    then runs prepare and forward on the current stream.  q, k, v: bf16
    [B, H, N, 128] contiguous CUDA tensors."""
    import torch
    B, H, N, d = q.shape
    p = default_params(B, H, N, d=d, **kw)
    ws = alloc_workspace(p, q.device)
    o = torch.empty_like(q)
    prepare(p, q, k, v, ws)
    forward(p, ws, o)
    return o
