"""Seeded synthetic inputs for VC-Attention FP8 (shared by the tests, the smoke
check and the benchmark; holds none of the attention method's arithmetic).

The workloads stand in for the activations the source pages measure on, which are
not available here: FLUX-style joint text/image attention (token counts from the
FLUX.3 Klein launch article: a 1024x1024 image is 4096 tokens of 128 channels,
4256 tokens for text-to-image and 8272 for image-to-image with one reference) and
Wan2.2-style 720p video clips (about 70k tokens for a 5 s clip, per the
noticiai.com.br VC-Attention article, section "Por que a atencao e o gargalo").

Random numbers come from splitmix64 (Steele, Lea and Flood; Vigna's reference
definition) used as a counter-based stream: output i of a stream with state s is
mix(s + (i + 1) * 0x9E3779B97F4A7C15).  Normals use the Box-Muller cosine branch in
fp64, then round to fp32 and to bf16 (both round-to-nearest-even).

Recipe per (batch b, head h):
  Q, K ~ N(0, 1) (N(0.5, 1) on reference tokens of the image-to-image workload);
  K gets a per-(head, channel) offset ~ N(0, 3) shared by all batch items;
  V ~ N(0, 1) (N(0.5, 1) on reference tokens), plus outliers: round(rate * N)
  tokens drawn without replacement get an independent N(0, sigma) on 4 distinct
  channels; the channels are drawn per head (per (batch, head) where the workload
  says the outlier channels change between batch items); text tokens of the
  text-to-image 1024^2 workload get twice the outlier sigma.
"""
from __future__ import annotations

import concurrent.futures as _fut
import os

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Workload catalogue.  "text" is the [start, end) range of text tokens, "ref" the
# range of reference-image tokens (shifted mean), "chan_per_batch" draws outlier
# channels per (batch, head) instead of per head.
WORKLOADS = {
    0: dict(name="tiny", B=1, H=2, N=1024, C=8, T=10, rho=0.005,
            rate=0.01, sigma=20.0, text=None, text_mult=1.0, ref=None, chan_per_batch=False),
    1: dict(name="flux_t2i_1024", B=1, H=24, N=4256, C=16, T=10, rho=0.005,
            rate=0.01, sigma=20.0, text=(0, 160), text_mult=2.0, ref=None, chan_per_batch=False),
    2: dict(name="flux_i2i_1024_ref", B=1, H=24, N=8272, C=16, T=10, rho=0.005,
            rate=0.01, sigma=20.0, text=(0, 80), text_mult=1.0, ref=(4176, 8272),
            chan_per_batch=False),
    3: dict(name="flux_t2i_2048_cfg", B=2, H=24, N=16544, C=32, T=10, rho=0.005,
            rate=0.01, sigma=20.0, text=(0, 160), text_mult=1.0, ref=None, chan_per_batch=True),
    4: dict(name="wan22_720p_5s", B=1, H=40, N=75600, C=64, T=10, rho=0.005,
            rate=0.005, sigma=30.0, text=None, text_mult=1.0, ref=None, chan_per_batch=False),
}
D = 128


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream(state: int, n: int, start: int = 0) -> np.ndarray:
    """Outputs start..start+n-1 of the splitmix64 stream with the given state."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        return _mix(np.uint64(state & 0xFFFFFFFFFFFFFFFF) + i * GOLDEN)


def subseed(*parts: int) -> int:
    """Fold integer parts into one 64-bit stream state."""
    s = np.uint64(0x243F6A8885A308D3)
    with np.errstate(over="ignore"):
        for p in parts:
            s = _mix(np.asarray([s ^ np.uint64(p & 0xFFFFFFFFFFFFFFFF)], dtype=np.uint64) + GOLDEN)[0]
    return int(s)


def normals(state: int, n: int, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """n fp64 normals (Box-Muller, cosine branch) from one stream."""
    x = stream(state, 2 * n)
    u1 = ((x[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53  # (0, 1]
    u2 = (x[1::2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53  # [0, 1)
    return mean + std * np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def draw_distinct(state: int, n: int, k: int) -> np.ndarray:
    """k distinct integers from [0, n) by a partial Fisher-Yates shuffle."""
    x = stream(state, k)
    swap: dict[int, int] = {}
    out = np.empty(k, dtype=np.int64)
    for i in range(k):
        j = i + int(x[i] % np.uint64(n - i))
        vi, vj = swap.get(i, i), swap.get(j, j)
        swap[i], swap[j] = vj, vi
        out[i] = vj
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bf16 bits, round-to-nearest-even at each step."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _head(wl: dict, cfg_id: int, seed: int, b: int, h: int, N: int):
    ref = wl["ref"]
    q = normals(subseed(seed, cfg_id, 1, b, h), N * D)
    k = normals(subseed(seed, cfg_id, 2, b, h), N * D)
    v = normals(subseed(seed, cfg_id, 3, b, h), N * D)
    q, k, v = (t.reshape(N, D) for t in (q, k, v))
    if ref is not None:
        for t in (q, k, v):
            t[ref[0]:ref[1]] += 0.5
    k += normals(subseed(seed, cfg_id, 4, h), D, 0.0, 3.0)[None, :]
    n_out = int(round(wl["rate"] * N))
    if n_out > 0:
        toks = draw_distinct(subseed(seed, cfg_id, 5, b, h), N, n_out)
        cb = b if wl["chan_per_batch"] else 0
        chans = draw_distinct(subseed(seed, cfg_id, 6, cb, h), D, 4)
        sig = np.full(n_out, wl["sigma"])
        if wl["text"] is not None and wl["text_mult"] != 1.0:
            t0, t1 = wl["text"]
            sig[(toks >= t0) & (toks < t1)] *= wl["text_mult"]
        add = normals(subseed(seed, cfg_id, 7, b, h), n_out * 4).reshape(n_out, 4) * sig[:, None]
        for ci in range(4):
            v[toks, chans[ci]] += add[:, ci]
    return to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v)


def make_inputs(cfg_id: int, seed: int = 0, heads=None, threads: int | None = None):
    """bf16 bit arrays (uint16) q, k, v of shape [B, H, N, 128] for a workload.

    heads: optional list of global head indices b*H+h to fill (others stay zero),
    for parity checks that sample heads of the very large workloads."""
    wl = WORKLOADS[cfg_id]
    B, H, N = wl["B"], wl["H"], wl["N"]
    q = np.zeros((B, H, N, D), np.uint16)
    k = np.zeros_like(q)
    v = np.zeros_like(q)
    todo = list(range(B * H)) if heads is None else list(heads)
    nthr = threads or min(16, os.cpu_count() or 1)

    def job(gh):
        b, h = divmod(gh, H)
        q[b, h], k[b, h], v[b, h] = _head(wl, cfg_id, seed, b, h, N)

    with _fut.ThreadPoolExecutor(nthr) as ex:
        list(ex.map(job, todo))
    return q, k, v


def make_custom(B: int, H: int, N: int, seed: int = 0, rate: float = 0.01, sigma: float = 20.0,
                koff: float = 3.0, vmean: float = 0.0):
    """Small generic inputs with the same recipe (used by edge-case tests)."""
    q = np.zeros((B, H, N, D), np.uint16)
    k = np.zeros_like(q)
    v = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            qq = normals(subseed(seed, 99, 1, b, h, N), N * D).reshape(N, D)
            kk = normals(subseed(seed, 99, 2, b, h, N), N * D).reshape(N, D)
            vv = normals(subseed(seed, 99, 3, b, h, N), N * D, vmean).reshape(N, D)
            kk += normals(subseed(seed, 99, 4, h), D, 0.0, koff)[None, :]
            n_out = int(round(rate * N))
            if n_out > 0:
                toks = draw_distinct(subseed(seed, 99, 5, b, h, N), N, n_out)
                chans = draw_distinct(subseed(seed, 99, 6, h), D, 4)
                add = normals(subseed(seed, 99, 7, b, h, N), n_out * 4).reshape(n_out, 4) * sigma
                for ci in range(4):
                    vv[toks, chans[ci]] += add[:, ci]
            q[b, h], k[b, h], v[b, h] = to_bf16_bits(qq), to_bf16_bits(kk), to_bf16_bits(vv)
    return q, k, v


def drift(v: np.ndarray, step: int, seed: int = 0, scale: float = 0.05) -> np.ndarray:
    """Values of a later denoising step: v (bf16 bits, any shape ending in 128)
    plus independent N(0, scale) noise per element from a stream seeded by
    (seed, step), rounded back to bf16.  Small steps keep the clusters close
    to those of the previous step, as consecutive diffusion steps do."""
    x = bf16_bits_to_f32(np.ascontiguousarray(v)).astype(np.float64)
    x = x + normals(subseed(seed, 0xD41F7, step), x.size, 0.0, scale).reshape(x.shape)
    return to_bf16_bits(x)
