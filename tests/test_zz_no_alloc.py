"""vc_attn_run_noalloc through the C ABI: prepare + forward with the library's
static per-GPU workspace must give the same output as vc_attn_prepare +
vc_attn_forward with a caller-allocated workspace, on two calls in a row (the
second smaller, so the array holds the first call's larger contents)."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import gpu_common as G  # noqa: E402

from synthetic import inputs  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_fp8_attention_amd as vc
    vc.lib()


def test_noalloc_matches_allocated_workspace_twice():
    import torch

    import precision_fp8_attention_amd as vc
    cases = [(1, 3, 1000, 8, vc.DEFAULT_FLAGS | vc.FP8_SCORES, 31),  # larger first
             (1, 2, 300, 5, vc.DEFAULT_FLAGS, 32)]                     # then smaller
    for B, H, N, C_, flags, seed in cases:
        G.log(f"[case] run_noalloc B={B} H={H} N={N} flags={flags}")
        p = G.lib_params(B, H, N, C_, rho=0.02, flags=flags)
        assert vc.workspace_size(p) <= vc.NOALLOC_WORKSPACE_BYTES
        q, k, v = inputs.make_custom(B, H, N, seed=seed)
        qd, kd, vd = G.to_device(q, k, v)
        _, o_ref = G.run(p, qd, kd, vd)
        o = torch.full_like(qd, float("nan"))
        vc.run_noalloc(p, qd, kd, vd, o)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"run_noalloc differs from prepare + forward (N={N})"
        G.check_output(p, q, k, v, o, list(range(B * H)), np.arange(N, dtype=np.int32),
                       label=f"noalloc_N{N}")
