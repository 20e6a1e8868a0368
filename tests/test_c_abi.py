"""The C ABI from plain C: tests/c_abi_driver.c (no Python, no torch) allocates
with hipMalloc, runs prepare + forward on its own stream, checks two error
paths, and writes O.  Its output must be bit-identical to the binding's for the
same inputs and parameters."""
import os
import subprocess
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import gpu_common as G  # noqa: E402

import precision_fp8_attention_amd as vc  # noqa: E402
from synthetic import inputs  # noqa: E402

pytestmark = pytest.mark.gpu
DRIVER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_driver.bin")


@pytest.mark.parametrize("flags", [vc.DEFAULT_FLAGS, vc.DEFAULT_FLAGS | vc.V4 | vc.SMOOTH_Q | vc.FP8_SCORES],
                         ids=["default", "v4_smooth_q_fp8"])
def test_c_caller_matches_binding(tmp_path, flags):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(DRIVER), f"{DRIVER} is missing: run __graft_entry__.build()"
    B, H, N, C_ = 1, 2, 700, 6
    q, k, v = inputs.make_custom(B, H, N, seed=3)
    fin, fout = tmp_path / "qkv.bin", tmp_path / "o.bin"
    with open(fin, "wb") as f:
        for x in (q, k, v):
            f.write(np.ascontiguousarray(x).tobytes())
    G.log(f"[case] C driver: B={B} H={H} N={N} C={C_} flags={flags}")
    r = subprocess.run([DRIVER, str(fin), str(fout), str(B), str(H), str(N), str(C_), str(flags)],
                       capture_output=True, text=True, timeout=120)
    G.log(r.stdout.strip())
    assert r.returncode == 0, r.stderr
    o_c = np.fromfile(fout, dtype=np.uint16).reshape(B, H, N, 128)
    p = vc.default_params(B, H, N, n_clusters=C_, flags=flags)
    _, o = G.run(p, *G.to_device(q, k, v))
    o_py = o.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(o_c, o_py)
