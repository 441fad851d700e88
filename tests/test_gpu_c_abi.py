"""A plain C program calls the library through include/attn_fwd.h (needs an MI355X).

tests/c_abi/attn_fwd_c_caller.c, built by gcc against the public header, the HIP runtime's
memory API and libattn_fwd.so (no Python, no torch), reads seeded inputs from a file, calls
attn_fwd on a stream of its own and writes O and LSE back; they are compared with the oracle on
the same stored inputs at the forward's tolerances (max |dO| 2e-2 for bf16 / fp16, 1e-4 for
fp32; max |dLSE| 1e-3).
"""
import os
import subprocess

import numpy as np
import pytest

from transformer_scaled_dot_amd import inputs

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CALLER = os.path.join(ROOT, "tests", "c_abi", "attn_fwd_c_caller")
TOL_O = {"bf16": 2e-2, "f16": 2e-2, "f32": 1e-4}


@pytest.mark.parametrize("dtype,D,causal", [("bf16", 128, True), ("f16", 64, False), ("f32", 64, True)])
def test_c_caller_matches_oracle(dtype, D, causal, tmp_path, oracle_impl):
    assert os.access(CALLER, os.X_OK), "tests/c_abi/attn_fwd_c_caller is not built"
    w = inputs.Workload("c_caller", dtype, 2, 3, 100, 130, D, causal, False, 1.0, 1.0, 61)
    x = inputs.make_inputs(w)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        for name in ("q", "k", "v"):
            f.write(np.ascontiguousarray(x[name]).tobytes())
    args = [CALLER, str(w.B), str(w.H), str(w.Nq), str(w.Nk), str(D), str(int(causal)),
            str(inputs.DTYPE_CODE[dtype]), str(src), str(dst)]
    print(" ".join(args), flush=True)
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0
    assert "D=96: " in r.stdout and "causal=2: " in r.stdout and "attn_fwd: " in r.stdout
    raw = np.fromfile(dst, dtype=np.uint8)
    n_o = w.B * w.H * w.Nq * D
    store = x["q"].dtype
    o = inputs.storage_to_f64(raw[: n_o * store.itemsize].view(store).reshape(w.B, w.H, w.Nq, D), dtype)
    lse = raw[n_o * store.itemsize:].view(np.float32).reshape(w.B, w.H, w.Nq).astype(np.float64)
    ro, rl = oracle_impl.attn(x["q"], x["k"], x["v"], dtype, float(x["scale"]), causal, None)
    assert float(np.max(np.abs(o - ro))) <= TOL_O[dtype]
    assert float(np.max(np.abs(lse - rl))) <= 1e-3
