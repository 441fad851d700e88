"""Seeded random shapes through every entry point, against the oracle (needs an MI355X).

Each case draws B, H, Nq, Nk in [1, 300] (and 24 larger cases: one or two slices, Nq, Nk in
[300, 3000], so the decode keys are split over workgroups), D in {64, 128}, a storage type, the causal flag, an
optional band, key lengths (some zero, some past Nk) and a scale (negative and zero included),
and checks the forward, the KV-cache decode entry point and (every other case) the backward
against the oracle at the usual tolerances.  The cases are fixed by the seed, so a failure names
a reproducible case.
"""
import numpy as np
import pytest
import torch

from gpu_util import compare, to_device, to_f64
from transformer_scaled_dot_amd import binding, inputs

pytestmark = pytest.mark.gpu

N_CASES = 200
N_LARGE = 24
TOL_G = {"bf16": (2e-2, 1e-3), "f16": (2e-2, 1e-3), "f32": (1e-4, 1e-1)}


def draw(i, large=False):
    r = np.random.default_rng((19000 if large else 9000) + i)
    if large:  # longer key loops and split decodes; few slices so the oracle stays quick
        B, H = 1, int(r.integers(1, 3))
        Nq, Nk = int(r.integers(300, 3001)), int(r.integers(300, 3001))
    else:
        B, H = int(r.integers(1, 4)), int(r.integers(1, 4))
        Nq, Nk = int(r.integers(1, 301)), int(r.integers(1, 301))
    D = int(r.choice([64, 128]))
    dtype = str(r.choice(["bf16", "f16", "f32"]))
    causal = bool(r.integers(0, 2))
    window = None if r.random() < 0.6 else int(r.integers(0, 160))
    kl = None if r.random() < 0.5 else r.integers(0, Nk + 20, size=B).astype(np.int32)
    scale = float(np.float32([1.0 / np.sqrt(D), -0.07, 0.0, 0.3][int(r.integers(0, 4))]))
    if large and window is not None:
        window *= 8  # bands of up to ~1300 keys: several tiles wide
    return dict(B=B, H=H, Nq=Nq, Nk=Nk, D=D, dtype=dtype, causal=causal, window=window, kl=kl,
                scale=scale, seed=(19000 if large else 9000) + i)


@pytest.mark.parametrize("i", range(N_LARGE))
def test_random_large_case(i, oracle_impl):
    run_case(i, draw(i, large=True), oracle_impl)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i, oracle_impl):
    run_case(i, draw(i), oracle_impl)


def run_case(i, c, oracle_impl):
    print(f"[random] case {i}: {c}", flush=True)
    w = inputs.Workload("r", c["dtype"], c["B"], c["H"], c["Nq"], c["Nk"], c["D"], c["causal"], False, 1.0, 1.0,
                       c["seed"])
    x = inputs.make_inputs(w)
    q, k, v = (to_device(x[n], c["dtype"]) for n in "qkv")
    kl_dev = None if c["kl"] is None else torch.from_numpy(c["kl"]).cuda()
    s = c["scale"]

    # forward (with the band when drawn)
    o, lse = binding.fwd(q, k, v, causal=c["causal"], key_lens=kl_dev, scale=s, window=c["window"])
    torch.cuda.synchronize()
    ro, rl = oracle_impl.attn(x["q"], x["k"], x["v"], c["dtype"], s, c["causal"], c["kl"], window=c["window"])
    compare(o, lse, ro, rl, c["dtype"], f"case {i} forward")

    # KV-cache decode: the queries are the last Nq positions of each cached sequence
    if c["Nq"] <= c["Nk"]:
        od, ld = binding.decode(q, k, v, causal=c["causal"], key_lens=kl_dev, scale=s)
        torch.cuda.synchronize()
        rod, rld = oracle_impl.attn(x["q"], x["k"], x["v"], c["dtype"], s, 2 if c["causal"] else 0, c["kl"])
        compare(od, ld, rod, rld, c["dtype"], f"case {i} decode")

    # backward, every other case
    if i % 2 == 0:
        do_np = inputs.make_grad_out(w)
        do = to_device(do_np, c["dtype"])
        got = binding.bwd(q, k, v, o, lse, do, causal=c["causal"], key_lens=kl_dev, scale=s, window=c["window"])
        torch.cuda.synchronize()
        want = oracle_impl.attn_bwd(x["q"], x["k"], x["v"], do_np, c["dtype"], s, c["causal"], c["kl"],
                                    window=c["window"])
        tol, floor = TOL_G[c["dtype"]]
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            a = to_f64(a)
            b = np.asarray(b).reshape(a.shape)
            assert np.all(np.isfinite(a)), f"case {i} {name}: non-finite"
            err = float(np.max(np.abs(a - b)))
            ref = float(np.max(np.abs(b)))
            assert err <= tol * max(ref, floor), f"case {i} {name}: max err {err:.3e}, max |ref| {ref:.3e}"
