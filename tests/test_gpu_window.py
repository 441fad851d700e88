"""Sliding-window (local band) attention on the HIP path against the fp64 oracle (needs an MI355X).

Row i attends only to keys j with |i - j| <= w, on top of the causal and padding rules.  Every
expected value comes from oracle/ (window argument) or from a closed form; tolerances as in
test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

import pins
from gpu_util import TOL_LSE, TOL_O, compare, run, sample_rows, to_device, to_f64
from transformer_scaled_dot_amd import binding, inputs

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


# name, B, H, Nq, Nk, D, causal, key_lens
SHAPES = [
    ("square_300_d64", 2, 3, 300, 300, 64, False, None),
    ("square_300_d128_causal", 2, 3, 300, 300, 128, True, None),
    ("nq_lt_nk_d128", 1, 2, 130, 257, 128, False, None),
    ("nq_gt_nk_causal_d64", 1, 2, 257, 130, 64, True, None),
    ("padded_d64", 4, 2, 200, 200, 64, False, [200, 150, 9, 0]),
    ("padded_causal_d128", 4, 2, 200, 200, 128, True, [200, 150, 9, 0]),
]
WINDOWS = [0, 1, 31, 63, 64, 65, 100, 255]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_window_parity(shape, dtype, oracle_impl):
    name, B, H, Nq, Nk, D, causal, kl = shape
    w = inputs.Workload(name, dtype, B, H, Nq, Nk, D, causal, kl is not None, 1.0, 1.0, 91)
    x = inputs.make_inputs(w)
    if kl is not None:
        x["key_lens"] = np.array(kl, np.int32)
    worst = (0.0, 0.0)
    for win in WINDOWS:
        log(f"[window] {name} {dtype} w={win}")
        o, lse = run(x, dtype, causal, window=win)
        ro, rl = oracle_impl.attn(x["q"], x["k"], x["v"], dtype, float(x["scale"]), causal,
                                  x["key_lens"], window=win)
        eo, el = compare(o, lse, ro, rl, dtype, f"{name}/{dtype}/w={win}")
        worst = (max(worst[0], eo), max(worst[1], el))
    log(f"[window] {name} {dtype}: max|dO|={worst[0]:.3e} max|dLSE|={worst[1]:.3e}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_wide_window_is_no_window_bitwise(dtype):
    """A band at least as wide as the sequence is the plain kernel, bit for bit."""
    rng = np.random.default_rng(5)
    B, H, N, D = 2, 2, 333, 128
    x = {n: pins.rand_store(rng, (B, H, N, D), dtype) for n in "qkv"}
    x["scale"] = np.float32(0.088)
    x["key_lens"] = np.array([333, 100], np.int32)
    for causal in (False, True):
        o1, l1 = run(x, dtype, causal)
        for win in (N, N + 1, 10 ** 6):
            o2, l2 = run(x, dtype, causal, window=win)
            assert torch.equal(o1, o2) and torch.equal(l1, l2), win


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_window_zero_query_mean(dtype):
    """Q = 0: O is the mean of V over the band's valid keys, LSE = ln of their count."""
    rng = np.random.default_rng(6)
    B, H, N, D = 2, 2, 260, 64
    q = pins.store(np.zeros((B, H, N, D)), dtype)
    k = pins.rand_store(rng, (B, H, N, D), dtype)
    v = pins.rand_store(rng, (B, H, N, D), dtype)
    kl = np.array([260, 120], np.int32)
    vd = inputs.storage_to_f64(v, dtype)
    for causal in (False, True):
        for win in (0, 7, 64, 130):
            x = {"q": q, "k": k, "v": v, "scale": np.float32(0.3), "key_lens": kl}
            o, lse = run(x, dtype, causal, window=win)
            o, lse = to_f64(o), to_f64(lse)
            for b in range(B):
                L = int(kl[b])
                for i in range(N):
                    keep = pins.window_set(i, L, causal, win)
                    if not keep:
                        assert np.all(o[b, :, i] == 0) and np.all(lse[b, :, i] == -np.inf)
                        continue
                    want = vd[b][:, keep].mean(axis=1)  # [H, D]: mean over the band's keys
                    assert np.max(np.abs(o[b, :, i] - want)) <= TOL_O[dtype]
                    assert np.max(np.abs(lse[b, :, i] - np.log(len(keep)))) <= TOL_LSE


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_window_zero_copies_v(dtype):
    """A band of width 0 keeps only key i: O[i] = V[i] exactly."""
    rng = np.random.default_rng(8)
    B, H, N, D = 1, 3, 190, 128
    x = {n: pins.rand_store(rng, (B, H, N, D), dtype) for n in "qkv"}
    x["scale"], x["key_lens"] = np.float32(0.088), None
    for causal in (False, True):
        o, _ = run(x, dtype, causal, window=0)
        assert torch.equal(o, to_device(x["v"], dtype))


@pytest.mark.parametrize("name", ["decoder_window512_causal_bf16_b4h32n4096d128",
                                  "longctx_window512_causal_bf16_b1h32n16384d128"])
def test_window_sampled_rows_full_size(name, oracle_impl):
    """The measured windowed workloads at full size: sampled rows against the oracle."""
    w = inputs.WORKLOADS[name]
    log(f"[window] {name} (sampled rows)")
    x = inputs.make_inputs(w)
    o, lse = run(x, w.dtype, w.causal, window=w.window)
    rows = sample_rows(w, 160)
    ro, rl = oracle_impl.attn_rows(x["q"], x["k"], x["v"], w.dtype, float(x["scale"]), w.causal,
                                   x["key_lens"], rows, window=w.window)
    eo, el = compare(o, lse, ro, rl, w.dtype, name, rows=rows)
    log(f"[window] {name}: {rows.size} rows, max|dO|={eo:.3e} max|dLSE|={el:.3e}")


def test_invalid_window_writes_nothing():
    q = torch.randn(1, 2, 64, 64, device="cuda", dtype=torch.bfloat16)
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 2, 64), 7.0, device="cuda")
    P = lambda t: t.data_ptr()
    for bad in (-2, -1000):
        rc = binding.attn_fwd_window(P(q), P(q), P(q), P(o), P(lse), 1, 2, 64, 64, 64, 0.125, 0, bad,
                                     None, 2, None)
        assert rc == -9
    with pytest.raises(ValueError):
        binding.fwd(q, q, q, window=-3)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
