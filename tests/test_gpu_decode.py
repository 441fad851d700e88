"""KV-cache decode (attn_decode) on the HIP path against the fp64 oracle (needs an MI355X).

The Nq queries are the last Nq positions of each cached sequence: with causal set, query i
sees keys j <= i + L_b - Nq (the oracle's causal=2).  Long caches are split over several
workgroups whose partial results are merged by log-sum-exp; every expected value comes from
oracle/, from the golden fixture or from a closed form.  Tolerances as in test_gpu_parity.py.
"""
import json
import os

import numpy as np
import pytest
import torch

import pins
from gpu_util import TOL_LSE, TOL_O, compare, run, run_decode, to_device, to_f64
from transformer_scaled_dot_amd import binding, inputs

pytestmark = pytest.mark.gpu

CODE = {"f32": 0, "f16": 1, "bf16": 2}


def log(msg):
    print(msg, flush=True)


def oracle_causal(causal):
    return 2 if causal else 0


# name, B, H, Nq, Nk, D, key_lens -- the comment gives the key split the sizes lead to
SHAPES = [
    ("q1_k5000_d128", 2, 4, 1, 5000, 128, None),                  # 16 splits, ragged last one
    ("q1_k100_d64", 1, 8, 1, 100, 64, None),                      # too short to split
    ("q4_k3000_d64_pad", 3, 2, 4, 3000, 64, [3000, 1777, 2]),     # 10 splits; L < Nq
    ("q17_k33000_d128", 1, 4, 17, 33000, 128, None),              # 58 splits
    ("q200_k1000_d64", 2, 2, 200, 1000, 64, None),                # 2 Q tiles x 3 splits
    ("q33_k700_d128_pad", 2, 3, 33, 700, 128, [700, 40]),         # 2 splits, one empty
    ("q64_k64_d128", 1, 2, 64, 64, 128, None),                    # Nq = Nk: top-left causal
    ("q1_k1_d64", 1, 1, 1, 1, 64, None),
    ("q3_k2048_d64_empty", 2, 2, 3, 2048, 64, [0, 2048]),         # one cache empty
]


def make_x(shape, dtype, seed=31):
    name, B, H, Nq, Nk, D, kl = shape
    w = inputs.Workload(name, dtype, B, H, Nq, Nk, D, True, kl is not None, 1.0, 1.0, seed,
                        kv_cache=True)
    x = inputs.make_inputs(w)
    x["key_lens"] = None if kl is None else np.array(kl, np.int32)
    return x


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_decode_parity(shape, dtype, oracle_impl):
    name, B, H, Nq, Nk, D, _ = shape
    x = make_x(shape, dtype)
    ws = binding.attn_decode_workspace_size(B, H, Nq, Nk, D, CODE[dtype])
    for causal in (False, True):
        log(f"[decode] {name} {dtype} causal={causal} workspace={ws}")
        o, lse = run_decode(x, dtype, causal)
        ro, rl = oracle_impl.attn(x["q"], x["k"], x["v"], dtype, float(x["scale"]),
                                  oracle_causal(causal), x["key_lens"])
        eo, el = compare(o, lse, ro, rl, dtype, f"{name}/{dtype}/causal={causal}")
        log(f"[decode] {name} {dtype} causal={causal}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")


def test_decode_golden_fixture():
    """The 50-digit fixture's cases without a window through attn_decode (D zero-padded to 64):
    bottom-right causal cases as causal, the non-causal ones as non-causal."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "bruteforce_tiny.json")) as f:
        cases = json.load(f)["cases"]
    n = 0
    for cs in cases:
        if cs.get("window") is not None or cs["causal"] is True:
            continue
        for dtype in ("bf16", "f16", "f32"):
            D = cs["D"]
            pad = lambda a: np.pad(np.array(a, np.float64), [(0, 0)] * 3 + [(0, 64 - D)])
            x = {n_: pins.store(pad(cs[n_]), dtype) for n_ in "qkv"}
            x["scale"] = np.float32(cs["scale"])
            x["key_lens"] = None if cs["key_lens"] is None else np.array(cs["key_lens"], np.int32)
            o, lse = run_decode(x, dtype, cs["causal"] == 2)
            o, lse = to_f64(o), to_f64(lse)
            assert np.all(o[..., D:] == 0)
            want_o = np.array(cs["o"], np.float64)
            want_l = np.array([[[float(v) for v in h] for h in b] for b in cs["lse"]])
            assert np.array_equal(np.isfinite(lse), np.isfinite(want_l)), cs["name"]
            assert np.max(np.abs(o[..., :D] - want_o)) <= TOL_O[dtype], cs["name"]
            fin = np.isfinite(want_l)
            assert np.max(np.abs(lse[fin] - want_l[fin]), initial=0) <= TOL_LSE, cs["name"]
        n += 1
    assert n >= 4


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unsplit_decode_is_attn_fwd_bitwise(dtype):
    """A cache too short to split runs the plain kernel: non-causal decode equals attn_fwd bit
    for bit, and with Nq = Nk the bottom-right causal mask is the top-left one."""
    rng = np.random.default_rng(41)
    for (B, H, Nq, Nk, D) in ((2, 3, 1, 300, 128), (2, 3, 5, 511, 64), (1, 2, 130, 130, 128)):
        assert binding.attn_decode_workspace_size(B, H, Nq, Nk, D, CODE[dtype]) == 0
        x = {"q": pins.rand_store(rng, (B, H, Nq, D), dtype),
             "k": pins.rand_store(rng, (B, H, Nk, D), dtype),
             "v": pins.rand_store(rng, (B, H, Nk, D), dtype),
             "scale": np.float32(0.1), "key_lens": None}
        o1, l1 = run(x, dtype, False)
        o2, l2 = run_decode(x, dtype, False)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        if Nq == Nk:
            o1, l1 = run(x, dtype, True)
            o2, l2 = run_decode(x, dtype, True)
            assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_decode_zero_query_mean(dtype):
    """Q = 0 across a split cache: O is the mean of V over the visible keys, LSE = ln(count)."""
    rng = np.random.default_rng(42)
    B, H, Nq, Nk, D = 2, 2, 3, 3000, 64
    v = pins.rand_store(rng, (B, H, Nk, D), dtype)
    x = {"q": pins.store(np.zeros((B, H, Nq, D)), dtype), "k": pins.rand_store(rng, (B, H, Nk, D), dtype),
         "v": v, "scale": np.float32(0.125), "key_lens": np.array([3000, 1501], np.int32)}
    assert binding.attn_decode_workspace_size(B, H, Nq, Nk, D, CODE[dtype]) > 0
    vd = inputs.storage_to_f64(v, dtype)
    for causal in (False, True):
        o, lse = run_decode(x, dtype, causal)
        o, lse = to_f64(o), to_f64(lse)
        for b in range(B):
            L = int(x["key_lens"][b])
            for i in range(Nq):
                n = L - Nq + i + 1 if causal else L
                want = vd[b, :, :n].mean(axis=1)
                assert np.max(np.abs(o[b, :, i] - want)) <= TOL_O[dtype], (causal, b, i)
                assert np.max(np.abs(lse[b, :, i] - np.log(n))) <= TOL_LSE, (causal, b, i)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_dominant_key(dtype):
    """One key aligned with the query and a logit 40 above every other: the output is that key's
    V row wherever the key sits among the splits (the other splits' weights are e^-40)."""
    rng = np.random.default_rng(43)
    B, H, Nq, Nk, D = 1, 2, 1, 4096, 128
    u = np.zeros(D)
    u[:2] = 1.0
    q = np.broadcast_to(u * 4.0, (B, H, Nq, D))
    k = rng.standard_normal((B, H, Nk, D)) * 0.01
    k[..., :2] = 0.0  # every other logit is exactly 0
    for j in (0, 255, 256, 2100, Nk - 1):
        kk = k.copy()
        kk[:, :, j] = u * 5.0  # logit <q, k_j> = 2 * 4 * 5 = 40 (scale 1), exact in every dtype
        x = {"q": pins.store(q, dtype), "k": pins.store(kk, dtype),
             "v": pins.rand_store(rng, (B, H, Nk, D), dtype), "scale": np.float32(1.0), "key_lens": None}
        o, lse = run_decode(x, dtype, True)
        want = inputs.storage_to_f64(x["v"], dtype)[:, :, j:j + 1]
        assert np.max(np.abs(to_f64(o) - want)) <= TOL_O[dtype], j
        assert np.max(np.abs(to_f64(lse) - 40.0)) <= TOL_LSE, j


def test_workspace_errors_write_nothing():
    B, H, Nq, Nk, D = 2, 2, 1, 4096, 64
    need = binding.attn_decode_workspace_size(B, H, Nq, Nk, D, 2)
    assert need > 0
    q = torch.randn(B, H, Nq, D, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(B, H, Nk, D, device="cuda", dtype=torch.bfloat16)
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, H, Nq), 7.0, device="cuda")
    ws = torch.empty(need + 64, dtype=torch.uint8, device="cuda")
    P = lambda t: t.data_ptr()
    args = (P(q), P(k), P(k), P(o), P(lse), B, H, Nq, Nk, D, 0.125, 1, None, 2)
    assert binding.attn_decode(*args, None, need, None) == -1
    assert binding.attn_decode(*args, P(ws) + 8, need, None) == -8
    assert binding.attn_decode(*args, P(ws), need - 1, None) == -10
    assert binding.attn_decode(*args, P(ws), 0, None) == -10
    with pytest.raises(binding.AttnError):
        binding.decode(q, k, k, causal=True, workspace=ws[: need - 16])
    with pytest.raises(ValueError):
        binding.decode(q, k, k, workspace=torch.empty(need, dtype=torch.uint8))
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())


def test_workspace_reuse(oracle_impl):
    """One caller-owned workspace (larger than needed) for two calls in a row, the second with a
    smaller cache: both match the oracle."""
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    for shape in (("a", 2, 4, 2, 6000, 128, [6000, 4500]), ("b", 1, 4, 1, 2500, 128, None)):
        x = make_x(shape, "bf16", seed=44)
        _, B, H, Nq, Nk, D, _ = shape
        assert 0 < binding.attn_decode_workspace_size(B, H, Nq, Nk, D, 2) <= ws.numel()
        o, lse = run_decode(x, "bf16", True, workspace=ws)
        ro, rl = oracle_impl.attn(x["q"], x["k"], x["v"], "bf16", float(x["scale"]), 2, x["key_lens"])
        compare(o, lse, ro, rl, "bf16", shape[0])


@pytest.mark.parametrize("name", [n for n, w in inputs.WORKLOADS.items() if w.kv_cache])
def test_decode_workloads_full_size(name, oracle_impl):
    """The measured decode workloads at full size, every row against the oracle."""
    w = inputs.WORKLOADS[name]
    log(f"[decode] {name} (all {w.B * w.H * w.Nq} rows)")
    x = inputs.make_inputs(w)
    o, lse = run_decode(x, w.dtype, w.causal)
    ro, rl = oracle_impl.attn(x["q"], x["k"], x["v"], w.dtype, float(x["scale"]),
                              oracle_causal(w.causal), x["key_lens"])
    eo, el = compare(o, lse, ro, rl, w.dtype, name)
    log(f"[decode] {name}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")


def test_decode_determinism_bitwise():
    w = inputs.WORKLOADS["kvdecode_bf16_b4h32q1k4096d128"]
    x = inputs.make_inputs(w)
    o1, l1 = run_decode(x, w.dtype, w.causal)
    for _ in range(3):
        o2, l2 = run_decode(x, w.dtype, w.causal)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
