"""Parity of the HIP path with the fp64 oracle, through the C ABI (needs an MI355X).

Every input comes from the seeded generator; every expected value from oracle/ (or from a
closed form).  Tolerances: max |dO| <= 2e-2 for bf16/fp16 storage, 1e-4 for fp32, and
max |dLSE| <= 1e-3; the -inf pattern of LSE (empty rows) must match exactly.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import pins
from gpu_util import TOL_LSE, TOL_O, compare, run, sample_rows, to_device, to_f64
from transformer_scaled_dot_amd import binding, inputs

pytestmark = pytest.mark.gpu

SMALL = ["tiny_f32_b1h2n128d64", "ragged_f16_b2h8n100d64", "bert_bf16_b32h12n512d64_pad",
         "bert_bf16_b32h12n512d64_pad_stress"]
LARGE = ["decoder_causal_bf16_b4h32n4096d128", "longctx_causal_bf16_b1h32n16384d128"]


def log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name", SMALL)
def test_parity_full_workload(name, oracle_impl):
    w = inputs.WORKLOADS[name]
    log(f"[parity] {name}")
    x = inputs.make_inputs(w)
    o, lse = run(x, w.dtype, w.causal)
    ro, rl = oracle_impl.attn(x["q"], x["k"], x["v"], w.dtype, float(x["scale"]), w.causal,
                              x["key_lens"])
    eo, el = compare(o, lse, ro, rl, w.dtype, name)
    log(f"[parity] {name}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")


@pytest.mark.parametrize("name", LARGE)
def test_parity_sampled_rows_full_size(name, oracle_impl):
    """Full-size workloads in the benchmark's launch configuration: sampled rows against the
    oracle, and at every row the properties that hold at any size."""
    w = inputs.WORKLOADS[name]
    log(f"[parity] {name} (sampled rows)")
    x = inputs.make_inputs(w)
    o, lse = run(x, w.dtype, w.causal)
    rows = sample_rows(w, 192)
    ro, rl = oracle_impl.attn_rows(x["q"], x["k"], x["v"], w.dtype, float(x["scale"]), w.causal,
                                   x["key_lens"], rows)
    eo, el = compare(o, lse, ro, rl, w.dtype, name, rows=rows)
    log(f"[parity] {name}: {rows.size} rows, max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    # every row: O is a convex combination of V rows, LSE finite
    vmax = float(torch.from_numpy(inputs.storage_to_f64(x["v"], w.dtype)).abs().max())
    assert torch.isfinite(lse).all()
    assert float(o.float().abs().max()) <= vmax + TOL_O[w.dtype]
    # causal row 0 of every (b, h) copies V[0] exactly
    v0 = to_device(x["v"], w.dtype)[:, :, 0]
    assert torch.equal(o[:, :, 0], v0)


def test_parity_every_row_decoder_4k(oracle_impl):
    """The 4K causal workload (B=4, H=32, D=128) at full size, in the benchmark's launch
    configuration: every one of its 524,288 rows against the oracle."""
    name = "decoder_causal_bf16_b4h32n4096d128"
    w = inputs.WORKLOADS[name]
    log(f"[parity] {name} (every row)")
    x = inputs.make_inputs(w)
    o, lse = run(x, w.dtype, w.causal)
    ro, rl = oracle_impl.attn(x["q"], x["k"], x["v"], w.dtype, float(x["scale"]), w.causal, x["key_lens"])
    eo, el = compare(o, lse, ro, rl, w.dtype, name)
    log(f"[parity] {name}: all {w.B * w.H * w.Nq} rows, max|dO|={eo:.3e} max|dLSE|={el:.3e}")


_LONGCTX = "longctx_causal_bf16_b1h32n16384d128"
_LONGCTX_RUN = {}


def _longctx_run():
    """Inputs and GPU outputs of the 16K causal workload, computed once for the tests below."""
    if not _LONGCTX_RUN:
        w = inputs.WORKLOADS[_LONGCTX]
        x = inputs.make_inputs(w)
        o, lse = run(x, w.dtype, w.causal)
        _LONGCTX_RUN.update(w=w, x=x, o=o, lse=lse)
    return _LONGCTX_RUN


@pytest.mark.parametrize("first_head", [0, 8, 16, 24])
def test_parity_every_row_longctx_16k(first_head, oracle_impl):
    """The 16K causal workload (B=1, H=32, D=128) at full size, in the benchmark's launch
    configuration: every row of heads first_head .. first_head + 7 against the oracle, so the four
    cases together cover all 524,288 rows (one launch, checked in four parts of ~25 s of oracle
    work each)."""
    r = _longctx_run()
    w, x, o, lse = r["w"], r["x"], r["o"], r["lse"]
    log(f"[parity] {_LONGCTX} heads {first_head}..{first_head + 7} (every row)")
    rows = np.arange(first_head * w.Nq, (first_head + 8) * w.Nq, dtype=np.int64)
    ro, rl = oracle_impl.attn_rows(x["q"], x["k"], x["v"], w.dtype, float(x["scale"]), w.causal,
                                   x["key_lens"], rows)
    eo, el = compare(o, lse, ro, rl, w.dtype, _LONGCTX, rows=rows)
    log(f"[parity] {_LONGCTX} heads {first_head}..{first_head + 7}: {rows.size} rows, "
        f"max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    if first_head == 24:
        _LONGCTX_RUN.clear()


# ------------------------------------------------------------------ long sequences
# More than 8K query rows at D = 128 (no band, no key split) run the 256-row, 8-wave workgroups;
# everything else the 128-row, 4-wave ones.  Both give each wave the same 32 rows and the same
# per-row arithmetic, so besides the oracle the 8-wave output must equal, bit for bit, that of a
# call with a band of width max(Nq, Nk) - 1 (no key is outside it, but a band keeps the 4-wave
# workgroups).
LONG = [
    # name, dtype, B, H, Nq, Nk, causal, key_lens
    ("long_causal_ragged_bf16", "bf16", 1, 2, 8300, 8300, True, None),
    ("long_causal_ragged_f16", "f16", 1, 2, 8300, 8300, True, None),
    ("long_noncausal_lens_bf16", "bf16", 2, 1, 8200, 8200, False, [5000, 8200]),
    ("long_causal_lens_f16", "f16", 2, 1, 8400, 8400, True, [8400, 3001]),
    ("long_causal_nq_gt_nk_bf16", "bf16", 1, 1, 9000, 4000, True, None),
    ("long_causal_nq_lt_nk_bf16", "bf16", 1, 1, 8500, 12000, True, None),
    # either side of the switch: 8192 rows keep the 4-wave workgroups, 8193 take the 8-wave ones
    # (whose last 256-row tile then holds a single row)
    ("boundary_8192_bf16", "bf16", 1, 2, 8192, 8192, True, None),
    ("boundary_8193_bf16", "bf16", 1, 2, 8193, 8193, True, None),
]


@pytest.mark.parametrize("case", LONG, ids=[c[0] for c in LONG])
def test_long_sequence_workgroups(case, oracle_impl):
    name, dtype, B, H, Nq, Nk, causal, kl = case
    log(f"[long] {name}")
    w = inputs.Workload(name, dtype, B, H, Nq, Nk, 128, causal, kl is not None, 0.5, 1.0, 91)
    x = inputs.make_inputs(w)
    if kl is not None:
        x["key_lens"] = np.array(kl, np.int32)
    o, lse = run(x, dtype, causal)
    o4, lse4 = run(x, dtype, causal, window=max(Nq, Nk) - 1)
    assert torch.equal(o.view(torch.int16), o4.view(torch.int16)), f"{name}: O differs from the 4-wave launch"
    assert torch.equal(lse, lse4), f"{name}: LSE differs from the 4-wave launch"
    rows = sample_rows(w, 512, block_m=256)
    ro, rl = oracle_impl.attn_rows(x["q"], x["k"], x["v"], dtype, float(x["scale"]), causal,
                                   x["key_lens"], rows)
    eo, el = compare(o, lse, ro, rl, dtype, name, rows=rows)
    log(f"[long] {name}: {rows.size} rows, max|dO|={eo:.3e} max|dLSE|={el:.3e}")


# ------------------------------------------------------------------ edge cases
EDGE = [
    # name, B, H, Nq, Nk, D, causal, key_lens, scale
    ("one_by_one", 1, 1, 1, 1, 64, False, None, None),
    ("single_query_long_keys", 1, 2, 1, 300, 128, False, None, None),
    ("causal_topleft_nq_lt_nk", 1, 2, 77, 200, 64, True, None, None),
    ("causal_topleft_nq_gt_nk", 1, 2, 200, 77, 128, True, None, None),
    ("ragged_causal_129", 2, 1, 129, 129, 128, True, None, None),
    ("ragged_191_noncausal", 1, 3, 191, 191, 64, False, None, None),
    ("lens_edges", 7, 2, 70, 130, 64, False, [0, 1, 63, 64, 65, 1000, -5], None),
    ("lens_edges_causal", 7, 1, 130, 130, 128, True, [0, 1, 63, 64, 65, 1000, -5], None),
    ("negative_scale", 1, 2, 96, 96, 64, False, None, -0.2),
    ("zero_scale_causal", 1, 2, 96, 96, 128, True, None, 0.0),
    ("big_scale", 1, 1, 64, 200, 64, False, None, 3.0),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge_cases(case, dtype, oracle_impl):
    name, B, H, Nq, Nk, D, causal, kl, scale = case
    log(f"[edge] {name} {dtype}")
    w = inputs.Workload(name, dtype, B, H, Nq, Nk, D, causal, kl is not None, 1.0, 1.0, 77,
                        scale=scale)
    x = inputs.make_inputs(w)
    if kl is not None:
        x["key_lens"] = np.array(kl, np.int32)
    o, lse = run(x, dtype, causal)
    ro, rl = oracle_impl.attn(x["q"], x["k"], x["v"], dtype, float(x["scale"]), causal, x["key_lens"])
    eo, el = compare(o, lse, ro, rl, dtype, f"{name}/{dtype}")
    log(f"[edge] {name} {dtype}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")


# ------------------------------------------------------------------ closed forms on the kernel
def _kernel(q, k, v, dtype, scale, causal=False, key_lens=None, window=None):
    x = {"q": q, "k": k, "v": v, "scale": np.float32(scale), "key_lens": key_lens}
    return run(x, dtype, causal, window=window)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_kernel_zero_query_mean(dtype, D):
    rng = np.random.default_rng(1)
    B, H, N = 3, 2, 150
    q = pins.store(np.zeros((B, H, N, D)), dtype)
    k = pins.rand_store(rng, (B, H, N, D), dtype)
    v = pins.rand_store(rng, (B, H, N, D), dtype)
    kl = np.array([150, 70, 1], np.int32)
    vd = inputs.storage_to_f64(v, dtype)
    for causal in (False, True):
        o, lse = _kernel(q, k, v, dtype, 0.125, causal, kl)
        o, lse = to_f64(o), to_f64(lse)
        for b in range(B):
            n = np.minimum(np.arange(N) + 1, kl[b]) if causal else np.full(N, kl[b])
            csum = np.cumsum(vd[b], axis=1)  # [H, N, D]
            want = csum[:, n - 1] / n[None, :, None]
            assert np.max(np.abs(o[b] - want)) <= TOL_O[dtype]
            assert np.max(np.abs(lse[b] - np.log(n)[None])) <= TOL_LSE


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_kernel_causal_row0_and_single_key_exact(dtype):
    rng = np.random.default_rng(2)
    q, k, v = (pins.rand_store(rng, (2, 3, 70, 128), dtype) for _ in range(3))
    o, _ = _kernel(q, k, v, dtype, 0.09, True)
    assert torch.equal(o[:, :, 0], to_device(v, dtype)[:, :, 0])
    k1, v1 = (pins.rand_store(rng, (2, 3, 1, 64), dtype) for _ in range(2))
    q1 = pins.rand_store(rng, (2, 3, 40, 64), dtype)
    o, lse = _kernel(q1, k1, v1, dtype, 0.125, False)
    assert torch.equal(o, to_device(v1, dtype).expand_as(o).contiguous())
    s = (inputs.storage_to_f64(q1, dtype) * inputs.storage_to_f64(k1, dtype)).sum(-1) * np.float32(0.125)
    assert np.max(np.abs(to_f64(lse) - s)) <= TOL_LSE


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_kernel_rows_sum_to_one(dtype):
    """V = 1 gives O = 1: the weights fed to P.V and the sum used to normalise agree."""
    rng = np.random.default_rng(3)
    q, k = (pins.rand_store(rng, (2, 4, 333, 128), dtype, 2.0) for _ in range(2))
    v = pins.store(np.ones((2, 4, 333, 128)), dtype)
    for causal in (False, True):
        o, _ = _kernel(q, k, v, dtype, 0.2, causal, np.array([333, 100], np.int32))
        assert float((o.double() - 1).abs().max()) <= TOL_O[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_kernel_query_permutation_bitwise(dtype):
    rng = np.random.default_rng(4)
    q = pins.rand_store(rng, (1, 2, 256, 64), dtype)
    k, v = (pins.rand_store(rng, (1, 2, 192, 64), dtype) for _ in range(2))
    o, lse = _kernel(q, k, v, dtype, 0.125)
    perm = rng.permutation(256)
    o2, lse2 = _kernel(np.ascontiguousarray(q[:, :, perm]), k, v, dtype, 0.125)
    pt = torch.from_numpy(perm).cuda()
    assert torch.equal(o2, o[:, :, pt]) and torch.equal(lse2, lse[:, :, pt])
    # joint K/V permutation: same result up to summation order
    pk = rng.permutation(192)
    o3, lse3 = _kernel(q, np.ascontiguousarray(k[:, :, pk]), np.ascontiguousarray(v[:, :, pk]), dtype, 0.125)
    assert float((o3.double() - o.double()).abs().max()) <= TOL_O[dtype]
    assert float((lse3 - lse).abs().max()) <= TOL_LSE


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_kernel_one_hot_dominant_key(dtype):
    rng = np.random.default_rng(5)
    D, N, jstar, c = 64, 300, 77, 16.0
    q = np.zeros((1, 1, N, D))
    q[..., 0] = c
    k = np.zeros((1, 1, N, D))
    k[0, 0, jstar, 0] = c
    v = pins.rand_store(rng, (1, 1, N, D), dtype)
    vd = inputs.storage_to_f64(v, dtype)[0, 0]
    g = c * c / 8
    for causal in (False, True):
        o, lse = _kernel(pins.store(q, dtype), pins.store(k, dtype), v, dtype, 0.125, causal)
        o, lse = to_f64(o)[0, 0], to_f64(lse)[0, 0]
        for i in range(N):
            n = i + 1 if causal else N
            if causal and i < jstar:
                want, wl = vd[:n].mean(0), math.log(n)
            else:
                eg = math.exp(g)
                want = (eg * vd[jstar] + vd[:n].sum(0) - vd[jstar]) / (eg + n - 1)
                wl = g + math.log1p((n - 1) * math.exp(-g))
            assert np.max(np.abs(o[i] - want)) <= TOL_O[dtype]
            assert abs(lse[i] - wl) <= TOL_LSE


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kernel_key_shift(dtype):
    rng = np.random.default_rng(6)
    B, H, N, D = 1, 2, 140, 64
    q = rng.integers(-3, 4, (B, H, N, D)).astype(np.float64)
    k = rng.integers(-3, 4, (B, H, N, D)).astype(np.float64)
    c = rng.integers(-2, 3, D).astype(np.float64)
    v = pins.rand_store(rng, (B, H, N, D), dtype)
    scale = 0.03125
    for causal in (False, True):
        o, lse = _kernel(pins.store(q, dtype), pins.store(k, dtype), v, dtype, scale, causal)
        o2, lse2 = _kernel(pins.store(q, dtype), pins.store(k + c, dtype), v, dtype, scale, causal)
        assert float((o2.double() - o.double()).abs().max()) <= TOL_O[dtype]
        d = to_f64(lse2) - to_f64(lse) - scale * (q @ c)
        assert np.max(np.abs(d)) <= TOL_LSE


def test_kernel_golden_bruteforce():
    """The 50-digit fixture, with D zero-padded to 64 (zeros change no dot product; padded V
    columns must come out exactly 0)."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "bruteforce_tiny.json")) as f:
        cases = json.load(f)["cases"]
    for cs in cases:
        if cs["causal"] == 2:
            continue  # queries at the end of a KV cache: attn_decode's cases (test_gpu_decode.py)
        for dtype in ("bf16", "f16", "f32"):
            D = cs["D"]
            pad = lambda a: np.pad(np.array(a, np.float64), [(0, 0)] * 3 + [(0, 64 - D)])
            q, k, v = (pins.store(pad(cs[n]), dtype) for n in "qkv")
            kl = None if cs["key_lens"] is None else np.array(cs["key_lens"], np.int32)
            o, lse = _kernel(q, k, v, dtype, cs["scale"], cs["causal"], kl, cs.get("window"))
            o, lse = to_f64(o), to_f64(lse)
            assert np.all(o[..., D:] == 0)
            want_o = np.array(cs["o"], np.float64)
            want_l = np.array([[[float(x) for x in h] for h in b] for b in cs["lse"]])
            assert np.array_equal(np.isfinite(lse), np.isfinite(want_l)), cs["name"]
            assert np.max(np.abs(o[..., :D] - want_o)) <= TOL_O[dtype], cs["name"]
            fin = np.isfinite(want_l)
            assert np.max(np.abs(lse[fin] - want_l[fin]), initial=0) <= TOL_LSE, cs["name"]


# ------------------------------------------------------------------ determinism, ABI behaviour
def test_determinism_bitwise():
    w = inputs.WORKLOADS["bert_bf16_b32h12n512d64_pad"]
    x = inputs.make_inputs(w)
    o1, l1 = run(x, w.dtype, w.causal)
    for _ in range(3):
        o2, l2 = run(x, w.dtype, w.causal)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_invalid_arguments_write_nothing():
    q = torch.randn(1, 2, 64, 64, device="cuda", dtype=torch.bfloat16)
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 2, 64), 7.0, device="cuda")
    P = lambda t: t.data_ptr()
    args = dict(B=1, H=2, Nq=64, Nk=64, D=64, scale=0.125, causal=0, key_lens=None, dtype=2, stream=None)
    bad = [
        (dict(D=96), -3),
        (dict(B=0), -2),
        (dict(Nk=0), -2),
        (dict(dtype=9), -4),
        (dict(scale=float("nan")), -5),
        (dict(scale=float("inf")), -5),
        (dict(causal=2), -7),
        (dict(Nq=(1 << 29) // 64), -2),
    ]
    for over, code in bad:
        a = {**args, **over}
        rc = binding.attn_fwd(P(q), P(q), P(q), P(o), P(lse), a["B"], a["H"], a["Nq"], a["Nk"], a["D"],
                              a["scale"], a["causal"], a["key_lens"], a["dtype"], a["stream"])
        assert rc == code, (over, rc)
    rc = binding.attn_fwd(None, P(q), P(q), P(o), P(lse), 1, 2, 64, 64, 64, 0.125, 0, None, 2, None)
    assert rc == -1
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_guard_bands_untouched(dtype):
    """Outputs are written exactly in place: canaries before and after O and LSE survive."""
    rng = np.random.default_rng(7)
    B, H, N, D = 2, 3, 200, 128
    x = {"q": pins.rand_store(rng, (B, H, N, D), dtype), "k": pins.rand_store(rng, (B, H, N, D), dtype),
         "v": pins.rand_store(rng, (B, H, N, D), dtype), "scale": np.float32(0.088), "key_lens": None}
    q, k, v = (to_device(x[n], dtype) for n in "qkv")
    G = 4096
    tdt = q.dtype
    obuf = torch.full((G + q.numel() + G,), -3.0, dtype=tdt, device="cuda")
    lbuf = torch.full((G + B * H * N + G,), -3.0, dtype=torch.float32, device="cuda")
    o = obuf[G:G + q.numel()].view(B, H, N, D)
    lse = lbuf[G:G + B * H * N].view(B, H, N)
    binding.fwd(q, k, v, causal=True, scale=0.088, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool((obuf[:G] == -3.0).all()) and bool((obuf[-G:] == -3.0).all())
    assert bool((lbuf[:G] == -3.0).all()) and bool((lbuf[-G:] == -3.0).all())
    assert bool(torch.isfinite(o.float()).all())


def test_no_device_allocation_by_the_library():
    w = inputs.WORKLOADS["decoder_causal_bf16_b4h32n4096d128"].with_(B=1, H=4)
    x = inputs.make_inputs(w)
    q, k, v = (to_device(x[n], "bf16") for n in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], device="cuda")
    binding.fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(5):
        binding.fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0
