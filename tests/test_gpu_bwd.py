"""Attention backward (attn_bwd) on the HIP path against the fp64 oracle (needs an MI355X).

The forward runs on the GPU (attn_fwd) to produce the O and LSE the backward takes; the
expected gradients come from oracle.attn_bwd on the same stored inputs.  Tolerance, per
gradient tensor: max |GPU - oracle| <= 2e-2 * max |oracle| for bf16 / fp16 (the forward's bf16
bound applied to the gradient scaled to unit size: P and dS are rounded to the input type
before their products, a relative error of about 2^-9 per term), with max |oracle| taken at least
1e-3; for fp32 storage (fp32 throughout) 1e-4 * max |oracle|, the forward's fp32 bound, with
max |oracle| taken at least 0.1; gradient rows that are zero by structure (keys no row may see,
rows that see no key) must be exactly zero.
"""
import numpy as np
import pytest
import torch

from gpu_util import to_device, to_f64
from transformer_scaled_dot_amd import binding, inputs

pytestmark = pytest.mark.gpu

# (relative bound, floor of max |oracle|) per storage type.  A gradient that is zero only by
# exact cancellation (one visible key per row: dP = Dr) keeps an fp32 residue of about 1e-6 on
# the GPU, where dP and Dr are formed separately; the bound never drops below 2e-5 (bf16, fp16)
# or 1e-5 (fp32).
TOLS = {"bf16": (2e-2, 1e-3), "f16": (2e-2, 1e-3), "f32": (1e-4, 1e-1)}
# Per-row check: each gradient row's error relative to its own largest entry (floored at
# ROW_FLOOR of the tensor's largest entry), so that a small row cannot hide a wrong result
# behind the tensor-wide bound.  The bound is looser than the tensor-wide one because a row's
# gradient can be much smaller than the terms summed into it: dq_i = sum_j dS_ij k_j with
# sum_j dS_ij = 0, so the rounding of dS to the input type (2^-9 relative per term) is measured
# against a partly cancelled sum (early causal rows, with few keys, show up to ~9 %).
ROW_FLOOR = 0.05
ROW_TOL = {"bf16": 0.25, "f16": 0.25, "f32": 1e-2}


def log(msg):
    print(msg, flush=True)


def run_fwd_bwd(x, dtype, causal, dlse=None, scale=None, window=None):
    """GPU forward then backward on stored inputs x (q, k, v, do, key_lens, scale)."""
    q, k, v, do = (to_device(x[n], dtype) for n in ("q", "k", "v", "do"))
    kl = None if x.get("key_lens") is None else torch.from_numpy(np.asarray(x["key_lens"], np.int32)).cuda()
    s = float(x["scale"]) if scale is None else float(scale)
    o, lse = binding.fwd(q, k, v, causal=causal, key_lens=kl, scale=s, window=window)
    g = None if dlse is None else torch.from_numpy(np.asarray(dlse, np.float32)).cuda()
    dq, dk, dv = binding.bwd(q, k, v, o, lse, do, causal=causal, key_lens=kl, scale=s, dlse=g, window=window)
    torch.cuda.synchronize()
    return dq, dk, dv


def unseen(x, causal, H, bh=None, window=None):
    """Masks of gradient rows that are zero by structure: dq rows that see no valid key, dk / dv
    rows of keys that no query row may see."""
    B, _, Nq, _ = x["q"].shape
    Nk = x["k"].shape[2]
    kl = np.full(B, Nk) if x.get("key_lens") is None else np.clip(np.asarray(x["key_lens"]), 0, Nk)
    i = np.arange(Nq)[None, :]
    j = np.arange(Nk)[None, :]
    L = np.repeat(kl, H)[:, None]
    lo = np.maximum(i - window, 0) if window is not None else np.zeros_like(i)
    hi = np.minimum(L, i + 1) if causal else np.broadcast_to(L, (L.shape[0], Nq))
    if window is not None:
        hi = np.minimum(hi, i + window + 1)
    rows = hi <= lo                                                            # [B*H, Nq]
    first = np.maximum(j - window, 0) if window is not None else np.zeros_like(j)
    if causal:
        first = np.maximum(first, j)
    keys = (j >= L) | (first > Nq - 1)                                         # [B*H, Nk]
    if bh is not None:
        rows, keys = rows[bh], keys[bh]
    return rows, keys


def compare_grads(got, want, what, bh=None, zero_rows=None, dtype="bf16"):
    tol, floor = TOLS[dtype]
    for n, (name, a, b) in enumerate(zip(("dq", "dk", "dv"), got, want)):
        a = to_f64(a)
        if bh is not None:
            a = a.reshape(-1, *a.shape[2:])[bh]
        b = np.asarray(b).reshape(a.shape)
        assert np.all(np.isfinite(a)), f"{what} {name}: non-finite"
        if zero_rows is not None:
            z = zero_rows[0 if n == 0 else 1].reshape(a.shape[:-1])
            assert np.all(a[z] == 0.0) and np.all(b[z] == 0.0), f"{what} {name}: rows that must be zero"
        scale = float(np.max(np.abs(b))) if b.size else 0.0
        err = float(np.max(np.abs(a - b))) if b.size else 0.0
        assert err <= tol * max(scale, floor), f"{what} {name}: max err {err:.3e} vs max |ref| {scale:.3e}"
        if b.size:
            # per row (one query's dq, one key's dk / dv): the error relative to that row's own
            # largest entry, with rows below ROW_FLOOR of the tensor's largest entry measured
            # against that floor instead (their size is set by cancellation, not by the inputs)
            ra, rb = a.reshape(-1, a.shape[-1]), b.reshape(-1, b.shape[-1])
            row_scale = np.maximum(np.max(np.abs(rb), axis=1), max(ROW_FLOOR * scale, floor))
            row_err = float(np.max(np.max(np.abs(ra - rb), axis=1) / row_scale))
            log(f"[bwd] {what} {name}: max err / max|ref| = {err / max(scale, floor):.3e}, "
                f"worst row err / row max|ref| = {row_err:.3e}")
            assert row_err <= ROW_TOL[dtype], f"{what} {name}: worst row error {row_err:.3e}"
        log(f"[bwd] {what} {name}: max err {err:.3e} (max |ref| {scale:.3e}, ratio {err / max(scale, 1e-30):.2e})")


def make(B, H, Nq, Nk, D, dtype, seed, kl=None, sigma=1.0):
    w = inputs.Workload("t", dtype, B, H, Nq, Nk, D, False, False, sigma, 1.0, seed)
    x = inputs.make_inputs(w)
    x["do"] = inputs.make_grad_out(w)
    x["key_lens"] = None if kl is None else np.array(kl, np.int32)
    return x


# name, B, H, Nq, Nk, D, key_lens
SHAPES = [
    ("n128_d64", 1, 2, 128, 128, 64, None),
    ("n300_d128", 2, 3, 300, 300, 128, None),
    ("nq130_nk257_d64", 2, 2, 130, 257, 64, None),
    ("nq257_nk130_d128", 1, 2, 257, 130, 128, None),
    ("padded_n200_d64", 4, 2, 200, 200, 64, [200, 150, 9, 0]),
    ("padded_q33_k700_d128", 2, 3, 33, 700, 128, [700, 40]),
    ("n1_d64", 1, 1, 1, 1, 64, None),
    ("n517_d128", 1, 2, 517, 517, 128, None),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_bwd_parity(shape, dtype, oracle_impl):
    name, B, H, Nq, Nk, D, kl = shape
    x = make(B, H, Nq, Nk, D, dtype, 51, kl)
    rng = np.random.default_rng(52)
    for causal in (False, True):
        for with_g in (False, True):
            g = rng.standard_normal((B, H, Nq)).astype(np.float32) if with_g else None
            log(f"[bwd] {name} {dtype} causal={causal} dlse={with_g}")
            got = run_fwd_bwd(x, dtype, causal, g)
            want = oracle_impl.attn_bwd(x["q"], x["k"], x["v"], x["do"], dtype, float(x["scale"]), causal,
                                        x["key_lens"], g)
            compare_grads(got, want, f"{name}/{dtype}/causal={causal}/dlse={with_g}",
                          zero_rows=unseen(x, causal, H), dtype=dtype)


WIN_SHAPES = [
    ("n300_d128", 2, 3, 300, 300, 128, None),
    ("nq130_nk257_d64", 2, 2, 130, 257, 64, None),
    ("padded_n200_d64", 4, 2, 200, 200, 64, [200, 150, 9, 0]),
    ("n517_d128", 1, 2, 517, 517, 128, None),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", WIN_SHAPES, ids=[s[0] for s in WIN_SHAPES])
def test_bwd_window_parity(shape, dtype, oracle_impl):
    """Backward of sliding-window attention against the oracle, bands from 0 to wider than a tile."""
    name, B, H, Nq, Nk, D, kl = shape
    x = make(B, H, Nq, Nk, D, dtype, 56, kl)
    rng = np.random.default_rng(57)
    for causal in (False, True):
        for w in (0, 1, 31, 64, 100, 255):
            g = rng.standard_normal((B, H, Nq)).astype(np.float32) if w % 2 else None
            log(f"[bwd] {name} {dtype} causal={causal} window={w}")
            got = run_fwd_bwd(x, dtype, causal, g, window=w)
            want = oracle_impl.attn_bwd(x["q"], x["k"], x["v"], x["do"], dtype, float(x["scale"]), causal,
                                        x["key_lens"], g, window=w)
            compare_grads(got, want, f"{name}/{dtype}/causal={causal}/w={w}",
                          zero_rows=unseen(x, causal, H, window=w), dtype=dtype)


def test_bwd_wide_window_is_no_window_bitwise():
    x = make(2, 2, 333, 333, 128, "bf16", 58, [333, 100])
    for causal in (False, True):
        a = run_fwd_bwd(x, "bf16", causal)
        for w in (333, 10 ** 6):
            b = run_fwd_bwd(x, "bf16", causal, window=w)
            assert all(torch.equal(t1, t2) for t1, t2 in zip(a, b)), w


def test_bwd_window_full_size_slices(oracle_impl):
    """The 4K decoder workload with a band of 512, whole (b, h) slices against the oracle."""
    w = inputs.WORKLOADS["decoder_window512_causal_bf16_b4h32n4096d128"]
    x = inputs.make_inputs(w)
    x["do"] = inputs.make_grad_out(w)
    got = run_fwd_bwd(x, w.dtype, w.causal, window=w.window)
    bh = np.array([0, 77, 127])
    want = oracle_impl.attn_bwd(x["q"], x["k"], x["v"], x["do"], w.dtype, float(x["scale"]), w.causal,
                                x["key_lens"], None, bh, window=w.window)
    compare_grads(got, want, "decoder window 512", bh=bh, zero_rows=unseen(x, w.causal, w.H, bh, w.window))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [-0.1, 0.0, 0.3])
def test_bwd_scale_values(scale, dtype, oracle_impl):
    """A negative scale (moved onto Q or K as a sign flip), zero and a large one."""
    x = make(2, 2, 150, 170, 128, dtype, 53, [170, 77])
    x["scale"] = np.float32(scale)
    for causal in (False, True):
        got = run_fwd_bwd(x, dtype, causal)
        want = oracle_impl.attn_bwd(x["q"], x["k"], x["v"], x["do"], dtype, float(x["scale"]), causal,
                                    x["key_lens"])
        compare_grads(got, want, f"{dtype}/scale={scale}/causal={causal}", zero_rows=unseen(x, causal, 2),
                      dtype=dtype)


def test_bwd_stress_logits(oracle_impl):
    """Q and K scaled x8 (logits of std ~64): P is sharply peaked."""
    x = make(2, 2, 200, 200, 64, "bf16", 54, [200, 131], sigma=8.0)
    for causal in (False, True):
        got = run_fwd_bwd(x, "bf16", causal)
        want = oracle_impl.attn_bwd(x["q"], x["k"], x["v"], x["do"], "bf16", float(x["scale"]), causal,
                                    x["key_lens"])
        compare_grads(got, want, f"stress/causal={causal}", zero_rows=unseen(x, causal, 2))


@pytest.mark.parametrize("name,bh", [
    ("bert_bf16_b32h12n512d64_pad", [0, 100, 383]),
    ("decoder_causal_bf16_b4h32n4096d128", [0, 127]),
    ("longctx_causal_bf16_b1h32n16384d128", [31]),
])
def test_bwd_workloads_sampled_slices(name, bh, oracle_impl):
    """The forward workloads at full size through the backward (dO from its own seeded stream);
    whole (b, h) slices are checked against the oracle."""
    w = inputs.WORKLOADS[name]
    x = inputs.make_inputs(w)
    x["do"] = inputs.make_grad_out(w)
    log(f"[bwd] {name}: GPU forward + backward")
    got = run_fwd_bwd(x, w.dtype, w.causal)
    log(f"[bwd] {name}: oracle on slices {bh}")
    want = oracle_impl.attn_bwd(x["q"], x["k"], x["v"], x["do"], w.dtype, float(x["scale"]), w.causal,
                                x["key_lens"], None, np.array(bh))
    compare_grads(got, want, name, bh=np.array(bh), zero_rows=unseen(x, w.causal, w.H, np.array(bh)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_deterministic_bitwise(dtype):
    """No atomics: two runs give identical bits."""
    x = make(2, 4, 600, 600, 128, dtype, 55, [600, 333])
    a = run_fwd_bwd(x, dtype, True)
    for _ in range(2):
        b = run_fwd_bwd(x, dtype, True)
        for t1, t2 in zip(a, b):
            assert torch.equal(t1, t2)


def test_bwd_errors_write_nothing():
    B, H, N, D = 1, 2, 64, 64
    t = lambda: torch.randn(B, H, N, D, device="cuda", dtype=torch.bfloat16)
    q, k, v, o, do = t(), t(), t(), t(), t()
    lse = torch.zeros(B, H, N, device="cuda")
    outs = [torch.full_like(q, 7.0) for _ in range(3)]
    need = binding.attn_bwd_workspace_size(B, H, N)
    ws = torch.empty(need + 64, dtype=torch.uint8, device="cuda")
    P = lambda x: x.data_ptr()
    base = (P(q), P(k), P(v), P(o), P(do), P(lse), None, *(P(x) for x in outs), B, H, N, N, D, 0.125, 1, None)
    assert binding.attn_bwd(*base, 2, None, need, None) == -1
    assert binding.attn_bwd(*base, 2, P(ws) + 8, need, None) == -8
    assert binding.attn_bwd(*base, 2, P(ws), need - 4, None) == -10
    assert binding.attn_bwd(*base, 3, P(ws), need, None) == -4
    with pytest.raises(ValueError):
        binding.bwd(q, k, v, o, lse, do.float())
    torch.cuda.synchronize()
    assert all(bool((x == 7.0).all()) for x in outs)
