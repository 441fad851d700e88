"""`attention`, the differentiable op over attn_fwd_window / attn_bwd_window (needs an MI355X).

Its gradients must be exactly what the backward entry point returns for the same dO (and dLSE),
whichever outputs the loss uses; attn_bwd itself is checked against the oracle in
test_gpu_bwd.py, and one case here is compared with the oracle directly.
"""
import numpy as np
import pytest
import torch

from gpu_util import to_f64
from transformer_scaled_dot_amd import attention, binding

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def leaf(shape, dtype, gen, sigma=1.0):
    return (torch.randn(*shape, generator=gen, device="cuda") * sigma).to(TDT[dtype]).requires_grad_(True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal,window,padded", [(True, None, True), (False, None, False), (True, 40, False)])
@pytest.mark.parametrize("use", ["o", "o+lse", "lse"])
def test_gradients_are_the_backward_entry_point(dtype, causal, window, padded, use):
    g = torch.Generator(device="cuda").manual_seed(71)
    B, H, N, D = 2, 3, 150, 128 if dtype == "bf16" else 64
    q, k, v = (leaf((B, H, N, D), dtype, g, 0.5) for _ in range(3))
    kl = torch.tensor([150, 77], dtype=torch.int32, device="cuda") if padded else None
    G = torch.randn(B, H, N, D, generator=g, device="cuda").to(TDT[dtype])
    gl = torch.randn(B, H, N, generator=g, device="cuda")
    o, lse = attention(q, k, v, causal=causal, key_lens=kl, window=window, return_lse=True)
    loss = 0
    if "o" in use.split("+"):
        loss = loss + (o.float() * G.float()).sum()
    if "lse" in use.split("+"):
        loss = loss + (torch.nan_to_num(lse, neginf=0.0) * gl).sum()
    loss.backward()
    torch.cuda.synchronize()
    # the same call through the entry points
    o2, lse2 = binding.fwd(q.detach(), k.detach(), v.detach(), causal=causal, key_lens=kl, window=window)
    assert torch.equal(o.detach(), o2) and torch.equal(lse.detach(), lse2)
    dout = G if "o" in use.split("+") else torch.zeros_like(G)
    dlse = None
    if "lse" in use.split("+"):
        dlse = torch.where(torch.isfinite(lse2), gl, torch.zeros_like(gl)).contiguous()
    want = binding.bwd(q.detach(), k.detach(), v.detach(), o2, lse2, dout, causal=causal, key_lens=kl,
                       window=window, dlse=dlse)
    torch.cuda.synchronize()
    for name, got, ref in zip(("dq", "dk", "dv"), (q.grad, k.grad, v.grad), want):
        assert torch.equal(got, ref), f"{dtype} {use} {name}"


def test_against_the_oracle(oracle_impl):
    """fp32 attention with both outputs in the loss, against the oracle's gradients."""
    from transformer_scaled_dot_amd import inputs

    w = inputs.Workload("t", "f32", 1, 2, 90, 110, 64, True, False, 1.0, 1.0, 72)
    x = inputs.make_inputs(w)
    do = inputs.make_grad_out(w)
    gl = np.random.default_rng(73).standard_normal((1, 2, 90)).astype(np.float32)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x[n])).cuda().requires_grad_(True) for n in "qkv")
    o, lse = attention(q, k, v, causal=True, scale=float(x["scale"]), return_lse=True)
    ((o * torch.from_numpy(do).cuda()).sum() + (lse * torch.from_numpy(gl).cuda()).sum()).backward()
    want = oracle_impl.attn_bwd(x["q"], x["k"], x["v"], do, "f32", float(x["scale"]), True, None, gl)
    for name, got, ref in zip(("dq", "dk", "dv"), (q.grad, k.grad, v.grad), want):
        ref = np.asarray(ref).reshape(got.shape)
        err = float(np.max(np.abs(to_f64(got) - ref)))
        assert err <= 1e-4 * max(float(np.max(np.abs(ref))), 0.1), (name, err)
