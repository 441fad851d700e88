"""Helpers for the GPU tests: move generator bytes to the device, run the HIP path, compare."""
from __future__ import annotations

import numpy as np
import torch

from transformer_scaled_dot_amd import binding, inputs

TOL_O = {"f32": 1e-4, "f16": 2e-2, "bf16": 2e-2}
TOL_LSE = 1e-3
TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_device(a: np.ndarray, dtype: str, dev="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(dev)


def to_storage(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Device tensor -> numpy storage form (bf16 as uint16 bits)."""
    c = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return c.view(torch.int16).numpy().view(np.uint16)
    return c.numpy()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().double().numpy()


def run(x: dict, dtype: str, causal: bool, scale=None, dev="cuda", window=None):
    q, k, v = (to_device(x[n], dtype, dev) for n in "qkv")
    kl = None if x.get("key_lens") is None else torch.from_numpy(np.asarray(x["key_lens"], np.int32)).to(dev)
    s = float(x["scale"]) if scale is None else float(scale)
    o, lse = binding.fwd(q, k, v, causal=causal, key_lens=kl, scale=s, window=window)
    torch.cuda.synchronize()
    return o, lse


def run_decode(x: dict, dtype: str, causal: bool, scale=None, dev="cuda", workspace=None):
    """attn_decode through the binding: the queries are the last Nq positions of each cache."""
    q, k, v = (to_device(x[n], dtype, dev) for n in "qkv")
    kl = None if x.get("key_lens") is None else torch.from_numpy(np.asarray(x["key_lens"], np.int32)).to(dev)
    s = float(x["scale"]) if scale is None else float(scale)
    o, lse = binding.decode(q, k, v, causal=causal, key_lens=kl, scale=s, workspace=workspace)
    torch.cuda.synchronize()
    return o, lse


def compare(o_dev, lse_dev, o_ref, lse_ref, dtype, what="", rows=None):
    """Max-abs comparison; -inf / non-finite patterns must be identical.  Returns the errors."""
    o = to_f64(o_dev)
    lse = to_f64(lse_dev)
    D = o.shape[-1]
    if rows is not None:
        o = o.reshape(-1, D)[rows]
        lse = lse.reshape(-1)[rows]
    o_ref = np.asarray(o_ref).reshape(o.shape)
    lse_ref = np.asarray(lse_ref).reshape(lse.shape)
    assert np.array_equal(np.isfinite(lse), np.isfinite(lse_ref)), f"{what}: LSE finiteness differs"
    assert np.array_equal(lse[~np.isfinite(lse)], lse_ref[~np.isfinite(lse_ref)]), f"{what}: LSE inf"
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    fin = np.isfinite(lse_ref)
    eo = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    el = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
    assert eo <= TOL_O[dtype], f"{what}: max|dO| = {eo:.3e} > {TOL_O[dtype]:.0e}"
    assert el <= TOL_LSE, f"{what}: max|dLSE| = {el:.3e} > {TOL_LSE:.0e}"
    return eo, el


def sample_rows(w: inputs.Workload, n_random: int, seed: int = 0, block_m: int = 128) -> np.ndarray:
    """Flat row ids: the first and last rows, both sides of every few tile boundaries, and random
    rows, spread over (b, h) slices."""
    rng = np.random.default_rng(seed)
    total = w.B * w.H * w.Nq
    picks = {0, total - 1}
    bhs = sorted({0, w.B * w.H - 1, *rng.integers(0, w.B * w.H, 6).tolist()})
    for bh in bhs:
        base = bh * w.Nq
        for t in range(0, w.Nq, max(block_m, w.Nq // 8)):
            for d in (-1, 0, 1, 31, 32, 63, 64):
                i = t + d
                if 0 <= i < w.Nq:
                    picks.add(base + i)
        picks.add(base + w.Nq - 1)
    picks.update(rng.integers(0, total, n_random).tolist())
    return np.array(sorted(picks), dtype=np.int64)
