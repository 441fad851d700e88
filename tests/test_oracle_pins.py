"""The oracle against what the pages and the mathematics fix (CPU only)."""
import math

import numpy as np
import pytest

import pins
from transformer_scaled_dot_amd import inputs


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, oracle_impl):
    pin(oracle_impl)


@pytest.mark.parametrize("name", [
    "tiny_f32_b1h2n128d64",
    "ragged_f16_b2h8n100d64",
    "bert_bf16_b32h12n512d64_pad",
    "bert_bf16_b32h12n512d64_pad_stress",
])
def test_oracle_matches_torch_sdpa_on_workload(name, oracle_impl):
    """Library special case at the parity workloads' own shapes and inputs (the BERT-shaped
    ones on a subset of batches to stay within seconds)."""
    w = inputs.WORKLOADS[name]
    x = inputs.make_inputs(w)
    q, k, v, kl = x["q"], x["k"], x["v"], x["key_lens"]
    if w.B > 4:
        sel = [0, 7, 19, 31]
        q, k, v = (np.ascontiguousarray(t[sel]) for t in (q, k, v))
        kl = kl[sel]
    o, lse = oracle_impl.attn(q, k, v, w.dtype, float(x["scale"]), w.causal, kl)
    ro, rl = pins.torch_sdpa_f64(q, k, v, w.dtype, float(x["scale"]), w.causal, kl)
    pins.close(o, ro, 1e-12, "O")
    pins.close(lse, rl, 1e-12 * max(1.0, float(np.abs(rl).max())), "lse")


@pytest.mark.parametrize("causal", [False, True])
def test_mask_fill_readings_agree(causal, oracle_impl):
    """The pages fill masked logits with -inf, with -1e9, or add (1 - mask) * -10000.  On rows
    that keep a key the three agree with leaving masked keys out (what the oracle does)."""
    import torch

    rng = np.random.default_rng(3)
    B, H, N, D = 2, 2, 16, 8
    q, k, v = (pins.rand_store(rng, (B, H, N, D), "f32", 2.0) for _ in range(3))
    kl = np.array([16, 9], np.int32)
    scale = float(np.float32(0.35))
    o, _ = oracle_impl.attn(q, k, v, "f32", scale, causal, kl)
    qd, kd, vd = (torch.from_numpy(t.astype(np.float64)) for t in (q, k, v))
    s = torch.matmul(qd, kd.transpose(-2, -1)) * scale
    keep = torch.arange(N)[None, :] < torch.from_numpy(kl.astype(np.int64))[:, None]
    keep = keep[:, None, None, :].expand(B, H, N, N)
    if causal:
        keep = keep & torch.ones(N, N, dtype=torch.bool).tril()
    for variant in ("neg_inf", "neg_1e9", "additive_1e4"):
        if variant == "neg_inf":
            t = s.masked_fill(~keep, float("-inf"))
        elif variant == "neg_1e9":
            t = s.masked_fill(~keep, -1e9)
        else:
            t = s + (1.0 - keep.double()) * -10000.0
        ref = torch.matmul(torch.softmax(t, dim=-1), vd).numpy()
        pins.close(o, ref, 1e-12, variant)


def test_oracle_full_workload_vs_rows(oracle_impl):
    """Row sampling (used at full sizes) returns exactly the full computation's rows."""
    w = inputs.WORKLOADS["ragged_f16_b2h8n100d64"]
    x = inputs.make_inputs(w)
    o, lse = oracle_impl.attn(x["q"], x["k"], x["v"], w.dtype, float(x["scale"]), w.causal)
    rows = np.array([0, 99, 100, 777, 1599], np.int64)
    o2, l2 = oracle_impl.attn_rows(x["q"], x["k"], x["v"], w.dtype, float(x["scale"]), w.causal,
                                   None, rows)
    assert np.array_equal(o2, o.reshape(-1, w.D)[rows])
    assert np.array_equal(l2, lse.reshape(-1)[rows])


def test_oracle_rejects_bad_arguments(oracle_impl):
    q = np.zeros((1, 1, 4, 8), np.float32)
    with pytest.raises(ValueError):
        oracle_impl.attn_rows(q, q, q, "f32", 1.0, rows=np.array([4], np.int64))
    with pytest.raises(TypeError):
        oracle_impl.attn(q.astype(np.float16), q, q, "f32", 1.0)
    assert math.isinf(oracle_impl.attn(q, q, q, "f32", 1.0, key_lens=np.array([0], np.int32))[1][0, 0, 0])
