"""The seeded generator: determinism, published SplitMix64 behaviour, rounding (CPU only)."""
import numpy as np
import pytest
import torch

from transformer_scaled_dot_amd import inputs

M64 = (1 << 64) - 1


def splitmix64_scalar(state, n):
    """Plain-integer SplitMix64 (one step at a time, as published)."""
    out = []
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & M64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
        out.append(z ^ (z >> 31))
    return out


def test_splitmix64_matches_scalar_definition():
    for state in (0, 1, 1234567, 0xDEADBEEFCAFEF00D):
        got = inputs.splitmix64(state, 0, 20).tolist()
        assert got == splitmix64_scalar(state, 20)
    # counter-based: any window equals the stream's slice
    assert inputs.splitmix64(99, 7, 5).tolist() == splitmix64_scalar(99, 12)[7:]


def test_splitmix64_known_first_output():
    # first output of the stream seeded with 0 (widely quoted value of the published generator)
    assert int(inputs.splitmix64(0, 0, 1)[0]) == 0xE220A8397B1DCDAF


def test_uniform_and_normal_statistics():
    u = inputs.uniforms(5, 0, 1 << 20)
    assert u.min() >= 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 2e-3
    z = inputs.normals(inputs.stream_state(5, 0), 1 << 20)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1.0) < 5e-3
    # chunking does not change the stream
    z2 = inputs.normals(inputs.stream_state(5, 0), 1001, chunk=37)
    assert np.array_equal(z2, z[:1001])


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 65504.0], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(inputs.f32_to_bf16_bits(x), want)


def test_f16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(100000).astype(np.float32) * 10
    st = inputs.to_storage(x.astype(np.float64), "f16")
    assert np.array_equal(st, torch.from_numpy(x).half().numpy())


@pytest.mark.parametrize("name", list(inputs.WORKLOADS)[:4])
def test_workload_inputs_deterministic(name):
    w = inputs.WORKLOADS[name]
    a = inputs.make_inputs(w)
    b = inputs.make_inputs(w)
    assert inputs.input_hashes(a) == inputs.input_hashes(b)
    assert a["q"].shape == (w.B, w.H, w.Nq, w.D) and a["k"].shape == (w.B, w.H, w.Nk, w.D)
    c = inputs.make_inputs(w, seed=w.seed + 100)
    assert inputs.sha256(c["q"]) != inputs.sha256(a["q"])
    if w.padded:
        kl = a["key_lens"]
        assert kl.dtype == np.int32 and kl.min() >= 64 and kl.max() <= 512
    assert a["scale"] == np.float32(1 / np.sqrt(w.D))


def test_stress_variant_scales_q_and_k_only():
    base = inputs.make_inputs(inputs.WORKLOADS["bert_bf16_b32h12n512d64_pad"])
    st = inputs.make_inputs(inputs.WORKLOADS["bert_bf16_b32h12n512d64_pad_stress"])
    # x8 is exact in binary, so the stressed bf16 values are the base values times 8
    qb = inputs.storage_to_f64(base["q"], "bf16")
    qs = inputs.storage_to_f64(st["q"], "bf16")
    assert np.array_equal(qs, 8 * qb)
    assert np.array_equal(st["v"], base["v"])
    assert np.array_equal(st["key_lens"], base["key_lens"])


def test_flop_formula():
    w = inputs.WORKLOADS["longctx_causal_bf16_b1h32n16384d128"]
    assert w.flops() == 4 * 32 * 16384 * 16384 * 128 / 2


def test_band_pair_count():
    """The windowed FLOP count is 4*B*H*D times the pairs with |i - j| <= w (and j <= i when
    causal), counted here by brute force on small shapes."""
    for causal in (False, True):
        for w in (0, 1, 5, 40):
            wl = inputs.Workload("t", "bf16", 2, 3, 37, 29, 64, causal, False, 1.0, 1.0, 1, window=w)
            brute = sum(1 for i in range(37) for j in range(29)
                        if abs(i - j) <= w and (not causal or j <= i))
            assert wl.band_pairs() == brute
            assert wl.flops() == 4.0 * 2 * 3 * 64 * brute


def test_cache_pair_count():
    """A KV-cache step's FLOP count is 4*B*H*D times the visible pairs: query i is position
    Nk - Nq + i of the sequence and sees keys j <= Nk - Nq + i when causal (brute force)."""
    for causal in (False, True):
        for nq, nk in ((1, 1), (1, 50), (7, 50), (50, 50), (60, 50)):
            wl = inputs.Workload("t", "bf16", 2, 3, nq, nk, 64, causal, False, 1.0, 1.0, 1, kv_cache=True)
            brute = sum(1 for i in range(nq) for j in range(nk) if not causal or j <= nk - nq + i)
            assert wl.cache_pairs() == brute
            assert wl.flops() == 4.0 * 2 * 3 * 64 * brute
    w = inputs.WORKLOADS["kvdecode_bf16_b1h32q1k16384d128"]
    assert w.flops() == 4.0 * 32 * 128 * 16384


def test_key_length_range():
    """Key lengths cover [lo, Nk] inclusive; the BERT-like batch keeps [64, 512]."""
    kl = inputs.make_key_lens(3, 20000, 40, 30)
    assert kl.min() == 30 and kl.max() == 40 and len(np.unique(kl)) == 11
    assert np.array_equal(inputs.make_key_lens(3, 32), inputs.make_key_lens(3, 32, 512, 64))
    w = inputs.WORKLOADS["kvdecode_ragged_bf16_b16h32q1k8192d128"]
    kl = inputs.make_key_lens(w.seed, w.B, w.Nk, w.len_lo)
    assert kl.shape == (16,) and kl.min() >= 1024 and kl.max() <= 8192
    with pytest.raises(ValueError):
        inputs.make_key_lens(1, 4, 10, 11)


def test_grad_out_stream():
    """dO has a stream of its own (4): N(0, 1), deterministic, different from Q."""
    w = inputs.Workload("t", "f32", 2, 3, 50, 60, 64, False, False, 1.0, 1.0, 9)
    a, b = inputs.make_grad_out(w), inputs.make_grad_out(w)
    assert a.shape == (2, 3, 50, 64) and np.array_equal(a, b)
    assert not np.array_equal(a, inputs.make_inputs(w)["q"])
    assert abs(float(a.mean())) < 0.05 and abs(float(a.std()) - 1.0) < 0.05
