"""The largest slices the ABI accepts (needs an MI355X).

Per (b, h) slice the kernels address Q, K, V and O with 32-bit byte offsets; the host accepts
N * D < 2^29 elements.  These tests run one slice at N = 2^22 - 1 (D = 128, the last accepted
length, with a ragged last tile) through the forward, the sliding-window forward and the
KV-cache decode, and compare sampled rows -- including the last ones -- with the oracle.

The inputs (4.2 M rows x 128 per tensor) come from torch's seeded CPU generator, normal draws
rounded to bfloat16: the counter-based generator of inputs.py would need tens of seconds for
them, and nothing here depends on its stream.
"""
import numpy as np
import pytest
import torch

from gpu_util import compare
from transformer_scaled_dot_amd import binding

pytestmark = pytest.mark.gpu

N = (1 << 22) - 1   # N * 128 < 2^29
D = 128


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def big():
    g = torch.Generator().manual_seed(20261203)
    out = {}
    for name, sigma in (("q", 0.5), ("k", 0.5), ("v", 1.0)):
        t = (torch.randn(1, 1, N, D, generator=g) * sigma).to(torch.bfloat16)
        out[name] = t
    log("[max] inputs ready")
    return out


def storage(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def rows_to_check():
    return np.array(sorted({0, 1, 63, 64, 127, 128, 4095, N // 2, N - 129, N - 65, N - 2, N - 1}), np.int64)


def test_forward_causal_max_length(big, oracle_impl):
    q, k, v = (big[n].cuda() for n in "qkv")
    log(f"[max] forward causal N={N}")
    o, lse = binding.fwd(q, k, v, causal=True, scale=1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    rows = rows_to_check()
    ro, rl = oracle_impl.attn_rows(storage(big["q"]), storage(big["k"]), storage(big["v"]), "bf16",
                                   float(np.float32(1.0 / np.sqrt(D))), True, None, rows)
    eo, el = compare(o, lse, ro, rl, "bf16", "max forward", rows=rows)
    log(f"[max] forward causal: max|dO|={eo:.3e} max|dLSE|={el:.3e}")


def test_window_max_length(big, oracle_impl):
    q, k, v = (big[n].cuda() for n in "qkv")
    log(f"[max] window 1000 N={N}")
    o, lse = binding.fwd(q, k, v, causal=False, scale=0.1, window=1000)
    torch.cuda.synchronize()
    rows = rows_to_check()
    ro, rl = oracle_impl.attn_rows(storage(big["q"]), storage(big["k"]), storage(big["v"]), "bf16",
                                   float(np.float32(0.1)), False, None, rows, window=1000)
    eo, el = compare(o, lse, ro, rl, "bf16", "max window", rows=rows)
    log(f"[max] window: max|dO|={eo:.3e} max|dLSE|={el:.3e}")


def test_decode_max_cache(big, oracle_impl):
    """Four new queries at the end of a cache of 2^22 - 1 keys, the valid length 5 short of it."""
    k, v = big["k"].cuda(), big["v"].cuda()
    q = big["q"][:, :, :4].contiguous()
    kl = np.array([N - 5], np.int32)
    log(f"[max] decode Nk={N}, workspace {binding.attn_decode_workspace_size(1, 1, 4, N, D, 2)} bytes")
    o, lse = binding.decode(q.cuda(), k, v, causal=True, key_lens=torch.from_numpy(kl).cuda(), scale=0.09)
    torch.cuda.synchronize()
    ro, rl = oracle_impl.attn(storage(q), storage(big["k"]), storage(big["v"]), "bf16",
                              float(np.float32(0.09)), 2, kl)
    eo, el = compare(o, lse, ro, rl, "bf16", "max decode")
    log(f"[max] decode: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
