"""The entry points under HIP graph capture (needs an MI355X).

The library enqueues only kernels on the caller's stream (no allocation, no memset, no host
synchronisation), so a capture of one call replays it.  Each test captures one call into a
torch CUDA (HIP) graph, changes the inputs in place between replays, runs the program's own
eager work and synchronisations in between, and checks every replay against an eager call on
the same inputs, bit for bit.
"""
import numpy as np
import pytest
import torch

from transformer_scaled_dot_amd import binding

pytestmark = pytest.mark.gpu


def replays(capture_fn, eager_fn, inputs, n=4, seed=7):
    """Capture capture_fn() on a side stream, then for n rounds: refill `inputs` in place,
    replay, compare with eager_fn() on the same inputs."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        capture_fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = capture_fn()
    for r in range(n):
        for t in inputs:
            t.copy_(torch.randn(t.shape, generator=g, device="cuda", dtype=torch.float32).to(t.dtype))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        want = eager_fn()
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {r} differs from the eager call"
        _ = (torch.randn(1000, device="cuda") * 2).sum().item()  # unrelated eager work in between


@pytest.mark.parametrize("causal,window", [(True, None), (False, None), (True, 64)])
def test_forward_graph_replays(causal, window):
    B, H, N, D = 2, 4, 333, 128
    q, k, v = (torch.empty(B, H, N, D, device="cuda", dtype=torch.bfloat16) for _ in range(3))
    kl = torch.tensor([333, 200], dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device="cuda")

    def cap():
        binding.fwd(q, k, v, causal=causal, key_lens=kl, window=window, out=o, lse=lse,
                    stream=torch.cuda.current_stream())
        return (o, lse)

    def eager():
        return binding.fwd(q, k, v, causal=causal, key_lens=kl, window=window)

    replays(cap, eager, [q, k, v])


def test_decode_graph_replays():
    """A split decode (two kernels and a workspace) captured as one graph."""
    B, H, Nq, Nk, D = 2, 4, 1, 6000, 128
    q = torch.empty(B, H, Nq, D, device="cuda", dtype=torch.bfloat16)
    k, v = (torch.empty(B, H, Nk, D, device="cuda", dtype=torch.bfloat16) for _ in range(2))
    kl = torch.tensor([6000, 4100], dtype=torch.int32, device="cuda")
    ws = torch.empty(binding.attn_decode_workspace_size(B, H, Nq, Nk, D, 2), dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0
    o = torch.empty_like(q)
    lse = torch.empty(B, H, Nq, device="cuda")

    def cap():
        binding.decode(q, k, v, causal=True, key_lens=kl, out=o, lse=lse, workspace=ws,
                       stream=torch.cuda.current_stream())
        return (o, lse)

    def eager():
        return binding.decode(q, k, v, causal=True, key_lens=kl)

    replays(cap, eager, [q, k, v])


def test_backward_graph_replays():
    """Forward and backward captured together, as one training step's attention would be."""
    B, H, N, D = 2, 4, 300, 128
    q, k, v, do = (torch.empty(B, H, N, D, device="cuda", dtype=torch.bfloat16) for _ in range(4))
    kl = torch.tensor([300, 170], dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(binding.attn_bwd_workspace_size(B, H, N), dtype=torch.uint8, device="cuda")

    def cap():
        st = torch.cuda.current_stream()
        binding.fwd(q, k, v, causal=True, key_lens=kl, out=o, lse=lse, stream=st)
        binding.bwd(q, k, v, o, lse, do, causal=True, key_lens=kl, dq=dq, dk=dk, dv=dv, workspace=ws,
                    stream=st)
        return (o, lse, dq, dk, dv)

    def eager():
        o2, l2 = binding.fwd(q, k, v, causal=True, key_lens=kl)
        return (o2, l2, *binding.bwd(q, k, v, o2, l2, do, causal=True, key_lens=kl))

    replays(cap, eager, [q, k, v, do])
    assert np.isfinite(dq.float().cpu().numpy()).all()


def test_concurrent_streams_match_sequential():
    """The library keeps no state: calls on two streams at once (default priority) give the same
    bits as the same calls one after the other."""
    g = torch.Generator(device="cuda").manual_seed(11)
    mk = lambda *s: torch.randn(*s, device="cuda", generator=g).to(torch.bfloat16)
    q1, k1, v1 = mk(2, 8, 700, 128), mk(2, 8, 700, 128), mk(2, 8, 700, 128)
    q2, k2, v2 = mk(1, 4, 1, 128), mk(1, 4, 9000, 128), mk(1, 4, 9000, 128)
    ref1 = binding.fwd(q1, k1, v1, causal=True)
    ref2 = binding.decode(q2, k2, v2, causal=True)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            a = binding.fwd(q1, k1, v1, causal=True, stream=s1)
        with torch.cuda.stream(s2):
            b = binding.decode(q2, k2, v2, causal=True, stream=s2)
        outs.append((a, b))
    torch.cuda.synchronize()
    for a, b in outs:
        assert torch.equal(a[0], ref1[0]) and torch.equal(a[1], ref1[1])
        assert torch.equal(b[0], ref2[0]) and torch.equal(b[1], ref2[1])
