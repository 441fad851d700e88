"""attn_decode_noalloc (the decode entry point that takes its split partials from the library's
static scratch instead of a caller workspace) against attn_decode with a workspace, through the
C ABI (needs an MI355X).  Two calls in a row, the second on a smaller input; outputs must be
bitwise those of attn_decode on the same inputs, and no device memory may be allocated by the
calls."""
import numpy as np
import pytest
import torch

from gpu_util import to_device
from transformer_scaled_dot_amd import binding, inputs

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 16 << 20  # ATTN_DECODE_SCRATCH_BYTES in include/attn_fwd.h

CASES = [
    # name, dtype, B, H, Nq, Nk, D, causal, padded  (first the larger input, then a smaller one)
    ("b2h8_q1_k4096_d128_bf16", "bf16", 2, 8, 1, 4096, 128, True, True),
    ("b1h4_q3_k1000_d64_f16", "f16", 1, 4, 3, 1000, 64, True, False),
]


def log(msg):
    print(msg, flush=True)


def call_both(w, x):
    dev = torch.device("cuda")
    q, k, v = (to_device(x[n], w.dtype) for n in "qkv")
    kl = None if x["key_lens"] is None else torch.from_numpy(x["key_lens"]).to(dev)
    code = inputs.DTYPE_CODE[w.dtype]
    stream = torch.cuda.current_stream().cuda_stream
    args = (w.B, w.H, w.Nq, w.Nk, w.D, float(x["scale"]), int(w.causal), None if kl is None else kl.data_ptr(), code)
    # reference: attn_decode with a caller workspace
    need = binding.attn_decode_workspace_size(w.B, w.H, w.Nq, w.Nk, w.D, code)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    o_ref = torch.full_like(q, float("nan"))
    l_ref = torch.full((w.B, w.H, w.Nq), float("nan"), device=dev)
    rc = binding.attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_ref.data_ptr(), l_ref.data_ptr(),
                             *args, ws.data_ptr(), need, stream)
    assert rc == binding.ATTN_OK, binding.STATUS.get(rc, rc)
    # the entry point under test: outputs preallocated, nothing else
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.H, w.Nq), float("nan"), device=dev)
    torch.cuda.synchronize()
    alloc0, free0 = torch.cuda.memory_allocated(), torch.cuda.mem_get_info()[0]
    rc = binding.attn_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                     *args, stream)
    torch.cuda.synchronize()
    alloc1, free1 = torch.cuda.memory_allocated(), torch.cuda.mem_get_info()[0]
    assert rc == binding.ATTN_OK, binding.STATUS.get(rc, rc)
    return (o, lse), (o_ref, l_ref), need, (alloc1 - alloc0, free0 - free1)


def make(case):
    name, dtype, B, H, Nq, Nk, D, causal, padded = case
    w = inputs.Workload(name, dtype, B, H, Nq, Nk, D, causal, padded, 0.5, 0.5, 31, kv_cache=True)
    return w, inputs.make_inputs(w)


def test_noalloc_matches_decode_two_calls():
    # Set-up: the first call on a device looks up that device's copy of the static scratch, which
    # the runtime materialises then (at most the scratch plus page rounding, once per process).
    w, x = make(CASES[-1])
    _, _, _, (d_alloc, d_free) = call_both(w, x)
    log(f"[noalloc] set-up call: torch alloc delta {d_alloc}, device free delta {d_free}")
    assert d_alloc == 0 and d_free <= SCRATCH_BYTES + (4 << 20)
    # Two calls in a row, the second on a smaller input: no device memory changes, and the
    # results are bitwise attn_decode's (same kernels, same key-split plan).
    for case in CASES:
        w, x = make(case)
        (o, lse), (o_ref, l_ref), need, (d_alloc, d_free) = call_both(w, x)
        log(f"[noalloc] {w.name}: scratch {need} bytes, torch alloc delta {d_alloc}, device free delta {d_free}")
        assert 0 < need <= SCRATCH_BYTES, f"{w.name}: the case must use the scratch and fit it"
        assert d_alloc == 0 and d_free == 0, f"{w.name}: device memory changed during the call"
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"{w.name}: O differs from attn_decode"
        assert torch.equal(lse, l_ref), f"{w.name}: LSE differs from attn_decode"
        assert bool(torch.isfinite(lse).all()), f"{w.name}: non-finite LSE"
