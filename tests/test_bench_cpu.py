"""bench.py's host-side accounting (CPU only): the visible-pair count behind the CPU baseline's
unit, the algorithmic bytes behind `roofline`, the traffic lookup and the one-GPU exit."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from transformer_scaled_dot_amd import inputs  # noqa: E402


def brute_pairs(w, key_lens):
    """Visible (query, key) pairs per flat row, by the definition of each mask."""
    out = []
    for b in range(w.B):
        L = w.Nk if key_lens is None else min(max(int(key_lens[b]), 0), w.Nk)
        for _h in range(w.H):
            for i in range(w.Nq):
                n = 0
                for j in range(w.Nk):
                    ok = j < L
                    if w.kv_cache and w.causal:
                        ok = ok and j <= i + L - w.Nq
                    elif w.causal:
                        ok = ok and j <= i
                    if w.window is not None:
                        ok = ok and abs(i - j) <= w.window
                    n += ok
                out.append(n)
    return np.array(out)


CASES = [
    dict(causal=False, window=None, kv_cache=False, kl=None),
    dict(causal=True, window=None, kv_cache=False, kl=None),
    dict(causal=True, window=3, kv_cache=False, kl=[13, 5]),
    dict(causal=False, window=4, kv_cache=False, kl=[20, 0]),
    dict(causal=True, window=None, kv_cache=True, kl=[20, 9]),
    dict(causal=False, window=None, kv_cache=False, kl=[7, 20]),
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_row_pairs_match_brute_force(case):
    nq = 3 if case["kv_cache"] else 17
    w = inputs.Workload("t", "bf16", 2, 2, nq, 20, 64, case["causal"], case["kl"] is not None, 1.0, 1.0, 1,
                        window=case["window"], kv_cache=case["kv_cache"])
    kl = None if case["kl"] is None else np.array(case["kl"], np.int32)
    rows = np.arange(w.B * w.H * w.Nq, dtype=np.int64)
    got = bench.row_pairs(w, rows, kl)
    np.testing.assert_array_equal(got, brute_pairs(w, kl))


def test_algorithmic_bytes_long_context():
    """Q, K, V read once, O written once (bf16), LSE in fp32: 539.0 MB at B=1, H=32, N=16384, D=128."""
    w = inputs.WORKLOADS["longctx_causal_bf16_b1h32n16384d128"]
    assert bench.algorithmic_bytes(w) == 4 * 32 * 16384 * 128 * 2 + 32 * 16384 * 4
    assert abs(bench.algorithmic_bytes(w) / 1e6 - 539.0) < 0.1
    # backward: Q, K, V, O, dO read and dQ, dK, dV written (bf16) plus the LSE
    assert bench.bwd_algorithmic_bytes(w) == 8 * 32 * 16384 * 128 * 2 + 32 * 16384 * 4


def test_algorithmic_bytes_counts_valid_cache_rows_only():
    w = inputs.WORKLOADS["kvdecode_ragged_bf16_b16h32q1k8192d128"]
    kl = np.array([8192, 100, 0, 20000] + [1] * 12, np.int32)  # clamped to [0, Nk]
    rows = 8192 + 100 + 0 + 8192 + 12
    want = 2 * (2 * 16 * 32 * 1 * 128 + 2 * 32 * rows * 128) + 4 * 16 * 32 * 1
    assert bench.algorithmic_bytes(w, kl) == want


def test_read_traffic_requires_matching_sources(tmp_path, monkeypatch):
    """A traffic figure is used only when its file was measured on the same kernel sources."""
    h = "ab" * 32
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "attn_fwd_wl_traffic.md").write_text(
        f"traffic_bytes_per_launch: 1.2345e+08\nkernel_source_sha256: {h}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_traffic("wl", h) == pytest.approx(1.2345e8)
    assert bench.read_traffic("wl", "cd" * 32) is None
    assert bench.read_traffic("other", h) is None


def test_committed_profiles_name_their_sources():
    """Every committed traffic summary states the kernel-source hash it was measured on, and the
    bench reads its figure back when given that hash."""
    pdir = os.path.join(ROOT, "profiles")
    files = [f for f in os.listdir(pdir) if f.endswith("_traffic.md")]
    assert files
    for f in files:
        text = open(os.path.join(pdir, f)).read()
        m = [ln.split(":", 1)[1].strip() for ln in text.splitlines() if ln.startswith("kernel_source_sha256:")]
        assert m and len(m[0]) == 64, f
        family, _, rest = f.partition("_")
        family = family + "_" + rest.split("_", 1)[0]  # attn_fwd / attn_bwd / attn_decode
        workload = rest.split("_", 1)[1][: -len("_traffic.md")]
        assert bench.read_traffic(workload, m[0], family) is not None, f


def test_kernel_source_hash_tracks_contents():
    assert bench.kernel_source_hash() == bench.kernel_source_hash()
    assert bench.kernel_source_hash() != bench.kernel_source_hash(bench.BWD_KERNEL_SOURCES)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
