"""Seeded synthetic inputs for the attention forward, shared by the HIP path and the oracle.

This module holds no attention arithmetic: it only draws numbers and rounds them to the
storage dtype.  Both sides of every parity check read the bytes produced here.

Recipe (one stream per tensor, all counter-based so any slice can be regenerated):

* SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014): output n >= 1 of a stream with start state s is mix(s + n*G mod 2^64),
  G = 0x9E3779B97F4A7C15, mix = the published two xor-shift-multiply rounds.
* The stream for tensor t (0 = Q, 1 = K, 2 = V, 3 = key lengths, 4 = dO, the gradient of O
  fed to the backward, N(0, 1)) starts at state mix(seed + (t+1)*G), i.e. the t-th output of
  the seed's own stream.
* Uniforms: u = (x >> 11) * 2^-53 in [0, 1).
* Normals: Box-Muller on consecutive pairs (u1, u2): r = sqrt(-2 ln(1 - u1)),
  z0 = r cos(2 pi u2), z1 = r sin(2 pi u2), in float64.
* Value = z * sigma (float64) -> float32 (round to nearest even) -> storage dtype
  (float16 by numpy's RNE cast; bfloat16 by RNE on the float32 bit pattern).
* Key lengths (padded workloads): lo + (x mod (Nk - lo + 1)), i.e. uniform on [lo, Nk]
  (lo = 64 unless the workload says otherwise: [64, 512] for the BERT-like batch).

The workloads mirror the shapes the pages measure: a tiny fp32 case, the (2, 100, 512)
toy split into 8 heads of 64, BERT-base encoder attention at 512 tokens with padding,
decoder attention at 4K and long-context attention at 16K with 32 heads of 128, the same
two with a sliding window, and KV-cache decode steps (one new query per sequence against a
4K, 16K or ragged 1K-8K cache of the decoder's 32 heads of 128).
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

DTYPES = ("f32", "f16", "bf16")
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(state: int, start: int, count: int) -> np.ndarray:
    """Outputs start+1 .. start+count (1-based) of the SplitMix64 stream with start state `state`."""
    with np.errstate(over="ignore"):
        n = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        return _mix(np.uint64(state) + n * GAMMA)


def stream_state(seed: int, tensor: int) -> int:
    return int(splitmix64(seed & 0xFFFFFFFFFFFFFFFF, tensor, 1)[0])


def uniforms(state: int, start: int, count: int) -> np.ndarray:
    x = splitmix64(state, start, count)
    return (x >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def normals(state: int, count: int, chunk: int = 1 << 20) -> np.ndarray:
    """`count` standard normals (float64) from Box-Muller pairs of the stream.  Chunks are
    independent slices of the counter-based stream, filled by a few threads (numpy releases
    the GIL inside its array loops); the result does not depend on the thread count."""
    out = np.empty(count, dtype=np.float64)
    npairs = (count + 1) // 2

    def fill(p0: int) -> None:
        np_ = min(chunk, npairs - p0)
        u = uniforms(state, 2 * p0, 2 * np_)
        u1, u2 = u[0::2], u[1::2]
        r = np.sqrt(-2.0 * np.log1p(-u1))
        th = (2.0 * np.pi) * u2
        z = np.empty(2 * np_, dtype=np.float64)
        z[0::2] = r * np.cos(th)
        z[1::2] = r * np.sin(th)
        lo = 2 * p0
        hi = min(count, lo + 2 * np_)
        out[lo:hi] = z[: hi - lo]

    starts = range(0, npairs, chunk)
    if len(starts) <= 1:
        for p0 in starts:
            fill(p0)
    else:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1, len(starts))) as ex:
            list(ex.map(fill, starts))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> float32 (RNE) -> storage dtype.  bf16 is returned as uint16 bits."""
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "f16":
        return x32.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values (used only to inspect data, e.g. in tests)."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    B: int
    H: int
    Nq: int
    Nk: int
    D: int
    causal: bool
    padded: bool
    sigma_qk: float
    sigma_v: float
    seed: int
    note: str = ""
    scale: float = field(default=None)  # defaults to 1/sqrt(D), rounded to float32
    window: int = field(default=None)   # local band |i - j| <= window, None for none
    kv_cache: bool = False  # queries are the last Nq positions of each key sequence (decode)
    len_lo: int = 64        # padded workloads: key lengths uniform on [len_lo, Nk]

    @property
    def scale_f32(self) -> np.float32:
        s = self.scale if self.scale is not None else 1.0 / np.sqrt(self.D)
        return np.float32(s)

    def band_pairs(self) -> int:
        """(query, key) pairs inside the band (and the causal triangle), padding ignored."""
        i = np.arange(self.Nq, dtype=np.int64)
        lo = np.maximum(i - self.window, 0)
        hi = np.minimum(i + 1 if self.causal else i + self.window + 1, self.Nk)
        hi = np.minimum(hi, i + self.window + 1)
        return int(np.maximum(hi - lo, 0).sum())

    def cache_pairs(self) -> int:
        """(query, key) pairs of a KV-cache step, padding ignored: query i (the (Nk - Nq + i)-th
        position) sees keys j <= i + Nk - Nq when causal, every key otherwise."""
        if not self.causal:
            return self.Nq * self.Nk
        i = np.arange(self.Nq, dtype=np.int64)
        return int(np.clip(i + 1 + self.Nk - self.Nq, 0, self.Nk).sum())

    def flops(self) -> float:
        """Metric FLOPs: 4*B*H*Nq*Nk*D, halved for causal (QK^T and PV, dense count).  With a
        local window: 4*B*H*D per (query, key) pair inside the band.  A KV-cache step counts
        4*B*H*D per visible (query, key) pair."""
        if self.window is not None:
            return 4.0 * self.B * self.H * self.D * self.band_pairs()
        if self.kv_cache:
            return 4.0 * self.B * self.H * self.D * self.cache_pairs()
        f = 4.0 * self.B * self.H * self.Nq * self.Nk * self.D
        return f / 2 if self.causal else f

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32_b1h2n128d64", "f32", 1, 2, 128, 128, 64, False, False, 1.0, 1.0, 1,
                 "tiny non-causal fp32, no mask"),
        Workload("ragged_f16_b2h8n100d64", "f16", 2, 8, 100, 100, 64, False, False, 1.0, 1.0, 2,
                 "(2,100,512) toy split into 8 heads of 64; N=100 is not a tile multiple"),
        Workload("bert_bf16_b32h12n512d64_pad", "bf16", 32, 12, 512, 512, 64, False, True, 1.0, 1.0, 3,
                 "BERT-base encoder attention, key padding lengths U[64,512]"),
        Workload("bert_bf16_b32h12n512d64_pad_stress", "bf16", 32, 12, 512, 512, 64, False, True, 8.0, 1.0, 3,
                 "same, Q and K scaled x8: logits of std ~64"),
        Workload("decoder_causal_bf16_b4h32n4096d128", "bf16", 4, 32, 4096, 4096, 128, True, False, 0.5, 0.5, 4,
                 "decoder causal attention at 4K"),
        Workload("longctx_causal_bf16_b1h32n16384d128", "bf16", 1, 32, 16384, 16384, 128, True, False, 0.5, 0.5, 5,
                 "long-context causal attention at 16K"),
        Workload("decoder_window512_causal_bf16_b4h32n4096d128", "bf16", 4, 32, 4096, 4096, 128, True, False,
                 0.5, 0.5, 6, "decoder causal attention at 4K with a sliding window of 512", window=512),
        Workload("longctx_window512_causal_bf16_b1h32n16384d128", "bf16", 1, 32, 16384, 16384, 128, True,
                 False, 0.5, 0.5, 7, "long-context causal attention at 16K with a sliding window of 512",
                 window=512),
        Workload("kvdecode_bf16_b4h32q1k4096d128", "bf16", 4, 32, 1, 4096, 128, True, False, 0.5, 0.5, 8,
                 "one decode step of the 4K decoder batch: 1 new query per sequence, full 4K cache",
                 kv_cache=True),
        Workload("kvdecode_bf16_b1h32q1k16384d128", "bf16", 1, 32, 1, 16384, 128, True, False, 0.5, 0.5, 9,
                 "one decode step at 16K context: 1 new query against a 16K cache", kv_cache=True),
        Workload("kvdecode_ragged_bf16_b16h32q1k8192d128", "bf16", 16, 32, 1, 8192, 128, True, True, 0.5,
                 0.5, 10, "one decode step of a serving batch: 16 caches of lengths U[1024, 8192]",
                 kv_cache=True, len_lo=1024),
    ]
}

# The measured workload of the benchmark and the parity workloads, in order.
BENCH_WORKLOAD = "longctx_causal_bf16_b1h32n16384d128"
PARITY_ORDER = list(WORKLOADS)


def make_key_lens(seed: int, B: int, Nk: int = 512, lo: int = 64) -> np.ndarray:
    """Valid key lengths uniform on [lo, Nk] (lo <= Nk)."""
    if not 0 <= lo <= Nk:
        raise ValueError("need 0 <= lo <= Nk")
    st = stream_state(seed, 3)
    x = splitmix64(st, 0, B)
    return (np.uint64(lo) + x % np.uint64(Nk - lo + 1)).astype(np.int32)


def make_tensor(seed: int, which: int, shape, sigma: float, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    z = normals(stream_state(seed, which), n)
    if sigma != 1.0:
        z *= sigma
    return to_storage(z, dtype).reshape(shape)


def make_grad_out(w: Workload, seed: int | None = None) -> np.ndarray:
    """dO for the backward: N(0, 1) in the storage dtype, [B, H, Nq, D] (stream 4)."""
    s = w.seed if seed is None else seed
    return make_tensor(s, 4, (w.B, w.H, w.Nq, w.D), 1.0, w.dtype)


def make_inputs(w: Workload, seed: int | None = None) -> dict:
    """Q, K, V (storage dtype, [B,H,N,D] contiguous), key lengths (int32[B] or None), scale (float32)."""
    s = w.seed if seed is None else seed
    q = make_tensor(s, 0, (w.B, w.H, w.Nq, w.D), w.sigma_qk, w.dtype)
    k = make_tensor(s, 1, (w.B, w.H, w.Nk, w.D), w.sigma_qk, w.dtype)
    v = make_tensor(s, 2, (w.B, w.H, w.Nk, w.D), w.sigma_v, w.dtype)
    kl = make_key_lens(s, w.B, w.Nk, w.len_lo) if w.padded else None
    return {"q": q, "k": k, "v": v, "key_lens": kl, "scale": w.scale_f32, "seed": s}


def sha256(a: np.ndarray | None) -> str | None:
    if a is None:
        return None
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def input_hashes(inp: dict) -> dict:
    return {n: sha256(inp[n]) for n in ("q", "k", "v", "key_lens")}
