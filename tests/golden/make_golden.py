"""Writes bruteforce_tiny.json: tiny attention cases and their exact (50-digit) results.

The pages print no worked attention example with numbers, so these expected values come
from the decimal brute-force reference in oracle/bruteforce.py (this script calls nothing
else).  Inputs are multiples of 1/8 in [-2, 2], exactly representable in fp32, fp16 and
bf16, so every dtype path reads the same values.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import bruteforce  # noqa: E402


def eighths(n, a, c):
    """Deterministic multiples of 1/8 in [-2, 2] from a small linear congruential walk."""
    out, x = [], a
    for _ in range(n):
        x = (x * 37 + c) % 33
        out.append((x - 16) / 8.0)
    return out


def tensor(B, H, N, D, a, c):
    flat = eighths(B * H * N * D, a, c)
    it = iter(flat)
    return [[[[next(it) for _ in range(D)] for _ in range(N)] for _ in range(H)] for _ in range(B)]


CASES = [
    # name, B, H, Nq, Nk, D, scale, causal, key_lens, window (None: no window)
    ("noncausal_q3_k4_d2", 1, 1, 3, 4, 2, 0.5, False, None, None),
    ("causal_q4_k4_d3", 1, 2, 4, 4, 3, 0.25, True, None, None),
    ("causal_topleft_q3_k5_d2", 1, 1, 3, 5, 2, 1.0, True, None, None),
    ("causal_topleft_q5_k3_d2", 1, 1, 5, 3, 2, 1.0, True, None, None),
    ("padded_lens_2_0_q3_k4_d2", 2, 1, 3, 4, 2, 0.5, False, [2, 0], None),
    ("padded_causal_lens_3_1_q4_k4_d4", 2, 1, 4, 4, 4, 0.5, True, [3, 1], None),
    ("wide_q2_k6_d4_scale2", 1, 1, 2, 6, 4, 2.0, False, None, None),
    ("window1_q6_k6_d2", 1, 1, 6, 6, 2, 0.5, False, None, 1),
    ("window2_causal_q6_k6_d3", 1, 1, 6, 6, 3, 0.5, True, None, 2),
    ("window0_q4_k5_d2", 1, 1, 4, 5, 2, 1.0, False, None, 0),
    ("window1_padded_lens_4_2_q5_k6_d2", 2, 1, 5, 6, 2, 0.5, False, [4, 2], 1),
    ("bottomright_q2_k5_d2", 1, 1, 2, 5, 2, 0.5, 2, None, None),
    ("bottomright_padded_lens_4_1_q3_k6_d2", 2, 1, 3, 6, 2, 1.0, 2, [4, 1], None),
]


def main():
    cases = []
    for i, (name, B, H, Nq, Nk, D, scale, causal, kl, window) in enumerate(CASES):
        q = tensor(B, H, Nq, D, 3 + i, 5)
        k = tensor(B, H, Nk, D, 7 + i, 11)
        v = tensor(B, H, Nk, D, 13 + i, 17)
        O, L = bruteforce.attention(q, k, v, scale, causal, kl, window=window)
        cases.append({
            "name": name, "B": B, "H": H, "Nq": Nq, "Nk": Nk, "D": D, "scale": scale,
            "causal": causal, "key_lens": kl, "window": window, "q": q, "k": k, "v": v,
            "o": [[[[format(x, ".30e") for x in row] for row in h] for h in b] for b in O],
            "lse": [[[("-inf" if x is None else format(x, ".30e")) for x in h] for h in b] for b in L],
        })
    doc = {
        "source": "oracle/bruteforce.py (Python decimal, 50 digits); inputs are exact eighths",
        "definition": "O = softmax(scale*q.k over the valid keys) V, LSE = natural log-sum-exp of "
                      "the scaled valid logits; causal keeps j <= i; empty rows give O=0, LSE=-inf",
        "cases": cases,
    }
    with open(os.path.join(HERE, "bruteforce_tiny.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
