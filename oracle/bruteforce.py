"""TEST INFRASTRUCTURE ONLY: a second, independent reference for tiny inputs.

Pure-Python `decimal` arithmetic at 50 significant digits (Decimal.exp and Decimal.ln are
correctly rounded), so for inputs that are exact binary fractions the result is the exact
attention output to ~1e-48.  It follows the same plain definition as attn_oracle.c but
shares no code with it: masked keys are left out of the softmax, the causal mask keeps
keys j <= i (causal = 2: j <= i + L_b - Nq, the queries being the last Nq positions), a window
w keeps keys with |i - j| <= w, and a row with no key gives O = 0 and LSE = -inf.
"""
from __future__ import annotations

from decimal import Decimal, localcontext
from fractions import Fraction


def _dec(x) -> Decimal:
    f = Fraction(x)  # exact for python floats / ints / Fractions
    return Decimal(f.numerator) / Decimal(f.denominator)


def attention_row(q_row, keys, values, scale, digits: int = 50):
    """O (list of Decimal) and LSE (Decimal, or None for an empty row) for one query row.

    q_row: [D]; keys, values: lists of [D] rows already restricted to the valid keys.
    """
    with localcontext() as ctx:
        ctx.prec = digits
        D = len(q_row)
        if not keys:
            return [Decimal(0)] * D, None
        sc = _dec(scale)
        qd = [_dec(x) for x in q_row]
        logits = []
        for kr in keys:
            acc = Decimal(0)
            for a, b in zip(qd, kr):
                acc += a * _dec(b)
            logits.append(sc * acc)
        m = max(logits)
        w = [(s - m).exp() for s in logits]
        tot = sum(w, Decimal(0))
        out = []
        for d in range(D):
            acc = Decimal(0)
            for wj, vr in zip(w, values):
                acc += wj * _dec(vr[d])
            out.append(acc / tot)
        return out, m + tot.ln()


def attention(q, k, v, scale, causal=False, key_lens=None, digits: int = 50, window=None):
    """q: nested lists [B][H][Nq][D]; k, v: [B][H][Nk][D].  Returns (O, LSE) as nested lists of
    Decimal (LSE None for empty rows)."""
    B, H = len(q), len(q[0])
    O, L = [], []
    for b in range(B):
        ob, lb = [], []
        for h in range(H):
            Nk = len(k[b][h])
            kb = Nk if key_lens is None else max(0, min(Nk, int(key_lens[b])))
            oh, lh = [], []
            shift = kb - len(q[b][h]) if causal == 2 else 0
            for i, qr in enumerate(q[b][h]):
                keep = [j for j in range(kb)
                        if (not causal or j <= i + shift) and (window is None or abs(i - j) <= window)]
                o, lse = attention_row(qr, [k[b][h][j] for j in keep], [v[b][h][j] for j in keep],
                                       scale, digits)
                oh.append(o)
                lh.append(lse)
            ob.append(oh)
            lb.append(lh)
        O.append(ob)
        L.append(lb)
    return O, L
