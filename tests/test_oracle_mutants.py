"""Plant plausible mistakes in copies of the oracle source (CPU only) and check that the pins
catch every one.  The real oracle is never modified: each mutant is a textual edit of a
temporary copy of attn_oracle.c, built with the oracle's own build command."""
import os

import pytest

import oracle
import pins

MUTANTS = [
    ("dropped scale", "s[j - jbeg] = scale * acc;", "s[j - jbeg] = acc;"),
    ("scale applied twice", "s[j - jbeg] = scale * acc;", "s[j - jbeg] = scale * scale * acc;"),
    ("q.q instead of q.k", "acc += qrow[d] * krow[d];", "acc += qrow[d] * qrow[d];"),
    ("wrong sign in the shift", "s[j] = exp(s[j] - m);", "s[j] = exp(s[j] + m);"),
    ("no max shift", "if (s[j] > m) m = s[j];", "if (s[j] > m) m = m;"),
    ("min instead of max", "if (s[j] > m) m = s[j];", "if (s[j] < m) m = s[j];"),
    ("missing normalisation", "for (int d = 0; d < D; ++d) o[d] /= l;", ""),
    ("log2 in the LSE", "*lse = m + log(l);", "*lse = m + log2(l);"),
    ("LSE without the max", "*lse = m + log(l);", "*lse = log(l);"),
    ("causal j < i", "jend = (int64_t)i + cb + 1;", "jend = (int64_t)i + cb;"),
    ("causal ignored", "if (causal && jend > (int64_t)i + cb + 1)", "if (0 && jend > (int64_t)i + cb + 1)"),
    ("key lengths ignored", "\n        L = key_lens[b];", "\n        L = Nk;"),
    ("key length off by one", "\n        L = key_lens[b];", "\n        L = key_lens[b] - 1;"),
    ("batch index from head", "int b = (int)(bh / H);", "int b = (int)(bh % H);"),
    ("K/V base uses Nq", "int64_t kbase = bh * (int64_t)Nk * D;", "int64_t kbase = bh * (int64_t)Nq * D;"),
    ("V rows reversed", "decode_row(v, dtype, kbase + (jbeg + j) * D, D, krow);",
     "decode_row(v, dtype, kbase + (jend - 1 - j) * D, D, krow);"),
    ("V read from K", "decode_row(v, dtype, kbase + (jbeg + j) * D, D, krow);",
     "decode_row(k, dtype, kbase + (jbeg + j) * D, D, krow);"),
    ("V rows not offset by the window start", "decode_row(v, dtype, kbase + (jbeg + j) * D, D, krow);",
     "decode_row(v, dtype, kbase + j * D, D, krow);"),
    ("logits not offset by the window start", "s[j - jbeg] = scale * acc;", "s[j] = scale * acc;"),
    ("window start off by one", "jbeg = (int64_t)i - window;", "jbeg = (int64_t)i - window + 1;"),
    ("window start ignored", "if (jbeg < (int64_t)i - window) jbeg = (int64_t)i - window;", ""),
    ("window end off by one", "jend = (int64_t)i + window + 1;", "jend = (int64_t)i + window;"),
    ("bottom-right shift ignored", "int64_t cb = causal == 2 ? L - Nq : 0;", "int64_t cb = 0;"),
    ("bottom-right shift from Nk", "int64_t cb = causal == 2 ? L - Nq : 0;", "int64_t cb = causal == 2 ? Nk - Nq : 0;"),
    ("bottom-right off by one", "int64_t cb = causal == 2 ? L - Nq : 0;", "int64_t cb = causal == 2 ? L - Nq - 1 : 0;"),
    ("window end ignored", "if (jend > (int64_t)i + window + 1) jend = (int64_t)i + window + 1;", ""),
    ("empty row LSE 0", "*lse = -INFINITY;", "*lse = 0.0;"),
    ("bf16 shift 15", "uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    ("fp16 bias off by one", "e - 25);", "e - 24);"),
    ("fp16 subnormal scale", "ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    ("sum of unshifted exps", "l += s[j];", "l += s[j] * exp(m);"),
    # backward
    ("bwd dq without scale", "dqi[d] += sh.scale * ds * Kd[j * D + d];", "dqi[d] += ds * Kd[j * D + d];"),
    ("bwd dq from V", "dqi[d] += sh.scale * ds * Kd[j * D + d];", "dqi[d] += sh.scale * ds * Vd[j * D + d];"),
    ("bwd dk without scale", "dkj[d] += sh.scale * ds * qi[d];", "dkj[d] += ds * qi[d];"),
    ("bwd dk from dO", "dkj[d] += sh.scale * ds * qi[d];", "dkj[d] += sh.scale * ds * gi[d];"),
    ("bwd dv weighted by dS", "dvj[d] += pij * gi[d];", "dvj[d] += ds * gi[d];"),
    ("bwd row term dropped (dq)", "const double ds = P[j] * (dP[j] - Dsum + g);", "const double ds = P[j] * (dP[j] + g);"),
    ("bwd row term dropped (dk)", "const double ds = pij * (dp - Dr[i] + g);", "const double ds = pij * (dp + g);"),
    ("bwd LSE gradient sign", "const double ds = P[j] * (dP[j] - Dsum + g);", "const double ds = P[j] * (dP[j] - Dsum - g);"),
    ("bwd LSE gradient ignored (dk)", "const double ds = pij * (dp - Dr[i] + g);", "const double ds = pij * (dp - Dr[i]);"),
    ("bwd row term without P", "Dsum += P[j] * acc;", "Dsum += acc;"),
    ("bwd P not normalised", "P[j] = exp(P[j] - m) / l;", "P[j] = exp(P[j] - m);"),
    ("bwd lse without max", "lse[i] = m + log(l);", "lse[i] = log(l);"),
    ("bwd visibility ignored in key pass", "if ((int64_t)j < bwd_jbeg(&sh, i) || (int64_t)j >= bwd_jend(&sh, L, i)) continue;", ""),
    ("bwd causal off by one", "if (sh->causal && jend > (int64_t)i + 1) jend = (int64_t)i + 1;",
     "if (sh->causal && jend > (int64_t)i) jend = (int64_t)i;"),
    ("bwd dO decoded from Q", "dOd[x] = dec(dO, dtype, (int64_t)(s_bh * nq + x));", "dOd[x] = dec(q, dtype, (int64_t)(s_bh * nq + x));"),
    ("bwd band start ignored (key pass)", "if ((int64_t)j < bwd_jbeg(&sh, i) || (int64_t)j >= bwd_jend(&sh, L, i)) continue;",
     "if ((int64_t)j >= bwd_jend(&sh, L, i)) continue;"),
    ("bwd band start ignored (row pass)", "const int64_t jb = bwd_jbeg(&sh, i), n = bwd_jend(&sh, L, i);",
     "const int64_t jb = 0, n = bwd_jend(&sh, L, i);"),
    ("bwd band end off by one", "if (sh->window >= 0 && jend > (int64_t)i + sh->window + 1) jend = (int64_t)i + sh->window + 1;",
     "if (sh->window >= 0 && jend > (int64_t)i + sh->window) jend = (int64_t)i + sh->window;"),
    ("bwd key lengths ignored", "            L = key_lens[b];\n            if (L < 0) L = 0;\n            if (L > Nk) L = Nk;\n        }\n        for (size_t x",
     "            L = Nk;\n        }\n        for (size_t x"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle.SRC) as f:
        return f.read()


@pytest.mark.slow
@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(desc, old, new, source, tmp_path):
    assert source.count(old) == 1, f"mutation anchor for {desc!r} must occur exactly once"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new))
    lib = oracle.build(str(src), str(tmp_path / "libmutant.so"))
    impl = oracle.Oracle(lib)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(impl)
        except (AssertionError, ValueError, FloatingPointError) as e:
            caught.append((pin.__name__, str(e)[:80]))
            break
    assert caught, f"no pin caught the planted mistake: {desc}"
    os.remove(lib)
