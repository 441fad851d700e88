"""The C-ABI library on the CPU: it loads, exports every declared symbol, and rejects bad
arguments on the host before touching a device (no compute call is made here)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from transformer_scaled_dot_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def declared_functions():
    names = []
    for fn in sorted(os.listdir(INCLUDE)):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(INCLUDE, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return names


def test_header_declares_the_entry_points():
    assert set(declared_functions()) == set(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"libattn_fwd.so does not export {name}"
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, flags=re.M), f"{name} is not a defined text symbol"


def test_status_strings():
    for code in binding.STATUS:
        s = binding.attn_status_str(code)
        assert isinstance(s, str) and s
    assert binding.attn_status_str(12345) == "unknown status"


FAKE = 0x1000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("over,code", [
    (dict(q=None), -1), (dict(lse=None), -1), (dict(B=0), -2), (dict(H=-1), -2),
    (dict(Nq=0), -2), (dict(Nk=0), -2), (dict(D=32), -3), (dict(D=256), -3), (dict(dtype=3), -4),
    (dict(dtype=-1), -4), (dict(scale=float("nan")), -5), (dict(scale=float("-inf")), -5),
    (dict(causal=-1), -6), (dict(causal=2), -6), (dict(Nk=1 << 23, D=64), -2),
    (dict(o=FAKE + 8), -8), (dict(q=FAKE + 2), -8), (dict(key_lens=FAKE + 2), -8),
])
def test_host_validation(over, code):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, Nq=8, Nk=8, D=64, scale=0.125,
             causal=0, key_lens=None, dtype=2, stream=None)
    a.update(over)
    rc = binding.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                          a["Nk"], a["D"], a["scale"], a["causal"], a["key_lens"], a["dtype"],
                          a["stream"])
    assert rc == code


@pytest.mark.parametrize("over,code", [
    (dict(window=-2), -9), (dict(window=-(1 << 30)), -9), (dict(q=None), -1), (dict(D=32), -3),
    (dict(causal=2), -6), (dict(o=FAKE + 8), -8), (dict(window=-2, causal=3), -6),
])
def test_host_validation_window(over, code):
    """attn_fwd_window checks its band argument on the host like the others."""
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, Nq=8, Nk=8, D=64, scale=0.125,
             causal=0, window=3, key_lens=None, dtype=2, stream=None)
    a.update(over)
    rc = binding.attn_fwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                                 a["Nk"], a["D"], a["scale"], a["causal"], a["window"],
                                 a["key_lens"], a["dtype"], a["stream"])
    assert rc == code


def test_missing_library_fails_loudly():
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from transformer_scaled_dot_amd import binding\n"
            "try:\n    binding.load_library('/nonexistent/libattn_fwd.so')\n"
            "except RuntimeError as e:\n    print('raised', e)\n") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True)
    assert out.stdout.startswith("raised") and "no fallback" in out.stdout


def test_package_import_loads_nothing():
    code = ("import sys; sys.path.insert(0, %r)\nimport transformer_scaled_dot_amd, "
            "transformer_scaled_dot_amd.inputs\nfrom transformer_scaled_dot_amd import binding\n"
            "print(binding._lib is None)") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True)
    assert out.stdout.strip() == "True"
