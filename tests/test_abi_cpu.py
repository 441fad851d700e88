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
    # and nothing else: launchers and kernels stay internal (hidden visibility)
    exported = set(re.findall(r"\bT (\S+)$", out, flags=re.M))
    assert exported == set(declared_functions()), f"unexpected exports: {sorted(exported - set(declared_functions()))}"


def header_status_codes():
    """The attn_status enum as include/attn_fwd.h declares it: {name: value}."""
    text = open(os.path.join(INCLUDE, "attn_fwd.h")).read()
    body = re.search(r"typedef enum \{([^{}]*)\} attn_status;", text).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"(ATTN_\w+)\s*=\s*(-?\d+)", body)}


def test_status_codes_pinned():
    """The seven codes of the interface's original set keep their values (a caller built against
    it reads them unchanged); the codes added later follow from -7 down; the binding mirrors the
    header exactly."""
    codes = header_status_codes()
    original = {"ATTN_OK": 0, "ATTN_ERR_NULL": -1, "ATTN_ERR_SHAPE": -2, "ATTN_ERR_HEAD_DIM": -3,
                "ATTN_ERR_DTYPE": -4, "ATTN_ERR_SCALE": -5, "ATTN_ERR_LAUNCH": -6}
    added = {"ATTN_ERR_FLAG": -7, "ATTN_ERR_ALIGN": -8, "ATTN_ERR_WINDOW": -9, "ATTN_ERR_WORKSPACE": -10,
             "ATTN_ERR_SCRATCH": -11}
    assert codes == {**original, **added}
    assert {v: k for k, v in codes.items()} == binding.STATUS


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
    (dict(causal=-1), -7), (dict(causal=2), -7), (dict(Nk=1 << 23, D=64), -2),
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
    (dict(causal=2), -7), (dict(o=FAKE + 8), -8), (dict(window=-2, causal=3), -7),
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


DECODE_OK = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, Nq=1, Nk=4096, D=64, scale=0.125,
                 causal=1, key_lens=None, dtype=2, ws=FAKE, ws_bytes=1 << 20, stream=None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), -1), (dict(B=0), -2), (dict(D=96), -3), (dict(dtype=5), -4),
    (dict(scale=float("inf")), -5), (dict(causal=2), -7), (dict(lse=FAKE + 4), -8),
    (dict(ws=None), -1), (dict(ws=FAKE + 8), -8), (dict(ws_bytes=0), -10), (dict(ws_bytes=4159), -10),
])
def test_host_validation_decode(over, code):
    """attn_decode rejects bad arguments and a missing, misaligned or short workspace on the host
    (B=H=Nq=1, Nk=4096, D=64 spreads the keys over 16 splits: 16 * (64 + 1) * 4 = 4160 bytes)."""
    a = dict(DECODE_OK)
    a.update(over)
    rc = binding.attn_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                             a["Nk"], a["D"], a["scale"], a["causal"], a["key_lens"], a["dtype"],
                             a["ws"], a["ws_bytes"], a["stream"])
    assert rc == code


def test_decode_workspace_size():
    """The workspace holds n_splits fp32 copies of O and LSE: n_splits * B*H*Nq * (D + 1) * 4
    bytes, with at most 64 splits of at least 256 keys; 0 when the cache is not split, or for
    arguments attn_decode would reject."""
    ws = binding.attn_decode_workspace_size
    assert ws(1, 1, 1, 4096, 64, 2) == 16 * 65 * 4
    assert ws(1, 1, 1, 511, 128, 2) == 0          # below two 256-key splits
    assert ws(1, 1, 1, 512, 128, 2) == 2 * 129 * 4
    assert ws(64, 32, 1, 1 << 20, 128, 2) == 0    # 2048 workgroups without a split
    for B, H, Nq, Nk, D, dt in ((1, 32, 1, 32768, 128, 2), (4, 32, 1, 4096, 128, 2),
                                (16, 32, 1, 8192, 128, 1), (2, 8, 200, 70000, 64, 0)):
        n = ws(B, H, Nq, Nk, D, dt)
        unit = B * H * Nq * (D + 1) * 4
        assert n % unit == 0 and 2 <= n // unit <= 64, (B, H, Nq, Nk, D, n)
        assert n // unit <= Nk // 256
    for bad in ((0, 1, 1, 4096, 64, 2), (1, 1, 1, 4096, 80, 2), (1, 1, 1, 4096, 64, 7),
                (1, 1, 0, 4096, 64, 2)):
        assert ws(*bad) == 0


BWD_OK = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dlse=None, dq=FAKE, dk=FAKE, dv=FAKE,
              B=2, H=3, Nq=40, Nk=50, D=128, scale=0.088, causal=1, key_lens=None, dtype=2,
              ws=FAKE, ws_bytes=1 << 20, stream=None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), -1), (dict(do=None), -1), (dict(dv=None), -1), (dict(lse=None), -1),
    (dict(B=0), -2), (dict(Nk=0), -2), (dict(D=96), -3), (dict(dtype=-1), -4), (dict(dtype=3), -4),
    (dict(scale=float("nan")), -5), (dict(causal=2), -7), (dict(dq=FAKE + 4), -8),
    (dict(dlse=FAKE + 4), -8), (dict(key_lens=FAKE + 1), -8), (dict(ws=None), -1),
    (dict(ws=FAKE + 8), -8), (dict(ws_bytes=2 * 2 * 3 * 64 * 4 - 1), -10), (dict(Nq=1 << 22, D=128), -2),
    (dict(B=4096, H=64, Nq=1024, D=64, ws_bytes=1 << 40), -2),
])
def test_host_validation_bwd(over, code):
    """attn_bwd checks every argument on the host before anything is enqueued."""
    a = dict(BWD_OK)
    a.update(over)
    rc = binding.attn_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dlse"], a["dq"], a["dk"],
                          a["dv"], a["B"], a["H"], a["Nq"], a["Nk"], a["D"], a["scale"], a["causal"],
                          a["key_lens"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])
    assert rc == code


def test_bwd_workspace_size():
    """Two fp32 planes of [B, H, Nq rounded up to 64]; 0 for an empty shape."""
    ws = binding.attn_bwd_workspace_size
    assert ws(2, 3, 40) == 2 * 2 * 3 * 64 * 4
    assert ws(1, 1, 32) == 2 * 64 * 4
    assert ws(1, 1, 65) == 2 * 128 * 4
    assert ws(1, 32, 16384) == 2 * 32 * 16384 * 4
    assert ws(0, 1, 1) == 0 and ws(1, 0, 1) == 0 and ws(1, 1, 0) == 0


@pytest.mark.parametrize("over,code", [
    (dict(window=-2), -9), (dict(window=-1000), -9), (dict(q=None), -1), (dict(dtype=3), -4),
    (dict(causal=2), -7), (dict(ws=None), -1),
])
def test_host_validation_bwd_window(over, code):
    """attn_bwd_window checks its band argument on the host like the others."""
    a = dict(BWD_OK, window=16)
    a.update(over)
    rc = binding.attn_bwd_window(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dlse"], a["dq"],
                                 a["dk"], a["dv"], a["B"], a["H"], a["Nq"], a["Nk"], a["D"], a["scale"],
                                 a["causal"], a["window"], a["key_lens"], a["dtype"], a["ws"], a["ws_bytes"],
                                 a["stream"])
    assert rc == code


def test_c_caller_is_built_and_checks_its_arguments():
    """The plain C caller (gcc, public header only) is built with the library; given no arguments
    it prints its usage and exits 1 before any GPU call."""
    caller = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "c_abi",
                          "attn_fwd_c_caller")
    assert os.access(caller, os.X_OK)
    r = subprocess.run([caller], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr


@pytest.mark.parametrize("over,code", [
    (dict(q=None), -1), (dict(D=96), -3), (dict(causal=2), -7), (dict(o=FAKE + 8), -8),
    # B=1, H=32, Nq=128, Nk=16384, D=128: 32 key splits of 128 rows need 67.6 MB of partials
    (dict(B=1, H=32, Nq=128, Nk=16384, D=128), -11),
])
def test_host_validation_decode_noalloc(over, code):
    """attn_decode_noalloc checks its arguments like attn_decode and refuses, on the host and
    before touching a device, a call whose split partials exceed its static scratch."""
    a = dict(DECODE_OK)
    a.update(over)
    rc = binding.attn_decode_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                                     a["Nk"], a["D"], a["scale"], a["causal"], a["key_lens"], a["dtype"],
                                     a["stream"])
    assert rc == code


def test_decode_noalloc_scratch_limit_matches_header():
    text = open(os.path.join(INCLUDE, "attn_fwd.h")).read()
    m = re.search(r"#define ATTN_DECODE_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == 16 << 20
    # just under and just over the limit: Nq queries per (b, h), 1024 split workgroups
    for nq, want in ((31, 0), (32, -11)):
        need = binding.attn_decode_workspace_size(1, 32, nq, 16384, 128, 2)
        rc = binding.attn_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 32, nq, 16384, 128, 0.1, 1, None, 2, None) \
            if want else None
        if want:
            assert need > 16 << 20 and rc == want
        else:
            assert need <= 16 << 20
