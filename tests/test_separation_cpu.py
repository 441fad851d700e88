"""The oracle and the GPU path share no code: the package, its kernels and the public headers never
import, include, link or name the oracle's modules or library, the oracle never reaches into the
package (the seeded input generators in `inputs.py` aside, which hold none of the method's
arithmetic), and importing the product or the bench leaves the oracle unloaded."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "transformer_scaled_dot_amd")
ORACLE = os.path.join(ROOT, "oracle")


def source_files(top, exts):
    for dirpath, dirnames, files in os.walk(top):
        dirnames[:] = [d for d in dirnames if d not in ("__pycache__", "_build")]
        for f in files:
            if f.endswith(exts):
                yield os.path.join(dirpath, f)


def code_lines(path):
    """Source lines with comments and docstring-only lines dropped (a mention is not a use)."""
    text = open(path, encoding="utf-8").read()
    if path.endswith(".py"):
        text = re.sub(r'"""(.*?)"""', "", text, flags=re.S)
        return [ln.split("#", 1)[0] for ln in text.splitlines()]
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return [ln.split("//", 1)[0] for ln in text.splitlines()]


def test_product_never_reaches_the_oracle():
    pattern = re.compile(r"\boracle\b|liboracle|attn_oracle")
    files = list(source_files(PKG, (".py", ".hip", ".h", ".cpp", ".c"))) + \
        list(source_files(os.path.join(ROOT, "include"), (".h",)))
    assert files
    for f in files:
        for n, ln in enumerate(code_lines(f), 1):
            assert not pattern.search(ln), f"{os.path.relpath(f, ROOT)}:{n} names the oracle: {ln.strip()}"


def test_oracle_never_reaches_the_product():
    allowed = {"transformer_scaled_dot_amd.inputs"}
    files = list(source_files(ORACLE, (".py", ".c", ".h")))
    assert any(f.endswith(".c") for f in files) and any(f.endswith(".py") for f in files)
    for f in files:
        for n, ln in enumerate(code_lines(f), 1):
            for mod in re.findall(r"transformer_scaled_dot_amd[\w.]*", ln):
                assert mod in allowed, f"{os.path.relpath(f, ROOT)}:{n} uses {mod}"
            assert not re.search(r"libattn_fwd|csrc|attn_common|attn_fwd\.h|attn_bwd\.h", ln), \
                f"{os.path.relpath(f, ROOT)}:{n}: {ln.strip()}"
            if f.endswith((".c", ".h")):
                inc = re.match(r'\s*#\s*include\s*"([^"]+)"', ln)
                assert inc is None or os.path.exists(os.path.join(ORACLE, inc.group(1))), \
                    f"{os.path.relpath(f, ROOT)}:{n} includes {inc.group(1)} from outside oracle/"


def test_importing_the_product_or_the_bench_loads_no_oracle():
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import transformer_scaled_dot_amd, transformer_scaled_dot_amd.inputs, bench\n"
            "from transformer_scaled_dot_amd import binding\n"
            "print(sorted(m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')))") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True, cwd=ROOT)
    assert out.stdout.strip() == "[]"


def test_input_generators_hold_no_attention_arithmetic():
    """inputs.py draws and shapes random tensors; it computes no softmax, exponential or product of
    Q and K (both sides compute those on their own)."""
    lines = code_lines(os.path.join(PKG, "inputs.py"))
    for n, ln in enumerate(lines, 1):
        assert not re.search(r"softmax|\bexp\(|logsumexp|\bmatmul\b|\w\s*@\s*\w|einsum|\.dot\(", ln), \
            f"inputs.py:{n}: {ln.strip()}"
