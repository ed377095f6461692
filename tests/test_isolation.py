"""The oracle and the product stay apart, and the product fails loudly.

* nothing in the package (Python or HIP sources) or its C header refers to
  the oracle, and the oracle refers to nothing of the package: they share no
  code, header, table or helper (the seeded input generator, which holds no
  arithmetic of the method, is the one module both consume);
* of the repository's top-level scripts only the benchmark's CPU-baseline
  leg and the smoke check may call the oracle;
* importing the binding without its built library raises ImportError
  (there is no CPU fallback).
"""
import glob
import os
import re
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "combine_epx_get_amd")


def _sources(*patterns):
    out = []
    for p in patterns:
        out += glob.glob(os.path.join(ROOT, p), recursive=True)
    return sorted(out)


def test_package_never_refers_to_the_oracle():
    for f in _sources("combine_epx_get_amd/**/*.py", "combine_epx_get_amd/csrc/*", "include/*.h"):
        if os.path.basename(f) == "workloads.py":
            continue   # the seeded input generator both sides consume (no method arithmetic)
        text = open(f, encoding="utf-8").read()
        assert not re.search(r"\boracle\b", text, re.IGNORECASE), f


def test_oracle_never_refers_to_the_package():
    for f in _sources("oracle/*.py", "oracle/*.c"):
        text = open(f, encoding="utf-8").read()
        assert "combine_epx_get_amd" not in text and "epx.h" not in text and "libepx" not in text, f


def test_only_the_baseline_and_smoke_call_the_oracle():
    bench = open(os.path.join(ROOT, "bench.py"), encoding="utf-8").read()
    # the oracle is imported inside the CPU-baseline leg only (one layer of
    # the oracle, and its timing)
    uses = [m.start() for m in re.finditer(r"import oracle|from oracle", bench)]
    spans = []
    for fn in ("def cpu_layer(", "def cpu_baseline("):
        start = bench.index(fn)
        spans.append((start, bench.index("\ndef ", start + 1)))
    assert uses and all(any(a < u < b for a, b in spans) for u in uses)
    entry = open(os.path.join(ROOT, "__graft_entry__.py"), encoding="utf-8").read()
    uses = [m.start() for m in re.finditer(r"import oracle|from oracle", entry)]
    smoke, build = entry.index("def smoke("), entry.index("def build(")
    assert all(u > smoke or (build < u < smoke and "oracle.build" in entry) for u in uses)


def test_binding_without_library_raises(tmp_path):
    pkg = tmp_path / "combine_epx_get_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(PKG, "epx.py"), pkg / "epx.py")
    (pkg / "__init__.py").write_text("")
    code = ("import sys; sys.path.insert(0, sys.argv[1])\n"
            "try:\n    import combine_epx_get_amd.epx\nexcept ImportError as e:\n    print('ImportError', e)\n")
    r = subprocess.run([sys.executable, "-c", code, str(tmp_path)], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ImportError"), (r.stdout, r.stderr)
