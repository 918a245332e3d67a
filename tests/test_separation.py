"""The oracle and the HIP path share nothing, and the product path has no
CPU fallback (CPU only).

- Nothing in the package imports the oracle; the oracle imports only numpy
  and the standard library; the seeded input generators (synth) import
  neither side.
- bench.py reaches the oracle only from its cpu_baseline functions, and
  __graft_entry__.py only from smoke() and, to compile the oracle's C twin
  (building the checker, not using it), from build().
- The oracle's C source includes only the C standard library.
- The HIP sources include only each other and include/.
- A missing library, or host tensors handed to an entry point, raise
  instead of computing anything on the CPU.
"""

import ast
import os

import pytest

import combine_moe_layout_06_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "combine_moe_layout_06_amd")


def _py_files(folder):
    for dirpath, _, names in os.walk(folder):
        for n in names:
            if n.endswith(".py"):
                yield os.path.join(dirpath, n)


def _imports(tree):
    """(top-level module name, enclosing function name or None) per import."""
    out = []

    def visit(node, func):
        for child in ast.iter_child_nodes(node):
            f = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else func
            if isinstance(child, ast.Import):
                out.extend((a.name.split(".")[0], func) for a in child.names)
            elif isinstance(child, ast.ImportFrom) and child.level == 0 and child.module:
                out.append((child.module.split(".")[0], func))
            visit(child, f)

    visit(tree, None)
    return out


def _parse(path):
    with open(path) as f:
        return ast.parse(f.read(), path)


def test_package_never_imports_the_oracle():
    for path in _py_files(PKG):
        mods = {m for m, _ in _imports(_parse(path))}
        assert "oracle" not in mods, path
        assert "synth" not in mods, path


def test_oracle_imports_only_numpy_and_the_standard_library():
    allowed = {"numpy", "__future__", "math", "typing", "dataclasses", "itertools",
               "functools", "struct", "ctypes", "os", "subprocess"}
    for path in _py_files(os.path.join(ROOT, "oracle")):
        mods = {m for m, _ in _imports(_parse(path))}
        assert mods <= allowed, (path, mods - allowed)


def test_input_generators_import_neither_side():
    for path in _py_files(os.path.join(ROOT, "synth")):
        mods = {m for m, _ in _imports(_parse(path))}
        assert not mods & {"oracle", "combine_moe_layout_06_amd", "torch"}, (path, mods)


def test_bench_reaches_the_oracle_only_from_its_cpu_baseline():
    uses = [(m, f) for m, f in _imports(_parse(os.path.join(ROOT, "bench.py"))) if m == "oracle"]
    assert uses, "bench.py times the oracle as its cpu_baseline"
    for _, func in uses:
        assert func is not None and func.startswith("cpu_baseline"), func


def test_graft_entry_reaches_the_oracle_only_from_smoke():
    uses = [(m, f) for m, f in _imports(_parse(os.path.join(ROOT, "__graft_entry__.py")))
            if m == "oracle"]
    assert uses
    for _, func in uses:
        assert func in ("smoke", "build"), func
    src = open(os.path.join(ROOT, "__graft_entry__.py")).read()
    build_src = src[src.index("def build"):src.index("def smoke")]
    assert "c_twin.build()" in build_src and "O." not in build_src


def test_oracle_c_source_includes_only_the_standard_library():
    std = {"<math.h>", "<stdint.h>", "<string.h>", "<stdlib.h>", "<stddef.h>"}
    for name in os.listdir(os.path.join(ROOT, "oracle")):
        if name.endswith((".c", ".h")):
            with open(os.path.join(ROOT, "oracle", name)) as f:
                for line in f:
                    if line.strip().startswith("#include"):
                        assert line.split()[1] in std, (name, line)


def test_hip_sources_include_only_their_own_headers():
    csrc = os.path.join(PKG, "csrc")
    own = set(os.listdir(csrc)) | set(os.listdir(os.path.join(ROOT, "include")))
    for name in os.listdir(csrc):
        with open(os.path.join(csrc, name)) as f:
            for line in f:
                s = line.strip()
                if s.startswith("#include \""):
                    inc = os.path.basename(s.split('"')[1])
                    assert inc in own, (name, s)


def test_missing_library_raises(monkeypatch):
    monkeypatch.setattr(M, "_lib", None)
    monkeypatch.setattr(M, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libmoe_layout.so"))
    with pytest.raises(RuntimeError, match="build"):
        M.lib()
    with pytest.raises(RuntimeError, match="build"):
        M.moe_layout_workspace_bytes(16, 8, 2)


def test_host_tensors_are_refused():
    torch = pytest.importorskip("torch")
    x = torch.zeros((4, 8), dtype=torch.int16)
    dst = torch.zeros((4, 2), dtype=torch.int32)
    w = torch.zeros((4, 2), dtype=torch.float32)
    out = torch.zeros((4, 8), dtype=torch.int16)
    with pytest.raises(ValueError, match="device tensor"):
        M.moe_combine(4, 8, 2, 8, x, dst, w, out)
