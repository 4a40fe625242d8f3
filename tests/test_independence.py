"""The oracle and the HIP path share no code: neither imports the other, the
oracle touches no GPU library, and the product package never imports the
oracle or any CPU fallback."""

import ast
import glob
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _imports(path):
    tree = ast.parse(open(path).read())
    mods = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            mods.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom):
            if node.level == 0 and node.module:
                mods.add(node.module.split(".")[0])
    return mods


def test_oracle_imports_only_numpy_and_itself():
    for f in glob.glob(os.path.join(ROOT, "oracle", "*.py")):
        bad = _imports(f) - {"numpy", "math", "__future__"}
        assert not bad, f"{f} imports {bad}"


def test_package_never_imports_the_oracle():
    for f in glob.glob(os.path.join(ROOT, "fp8_block_scaled_dsmoe_amd", "**", "*.py"), recursive=True):
        mods = _imports(f)
        assert "oracle" not in mods and "numpy" not in mods, f"{f} imports {mods}"


def test_kernel_sources_do_not_mention_the_oracle():
    for f in glob.glob(os.path.join(ROOT, "fp8_block_scaled_dsmoe_amd", "csrc", "*")):
        assert "oracle" not in open(f).read().lower(), f
