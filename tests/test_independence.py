"""The product path and the oracle share no code: no product module imports or
loads anything under oracle/, the oracle imports nothing from the product
package, and the HIP sources include nothing from oracle/. Only bench.py's
CPU-baseline leg and the smoke check reach the oracle, through oracle.ref."""
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "embeddings_a2av_virtual_amd")


def _files(root, exts):
    for dp, _, fs in os.walk(root):
        if "__pycache__" in dp:
            continue
        for f in fs:
            if f.endswith(exts):
                yield os.path.join(dp, f)


def test_product_does_not_touch_the_oracle():
    for path in _files(PKG, (".py", ".hip", ".hpp", ".h", ".cpp")):
        text = open(path).read()
        assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), path
        assert not re.search(r"a2av_ref|liba2av_ref", text), path


def test_oracle_does_not_touch_the_product():
    for path in _files(os.path.join(ROOT, "oracle"), (".py", ".c", ".h")):
        text = open(path).read()
        assert not re.search(r"^\s*(from|import)\s+embeddings_a2av_virtual_amd", text, re.M), path
        assert not re.search(r"#include\s+[<\"][^>\"]*a2av\.h[>\"]", text), path
        assert "liba2av.so" not in text, path


def test_oracle_users_are_the_allowed_ones():
    users = []
    for path in _files(ROOT, (".py",)):
        rel = os.path.relpath(path, ROOT)
        if rel.startswith(("_work", "oracle", "tests", ".")):
            continue
        if re.search(r"^\s*(from|import)\s+oracle\b", open(path).read(), re.M):
            users.append(rel)
    assert sorted(users) == ["__graft_entry__.py", "bench.py"], users


def test_bench_reaches_the_oracle_only_in_cpu_legs():
    text = open(os.path.join(ROOT, "bench.py")).read()
    # every import of the oracle sits in a function whose CPU leg is switched by --no-cpu
    funcs = re.findall(r"def (\w+)\([^)]*\):(?:(?!\ndef ).)*?from oracle", text, re.S)
    assert set(funcs) <= {"cpu_baseline", "row_benchmarks"}, funcs
