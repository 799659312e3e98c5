"""Plant plausible mistakes in copies of the allocator model; the pins must catch each one.

Each mutant is a one-line edit of oracle/range_alloc.py, loaded from a
temporary file in a child process and run through alloc_pins.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCE = os.path.join(ROOT, "oracle", "range_alloc.py")

MUTANTS = {
    "first_fit_from_the_top": ("for s in range(0, self.num_blocks - n + 1, self.A):",
                               "for s in reversed(range(0, self.num_blocks - n + 1, self.A)):"),
    "grows_cached_extent": ("if (last is not None and last.refs == 1 and last.key is None",
                            "if (last is not None and last.refs == 1"),
    "evicts_newest_first": ("ext = self.lru.pop(0)", "ext = self.lru.pop()"),
    "evicts_one_too_many": ("while self._free_count() < n:",
                            "while self._free_count() <= n and self.lru:"),
    "release_frees_cached": ("if e.key is not None:\n                    self.lru.append(e)",
                             "if False:\n                    self.lru.append(e)"),
    "split_misplaces_prefix": ("mid = Extent(e.start + head, count)",
                               "mid = Extent(e.start, count)"),
    "acquire_leaves_lru": ("if e.refs == 0:\n            self.lru.remove(e)",
                           "if False:\n            self.lru.remove(e)"),
    "runs_taken_from_the_top": ("for s, ln in self.free_runs():",
                                "for s, ln in reversed(self.free_runs()):"),
    "no_space_check_ignores_cache": ("if self._free_count() + sum(e.len for e in self.lru) < n:",
                                     "if self._free_count() < n:"),
}

CHILD = r"""
import importlib.util, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
spec = importlib.util.spec_from_file_location("mutated_range_alloc", {path!r})
mod = importlib.util.module_from_spec(spec); spec.loader.exec_module(mod)
import alloc_pins as AP
AP.pin_allocator(lambda *a: mod.RangeAllocOracle(*a))
print("ALL PINS PASSED")
"""


def run_child(path):
    return subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, tests=HERE, path=path)],
                          capture_output=True, text=True, timeout=300)


def test_unmutated_copy_passes(tmp_path):
    p = tmp_path / "copy.py"
    p.write_text(open(SOURCE).read())
    r = run_child(str(p))
    assert r.returncode == 0 and "ALL PINS PASSED" in r.stdout, r.stderr[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    p = tmp_path / "mutant.py"
    p.write_text(src.replace(old, new))
    r = run_child(str(p))
    assert r.returncode != 0 and "ALL PINS PASSED" not in r.stdout, f"mutant {name} survived"
