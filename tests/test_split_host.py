"""Host logic of the streaming kernels' token splits (csrc/split.h), on the
CPU: tests/split_check.cpp walks the forward's plan for 8,160 shapes and
device sizes the way the kernels walk it (segments, piece slots, the scan's
slot ranges, the folded prefix's arrivals) and checks coverage and slot
invariants.  Each altered copy of the header below plants one plausible
mistake, which the check must report."""
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
HEADER = ROOT / "block_causal_linear_phi_amd" / "csrc" / "split.h"
CHECK = ROOT / "tests" / "split_check.cpp"

# (name, original text, altered text)
MUTANTS = [
    ("padded_block_one_short", "s->Nbp = (int)(J * Lb);", "s->Nbp = (int)(J * Lb) - 1;"),
    ("last_slot_off_by_one", "return (bhc * Nbp + Nbp - 1) / L + bhc;", "return (bhc * Nbp + Nbp - 2) / L + bhc;"),
    ("token_range_not_clamped", "jend < Nb ? jend : Nb};", "jend};"),
    ("last_arriving_workgroup_off_by_one", "return (seq_end_pos(bh, nb, Nbp) - 1) / L; }",
     "return (seq_end_pos(bh, nb, Nbp) - 2) / L; }"),
]


def _compiler():
    for cxx in ("g++", "c++", "clang++"):
        if shutil.which(cxx):
            return cxx
    pytest.skip("no host C++ compiler")


def _build_and_run(tmp_path, header):
    exe = tmp_path / "split_check"
    subprocess.run([_compiler(), "-O2", "-std=c++17", f'-DSPLIT_H="{header}"', "-o", str(exe), str(CHECK)],
                   check=True, capture_output=True, text=True)
    return subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)


def test_split_invariants(tmp_path):
    r = _build_and_run(tmp_path, HEADER)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_split_check_catches(tmp_path, name, old, new):
    text = HEADER.read_text()
    assert text.count(old) == 1, name
    mutant = tmp_path / "split.h"
    mutant.write_text(text.replace(old, new))
    r = _build_and_run(tmp_path, mutant)
    assert r.returncode != 0 and "FAIL" in r.stdout, (name, r.stdout)
