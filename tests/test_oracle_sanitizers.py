"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

``oracle/oracle.c`` is compiled together with ``oracle_sanitize_driver.c``,
which calls every oracle function on small seeded cases with each buffer in
its own exact-size heap block; any out-of-bounds access, signed overflow or
other undefined behaviour aborts the run.
"""
import os
import shutil
import subprocess

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "oracle_sanitize_driver.c")


def _have_sanitizers() -> bool:
    if shutil.which("gcc") is None:
        return False
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return os.path.isabs(out) and os.path.exists(out)


@pytest.mark.skipif(not _have_sanitizers(), reason="gcc with AddressSanitizer runtime not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra",
           oracle.SOURCE, DRIVER, "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stdout[-2000:] + res.stderr[-4000:]


@pytest.mark.skipif(not _have_sanitizers(), reason="gcc with AddressSanitizer runtime not available")
@pytest.mark.parametrize("name,old,new", [
    ("all_gather_writes_one_past", "memcpy((char*)y[q] + at * esize, x[r], counts[r] * esize);",
     "memcpy((char*)y[q] + at * esize, x[r], counts[r] * esize + (r == nranks - 1 ? esize : 0));"),
    ("reduce_scatter_reads_next_chunk", "fold_one(x, (size_t)r * m, nranks, i, dtype, op, y[r], i);",
     "fold_one(x, (size_t)(r + 1) * m, nranks, i, dtype, op, y[r], i);"),
])
def test_planted_overrun_is_caught(tmp_path, name, old, new):
    """The driver really reaches the edges: an off-by-one planted in a copy of
    the oracle makes the sanitized run fail."""
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, name
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    exe = str(tmp_path / "oracle_sanitize_mutant")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    str(mutated), DRIVER, "-o", exe], check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:verify_asan_link_order=0")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode != 0 and "AddressSanitizer" in res.stderr, name
