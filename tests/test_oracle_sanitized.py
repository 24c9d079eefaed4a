"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code only, gcc):
every pin and the tiny-prefill and decode workloads (the latter with its 6.44 GB pool) run
clean, and a copy of the oracle with a planted one-past-the-end write is stopped, which shows
the instrumentation is live.  Each run is a child process with the sanitizer runtime
preloaded (tests/oracle_sanitized_run.py)."""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-g"]


def _runtime():
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                         text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.fixture(scope="module")
def san(tmp_path_factory):
    rt = _runtime()
    if rt is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    d = tmp_path_factory.mktemp("sanitized")
    lib = obuild.build(SAN_FLAGS, out=str(d / "libqsa_ref_san.so"))
    src = open(obuild.SRC).read()
    old = "for (int64_t c = 0; c < numBlocks; ++c) ids[r * numBlocks + c] = (int32_t)c;"
    assert src.count(old) == 1
    bad_src = d / "qsa_ref_oob.c"
    bad_src.write_text(src.replace(old, old.replace("c < numBlocks", "c <= numBlocks")))
    bad = str(d / "libqsa_ref_oob.so")
    subprocess.run(["gcc", *obuild.FLAGS, *SAN_FLAGS, "-Wno-error", str(bad_src), "-o", bad,
                    "-lm"], check=True)
    env = dict(os.environ, LD_PRELOAD=rt, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return lib, bad, env


def _run(env, lib, what):
    return subprocess.run([sys.executable, "-m", "tests.oracle_sanitized_run", lib, what],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.mark.parametrize("what", ["pins", "workloads"])
def test_oracle_clean_under_sanitizers(san, what):
    lib, _, env = san
    r = _run(env, lib, what)
    assert r.returncode == 0 and "done" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_sanitizer_catches_planted_overflow(san):
    _, bad, env = san
    r = _run(env, bad, "oob")
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
