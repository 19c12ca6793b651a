"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle's C source is compiled with -fsanitize=address,undefined (every
finding fatal) into a temporary library, and the pin suites run in a child
interpreter that loads it in place of the oracle (PSO_ORACLE_LIB) with the
sanitizer runtime preloaded: an out-of-bounds access, use after free, signed
overflow, misaligned access or invalid shift anywhere the pins reach ends the
run with a report."""
import os
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "polestar_oracle.c")
PIN_SUITES = ["test_oracle_attn_kl.py", "test_oracle_commit.py", "test_oracle_cosine.py",
              "test_oracle_formats.py", "test_oracle_kmeans.py", "test_oracle_topk_gather.py"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _sanitized_run(tmp, source, suites):
    """Compile `source` (the oracle's text) with the sanitizers, run the given
    pin suites against it in a child interpreter; return (returncode, output)."""
    src = os.path.join(tmp, "polestar_oracle.c")
    open(src, "w").write(source)
    open(os.path.join(tmp, "polestar_oracle.h"), "w").write(open(SRC[:-2] + ".h").read())
    lib = os.path.join(tmp, "libpolestar_oracle_asan.so")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-Werror", "-ffp-contract=off",
           "-fno-fast-math", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fPIC", "-shared", src, "-o", lib, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env.update(PSO_ORACLE_LIB=lib, LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # -s: the sanitizers report on stderr, which pytest would otherwise capture
    # and lose when the report ends the process
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *[os.path.join(HERE, f) for f in suites]], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    return p.returncode, p.stdout + p.stderr


needs_asan = pytest.mark.skipif(_runtime("libasan.so") is None,
                                reason="gcc's AddressSanitizer runtime is not installed")


@needs_asan
def test_pins_pass_under_address_and_undefined_behaviour_sanitizers():
    with tempfile.TemporaryDirectory(prefix="pso_asan_") as tmp:
        rc, out = _sanitized_run(tmp, open(SRC).read(), PIN_SUITES)
        assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
        assert rc == 0, out[-4000:]
        assert " passed" in out


@needs_asan
def test_the_sanitized_run_catches_a_planted_overread():
    """The same run on a copy of the oracle whose row-norm loop reads one
    element past each row (past the end of the buffer on the last row) must
    end with an AddressSanitizer report."""
    planted = open(SRC).read().replace(
        "row_norm[r] = row_norm_one(H, dtype, r * (size_t)s->d, s->d);",
        "row_norm[r] = row_norm_one(H, dtype, r * (size_t)s->d, s->d + 1);")
    assert planted != open(SRC).read()
    with tempfile.TemporaryDirectory(prefix="pso_asan_") as tmp:
        rc, out = _sanitized_run(tmp, planted, ["test_oracle_kmeans.py"])
        assert rc != 0 and "AddressSanitizer" in out, out[-2000:]
