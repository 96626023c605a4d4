"""Race and ordering checks of the sliding engine's host logic on the CPU.

engine.cpp, adam.cpp and layout.cpp are compiled unchanged with g++ against
a fake HIP runtime (tests/engine_cpu/fake_hip.cpp: one worker thread per
stream, events with the runtime's ordering rules and nothing more) and
stand-in kernels that touch the real buffers (fake_kernels.cpp).  The
driver (engine_check.cpp) runs 18 engine configurations -- synchronous and
pipelined steps, checkpointing, host or device head Adam, windows 2 and 3,
keep-turnaround without Adam (also past two windows, windows 2 and 3, and
with checkpointing), no head, fp32, fp16 loss scaling with and
without an injected non-finite layer -- and compares every loss, master,
moment and parameter bit for bit with a sequential model of the same steps.
Every "device" buffer (pool, activation region, workspace, head scratch)
starts as all-ones bytes (NaN in every storage dtype), so a stand-in that
reads device memory before the engine's data reached it breaks the match.

* ThreadSanitizer build: random delays in every stream (FAKE_HIP_JITTER_US)
  vary the interleavings; any access the engine leaves unordered is
  reported.  Small delays give many interleavings quickly, 2 ms delays let
  slow copies expose waits that fast ones hide behind the engine's own
  event polling.
* AddressSanitizer + UndefinedBehaviorSanitizer build of the same.
* Mutation checks: the forward's wait for its parameters removed from a
  copy of engine.cpp, or an upload that waits for the wrong forward, must
  be reported.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "layer_sliding_offloaded_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "engine_cpu")
ADAM_FLAGS = ["-mavx2", "-mfma", "-mf16c", "-fno-math-errno", "-ffp-contract=off"]  # as the library builds it

SOURCES = [
    (os.path.join(CSRC, "adam.cpp"), ADAM_FLAGS),
    (os.path.join(CSRC, "engine.cpp"), ["-mf16c"]),
    (os.path.join(CSRC, "layout.cpp"), []),
    (os.path.join(HERE, "fake_hip.cpp"), []),
    (os.path.join(HERE, "fake_kernels.cpp"), ["-mf16c"]),
    (os.path.join(HERE, "engine_check.cpp"), ["-mf16c"]),
]
SANITIZERS = {
    "tsan": ["-fsanitize=thread"],
    "asan": ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"],
}

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not available")


def _compile(out_dir, san, sources, extra=()):
    flags = ["-std=c++17", "-O1", "-g", "-pthread", "-I", os.path.join(HERE, "fake_hip"), "-I", CSRC,
             *SANITIZERS[san]]
    objs = []

    def one(item):
        src, own = item
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        subprocess.run(["g++", *flags, *own, "-c", src, "-o", obj], check=True, capture_output=True, text=True)
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(one, list(sources) + [(e, []) for e in extra]))
    exe = os.path.join(out_dir, "engine_check")
    subprocess.run(["g++", "-pthread", *SANITIZERS[san], *objs, "-o", exe], check=True, capture_output=True,
                   text=True)
    return exe


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    out = {}
    for san in SANITIZERS:
        d = str(tmp_path_factory.mktemp(f"engine_{san}"))
        extra = [os.path.join(HERE, "tsan_clockwait.cpp")] if san == "tsan" else []
        try:
            out[san] = _compile(d, san, SOURCES, extra)
        except subprocess.CalledProcessError as e:
            pytest.fail(f"{san} build failed:\n{e.stderr[-3000:]}")
    return out


def _run(exe, jitter, seed, *scenarios, san="tsan"):
    env = dict(os.environ, FAKE_HIP_JITTER_US=str(jitter), FAKE_HIP_SEED=str(seed))
    env["TSAN_OPTIONS"] = "halt_on_error=1 exitcode=66"
    env["ASAN_OPTIONS"] = "detect_leaks=1"
    env.pop("SF_FAULT_ADAM_JOB", None)
    p = subprocess.run([exe, *scenarios], env=env, capture_output=True, text=True, timeout=600)
    print(p.stdout[-2000:], file=sys.stderr)
    return p


@pytest.mark.parametrize("jitter,seed", [(0, 1), (30, 2), (2000, 3)], ids=["no-delay", "delay-30us", "delay-2ms"])
def test_engine_matches_sequential_model_without_races(builds, jitter, seed):
    p = _run(builds["tsan"], jitter, seed)
    assert "ThreadSanitizer" not in p.stderr, p.stderr[-6000:]
    assert p.returncode == 0, p.stdout[-3000:] + p.stderr[-3000:]
    assert "18 scenarios, 0 failures" in p.stdout


def test_engine_memory_and_undefined_behaviour(builds):
    p = _run(builds["asan"], 30, 5, san="asan")
    assert "Sanitizer" not in p.stderr and "runtime error" not in p.stderr, p.stderr[-6000:]
    assert p.returncode == 0, p.stdout[-3000:]
    assert "18 scenarios, 0 failures" in p.stdout


def test_checker_reports_a_missing_wait(tmp_path):
    """Plant a bug in a copy of engine.cpp: the compute stream no longer
    waits for a layer's parameters before its forward.  The checker must
    fail the scenario (a race report, a wrong result, or both)."""
    src = open(os.path.join(CSRC, "engine.cpp")).read()
    line = "    SF_HIP(hipStreamWaitEvent(e->s_comp, gs ? e->ev_gslot_ready[ug] : e->ev_param_ready[u], 0));\n"
    assert src.count(line) == 1
    mutant = tmp_path / "engine.cpp"
    mutant.write_text(src.replace(line, ""))
    sources = [(str(mutant), ["-mf16c"]) if s.endswith("engine.cpp") else (s, f) for s, f in SOURCES]
    exe = _compile(str(tmp_path), "tsan", sources, [os.path.join(HERE, "tsan_clockwait.cpp")])
    # the mutant's sources include the library headers from CSRC
    p = _run(exe, 50, 1, "adam-sync", "adam-pipe")
    assert p.returncode != 0
    assert "ThreadSanitizer: data race" in p.stderr or "FAIL:" in p.stdout


def test_checker_reports_a_wrong_upload_dependency(tmp_path):
    """Plant a bug in a copy of engine.cpp: without Adam after a preloaded
    start, the second page's uploads wait for the forward 2W layers back (none)
    instead of W back, so they overwrite parameters a forward still reads.
    The configurations with gradient-region pages must fail."""
    src = open(os.path.join(CSRC, "engine.cpp")).read()
    line = "  auto dep = [&](int j) { return params_first && j < 2 * W ? j - W : j - 2 * W; };\n"
    assert src.count(line) == 1
    mutant = tmp_path / "engine.cpp"
    mutant.write_text(src.replace(line, "  auto dep = [&](int j) { return j - 2 * W; };\n"))
    sources = [(str(mutant), ["-mf16c"]) if s.endswith("engine.cpp") else (s, f) for s, f in SOURCES]
    exe = _compile(str(tmp_path), "tsan", sources, [os.path.join(HERE, "tsan_clockwait.cpp")])
    p = _run(exe, 30, 1, "noadam-keep-pipe-l8", "noadam-keep-l7", "noadam-keep-pipe-l5", "noadam-keep-pipe-w3-l10")
    assert p.returncode != 0
    assert "ThreadSanitizer: data race" in p.stderr or "FAIL:" in p.stdout

