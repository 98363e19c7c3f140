"""The host slot manager (csrc/slot_lru.hpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer by the host compiler (no GPU code), run on random traces
under both route rules and compared step by step with the oracle (LRU)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.lru import LayerLRU

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "expert_slot_cache_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("san") / "slot_lru_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", CSRC, os.path.join(ROOT, "tests", "native", "slot_lru_driver.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, E, N, rule, steps):
    lines = [f"{E} {N} {1 if rule == 'static' else 0} {len(steps)}"]
    for ids in steps:
        T, K = ids.shape
        lines.append(f"{T} {K} " + " ".join(str(int(v)) for v in ids.ravel()))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env, timeout=60)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-2000:]
    return r.stdout.splitlines()


@pytest.mark.parametrize("rule", ["distinct", "static"])
@pytest.mark.parametrize("E,N,K,Tmax", [(8, 3, 2, 2), (24, 6, 4, 3), (64, 16, 8, 2), (10, 0, 2, 1), (12, 12, 3, 4)])
def test_sanitized_slot_manager_matches_oracle(driver, E, N, K, Tmax, rule):
    rng = np.random.default_rng(E * 131 + N * 7 + K + (rule == "static"))
    steps = []
    for _ in range(300):
        T = int(rng.integers(1, Tmax + 1))
        p = rng.dirichlet(np.full(E, 0.3))
        steps.append(np.stack([rng.choice(E, size=K, replace=False, p=p) for _ in range(T)]).astype(np.int32))
    out = _run(driver, E, N, rule, steps)
    ref = LayerLRU(E, N, rule)
    for s, ids in enumerate(steps):
        r = ref.step(ids)
        f = out[s].split()
        assert f[0] == "step"
        got = [int(v) for v in f[3:]]
        assert (int(f[1]), int(f[2])) == (r.path, len(r.misses)), s
        assert [tuple(got[i:i + 3]) for i in range(0, len(got), 3)] == [tuple(m) for m in r.misses], s
    tail = {ln.split()[0]: [int(v) for v in ln.split()[1:]] for ln in out[len(steps):]}
    assert tail["map"] == ref.map
    assert tail["owner"] == ref.owner
    lo = ref.lru_order()
    assert tail["order"] == lo + [-1] * (N - len(lo))
    assert tail["counters"] == [ref.steps, ref.hits, ref.misses, ref.fallbacks]
