"""The work protocol of the persistent IKBO-LCB launch (request and candidate tiles claimed from
counters, split-K arrivals, per-request-tile ready flags, bounded waits), restated on the host
with std::atomic in tests/protocol/lcb_fused_model.cpp and run under ThreadSanitizer: every item is
claimed once, the data each side reads is ordered after its writer by the flags, published results
are exact, and with the flags withheld every wait gives up and the run still ends. CPU only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "protocol", "lcb_fused_model.cpp")


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("model") / "lcb_fused_model")
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-pthread", "-fsanitize=thread", SRC, "-o", exe])
    return exe


# (workgroups, request tiles, splits, candidate tiles, publish, wait bound in us)
CASES = [(16, 4, 3, 37, 1, 2000000), (32, 1, 16, 8, 1, 2000000), (8, 9, 1, 200, 1, 2000000),
         (24, 5, 4, 60, 0, 200), (4, 2, 2, 3, 0, 0)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "W%d_Q%d_S%d_T%d_pub%d" % c[:5])
def test_protocol_under_thread_sanitizer(model, case):
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")
    r = subprocess.run([model] + [str(v) for v in case], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                       timeout=300, env=env)
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr[-2000:])
    assert "ok" in r.stdout
