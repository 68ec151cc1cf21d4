"""Race test: the GPU parity suite (all but the full-size cases) run against
the timing-perturbed build libfa_stress.so (compiled with -DFA_STRESS:
wave-uniform pseudo-random pauses of 0..7 x 64 cycles where waves hand LDS
buffers to one another, in every kernel). A missing wait or barrier that the
usual timing hides would show as a parity or determinism failure. Runs in a
child process, which loads the stress library through AWARE_ATTENTION_LIB."""
import os
import subprocess
import sys

import pytest

from tests.gpu_util import say, torch_or_skip

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STRESS_LIB = os.path.join(ROOT, "aware_attention_amd", "libfa_stress.so")
SUITE = ["tests/test_gpu_parity.py", "tests/test_gpu_band.py", "tests/test_gpu_mx8.py",
         "tests/test_gpu_backward.py", "tests/test_gpu_local.py", "tests/test_gpu_d256.py",
         "tests/test_gpu_padded.py", "tests/test_gpu_general.py", "tests/test_gpu_decode.py",
         "tests/test_gpu_rescale.py"]


def test_parity_suite_under_timing_jitter():
    torch_or_skip()
    assert os.path.exists(STRESS_LIB), f"{STRESS_LIB} is not built (python -m aware_attention_amd.build --stress)"
    env = dict(os.environ, AWARE_ATTENTION_LIB=STRESS_LIB)
    probe = subprocess.run([sys.executable, "-c", "import aware_attention_amd._lib as L; L.load(); "
                            "print(L.LIB_PATH)"], env=env, cwd=ROOT, capture_output=True, text=True,
                           timeout=120)
    assert probe.returncode == 0 and probe.stdout.strip().endswith("libfa_stress.so"), probe.stderr
    say("parity suite against libfa_stress.so")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          "-k", "not full_size", "--timeout", "200", "--timeout-method", "thread",
                          *SUITE], env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    tail = "\n".join(res.stdout.splitlines()[-15:])
    print(tail, flush=True)
    assert res.returncode == 0, tail
