"""The measurement probes of libleapq_probe.so on the GPU: the append's memory
traffic without arithmetic, the plain streaming read and the matrix/VALU
co-execution probe run and return positive times (their rates are measured
by bench.py and the profiling programs)."""
import pytest

from quantized_recurrent_state_amd import profiling
from tests.gpu_harness import progress

pytestmark = pytest.mark.gpu


def test_append_pattern_probe_runs():
    progress("  probe: append pattern, 256 heads, n = 0 and 7; streaming read of 4 MB")
    t = profiling.append_pattern(256, 4, 16, 2, 512, [0, 7], reps=3)
    assert set(t) == {0, 7} and all(v > 0.0 for v in t.values()), t
    t32 = profiling.append_pattern(64, 0, 4, 4, 256, [3], reps=2)  # C = 0, fp32 keys, bf16-sized corrections
    assert t32[3] > 0.0
    assert profiling.read_ceiling(4 << 20, reps=3) > 0.0


def test_coexec_probe_runs():
    progress("  probe: matrix/VALU co-execution, both accumulator forms, 1 launch each")
    for agpr in (False, True):
        t = profiling.coexec(agpr, lds=40960, reps=1)
        assert set(t) == {0, 1, 2} and all(v > 0.0 for v in t.values()), t
