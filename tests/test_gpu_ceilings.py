"""The ceiling probes run and report figures inside the physical bounds: a
read-only stream and the decode batch's paged reads below the 8 TB/s HBM
peak, the bf16 library GEMM below the 2.5 PFLOP/s dense peak, and a
transcendental issuing no faster than an FMA.  The figures themselves are
measurements, printed for the record, not asserted."""
import pytest
import torch

import ceilings
from gpu_common import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def test_read_probes_stay_below_the_hbm_peak():
    for nt in (False, True):
        r = ceilings.stream_read(nbytes=1 << 30, reps=5, nt=nt)
        p = ceilings.paged_read(reps=5, nt=nt)
        say(f"[gpu] non-temporal={nt}: stream read {r}; paged read {p}")
        for x in (r, p):
            assert 500.0 < x["GB/s"] < 1.05 * ceilings.HBM_PEAK_GBS


def test_issue_rate_of_exp_and_fma():
    r = ceilings.issue_rate(iters=1024, reps=2)
    say(f"[gpu] issue rate {r}")
    fma, ex = r["fma"]["cycles_per_instruction"], r["exp"]["cycles_per_instruction"]
    assert 1.0 <= fma <= ex
    assert r["fma"]["clock_mhz"] > 100.0


def test_library_gemm_below_the_dense_peak():
    g = ceilings.gemm(n=4096, reps=5)
    say(f"[gpu] bf16 GEMM {g}")
    assert 100.0 < g["TFLOP/s"] < 2600.0
