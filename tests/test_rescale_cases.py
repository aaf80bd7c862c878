"""The ramped-score prefill cases reach the kernel's rescale of the reference
maximum on both code paths (host emulation of the kernel's tile maxima; no
GPU).  The GPU parity test of the same cases is ``test_prefill_rescale_branch``
in test_parity_gpu.py."""
import numpy as np
import pytest

from tests.rescale_emu import rescale_events
from workloads import prefill_inputs, prefill_ramp_inputs

# B, N, M, Hq, Hkv, d, dtype, causal: causal with N == M and N < M, non-causal,
# fp16 and bf16, head dims 64 and 128, GQA and MHA
RESCALE_CASES = [
    (1, 1024, 1024, 4, 2, 128, "bf16", True),
    (1, 1024, 1024, 4, 4, 64, "f16", True),
    (1, 300, 1000, 4, 1, 128, "f16", True),
    (1, 200, 700, 4, 2, 64, "bf16", True),
    (1, 256, 1000, 2, 2, 64, "bf16", False),
    (2, 512, 512, 8, 2, 128, "f16", False),
]
RESCALE_SEED = 11


def rescale_case_inputs(case):
    B, N, M, Hq, Hkv, d, dt, causal = case
    q, k, v = prefill_ramp_inputs(B, Hq, Hkv, N, M, d, dt, seed=RESCALE_SEED)
    return q, k, v, float(np.float32(d ** -0.5))


@pytest.mark.parametrize("case", RESCALE_CASES, ids=lambda c: "x".join(map(str, c)))
def test_ramp_inputs_rescale_on_both_paths(case):
    q, k, v, scale = rescale_case_inputs(case)
    ev = rescale_events(q, k, scale, case[-1])
    assert ev["fast"] > 0 and ev["general"] > 0, ev
    # |O| stays below 2, where the bf16 output's half-ulp is below the bound
    assert float(v.abs().max()) < 1.5


def test_plain_inputs_never_rescale():
    """The i.i.d. N(0, 1) inputs of the other parity cases never move the
    reference max (which is why the ramped cases exist)."""
    q, k, _ = prefill_inputs(2, 8, 2, 1024, 1024, 128, "bf16", 0)
    ev = rescale_events(q, k, float(np.float32(128 ** -0.5)), True)
    assert ev["fast"] == 0 and ev["general"] == 0 and ev["max_jump"] < 8.0, ev
