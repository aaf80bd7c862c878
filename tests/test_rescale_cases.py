"""The ramped-score prefill cases reach the kernel's rescale of the reference
maximum on both code paths, and with bf16 and with fp16 P both outcomes of
the max-free pass (kept with weights far above the reference, or rerun with
the exact steps, which rescale), by host emulation of the kernel's tile maxima and row sums (no GPU).
The GPU parity test of the same cases is ``test_prefill_rescale_branch`` in
test_parity_gpu.py."""
import numpy as np
import pytest

from tests.rescale_emu import rescale_events
from workloads import prefill_inputs, prefill_ramp_inputs

# B, N, M, Hq, Hkv, d, dtype, causal[, ramp slope (default 6)]: causal with
# N == M and N < M, non-causal, fp16 and bf16, head dims 64 and 128, GQA and
# MHA; fp16 workgroups outgrow their max-free pass (weights past 2^15) within
# a few tiles, the last bf16 cases are long enough to outgrow it too (row sums
# past 2^100), and the steep one jumps by more than 126 log2 units in one tile
RESCALE_CASES = [
    (1, 1024, 1024, 4, 2, 128, "bf16", True),
    (1, 1024, 1024, 4, 4, 64, "f16", True),
    (1, 300, 1000, 4, 1, 128, "f16", True),
    (1, 200, 700, 4, 2, 64, "bf16", True),
    (1, 256, 1000, 2, 2, 64, "bf16", False),
    (2, 512, 512, 8, 2, 128, "f16", False),
    (1, 2048, 2048, 2, 2, 64, "bf16", True),
    (1, 512, 2048, 2, 2, 64, "bf16", False),
    (1, 1024, 4096, 4, 2, 128, "bf16", False),
    (1, 512, 512, 2, 2, 64, "bf16", True, 176.0),
    # head dim 256
    (1, 256, 1000, 2, 2, 256, "bf16", False),
    (1, 256, 700, 4, 2, 256, "f16", True),
    (1, 512, 4096, 2, 1, 256, "bf16", False),
]
RESCALE_SEED = 11


def rescale_case_inputs(case):
    B, N, M, Hq, Hkv, d, dt, causal = case[:8]
    slope = case[8] if len(case) > 8 else 6.0
    q, k, v = prefill_ramp_inputs(B, Hq, Hkv, N, M, d, dt, seed=RESCALE_SEED, slope=slope)
    return q, k, v, float(np.float32(d ** -0.5))


def case_events(case):
    q, k, v, scale = rescale_case_inputs(case)
    return rescale_events(q, k, scale, case[7], max_free=True, p_dtype=case[6])


def check_case_events(case, ev):
    """What a ramped case must reach: growth that the max-free first pass
    keeps, or a rerun whose exact steps rescale; no workgroup too close to
    call."""
    assert ev["uncertain"] == 0, ev
    assert ev["free_growth"] > 0 or (ev["restart"] > 0 and ev["fast"] > 0), ev


@pytest.mark.parametrize("case", RESCALE_CASES, ids=lambda c: "x".join(map(str, c)))
def test_ramp_inputs_rescale_on_both_paths(case):
    check_case_events(case, case_events(case))
    # |O| stays below 2, where the bf16 output's half-ulp is below the bound
    _, _, v, _ = rescale_case_inputs(case)
    assert float(v.abs().max()) < 1.5


def test_general_path_rescales_with_both_dtypes():
    """The masked (general) steps move the reference in the exact passes: the
    reruns of both dtypes reach that rescale, not only the steady-state one."""
    for dt in ("bf16", "f16"):
        evs = [case_events(c) for c in RESCALE_CASES if c[6] == dt]
        assert any(ev["general"] > 0 and ev["restart"] > 0 for ev in evs), (dt, evs)


def test_f16_cases_reach_both_outcomes_of_the_max_free_pass():
    """Some fp16 workgroups keep a max-free pass whose steady tiles exceeded
    the reference by more than 8 (weights up to 2^15, within fp16's range),
    and some rerun the pass with the exact steps, which then rescale on the
    steady-state path."""
    evs = [case_events(c) for c in RESCALE_CASES if c[6] == "f16"]
    assert any(ev["free_growth"] > 0 and ev["restart"] > 0 for ev in evs), evs
    assert any(ev["restart"] > 0 and ev["fast"] > 0 for ev in evs), evs


def test_bf16_cases_reach_both_outcomes_of_the_max_free_pass():
    """Some bf16 workgroups keep a max-free pass whose steady tiles exceeded
    the reference by far more than 8 (up to about 2^100 in the row sums), and
    some rerun the pass with the exact steps, which then rescale on the
    steady-state path."""
    evs = [case_events(c) for c in RESCALE_CASES if c[6] == "bf16"]
    assert any(ev["free_growth"] > 0 and ev["max_jump"] > 60 for ev in evs), evs
    assert any(ev["restart"] > 0 and ev["fast"] > 0 for ev in evs), evs
    assert any(ev["free_growth"] > 0 and ev["restart"] > 0 for ev in evs), evs
    # a rerun whose reference moves by more than 126 log2 units in one tile:
    # alpha flushes to zero and the earlier (negligible) weights drop out
    assert any(ev["max_lag"] > 126.5 and ev["restart"] > 0 for ev in evs), evs


def test_plain_inputs_never_rescale():
    """The i.i.d. N(0, 1) inputs of the other parity cases never move the
    reference max (which is why the ramped cases exist)."""
    q, k, _ = prefill_inputs(2, 8, 2, 1024, 1024, 128, "bf16", 0)
    for free in (False, True):
        ev = rescale_events(q, k, float(np.float32(128 ** -0.5)), True, max_free=free)
        assert ev["fast"] == 0 and ev["general"] == 0 and ev["max_jump"] < 8.0, ev
        assert ev["restart"] == 0 and ev["free_growth"] == 0 and ev["uncertain"] == 0, ev
