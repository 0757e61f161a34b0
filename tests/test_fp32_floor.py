"""The FP32 precision floor of narrow keys, measured: the multi-query backward with a 3-column key
(R = 3) over D = 1024 columns. Its slice gradient's terms are dp_{m,s} = <dY_m, v_s> sums over all
D columns (magnitude ~ sqrt(D)) that cancel in dp - delta, so any FP32 evaluation carries an error
~ eps32 * sqrt(D) * |dp| into the three slice columns; relative to the rms of dvalues that exceeds
the literal 1e-5 bound. A plain FP32 evaluation (sequential float32 sums, tests/fp32_floor.py)
shows it against the FP64 oracle; the GPU parity case of the same inputs is held to a small
multiple of this measured floor. Shrinking D lowers the floor below 1e-5 (D = 64)."""
import numpy as np
import pytest

import attnres_workloads as W
import oracle
from fp32_floor import fp32_floor
from parity import TOL_F32

# the inputs of the GPU case in tests/test_gpu_multi.py (seed = 2000 + S * M + D)
CASE = dict(S=3, N=97, D=1024, R=3, M=3)


def _floor(D):
    S, N, R, M = CASE["S"], CASE["N"], CASE["R"], CASE["M"]
    V, Q, G = W.multi_case(S, N, D, R, M, "f32", seed=2000 + S * M + D)
    ref = oracle.run_multi(V, Q, G)["dvalues"]
    return fp32_floor(V.numpy(), Q.numpy(), G.numpy(), ref)


def test_fp32_evaluation_of_a_narrow_key_exceeds_the_literal_bound():
    floor = _floor(CASE["D"])
    print(f"FP32 floor at D={CASE['D']}, R=3: {floor:.3g} x rms")
    assert floor > TOL_F32            # the literal bound is below what FP32 can reach here
    assert floor < 10 * TOL_F32       # and the floor is eps32-sized, not a formula error


def test_fp32_floor_falls_with_the_row_width():
    assert _floor(64) < TOL_F32 < _floor(CASE["D"])


@pytest.mark.parametrize("D", [64, 256])
def test_fp32_evaluation_matches_the_oracle_on_wide_keys(D):
    # with R = D there is no cancelling narrow slice: plain FP32 meets the literal bound, so the
    # floor above is the narrow key's, not a defect of this evaluation
    S, N, M = 4, 33, 3
    V, Q, G = W.multi_case(S, N, D, D, M, "f32", seed=77 + D)
    ref = oracle.run_multi(V, Q, G)["dvalues"]
    assert fp32_floor(V.numpy(), Q.numpy(), G.numpy(), ref) <= TOL_F32
