"""CPU checks of the GPU tests' parity helpers: the threaded oracle driver
returns what single oracle calls return, and the bf16-out bound is the plain
2e-2 except on elements with |ref| >= 4."""
import numpy as np
import pytest

import oracle
from gpu_common import assert_bf16_out_close, oracle_decode_parallel, oracle_rows_parallel


def _inputs(L=300, Hq=4, Hkv=2, D=16, seed=3):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((1, L, Hq, D)), rng.standard_normal((1, L, Hkv, D)),
            rng.standard_normal((1, L, Hkv, D)))


def test_parallel_rows_equal_one_call():
    q, k, v = _inputs()
    rows = np.array([0, 1, 5, 63, 64, 65, 100, 150, 151, 299])
    ref, ref_lse = oracle.bifocal_attention(q, k, v, 20, 64, 1e4, 0.25, rows=rows)
    got, got_lse = oracle_rows_parallel(q, k, v, rows, 20, 64, 1e4, 0.25, workers=3)
    assert got.shape == ref.shape and got_lse.shape == ref_lse.shape
    assert np.max(np.abs(got - ref)) <= 1e-12 and np.max(np.abs(got_lse - ref_lse)) <= 1e-12


def test_parallel_decode_equal_one_call():
    q, k, v = _inputs(L=200)
    steps = [(q[:, L - 1], L) for L in (1, 50, 129, 200)]
    got = oracle_decode_parallel(steps, k, v, 10, 64, 1e4, 0.25, workers=2)
    for (qt, L), (o, ls) in zip(steps, got):
        ro, rl = oracle.decode_attention(qt, k, v, L, 10, 64, 1e4, 0.25)
        assert np.max(np.abs(o - ro)) <= 1e-12 and np.max(np.abs(ls - rl)) <= 1e-12


def test_bf16_bound_is_plain_below_four():
    ref = np.array([1.0, -3.9, 0.0])
    assert_bf16_out_close(ref + 0.0199, ref)
    with pytest.raises(AssertionError):
        assert_bf16_out_close(ref + np.array([0.0, 0.021, 0.0]), ref)


def test_bf16_bound_widens_by_half_ulp_from_four():
    ref = np.array([5.0, 1.0])
    # 2e-2 + 2^-8 * 5 = 0.0395 allowed at 5.0
    assert_bf16_out_close(ref + np.array([0.039, 0.0]), ref)
    with pytest.raises(AssertionError):
        assert_bf16_out_close(ref + np.array([0.041, 0.0]), ref)
