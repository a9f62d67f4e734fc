"""The GPU tests' comparators, checked on the CPU: an output element that is
NaN (never written into the NaN-filled buffer, or computed as NaN), a head
left unwritten, an infinite element or LSE, and bits that differ must all
fail; values within the stated bound must pass."""

import numpy as np
import pytest
import torch

from parity_utils import LSE_ATOL, TOL_BF16, compare, same_bits


def case(T=2, H=4, seed=0):
    g = np.random.default_rng(seed)
    ref = {"out": g.standard_normal((T, H, 512)) * 0.05,
           "lse": g.standard_normal((T, H)) * 3.0}
    out = torch.from_numpy(ref["out"]).to(torch.bfloat16)
    lse = torch.from_numpy(ref["lse"]).to(torch.float32)
    return out, lse, ref


def test_matching_outputs_pass():
    out, lse, ref = case()
    e, le = compare(out, lse, ref, TOL_BF16, what="match")
    assert e < 1e-3 and le < 1e-6


def test_one_nan_element_fails():
    out, lse, ref = case()
    out[1, 2, 300] = float("nan")
    with pytest.raises(AssertionError, match="not finite"):
        compare(out, lse, ref, TOL_BF16, what="nan element")


def test_unwritten_head_fails():
    """A head the kernel never wrote keeps the NaN fill of run_decode."""
    out, lse, ref = case()
    out[0, 3, :] = float("nan")
    with pytest.raises(AssertionError):
        compare(out, lse, ref, TOL_BF16, what="unwritten head")


def test_infinite_element_fails():
    out, lse, ref = case()
    out[0, 0, 0] = float("inf")
    with pytest.raises(AssertionError):
        compare(out, lse, ref, TOL_BF16, what="inf element")


def test_out_of_tolerance_element_fails():
    out, lse, ref = case()
    out[1, 0, 7] = float(ref["out"][1, 0, 7]) + 0.05
    with pytest.raises(AssertionError, match="out of tolerance"):
        compare(out, lse, ref, TOL_BF16, what="off element")


@pytest.mark.parametrize("bad", [float("nan"), float("inf"), 2 * LSE_ATOL])
def test_bad_lse_fails(bad):
    out, lse, ref = case()
    lse[1, 1] = bad if bad != 2 * LSE_ATOL else float(ref["lse"][1, 1]) + bad
    with pytest.raises(AssertionError):
        compare(out, lse, ref, TOL_BF16, what="bad lse")


def test_neg_inf_lse_must_match_the_oracle():
    out, lse, ref = case()
    ref["lse"][0, 0] = -np.inf
    with pytest.raises(AssertionError, match="-inf"):
        compare(out, lse, ref, TOL_BF16, what="missing -inf")
    lse[0, 0] = -float("inf")
    compare(out, lse, ref, TOL_BF16, what="both -inf")


def test_same_bits_rejects_nan_and_differences():
    a = torch.randn(3, 8).to(torch.bfloat16)
    same_bits(a, a.clone())
    b = a.clone()
    b[1, 1] = float("nan")
    with pytest.raises(AssertionError, match="NaN"):
        same_bits(b, b.clone())            # both unwritten: still a failure
    c = a.clone()
    c[2, 3] = c[2, 3] * 2 + 1
    with pytest.raises(AssertionError, match="bits differ"):
        same_bits(a, c)
    l = torch.tensor([-float("inf"), 1.5])
    same_bits(l, l.clone())                 # -inf (an empty token) is a value
