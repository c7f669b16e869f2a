"""CPU model of the two-term e4m3 split that feeds a bf16 indexer query to the
fp8 matrix cores: with one exponent s per query (max|q| * 2^s in [128, 256)),
X = q * 2^s is split as hi = e4m3(X) and lo = e4m3(16 (X - hi)), and the MFMAs
see hi + lo / 16. The model uses torch's e4m3fn cast (round to nearest even),
the rounding of the gfx950 conversion for in-range values, and checks the bound
the kernel states, over every finite bf16 value below the maximum:

* exact wherever |X| >= 2^-6 (e4m3's smallest normal), which includes every
  element with |q| >= 2^-13 max|q|;
* elsewhere |X - (hi + lo/16)| <= 2^-14, i.e. an error of at most
  2^-14 2^-s <= 2^-21 max|q| in q.

A plausible mistake (residual not scaled by 16, a wrong exponent choice, a
claim of exactness down to 2^-21 max|q|) fails one of the assertions."""
import math

import numpy as np
import pytest
import torch


def _bf16_all_finite():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    x = bits.view(torch.bfloat16).float()
    return x[torch.isfinite(x)]


def _split(X):
    hi = X.to(torch.float8_e4m3fn).float()
    r = (X - hi) * 16.0
    lo = r.to(torch.float8_e4m3fn).float()
    return hi, lo


def _exponent(amax):
    # s with amax * 2^s in [128, 256)
    _, e = math.frexp(amax)
    return 8 - e


@pytest.mark.parametrize("amax", [1.0, 1.5, 3.99, 4.0, 0.0123, 300.0])
def test_split_bound_over_all_bf16_values(amax):
    amax = float(torch.tensor(amax).to(torch.bfloat16).float())
    s = _exponent(amax)
    x = _bf16_all_finite().double()
    x = x[x.abs() <= amax]
    X = x * 2.0 ** s
    assert float(X.abs().max()) < 256.0
    hi, lo = _split(X.float())
    rep = hi.double() + lo.double() / 16.0
    err = (rep - X).abs()
    normal = X.abs() >= 2.0 ** -6
    assert torch.all(err[normal] == 0), "the split must be exact at or above e4m3's smallest normal"
    assert float(err.max()) <= 2.0 ** -14
    # in units of the query: at most 2^-21 of its largest magnitude
    assert float((err / 2.0 ** s).max()) <= 2.0 ** -21 * amax
    # every element with |q| >= 2^-13 max|q| is exact, whatever the octave of amax
    assert torch.all(err[x.abs() >= 2.0 ** -13 * amax] == 0)
    # and the bound is tight: some element below the normal range is inexact
    assert float(err.max()) > 0.0


def test_exactness_does_not_reach_2_to_minus_21():
    """Elements between 2^-21 and 2^-14 of the maximum are not all exact (the
    residual underflows into e4m3's subnormal steps of 2^-9)."""
    amax = 2.0
    s = _exponent(amax)
    x = _bf16_all_finite().double()
    x = x[(x.abs() >= 2.0 ** -21 * amax) & (x.abs() < 2.0 ** -14 * amax)]
    X = (x * 2.0 ** s).float()
    hi, lo = _split(X)
    err = (hi.double() + lo.double() / 16.0 - X.double()).abs()
    assert float(err.max()) > 0.0


def test_dropping_the_residual_breaks_the_bound():
    """hi alone (a one-term e4m3 query) is off by up to 2^-5 relative: well
    outside the stated bound, so the residual term matters."""
    x = _bf16_all_finite().double()
    x = x[(x.abs() <= 1.0) & (x.abs() >= 0.5)]
    X = (x * 2.0 ** _exponent(1.0)).float()
    hi, _ = _split(X)
    rel = ((hi.double() - X.double()).abs() / X.double().abs()).max()
    assert float(rel) > 2.0 ** -6
