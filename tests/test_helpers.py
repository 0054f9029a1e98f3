"""CPU checks of the parity metrics themselves: a metric that cannot see a
mistake would let a wrong kernel pass."""
import numpy as np
import pytest

import oracle
from helpers import as_real_pairs, assert_spectrum_parity, max_abs, rel_l2, sum_bar


def _spectrum_ref(N=64, L=64, seed=0):
    z = np.random.default_rng(seed).standard_normal((2, 3, N)) * 2
    zs = oracle.softmax(z)
    line = np.zeros((2, 3, L))
    line[..., :N] = zs
    return np.fft.fft(line, axis=-1) / L


def test_metrics_refuse_complex():
    a = np.ones(4, dtype=np.complex64)
    with pytest.raises(TypeError):
        rel_l2(a, a)
    with pytest.raises(TypeError):
        max_abs(a, a)


def test_spectrum_check_sees_imaginary_parts():
    ref = _spectrum_ref()
    assert_spectrum_parity(ref.astype(np.complex64), ref, "exact")
    # a spectrum with every imaginary part negated (the conjugate: the
    # reversed filter) must fail, as must one with the parts swapped
    with pytest.raises(AssertionError):
        assert_spectrum_parity(np.conj(ref).astype(np.complex64), ref, "conjugated")
    with pytest.raises(AssertionError):
        assert_spectrum_parity((ref.imag + 1j * ref.real).astype(np.complex64), ref, "swapped")
    # the real parts alone agree, which a real-only metric would accept
    assert rel_l2(np.conj(ref).real, ref.real) == 0.0
    assert rel_l2(as_real_pairs(np.conj(ref)), as_real_pairs(ref)) > 0.1


def test_sum_bar_matches_fp32_accumulation():
    """The derived weight-gradient bar covers a plain fp32 sequential sum of
    K random products (the worst order: one running accumulator), and is not
    so loose that a one-ulp-per-term systematic bias of the inputs passes."""
    rng = np.random.default_rng(5)
    K, C = 8000, 64
    a = rng.standard_normal((K, C)).astype(np.float32)
    b = (rng.standard_normal((K, C)) * 0.05).astype(np.float32)
    exact = np.sum(a.astype(np.float64) * b.astype(np.float64), axis=0)
    acc = np.zeros(C, dtype=np.float32)
    for t in range(K):
        acc = (acc + a[t] * b[t]).astype(np.float32)
    err = np.max(np.abs(acc - exact))
    bar = sum_bar(K, float(np.sqrt(np.mean(a.astype(np.float64) ** 2))),
                  float(np.sqrt(np.mean(b.astype(np.float64) ** 2))), eps_in=0.0)
    assert err <= bar, (err, bar)
    # a systematic relative error of 1e-3 in b (say, a dropped rounding
    # correction) is caught by the bar with the input term included
    biased = np.sum(a.astype(np.float64) * (b.astype(np.float64) * (1 + 1e-3)), axis=0)
    assert np.max(np.abs(biased - exact)) > sum_bar(K, 1.0, 0.05)
