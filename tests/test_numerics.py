"""Host-side checks of numerical methods the HIP kernels use (no GPU)."""


def test_as7126_erf_error_bound():
    """The library's GELU uses Abramowitz & Stegun 7.1.26 for erf (|error| <= 1.5e-7);
    check the published bound of that formula against math.erf in float64."""
    from math import erf, exp
    p, a = 0.3275911, (0.254829592, -0.284496736, 1.421413741, -1.453152027, 1.061405429)
    worst = 0.0
    for i in range(20001):
        z = i * 6.0 / 20000
        t = 1.0 / (1.0 + p * z)
        approx = 1.0 - sum(c * t ** (k + 1) for k, c in enumerate(a)) * exp(-z * z)
        worst = max(worst, abs(approx - erf(z)))
    assert worst <= 1.5e-7
