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


def test_as7127_erf_error_bound():
    """For binary16 outputs the GELU takes erf from Abramowitz & Stegun 7.1.27
    (|error| <= 5e-4, one reciprocal, no exponential); check the published
    bound against math.erf in float64, and what it means for GELU(x): at most
    5e-4 |x| / 2, below 3e-3 of max |GELU| over any range |x| <= L (L >= 1)."""
    from math import erf, sqrt
    a = (0.278393, 0.230389, 0.000972, 0.078108)
    worst = worst_gelu = 0.0
    for i in range(40001):
        z = i * 8.0 / 40000
        approx = 1.0 - 1.0 / (1.0 + sum(c * z ** (k + 1) for k, c in enumerate(a))) ** 4
        worst = max(worst, abs(approx - erf(z)))
        x = z * sqrt(2.0)
        worst_gelu = max(worst_gelu, 0.5 * x * abs(approx - erf(z)) / max(1.0, x))
    assert worst <= 5e-4
    assert worst_gelu <= 2.5e-4
