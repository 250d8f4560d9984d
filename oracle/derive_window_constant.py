"""Recompute the oracle's window constant C0 from the Gaussian model.

For X ~ N(0, sigma^2) the 7-binade window [2^a, 2^(a+7)) beats the window one
binade lower exactly while 2^(a-1) / sigma <= u*, where u* is the root of
    Phi(256 u) - Phi(128 u) = Phi(2 u) - Phi(u).
So the best window is the largest a with var >= C0 * 4^a, C0 = 1 / (4 u*^2).
Printed: u*, C0 to 40 digits, the nearest fp64 as a hex literal, and the
Gaussian escape probability at both ends of a window's sigma range.
"""
import mpmath as mp


def derive(dps: int = 50):
    mp.mp.dps = dps
    Phi = mp.ncdf
    h = lambda u: (Phi(256 * u) - Phi(128 * u)) - (Phi(2 * u) - Phi(u))
    u = mp.findroot(h, 0.019)
    C0 = 1 / (4 * u * u)
    return u, C0


def escape_probability(t):
    """P(|Z| outside [2^-t, 2^(7-t))) for standard normal Z."""
    lo = mp.mpf(2) ** (-t)
    return 1 - 2 * (mp.ncdf(128 * lo) - mp.ncdf(lo))


if __name__ == "__main__":
    u, C0 = derive()
    t = mp.log(C0, 2) / 2
    print("u* =", mp.nstr(u, 40))
    print("C0 =", mp.nstr(C0, 40), "=", float(C0).hex())
    print("escape probability: best case", mp.nstr(
        min(escape_probability(t + x / mp.mpf(200)) for x in range(201)), 6),
        "worst case", mp.nstr(escape_probability(t), 6))
