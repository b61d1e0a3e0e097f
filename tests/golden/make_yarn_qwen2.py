"""Writes yarn_qwen2.txt: YaRN-scaled RoPE frequencies for Qwen2's
long-context setting, from the closed form in exact/decimal arithmetic.

This script does not import the oracle: the file it writes is a pin *of* the
oracle, so its values come from the closed form alone (Python's `decimal`
at 40 digits for the powers and logarithms, `fractions` for the ramp).

    python tests/golden/make_yarn_qwen2.py > tests/golden/yarn_qwen2.txt

The setting (the pages: Qwen2 trains at 32K and turns YaRN on at inference
to reach 128K, "Qwen-2 详解" (yudonglee.me) §6.2; the Qwen2
technical-report walkthrough (aicoding.csdn.net) §5.3 gives the scaled
frequency theta_i' = theta_i / s * alpha_i with a per-dimension ramp and a
logit rescale; theta = 1e6 from the same page §5.2): head size d = 128,
base 1e6, original window 32768, factor s = 4, beta_fast = 32,
beta_slow = 1.  The ramp is the reading the library takes from the YaRN
paper (Peng et al., 2023), blended linearly in the pair index.
"""

from decimal import Decimal, getcontext
from fractions import Fraction

getcontext().prec = 40

D_HEAD = 128
THETA = Decimal(10) ** 6
L_ORIG = Decimal(32768)
FACTOR = 4
BETA_FAST, BETA_SLOW = 32, 1
PI = Decimal("3.141592653589793238462643383279502884197")
PAIRS = [0] + list(range(20, 44)) + [63]


def corr_dim(n_turns):
    """Pair index whose frequency turns n_turns times over L_ORIG."""
    return Decimal(D_HEAD) * (L_ORIG / (2 * PI * Decimal(n_turns))).ln() / (2 * THETA.ln())


def main():
    d_fast, d_slow = corr_dim(BETA_FAST), corr_dim(BETA_SLOW)
    lo = int(d_fast.to_integral_value(rounding="ROUND_FLOOR"))
    hi = int(d_slow.to_integral_value(rounding="ROUND_CEILING"))
    mscale = Decimal("0.1") * Decimal(FACTOR).ln() + 1
    print("# YaRN-scaled RoPE frequencies, Qwen2 long-context setting.")
    print("# Sources: \"Qwen-2 详解\" (yudonglee.me) §6.2 (YaRN at inference, 32K -> 128K);")
    print("#   Qwen2 technical-report walkthrough (aicoding.csdn.net) §5.2 (theta = 1e6),")
    print("#   §5.3 (theta_i' = theta_i / s * alpha_i, logits rescaled).  Ramp: YaRN paper")
    print("#   (Peng et al., 2023), linear in the pair index between the correction dims.")
    print("# d = 128, theta = 1e6, L_orig = 32768, s = 4, beta_fast = 32, beta_slow = 1.")
    print("# Pair j turns n = L_orig * omega_j / (2 pi) times over the window,")
    print("#   omega_j = theta^(-2j/d) = 10^(-3j/32).  The pair index of n turns is")
    print("#   D(n) = d ln(L_orig / (2 pi n)) / (2 ln theta):")
    print(f"#   D(32) = {d_fast:.12f} -> floor {lo};  D(1) = {d_slow:.12f} -> ceil {hi}.")
    print(f"# r_j = clamp((j - {lo}) / ({hi} - {lo}), 0, 1);  omega'_j = omega_j (1 - r_j)"
          " + (omega_j / s) r_j.")
    print(f"# attention factor on cos and sin: 0.1 ln 4 + 1 = {mscale:.17f}")
    print("# Written by tests/golden/make_yarn_qwen2.py (decimal arithmetic, no oracle).")
    print("# columns: pair j, ramp r_j (exact), omega_j, omega'_j")
    print(f"lo {lo}")
    print(f"hi {hi}")
    print(f"mscale {mscale:.17e}")
    for j in PAIRS:
        w = Decimal(10) ** (Decimal(-3 * j) / Decimal(32))
        r = min(max(Fraction(j - lo, hi - lo), Fraction(0)), Fraction(1))
        rd = Decimal(r.numerator) / Decimal(r.denominator)
        wp = w * (1 - rd) + (w / FACTOR) * rd
        print(f"{j} {r} {w:.17e} {wp:.17e}")


if __name__ == "__main__":
    main()
