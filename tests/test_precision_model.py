"""CPU model of the encode's projection arithmetic (no GPU).

The encode multiplies on bf16 MFMA units with fp32 accumulation. The mean is
subtracted before the transform (page "KV Cache Transform Coding for Compact
Storage in LLM Inference", section 2B), and how that subtraction is arranged
decides whether the rounding error scales with the centred token |x - mu| or
with |x|. The kernel centres each token on mu_hi = bf16(mu32) in fp32, splits
d = x - mu_hi into bf16 terms (two for bf16 input, three for f32) and starts
its accumulators at -(mu32 - mu_hi) V'. These tests check the facts that
argument rests on, and model the code mismatch rate of that arithmetic
against the oracle's exact projection, next to the rejected alternative of
folding the mean into the product (x V' - mu V').
"""
import numpy as np

import oracle.kvtc_oracle as O


def _f32(x):
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def _bf16(x):
    return O.bf16_rne(np.asarray(x, np.float32)).astype(np.float64)


def _split(d, n):
    """d (fp32 values) -> n bf16 terms, each the rounding of what is left."""
    terms, rem = [], np.asarray(d, np.float64)
    for _ in range(n):
        t = _bf16(rem)
        terms.append(t)
        rem = rem - t            # exact in fp32 (|rem| <= half an ulp of t)
    return terms, rem


def test_two_terms_hold_a_bf16_difference_exactly():
    """x, mu_hi bf16 within a factor 2^8 of each other: x - mu_hi is exact in
    fp32 and equals the sum of its two-term bf16 split."""
    rng = np.random.default_rng(1)
    e = rng.integers(-20, 20, 200000)
    x = _bf16(rng.uniform(1, 2, e.size) * 2.0 ** e * rng.choice([-1, 1], e.size))
    m = _bf16(x * rng.uniform(2.0 ** -7.9, 2.0 ** 7.9, e.size) * rng.choice([-1, 1], e.size))
    d = _f32(x - m)
    assert np.array_equal(d, x - m)                  # no rounding in fp32
    (t1, t2), rem = _split(d, 2)
    assert np.array_equal(t1 + t2, d) and not np.any(rem)


def test_three_terms_hold_any_fp32_value_exactly():
    rng = np.random.default_rng(2)
    d = _f32(rng.standard_normal(200000) * 2.0 ** rng.integers(-30, 30, 200000))
    (t1, t2, t3), rem = _split(d, 3)
    assert np.array_equal(t1 + t2 + t3, d) and not np.any(rem)


def _mismatch_rate(mu_ratio, scheme, seed=3, F=512, T=1500):
    """Code mismatches of a model of the kernel's arithmetic (each 16-feature
    MFMA chunk summed exactly and added to the fp32 accumulator with one
    rounding) against the oracle's exact projection, widths 8/8/7/7/6/4."""
    rng = np.random.default_rng(seed)
    G, widths = 16, [8, 8, 7, 7, 6, 4]
    r = G * len(widths)
    V = np.linalg.qr(rng.standard_normal((F, F)))[0][:, :r]
    Vb = _bf16(V)
    mu = _f32(mu_ratio * rng.standard_normal(F))
    z = rng.standard_normal((T, r)) * np.arange(1, r + 1) ** -1.2 * 10
    x = _bf16(z @ V.T + mu + 0.05 * rng.standard_normal((T, F)))
    exact = _f32((x - mu) @ Vb)
    if scheme == "folded":                          # x V' - mu V'
        acc, terms = np.tile(-_f32(mu @ Vb), (T, 1)), [x]
    else:                                           # centred on mu_hi, two terms
        mhi = _bf16(mu)
        acc = np.tile(-_f32((mu - mhi) @ Vb), (T, 1))
        terms, _ = _split(_f32(x - mhi), 2)
    for k in range(0, F, 16):
        for t in terms:
            acc = _f32(acc + t[:, k:k + 16] @ Vb[k:k + 16])
    bad = tot = 0
    for a, b in enumerate(widths):
        sl = slice(a * G, (a + 1) * G)
        bad += np.count_nonzero(O.quantize_fp32(exact[:, sl], b)[0] != O.quantize_fp32(acc[:, sl], b)[0])
        tot += T * G
    return bad / tot


def test_centred_split_keeps_codes_within_the_bar_at_any_mean():
    for ratio in (0.5, 10.0, 100.0):
        assert _mismatch_rate(ratio, "centred") <= 1e-4, ratio


def test_folding_the_mean_into_the_product_does_not():
    # the alternative the kernel does not use: the error grows with |x|
    assert _mismatch_rate(100.0, "folded") > 1e-4
