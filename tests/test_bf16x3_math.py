"""The arithmetic the bf16 matrix-pipe kernels rest on, checked on the host in numpy (no GPU):

* an f32 value x taken as three bf16 terms, hi = bf16(x), mid = bf16(x - hi),
  lo = bf16(x - hi - mid), rounding to nearest even: both subtractions are exact in f32, each
  remainder is at most 2^-8 of the value it is taken from, and hi + mid + lo == x exactly;
* a product a*b formed from the six leading term products (ah bh, ah bm, am bh, ah bl, al bh,
  am bm), each exact in f32: within 2^-23 |a||b| (the dropped am bl + al bm), and typically far
  closer; summed over a dot product, closer to the exact value than f32-rounded products;
* truncation instead of rounding gives exact three-term sums too, but its remainders are up to
  2^-7, so the six-product form misses by up to about 2^-21, which is why the kernels round.

The bf16 rounding here is written from the IEEE definition (round the f32 bit pattern to its
upper 16 bits, ties to even); it shares nothing with the kernels."""
import numpy as np
import pytest


def bf16_rne(x):
    """f32 array -> f32 array of the nearest bf16 values (ties to even); finite inputs."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def bf16_trunc(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    return (u & np.uint32(0xFFFF0000)).view(np.float32)


def split3(x, rnd=bf16_rne):
    x = np.asarray(x, dtype=np.float32)
    hi = rnd(x)
    r = (x - hi).astype(np.float32)
    mid = rnd(r)
    t = (r - mid).astype(np.float32)
    lo = rnd(t)
    return hi, mid, lo, r, t


def samples(n=200000, seed=0):
    rng = np.random.default_rng(seed)
    # significands across the f32 range of interest, exponents from 2^-40 to 2^40, both signs
    mant = rng.uniform(1.0, 2.0, n)
    expo = rng.integers(-40, 41, n)
    x = (np.sign(rng.standard_normal(n)) * mant * np.exp2(expo)).astype(np.float32)
    # plus values at and next to bf16 rounding ties and powers of two
    u = rng.integers(0, 1 << 16, 4096, dtype=np.uint64) << 16
    with np.errstate(invalid="ignore"):
        ties = (u | 0x8000).astype(np.uint32).view(np.float32) * np.float32(1.0)
    ties = ties[np.isfinite(ties) & (np.abs(ties) >= 2.0 ** -40) & (np.abs(ties) <= 2.0 ** 40)]
    near = np.nextafter(ties, np.float32(np.inf)).astype(np.float32)
    return np.concatenate([x, ties.astype(np.float32), near])


def test_bf16_rounding_matches_a_direct_definition():
    # nearest of the two bf16 neighbours, ties to the even one
    x = samples(20000, seed=1)
    lo = bf16_trunc(x).astype(np.float64)
    step = np.exp2(np.floor(np.log2(np.abs(lo))) - 7)          # bf16 spacing at |lo|
    hi = lo + np.sign(lo) * step
    got = bf16_rne(x).astype(np.float64)
    d_lo, d_hi = np.abs(x - lo), np.abs(x - hi)
    want = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    even_lo = ((bf16_trunc(x).view(np.uint32) >> 16) & 1) == 0
    want = np.where(tie, np.where(even_lo, lo, hi), want)
    assert np.array_equal(got, want)


def test_three_term_split_is_exact():
    x = samples()
    hi, mid, lo, r, t = split3(x)
    xd = x.astype(np.float64)
    # the two f32 subtractions are exact
    assert np.array_equal(r.astype(np.float64), xd - hi.astype(np.float64))
    assert np.array_equal(t.astype(np.float64), r.astype(np.float64) - mid.astype(np.float64))
    # each remainder is at most half a bf16 step: 2^-8 of the value it is taken from
    assert np.all(np.abs(r.astype(np.float64)) <= np.abs(xd) * 2.0 ** -8)
    assert np.all(np.abs(t.astype(np.float64)) <= np.abs(r.astype(np.float64)) * 2.0 ** -8)
    # x - hi keeps at most 16 significant bits and x - hi - mid at most 8: lo is exact
    assert np.array_equal(lo, t)
    assert np.array_equal(hi.astype(np.float64) + mid.astype(np.float64) + lo.astype(np.float64), xd)
    # the terms are bf16 values
    for term in (hi, mid, lo):
        assert np.all((term.view(np.uint32) & 0xFFFF) == 0)


def six_products(a, b, rnd=bf16_rne):
    ah, am, al = split3(a, rnd)[:3]
    bh, bm, bl = split3(b, rnd)[:3]
    terms = [(ah, bh), (ah, bm), (am, bh), (ah, bl), (al, bh), (am, bm)]
    # every term product is exact in f32: two 8-bit significands
    for p, q in terms:
        prod32 = (p * q).astype(np.float64)
        assert np.array_equal(prod32, p.astype(np.float64) * q.astype(np.float64))
    return sum(p.astype(np.float64) * q.astype(np.float64) for p, q in terms)


def test_six_product_form_against_the_product():
    rng = np.random.default_rng(2)
    a = samples(100000, seed=3)
    b = samples(100000, seed=4)
    n = min(len(a), len(b))
    a, b = a[:n], b[rng.permutation(len(b))][:n]
    exact = a.astype(np.float64) * b.astype(np.float64)
    rel = np.abs(six_products(a, b) - exact) / np.abs(exact)
    # the dropped terms: |am bl| + |al bm| <= 2 * 2^-8 * 2^-16 (plus al bl, 2^-32)
    assert rel.max() <= 2.0 ** -23
    assert np.median(rel) <= 2.0 ** -27
    # f32's own rounding of a product: up to 2^-24, median about 2^-25.5
    f32_rel = np.abs((a * b).astype(np.float64) - exact) / np.abs(exact)
    assert np.median(rel) < np.median(f32_rel) / 8


def test_truncation_would_not_meet_the_bound():
    # exact as a three-term sum, but its remainders are 2 bits larger, so the six-product form
    # drops terms up to about 2^-21 relative
    a = samples(100000, seed=5)
    b = samples(100000, seed=6)
    hi, mid, lo, _, _ = split3(a, bf16_trunc)
    assert np.array_equal(hi.astype(np.float64) + mid.astype(np.float64) + lo.astype(np.float64),
                          a.astype(np.float64))
    n = min(len(a), len(b))
    a, b = a[:n], b[:n]
    exact = a.astype(np.float64) * b.astype(np.float64)
    rel = np.abs(six_products(a, b, bf16_trunc) - exact) / np.abs(exact)
    assert rel.max() > 2.0 ** -22


@pytest.mark.parametrize("hd", [64, 128])
def test_dot_products_stay_within_f32_rounding_scale(hd):
    # a score q.k summed over hd six-product terms is as close to the f64 dot as the f32 dot
    rng = np.random.default_rng(hd)
    q = rng.standard_normal((4096, hd)).astype(np.float32)
    k = rng.standard_normal((4096, hd)).astype(np.float32)
    exact = np.sum(q.astype(np.float64) * k.astype(np.float64), axis=1)
    six = np.sum(six_products(q.ravel(), k.ravel()).reshape(4096, hd), axis=1)
    f32 = np.sum((q * k).astype(np.float64), axis=1)          # f32-rounded products, exact sum
    scale = np.sum(np.abs(q.astype(np.float64) * k.astype(np.float64)), axis=1)
    six_err = np.max(np.abs(six - exact) / scale)
    assert six_err <= 2.0 ** -26
    assert six_err < np.max(np.abs(f32 - exact) / scale)
