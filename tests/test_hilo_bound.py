"""The certificate of the fp16 hi/lo nearest-centroid scores, on the CPU.

The GPU search scores a centroid c against a sub-vector x as
    s^ = fl32( C + sum_j c_j hi_j + sum_j c_j lo_j ),  C = ||c||^2 (1 +- 2^-15) 2^s
with X = fl32(-2x) 2^s, hi = fl16(X), lo = fl16(X - hi), and keeps every
centroid whose s^ - E is within the best s^ + E, E = 2^-15 (||x||^2 + ||c||^2)
(in units of 2^s).  Here the scores are emulated with the matrix cores'
accumulation modelled pessimistically: every one of the additions is
rounded to fp32 and then pushed a further ulp (2u in all) in the direction
that hurts most.  The emulated error must stay within E, and the true
nearest centroid must survive the candidate test, for rows far below the
scale's maximum (workgroup scale) as well as for each row's own scale."""
import numpy as np
import pytest

U = 2.0 ** -24


def f32(x):
    return np.float64(np.float32(x))


def push(v, direction):
    """fl32(v), then one more ulp in `direction` (+1 / -1)."""
    r = np.float32(v)
    return np.float64(np.nextafter(r, np.float32(np.inf if direction > 0 else -np.inf)))


def split(x, sc):
    X = np.array([f32(f32(-2.0 * xi) * sc) for xi in x])
    hi = X.astype(np.float16).astype(np.float64)
    lo = (X - hi).astype(np.float16).astype(np.float64)
    return hi, lo


def scale_for(mx):
    if mx == 0:
        return 1.0
    e = np.frexp(np.float32(mx))[1]
    return 2.0 ** min(max(15 - int(e), -60), 60)


def emulated(c, x, sc, direction, bound_sign, l1_term):
    """Worst-case modelled s^ (units of 2^s) with the norm term of sign
    bound_sign; l1_term: the workgroup-scale tables' 2^-24 ||c||_1."""
    hi, lo = split(x, sc)
    n = f32(np.sum(c.astype(np.float64) ** 2))
    l1 = float(np.sum(np.abs(c))) if l1_term else 0.0
    term = f32(n * (1 + bound_sign * 2.0 ** -15) * sc + bound_sign * 2.0 ** -24 * l1)
    acc = term
    for p in list(c * hi) + list(c * lo):      # products exact in fp64 (and fp32)
        acc = push(acc + p, direction)
    return acc


def check_rows(cents, xs, sc_fn, l1_term):
    for x in xs:
        mxs = sc_fn(x)
        xx = f32(np.sum(x.astype(np.float64) ** 2))
        exact = np.array([np.sum((c.astype(np.float64)) ** 2) - 2 * np.dot(x, c.astype(np.float64))
                          for c in cents])
        lo_s = np.array([emulated(c, x, mxs, -1, -1, l1_term) for c in cents]) / mxs
        hi_s = np.array([emulated(c, x, mxs, +1, +1, l1_term) for c in cents]) / mxs
        n2 = np.sum(cents.astype(np.float64) ** 2, axis=1)
        E = 2.0 ** -15 * (xx + n2) + 1e-30
        if l1_term:
            E = E + 2.0 ** -24 * np.sum(np.abs(cents.astype(np.float64)), axis=1) / mxs
        # the modelled scores, with their norm-term margins, bracket the exact score
        assert np.all(lo_s <= exact + 1e-300) and np.all(hi_s >= exact - 1e-300)
        # and stay within 2E of it (the margins plus the modelled error)
        assert np.all(exact - lo_s <= 2 * E) and np.all(hi_s - exact <= 2 * E)
        # the exact nearest survives the candidate test
        thr = np.min(hi_s) + 2.0 * 2.0 ** -15 * xx
        best = int(np.argmin(exact))
        assert lo_s[best] <= thr


@pytest.mark.parametrize("d", [4, 8])
def test_hilo_certificate_own_scale(d):
    rng = np.random.default_rng(11 + d)
    cents = (rng.standard_normal((48, d)) * np.exp2(rng.integers(-14, 8, (48, 1)))).astype(np.float16)
    cents[0] = 0
    cents[1, : d // 2] = np.float16(2.0 ** -20)            # subnormal fp16 channels
    xs = [rng.standard_normal(d) * 2.0 ** k for k in (-30, -12, -3, 0, 5, 12)]
    xs.append(cents[5].astype(np.float64) * (1 + 2.0 ** -20))   # a near-tie with a centroid
    xs.append(np.zeros(d))

    def own(x):
        return scale_for(float(np.max(np.abs(-2.0 * np.asarray(x, np.float32)))))
    check_rows(cents, xs, own, False)


@pytest.mark.parametrize("d", [4, 8])
def test_hilo_certificate_workgroup_scale(d):
    """One scale for rows spanning 2^-30 .. 2^12: the small rows' lo parts are
    subnormal, covered by the 2^-24 ||c||_1 term of the norm tables."""
    rng = np.random.default_rng(21 + d)
    cents = (rng.standard_normal((48, d)) * np.exp2(rng.integers(-16, 6, (48, 1)))).astype(np.float16)
    xs = [rng.standard_normal(d) * 2.0 ** k for k in (-30, -20, -10, -3, 0, 6, 12)]
    mx = max(float(np.max(np.abs(-2.0 * np.asarray(x, np.float32)))) for x in xs)
    sc = scale_for(mx)
    check_rows(cents, xs, lambda x: sc, True)


def test_hilo_split_is_exact_to_the_stated_bound():
    """X - (hi + lo) within 2^-22 |X| + 2^-25, and the products exact in fp32."""
    rng = np.random.default_rng(5)
    X = np.concatenate([rng.uniform(-2 ** 15, 2 ** 15, 20000),
                        rng.standard_normal(20000) * 2.0 ** rng.integers(-30, 15, 20000)])
    X = X.astype(np.float32).astype(np.float64)
    hi = X.astype(np.float16).astype(np.float64)
    lo = (X - hi).astype(np.float16).astype(np.float64)
    assert np.all(np.abs(X - (hi + lo)) <= 2.0 ** -22 * np.abs(X) + 2.0 ** -25)
    c = rng.standard_normal(40000).astype(np.float16).astype(np.float64)
    assert np.all((c * hi).astype(np.float32).astype(np.float64) == c * hi)
