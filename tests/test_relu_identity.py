"""The block-score kernel sums the per-head ReLUs as p + relu(d) = max(p + d, p) for p >= +0
(relu(d) = d > 0 ? d : +0, max = IEEE maxNum, which returns the number when one operand is a
quiet NaN).  Checked here bit for bit in IEEE binary32 (numpy float32 arithmetic, np.fmax is
maxNum) over special values and random ones, against the plain sequential form."""
import numpy as np

F = np.float32


def relu(d):
    return np.where(d > F(0), d, F(0)).astype(F)


def specials():
    fm = np.finfo(F)
    v = [0.0, -0.0, 1e-45, -1e-45, fm.tiny, -fm.tiny, 1.0, -1.0, 0.5, -0.5, 3.0e-39, fm.max,
         -fm.max, np.inf, -np.inf, np.nan, 1e30, -1e30, 2.0 ** -24, -2.0 ** -24]
    return np.array(v, F)


def test_identity_on_special_and_random_values():
    rng = np.random.default_rng(0)
    p = np.concatenate([np.abs(specials()[~np.isnan(specials())]),
                        np.abs(rng.standard_normal(4000).astype(F)) * F(10) ** rng.integers(
                            -40, 38, 4000).astype(F)]).astype(F)
    p = p[~np.isnan(p)]
    p = p[np.signbit(p) == 0]                     # p >= +0
    d = np.concatenate([specials(), rng.standard_normal(4000).astype(F) *
                        F(10) ** rng.integers(-40, 38, 4000).astype(F)]).astype(F)
    P, D = np.meshgrid(p, d, indexing="ij")
    with np.errstate(all="ignore"):
        want = (P + relu(D)).astype(F)
        got = np.fmax((P + D).astype(F), P).astype(F)
    assert np.array_equal(want.view(np.uint32), got.view(np.uint32))


def test_head_sum_chain_matches_sequential_sum():
    rng = np.random.default_rng(1)
    sp = specials()
    d = rng.choice(np.concatenate([sp, rng.standard_normal(64).astype(F)]), (200000, 4))
    d = d.astype(F)
    with np.errstate(all="ignore"):
        want = F(0) + relu(d[:, 0])
        for h in range(1, 4):
            want = (want + relu(d[:, h])).astype(F)
        p = relu(d[:, 0])
        for h in range(1, 4):
            p = np.fmax((p + d[:, h]).astype(F), p).astype(F)
    assert np.array_equal(want.view(np.uint32), p.view(np.uint32))
