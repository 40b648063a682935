"""Pins of the oracle's backward (hstu_full_bwd) to something other than itself.

The pages give no backward formula, so the independent reference is the
derivative itself: central finite differences of the oracle's forward
(already pinned by brute force and closed forms) in float64, for every
element of every differentiable input. A dropped term, a wrong sign or a
transposed operand anywhere in the chain rule fails these."""
import numpy as np
import pytest

import oracle


def _case(seed, lengths, H, d, n_pos, n_time, per_head_pos, per_head_time, affine):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    gaps = rng.choice([0, 1, 3, 9, 40, 150], size=T)   # several time buckets, some clamped
    ts = np.cumsum(gaps).astype(np.int64)
    x = dict(
        q=rng.normal(size=(T, H, d)), k=rng.normal(size=(T, H, d)), v=rng.normal(size=(T, H, d)),
        u=rng.normal(size=(T, H * d)),
        pos_tab=rng.normal(scale=0.5, size=(H, n_pos) if per_head_pos else (n_pos,)),
        time_tab=rng.normal(scale=0.5, size=(H, n_time) if per_head_time else (n_time,)),
        gamma=rng.normal(1.0, 0.3, size=H * d) if affine else None,
        beta=rng.normal(0.0, 0.3, size=H * d) if affine else None,
    )
    dy = rng.normal(size=(T, H * d))
    return x, ts, off, dy


def _loss(x, ts, off, dy, alpha, norm_n):
    y, _ = oracle.hstu_full(x["q"], x["k"], x["v"], x["u"], ts, off, x["pos_tab"], x["time_tab"], alpha, norm_n,
                            x["gamma"], x["beta"])
    return float((y * dy).sum())


CASES = [
    # lengths, H, d, n_pos, n_time, per-head pos, per-head time, affine, alpha, norm_n
    ([3, 0, 5], 2, 4, 4, 6, True, False, True, 0.7, 0),
    ([6, 2], 2, 3, 8, 4, False, True, False, 1.3, 5),
    ([1, 4], 1, 2, 2, 3, False, False, True, 1.0, 0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_backward_matches_central_differences(case):
    lengths, H, d, n_pos, n_time, php, pht, aff, alpha, norm_n = CASES[case]
    x, ts, off, dy = _case(40 + case, lengths, H, d, n_pos, n_time, php, pht, aff)
    g = oracle.hstu_full_bwd(x["q"], x["k"], x["v"], x["u"], ts, off, dy, x["pos_tab"], x["time_tab"], alpha,
                             norm_n, x["gamma"], x["beta"])
    names = {"q": "dq", "k": "dk", "v": "dv", "u": "du", "pos_tab": "dpos", "time_tab": "dtime",
             "gamma": "dgamma", "beta": "dbeta"}
    eps = 1e-6
    for name, gname in names.items():
        if x[name] is None:
            assert g[gname] is None
            continue
        ana = np.asarray(g[gname]).reshape(np.shape(x[name]))
        num = np.zeros_like(ana)
        base = x[name]
        for idx in np.ndindex(base.shape):
            keep = base[idx]
            base[idx] = keep + eps
            lp = _loss(x, ts, off, dy, alpha, norm_n)
            base[idx] = keep - eps
            lm = _loss(x, ts, off, dy, alpha, norm_n)
            base[idx] = keep
            num[idx] = (lp - lm) / (2 * eps)
        scale = max(np.abs(num).max(), 1e-12)
        assert np.abs(ana - num).max() / scale < 1e-6, (name, np.abs(ana - num).max(), scale)


def test_zero_upstream_gives_zero_gradients():
    x, ts, off, dy = _case(7, [4, 3], 2, 4, 4, 6, True, True, True)
    g = oracle.hstu_full_bwd(x["q"], x["k"], x["v"], x["u"], ts, off, np.zeros_like(dy), x["pos_tab"],
                             x["time_tab"], 1.0, 0, x["gamma"], x["beta"])
    for key, val in g.items():
        assert val is not None and not np.any(val), key


def test_masked_future_keys_get_no_query_gradient():
    """Query i only sees keys <= i: perturbing dy of the first row moves no key beyond it."""
    x, ts, off, dy = _case(8, [5], 1, 3, 4, 6, False, False, False)
    dy0 = np.zeros_like(dy)
    dy0[0] = dy[0]
    g = oracle.hstu_full_bwd(x["q"], x["k"], x["v"], x["u"], ts, off, dy0, x["pos_tab"], x["time_tab"])
    assert not np.any(g["dk"][1:]) and not np.any(g["dv"][1:]) and not np.any(g["dq"][1:])
    assert np.any(g["dk"][0]) and np.any(g["dv"][0])


def test_silu_grad_closed_forms():
    assert oracle.silu_grad(0.0) == 0.5
    x = np.array([-40.0, -3.0, 0.25, 2.0, 60.0])
    sg = 1 / (1 + np.exp(-x))
    np.testing.assert_allclose(oracle.silu_grad(x), sg + x * sg * (1 - sg), rtol=1e-15)
    assert abs(oracle.silu_grad(60.0) - 1.0) < 1e-20 + 1e-15


@pytest.mark.parametrize("case", range(len(CASES)))
def test_magnitudes_bound_the_gradients(case):
    """Each magnitude is the same sum over absolute values, so it bounds |g| (triangle inequality)."""
    lengths, H, d, n_pos, n_time, php, pht, aff, alpha, norm_n = CASES[case]
    x, ts, off, dy = _case(50 + case, lengths, H, d, n_pos, n_time, php, pht, aff)
    g = oracle.hstu_full_bwd(x["q"], x["k"], x["v"], x["u"], ts, off, dy, x["pos_tab"], x["time_tab"], alpha,
                             norm_n, x["gamma"], x["beta"], magnitudes=True)
    for name in ("dq", "dk", "dv", "du", "dpos", "dtime", "dgamma", "dbeta"):
        if g[name] is None:
            continue
        assert np.all(g["mag_" + name] >= np.abs(g[name]) * (1 - 1e-12)), name
    assert oracle.max_rel_err_vs_magnitude(g["dq"].reshape(len(g["dq"]), -1), g["dq"].reshape(len(g["dq"]), -1),
                                           g["mag_dq"].reshape(len(g["dq"]), -1)) == 0.0


def test_magnitude_equals_value_without_cancellation():
    """One token, one head: dv = a dO has a single term, so |dv| equals its magnitude."""
    x, ts, off, dy = _case(9, [1], 1, 4, 4, 6, False, False, True)
    g = oracle.hstu_full_bwd(x["q"], x["k"], x["v"], x["u"], ts, off, dy, x["pos_tab"], x["time_tab"],
                             magnitudes=True)
    np.testing.assert_allclose(g["mag_dv"], np.abs(g["dv"]), rtol=1e-14)
    # dq's terms carry the sum over d inside da = dO . v, so there it only bounds
    assert np.all(g["mag_dq"] >= np.abs(g["dq"]))
