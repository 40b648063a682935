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


# ---------------------------------------------------------------- root-sum-square scale

def _rss_brute_force(x, ts, off, dy, alpha, H, d, eps=1e-5):
    """Every term of every gradient entry enumerated one by one in loops.

    dO of token i, feature c (c over the H * d values of the token) is
    written out as the norm backward's terms r g_c, -r g_e / D (each e) and
    -r n_c g_e n_e / D (each e), with g = dY u gamma, n the normalised
    output, r = 1 / sqrt(var + eps) and D = H * d. Then, per head:
    dq_ic = alpha / N * sum_j sum_e SiLU'(s_ij) dO_ie v_je k_jc (j <= i),
    dk_jc the same over i >= j with q_ic, dv_jc = sum_i a_ij dO_ic, a table
    entry = sum over its pairs and e of SiLU'(s_ij) dO_ie v_je / N. Returns
    the square roots of the summed squares.
    """
    T = len(ts)
    D = H * d
    _, o = oracle.hstu_full(x["q"], x["k"], x["v"], x["u"], ts, off, x["pos_tab"], x["time_tab"], alpha, 0,
                            x["gamma"], x["beta"])
    g = dy * x["u"] * (x["gamma"] if x["gamma"] is not None else 1.0)
    do_terms = []                                       # do_terms[i][c] = list of the terms of dO_ic
    for i in range(T):
        mu = o[i].mean()
        r = 1.0 / np.sqrt(((o[i] - mu) ** 2).mean() + eps)
        n = (o[i] - mu) * r
        do_terms.append([[r * g[i, c]] + [-r * g[i, e] / D for e in range(D)]
                         + [-r * n[c] * g[i, e] * n[e] / D for e in range(D)] for c in range(D)])
    out = {k: np.zeros((T, H, d)) for k in ("dq", "dk", "dv")}
    npos, ntime = len(x["pos_tab"]), len(x["time_tab"])
    out["dpos"], out["dtime"] = np.zeros(npos), np.zeros(ntime)
    for b in range(len(off) - 1):
        s0, s1 = int(off[b]), int(off[b + 1])
        N = s1 - s0
        for h in range(H):
            for i in range(s0, s1):
                for j in range(s0, i + 1):
                    pb, tb = oracle.pos_bucket(i - j, npos), oracle.time_bucket(ts[i] - ts[j], ntime)
                    sc = alpha * float(np.dot(x["q"][i, h], x["k"][j, h])) + x["pos_tab"][pb] + x["time_tab"][tb]
                    a, sg = float(oracle.silu(sc)) / N, float(oracle.silu_grad(sc)) / N
                    for c in range(d):
                        for t in do_terms[i][h * d + c]:
                            out["dv"][j, h, c] += (a * t) ** 2
                    for e in range(d):
                        for t in do_terms[i][h * d + e]:
                            w = sg * t * x["v"][j, h, e]  # one term of ds_ij
                            out["dpos"][pb] += w ** 2
                            out["dtime"][tb] += w ** 2
                            for c in range(d):
                                out["dq"][i, h, c] += (alpha * w * x["k"][j, h, c]) ** 2
                                out["dk"][j, h, c] += (alpha * w * x["q"][i, h, c]) ** 2
    return {k: np.sqrt(v) for k, v in out.items()}


def test_rss_matches_term_by_term_enumeration():
    x, ts, off, dy = _case(11, [3, 1], 2, 2, 4, 6, False, False, True)
    alpha = 0.8
    g = oracle.hstu_full_bwd(x["q"], x["k"], x["v"], x["u"], ts, off, dy, x["pos_tab"], x["time_tab"],
                             alpha, 0, x["gamma"], x["beta"], magnitudes=True)
    bf = _rss_brute_force(x, ts, off, dy, alpha, 2, 2)
    for name in ("dq", "dk", "dv", "dpos", "dtime"):
        np.testing.assert_allclose(g["rss_" + name], bf[name], rtol=1e-12, atol=1e-300, err_msg=name)


def _term_counts(lengths, H, d, n_pos, n_time, ts):
    """Number of terms of each gradient entry once dO is written out (2 D + 1
    terms each, D = H d): dq_ic sums over keys j <= i and features e, dk_jc
    over queries i >= j and e, dv_jc over queries i >= j, a table entry over
    its pairs and e (and the heads, for a shared table)."""
    T = sum(lengths)
    nt = 2 * H * d + 1
    nq, nk = np.zeros(T), np.zeros(T)
    npos, ntime = np.zeros(n_pos), np.zeros(n_time)
    s0 = 0
    for L in lengths:
        for i in range(L):
            for j in range(i + 1):
                nq[s0 + i] += 1
                nk[s0 + j] += 1
                npos[min(i - j, n_pos - 1)] += 1
                dt = abs(int(ts[s0 + i]) - int(ts[s0 + j]))
                ntime[min(int(np.floor(np.log2(dt + 1))), n_time - 1)] += 1
        s0 += L
    return {"dq": nq[:, None, None] * d * nt, "dk": nk[:, None, None] * d * nt, "dv": nk[:, None, None] * nt,
            "dpos": npos * d * H * nt, "dtime": ntime * d * H * nt}


@pytest.mark.parametrize("case", range(len(CASES)))
def test_rss_bounds_the_gradient(case):
    """Cauchy-Schwarz: a sum of n terms is at most sqrt(n) times their
    root-sum-square; with n counted from the mask, |g| <= sqrt(n) rss."""
    lengths, H, d, n_pos, n_time, php, pht, aff, alpha, norm_n = CASES[case]
    x, ts, off, dy = _case(60 + case, lengths, H, d, n_pos, n_time, False, False, aff)
    g = oracle.hstu_full_bwd(x["q"], x["k"], x["v"], x["u"], ts, off, dy, x["pos_tab"], x["time_tab"], alpha,
                             norm_n, x["gamma"], x["beta"], magnitudes=True)
    n = _term_counts(lengths, H, d, n_pos, n_time, ts)
    for name in ("dq", "dk", "dv", "dpos", "dtime"):
        r, v = g["rss_" + name], np.abs(g[name])
        assert np.all(v <= np.sqrt(np.broadcast_to(n[name], r.shape)) * r * (1 + 1e-12)), name
        assert np.all(r[v > 0] > 0), name


def _bf16(x):
    import workloads as W
    return W.round_to_bf16(np.asarray(x, dtype=np.float32)).astype(np.float64)


def _bwd_case():
    import workloads as W
    inp = W.jagged("rss_bar", 61, [1, 77, 300, 130, 64, 129], 2, 128, "bf16", 128, 128)
    dy = W.upstream_grad(62, inp.u.shape)
    return inp, dy


def test_bf16_rounding_model_passes_the_gradient_bar():
    """The bar against the error model it comes from: a backward whose dO, P
    and dS are rounded to bf16, whose dO comes from an output recomputed with
    the bf16 P, and whose results are returned in bf16 (the roundings the GPU
    path makes) stays well under it."""
    from tolerances import GRAD_RSS_BF16
    inp, dy = _bwd_case()
    ref = oracle.hstu_full_bwd(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, dy, inp.tables.pos,
                               inp.tables.time, magnitudes=True)
    T, H, d = inp.q.shape
    off = inp.seq_offsets
    pieces = []
    for b in range(len(off) - 1):
        s0, s1 = int(off[b]), int(off[b + 1])
        L = s1 - s0
        if L == 0:
            continue
        i = np.arange(L)
        allowed = i[None, :] <= i[:, None]
        rel = np.where(allowed, i[:, None] - i[None, :], 0)
        t = inp.ts[s0:s1].astype(np.int64)
        dt = t[:, None] - t[None, :]
        bias = (inp.tables.pos[oracle.pos_bucket(rel, 128)] + inp.tables.time[oracle.time_bucket(dt, 128)])
        for h in range(H):
            q, k, v = (a[s0:s1, h].astype(np.float64) for a in (inp.q, inp.k, inp.v))
            s = q @ k.T + bias
            pieces.append((s0, s1, h, q, k, v, s, allowed, _bf16(np.where(allowed, oracle.silu(s), 0.0) / L)))
    # the recomputed forward multiplies the bf16 P too; dO comes from that O
    o = np.zeros((T, H, d))
    for s0, s1, h, q, k, v, s, allowed, p in pieces:
        o[s0:s1, h] = p @ v
    do = _bf16(oracle.layer_norm_gate_bwd(o.reshape(T, -1), inp.u, dy)[0]).reshape(T, H, d)
    sim = {name: np.zeros((T, H, d)) for name in ("dq", "dk", "dv")}
    for s0, s1, h, q, k, v, s, allowed, p in pieces:
        ds = _bf16(np.where(allowed, (do[s0:s1, h] @ v.T) * oracle.silu_grad(s), 0.0) / (s1 - s0))
        sim["dq"][s0:s1, h] = _bf16(ds @ k)
        sim["dk"][s0:s1, h] = _bf16(ds.T @ q)
        sim["dv"][s0:s1, h] = _bf16(p.T @ do[s0:s1, h])
    for name in ("dq", "dk", "dv"):
        err = oracle.max_err_vs_scale(sim[name], ref[name], ref["rss_" + name])
        assert 0.1 * GRAD_RSS_BF16 < err < 0.75 * GRAD_RSS_BF16, (name, err)


def test_gradient_bar_catches_a_skipped_key_tile():
    """The oracle's own gradients with the keys 64..127 of one user dropped
    (what a kernel that skips one key tile returns) fail the bar by far; the
    per-row magnitude metric let this through."""
    from tolerances import GRAD_RSS_BF16
    inp, dy = _bwd_case()
    args = (inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, dy, inp.tables.pos, inp.tables.time)
    ref = oracle.hstu_full_bwd(*args, magnitudes=True)

    def drop(b, allowed):
        if b == 2:                                      # the 300-token user
            allowed[:, 64:128] = False
        return allowed

    bad = oracle.hstu_full_bwd(*args, pair_mask=drop)
    T = len(inp.q)
    for name in ("dq", "dk", "dv"):
        err = oracle.max_err_vs_scale(bad[name], ref[name], ref["rss_" + name])
        assert err > 10 * GRAD_RSS_BF16, (name, err)
    for name in ("dpos", "dtime"):
        assert oracle.max_err_vs_scale(bad[name], ref[name], ref["rss_" + name]) > 5 * GRAD_RSS_BF16, name
    # the old per-row magnitude metric on dq stays under its 2e-2 bar
    m = oracle.max_rel_err_vs_magnitude(bad["dq"].reshape(T, -1), ref["dq"].reshape(T, -1),
                                        ref["mag_dq"].reshape(T, -1))
    assert m > 0
    # nothing dropped: identical
    same = oracle.hstu_full_bwd(*args, pair_mask=lambda b, a: a)
    for name in ("dq", "dk", "dv", "dpos", "dtime"):
        assert np.array_equal(same[name], ref[name]), name
