"""Pins for the fp64 oracle: closed forms, exhaustive checks, brute force, invariants.

Each test fixes the oracle to something other than itself: a closed form of
the definition for specially built inputs, an exhaustive integer check, a
textbook routine (np.convolve, np.cumsum), or an invariant the pages state
(cached reuse equals recompute; M-FALCON only changes mask and bias so that
candidates do not interact; causal next-action modelling).
"""
import math

import numpy as np
import pytest

import oracle
import oracle.hstu as oracle_hstu
import workloads as W
from tolerances import TOL


def _rand_case(rng, lengths, H, d, n_pos=5, n_time=6, per_head=False, ts_spread=50):
    T = int(sum(lengths))
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d))
    u = rng.standard_normal((T, H * d))
    ts = np.zeros(T, dtype=np.int64)
    o = 0
    for L in lengths:
        ts[o:o + L] = 1000 + np.cumsum(rng.integers(0, ts_spread, size=L))
        o += L
    pshape = (H, n_pos) if per_head else (n_pos,)
    tshape = (H, n_time) if per_head else (n_time,)
    pos = rng.standard_normal(pshape) if n_pos else None
    tim = rng.standard_normal(tshape) if n_time else None
    off = W.offsets_from_lengths(lengths)
    return q, k, v, u, ts, off, pos, tim


def _brute(q, k, v, u, ts, off, pos, tim, alpha=1.0, norm_n=0, gamma=None, beta=None, eps=1e-5):
    """Scalar loops with math.exp, one (i, j) pair at a time."""
    T, H, d = q.shape
    z = [[0.0] * (H * d) for _ in range(T)]
    for b in range(len(off) - 1):
        s0, s1 = int(off[b]), int(off[b + 1])
        L = s1 - s0
        N = norm_n if norm_n > 0 else L
        for h in range(H):
            for i in range(L):
                for j in range(i + 1):
                    s = alpha * sum(float(q[s0 + i, h, c]) * float(k[s0 + j, h, c]) for c in range(d))
                    if pos is not None:
                        p = pos if pos.ndim == 1 else pos[h]
                        s += float(p[min(i - j, len(p) - 1)])
                    if tim is not None:
                        t = tim if tim.ndim == 1 else tim[h]
                        x = abs(int(ts[s0 + i]) - int(ts[s0 + j])) + 1
                        bkt = 0
                        while (1 << (bkt + 1)) <= x:
                            bkt += 1
                        s += float(t[min(bkt, len(t) - 1)])
                    a = s / (1.0 + math.exp(-s)) / N
                    for c in range(d):
                        z[s0 + i][h * d + c] += a * float(v[s0 + j, h, c])
    y = np.zeros((T, H * d))
    for t in range(T):
        row = z[t]
        mu = sum(row) / len(row)
        var = sum((x - mu) ** 2 for x in row) / len(row)
        for c in range(H * d):
            n = (row[c] - mu) / math.sqrt(var + eps)
            if gamma is not None:
                n *= float(gamma[c])
            if beta is not None:
                n += float(beta[c])
            y[t, c] = n * float(u[t, c])
    return y


# ---------------------------------------------------------------- buckets

def test_time_bucket_exhaustive_against_doubling():
    dt = np.arange(0, (1 << 20) + 1, dtype=np.int64)
    got = oracle.time_bucket(dt, 64)
    # floor(log2(dt + 1)) by doubling: count how many powers of two are <= dt + 1
    x = dt + 1
    want = np.zeros_like(dt)
    p = np.int64(2)
    while p <= x.max():
        want += (x >= p)
        p *= 2
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.time_bucket(-dt, 64), want)          # |dt|
    assert np.array_equal(oracle.time_bucket(dt, 7), np.minimum(want, 6))  # clamp


def test_time_bucket_large_and_boundaries():
    for k in range(1, 52):
        v = (1 << k) - 1     # dt + 1 = 2**k exactly -> bucket k
        assert int(oracle.time_bucket(np.array([v]), 64)[0]) == k
        assert int(oracle.time_bucket(np.array([v - 1]), 64)[0]) == k - 1


def test_pos_bucket_clamp():
    assert list(oracle.pos_bucket(np.arange(8), 5)) == [0, 1, 2, 3, 4, 4, 4, 4]


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("case", range(6))
def test_matches_brute_force_tiny(case):
    rng = np.random.default_rng(100 + case)
    lengths = [[0, 1, 3], [5], [2, 0, 7], [1], [4, 6], [8, 3]][case]
    H, d = [(1, 1), (2, 3), (2, 4), (1, 2), (2, 2), (1, 4)][case]
    per_head = case % 2 == 1
    alpha = [1.0, 0.5, 1.0, 2.0, 1.0, 0.7][case]
    norm_n = [0, 0, 3, 0, 0, 11][case]
    q, k, v, u, ts, off, pos, tim = _rand_case(rng, lengths, H, d, per_head=per_head)
    gamma = rng.standard_normal(H * d) if case in (2, 4) else None
    beta = rng.standard_normal(H * d) if case in (2, 5) else None
    y, _ = oracle.hstu_full(q, k, v, u, ts, off, pos, tim, alpha, norm_n, gamma, beta)
    yb = _brute(q, k, v, u, ts, off, pos, tim, alpha, norm_n, gamma, beta)
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-12)


def test_tiny_config_matches_brute_force():
    inp = W.tiny_fp32()
    y, _ = oracle.hstu_full(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, inp.tables.pos, None)
    # brute force on the first 12 tokens of each sequence is exact for those rows
    # only if N is the full length: pass it through norm_n per sequence.
    for b in range(inp.batch):
        s0 = int(inp.seq_offsets[b])
        L = int(inp.lengths[b])
        n = 12
        sl = slice(s0, s0 + n)
        yb = _brute(inp.q[sl], inp.k[sl], inp.v[sl], inp.u[sl], inp.ts[sl], np.array([0, n]),
                    inp.tables.pos, None, norm_n=L)
        np.testing.assert_allclose(y[sl], yb, rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------- closed forms

def test_single_token_closed_form():
    rng = np.random.default_rng(7)
    H, d = 2, 3
    q, k, v = (rng.standard_normal((1, H, d)) for _ in range(3))
    u = rng.standard_normal((1, H * d))
    pos = np.array([0.3, -1.0])
    tim = np.array([-0.2, 5.0, 5.0])
    ts = np.array([123], dtype=np.int64)
    y, o = oracle.hstu_full(q, k, v, u, ts, [0, 1], pos, tim, alpha=0.5)
    for h in range(H):
        s = 0.5 * float(q[0, h] @ k[0, h]) + 0.3 - 0.2
        a = s / (1 + math.exp(-s))
        np.testing.assert_allclose(o[0, h * d:(h + 1) * d], a * v[0, h], rtol=1e-14)
    z = o[0]
    want = (z - z.mean()) / math.sqrt(z.var() + 1e-5) * u[0]
    np.testing.assert_allclose(y[0], want, rtol=1e-13)


@pytest.mark.parametrize("s_target", [2.5, 64.0, -64.0])
def test_constant_score_is_scaled_prefix_sum(s_target):
    """q_i = q, k_j = k and no bias: every allowed score is alpha q.k, so
    o_i = SiLU(s) / N * (v_0 + ... + v_i), a prefix sum."""
    rng = np.random.default_rng(11)
    L, H, d, alpha = 9, 1, 4, 0.5
    qv = np.array([1.0, 0.0, 0.0, 0.0])
    kv = np.array([2 * s_target, 0.0, 0.0, 0.0])
    q = np.tile(qv, (L, H, 1))
    k = np.tile(kv, (L, H, 1))
    v = rng.standard_normal((L, H, d))
    u = np.ones((L, H * d))
    ts = np.arange(L, dtype=np.int64)
    beta = rng.standard_normal(H * d)
    y, o = oracle.hstu_full(q, k, v, u, ts, [0, L], None, None, alpha=alpha, beta=beta)
    sil = s_target / (1 + math.exp(-s_target))
    want = sil / L * np.cumsum(v[:, 0, :], axis=0)
    np.testing.assert_allclose(o, want, rtol=1e-13, atol=1e-300)
    if s_target < 0:
        # o is ~1e-27 times v: LayerNorm of a near-zero row contributes ~1e-25, y = beta * u
        np.testing.assert_allclose(y, np.tile(beta, (L, 1)), atol=1e-20)


def test_position_bias_only_is_causal_convolution():
    """Q = K = 0 with a position table only: a_ij = w[i - j], w[r] = SiLU(P[min(r, n_pos - 1)]) / N,
    so each channel of o is the causal convolution of w with v."""
    rng = np.random.default_rng(12)
    L, H, d = 40, 2, 3
    P = rng.standard_normal(7)
    q = np.zeros((L, H, d))
    k = np.zeros((L, H, d))
    v = rng.standard_normal((L, H, d))
    u = np.ones((L, H * d))
    ts = np.arange(L, dtype=np.int64) * 1000
    _, o = oracle.hstu_full(q, k, v, u, ts, [0, L], P, None)
    w = np.array([P[min(r, 6)] / (1 + math.exp(-P[min(r, 6)])) for r in range(L)]) / L
    for h in range(H):
        for c in range(d):
            want = np.convolve(w, v[:, h, c])[:L]
            np.testing.assert_allclose(o[:, h * d + c], want, rtol=1e-12, atol=1e-14)


def test_time_bias_only_closed_form():
    """Timestamps 2**i - 1: for 0 < j < i, |ts_i - ts_j| + 1 = 2**i - 2**j + 1 lies in
    (2**(i-1), 2**i), so the bucket is i - 1; for j = 0 it is exactly 2**i (bucket i);
    the diagonal has bucket 0."""
    rng = np.random.default_rng(13)
    L, H, d, nt = 12, 1, 2, 8
    Tt = rng.standard_normal(nt)
    ts = (1 << np.arange(L, dtype=np.int64)) - 1
    q = np.zeros((L, H, d))
    k = np.zeros((L, H, d))
    v = rng.standard_normal((L, H, d))
    u = np.ones((L, H * d))
    _, o = oracle.hstu_full(q, k, v, u, ts, [0, L], None, Tt)
    sil = lambda x: x / (1 + math.exp(-x))
    for i in range(L):
        want = sil(Tt[0]) * v[i, 0]
        for j in range(i):
            bkt = i if j == 0 else i - 1
            want = want + sil(Tt[min(bkt, nt - 1)]) * v[j, 0]
        np.testing.assert_allclose(o[i], want / L, rtol=1e-12, atol=1e-15)


def test_layer_norm_closed_forms():
    rng = np.random.default_rng(14)
    z = rng.standard_normal((5, 16)) * 3
    y = oracle.layer_norm_gate(z, np.ones_like(z))
    var = z.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-14)
    np.testing.assert_allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-12)
    # the norm spans all heads of a token: H = 2, d = 1, z = [a, b] gives +-|a-b|/2 / sqrt((a-b)^2/4 + eps)
    a, b = 0.7, -0.1
    yy = oracle.layer_norm_gate(np.array([[a, b]]), np.array([[1.0, 1.0]]))
    m = abs(a - b) / 2 / math.sqrt((a - b) ** 2 / 4 + 1e-5)
    np.testing.assert_allclose(yy[0], [m, -m], rtol=1e-13)


def test_zero_v_gives_beta_times_u():
    rng = np.random.default_rng(15)
    q, k, v, u, ts, off, pos, tim = _rand_case(rng, [6, 3], 2, 4)
    v[:] = 0
    beta = rng.standard_normal(8)
    y, _ = oracle.hstu_full(q, k, v, u, ts, off, pos, tim)
    assert np.all(y == 0)
    y, _ = oracle.hstu_full(q, k, v, u, ts, off, pos, tim, beta=beta)
    np.testing.assert_allclose(y, beta * u, rtol=1e-15)


# ---------------------------------------------------------------- invariants

def test_causality_under_perturbation():
    rng = np.random.default_rng(16)
    q, k, v, u, ts, off, pos, tim = _rand_case(rng, [30], 2, 4)
    y, _ = oracle.hstu_full(q, k, v, u, ts, off, pos, tim, norm_n=30)
    i = 17
    q2, k2, v2, u2, ts2 = q.copy(), k.copy(), v.copy(), u.copy(), ts.copy()
    q2[i + 1:] += 1
    k2[i + 1:] -= 2
    v2[i + 1:] *= 3
    u2[i + 1:] = 0
    ts2[i + 1:] += 10 ** 6
    y2, _ = oracle.hstu_full(q2, k2, v2, u2, ts2, off, pos, tim, norm_n=30)
    assert np.array_equal(y[:i + 1], y2[:i + 1])
    assert not np.allclose(y[i + 1:], y2[i + 1:])


def test_jagged_batch_equals_per_sequence_runs():
    rng = np.random.default_rng(17)
    lengths = [5, 0, 12, 1, 7]
    q, k, v, u, ts, off, pos, tim = _rand_case(rng, lengths, 2, 3)
    y, _ = oracle.hstu_full(q, k, v, u, ts, off, pos, tim)
    for b in range(len(lengths)):
        sl = slice(int(off[b]), int(off[b + 1]))
        yb, _ = oracle.hstu_full(q[sl], k[sl], v[sl], u[sl], ts[sl], [0, lengths[b]], pos, tim)
        assert np.array_equal(y[sl], yb)


def test_cached_equals_full_recompute():
    inp = W.cached("c", 21, [0, 70, 64, 130], [5, 64, 1, 0], H=2, d=8, dtype="f32", n_pos=16, n_time=16)
    h = inp.hist
    yfull, _ = oracle.hstu_full(h.q, h.k, h.v, h.u, h.ts, h.seq_offsets, h.tables.pos, h.tables.time)
    _, new_rows = inp.split()
    y, _ = oracle.hstu_cached(h.q[new_rows], h.u[new_rows], h.ts[new_rows], h.k, h.v, h.ts, h.seq_offsets,
                              inp.cache_lens, inp.new_offsets(), h.tables.pos, h.tables.time)
    np.testing.assert_allclose(y, yfull[new_rows], rtol=1e-12, atol=1e-12)


def _mf_case(seed, hist, cand, H=2, d=4):
    ci = W.candidates("m", seed, hist, cand, H=H, d=d, dtype="f32", n_pos=16, n_time=16)
    return ci.inputs, ci.hist_lens, ci.num_candidates


def test_mfalcon_candidate_equals_full_path_on_history_plus_candidate():
    inp, n, m = _mf_case(31, [9, 20], [4, 3])
    y, _ = oracle.hstu_mfalcon(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, m,
                               inp.tables.pos, inp.tables.time)
    for b in range(2):
        s0 = int(inp.seq_offsets[b])
        hist = np.arange(s0, s0 + n[b])
        for c in range(s0 + n[b], s0 + n[b] + m[b]):
            idx = np.concatenate([hist, [c]])
            yf, _ = oracle.hstu_full(inp.q[idx], inp.k[idx], inp.v[idx], inp.u[idx], inp.ts[idx],
                                     [0, len(idx)], inp.tables.pos, inp.tables.time)
            np.testing.assert_allclose(y[c], yf[-1], rtol=1e-12, atol=1e-12)
            # history rows equal the full path on history + [c] as well (causal)
            np.testing.assert_allclose(y[hist], yf[:-1], rtol=1e-12, atol=1e-12)


def test_mfalcon_candidates_do_not_interact():
    inp, n, m = _mf_case(32, [15], [6])
    y, _ = oracle.hstu_mfalcon(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, m,
                               inp.tables.pos, inp.tables.time)
    q, k, v = inp.q.copy(), inp.k.copy(), inp.v.copy()
    other = np.arange(15 + 3, 21)  # candidates 3..5 perturbed
    q[other] += 5
    k[other] -= 1
    v[other] *= -2
    y2, _ = oracle.hstu_mfalcon(q, k, v, inp.u, inp.ts, inp.seq_offsets, m, inp.tables.pos, inp.tables.time)
    assert np.array_equal(y[:18], y2[:18])
    # removing candidates changes nothing for the others either
    keep = np.arange(0, 17)
    y3, _ = oracle.hstu_mfalcon(inp.q[keep], inp.k[keep], inp.v[keep], inp.u[keep], inp.ts[keep], [0, 17],
                                [2], inp.tables.pos, inp.tables.time)
    assert np.array_equal(y[:17], y3)


def test_mfalcon_history_rows_are_full_path_with_fixed_n():
    inp, n, m = _mf_case(33, [11, 0, 6], [2, 3, 0])
    y, _ = oracle.hstu_mfalcon(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, m,
                               inp.tables.pos, inp.tables.time)
    for b in range(3):
        s0 = int(inp.seq_offsets[b])
        h = np.arange(s0, s0 + n[b])
        if len(h) == 0:
            continue
        yf, _ = oracle.hstu_full(inp.q[h], inp.k[h], inp.v[h], inp.u[h], inp.ts[h], [0, len(h)],
                                 inp.tables.pos, inp.tables.time, norm_n=int(n[b]) + 1)
        np.testing.assert_allclose(y[h], yf, rtol=1e-13, atol=1e-13)


def test_mfalcon_candidate_without_history_is_self_only():
    inp, n, m = _mf_case(34, [0], [3], H=1, d=2)
    pos, tim = inp.tables.pos, inp.tables.time
    y, o = oracle.hstu_mfalcon(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, m, pos, tim)
    for c in range(3):
        s = float(inp.q[c, 0].astype(np.float64) @ inp.k[c, 0].astype(np.float64)) + float(pos[0]) + float(tim[0])
        np.testing.assert_allclose(o[c], s / (1 + math.exp(-s)) * inp.v[c, 0].astype(np.float64), rtol=1e-13)


def test_full_rows_sampler_matches_full():
    inp = W.jagged("r", 41, [33, 70], 2, 8, "f32", 16, 16)
    y, _ = oracle.hstu_full(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, inp.tables.pos, inp.tables.time)
    rows = np.array([0, 5, 32, 33, 34, 102])
    yr = oracle.hstu_full_rows(rows, inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets,
                               inp.tables.pos, inp.tables.time)
    np.testing.assert_allclose(yr, y[rows], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- paged append

def test_kv_append_lands_in_logical_order():
    inp = W.cached("p", 51, [3, 64, 0], [70, 1, 2], H=2, d=4, dtype="f32", n_pos=4, n_time=4, page_size=8)
    h = inp.hist
    P = inp.num_pages
    kp = np.zeros((P, 2, 8, 4))
    vp = np.zeros((P, 2, 8, 4))
    tp = np.zeros((P, 8), dtype=np.int64)
    pre, new = inp.split()
    # prefill the prefix as an append onto an empty cache, then append the new tokens
    kp, vp, tp = oracle.kv_append_pages(kp, vp, tp, inp.page_table, np.zeros(3, np.int32), inp.prefix_offsets(),
                                        h.k[pre], h.v[pre], h.ts[pre], page_size=8)
    kp, vp, tp = oracle.kv_append_pages(kp, vp, tp, inp.page_table, inp.cache_lens, inp.new_offsets(),
                                        h.k[new], h.v[new], h.ts[new], page_size=8)
    for b in range(3):
        L = int(inp.cache_lens[b] + inp.new_lens[b])
        s0 = int(h.seq_offsets[b])
        for p in range(L):
            page = inp.page_table[b, p // 8]
            assert np.array_equal(kp[page, :, p % 8], h.k[s0 + p])
            assert np.array_equal(vp[page, :, p % 8], h.v[s0 + p])
            assert tp[page, p % 8] == h.ts[s0 + p]
    used = set(inp.page_table[inp.page_table >= 0].tolist())
    for page in set(range(P)) - used:
        assert not kp[page].any() and not vp[page].any()


# ---------------------------------------------------------------- layer

def test_layer_split_order_and_rows():
    """U, V, Q, K come from consecutive H*d column blocks of SiLU(X W1)."""
    H, d, D = 1, 2, 3
    hd = H * d
    # two tokens; token 0 carries feature 0 only, token 1 feature 1 only.
    x = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 0.0]])
    w1 = np.zeros((D, 4 * hd))
    w1[:, 0:hd] = 1.0          # U = SiLU(1) for both tokens
    w1[0, hd:2 * hd] = [1.0, -1.0]   # V row 0: token 0 only
    w1[1, 2 * hd] = 3.0        # Q: token 1 only, channel 0
    w1[0, 3 * hd] = 2.0        # K: token 0 only, channel 0
    w2 = np.eye(hd)
    ts = np.array([0, 5], dtype=np.int64)
    y = oracle.hstu_layer(x, w1, w2, ts, [0, 2], H, d)
    sil = lambda t: t / (1 + math.exp(-t))
    # token 1 row: keys 0 and 1; s_10 = q1.k0 = SiLU(3) * SiLU(2); s_11 = q1.k1 = 0
    s10 = sil(3.0) * sil(2.0)
    v0 = np.array([sil(1.0), sil(-1.0)])
    o1 = sil(s10) * v0 / 2           # v1 = SiLU(0) = 0
    z = o1
    want1 = (z - z.mean()) / math.sqrt(z.var() + 1e-5) * sil(1.0)
    np.testing.assert_allclose(y[1], want1, rtol=1e-12)
    yr = oracle.hstu_layer(x, w1, w2, ts, [0, 2], H, d, rows=[1])
    np.testing.assert_allclose(yr[0], y[1], rtol=1e-13)


def test_layer_rows_match_full_layer():
    li = W.full_layer(seed=62, batch=3, embed=16, num_heads=2, head_dim=4, lengths=[5, 9, 1])
    y = oracle.hstu_layer(li.x, li.w1, li.w2, li.ts, li.seq_offsets, 2, 4, li.tables.pos, li.tables.time)
    rows = np.array([0, 4, 5, 11, 13, 14])
    yr = oracle.hstu_layer(li.x, li.w1, li.w2, li.ts, li.seq_offsets, 2, 4, li.tables.pos, li.tables.time,
                           rows=rows)
    np.testing.assert_allclose(yr, y[rows], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- metric, counts

def test_max_rel_row_error():
    ref = np.array([[1.0, -2.0], [0.0, 0.0]])
    assert oracle.max_rel_row_error(ref, ref) == 0.0
    assert oracle.max_rel_row_error(ref + [[0.02, 0], [0, 0]], ref) == pytest.approx(0.01)
    assert oracle.max_rel_row_error(ref + [[0, 0], [0, 1e-3]], ref) == float("inf")
    # no rows at all (a batch whose users have no new tokens)
    assert oracle.max_rel_row_error(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0
    with pytest.raises(ValueError):
        oracle.max_rel_row_error(np.zeros((1, 4)), np.zeros((0, 4)))


def test_max_err_vs_scale_hand_computed():
    g_ref = np.array([1.5, 2.0, 0.0, -4.0])
    g = np.array([1.0, 2.0, 0.0, -3.0])
    scale = np.array([2.0, 1.0, 0.0, 8.0])
    # entries: 0.5 / 2, 0 / 1, exact zero with zero scale, 1 / 8
    assert oracle.max_err_vs_scale(g, g_ref, scale) == 0.25
    assert oracle.max_err_vs_scale(g.reshape(2, 2), g_ref.reshape(2, 2), scale.reshape(2, 2)) == 0.25
    bad = g.copy()
    bad[2] = 1e-30                                      # nonzero where no term exists
    assert oracle.max_err_vs_scale(bad, g_ref, scale) == float("inf")
    assert oracle.max_err_vs_scale(np.zeros(0), np.zeros(0), np.zeros(0)) == 0.0


def test_max_rel_err_vs_magnitude_hand_computed():
    g_ref = np.array([[1.0, 1.0], [3.0, 3.0]])
    g = np.array([[1.0, 2.0], [3.0, 4.0]])
    mag = np.array([[2.0, 4.0], [1.0, 8.0]])
    # row 0: max |diff| 1 over max magnitude 4; row 1: 1 over 8
    assert oracle.max_rel_err_vs_magnitude(g, g_ref, mag) == 0.25
    # a 1-D input is one row: max |diff| 1 over max magnitude 8
    assert oracle.max_rel_err_vs_magnitude(g.reshape(-1), g_ref.reshape(-1), mag.reshape(-1)) == 0.125
    assert oracle.max_rel_err_vs_magnitude(g, g_ref, np.array([[0.0, 0.0], [1.0, 8.0]])) == float("inf")


def _count_pairs_from_oracle_masks(kind, lengths, extra):
    """Pairs the oracle's own masks allow, read off its pre-norm output.

    With q = k = 0, v = 1, no time table and a constant position table c,
    every allowed pair contributes SiLU(c) / N to each feature of its row's
    output, so row i's output times N / SiLU(c) is its number of keys.
    """
    c = 1.5
    sc = c / (1 + np.exp(-c))
    H, d = 1, 2
    ptab = np.full(4, c)
    if kind == "full":
        T = sum(lengths)
        off = np.concatenate([[0], np.cumsum(lengths)])
        z = np.zeros((T, H, d))
        _, o = oracle.hstu_full(z, z, np.ones((T, H, d)), np.ones((T, H * d)), np.arange(T), off, ptab, None,
                                norm_n=1)
    elif kind == "cached":
        new, cache = list(lengths), list(extra)
        M, K = sum(new), sum(a + b for a, b in zip(new, cache))
        noff = np.concatenate([[0], np.cumsum(new)])
        hoff = np.concatenate([[0], np.cumsum([a + b for a, b in zip(new, cache)])])
        _, o = oracle.hstu_cached(np.zeros((M, H, d)), np.ones((M, H * d)), np.arange(M), np.zeros((K, H, d)),
                                  np.ones((K, H, d)), np.arange(K), hoff, cache, noff, ptab, None, norm_n=1)
    else:
        hist, cand = list(lengths), list(extra)
        L = [a + b for a, b in zip(hist, cand)]
        T = sum(L)
        off = np.concatenate([[0], np.cumsum(L)])
        z = np.zeros((T, H, d))
        _, o = oracle.hstu_mfalcon(z, z, np.ones((T, H, d)), np.ones((T, H * d)), np.arange(T), off, cand, ptab,
                                   None, norm_n=1)
    per_row = np.asarray(o)[:, 0] / sc
    assert np.allclose(per_row, np.round(per_row))
    return int(round(per_row.sum()))


def test_pair_counts():
    assert oracle.pair_count("full", [8192] * 8) == 268_468_224
    assert oracle.pair_count("cached", [128] * 8, [8192] * 8) == 8 * (128 * 8192 + 128 * 129 // 2)
    assert oracle.pair_count("mfalcon", [4096] * 4, [1024] * 4) == 4 * (4096 * 4097 // 2 + 1024 * 4097)


@pytest.mark.parametrize("lengths", [[7], [0, 1, 5, 3], [2, 0]])
def test_pair_count_full_enumerated(lengths):
    # causal: every key at or before the query
    brute = sum(1 for L in lengths for i in range(L) for j in range(L) if j <= i)
    assert oracle.pair_count("full", lengths) == brute
    assert _count_pairs_from_oracle_masks("full", lengths, None) == brute


@pytest.mark.parametrize("new,cache", [([3], [5]), ([1, 4, 0], [0, 2, 6]), ([2, 2], [64, 1])])
def test_pair_count_cached_enumerated(new, cache):
    # new token m of a user with C cached tokens sits at position C + m and
    # sees keys 0 .. C + m of the C + M key sequence
    brute = sum(1 for M, C in zip(new, cache) for m in range(M) for j in range(C + M) if j <= C + m)
    assert oracle.pair_count("cached", new, cache) == brute
    assert _count_pairs_from_oracle_masks("cached", new, cache) == brute


@pytest.mark.parametrize("hist,cand", [([4], [3]), ([0, 3, 5], [2, 0, 1]), ([6, 1], [1, 4])])
def test_pair_count_mfalcon_enumerated(hist, cand):
    # history rows causal over the history; a candidate sees the whole
    # history and itself, never another candidate
    brute = 0
    for n, m in zip(hist, cand):
        for i in range(n + m):
            for j in range(n + m):
                if i < n:
                    brute += j <= i
                else:
                    brute += j < n or j == i
    assert oracle.pair_count("mfalcon", hist, cand) == brute
    assert _count_pairs_from_oracle_masks("mfalcon", hist, cand) == brute


def test_dense_matches_loops_and_split_order():
    rng = np.random.default_rng(5)
    a = rng.integers(-3, 4, size=(5, 4)).astype(np.float64)
    b = rng.integers(-3, 4, size=(4, 6)).astype(np.float64)
    ref = np.zeros((5, 6))
    for i in range(5):
        for j in range(6):
            ref[i, j] = sum(a[i, k] * b[k, j] for k in range(4))
    np.testing.assert_array_equal(oracle.dense(a, b), ref)
    blocks = oracle.dense(a, b, apply_silu=True, split_width=2)
    assert len(blocks) == 3
    for i, blk in enumerate(blocks):
        expect = [[x / (1 + math.exp(-x)) for x in row] for row in ref[:, 2 * i:2 * i + 2]]
        np.testing.assert_allclose(blk, expect, rtol=1e-15, atol=1e-300)


def test_time_bucket_edge_input_detects_a_shifted_edge(monkeypatch):
    """The GPU test on workloads.time_bucket_edges can see a kernel that puts
    pairs at a bucket's lower edge (|dt| = 2^b - 1, b >= 7: only in key tiles
    away from the diagonal) one bucket too low: planted in the oracle, that
    mistake moves the output by more than four times the bf16 bar."""
    inp = W.time_bucket_edges()
    args = (inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, inp.tables.pos, inp.tables.time)
    y_ok, _ = oracle.hstu_full(*args)
    right = oracle_hstu.time_bucket

    def shifted(dt, n_time):
        a = np.abs(np.asarray(dt, dtype=np.int64))
        b = right(dt, n_time)
        x = a + 1
        return np.where((a >= 64) & ((x & (x - 1)) == 0), b - 1, b)

    monkeypatch.setattr(oracle_hstu, "time_bucket", shifted)
    y_bad, _ = oracle.hstu_full(*args)
    assert oracle.max_rel_row_error(y_bad, y_ok) > 4 * TOL["bf16"]
