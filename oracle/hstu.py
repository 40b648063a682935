"""Plain fp64 CPU oracle for the HSTU attention layer (test infrastructure).

This module is test infrastructure. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the library never calls it. It
shares no code with the HIP path and imports nothing from it.

What is computed, and where the pages say so:

* Pointwise SiLU attention in place of softmax, plus a relative attention
  bias: "Generative recommenders at scale", section "Inside NVIDIA's
  GPU-native stack for HSTU and Semantic IDs"; "How Generative Recommenders
  Are Redefining RecSys at Scale", Takeaways (SiLU-based weighting, relative
  attention bias, elementwise gating before the output projection).
* Timestamp-ordered user sequences (position and time are the two relative
  quantities the bias depends on): same summary page, description.
* Causal next-action modelling over user histories of very different
  lengths: "Generative recommenders at scale", section "Inside NVIDIA's ...";
  "HSTU Generative Recommenders: Deploy on GPU Cloud", section "Scaling
  Training and Serving Across Multiple GPUs" (wildly variable lengths).
* Cached prefix, only new tokens computed: "Deploying an HSTU Generative
  Recommender with NVIDIA Dynamo-Triton", section "Technical Stack and
  Performance Gains"; page "recomendador-generativo-hstu-dynamo-triton",
  section "Como o recomendador generativo HSTU reutiliza o histórico" (paged
  GPU table with append).
* M-FALCON: candidates scored in one pass by changing the mask and the
  relative bias so the history computation is shared: "HSTU Generative
  Recommenders: Deploy on GPU Cloud", section "M-FALCON: Microbatched
  Attention for Scoring Multiple Candidates at Once".

The pages print no equation. The definition used here, per sequence b with
L_b tokens and head h, local indices 0 <= j <= i < L_b:

    s_ij = alpha * <q_i, k_j> + P[min(i - j, n_pos - 1)]
                              + T[min(floor(log2(|ts_i - ts_j| + 1)), n_time - 1)]
    a_ij = SiLU(s_ij) / N_b         (zero where the mask forbids (i, j))
    o_i  = sum_j a_ij v_j
    y_i  = (LayerNorm over the H*d values of token i)(o_i) * gamma + beta, times u_i

Readings where the pages are silent (each one is also listed in the design
notes): N_b is the per-sequence number of keys the sequence spans (L_b for the
full path, C_b + M_b when M_b new tokens follow a cached prefix of C_b, n_b + 1
for M-FALCON with history n_b); alpha = 1 unless given; the position bucket is
a linear clamp; the time bucket is the integer floor of log2(|dt| + 1) in
seconds, clamped; one table is shared by all heads unless a [H, n] table is
given; the mask is applied after SiLU (a_ij = 0, never -inf); the causal
diagonal is included; LayerNorm uses the population variance with eps = 1e-5
over all H*d values of a token, gamma = 1, beta = 0 unless given. Candidates
of M-FALCON sit at position n_b, attend to every history key and to themselves
(relative position 0, dt = 0) and to no other candidate.

Everything is evaluated in float64. Inputs that the GPU receives in bf16 are
already bf16 values here (the input generators round them), so both sides see
the same numbers.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "time_bucket", "pos_bucket", "silu", "layer_norm_gate",
    "hstu_full", "hstu_full_rows", "hstu_cached", "hstu_mfalcon",
    "kv_append_pages", "hstu_layer", "max_rel_row_error", "pair_count",
    "silu_grad", "layer_norm_gate_bwd", "hstu_full_bwd", "max_rel_err_vs_magnitude", "max_err_vs_scale",
    "dense",
]


# ----------------------------------------------------------------------------
# Buckets and the relative attention bias
# ----------------------------------------------------------------------------

def time_bucket(dt, n_time: int) -> np.ndarray:
    """min(floor(log2(|dt| + 1)), n_time - 1) for integer seconds dt.

    floor(log2(x)) for an integer x >= 1 is one less than its bit length. For
    x below 2**53 the float64 conversion is exact, and frexp returns x = m*2**e
    with m in [0.5, 1), so floor(log2(x)) = e - 1 exactly.
    """
    x = np.abs(np.asarray(dt, dtype=np.int64)) + 1
    if np.any(x >= (1 << 53)):
        raise ValueError("time difference too large for the exact bucket")
    _, e = np.frexp(x.astype(np.float64))
    return np.minimum(e.astype(np.int64) - 1, n_time - 1)


def pos_bucket(rel, n_pos: int) -> np.ndarray:
    """min(rel, n_pos - 1) for relative positions rel >= 0 (linear clamp)."""
    rel = np.asarray(rel, dtype=np.int64)
    return np.minimum(rel, n_pos - 1)


def _table_row(tab, h):
    if tab is None:
        return None
    tab = np.asarray(tab, dtype=np.float64)
    return tab if tab.ndim == 1 else tab[h]


def _bias(rel_pos, dt, pos_tab, time_tab, h):
    """Relative attention bias P[pos bucket] + T[time bucket] (0 for a missing table)."""
    b = np.zeros(np.shape(rel_pos), dtype=np.float64)
    p = _table_row(pos_tab, h)
    if p is not None:
        b = b + p[pos_bucket(rel_pos, len(p))]
    t = _table_row(time_tab, h)
    if t is not None:
        b = b + t[time_bucket(dt, len(t))]
    return b


def silu(x):
    """SiLU(x) = x / (1 + exp(-x)) in float64 (exp overflow gives the limit -0.0)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def layer_norm_gate(z, u, gamma=None, beta=None, eps=1e-5):
    """Per token: ((z - mean) / sqrt(var + eps) * gamma + beta) * u, over the last axis.

    The variance is the population variance. This is the Norm(AV) followed by
    the elementwise gating with U ("How Generative Recommenders Are Redefining
    RecSys at Scale", Takeaways: gating before the output projection).
    """
    z = np.asarray(z, dtype=np.float64)
    mu = z.mean(axis=-1, keepdims=True)
    var = ((z - mu) ** 2).mean(axis=-1, keepdims=True)
    n = (z - mu) / np.sqrt(var + eps)
    if gamma is not None:
        n = n * np.asarray(gamma, dtype=np.float64)
    if beta is not None:
        n = n + np.asarray(beta, dtype=np.float64)
    return n * np.asarray(u, dtype=np.float64)


# ----------------------------------------------------------------------------
# One (sequence, head) block of SiLU attention
# ----------------------------------------------------------------------------

def _attend(q, k, v, q_pos, k_pos, q_ts, k_ts, allowed, pos_tab, time_tab, h, alpha, n_norm):
    """o = (SiLU(alpha q k^T + bias) masked) / N @ v for one head.

    q [m, d], k and v [n, d]; positions and timestamps give the relative
    position (q_pos - k_pos) and time difference (q_ts - k_ts) of each pair;
    ``allowed`` [m, n] is the mask, applied after SiLU.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rel = np.asarray(q_pos, dtype=np.int64)[:, None] - np.asarray(k_pos, dtype=np.int64)[None, :]
    dt = np.asarray(q_ts, dtype=np.int64)[:, None] - np.asarray(k_ts, dtype=np.int64)[None, :]
    s = alpha * (q @ k.T)
    # the bias is only looked up where the pair is allowed (rel >= 0 there)
    relc = np.where(allowed, rel, 0)
    s = s + _bias(relc, dt, pos_tab, time_tab, h)
    a = np.where(allowed, silu(s), 0.0) / float(n_norm)
    return a @ v


def _heads(x):
    x = np.asarray(x)
    return x.shape[1], x.shape[2]


# ----------------------------------------------------------------------------
# Full causal path over jagged sequences
# ----------------------------------------------------------------------------

def hstu_full(q, k, v, u, ts, seq_offsets, pos_tab=None, time_tab=None, alpha=1.0, norm_n=0,
              gamma=None, beta=None, eps=1e-5):
    """Causal HSTU attention over packed jagged sequences, then LayerNorm and U gating.

    q, k, v: [T, H, d]; u: [T, H*d]; ts: int64 [T]; seq_offsets: [B+1].
    Returns (y [T, H*d], o [T, H*d]) in float64, o being the attention output
    before the norm.
    """
    H, d = _heads(q)
    T = q.shape[0]
    off = np.asarray(seq_offsets, dtype=np.int64)
    o = np.zeros((T, H, d), dtype=np.float64)
    for b in range(len(off) - 1):
        s0, s1 = int(off[b]), int(off[b + 1])
        L = s1 - s0
        if L == 0:
            continue
        pos = np.arange(L)
        allowed = pos[None, :] <= pos[:, None]
        n_norm = norm_n if norm_n > 0 else L
        t = ts[s0:s1]
        for h in range(H):
            o[s0:s1, h] = _attend(q[s0:s1, h], k[s0:s1, h], v[s0:s1, h], pos, pos, t, t, allowed,
                                  pos_tab, time_tab, h, alpha, n_norm)
    o = o.reshape(T, H * d)
    return layer_norm_gate(o, u, gamma, beta, eps), o


def hstu_full_rows(rows, q, k, v, u, ts, seq_offsets, pos_tab=None, time_tab=None, alpha=1.0,
                   norm_n=0, gamma=None, beta=None, eps=1e-5):
    """The full path evaluated only at the given packed token rows.

    Row i of sequence b needs keys 0..i of b only, so a sample of rows of a
    large batch costs O(rows * L * H * d). Returns y for those rows.
    """
    H, d = _heads(q)
    off = np.asarray(seq_offsets, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), H * d), dtype=np.float64)
    seq_of = np.searchsorted(off, rows, side="right") - 1
    for r, (t, b) in enumerate(zip(rows, seq_of)):
        s0, s1 = int(off[b]), int(off[b + 1])
        i = int(t) - s0
        L = s1 - s0
        n_norm = norm_n if norm_n > 0 else L
        kpos = np.arange(i + 1)
        allowed = np.ones((1, i + 1), dtype=bool)
        z = np.zeros((H, d))
        for h in range(H):
            z[h] = _attend(q[t:t + 1, h], k[s0:s0 + i + 1, h], v[s0:s0 + i + 1, h], [i], kpos,
                           ts[t:t + 1], ts[s0:s0 + i + 1], allowed, pos_tab, time_tab, h, alpha, n_norm)[0]
        out[r] = layer_norm_gate(z.reshape(1, -1), u[t:t + 1], gamma, beta, eps)[0]
    return out


# ----------------------------------------------------------------------------
# KV-cache delta path
# ----------------------------------------------------------------------------

def hstu_cached(q_new, u_new, ts_new, k_hist, v_hist, ts_hist, hist_offsets, cache_lens,
                new_offsets, pos_tab=None, time_tab=None, alpha=1.0, norm_n=0,
                gamma=None, beta=None, eps=1e-5):
    """New tokens attend causally to the cached prefix and to the new tokens.

    Per user b the logical key sequence (k_hist, v_hist, ts_hist rows
    hist_offsets[b] .. hist_offsets[b+1]) has C_b + M_b tokens: the C_b cached
    prefix tokens followed by the M_b new ones (already appended). Query m of
    user b (packed row new_offsets[b] + m) sits at position C_b + m and attends
    to keys 0 .. C_b + m. N_b = C_b + M_b.
    Returns (y_new [M, H*d], o_new [M, H*d]).
    """
    H, d = _heads(q_new)
    M = q_new.shape[0]
    hoff = np.asarray(hist_offsets, dtype=np.int64)
    noff = np.asarray(new_offsets, dtype=np.int64)
    o = np.zeros((M, H, d), dtype=np.float64)
    for b in range(len(noff) - 1):
        m0, m1 = int(noff[b]), int(noff[b + 1])
        Mb = m1 - m0
        if Mb == 0:
            continue
        C = int(cache_lens[b])
        h0, h1 = int(hoff[b]), int(hoff[b + 1])
        if h1 - h0 != C + Mb:
            raise ValueError("history length must equal cache_len + new tokens")
        qpos = C + np.arange(Mb)
        kpos = np.arange(C + Mb)
        allowed = kpos[None, :] <= qpos[:, None]
        n_norm = norm_n if norm_n > 0 else C + Mb
        for h in range(H):
            o[m0:m1, h] = _attend(q_new[m0:m1, h], k_hist[h0:h1, h], v_hist[h0:h1, h], qpos, kpos,
                                  ts_new[m0:m1], ts_hist[h0:h1], allowed, pos_tab, time_tab, h, alpha, n_norm)
    o = o.reshape(M, H * d)
    return layer_norm_gate(o, u_new, gamma, beta, eps), o


def kv_append_pages(k_pages, v_pages, ts_pages, page_table, cache_lens, new_offsets, k_new, v_new,
                    ts_new, page_size=64):
    """Paged KV append: new token m of user b lands at logical position C_b + m.

    That position lives in page page_table[b, (C_b + m) // page_size] at slot
    (C_b + m) % page_size. Pages are [num_pages, H, page_size, d] for K and V
    and [num_pages, page_size] for timestamps. Returns updated copies.
    Page-table operations are named in "recomendador-generativo-hstu-dynamo-
    triton", section "Como o recomendador generativo HSTU reutiliza o histórico".
    """
    k_pages = np.array(k_pages, copy=True)
    v_pages = np.array(v_pages, copy=True)
    ts_pages = np.array(ts_pages, copy=True)
    noff = np.asarray(new_offsets, dtype=np.int64)
    for b in range(len(noff) - 1):
        for t in range(int(noff[b]), int(noff[b + 1])):
            p = int(cache_lens[b]) + (t - int(noff[b]))
            page = int(page_table[b, p // page_size])
            if page < 0:
                raise ValueError("token position has no page")
            slot = p % page_size
            k_pages[page, :, slot, :] = k_new[t]
            v_pages[page, :, slot, :] = v_new[t]
            ts_pages[page, slot] = ts_new[t]
    return k_pages, v_pages, ts_pages


# ----------------------------------------------------------------------------
# M-FALCON candidate path
# ----------------------------------------------------------------------------

def hstu_mfalcon(q, k, v, u, ts, seq_offsets, num_candidates, pos_tab=None, time_tab=None, alpha=1.0,
                 norm_n=0, gamma=None, beta=None, eps=1e-5):
    """History rows causal over the history; each candidate attends to the history and itself.

    User b spans [history (n_b) | candidates (m_b = num_candidates[b])]. A
    candidate sits at position n_b: key j < n_b has relative position n_b - j
    and time difference ts_c - ts_j; its own key has relative position 0 and
    time difference 0. Candidates do not see each other. N_b = n_b + 1.
    Returns (y [T, H*d], o [T, H*d]).
    """
    H, d = _heads(q)
    T = q.shape[0]
    off = np.asarray(seq_offsets, dtype=np.int64)
    o = np.zeros((T, H, d), dtype=np.float64)
    for b in range(len(off) - 1):
        s0, s1 = int(off[b]), int(off[b + 1])
        L = s1 - s0
        m = int(num_candidates[b])
        n = L - m
        if n < 0:
            raise ValueError("more candidates than tokens")
        n_norm = norm_n if norm_n > 0 else n + 1
        if n > 0:
            hp = np.arange(n)
            allowed = hp[None, :] <= hp[:, None]
            th = ts[s0:s0 + n]
            for h in range(H):
                o[s0:s0 + n, h] = _attend(q[s0:s0 + n, h], k[s0:s0 + n, h], v[s0:s0 + n, h], hp, hp,
                                          th, th, allowed, pos_tab, time_tab, h, alpha, n_norm)
        for c in range(s0 + n, s1):
            # keys: history 0..n-1 at positions 0..n-1, then the candidate itself at position n
            kidx = np.concatenate([np.arange(s0, s0 + n), [c]])
            kpos = np.concatenate([np.arange(n), [n]])
            allowed = np.ones((1, n + 1), dtype=bool)
            for h in range(H):
                o[c, h] = _attend(q[c:c + 1, h], k[kidx, h], v[kidx, h], [n], kpos, ts[c:c + 1], ts[kidx],
                                  allowed, pos_tab, time_tab, h, alpha, n_norm)[0]
    o = o.reshape(T, H * d)
    return layer_norm_gate(o, u, gamma, beta, eps), o


# ----------------------------------------------------------------------------
# Full HSTU layer around the attention
# ----------------------------------------------------------------------------

def dense(a, b, apply_silu=False, split_width=None):
    """One of the layer's dense products: a @ b in float64, then SiLU if asked
    (f1 is SiLU(X W1), f2 is a plain product; "How Generative Recommenders Are
    Redefining RecSys at Scale", Takeaways). With split_width w the columns
    are returned as the list of blocks [i*w, (i+1)*w) (U, V, Q, K for f1)."""
    c = np.asarray(a, dtype=np.float64) @ np.asarray(b, dtype=np.float64)
    if apply_silu:
        c = silu(c)
    if split_width is None:
        return c
    return [c[:, i:i + split_width] for i in range(0, c.shape[1], split_width)]


def hstu_layer(x, w1, w2, ts, seq_offsets, num_heads, head_dim, pos_tab=None, time_tab=None, alpha=1.0,
               gamma=None, beta=None, eps=1e-5, rows=None):
    """f2(Norm(A V) * U) with U, V, Q, K = split(SiLU(f1(X))).

    f1 and f2 are plain matrix products with no bias; the f1 output is split,
    in this order, into U, V, Q, K of width H*d each ("How Generative
    Recommenders Are Redefining RecSys at Scale", Takeaways: gating before the
    output projection). If ``rows`` is given only those packed rows of the
    output are computed (their sequences' f1 outputs are still needed).
    """
    x = np.asarray(x, dtype=np.float64)
    hd = num_heads * head_dim
    off = np.asarray(seq_offsets, dtype=np.int64)
    if rows is None:
        f1 = silu(x @ np.asarray(w1, dtype=np.float64))
        u, vv, qq, kk = (f1[:, i * hd:(i + 1) * hd] for i in range(4))
        T = x.shape[0]
        sh = (T, num_heads, head_dim)
        y, _ = hstu_full(qq.reshape(sh), kk.reshape(sh), vv.reshape(sh), u, ts, off, pos_tab, time_tab,
                         alpha, 0, gamma, beta, eps)
        return y @ np.asarray(w2, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    seq_of = np.searchsorted(off, rows, side="right") - 1
    out = np.zeros((len(rows), np.asarray(w2).shape[1]))
    w1d = np.asarray(w1, dtype=np.float64)
    for b in np.unique(seq_of):
        s0, s1 = int(off[b]), int(off[b + 1])
        sel = np.nonzero(seq_of == b)[0]
        last = int(rows[sel].max()) + 1
        f1 = silu(x[s0:last] @ w1d)
        u, vv, qq, kk = (f1[:, i * hd:(i + 1) * hd] for i in range(4))
        sh = (last - s0, num_heads, head_dim)
        # rows of a causal sequence only need its first (row + 1) tokens; the
        # sequence length still sets N, passed here as norm_n.
        y = hstu_full_rows(rows[sel] - s0, qq.reshape(sh), kk.reshape(sh), vv.reshape(sh), u,
                           ts[s0:last], np.array([0, last - s0]), pos_tab, time_tab, alpha, s1 - s0,
                           gamma, beta, eps)
        out[sel] = y @ np.asarray(w2, dtype=np.float64)
    return out


# ----------------------------------------------------------------------------
# Backward of the full causal path (training)
# ----------------------------------------------------------------------------
#
# Training is the pages' other workload ("HSTU Generative Recommenders: Deploy
# on GPU Cloud", section "Scaling Training and Serving Across Multiple GPUs";
# "Generative recommenders at scale", section "Inside NVIDIA's GPU-native stack
# for HSTU and Semantic IDs": model FLOP utilisation of HSTU training). The
# pages print no backward formula; the gradients below are the chain rule of
# the forward definition at the top of this module, written out step by step.

def silu_grad(x):
    """d SiLU(x) / dx = sigma(x) * (1 + x * (1 - sigma(x))) in float64."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        sg = 1.0 / (1.0 + np.exp(-x))
    return sg * (1.0 + x * (1.0 - sg))


def layer_norm_gate_bwd(z, u, dy, gamma=None, beta=None, eps=1e-5):
    """Gradients of y = ((z - mean) / sqrt(var + eps) * gamma + beta) * u, per token.

    Returns (dz, du, dgamma, dbeta); dgamma and dbeta are None when gamma or
    beta is None. With n = (z - mean) * r, r = 1 / sqrt(var + eps) and
    g = dy * u * gamma (the gradient reaching n), the population-variance
    normalisation gives dz = r * (g - mean(g) - n * mean(g * n)).
    """
    z = np.asarray(z, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    mu = z.mean(axis=-1, keepdims=True)
    var = ((z - mu) ** 2).mean(axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(var + eps)
    n = (z - mu) * r
    gam = np.ones(z.shape[-1]) if gamma is None else np.asarray(gamma, dtype=np.float64)
    bet = np.zeros(z.shape[-1]) if beta is None else np.asarray(beta, dtype=np.float64)
    du = dy * (n * gam + bet)
    dn_aff = dy * u                       # gradient reaching n * gamma + beta
    dgamma = None if gamma is None else (dn_aff * n).sum(axis=0)
    dbeta = None if beta is None else dn_aff.sum(axis=0)
    g = dn_aff * gam
    dz = r * (g - g.mean(axis=-1, keepdims=True) - n * (g * n).mean(axis=-1, keepdims=True))
    return dz, du, dgamma, dbeta


def hstu_full_bwd(q, k, v, u, ts, seq_offsets, dy, pos_tab=None, time_tab=None, alpha=1.0, norm_n=0,
                  gamma=None, beta=None, eps=1e-5, magnitudes=False, pair_mask=None):
    """Gradients of the full causal path (hstu_full) for an upstream gradient dy [T, H*d].

    Per sequence and head, with s = alpha q k^T + bias, a = SiLU(s) / N on
    allowed pairs and o = a v:
        da = do v^T,   dv = a^T do,
        ds = da * SiLU'(s) / N on allowed pairs (0 elsewhere),
        dq = alpha ds k,   dk = alpha ds^T q,
        dP[c] = sum of ds over pairs whose position bucket is c,
        dT[c] = sum of ds over pairs whose time bucket is c,
    a shared (1-D) table summing over heads, a per-head ([H, n]) table per row.
    The norm and gating gradients come from layer_norm_gate_bwd.
    Returns a dict with dq, dk, dv ([T, H, d]), du ([T, H*d]), dpos, dtime
    (shaped like the tables, None without one), dgamma, dbeta.

    With magnitudes=True the dict also holds, under "mag_<name>", the same
    sums taken over absolute values (|do| |v|^T for da, |da| |SiLU'| / N for
    ds, and so on): the scale against which rounding errors of the summed
    terms are measured (a gradient that is small only by cancellation has a
    large magnitude). It also holds, under "rss_<name>" for dq, dk, dv, dpos
    and dtime, the root-sum-square of the terms: every gradient entry written
    out as one sum of products of leaf factors (dq_ic = alpha / N * sum over
    keys j and features e of SiLU'(s_ij) do_ie v_je k_jc; dv_jc = sum over i
    of a_ij do_ic; a table entry = sum over its pairs and features of
    SiLU'(s_ij) do_ie v_je / N; and each do_ie itself written out as the
    terms of the norm's backward, r (g_e - mean g - n_e mean(g n)) with
    g = dY u gamma), with each term squared, the squares added, and the
    root taken. Independent relative rounding errors of size eps per
    term give an error whose spread is about eps times this scale, whatever
    the signs, so it is the natural unit for a rounding error; a term that
    is missing altogether costs about its own size, which on random data is
    the scale itself.

    pair_mask, when given, is called as pair_mask(b, allowed) for sequence b
    and returns the pairs the gradient sums keep (a subset of ``allowed``);
    the recomputed forward is not affected. Tests use it to show what a
    backward that skips pairs (one key tile, say) would return.
    """
    H, d = _heads(q)
    T = q.shape[0]
    off = np.asarray(seq_offsets, dtype=np.int64)
    _, o = hstu_full(q, k, v, u, ts, off, pos_tab, time_tab, alpha, norm_n, gamma, beta, eps)
    do, du, dgamma, dbeta = layer_norm_gate_bwd(o, u, dy, gamma, beta, eps)
    do = do.reshape(T, H, d)
    dq = np.zeros((T, H, d))
    dk = np.zeros((T, H, d))
    dv = np.zeros((T, H, d))
    dpos = None if pos_tab is None else np.zeros(np.shape(pos_tab))
    dtime = None if time_tab is None else np.zeros(np.shape(time_tab))
    mag = {}
    do_r2 = None
    if magnitudes:
        # dO written out as the terms of the norm's backward, r (g_c - mean_e
        # g_e - n_c mean_e g_e n_e) with g = dY u gamma: the sum of their
        # squares stands for dO^2 in the root-sum-square of everything
        # downstream (dO's own size can be small by cancellation while its
        # terms, and any error they carry, are not)
        z = np.asarray(o, dtype=np.float64)
        D = z.shape[-1]
        mu = z.mean(axis=-1, keepdims=True)
        rr = 1.0 / np.sqrt(((z - mu) ** 2).mean(axis=-1, keepdims=True) + eps)
        nn = (z - mu) * rr
        gg = np.asarray(dy, dtype=np.float64) * np.asarray(u, dtype=np.float64)
        if gamma is not None:
            gg = gg * np.asarray(gamma, dtype=np.float64)
        do_r2 = (rr ** 2 * (gg ** 2 + (gg ** 2).sum(axis=-1, keepdims=True) / D ** 2
                            + nn ** 2 * ((gg * nn) ** 2).sum(axis=-1, keepdims=True) / D ** 2)).reshape(T, H, d)
        mag = {"mag_dq": np.zeros((T, H, d)), "mag_dk": np.zeros((T, H, d)), "mag_dv": np.zeros((T, H, d)),
               "mag_du": np.abs(du),
               "mag_dpos": None if dpos is None else np.zeros_like(dpos),
               "mag_dtime": None if dtime is None else np.zeros_like(dtime)}
        mag.update({"rss_dq": np.zeros((T, H, d)), "rss_dk": np.zeros((T, H, d)), "rss_dv": np.zeros((T, H, d)),
                    "rss_dpos": None if dpos is None else np.zeros_like(dpos),
                    "rss_dtime": None if dtime is None else np.zeros_like(dtime)})
        if dgamma is not None or dbeta is not None:
            z = np.asarray(o, dtype=np.float64)
            mu = z.mean(axis=-1, keepdims=True)
            nrm = (z - mu) / np.sqrt(((z - mu) ** 2).mean(axis=-1, keepdims=True) + eps)
            gu = np.abs(np.asarray(dy, dtype=np.float64) * np.asarray(u, dtype=np.float64))
            mag["mag_dgamma"] = None if dgamma is None else (gu * np.abs(nrm)).sum(axis=0)
            mag["mag_dbeta"] = None if dbeta is None else gu.sum(axis=0)
    for b in range(len(off) - 1):
        s0, s1 = int(off[b]), int(off[b + 1])
        L = s1 - s0
        if L == 0:
            continue
        pos = np.arange(L)
        allowed = pos[None, :] <= pos[:, None]
        n_norm = norm_n if norm_n > 0 else L
        rel = np.where(allowed, pos[:, None] - pos[None, :], 0)
        kept = allowed if pair_mask is None else (np.asarray(pair_mask(b, allowed.copy()), dtype=bool) & allowed)
        t = np.asarray(ts[s0:s1], dtype=np.int64)
        dt = t[:, None] - t[None, :]
        for h in range(H):
            qh = np.asarray(q[s0:s1, h], dtype=np.float64)
            kh = np.asarray(k[s0:s1, h], dtype=np.float64)
            vh = np.asarray(v[s0:s1, h], dtype=np.float64)
            s = alpha * (qh @ kh.T) + _bias(rel, dt, pos_tab, time_tab, h)
            a = np.where(allowed, silu(s), 0.0) / float(n_norm)
            doh = do[s0:s1, h]
            dv[s0:s1, h] = a.T @ doh
            da = doh @ vh.T
            ds = np.where(kept, da * silu_grad(s), 0.0) / float(n_norm)
            if pair_mask is not None:
                dv[s0:s1, h] = np.where(kept, a, 0.0).T @ doh
            dq[s0:s1, h] = alpha * (ds @ kh)
            dk[s0:s1, h] = alpha * (ds.T @ qh)
            if dpos is not None:
                row = dpos if dpos.ndim == 1 else dpos[h]
                np.add.at(row, pos_bucket(rel[kept], row.shape[0]), ds[kept])
            if dtime is not None:
                row = dtime if dtime.ndim == 1 else dtime[h]
                np.add.at(row, time_bucket(dt[kept], row.shape[0]), ds[kept])
            if magnitudes:
                ds_m = np.where(allowed, (np.abs(doh) @ np.abs(vh).T) * np.abs(silu_grad(s)), 0.0) / float(n_norm)
                mag["mag_dq"][s0:s1, h] = abs(alpha) * (ds_m @ np.abs(kh))
                mag["mag_dk"][s0:s1, h] = abs(alpha) * (ds_m.T @ np.abs(qh))
                mag["mag_dv"][s0:s1, h] = np.abs(a).T @ np.abs(doh)
                # squared root-sum-square of the terms of each ds_ij, then of
                # each gradient entry (sums of squares of the same terms)
                dor2 = do_r2[s0:s1, h]
                ds_r2 = np.where(allowed, (dor2 @ (vh ** 2).T) * silu_grad(s) ** 2, 0.0) / float(n_norm) ** 2
                mag["rss_dq"][s0:s1, h] = abs(alpha) * np.sqrt(ds_r2 @ kh ** 2)
                mag["rss_dk"][s0:s1, h] = abs(alpha) * np.sqrt(ds_r2.T @ qh ** 2)
                mag["rss_dv"][s0:s1, h] = np.sqrt((a ** 2).T @ dor2)
                for key, rel_or_dt, fn, w in (("mag_dpos", rel, pos_bucket, ds_m), ("mag_dtime", dt, time_bucket, ds_m),
                                              ("rss_dpos", rel, pos_bucket, ds_r2),
                                              ("rss_dtime", dt, time_bucket, ds_r2)):
                    if mag[key] is not None:
                        row = mag[key] if mag[key].ndim == 1 else mag[key][h]
                        np.add.at(row, fn(rel_or_dt[allowed], row.shape[0]), w[allowed])
    for key in ("rss_dpos", "rss_dtime"):  # sums of squares so far
        if mag.get(key) is not None:
            mag[key] = np.sqrt(mag[key])
    out = {"dq": dq, "dk": dk, "dv": dv, "du": du, "dpos": dpos, "dtime": dtime,
           "dgamma": dgamma, "dbeta": dbeta}
    out.update(mag)
    return out


# ----------------------------------------------------------------------------
# Comparison metric and work count
# ----------------------------------------------------------------------------

def max_rel_row_error(y, y_ref, zero_row_atol=1e-6):
    """max over rows t of ||y_t - y*_t||_inf / ||y*_t||_inf.

    Elementwise relative error is ill-posed because outputs cross zero; rows
    whose reference is identically zero must instead satisfy
    ||y_t||_inf <= zero_row_atol (reported as inf otherwise).
    """
    y_ref = np.asarray(y_ref, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if y_ref.size == 0:
        if y.size != 0:
            raise ValueError("output has values where the reference has none")
        return 0.0
    y = y.reshape(len(y_ref), -1)
    y_ref = y_ref.reshape(len(y_ref), -1)
    num = np.abs(y - y_ref).max(axis=1)
    den = np.abs(y_ref).max(axis=1)
    zero = den == 0
    err = np.where(zero, 0.0, num / np.where(zero, 1.0, den))
    if np.any(zero & (np.abs(y).max(axis=1) > zero_row_atol)):
        return float("inf")
    return float(err.max())


def max_rel_err_vs_magnitude(g, g_ref, mag):
    """max over rows t of ||g_t - g*_t||_inf / ||mag_t||_inf.

    mag is the same sum as g* over absolute values of the terms, so this is
    the error relative to the size of what was added up; it stays meaningful
    for a row whose gradient is small through cancellation. A 1-D input is
    one row. Rows whose magnitude is zero must match exactly (else inf).
    """
    g = np.asarray(g, dtype=np.float64)
    g_ref = np.asarray(g_ref, dtype=np.float64)
    mag = np.asarray(mag, dtype=np.float64)
    n = len(g_ref) if g_ref.ndim > 1 else 1
    g, g_ref, mag = (x.reshape(n, -1) for x in (g, g_ref, mag))
    num = np.abs(g - g_ref).max(axis=1)
    den = mag.max(axis=1)
    zero = den == 0
    if np.any(zero & (num > 0)):
        return float("inf")
    return float(np.where(zero, 0.0, num / np.where(zero, 1.0, den)).max()) if n else 0.0


def max_err_vs_scale(g, g_ref, scale):
    """max over entries of |g - g*| / scale, entry by entry.

    scale has g*'s shape (the root-sum-square of each entry's terms, say).
    Entries whose scale is zero are sums of no terms and must be exactly zero
    in g as well (else inf). Empty inputs give 0.
    """
    g = np.asarray(g, dtype=np.float64).reshape(-1)
    g_ref = np.asarray(g_ref, dtype=np.float64).reshape(-1)
    scale = np.asarray(scale, dtype=np.float64).reshape(-1)
    if g_ref.size == 0:
        return 0.0
    err = np.abs(g - g_ref)
    zero = scale == 0
    if np.any(zero & (err > 0)):
        return float("inf")
    return float(np.where(zero, 0.0, err / np.where(zero, 1.0, scale)).max())


def pair_count(kind, lengths, extra=None):
    """Number of allowed (query, key) pairs, the unit of algorithmic work.

    full: sum L(L+1)/2; cached (extra = cache_lens, lengths = new lengths):
    sum over new rows of the keys they see; mfalcon (lengths = history,
    extra = candidates): n(n+1)/2 + m(n+1).
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    if kind == "full":
        return int(np.sum(lengths * (lengths + 1) // 2))
    if kind == "cached":
        C = np.asarray(extra, dtype=np.int64)
        M = lengths
        return int(np.sum(M * C + M * (M + 1) // 2))
    if kind == "mfalcon":
        n = lengths
        m = np.asarray(extra, dtype=np.int64)
        return int(np.sum(n * (n + 1) // 2 + m * (n + 1)))
    raise ValueError(kind)
