"""GPU parity: the HIP library against the fp64 oracle on the same seeded inputs.

Bar: max over token rows of ||y - y*||_inf / ||y*||_inf within 1e-4 (fp32)
and 2e-2 (bf16). The bf16 bound covers bf16 rounding of the SiLU weights
before the second product, fp32 accumulation over up to 8,192 keys and the
bf16 rounding of the output (2^-9 relative); measured errors are far below it.
Integer work (paged append) is compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from devutil import TOL, dev, params_for, run_full, tdtype, to_np

hs = pytest.importorskip("hstu_jagged_silu_amd")
pytestmark = pytest.mark.gpu


def oracle_full(inp, **kw):
    y, _ = oracle.hstu_full(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, inp.tables.pos,
                            inp.tables.time, **kw)
    return y


def check(y_gpu, y_ref, dtype, what=""):
    err = oracle.max_rel_row_error(to_np(y_gpu), y_ref)
    print(f"{what} max row rel err {err:.3e}")
    assert err <= TOL[dtype], f"{what}: {err}"
    return err


# ---------------------------------------------------------------- full path

def test_tiny_fp32_full():
    inp = W.tiny_fp32()
    check(run_full(inp), oracle_full(inp), "f32", "tiny fp32")


def test_training_shape_bf16_full():
    inp = W.training_shape()
    check(run_full(inp), oracle_full(inp), "bf16", "jagged B32 bf16")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("bf16", 32), ("f32", 32), ("f32", 64),
                                     ("f32", 128)])
def test_ragged_edge_lengths(dtype, d):
    lengths = [0, 1, 2, 63, 64, 65, 127, 128, 129, 200, 0, 257]
    inp = W.jagged(f"edge_{dtype}_{d}", 70 + d, lengths, 2, d, dtype, 128, 128)
    check(run_full(inp), oracle_full(inp), dtype, f"ragged {dtype} d={d}")


def test_per_head_tables_alpha_norm_affine():
    inp = W.jagged("opts", 77, [150, 33, 260], 3, 64, "bf16", 0, 0)
    rng = np.random.default_rng(5)
    pos = (rng.standard_normal((3, 40)) * 0.5).astype(np.float32)
    tim = (rng.standard_normal((3, 20)) * 0.5).astype(np.float32)
    lw = (1 + 0.1 * rng.standard_normal(192)).astype(np.float32)
    lb = (0.1 * rng.standard_normal(192)).astype(np.float32)
    p = hs.LayerParams(num_heads=3, head_dim=64, dtype=torch.bfloat16, alpha=0.25, norm_n=100,
                       pos_tab=dev(pos), time_tab=dev(tim), ln_w=dev(lw), ln_b=dev(lb), ln_eps=1e-3)
    y = run_full(inp, params=p)
    y_ref, _ = oracle.hstu_full(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, pos, tim, alpha=0.25,
                                norm_n=100, gamma=lw, beta=lb, eps=1e-3)
    check(y, y_ref, "bf16", "per-head tables, alpha, fixed N, affine")


def test_no_tables_and_position_only():
    for n_pos, n_time in ((0, 0), (64, 0), (0, 64)):
        inp = W.jagged("tabs", 80 + n_pos + n_time, [100, 300], 2, 128, "bf16", n_pos, n_time)
        check(run_full(inp), oracle_full(inp), "bf16", f"tables pos={n_pos} time={n_time}")


def test_unordered_and_huge_timestamps():
    """Timestamps out of order (the |dt| path) and gaps beyond 2^31 s (the 64-bit path)."""
    inp = W.jagged("ts", 81, [300, 190], 2, 64, "bf16", 32, 64)
    rng = np.random.default_rng(3)
    inp.ts = rng.permutation(inp.ts)
    check(run_full(inp), oracle_full(inp), "bf16", "shuffled ts")
    inp.ts = (np.arange(inp.total, dtype=np.int64) * (3 << 29)) + 1_700_000_000
    inp.ts[::7] -= 1 << 40
    check(run_full(inp), oracle_full(inp), "bf16", "huge ts")


def test_time_bucket_edges_unit_gap():
    """Timestamps one second apart: |dt| is the distance, so every row has
    pairs exactly at a time bucket's lower edge 2^b - 1, most of them in key
    tiles that span two buckets (the threshold path of the kernel); the time
    table is scaled so that a pair in the wrong bucket shows (a CPU pin
    plants that mistake in the oracle and sees it)."""
    inp = W.time_bucket_edges()
    check(run_full(inp), oracle_full(inp), "bf16", "time bucket edges")


def test_maximum_sizes_sampled_rows():
    """The largest supported shapes: H*d = 2,048 (16 heads of 128), a 2,048-entry
    position table, 64 time buckets, users longer than the position table."""
    inp = W.jagged("max", 99, [3000, 2500, 40], 16, 128, "bf16", 2048, 64)
    inp.tables.pos *= 25.0   # large enough to move the outputs (the draws have variance 0.02)
    y = to_np(run_full(inp))
    rng = np.random.default_rng(10)
    rows = np.unique(np.concatenate([[0, 2046, 2047, 2048, 2999, 3000, 5047, 5048, 5499, 5500, 5539],
                                     rng.integers(0, inp.total, size=30)]))
    y_ref = oracle.hstu_full_rows(rows, inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, inp.tables.pos,
                                  inp.tables.time)
    err = oracle.max_rel_row_error(y[rows], y_ref)
    print(f"maximum sizes sampled rows max row rel err {err:.3e}")
    assert err <= TOL["bf16"]
    assert np.isfinite(y).all()


def test_long_sequences_sampled_rows():
    """8 users x 8,192 tokens, 4 x 128, bf16 (the benchmark's workload): sampled rows."""
    inp = W.long_seq()
    y = to_np(run_full(inp))
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([
        [0, 1, 127, 128, 8191, 8192, 65535, 4096 + 8192 * 3],
        rng.integers(0, inp.total, size=40)]))
    y_ref = oracle.hstu_full_rows(rows, inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, inp.tables.pos,
                                  inp.tables.time)
    err = oracle.max_rel_row_error(y[rows], y_ref)
    print(f"8x8192 sampled rows max row rel err {err:.3e}")
    assert err <= TOL["bf16"]
    assert np.isfinite(y).all()


def test_long_sequences_one_whole_user():
    """8 users x 8,192 tokens, 4 x 128, bf16 (the benchmark's workload, in the
    benchmark's launch): every row and head of the last user against the
    oracle run on that user alone (users are independent: a jagged batch
    equals per-user runs)."""
    inp = W.long_seq()
    y = to_np(run_full(inp))
    b = len(inp.seq_offsets) - 2
    s0, s1 = int(inp.seq_offsets[b]), int(inp.seq_offsets[b + 1])
    assert s1 - s0 == 8192
    print(f"user {b}: rows {s0} .. {s1 - 1}, running the oracle on the whole user", flush=True)
    y_ref, _ = oracle.hstu_full(inp.q[s0:s1], inp.k[s0:s1], inp.v[s0:s1], inp.u[s0:s1], inp.ts[s0:s1],
                                np.array([0, s1 - s0]), inp.tables.pos, inp.tables.time)
    err = oracle.max_rel_row_error(y[s0:s1], y_ref)
    print(f"8x8192 whole user {b} (8,192 rows x 4 heads) max row rel err {err:.3e}")
    assert err <= TOL["bf16"]
    assert np.isfinite(y).all()


def test_more_than_4096_items_sampled_rows():
    """64 users x 8 heads: 4,608 work items, more than the scheduler keeps in
    registers between its histogram and scatter passes (the rest are rebuilt)."""
    rng = np.random.default_rng(133)
    lengths = [int(x) for x in rng.integers(1025, 1153, size=64)]   # 9 query tiles each
    inp = W.jagged("many_items", 133, lengths, 8, 64, "bf16", 128, 128)
    assert sum(8 * ((L + 127) // 128) for L in lengths) > 4096
    y = to_np(run_full(inp))
    rows = np.unique(np.concatenate([[0, inp.total - 1], rng.integers(0, inp.total, size=40)]))
    y_ref = oracle.hstu_full_rows(rows, inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, inp.tables.pos,
                                  inp.tables.time)
    err = oracle.max_rel_row_error(y[rows], y_ref)
    print(f"4,608 items sampled rows max row rel err {err:.3e}")
    assert err <= TOL["bf16"]
    assert np.isfinite(y).all()


# ---------------------------------------------------------------- invariants

def test_jagged_batch_equals_per_sequence_bitwise():
    inp = W.jagged("inv", 90, [300, 1, 129], 2, 128, "bf16", 128, 128)
    y = to_np(run_full(inp))
    for b in range(inp.batch):
        s0, s1 = int(inp.seq_offsets[b]), int(inp.seq_offsets[b + 1])
        one = W.JaggedInputs("one", "bf16", 2, 128, inp.lengths[b:b + 1], np.array([0, s1 - s0], np.int32),
                             inp.ts[s0:s1], inp.q[s0:s1], inp.k[s0:s1], inp.v[s0:s1], inp.u[s0:s1], inp.tables)
        assert np.array_equal(to_np(run_full(one)), y[s0:s1])


def test_causality_bitwise():
    inp = W.jagged("caus", 91, [500], 2, 128, "bf16", 128, 128)
    p = params_for("bf16", 2, 128, inp.tables, norm_n=500)
    y = to_np(run_full(inp, params=p))
    i = 200
    inp.q[i + 1:] = -inp.q[i + 1:]
    inp.k[i + 1:] *= 2
    inp.v[i + 1:] = 0
    inp.ts[i + 1:] += 10 ** 7
    y2 = to_np(run_full(inp, params=p))
    assert np.array_equal(y[:i + 1], y2[:i + 1])


def test_zero_v_gives_zero():
    inp = W.jagged("zv", 92, [70, 130], 2, 64, "bf16", 16, 16)
    inp.v[:] = 0
    assert np.all(to_np(run_full(inp)) == 0)


# ---------------------------------------------------------------- paged append + cached path

def _prefill(ci, cache, p):
    """Fill every user's cached prefix by appending it to empty caches."""
    h = ci.hist
    dt = tdtype(ci.dtype)
    pre, new = ci.split()
    zeros = dev(np.zeros(ci.batch, np.int32))
    hs.hstu_kv_append(cache, dev(ci.prefix_offsets()), zeros, dev(h.k[pre], dt), dev(h.v[pre], dt),
                      dev(h.ts[pre]), p)
    hs.hstu_kv_append(cache, dev(ci.new_offsets()), dev(ci.cache_lens), dev(h.k[new], dt), dev(h.v[new], dt),
                      dev(h.ts[new]), p)
    return pre, new


def _cache_for(ci, p):
    return hs.PagedKVCache.empty(ci.num_pages, ci.num_heads, ci.head_dim, dev(ci.page_table),
                                 dtype=tdtype(ci.dtype))


def test_kv_append_bit_exact():
    ci = W.cached("app", 95, [0, 70, 64, 1], [5, 64, 130, 0], H=2, d=64, dtype="bf16")
    p = params_for("bf16", 2, 64)
    cache = _cache_for(ci, p)
    pre, new = _prefill(ci, cache, p)
    torch.cuda.synchronize()
    h = ci.hist
    P = ci.num_pages
    kp, vp, tp = oracle.kv_append_pages(np.zeros((P, 2, 64, 64), np.float32), np.zeros((P, 2, 64, 64), np.float32),
                                        np.zeros((P, 64), np.int64), ci.page_table, np.zeros(4, np.int32),
                                        ci.prefix_offsets(), h.k[pre], h.v[pre], h.ts[pre])
    kp, vp, tp = oracle.kv_append_pages(kp, vp, tp, ci.page_table, ci.cache_lens, ci.new_offsets(), h.k[new],
                                        h.v[new], h.ts[new])
    assert np.array_equal(cache.k_pages.float().cpu().numpy(), kp)
    assert np.array_equal(cache.v_pages.float().cpu().numpy(), vp)
    assert np.array_equal(cache.ts_pages.cpu().numpy(), tp)


def _run_cached(ci, p=None):
    dt = tdtype(ci.dtype)
    p = p or params_for(ci.dtype, ci.num_heads, ci.head_dim, ci.hist.tables)
    cache = _cache_for(ci, p)
    pre, new = _prefill(ci, cache, p)
    h = ci.hist
    max_total = int((ci.cache_lens + ci.new_lens).max())
    y = hs.hstu_attn_fwd_cached(dev(h.q[new], dt), dev(h.u[new], dt), dev(h.ts[new]), dev(ci.new_offsets()),
                                dev(ci.cache_lens), int(max(1, ci.new_lens.max())), max_total, cache, p)
    torch.cuda.synchronize()
    return y, new


def test_kv_cache_delta_config():
    """8 users, 8,192 cached tokens in 64-token pages + 128 new tokens each."""
    ci = W.kv_cache_delta()
    y, new = _run_cached(ci)
    h = ci.hist
    y_ref, _ = oracle.hstu_cached(h.q[new], h.u[new], h.ts[new], h.k, h.v, h.ts, h.seq_offsets, ci.cache_lens,
                                  ci.new_offsets(), h.tables.pos, h.tables.time)
    check(y, y_ref, "bf16", "kv delta vs oracle")
    # cached delta equals full recompute over 8,320 tokens (rows of the full oracle)
    rows = new[np.random.default_rng(1).integers(0, len(new), 24)]
    y_full = oracle.hstu_full_rows(rows, h.q, h.k, h.v, h.u, h.ts, h.seq_offsets, h.tables.pos, h.tables.time)
    pos = np.searchsorted(new, rows)
    err = oracle.max_rel_row_error(to_np(y)[pos], y_full)
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 32)])
def test_cached_edge_cases(dtype, d):
    ci = W.cached("cedge", 96, [0, 1, 63, 64, 700, 1500, 3], [5, 1, 129, 64, 2, 0, 300], H=2, d=d, dtype=dtype,
                  n_pos=128, n_time=64)
    y, new = _run_cached(ci)
    h = ci.hist
    y_ref, _ = oracle.hstu_cached(h.q[new], h.u[new], h.ts[new], h.k, h.v, h.ts, h.seq_offsets, ci.cache_lens,
                                  ci.new_offsets(), h.tables.pos, h.tables.time)
    check(y, y_ref, dtype, f"cached edges {dtype}")


def test_cached_more_than_64_users():
    """70 users: the epilogue finds a row's user by a loop over 64-entry blocks
    of the offsets (one wave-wide load covers up to 64 users)."""
    rng = np.random.default_rng(134)
    cache_lens = [int(x) for x in rng.integers(0, 300, size=70)]
    new_lens = [int(x) for x in rng.integers(0, 40, size=70)]
    ci = W.cached("cmany", 134, cache_lens, new_lens, H=2, d=64, dtype="bf16", n_pos=128, n_time=64)
    y, new = _run_cached(ci)
    h = ci.hist
    y_ref, _ = oracle.hstu_cached(h.q[new], h.u[new], h.ts[new], h.k, h.v, h.ts, h.seq_offsets, ci.cache_lens,
                                  ci.new_offsets(), h.tables.pos, h.tables.time)
    check(y, y_ref, "bf16", "cached 70 users")


def test_cached_equals_gpu_full_path():
    ci = W.cached("cvf", 97, [200, 513], [70, 130], H=2, d=128, dtype="bf16")
    y, new = _run_cached(ci)
    yf = run_full(ci.hist)
    err = oracle.max_rel_row_error(to_np(y), to_np(yf)[new])
    assert err <= 1e-2, err


# ---------------------------------------------------------------- M-FALCON

def _run_mfalcon(ci, p=None):
    inp = ci.inputs
    dt = tdtype(inp.dtype)
    p = p or params_for(inp.dtype, inp.num_heads, inp.head_dim, inp.tables)
    y = hs.hstu_mfalcon_fwd(dev(inp.q, dt), dev(inp.k, dt), dev(inp.v, dt), dev(inp.u, dt), dev(inp.ts),
                            dev(inp.seq_offsets), dev(ci.num_candidates), max(1, inp.max_len), p)
    torch.cuda.synchronize()
    return y


def _oracle_mfalcon(ci):
    inp = ci.inputs
    y, _ = oracle.hstu_mfalcon(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, ci.num_candidates,
                               inp.tables.pos, inp.tables.time)
    return y


def test_mfalcon_config():
    """4 users, 4,096 history tokens + 1,024 candidates each."""
    ci = W.mfalcon_scoring()
    check(_run_mfalcon(ci), _oracle_mfalcon(ci), "bf16", "M-FALCON B4 4096+1024")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 32), ("bf16", 64)])
def test_mfalcon_edge_cases(dtype, d):
    ci = W.candidates("medge", 98, [0, 1, 64, 100, 129, 300], [3, 0, 130, 1, 64, 0], H=2, d=d, dtype=dtype)
    check(_run_mfalcon(ci), _oracle_mfalcon(ci), dtype, f"M-FALCON edges {dtype} d={d}")


def test_mfalcon_candidates_independent_bitwise():
    ci = W.candidates("mind", 99, [257], [200], H=2, d=128, dtype="bf16")
    y = to_np(_run_mfalcon(ci))
    inp = ci.inputs
    other = np.arange(257 + 100, 457)
    inp.q[other] *= -1
    inp.k[other] += 1
    inp.v[other] = 0
    y2 = to_np(_run_mfalcon(ci))
    assert np.array_equal(y[:357], y2[:357])


# ---------------------------------------------------------------- norm input

FP32_IN = 1  # HSTU_FLAG_FP32_NORM_INPUT


def _both_norm_inputs(inp, ref, label, **pkw):
    """The bf16 full path with the norm-ready store (default) and with the fp32
    round trip, each against the oracle, and against each other."""
    ys = []
    for flags in (0, FP32_IN):
        p = params_for(inp.dtype, inp.num_heads, inp.head_dim, inp.tables, flags=flags, **pkw)
        ys.append(to_np(run_full(inp, p)))
        err = oracle.max_rel_row_error(ys[-1], ref)
        print(f"{label} flags={flags}: max row rel err {err:.3e}", flush=True)
        assert err <= TOL["bf16"]
    assert oracle.max_rel_row_error(ys[0], ys[1]) <= TOL["bf16"]
    return ys


@pytest.mark.parametrize("d", [128, 64, 32])
def test_norm_ready_store_ragged_all_head_dims(d):
    inp = W.jagged(f"normready_d{d}", 401, [1, 77, 200, 130, 0, 64, 129, 300], 4, d, "bf16", 128, 128)
    _both_norm_inputs(inp, oracle_full(inp), f"norm-ready d={d}")


def test_norm_ready_store_training_shape_and_affine():
    inp = W.training_shape()
    w, b = W.affine_terms(402, 512)
    ref, _ = oracle.hstu_full(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, inp.tables.pos,
                              inp.tables.time, gamma=w, beta=b)
    _both_norm_inputs(inp, ref, "training shape + affine", ln_w=dev(w), ln_b=dev(b))


def test_norm_ready_store_sixteen_heads():
    # H * d = 2,048: the finisher merges 16 heads' statistics per row
    inp = W.jagged("normready_h16", 403, [700, 45, 300], 16, 128, "bf16", 256, 64)
    _both_norm_inputs(inp, oracle_full(inp), "16 heads")


def test_norm_ready_store_large_common_offset():
    """V = N(0, 1) + 40 with one head: every output row is a large common
    offset plus a small spread. The store keeps deviations from the head's
    mean, so bf16 rounding stays relative to the spread (a bf16 copy of O
    itself would lose the spread to rounding of the offset, about 40 x 2^-9
    of the row sum against a spread of the row sum over sqrt(keys)). One head,
    because the bf16 P of each head scales the offset by its own rounding
    error, which the norm removes only when the row is one head."""
    inp = W.jagged("normready_offset", 404, [150, 400, 64], 1, 128, "bf16", 128, 128)
    inp.v = W.round_to_bf16((inp.v + 40.0).astype(np.float32))
    _both_norm_inputs(inp, oracle_full(inp), "common offset 40")


def test_norm_ready_store_mfalcon():
    ci = W.candidates("normready_mf", 405, [300, 0, 129], [50, 7, 64])
    ref = _oracle_mfalcon(ci)
    inp = ci.inputs
    ys = []
    for flags in (0, FP32_IN):
        ys.append(to_np(_run_mfalcon(ci, params_for(inp.dtype, inp.num_heads, inp.head_dim, inp.tables,
                                                     flags=flags))))
        err = oracle.max_rel_row_error(ys[-1], ref)
        print(f"M-FALCON flags={flags}: max row rel err {err:.3e}", flush=True)
        assert err <= TOL["bf16"]
