"""GPU parity sweep: seeded random small configurations of every forward
path, and of the backward, against the fp64 oracle, through the C ABI. Each case draws its own
batch of ragged lengths (empty users, single tokens, exact tile multiples and
tile + 1 included by construction), head count and head size, dtype, tables
(position, time, both, none; shared or per head), alpha, a fixed N, and the
norm's affine terms. Bars as everywhere: max row error 1e-4 (fp32), 2e-2
(bf16); for gradients the per-entry root-sum-square bar of the backward
tests."""
import numpy as np
import pytest
import torch

import hstu_jagged_silu_amd as hs
import oracle
import workloads as W

from devutil import GRAD_RSS_BF16, TOL, dev, tdtype, to_np

pytestmark = pytest.mark.gpu

N_CASES = 24


def _case(seed):
    rng = np.random.default_rng(seed)
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    d = int(rng.choice([32, 64, 128]))
    H = int(rng.choice([1, 2, 3, 4]))
    B = int(rng.integers(1, 7))
    special = [0, 1, 63, 64, 65, 127, 128, 129, 256]
    lengths = [int(rng.choice(special)) if rng.random() < 0.5 else int(rng.integers(1, 400)) for _ in range(B)]
    n_pos = int(rng.choice([1, 16, 128, 300]))
    n_time = int(rng.choice([1, 8, 64, 128]))
    opts = dict(
        pos=rng.random() < 0.8, time=rng.random() < 0.8, per_head=rng.random() < 0.3,
        alpha=float(rng.choice([1.0, 0.5, 1.7])), norm_n=int(rng.choice([0, 0, 500])),
        affine=rng.random() < 0.4, seed=seed)
    return dtype, d, H, lengths, n_pos, n_time, opts


def _params(inp, dtype, H, d, opts):
    pos, tim = inp.tables.pos, inp.tables.time
    if opts["per_head"]:
        pos = np.stack([pos * (1.0 + 0.3 * h) for h in range(H)]).astype(np.float32)
        tim = np.stack([tim * (1.0 - 0.2 * h) for h in range(H)]).astype(np.float32)
    pos = pos if opts["pos"] else None
    tim = tim if opts["time"] else None
    w, b = W.affine_terms(opts["seed"] + 7, H * d) if opts["affine"] else (None, None)
    p = hs.LayerParams(num_heads=H, head_dim=d, dtype=tdtype(dtype), alpha=opts["alpha"], norm_n=opts["norm_n"],
                       pos_tab=None if pos is None else dev(pos), time_tab=None if tim is None else dev(tim),
                       ln_w=None if w is None else dev(w), ln_b=None if b is None else dev(b))
    return p, pos, tim, w, b


@pytest.mark.parametrize("seed", range(N_CASES))
def test_full_path_random_config(seed):
    dtype, d, H, lengths, n_pos, n_time, opts = _case(1000 + seed)
    inp = W.jagged(f"sweep{seed}", 1000 + seed, lengths, H, d, dtype, n_pos, n_time)
    p, pos, tim, w, b = _params(inp, dtype, H, d, opts)
    print(f"case {seed}: {dtype} d={d} H={H} lengths={lengths} {opts}", flush=True)
    dt = tdtype(dtype)
    y = hs.hstu_attn_fwd(dev(inp.q, dt), dev(inp.k, dt), dev(inp.v, dt), dev(inp.u, dt), dev(inp.ts),
                         dev(inp.seq_offsets), max(1, inp.max_len), p)
    torch.cuda.synchronize()
    ref, _ = oracle.hstu_full(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, pos, tim, opts["alpha"],
                              opts["norm_n"], w, b)
    err = oracle.max_rel_row_error(to_np(y), ref)
    print(f"  max row rel err {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("seed", range(N_CASES))
def test_mfalcon_random_config(seed):
    dtype, d, H, lengths, n_pos, n_time, opts = _case(2000 + seed)
    rng = np.random.default_rng(3000 + seed)
    cand = [int(rng.integers(0, 150)) for _ in lengths]
    ci = W.candidates(f"msweep{seed}", 2000 + seed, lengths, cand, H=H, d=d, dtype=dtype, n_pos=n_pos,
                      n_time=n_time)
    inp = ci.inputs
    p, pos, tim, w, b = _params(inp, dtype, H, d, opts)
    print(f"case {seed}: {dtype} d={d} H={H} history={lengths} candidates={cand} {opts}", flush=True)
    dt = tdtype(dtype)
    y = hs.hstu_mfalcon_fwd(dev(inp.q, dt), dev(inp.k, dt), dev(inp.v, dt), dev(inp.u, dt), dev(inp.ts),
                            dev(inp.seq_offsets), dev(ci.num_candidates), max(1, inp.max_len), p)
    torch.cuda.synchronize()
    ref, _ = oracle.hstu_mfalcon(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, ci.num_candidates, pos, tim,
                                 opts["alpha"], opts["norm_n"], w, b)
    err = oracle.max_rel_row_error(to_np(y), ref)
    print(f"  max row rel err {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("seed", range(N_CASES))
def test_cached_random_config(seed):
    dtype, d, H, lengths, n_pos, n_time, opts = _case(4000 + seed)
    rng = np.random.default_rng(5000 + seed)
    new = [int(rng.integers(0, 200)) for _ in lengths]
    ci = W.cached(f"csweep{seed}", 4000 + seed, lengths, new, H=H, d=d, dtype=dtype, n_pos=n_pos, n_time=n_time)
    h = ci.hist
    p, pos, tim, w, b = _params(h, dtype, H, d, opts)
    print(f"case {seed}: {dtype} d={d} H={H} cached={lengths} new={new} {opts}", flush=True)
    dt = tdtype(dtype)
    cache = hs.PagedKVCache.empty(ci.num_pages, H, d, dev(ci.page_table), dtype=dt)
    pre, newi = ci.split()
    Bn = len(lengths)
    hs.hstu_kv_append(cache, dev(ci.prefix_offsets()), dev(np.zeros(Bn, np.int32)), dev(h.k[pre], dt),
                      dev(h.v[pre], dt), dev(h.ts[pre]), p)
    hs.hstu_kv_append(cache, dev(ci.new_offsets()), dev(ci.cache_lens), dev(h.k[newi], dt), dev(h.v[newi], dt),
                      dev(h.ts[newi]), p)
    max_total = int(max(1, (ci.cache_lens + ci.new_lens).max()))
    y = hs.hstu_attn_fwd_cached(dev(h.q[newi], dt), dev(h.u[newi], dt), dev(h.ts[newi]), dev(ci.new_offsets()),
                                dev(ci.cache_lens), int(max(1, ci.new_lens.max())), max_total, cache, p)
    torch.cuda.synchronize()
    ref, _ = oracle.hstu_cached(h.q[newi], h.u[newi], h.ts[newi], h.k, h.v, h.ts, h.seq_offsets, ci.cache_lens,
                                ci.new_offsets(), pos, tim, opts["alpha"], opts["norm_n"], w, b)
    err = oracle.max_rel_row_error(to_np(y), ref)
    print(f"  max row rel err {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("seed", range(10))
def test_backward_random_config(seed):
    dtype, d, H, lengths, n_pos, n_time, opts = _case(6000 + seed)
    n_pos = min(n_pos, 512)                    # the backward's largest position table
    inp = W.jagged(f"bsweep{seed}", 6000 + seed, lengths, H, d, "bf16", n_pos, n_time)
    p, pos, tim, w, b = _params(inp, "bf16", H, d, opts)
    print(f"case {seed}: bf16 d={d} H={H} lengths={lengths} {opts}", flush=True)
    dy = W.upstream_grad(7000 + seed, inp.u.shape)
    bf = torch.bfloat16
    g = hs.hstu_attn_bwd(dev(inp.q, bf), dev(inp.k, bf), dev(inp.v, bf), dev(inp.u, bf), dev(inp.ts),
                         dev(inp.seq_offsets), max(1, inp.max_len), dev(dy, bf), p)
    torch.cuda.synchronize()
    ref = oracle.hstu_full_bwd(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, dy, pos, tim, opts["alpha"],
                               opts["norm_n"], w, b, magnitudes=True)
    for name, rname in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("d_pos_tab", "dpos"), ("d_time_tab", "dtime")):
        if ref[rname] is None:
            assert g[name] is None, name
            continue
        r = np.asarray(ref[rname])
        err = oracle.max_err_vs_scale(to_np(g[name]).reshape(r.shape), r, ref["rss_" + rname])
        print(f"  {name} {err:.3e}")
        assert err <= GRAD_RSS_BF16, (name, err)
    for name, rname in (("du", "du"), ("d_ln_w", "dgamma"), ("d_ln_b", "dbeta")):
        if ref[rname] is None:
            assert g[name] is None, name
            continue
        err = oracle.max_rel_err_vs_magnitude(to_np(g[name]), np.asarray(ref[rname]), np.asarray(ref["mag_" + rname]))
        print(f"  {name} {err:.3e}")
        assert err <= TOL["bf16"], (name, err)
