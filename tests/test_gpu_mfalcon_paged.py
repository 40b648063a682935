"""GPU parity of M-FALCON over a paged history (hstu_mfalcon_fwd_cached): the
candidates' outputs against the fp64 oracle's candidate rows of M-FALCON on
[history | candidates], and against the jagged GPU path."""
import numpy as np
import pytest
import torch

import hstu_jagged_silu_amd as hs
import oracle
import workloads as W

from devutil import TOL, dev, params_for, tdtype, to_np

pytestmark = pytest.mark.gpu


def run_paged(ci, p=None, seed=7):
    """Append every user's history to a fresh page pool, then score the candidates."""
    inp = ci.inputs
    dt = tdtype(inp.dtype)
    p = p or params_for(inp.dtype, inp.num_heads, inp.head_dim, inp.tables)
    hist, cand = ci.split()
    num_pages, table = ci.history_pages(seed)
    cache = hs.PagedKVCache.empty(num_pages, inp.num_heads, inp.head_dim, dev(table), dtype=dt)
    hoff = W.offsets_from_lengths(ci.hist_lens)
    coff = W.offsets_from_lengths(ci.num_candidates)
    if len(hist):
        hs.hstu_kv_append(cache, dev(hoff), dev(np.zeros(len(ci.hist_lens), np.int32)), dev(inp.k[hist], dt),
                          dev(inp.v[hist], dt), dev(inp.ts[hist]), p)
    y = hs.hstu_mfalcon_fwd_cached(dev(inp.q[cand], dt), dev(inp.k[cand], dt), dev(inp.v[cand], dt),
                                   dev(inp.u[cand], dt), dev(inp.ts[cand]), dev(coff), dev(ci.hist_lens),
                                   int(max(1, ci.num_candidates.max())), int(max(1, ci.hist_lens.max())), cache, p)
    torch.cuda.synchronize()
    return to_np(y), cand


def oracle_candidates(ci, cand):
    inp = ci.inputs
    y, _ = oracle.hstu_mfalcon(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, ci.num_candidates,
                               inp.tables.pos, inp.tables.time)
    return y[cand]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 32), ("bf16", 64)])
def test_paged_mfalcon_edge_cases(dtype, d):
    # empty history, one token, page boundaries, a history longer than one key split
    ci = W.candidates("pmedge", 101, [0, 1, 64, 100, 129, 300, 1100], [3, 2, 130, 1, 64, 5, 7], H=2, d=d,
                      dtype=dtype)
    y, cand = run_paged(ci)
    err = oracle.max_rel_row_error(y, oracle_candidates(ci, cand))
    print(f"paged M-FALCON edges {dtype} d={d}: max row rel err {err:.3e}")
    assert err <= TOL[dtype]


def test_paged_mfalcon_config_vs_oracle_and_jagged():
    """4 users, 4,096 history tokens in pages + 1,024 candidates each."""
    ci = W.mfalcon_scoring()
    y, cand = run_paged(ci)
    err = oracle.max_rel_row_error(y, oracle_candidates(ci, cand))
    print(f"paged M-FALCON B4 4096+1024 vs oracle: max row rel err {err:.3e}")
    assert err <= TOL["bf16"]
    inp = ci.inputs
    bf = torch.bfloat16
    p = params_for("bf16", 4, 128, inp.tables)
    yj = to_np(hs.hstu_mfalcon_fwd(dev(inp.q, bf), dev(inp.k, bf), dev(inp.v, bf), dev(inp.u, bf), dev(inp.ts),
                                   dev(inp.seq_offsets), dev(ci.num_candidates), inp.max_len, p))
    torch.cuda.synchronize()
    assert oracle.max_rel_row_error(y, yj[cand]) <= TOL["bf16"]


def test_paged_candidates_independent_bitwise():
    ci = W.candidates("pmind", 102, [700], [200], H=2, d=128, dtype="bf16")
    y, cand = run_paged(ci)
    inp = ci.inputs
    other = cand[100:]
    inp.q[other] *= -1
    inp.k[other] += 1
    inp.v[other] = 0
    y2, _ = run_paged(ci)
    assert np.array_equal(y[:100], y2[:100])
