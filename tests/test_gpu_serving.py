"""GPU check of the multi-layer cached serving loop: a page manager shared by
two layers, histories that grow over requests, a pool small enough that a
user is evicted and has to send its whole history again. Each request sends
only the uncached rows, as device tensors, into preallocated buffers; every
request's outputs, per layer, are compared with the oracle's cached path over
the user's full history (which is also the full recompute of those rows)."""
import numpy as np
import pytest
import torch

import hstu_jagged_silu_amd as hs
import oracle
import workloads as W
from hstu_jagged_silu_amd.serving import CachedServing

from devutil import TOL, dev, to_np

pytestmark = pytest.mark.gpu


def test_two_layer_serving_with_eviction():
    H, d, final = 2, 128, {11: 140, 22: 230, 33: 150}
    # per user and layer: the whole final history, drawn once (seeded)
    users = {}
    for seed, (uid, L) in enumerate(final.items()):
        inp = [W.jagged(f"srv{uid}_{l}", 300 + 10 * seed + l, [L], H, d, "bf16", 128, 128) for l in range(2)]
        users[uid] = inp
    tables = users[11][0].tables
    params = [hs.LayerParams(num_heads=H, head_dim=d, dtype=torch.bfloat16, pos_tab=dev(tables.pos),
                             time_tab=dev(tables.time)) for _ in range(2)]
    # 8 pages of 64 tokens. Request 0: users 11 and 22 take 6 pages. Request 1: 11 grows
    # and 33 arrives, so 22 (not in the request) is evicted. Request 2: 22 comes back and
    # evicts 33, the least recently used user outside the request.
    srv = CachedServing(params, num_pages=8, max_pages_per_seq=4, max_users=4, max_batch=2, max_new_tokens=400)
    requests = [({11: 100, 22: 200}, 0), ({11: 130, 33: 150}, 1), ({22: 230, 11: 140}, 1)]
    ws_ptr = srv.workspace.data_ptr()
    for step, (lens, expect_evictions) in enumerate(requests):
        ids = list(lens)
        ev0 = srv.pm.stats()["evictions"]

        def fetch(req):
            # only the uncached rows of each user travel to the device
            sl = [slice(int(c), int(lens[u])) for u, c in zip(ids, req.cache_lens)]
            ts_new = dev(np.concatenate([users[u][0].ts[s] for u, s in zip(ids, sl)]))
            layers = []
            for l in range(2):
                parts = [[x[s] for x in (users[u][l].q, users[u][l].k, users[u][l].v, users[u][l].u)]
                         for u, s in zip(ids, sl)]
                layers.append(tuple(dev(np.concatenate([p[i] for p in parts]), torch.bfloat16) for i in range(4)))
            return ts_new, layers

        req, ys = srv.step(ids, [lens[u] for u in ids], fetch)
        torch.cuda.synchronize()
        cache_lens, new_off = req.cache_lens, req.new_offsets
        assert srv.pm.stats()["evictions"] - ev0 == expect_evictions
        assert srv.workspace.data_ptr() == ws_ptr and all(y.data_ptr() == o.data_ptr() for y, o in zip(ys, srv.outputs))
        hoff = W.offsets_from_lengths(np.array([lens[u] for u in ids]))
        ts_hist = np.concatenate([users[u][0].ts[:lens[u]] for u in ids])
        ts_new = np.concatenate([users[u][0].ts[c:lens[u]] for u, c in zip(ids, cache_lens)])
        for l in range(2):
            hist = [(users[u][l], c, lens[u]) for u, c in zip(ids, cache_lens)]
            q_new = np.concatenate([x.q[c:L] for x, c, L in hist])
            u_new = np.concatenate([x.u[c:L] for x, c, L in hist])
            k_hist = np.concatenate([x.k[:L] for x, _, L in hist])
            v_hist = np.concatenate([x.v[:L] for x, _, L in hist])
            y_ref, _ = oracle.hstu_cached(q_new, u_new, ts_new, k_hist, v_hist, ts_hist, hoff, cache_lens, new_off,
                                          tables.pos, tables.time)
            err = oracle.max_rel_row_error(to_np(ys[l]), y_ref)
            print(f"request {step} layer {l}: cache_lens {list(cache_lens)} max row rel err {err:.3e}")
            assert err <= TOL["bf16"]
    # user 22 came back after its eviction with nothing cached
    assert list(cache_lens) == [0, 130]


def test_failed_run_commits_nothing():
    """A request whose run raises (here: the caller sends too few rows) is not
    committed; the users' next request reuses the reserved pages."""
    H, d = 1, 128
    inp = W.jagged("srv_fail", 310, [100], H, d, "bf16", 128, 128)
    p = hs.LayerParams(num_heads=H, head_dim=d, dtype=torch.bfloat16, pos_tab=dev(inp.tables.pos),
                       time_tab=dev(inp.tables.time))
    srv = CachedServing([p], num_pages=4, max_pages_per_seq=4, max_users=2, max_batch=1, max_new_tokens=128)

    def short(req):
        n = req.total_new - 1
        return dev(inp.ts[:n]), [tuple(dev(x[:n], torch.bfloat16) for x in (inp.q, inp.k, inp.v, inp.u))]

    with pytest.raises(ValueError):
        srv.step([5], [100], short)
    assert srv.pm.lookup(5) == 0 and srv.pm.stats()["free_pages"] == 2

    def full(req):
        return dev(inp.ts[:100]), [tuple(dev(x[:100], torch.bfloat16) for x in (inp.q, inp.k, inp.v, inp.u))]

    req, ys = srv.step([5], [100], full)
    torch.cuda.synchronize()
    assert list(req.cache_lens) == [0] and srv.pm.lookup(5) == 100 and srv.pm.stats()["free_pages"] == 2
    y_ref, _ = oracle.hstu_full(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, inp.tables.pos, inp.tables.time)
    assert oracle.max_rel_row_error(to_np(ys[0]), y_ref) <= TOL["bf16"]
