"""GPU check of the multi-layer cached serving loop: a page manager shared by
two layers, histories that grow over requests, a pool small enough that a
user is evicted and has to send its whole history again. Every request's
outputs, per layer, are compared with the oracle's cached path over the
user's full history (which is also the full recompute of those rows)."""
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
    srv = CachedServing(params, num_pages=8, max_pages_per_seq=4, max_users=4)
    requests = [({11: 100, 22: 200}, 0), ({11: 130, 33: 150}, 1), ({22: 230, 11: 140}, 1)]
    for step, (lens, expect_evictions) in enumerate(requests):
        ids = list(lens)
        ev0 = srv.pm.stats()["evictions"]
        ts = [users[u][0].ts[:lens[u]] for u in ids]   # one timestamp sequence per user, shared by layers
        layers = [[(users[u][l].q[:lens[u]], users[u][l].k[:lens[u]], users[u][l].v[:lens[u]],
                    users[u][l].u[:lens[u]]) for u in ids] for l in range(2)]
        cache_lens, new_off, ys = srv.step(ids, ts, layers)
        torch.cuda.synchronize()
        assert srv.pm.stats()["evictions"] - ev0 == expect_evictions
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
