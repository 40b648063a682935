"""Multi-layer cached serving loop over the paged KV cache.

One request step for a batch of users: the page manager says how many of
each user's tokens are already cached (0 after an eviction), only the
uncached suffix is sent, and every layer appends that suffix's K, V and
timestamps to its own page pool and runs the cached forward over the whole
history. This is the reuse of a cached history prefix across requests that
"Deploying an HSTU Generative Recommender with NVIDIA Dynamo-Triton"
(section "Technical Stack and Performance Gains") and page
"recomendador-generativo-hstu-dynamo-triton" (section "Como o recomendador
generativo HSTU reutiliza o histórico") describe; the layers' own weights are
outside this library, so each layer's Q, K, V, U rows come from the caller.

Argument marshalling only: every step runs in the library's kernels.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np
import torch

from . import (HSTU_FN_CACHED, LayerParams, PageManager, PagedKVCache, hstu_attn_fwd_cached,
               hstu_kv_append, hstu_workspace_size)


class CachedServing:
    """Page manager plus one page pool per layer (all layers share page ids)."""

    def __init__(self, params: Sequence[LayerParams], num_pages: int, max_pages_per_seq: int, max_users: int,
                 device: str = "cuda"):
        if not params:
            raise ValueError("need at least one layer")
        self.params = list(params)
        self.pm = PageManager(num_pages, max_pages_per_seq, max_users)
        self.device = device
        self.max_pages_per_seq = max_pages_per_seq
        self.pools = [PagedKVCache.empty(num_pages, p.num_heads, p.head_dim, None, dtype=p.dtype, device=device)
                      for p in self.params]

    def step(self, user_ids: Sequence[int], ts: Sequence[np.ndarray],
             layers: Sequence[Sequence[Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]]]):
        """Serve one request for a batch of users.

        user_ids: B distinct 64-bit ids. ts[b]: int64 [L_b], user b's whole
        history so far (timestamps). layers[l][b] = (q, k, v, u) of user b's
        whole history at layer l ([L_b, H, d] and [L_b, H*d], host arrays).
        Returns (cache_lens int32 [B] before the step, new_offsets int32
        [B+1], list over layers of y [T_new, H*d] on the device): y holds the
        rows cache_lens[b] .. L_b - 1 of each user, packed.
        """
        B = len(user_ids)
        if B == 0:
            return np.zeros(0, np.int32), np.zeros(1, np.int32), []
        if len(ts) != B or any(len(layer) != B for layer in layers) or len(layers) != len(self.params):
            raise ValueError("one entry per user and per layer expected")
        lens = np.array([len(t) for t in ts], dtype=np.int64)
        cached = np.array([max(self.pm.lookup(u), 0) for u in user_ids], dtype=np.int64)
        if np.any(cached > lens):
            raise ValueError("a user's history is shorter than what is cached for it")
        n_new = (lens - cached).astype(np.int32)
        cache_lens, table, _ = self.pm.reserve(user_ids, n_new)
        assert np.array_equal(cache_lens, cached.astype(np.int32))
        new_off = np.zeros(B + 1, dtype=np.int32)
        new_off[1:] = np.cumsum(n_new)
        dev = lambda x, dt=None: (torch.from_numpy(np.ascontiguousarray(x)).to(dt) if dt is not None else
                                  torch.from_numpy(np.ascontiguousarray(x))).to(self.device)
        sl = [slice(int(c), int(l)) for c, l in zip(cached, lens)]
        ts_new = dev(np.concatenate([np.asarray(t, dtype=np.int64)[s] for t, s in zip(ts, sl)]))
        off_t, cl_t, table_t = dev(new_off), dev(cache_lens), dev(table)
        max_new = int(max(1, n_new.max()))
        max_total = int(max(1, lens.max()))
        T_new = int(new_off[-1])
        outs: List[torch.Tensor] = []
        for p, pool, layer in zip(self.params, self.pools, layers):
            pool.page_table = table_t
            # the uncached suffix of every user, packed: q, k, v, u
            parts = [[np.asarray(x)[sl[b]] for x in layer[b]] for b in range(B)]
            q, k, v, u = (dev(np.concatenate([parts[b][i] for b in range(B)]), p.dtype) for i in range(4))
            hstu_kv_append(pool, off_t, cl_t, k, v, ts_new, p)
            ws = torch.empty(hstu_workspace_size(HSTU_FN_CACHED, p, B, T_new, max_total), dtype=torch.uint8,
                             device=self.device)
            outs.append(hstu_attn_fwd_cached(q, u, ts_new, off_t, cl_t, max_new, max_total, pool, p, workspace=ws))
        self.pm.commit(user_ids, n_new)
        return cache_lens, new_off, outs
