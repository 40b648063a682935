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

Everything the loop needs on the device is allocated once, in the
constructor, for the largest request it accepts: the page pools, the
workspace, the per-layer outputs and the per-request index arrays (page
table rows, offsets, cached lengths, staged through pinned host buffers). A
step copies those index arrays (a few KiB) to the device and launches the
library's kernels; the token rows arrive as device tensors.

Argument marshalling only: every step runs in the library's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, List, Sequence, Tuple

import numpy as np
import torch

from . import (HSTU_FN_CACHED, PAGE_SIZE, LayerParams, PageManager, PagedKVCache, hstu_attn_fwd_cached,
               hstu_kv_append, hstu_workspace_size)


@dataclass
class Request:
    """One reserved request: user ids, cached tokens per user before it, new
    tokens per user and their packed offsets (host arrays)."""
    user_ids: List[int]
    cache_lens: np.ndarray   # int32 [B]
    n_new: np.ndarray        # int32 [B]
    new_offsets: np.ndarray  # int32 [B + 1]
    page_table: np.ndarray   # int32 [B, max_pages_per_seq]
    done: bool = False

    @property
    def total_new(self) -> int:
        return int(self.new_offsets[-1])


class CachedServing:
    """Page manager plus one page pool per layer (all layers share page ids),
    with every device buffer of a step preallocated."""

    def __init__(self, params: Sequence[LayerParams], num_pages: int, max_pages_per_seq: int, max_users: int,
                 max_batch: int, max_new_tokens: int, device: str = "cuda"):
        if not params:
            raise ValueError("need at least one layer")
        if max_batch < 1 or max_new_tokens < 1:
            raise ValueError("max_batch and max_new_tokens must be >= 1")
        self.params = list(params)
        self.pm = PageManager(num_pages, max_pages_per_seq, max_users)
        self.device = device
        self.max_pages_per_seq = max_pages_per_seq
        self.max_batch, self.max_new_tokens = max_batch, max_new_tokens
        self.max_total = max_pages_per_seq * PAGE_SIZE
        self.pools = [PagedKVCache.empty(num_pages, p.num_heads, p.head_dim, None, dtype=p.dtype, device=device)
                      for p in self.params]
        nbytes = max(hstu_workspace_size(HSTU_FN_CACHED, p, max_batch, max_new_tokens, self.max_total)
                     for p in self.params)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.outputs = [torch.empty((max_new_tokens, p.num_heads * p.head_dim), dtype=p.dtype, device=device)
                        for p in self.params]
        # per-request index arrays: pinned host staging, device copies
        pin = torch.cuda.is_available()
        self._h_table = torch.full((max_batch, max_pages_per_seq), -1, dtype=torch.int32, pin_memory=pin)
        self._h_off = torch.zeros(max_batch + 1, dtype=torch.int32, pin_memory=pin)
        self._h_lens = torch.zeros(max_batch, dtype=torch.int32, pin_memory=pin)
        self._d_table = torch.full((max_batch, max_pages_per_seq), -1, dtype=torch.int32, device=device)
        self._d_off = torch.zeros(max_batch + 1, dtype=torch.int32, device=device)
        self._d_lens = torch.zeros(max_batch, dtype=torch.int32, device=device)
        self._staged = None   # event after the last staging copies: the pinned buffers are free once it completes

    def begin(self, user_ids: Sequence[int], hist_lens: Sequence[int]) -> Request:
        """Reserve pages for a request. hist_lens[b] is user b's whole history
        length after this request. The caller then sends, for user b, the rows
        cache_lens[b] .. hist_lens[b] - 1 (all of them after an eviction)."""
        B = len(user_ids)
        if B > self.max_batch:
            raise ValueError(f"batch {B} above max_batch {self.max_batch}")
        lens = np.asarray(hist_lens, dtype=np.int64).reshape(-1)
        if len(lens) != B:
            raise ValueError("one history length per user expected")
        cached = np.array([max(self.pm.lookup(u), 0) for u in user_ids], dtype=np.int64)
        if np.any(cached > lens):
            raise ValueError("a user's history is shorter than what is cached for it")
        n_new = (lens - cached).astype(np.int32)
        if int(n_new.sum()) > self.max_new_tokens:
            raise ValueError(f"{int(n_new.sum())} new tokens above max_new_tokens {self.max_new_tokens}")
        if B and int(lens.max()) > self.max_total:
            raise ValueError("a history longer than max_pages_per_seq pages")
        if B == 0:
            return Request([], np.zeros(0, np.int32), n_new, np.zeros(1, np.int32),
                           np.zeros((0, self.max_pages_per_seq), np.int32))
        cache_lens, table, _ = self.pm.reserve(list(user_ids), n_new)
        if not np.array_equal(cache_lens, cached.astype(np.int32)):
            raise RuntimeError("page manager and lookup disagree on the cached lengths")
        new_off = np.zeros(B + 1, dtype=np.int32)
        new_off[1:] = np.cumsum(n_new)
        return Request(list(user_ids), cache_lens, n_new, new_off, table)

    def run(self, req: Request, ts_new: torch.Tensor,
            layers: Sequence[Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]]) -> List[torch.Tensor]:
        """Append and attend for every layer. ts_new: int64 [T_new] device
        timestamps of the packed new rows; layers[l] = (q, k, v, u) device
        tensors of those rows at layer l ([T_new, H, d] and [T_new, H*d]).
        Returns per layer a view [T_new, H*d] of that layer's preallocated
        output (overwritten by the next run)."""
        B, T = len(req.user_ids), req.total_new
        if len(layers) != len(self.params):
            raise ValueError("one (q, k, v, u) per layer expected")
        if B == 0 or T == 0:
            return [o[:0] for o in self.outputs]
        if ts_new.shape[0] != T:
            raise ValueError(f"ts_new must hold {T} rows")
        if self._staged is not None:
            self._staged.synchronize()
        self._h_table[:B].copy_(torch.from_numpy(req.page_table))
        self._h_off[:B + 1].copy_(torch.from_numpy(req.new_offsets))
        self._h_lens[:B].copy_(torch.from_numpy(req.cache_lens))
        self._d_table[:B].copy_(self._h_table[:B], non_blocking=True)
        self._d_off[:B + 1].copy_(self._h_off[:B + 1], non_blocking=True)
        self._d_lens[:B].copy_(self._h_lens[:B], non_blocking=True)
        self._staged = torch.cuda.Event()
        self._staged.record()
        off, lens = self._d_off[:B + 1], self._d_lens[:B]
        max_new = int(max(1, req.n_new.max()))
        max_total = int(max(1, (req.cache_lens + req.n_new).max()))
        outs = []
        for p, pool, (q, k, v, u), y in zip(self.params, self.pools, layers, self.outputs):
            if q.shape[0] != T or k.shape[0] != T or v.shape[0] != T or u.shape[0] != T:
                raise ValueError(f"every layer's q, k, v, u must hold {T} rows")
            pool.page_table = self._d_table
            hstu_kv_append(pool, off, lens, k, v, ts_new, p)
            outs.append(hstu_attn_fwd_cached(q, u, ts_new, off, lens, max_new, max_total, pool, p, y=y[:T],
                                             workspace=self.workspace))
        return outs

    def commit(self, req: Request) -> None:
        """Advance the users' cached lengths by the new tokens (after run)."""
        if req.done:
            raise ValueError("request already committed")
        if req.user_ids:
            self.pm.commit(req.user_ids, req.n_new)
        req.done = True

    def step(self, user_ids: Sequence[int], hist_lens: Sequence[int],
             fetch: Callable[[Request], Tuple[torch.Tensor, Sequence[Tuple[torch.Tensor, ...]]]]):
        """begin, then fetch(request) -> (ts_new, layers) device tensors of the
        rows the request needs, then run; commits only when run succeeds (an
        uncommitted reservation is replaced by the users' next request, its
        pages kept). Returns (request, per-layer outputs)."""
        req = self.begin(user_ids, hist_lens)
        ts_new, layers = fetch(req)
        outs = self.run(req, ts_new, layers)
        self.commit(req)
        return req, outs
