"""HIP graph capture of the library's calls, through torch.cuda.CUDAGraph.

The entry points allocate nothing, record no memset and never wait on the
host, so a caller can capture them: the serving loop (paged append, then the
cached forward) and the full forward are captured here. Each graph is
replayed several times with eager work and host synchronisations between
the replays, and every replay is checked bitwise against the eager result of
the same calls (the kernels are deterministic)."""
import numpy as np
import pytest
import torch

import hstu_jagged_silu_amd as hs
import workloads as W

from devutil import dev, params_for, tdtype

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _capture(fn):
    """Capture fn() into a graph (after one eager warm-up on a side stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_full_forward_graph_replays():
    inp = W.jagged("graph_full", 131, [300, 1, 77, 512, 0, 129], 2, 128, "bf16", 128, 128)
    p = params_for("bf16", 2, 128, inp.tables)
    q, k, v, u = (dev(x, torch.bfloat16) for x in (inp.q, inp.k, inp.v, inp.u))
    ts, offs = dev(inp.ts), dev(inp.seq_offsets)
    T, B = q.shape[0], offs.shape[0] - 1
    ws = torch.empty(hs.hstu_workspace_size(hs.HSTU_FN_FULL, p, B, T, inp.max_len), dtype=torch.uint8,
                     device="cuda")
    y_eager = hs.hstu_attn_fwd(q, k, v, u, ts, offs, inp.max_len, p, workspace=ws)
    torch.cuda.synchronize()
    y = torch.empty_like(y_eager)
    g = _capture(lambda: hs.hstu_attn_fwd(q, k, v, u, ts, offs, inp.max_len, p, y=y, workspace=ws))
    for r in range(REPLAYS):
        y.fill_(float("nan"))
        # eager work between replays: the same call into another buffer
        y_other = hs.hstu_attn_fwd(q, k, v, u, ts, offs, inp.max_len, p, workspace=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {r}"
        assert torch.equal(y_other, y_eager)


def test_serving_step_graph_replays():
    """Append of the new tokens + cached forward, captured as one graph.
    Replaying rewrites the same page slots, so every replay must leave the
    pages and the output exactly as the eager step did."""
    ci = W.cached("graph_srv", 132, [200, 0, 64, 1000], [37, 5, 64, 128], H=2, d=128, dtype="bf16")
    p = params_for("bf16", 2, 128, ci.hist.tables)
    dt = tdtype("bf16")
    h = ci.hist
    pre, new = ci.split()
    cache = hs.PagedKVCache.empty(ci.num_pages, 2, 128, dev(ci.page_table), dtype=dt)
    hs.hstu_kv_append(cache, dev(ci.prefix_offsets()), dev(np.zeros(ci.batch, np.int32)), dev(h.k[pre], dt),
                      dev(h.v[pre], dt), dev(h.ts[pre]), p)
    k_new, v_new, ts_new = dev(h.k[new], dt), dev(h.v[new], dt), dev(h.ts[new])
    q_new, u_new = dev(h.q[new], dt), dev(h.u[new], dt)
    new_offs, cache_lens = dev(ci.new_offsets()), dev(ci.cache_lens)
    max_new = int(max(1, ci.new_lens.max()))
    max_total = int((ci.cache_lens + ci.new_lens).max())
    T, B = q_new.shape[0], ci.batch
    ws = torch.empty(hs.hstu_workspace_size(hs.HSTU_FN_CACHED, p, B, T, max_total), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty_like(u_new)

    def step():
        hs.hstu_kv_append(cache, new_offs, cache_lens, k_new, v_new, ts_new, p)
        hs.hstu_attn_fwd_cached(q_new, u_new, ts_new, new_offs, cache_lens, max_new, max_total, cache, p, y=y,
                                workspace=ws)

    step()
    torch.cuda.synchronize()
    y_eager = y.clone()
    pages_eager = (cache.k_pages.clone(), cache.v_pages.clone(), cache.ts_pages.clone())
    g = _capture(step)
    for r in range(REPLAYS):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {r}"
        assert torch.equal(cache.k_pages, pages_eager[0]) and torch.equal(cache.v_pages, pages_eager[1])
        assert torch.equal(cache.ts_pages, pages_eager[2])
        # eager work between replays: one eager step on the same buffers
        step()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager)
