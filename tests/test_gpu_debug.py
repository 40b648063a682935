"""Debug mode (HSTU_DEBUG=1): device-side content checks before the attention.

Bad index content (offsets, lengths, candidate counts, cache lengths, page
entries) must set the documented bits in the workspace header and keep every
kernel inside its buffers; valid content must give 0 and the same output as
a call without the debug mode.
"""
import os

import numpy as np
import pytest
import torch

import workloads as W
from devutil import dev, params_for, run_full, to_np

hs = pytest.importorskip("hstu_jagged_silu_amd")
pytestmark = pytest.mark.gpu


@pytest.fixture
def debug_env():
    old = os.environ.get("HSTU_DEBUG")
    os.environ["HSTU_DEBUG"] = "1"
    yield
    if old is None:
        os.environ.pop("HSTU_DEBUG", None)
    else:
        os.environ["HSTU_DEBUG"] = old


def _full_call(inp, offsets, max_len, ws=None):
    bf = torch.bfloat16
    q, k, v, u = (dev(x, bf) for x in (inp.q, inp.k, inp.v, inp.u))
    p = params_for("bf16", inp.num_heads, inp.head_dim, inp.tables)
    B = len(offsets) - 1
    nbytes = hs.hstu_workspace_size(hs.HSTU_FN_FULL, p, B, inp.total, max_len)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda") if ws is None else ws
    y = hs.hstu_attn_fwd(q, k, v, u, dev(inp.ts), dev(np.asarray(offsets, np.int32)), max_len, p, workspace=ws)
    return y, ws


def test_valid_content_flags_zero_and_matches(debug_env):
    inp = W.jagged("dbg", 95, [70, 0, 130], 2, 128, "bf16", 128, 128)
    y, ws = _full_call(inp, inp.seq_offsets, inp.max_len)
    assert hs.debug_flag(ws) == 0
    del os.environ["HSTU_DEBUG"]
    assert np.array_equal(to_np(y), to_np(run_full(inp)))


@pytest.mark.parametrize("case,bits", [
    ("decreasing", hs.HSTU_DEBUG_BAD_OFFSETS),
    ("negative_start", hs.HSTU_DEBUG_BAD_OFFSETS),
    ("end_not_total", hs.HSTU_DEBUG_BAD_OFFSETS),
    ("too_long", hs.HSTU_DEBUG_BAD_LENGTH),
])
def test_bad_offsets_and_lengths(debug_env, case, bits):
    inp = W.jagged("dbg2", 96, [70, 60, 70], 2, 128, "bf16", 128, 128)
    off = [int(x) for x in inp.seq_offsets]   # [0, 70, 130, 200]
    max_len = inp.max_len
    if case == "decreasing":
        off[1], off[2] = 150, 100
    elif case == "negative_start":
        off[0] = -64
    elif case == "end_not_total":
        off[3] = 190
    else:
        max_len = 64
    print("case", case, off, max_len, flush=True)
    _, ws = _full_call(inp, off, max_len)
    assert hs.debug_flag(ws) & bits


def test_bad_candidate_count(debug_env):
    ci = W.candidates("dbg3", 97, [100, 50], [20, 10])
    inp = ci.inputs
    bf = torch.bfloat16
    q, k, v, u = (dev(x, bf) for x in (inp.q, inp.k, inp.v, inp.u))
    p = params_for("bf16", inp.num_heads, inp.head_dim, inp.tables)
    nc = np.array(ci.num_candidates, np.int32)
    nc[1] = 61   # more candidates than the user's 60 rows
    ws = torch.zeros(hs.hstu_workspace_size(hs.HSTU_FN_MFALCON, p, 2, inp.total, inp.max_len), dtype=torch.uint8,
                     device="cuda")
    hs.hstu_mfalcon_fwd(q, k, v, u, dev(inp.ts), dev(inp.seq_offsets), dev(nc), inp.max_len, p, workspace=ws)
    assert hs.debug_flag(ws) == hs.HSTU_DEBUG_BAD_CANDIDATES


def test_bad_cache_len_and_page(debug_env):
    ci = W.cached("dbg4", 98, [130, 64], [5, 70], H=2, d=128)
    h = ci.hist
    bf = torch.bfloat16
    p = params_for("bf16", 2, 128, h.tables)
    pre, new = ci.split()
    cache = hs.PagedKVCache.empty(ci.num_pages, 2, 128, dev(ci.page_table), dtype=bf)
    hs.hstu_kv_append(cache, dev(ci.prefix_offsets()), dev(np.zeros(ci.batch, np.int32)),
                      dev(h.k[pre], bf), dev(h.v[pre], bf), dev(h.ts[pre]), p)
    qn, un, kn, vn = (dev(x[new], bf) for x in (h.q, h.u, h.k, h.v))
    tsn, noff = dev(h.ts[new]), dev(ci.new_offsets())
    max_total = int((ci.cache_lens + ci.new_lens).max())
    max_new = int(ci.new_lens.max())
    hs.hstu_kv_append(cache, noff, dev(ci.cache_lens), kn, vn, tsn, p)

    def run(cache_lens, table):
        c = hs.PagedKVCache(cache.k_pages, cache.v_pages, cache.ts_pages, dev(table))
        ws = torch.zeros(hs.hstu_workspace_size(hs.HSTU_FN_CACHED, p, ci.batch, len(new), max_total),
                         dtype=torch.uint8, device="cuda")
        hs.hstu_attn_fwd_cached(qn, un, tsn, noff, dev(np.asarray(cache_lens, np.int32)), max_new, max_total, c, p,
                                workspace=ws)
        return hs.debug_flag(ws)

    assert run(ci.cache_lens, ci.page_table) == 0
    bad_len = np.array(ci.cache_lens, np.int32)
    bad_len[0] = -1
    assert run(bad_len, ci.page_table) & hs.HSTU_DEBUG_BAD_CACHE_LEN
    bad_tab = np.array(ci.page_table, np.int32)
    bad_tab[1, 0] = ci.num_pages + 3   # outside the pool
    assert run(ci.cache_lens, bad_tab) == hs.HSTU_DEBUG_BAD_PAGE
    bad_tab = np.array(ci.page_table, np.int32)
    bad_tab[0, 1] = -1                 # a needed page missing
    assert run(ci.cache_lens, bad_tab) == hs.HSTU_DEBUG_BAD_PAGE
