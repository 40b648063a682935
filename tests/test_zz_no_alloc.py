"""GPU check of hstu_attn_fwd_cached_noalloc, the cached path for callers that
cannot allocate (its scratch is the library's per-GPU array), against
hstu_attn_fwd_cached with a workspace of its own, through the C ABI. Two
calls in a row, the second smaller, so the second runs on the scratch the
first left behind. Both entry points run the same kernels in the same order,
so the results must agree bit for bit (and so within the bf16 bar); both are
also checked against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import hstu_jagged_silu_amd as hs
import oracle
import workloads as W

from devutil import TOL, dev, to_np

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _cached_case(cc):
    h = cc.hist
    H, d = h.num_heads, h.head_dim
    p = hs.LayerParams(num_heads=H, head_dim=d, dtype=BF, pos_tab=dev(h.tables.pos), time_tab=dev(h.tables.time))
    cache = hs.PagedKVCache.empty(cc.num_pages, H, d, dev(cc.page_table), dtype=BF)
    pre, new = cc.split()
    B = len(cc.cache_lens)
    hs.hstu_kv_append(cache, dev(cc.prefix_offsets()), dev(np.zeros(B, np.int32)), dev(h.k[pre], BF),
                      dev(h.v[pre], BF), dev(h.ts[pre]), p)
    hs.hstu_kv_append(cache, dev(cc.new_offsets()), dev(cc.cache_lens), dev(h.k[new], BF), dev(h.v[new], BF),
                      dev(h.ts[new]), p)
    new_lens = np.diff(cc.new_offsets())
    max_new = int(new_lens.max())
    max_total = int((np.asarray(cc.cache_lens) + new_lens).max())
    args = (dev(h.q[new], BF), dev(h.u[new], BF), dev(h.ts[new]), dev(cc.new_offsets()), dev(cc.cache_lens),
            max_new, max_total, cache, p)
    y_ref, _ = oracle.hstu_cached(h.q[new], h.u[new], h.ts[new], h.k, h.v, h.ts, h.seq_offsets, cc.cache_lens,
                                  cc.new_offsets(), h.tables.pos, h.tables.time)
    return args, y_ref


def test_noalloc_matches_cached_twice_second_smaller():
    cases = [W.cached("noalloc_a", 501, [300, 0, 1000, 65], [40, 64, 17, 130]),
             W.cached("noalloc_b", 502, [100], [20])]
    for cc in cases:
        args, y_ref = _cached_case(cc)
        print(f"case {cc.hist.name}: cache {list(cc.cache_lens)}", flush=True)
        y_ws = hs.hstu_attn_fwd_cached(*args)
        y_na = torch.full_like(y_ws, float("nan"))
        hs.hstu_attn_fwd_cached_noalloc(*args, y_na)
        torch.cuda.synchronize()
        a, b = to_np(y_ws), to_np(y_na)
        err = oracle.max_rel_row_error(b, a)
        print(f"  no-alloc vs workspace: max row rel err {err:.3e}, bitwise equal {np.array_equal(a, b)}", flush=True)
        assert err <= TOL["bf16"]
        assert np.array_equal(a, b)
        assert oracle.max_rel_row_error(b, y_ref) <= TOL["bf16"]


def test_noalloc_oversize_is_rejected():
    cc = W.cached("noalloc_c", 503, [200], [30])
    args, _ = _cached_case(cc)
    y = torch.empty_like(args[1])
    # claim 65,536 new rows (256 keys, within the page table): a workspace of
    # 128 MiB, more than the scratch holds; the call returns before any launch
    q, u, ts, off, lens, _, _, cache, p = args
    c = cache.c_struct(p)
    pc = p.c_struct(None)
    need = hs.hstu_workspace_size(hs.HSTU_FN_CACHED, p, 1, 65536, 256)
    assert need > hs.HSTU_NOALLOC_SCRATCH_BYTES
    r = hs.lib().hstu_attn_fwd_cached_noalloc(ctypes.byref(pc), 1, off.data_ptr(), lens.data_ptr(), 65536, 256,
                                              65536, q.data_ptr(), u.data_ptr(), ts.data_ptr(), ctypes.byref(c),
                                              y.data_ptr(), None)
    assert r == 3  # HSTU_ERR_WORKSPACE
