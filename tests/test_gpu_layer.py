"""GPU parity of the full HSTU layer (f1 + SiLU, split U/V/Q/K, attention,
f2) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import hstu_jagged_silu_amd as hs
import oracle
import workloads as W

from devutil import TOL, dev, to_np

pytestmark = pytest.mark.gpu


PRODUCTS = [hs.HSTU_PRODUCTS_HIPBLASLT, hs.HSTU_PRODUCTS_OWN, hs.HSTU_PRODUCTS_AUTO]


def run_layer(inp, **kw):
    bf = torch.bfloat16
    p = hs.LayerParams(num_heads=inp.num_heads, head_dim=inp.head_dim, dtype=bf,
                       pos_tab=dev(inp.tables.pos), time_tab=dev(inp.tables.time))
    out = hs.hstu_layer_fwd(dev(inp.x, bf), dev(inp.w1, bf), dev(inp.w2, bf), dev(inp.ts), dev(inp.seq_offsets),
                            max(1, inp.max_len), p, **kw)
    torch.cuda.synchronize()
    return to_np(out)


@pytest.mark.parametrize("products", PRODUCTS)
def test_small_layer_all_rows(products):
    inp = W.full_layer(seed=21, batch=4, embed=256, num_heads=2, head_dim=128, lengths=[1, 77, 200, 130])
    y = run_layer(inp, products=products)
    y_ref = oracle.hstu_layer(inp.x, inp.w1, inp.w2, inp.ts, inp.seq_offsets, inp.num_heads, inp.head_dim,
                              inp.tables.pos, inp.tables.time)
    err = oracle.max_rel_row_error(y, y_ref)
    print(f"small layer max row rel err {err:.3e}")
    assert err <= TOL["bf16"]


def test_layer_head_dim_64_and_empty_user():
    inp = W.full_layer(seed=22, batch=3, embed=128, num_heads=4, head_dim=64, lengths=[65, 0, 190])
    y = run_layer(inp)
    y_ref = oracle.hstu_layer(inp.x, inp.w1, inp.w2, inp.ts, inp.seq_offsets, inp.num_heads, inp.head_dim,
                              inp.tables.pos, inp.tables.time)
    assert oracle.max_rel_row_error(y, y_ref) <= TOL["bf16"]


@pytest.mark.parametrize("products", PRODUCTS)
def test_full_size_layer_sampled_rows(products):
    """Batch 16, lognormal lengths (median 2,048) capped at 8,192, E = 1,024, 8 x 128: sampled rows,
    from the shortest users and from the longest."""
    inp = W.full_layer()
    y = run_layer(inp, products=products)
    assert np.isfinite(y).all()
    off = inp.seq_offsets
    rng = np.random.default_rng(11)
    # rows from the three shortest non-empty users and the two longest (8,192
    # tokens: the last query tile, every key tile) plus the first and last row
    # of the whole batch; the oracle recomputes f1 for each sampled user's prefix
    lens = np.diff(off)
    order = [b for b in np.argsort(lens, kind="stable") if lens[b] > 0]
    users = order[:3] + order[-2:]
    rows = [0, int(off[-1]) - 1]
    for b in users:
        s0, s1 = int(off[b]), int(off[b + 1])
        rows += [s0, s1 - 1] + list(rng.integers(s0, s1, size=2))
    rows = np.unique(np.array(rows, dtype=np.int64))
    y_ref = oracle.hstu_layer(inp.x, inp.w1, inp.w2, inp.ts, inp.seq_offsets, inp.num_heads, inp.head_dim,
                              inp.tables.pos, inp.tables.time, rows=rows)
    err = oracle.max_rel_row_error(y[rows], y_ref)
    print(f"full-size layer ({inp.total} tokens) sampled rows max row rel err {err:.3e}")
    assert err <= TOL["bf16"]


def test_layer_repeat_is_deterministic_and_workspace_reuse():
    inp = W.full_layer(seed=23, batch=2, embed=128, num_heads=2, head_dim=128, lengths=[300, 45])
    p = hs.LayerParams(num_heads=2, head_dim=128, dtype=torch.bfloat16, pos_tab=dev(inp.tables.pos),
                       time_tab=dev(inp.tables.time))
    nbytes = hs.hstu_layer_workspace_size(p, 128, 2, inp.total, 300)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    bf = torch.bfloat16
    args = (dev(inp.x, bf), dev(inp.w1, bf), dev(inp.w2, bf), dev(inp.ts), dev(inp.seq_offsets), 300, p)
    a = to_np(hs.hstu_layer_fwd(*args, workspace=ws))
    ws.fill_(0xFF)
    b = to_np(hs.hstu_layer_fwd(*args, workspace=ws))
    torch.cuda.synchronize()
    assert np.array_equal(a, b)
