"""GPU parity of the backward (hstu_attn_bwd) against the fp64 oracle's
hstu_full_bwd, through the C ABI.

Error metric: per output, max over rows of ||g - g*||_inf / ||m*||_inf, where
m* is the oracle's same sum over absolute values of the terms (its
"magnitude"; bias tables and affine terms are one row each). A gradient
entry is a sum of products whose factors reach the MFMAs rounded to bf16
(dO, P, dS; relative error at most 2^-8 each) and is returned rounded to
bf16, so its error is bounded by a few times 2^-8 of that magnitude; the
bar is 2e-2 (about 5 x 2^-8), the forward's bf16 bar. Measuring against the
value itself instead would fail rows whose gradient is small only through
cancellation (the first token of a user, for one)."""
import numpy as np
import pytest
import torch

import hstu_jagged_silu_amd as hs
import oracle
import workloads as W

from devutil import TOL, dev, to_np

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def run_bwd(inp, dy, per_head_tables=False, affine=None, alpha=1.0, norm_n=0, tables=True, **kw):
    H, d = inp.num_heads, inp.head_dim
    pos = inp.tables.pos if tables else None
    tim = inp.tables.time if tables else None
    if per_head_tables and pos is not None:
        pos = np.stack([pos * (1 + 0.5 * h) for h in range(H)]).astype(np.float32)
    ln_w, ln_b = affine if affine is not None else (None, None)
    p = hs.LayerParams(num_heads=H, head_dim=d, dtype=BF, alpha=alpha, norm_n=norm_n,
                       pos_tab=None if pos is None else dev(pos), time_tab=None if tim is None else dev(tim),
                       ln_w=None if ln_w is None else dev(ln_w), ln_b=None if ln_b is None else dev(ln_b))
    g = hs.hstu_attn_bwd(dev(inp.q, BF), dev(inp.k, BF), dev(inp.v, BF), dev(inp.u, BF), dev(inp.ts),
                         dev(inp.seq_offsets), max(1, inp.max_len), dev(dy, BF), p, **kw)
    torch.cuda.synchronize()
    ref = oracle.hstu_full_bwd(inp.q, inp.k, inp.v, inp.u, inp.ts, inp.seq_offsets, dy, pos, tim, alpha, norm_n,
                               ln_w, ln_b, magnitudes=True)
    return g, ref


def check(g, ref, tol=TOL["bf16"], label=""):
    errs = {}
    for name, rname in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("du", "du"), ("d_pos_tab", "dpos"),
                        ("d_time_tab", "dtime"), ("d_ln_w", "dgamma"), ("d_ln_b", "dbeta")):
        if ref[rname] is None:
            assert g[name] is None, name
            continue
        r = np.asarray(ref[rname])
        m = np.asarray(ref["mag_" + rname])
        x = to_np(g[name])
        if rname in ("dq", "dk", "dv"):
            x, r, m = (t.reshape(r.shape[0], -1) for t in (x, r, m))
        errs[name] = oracle.max_rel_err_vs_magnitude(x, r, m)
    print(label, " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= tol, (k, v)


@pytest.mark.parametrize("d", [128, 64, 32])
def test_ragged_lengths_all_gradients(d):
    inp = W.jagged(f"bwd_ragged_d{d}", 61, [1, 77, 200, 130, 0, 64, 129], 2, d, "bf16", 128, 128)
    dy = W.upstream_grad(62, inp.u.shape)
    g, ref = run_bwd(inp, dy, affine=W.affine_terms(63, 2 * d))
    check(g, ref, label=f"ragged d={d}")


def test_largest_position_table():
    # the backward's largest position table (512 buckets), users longer than it
    inp = W.jagged("bwd_maxpos", 66, [700, 300], 2, 64, "bf16", 512, 64)
    inp.tables.pos *= 25.0
    dy = W.upstream_grad(67, inp.u.shape)
    g, ref = run_bwd(inp, dy, affine=W.affine_terms(68, 2 * 64))
    check(g, ref, label="512 position buckets")


def test_per_head_tables_alpha_norm_no_affine():
    inp = W.jagged("bwd_opts", 64, [300, 45, 190], 4, 128, "bf16", 64, 40)
    dy = W.upstream_grad(65, inp.u.shape)
    g, ref = run_bwd(inp, dy, per_head_tables=True, alpha=0.35, norm_n=512)
    check(g, ref, label="per-head tables, alpha, N")


def test_no_tables():
    inp = W.jagged("bwd_notab", 66, [150, 260], 2, 128, "bf16", 0, 0)
    dy = W.upstream_grad(67, inp.u.shape)
    g, ref = run_bwd(inp, dy, tables=False, affine=W.affine_terms(68, 256))
    check(g, ref, label="no tables")


def test_training_shape_config():
    """Batch 32, lengths U[64, 1024], 4 x 128, position 128 + time 128 buckets: every gradient."""
    inp = W.training_shape()
    dy = W.upstream_grad(69, inp.u.shape)
    g, ref = run_bwd(inp, dy, affine=W.affine_terms(70, 512))
    check(g, ref, label="training shape")


def test_repeat_is_bitwise_and_workspace_reuse():
    inp = W.jagged("bwd_rep", 71, [333, 64, 512], 2, 128, "bf16", 128, 128)
    dy = W.upstream_grad(72, inp.u.shape)
    H, d = 2, 128
    w, b = W.affine_terms(73, H * d)
    p = hs.LayerParams(num_heads=H, head_dim=d, dtype=BF, pos_tab=dev(inp.tables.pos), time_tab=dev(inp.tables.time),
                       ln_w=dev(w), ln_b=dev(b))
    nbytes = hs.hstu_workspace_size(hs.HSTU_FN_FULL_BWD, p, 3, inp.total, 512)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    args = (dev(inp.q, BF), dev(inp.k, BF), dev(inp.v, BF), dev(inp.u, BF), dev(inp.ts), dev(inp.seq_offsets), 512,
            dev(dy, BF), p)
    a = hs.hstu_attn_bwd(*args, workspace=ws)
    torch.cuda.synchronize()
    a = {k: v.clone() for k, v in a.items()}
    ws.fill_(0xFF)
    c = hs.hstu_attn_bwd(*args, workspace=ws)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], c[k]), k


def test_single_token_users_and_empty_batch():
    inp = W.jagged("bwd_single", 74, [1, 1, 2], 2, 128, "bf16", 128, 128)
    dy = W.upstream_grad(75, inp.u.shape)
    g, ref = run_bwd(inp, dy, affine=W.affine_terms(76, 256))
    check(g, ref, label="single tokens")
    # an empty batch writes zero table and affine gradients
    e = W.jagged("bwd_empty", 77, [0, 0], 2, 128, "bf16", 128, 128)
    w, b = W.affine_terms(78, 256)
    p = hs.LayerParams(num_heads=2, head_dim=128, dtype=BF, pos_tab=dev(e.tables.pos), time_tab=dev(e.tables.time),
                       ln_w=dev(w), ln_b=dev(b))
    z = torch.zeros((0, 2, 128), dtype=BF, device="cuda")
    zu = torch.zeros((0, 256), dtype=BF, device="cuda")
    out = hs.hstu_attn_bwd(z, z, z, zu, torch.zeros(0, dtype=torch.int64, device="cuda"), dev(e.seq_offsets), 1,
                           zu, p)
    torch.cuda.synchronize()
    for k in ("d_pos_tab", "d_time_tab", "d_ln_w", "d_ln_b"):
        assert not torch.any(out[k]), k
