"""Helpers shared by the GPU tests: move generated inputs to the device and
call the library through its binding."""
import numpy as np
import torch

import hstu_jagged_silu_amd as hs

from tolerances import GRAD_RSS_BF16, TOL  # noqa: F401


def tdtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def params_for(inp_dtype, H, d, tables=None, **kw):
    pos = tables.pos if tables is not None else None
    tim = tables.time if tables is not None else None
    return hs.LayerParams(num_heads=H, head_dim=d, dtype=tdtype(inp_dtype),
                          pos_tab=None if pos is None else dev(pos),
                          time_tab=None if tim is None else dev(tim), **kw)


def run_full(inp, params=None, **kw):
    dt = tdtype(inp.dtype)
    p = params or params_for(inp.dtype, inp.num_heads, inp.head_dim, inp.tables)
    y = hs.hstu_attn_fwd(dev(inp.q, dt), dev(inp.k, dt), dev(inp.v, dt), dev(inp.u, dt), dev(inp.ts),
                         dev(inp.seq_offsets), max(1, inp.max_len), p, **kw)
    torch.cuda.synchronize()
    return y


def to_np(y):
    return y.float().cpu().numpy().astype(np.float64)
