"""GPU parity of the library's own dense product (hstu_matmul_bf16, the
layer's f1 with SiLU + U/V/Q/K split and its f2) against the oracle's dense
product, through the C ABI. Inputs are bf16 values, so the oracle's fp64
product is exact; the GPU accumulates in fp32 and rounds the output to bf16
(relative 2^-9), so the bar is the forward's bf16 bar on row-relative error."""
import numpy as np
import pytest
import torch

import hstu_jagged_silu_amd as hs
import oracle
import workloads as W

from devutil import TOL, dev, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K", [(300, 256, 64), (1, 256, 64), (1000, 512, 128), (256, 768, 1024), (4097, 1024, 256)])
def test_plain_product(M, N, K):
    a, b = W.dense_operands(M + N + K, M, N, K)
    c = hs.hstu_matmul_bf16(dev(a, torch.bfloat16), dev(b, torch.bfloat16))
    torch.cuda.synchronize()
    err = oracle.max_rel_row_error(to_np(c), oracle.dense(a, b))
    print(f"M={M} N={N} K={K}: max row rel err {err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("M,w,K", [(777, 64, 128), (4097, 256, 1024), (129, 512, 64)])
def test_silu_split_product(M, w, K):
    N = 4 * w
    a, b = W.dense_operands(M * 3 + w, M, N, K)
    c = hs.hstu_matmul_bf16(dev(a, torch.bfloat16), dev(b, torch.bfloat16), epilogue=hs.HSTU_EPI_SILU_SPLIT,
                            split_width=w)
    torch.cuda.synchronize()
    ref = oracle.dense(a, b, apply_silu=True, split_width=w)
    got = to_np(c)
    for i in range(4):
        err = oracle.max_rel_row_error(got[i], ref[i])
        print(f"M={M} w={w} K={K} block {i}: max row rel err {err:.3e}")
        assert err <= TOL["bf16"]


def test_layer_shapes_f1_f2():
    """The 16-user lognormal layer workload: X [T, 1024] W1 [1024, 4096] with SiLU + split, then f2."""
    inp = W.full_layer()
    T, E = inp.x.shape
    HD = inp.num_heads * inp.head_dim
    x, w1, w2 = dev(inp.x, torch.bfloat16), dev(inp.w1, torch.bfloat16), dev(inp.w2, torch.bfloat16)
    uvqk = hs.hstu_matmul_bf16(x, w1, epilogue=hs.HSTU_EPI_SILU_SPLIT, split_width=HD)
    y = hs.hstu_matmul_bf16(uvqk[0].contiguous(), w2)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(T - 8, T), np.random.default_rng(3).integers(0, T, 64)]))
    ref = oracle.dense(inp.x[rows], inp.w1, apply_silu=True, split_width=HD)
    got = to_np(uvqk)
    for i in range(4):
        assert oracle.max_rel_row_error(got[i][rows], ref[i]) <= TOL["bf16"]
    # f2 on the GPU's own U (bf16) as input
    u = got[0][rows].astype(np.float32)
    assert oracle.max_rel_row_error(to_np(y)[rows], oracle.dense(u, inp.w2)) <= TOL["bf16"]


def test_rejects_unsupported_shapes():
    a = torch.zeros((10, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hs.HstuError):
        hs.hstu_matmul_bf16(a, torch.zeros((64, 100), dtype=torch.bfloat16, device="cuda"))
    assert hs.hstu_matmul_bf16(a[:0], torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")).shape == (0, 256)
