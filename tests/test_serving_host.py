"""Host side of the cached serving loop (no GPU): what begin() reserves and
returns, the limits fixed at construction, commit and its single use."""
import numpy as np
import pytest
import torch

hs = pytest.importorskip("hstu_jagged_silu_amd")
from hstu_jagged_silu_amd.serving import CachedServing  # noqa: E402


def _srv(**kw):
    p = hs.LayerParams(num_heads=1, head_dim=32, dtype=torch.bfloat16)
    args = dict(num_pages=6, max_pages_per_seq=3, max_users=3, max_batch=2, max_new_tokens=200)
    args.update(kw)
    return CachedServing([p, p], device="cpu", **args)


def test_begin_commit_and_growth():
    srv = _srv()
    assert srv.outputs[0].shape == (200, 32) and srv.workspace.numel() > 0
    req = srv.begin([7, 8], [70, 10])
    assert list(req.cache_lens) == [0, 0] and list(req.n_new) == [70, 10] and list(req.new_offsets) == [0, 70, 80]
    assert (req.page_table[0] >= 0).sum() == 2 and (req.page_table[1] >= 0).sum() == 1
    srv.commit(req)
    with pytest.raises(ValueError):
        srv.commit(req)
    req = srv.begin([7], [130])                          # only the 60 new rows are sent
    assert list(req.cache_lens) == [70] and req.total_new == 60
    srv.commit(req)
    assert srv.pm.lookup(7) == 130


def test_limits_fixed_at_construction():
    srv = _srv()
    with pytest.raises(ValueError, match="max_batch"):
        srv.begin([1, 2, 3], [1, 1, 1])
    with pytest.raises(ValueError, match="max_new_tokens"):
        srv.begin([1, 2], [150, 60])
    with pytest.raises(ValueError, match="max_pages_per_seq"):
        srv.begin([1], [3 * 64 + 1])
    srv.commit(srv.begin([1], [100]))
    with pytest.raises(ValueError, match="shorter"):
        srv.begin([1], [99])
    assert srv.pm.stats()["users"] == 1


def test_uncommitted_request_is_replaced():
    srv = _srv()
    srv.begin([4], [130])                                # never run or committed
    assert srv.pm.lookup(4) == 0 and srv.pm.stats()["free_pages"] == 3
    req = srv.begin([4], [130])                          # same pages, nothing leaked
    assert list(req.cache_lens) == [0] and srv.pm.stats()["free_pages"] == 3
    srv.commit(req)
    assert srv.pm.lookup(4) == 130
