"""Host logic of the paged KV-cache manager (hstu_pm_*, no GPU): allocation,
growth across page boundaries, LRU eviction, pinning of the request's own
users, failure atomicity, reservations that are replaced or only partly
committed, and a randomized comparison with a small Python model of the
documented rules."""
import numpy as np
import pytest

hs = pytest.importorskip("hstu_jagged_silu_amd")


def pages(n):
    return (n + 63) // 64


def test_allocation_and_growth():
    pm = hs.PageManager(num_pages=10, max_pages_per_seq=4, max_users=3)
    lens, table, ev = pm.reserve([7, 8], [70, 10])
    assert list(lens) == [0, 0] and ev == 0
    assert (table[0] >= 0).sum() == 2 and (table[1] >= 0).sum() == 1
    assert len(set(table[table >= 0].tolist())) == 3
    pm.commit([7, 8], [70, 10])
    assert pm.lookup(7) == 70 and pm.lookup(8) == 10 and pm.lookup(9) == -1
    lens, table2, _ = pm.reserve([7], [60])            # 130 tokens: a third page
    assert list(lens) == [70]
    assert list(table2[0, :2]) == list(table[0, :2]) and table2[0, 2] >= 0 and table2[0, 3] == -1
    pm.commit([7], [60])
    assert pm.stats() == {"free_pages": 6, "users": 2, "evictions": 0}


def test_lru_eviction_and_pinning():
    pm = hs.PageManager(num_pages=4, max_pages_per_seq=4, max_users=8)
    for u in (1, 2):
        pm.reserve([u], [128])
        pm.commit([u], [128])
    assert pm.lookup(1) == 128                          # user 1 is now the most recently used
    lens, _, ev = pm.reserve([3], [64])                 # needs one page: evicts user 2
    assert ev == 1 and pm.lookup(2) == -1 and pm.lookup(1) == 128
    pm.commit([3], [64])
    # one page is free; user 1 needs two more and is in the request, so user 3
    # goes even though it is newer
    lens, _, ev = pm.reserve([1], [128])
    assert ev == 1 and pm.lookup(3) == -1 and list(lens) == [128]


def test_failures_change_nothing():
    pm = hs.PageManager(num_pages=4, max_pages_per_seq=3, max_users=2)
    pm.reserve([1], [128])
    pm.commit([1], [128])
    before = pm.stats()
    with pytest.raises(hs.HstuError, match="WORKSPACE"):
        pm.reserve([1, 2], [64, 128])                   # 1 + 2 pages while user 1 keeps 2 of 4
    assert pm.stats() == before and pm.lookup(1) == 128
    with pytest.raises(hs.HstuError, match="UNSUPPORTED"):
        pm.reserve([1], [200])                          # beyond 3 pages per user
    with pytest.raises(hs.HstuError, match="INVALID"):
        pm.reserve([5, 5], [1, 1])                      # duplicate id
    with pytest.raises(hs.HstuError, match="INVALID"):
        pm.commit([1], [64])                            # not reserved
    with pytest.raises(hs.HstuError, match="INVALID"):
        pm.evict(42)
    assert pm.stats() == before
    pm.evict(1)
    assert pm.stats()["free_pages"] == 4 and pm.lookup(1) == -1


class Model:
    """The documented rules, written independently of the C++ code."""

    def __init__(self, num_pages, max_pages, max_users):
        self.P, self.M, self.U = num_pages, max_pages, max_users
        self.len, self.npages, self.last = {}, {}, {}
        self.clock = 0

    def used_pages(self):
        return sum(self.npages.values())

    def lookup(self, u):
        if u not in self.len:
            return -1
        self.clock += 1
        self.last[u] = self.clock
        return self.len[u]

    def reserve(self, ids, n_new):
        have = {u: self.len.get(u, 0) for u in ids}
        if any(pages(have[u] + n) > self.M for u, n in zip(ids, n_new)):
            return "UNSUPPORTED", None
        need_slots = sum(u not in self.len for u in ids)
        # after the call the batch's users hold exactly pages(len + n) pages
        # each (a reservation never committed is replaced, not added to)
        want = sum(pages(have[u] + n) for u, n in zip(ids, n_new))
        pinned = [u for u in ids if u in self.len]
        if need_slots > self.U - len(pinned) or want > self.P:
            return "WORKSPACE", None
        ev = 0
        others = lambda: sum(p for u, p in self.npages.items() if u not in ids)
        while (self.U - len(self.len) < need_slots) or (others() + want > self.P):
            victim = min((u for u in self.len if u not in pinned), key=lambda u: self.last[u])
            del self.len[victim], self.npages[victim], self.last[victim]
            ev += 1
        lens = []
        for u, n in zip(ids, n_new):
            lens.append(self.len.get(u, 0))
            self.len.setdefault(u, 0)
            self.npages[u] = pages(self.len[u] + n)
            self.clock += 1
            self.last[u] = self.clock
        return "OK", (lens, ev)

    def commit(self, ids, n_new):
        for u, n in zip(ids, n_new):
            self.len[u] += n


def test_randomized_against_model():
    rng = np.random.default_rng(0)
    P, M, U = 40, 6, 7
    pm, ref = hs.PageManager(P, M, U), Model(P, M, U)
    for _ in range(400):
        if rng.random() < 0.2:
            u = int(rng.integers(0, 12))
            assert pm.lookup(u) == ref.lookup(u)
            continue
        ids = rng.choice(12, size=int(rng.integers(1, 5)), replace=False).tolist()
        n_new = rng.integers(0, 150, size=len(ids)).tolist()
        status, res = ref.reserve(ids, n_new)
        if status != "OK":
            with pytest.raises(hs.HstuError, match=status):
                pm.reserve(ids, n_new)
            continue
        lens, table, ev = pm.reserve(ids, n_new)
        assert list(lens) == res[0] and ev == res[1]
        # each user's page row: exactly pages(len + n) leading ids, no page shared
        for i, (u, n) in enumerate(zip(ids, n_new)):
            k = pages(res[0][i] + n)
            assert (table[i, :k] >= 0).all() and (table[i, k:] == -1).all()
        assert len(set(table[table >= 0].tolist())) == int((table >= 0).sum())
        # commit all, part (fewer tokens than reserved) or nothing (an
        # abandoned reservation, replaced by the user's next reserve)
        r = rng.random()
        if r < 0.6:
            done = n_new
        elif r < 0.8:
            done = [int(rng.integers(0, n + 1)) for n in n_new]
        else:
            done = None
        if done is not None:
            pm.commit(ids, done)
            ref.commit(ids, done)
        st = pm.stats()
        assert st["users"] == len(ref.len) and st["free_pages"] == P - ref.used_pages()
    for u in list(ref.len):
        pm.evict(u)
    assert pm.stats()["free_pages"] == P and pm.stats()["users"] == 0


def test_repeated_reserve_reuses_pages():
    # two reserves without a commit between them: the second reuses the
    # first's pages, and eviction returns every page to the pool
    pm = hs.PageManager(num_pages=6, max_pages_per_seq=4, max_users=2)
    _, t1, _ = pm.reserve([1], [130])                   # 3 pages
    assert pm.stats()["free_pages"] == 3
    _, t2, _ = pm.reserve([1], [130])                   # the same 3 pages again
    assert list(t2[0]) == list(t1[0]) and pm.stats()["free_pages"] == 3
    _, t3, _ = pm.reserve([1], [10])                    # a smaller request gives 2 back
    assert list(t3[0, :1]) == list(t1[0, :1]) and (t3[0, 1:] == -1).all()
    assert pm.stats()["free_pages"] == 5
    pm.commit([1], [10])
    assert pm.lookup(1) == 10
    _, t4, _ = pm.reserve([1], [200])                   # 210 tokens: 4 pages, the first kept
    assert t4[0, 0] == t1[0, 0] and (t4[0] >= 0).all() and len(set(t4[0].tolist())) == 4
    pm.commit([1], [100])                               # part of the reservation
    assert pm.stats()["free_pages"] == 2                # the 4th page stays reserved
    pm.evict(1)
    assert pm.stats() == {"free_pages": 6, "users": 0, "evictions": 1}


def test_reserve_twice_then_full_pool():
    # a reservation that is replaced must not shrink the pool: after it the
    # whole pool still fits one request
    pm = hs.PageManager(num_pages=4, max_pages_per_seq=4, max_users=2)
    pm.reserve([1], [256])
    pm.reserve([1], [256])
    pm.commit([1], [256])
    assert pm.stats()["free_pages"] == 0
    pm.evict(1)
    lens, table, ev = pm.reserve([2], [256])
    assert ev == 0 and (table[0] >= 0).all() and pm.stats()["free_pages"] == 0
