"""The library's page allocator (host code; VeriCache review, §Implementation notes, "Page table
tricks": compressed-resident and full-transient pages kept apart) against a plain model of its
definition: two disjoint id ranges, each with a LIFO free stack that starts with the lowest id
on top; a failed call changes nothing."""
import numpy as np
import pytest

from lossless_kv_cache_vc_amd import vc
from lossless_kv_cache_vc_amd.vc import PAGE_RESIDENT as RES, PAGE_TRANSIENT as TR


class Model:
    def __init__(self, nb, nr):
        self.nr = nr
        self.free = {RES: list(range(nr - 1, -1, -1)), TR: list(range(nb - 1, nr - 1, -1))}
        self.used = set()

    def alloc(self, kind, n):
        if len(self.free[kind]) < n:
            return None
        out = [self.free[kind].pop() for _ in range(n)]
        self.used.update(out)
        return out

    def release(self, kind, ids):
        ok = all(i in self.used and (i < self.nr) == (kind == RES) for i in ids) and len(set(ids)) == len(ids)
        if ok:
            for i in ids:
                self.used.discard(i)
                self.free[kind].append(i)
        return ok


def _expect(code, fn):
    with pytest.raises(vc.VCError) as e:
        fn()
    assert e.value.code == code, str(e.value)


def test_fresh_allocator_hands_out_ascending_ids_per_kind():
    a = vc.PageAllocator(10, 4)
    assert a.free_count(RES) == 4 and a.free_count(TR) == 6
    assert a.alloc(RES, 3) == [0, 1, 2]
    assert a.alloc(TR, 2) == [4, 5]
    a.release(RES, [1])
    assert a.alloc(RES, 1) == [1]          # LIFO: the freed block comes back first
    _expect(vc.VC_ENOMEM, lambda: a.alloc(RES, 2))
    assert a.free_count(RES) == 1          # nothing was taken by the failed call
    assert a.free_count(2) == -1


def test_bad_releases_change_nothing():
    a = vc.PageAllocator(8, 4)
    r = a.alloc(RES, 2)
    t = a.alloc(TR, 2)
    _expect(vc.VC_EINVAL, lambda: a.release(TR, [r[0]]))          # other kind
    _expect(vc.VC_EINVAL, lambda: a.release(RES, [3]))            # not allocated
    _expect(vc.VC_EINVAL, lambda: a.release(RES, [r[0], r[0]]))   # twice in one call
    _expect(vc.VC_EINVAL, lambda: a.release(RES, [r[0], 99]))     # out of range, after a good id
    assert a.free_count(RES) == 2 and a.free_count(TR) == 2
    a.release(RES, r)
    _expect(vc.VC_EINVAL, lambda: a.release(RES, r))              # double free
    a.release(TR, t)
    assert a.free_count(RES) == 4 and a.free_count(TR) == 4


def test_bad_creation_and_kinds():
    _expect(vc.VC_EINVAL, lambda: vc.PageAllocator(4, 5))
    _expect(vc.VC_EINVAL, lambda: vc.PageAllocator(-1, 0))
    a = vc.PageAllocator(4, 2)
    _expect(vc.VC_EINVAL, lambda: a.alloc(7, 1))
    _expect(vc.VC_EINVAL, lambda: a.alloc(RES, -1))
    assert a.alloc(RES, 0) == []


def test_random_sequences_follow_the_model():
    rng = np.random.default_rng(0)
    for trial in range(20):
        nb = int(rng.integers(1, 200))
        nr = int(rng.integers(0, nb + 1))
        a, m = vc.PageAllocator(nb, nr), Model(nb, nr)
        live = {RES: [], TR: []}
        for _ in range(300):
            kind = int(rng.integers(0, 2))
            if rng.random() < 0.55:
                n = int(rng.integers(0, 12))
                want = m.alloc(kind, n)
                if want is None:
                    _expect(vc.VC_ENOMEM, lambda: a.alloc(kind, n))
                else:
                    assert a.alloc(kind, n) == want
                    live[kind] += want
            elif live[kind]:
                k = int(rng.integers(1, len(live[kind]) + 1))
                pick = list(rng.choice(live[kind], size=k, replace=False))
                assert m.release(kind, pick)
                a.release(kind, pick)
                live[kind] = [i for i in live[kind] if i not in pick]
            assert a.free_count(RES) == len(m.free[RES]) and a.free_count(TR) == len(m.free[TR])
        # kinds never mix, ids never repeat
        assert all(i < nr for i in live[RES]) and all(i >= nr for i in live[TR])
        assert len(set(live[RES]) | set(live[TR])) == len(live[RES]) + len(live[TR])


def test_page_rows_grow_and_shrink():
    a = vc.PageAllocator(16, 8)
    row = np.full(6, -1, dtype=np.int32)
    a.extend_row(RES, row, 0, 17)                 # 17 tokens: 2 pages
    assert list(row) == [0, 1, -1, -1, -1, -1]
    a.extend_row(RES, row, 17, 32)                # still 2 pages
    assert list(row[:3]) == [0, 1, -1]
    a.extend_row(RES, row, 32, 33)                # a third page
    assert list(row[:3]) == [0, 1, 2] and a.free_count(RES) == 5
    _expect(vc.VC_EINVAL, lambda: a.extend_row(RES, row, 33, 16 * 6 + 1))   # beyond the row
    _expect(vc.VC_EINVAL, lambda: a.extend_row(RES, row, 33, 20))           # shrinking is truncate
    small = vc.PageAllocator(3, 3)
    r2 = np.full(4, -1, dtype=np.int32)
    small.extend_row(RES, r2, 0, 32)
    _expect(vc.VC_ENOMEM, lambda: small.extend_row(RES, r2, 32, 64))       # needs 2, 1 free
    assert list(r2) == [0, 1, -1, -1] and small.free_count(RES) == 1        # unchanged
    # a rollback across a page boundary frees the page; within a page it frees nothing
    a.truncate_row(RES, row, 33, 32)
    assert list(row[:3]) == [0, 1, -1] and a.free_count(RES) == 6
    a.truncate_row(RES, row, 32, 20)
    assert list(row[:2]) == [0, 1] and a.free_count(RES) == 6
    a.truncate_row(RES, row, 20, 0)
    assert (row == -1).all() and a.free_count(RES) == 8
    _expect(vc.VC_EINVAL, lambda: a.truncate_row(RES, row, 10, 20))


def test_transient_full_cache_cycle():
    """A full cache reloaded into transient pages for one verify and freed after it leaves the
    resident pool untouched."""
    a = vc.PageAllocator(40, 24)
    comp = np.full(8, -1, dtype=np.int32)
    a.extend_row(RES, comp, 0, 100)
    for _ in range(3):
        full = np.full(16, -1, dtype=np.int32)
        a.extend_row(TR, full, 0, 250)
        assert (full[:16] >= 24).all()
        a.truncate_row(TR, full, 250, 0)
        assert a.free_count(TR) == 16
    assert a.free_count(RES) == 24 - 7 and (comp[:7] < 24).all()
