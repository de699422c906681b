"""CPU tests of the expert-slot cache policy (LRU over (layer, expert) keys).

The C++ policy (expert_ffn_execution_amd/csrc/slot_policy.h) runs behind a
small shim with a mock copy engine; its decisions are compared with an
independent textbook LRU model written here with an OrderedDict.
"""
import ctypes as C
import os
import subprocess
from collections import OrderedDict

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "native", "policy_shim.cpp")
LIB = os.path.join(HERE, "native", "_build", "libpolicy_shim.so")

OK, INVALID, UNSUPPORTED, CAPACITY, BUSY, HIP, WARN = 0, 1, 2, 3, 5, 6, 100
GLOBAL, PER_LAYER = 0, 1


def build_shim():
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-Wall",
                    f"-I{os.path.join(ROOT, 'include')}", SRC, "-o", LIB], check=True)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < max(
            os.path.getmtime(SRC),
            os.path.getmtime(os.path.join(ROOT, "expert_ffn_execution_amd", "csrc", "slot_policy.h"))):
        build_shim()
    L = C.CDLL(LIB)
    P = C.c_void_p
    L.pol_create.restype = P
    L.pol_create.argtypes = [C.c_int] * 4
    for f in ("pol_destroy", "pol_complete_all", "pol_fail_next_copy"):
        getattr(L, f).argtypes = [P]
    L.pol_map.argtypes = [P, C.c_int, P, C.c_int, P, P]
    L.pol_release.argtypes = [P, C.c_int]
    L.pol_prefetch.argtypes = [P, C.c_int, P, C.c_int, P]
    L.pol_evict.argtypes = [P, C.c_int, C.c_int]
    L.pol_lookup.argtypes = [P, C.c_int, C.c_int]
    L.pol_resize.argtypes = [P, C.c_int, C.c_int]
    L.pol_set_auto_complete.argtypes = [P, C.c_int]
    L.pol_log.argtypes = [P, P, C.c_int]
    L.pol_stats.argtypes = [P, P]
    return L


class Cache:
    def __init__(self, lib, L, E, S, scope=GLOBAL):
        self.lib, self.h = lib, lib.pol_create(L, E, S, scope)

    def __del__(self):
        self.lib.pol_destroy(self.h)

    def map(self, layer, experts):
        arr = (C.c_int * max(1, len(experts)))(*experts)
        slots = (C.c_int * max(1, len(experts)))()
        st = (C.c_int * 4)()
        r = self.lib.pol_map(self.h, layer, arr, len(experts), slots, st)
        return r, list(slots)[:len(experts)], list(st)

    def prefetch(self, layer, experts):
        arr = (C.c_int * max(1, len(experts)))(*experts)
        got = C.c_int()
        r = self.lib.pol_prefetch(self.h, layer, arr, len(experts), C.byref(got))
        return r, got.value

    def release(self, layer):
        return self.lib.pol_release(self.h, layer)

    def evict(self, layer, expert=-1):
        return self.lib.pol_evict(self.h, layer, expert)

    def lookup(self, layer, expert):
        return self.lib.pol_lookup(self.h, layer, expert)

    def log(self):
        buf = (C.c_int * 65536)()
        n = self.lib.pol_log(self.h, buf, 65536)
        v = list(buf)[:n]
        return [tuple(v[i:i + 4]) for i in range(0, n, 4)]

    def stats(self):
        out = (C.c_longlong * 12)()
        self.lib.pol_stats(self.h, out)
        keys = ["maps", "demand", "hits", "prefetch_hits", "misses", "prefetch_issued",
                "evictions", "bytes_h2d", "resident", "held", "in_flight", "n_slots"]
        return dict(zip(keys, list(out)))


class RefLRU:
    """Textbook LRU over (layer, expert) keys: free slots are filled lowest first;
    otherwise the least recently used key that is neither held nor part of the
    current request is evicted.  A request touches its resident keys first, then
    brings in its missing keys, each in ascending expert order."""

    def __init__(self, L, E, S, scope=GLOBAL):
        self.S, self.L, self.scope = S, L, scope
        self.slot_of = {}                 # key -> slot
        self.key_at = [None] * S
        self.lru = OrderedDict()          # key -> None, least recent first
        self.held = set()

    def _range(self, layer):
        if self.scope == PER_LAYER:
            w = self.S // self.L
            return range(layer * w, (layer + 1) * w)
        return range(self.S)

    def _victim(self, layer, request):
        rng = self._range(layer)
        for s in rng:
            if self.key_at[s] is None:
                return s
        for key in self.lru:
            s = self.slot_of[key]
            if s in rng and key not in self.held and key not in request:
                return s
        return None

    def _place(self, key, s):
        old = self.key_at[s]
        if old is not None:
            del self.slot_of[old]
            del self.lru[old]
        self.key_at[s] = key
        self.slot_of[key] = s
        self.lru[key] = None

    def map(self, layer, experts):
        req = {(layer, e) for e in experts}
        missing = [e for e in experts if (layer, e) not in self.slot_of]
        rng = self._range(layer)
        room = sum(1 for s in rng if self.key_at[s] is None or
                   (self.key_at[s] not in self.held and self.key_at[s] not in req))
        if len(missing) > room:
            return CAPACITY, None
        for e in experts:
            if (layer, e) in self.slot_of:
                self.lru.move_to_end((layer, e))
                self.held.add((layer, e))
        copies = []
        for e in missing:
            s = self._victim(layer, req)
            self._place((layer, e), s)
            self.held.add((layer, e))
            copies.append((s, layer, e))
        return OK, ([self.slot_of[(layer, e)] for e in experts], copies)

    def prefetch(self, layer, experts):
        req = {(layer, e) for e in experts}
        for e in experts:
            if (layer, e) in self.slot_of:
                self.lru.move_to_end((layer, e))
        copies = []
        for e in experts:
            if (layer, e) in self.slot_of:
                continue
            s = self._victim(layer, req)
            if s is None:
                return WARN, copies
            self._place((layer, e), s)
            copies.append((s, layer, e))
        return OK, copies

    def release(self, layer):
        self.held = {k for k in self.held if k[0] != layer}


def _copies(log):
    return [(s, l, e) for kind, s, l, e in log if kind == 0]


@pytest.mark.parametrize("scope", [GLOBAL, PER_LAYER])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_textbook_lru(lib, scope, seed):
    L, E, S = 4, 16, 24 if scope == GLOBAL else 24
    rng = np.random.default_rng(seed)
    c, ref = Cache(lib, L, E, S, scope), RefLRU(L, E, S, scope)
    skew = np.exp(-1.1 * np.log(np.arange(1, E + 1)))
    skew /= skew.sum()
    for step in range(200):
        layer = step % L
        n = int(rng.integers(1, 6))
        experts = sorted(set(rng.choice(E, size=n, p=skew).tolist()))
        r, slots, _ = c.map(layer, experts)
        rr, payload = ref.map(layer, experts)
        assert r == rr, (step, r, rr)
        if r == OK:
            ref_slots, ref_copies = payload
            assert slots == ref_slots, step
            assert _copies(c.log()) == ref_copies, step
        nxt = (layer + 1) % L
        pf = sorted(set(rng.choice(E, size=int(rng.integers(0, 4)), p=skew).tolist()))
        r1, _ = c.prefetch(nxt, pf)
        r2, ref_copies = ref.prefetch(nxt, pf)
        assert r1 == r2 and _copies(c.log()) == ref_copies, step
        assert c.release(layer) == OK
        ref.release(layer)
        for l2 in range(L):
            for e in range(E):
                assert c.lookup(l2, e) == ref.slot_of.get((l2, e), -1)


def test_held_slots_are_never_evicted(lib):
    c = Cache(lib, 2, 8, 6)
    assert c.map(0, [0, 1, 2, 3])[0] == OK           # held until release
    r, issued = c.prefetch(1, [0, 1, 2, 3, 4])      # only 2 free slots
    assert r == WARN and issued == 2
    for e in range(4):
        assert c.lookup(0, e) >= 0
    assert c.map(1, [0, 1, 2])[0] == CAPACITY        # 2 prefetched + 1 more > room
    c.release(0)
    r, slots, st = c.map(1, [0, 1, 2])
    assert r == OK and st == [3, 0, 2, 1]             # 2 prefetch hits, 1 miss


def test_capacity_error_changes_nothing(lib):
    c = Cache(lib, 1, 16, 4)
    assert c.map(0, [0, 1, 2, 3])[0] == OK
    c.log()
    before = [c.lookup(0, e) for e in range(16)]
    assert c.map(0, [0, 1, 2, 3, 4])[0] == CAPACITY
    assert [c.lookup(0, e) for e in range(16)] == before
    assert c.log() == []


def test_request_never_evicts_its_own_experts(lib):
    c = Cache(lib, 1, 8, 2)
    assert c.map(0, [1])[0] == OK
    c.release(0)
    assert c.map(0, [2])[0] == OK
    c.release(0)
    # expert 1 is the LRU entry; a request for [0, 1] must keep 1 and evict 2
    r, slots, st = c.map(0, [0, 1])
    assert r == OK and st == [2, 1, 0, 1]
    assert c.lookup(0, 1) >= 0 and c.lookup(0, 2) == -1


def test_in_flight_and_held_entries_are_busy(lib):
    c = Cache(lib, 2, 8, 8)
    lib.pol_set_auto_complete(c.h, 0)
    assert c.prefetch(1, [3])[0] == OK
    assert c.evict(1, 3) == BUSY                     # copy in flight
    lib.pol_complete_all(c.h)
    assert c.evict(1, 3) == OK and c.lookup(1, 3) == -1
    lib.pol_set_auto_complete(c.h, 1)
    assert c.map(0, [5])[0] == OK
    assert c.evict(0, 5) == BUSY and c.evict(0) == BUSY
    c.release(0)
    assert c.evict(0) == OK and c.lookup(0, 5) == -1


def test_in_flight_entries_are_not_victims(lib):
    c = Cache(lib, 2, 8, 3)
    lib.pol_set_auto_complete(c.h, 0)
    assert c.prefetch(1, [0, 1, 2]) == (OK, 3)
    assert c.prefetch(0, [4]) == (WARN, 0)           # everything in flight
    lib.pol_complete_all(c.h)
    assert c.prefetch(0, [4]) == (OK, 1)


def test_map_waits_for_in_flight_copies(lib):
    c = Cache(lib, 1, 8, 4)
    lib.pol_set_auto_complete(c.h, 0)
    c.prefetch(0, [2])
    c.log()
    r, slots, st = c.map(0, [2])
    assert r == OK and st == [1, 0, 1, 0]
    assert (1, slots[0], -1, -1) in c.log()          # compute waits on the fill


def test_map_waits_for_landing_copies_it_must_evict(lib):
    """A request that fits once in-flight copies land is served: the host
    waits for the least recently used of them (engine call 4) and evicts it,
    as the textbook LRU (which has no copies in flight) would; a request that
    does not fit even then is refused and changes nothing."""
    c = Cache(lib, 2, 8, 4)
    lib.pol_set_auto_complete(c.h, 0)
    assert c.prefetch(1, [0, 1, 2, 3]) == (OK, 4)            # four copies in flight
    c.log()
    r, slots, st = c.map(0, [5, 6])
    assert r == OK and st == [2, 0, 0, 2]
    waits = [e for e in c.log() if e[0] == 4]
    assert len(waits) == 2 and {w[1] for w in waits} == {0, 1}  # the two oldest: (1, 0), (1, 1)
    assert c.lookup(1, 0) == -1 and c.lookup(1, 1) == -1 and c.lookup(1, 2) >= 0
    c.release(0)
    lib.pol_set_auto_complete(c.h, 1)
    assert c.map(0, [5])[0] == OK                             # held: 1, room: 3
    before = [c.lookup(l, e) for l in range(2) for e in range(8)]
    c.log()
    assert c.map(0, [1, 2, 3, 4, 5])[0] == CAPACITY           # 4 misses > 3 other slots
    assert [c.lookup(l, e) for l in range(2) for e in range(8)] == before and c.log() == []


def test_release_records_last_reader_and_copy_failure_retries(lib):
    c = Cache(lib, 1, 8, 4)
    assert c.map(0, [1, 2])[0] == OK
    c.log()
    c.release(0)
    assert sorted(e[1] for e in c.log() if e[0] == 2) == sorted([c.lookup(0, 1), c.lookup(0, 2)])
    lib.pol_fail_next_copy(c.h)
    assert c.map(0, [5])[0] == HIP
    assert c.lookup(0, 5) == -1                      # not marked resident
    r, _, st = c.map(0, [5])                         # the next map copies again
    assert r == OK and st[3] == 1


def test_stats_and_invalid_lists(lib):
    c = Cache(lib, 2, 8, 8)
    assert c.map(0, [3, 1])[0] == INVALID             # not ascending
    assert c.map(0, [1, 1])[0] == INVALID             # duplicate
    assert c.map(2, [1])[0] == INVALID                # bad layer
    assert c.map(0, [8])[0] == INVALID                # bad expert
    c.map(0, [1, 2])
    c.release(0)
    c.map(0, [1, 3])
    s = c.stats()
    assert s["maps"] == 2 and s["demand"] == 4 and s["hits"] == 1 and s["misses"] == 3
    assert s["bytes_h2d"] == 3 * 1000 and s["resident"] == 3 and s["held"] == 2


# ---------------------------------------------------------------------------
# resize (elastic slot budget)
# ---------------------------------------------------------------------------
def _resize(lib, c, n, moved=False):
    return lib.pol_resize(c.h, n, 1 if moved else 0)


def _ref_resize(ref, n, moved=False):
    """Reference resize: evict least-recently-used keys until the residents
    fit; keys below n stay put, the others move, in ascending old slot, to the
    lowest free slot below n.  Returns the (src, dst) copies."""
    assert not ref.held
    while len(ref.slot_of) > n:
        key = next(iter(ref.lru))
        s = ref.slot_of.pop(key)
        ref.key_at[s] = None
        del ref.lru[key]
    new_at = [None] * n
    for s in range(min(n, ref.S)):
        new_at[s] = ref.key_at[s]
    moves = [(s, s) for s in range(min(n, ref.S)) if moved and new_at[s] is not None]
    d = 0
    for s in range(n, ref.S):
        if ref.key_at[s] is None:
            continue
        while new_at[d] is not None:
            d += 1
        new_at[d] = ref.key_at[s]
        moves.append((s, d))
    ref.key_at, ref.S = new_at, n
    ref.slot_of = {k: s for s, k in enumerate(new_at) if k is not None}
    return sorted(moves)


def _moves(log):
    return sorted((s, d) for kind, s, d, _ in log if kind == 3)


def test_resize_shrink_evicts_lru_and_relocates(lib):
    c = Cache(lib, 1, 16, 8)
    for e in range(8):                     # LRU order: 0 (oldest) .. 7
        assert c.map(0, [e])[0] == OK
        c.release(0)
    c.log()
    assert _resize(lib, c, 5) == OK
    assert [c.lookup(0, e) for e in range(3)] == [-1, -1, -1]     # three oldest evicted
    # experts 3, 4 kept slots 3, 4; experts 5, 6, 7 moved to the freed slots 0, 1, 2
    assert [c.lookup(0, e) for e in range(3, 8)] == [3, 4, 0, 1, 2]
    assert _moves(c.log()) == [(5, 0), (6, 1), (7, 2)]
    s = c.stats()
    assert s["n_slots"] == 5 and s["resident"] == 5 and s["evictions"] == 3
    r, slots, st = c.map(0, [3, 4, 5, 6, 7])                      # all hits, no copies
    assert r == OK and st == [5, 5, 0, 0] and _copies(c.log()) == []


def test_resize_grow_keeps_everything_in_place(lib):
    c = Cache(lib, 1, 16, 4)
    assert c.map(0, [1, 2, 3, 4])[0] == OK
    c.release(0)
    before = [c.lookup(0, e) for e in range(16)]
    c.log()
    assert _resize(lib, c, 8) == OK
    assert [c.lookup(0, e) for e in range(16)] == before and _moves(c.log()) == []
    r, slots, st = c.map(0, [5, 6, 7, 8])                         # misses fill the new slots
    assert r == OK and sorted(slots) == [4, 5, 6, 7] and st[3] == 4


def test_resize_into_a_new_array_copies_every_survivor(lib):
    c = Cache(lib, 1, 16, 6)
    assert c.map(0, [0, 2, 4, 6, 8, 10])[0] == OK
    c.release(0)
    c.log()
    assert _resize(lib, c, 4, moved=True) == OK
    mv = _moves(c.log())
    assert len(mv) == 4 and all(d < 4 for _, d in mv)
    assert sorted(d for _, d in mv) == [0, 1, 2, 3]


def test_resize_busy_and_bad_arguments_change_nothing(lib):
    c = Cache(lib, 2, 8, 6)
    assert c.map(0, [1, 2])[0] == OK                              # held
    before = [c.lookup(0, e) for e in range(8)]
    assert _resize(lib, c, 3) == BUSY
    assert [c.lookup(0, e) for e in range(8)] == before and c.stats()["n_slots"] == 6
    c.release(0)
    lib.pol_set_auto_complete(c.h, 0)
    assert c.prefetch(1, [0, 1, 2, 3])[0] == OK                   # four copies in flight
    assert _resize(lib, c, 3) == BUSY                             # cannot drop in-flight entries
    assert _resize(lib, c, 0) == INVALID
    lib.pol_complete_all(c.h)
    assert _resize(lib, c, 3) == OK and c.stats()["resident"] == 3
    p = Cache(lib, 2, 8, 6, PER_LAYER)
    assert _resize(lib, p, 4) == UNSUPPORTED


def test_resize_in_flight_entries_survive_and_stay_in_flight(lib):
    c = Cache(lib, 1, 8, 4)
    lib.pol_set_auto_complete(c.h, 0)
    assert c.prefetch(0, [0, 1, 2, 3])[0] == OK                   # slots 0..3 in flight
    assert _resize(lib, c, 4, moved=True) == OK
    assert c.stats()["in_flight"] == 4                            # now the moves are in flight
    assert c.evict(0, 3) == BUSY
    lib.pol_complete_all(c.h)
    assert c.evict(0, 3) == OK


def test_resize_failed_copy_empties_the_cache(lib):
    c = Cache(lib, 1, 8, 6)
    assert c.map(0, [0, 1, 2, 3, 4, 5])[0] == OK
    c.release(0)
    lib.pol_fail_next_copy(c.h)
    assert _resize(lib, c, 4, moved=True) == HIP
    s = c.stats()
    assert s["n_slots"] == 4 and s["resident"] == 0
    assert all(c.lookup(0, e) == -1 for e in range(8))
    assert c.map(0, [0, 1])[0] == OK                              # usable again


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_resize_matches_reference_under_traffic(lib, seed):
    """Random maps, prefetches and resizes (between steps, nothing held)
    against the reference LRU and the reference resize."""
    L, E = 3, 12
    rng = np.random.default_rng(seed)
    S = 10
    c, ref = Cache(lib, L, E, S), RefLRU(L, E, S)
    skew = np.exp(-1.1 * np.log(np.arange(1, E + 1)))
    skew /= skew.sum()
    for step in range(150):
        layer = step % L
        n = int(rng.integers(1, 5))
        experts = sorted(set(rng.choice(E, size=n, p=skew).tolist()))
        r, slots, _ = c.map(layer, experts)
        rr, payload = ref.map(layer, experts)
        assert r == rr, step
        if r == OK:
            assert slots == payload[0] and _copies(c.log()) == payload[1], step
        pf = sorted(set(rng.choice(E, size=int(rng.integers(0, 3)), p=skew).tolist()))
        r1, _ = c.prefetch((layer + 1) % L, pf)
        r2, ref_copies = ref.prefetch((layer + 1) % L, pf)
        assert r1 == r2 and _copies(c.log()) == ref_copies, step
        c.release(layer)
        ref.release(layer)
        if step % 7 == 6:
            n_new = int(rng.integers(4, 14))
            moved = bool(rng.integers(0, 2))
            assert _resize(lib, c, n_new, moved) == OK, step
            assert _moves(c.log()) == _ref_resize(ref, n_new, moved), step
            assert c.stats()["n_slots"] == n_new
        for l2 in range(L):
            for e in range(E):
                assert c.lookup(l2, e) == ref.slot_of.get((l2, e), -1), (step, l2, e)
