"""Host model of the staged cluster scorer's hand-counted memory waits (CPU only).

The staged kernel (score_mfma_stage_kernel in score_mfma.hip) streams key tiles into LDS with
memory-to-LDS loads and waits for them with hand-counted `s_waitcnt vmcnt(n)`: vector memory
operations of one wave complete in issue order for this counter, so `vmcnt(n)` means "every
operation but the newest n has completed".  A count that is one too large lets a wave read a tile
slot, a flag or a partial sum before it has landed; the GPU tests would see that only as a rare
wrong score.

This test replays, for one wave, the order in which the kernel issues its vector memory
operations (tile loads, the next stream's operand and pivot loads, the partial-sum stores, the
arrival flag store, the flag and partial-sum fetches) and its waits, over every branch of the
round structure (rounds, items per round, the deferred items, the early fetch taken or not, wave 0
or another wave, keys turned or not), and asserts at every point where the kernel reads data that
the wait before it covers that data:
  * a tile slot is read (read_item) only after all loads of that tile completed;
  * the fetched arrival flags are read only after their load completed;
  * the fetched partial sums are merged only after their loads completed;
  * the arrival flag is stored only after the partial sums it announces were stored;
  * each wave's share of the next stream's operands (and wave 0's pivots) has landed before the
    end-of-round barrier, after which every wave reads all of them.
Operations the compiler adds (the F stores, spin loads) are newer than the ones modelled and can
only make a fixed `vmcnt(n)` wait for more, so leaving them out keeps the check conservative.

The deferral constants and the wait table (vmcnt per count of extra operations, for four- and
five-load tiles) are read from the kernel source, so the model cannot silently disagree with
them; the order of operations follows the kernel's main loop and must be kept in step with it.
"""
import itertools
import os
import re

import pytest

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "kv_cache_compression_tria_amd", "csrc", "score_mfma.hip")


def _source():
    with open(SRC) as fh:
        return fh.read()


def _const(src, name):
    m = re.search(r"constexpr int %s = (\d+);" % name, src)
    assert m, name
    return int(m.group(1))


def _wait_tables(src):
    """vmcnt per extra-operation count e = 0..4 and e >= 5, for plain (4-load) and turned
    (5-load) tiles, from the wait_ring lambda."""
    body = src[src.index("auto wait_ring = [&](int e) {"):]
    body = body[:body.index("\n    };")]
    rot_part, plain_part = body.split("} else {")
    tables = {}
    for rot, part in ((True, rot_part), (False, plain_part)):
        pairs = re.findall(r"case (\d+): asm volatile\(\"s_waitcnt vmcnt\((\d+)\)", part)
        dflt = re.findall(r"default: asm volatile\(\"s_waitcnt vmcnt\((\d+)\)", part)
        assert [int(c) for c, _ in pairs] == [0, 1, 2, 3, 4] and len(dflt) == 1, part
        tables[rot] = [int(v) for _, v in pairs] + [int(dflt[0])]
    return tables


class Wave:
    """Vector memory operations of one wave, completing in issue order."""

    def __init__(self):
        self.ops = []
        self.done = 0

    def issue(self, label):
        self.ops.append(label)

    def wait(self, n):                  # s_waitcnt vmcnt(n)
        self.done = max(self.done, len(self.ops) - n)

    def landed(self, label):
        idx = [i for i, lab in enumerate(self.ops) if lab == label]
        assert idx, f"{label} was never issued"
        return max(idx) < self.done


def replay(*, wid, rounds, nt, rot, early, ps, g, defer, flags_item, table):
    """One wave of the staged kernel; early(r) says whether wave 0's early fetch of round r's
    partial sums finds every flag set."""
    w = Wave()
    lpt = 5 if rot else 4               # loads per tile: four 1 KB row loads (+ the positions)

    def wait_ring(e):
        w.wait(table[min(e, 5)])

    def load_item(i):
        for _ in range(lpt):
            w.issue(("tile", i))

    def stage_ops(rn):
        w.issue(("ops", rn))
        if wid != 0:
            return 1
        w.issue(("piv", rn))
        return 2

    def publish(r):
        if wid != 0:
            return 0
        w.issue(("pub", r))
        w.issue(("pub", r))
        return 2

    def count_arrival(r):
        if wid != 0:
            return 0
        assert w.landed(("pub", r)), f"arrival of round {r} stored before its partial sums landed"
        w.issue(("arr", r))
        return 1

    fetched_early = {}

    def fetch_flags(r):
        if wid != 0:
            return 0
        w.issue(("flags", r))
        return 1

    def fetch_parts(r):
        if wid != 0:
            return 0
        assert w.landed(("flags", r)), f"flags of round {r} read before they landed"
        fetched_early[r] = early(r)
        if not fetched_early[r]:
            return 0
        ni = (ps * g * 2 + 63) // 64
        for _ in range(ni):
            w.issue(("parts", r))
        return ni

    def score_item(i, e_prev, rn_ops, pub_r, cnt):
        wait_ring(e_prev)
        assert w.landed(("tile", i)), f"tile of item {i} read before it landed (wait count {e_prev})"
        load_item(i + 2)
        e = 0
        if rn_ops >= 0:
            e += stage_ops(rn_ops)
        if pub_r >= 0:
            e += publish(pub_r)
        if cnt >= 0:
            e += count_arrival(cnt)
        return e

    def finish(r, e):
        if wid == 0 and fetched_early.get(r, False):
            wait_ring(e)
            assert w.landed(("parts", r)), f"partials of round {r} merged before they landed"
        elif wid == 0:
            w.wait(0)                   # the flag spin, then the partials' loads and vmcnt(0)

    load_item(0)
    load_item(1)
    ops_li = max(nt - 3, 0)
    e = 0
    for r in range(rounds):
        more = r + 1 < rounds
        rn = r + 1 if more else -1
        li = 0
        if r > 0:
            nd = min(defer, nt)
            fetch = nd > flags_item + 3
            for q in range(nd):
                e = score_item(r * nt + q, e, rn if q == ops_li else -1, r - 1 if q == 0 else -1,
                               r - 1 if q == 2 else -1)
                if q == flags_item and fetch:
                    e += fetch_flags(r - 1)
                if q == flags_item + 2 and fetch:
                    e += fetch_parts(r - 1)
            if nd < 3:
                if nd == 0:
                    publish(r - 1)
                w.wait(0)
                count_arrival(r - 1)
            finish(r - 1, e)
            e = 0
            li = nd
        for li in range(li, nt):
            e = score_item(r * nt + li, e, rn if li == ops_li else -1, -1, -1)
        if more and nt < 3:
            w.wait(0)
            e = 0
        if more:
            # end-of-round barrier: every wave then reads all operand chunks and the pivots
            assert w.landed(("ops", rn)), f"operands of round {rn} not landed at the barrier"
            if wid == 0:
                assert w.landed(("piv", rn)), f"pivots of round {rn} not landed at the barrier"
    publish(rounds - 1)
    w.wait(0)
    count_arrival(rounds - 1)
    finish(rounds - 1, 0)
    return w


@pytest.fixture(scope="module")
def kernel():
    src = _source()
    return {"defer": _const(src, "kStageDefer"), "flags_item": _const(src, "kStageFlags"),
            "tables": _wait_tables(src)}


def test_wait_tables_read_from_the_kernel(kernel):
    """Sanity of what was parsed: a plain tile's wait leaves its 4 loads plus e operations
    outstanding, a turned tile's 5 plus e, capped at e = 5."""
    assert kernel["tables"][False] == [4 + e for e in range(6)]
    assert kernel["tables"][True] == [5 + e for e in range(6)]
    assert kernel["flags_item"] + 3 < kernel["defer"]


EARLY = {"always": lambda r: True, "never": lambda r: False, "alternate": lambda r: r % 2 == 0}


@pytest.mark.parametrize("rot", [False, True])
@pytest.mark.parametrize("wid", [0, 1])
@pytest.mark.parametrize("early", sorted(EARLY))
def test_every_wait_covers_what_follows(kernel, rot, wid, early):
    cases = 0
    for rounds, nt, (ps, g) in itertools.product([1, 2, 3, 5], [1, 2, 3, 4, 5, 15, 16, 17, 18, 22, 32, 64],
                                                 [(1, 4), (16, 8), (32, 8), (4, 3)]):
        replay(wid=wid, rounds=rounds, nt=nt, rot=rot, early=EARLY[early], ps=ps, g=g, defer=kernel["defer"],
               flags_item=kernel["flags_item"], table=kernel["tables"][rot])
        cases += 1
    assert cases == 4 * 12 * 4


def test_the_model_catches_a_count_one_too_large(kernel):
    """Plant a wait that allows one operation too many (the kernel's table plus one): the model
    must report a read before its data landed."""
    bad = [n + 1 for n in kernel["tables"][False]]
    with pytest.raises(AssertionError):
        replay(wid=0, rounds=3, nt=16, rot=False, early=EARLY["always"], ps=16, g=8, defer=kernel["defer"],
               flags_item=kernel["flags_item"], table=bad)


def test_the_model_catches_plain_tiles_waited_with_the_turned_table(kernel):
    """Four-load tiles waited for with the five-load (turned-key) table leave one load of the tile
    about to be read outstanding: the model must report it."""
    with pytest.raises(AssertionError):
        replay(wid=1, rounds=2, nt=16, rot=False, early=EARLY["never"], ps=16, g=8, defer=kernel["defer"],
               flags_item=kernel["flags_item"], table=kernel["tables"][True])
