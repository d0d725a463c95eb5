"""CPU model of the sliced stochastic walk's exchange protocol (host logic; no GPU).

The kernel's slices of one sequence exchange one record per step r: each slice
writes its words into slot r & 1, tagged r + 1 in the high half, then polls every
peer's words in that slot until their tags read r + 1 (relaxed device-scope
atomics: each word is single-copy atomic, nothing else is ordered).  Slices run
at any relative speed.  The model runs slices as interleaved step machines over
a shared word store, one word access per step, in random orders, and checks that
every value read is the peer's value of the same step and that every slice
finishes.  Planted protocol mistakes (one slot instead of two, tags not cleared
between calls, a slice that runs ahead without reading) must make it fail.
"""
import numpy as np
import pytest


def run_model(NS, steps, seed, *, slots=2, clear=True, stale=None, skip_reads=False, max_ticks=60000):
    """Returns (ok, reason).  `stale`: words left by an earlier call (before a clear)."""
    rng = np.random.default_rng(seed)
    W = 2  # words per record (the kernel uses 16; the protocol does not depend on it)
    mem = {}
    if stale is not None:
        mem.update(stale)
    if clear:
        mem = {k: (0, 0) for k in mem}
    value = lambda s, r, j: (s * 1000 + r) * 10 + j  # slice s's word j of step r

    def slice_machine(s):
        for r in range(steps):
            slot = r % slots
            tag = r + 1
            for j in range(W):
                mem[(slot, s, j)] = (tag, value(s, r, j))
                yield
            if skip_reads and s == 0 and r % 2 == 0:
                continue
            for t in range(NS):
                if t == s:
                    continue
                for j in range(W):
                    while True:
                        tg, v = mem.get((slot, t, j), (0, 0))
                        yield
                        if tg == tag:
                            break
                    if v != value(t, r, j):
                        raise AssertionError(f"slice {s} step {r} read {v} from slice {t} word {j}, "
                                             f"expected {value(t, r, j)}")
    machines = {s: slice_machine(s) for s in range(NS)}
    speed = rng.uniform(0.1, 1.0, NS)  # relative speeds: some slices run far ahead
    ticks = 0
    try:
        while machines:
            ticks += 1
            if ticks > max_ticks:
                return False, "no progress (a slice waits forever)"
            alive = list(machines)
            p = speed[alive] / speed[alive].sum()
            s = alive[rng.choice(len(alive), p=p)]
            try:
                next(machines[s])
            except StopIteration:
                del machines[s]
    except AssertionError as e:
        return False, str(e)
    return True, ""


@pytest.mark.parametrize("NS", [2, 3, 5, 16])
def test_protocol_delivers_each_step(NS):
    for seed in range(6 if NS < 16 else 2):
        ok, why = run_model(NS, steps=8, seed=seed)
        assert ok, (NS, seed, why)


# an earlier call that ran two steps leaves tag 1 in slot 0 and tag 2 in slot 1:
# exactly the tags this call's first two steps poll for
STALE = {(r % 2, s, j): (r + 1, -1) for r in range(2) for s in range(4) for j in range(2)}


def test_protocol_ignores_an_earlier_calls_words_once_cleared():
    for seed in range(6):
        ok, why = run_model(4, steps=6, seed=seed, stale=STALE, clear=True)
        assert ok, why


def test_planted_single_slot_fails():
    """With one slot, a slice that runs ahead overwrites a record a slow peer has
    not read yet; the slow peer then reads a later step's value or waits forever."""
    assert any(not run_model(4, steps=8, seed=seed, slots=1, max_ticks=20000)[0] for seed in range(10))


def test_planted_uncleared_tags_fail():
    """Without the clear, a record of an earlier call carries the tags this call
    polls for, and a slice takes that stale value."""
    assert any(not run_model(4, steps=6, seed=seed, stale=STALE, clear=False, max_ticks=20000)[0]
               for seed in range(10))


def test_planted_run_ahead_without_reading_fails():
    """A slice that skips reading a step can overwrite its slot two steps later
    while a peer still polls it."""
    assert any(not run_model(3, steps=10, seed=seed, skip_reads=True, max_ticks=20000)[0]
               for seed in range(15))
