"""A model of the completion-word protocol that the greedy head and the
in-kernel split-K combine use to elect the last workgroup (arrive.hpp):
a 64-bit word, high half the dispatch's tag, low half the count.

Each workgroup's arrival is a sequence of atomic steps on the word
(increment; if the returned value lacks the tag: compare-and-swap to
(tag, 1), or a second increment once the tag is there). The dispatch's
first workgroup may claim the word at any point before or between the
arrivals (read, then compare-and-swap to (tag, 0)). The model runs every
such sequence step by step under random interleavings, from random,
adversarial and stale initial words, and checks what the kernels rely on:
exactly one workgroup sees itself as the last, only after every workgroup
has counted itself in, and the word ends as (tag, total)."""
import random

import pytest

MASK = (1 << 64) - 1


def arrival(word, tag, total, state):
    """Generator of one workgroup's atomic steps; `word` is a one-element
    list (the memory), `state` collects the outcome."""
    old = word[0]
    word[0] = (old + 1) & MASK                     # increment
    yield
    if old >> 32 != tag:
        cur = (old + 1) & MASK
        while True:
            if cur >> 32 == tag:
                old = word[0]
                word[0] = (old + 1) & MASK          # second increment
                yield
                break
            now = word[0]                           # compare-and-swap
            if now == cur:
                word[0] = (tag << 32) | 1
                old = tag << 32
                yield
                break
            cur = now
            yield
    state["count"] = old & 0xFFFFFFFF
    state["last"] = (old & 0xFFFFFFFF) == total - 1
    state["done"] = True


def preclaim(word, tag):
    cur = word[0]                                   # read
    yield
    while cur >> 32 != tag:
        now = word[0]                               # compare-and-swap
        if now == cur:
            word[0] = tag << 32
            yield
            return
        cur = now
        yield


def run(initial, tag, total, seed, with_preclaim, preclaim_first):
    rng = random.Random(seed)
    word = [initial & MASK]
    states = [dict(done=False) for _ in range(total)]
    gens = [arrival(word, tag, total, st) for st in states]
    pre = preclaim(word, tag) if with_preclaim else None
    if pre is not None and preclaim_first:
        for _ in pre:
            pass
        pre = None
    live = list(range(total)) + ([-1] if pre is not None else [])
    last_seen_when = None
    while live:
        i = rng.choice(live)
        g = pre if i == -1 else gens[i]
        try:
            next(g)
        except StopIteration:
            live.remove(i)
            if i >= 0 and states[i]["last"]:
                # every other workgroup must have counted itself in already
                last_seen_when = sum(1 for st in states if st.get("done"))
    lasts = [k for k, st in enumerate(states) if st["last"]]
    assert len(lasts) == 1, f"{len(lasts)} workgroups saw themselves last"
    assert word[0] == (tag << 32) | total, hex(word[0])
    counts = sorted(st["count"] for st in states)
    assert counts == list(range(total)), counts
    assert last_seen_when is not None


TAG = 0x5EED1234


@pytest.mark.parametrize("initial", [
    0,                                   # zeroed workspace
    (TAG - 1) << 32 | 255,               # the previous dispatch, finished
    (TAG - 1) << 32 | 0xFFFFFFFF,        # a carry into the tag half
    (TAG ^ 0xFFFF) << 32 | 17,           # a torn call
    0xA5A5A5A5A5A5A5A5,                  # fill pattern
    MASK,                                # all ones: the increment wraps
])
@pytest.mark.parametrize("with_preclaim,preclaim_first", [(False, False), (True, False), (True, True)])
def test_one_last_workgroup(initial, with_preclaim, preclaim_first):
    for seed in range(60):
        for total in (1, 2, 3, 7, 32):
            run(initial, TAG, total, seed * 97 + total, with_preclaim, preclaim_first)


def test_random_initial_words():
    rng = random.Random(4)
    for seed in range(300):
        initial = rng.getrandbits(64)
        if initial >> 32 == TAG:
            continue   # a stale word carrying this very tag (the 2^-32 case the design accepts)
        run(initial, TAG, rng.choice([1, 2, 5, 16, 64]), seed, rng.random() < 0.7, rng.random() < 0.5)


def test_mutant_protocol_is_caught():
    """A protocol that trusts any returned count (no tag check) elects no
    or several last workgroups from a stale word: the model notices."""
    def naive(word, tag, total, state):
        old = word[0]
        word[0] = (old + 1) & MASK
        yield
        state["count"] = old & 0xFFFFFFFF
        state["last"] = (old & 0xFFFFFFFF) == total - 1
        state["done"] = True

    global arrival
    saved = arrival
    arrival = naive
    try:
        with pytest.raises(AssertionError):
            run((TAG - 1) << 32 | 255, TAG, 8, 1, False, False)
    finally:
        arrival = saved
