"""Pin the oracle's lazy-layer queue and KV accounting.

Chinese write-up, "solution 2" / project page, Figure 2 caption: after each
layer its (lazy ratio, layer) enters a priority queue; while more than C
layers are queued the highest ratio leaves and its KV becomes streaming.
Pins: a brute-force scan simulation (no heap), the closed form "the final
full layers are the C lowest scores" (which is also the offline rule of the
press-release page, "LightTransfer method": replace the 50% of layers with
the highest ratio), exhaustive small cases with ties, capacity edges, and the
byte totals of the 64-layer 32K workload.
"""
import itertools
import random

import pytest

import oracle


def scan_simulation(scores, C):
    """Push, then remove the max by a linear scan while size > C (equal
    scores: lower layer index leaves first)."""
    held, ev = [], []
    for l, s in enumerate(scores):
        held.append((s, l))
        e = -1
        if len(held) > C:
            best = max(held, key=lambda t: (t[0], -t[1]))
            held.remove(best)
            e = best[1]
        ev.append(e)
    return ev


def closed_form_kept(scores, C):
    order = sorted(range(len(scores)), key=lambda l: (scores[l], -l))
    return set(order[:C])


@pytest.mark.parametrize("seed", range(200))
def test_queue_random(seed):
    rnd = random.Random(seed)
    L = rnd.randint(1, 40)
    C = rnd.randint(0, L)
    scores = [rnd.choice([rnd.random(), round(rnd.random(), 1)]) for _ in range(L)]
    ev, st = oracle.select_lazy_layers(scores, C)
    assert ev == scan_simulation(scores, C)
    kept = {l for l in range(L) if not st[l]}
    assert kept == closed_form_kept(scores, C)
    assert sum(st) == L - C
    assert sorted(e for e in ev if e >= 0) == sorted(l for l in range(L) if st[l])


def test_queue_exhaustive_with_ties():
    vals = (0.0, 0.5, 1.0)
    for L in range(1, 7):
        for scores in itertools.product(vals, repeat=L):
            for C in range(0, L + 1):
                ev, st = oracle.select_lazy_layers(list(scores), C)
                assert ev == scan_simulation(list(scores), C)
                assert {l for l in range(L) if not st[l]} == closed_form_kept(list(scores), C)


def test_queue_capacity_edges():
    s = [0.3, 0.9, 0.1, 0.5]
    ev, st = oracle.select_lazy_layers(s, 4)
    assert ev == [-1] * 4 and st == [0] * 4
    ev, st = oracle.select_lazy_layers(s, 0)
    assert ev == [0, 1, 2, 3] and st == [1] * 4
    with pytest.raises(ValueError):
        oracle.select_lazy_layers(s, 5)
    with pytest.raises(ValueError):
        oracle.select_lazy_layers([0.1, float("nan")], 1)


def test_tie_breaks_lower_index_first():
    ev, st = oracle.select_lazy_layers([0.5, 0.5, 0.5], 1)
    assert ev == [-1, 0, 1] and st == [1, 1, 0]


def test_layer_score_is_mean():
    assert oracle.layer_score([0.25, 0.75, 0.5]) == 0.5


def test_kv_accounting_driver_workload():
    """64 layers of B1 Hkv8 N32768 D128 bf16, S4 R1020, capacity 32: all-full
    8192 MiB, final 4224 MiB (32 full + 32 streaming), transient peak
    4348 MiB (33 full + 31 streaming, at the last layer)."""
    MiB = 1 << 20
    full, stream = oracle.kv_bytes(1, 8, 32768, 128, 2, 4, 1020)
    assert full == 128 * MiB and stream == 4 * MiB
    scores = [random.Random(1).random() for _ in range(64)]
    ev, st = oracle.select_lazy_layers(scores, 32)
    acc = oracle.kv_accounting(ev, full, stream)
    assert acc["retained"][-1] == 4224 * MiB
    assert max(acc["transient"]) == 4348 * MiB
    assert acc["transient"][-1] == 4348 * MiB
    assert 64 * full == 8192 * MiB
    # every step stays within C+1 full layers plus the rest streaming
    for l, t in enumerate(acc["transient"]):
        nf = min(l, 32) + 1
        assert t == nf * full + (l + 1 - nf) * stream


# Eviction before the push (project page, Figure 2 caption: when the queue is
# full the laziest layer leaves to free memory for the current one).

def scan_simulation_before(scores, C):
    """With C layers held, remove the max by a linear scan (equal scores:
    lower layer index), then add the current layer; C == 0 holds nothing."""
    held, ev = [], []
    for l, s in enumerate(scores):
        e = -1
        if C == 0:
            e = l
        else:
            if len(held) == C:
                best = max(held, key=lambda t: (t[0], -t[1]))
                held.remove(best)
                e = best[1]
            held.append((s, l))
        ev.append(e)
    return ev


def closed_form_kept_before(scores, C):
    """The last layer always stays (for C >= 1), with the C-1 lowest of the
    earlier layers under (score, -index); proof by induction on the steps."""
    L = len(scores)
    if C == 0:
        return set()
    order = sorted(range(L - 1), key=lambda l: (scores[l], -l))
    return {L - 1} | set(order[:C - 1])


@pytest.mark.parametrize("seed", range(200))
def test_queue_before_random(seed):
    rnd = random.Random(1000 + seed)
    L = rnd.randint(1, 40)
    C = rnd.randint(0, L)
    scores = [rnd.choice([rnd.random(), round(rnd.random(), 1)]) for _ in range(L)]
    ev, st = oracle.select_lazy_layers(scores, C, policy="before")
    assert ev == scan_simulation_before(scores, C)
    kept = {l for l in range(L) if not st[l]}
    assert kept == closed_form_kept_before(scores, C)
    assert sum(st) == L - C
    if C >= 1:
        assert all(ev[l] != l for l in range(L))  # the current layer always enters


def test_queue_before_exhaustive_with_ties():
    vals = (0.0, 0.5, 1.0)
    for L in range(1, 7):
        for scores in itertools.product(vals, repeat=L):
            for C in range(0, L + 1):
                ev, st = oracle.select_lazy_layers(list(scores), C, policy="before")
                assert ev == scan_simulation_before(list(scores), C)


def test_queue_before_edges():
    scores = [0.3, 0.9, 0.1, 0.7, 0.5]
    ev, st = oracle.select_lazy_layers(scores, 0, policy="before")
    assert ev == [0, 1, 2, 3, 4] and st == [1] * 5
    ev, st = oracle.select_lazy_layers(scores, 5, policy="before")
    assert ev == [-1] * 5 and st == [0] * 5
    # C = 2: step 2 evicts 1 (0.9 > 0.3); step 3 evicts 0 (0.3 > 0.1); step 4 evicts 3
    ev, st = oracle.select_lazy_layers(scores, 2, policy="before")
    assert ev == [-1, -1, 1, 0, 3]
    # the two timings differ: after-push evicts the current layer 1 at step 2
    ev_after, _ = oracle.select_lazy_layers(scores, 2)
    assert ev_after == [-1, -1, 1, 3, 4]


def test_queue_policy_rejected():
    with pytest.raises(ValueError):
        oracle.select_lazy_layers([0.1], 1, policy="sometimes")


def test_kv_accounting_before_push():
    """Same 64-layer workload with eviction before the push: the victim is
    freed before the current layer is stored, so at step l >= C the KV is C
    full layers plus l+1-C streaming ones; the peak is the final 4224 MiB
    (32 full + 32 streaming) instead of 4348 MiB (33 full + 31 streaming)."""
    MiB = 1 << 20
    full, stream = oracle.kv_bytes(1, 8, 32768, 128, 2, 4, 1020)
    scores = [random.Random(2).random() for _ in range(64)]
    ev, st = oracle.select_lazy_layers(scores, 32, policy="before")
    acc = oracle.kv_accounting(ev, full, stream, policy="before")
    assert acc["retained"][-1] == 4224 * MiB
    assert max(acc["transient"]) == 4224 * MiB
    for l, t in enumerate(acc["transient"]):
        nf = min(l + 1, 32)
        assert t == nf * full + (l + 1 - nf) * stream
    # with C = 0 every layer is converted at its own step: never two full layers
    ev0, _ = oracle.select_lazy_layers(scores, 0, policy="before")
    acc0 = oracle.kv_accounting(ev0, full, stream, policy="before")
    assert all(t == full + l * stream for l, t in enumerate(acc0["transient"]))


def test_kv_accounting_with_emitted_slices():
    """With the streaming slice written by every layer's prefill, a layer at
    full size also holds its 4 MiB slice: final 32 x 132 + 32 x 4 = 4352 MiB,
    peak 33 x 132 + 31 x 4 = 4480 MiB (after push), 4352 MiB (before push)."""
    MiB = 1 << 20
    full, stream = oracle.kv_bytes(1, 8, 32768, 128, 2, 4, 1020)
    scores = [random.Random(3).random() for _ in range(64)]
    for policy, peak in (("after", 4480), ("before", 4352)):
        ev, _ = oracle.select_lazy_layers(scores, 32, policy=policy)
        acc = oracle.kv_accounting(ev, full, stream, policy=policy, emit=True)
        assert acc["retained"][-1] == 4352 * MiB
        assert max(acc["transient"]) == peak * MiB
        plain = oracle.kv_accounting(ev, full, stream, policy=policy)
        # the difference is exactly one slice per layer still at full size
        for l, (a, b) in enumerate(zip(acc["retained"], plain["retained"])):
            n_full = (l + 1) - sum(1 for x in ev[:l + 1] if x >= 0)
            assert a - b == n_full * stream
