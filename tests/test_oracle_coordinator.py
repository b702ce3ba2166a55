"""Pins of the coordinator oracle ([codex] 5.1-5.3 and section 7) against
what the pages fix: the trace life cycle, the fetch-compute-release loop of
the pages' diagram (worked by hand below), the limits (prefetch bucket,
max live, reuse distance) as invariants, persistence, ds_id order, the
re-recording after a changed module order, a closed form for the elements
gathered per step, and the published FNV-1a test vectors (CPU only)."""

import random

import pytest
from hypothesis import given, settings, strategies as st

from oracle import coordinator as co
from synth import get_config
from synth.modules import module_table, step_order

C, P = co.CURRENT, co.PREFETCH


def _chain(n_mod=4, numel=10, **cfg):
    ids = list(range(n_mod))
    return co.Coordinator({d: numel for d in ids}, {d: False for d in ids}, [[d] for d in ids],
                          co.CoordConfig(**cfg))


def _run_step(c, order):
    ev = []
    for m in order:
        ev.append(("fetch", m, c.fetch(m)))
        ev.append(("release", m, c.release(m)))
    return ev


def test_fnv1a_published_vectors():
    assert co.fnv1a64_bytes(b"") == 0xCBF29CE484222325
    assert co.fnv1a64_bytes(b"a") == 0xAF63DC4C8601EC8C
    assert co.fnv1a64_bytes(b"foobar") == 0x85944171F73967E8


def test_trace_life_cycle():
    """[codex] 5.1: step 0 without a trace, step 1 records, from step 2 on
    the script drives prefetching."""
    c = _chain(prefetch_bucket_size=10, max_live_parameters=10**9, max_reuse_distance=0)
    assert c.mode == co.INVALID
    for step, mode_during, mode_after in ((0, co.INVALID, co.RECORD), (1, co.RECORD, co.COMPLETE),
                                          (2, co.COMPLETE, co.COMPLETE), (3, co.COMPLETE, co.COMPLETE)):
        assert c.mode == mode_during
        ev = _run_step(c, [0, 1, 2, 3])
        prefetches = [ops for kind, _, ops in ev if kind == "fetch" for k, _ in ops if k == P]
        assert bool(prefetches) == (step >= 2)
        assert c.reset_step() == mode_after
    assert c.trace == [0, 1, 2, 3]
    assert c.script == [(0, 0), (1, 1), (2, 2), (3, 3)]


def test_fetch_compute_release_loop_of_the_diagram():
    """[codex] section 2's loop: while module i computes, module i+1's
    parameters are prefetched; after it, module i's are released."""
    c = _chain(prefetch_bucket_size=10, max_live_parameters=10**9, max_reuse_distance=0)
    for _ in range(2):
        _run_step(c, [0, 1, 2, 3])
        c.reset_step()
    assert _run_step(c, [0, 1, 2, 3]) == [
        ("fetch", 0, [(C, [0]), (P, [1])]), ("release", 0, [0]),
        ("fetch", 1, [(P, [2])]), ("release", 1, [1]),
        ("fetch", 2, [(P, [3])]), ("release", 2, [2]),
        ("fetch", 3, []), ("release", 3, [3]),
    ]


def test_prefetch_bucket_and_max_live_by_hand():
    # a 20-element bucket takes the next two modules at once
    c = _chain(prefetch_bucket_size=20, max_live_parameters=10**9, max_reuse_distance=0)
    for _ in range(2):
        _run_step(c, [0, 1, 2, 3])
        c.reset_step()
    assert [e[2] for e in _run_step(c, [0, 1, 2, 3])[0::2]] == [[(C, [0]), (P, [1, 2])], [(P, [3])], [], []]
    # max_live 20 stops it at one module: the current one is live too
    c = _chain(prefetch_bucket_size=20, max_live_parameters=20, max_reuse_distance=0)
    for _ in range(2):
        _run_step(c, [0, 1, 2, 3])
        c.reset_step()
    assert [e[2] for e in _run_step(c, [0, 1, 2, 3])[0::2]] == [[(C, [0]), (P, [1])], [(P, [2])], [(P, [3])], []]


def test_forward_backward_turn_by_hand():
    """Forward then backward over a 4-module chain.  At the fetch of module 2
    the prefetcher takes module 3 (script position 3) and walks on past the
    live entries that follow -- 3 again at position 4 and 2 itself at
    position 5 -- marking those later uses, until module 1 (position 6) does
    not fit the full bucket.  So module 2's and module 3's parameters are
    kept over the turn (a marked use is never released: the prefetcher has
    passed it and would not gather it again), and the backward gathers only
    modules 1 and 0 again, both ahead of time."""
    c = _chain(prefetch_bucket_size=10, max_live_parameters=10**9, max_reuse_distance=0)
    order = [0, 1, 2, 3, 3, 2, 1, 0]
    for _ in range(2):
        _run_step(c, order)
        c.reset_step()
    assert _run_step(c, order) == [
        ("fetch", 0, [(C, [0]), (P, [1])]), ("release", 0, [0]),
        ("fetch", 1, [(P, [2])]), ("release", 1, [1]),
        ("fetch", 2, [(P, [3])]), ("release", 2, []),
        ("fetch", 3, [(P, [1])]), ("release", 3, []),
        ("fetch", 3, [(P, [0])]), ("release", 3, [3]),
        ("fetch", 2, []), ("release", 2, [2]),
        ("fetch", 1, []), ("release", 1, [1]),
        ("fetch", 0, []), ("release", 0, [0]),
    ]


def test_reuse_distance_keeps_parameters_used_again_within_the_window():
    """Module 0 is used again after two 10-element modules: distance 20."""
    order = [0, 1, 2, 0]
    for dist, kept in ((19, False), (20, True)):
        c = _chain(n_mod=3, prefetch_bucket_size=0, max_live_parameters=10**9, max_reuse_distance=dist)
        for _ in range(2):
            _run_step(c, order)
            c.reset_step()
        ev = _run_step(c, order)
        assert ev[1] == ("release", 0, [] if kept else [0])
        assert ev[6] == ("fetch", 0, [] if kept else [(C, [0])])


def test_dynamic_order_drops_the_trace_and_records_again():
    """[codex] section 7: a different module order invalidates the script;
    prefetching stops for the rest of the step; the next step records."""
    c = _chain(prefetch_bucket_size=10, max_live_parameters=10**9, max_reuse_distance=0)
    for _ in range(2):
        _run_step(c, [0, 1, 2, 3])
        c.reset_step()
    ev = _run_step(c, [0, 2, 1, 3])
    assert c.invalidations == 1 and c.mode == co.INVALID
    assert ev[0][2] == [(C, [0]), (P, [1])]
    assert all(k == C for e in ev[2::2] for k, _ in e[2])      # no prefetch after the mismatch
    assert c.reset_step() == co.RECORD
    _run_step(c, [0, 2, 1, 3])
    assert c.reset_step() == co.COMPLETE and c.trace == [0, 2, 1, 3]
    assert _run_step(c, [0, 2, 1, 3])[0][2] == [(C, [0]), (P, [2])]
    # a step with fewer fetches than the script is a mismatch at its end
    _run_step(c, [0, 2])
    c.release_all()
    assert c.reset_step() == co.RECORD and c.invalidations == 2


def _model(name):
    cfg = get_config(name)
    names, mods = module_table(cfg)
    numel = {d: p.numel for d, p in enumerate(cfg.params)}
    pers = {d: p.numel < cfg.threshold for d, p in enumerate(cfg.params)}
    return cfg, mods, numel, pers, step_order(cfg)


def _live(c):
    return {d for d, s in c.status.items() if s != co.NOT_AVAILABLE and not c.persistent[d]}


def _check_invariants(c, mods, live, ev, cfg):
    """Replays the event log from the live set at the start of the step."""
    live = set(live)
    for kind, m, ops in ev:
        if kind == "fetch":
            ids = [d for _, g in ops for d in g]
            assert len(ids) == len(set(ids))                            # nothing gathered twice at once
            assert all(not c.persistent[d] for d in ids)                # persistent: never gathered
            assert all(d not in live for d in ids)                      # never gather a live parameter
            for k, g in ops:
                assert g == sorted(g)                                   # ds_id order
            if ops and ops[-1][0] == P:
                g = ops[-1][1]
                pre = sum(c.numel[d] for d in live) + sum(c.numel[d] for k, gg in ops if k == C for d in gg)
                assert pre + sum(c.numel[d] for d in g) <= cfg.max_live_parameters
                assert len(g) == 1 or sum(c.numel[d] for d in g) <= cfg.prefetch_bucket_size
            live |= set(ids)
            assert all(d in live for d in mods[m] if not c.persistent[d])  # computable
        else:
            assert all(d in live and not c.persistent[d] for d in ops)
            live -= set(ops)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_workload_traces_keep_the_invariants(name):
    cfg_, mods, numel, pers, order = _model(name)
    for cfg in (co.CoordConfig(), co.CoordConfig(int(5e7), int(2e8), 0), co.CoordConfig(int(1e6), int(1e9), int(5e8))):
        c = co.Coordinator(numel, pers, mods, cfg)
        for step in range(4):
            live0 = _live(c)
            ev = _run_step(c, order)
            _check_invariants(c, mods, live0, ev, cfg)
            c.release_all()
            c.reset_step()


@pytest.mark.parametrize("name", ["c2", "c4"])
def test_gathered_elements_closed_form_without_prefetch_or_reuse(name):
    """No prefetch, reuse distance 0: a module's parameters are released at
    once unless the very next fetch uses them.  Llama: forward gathers every
    partitioned parameter once, backward again except lm_head (fetched twice
    in a row at the turn): 2F - lm_head.  GPT-2: the tied wte has four uses
    (embedding and head, forward and backward); only the two at the turn are
    adjacent, so it is gathered three times: 2F + wte."""
    cfg_, mods, numel, pers, order = _model(name)
    c = co.Coordinator(numel, pers, mods, co.CoordConfig(0, int(1e12), 0))
    for _ in range(2):
        _run_step(c, order)
        c.reset_step()
    ev = _run_step(c, order)
    got = sum(numel[d] for kind, _, ops in ev if kind == "fetch" for _, g in ops for d in g)
    F = sum(n for d, n in numel.items() if not pers[d])
    head = numel[[d for d, p in enumerate(cfg_.params) if p.name in ("lm_head.weight", "wte")][0]]
    if name == "c4":
        assert got == 2 * F - head
    else:
        assert got == 2 * F + head


@settings(max_examples=150, deadline=None)
@given(st.integers(0, 10**6))
def test_random_structures_keep_the_invariants(seed):
    rng = random.Random(seed)
    n_p = rng.randint(1, 12)
    numel = {d: rng.randint(1, 50) for d in range(n_p)}
    pers = {d: rng.random() < 0.2 for d in range(n_p)}
    mods = [rng.sample(range(n_p), rng.randint(1, min(3, n_p))) for _ in range(rng.randint(1, 6))]
    order = [rng.randrange(len(mods)) for _ in range(rng.randint(1, 12))]
    cfg = co.CoordConfig(rng.choice([0, 1, 30, 100]), rng.choice([0, 40, 200, 10**9]), rng.choice([0, 20, 10**9]))
    c = co.Coordinator(numel, pers, [sorted(m) for m in mods], cfg)
    for step in range(4):
        o = order if step != 3 or rng.random() < 0.5 else order[::-1]
        live0 = _live(c)
        ev = _run_step(c, o)
        _check_invariants(c, c.modules, live0, ev, cfg)
        assert _live(c) == {d for d, s in c.status.items() if s != co.NOT_AVAILABLE and not c.persistent[d]}
        c.release_all()
        c.reset_step()
