"""The static validator (Safety Gate) and the CPU schedule simulator.

Real lowerings over a spread of shapes, queue counts, split counts and sync modes must all be
accepted; a generated corpus of unsafe mutants of real lowerings (dropped waits, lowered or
raised thresholds, wrong step lag, swapped queue entries, back edges, aliased output ranges,
dropped signals, removed producers, shared flag slots) must all be rejected: zero false
accepts.  Each mutation kind is unsafe by construction (the comment at each generator says
why); the simulator confirms deadlocks and races on tiny schedules.
"""
import ctypes
import random

import pytest

import persistent_megakernel_02_amd as pmk
from persistent_megakernel_02_amd import _lib
from synthgen import WORKLOADS

OPS = {1: "QKV", 2: "ATTN", 3: "OPROJ", 4: "GATEUP", 5: "DOWN", 6: "LMHEAD", 7: "TOKEN", 8: "COMBINE"}


class Sched:
    def __init__(self, w, n_cus, **kw):
        self.lib = pmk.load()
        self.h = ctypes.c_void_p()
        cfg = pmk.model_config(w)
        st = self.lib.pmk_schedule_build(ctypes.byref(cfg), ctypes.byref(pmk.schedule_config(**kw)), n_cus,
                                         ctypes.byref(self.h))
        assert st == 0, self.lib.pmk_last_global_error()

    def __del__(self):
        if self.h:
            self.lib.pmk_schedule_free(self.h)

    @property
    def n_tasks(self):
        return self.lib.pmk_schedule_num_tasks(self.h)

    @property
    def n_queues(self):
        return self.lib.pmk_schedule_num_queues(self.h)

    def task(self, i):
        t = pmk.pmk_task()
        assert self.lib.pmk_schedule_get_task(self.h, i, ctypes.byref(t)) == 0
        return t

    def set_task(self, i, t):
        assert self.lib.pmk_schedule_set_task(self.h, i, ctypes.byref(t)) == 0

    def queue(self, q):
        n = ctypes.c_int32()
        p = self.lib.pmk_schedule_queue(self.h, q, ctypes.byref(n))
        return [p[i] for i in range(n.value)]

    def set_queue(self, q, lst):
        arr = (ctypes.c_int32 * len(lst))(*lst)
        assert self.lib.pmk_schedule_set_queue(self.h, q, arr, len(lst)) == 0

    def producers(self, c):
        return self.lib.pmk_schedule_counter_producers(self.h, c)

    def set_producers(self, c, p):
        assert self.lib.pmk_schedule_set_counter_producers(self.h, c, p) == 0

    def validate(self):
        buf = ctypes.create_string_buffer(512)
        st = self.lib.pmk_schedule_validate(self.h, buf, 512)
        return st, buf.value.decode()

    def simulate(self, steps=3, seed=1):
        buf = ctypes.create_string_buffer(512)
        st = self.lib.pmk_schedule_simulate(self.h, steps, seed, buf, 512)
        return st, buf.value.decode()


REAL = [("tiny", n, {}) for n in (1, 2, 3, 4, 7, 8, 16, 64, 256)] + \
       [("tiny", 8, dict(attn_splits=s)) for s in (1, 2, 5)] + \
       [("tiny", 8, dict(sync_mode=pmk.PMK_SYNC_COUNTERS))] + \
       [("1b", n, {}) for n in (16, 100, 256)] + [("2b", 256, {}), ("8b", 256, {}), ("8b_fp8", 256, {}),
                                                  ("8b", 304, dict(attn_splits=16))]


@pytest.mark.parametrize("name,n_cus,kw", REAL)
def test_real_lowerings_are_accepted(name, n_cus, kw):
    s = Sched(WORKLOADS[name], n_cus, **kw)
    st, msg = s.validate()
    assert st == 0, msg


# 128 splits (8192 positions, 64 per split) x 4 heads x (64 + 4) fp32 partials per kv head:
# 136 KiB for one combine, so the builder splits each head group over 4 combines (one q head each)
SPLIT_COMBINE = WORKLOADS["tiny"].with_(name="tiny_split_combine", n_q=8, n_kv=2, prompt=8160, steps=32)


@pytest.mark.parametrize("name,n_cus,want", [("tiny_split_combine", 256, 4), ("2b", 256, 5), ("8b", 256, 2),
                                             ("8b_fp8", 256, 2), ("1b", 256, 1)])
def test_combines_per_kv_head(name, n_cus, want):
    """Several COMBINE tasks per kv head, each over a range of its q heads, when one would read too
    many partials (and the O-projection tiles still fit); together they cover every head once."""
    w = SPLIT_COMBINE if name == "tiny_split_combine" else WORKLOADS[name]
    s = Sched(w, n_cus)
    comb = [s.task(i) for i in range(s.n_tasks) if s.task(i).op == 8 and s.task(i).layer == 0]
    grp = w.n_q // w.n_kv
    for g in range(w.n_kv):
        ranges = sorted((t.a1 & 255, t.a1 >> 8) for t in comb if t.a0 == g)
        assert len(ranges) == want
        assert ranges[0][0] == 0 and ranges[-1][1] == grp
        assert all(a[1] == b[0] for a, b in zip(ranges, ranges[1:]))
    st, msg = s.validate()
    assert st == 0, msg


@pytest.mark.parametrize("max_seq,want_s", [(512, 1), (513, 2), (1024, 2), (1100, 3)])
def test_split_count_keeps_chunks_within_two_groups_per_wave(max_seq, want_s):
    """An attention task holds at most 512 positions (8 waves x two 32-position groups): asking for
    one split raises the count to ceil(max_seq / 512), and the lowering validates."""
    w = WORKLOADS["tiny"].with_(prompt=max_seq - 32, steps=32)
    s = Sched(w, 8, attn_splits=1)
    tasks = [s.task(i) for i in range(s.n_tasks)]
    assert sum(1 for t in tasks if t.op == 2 and t.layer == 0 and t.a0 == 0) == want_s
    st, msg = s.validate()
    assert st == 0, msg


@pytest.mark.parametrize("n_cus", [2, 5, 8])
def test_simulator_runs_real_lowerings_clean(n_cus):
    s = Sched(WORKLOADS["tiny"], n_cus)
    for seed in (1, 2):
        st, msg = s.simulate(steps=3, seed=seed)
        assert st == 0, msg


# ------------------------------------------------------------------------------------------------
# mutation corpus
# ------------------------------------------------------------------------------------------------
def mutants(w, n_cus, rng, per_kind):
    """Yield (kind, mutate(sched)) pairs; every mutant is unsafe by construction."""
    base = Sched(w, n_cus)
    NT, NQ = base.n_tasks, base.n_queues
    tasks = [base.task(i) for i in range(NT)]
    q0 = set(base.queue(0))
    # the first QKV tasks on the queue that ends with the TOKEN task are already ordered after the
    # previous step's LM head by program order, so their wait is redundant (dropping it is safe)
    waiting = [i for i, t in enumerate(tasks) if t.wait_ctr >= 0 and not (t.op == 1 and t.layer == 0 and i in q0)]
    # tasks whose queue already joined the same counter earlier in the step (lag 0, full count):
    # their own wait is redundant, so weakening it is safe
    joined_before = set()
    for q in range(NQ):
        seen = set()
        for i in base.queue(q):
            t = tasks[i]
            if t.wait_ctr >= 0 and t.wait_ctr in seen:
                joined_before.add(i)
            if t.wait_ctr >= 0 and t.wait_lag == 0 and t.wait_count == base.producers(t.wait_ctr):
                seen.add(t.wait_ctr)
    # tasks whose counter's producers all run earlier on their own queue (one attention split per
    # kv head: the combine after it): program order already orders them, so the wait is redundant
    queue_pos = {}
    for q in range(NQ):
        for k, i in enumerate(base.queue(q)):
            queue_pos[i] = (q, k)
    producers_of = {}
    for i, t in enumerate(tasks):
        if t.signal_ctr >= 0:
            producers_of.setdefault(t.signal_ctr, []).append(i)
    for i, t in enumerate(tasks):
        if t.wait_ctr >= 0:
            q, k = queue_pos[i]
            if all(queue_pos[p][0] == q and queue_pos[p][1] < k for p in producers_of.get(t.wait_ctr, [])):
                joined_before.add(i)
    weakenable = [i for i in waiting if i not in joined_before]
    signalling = [i for i, t in enumerate(tasks) if t.signal_ctr >= 0]
    full = [i for i in waiting if tasks[i].wait_count == base.producers(tasks[i].wait_ctr)
            and base.producers(tasks[i].wait_ctr) > 1]

    def drop_wait(s, i):      # the task reads data other queues produce in the same (or previous) step
        t = s.task(i); t.wait_ctr = -1; s.set_task(i, t)

    def lower_threshold(s, i):  # join incomplete: a reader of a multi-producer region waits for fewer
        t = s.task(i); t.wait_count = max(1, t.wait_count - 1 - rng.randrange(t.wait_count - 1 or 1)); s.set_task(i, t)

    def raise_threshold(s, i):  # never satisfiable
        t = s.task(i); t.wait_count = s.producers(t.wait_ctr) + 1 + rng.randrange(3); s.set_task(i, t)

    def zero_threshold(s, i):
        t = s.task(i); t.wait_count = 0; s.set_task(i, t)

    def wrong_lag(s, i):        # waits for the previous step's producers: reads stale data
        t = s.task(i); t.wait_lag = 1 - t.wait_lag; s.set_task(i, t)

    def back_edge(s, i):        # waits on a counter produced later in the same step (by its dependants;
        t = s.task(i)           # another kv head's attention splits do not depend on an ATTN task)
        own = max(t.signal_ctr, t.wait_ctr if t.wait_lag == 0 else -1)
        later = sorted({tasks[j].signal_ctr for j in signalling
                        if tasks[j].signal_ctr > own and not (t.op == 2 and tasks[j].op == 2)})
        t.wait_ctr = rng.choice(later)
        t.wait_lag = 0
        t.wait_count = s.producers(t.wait_ctr)
        s.set_task(i, t)

    def drop_signal(s, i):      # the counter never reaches its producer count
        t = s.task(i); t.signal_ctr = -1; s.set_task(i, t)

    def remove_producer(s, i):  # declared producer count no longer matches the signalling tasks
        c = s.task(i).signal_ctr; s.set_producers(c, s.producers(c) - 1)

    def shared_slot(s, i):      # two producers publish through one flag word
        t = s.task(i)
        peers = [j for j in signalling if tasks[j].signal_ctr == t.signal_ctr and j != i]
        if peers:
            t.signal_slot = tasks[rng.choice(peers)].signal_slot
        else:
            t.signal_slot = t.signal_slot + 1
        s.set_task(i, t)

    def alias_rows(s, i):       # two tasks of one phase produce the same output, so some output of
        t = s.task(i)           # the phase is produced by none (or an empty range: integrity)
        peers = [j for j in signalling if tasks[j].op == t.op and tasks[j].layer == t.layer and j != i]
        if t.op in (3, 5, 6) and peers:
            p = tasks[rng.choice(peers)]
            t.a0, t.a1 = p.a0, p.a1
        elif t.op == 2 and peers:   # ATTN: another task's (kv head, split)
            p = tasks[rng.choice(peers)]
            t.a0, t.a1 = p.a0, p.a1
        elif t.op == 8:             # COMBINE: another combine's (kv head, head range), or an invalid one
            if peers:
                p = tasks[rng.choice(peers)]
                t.a0, t.a1 = p.a0, p.a1
            else:
                t.a1 = 1            # head range [1, 0): empty
        else:
            t.a1 = t.a0
        s.set_task(i, t)

    def swap_queue(s, q):       # a task moved before the task whose signal it needs (its full-count
        lst = s.queue(q)        # wait then includes a producer queued behind it: deadlock)
        pairs = [k for k in range(len(lst) - 1)
                 if tasks[lst[k + 1]].wait_ctr >= 0 and tasks[lst[k + 1]].wait_ctr == tasks[lst[k]].signal_ctr
                 and tasks[lst[k + 1]].wait_lag == 0
                 and tasks[lst[k + 1]].wait_count == base.producers(tasks[lst[k + 1]].wait_ctr)]
        if not pairs:
            lst = lst + lst[:1]  # duplicate entry: integrity
        else:
            k = rng.choice(pairs)
            lst[k], lst[k + 1] = lst[k + 1], lst[k]
        s.set_queue(q, lst)

    def drop_from_queue(s, q):  # a task in no queue
        lst = s.queue(q)
        if lst:
            lst.pop(rng.randrange(len(lst)))
        s.set_queue(q, lst)

    kinds = [("drop_wait", drop_wait, weakenable),
             ("lower_threshold", lower_threshold, [i for i in full if i not in joined_before]),
             ("raise_threshold", raise_threshold, waiting), ("zero_threshold", zero_threshold, waiting),
             ("wrong_lag", wrong_lag, weakenable), ("back_edge", back_edge, [i for i in waiting if tasks[i].op not in (6, 7)]),
             ("drop_signal", drop_signal, signalling), ("remove_producer", remove_producer, signalling),
             ("shared_slot", shared_slot, signalling), ("alias_rows", alias_rows, signalling)]
    for kind, fn, sites in kinds:
        for i in rng.sample(sites, min(per_kind, len(sites))):
            yield kind, (lambda s, fn=fn, i=i: fn(s, i))
    for kind, fn in (("swap_queue", swap_queue), ("drop_from_queue", drop_from_queue)):
        for _ in range(per_kind):
            q = rng.randrange(NQ)
            yield kind, (lambda s, fn=fn, q=q: fn(s, q))


def test_mutation_corpus_has_no_false_accepts():
    rng = random.Random(20260609)
    total, by_kind, accepted = 0, {}, []
    for name, n_cus, per_kind in (("tiny", 4, 40), ("tiny", 8, 40), ("tiny", 32, 20), ("1b", 16, 10),
                                  ("tiny_split_combine", 256, 10)):
        w = SPLIT_COMBINE if name == "tiny_split_combine" else WORKLOADS[name]
        for kind, mutate in mutants(w, n_cus, rng, per_kind):
            s = Sched(w, n_cus)
            mutate(s)
            st, msg = s.validate()
            total += 1
            by_kind[kind] = by_kind.get(kind, 0) + 1
            if st == 0:
                accepted.append((name, n_cus, kind))
    print(f"mutants: {total} {by_kind}")
    assert total >= 800
    assert not accepted, f"false accepts: {accepted[:10]}"


def test_swapping_across_a_dependency_is_a_deadlock():
    s = Sched(WORKLOADS["tiny"], 4)
    q = s.queue(0)
    # the queue's ATTN(0) waits for all QKV(0) tasks, including this queue's own, which now follows it
    i_qkv = next(k for k, t in enumerate(q) if s.task(t).op == 1)
    i_attn = next(k for k, t in enumerate(q) if s.task(t).op == 2)
    q[i_qkv], q[i_attn] = q[i_attn], q[i_qkv]
    s.set_queue(0, q)
    st, msg = s.validate()
    assert st == _lib.PMK_ERR_SCHEDULE_INVALID and msg.startswith("deadlock"), msg
    st, msg = s.simulate(steps=2)
    assert st == _lib.PMK_ERR_TIMEOUT and "deadlock" in msg, msg


def test_simulator_catches_a_race_the_validator_rejects():
    s = Sched(WORKLOADS["tiny"], 16)
    gu = [i for i in range(s.n_tasks) if s.task(i).op == 4 and s.task(i).layer == 0]
    for i in gu:
        t = s.task(i)
        t.wait_ctr = -1
        s.set_task(i, t)
    st, msg = s.validate()
    assert st == _lib.PMK_ERR_SCHEDULE_INVALID and msg.startswith("race"), msg
    caught = [s.simulate(steps=2, seed=k) for k in range(5)]
    assert any(st == _lib.PMK_ERR_SCHEDULE_INVALID and "race" in m for st, m in caught), caught


def test_weighted_row_splits_are_accepted_and_proportional():
    """Speed-weighted GEMV splits (what tuning installs) pass the validator and follow the weights."""
    lib = pmk.load()
    for name, n_cus in (("tiny", 8), ("1b", 64), ("8b", 256)):
        w = WORKLOADS[name]
        rng = random.Random(7)
        weights = (ctypes.c_float * (8 * n_cus))(*[0.7 + 0.6 * rng.random() for _ in range(8 * n_cus)])
        h = ctypes.c_void_p()
        cfg = pmk.model_config(w)
        st = lib.pmk_schedule_build_weighted(ctypes.byref(cfg), ctypes.byref(pmk.schedule_config()), n_cus, weights,
                                             ctypes.byref(h))
        assert st == 0, lib.pmk_last_global_error()
        buf = ctypes.create_string_buffer(512)
        assert lib.pmk_schedule_validate(h, buf, 512) == 0, buf.value.decode()
        # the LM head rows of each queue follow its weight (within rounding)
        t = pmk.pmk_task()
        rows, wts = [], []
        for i in range(lib.pmk_schedule_num_tasks(h)):
            assert lib.pmk_schedule_get_task(h, i, ctypes.byref(t)) == 0
            if t.op == 6:
                rows.append(t.a1 - t.a0)
                wts.append(weights[6 * n_cus + t.signal_slot])
        total = sum(rows)
        for r, x in zip(rows, wts):
            assert abs(r - total * x / sum(wts)) <= 1.5
        lib.pmk_schedule_free(h)
