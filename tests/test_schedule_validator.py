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
                                                  ("8b", 304, dict(attn_splits=16))] + \
       [("8b", 256, dict(combine_parts=cp, combine_o_share=sh)) for cp in (1, 2, 4) for sh in (1, 2, 3)] + \
       [("1b", 256, dict(combine_parts=4, combine_o_share=3)), ("8b", 256, dict(attn_splits=24)),
        ("8b", 256, dict(attn_splits=16, combine_o_share=3))]


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
# What the kernel executes (mirrored from the task functions): the readers of step-tagged vectors
# (QKV of layers after the first, ATTN, OPROJ, GATEUP, LMHEAD) poll the tags in both sync modes, so
# their counter wait only adds ordering; in flags mode they do not execute it at all, and the
# producers of those vectors (QKV, COMBINE, OPROJ, DOWN) publish no flag.
def tag_reader(t):
    return (t.op == 1 and t.layer > 0) or t.op in (2, 3, 4, 6)


def exec_wait(t, mode):
    if mode == pmk.PMK_SYNC_FLAGS and tag_reader(t):
        return -1
    return t.wait_ctr


def exec_signal(t, mode):
    if mode == pmk.PMK_SYNC_FLAGS and t.op in (1, 8, 3, 5):
        return -1
    return t.signal_ctr


def qkv_groups(w, t):
    """kv groups whose q, k or v rows a QKV task writes."""
    hd, qd, kvd, grp = w.head_dim, w.n_q * w.head_dim, w.n_kv * w.head_dim, w.n_q // w.n_kv
    gs = set()
    for r in range(t.a0, t.a1):
        gs.add((r // hd) // grp if r < qd else ((r - qd) // hd if r < qd + kvd else (r - qd - kvd) // hd))
    return gs


def mutants(w, n_cus, rng, per_kind, mode=pmk.PMK_SYNC_FLAGS):
    """Yield (kind, mutate(sched)) pairs; every mutant is unsafe by construction in `mode`."""
    base = Sched(w, n_cus, sync_mode=mode)
    NT, NQ = base.n_tasks, base.n_queues
    tasks = [base.task(i) for i in range(NT)]
    q0 = set(base.queue(0))
    # waits that protect data read without a tag: the first layer's QKV (the token of the previous
    # step), COMBINE (attention partials), DOWN (h), TOKEN (the step's key).  The first QKV tasks on
    # the queue that ends with the TOKEN task are already ordered after the previous step's LM head
    # by program order, so their wait is redundant (dropping it is safe)
    waiting = [i for i, t in enumerate(tasks) if exec_wait(t, mode) >= 0 and not tag_reader(t)
               and not (t.op == 1 and t.layer == 0 and i in q0)]
    declared = [i for i, t in enumerate(tasks) if t.wait_ctr >= 0]
    executed = [i for i, t in enumerate(tasks) if exec_wait(t, mode) >= 0]
    # tasks whose queue already joined the same counter earlier in the step (lag 0, full count):
    # their own wait is redundant, so weakening it is safe
    joined_before = set()
    for q in range(NQ):
        seen = set()
        for i in base.queue(q):
            t = tasks[i]
            if t.wait_ctr >= 0 and t.wait_ctr in seen:
                joined_before.add(i)
            if exec_wait(t, mode) >= 0 and t.wait_lag == 0 and t.wait_count == base.producers(t.wait_ctr):
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
    # counters whose producers publish nothing in this mode (flags: QKV, COMBINE, OPROJ, DOWN)
    flagless = sorted({t.signal_ctr for t in tasks if t.signal_ctr >= 0 and exec_signal(t, mode) < 0})

    def drop_wait(s, i):      # the task reads data other queues produce in the same (or previous) step
        t = s.task(i); t.wait_ctr = -1; s.set_task(i, t)

    def lower_threshold(s, i):  # join incomplete: a reader of a multi-producer region waits for fewer
        t = s.task(i); t.wait_count = max(1, t.wait_count - 1 - rng.randrange(t.wait_count - 1 or 1)); s.set_task(i, t)

    def raise_threshold(s, i):  # never satisfiable (and outside 1 <= t <= producers)
        t = s.task(i); t.wait_count = s.producers(t.wait_ctr) + 1 + rng.randrange(3); s.set_task(i, t)

    def zero_threshold(s, i):
        t = s.task(i); t.wait_count = 0; s.set_task(i, t)

    def wrong_lag(s, i):        # waits for the previous step's producers: reads stale data
        t = s.task(i); t.wait_lag = 1 - t.wait_lag; s.set_task(i, t)

    def back_edge(s, i):        # an executed wait on a counter produced later in the same step (by its
        t = s.task(i)           # dependants; another kv head's attention splits do not depend on it)
        own = max(t.signal_ctr, t.wait_ctr if t.wait_lag == 0 else -1)

        def dependant(j):       # in flags mode an attention split polls only its own group's q, k, v
            a = tasks[j]
            if t.op == 2 and a.op == 2:
                return False
            if mode == pmk.PMK_SYNC_FLAGS and t.op == 1 and a.op == 2 and a.layer == t.layer:
                return a.a0 in qkv_groups(w, t)
            return True
        later = sorted({tasks[j].signal_ctr for j in signalling
                        if tasks[j].signal_ctr > own and exec_signal(tasks[j], mode) >= 0 and dependant(j)})
        t.wait_ctr = rng.choice(later)
        t.wait_lag = 0
        t.wait_count = s.producers(t.wait_ctr)
        s.set_task(i, t)

    def flagless_wait(s, i):    # flags mode: an executed wait on a counter whose producers publish no
        t = s.task(i)           # flag never ends, wherever program order already puts its producers
        t.wait_ctr = rng.choice(flagless)
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

    def depends(c, p):
        """Does task c wait, in this mode, for task p of the same step (executed full wait on p's
        executed signal, or a tagged read of what p writes)?"""
        tc, tp = tasks[c], tasks[p]
        if exec_wait(tc, mode) >= 0 and tc.wait_ctr == exec_signal(tp, mode) and tc.wait_lag == 0 \
                and tc.wait_count == base.producers(tc.wait_ctr):
            return True
        if tc.op == 2 and tp.op == 1 and tp.layer == tc.layer:      # q, k, v of its group
            return tc.a0 in qkv_groups(w, tp)
        if tc.op == 4 and tp.op == 3 and tp.layer == tc.layer:      # all of xm
            return True
        if tc.op == 3 and tp.op == 8 and tp.layer == tc.layer:      # all of o
            return True
        if tc.op == 1 and tp.op == 5 and tp.layer == tc.layer - 1:  # all of x
            return True
        if tc.op == 6 and tp.op == 5 and tp.layer == w.layers - 1:
            return True
        return False

    def swap_queue(s, q):       # a task moved before a task it waits for: deadlock
        lst = s.queue(q)
        pairs = [k for k in range(len(lst) - 1) if depends(lst[k + 1], lst[k])]
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
             ("raise_threshold", raise_threshold, declared), ("zero_threshold", zero_threshold, declared),
             ("wrong_lag", wrong_lag, weakenable),
             ("back_edge", back_edge, [i for i in executed if tasks[i].op not in (6, 7)]),
             ("drop_signal", drop_signal, signalling), ("remove_producer", remove_producer, signalling),
             ("shared_slot", shared_slot, signalling), ("alias_rows", alias_rows, signalling)]
    if mode == pmk.PMK_SYNC_FLAGS and flagless:
        kinds.append(("flagless_wait", flagless_wait, executed))
    for kind, fn, sites in kinds:
        for i in rng.sample(sites, min(per_kind, len(sites))):
            yield kind, (lambda s, fn=fn, i=i: fn(s, i))
    for kind, fn in (("swap_queue", swap_queue), ("drop_from_queue", drop_from_queue)):
        for _ in range(per_kind):
            q = rng.randrange(NQ)
            yield kind, (lambda s, fn=fn, q=q: fn(s, q))


@pytest.mark.parametrize("mode", [pmk.PMK_SYNC_FLAGS, pmk.PMK_SYNC_COUNTERS], ids=["flags", "counters"])
def test_mutation_corpus_has_no_false_accepts(mode):
    rng = random.Random(20260609 + mode)
    total, by_kind, accepted = 0, {}, []
    for name, n_cus, per_kind in (("tiny", 4, 40), ("tiny", 8, 40), ("tiny", 32, 20), ("1b", 16, 10),
                                  ("tiny_split_combine", 256, 10)):
        w = SPLIT_COMBINE if name == "tiny_split_combine" else WORKLOADS[name]
        for kind, mutate in mutants(w, n_cus, rng, per_kind, mode):
            s = Sched(w, n_cus, sync_mode=mode)
            mutate(s)
            st, msg = s.validate()
            total += 1
            by_kind[kind] = by_kind.get(kind, 0) + 1
            if st == 0:
                accepted.append((name, n_cus, kind))
    print(f"mutants: {total} {by_kind}")
    assert total >= 800
    assert not accepted, f"false accepts: {accepted[:10]}"


def _counter_of(s, op, layer):
    for i in range(s.n_tasks):
        t = s.task(i)
        if t.op == op and t.layer == layer and t.signal_ctr >= 0:
            return t.signal_ctr
    raise AssertionError((op, layer))


def test_flags_mode_rejects_a_wait_the_counter_model_accepts():
    """A combine retargeted to wait for all QKV tasks of its layer (which on two queues all run
    before it, with its attention split ahead of it on its own queue): with counters every such wait
    completes and the schedule is safe; in flags mode QKV tasks publish no flag, so the combine would
    wait forever: the validator models what each mode runs and rejects only the flags schedule."""
    results = {}
    for mode in (pmk.PMK_SYNC_COUNTERS, pmk.PMK_SYNC_FLAGS):
        s = Sched(WORKLOADS["tiny"], 2, sync_mode=mode)
        for i in range(s.n_tasks):
            t = s.task(i)
            if t.op == 8:
                t.wait_ctr = _counter_of(s, 1, t.layer)
                t.wait_count = s.producers(t.wait_ctr)
                s.set_task(i, t)
        results[mode] = s.validate()
        if mode == pmk.PMK_SYNC_FLAGS:
            assert s.simulate(steps=2)[0] == _lib.PMK_ERR_TIMEOUT
        else:
            assert s.simulate(steps=2) == (0, "")
    assert results[pmk.PMK_SYNC_COUNTERS] == (0, ""), results
    st, msg = results[pmk.PMK_SYNC_FLAGS]
    assert st == _lib.PMK_ERR_SCHEDULE_INVALID and msg.startswith("deadlock"), msg


def test_attention_ahead_of_another_groups_qkv_is_safe_only_with_flags():
    """An attention task of kv group g moved ahead of a QKV task (on its queue) that writes only
    another group's rows: with counters the attention waits for every QKV task, including that one
    (deadlock); with flags it polls only its own group's q, k and v, so the schedule is safe."""
    w = WORKLOADS["tiny"].with_(name="tiny_4kv", n_q=8, n_kv=4)
    for mode, want in ((pmk.PMK_SYNC_COUNTERS, "deadlock"), (pmk.PMK_SYNC_FLAGS, "")):
        s = Sched(w, 4, sync_mode=mode)
        done = False
        for q in range(s.n_queues):
            lst = s.queue(q)
            for k in range(len(lst) - 1):
                a, b = s.task(lst[k]), s.task(lst[k + 1])
                if a.op == 1 and b.op == 2 and a.layer == b.layer and b.a0 not in qkv_groups(w, a):
                    lst[k], lst[k + 1] = lst[k + 1], lst[k]
                    s.set_queue(q, lst)
                    done = True
                    break
            if done:
                break
        assert done
        st, msg = s.validate()
        if want:
            assert st == _lib.PMK_ERR_SCHEDULE_INVALID and msg.startswith(want), msg
        else:
            assert st == 0, msg
            assert s.simulate(steps=3) == (0, "")


def test_swapping_across_a_dependency_is_a_deadlock():
    s = Sched(WORKLOADS["tiny"], 4)
    q = s.queue(0)
    # the queue's ATTN(0) polls q and the current K/V of its group, which this queue's own QKV task
    # writes; that task now follows it
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
    # the down projections no longer wait for the gate/up tasks whose h they read
    dn = [i for i in range(s.n_tasks) if s.task(i).op == 5 and s.task(i).layer == 0]
    for i in dn:
        t = s.task(i)
        t.wait_ctr = -1
        s.set_task(i, t)
    st, msg = s.validate()
    assert st == _lib.PMK_ERR_SCHEDULE_INVALID and msg.startswith("race"), msg
    caught = [s.simulate(steps=2, seed=k) for k in range(5)]
    assert any(st == _lib.PMK_ERR_SCHEDULE_INVALID and "race" in m for st, m in caught), caught


def test_kv_cache_rows_are_checked():
    """The KV cache is part of the access model: dropping the QKV task that appends a kv head's V
    rows leaves the next step's attention reading a row no task wrote (coverage)."""
    s = Sched(WORKLOADS["tiny"], 8)
    w = WORKLOADS["tiny"]
    qd, kvd = w.n_q * w.head_dim, w.n_kv * w.head_dim
    for i in range(s.n_tasks):
        t = s.task(i)
        if t.op == 1 and t.layer == 0 and t.a0 >= qd + kvd:  # a task of V rows only
            t.a1 = t.a0  # empty
            s.set_task(i, t)
            break
    else:
        raise AssertionError("no V-only QKV task")
    st, msg = s.validate()
    assert st == _lib.PMK_ERR_SCHEDULE_INVALID, msg


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


def test_simulator_under_thread_sanitizer(tmp_path):
    """The host simulator, built with g++ under ThreadSanitizer, runs clean and failing schedules in
    both sync modes without a data-race report (its shared stamps and counters are atomics)."""
    import os
    import shutil
    import subprocess
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = str(tmp_path / "sim_tsan")
    build = subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread",
                            os.path.join(root, "persistent_megakernel_02_amd", "csrc", "schedule.cpp"),
                            os.path.join(root, "tests", "tsan_simulate.cpp"), "-o", exe],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                         env=dict(os.environ, TSAN_OPTIONS="halt_on_error=1"))
    out = run.stdout + run.stderr
    assert "ThreadSanitizer" not in out, out[-3000:]
    assert run.returncode == 0, out[-3000:]
