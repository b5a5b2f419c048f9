"""GPU error paths: the watchdog, capacity and argument checks.

The watchdog is forced from the host: a spin limit of one poll makes the first wait that is not
met at once give up, record {cu, task, expected, seen}, raise the abort word that every other
wait also reads, and let the whole grid drain (no kernel faults or hangs; every wait is bounded).
A fresh context afterwards decodes normally.
"""
import numpy as np
import pytest

import synthgen
from persistent_megakernel_02_amd import _lib
from tests.parity import log

pytestmark = pytest.mark.gpu

TINY = synthgen.WORKLOADS["tiny"]


def _decoder(sched=None):
    import torch
    import persistent_megakernel_02_amd as pmk
    w = TINY
    wts = synthgen.make_weights(w, gain_std=0.1)
    dec = pmk.Decoder(pmk.model_config(w), 0, sched)
    dec.load_weights(pmk.DeviceWeights(wts))
    k, v, _ = synthgen.make_kv(w, w.prompt)
    dec.load_kv(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), w.prompt, 5)
    torch.cuda.synchronize()
    return dec


def test_watchdog_times_out_and_the_grid_drains():
    import torch
    import persistent_megakernel_02_amd as pmk
    dec = _decoder(pmk.schedule_config(spin_limit=1))
    log("tiny: decode with a one-poll spin limit")
    toks, _, nd = dec.decode(8)
    torch.cuda.synchronize()
    err = dec.poll_error()
    log(f"watchdog: code {err.code} cu {err.cu} task {err.task} expected {err.expected} seen {err.seen}")
    assert err.code == _lib.PMK_ERR_TIMEOUT
    assert 0 <= err.cu < dec.schedule_info().n_cus
    assert 0 <= err.task < dec.schedule_info().n_tasks or err.task == -1
    dec.close()
    # the device is fine: a fresh context decodes without error, deterministically
    runs = []
    for _ in range(2):
        d2 = _decoder()
        t2, _, n2 = d2.decode(8)
        torch.cuda.synchronize()
        assert d2.poll_error().code == 0
        assert int(n2.item()) == 8
        runs.append(t2.cpu().numpy())
        d2.close()
    assert np.array_equal(runs[0], runs[1])
    assert ((runs[0] >= 0) & (runs[0] < TINY.vocab)).all()


def test_capacity_and_argument_errors():
    import torch
    dec = _decoder()
    room = TINY.max_seq - TINY.prompt
    with pytest.raises(_lib.PmkError) as e:
        dec.decode(room + 1)
    assert e.value.status == _lib.PMK_ERR_CAPACITY
    with pytest.raises(_lib.PmkError) as e:
        dec.decode(0)
    assert e.value.status == _lib.PMK_ERR_INVALID_ARG
    assert dec.position() == TINY.prompt  # rejected calls change nothing
    toks, _, nd = dec.decode(room)         # exactly to max_seq
    torch.cuda.synchronize()
    assert int(nd.item()) == room and dec.poll_error().code == 0
    assert dec.position() == TINY.max_seq
    with pytest.raises(_lib.PmkError) as e:
        dec.decode(1)
    assert e.value.status == _lib.PMK_ERR_CAPACITY
    dec.close()
