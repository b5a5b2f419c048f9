"""The entry point that allocates nothing, pmk_bind_static_workspace: the workspace is the library's
static device array, so a caller that cannot allocate device memory only brings the arena and the KV
cache.  Its decode must equal, bit for bit, the same decode on a caller-allocated workspace
(pmk_bind), and match the oracle; two calls in a row, the second on a smaller model, check that
nothing of the first call's contents of the shared array leaks into the second."""
import ctypes

import numpy as np
import pytest

import synthgen
from synthgen import WORKLOADS
from tests.parity import check, gpu_run, log, oracle_teacher_forced


def _compare(w, wts, prompt, label):
    import persistent_megakernel_02_amd as pmk
    runs = {}
    for mode_name, mode in (("megakernel", pmk.PMK_MODE_MEGAKERNEL), ("graph", pmk.PMK_MODE_GRAPH)):
        log(f"{label}/{mode_name}: caller workspace, then the static workspace")
        ref = gpu_run(w, wts, w.steps, mode=mode, prompt=prompt)
        got = gpu_run(w, wts, w.steps, mode=mode, prompt=prompt, static_workspace=True)
        assert got.first == ref.first
        assert np.array_equal(got.tokens, ref.tokens), mode_name
        assert np.array_equal(got.logits, ref.logits), mode_name
        runs[mode_name] = got
    oref, first_ok = oracle_teacher_forced(w, wts, runs["megakernel"], prompt=prompt)
    check(w, runs["megakernel"], oref, first_ok, f"{label}/static workspace")


@pytest.mark.gpu
def test_static_workspace_equals_caller_workspace_on_two_calls():
    w1 = WORKLOADS["tiny"]
    wts1 = synthgen.make_weights(w1, std=0.1, gain_std=0.1)
    _compare(w1, wts1, synthgen.make_prompt(w1), "tiny")
    # second call: a smaller model and prompt (one layer, 5-token prompt, 9 steps) on the same array
    w2 = w1.with_(name="tiny_1layer", layers=1, prompt=5, steps=9)
    wts2 = synthgen.make_weights(w2, std=0.1, gain_std=0.1)
    _compare(w2, wts2, synthgen.make_prompt(w2), "tiny 1 layer")


@pytest.mark.gpu
def test_a_later_static_bind_takes_the_array_over():
    """Two contexts on one device: the second static bind takes the array, and the first context's
    device calls then fail cleanly instead of racing on shared memory."""
    import torch
    import persistent_megakernel_02_amd as pmk
    w = WORKLOADS["tiny"]
    wts = synthgen.make_weights(w)
    a = pmk.Decoder(pmk.model_config(w), 0, static_workspace=True)
    a.load_weights(pmk.DeviceWeights(wts))
    b = pmk.Decoder(pmk.model_config(w), 0, static_workspace=True)
    b.load_weights(pmk.DeviceWeights(wts))
    prompt = torch.from_numpy(synthgen.make_prompt(w)).cuda()
    with pytest.raises(pmk.PmkError):
        a.prefill(prompt)
    b.prefill(prompt)
    toks, _, _ = b.decode(4)
    torch.cuda.synchronize()
    assert (toks.cpu().numpy() >= 0).all()
    a.close()
    b.close()


def test_static_bind_rejects_a_workspace_beyond_its_maximum():
    """The maximum is checked before anything else, also without a device: a schedule whose
    workspace exceeds the static array (the 8B model with a 64-step trace ring, or with the chunk
    buffers of the batched prefill) is refused with a clear error; one that fits reaches the device
    check."""
    import persistent_megakernel_02_amd as pmk
    from persistent_megakernel_02_amd import _lib
    lib = pmk.load()
    for name, trace, chunk, want in (("8b", 64, -1, _lib.PMK_ERR_CAPACITY), ("8b", 0, 0, _lib.PMK_ERR_CAPACITY),
                                     ("8b", 0, -1, _lib.PMK_ERR_NOT_BOUND), ("tiny", 0, 0, _lib.PMK_ERR_NOT_BOUND)):
        ctx = ctypes.c_void_p()
        st = lib.pmk_create(ctypes.byref(pmk.model_config(WORKLOADS[name])),
                            ctypes.byref(pmk.schedule_config(trace_steps=trace, prefill_chunk=chunk)), -1,
                            ctypes.byref(ctx))
        assert st == 0
        got = lib.pmk_bind_static_workspace(ctx, 256, 512)
        msg = lib.pmk_last_error(ctx).decode()
        lib.pmk_destroy(ctx)
        assert got == want, (name, trace, chunk, got, msg)
        if want == _lib.PMK_ERR_CAPACITY:
            assert "static workspace holds at most" in msg
