"""GPU parity: the decode path through the C ABI against the CPU oracle (teacher-forced).

Tolerance (stated by the workload): logits within max-abs 2e-2 for fp16/bf16, 1e-1 for fp8, and
identical greedy tokens wherever the oracle's top-2 gap exceeds 1e-2.  Small workloads run the
full prefill + decode; the full-size workloads start from synthetic KV contents of their full
prompt length (a generator input given to both sides) and compare sampled decode steps.
"""
import numpy as np
import pytest

import synthgen
from synthgen import WORKLOADS
from tests.parity import check, gpu_run, log, oracle_teacher_forced

pytestmark = pytest.mark.gpu

TINY = WORKLOADS["tiny"]
TINY_FP8 = TINY.with_(name="tiny_fp8", wdtype="fp8", kvdtype="fp8", n_q=4, n_kv=2, head_dim=128, hidden=512,
                      ffn=1024)


@pytest.fixture(scope="module")
def tiny():
    return synthgen.make_weights(TINY, gain_std=0.1)


def _modes():
    import persistent_megakernel_02_amd as pmk
    return [("megakernel", pmk.PMK_MODE_MEGAKERNEL), ("graph", pmk.PMK_MODE_GRAPH), ("per_op", pmk.PMK_MODE_PER_OP)]


@pytest.mark.parametrize("mode_name", ["megakernel", "graph", "per_op"])
def test_tiny_full_prefill_and_decode(tiny, mode_name):
    mode = dict(_modes())[mode_name]
    prompt = synthgen.make_prompt(TINY)
    log(f"tiny {mode_name}: prefill {len(prompt)} + decode {TINY.steps}")
    run = gpu_run(TINY, tiny, TINY.steps, mode=mode, prompt=prompt)
    ref, first_ok = oracle_teacher_forced(TINY, tiny, run, prompt=prompt)
    check(TINY, run, ref, first_ok, f"tiny/{mode_name}")


def test_tiny_varied_token_stream():
    """At N(0, 0.02) weights the tiny model's greedy stream repeats one token; at N(0, 0.1) (gains
    1 + N(0, 0.1)) it changes at nearly every step, with wide top-2 gaps, so the emitted tokens
    themselves are compared with the oracle's, in every mode, along with the logits."""
    w = TINY.with_(steps=32)
    wts = synthgen.make_weights(w, std=0.1, gain_std=0.1)
    prompt = synthgen.make_prompt(w)
    runs = {name: gpu_run(w, wts, w.steps, mode=m, prompt=prompt) for name, m in _modes()}
    base = runs["megakernel"]
    ref, first_ok = oracle_teacher_forced(w, wts, base, prompt=prompt)
    check(w, base, ref, first_ok, "tiny/varied stream")
    toks = [base.first] + [int(t) for t in base.tokens]
    assert len(set(toks)) > len(toks) // 2, toks
    for name, r in runs.items():
        assert np.array_equal(r.tokens, base.tokens), name
        assert np.array_equal(r.logits, base.logits), name


def test_tiny_counter_sync_mode(tiny):
    import persistent_megakernel_02_amd as pmk
    prompt = synthgen.make_prompt(TINY)
    run = gpu_run(TINY, tiny, TINY.steps, prompt=prompt, sched=pmk.schedule_config(sync_mode=pmk.PMK_SYNC_COUNTERS))
    ref, first_ok = oracle_teacher_forced(TINY, tiny, run, prompt=prompt)
    check(TINY, run, ref, first_ok, "tiny/counters")


def test_modes_agree_bitwise_and_chunking(tiny):
    """The three modes run the same task functions in the same order: identical logits.  Decoding in
    chunks (the KV cache, position and next-token slot persist between calls) equals one call."""
    prompt = synthgen.make_prompt(TINY)
    runs = {name: gpu_run(TINY, tiny, TINY.steps, mode=m, prompt=prompt) for name, m in _modes()}
    base = runs["megakernel"]
    for name, r in runs.items():
        assert np.array_equal(r.tokens, base.tokens), name
        assert np.array_equal(r.logits, base.logits), name
    chunked = gpu_run(TINY, tiny, TINY.steps, prompt=prompt, chunks=[5, 11, 16])
    assert np.array_equal(chunked.tokens, base.tokens)
    assert np.array_equal(chunked.logits, base.logits)
    again = gpu_run(TINY, tiny, TINY.steps, prompt=prompt)
    assert np.array_equal(again.logits, base.logits)  # deterministic


@pytest.mark.parametrize("name", ["tiny", "1b"])
def test_tuned_schedule_keeps_parity(name, tiny):
    """pmk_tune re-splits the GEMV rows by measured speed, keeps the split only if it runs faster and
    restores the position and next token: decoding afterwards still matches the oracle, and the
    modes still agree bitwise."""
    import torch
    import persistent_megakernel_02_amd as pmk
    w = synthgen.WORKLOADS[name]
    wts = tiny if name == "tiny" else synthgen.make_weights(w)
    dec = pmk.Decoder(pmk.model_config(w), 0, pmk.schedule_config(trace_steps=4))
    dec.load_weights(pmk.DeviceWeights(wts))
    prompt = synthgen.make_prompt(w)
    first = dec.prefill(torch.from_numpy(np.ascontiguousarray(prompt, np.int32)).cuda())
    torch.cuda.synchronize()
    pos = dec.position()
    log(f"{name}: tune at position {pos}")
    h0 = dec.schedule_info().hash
    k1 = dec.tune(4)
    h1 = dec.schedule_info().hash
    k2 = dec.tune(4)
    h2 = dec.schedule_info().hash
    # a re-split that did not run faster is undone: the schedule in force before comes back
    if not k1:
        assert h1 == h0
    if not k2:
        assert h2 == h1
    log(f"{name}: re-splits kept {k1}, {k2}")
    assert dec.position() == pos
    assert dec.poll_error().code == 0
    log(f"{name}: schedule hash {h0:#x} -> {dec.schedule_info().hash:#x}")
    steps = 8
    runs = {}
    for mname, m in _modes():
        runs[mname] = gpu_run(w, wts, steps, mode=m, prompt=prompt, dec=dec)
    ref, first_ok = oracle_teacher_forced(w, wts, runs["megakernel"], prompt=prompt)
    check(w, runs["megakernel"], ref, first_ok, f"{name}/tuned")
    for mname, r in runs.items():
        assert np.array_equal(r.logits, runs["megakernel"].logits), mname


def test_tiny_eos_stops_early(tiny):
    import torch
    import persistent_megakernel_02_amd as pmk
    prompt = synthgen.make_prompt(TINY)
    ref = gpu_run(TINY, tiny, TINY.steps, prompt=prompt)
    eos = int(ref.tokens[3])
    stop = int(np.argmax(ref.tokens == eos)) + 1
    for _, mode in _modes():
        dec = pmk.Decoder(pmk.model_config(TINY), 0)
        dec.load_weights(pmk.DeviceWeights(tiny))
        dec.set_mode(mode)
        dec.prefill(torch.from_numpy(prompt).cuda())
        toks, _, nd = dec.decode(TINY.steps, eos=eos)
        torch.cuda.synchronize()
        assert int(nd.item()) == stop
        assert np.array_equal(toks.cpu().numpy()[:stop], ref.tokens[:stop])
        dec.close()


def test_tiny_fp8_prefill_and_decode():
    w = TINY_FP8
    wts = synthgen.make_weights(w, gain_std=0.1)
    prompt = synthgen.make_prompt(w)
    scales = np.full((w.layers, w.n_kv, 2), 4.0 / 448.0, np.float32)
    run = gpu_run(w, wts, w.steps, prompt=prompt, kv_scales=scales)
    ref, first_ok = oracle_teacher_forced(w, wts, run, prompt=prompt, kv_scales=scales)
    check(w, run, ref, first_ok, "tiny_fp8")


def test_tiny_fp8_varied_token_stream():
    """The FP8 path (block-scaled weights, FP8 KV at a fixed scale given to both sides) with
    weights ~N(0, 0.05): 32 distinct tokens in 33, tokens and logits against the oracle, and the
    modes bitwise equal."""
    w = TINY_FP8.with_(steps=32)
    wts = synthgen.make_weights(w, std=0.05, gain_std=0.1)
    prompt = synthgen.make_prompt(w)
    scales = np.full((w.layers, w.n_kv, 2), 4.0 / 448.0, np.float32)
    runs = {name: gpu_run(w, wts, w.steps, mode=m, prompt=prompt, kv_scales=scales) for name, m in _modes()}
    base = runs["megakernel"]
    ref, first_ok = oracle_teacher_forced(w, wts, base, prompt=prompt, kv_scales=scales)
    check(w, base, ref, first_ok, "tiny_fp8/varied stream")
    toks = [base.first] + [int(t) for t in base.tokens]
    assert len(set(toks)) > len(toks) // 2, toks
    for name, r in runs.items():
        assert np.array_equal(r.tokens, base.tokens), name
        assert np.array_equal(r.logits, base.logits), name


@pytest.mark.parametrize("mode_name", ["megakernel", "per_op"])
def test_tiny_one_token_prompt_and_one_step(tiny, mode_name):
    """The smallest call: a one-token prompt (one position in the cache, every split but the first
    empty) and a single decode step."""
    mode = dict(_modes())[mode_name]
    w = TINY.with_(prompt=1, steps=1)
    prompt = synthgen.make_prompt(w)
    run = gpu_run(w, tiny, 1, mode=mode, prompt=prompt)
    ref, first_ok = oracle_teacher_forced(w, tiny, run, prompt=prompt)
    check(w, run, ref, first_ok, f"tiny/one token/{mode_name}")


@pytest.mark.parametrize("wname", ["tiny", "tiny_fp8"])
def test_long_split_two_groups_per_wave(wname):
    """One attention split over up to 332 positions (11 groups of 32 for eight waves): once the
    split passes 256 positions some waves take a second group, whose K/V rows load after the wait,
    with an online rescale of the wave's softmax.  Prefill crosses that point, decode stays past it;
    the modes still agree bitwise."""
    import persistent_megakernel_02_amd as pmk
    base = TINY if wname == "tiny" else TINY_FP8
    w = base.with_(name=f"{wname}_long", prompt=300, steps=32)
    wts = synthgen.make_weights(w, gain_std=0.1)
    prompt = synthgen.make_prompt(w)
    scales = np.full((w.layers, w.n_kv, 2), 4.0 / 448.0, np.float32) if w.kvdtype == "fp8" else None
    sched = pmk.schedule_config(attn_splits=1)
    runs = {name: gpu_run(w, wts, w.steps, mode=m, prompt=prompt, sched=sched, kv_scales=scales)
            for name, m in _modes()}
    ref, first_ok = oracle_teacher_forced(w, wts, runs["megakernel"], prompt=prompt, kv_scales=scales)
    check(w, runs["megakernel"], ref, first_ok, f"{wname}/one split")
    for name, r in runs.items():
        assert np.array_equal(r.logits, runs["megakernel"].logits), name


def test_split_combines_match_oracle_and_modes():
    """128 splits x 4 heads (requested): each kv head's combine is split over 4 tasks (one q head each); from
    synthetic KV of 2016 positions, megakernel, graph and per-op decode agree bitwise and match the
    oracle."""
    import persistent_megakernel_02_amd as pmk
    w = TINY.with_(name="tiny_split_combine", n_q=8, n_kv=2, prompt=2016, steps=16)
    wts = synthgen.make_weights(w, gain_std=0.1)
    k, v, scales = synthgen.make_kv(w, w.prompt)
    nxt = int(synthgen.make_prompt(w, 1)[0])
    sched = pmk.schedule_config(attn_splits=128)
    runs = {name: gpu_run(w, wts, w.steps, mode=m, kv=(k, v, w.prompt), next_token=nxt, sched=sched)
            for name, m in _modes()}
    ref, _ = oracle_teacher_forced(w, wts, runs["megakernel"], kv=(k, v, w.prompt))
    check(w, runs["megakernel"], ref, True, "tiny/split combines")
    for name, r in runs.items():
        assert np.array_equal(r.logits, runs["megakernel"].logits), name


# ------------------------------------------------------------------------------------------------
# workloads at their full model size: synthetic KV of the full prompt length, sampled decode steps
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name,steps", [("1b", 6), ("2b", 4), ("8b", 3), ("8b_fp8", 3)])
def test_full_size_decode_from_synthetic_kv(name, steps):
    w = WORKLOADS[name]
    log(f"{name}: generating weights")
    wts = synthgen.make_weights(w)
    k, v, scales = synthgen.make_kv(w, w.prompt)
    kv = (k, v, w.prompt)
    nxt = int(synthgen.make_prompt(w, 1)[0])
    log(f"{name}: GPU decode from KV {w.prompt}")
    run = gpu_run(w, wts, steps, kv=kv, next_token=nxt, kv_scales=scales)
    log(f"{name}: oracle {steps} steps")
    ref, _ = oracle_teacher_forced(w, wts, run, kv=kv, kv_scales=scales)
    check(w, run, ref, True, name)


def test_1b_prefill_short_prompt():
    w = WORKLOADS["1b"].with_(prompt=24, steps=8)
    wts = synthgen.make_weights(w)
    prompt = synthgen.make_prompt(w)
    run = gpu_run(w, wts, w.steps, prompt=prompt)
    ref, first_ok = oracle_teacher_forced(w, wts, run, prompt=prompt)
    check(w, run, ref, first_ok, "1b/prefill24")
