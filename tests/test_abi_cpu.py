"""CPU tests of the C-ABI library: it loads, exports every declared symbol, enforces the
operation contract, sizes its buffers, and builds deterministic schedules without a device."""
import ctypes
import os
import re

import pytest

import persistent_megakernel_02_amd as pmk
from persistent_megakernel_02_amd import _lib
import synthgen
from synthgen import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "pmk.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pmk_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = pmk.load()
    names = declared_functions()
    assert len(names) >= 30
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"{n} has no binding"
    assert lib.pmk_abi_version() == 6


def create(cfg, sched=None):
    lib = pmk.load()
    ctx = ctypes.c_void_p()
    st = lib.pmk_create(ctypes.byref(cfg), ctypes.byref(sched) if sched else None, -1, ctypes.byref(ctx))
    return st, ctx, (lib.pmk_last_global_error() or b"").decode()


@pytest.mark.parametrize("change,needle", [
    (dict(has_bias=1), "biased"),
    (dict(tie_embeddings=1), "tied"),
    (dict(head_dim=96), "head_dim"),
    (dict(n_kv_heads=3), "multiple"),
    (dict(n_q_heads=32, n_kv_heads=2), "at most 8"),
    (dict(weight_dtype=pmk.PMK_DT_BF16, kv_dtype=pmk.PMK_DT_F16), "formats"),
    (dict(weight_dtype=pmk.PMK_DT_INT8, kv_dtype=pmk.PMK_DT_FP8_E4M3), "formats"),
    (dict(weight_dtype=pmk.PMK_DT_INT4, kv_dtype=pmk.PMK_DT_BF16, hidden=272), "32 for int4"),
    (dict(weight_dtype=pmk.PMK_DT_INT8, kv_dtype=pmk.PMK_DT_BF16, hidden=264), "16 for fp8 and int8"),
    (dict(hidden=260), "multiples"),
    (dict(vocab=0), "positive"),
])
def test_contract_rejections(change, needle):
    cfg = pmk.model_config(WORKLOADS["tiny"])
    for k, v in change.items():
        setattr(cfg, k, v)
    st, ctx, msg = create(cfg)
    assert st == _lib.PMK_ERR_UNSUPPORTED and needle in msg, msg


def test_fp8_kv_rows_must_cover_a_cache_line():
    cfg = pmk.model_config(WORKLOADS["tiny"].with_(wdtype="fp8", kvdtype="fp8"))  # head_dim 64 -> 64-byte rows
    st, _, msg = create(cfg)
    assert st == _lib.PMK_ERR_UNSUPPORTED and "128 bytes" in msg


def test_sizes_and_device_less_context():
    lib = pmk.load()
    for name in ("tiny", "8b", "8b_fp8", "8b_int8", "8b_int4"):
        w = WORKLOADS[name]
        st, ctx, msg = create(pmk.model_config(w))
        assert st == 0, msg
        s = pmk.pmk_sizes()
        assert lib.pmk_buffer_sizes(ctx, ctypes.byref(s)) == 0
        seqcap = (w.max_seq + 31) // 32 * 32  # the V cache is stored in blocks of 32 positions
        kv_half = w.layers * w.n_kv * seqcap * w.head_dim * (1 if w.kvdtype == "fp8" else 2)
        assert s.kv_bytes == 2 * ((kv_half + 255) // 256 * 256)
        # the arena holds at least every streamed weight byte
        assert s.arena_bytes >= w.weight_bytes()
        # device calls on a device-less context are refused, not crashed
        assert lib.pmk_bind(ctx, 256, 512, 768) == _lib.PMK_ERR_NOT_BOUND
        assert lib.pmk_decode_n_tokens(ctx, 4, 256, None, -1, None, None) == _lib.PMK_ERR_NOT_BOUND
        lib.pmk_destroy(ctx)


def test_schedule_hash_is_deterministic_and_config_sensitive():
    lib = pmk.load()
    cfg = pmk.model_config(WORKLOADS["1b"])
    hashes = []
    for sync in (pmk.PMK_SYNC_FLAGS, pmk.PMK_SYNC_FLAGS, pmk.PMK_SYNC_COUNTERS):
        st, ctx, msg = create(cfg, pmk.schedule_config(sync_mode=sync))
        assert st == 0, msg
        info = pmk.pmk_schedule_info()
        lib.pmk_schedule_get_info(ctx, ctypes.byref(info))
        hashes.append(info.hash)
        lib.pmk_destroy(ctx)
    assert hashes[0] == hashes[1] != hashes[2]


def test_null_and_bad_arguments():
    lib = pmk.load()
    ctx = ctypes.c_void_p()
    assert lib.pmk_create(None, None, -1, ctypes.byref(ctx)) == _lib.PMK_ERR_INVALID_ARG
    assert lib.pmk_buffer_sizes(None, None) == _lib.PMK_ERR_INVALID_ARG
    assert lib.pmk_set_mode(None, 0) == _lib.PMK_ERR_INVALID_ARG
    st, ctx, _ = create(pmk.model_config(WORKLOADS["tiny"]))
    assert lib.pmk_set_mode(ctx, 7) == _lib.PMK_ERR_INVALID_ARG
    assert lib.pmk_set_trace(ctx, 1) == _lib.PMK_ERR_INVALID_ARG  # no trace buffer in this schedule
    assert lib.pmk_status_str(_lib.PMK_ERR_CAPACITY) == b"KV capacity exceeded"
    lib.pmk_destroy(ctx)
    cfg = pmk.model_config(WORKLOADS["tiny"])
    for bad in (dict(prefill_chunk=100), dict(prefill_chunk=2048), dict(prefill_chunk=-2), dict(prefill_ksplit=3),
                dict(prefill_ksplit=-1), dict(combine_o_copy=3), dict(combine_o_copy=-1)):
        st, _, msg = create(cfg, pmk.schedule_config(**bad))
        name = next(iter(bad))
        assert st == _lib.PMK_ERR_INVALID_ARG and name in msg, (bad, st, msg)
    for good in (dict(prefill_ksplit=1), dict(prefill_ksplit=2), dict(prefill_chunk=-1), dict(combine_o_copy=1),
                 dict(combine_o_copy=2)):
        st, ctx, msg = create(cfg, pmk.schedule_config(**good))
        assert st == 0, (good, msg)
        lib.pmk_destroy(ctx)


def test_workload_byte_accounting():
    # bytes streamed per token (weights incl. fp8 block scales, gains, one embedding row, LM head)
    # and the mean KV bytes over the decode steps, for the workloads' shapes
    expect = {"tiny": (3_427_328, 3_460_608), "1b": (2_077_368_320, 2_096_259_072),
              "2b": (3_742_382_080, 3_803_750_400), "8b": (15_009_857_536, 15_563_571_200),
              "8b_fp8": (7_507_031_296, 8_052_323_584),
              # int8 / int4: 7,504,658,432 weights at 1 or 1/2 byte, 58,630,144 bf16 group scales,
              # 540,672 bytes of gains and embedding row; bf16 KV as in 8b
              "8b_int8": (7_622_459_392, 8_176_173_056), "8b_int4": (3_870_130_176, 4_423_843_840)}
    for name, (wb, total) in expect.items():
        w = WORKLOADS[name]
        assert w.weight_bytes() == wb
        assert round(w.mean_bytes_per_token()) == total
