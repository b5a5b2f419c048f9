"""Pins of the CPU oracle against what the definitions and the mathematics fix.

Each test ties an oracle function to something other than itself: a library routine for
the storage formats, a closed form, an invariant, or a brute-force fp64 recomputation of
the whole sequence without a KV cache (tests/brute.py).  A plausible slip in the oracle
(a dropped term, a wrong sign, index or transposition, the wrong RoPE pairing, a wrong
GQA group map, a missing eps) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthgen
from synthgen import WORKLOADS
from tests import brute

RNG = np.random.default_rng(1234)


# ------------------------------------------------------------------------------------------------
# storage formats
# ------------------------------------------------------------------------------------------------
def test_f16_decode_exhaustive():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(oracle.F16, codes)
    ref = codes.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_decode_exhaustive():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(oracle.BF16, codes)
    ref = (codes.astype(np.uint32) << 16).view(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _f16_probe_values():
    v = np.concatenate([
        RNG.standard_normal(20000).astype(np.float32) * np.float32(0.02),
        RNG.standard_normal(20000).astype(np.float32) * np.float32(3000.0),
        (RNG.random(5000) * 2 ** -14).astype(np.float32),        # binary16 subnormals
        (RNG.random(2000) * 2 ** -24).astype(np.float32),        # below the smallest subnormal
        np.array([65504, 65519.99, 65520, 70000, 1e30, -65520, 0.0, -0.0, 2 ** -25, 2 ** -24, 3 * 2 ** -26],
                 np.float32),
    ])
    # exact midpoints between neighbouring binary16 values (ties must go to even)
    h = RNG.integers(0, 0x7bff, 5000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    return np.concatenate([v, mid, -mid])


def test_f16_encode_matches_numpy_rne():
    v = _f16_probe_values()
    got = oracle.encode(oracle.F16, v)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_encode_matches_torch_rne():
    v = np.concatenate([RNG.standard_normal(50000).astype(np.float32) * s for s in (1e-3, 1.0, 1e6)])
    u = (RNG.integers(0, 2 ** 16, 5000).astype(np.uint32) << 16) | 0x8000  # exact ties
    v = np.concatenate([v, u.view(np.float32)])
    v = v[np.isfinite(v)]
    got = oracle.encode(oracle.BF16, v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode(oracle.E4M3, codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7e] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_encode_rne_and_saturation():
    v = np.concatenate([RNG.standard_normal(40000).astype(np.float32) * s for s in (0.01, 1.0, 100.0)])
    v = v[np.abs(v) <= 448.0]
    got = oracle.encode(oracle.E4M3, v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    sat = oracle.encode(oracle.E4M3, np.array([449.0, 1e6, -1e9, 464.0], np.float32))
    assert list(sat) == [0x7e, 0x7e, 0xfe, 0x7e]


# ------------------------------------------------------------------------------------------------
# GEMV
# ------------------------------------------------------------------------------------------------
def test_gemv_identity_and_one_hot():
    n = 96
    eye = np.eye(n, dtype=np.float16).view(np.uint16)
    x = RNG.standard_normal(n).astype(np.float32)
    assert np.array_equal(oracle.gemv(oracle.F16, eye, x), x)
    W = synthgen.normal(7, 1, (40, 72), 0.5, synthgen.FMT_BF16)  # 40 rows x 72 cols
    Wd = brute.dec16(W, "bf16")
    for j in (0, 13, 71):
        e = np.zeros(72, np.float32)
        e[j] = 1.0
        assert np.array_equal(oracle.gemv(oracle.BF16, W, e), Wd[:, j].astype(np.float32))


@pytest.mark.parametrize("fmt", ["f16", "bf16", "fp8"])
def test_gemv_within_fp32_error_bound(fmt):
    rows, cols = 300, 520
    raw = synthgen.normal(11, 2, (rows, cols), 0.02, synthgen.FMT_BF16 if fmt != "f16" else synthgen.FMT_F16)
    x = RNG.standard_normal(cols).astype(np.float32)
    if fmt == "fp8":
        q, S = synthgen.quant_e4m3_block(raw)
        Wd = brute.dec_e4m3(q) * np.repeat(np.repeat(S.astype(np.float64), 128, 0), 128, 1)[:rows, :cols]
        got = oracle.gemv(oracle.E4M3, q, x, S)
        terms = cols + 1  # the dequantisation product adds one rounding per term
    else:
        Wd = brute.dec16(raw, fmt)
        got = oracle.gemv(oracle.FMT[fmt], raw, x)
        terms = cols
    ref = Wd @ x.astype(np.float64)
    u = 2.0 ** -24
    gamma = terms * u / (1 - terms * u)
    bound = gamma * (np.abs(Wd) @ np.abs(x.astype(np.float64)))
    assert np.all(np.abs(got - ref) <= bound)
    assert np.abs(ref).max() > 10 * bound.max()  # not vacuous


# ------------------------------------------------------------------------------------------------
# weight-only integer formats (W8A16 / W4A16): codes, group scales, binary16 activations
# ------------------------------------------------------------------------------------------------
def _bf16_bits(v) -> np.ndarray:
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_int8_codes_are_twos_complement_bytes():
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    S = _bf16_bits([[1.0, 1.0]])
    got = oracle.weight_matrix(oracle.I8, codes.view(np.int8), S)
    assert np.array_equal(got[0], codes[0].view(np.int8).astype(np.float32))
    assert got[0, 0x80] == -128 and got[0, 0xFF] == -1 and got[0, 0x7F] == 127


def test_int4_codes_low_nibble_is_the_even_column():
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)  # 512 columns
    S = _bf16_bits([[1.0] * 4])
    got = oracle.weight_matrix(oracle.I4, b, S)[0]
    lo = (b[0].astype(np.int64) & 15 ^ 8) - 8  # 4-bit two's complement by the xor-subtract identity
    hi = (b[0].astype(np.int64) >> 4 ^ 8) - 8
    assert np.array_equal(got[0::2], lo.astype(np.float32))
    assert np.array_equal(got[1::2], hi.astype(np.float32))
    # hand-decoded bytes: 0x8F holds (-1, -8), 0x70 holds (0, 7)
    assert list(got[2 * 0x8F: 2 * 0x8F + 2]) == [-1.0, -8.0]
    assert list(got[2 * 0x70: 2 * 0x70 + 2]) == [0.0, 7.0]


@pytest.mark.parametrize("fmt", ["int8", "int4"])
def test_int_group_scales_index_row_and_128_column_group(fmt):
    rows, cols = 3, 300  # groups of 128, 128 and a ragged 44
    ng = 3
    if fmt == "int8":
        codes = np.ones((rows, cols), np.int8)
    else:
        codes = np.full((rows, cols // 2), 0x11, np.uint8)  # +1 in both nibbles
    S = _bf16_bits([[2.0 ** (3 * r + g) for g in range(ng)] for r in range(rows)])
    y = oracle.gemv(oracle.FMT[fmt], codes, np.ones(cols, np.float32), S)
    ref = [128 * 2.0 ** (3 * r) + 128 * 2.0 ** (3 * r + 1) + 44 * 2.0 ** (3 * r + 2) for r in range(rows)]
    assert list(y) == ref


@pytest.mark.parametrize("fmt", ["int8", "int4"])
def test_int_gemv_rounds_the_activation_to_binary16(fmt):
    cols = 256
    codes = np.ones((1, cols), np.int8) if fmt == "int8" else np.full((1, cols // 2), 0x11, np.uint8)
    S = _bf16_bits([[1.0, 1.0]])
    # 1 + 2^-12 is below half a binary16 step at 1 (2^-11): it rounds to 1
    y = oracle.gemv(oracle.FMT[fmt], codes, np.full(cols, 1 + 2.0 ** -12, np.float32), S)
    assert y[0] == cols
    # 1 + 3 * 2^-11 lies halfway between 1 + 2^-10 and 1 + 2^-9: the tie goes to the even 1 + 2^-9
    y = oracle.gemv(oracle.FMT[fmt], codes, np.full(cols, 1 + 3 * 2.0 ** -11, np.float32), S)
    assert y[0] == cols * (1 + 2.0 ** -9)


@pytest.mark.parametrize("fmt", ["int8", "int4"])
def test_int_gemv_within_fp32_error_bound(fmt):
    rows, cols = 200, 640
    raw = synthgen.normal(12, 3, (rows, cols), 0.02, synthgen.FMT_BF16)
    q, S = synthgen.quant_int_group(raw, 8 if fmt == "int8" else 4)
    x = RNG.standard_normal(cols).astype(np.float32)
    Wd = brute.int_codes(q, fmt) * np.repeat(brute.dec16(S, "bf16"), 128, 1)[:, :cols]
    x16 = x.astype(np.float16).astype(np.float64)  # numpy's own nearest-even binary16 rounding
    got = oracle.gemv(oracle.FMT[fmt], q, x, S)
    ref = Wd @ x16
    u = 2.0 ** -24
    gamma = cols * u / (1 - cols * u)  # code * bf16 scale is exact in fp32
    bound = gamma * (np.abs(Wd) @ np.abs(x16))
    assert np.all(np.abs(got - ref) <= bound)
    assert np.abs(ref).max() > 10 * bound.max()
    # the binary16 rounding is visible: unrounded activations give results far outside the oracle's
    # distance from the rounded reference
    assert np.abs(Wd @ x.astype(np.float64) - ref).max() > 20 * np.abs(got - ref).max()


@pytest.mark.parametrize("bits", [8, 4])
def test_int_quantiser_reconstructs_each_weight_within_half_a_step(bits):
    """The generator's group quantiser (shared input data, not oracle arithmetic)."""
    rows, cols = 64, 300
    raw = synthgen.normal(13, 4, (rows, cols), 0.02, synthgen.FMT_BF16)
    q, S = synthgen.quant_int_group(raw, bits)
    fmt = "int8" if bits == 8 else "int4"
    s = np.repeat(brute.dec16(S, "bf16"), 128, 1)[:, :cols]
    w = brute.dec16(raw, "bf16")
    qmax = 127 if bits == 8 else 7
    codes = brute.int_codes(q, fmt)
    assert np.abs(codes).max() == qmax  # the group maximum maps to the largest code
    # half a step, plus the clamp when bf16 rounded the scale down (|w| / s <= qmax (1 + 2^-8))
    assert np.all(np.abs(w - codes * s) <= s * (0.5 + qmax * 2.0 ** -8))


# ------------------------------------------------------------------------------------------------
# RMSNorm
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("c", [0.003, 0.5, -2.0, 40.0])
def test_rmsnorm_constant_vector_closed_form(c):
    n, eps = 256, 1e-5
    g = (1.0 + 0.1 * RNG.standard_normal(n)).astype(np.float32)
    y = oracle.rmsnorm(np.full(n, c, np.float32), g, eps)
    ref = c / math.sqrt(c * c + eps) * g.astype(np.float64)
    np.testing.assert_allclose(y, ref, rtol=3e-6, atol=0)


def test_rmsnorm_uses_mean_and_eps():
    # mean (not sum) of squares: a vector of n ones has rms 1, so y = g/sqrt(1+eps)
    n = 4096
    g = np.ones(n, np.float32)
    y = oracle.rmsnorm(np.ones(n, np.float32), g, 0.5)
    np.testing.assert_allclose(y, 1 / math.sqrt(1.5), rtol=1e-6)


# ------------------------------------------------------------------------------------------------
# RoPE
# ------------------------------------------------------------------------------------------------
def test_rope_position_zero_is_identity():
    u = RNG.standard_normal(128).astype(np.float32)
    assert np.array_equal(oracle.rope(u, 0, 500000.0), u)


def test_rope_preserves_norm():
    u = RNG.standard_normal(128).astype(np.float32)
    for p in (1, 17, 4095):
        r = oracle.rope(u, p, 10000.0)
        assert abs(np.linalg.norm(r.astype(np.float64)) - np.linalg.norm(u.astype(np.float64))) < 1e-5


def test_rope_basis_vectors_rotate_half_pairs():
    hd, theta = 64, 10000.0
    for p in (1, 7, 300):
        for i in (0, 5, 31):
            phi = p * theta ** (-2.0 * i / hd)
            e = np.zeros(hd, np.float32)
            e[i] = 1.0
            r = oracle.rope(e, p, theta)
            expect = np.zeros(hd)
            expect[i], expect[i + hd // 2] = math.cos(phi), math.sin(phi)
            np.testing.assert_allclose(r, expect, atol=1e-7)
            e = np.zeros(hd, np.float32)
            e[i + hd // 2] = 1.0
            r = oracle.rope(e, p, theta)
            expect = np.zeros(hd)
            expect[i], expect[i + hd // 2] = -math.sin(phi), math.cos(phi)
            np.testing.assert_allclose(r, expect, atol=1e-7)


def test_rope_inner_product_depends_on_offset_only():
    q = RNG.standard_normal(128).astype(np.float32)
    k = RNG.standard_normal(128).astype(np.float32)
    a = np.dot(oracle.rope(q, 9, 10000.0).astype(np.float64), oracle.rope(k, 4, 10000.0))
    b = np.dot(oracle.rope(q, 105, 10000.0).astype(np.float64), oracle.rope(k, 100, 10000.0))
    c = np.dot(oracle.rope(q, 5, 10000.0).astype(np.float64), oracle.rope(k, 0, 10000.0))
    assert abs(a - b) < 1e-4 and abs(a - c) < 1e-4


# ------------------------------------------------------------------------------------------------
# attention
# ------------------------------------------------------------------------------------------------
def _f16(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def test_attention_single_token_returns_v():
    hd = 64
    q = RNG.standard_normal(hd).astype(np.float32)
    K = _f16(RNG.standard_normal((1, hd)))
    V = _f16(RNG.standard_normal((1, hd)))
    out = oracle.attend(q, K, V, oracle.F16)
    assert np.array_equal(out, V.view(np.float16).astype(np.float32)[0])


def test_attention_identical_keys_give_mean_of_v():
    hd, T = 64, 37
    q = RNG.standard_normal(hd).astype(np.float32)
    K = np.repeat(_f16(RNG.standard_normal((1, hd))), T, 0)
    Vf = RNG.standard_normal((T, hd))
    V = _f16(Vf)
    out = oracle.attend(q, K, V, oracle.F16)
    np.testing.assert_allclose(out, V.view(np.float16).astype(np.float64).mean(0), atol=2e-6)


def test_attention_two_keys_closed_form_scale():
    hd = 128
    q = np.zeros(hd, np.float32)
    q[0] = 4.0
    K = np.zeros((2, hd), np.float32)
    K[0, 0], K[1, 0] = 1.5, -0.5   # scores 6 and -2 before the 1/sqrt(hd) scale
    V = np.zeros((2, hd), np.float32)
    V[0, :], V[1, :] = 1.0, -3.0
    out = oracle.attend(q, _f16(K), _f16(V), oracle.F16)
    w0 = 1.0 / (1.0 + math.exp(-(6.0 - (-2.0)) / math.sqrt(hd)))
    np.testing.assert_allclose(out, w0 * 1.0 + (1 - w0) * (-3.0), rtol=1e-6)


def test_attention_fp8_scales_apply_to_k_and_v():
    hd = 64
    q = np.zeros(hd, np.float32)
    q[3] = 2.0
    Kc = np.zeros((2, hd), np.uint8)
    Kc[0, 3] = 0x38  # 1.0
    Vc = np.zeros((2, hd), np.uint8)
    Vc[0, :] = 0x40  # 2.0
    Vc[1, :] = 0xC0  # -2.0
    out = oracle.attend(q, Kc, Vc, oracle.E4M3, ks=0.5, vs=0.25)
    s0 = 2.0 * 1.0 * 0.5 / math.sqrt(hd)
    w0 = 1 / (1 + math.exp(-s0))
    np.testing.assert_allclose(out, w0 * 0.5 + (1 - w0) * (-0.5), rtol=1e-6)


def test_attention_shift_invariance():
    hd, T = 64, 20
    q = np.zeros(hd, np.float32)
    q[:8] = RNG.standard_normal(8)
    Kf = np.zeros((T, hd))
    Kf[:, :8] = RNG.standard_normal((T, 8))
    Vf = RNG.standard_normal((T, hd))
    base = oracle.attend(q, _f16(Kf), _f16(Vf), oracle.F16)
    q2 = q.copy()
    q2[40] = 1.0
    K2 = Kf.copy()
    K2[:, 40] = 3.0   # every score shifts by 3/sqrt(hd)
    out = oracle.attend(q2, _f16(K2), _f16(Vf), oracle.F16)
    np.testing.assert_allclose(out, base, atol=1e-6)


# ------------------------------------------------------------------------------------------------
# SwiGLU activation and greedy choice
# ------------------------------------------------------------------------------------------------
def test_silu_values_and_limits():
    assert oracle.silu(0.0) == 0.0
    for z in (-3.0, -0.5, 0.25, 1.0, 4.0):
        assert abs(oracle.silu(z) - z / (1 + math.exp(-z))) <= 2e-7 * max(1.0, abs(z))
    assert abs(oracle.silu(30.0) - 30.0) < 1e-5
    assert abs(oracle.silu(-30.0)) < 1e-10


def test_argmax_ties_lowest_index_and_nan():
    v = np.array([0.5, 2.0, -1.0, 2.0, 2.0], np.float32)
    assert oracle.argmax(v) == 1
    v[0] = np.nan
    assert oracle.argmax(v) == -1


# ------------------------------------------------------------------------------------------------
# whole model
# ------------------------------------------------------------------------------------------------
TINY = WORKLOADS["tiny"]


@pytest.fixture(scope="module")
def tiny_weights():
    return synthgen.make_weights(TINY, gain_std=0.1)


def test_tiny_model_matches_fp64_brute_force(tiny_weights):
    m = oracle.OracleModel(tiny_weights)
    prompt = synthgen.make_prompt(TINY)
    tok, lg = m.prefill(prompt)
    ref = brute.logits_all(tiny_weights, prompt)
    assert np.abs(lg - ref).max() < 1e-4 and np.abs(ref).max() > 0.1
    toks = list(prompt) + [tok]
    for _ in range(5):
        tok, lg = m.step(toks[-1])
        ref = brute.logits_all(tiny_weights, toks)
        assert np.abs(lg - ref).max() < 1e-4
        assert tok == int(np.argmax(lg))
        toks.append(tok)


def test_prefill_block_size_and_decode_consistency(tiny_weights):
    prompt = synthgen.make_prompt(TINY, 24)
    outs = []
    for block in (1, 5, 64):
        m = oracle.OracleModel(tiny_weights)
        outs.append(m.prefill(prompt, block=block))
    for t, lg in outs[1:]:
        assert t == outs[0][0] and np.array_equal(lg, outs[0][1])
    # prefill of P tokens then decode of the rest == prefill of all of them (same last-position logits)
    m = oracle.OracleModel(tiny_weights)
    m.prefill(prompt[:10])
    for t in prompt[10:]:
        _, lg = m.step(int(t))
    assert np.array_equal(lg, outs[0][1])


def test_zero_layers_closed_form():
    w = TINY.with_(layers=0)
    wts = synthgen.make_weights(w, gain_std=0.1)
    m = oracle.OracleModel(wts)
    tok = 77
    _, lg = m.prefill(np.array([tok], np.int32))
    x = brute.dec16(wts.embed, "f16")[tok]
    g = brute.dec16(wts.final_norm, "f16")
    ref = brute.dec16(wts.lm_head, "f16") @ (x / np.sqrt((x * x).mean() + w.eps) * g)
    assert np.abs(lg - ref).max() < 1e-5


def test_zero_wo_wd_makes_logits_context_free():
    wts = synthgen.make_weights(TINY, zero=("wo", "w_down"))
    a = oracle.OracleModel(wts)
    b = oracle.OracleModel(wts)
    a.prefill(np.array([1, 2, 3, 900], np.int32))
    b.prefill(np.array([500, 11], np.int32))
    _, la = a.step(42)
    _, lb = b.step(42)
    assert np.array_equal(la, lb)


def test_zero_wq_gives_uniform_attention():
    w = TINY.with_(layers=1)
    wts = synthgen.make_weights(w, zero=("wq",))
    m = oracle.OracleModel(wts)
    prompt = synthgen.make_prompt(w, 9)
    _, lg = m.prefill(prompt)
    ref = brute.logits_all(wts, prompt, attn_override="uniform")
    assert np.abs(lg - ref).max() < 1e-4


def test_gqa_equals_mha_with_repeated_kv_heads(tiny_weights):
    w = TINY
    grp = w.n_q // w.n_kv
    mha_w = w.with_(n_kv=w.n_q)
    mha = synthgen.make_weights(mha_w, gain_std=0.1)
    hd = w.head_dim
    for l in range(w.layers):
        for k in ("wq", "wo", "w_gate", "w_up", "w_down", "attn_norm", "ffn_norm"):
            mha.layers[l][k] = tiny_weights.layers[l][k]
        for k in ("wk", "wv"):
            src = tiny_weights.layers[l][k].reshape(w.n_kv, hd, w.hidden)
            mha.layers[l][k] = np.ascontiguousarray(np.repeat(src, grp, axis=0).reshape(w.n_q * hd, w.hidden))
    mha.embed, mha.lm_head, mha.final_norm = tiny_weights.embed, tiny_weights.lm_head, tiny_weights.final_norm
    prompt = synthgen.make_prompt(w, 12)
    t1, l1 = oracle.OracleModel(tiny_weights).prefill(prompt)
    t2, l2 = oracle.OracleModel(mha).prefill(prompt)
    assert t1 == t2 and np.array_equal(l1, l2)


def test_loaded_kv_equals_prefilled_kv(tiny_weights):
    prompt = synthgen.make_prompt(TINY)
    a = oracle.OracleModel(tiny_weights)
    a.prefill(prompt)
    k, v = a.read_kv(len(prompt))
    b = oracle.OracleModel(tiny_weights)
    b.load_kv(k, v, len(prompt))
    ta, la = a.step(5)
    tb, lb = b.step(5)
    assert ta == tb and np.array_equal(la, lb)


def test_synthetic_kv_decode_matches_brute_force():
    w = TINY.with_(layers=1)
    wts = synthgen.make_weights(w, gain_std=0.1)
    k, v, _ = synthgen.make_kv(w, 30)
    m = oracle.OracleModel(wts)
    m.load_kv(k, v, 30)
    _, lg = m.step(3)
    ref = brute.logits_all(wts, [3], cached_kv=(brute.dec16(k, "f16"), brute.dec16(v, "f16")))
    assert np.abs(lg - ref).max() < 1e-4


def test_fp8_model_matches_fp64_brute_force():
    w = TINY.with_(wdtype="fp8", kvdtype="fp8", hidden=256, ffn=384, layers=2)
    wts = synthgen.make_weights(w)
    scales = np.full((w.layers, w.n_kv, 2), 4.0 / 448.0, np.float32)
    m = oracle.OracleModel(wts)
    m.set_kv_scales(scales)
    prompt = synthgen.make_prompt(w, 8)
    tok, lg = m.prefill(prompt)
    ref = brute.logits_all(wts, prompt, kv_scales=scales)
    assert np.abs(lg - ref).max() < 2e-3 and np.abs(ref).max() > 0.1
    _, lg2 = m.step(tok)
    ref2 = brute.logits_all(wts, list(prompt) + [tok], kv_scales=scales)
    assert np.abs(lg2 - ref2).max() < 2e-3


@pytest.mark.parametrize("fmt", ["int8", "int4"])
def test_int_model_matches_fp64_brute_force(fmt):
    w = TINY.with_(wdtype=fmt, kvdtype="bf16", hidden=256, ffn=384, layers=2)
    wts = synthgen.make_weights(w, gain_std=0.1)
    m = oracle.OracleModel(wts)
    prompt = synthgen.make_prompt(w, 8)
    tok, lg = m.prefill(prompt)
    ref = brute.logits_all(wts, prompt)
    assert np.abs(lg - ref).max() < 2e-3 and np.abs(ref).max() > 0.1
    _, lg2 = m.step(tok)
    ref2 = brute.logits_all(wts, list(prompt) + [tok])
    assert np.abs(lg2 - ref2).max() < 2e-3


def test_oracle_matches_its_recorded_tiny_run():
    """Regression fixture written by tests/golden/make_golden.py (oracle + generator only)."""
    import json
    import os
    from tests.golden.make_golden import run
    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle_greedy.json")) as f:
        gold = json.load(f)
    now = run()
    assert now["tokens"] == gold["tokens"] and now["prompt"] == gold["prompt"]
    for k, v in gold["logits_head"].items():
        assert np.array_equal(np.float32(now["logits_head"][k]), np.float32(v)), k


# ---------------------------------------------------------------------------------------------
# static FP8 KV scales derived from a prompt: the largest |k| (after RoPE) and |v| per (layer, kv
# head) over the appended rows, S = amax / 448 (a reading of the pages' static per-head FP8-KV
# scale: "Netra Kernel" summary, details, FP8-KV attention with explicit scale semantics)
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("kvfmt", ["f16", "fp8"])
def test_kv_amax_matches_brute_force_values(kvfmt):
    """The recorded maxima equal the largest |k|, |v| of an independent fp64 recomputation of the
    prompt (same rounding of earlier layers' KV into the cache format, scale 1)."""
    w = TINY.with_(kvdtype=kvfmt, wdtype=kvfmt, hidden=256, ffn=384, head_dim=128 if kvfmt == "fp8" else 64)
    wts = synthgen.make_weights(w, gain_std=0.1)
    m = oracle.OracleModel(wts)
    ones = np.ones((w.layers, w.n_kv, 2), np.float32)
    if kvfmt == "fp8":
        m.set_kv_scales(ones)
    prompt = synthgen.make_prompt(w, 12)
    m.prefill(prompt)
    got = m.kv_amax()
    kv = []
    brute.logits_all(wts, prompt, kv_scales=ones if kvfmt == "fp8" else None, collect_kv=kv)
    ref = np.array([[[np.abs(K[:, g]).max(), np.abs(V[:, g]).max()] for g in range(w.n_kv)] for K, V in kv])
    assert ref.min() > 0.05
    np.testing.assert_allclose(got, ref, rtol=2e-3)
    # the maxima restart from zero after a reset
    m.reset_kv_amax()
    assert (m.kv_amax() == 0).all()


@pytest.mark.parametrize("kvfmt", ["bf16", "fp8"])
def test_kv_amax_rounds_to_the_largest_cache_element(kvfmt):
    """Round-to-nearest-even (saturating for E4M3) is monotone in |x|, so the largest |cache
    element| of each (layer, head, K|V) is the maximum rounded into the cache format: exact."""
    w = TINY.with_(kvdtype=kvfmt, wdtype="fp8" if kvfmt == "fp8" else kvfmt, hidden=256, ffn=384, head_dim=128)
    wts = synthgen.make_weights(w, gain_std=0.1)
    m = oracle.OracleModel(wts)
    if kvfmt == "fp8":
        m.set_kv_scales(np.ones((w.layers, w.n_kv, 2), np.float32))
    P = 10
    m.prefill(synthgen.make_prompt(w, P))
    amax = m.kv_amax()
    k, v = m.read_kv(P)
    fmt = oracle.FMT[kvfmt]
    for l in range(w.layers):
        for g in range(w.n_kv):
            for j, c in enumerate((k, v)):
                largest = np.abs(oracle.decode(fmt, c[l, g])).max()
                rounded = abs(float(oracle.decode(fmt, oracle.encode(fmt, amax[l, g, j:j + 1]))[0]))
                assert largest == rounded, (l, g, j, largest, rounded)


def test_derived_fp8_scales_map_layer0_maximum_to_448_and_zero_to_one():
    """With S = amax / 448 the largest calibrated value of layer 0 (whose k and v do not depend on
    the cache contents) becomes the largest E4M3 magnitude; a head whose values are all zero keeps
    scale 1 (here every v, by zeroing Wv)."""
    w = TINY.with_(wdtype="fp8", kvdtype="fp8", hidden=256, ffn=384, head_dim=128)
    wts = synthgen.make_weights(w, gain_std=0.1)
    for d in wts.layers:
        d["wv"][...] = 0
    prompt = synthgen.make_prompt(w, 12)
    cal = oracle.OracleModel(wts)
    cal.set_kv_scales(np.ones((w.layers, w.n_kv, 2), np.float32))
    cal.prefill(prompt)
    amax = cal.kv_amax()
    S = cal.kv_scales_from_amax()
    assert (amax[..., 1] == 0).all() and (S[..., 1] == 1.0).all()
    assert (S[..., 0] > 0).all() and (S[..., 0] != 1.0).all()
    m = oracle.OracleModel(wts)
    m.set_kv_scales(S)
    m.prefill(prompt)
    k, _ = m.read_kv(len(prompt))
    for g in range(w.n_kv):
        assert np.abs(oracle.decode(oracle.E4M3, k[0, g])).max() == 448.0


# ---------------------------------------------------------------------------------------------
# teacher-forced rounding of the appended KV row (the parity protocol's teacher forcing extended
# from the input token to the step's rounding decisions)
# ---------------------------------------------------------------------------------------------
def test_forced_kv_row_equal_to_own_row_changes_nothing(tiny_weights):
    m1, m2 = oracle.OracleModel(tiny_weights), oracle.OracleModel(tiny_weights)
    prompt = synthgen.make_prompt(TINY, 6)
    for m in (m1, m2):
        m.prefill(prompt[:5])
    tok, lg = m1.step(int(prompt[5]))
    k, v = m1.read_kv(6)
    tok2, lg2, own_k, own_v = m2.step_forced(int(prompt[5]), k[:, :, 5], v[:, :, 5])
    assert tok2 == tok and np.array_equal(lg2, lg)
    assert np.array_equal(own_k, k[:, :, 5]) and np.array_equal(own_v, v[:, :, 5])


@pytest.mark.parametrize("kvfmt", ["f16", "fp8"])
def test_forced_kv_row_matches_brute_force(kvfmt):
    """A step that appends a perturbed row (every code of layer 0 moved by one, every V code of the
    last layer by one) against an fp64 recomputation that uses the same row: the forced row is what
    the step's attention reads, and the step's own codes are still reported."""
    w = TINY.with_(kvdtype=kvfmt, wdtype=kvfmt, hidden=256, ffn=384, head_dim=128 if kvfmt == "fp8" else 64)
    wts = synthgen.make_weights(w, gain_std=0.1)
    scales = np.full((w.layers, w.n_kv, 2), 4.0 / 448.0, np.float32) if kvfmt == "fp8" else None
    prompt = synthgen.make_prompt(w, 7)
    ref_m = oracle.OracleModel(wts)
    m = oracle.OracleModel(wts)
    for x in (ref_m, m):
        if scales is not None:
            x.set_kv_scales(scales)
        x.prefill(prompt[:6])
    ref_m.step(int(prompt[6]))
    own_k, own_v = ref_m.read_kv(7)
    fk, fv = own_k[:, :, 6].copy(), own_v[:, :, 6].copy()
    fk[0] = fk[0] + 1
    fv[0] = fv[0] + 1
    fv[-1] = fv[-1] + 1
    _, lg, ok, ov = m.step_forced(int(prompt[6]), fk, fv)
    # layer 0's own k, v do not depend on the forced row (later layers' do: they read it)
    assert np.array_equal(ok[0], own_k[0, :, 6]) and np.array_equal(ov[0], own_v[0, :, 6])
    assert not np.array_equal(ok[-1], own_k[-1, :, 6])
    k_after, v_after = m.read_kv(7)
    assert np.array_equal(k_after[:, :, 6], fk) and np.array_equal(v_after[:, :, 6], fv)
    fmt = oracle.FMT[kvfmt]
    deq = []
    for j, row in enumerate((fk, fv)):
        d = oracle.decode(fmt, row).astype(np.float64)
        if kvfmt == "fp8":
            d = d * scales[:, :, j][:, :, None]
        deq.append(d)
    ref = brute.logits_all(wts, prompt, kv_scales=scales, forced_last=tuple(deq))
    assert np.abs(lg - ref).max() < 2e-3 and np.abs(ref).max() > 0.05
    plain = brute.logits_all(wts, prompt, kv_scales=scales)
    assert np.abs(plain - ref).max() > 10 * np.abs(lg - ref).max()  # the forcing is visible
