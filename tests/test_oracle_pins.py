"""Pins for the CPU oracle: each test checks it against something other than
itself (a library routine, the OCP format definitions, exact arithmetic, a
closed form, an invariant of the layer's mathematics, or an expert-centric
brute force).  CPU only.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from moe_decode_gate_amd import inputs as gen


# ---------------------------------------------------------------- formats --

def test_e4m3_table_matches_torch_all_codes():
    ours = oracle.e4m3_table()
    lib = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert sorted(np.flatnonzero(nan)) == [0x7F, 0xFF]          # S.1111.111 only: the FN variant
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0x7E, 448.0), (0xFE, -448.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
    (0x08, 2.0 ** -6), (0x40, 2.0), (0x3C, 1.5), (0x00, 0.0), (0x78, 256.0),
])
def test_e4m3_format_definition_values(code, value):
    # OCP 8-bit FP E4M3: bias 7, subnormal step 2^-9, largest finite 1.75 * 2^8.
    assert oracle.e4m3_table()[code] == value


def test_e4m3_negative_zero_and_nan():
    t = oracle.e4m3_table()
    assert t[0x80] == 0.0 and math.copysign(1.0, t[0x80]) < 0
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])


def test_e8m0_table_matches_torch_all_scales():
    ours = oracle.e8m0_table()
    lib = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert math.isnan(ours[255]) and math.isnan(lib[255])
    assert np.array_equal(ours[:255], lib[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def test_dequant_is_exact_product_all_65536():
    t = oracle.e4m3_table()
    for s in range(256):
        for c in range(0, 256, 17 if s % 3 else 1):
            v = oracle.dequant(c, s)
            if c in (0x7F, 0xFF) or s == 255:
                assert math.isnan(v)
            else:
                assert v == math.ldexp(t[c], s - 127)


def test_bf16_rne_matches_torch(rng):
    f = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),          # subnormal range
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38, 1e-45], np.float32),
    ])
    # exact ties: low 16 bits == 0x8000, both parities of the kept LSB
    ties = (rng.integers(0x3F000000, 0x40800000, 4000, dtype=np.uint32) & 0xFFFF0000) | 0x8000
    f = np.concatenate([f, ties.view(np.float32)])
    lib = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([oracle.bf16_rne(float(v)) for v in f], np.uint16)
    assert np.array_equal(ours, lib)


def test_bf16_rne_nan_stays_nan():
    b = oracle.bf16_rne(float("nan"))
    assert (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0


def test_bf16_value_roundtrip(rng):
    bits = rng.integers(0, 65536, 5000, dtype=np.uint16)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = np.array([oracle.bf16_value(int(b)) for b in bits])
    fin = ~np.isnan(lib)
    assert np.array_equal(ours[fin], lib[fin]) and np.all(np.isnan(ours[~fin]))


def test_round_f32_matches_numpy(rng):
    v = rng.standard_normal(5000) * 10.0 ** rng.integers(-30, 30, 5000)
    ours = np.array([oracle.round_f32(float(a)) for a in v], np.float32)
    assert np.array_equal(ours, v.astype(np.float32))


def test_silu_matches_torch_and_is_stable():
    g = np.concatenate([np.linspace(-40, 40, 2001), [-750.0, -1e6, 750.0, 1e6, 0.0]])
    lib = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    ours = np.array([oracle.silu(float(a)) for a in g])
    assert np.all(np.isfinite(ours))
    np.testing.assert_allclose(ours, lib, rtol=1e-15, atol=1e-300)
    assert oracle.silu(64.0) == 64.0 * (1.0 / (1.0 + math.exp(-64.0)))


# ----------------------------------------------------------- the layer --

def _tiny_layer(E, K, H, I, seed, std=0.02):
    spec = gen.LayerSpec(E=E, K=K, H=H, I=I, seed=seed)
    return spec, gen.make_layer(spec, std=std)


def _dense_reference(x, ids, w, L):
    """sum_k w_k * MLP_{e_k}(x) with torch float64 matmuls on torch-decoded
    weights; the intermediate is rounded FP64 -> FP32 -> BF16 by torch."""
    def deq(codes, scales):
        v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
        s = torch.from_numpy(scales).view(torch.float8_e8m0fnu).to(torch.float64)
        return v * s.repeat_interleave(32, dim=-1)
    E, I2, H = L.wgu.shape
    I = I2 // 2
    xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    B, K = ids.shape
    y = torch.zeros(B, H, dtype=torch.float64)
    act = np.zeros((B, K, I), np.uint16)
    for b in range(B):
        for k in range(K):
            e = int(ids[b, k])
            gu = deq(L.wgu[e], L.sgu[e])
            dn = deq(L.wd[e], L.sd[e])
            g = gu[:I] @ xf[b]
            u = gu[I:] @ xf[b]
            a = (torch.nn.functional.silu(g) * u).to(torch.float32).to(torch.bfloat16)
            act[b, k] = a.view(torch.int16).numpy().view(np.uint16)
            y[b] += float(w[b, k]) * (dn @ a.to(torch.float64))
    return y.numpy(), act


@pytest.mark.parametrize("E,K,H,I,B", [(4, 1, 64, 32, 2), (4, 2, 64, 32, 3), (8, 2, 128, 64, 1)])
def test_oracle_matches_expert_centric_brute_force(E, K, H, I, B):
    spec, L = _tiny_layer(E, K, H, I, seed=77 + E + K + B, std=0.3)
    t = gen.make_tokens(spec, B)
    y, act = oracle.moe_decode(t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd)
    yb, actb, _ = brute.moe_decode(t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd)
    assert np.array_equal(act, actb)
    np.testing.assert_allclose(y, np.array(yb), rtol=1e-13, atol=1e-300)


@pytest.mark.parametrize("K", [1, 2, 4])
def test_oracle_matches_dense_swiglu_reference(K):
    spec, L = _tiny_layer(16, K, 256, 96, seed=300 + K, std=0.1)
    t = gen.make_tokens(spec, 4)
    y, act = oracle.moe_decode(t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd)
    yr, actr = _dense_reference(t.x, t.ids, t.w, L)
    assert np.array_equal(act, actr)
    np.testing.assert_allclose(y, yr, rtol=1e-12, atol=1e-15)


def test_k1_unit_weight_is_one_dense_mlp():
    spec, L = _tiny_layer(3, 1, 64, 64, seed=9, std=0.2)
    t = gen.make_tokens(spec, 2)
    t.w[:] = 1.0
    y, _ = oracle.moe_decode(t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd)
    yr, _ = _dense_reference(t.x, t.ids, t.w, L)
    np.testing.assert_allclose(y, yr, rtol=1e-12, atol=1e-15)


@pytest.fixture(scope="module")
def small():
    spec, L = _tiny_layer(8, 3, 128, 64, seed=4242, std=0.1)
    t = gen.make_tokens(spec, 5)
    return spec, L, t


def _y(t, L, ids=None, w=None, x=None, sd=None):
    y, _ = oracle.moe_decode(t.x if x is None else x, t.ids if ids is None else ids,
                             t.w if w is None else w, L.wgu, L.sgu, L.wd, L.sd if sd is None else sd)
    return y


def test_invariant_linear_in_router_weights(small):
    spec, L, t = small
    # weights with few significant bits, so that w1 + w2 is exact in FP32
    w1 = (np.round(t.w * 256) / 256).astype(np.float32)
    w2 = (np.random.default_rng(5).integers(-64, 64, t.w.shape) / 32.0).astype(np.float32)
    # y(w1 + w2) = y(w1) + y(w2) and y(2 w) = 2 y(w): the combine is linear in w
    y12 = _y(t, L, w=(w1 + w2).astype(np.float32))
    ysum = _y(t, L, w=w1) + _y(t, L, w=w2)
    np.testing.assert_allclose(y12, ysum, rtol=0, atol=1e-13 * np.abs(ysum).max())
    np.testing.assert_array_equal(_y(t, L, w=(2 * w1).astype(np.float32)), 2 * _y(t, L, w=w1))


def test_invariant_zero_weight_slot_contributes_nothing(small):
    spec, L, t = small
    w = t.w.copy(); w[:, 1] = 0.0
    ids2 = t.ids.copy(); ids2[:, 1] = (ids2[:, 1] + 3) % spec.E
    np.testing.assert_array_equal(_y(t, L, w=w), _y(t, L, w=w, ids=ids2))
    # and equals the layer with that slot removed
    keep = [0, 2]
    y_removed, _ = oracle.moe_decode(t.x, t.ids[:, keep].copy(), t.w[:, keep].copy(), L.wgu, L.sgu, L.wd, L.sd)
    np.testing.assert_allclose(_y(t, L, w=w), y_removed, rtol=1e-14, atol=1e-300)


def test_invariant_slot_permutation(small):
    spec, L, t = small
    p = [2, 0, 1]
    np.testing.assert_allclose(_y(t, L, ids=t.ids[:, p].copy(), w=t.w[:, p].copy()), _y(t, L),
                               rtol=1e-14, atol=1e-300)


def test_invariant_duplicate_expert_equals_summed_weight(small):
    spec, L, t = small
    ids = t.ids.copy(); ids[:, 1] = ids[:, 0]
    w = (np.round(t.w * 1024) / 1024).astype(np.float32)       # so that w0 + w1 is exact
    wsum = w.copy(); wsum[:, 0] = w[:, 0] + w[:, 1]; wsum[:, 1] = 0.0
    y_dup, y_sum = _y(t, L, ids=ids, w=w), _y(t, L, ids=ids, w=wsum)
    np.testing.assert_allclose(y_dup, y_sum, rtol=0, atol=1e-13 * np.abs(y_sum).max())


def test_invariant_token_permutation(small):
    spec, L, t = small
    p = np.array([3, 1, 4, 0, 2])
    yp = _y(t, L, ids=t.ids[p].copy(), w=t.w[p].copy(), x=t.x[p].copy())
    np.testing.assert_array_equal(yp, _y(t, L)[p])


@pytest.mark.parametrize("shift", [1, -3, 5])
def test_invariant_down_scale_shift_scales_output_exactly(small, shift):
    spec, L, t = small
    sd = (L.sd.astype(np.int32) + shift).astype(np.uint8)
    np.testing.assert_array_equal(_y(t, L, sd=sd), _y(t, L) * 2.0 ** shift)


def test_fingerprint_closed_form():
    """Exact closed form.  Gate rows all 2.0 and x all 1.0 give g = 2H = 64,
    and SiLU(64) rounds to exactly 64.  Up rows of expert e hold the single
    code (e+1) at h = 0, so u = e+1 and act = 64 (e+1), exact in BF16.  Down
    row h holds 1.0 at column h (H = I), scale 2^0.  Hence
        y[b,h] = sum_k w[b,k] * 64 * (ids[b,k] + 1)
    for every h: a wrong expert, slot, weight or row index changes the value.
    """
    E, K, H, I = 6, 3, 32, 32
    wgu = np.zeros((E, 2 * I, H), np.uint8)
    sgu = np.full((E, 2 * I, H // 32), 127, np.uint8)
    wgu[:, :I, :] = 0x40                                       # 2.0
    code_of = {1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, 5: 0x4A, 6: 0x4C}   # 1,2,3,4,5,6 in E4M3
    for e in range(E):
        wgu[e, I:, 0] = code_of[e + 1]
    wd = np.zeros((E, H, I), np.uint8)
    sd = np.full((E, H, I // 32), 127, np.uint8)
    for h in range(H):
        wd[:, h, h % I] = 0x38
    x = np.full((2, H), 0x3F80, np.uint16)                     # bf16 1.0
    ids = np.array([[0, 3, 5], [2, 2, 4]], np.int32)
    w = np.array([[0.5, 0.25, 0.125], [0.5, 0.5, 2.0 ** -6]], np.float32)
    y, act = oracle.moe_decode(x, ids, w, wgu, sgu, wd, sd)
    expect = np.array([sum(float(w[b, k]) * 64 * (ids[b, k] + 1) for k in range(K)) for b in range(2)])
    np.testing.assert_array_equal(y, np.repeat(expect[:, None], H, axis=1))
    for b in range(2):
        for k in range(K):
            assert oracle.bf16_value(int(act[b, k, 0])) == 64.0 * (ids[b, k] + 1)


def test_oracle_rejects_out_of_range_ids():
    spec, L = _tiny_layer(4, 2, 64, 32, seed=1)
    t = gen.make_tokens(spec, 2)
    ids = t.ids.copy(); ids[1, 1] = 4
    with pytest.raises(ValueError):
        oracle.moe_decode(t.x, ids, t.w, L.wgu, L.sgu, L.wd, L.sd)
    ids[1, 1] = -1
    with pytest.raises(ValueError):
        oracle.moe_decode(t.x, ids, t.w, L.wgu, L.sgu, L.wd, L.sd)


def test_oracle_thread_count_does_not_change_result(small):
    spec, L, t = small
    y1, a1 = oracle.moe_decode(t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd, nthreads=1)
    y4, a4 = oracle.moe_decode(t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd, nthreads=4)
    assert np.array_equal(a1, a4) and np.array_equal(y1, y4)


def test_nan_code_propagates(small):
    spec, L, t = small
    wd = L.wd.copy()
    e = int(t.ids[0, 0])
    wd[e, 7, 3] = 0x7F
    y, _ = oracle.moe_decode(t.x, t.ids, t.w, L.wgu, L.sgu, wd, L.sd)
    assert math.isnan(y[0, 7])
    assert np.isfinite(np.delete(y[0], 7)).all()


def test_golden_tiny_layer_regression():
    """The tiny layer's generator bits and oracle output are those stored by
    tests/golden/make_golden.py (oracle + generator only)."""
    import hashlib
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_layer.json")
    ref = json.load(open(path))
    spec = gen.CONFIGS["tiny"]["spec"]
    L = gen.make_layer(spec)
    t = gen.make_tokens(spec, 1)
    h = hashlib.sha256()
    for a in (L.wgu, L.sgu, L.wd, L.sd):
        h.update(a.tobytes())
    assert h.hexdigest() == ref["weights_sha256"]
    y, act = oracle.moe_decode(t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd)
    assert act.ravel().tolist() == ref["act_bits"]
    assert [float(v).hex() for v in y.ravel()] == ref["y"]


# ----------------------------------------------------------------- router --

def test_route_matches_numpy_topk_and_scipy_softmax(rng):
    import scipy.special
    logits = rng.standard_normal((50, 128)).astype(np.float32)
    ids, w = oracle.route(logits, 8)
    # library top-k: stable argsort on (-logit) keeps the lower index first among equals
    ref_ids = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :8]
    assert np.array_equal(ids, ref_ids)
    chosen = np.take_along_axis(logits.astype(np.float64), ref_ids, axis=1)
    np.testing.assert_allclose(w, scipy.special.softmax(chosen, axis=1), rtol=1e-14)
    # renormalised full softmax restricted to the chosen set is the same thing
    full = scipy.special.softmax(logits.astype(np.float64), axis=1)
    sel = np.take_along_axis(full, ref_ids, axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-12)


def test_route_ties_and_invariants():
    logits = np.zeros((3, 16), np.float32)
    logits[0, [3, 7, 11]] = 2.0                      # three-way tie: indices ascending
    logits[1, :] = -1.0                               # all equal: 0, 1, 2, ...
    logits[2, 5] = 5.0
    ids, w = oracle.route(logits, 4)
    assert ids[0].tolist() == [3, 7, 11, 0]
    assert ids[1].tolist() == [0, 1, 2, 3]
    assert ids[2, 0] == 5
    np.testing.assert_allclose(w[1], 0.25, rtol=0)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-15)
    # shift invariance and K = 1
    g = np.random.default_rng(3).standard_normal((4, 32)).astype(np.float32)
    i1, w1 = oracle.route(g, 5)
    i2, w2 = oracle.route(g + np.float32(8.0), 5)
    assert np.array_equal(i1, i2)
    np.testing.assert_allclose(w1, w2, rtol=1e-6)     # FP32 inputs: the shift itself rounds
    i3, w3 = oracle.route(g, 1)
    assert np.array_equal(i3[:, 0], i1[:, 0]) and (w3 == 1.0).all()
    with pytest.raises(ValueError):
        oracle.route(g, 33)


def test_route_agrees_with_generator_softmax_routing():
    spec = gen.LayerSpec(E=128, K=8, H=64, I=32, seed=12)
    t = gen.make_tokens(spec, 16)
    ids, w = oracle.route(gen.make_logits(spec, 16), 8)
    assert np.array_equal(ids, t.ids)                 # same draws, FP32 ranking keeps the order
    np.testing.assert_allclose(w, t.w, rtol=1e-6)


# ------------------------------------------------- accuracy experiment --

def test_e4m3_encode_matches_torch(rng):
    # FP32-representable values, so torch's FP32 -> E4M3 conversion sees the same input
    v = np.concatenate([
        rng.uniform(-448, 448, 20000), rng.standard_normal(5000) * 0.01,
        rng.standard_normal(2000) * 2.0 ** -8,                       # subnormal range
    ]).astype(np.float32)
    t = oracle.e4m3_table()
    finite = np.sort(np.unique(t[np.isfinite(t)]))
    mids = ((finite[1:] + finite[:-1]) / 2).astype(np.float32)     # exact ties
    v = np.concatenate([v, mids, -mids, finite.astype(np.float32)])
    ours = np.array([oracle.e4m3_encode(float(a)) for a in v], np.uint8)
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # -0 vs +0 encodings of zero agree in value
    same = (ours == lib) | ((t[ours] == 0) & (t[lib] == 0))
    assert same.all(), v[~same][:10]


def test_mxfp8_quantize_matches_generator(rng):
    v = (rng.standard_normal((37, 256)) * 10.0 ** rng.integers(-3, 2, (37, 1))).astype(np.float32)
    v[3, :32] = 0.0                                                  # an all-zero block
    c1, s1 = oracle.mxfp8_quantize(v.astype(np.float64))
    c2, s2 = gen.quantize_mxfp8(v)
    assert np.array_equal(s1, s2)
    t = oracle.e4m3_table()
    assert np.array_equal(t[c1], t[c2])


def test_mxfp8_quantize_scale_rule_from_the_format(rng):
    """The MX shared scale, pinned by what the OCP MX definition fixes rather
    than by a second copy of the formula: the scale is a power of two that
    puts the block's largest magnitude in the top binade of the element
    format, [2^8, 2^9) for E4M3 (whose largest normal is 1.75 * 2^8 = 448);
    the block maximum's code is then in that binade or saturated at 448; the
    scale byte moves one for one with a power-of-two rescale of the block; and
    every element is within half an E4M3 spacing of its scaled value (or
    saturated)."""
    t = oracle.e4m3_table()
    v = (rng.standard_normal((64, 256)) * 10.0 ** rng.integers(-6, 4, (64, 1))).astype(np.float64)
    codes, sb = oracle.mxfp8_quantize(v)
    blk = v.reshape(64, 8, 32)
    amax = np.abs(blk).max(axis=-1)
    scaled_max = amax * 2.0 ** (127 - sb.astype(np.float64))
    assert ((scaled_max >= 256.0) & (scaled_max < 512.0)).all()
    q = t[codes].reshape(64, 8, 32)
    qmax = np.abs(q).max(axis=-1)
    assert ((qmax >= 256.0) & (qmax <= 448.0)).all()
    # elements: nearest E4M3 value of the scaled input, or saturated at +-448
    sc = blk * 2.0 ** (127 - sb.astype(np.float64))[..., None]
    finite = np.sort(np.unique(np.abs(t[np.isfinite(t)])))
    idx = np.clip(np.searchsorted(finite, np.abs(sc)), 1, len(finite) - 1)
    gap = finite[idx] - finite[idx - 1]
    inside = np.abs(sc) <= 448.0
    assert (np.abs(np.abs(q) - np.abs(sc))[inside] <= gap[inside] / 2 + 1e-300).all()
    assert (np.abs(q)[~inside] == 448.0).all()
    assert (np.sign(q) == np.sign(sc))[np.abs(q) > 0].all()
    # a power-of-two rescale of the input moves every scale byte by the same amount
    for k in (-5, 3, 17):
        c2, s2 = oracle.mxfp8_quantize(np.ldexp(v, k))
        assert np.array_equal(c2, codes) and np.array_equal(s2.astype(int), sb.astype(int) + k)
    # worked values: a block whose largest magnitude is 1.0 has shared exponent -8 (byte 119) and
    # its maximum encodes 256 = 2^8 (code 0x78); one whose largest is 0.875 * 2^-3 keeps exponent -12
    one = np.zeros(32); one[5] = 1.0; one[6] = -0.25
    c, s = oracle.mxfp8_quantize(one)
    assert s[0] == 119 and c[5] == 0x78 and t[c[6]] == -64.0
    b = np.zeros(32); b[0] = 0.875 * 2.0 ** -3                       # = 1.75 * 2^-4
    c, s = oracle.mxfp8_quantize(b)
    assert s[0] == 127 - 12 and t[c[0]] == 448.0
    # a largest magnitude just below the next binade scales to 511.75 and saturates at 448
    b[0] = 1.9990234375 * 2.0 ** -3
    c, s = oracle.mxfp8_quantize(b)
    assert s[0] == 127 - 11 and t[c[0]] == 448.0
    # the scale byte is clamped to E8M0's finite range [0, 254] (255 encodes NaN): far above it the
    # elements saturate, far below they underflow to zero
    c, s = oracle.mxfp8_quantize(np.full(32, 2.0 ** 140))
    assert s[0] == 254 and (t[c] == 448.0).all()
    c, s = oracle.mxfp8_quantize(np.full(32, -(2.0 ** -140)))
    assert s[0] == 0 and (t[c] == 0.0).all()


def _dense_exact(x, ids, w, L):
    def deq(codes, scales):
        v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
        s = torch.from_numpy(scales).view(torch.float8_e8m0fnu).to(torch.float64)
        return v * s.repeat_interleave(32, dim=-1)
    E, I2, H = L.wgu.shape
    I = I2 // 2
    xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    y = torch.zeros(ids.shape[0], H, dtype=torch.float64)
    for b in range(ids.shape[0]):
        for k in range(ids.shape[1]):
            e = int(ids[b, k])
            gu, dn = deq(L.wgu[e], L.sgu[e]), deq(L.wd[e], L.sd[e])
            a = torch.nn.functional.silu(gu[:I] @ xf[b]) * (gu[I:] @ xf[b])
            y[b] += float(w[b, k]) * (dn @ a)
    return y.numpy()


def test_exact_reference_matches_dense_torch():
    spec, L = _tiny_layer(16, 4, 256, 96, seed=71, std=0.1)
    t = gen.make_tokens(spec, 3)
    y = oracle.moe_decode_exact(t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd)
    np.testing.assert_allclose(y, _dense_exact(t.x, t.ids, t.w, L), rtol=1e-12, atol=1e-15)


def test_dense_weights_reference_equals_exact_oracle_on_mxfp8_values():
    """The FP64 reference with real-valued weights, given the MXFP8 weights'
    exact values, is the C oracle's unrounded layer (to FP64 summation order);
    and it is linear in the down weights (doubling them doubles y)."""
    spec, L = _tiny_layer(12, 3, 192, 96, seed=73, std=0.1)
    t = gen.make_tokens(spec, 4)
    t4, t8 = oracle.e4m3_table(), oracle.e8m0_table()
    gu = lambda e: t4[L.wgu[e]] * np.repeat(t8[L.sgu[e]], 32, axis=-1)
    dn = lambda e: t4[L.wd[e]] * np.repeat(t8[L.sd[e]], 32, axis=-1)
    y = oracle.moe_decode_dense_weights(t.x, t.ids, t.w, gu, dn)
    ref = oracle.moe_decode_exact(t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)
    y2 = oracle.moe_decode_dense_weights(t.x, t.ids, t.w, gu, lambda e: 2.0 * dn(e))
    np.testing.assert_allclose(y2, 2.0 * y, rtol=1e-14, atol=1e-16)


def test_conventional_numerics_match_torch_composition():
    """The conventional path rebuilt from library routines: torch's FP8 and
    BF16 conversions (via the generator's quantizer) and float64 matmuls."""
    spec, L = _tiny_layer(16, 4, 256, 96, seed=72, std=0.1)
    t = gen.make_tokens(spec, 3)
    y = oracle.moe_decode_conventional(t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd)

    def deq(codes, scales):
        v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
        s = torch.from_numpy(scales).view(torch.float8_e8m0fnu).to(torch.float64)
        return v * s.repeat_interleave(32, dim=-1)

    def bf16(a):
        return a.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    I = spec.I
    xf = torch.from_numpy(t.x.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    xq = deq(*gen.quantize_mxfp8(xf))
    ref = torch.zeros(3, spec.H, dtype=torch.float64)
    for b in range(3):
        for k in range(spec.K):
            e = int(t.ids[b, k])
            gu, dn = deq(L.wgu[e], L.sgu[e]), deq(L.wd[e], L.sd[e])
            a = bf16(torch.nn.functional.silu(gu[:I] @ xq[b]) * (gu[I:] @ xq[b]))
            aq = deq(*gen.quantize_mxfp8(a.to(torch.float32).numpy()))
            ref[b] += float(t.w[b, k]) * bf16(dn @ aq)
    ref = bf16(ref).numpy()
    # BF16 decisions taken on sums in a different order: allow one-ulp flips, mostly exact
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert (np.abs(y - ref) <= ulp * 1.01).all()
    assert (y == ref).mean() > 0.97


def test_conventional_equals_plain_when_activations_are_mxfp8_exact():
    """If x and every intermediate are already MXFP8 values and the expert
    outputs are BF16-exact, the conventional path's roundings are identities:
    the fingerprint layer (integer activations) gives the closed form."""
    E, K, H, I = 6, 3, 32, 32
    wgu = np.zeros((E, 2 * I, H), np.uint8); sgu = np.full((E, 2 * I, 1), 127, np.uint8)
    wgu[:, :I, :] = 0x40
    for e in range(E):
        wgu[e, I:, 0] = [0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C][e]
    wd = np.zeros((E, H, I), np.uint8); sd = np.full((E, H, 1), 127, np.uint8)
    for h in range(H):
        wd[:, h, h % I] = 0x38
    x = np.full((2, H), 0x3F80, np.uint16)
    ids = np.array([[0, 3, 5], [2, 1, 4]], np.int32)
    w = np.array([[0.5, 0.25, 0.125], [0.5, 0.25, 0.25]], np.float32)
    yc = oracle.moe_decode_conventional(x, ids, w, wgu, sgu, wd, sd)
    ye = oracle.moe_decode_exact(x, ids, w, wgu, sgu, wd, sd)
    expect = np.array([sum(float(w[b, k]) * 64 * (ids[b, k] + 1) for k in range(K)) for b in range(2)])
    np.testing.assert_array_equal(yc, np.repeat(expect[:, None], H, axis=1))
    np.testing.assert_allclose(ye, yc, rtol=1e-14)
