"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Inputs are the seeded synthetic layers of the shapes the warp-decode pages
measure (128 experts, top-8, hidden 2048; "Better MoE model inference with
warp decode", Key claims) plus a larger layer, a tiny one and ragged/edge
shapes.  Gates (see tests/gpu_common.py): the intermediate matches the
oracle's BF16 bits except for rare flips (one ulp, or a few ulps on values
far below their row's scale); outputs reach cosine
>= 0.99999 and max |err| <= 4e-3 at unit output scale, and every element
lies within half a BF16 ulp (plus FP32 summation noise) of the FP64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_decode_gate_amd import inputs as gen
from tests.gpu_common import (DevLayer, DevTokens, act_flip_propagation, act_flip_stats, assert_act_flips, assert_output_parity, bits_of, log,
                              run_layer, shifted, unit_shift, bf16_bits_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_decode_gate_amd import binding  # noqa: F401  (fails loudly if the library is missing)
    torch.cuda.set_device(0)


_LAYERS = {}


def layer_for(spec: gen.LayerSpec, experts=None):
    key = (spec, None if experts is None else tuple(sorted(set(int(e) for e in experts))))
    if key not in _LAYERS:
        _LAYERS.clear()                       # keep at most one big layer resident
        log(f"[gen] layer {spec} experts={'all' if experts is None else len(key[1])}")
        _LAYERS[key] = DevLayer(gen.make_layer(spec, experts=experts, threads=16))
    return _LAYERS[key]


CASES = {
    # name: (spec, B, routing, generate only routed experts)
    "tiny_b1": (gen.CONFIGS["tiny"]["spec"], 1, "softmax", False),
    "tiny_b7": (gen.CONFIGS["tiny"]["spec"], 7, "softmax", False),
    "qwen3_b1": (gen.CONFIGS["qwen3"]["spec"], 1, "softmax", True),
    "qwen3_b32": (gen.CONFIGS["qwen3_b32"]["spec"], 32, "softmax", True),
    "large_b1": (gen.CONFIGS["large"]["spec"], 1, "zipf", True),
    "large_b8": (gen.CONFIGS["large"]["spec"], 8, "zipf", True),
    "large_b32": (gen.CONFIGS["large"]["spec"], 32, "zipf", True),
    "ragged": (gen.LayerSpec(E=5, K=3, H=96, I=160, seed=501), 3, "softmax", False),
    "k1_e1": (gen.LayerSpec(E=1, K=1, H=64, I=32, seed=502), 2, "softmax", False),
    "wide_h8192": (gen.LayerSpec(E=4, K=2, H=8192, I=64, seed=503), 2, "softmax", False),
    "deep_ki16384": (gen.LayerSpec(E=6, K=4, H=64, I=4096, seed=504), 2, "softmax", False),
    "b64": (gen.LayerSpec(E=16, K=4, H=256, I=96, seed=505), 64, "softmax", False),
    # H/32 = 9 scale bytes per row: rows start off 4-byte boundaries (byte-wise scale loads)
    "h288": (gen.LayerSpec(E=6, K=2, H=288, I=64, seed=506), 3, "softmax", False),
    # 12 and 28 scale bytes per row: the matrix-core kernels' last batch of 4 steps is partial and
    # its 8-byte scale window would end past the row (a wrong window once gave cosine 0.994)
    "scale_rows_4mod8": (gen.LayerSpec(E=12, K=5, H=384, I=896, seed=507), 40, "softmax", False),
}


MODES = {
    0: (None, None),                                   # the library's defaults for the batch size
    1: (dict(math=1, form=1), dict(math=1)),           # FP32 math, token form
    2: (dict(math=2, form=1), dict(math=2)),           # BF16-pair math, token form
    3: (dict(form=3), None),                           # gate/up on the matrix cores (expert form)
    4: (dict(form=3), dict(form=3)),                   # both on the matrix cores (8-wave down)
    5: (None, dict(form=3, waves_per_block=16, token_split=1)),   # down on the matrix cores, 16 waves
    6: (None, dict(form=3, waves_per_block=16, token_split=2)),   # two token ranges per output block
}


@pytest.mark.parametrize("math", list(MODES))
@pytest.mark.parametrize("name", list(CASES))
def test_layer_parity(name, math):
    """Each case under the library's defaults, the two VALU math modes of the
    token form, the matrix-core expert form of gate/up, and down on the matrix
    cores (8 and 16 waves per workgroup)."""
    spec, B, routing, only_routed = CASES[name]
    cfg_gu, cfg_dn = MODES[math]
    log(f"[case] {name} B={B} routing={routing} mode={math}")
    t = gen.make_tokens(spec, B, routing=routing)
    dl = layer_for(spec, experts=t.ids.ravel() if only_routed else None)
    L = dl.host
    dt = DevTokens(t)
    y64, act_o = oracle.moe_decode(t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd, nthreads=16)
    k = unit_shift(y64)
    sd_k = shifted(dl.sd, k)

    act, out = run_layer(dl, dt, sd=sd_k, cfg_gu=cfg_gu, cfg_dn=cfg_dn)
    frac, ulps, within = act_flip_stats(bits_of(act), act_o)
    log(f"[act] {name}: flip fraction {frac:.2e}, max {ulps:.2f} ulp, all within bound: {within}, n={act_o.size}")
    # rare flips; each within one ulp, or (cancellation) within 2^-14 of the row's scale
    assert_act_flips(frac, act_o.size, within, name)

    # down kernel alone, fed the oracle's intermediate: only FP32 summation and output rounding differ
    from moe_decode_gate_amd import binding as wd
    act_dev = torch.from_numpy(act_o.view(np.int16)).cuda().view(torch.bfloat16)
    out_k2 = wd.down(act_dev, dt.ids, dt.w, dl.wd, sd_k, cfg=cfg_dn)
    torch.cuda.synchronize()
    assert_output_parity(bits_of(out_k2), y64 * 2.0 ** k, f"{name} down-only (Sd{k:+d})")
    # whole layer against the oracle's down projection of the GPU's own intermediate
    y_of_gpu_act = oracle.down(bits_of(act), t.ids, t.w, L.wd, L.sd, nthreads=16)
    assert_output_parity(bits_of(out), y_of_gpu_act * 2.0 ** k, f"{name} layer vs oracle(act_gpu) (Sd{k:+d})")
    # whole layer against the oracle end to end: the down-stage bound plus the exact
    # propagation of the intermediate values where the GPU's differ from the oracle's
    prop = act_flip_propagation(bits_of(act), act_o, t.ids, t.w, L.wd, L.sd)
    assert_output_parity(bits_of(out), y64 * 2.0 ** k, f"{name} layer (Sd{k:+d})", extra=prop * 2.0 ** k)
    # the literal, unshifted data: cosine and per-element bounds still hold
    if k != 0:
        _, out0 = run_layer(dl, dt, cfg_gu=cfg_gu, cfg_dn=cfg_dn)
        assert_output_parity(bits_of(out0), y64, f"{name} layer (unshifted)", unit_scale=False, extra=prop)


@pytest.mark.parametrize("math", [1, 2])
def test_dequant_probe_matches_format_definition(math):
    """The hardware conversion, exactly as the kernels use it (math mode 1:
    to FP32; 2: to BF16), against the OCP E4M3 x E8M0 definition for all 256
    codes x 256 scale bytes x 4 byte lanes.  Both targets hold every product
    whose magnitude is a normal FP32 number exactly."""
    from moe_decode_gate_amd import binding as wd
    got = wd.dequant_probe()[math - 1].cpu().numpy().astype(np.float64)   # [s, c, lane]
    t4, t8 = oracle.e4m3_table(), oracle.e8m0_table()
    codes = (np.arange(256)[:, None] + np.arange(4)[None, :]) & 255    # [c, lane]
    exact = t8[:, None, None] * t4[codes][None, :, :]                  # FP64 exact product
    with np.errstate(over="ignore"):
        want32 = exact.astype(np.float32).astype(np.float64)
    s_idx = np.arange(256)[:, None, None] * np.ones((1, 256, 4))
    nan_code = np.isnan(t4[codes])[None].repeat(256, 0)
    normal = (np.abs(want32) >= 2.0 ** -126) & np.isfinite(want32)
    zero = exact == 0
    core = (s_idx >= 1) & (s_idx <= 254) & ~nan_code & (normal | zero)
    bad = core & (got != want32)
    log(f"[probe] core cases {int(core.sum())}, mismatches {int(bad.sum())}")
    assert not bad.any(), np.argwhere(bad)[:10]
    # signed zeros
    assert np.array_equal(np.signbit(got[core & zero]), np.signbit(exact[core & zero]))
    # NaN codes stay NaN for every scale in range
    assert np.isnan(got[(s_idx >= 1) & (s_idx <= 254) & nan_code]).all()
    # the remaining classes: FP32-overflowing and FP32-subnormal products, E8M0 bytes 0 and 255
    rest = ~core & ~nan_code
    inr = (s_idx >= 1) & (s_idx <= 254)
    for name, m in (("fp32 overflow", rest & inr & ~np.isfinite(want32)),
                    ("fp32 subnormal", rest & inr & np.isfinite(want32)),
                    ("s=0", rest & (s_idx == 0)), ("s=255", rest & (s_idx == 255))):
        eq = (got[m] == want32[m]) | (np.isnan(got[m]) & np.isnan(want32[m]))
        log(f"[probe] {name}: {int(m.sum())} cases, {int(eq.sum())} equal to FP32(exact); "
            f"zeros {int((got[m] == 0).sum())}, inf {int(np.isinf(got[m]).sum())}, nan {int(np.isnan(got[m]).sum())}")
    # E8M0 byte 255 is NaN for every code; overflow gives a signed infinity
    assert np.isnan(got[s_idx == 255]).all()
    ovf = rest & inr & ~np.isfinite(want32)
    assert np.array_equal(got[ovf], want32[ovf])
    sub = rest & ((s_idx == 0) | inr) & np.isfinite(want32) & ~(s_idx == 255)
    if math == 1:
        # FP32 conversion: exact also for subnormal products and E8M0 byte 0 (2^-127)
        assert np.array_equal(got[sub], want32[sub])
    else:
        # BF16 conversion: FP32-subnormal products land on BF16 subnormals (step 2^-133),
        # rounded to nearest
        assert (np.abs(got[sub] - exact[sub]) <= 2.0 ** -134).all()
