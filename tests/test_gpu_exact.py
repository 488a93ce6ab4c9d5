"""Bit-exact GPU checks of indexing, routing and determinism.

All arithmetic in the fingerprint layer is exact in FP32, so any wrong expert,
row, column, scale block, slot or router weight shows up as a changed integer.
The remaining tests compare the HIP path with itself under transformations
that must leave the bits unchanged (token permutation, launch configuration,
zero-weight slots) or scale them exactly (down-projection E8M0 shift).
"""
import numpy as np
import pytest
import torch

import oracle

from moe_decode_gate_amd import inputs as gen
from tests.gpu_common import (DevLayer, DevTokens, act_flip_stats, assert_act_flips, assert_output_parity, bits_of, log,
                              run_layer, shifted)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _e4m3_int(v: int) -> int:
    """E4M3 code of a small positive integer 1..15 (exact)."""
    if v == 1:
        return 0x38
    e = v.bit_length() - 1
    m = (v - (1 << e)) << (3 - e) if e <= 3 else 0
    return ((e + 7) << 3) | m


def fingerprint_layer(E, K, H, I):
    """x = 1; gate row = code 1.0 under scale 2^1 (value 2) so g = 2H and
    SiLU(g) = g exactly in FP32; up row j of expert e = the single integer
    u(e,j) = (7e + 3j) % 15 + 1 at column j % H; down row h of expert e = one
    1.0 at column i(e,h) = (h + e) % I with block scale 2^((h + e) % 3).
    Scale bytes of the other blocks are 2^-20 so a wrong block is visible."""
    wgu = np.zeros((E, 2 * I, H), np.uint8)
    sgu = np.full((E, 2 * I, H // 32), 127 - 20, np.uint8)
    wgu[:, :I, :] = 0x38
    sgu[:, :I, :] = 128
    u = np.zeros((E, I), np.int64)
    for e in range(E):
        for j in range(I):
            u[e, j] = (7 * e + 3 * j) % 15 + 1
            wgu[e, I + j, j % H] = _e4m3_int(int(u[e, j]))
            sgu[e, I + j, (j % H) // 32] = 127
    wd = np.zeros((E, H, I), np.uint8)
    sd = np.full((E, H, I // 32), 127 - 20, np.uint8)
    for e in range(E):
        for h in range(H):
            i = (h + e) % I
            wd[e, h, i] = 0x38
            sd[e, h, i // 32] = 127 + (h + e) % 3
    spec = gen.LayerSpec(E=E, K=K, H=H, I=I, seed=0)
    return gen.Layer(spec, wgu, sgu, wd, sd, tuple(range(E))), u


def fingerprint_expect(u, ids, w, H, I):
    """Closed form: act[b,k,j] = 2H u(e,j); y[b,h] = sum_k w_k 2H u(e, i) 2^((h+e)%3), i = (h+e)%I."""
    B, K = ids.shape
    y = np.zeros((B, H), np.float64)
    act = np.zeros((B, K, I), np.float64)
    for b in range(B):
        for k in range(K):
            e = int(ids[b, k])
            act[b, k] = 2 * H * u[e]
            for h in range(H):
                y[b, h] += float(w[b, k]) * 2 * H * u[e, (h + e) % I] * 2.0 ** ((h + e) % 3)
    return act, y


def _bf16_bits(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


FINGERPRINT_CFGS = {
    "defaults": (None, None),
    "token-f32": (dict(form=1, math=1), dict(math=1)),
    "token-dot2": (dict(form=1, math=2), dict(math=2)),
    "expert": (dict(form=2), dict(math=2, rows_per_wave=8)),
    "lanes16": (dict(form=1, lanes_per_row=16, rows_per_wave=2), dict(math=1, rows_per_wave=4)),
    "matrix-cores": (dict(form=3), None),
    "matrix-cores-both": (dict(form=3), dict(form=3)),
    "matrix-core-down-16w": (None, dict(form=3, waves_per_block=16, token_split=1)),
    "matrix-core-down-2-ranges": (None, dict(form=3, waves_per_block=16, token_split=2)),
}


@pytest.mark.parametrize("cfgname", list(FINGERPRINT_CFGS))
@pytest.mark.parametrize("E,K,H,I,B", [(128, 8, 2048, 768, 32), (8, 2, 128, 64, 3), (5, 3, 96, 160, 4)])
def test_routing_fingerprint_bit_exact(E, K, H, I, B, cfgname):
    cfg_gu, cfg_dn = FINGERPRINT_CFGS[cfgname]
    if cfgname == "lanes16" and H > 2048:
        pytest.skip("16 lanes per row holds at most H = 2048")
    log(f"[case] fingerprint E={E} K={K} H={H} I={I} B={B} cfg={cfgname}")
    L, u = fingerprint_layer(E, K, H, I)
    rng = np.random.default_rng(E + K + H + I + B)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(B)]).astype(np.int32)
    w = np.array([[2.0 ** -(k + 1) for k in range(K)]] * B, np.float32)
    x = np.full((B, H), 0x3F80, np.uint16)
    dl, dt = DevLayer(L), DevTokens(gen.Tokens(x=x, ids=ids, w=w))
    act, out = run_layer(dl, dt, cfg_gu=cfg_gu, cfg_dn=cfg_dn)
    act_e, y_e = fingerprint_expect(u, ids, w, H, I)
    assert np.array_equal(bits_of(act), _bf16_bits(act_e))       # act values are exact in BF16
    assert np.array_equal(bits_of(out), _bf16_bits(y_e))         # y exact in FP32, then one RNE


@pytest.fixture(scope="module")
def mid():
    spec = gen.LayerSpec(E=32, K=4, H=1536, I=320, seed=77)     # both kernels with a lane tail
    L = gen.make_layer(spec, threads=16)
    t = gen.make_tokens(spec, 9)
    return DevLayer(L), t


def test_token_permutation_bit_exact(mid):
    dl, t = mid
    _, out = run_layer(dl, DevTokens(t))
    p = np.random.default_rng(0).permutation(t.ids.shape[0])
    tp = gen.Tokens(x=t.x[p].copy(), ids=t.ids[p].copy(), w=t.w[p].copy())
    _, outp = run_layer(dl, DevTokens(tp))
    assert np.array_equal(bits_of(outp), bits_of(out)[p])


@pytest.mark.parametrize("k", [1, 3, -2])
def test_down_scale_shift_scales_output_exactly(mid, k):
    dl, t = mid
    dt = DevTokens(t)
    _, out = run_layer(dl, dt)
    _, outk = run_layer(dl, dt, sd=shifted(dl.sd, k))
    want = (torch.from_numpy(bits_of(out).view(np.int16)).view(torch.bfloat16).float() * 2.0 ** k)
    assert np.array_equal(bits_of(outk), want.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_zero_weight_slot_ignores_its_expert(mid):
    dl, t = mid
    w = t.w.copy(); w[:, 2] = 0.0
    ids2 = t.ids.copy(); ids2[:, 2] = (ids2[:, 2] + 5) % dl.spec.E
    _, a = run_layer(dl, DevTokens(gen.Tokens(x=t.x, ids=t.ids, w=w)))
    _, b = run_layer(dl, DevTokens(gen.Tokens(x=t.x, ids=ids2, w=w)))
    assert np.array_equal(bits_of(a), bits_of(b))


def test_deterministic_and_full_coverage(mid):
    """Outputs pre-filled with NaN are fully overwritten; reruns are bit-identical."""
    from moe_decode_gate_amd import binding as wd
    dl, t = mid
    dt = DevTokens(t)
    B, K = t.ids.shape
    act = torch.full((B, K, dl.spec.I), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = torch.full((B, dl.spec.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    wd.gate_up(dt.x, dt.ids, dl.wgu, dl.sgu, act=act)
    wd.down(act, dt.ids, dt.w, dl.wd, dl.sd, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(act.float()).all() and torch.isfinite(out.float()).all()
    a1, o1 = bits_of(act), bits_of(out)
    for _ in range(3):
        a2, o2 = run_layer(dl, dt)
        assert np.array_equal(bits_of(a2), a1) and np.array_equal(bits_of(o2), o1)


def test_launch_configurations_agree_bitwise(mid):
    """Rows per wave, waves per workgroup, work order and XCD numbering change
    only which wave computes an output, never how: results are bit-identical.
    (Lanes per gate/up row changes the summation order; see the next test.)"""
    dl, t = mid
    dt = DevTokens(t)
    for math in (1, 2):
        base = dict(math=math, form=1, lanes_per_row=64, weight_loads=1)
        a0, o0 = run_layer(dl, dt, cfg_gu=base, cfg_dn=base)
        a0, o0 = bits_of(a0), bits_of(o0)
        for r in (1, 2, 4, 8):
            for wpb in (1, 3, 4):
                for order in (1, 2):
                    for remap in (1, 2):
                        cfg = dict(rows_per_wave=r, waves_per_block=wpb, order=order, xcd_remap=remap, math=math,
                                   form=1, lanes_per_row=64, weight_loads=1)
                        cfg_gu = dict(cfg, rows_per_wave=min(r, 4))
                        a, o = run_layer(dl, dt, cfg_gu=cfg_gu, cfg_dn=cfg)
                        assert np.array_equal(bits_of(a), a0), cfg
                        assert np.array_equal(bits_of(o), o0), cfg


@pytest.mark.parametrize("lpr", [16, 32, 64])
def test_gate_up_lane_groups(mid, lpr):
    """Gate/up with 16, 32 or 64 lanes per row: every row/order/grouping gives
    the same bits for a fixed lane count, and all lane counts stay within the
    intermediate parity bounds of each other (only the FP32 summation order
    differs)."""
    from tests.gpu_common import act_flip_stats
    dl, t = mid
    dt = DevTokens(t)
    ref, _ = run_layer(dl, dt, cfg_gu=dict(math=2, lanes_per_row=64), cfg_dn=dict(math=2))
    a0 = None
    for r in (1, 2, 4):
        for order in (1, 2):
            for remap in (1, 2):
                cfg = dict(rows_per_wave=r, order=order, xcd_remap=remap, math=2, lanes_per_row=lpr)
                a, _ = run_layer(dl, dt, cfg_gu=cfg, cfg_dn=dict(math=2))
                if a0 is None:
                    a0 = bits_of(a)
                assert np.array_equal(bits_of(a), a0), cfg
    frac, ulps, within = act_flip_stats(a0, bits_of(ref))
    assert_act_flips(frac, a0.size, within, f"lanes per row {lpr}")


@pytest.mark.parametrize("B", [1, 9, 40])
def test_gate_up_expert_form_matches_token_form(B):
    """The expert form (one wave per expert row block, serving every slot
    routed to it) keeps the token form's lane layout and summation order:
    its intermediate is bit-identical, for any routing (duplicates, unused
    experts, many tokens per expert)."""
    spec = gen.LayerSpec(E=16, K=4, H=1536, I=320, seed=91)
    dl = DevLayer(gen.make_layer(spec, threads=16))
    t = gen.make_tokens(spec, B, routing="zipf")
    t.ids[0, 1] = t.ids[0, 0]                      # a duplicated expert within a token
    dt = DevTokens(t)
    ref, _ = run_layer(dl, dt, cfg_gu=dict(form=1, math=2, lanes_per_row=64, weight_loads=1))
    for r in (1, 2, 4):
        for order in (1, 2):
            for remap in (1, 2):
                a, _ = run_layer(dl, dt, cfg_gu=dict(form=2, rows_per_wave=r, order=order, xcd_remap=remap))
                assert np.array_equal(bits_of(a), bits_of(ref)), (r, order, remap)


def test_gate_up_expert_form_bad_ids():
    spec = gen.LayerSpec(E=16, K=4, H=1536, I=320, seed=92)
    dl = DevLayer(gen.make_layer(spec, threads=16))
    t = gen.make_tokens(spec, 12)
    ids = t.ids.copy(); ids[3, 2] = 16; ids[7, 0] = -5
    dt = DevTokens(gen.Tokens(x=t.x, ids=ids, w=t.w))
    a, o = run_layer(dl, dt, cfg_gu=dict(form=2))
    af = a.float().cpu().numpy()
    assert np.isnan(af[3, 2]).all() and np.isnan(af[7, 0]).all()
    assert np.isfinite(np.delete(af.reshape(-1, spec.I), [3 * 4 + 2, 7 * 4 + 0], axis=0)).all()
    of = o.float().cpu().numpy()
    assert np.isnan(of[3]).all() and np.isnan(of[7]).all()


@pytest.mark.parametrize("B", [3, 40, 64])
def test_gate_up_matrix_core_form(B):
    """The expert form on the matrix cores sums in another order than the token
    form (the matrix core's FP32 accumulation), so it is held to the oracle:
    rare one-ulp flips only.  Zipf routing over 16 experts puts more than 16
    slots on popular experts (several slot groups per wave), and one token
    repeats an expert; reruns are bit-identical."""
    spec = gen.LayerSpec(E=16, K=4, H=1536, I=320, seed=93)
    L = gen.make_layer(spec, threads=16)
    dl = DevLayer(L)
    t = gen.make_tokens(spec, B, routing="zipf")
    t.ids[0, 1] = t.ids[0, 0]
    dt = DevTokens(t)
    a, _ = run_layer(dl, dt, cfg_gu=dict(form=3))
    ref = oracle.gate_up(t.x, t.ids, L.wgu, L.sgu, nthreads=16)
    frac, ulps, within = act_flip_stats(bits_of(a), ref)
    log(f"[mfma form] B={B}: max slots per expert {np.bincount(t.ids.ravel()).max()}, flips {frac:.2e}, "
        f"max {ulps:.1f} ulp")
    assert_act_flips(frac, ref.size, within, f"matrix-core gate/up B={B}")
    for _ in range(2):
        a2, _ = run_layer(dl, dt, cfg_gu=dict(form=3))
        assert np.array_equal(bits_of(a2), bits_of(a))


def test_gate_up_matrix_core_form_bad_ids():
    spec = gen.LayerSpec(E=16, K=4, H=1536, I=320, seed=94)
    dl = DevLayer(gen.make_layer(spec, threads=16))
    t = gen.make_tokens(spec, 12)
    ids = t.ids.copy(); ids[3, 2] = 16; ids[7, 0] = -5
    dt = DevTokens(gen.Tokens(x=t.x, ids=ids, w=t.w))
    a, o = run_layer(dl, dt, cfg_gu=dict(form=3))
    af = a.float().cpu().numpy()
    assert np.isnan(af[3, 2]).all() and np.isnan(af[7, 0]).all()
    assert np.isfinite(np.delete(af.reshape(-1, spec.I), [3 * 4 + 2, 7 * 4 + 0], axis=0)).all()
    of = o.float().cpu().numpy()
    assert np.isnan(of[3]).all() and np.isnan(of[7]).all()


@pytest.mark.parametrize("H,B,routing", [(1536, 3, "zipf"), (1536, 40, "zipf"), (1536, 64, "zipf"),
                                          (256, 24, "softmax"), (768, 33, "zipf"), (2048, 32, "softmax"),
                                          (4096, 8, "zipf"), (1280, 100, "zipf")])
def test_gate_up_lds_form_matches_register_form(H, B, routing):
    """The matrix-core gate/up that streams its codes into LDS (form 4) does
    the same products in the same order as the register-staged one (form 3),
    so the intermediate is bit-identical -- over one and several batches per
    row (H = 256 .. 4096), one and several 16-slot groups per expert (Zipf
    routing over 16 experts: up to ~70 slots on one expert at B = 100), a token
    that repeats an expert, and experts no slot uses; reruns are identical.
    Form 3 with 16 slots per pass over an expert's rows gives the same bits as
    32 (two 16-slot tiles per weight batch).  Both without the H split, which
    sums the two halves of H separately."""
    spec = gen.LayerSpec(E=16, K=4, H=H, I=320, seed=96 + H + B)
    L = gen.make_layer(spec, threads=16)
    dl = DevLayer(L)
    t = gen.make_tokens(spec, B, routing=routing)
    t.ids[0, 1] = t.ids[0, 0]
    dt = DevTokens(t)
    a3, _ = run_layer(dl, dt, cfg_gu=dict(form=3, h_split=1))
    a4, _ = run_layer(dl, dt, cfg_gu=dict(form=4))
    log(f"[lds form] H={H} B={B}: max slots per expert {np.bincount(t.ids.ravel()).max()}")
    assert np.array_equal(bits_of(a4), bits_of(a3))
    a4b, _ = run_layer(dl, dt, cfg_gu=dict(form=4, waves_per_block=2))
    assert np.array_equal(bits_of(a4b), bits_of(a3))
    a16, _ = run_layer(dl, dt, cfg_gu=dict(form=3, h_split=1, slots_per_pass=16))
    assert np.array_equal(bits_of(a16), bits_of(a3))
    if B <= 40:
        ref = oracle.gate_up(t.x, t.ids, L.wgu, L.sgu, nthreads=16)
        frac, ulps, within = act_flip_stats(bits_of(a4), ref)
        assert_act_flips(frac, ref.size, within, f"lds gate/up H={H} B={B}")


@pytest.mark.parametrize("H,B,routing", [(512, 3, "zipf"), (1024, 24, "softmax"), (2048, 32, "softmax"),
                                          (1536, 40, "zipf"), (4096, 8, "zipf"), (1536, 100, "zipf")])
def test_gate_up_h_split(H, B, routing):
    """The matrix-core gate/up with each (expert, 16 rows) served by a pair of
    waves, one per half of the H axis (h_split 2): held to the oracle's
    intermediate like the other forms; 16 and 32 slots per pass give the same
    bits; reruns are identical; a token's values do not depend on the other
    tokens (a reversed batch gives the reversed intermediate bit for bit); ids
    outside [0, E) give NaN rows."""
    spec = gen.LayerSpec(E=16, K=4, H=H, I=320, seed=196 + H + B)
    L = gen.make_layer(spec, threads=16)
    dl = DevLayer(L)
    t = gen.make_tokens(spec, B, routing=routing)
    t.ids[0, 1] = t.ids[0, 0]
    dt = DevTokens(t)
    a2, _ = run_layer(dl, dt, cfg_gu=dict(form=3, h_split=2))
    log(f"[h split] H={H} B={B}: max slots per expert {np.bincount(t.ids.ravel()).max()}")
    again, _ = run_layer(dl, dt, cfg_gu=dict(form=3, h_split=2))
    assert np.array_equal(bits_of(again), bits_of(a2))
    a16, _ = run_layer(dl, dt, cfg_gu=dict(form=3, h_split=2, slots_per_pass=16))
    assert np.array_equal(bits_of(a16), bits_of(a2))
    rev = gen.Tokens(x=t.x[::-1].copy(), ids=t.ids[::-1].copy(), w=t.w[::-1].copy())
    ar, _ = run_layer(dl, DevTokens(rev), cfg_gu=dict(form=3, h_split=2))
    assert np.array_equal(bits_of(ar)[::-1], bits_of(a2))
    if B <= 40:
        ref = oracle.gate_up(t.x, t.ids, L.wgu, L.sgu, nthreads=16)
        frac, ulps, within = act_flip_stats(bits_of(a2), ref)
        assert_act_flips(frac, ref.size, within, f"h-split gate/up H={H} B={B}")
    ids = t.ids.copy(); ids[1, 2] = 16; ids[B - 1, 0] = -5
    ab, _ = run_layer(dl, DevTokens(gen.Tokens(x=t.x, ids=ids, w=t.w)), cfg_gu=dict(form=3, h_split=2))
    af = ab.float().cpu().numpy()
    assert np.isnan(af[1, 2]).all() and np.isnan(af[B - 1, 0]).all()


def test_gate_up_lds_form_bad_ids_and_default():
    """Form 4 writes NaN rows for ids outside [0, E), and its intermediate is
    bit-identical to the default's (form 3 from B = 18)."""
    spec = gen.LayerSpec(E=16, K=4, H=1024, I=320, seed=97)
    dl = DevLayer(gen.make_layer(spec, threads=16))
    t = gen.make_tokens(spec, 30)
    ids = t.ids.copy(); ids[3, 2] = 16; ids[7, 0] = -5
    dt = DevTokens(gen.Tokens(x=t.x, ids=ids, w=t.w))
    a, o = run_layer(dl, dt, cfg_gu=dict(form=4))
    af = a.float().cpu().numpy()
    assert np.isnan(af[3, 2]).all() and np.isnan(af[7, 0]).all()
    assert np.isfinite(np.delete(af.reshape(-1, spec.I), [3 * 4 + 2, 7 * 4 + 0], axis=0)).all()
    a_def, _ = run_layer(dl, dt)
    assert np.array_equal(bits_of(a_def), bits_of(a))


def _down(act, ids, w, dl, cfg):
    from moe_decode_gate_amd import binding as wd
    out = wd.down(act, ids, w, dl.wd, dl.sd, cfg=cfg)
    torch.cuda.synchronize()
    return bits_of(out)


@pytest.mark.parametrize("B,W", [(3, 8), (32, 16), (40, 8), (64, 8), (64, 16)])
def test_down_matrix_core_form(B, W):
    """Down on the matrix cores sums in another order than the token form (the
    matrix core's FP32 accumulation; each token's slots folded in expert
    order), so it is held to the oracle's down projection of the same
    intermediate.  Zipf routing over 16 experts puts more slots on popular
    experts than one slot group holds, and two tokens repeat an expert (one of
    them three times).  Reruns are bit-identical; permuting the tokens permutes
    the output rows exactly (each result column of the matrix instruction
    depends only on its own slot), and so does reversing the top-k order of
    tokens without a repeated expert."""
    from moe_decode_gate_amd import binding as wd
    spec = gen.LayerSpec(E=16, K=4, H=1536, I=320, seed=96)
    L = gen.make_layer(spec, threads=16)
    dl = DevLayer(L)
    t = gen.make_tokens(spec, B, routing="zipf")
    t.ids[0, 1] = t.ids[0, 0]
    if B > 2:
        t.ids[2, 1] = t.ids[2, 2] = t.ids[2, 0]
    dt = DevTokens(t)
    cfg = dict(form=3, waves_per_block=W, token_split=1)
    act = wd.gate_up(dt.x, dt.ids, dl.wgu, dl.sgu)
    torch.cuda.synchronize()
    ob = _down(act, dt.ids, dt.w, dl, cfg)
    y64 = oracle.down(bits_of(act), t.ids, t.w, L.wd, L.sd, nthreads=16)
    log(f"[mfma down] B={B} W={W}: max slots per expert {np.bincount(t.ids.ravel()).max()}")
    assert_output_parity(ob, y64, f"down matrix cores B={B} W={W}", unit_scale=False)
    for _ in range(2):
        assert np.array_equal(_down(act, dt.ids, dt.w, dl, cfg), ob)
    perm = np.random.default_rng(B).permutation(B)
    pt = torch.from_numpy(perm).cuda()
    assert np.array_equal(_down(act[pt].contiguous(), dt.ids[pt].contiguous(), dt.w[pt].contiguous(), dl, cfg),
                          ob[perm])
    rev = _down(act.flip(1).contiguous(), dt.ids.flip(1).contiguous(), dt.w.flip(1).contiguous(), dl, cfg)
    plain = np.array([len(set(r)) == spec.K for r in t.ids])
    assert np.array_equal(rev[plain], ob[plain])
    # the batch cut into token ranges, one workgroup per range and block: a token's sums
    # do not depend on the other tokens, so the output is the same bit for bit
    for S in (2, 4):
        log(f"[mfma down] B={B} W={W} token_split={S}")
        assert np.array_equal(_down(act, dt.ids, dt.w, dl, dict(cfg, token_split=S)), ob)


@pytest.mark.parametrize("B,S", [(64, 2), (50, 4), (33, 2)])
def test_down_matrix_core_token_split_16_waves(B, S):
    """16 waves with token ranges, held to the oracle's down projection of the
    same intermediate; each range's rows equal, bit for bit, a run on that
    range's tokens alone."""
    from moe_decode_gate_amd import binding as wd
    spec = gen.LayerSpec(E=16, K=4, H=1536, I=320, seed=98)
    L = gen.make_layer(spec, threads=16)
    dl = DevLayer(L)
    t = gen.make_tokens(spec, B, routing="zipf")
    dt = DevTokens(t)
    act = wd.gate_up(dt.x, dt.ids, dl.wgu, dl.sgu)
    torch.cuda.synchronize()
    y64 = oracle.down(bits_of(act), t.ids, t.w, L.wd, L.sd, nthreads=16)
    ob = _down(act, dt.ids, dt.w, dl, dict(form=3, waves_per_block=16, token_split=S))
    assert_output_parity(ob, y64, f"down matrix cores B={B} W=16 S={S}", unit_scale=False)
    # each range's tokens alone give their rows bit for bit
    tpr = -(-B // S)
    for r0 in range(0, B, tpr):
        sl = slice(r0, min(B, r0 + tpr))
        part = _down(act[sl].contiguous(), dt.ids[sl].contiguous(), dt.w[sl].contiguous(), dl,
                     dict(form=3, waves_per_block=16))
        assert np.array_equal(part, ob[sl])


def test_down_matrix_core_form_bad_ids():
    """A token with an id outside [0, E) gets a NaN row; every other token's
    row is bit-identical to a run where that slot names a valid expert."""
    from moe_decode_gate_amd import binding as wd
    spec = gen.LayerSpec(E=16, K=4, H=1536, I=320, seed=97)
    dl = DevLayer(gen.make_layer(spec, threads=16))
    t = gen.make_tokens(spec, 24)
    dt = DevTokens(t)
    act = wd.gate_up(dt.x, dt.ids, dl.wgu, dl.sgu)
    ids = t.ids.copy()
    ids[3, 2] = 16
    ids[7, 0] = -5
    for W, S in ((8, 1), (16, 1), (8, 2), (16, 4)):
        cfg = dict(form=3, waves_per_block=W, token_split=S)
        ok = _down(act, dt.ids, dt.w, dl, cfg)
        bad = _down(act, torch.from_numpy(ids).cuda(), dt.w, dl, cfg)
        yb = (bad.astype(np.uint32) << 16).view(np.float32)
        assert np.isnan(yb[3]).all() and np.isnan(yb[7]).all()
        keep = np.ones(24, bool)
        keep[[3, 7]] = False
        assert np.array_equal(bad[keep], ok[keep])


def test_weight_load_modes_agree_bitwise(mid):
    """Cached and non-temporal weight loads read the same bytes."""
    dl, t = mid
    dt = DevTokens(t)
    runs = []
    for wl in (1, 2):
        runs.append(run_layer(dl, dt, cfg_gu=dict(weight_loads=wl, math=2, form=1, rows_per_wave=1),
                              cfg_dn=dict(weight_loads=wl, math=2, rows_per_wave=1)))
    (a1, o1), (a2, o2) = runs
    assert np.array_equal(bits_of(a1), bits_of(a2)) and np.array_equal(bits_of(o1), bits_of(o2))


def test_fused_entry_matches_two_calls(mid):
    from moe_decode_gate_amd import binding as wd
    dl, t = mid
    dt = DevTokens(t)
    _, o = run_layer(dl, dt)
    out = wd.moe_decode(dt.x, dt.ids, dt.w, dl.wgu, dl.sgu, dl.wd, dl.sd)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out), bits_of(o))


def test_side_stream(mid):
    from moe_decode_gate_amd import binding as wd
    dl, t = mid
    dt = DevTokens(t)
    _, o = run_layer(dl, dt)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = wd.moe_decode(dt.x, dt.ids, dt.w, dl.wgu, dl.sgu, dl.wd, dl.sd)
    s.synchronize()
    assert np.array_equal(bits_of(out), bits_of(o))


@pytest.mark.parametrize("B", [32, 64])
def test_graph_replays_match_eager(B):
    """The defaults (B=32: gate/up on the matrix cores, down with 8 rows per
    wave; B=64: both on the matrix cores) captured in a HIP graph: every replay,
    with eager work and synchronisation in between and the outputs cleared
    first, reproduces the eager result bit for bit."""
    from moe_decode_gate_amd import binding as wd
    spec = gen.LayerSpec(E=32, K=4, H=1536, I=320, seed=95)
    dl = DevLayer(gen.make_layer(spec, threads=16))
    t = gen.make_tokens(spec, B)
    dt = DevTokens(t)
    eager_act, eager_out = run_layer(dl, dt)
    act = torch.empty_like(eager_act)
    out = torch.empty_like(eager_out)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        wd.gate_up(dt.x, dt.ids, dl.wgu, dl.sgu, act=act, stream=s)
        wd.down(act, dt.ids, dt.w, dl.wd, dl.sd, out=out, stream=s)
    for i in range(3):
        act.fill_(0)
        out.fill_(0)
        run_layer(dl, dt)                                   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(act), bits_of(eager_act)), i
        assert np.array_equal(bits_of(out), bits_of(eager_out)), i


def test_out_of_range_id_poisons_only_its_token(mid):
    """An expert id outside [0, E) is never dereferenced: its intermediate row
    is NaN and its token's outputs are NaN; other tokens are unchanged."""
    dl, t = mid
    a0, o0 = run_layer(dl, DevTokens(t))
    ids = t.ids.copy()
    ids[2, 1] = dl.spec.E
    ids[5, 3] = -1
    a, o = run_layer(dl, DevTokens(gen.Tokens(x=t.x, ids=ids, w=t.w)))
    af, of = a.float().cpu().numpy(), o.float().cpu().numpy()
    assert np.isnan(af[2, 1]).all() and np.isnan(af[5, 3]).all()
    assert np.isnan(of[2]).all() and np.isnan(of[5]).all()
    keep = [b for b in range(ids.shape[0]) if b not in (2, 5)]
    assert np.array_equal(bits_of(o)[keep], bits_of(o0)[keep])


def test_empty_batch():
    from moe_decode_gate_amd import binding as wd
    spec = gen.LayerSpec(E=4, K=2, H=64, I=32, seed=1)
    dl = DevLayer(gen.make_layer(spec))
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    w = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    out = wd.moe_decode(x, ids, w, dl.wgu, dl.sgu, dl.wd, dl.sd)
    torch.cuda.synchronize()
    assert out.shape == (0, 64)
