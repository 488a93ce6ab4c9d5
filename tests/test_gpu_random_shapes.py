"""GPU parity on seeded random layer shapes and launch configurations.

Each case draws E, top-k, H, I (multiples of 32, K * I <= 16384), a batch size
and a routing law, runs gate/up and down through the C ABI under a drawn
configuration (library defaults, the matrix-core gate/up, the matrix-core down
with 8 or 16 waves and 1, 2 or 4 token ranges) and holds the result to the
oracle: the intermediate to its BF16 bits up to rare one-ulp flips, and the
output to the oracle's down projection of the GPU's own intermediate (half a
BF16 ulp plus FP32 summation, at unit output scale by an exact E8M0 shift).
The matrix-core down is also run on the token form's intermediate and must
give, bit for bit, the output of a run without token ranges.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_decode_gate_amd import inputs as gen
from tests.gpu_common import (DevLayer, DevTokens, act_flip_stats, assert_act_flips, assert_output_parity, bits_of, log, run_layer,
                              shifted, unit_shift)

pytestmark = pytest.mark.gpu

DOWN_CFGS = [None, dict(form=3, waves_per_block=8, token_split=1), dict(form=3, waves_per_block=8, token_split=2),
             dict(form=3, waves_per_block=16, token_split=1), dict(form=3, waves_per_block=16, token_split=2),
             dict(form=3, waves_per_block=16, token_split=4), dict(form=3, waves_per_block=8, token_split=4)]


def _cases(n=14, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = int(rng.integers(1, 161))
        K = int(rng.integers(1, min(E, 8) + 1))
        H = 32 * int(rng.integers(1, 65))
        I = 32 * int(rng.integers(1, 49))
        if K * I > 16384:
            continue
        B = int(rng.integers(1, 65))
        if B * K > 512 or B * K * H * I > 2 ** 28:     # the oracle finishes each case in seconds
            continue
        routing = "zipf" if rng.random() < 0.4 else "softmax"
        gu = dict(form=3) if rng.random() < 0.5 else None
        dn = DOWN_CFGS[int(rng.integers(0, len(DOWN_CFGS)))]
        out.append((len(out), E, K, H, I, B, routing, gu, dn, int(rng.integers(1, 2 ** 31))))
    return out


CASES = _cases()


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_decode_gate_amd import binding  # noqa: F401  (fails loudly if the library is missing)
    torch.cuda.set_device(0)


@pytest.mark.parametrize("case", CASES, ids=[f"c{c[0]}" for c in CASES])
def test_random_shape_parity(case):
    from moe_decode_gate_amd import binding as wd
    n, E, K, H, I, B, routing, cfg_gu, cfg_dn, seed = case
    log(f"[case] c{n}: E={E} K={K} H={H} I={I} B={B} routing={routing} gate/up={cfg_gu} down={cfg_dn}")
    spec = gen.LayerSpec(E=E, K=K, H=H, I=I, seed=seed)
    t = gen.make_tokens(spec, B, routing=routing)
    L = gen.make_layer(spec, experts=t.ids.ravel(), threads=16)
    dl, dt = DevLayer(L), DevTokens(t)
    y64, act_o = oracle.moe_decode(t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd, nthreads=16)
    k = unit_shift(y64)
    sd_k = shifted(dl.sd, k)

    act, out = run_layer(dl, dt, sd=sd_k, cfg_gu=cfg_gu, cfg_dn=cfg_dn)
    frac, ulps, within = act_flip_stats(bits_of(act), act_o)
    log(f"[act] c{n}: flip fraction {frac:.2e}, max {ulps:.2f} ulp, within bound: {within}")
    assert_act_flips(frac, act_o.size, within, f"c{n}")
    y_of_gpu_act = oracle.down(bits_of(act), t.ids, t.w, L.wd, L.sd, nthreads=16)
    assert_output_parity(bits_of(out), y_of_gpu_act * 2.0 ** k, f"c{n} layer vs oracle(act_gpu)")

    # the matrix-core down: token ranges change nothing, bit for bit
    if B * K <= 512:
        base = wd.down(act, dt.ids, dt.w, dl.wd, sd_k, cfg=dict(form=3, waves_per_block=8, token_split=1))
        for S in (2, 4):
            got = wd.down(act, dt.ids, dt.w, dl.wd, sd_k, cfg=dict(form=3, waves_per_block=8, token_split=S))
            torch.cuda.synchronize()
            assert np.array_equal(bits_of(got), bits_of(base)), (n, S)


GU_CFGS = [None, dict(form=1, math=1), dict(form=1, math=2, lanes_per_row=64, rows_per_wave=1),
           dict(form=1, math=2, lanes_per_row=32, rows_per_wave=4), dict(form=1, math=2, lanes_per_row=16, rows_per_wave=2),
           dict(form=1, math=2, weight_loads=2), dict(form=2), dict(form=3)]
DN_CFGS = [None, dict(math=1, rows_per_wave=1), dict(math=2, rows_per_wave=2), dict(math=1, rows_per_wave=4),
           dict(math=2, rows_per_wave=8), dict(math=1, rows_per_wave=8), dict(math=2, rows_per_wave=1, weight_loads=2),
           dict(form=3, waves_per_block=16, token_split=2), dict(form=3, waves_per_block=8, token_split=1)]


def _cases_wide(n=12, seed=20261203, bmax=64):
    """Wider ranges: up to 1024 experts, top-16, H up to 8192, I up to 4096, and
    tokens that name one expert twice."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = int(rng.choice([1, 3, 17, 64, 200, 513, 1024]))
        K = int(rng.integers(1, min(E, 16) + 1))
        H = 32 * int(rng.integers(1, 257))
        I = 32 * int(rng.integers(1, 129))
        B = int(rng.integers(1, bmax + 1))
        if K * I > 16384 or B * K * H * I > 2 ** 28 or E * 3 * H * I > 3 * 2 ** 29:
            continue
        dup = K >= 2 and rng.random() < 0.5
        gu = GU_CFGS[int(rng.integers(0, len(GU_CFGS)))]
        dn = DN_CFGS[int(rng.integers(0, len(DN_CFGS)))]
        out.append((len(out), E, K, H, I, B, dup, gu, dn, int(rng.integers(1, 2 ** 31))))
    return out


WIDE = _cases_wide()
# batches past the matrix-core down's 64 tokens (token form only)
WIDE += [(len(WIDE) + c[0],) + c[1:] for c in _cases_wide(n=6, seed=20261204, bmax=300) if c[5] > 64]


@pytest.mark.parametrize("case", WIDE, ids=[f"w{c[0]}" for c in WIDE])
def test_random_wide_parity(case):
    """Every launch family on the wider shapes; a drawn configuration that the
    library does not build for the shape (status WD_ERR_UNSUPPORTED, checked on
    the host) runs under the defaults instead."""
    from moe_decode_gate_amd import binding as wd
    n, E, K, H, I, B, dup, cfg_gu, cfg_dn, seed = case
    log(f"[case] w{n}: E={E} K={K} H={H} I={I} B={B} dup={dup} gate/up={cfg_gu} down={cfg_dn}")
    spec = gen.LayerSpec(E=E, K=K, H=H, I=I, seed=seed)
    t = gen.make_tokens(spec, B, routing="softmax")
    if dup:
        t.ids[::2, 1] = t.ids[::2, 0]                   # every other token names its first expert twice
    L = gen.make_layer(spec, experts=t.ids.ravel(), threads=16)
    dl, dt = DevLayer(L), DevTokens(t)
    y64, act_o = oracle.moe_decode(t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd, nthreads=16)
    k = unit_shift(y64)
    sd_k = shifted(dl.sd, k)

    def run(cfg, fn, what):
        try:
            return fn(cfg)
        except wd.WDError as err:
            if err.status != -7:
                raise
            log(f"[case] w{n}: {what} {cfg} not built for this shape; defaults instead")
            return fn(None)

    act = run(cfg_gu, lambda c: wd.gate_up(dt.x, dt.ids, dl.wgu, dl.sgu, cfg=c), "gate/up")
    out = run(cfg_dn, lambda c: wd.down(act, dt.ids, dt.w, dl.wd, sd_k, cfg=c), "down")
    torch.cuda.synchronize()
    frac, ulps, within = act_flip_stats(bits_of(act), act_o)
    log(f"[act] w{n}: flip fraction {frac:.2e}, max {ulps:.2f} ulp, within bound: {within}")
    assert_act_flips(frac, act_o.size, within, f"w{n}")
    y_of_gpu_act = oracle.down(bits_of(act), t.ids, t.w, L.wd, L.sd, nthreads=16)
    assert_output_parity(bits_of(out), y_of_gpu_act * 2.0 ** k, f"w{n} layer vs oracle(act_gpu)")


@pytest.mark.parametrize("case", CASES[:8], ids=[f"c{c[0]}" for c in CASES[:8]])
def test_random_fused_entry_and_graph(case):
    """wd_moe_decode (both kernels, library defaults, one workspace) gives the
    two separate calls' output bit for bit, eagerly and replayed three times
    from a HIP graph with eager work in between."""
    from moe_decode_gate_amd import binding as wd
    n, E, K, H, I, B, routing, _, _, seed = case
    log(f"[case] fused c{n}: E={E} K={K} H={H} I={I} B={B} routing={routing}")
    spec = gen.LayerSpec(E=E, K=K, H=H, I=I, seed=seed)
    t = gen.make_tokens(spec, B, routing=routing)
    L = gen.make_layer(spec, experts=t.ids.ravel(), threads=16)
    dl, dt = DevLayer(L), DevTokens(t)
    _, ref = run_layer(dl, dt)
    ref = bits_of(ref)
    ws = torch.empty(max(wd.workspace_bytes(B, K, I), 16), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
    wd.moe_decode(dt.x, dt.ids, dt.w, dl.wgu, dl.sgu, dl.wd, dl.sd, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out), ref)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            wd.moe_decode(dt.x, dt.ids, dt.w, dl.wgu, dl.sgu, dl.wd, dl.sd, out=out, workspace=ws)
    torch.cuda.synchronize()
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(out), ref)
