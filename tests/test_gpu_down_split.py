"""The down kernel's expert split on the GPU (wd_launch.expert_split 2): two
workgroups per block of 16 outputs, one for the experts with even ids and one
for odd, all tokens each; the two hand their FP32 partial sums over through one
scratch cell per output (an atomic exchange), and whichever comes second adds
them (even class + odd class) and writes the output; every call leaves the
cells zero.

Held to the oracle's down projection of the GPU's own intermediate; a token's
result depends on its own slots only (token permutation exact, a run on a
subset of the tokens gives their rows bit for bit); reruns, graph replays and
the whole-layer entry points agree bit for bit; the cells return to zero."""
import numpy as np
import pytest
import torch

import oracle
from moe_decode_gate_amd import inputs as gen
from tests.gpu_common import DevLayer, DevTokens, assert_output_parity, bits_of, log, shifted, unit_shift

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _down(wd, act, ids, w, dl, cfg, sd=None):
    out = wd.down(act, ids, w, dl.wd, dl.sd if sd is None else sd, cfg=cfg)
    torch.cuda.synchronize()
    return bits_of(out)


def _cells_zero(scr):
    return not scr.cpu().numpy().any()


CASES = [
    ("zipf16", gen.LayerSpec(E=16, K=4, H=1536, I=320, seed=120), 3, "zipf", 16),
    ("zipf16", gen.LayerSpec(E=16, K=4, H=1536, I=320, seed=121), 40, "zipf", 8),
    ("zipf16", gen.LayerSpec(E=16, K=4, H=1536, I=320, seed=122), 64, "zipf", 16),
    ("qwen3", gen.LayerSpec(E=128, K=8, H=2048, I=768, seed=123), 32, "softmax", 16),
    ("qwen3", gen.LayerSpec(E=128, K=8, H=2048, I=768, seed=124), 2, "softmax", 16),
    ("odd_h", gen.LayerSpec(E=24, K=6, H=800, I=256, seed=125), 48, "zipf", 8),
]


@pytest.mark.parametrize("name,spec,B,routing,W", CASES, ids=[f"{c[0]}-B{c[2]}-W{c[4]}" for c in CASES])
def test_down_expert_split(name, spec, B, routing, W):
    from moe_decode_gate_amd import binding as wd
    L = gen.make_layer(spec, threads=16)
    dl = DevLayer(L)
    t = gen.make_tokens(spec, B, routing=routing)
    t.ids[0, 1] = t.ids[0, 0]                         # a repeated expert
    dt = DevTokens(t)
    act = wd.gate_up(dt.x, dt.ids, dl.wgu, dl.sgu)
    torch.cuda.synchronize()
    y64 = oracle.down(bits_of(act), t.ids, t.w, L.wd, L.sd, nthreads=16)
    k = unit_shift(y64)
    sd = shifted(dl.sd, k)
    scr = wd.down_scratch(B, spec.H)
    cfg = dict(form=3, waves_per_block=W, expert_split=2, down_scratch=scr)
    ob = _down(wd, act, dt.ids, dt.w, dl, cfg, sd)
    log(f"[expert split] {name} B={B} W={W}: experts used {np.unique(t.ids).size}, shift {k}")
    assert_output_parity(ob, y64 * 2.0 ** k, f"down expert split {name} B={B} W={W}",
                         unit_scale=0.5 <= np.abs(y64 * 2.0 ** k).max() < 1.0)
    assert _cells_zero(scr)
    for _ in range(2):                                # reruns on the same scratch: identical
        assert np.array_equal(_down(wd, act, dt.ids, dt.w, dl, cfg, sd), ob)
    assert _cells_zero(scr)
    # a token's result depends on its own slots only
    perm = np.random.default_rng(B).permutation(B)
    pt = torch.from_numpy(perm).cuda()
    assert np.array_equal(_down(wd, act[pt].contiguous(), dt.ids[pt].contiguous(), dt.w[pt].contiguous(), dl, cfg,
                                sd), ob[perm])
    if B > 2:
        sub = slice(1, B - 1)
        part = _down(wd, act[sub].contiguous(), dt.ids[sub].contiguous(), dt.w[sub].contiguous(), dl,
                     dict(cfg, down_scratch=wd.down_scratch(B - 2, spec.H)), sd)
        assert np.array_equal(part, ob[sub])


@pytest.mark.parametrize("B", [16, 32])
def test_whole_layer_entry_points_use_the_split(B):
    """wd_moe_decode with the layer workspace (the binding's default) and the
    no-allocation entry point run the expert split, bit-identical to gate/up
    followed by the split down; with a workspace of act alone wd_moe_decode
    runs the down kernel without the split (held to the oracle too).  B = 16 clears the
    split's cells from the token-form gate/up, B = 32 from the matrix-core one."""
    from moe_decode_gate_amd import binding as wd
    spec = gen.LayerSpec(E=128, K=8, H=2048, I=768, seed=126)
    L = gen.make_layer(spec, threads=16)
    dl = DevLayer(L)
    t = gen.make_tokens(spec, B)
    dt = DevTokens(t)
    act = wd.gate_up(dt.x, dt.ids, dl.wgu, dl.sgu)
    ref = _down(wd, act, dt.ids, dt.w, dl, dict(down_scratch=wd.down_scratch(B, spec.H)))
    full = wd.moe_decode(dt.x, dt.ids, dt.w, dl.wgu, dl.sgu, dl.wd, dl.sd)
    # a workspace of garbage: the call clears the cells itself
    ws = torch.randint(0, 255, (wd.layer_workspace_bytes(B, spec.K, spec.H, spec.I),), dtype=torch.uint8,
                       device="cuda")
    full2 = wd.moe_decode(dt.x, dt.ids, dt.w, dl.wgu, dl.sgu, dl.wd, dl.sd, workspace=ws)
    na = wd.moe_decode_noalloc(dt.x, dt.ids, dt.w, dl.wgu, dl.sgu, dl.wd, dl.sd)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(full), ref) and np.array_equal(bits_of(full2), ref)
    assert np.array_equal(bits_of(na), ref)
    small = torch.empty(wd.workspace_bytes(B, spec.K, spec.I), dtype=torch.uint8, device="cuda")
    ranges = wd.moe_decode(dt.x, dt.ids, dt.w, dl.wgu, dl.sgu, dl.wd, dl.sd, workspace=small)
    torch.cuda.synchronize()
    y64, _ = oracle.moe_decode(t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd, nthreads=16)
    for got, what in ((bits_of(ranges), "token ranges"), (ref, "expert split")):
        r = assert_output_parity(got, oracle.down(bits_of(act), t.ids, t.w, L.wd, L.sd, nthreads=16), what,
                                 unit_scale=False)
        assert r["cos"] >= 0.99999


def test_expert_split_graph_replays():
    """Captured in a HIP graph, the split down reproduces the eager result on
    every replay (the cells it leaves at zero are what the next replay
    needs), with eager work in between."""
    from moe_decode_gate_amd import binding as wd
    spec = gen.LayerSpec(E=64, K=8, H=2048, I=512, seed=127)
    dl = DevLayer(gen.make_layer(spec, threads=16))
    B = 24
    dt = DevTokens(gen.make_tokens(spec, B))
    act = wd.gate_up(dt.x, dt.ids, dl.wgu, dl.sgu)
    scr = wd.down_scratch(B, spec.H)
    cfg = dict(form=3, expert_split=2, down_scratch=scr)
    eager = _down(wd, act, dt.ids, dt.w, dl, cfg)
    out = torch.empty((B, spec.H), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(3):
            wd.down(act, dt.ids, dt.w, dl.wd, dl.sd, out=out, cfg=cfg, stream=s)
    for rep in range(3):
        out.fill_(float("nan"))
        _down(wd, act, dt.ids, dt.w, dl, cfg)         # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(out), eager), rep
        assert _cells_zero(scr)


def test_expert_split_bad_ids():
    """An id outside [0, E) belongs to neither class: its token's outputs are NaN
    and the other tokens keep their bits."""
    from moe_decode_gate_amd import binding as wd
    spec = gen.LayerSpec(E=16, K=4, H=1536, I=320, seed=128)
    dl = DevLayer(gen.make_layer(spec, threads=16))
    B = 12
    t = gen.make_tokens(spec, B)
    dt = DevTokens(t)
    act = wd.gate_up(dt.x, dt.ids, dl.wgu, dl.sgu)
    scr = wd.down_scratch(B, spec.H)
    cfg = dict(form=3, expert_split=2, down_scratch=scr)
    ok = _down(wd, act, dt.ids, dt.w, dl, cfg)
    ids = dt.ids.clone()
    ids[3, 2] = 16
    ids[7, 0] = -5
    bad = _down(wd, act, ids, dt.w, dl, cfg)
    f = (bad & 0x7FFF) > 0x7F80
    assert f[3].all() and f[7].all()
    keep = [b for b in range(B) if b not in (3, 7)]
    assert np.array_equal(bad[keep], ok[keep])
    assert _cells_zero(scr)


WIDE = [
    ("qwen3", gen.LayerSpec(E=128, K=8, H=2048, I=768, seed=130), 96, "softmax"),
    ("qwen3", gen.LayerSpec(E=128, K=8, H=2048, I=768, seed=131), 128, "softmax"),
    ("zipf16", gen.LayerSpec(E=16, K=4, H=1536, I=320, seed=132), 100, "zipf"),
    ("odd_h", gen.LayerSpec(E=24, K=6, H=800, I=256, seed=133), 80, "zipf"),
    ("qwen3", gen.LayerSpec(E=128, K=8, H=2048, I=768, seed=135), 256, "softmax"),
    ("zipf16", gen.LayerSpec(E=16, K=4, H=1536, I=320, seed=136), 300, "zipf"),
]


@pytest.mark.parametrize("name,spec,B,routing", WIDE, ids=[f"{c[0]}-B{c[2]}" for c in WIDE])
def test_down_wide_variant(name, spec, B, routing):
    """Past 64 tokens or 512 slots the matrix-core down runs its 8-wave variant
    with room for 128 tokens and 1,024 slots: with the expert split (scratch),
    with one token range and with two (no scratch); past 128 tokens or 1,024
    slots in token ranges of at most that size.  Each held to the oracle's down
    projection of the GPU's own intermediate; different range cuts agree bit
    for bit (a token's result depends on its own slots only), and a token
    permutation permutes the outputs exactly."""
    from moe_decode_gate_amd import binding as wd
    L = gen.make_layer(spec, threads=16)
    dl = DevLayer(L)
    t = gen.make_tokens(spec, B, routing=routing)
    t.ids[0, 1] = t.ids[0, 0]                         # a repeated expert
    dt = DevTokens(t)
    act = wd.gate_up(dt.x, dt.ids, dl.wgu, dl.sgu)
    torch.cuda.synchronize()
    y64 = oracle.down(bits_of(act), t.ids, t.w, L.wd, L.sd, nthreads=16)
    k = unit_shift(y64)
    sd = shifted(dl.sd, k)
    scr = wd.down_scratch(B, spec.H)
    unit = 0.5 <= np.abs(y64 * 2.0 ** k).max() < 1.0
    log(f"[wide down] {name} B={B}: slots {B * spec.K}, max slots per expert {np.bincount(t.ids.ravel()).max()}")
    split = _down(wd, act, dt.ids, dt.w, dl, dict(form=3, down_scratch=scr), sd)   # the default
    if B <= 128:
        one = _down(wd, act, dt.ids, dt.w, dl, dict(form=3, token_split=1), sd)
        two = _down(wd, act, dt.ids, dt.w, dl, dict(form=3, token_split=2, waves_per_block=8), sd)
        runs = ((split, "expert split"), (one, "one range"), (two, "two ranges"))
    else:                                             # past 128 tokens: two (or four) ranges
        one = _down(wd, act, dt.ids, dt.w, dl, dict(form=3, token_split=4), sd)
        two = _down(wd, act, dt.ids, dt.w, dl, dict(form=3, token_split=4, waves_per_block=8), sd)
        runs = ((split, "default ranges"), (one, "four ranges"), (two, "four ranges, 8 waves"))
        assert np.array_equal(split, one)             # a token's result: its own slots only
    for got, what in runs:
        assert_output_parity(got, y64 * 2.0 ** k, f"wide down {name} B={B} {what}", unit_scale=unit)
    assert np.array_equal(one, two)
    assert _cells_zero(scr)
    perm = np.random.default_rng(B).permutation(B)
    pt = torch.from_numpy(perm).cuda()
    assert np.array_equal(_down(wd, act[pt].contiguous(), dt.ids[pt].contiguous(), dt.w[pt].contiguous(), dl,
                                dict(form=3, down_scratch=scr), sd), split[perm])
    # the layer entry point picks this variant by default
    full = wd.moe_decode(dt.x, dt.ids, dt.w, dl.wgu, dl.sgu, dl.wd, sd)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(full), split)


def test_down_wide_variant_bad_ids():
    """A bad id at B = 96: that token's outputs are NaN (tokens past 64 included),
    the others keep their bits."""
    from moe_decode_gate_amd import binding as wd
    spec = gen.LayerSpec(E=16, K=4, H=1536, I=320, seed=134)
    dl = DevLayer(gen.make_layer(spec, threads=16))
    B = 96
    t = gen.make_tokens(spec, B)
    dt = DevTokens(t)
    act = wd.gate_up(dt.x, dt.ids, dl.wgu, dl.sgu)
    cfg = dict(form=3, down_scratch=wd.down_scratch(B, spec.H))
    ok = _down(wd, act, dt.ids, dt.w, dl, cfg)
    ids = dt.ids.clone()
    ids[5, 1] = 16
    ids[90, 3] = -2
    bad = _down(wd, act, ids, dt.w, dl, cfg)
    f = (bad & 0x7FFF) > 0x7F80
    assert f[5].all() and f[90].all()
    keep = [b for b in range(B) if b not in (5, 90)]
    assert np.array_equal(bad[keep], ok[keep])
