"""GPU router (top-k gating) against the oracle: expert ids bit-exact (the
choice is made on the exact input logits), weights within FP32 rounding of the
FP64 softmax; and the routed layer end to end."""
import numpy as np
import pytest
import torch

import oracle
from moe_decode_gate_amd import inputs as gen
from tests.gpu_common import DevLayer, act_flip_propagation, assert_output_parity, bits_of, log, shifted, unit_shift

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


@pytest.mark.parametrize("B,E,K", [(1, 128, 8), (33, 128, 8), (64, 256, 8), (5, 1000, 64), (3, 8, 1),
                                   (7, 100, 7), (2, 64, 64), (9, 1024, 2)])
def test_route_matches_oracle(B, E, K):
    from moe_decode_gate_amd import binding as wd
    log(f"[case] route B={B} E={E} K={K}")
    logits = np.random.default_rng(B * 1000 + E + K).standard_normal((B, E)).astype(np.float32)
    ids, w = wd.route(torch.from_numpy(logits).cuda(), K)
    torch.cuda.synchronize()
    ids_o, w_o = oracle.route(logits, K)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    np.testing.assert_allclose(w.cpu().numpy().astype(np.float64), w_o, rtol=2e-6, atol=1e-9)


def test_route_ties_take_lower_index():
    from moe_decode_gate_amd import binding as wd
    logits = np.zeros((4, 200), np.float32)
    logits[0, [150, 3, 77, 64, 128]] = 1.0
    logits[1, :] = -2.0
    logits[2, ::3] = 0.5
    logits[3, [199, 63, 64, 127, 128, 191, 192, 0]] = 3.0
    ids, w = wd.route(torch.from_numpy(logits).cuda(), 8)
    torch.cuda.synchronize()
    ids_o, w_o = oracle.route(logits, 8)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    assert ids_o[0, :5].tolist() == [3, 64, 77, 128, 150]
    np.testing.assert_allclose(w.cpu().numpy(), w_o, rtol=2e-6)


def test_routed_layer_end_to_end():
    """logits -> wd_route -> wd_moe_decode against oracle.route -> oracle.moe_decode."""
    from moe_decode_gate_amd import binding as wd
    spec = gen.CONFIGS["qwen3_b32"]["spec"]
    B = 32
    logits = gen.make_logits(spec, B, step=5)
    ids_o, w_o = oracle.route(logits, spec.K)
    L = gen.make_layer(spec, experts=ids_o.ravel(), threads=16)
    dl = DevLayer(L)
    t = gen.make_tokens(spec, B, step=5)
    y64, act_o = oracle.moe_decode(t.x, ids_o, w_o.astype(np.float32), L.wgu, L.sgu, L.wd, L.sd, nthreads=16)
    k = unit_shift(y64)
    x = torch.from_numpy(t.x.view(np.int16)).cuda().view(torch.bfloat16)
    ids, w = wd.route(torch.from_numpy(logits).cuda(), spec.K)
    out = wd.moe_decode(x, ids, w, dl.wgu, dl.sgu, dl.wd, shifted(dl.sd, k))
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    act = wd.gate_up(x, ids, dl.wgu, dl.sgu)            # the intermediate wd_moe_decode formed
    torch.cuda.synchronize()
    prop = act_flip_propagation(bits_of(act), act_o, ids_o, w_o, L.wd, L.sd)
    assert_output_parity(bits_of(out), y64 * 2.0 ** k, "routed qwen3 B=32", extra=prop * 2.0 ** k)
