"""How far a NaN weight reaches (GPU, through the C ABI).

One E4M3 NaN code (0x7F) is planted in one expert's weights.  The outputs that
use that weight must become NaN -- exactly the ones the oracle makes NaN on the
same codes -- and every other output must keep the bits of the run without
the NaN.  A NaN in a down-projection row h of expert e reaches out[b, h] of
each token b routed to e (NaN times anything, zero included, is NaN); a NaN
in a gate or up row j of e makes act[b, k, j] NaN for those tokens and, through
the down projection, their whole output row.  Checked under the token forms
(small batch) and the matrix-core forms (from B = 18), whose tiles share a weight
row across several tokens and must still keep the NaN to the columns of the
tokens that use it."""
import numpy as np
import pytest
import torch

import oracle
from moe_decode_gate_amd import inputs as gen
from tests.gpu_common import DevLayer, DevTokens, bits_of, log, run_layer

pytestmark = pytest.mark.gpu

NAN_CODE = 0x7F


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


@pytest.fixture(scope="module")
def layer():
    spec = gen.LayerSpec(E=32, K=4, H=512, I=256, seed=20260077)
    return gen.make_layer(spec, threads=16)


def _planted(L, where, e):
    """A copy of the layer with one NaN code: in a down row ('down'), a gate
    row ('gate') or an up row ('up') of expert e."""
    wgu, wd = L.wgu.copy(), L.wd.copy()
    I = L.spec.I
    if where == "down":
        wd[e, 37, 101] = NAN_CODE
    elif where == "gate":
        wgu[e, 19, 300] = NAN_CODE
    else:
        wgu[e, I + 200, 5] = NAN_CODE
    return gen.Layer(L.spec, wgu, L.sgu, wd, L.sd, L.experts)


@pytest.mark.parametrize("B", [4, 32, 40])
@pytest.mark.parametrize("where", ["down", "gate", "up"])
def test_nan_weight_poisons_exactly_its_users(layer, where, B):
    spec = layer.spec
    t = gen.make_tokens(spec, B, step=B)
    e = int(np.bincount(t.ids.ravel(), minlength=spec.E).argmax())      # the most used expert
    users = np.array([e in row for row in t.ids])
    assert 0 < users.sum() < B
    t.w[np.argmax(users), list(t.ids[np.argmax(users)]).index(e)] = 0.0  # a zero weight does not hide NaN
    dt = DevTokens(t)
    _, clean = run_layer(DevLayer(layer), dt)
    P = _planted(layer, where, e)
    act, out = run_layer(DevLayer(P), dt)
    got, ref = bits_of(out), bits_of(clean)
    nan_gpu = (got & 0x7FFF) > 0x7F80
    y64, act_o = oracle.moe_decode(t.x, t.ids, t.w, P.wgu, P.sgu, P.wd, P.sd, nthreads=16)
    nan_ora = np.isnan(y64)
    log(f"[nan] {where} B={B} expert {e}: {int(users.sum())} users, {int(nan_gpu.sum())} NaN outputs "
        f"(oracle {int(nan_ora.sum())})")
    assert np.array_equal(nan_gpu, nan_ora)
    if where == "down":
        expect = np.stack([np.flatnonzero(users), np.full(int(users.sum()), 37)], 1)
        assert np.array_equal(np.argwhere(nan_ora), expect)
    else:
        assert np.array_equal(nan_ora.all(axis=1), users) and not nan_ora[~users].any()
        a = bits_of(act)
        assert np.array_equal((a & 0x7FFF) > 0x7F80, (act_o & 0x7FFF) > 0x7F80)
    assert np.array_equal(got[~nan_gpu], ref[~nan_gpu])
