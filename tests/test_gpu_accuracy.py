"""Accuracy experiment: the GPU layer's output and the conventional path's
numerics (activations rounded through MXFP8, per-expert outputs in BF16)
against the FP64 layer with unrounded activations.  The GPU's error must be
the oracle's own warp-decode error (the same roundings) and smaller than the
conventional path's."""
import numpy as np
import pytest
import torch

import oracle
from moe_decode_gate_amd import inputs as gen
from moe_decode_gate_amd import binding as wd
from tests.gpu_common import DevLayer, DevTokens, bf16_bits_to_f64, bits_of, log, run_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


@pytest.mark.parametrize("name,B,routing", [("qwen3_b32", 32, "softmax"), ("large", 8, "zipf")])
def test_accuracy_vs_unrounded_reference(name, B, routing):
    spec = gen.CONFIGS[name]["spec"]
    t = gen.make_tokens(spec, B, routing=routing)
    L = gen.make_layer(spec, experts=t.ids.ravel(), threads=16)
    dl = DevLayer(L)
    _, out = run_layer(dl, DevTokens(t))
    args = (t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd)
    gt = oracle.moe_decode_exact(*args, nthreads=16)
    y_wd, _ = oracle.moe_decode(*args, nthreads=16)
    y_wd_bf16 = bf16_bits_to_f64(np.array([oracle.bf16_rne(float(v)) for v in y_wd.ravel()],
                                          np.uint16)).reshape(y_wd.shape)
    cv = oracle.moe_decode_conventional(*args, nthreads=16)
    got = bf16_bits_to_f64(bits_of(out))
    dt = DevTokens(t)
    ec = bf16_bits_to_f64(bits_of(wd.ec_moe_decode(dt.x, dt.ids, dt.w, dl.wgu, dl.sgu, dl.wd, dl.sd)))
    n = float(np.linalg.norm(gt))
    e_gpu, e_wd, e_cv, e_ec = (float(np.linalg.norm(a - gt)) / n for a in (got, y_wd_bf16, cv, ec))
    log(f"[accuracy] {name} B={B}: rel L2 error gpu {e_gpu:.3e}, oracle warp-decode {e_wd:.3e}, "
        f"conventional {e_cv:.3e} (GPU expert-centric path {e_ec:.3e}), conventional / gpu = {e_cv / e_gpu:.2f}")
    assert abs(e_gpu - e_wd) <= 0.05 * e_wd          # same roundings, FP32 vs FP64 sums
    assert e_cv > e_gpu
    # the GPU expert-centric path has the conventional roundings plus its matrix instruction's
    # truncated sums (relative error ~2^-14, far below the MXFP8 activation rounding)
    assert abs(e_ec - e_cv) <= 0.05 * e_cv
