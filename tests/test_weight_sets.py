"""Weight sets on disk: .npy codes and E8M0 bytes plus a JSON manifest (shape,
seed, quantizer rule, per-file SHA-256), so runs are reproducible from the files
or from the manifest alone."""
import json
import os

import numpy as np
import pytest

from moe_decode_gate_amd import inputs as gen


def _layer():
    spec = gen.CONFIGS["tiny"]["spec"]
    return gen.make_layer(spec, experts=(0, 2, 5), threads=2)


def test_round_trip_is_bit_exact(tmp_path):
    L = _layer()
    man = gen.save_layer(L, str(tmp_path))
    R = gen.load_layer(str(tmp_path))
    assert R.spec == L.spec and R.experts == L.experts
    for name in ("wgu", "sgu", "wd", "sd"):
        assert np.array_equal(getattr(R, name), getattr(L, name)), name
    assert man["format"] == gen.MANIFEST_FORMAT


def test_manifest_states_shape_seed_and_rule(tmp_path):
    L = _layer()
    gen.save_layer(L, str(tmp_path), std=0.02)
    man = json.load(open(os.path.join(str(tmp_path), "manifest.json")))
    sp = L.spec
    assert man["spec"] == {"E": sp.E, "K": sp.K, "H": sp.H, "I": sp.I, "seed": sp.seed}
    assert man["experts"] == [0, 2, 5] and man["std"] == 0.02
    assert "floor(log2" in man["quantizer"]["shared_exponent"] and man["quantizer"]["block"] == 32
    assert man["arrays"]["wgu"]["shape"] == [sp.E, 2 * sp.I, sp.H]
    assert man["arrays"]["sd"]["shape"] == [sp.E, sp.H, sp.I // 32]


def test_manifest_alone_regenerates_the_weights(tmp_path):
    L = _layer()
    gen.save_layer(L, str(tmp_path))
    man = json.load(open(os.path.join(str(tmp_path), "manifest.json")))
    again = gen.make_layer(gen.LayerSpec(**man["spec"]), experts=man["experts"], std=man["std"], threads=2)
    R = gen.load_layer(str(tmp_path))
    for name in ("wgu", "sgu", "wd", "sd"):
        assert np.array_equal(getattr(again, name), getattr(R, name)), name


def test_a_changed_byte_is_refused(tmp_path):
    gen.save_layer(_layer(), str(tmp_path))
    fn = os.path.join(str(tmp_path), "wd.npy")
    raw = bytearray(open(fn, "rb").read())
    raw[-1] ^= 0x01
    open(fn, "wb").write(bytes(raw))
    with pytest.raises(ValueError, match="SHA-256"):
        gen.load_layer(str(tmp_path))
    R = gen.load_layer(str(tmp_path), verify=False)      # the check can be skipped, the shape still holds
    assert R.wd.shape == _layer().wd.shape


def test_wrong_shape_or_format_is_refused(tmp_path):
    L = _layer()
    gen.save_layer(L, str(tmp_path))
    np.save(os.path.join(str(tmp_path), "sd.npy"), L.sd[:, :, :1].copy(), allow_pickle=False)
    with pytest.raises(ValueError, match="needs uint8"):
        gen.load_layer(str(tmp_path), verify=False)
    mp = os.path.join(str(tmp_path), "manifest.json")
    man = json.load(open(mp))
    man["format"] = "something else"
    json.dump(man, open(mp, "w"))
    with pytest.raises(ValueError, match="format"):
        gen.load_layer(str(tmp_path))
