"""C-ABI checks that need no GPU: the library loads, exports every function
include/wd.h declares, and rejects bad arguments on the host before any
device call."""
import ctypes as C

import pytest
import torch

from moe_decode_gate_amd import binding as wd

A = 0x10000          # a 16-byte-aligned stand-in address; never dereferenced here
lib = wd.raw

# Calls that pass every host check return WD_ERR_DEVICE (-5) here, where there is
# no GPU; on a machine with one they would launch on the stand-in addresses.
pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="host-side argument checks with stand-in addresses need a machine without a GPU")


def test_every_declared_symbol_is_exported():
    names = wd.header_functions()
    assert {"wd_gate_up", "wd_down", "wd_moe_decode", "wd_workspace_bytes", "wd_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(-8, 1):
        assert lib.wd_status_string(s)
    assert lib.wd_status_string(123) == b"unknown status"


def test_workspace_bytes():
    assert lib.wd_workspace_bytes(32, 8, 768) == 32 * 8 * 768 * 2
    assert lib.wd_workspace_bytes(0, 8, 768) == 0
    assert lib.wd_workspace_bytes(1, 0, 768) == 0
    assert lib.wd_workspace_bytes(1, 8, 100) == 0


def gu(x=A, ids=A, w=A, s=A, act=A, B=1, K=8, E=128, H=2048, I=768):
    return lib.wd_gate_up(x, ids, w, s, act, B, K, E, H, I, None)


def dn(act=A, ids=A, tw=A, w=A, s=A, out=A, B=1, K=8, E=128, H=2048, I=768):
    return lib.wd_down(act, ids, tw, w, s, out, B, K, E, H, I, None)


def md(ws_bytes=1 << 20, ws=A, **kw):
    d = dict(x=A, ids=A, tw=A, wgu=A, sgu=A, wd=A, sd=A, out=A, B=1, K=8, E=128, H=2048, I=768)
    d.update(kw)
    return lib.wd_moe_decode(d["x"], d["ids"], d["tw"], d["wgu"], d["sgu"], d["wd"], d["sd"], ws, ws_bytes,
                             d["out"], d["B"], d["K"], d["E"], d["H"], d["I"], None)


@pytest.mark.parametrize("kw", [dict(H=100), dict(I=48), dict(K=0), dict(E=0), dict(B=-1), dict(H=0), dict(I=16)])
def test_bad_dims(kw):
    assert gu(**kw) == -2
    assert dn(**kw) == -2
    assert md(**kw) == -2


@pytest.mark.parametrize("kw", [dict(H=8192 + 32), dict(K=32, I=1024)])
def test_unsupported_sizes(kw):
    assert gu(**kw) == -7 or dn(**kw) == -7


def test_null_pointers():
    assert gu(x=None) == -1 and gu(w=None) == -1 and gu(act=None) == -1
    assert dn(tw=None) == -1 and dn(out=None) == -1 and dn(s=None) == -1
    assert md(ws=None) == -1 and md(wd=None) == -1


def test_misaligned():
    assert gu(x=A + 8) == -3 and gu(w=A + 4) == -3 and gu(ids=A + 2) == -3
    assert dn(act=A + 8) == -3 and dn(out=A + 1) == -3 and dn(tw=A + 2) == -3
    assert md(ws=A + 8) == -3


def test_workspace_too_small():
    assert md(ws_bytes=1 * 8 * 768 * 2 - 1) == -4


def test_empty_batch_launches_nothing():
    # B = 0 is valid and returns before any device query, with NULL activations
    assert gu(x=None, ids=None, act=None, B=0) == 0
    assert dn(act=None, ids=None, tw=None, out=None, B=0) == 0
    assert md(ws=None, ws_bytes=0, x=None, ids=None, tw=None, out=None, B=0) == 0


def test_bad_launch_config_rejected():
    for cfg in (wd.Launch(3, 0, 0, 0), wd.Launch(0, 5, 0, 0), wd.Launch(0, 0, 3, 0), wd.Launch(0, 0, 0, 7),
                wd.Launch(0, 0, 0, -1), wd.Launch(0, 0, 0, 0, None, None, 3), wd.Launch(lanes_per_row=8)):
        assert lib.wd_gate_up_ex(A, A, A, A, A, 1, 8, 128, 2048, 768, C.byref(cfg), None) == -7
        assert lib.wd_down_ex(A, A, A, A, A, A, 1, 8, 128, 2048, 768, C.byref(cfg), None) == -7


def test_lanes_per_row_limits():
    # grouped rows apply to the gate/up kernel only, and need the row's chunks to fit the lanes
    assert lib.wd_down_ex(A, A, A, A, A, A, 1, 8, 128, 2048, 768, C.byref(wd.Launch(lanes_per_row=16)), None) == -7
    assert lib.wd_gate_up_ex(A, A, A, A, A, 1, 8, 128, 8192, 768, C.byref(wd.Launch(lanes_per_row=16)), None) == -7


def test_defaults_cover_every_supported_shape():
    """With no launch configuration, every size the library accepts gets a
    compiled kernel variant: the call passes all host checks (and reaches the
    device check, -5 here) instead of returning WD_ERR_UNSUPPORTED."""
    n = 0
    for H in (32, 96, 288, 2048, 4096, 4128, 6304, 8192):
        for I in (32, 96, 768, 896, 1536, 4096, 8192):
            for K in (1, 2, 3, 8, 16):
                if K * I > 16384:
                    continue
                for E in (1, 16, 128, 1024, 2000):
                    if K > E:
                        continue
                    for B in (1, 2, 3, 4, 5, 7, 8, 16, 23, 24, 31, 32, 48, 56, 64, 65, 200):
                        rg = lib.wd_gate_up_ex(A, A, A, A, A, B, K, E, H, I, None, None)
                        rd = lib.wd_down_ex(A, A, A, A, A, A, B, K, E, H, I, None, None)
                        assert (rg, rd) == (-5, -5), (B, K, E, H, I, rg, rd)
                        n += 1
    assert n > 1000


def test_helpers_reject_bad_arguments():
    assert lib.wd_dequant_probe(None, None) == -1
    assert lib.wd_dequant_probe(A + 4, None) == -3
    assert lib.wd_stream_read(A, 15, A, 0, 4, None, None, None) == -3
    assert lib.wd_stream_read(A, 16, A, lib.wd_stream_blocks() + 1, 4, None, None, None) == -7
    assert lib.wd_stream_read(A, 16, A, 0, 3, None, None, None) == -7
    assert lib.wd_stream_copy(None, A, 16, 0, None) == -1
    assert lib.wd_gpu_sleep(-1, None) == -7


def test_route_rejects_bad_arguments():
    assert lib.wd_route(A, 1, 128, 0, A, A, None) == -2
    assert lib.wd_route(A, 1, 8, 9, A, A, None) == -2
    assert lib.wd_route(A, -1, 8, 2, A, A, None) == -2
    assert lib.wd_route(A, 1, 2048, 8, A, A, None) == -7
    assert lib.wd_route(A, 1, 128, 65, A, A, None) == -7
    assert lib.wd_route(None, 1, 128, 8, A, A, None) == -1
    assert lib.wd_route(A + 2, 1, 128, 8, A, A, None) == -3
    assert lib.wd_route(None, 0, 128, 8, None, None, None) == 0


def test_chunk_to_slot_division_is_exact():
    # The down kernel maps chunk c to slot c // (I/16) by (c * magic) >> 22 with
    # magic = 2^22 // nci + 1; exact for every chunk of every supported size.
    for nci in range(2, 1025, 2):                  # I = 16 * nci, I a multiple of 32
        magic = (1 << 22) // nci + 1
        K_max = 16384 // (16 * nci)
        for c in range(min(1024, K_max * nci)):
            assert (c * magic) >> 22 == c // nci


# ---- expert-centric path (include/ec.h) -----------------------------------

def ec(ws_bytes=1 << 30, ws=A, cfg=None, **kw):
    d = dict(x=A, ids=A, tw=A, wgu=A, sgu=A, wd=A, sd=A, out=A, B=1, K=8, E=128, H=2048, I=768)
    d.update(kw)
    args = (d["x"], d["ids"], d["tw"], d["wgu"], d["sgu"], d["wd"], d["sd"], ws, ws_bytes, d["out"],
            d["B"], d["K"], d["E"], d["H"], d["I"])
    if cfg is None:
        return lib.ec_moe_decode(*args, None)
    return lib.ec_moe_decode_ex(*args, C.byref(cfg), None)


def test_ec_workspace_layout():
    for B, K, E, H, I in [(1, 8, 128, 2048, 768), (32, 8, 128, 2048, 768), (64, 8, 128, 4096, 1536),
                          (7, 4, 16, 160, 96), (512, 8, 128, 2048, 768)]:
        lay = wd.ec_workspace_layout(B, K, E, H, I)
        offs = [lay[n] for n in wd.EC_WS]
        assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
        assert lay["total"] == lib.ec_workspace_bytes(B, K, E, H, I)
        pairs = B * K
        tiles = (pairs + 15 * min(E, pairs)) // 16
        rows = 16 * tiles
        assert lay["row_pair"] - lay["tile_expert"] >= 4 * tiles
        assert lay["xs"] - lay["xq"] >= rows * H
        assert lay["aq"] - lay["act"] >= 2 * rows * I
        assert lay["out_pair"] - lay["aq"] >= rows * I + rows * I // 32
        assert lay["total"] - lay["out_pair"] >= 2 * pairs * H


def test_ec_tile_bound_is_tight_enough():
    # sum over experts of ceil(count/16) never exceeds the bound, whatever the routing
    import numpy as np
    rng = np.random.default_rng(1)
    for _ in range(200):
        E = int(rng.integers(1, 300)); pairs = int(rng.integers(1, 4097))
        counts = np.bincount(rng.integers(0, E, pairs), minlength=E)
        assert int(((counts + 15) // 16).sum()) <= (pairs + 15 * min(E, pairs)) // 16


def test_ec_rejects_bad_arguments():
    assert lib.ec_workspace_bytes(0, 8, 128, 2048, 768) == 0
    assert lib.ec_workspace_bytes(1, 8, 128, 100, 768) == 0
    assert ec(H=100) == -2 and ec(I=48) == -2 and ec(K=0) == -2 and ec(K=9, E=8) == -2 and ec(B=-1) == -2
    assert ec(E=1025) == -7 and ec(H=8192 + 32) == -7 and ec(I=8192 + 32) == -7 and ec(B=513) == -7
    assert ec(x=None) == -1 and ec(ws=None) == -1 and ec(sd=None) == -1 and ec(out=None) == -1
    assert ec(x=A + 8) == -3 and ec(ws=A + 16) == -3 and ec(out=A + 2) == -3
    assert ec(ws_bytes=lib.ec_workspace_bytes(1, 8, 128, 2048, 768) - 1) == -4
    assert ec(cfg=wd.ECLaunch(last_stage=6)) == -7
    # out is optional when the last stage run is not the combine
    assert ec(out=None, cfg=wd.ECLaunch(last_stage=9)) == -7
    assert ec(B=0, x=None, ids=None, tw=None, out=None, ws=None, ws_bytes=0) == 0
    assert lib.ec_workspace_layout(1, 8, 128, 2048, 768, None) == -1


def test_matrix_core_form_limits():
    # form 3 (gate/up on the matrix cores) has a fixed lane layout, BF16 operands and cached loads
    def gux(**kw):
        return lib.wd_gate_up_ex(A, A, A, A, A, 1, 8, 128, 2048, 768, C.byref(wd.Launch(**kw)), None)

    assert gux(form=3, rows_per_wave=2) == -7
    assert gux(form=3, lanes_per_row=32) == -7
    assert gux(form=3, math=1) == -7
    assert gux(form=3, weight_loads=2) == -7
    assert gux(form=5) == -7
    assert gux(form=4, rows_per_wave=2) == -7 and gux(form=4, math=1) == -7
    # slots per pass over an expert's rows: 16 or 32, the register-staged matrix-core gate/up only
    assert gux(form=3, slots_per_pass=32) == -5 and gux(form=3, slots_per_pass=16) == -5
    assert gux(form=3, slots_per_pass=8) == -7 and gux(form=3, slots_per_pass=64) == -7
    assert gux(form=1, slots_per_pass=32) == -7 and gux(form=4, slots_per_pass=32) == -7
    assert lib.wd_down_ex(A, A, A, A, A, A, 32, 8, 128, 2048, 768, C.byref(wd.Launch(form=3, slots_per_pass=32)),
                          None) == -7
    # the H axis split over a pair of waves: the register-staged matrix-core gate/up, H a multiple
    # of 512, two waves per workgroup
    assert gux(form=3, h_split=2) == -5 and gux(form=3, h_split=1) == -5
    assert gux(form=3, h_split=2, waves_per_block=2) == -5
    assert gux(form=3, h_split=2, waves_per_block=4) == -7 and gux(form=3, h_split=3) == -7
    assert gux(form=1, h_split=2) == -7 and gux(form=4, h_split=2) == -7
    assert lib.wd_gate_up_ex(A, A, A, A, A, 1, 8, 128, 1536 + 256, 768, C.byref(wd.Launch(form=3, h_split=2)),
                             None) == -7
    assert lib.wd_down_ex(A, A, A, A, A, A, 32, 8, 128, 2048, 768, C.byref(wd.Launch(form=3, h_split=2)),
                          None) == -7

    # down on the matrix cores: 8 or 16 waves per workgroup, B <= 64, B * K <= 512, E <= 1024;
    # accepted configurations get as far as the device check (-5 here)
    def dnx(B=1, K=8, E=128, **kw):
        return lib.wd_down_ex(A, A, A, A, A, A, B, K, E, 2048, 768, C.byref(wd.Launch(**kw)), None)

    assert dnx(form=3) == -5
    assert dnx(B=64, form=3) == -5
    assert dnx(B=32, form=3, waves_per_block=16) == -5
    assert dnx(B=33, form=3, waves_per_block=16, token_split=1) == -5
    assert dnx(B=64, form=3, waves_per_block=16, token_split=1) == -5
    # past 64 tokens or 512 slots: the 8-wave variant with room for 128 tokens and 1,024 slots
    assert dnx(B=65, form=3) == -5 and dnx(B=128, form=3) == -5 and dnx(B=40, K=16, form=3) == -5
    assert dnx(B=128, form=3, token_split=2) == -5
    assert dnx(B=65, form=3, waves_per_block=16) == -7 and dnx(B=40, K=16, form=3, waves_per_block=16) == -7
    # past 128 tokens or 1,024 slots: token ranges of up to 128 tokens and 1,024 slots each
    assert dnx(B=129, form=3) == -5 and dnx(B=256, form=3) == -5 and dnx(B=512, form=3) == -5
    assert dnx(B=72, K=16, form=3) == -5           # 1,152 slots: two ranges
    assert dnx(B=129, form=3, token_split=1) == -7 and dnx(B=72, K=16, form=3, token_split=1) == -7
    assert dnx(B=256, form=3, token_split=4) == -5 and dnx(B=256, form=3, token_split=2, waves_per_block=16) == -7
    assert dnx(B=513, form=3) == -7 and dnx(B=512, form=3, token_split=2) == -7
    assert dnx(E=1025, K=8, form=3) == -7
    assert dnx(form=3, waves_per_block=4) == -7
    assert dnx(form=3, rows_per_wave=2) == -7
    assert dnx(form=3, math=1) == -7
    assert dnx(form=3, lanes_per_row=32) == -7
    assert dnx(form=3, weight_loads=2) == -7
    assert dnx(form=2) == -7
    # token ranges per 16-output block: 1, 2 or 4, matrix-core down only
    assert dnx(B=64, form=3, waves_per_block=16, token_split=2) == -5
    assert dnx(B=64, form=3, waves_per_block=16, token_split=4) == -5
    assert dnx(B=33, form=3, waves_per_block=16, token_split=2) == -5
    assert dnx(B=33, form=3, waves_per_block=16) == -5     # default: two ranges at H / 16 = 128 blocks
    assert dnx(B=64, form=3, token_split=3) == -7
    assert dnx(B=64, form=3, token_split=8) == -7
    assert dnx(B=8, form=1, token_split=2) == -7
    assert gux(form=3, token_split=2) == -7 and gux(token_split=2) == -7
    # the default picks it only where it applies; a tuned field keeps the token form
    assert dnx(B=64, E=2048) == -5 and dnx(B=64, K=16) == -5 and dnx(B=64, waves_per_block=2) == -5


def na(**kw):
    d = dict(x=A, ids=A, tw=A, wgu=A, sgu=A, wd=A, sd=A, out=A, B=1, K=8, E=128, H=2048, I=768)
    d.update(kw)
    return lib.wd_moe_decode_noalloc(d["x"], d["ids"], d["tw"], d["wgu"], d["sgu"], d["wd"], d["sd"], d["out"],
                                     d["B"], d["K"], d["E"], d["H"], d["I"], None)


def test_noalloc_host_checks():
    """The no-allocation entry point: the act[B,K,I] of the call must fit the
    4 MiB scratch (341 tokens of the 128-expert / top-8 / I 768 layer); larger
    calls return WD_ERR_SCRATCH before any device call."""
    assert wd.NOALLOC_SCRATCH_BYTES == 4 << 20
    assert na(B=341) == -5                              # fits: reaches the device check
    assert na(B=342) == -8
    assert na(B=128, K=8, I=2048) == -5 and na(B=129, K=8, I=2048) == -8
    assert lib.wd_status_string(-8) and b"scratch" in lib.wd_status_string(-8)
    assert na(B=0, x=None, ids=None, tw=None, out=None) == 0
    assert na(out=None) == -1 and na(wd=None) == -1
    assert na(x=A + 8) == -3 and na(out=A + 1) == -3
    assert na(H=100) == -2 and na(K=32, I=1024) == -7


def test_lds_gate_up_form_limits():
    """Form 4 (matrix-core gate/up streaming its codes into LDS) needs rows of
    a multiple of 256 elements, 4-byte-aligned scale bytes, x within 2 GB and
    2 or 4 waves per workgroup; it is gate/up only."""
    def g(H=2048, B=32, s=A, **kw):
        return lib.wd_gate_up_ex(A, A, A, s, A, B, 8, 128, H, 768, C.byref(wd.Launch(form=4, **kw)), None)
    assert g() == -5 and g(B=1) == -5 and g(waves_per_block=2) == -5
    assert g(H=96) == -7 and g(H=288) == -7 and g(s=A + 2) == -7 and g(waves_per_block=3) == -7
    assert g(H=8192, B=131072) == -7                     # x of 2 GB: past the buffer resource's range
    assert lib.wd_down_ex(A, A, A, A, A, A, 32, 8, 128, 2048, 768, C.byref(wd.Launch(form=4)), None) == -7


def test_down_expert_split_host_checks():
    """The down kernel's expert split needs scratch of wd_down_scratch_bytes(B, H)
    (256-byte aligned), the matrix-core form and no token ranges."""
    assert lib.wd_down_scratch_bytes(32, 2048) == 32 * 2048 * 8          # one 8-byte cell per output
    assert lib.wd_down_scratch_bytes(1, 4096) == 4096 * 8
    assert lib.wd_down_scratch_bytes(0, 2048) == 0 and lib.wd_down_scratch_bytes(1, 100) == 0
    assert lib.wd_layer_workspace_bytes(32, 8, 2048, 768) == 32 * 8 * 768 * 2 + lib.wd_down_scratch_bytes(32, 2048)
    assert lib.wd_layer_workspace_bytes(1, 8, 2048, 96) == 1536 + lib.wd_down_scratch_bytes(1, 2048)
    assert lib.wd_layer_workspace_bytes(1, 1, 2048, 96) == 256 + lib.wd_down_scratch_bytes(1, 2048)  # act padded
    need = lib.wd_down_scratch_bytes(32, 2048)

    def dnx(scr=A, nbytes=need, B=32, **kw):
        cfg = wd.Launch(down_scratch=scr, down_scratch_bytes=nbytes, **kw)
        return lib.wd_down_ex(A, A, A, A, A, A, B, 8, 128, 2048, 768, C.byref(cfg), None)

    assert dnx(form=3, expert_split=2) == -5
    assert dnx() == -5                                        # the default takes it
    assert dnx(form=3, expert_split=2, token_split=2) == -7
    assert dnx(form=3, expert_split=2, nbytes=need - 1) == -7
    assert dnx(form=3, expert_split=2, scr=A + 16) == -7      # scratch not 256-byte aligned
    assert dnx(form=1, expert_split=2) == -7
    assert dnx(form=3, expert_split=3) == -7
    assert dnx(scr=None, nbytes=0, form=3, expert_split=2) == -7
    assert lib.wd_gate_up_ex(A, A, A, A, A, 32, 8, 128, 2048, 768, C.byref(wd.Launch(expert_split=2)), None) == -7
