"""Python binding of libwd.so (the C ABI in include/wd.h and include/ec.h).

Argument marshalling only: the functions check dtypes, devices, contiguity
and shapes of torch tensors, then pass raw device pointers, sizes and the
current HIP stream to the library.  All computation happens in the library's
HIP kernels.  Importing this module fails loudly when the library has not
been built (python -m moe_decode_gate_amd.build).
"""
from __future__ import annotations

import ctypes as C
import os
import re
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libwd.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "wd.h")
EC_HEADER = os.path.join(os.path.dirname(_PKG), "include", "ec.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                      "(python -m moe_decode_gate_amd.build)")
_lib = C.CDLL(LIB_PATH)

WD_OK = 0
STATUS = {0: "WD_OK", -1: "WD_ERR_NULL", -2: "WD_ERR_DIMS", -3: "WD_ERR_ALIGN", -4: "WD_ERR_WORKSPACE",
          -5: "WD_ERR_DEVICE", -6: "WD_ERR_LAUNCH", -7: "WD_ERR_UNSUPPORTED", -8: "WD_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 4 << 20      # WD_NOALLOC_SCRATCH_BYTES in include/wd.h


class WDError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.wd_status_string(status).decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")


class Launch(C.Structure):
    """Launch configuration (wd_launch); 0 fields take the library default.
    start_event / stop_event: raw hipEvent_t handles (e.g. torch.cuda.Event's
    cuda_event after one record()) that receive the kernel's own start/end."""
    _fields_ = [("rows_per_wave", C.c_int), ("waves_per_block", C.c_int),
                ("order", C.c_int), ("xcd_remap", C.c_int),
                ("start_event", C.c_void_p), ("stop_event", C.c_void_p), ("math", C.c_int),
                ("lanes_per_row", C.c_int), ("form", C.c_int), ("weight_loads", C.c_int),
                ("token_split", C.c_int), ("lds_bytes", C.c_int), ("expert_split", C.c_int),
                ("down_scratch", C.c_void_p), ("down_scratch_bytes", C.c_size_t),
                ("slots_per_pass", C.c_int), ("h_split", C.c_int)]


class ECLaunch(C.Structure):
    """Expert-centric launch settings (ec_launch): last_stage (0 = all five),
    keep_intermediate, and per-stage start/stop hipEvent_t handles."""
    _fields_ = [("last_stage", C.c_int), ("keep_intermediate", C.c_int),
                ("start_event", C.c_void_p * 5), ("stop_event", C.c_void_p * 5)]


# Workspace regions of the expert-centric path (enum in include/ec.h).
EC_WS = ("header", "tile_expert", "row_pair", "xq", "xs", "act", "aq", "out_pair", "total")

_P, _I, _S = C.c_void_p, C.c_int, C.c_size_t
_sig = {
    "wd_gate_up": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "wd_gate_up_ex": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, C.POINTER(Launch), _P]),
    "wd_down": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "wd_down_ex": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, C.POINTER(Launch), _P]),
    "wd_moe_decode": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _S, _P, _I, _I, _I, _I, _I, _P]),
    "wd_moe_decode_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "wd_workspace_bytes": (_S, [_I, _I, _I]),
    "wd_down_scratch_bytes": (_S, [_I, _I]),
    "wd_layer_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "wd_route": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "wd_status_string": (C.c_char_p, [_I]),
    "wd_dequant_probe": (_I, [_P, _P]),
    "wd_stream_read": (_I, [_P, _S, _P, _I, _I, _P, _P, _P]),
    "wd_stream_blocks": (_I, []),
    "wd_stream_copy": (_I, [_P, _P, _S, _I, _P]),
    "wd_gpu_sleep": (_I, [_I, _P]),
    "ec_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "ec_workspace_layout": (_I, [_I, _I, _I, _I, _I, C.POINTER(C.c_size_t)]),
    "ec_moe_decode": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _S, _P, _I, _I, _I, _I, _I, _P]),
    "ec_mma_probe": (_I, [_P, _P, _P, _P, _P, _I, _P]),
    "ec_moe_decode_ex": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _S, _P, _I, _I, _I, _I, _I,
                              C.POINTER(ECLaunch), _P]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype, _f.argtypes = _res, _args


def header_functions(paths=(HEADER, EC_HEADER)):
    """Names of the functions include/wd.h and include/ec.h declare."""
    names = set()
    for path in ([paths] if isinstance(paths, str) else paths):
        text = open(path).read()
        names |= set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*((?:wd|ec)_[a-z_0-9]+)\s*\(", text, re.M))
    return sorted(names)


def _check(rc: int, where: str):
    if rc != WD_OK:
        raise WDError(rc, where)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtypes, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    return t


_U8 = (torch.uint8, torch.float8_e4m3fn, torch.float8_e8m0fnu)
_BF16 = (torch.bfloat16, torch.uint16, torch.int16)


def _dims(w_gu: torch.Tensor):
    E, I2, H = w_gu.shape
    return E, H, I2 // 2


def _cfg(cfg):
    if cfg is None:
        return None
    if isinstance(cfg, Launch):
        return C.byref(cfg)
    cfg = dict(cfg)
    scr = cfg.pop("down_scratch", None)
    if isinstance(scr, torch.Tensor):     # a device tensor: its pointer and size
        cfg["down_scratch"], cfg["down_scratch_bytes"] = scr.data_ptr(), scr.numel() * scr.element_size()
    elif scr is not None:
        cfg["down_scratch"] = scr
    return C.byref(Launch(**cfg))


def gate_up(x, topk_ids, w_gu, s_gu, act=None, cfg=None, stream=None):
    """act[B,K,I] (bf16) = BF16(SiLU(Gate x) * Up x) per (token, slot)."""
    E, H, I = _dims(w_gu)
    B, K = topk_ids.shape
    _dev(x, "x", _BF16, (B, H)); _dev(topk_ids, "topk_ids", (torch.int32,))
    _dev(w_gu, "w_gu", _U8, (E, 2 * I, H)); _dev(s_gu, "s_gu", _U8, (E, 2 * I, H // 32))
    if act is None:
        act = torch.empty((B, K, I), dtype=torch.bfloat16, device=x.device)
    _dev(act, "act", _BF16, (B, K, I))
    if cfg is None:
        rc = _lib.wd_gate_up(_ptr(x), _ptr(topk_ids), _ptr(w_gu), _ptr(s_gu), _ptr(act), B, K, E, H, I,
                             _stream(stream))
    else:
        rc = _lib.wd_gate_up_ex(_ptr(x), _ptr(topk_ids), _ptr(w_gu), _ptr(s_gu), _ptr(act), B, K, E, H, I,
                                _cfg(cfg), _stream(stream))
    _check(rc, "wd_gate_up")
    return act


def down(act, topk_ids, topk_w, w_d, s_d, out=None, cfg=None, stream=None):
    """out[B,H] (bf16) = sum_k topk_w[b,k] * Down_e act[b,k]."""
    E, H, I = w_d.shape
    B, K = topk_ids.shape
    _dev(act, "act", _BF16, (B, K, I)); _dev(topk_ids, "topk_ids", (torch.int32,))
    _dev(topk_w, "topk_w", (torch.float32,), (B, K))
    _dev(w_d, "w_d", _U8); _dev(s_d, "s_d", _U8, (E, H, I // 32))
    if out is None:
        out = torch.empty((B, H), dtype=torch.bfloat16, device=act.device)
    _dev(out, "out", _BF16, (B, H))
    if cfg is None:
        rc = _lib.wd_down(_ptr(act), _ptr(topk_ids), _ptr(topk_w), _ptr(w_d), _ptr(s_d), _ptr(out),
                          B, K, E, H, I, _stream(stream))
    else:
        rc = _lib.wd_down_ex(_ptr(act), _ptr(topk_ids), _ptr(topk_w), _ptr(w_d), _ptr(s_d), _ptr(out),
                             B, K, E, H, I, _cfg(cfg), _stream(stream))
    _check(rc, "wd_down")
    return out


def route(logits, K: int, topk_ids=None, topk_w=None, stream=None):
    """(topk_ids [B,K] int32, topk_w [B,K] fp32) from router logits [B,E] fp32."""
    _dev(logits, "logits", (torch.float32,))
    B, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((B, K), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((B, K), dtype=torch.float32, device=logits.device)
    _dev(topk_ids, "topk_ids", (torch.int32,), (B, K)); _dev(topk_w, "topk_w", (torch.float32,), (B, K))
    _check(_lib.wd_route(_ptr(logits), B, E, K, _ptr(topk_ids), _ptr(topk_w), _stream(stream)), "wd_route")
    return topk_ids, topk_w


def workspace_bytes(B: int, K: int, I: int) -> int:
    return _lib.wd_workspace_bytes(B, K, I)


def down_scratch_bytes(B: int, H: int) -> int:
    return _lib.wd_down_scratch_bytes(B, H)


def layer_workspace_bytes(B: int, K: int, H: int, I: int) -> int:
    return _lib.wd_layer_workspace_bytes(B, K, H, I)


def down_scratch(B: int, H: int, device="cuda") -> torch.Tensor:
    """Zeroed scratch for the down kernel's expert split (wd_launch.down_scratch);
    every call leaves its cells zero again, so it can be reused by calls in
    stream order."""
    return torch.zeros(max(down_scratch_bytes(B, H), 256), dtype=torch.uint8, device=device)


def moe_decode(x, topk_ids, topk_w, w_gu, s_gu, w_d, s_d, out=None, workspace=None, stream=None):
    """The whole layer (gate/up then down) on one stream; returns out[B,H] bf16."""
    E, H, I = _dims(w_gu)
    B, K = topk_ids.shape
    _dev(x, "x", _BF16, (B, H)); _dev(topk_ids, "topk_ids", (torch.int32,))
    _dev(topk_w, "topk_w", (torch.float32,), (B, K))
    _dev(w_gu, "w_gu", _U8, (E, 2 * I, H)); _dev(s_gu, "s_gu", _U8, (E, 2 * I, H // 32))
    _dev(w_d, "w_d", _U8, (E, H, I)); _dev(s_d, "s_d", _U8, (E, H, I // 32))
    if out is None:
        out = torch.empty((B, H), dtype=torch.bfloat16, device=x.device)
    _dev(out, "out", _BF16, (B, H))
    need = layer_workspace_bytes(B, K, H, I)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _dev(workspace, "workspace", (torch.uint8, torch.bfloat16))
    rc = _lib.wd_moe_decode(_ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(w_gu), _ptr(s_gu), _ptr(w_d), _ptr(s_d),
                            _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
                            B, K, E, H, I, _stream(stream))
    _check(rc, "wd_moe_decode")
    return out


def moe_decode_noalloc(x, topk_ids, topk_w, w_gu, s_gu, w_d, s_d, out=None, stream=None):
    """The whole layer through wd_moe_decode_noalloc: the intermediate lives in
    the library's per-GPU scratch array (no workspace).  Calls overlapping in
    time on one GPU race on that array."""
    E, H, I = _dims(w_gu)
    B, K = topk_ids.shape
    _dev(x, "x", _BF16, (B, H)); _dev(topk_ids, "topk_ids", (torch.int32,))
    _dev(topk_w, "topk_w", (torch.float32,), (B, K))
    _dev(w_gu, "w_gu", _U8, (E, 2 * I, H)); _dev(s_gu, "s_gu", _U8, (E, 2 * I, H // 32))
    _dev(w_d, "w_d", _U8, (E, H, I)); _dev(s_d, "s_d", _U8, (E, H, I // 32))
    if out is None:
        out = torch.empty((B, H), dtype=torch.bfloat16, device=x.device)
    _dev(out, "out", _BF16, (B, H))
    rc = _lib.wd_moe_decode_noalloc(_ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(w_gu), _ptr(s_gu), _ptr(w_d),
                                    _ptr(s_d), _ptr(out), B, K, E, H, I, _stream(stream))
    _check(rc, "wd_moe_decode_noalloc")
    return out


def dequant_probe(device="cuda", stream=None) -> torch.Tensor:
    """[2 math modes (FP32, BF16), 256 scales, 256 codes, 4 byte lanes] conversions (see wd.h)."""
    out = torch.empty((2, 256, 256, 4), dtype=torch.float32, device=device)
    _check(_lib.wd_dequant_probe(_ptr(out), _stream(stream)), "wd_dequant_probe")
    return out


def stream_blocks() -> int:
    return _lib.wd_stream_blocks()


def stream_read(buf: torch.Tensor, sink: torch.Tensor, blocks: int = 0, unroll: int = 4, start_event=None,
                stop_event=None, stream=None):
    """start_event / stop_event: raw hipEvent_t handles that receive the kernel's own start and end."""
    nbytes = buf.numel() * buf.element_size()
    _check(_lib.wd_stream_read(_ptr(buf), nbytes, _ptr(sink), blocks, unroll, start_event, stop_event,
                               _stream(stream)), "wd_stream_read")


def stream_copy(dst: torch.Tensor, src: torch.Tensor, blocks: int = 0, stream=None):
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    _check(_lib.wd_stream_copy(_ptr(dst), _ptr(src), nbytes, blocks, _stream(stream)), "wd_stream_copy")


def gpu_sleep(units: int, stream=None):
    _check(_lib.wd_gpu_sleep(units, _stream(stream)), "wd_gpu_sleep")


def ec_workspace_bytes(B: int, K: int, E: int, H: int, I: int) -> int:
    return _lib.ec_workspace_bytes(B, K, E, H, I)


def ec_workspace_layout(B: int, K: int, E: int, H: int, I: int) -> dict:
    """Byte offsets of the expert-centric workspace regions (EC_WS names)."""
    off = (C.c_size_t * len(EC_WS))()
    _check(_lib.ec_workspace_layout(B, K, E, H, I, off), "ec_workspace_layout")
    return dict(zip(EC_WS, list(off)))


def ec_moe_decode(x, topk_ids, topk_w, w_gu, s_gu, w_d, s_d, out=None, workspace=None, cfg=None, stream=None):
    """The expert-centric layer (align, gather, gate/up, down, combine); returns out[B,H] bf16.
    cfg: an ECLaunch (or None).  With cfg.last_stage in 1..4 out is left untouched."""
    E, H, I = _dims(w_gu)
    B, K = topk_ids.shape
    _dev(x, "x", _BF16, (B, H)); _dev(topk_ids, "topk_ids", (torch.int32,))
    _dev(topk_w, "topk_w", (torch.float32,), (B, K))
    _dev(w_gu, "w_gu", _U8, (E, 2 * I, H)); _dev(s_gu, "s_gu", _U8, (E, 2 * I, H // 32))
    _dev(w_d, "w_d", _U8, (E, H, I)); _dev(s_d, "s_d", _U8, (E, H, I // 32))
    if out is None:
        out = torch.empty((B, H), dtype=torch.bfloat16, device=x.device)
    _dev(out, "out", _BF16, (B, H))
    need = ec_workspace_bytes(B, K, E, H, I)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _dev(workspace, "workspace", (torch.uint8,))
    args = (_ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(w_gu), _ptr(s_gu), _ptr(w_d), _ptr(s_d),
            _ptr(workspace), workspace.numel(), _ptr(out), B, K, E, H, I)
    if cfg is None:
        rc = _lib.ec_moe_decode(*args, _stream(stream))
    else:
        rc = _lib.ec_moe_decode_ex(*args, C.byref(cfg), _stream(stream))
    _check(rc, "ec_moe_decode")
    return out


def ec_mma_probe(a, b, sa, sb, stream=None) -> torch.Tensor:
    """out[n,16,16] fp32 from one MX matrix instruction per block (see ec.h)."""
    n = a.shape[0]
    _dev(a, "a", _U8, (n, 16, 128)); _dev(b, "b", _U8, (n, 16, 128))
    _dev(sa, "sa", _U8, (n, 16, 4)); _dev(sb, "sb", _U8, (n, 16, 4))
    out = torch.empty((n, 16, 16), dtype=torch.float32, device=a.device)
    _check(_lib.ec_mma_probe(_ptr(a), _ptr(b), _ptr(sa), _ptr(sb), _ptr(out), n, _stream(stream)), "ec_mma_probe")
    return out


# Raw entry points for callers that manage pointers themselves (tests, bench).
raw = _lib
