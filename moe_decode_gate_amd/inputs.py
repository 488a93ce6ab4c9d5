"""Seeded synthetic inputs for the MoE decode layer.

This module is shared by the CPU oracle's tests and by the HIP path: it only
*draws* inputs.  It holds none of the layer's arithmetic (no dequantization,
no dot products, no activation function).  Everything it returns is a plain
NumPy array of the exact bits both sides consume:

* expert weights as MXFP8: OCP E4M3 ("FN") element codes, uint8, plus one
  E8M0 exponent byte per 32 consecutive elements along the reduction axis;
* activations x as BF16 bit patterns (uint16);
* routing as int32 expert ids and float32 router weights.

Workload shapes follow the Qwen-3-style MoE decode layer the warp-decode
write-ups measure (128 experts, top-8, hidden 2048; "Better MoE model
inference with warp decode", Key claims / section "Buffer elimination").
Weights are drawn N(0, 0.02) in fp32 and quantized per 32-element block with
the OCP MX scale rule (shared exponent = floor(log2(max|v|)) - emax_elem,
emax_elem = 8 for E4M3), elements rounded to nearest-even with saturation at
+-448.  Every expert of every tensor draws from its own child stream of a
``numpy.random.SeedSequence``, so an expert's bits do not depend on which other
experts were generated, and generation parallelises over experts.
"""

from __future__ import annotations

import dataclasses
import hashlib
import json
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = [
    "LayerSpec", "CONFIGS", "Layer", "Tokens",
    "quantize_mxfp8", "bf16_bits", "make_layer", "make_tokens",
    "layer_unique_bytes", "expert_bytes", "make_logits", "expert_weights_fp32",
    "save_layer", "load_layer", "MANIFEST_FORMAT",
]

BLOCK = 32          # MX block: elements sharing one E8M0 scale
E4M3_MAX = 448.0    # largest finite E4M3FN magnitude
E4M3_EMAX = 8       # exponent of the largest E4M3FN binade (448 = 1.75 * 2^8)

# Seed streams: one spawn key per tensor kind.
_KIND_WGU, _KIND_WD, _KIND_X, _KIND_ROUTE = 0, 1, 2, 3


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """Shape of one MoE decode layer."""
    E: int          # experts
    K: int          # experts routed per token (top-k)
    H: int          # hidden size (gate/up reduction axis, down output axis)
    I: int          # expert intermediate size (down reduction axis)
    seed: int       # root seed

    def __post_init__(self):
        if self.H % BLOCK or self.I % BLOCK:
            raise ValueError("H and I must be multiples of 32 (one E8M0 scale per 32 elements)")
        if not (1 <= self.K <= self.E):
            raise ValueError("need 1 <= K <= E")


# Workloads (sizes of the layer the pages measure, plus a tiny one that a
# pure-Python checker finishes quickly).
CONFIGS = {
    "tiny":   dict(spec=LayerSpec(E=8, K=2, H=128, I=64, seed=20260000), batches=(1,), routing="softmax"),
    "qwen3":  dict(spec=LayerSpec(E=128, K=8, H=2048, I=768, seed=20260001), batches=(1,), routing="softmax"),
    "qwen3_b32": dict(spec=LayerSpec(E=128, K=8, H=2048, I=768, seed=20260002), batches=(32,), routing="softmax"),
    "large":  dict(spec=LayerSpec(E=128, K=8, H=4096, I=1536, seed=20260003), batches=(1, 8, 32), routing="zipf"),
    "stack":  dict(spec=LayerSpec(E=128, K=8, H=2048, I=768, seed=20260400), batches=(1, 2, 4, 8, 16, 32, 64),
                   routing="softmax"),
}


@dataclasses.dataclass
class Layer:
    """One layer's MXFP8 expert weights (host arrays).

    wgu: [E, 2I, H] uint8 E4M3 codes; rows [0, I) are gate rows, [I, 2I) up rows.
    sgu: [E, 2I, H/32] uint8 E8M0 exponents.
    wd:  [E, H, I] uint8 E4M3 codes.
    sd:  [E, H, I/32] uint8 E8M0 exponents.
    experts: which experts hold drawn values (others are all-zero codes with
             scale byte 127, i.e. exactly zero weights).
    """
    spec: LayerSpec
    wgu: np.ndarray
    sgu: np.ndarray
    wd: np.ndarray
    sd: np.ndarray
    experts: tuple


@dataclasses.dataclass
class Tokens:
    """One decode batch: x as bf16 bits [B,H], ids int32 [B,K], w float32 [B,K]."""
    x: np.ndarray
    ids: np.ndarray
    w: np.ndarray


def bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float values to BF16 (nearest-even, via torch) and return the bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def quantize_mxfp8(v: np.ndarray):
    """Quantize fp32 values along the last axis to MXFP8 (OCP MX rule).

    Returns (codes uint8 with v's shape, scales uint8 with last axis / 32).
    Shared exponent per 32-block: floor(log2(amax)) - 8, stored biased by 127
    and clamped to [0, 254]; an all-zero block gets scale byte 0.  Elements are
    divided by 2^shared (exact), clamped to +-448 and rounded to the nearest
    E4M3FN value, ties to even (torch's float8_e4m3fn conversion).
    """
    v = np.asarray(v, dtype=np.float32)
    if v.shape[-1] % BLOCK:
        raise ValueError("last axis must be a multiple of 32")
    blk = v.reshape(v.shape[:-1] + (v.shape[-1] // BLOCK, BLOCK))
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(amax)                 # amax = m * 2^ex, m in [0.5, 1)
    shared = ex.astype(np.int32) - 1 - E4M3_EMAX
    sbyte = np.clip(shared + 127, 0, 254)
    sbyte = np.where(amax > 0, sbyte, 0).astype(np.uint8)
    q = np.ldexp(blk, -(sbyte.astype(np.int32) - 127)[..., None])
    q = np.clip(q, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(q.reshape(v.shape)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes.copy(), sbyte


def _expert_stream(spec: LayerSpec, kind: int, e: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(spec.seed, spawn_key=(kind, e)))


def expert_weights_fp32(spec: LayerSpec, e: int, std: float = 0.02):
    """Expert e's weights as drawn, before MXFP8 quantization: (gate/up [2I, H],
    down [H, I]) float32, from the same streams make_layer quantizes."""
    rg = _expert_stream(spec, _KIND_WGU, e)
    gu = rg.standard_normal((2 * spec.I, spec.H), dtype=np.float32) * np.float32(std)
    rd = _expert_stream(spec, _KIND_WD, e)
    dn = rd.standard_normal((spec.H, spec.I), dtype=np.float32) * np.float32(std)
    return gu, dn


def _draw_expert(spec: LayerSpec, e: int, std: float):
    gu, dn = expert_weights_fp32(spec, e, std)
    return quantize_mxfp8(gu), quantize_mxfp8(dn)


def make_layer(spec: LayerSpec, experts: Optional[Sequence[int]] = None, std: float = 0.02,
               threads: int = 8) -> Layer:
    """Draw a layer's MXFP8 weights.  `experts` limits which experts get drawn
    values (default: all); the rest are exact zeros (code 0, scale byte 127)."""
    E, H, I = spec.E, spec.H, spec.I
    ex = tuple(range(E)) if experts is None else tuple(sorted(set(int(e) for e in experts)))
    wgu = np.zeros((E, 2 * I, H), np.uint8)
    sgu = np.full((E, 2 * I, H // BLOCK), 127, np.uint8)
    wd = np.zeros((E, H, I), np.uint8)
    sd = np.full((E, H, I // BLOCK), 127, np.uint8)

    def one(e):
        (c1, s1), (c2, s2) = _draw_expert(spec, e, std)
        wgu[e], sgu[e], wd[e], sd[e] = c1, s1, c2, s2

    with ThreadPoolExecutor(max(1, threads)) as pool:
        list(pool.map(one, ex))
    return Layer(spec, wgu, sgu, wd, sd, ex)


def make_tokens(spec: LayerSpec, B: int, routing: str = "softmax", step: int = 0,
                zipf_s: float = 1.2) -> Tokens:
    """Draw one decode batch.

    x: N(0,1) rounded to BF16.
    routing "softmax": router logits N(0,1) over all E experts, the top-K by
      logit (descending; continuous draws make ties a null event, broken toward
      the lower index), weights = softmax over the chosen K logits (the full
      softmax renormalised over the top-K).  Ids of one token are distinct and,
      over tokens, a uniformly random K-subset.
    routing "zipf": a seeded permutation pi ranks the experts; expert pi[r] has
      popularity (r+1)^(-s).  Each token draws K distinct experts without
      replacement with probabilities proportional to popularity; weights are
      the softmax of N(0,1) logits over the chosen K, listed in descending order.
    """
    E, K, H = spec.E, spec.K, spec.H
    rx = np.random.default_rng(np.random.SeedSequence(spec.seed, spawn_key=(_KIND_X, step, B)))
    x = bf16_bits(rx.standard_normal((B, H)))
    rr = np.random.default_rng(np.random.SeedSequence(spec.seed, spawn_key=(_KIND_ROUTE, step, B)))
    if routing == "softmax":
        logits = rr.standard_normal((B, E))
        ids = np.argsort(-logits, axis=1, kind="stable")[:, :K]
        chosen = np.take_along_axis(logits, ids, axis=1)
    elif routing == "zipf":
        perm = np.random.default_rng(np.random.SeedSequence(spec.seed, spawn_key=(_KIND_ROUTE, 999))).permutation(E)
        pop = np.empty(E)
        pop[perm] = (np.arange(E) + 1.0) ** (-zipf_s)
        pop /= pop.sum()
        ids = np.stack([rr.choice(E, size=K, replace=False, p=pop) for _ in range(B)])
        chosen = np.sort(rr.standard_normal((B, K)), axis=1)[:, ::-1]
    else:
        raise ValueError(routing)
    z = np.exp(chosen - chosen.max(axis=1, keepdims=True))
    w = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return Tokens(x=x, ids=np.ascontiguousarray(ids, dtype=np.int32), w=np.ascontiguousarray(w))


def make_logits(spec: LayerSpec, B: int, step: int = 0) -> np.ndarray:
    """Router logits [B, E] as float32: the same N(0,1) draws that make_tokens'
    softmax routing ranks, rounded to FP32 (the router's input precision)."""
    rr = np.random.default_rng(np.random.SeedSequence(spec.seed, spawn_key=(_KIND_ROUTE, step, B)))
    return np.ascontiguousarray(rr.standard_normal((B, spec.E)).astype(np.float32))


def expert_bytes(spec: LayerSpec) -> int:
    """MXFP8 bytes (codes + E8M0 scales) of one expert: gate/up plus down."""
    H, I = spec.H, spec.I
    return 2 * I * H + 2 * I * (H // BLOCK) + H * I + H * (I // BLOCK)


def layer_unique_bytes(spec: LayerSpec, ids: np.ndarray) -> int:
    """Weight bytes a layer step must read at least once: every expert routed
    by at least one token, counted once."""
    return int(np.unique(np.asarray(ids)).size) * expert_bytes(spec)


# ---- weight sets on disk ----------------------------------------------------

MANIFEST_FORMAT = "moe-decode-mxfp8-layer/1"
_ARRAYS = ("wgu", "sgu", "wd", "sd")


def _sha256(path: str) -> str:
    h = hashlib.sha256()
    with open(path, "rb") as f:
        for chunk in iter(lambda: f.read(1 << 22), b""):
            h.update(chunk)
    return h.hexdigest()


def save_layer(L: Layer, path: str, std: float = 0.02) -> dict:
    """Write a layer's weight set to directory `path`: wgu/sgu/wd/sd as .npy files
    (uint8 codes and E8M0 bytes, exactly the bits the kernels read) and
    manifest.json holding the shape, the seed and the quantizer rule that
    produced them, and each file's shape, dtype and SHA-256, so a run can be
    reproduced from the files or regenerated from the manifest alone.  Returns
    the manifest."""
    os.makedirs(path, exist_ok=True)
    arrays = {}
    for name in _ARRAYS:
        a = np.ascontiguousarray(getattr(L, name))
        fn = name + ".npy"
        np.save(os.path.join(path, fn), a, allow_pickle=False)
        arrays[name] = {"file": fn, "shape": list(a.shape), "dtype": str(a.dtype),
                        "sha256": _sha256(os.path.join(path, fn))}
    sp = L.spec
    man = {
        "format": MANIFEST_FORMAT,
        "spec": {"E": sp.E, "K": sp.K, "H": sp.H, "I": sp.I, "seed": sp.seed},
        "experts": [int(e) for e in L.experts],
        "std": std,
        "generator": "per expert and tensor kind a numpy SeedSequence(seed, spawn_key=(kind, expert)) "
                     "stream (kind 0: gate/up [2I, H], 1: down [H, I]), N(0, std) in float32; "
                     "experts not listed are exact zeros (code 0, scale byte 127)",
        "quantizer": {"block": BLOCK, "element": "OCP E4M3FN", "scale": "OCP E8M0, bias 127",
                      "shared_exponent": "floor(log2(max|v| of the block)) - 8, byte clamped to [0, 254]; "
                                         "an all-zero block gets byte 0",
                      "elements": "v / 2^shared clamped to +-448, rounded to nearest E4M3FN, ties to even"},
        "layout": {"wgu": "[E, 2I, H] rows [0, I) gate, [I, 2I) up", "sgu": "[E, 2I, H/32]",
                   "wd": "[E, H, I]", "sd": "[E, H, I/32]"},
        "arrays": arrays,
    }
    with open(os.path.join(path, "manifest.json"), "w") as f:
        json.dump(man, f, indent=1, sort_keys=True)
    return man


def load_layer(path: str, verify: bool = True) -> Layer:
    """Read a weight set written by save_layer.  Arrays are loaded without
    unpickling (allow_pickle=False); their shapes and dtypes must match the
    manifest and the layer shape it states, and with `verify` each file's
    SHA-256 must match too.  Raises ValueError on any mismatch."""
    with open(os.path.join(path, "manifest.json")) as f:
        man = json.load(f)
    if man.get("format") != MANIFEST_FORMAT:
        raise ValueError(f"unknown weight-set format {man.get('format')!r}")
    spec = LayerSpec(**man["spec"])
    E, H, I = spec.E, spec.H, spec.I
    want = {"wgu": (E, 2 * I, H), "sgu": (E, 2 * I, H // BLOCK), "wd": (E, H, I), "sd": (E, H, I // BLOCK)}
    out = {}
    for name in _ARRAYS:
        ent = man["arrays"][name]
        fn = os.path.join(path, ent["file"])
        if verify and _sha256(fn) != ent["sha256"]:
            raise ValueError(f"{ent['file']}: SHA-256 does not match the manifest")
        a = np.load(fn, allow_pickle=False)
        if a.dtype != np.uint8 or tuple(a.shape) != want[name] or list(a.shape) != ent["shape"]:
            raise ValueError(f"{ent['file']}: {a.dtype} {a.shape}, the manifest's layer needs uint8 {want[name]}")
        out[name] = a
    return Layer(spec, out["wgu"], out["sgu"], out["wd"], out["sd"], tuple(man["experts"]))
