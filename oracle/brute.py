"""Expert-centric brute force for tiny layers.  Test infrastructure only.

An independent second computation of the MoE decode layer used to pin the C
oracle.  It deliberately takes the *other* route through the same mathematics:
the conventional expert-centric dataflow the warp-decode write-ups contrast
their method with ("Better MoE model inference with warp decode", Key claims,
section "The conventional MoE path": route, gather the tokens of each expert,
run each expert on its tokens, scatter the expert outputs back, combine with
the router weights), in exact rational arithmetic:

* element values come from torch's float8_e4m3fn / float8_e8m0fnu decoders
  (a library routine, not the oracle's closed form);
* every dot product is an exact ``fractions.Fraction`` sum;
* the intermediate is rounded FP64 -> FP32 -> BF16 with torch conversions;
* the router combine is done after the scatter, on exact values.

Only SiLU's sigmoid goes through ``math.exp`` (FP64).  Feasible for layers of
a few thousand weights per expert.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch


def _deq_rows(codes: np.ndarray, scales: np.ndarray):
    """Decode MXFP8 rows [R, n] into lists of exact Fractions via torch dtypes."""
    v = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e8m0fnu).to(torch.float64)
    s = s.repeat_interleave(32, dim=-1)
    vals = (v * s).tolist()         # exact: <=4 significant bits times a power of two
    return [[Fraction(a) for a in row] for row in vals]


def _bf16_to_fraction(bits: np.ndarray):
    f = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64)
    return [[Fraction(a) for a in row] for row in f.tolist()]


def _act_round(a: float) -> int:
    t = torch.tensor([a], dtype=torch.float64).to(torch.float32).to(torch.bfloat16)
    return int(t.view(torch.int16).item()) & 0xFFFF


def _bf16_bits_to_float(bits: int) -> float:
    t = torch.from_numpy(np.array([bits], np.uint16).view(np.int16)).view(torch.bfloat16)
    return float(t.to(torch.float64).item())


def moe_decode(x, ids, w, wgu, sgu, wd, sd):
    """Returns (y as float list [B][H], act bits [B,K,I] uint16, y exact Fractions)."""
    E, I2, H = wgu.shape
    I = I2 // 2
    B, K = ids.shape
    xs = _bf16_to_fraction(x)
    # 1. route: which (token, slot) pairs each expert serves
    served = {}
    for b in range(B):
        for k in range(K):
            e = int(ids[b, k])
            if not 0 <= e < E:
                raise ValueError("expert id out of range")
            served.setdefault(e, []).append((b, k))
    act = np.zeros((B, K, I), np.uint16)
    expert_out = {}
    for e, pairs in served.items():
        gu = _deq_rows(wgu[e], sgu[e])          # [2I][H]
        dn = _deq_rows(wd[e], sd[e])            # [H][I]
        # 2. gather this expert's tokens and run the expert on all of them
        for (b, k) in pairs:
            xb = xs[b]
            inter = []
            for j in range(I):
                g = sum((gu[j][h] * xb[h] for h in range(H)), Fraction(0))
                u = sum((gu[I + j][h] * xb[h] for h in range(H)), Fraction(0))
                gf = float(g)
                sig = 1.0 / (1.0 + math.exp(-gf)) if gf >= 0 else math.exp(gf) / (1.0 + math.exp(gf))
                bits = _act_round(gf * sig * float(u))
                act[b, k, j] = bits
                inter.append(Fraction(_bf16_bits_to_float(bits)))
            out = [sum((dn[h][i] * inter[i] for i in range(I)), Fraction(0)) for h in range(H)]
            expert_out[(b, k)] = out            # 3. scatter back to (token, slot)
    # 4. combine with the router weights
    y = []
    for b in range(B):
        row = [Fraction(0)] * H
        for k in range(K):
            wk = Fraction(float(w[b, k]))
            o = expert_out[(b, k)]
            row = [row[h] + wk * o[h] for h in range(H)]
        y.append(row)
    return [[float(v) for v in row] for row in y], act, y
