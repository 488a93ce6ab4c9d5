// The two gfx950 kernels of the output-neuron-centric MoE decode layer.
//
// Gate/up (the write-ups' moe_gate_up_3d_batched) and down
// (moe_down_3d_batched): "Better MoE model inference with warp decode", Key
// claims, section "How the two kernels work", and the Chinese summary's
// 技术原理 section with its Gate/Up and Down kernel subsections.
//
// Token forms (the pages' design; the defaults for small batches): each 64-lane
// wave owns output values for its whole life, streams the MXFP8 weight rows
// it needs straight from HBM into registers, converts them as it reads them,
// keeps a private FP32 accumulator and finishes with a cross-lane butterfly;
// waves never exchange data, so there is no LDS traffic, no barrier and no
// atomic.
//
// Expert forms on the matrix cores (the defaults from about 20 tokens, where tokens
// share experts; a departure from the pages' design): gate/up takes one wave
// per (expert, 16 intermediate rows) and down one workgroup per (16 output
// dims, token range or class of experts); both stage weight tiles through LDS
// (their own wave's region, or with the down kernel's workgroup barrier the
// per-slot products), and compute the same FP32 sums of exact products on
// v_mfma_f32_16x16x32_bf16 in another order.  Gate/up keeps no atomic and no
// buffer besides the intermediate; the down kernel's expert split adds a
// scratch cell per output, through which the two workgroups of a block hand
// over their FP32 partial sums (one atomic exchange per output).
#pragma once

#include <type_traits>

#include "wd_device.h"

namespace wd {

// Kernel arguments shared by both kernels.
struct LayerArgs {
    const uint16_t *x;       // [B,H] bf16
    const int32_t *ids;      // [B,K]
    const float *tw;         // [B,K]
    const uint8_t *w;        // gate/up: [E,2I,H] codes; down: [E,H,I] codes
    const uint8_t *s;        // matching E8M0 bytes
    const uint16_t *act_in;  // down: [B,K,I] bf16
    uint16_t *out;           // gate/up: act [B,K,I]; down: out [B,H]
    int B, K, E, H, I;
    int nwaves;              // logical waves in the grid
    int nrowblk;             // row blocks (I / R for gate/up, H / R for down)
    int order;               // 1: row-block major, 2: token/slot major
    int remap;               // 1: XCD-contiguous workgroup numbering
    uint32_t nci_magic;      // down: floor(2^22 / (I/16)) + 1; (c * magic) >> 22 == c / (I/16) for all chunks c
    int tsplit;              // down, matrix-core form: workgroups per 16-output block, each for its own tokens
    int nblocks;             // workgroups in the grid
    int wpb;                 // waves per workgroup
    int esplit;              // down, matrix-core form: workgroups per 16-output block, each for one class of experts
    uint64_t *dcell;         // down, expert split: one cell per output [H/16][B][16], zero between calls
    uint4 *zero_ptr;         // gate/up: 16-byte words the workgroups set to zero first (or null)
    int zero_n;
};

// The workgroups clear zero_n 16-byte words at zero_ptr, each its own share
// (the down kernel's expert-split cells, when both kernels run as one layer:
// the down kernel, launched after this one on the same stream, finds them
// zero).
__device__ __forceinline__ void zero_words(const LayerArgs &a) {
    if (a.zero_n > 0) {
        const uint4 z = {0u, 0u, 0u, 0u};
        for (int i = (int)(blockIdx.x * blockDim.x + threadIdx.x); i < a.zero_n; i += a.nblocks * (int)blockDim.x)
            a.zero_ptr[i] = z;
    }
}

// Makes the compiler load the kernel arguments a wave needs first in one
// batch at the start (an empty asm that takes them as scalar operands), so
// that they arrive with one wait instead of several sequential ones spread
// over the wave's opening instructions.
__device__ __forceinline__ void args_early(const LayerArgs &a) {
    asm volatile("" ::"s"(a.ids), "s"(a.w), "s"(a.s), "s"(a.B), "s"(a.K), "s"(a.H), "s"(a.I), "s"(a.nwaves),
                 "s"(a.nrowblk), "s"(a.order), "s"(a.remap), "s"(a.nblocks), "s"(a.wpb));
}

// (expert e, row block jb) of unit u of the expert forms of gate/up.
//   order 1: row-block major with a skew, u = i * E + e, jb = (i + e) % nrowblk:
//            with XCD-contiguous numbering every XCD gets the same share of
//            every expert's rows, whichever experts the batch routes to, and
//            the waves resident together read different row offsets of their
//            experts (expert regions are a power-of-two multiple apart, and
//            equal offsets would load the same memory channels);
//   order 2: expert major, u = e * nrowblk + jb;
//   order 3: row-block major without the skew, u = jb * E + e.
__device__ __forceinline__ void expert_unit(const LayerArgs &a, int u, int &e, int &jb) {
    if (a.order == 2) {
        e = u / a.nrowblk; jb = u - e * a.nrowblk;
    } else {
        const int i = u / a.E;
        e = u - i * a.E;
        jb = a.order == 1 ? (i + e) % a.nrowblk : i;
    }
}

// Logical wave index of the calling wave (wave-uniform, kept in an SGPR).
// The grid and workgroup sizes come from the kernel's own arguments, loaded
// with the rest of them, rather than from the dispatch's hidden arguments,
// which would put two more dependent scalar loads ahead of a wave's first
// weight load.
__device__ __forceinline__ int logical_wave(const LayerArgs &a) {
    const int g = a.remap == 1 ? xcd_logical((int)blockIdx.x, a.nblocks) : (int)blockIdx.x;
    return __builtin_amdgcn_readfirstlane(g * a.wpb + (int)(threadIdx.x >> 6));
}

// Leading scalar arguments of the kernels launched with LayerArgs: the values a wave needs to
// find its place in the grid and to address its first routing-id load, ahead of the LayerArgs
// block (which repeats them).  The library is built with kernel-argument preloading, so the
// dispatch puts these in SGPRs before the wave starts and the id load goes out at once, instead
// of after a scalar load of the argument block (about 0.2 us per launch of a one-token layer).
#define WD_LEAD_PARAMS                                                                              \
    const int32_t *__restrict__ l_ids, int l_nwaves, int l_nblocks, int l_wpb, int l_remap, int l_order, \
        int l_B, int l_K, int l_nrowblk, uint32_t l_nci_magic, int l_I

// logical_wave from the leading arguments
__device__ __forceinline__ int lead_wave(int remap, int nblocks, int wpb) {
    const int g = remap == 1 ? xcd_logical((int)blockIdx.x, nblocks) : (int)blockIdx.x;
    return __builtin_amdgcn_readfirstlane(g * wpb + (int)(threadIdx.x >> 6));
}

// ---------------------------------------------------------------------------
// Gate/up: one wave per (token b, slot k, block of G * R intermediate rows).
//
// The wave is cut into G = 64 / LPR groups of LPR lanes; each group owns one
// row at a time (R rows in turn), so the wave works on G rows at once and
// their cross-lane reductions run side by side in the same instructions.
// Lane t of a group owns the 16-element chunks c = t + LPR * i (i < CPL) of
// the H axis: each 16-byte code load instruction covers G contiguous
// LPR * 16-byte row segments.  x[b] is loaded once per wave and reused by the
// gate and the up row of every row the lane touches.  MATH selects the
// arithmetic: kMathF32 converts each MXFP8 pair to FP32 and accumulates with
// FMAs; kMathDot2 converts it to a BF16 pair (also exact) and accumulates two
// products per v_dot2_f32_bf16 into FP32, using x as stored.  TAIL handles
// H / 16 not a multiple of LPR * CPL (lanes past the row end add nothing).
// NT loads the weights non-temporally (for batches where no other wave reads
// the same rows).  The row handled by group g at step r is
// j = jb * G * R + r * G + g.
// ---------------------------------------------------------------------------
template <int CPL, int R, int LPR, bool TAIL, int MATH, bool NT>
__global__ __launch_bounds__(256) void gate_up_kernel(WD_LEAD_PARAMS, LayerArgs a) {
    constexpr int G = 64 / LPR;
    const int lane = threadIdx.x & 63;
    const int grp = lane / LPR, tl = lane % LPR;
    const int t = lead_wave(l_remap, l_nblocks, l_wpb);
    if (t >= l_nwaves) {                             // wave-uniform exit
        zero_words(a);
        return;
    }

    int b, k, jb;
    if (l_order == 1) {                              // t = (jb * B + b) * K + k
        k = t % l_K; const int r = t / l_K; b = r % l_B; jb = r / l_B;
    } else {                                         // t = (b * K + k) * nrowblk + jb
        jb = t % l_nrowblk; const int r = t / l_nrowblk; k = r % l_K; b = r / l_K;
    }
    int e = sload(l_ids + b * l_K + k);              // (b, k) is wave-uniform
    args_early(a);
    const int H = a.H, I = a.I;
    const int NC = H >> 4;                           // chunks per row
    const bool bad = (unsigned)e >= (unsigned)a.E;   // never read out of bounds for a bad id
    if (bad) e = 0;

    // x[b] in registers, chunk by chunk: FP32 (MATH == kMathF32) or the stored
    // BF16 pairs (kMathDot2).
    float xv[MATH == kMathF32 ? CPL : 1][16];
    u32x4 xp0[CPL], xp1[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = tl + LPR * i;
        const int cc = (!TAIL || c < NC) ? c : 0;
        const uint16_t *xp = a.x + (size_t)b * H + cc * 16;
        xp0[i] = ld16(xp);
        xp1[i] = ld16(xp + 8);
        if constexpr (MATH == kMathF32) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xv[i][2 * q] = bf16_lo(xp0[i][q]);
                xv[i][2 * q + 1] = bf16_hi(xp0[i][q]);
                xv[i][8 + 2 * q] = bf16_lo(xp1[i][q]);
                xv[i][8 + 2 * q + 1] = bf16_hi(xp1[i][q]);
            }
        }
    }

    const size_t nbr = (size_t)(H >> 5);             // scale bytes per row
    const size_t erow = (size_t)e * 2 * I;           // first row of expert e
    const int jbase = jb * (G * R) + grp;
    float res[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int j = jbase + r * G;
        const uint8_t *wg = a.w + (erow + j) * (size_t)H;
        const uint8_t *wu = wg + (size_t)I * H;
        const uint8_t *sg = a.s + (erow + j) * nbr;
        const uint8_t *su = sg + (size_t)I * nbr;
        // the row's loads, all issued before the first is used (the compiler would otherwise
        // wait for each chunk's before issuing the next)
        u32x4 qg[CPL], qu[CPL];
        uint8_t bg[CPL], bu[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = tl + LPR * i;
            const int cc = (!TAIL || c < NC) ? c : 0;
            qg[i] = ldw<NT>(wg + cc * 16);
            qu[i] = ldw<NT>(wu + cc * 16);
            bg[i] = sg[cc >> 1];
            bu[i] = su[cc >> 1];
        }
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const bool ok = !TAIL || tl + LPR * i < NC;
            const float fg = e8m0_operand(bg[i]);
            const float fu = e8m0_operand(bu[i]);
            float g2, u2;
            if constexpr (MATH == kMathF32) {
                g2 = dot16_f32(qg[i], fg, xv[i], g);
                u2 = dot16_f32(qu[i], fu, xv[i], u);
            } else {
                g2 = dot16_dot2(qg[i], fg, xp0[i], xp1[i], g);
                u2 = dot16_dot2(qu[i], fu, xp0[i], xp1[i], u);
            }
            g = ok ? g2 : g;                         // lanes past the row end add nothing
            u = ok ? u2 : u;
        }
        g = group_sum<LPR>(g);
        u = group_sum<LPR>(u);
        // SiLU(g) * u in FP32; sigmoid written so that exp never overflows.
        const float en = expf(-__builtin_fabsf(g));
        const float sig = g >= 0.f ? 1.f / (1.f + en) : en / (1.f + en);
        res[r] = bad ? __builtin_nanf("") : g * sig * u;
    }
    // lane t < R of group g stores the group's row of step t
    float mine = res[0];
#pragma unroll
    for (int r = 1; r < R; ++r) mine = tl == r ? res[r] : mine;
    if (tl < R)
        a.out[((size_t)b * a.K + k) * I + (size_t)(jbase + tl * G)] = to_bf16(mine);
    zero_words(a);                                   // last: its branch would split the loads' schedule
}

// ---------------------------------------------------------------------------
// Gate/up, expert form: one wave per (expert e, block of R rows), serving every
// (token, slot) routed to e.
//
// For batches in which tokens share experts, the token form above reads each
// routed expert row once per (token, slot) that uses it.  Here the wave first
// finds, with a ballot over topk_ids, the slots routed to its expert (no
// index buffer and no extra kernel), loads and converts its R gate rows and R
// up rows once, then walks those slots: for each it loads x[b] (the next
// slot's x is fetched while the current one is computed), forms the R gate and
// up dot products against the registers, reduces them across the wave and
// writes act[b,k,rows].  Each lane keeps the chunk layout of the token form
// with 64 lanes per row (chunk c = lane + 64 i, BF16 pairs through
// v_dot2_f32_bf16), so every act value is bit-identical to that form's.
// Waves whose expert no token uses exit after the ballot.  Slots with an id
// outside [0, E) get NaN rows from the waves of expert 0.
// Wave t handles (expert t % E, row block t / E) in row-block-major order
// (order 1), else (expert t / nrowblk, row block t % nrowblk).
// ---------------------------------------------------------------------------
template <int CPL, int R, bool TAIL>
__global__ __launch_bounds__(256) void gate_up_expert_kernel(WD_LEAD_PARAMS, LayerArgs a) {
    zero_words(a);
    const int lane = threadIdx.x & 63;
    const int t = lead_wave(l_remap, l_nblocks, l_wpb);
    if (t >= l_nwaves) return;
    int e, jb;
    expert_unit(a, t, e, jb);
    const int BK = a.B * a.K, H = a.H, I = a.I, NC = H >> 4;

    // which slots use this expert (and, for expert 0, which ids are invalid)
    uint64_t any = 0, bad_any = 0;
    for (int base = 0; base < BK; base += 64) {
        const int sl = base + lane;
        const int id = sl < BK ? a.ids[sl] : 0;
        any |= __builtin_amdgcn_ballot_w64(sl < BK && id == e);
        bad_any |= __builtin_amdgcn_ballot_w64(e == 0 && sl < BK && (unsigned)id >= (unsigned)a.E);
    }
    if (bad_any) {
        for (int base = 0; base < BK; base += 64) {
            const int sl = base + lane;
            const int id = sl < BK ? a.ids[sl] : 0;
            uint64_t m = __builtin_amdgcn_ballot_w64(sl < BK && (unsigned)id >= (unsigned)a.E);
            while (m) {
                const int s0 = base + (int)__builtin_ctzll(m);
                m &= m - 1;
                if (lane < R) a.out[(size_t)s0 * I + (size_t)jb * R + lane] = 0x7FC0;   // BF16 quiet NaN
            }
        }
    }
    if (!any) return;

    // the wave's R gate rows and R up rows, converted once to BF16 pairs
    const size_t nbr = (size_t)(H >> 5);
    const size_t erow = (size_t)e * 2 * I + (size_t)jb * R;
    uint32_t wg[R][CPL][8], wu[R][CPL][8];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint8_t *pg = a.w + (erow + r) * (size_t)H;
        const uint8_t *pu = pg + (size_t)I * H;
        const uint8_t *sg = a.s + (erow + r) * nbr;
        const uint8_t *su = sg + (size_t)I * nbr;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            const int cc = (!TAIL || c < NC) ? c : 0;
            const u32x4 qg = ld16(pg + cc * 16), qu = ld16(pu + cc * 16);
            const float fg = e8m0_operand(sg[cc >> 1]), fu = e8m0_operand(su[cc >> 1]);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                mx_word_bf16(qg[d], fg, wg[r][i][2 * d], wg[r][i][2 * d + 1]);
                mx_word_bf16(qu[d], fu, wu[r][i][2 * d], wu[r][i][2 * d + 1]);
            }
        }
    }

    // walk the slots routed to e, in slot order
    int base = 0;
    uint64_t m = 0;
    auto next_slot = [&]() -> int {
        while (m == 0) {
            if (base >= BK) return -1;
            const int sl = base + lane;
            const int id = sl < BK ? a.ids[sl] : 0;
            m = __builtin_amdgcn_ballot_w64(sl < BK && id == e);
            base += 64;
        }
        const int s0 = base - 64 + (int)__builtin_ctzll(m);
        m &= m - 1;
        return s0;
    };
    auto load_x = [&](int sl, u32x4 *x0, u32x4 *x1) {
        const uint16_t *xb = a.x + (size_t)(sl / a.K) * H;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            const int cc = (!TAIL || c < NC) ? c : 0;
            x0[i] = ld16(xb + cc * 16);
            x1[i] = ld16(xb + cc * 16 + 8);
        }
    };
    int cur = next_slot();
    u32x4 xa0[CPL], xa1[CPL];
    load_x(cur, xa0, xa1);
    while (cur >= 0) {
        const int nxt = next_slot();
        u32x4 xn0[CPL], xn1[CPL];
        if (nxt >= 0) load_x(nxt, xn0, xn1);
        float res[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float g = 0.f, u = 0.f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const bool ok = !TAIL || lane + 64 * i < NC;
                const float g2 = dot16_pre(wg[r][i], xa0[i], xa1[i], g);
                const float u2 = dot16_pre(wu[r][i], xa0[i], xa1[i], u);
                g = ok ? g2 : g;
                u = ok ? u2 : u;
            }
            g = wave_sum(g);
            u = wave_sum(u);
            const float en = expf(-__builtin_fabsf(g));
            const float sig = g >= 0.f ? 1.f / (1.f + en) : en / (1.f + en);
            res[r] = g * sig * u;
        }
        float mine = res[0];
#pragma unroll
        for (int r = 1; r < R; ++r) mine = lane == r ? res[r] : mine;
        if (lane < R) a.out[(size_t)cur * I + (size_t)jb * R + lane] = to_bf16(mine);
        if (nxt >= 0) {
#pragma unroll
            for (int i = 0; i < CPL; ++i) { xa0[i] = xn0[i]; xa1[i] = xn1[i]; }
        }
        cur = nxt;
    }
}

// ---------------------------------------------------------------------------
// Gate/up, expert form on the matrix cores: one wave per (expert e, block of 16
// intermediate rows j0 .. j0+15), serving the slots routed to e in groups of up
// to 16.  The wave issues its first weight loads before it reads topk_ids (they
// do not depend on the routing), scans the ids 512 slots at a time with
// independent loads, and keeps one batch of weight loads in flight ahead of
// the batch it computes.
//
// For a group of T slots the wave forms the 16 x T tiles G = Wg[e, j0:j0+16, :] X
// and U = Wu[e, j0:j0+16, :] X, whose columns are the x rows of the group's
// tokens, with v_mfma_f32_16x16x32_bf16: the weights are converted MXFP8 ->
// BF16 in registers (exact for every normal product), x is used as stored
// (BF16) and the matrix core accumulates the products in FP32 (measured on
// MI355X to within a few 2^-24 of the sum of |products|, like sequential FP32
// addition).  Operand layout: lane l holds weight row l % 16 (A) and the
// group's column l % 16 (B), elements 8 (l / 16) + 0..7 of the instruction's
// 32.  One 16-byte code load per lane and row covers elements
// 64 s + 16 (l / 16) + 0..15 of step s and feeds two instructions (first 8,
// last 8); x is loaded with the same mapping, so each product pairs the weight
// and the x element of the same h.  The result lane l holds column l % 16,
// rows 4 (l / 16) + 0..3: SiLU(g) * u in FP32, rounded to BF16, one 8-byte
// store per lane.  The slots are found by a ballot over topk_ids as in the
// expert form above; slots with an id outside [0, E) get NaN rows from expert
// 0's waves.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaSteps = 4;    // 64-element steps whose loads are issued together

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

struct MfmaBatch {                      // one wave's loads for kMfmaSteps 64-element steps
    u32x4 v[8];                         // codes, coalesced: instruction j holds 4 rows x 256 B
    uint64_t sg, su;                    // the lane's row's 2 * kMfmaSteps E8M0 bytes of these steps
};
static_assert(kMfmaSteps == 4, "one 8-byte scale load and 256 bytes per row cover a batch");

template <bool SC8, int NGMAX, int HS>
__global__ __launch_bounds__(256) void gate_up_mfma_kernel(WD_LEAD_PARAMS, LayerArgs a) {
    static_assert(HS == 1 || HS == 2, "one wave per unit, or a pair splitting H");
    constexpr int kWpb = HS == 2 ? 2 : 4;             // waves per workgroup
    // per wave: the batch's 16 gate and 16 up rows x 256 bytes, 16-byte slots XOR-swizzled by row,
    // and each lane's E8M0 bytes of the batch (kept in LDS: a register copy of the prefetched
    // bytes would make the compute wait for the whole prefetch)
    __shared__ u32x4 tile[kWpb][2][16][16];
    __shared__ uint64_t stile[kWpb][2][64];
    __shared__ f32x4 xch[HS == 2 ? NGMAX : 1][2][64];  // HS 2: the second wave's sums for the first
    const int lane = threadIdx.x & 63;
    const int lw = lead_wave(l_remap, l_nblocks, l_wpb);
    if (lw >= l_nwaves) {                             // with HS 2, nwaves is even: pairs exit together
        zero_words(a);
        return;
    }
    // HS 2: the two waves of a workgroup serve one unit, each over its half of the H axis (an
    // equal number of whole 256-element batches); the second hands its FP32 sums to the first,
    // which adds them to its own (first half + second half) and writes the results
    const int unit = HS == 2 ? lw >> 1 : lw;
    const int half = HS == 2 ? lw & 1 : 0;
    int e, jb;
    expert_unit(a, unit, e, jb);
    const int BK = a.B * a.K, H = a.H, I = a.I;
    const int r16 = lane & 15, q = lane >> 4;
    u32x4(*wt)[16][16] = tile[threadIdx.x >> 6];

    const size_t nbr = (size_t)(H >> 5);
    const size_t grow = (size_t)e * 2 * I + (size_t)jb * 16 + r16;
    const uint8_t *sg = a.s + grow * nbr;
    const uint8_t *su = sg + (size_t)I * nbr;
    const int s_all = (H + 63) >> 6;                  // 64-element steps of a row
    const int s_lo = half * (s_all / HS), s_hi = HS == 2 && half == 0 ? s_all / 2 : s_all;
    const u32x4 zero = {0u, 0u, 0u, 0u};

    // Weight and scale loads are unconditional (offsets past H are clamped; the selects
    // in the compute step zero what they brought) and every batch issues the same loads,
    // so no branch separates them and each wait counts exactly the loads it needs.
    // The E8M0 bytes of a batch (blocks 2 s0 .. 2 s0 + 7 of the lane's row) come in
    // one 8-byte load when every batch's window lies inside its row (SC8: H a multiple
    // of 256, so a row holds a multiple of 8 bytes, and the scale array 4-byte aligned),
    // else byte by byte (a last batch of fewer than 4 steps ends past the row).
    // Codes come coalesced: instruction j reads rows 4 (j % 4) + l / 16 of the gate
    // (j < 4) or up (j >= 4) block, 16 bytes per lane, the 16 lanes of a row covering its
    // 256 bytes of the batch in slot order p = l % 16 holding segment p ^ row (the swizzle
    // that makes the operand-layout reads from LDS conflict-free).
    const uint8_t *pg0 = a.w + ((size_t)e * 2 * I + (size_t)jb * 16) * (size_t)H;
    const uint8_t *pu0 = pg0 + (size_t)I * H;
    const int wrow = lane >> 4, wslot = lane & 15;
    // an in-bounds address in x (at least 64 bytes) for the code loads whose data is not used
    const uint8_t *xdum = reinterpret_cast<const uint8_t *>(a.x) + 16 * (lane & 3);
    auto load_batch = [&](int s0, MfmaBatch &bt, bool dummy) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 4 * (j & 3) + wrow;
            const int k = 64 * s0 + 16 * (wslot ^ r);
            const uint8_t *base = (j < 4 ? pg0 : pu0) + (size_t)r * H;
            // non-temporal: a pass reads the rows once, and keeping them out of the way leaves the
            // caches to the routing ids and x, which every wave reads (bit-identical; B = 32
            // 69.6 -> 67.9 us; an expert with more than a pass's slots reads its rows again in
            // the next pass, from memory, and is still faster so)
            bt.v[j] = ldw<true>(dummy ? xdum : base + (k < H ? k : 0));   // past H: clamped, zeroed when read
        }
        if constexpr (SC8) {
            const int o = 2 * s0 + 8 <= (int)nbr ? 2 * s0 : 0;   // always 2 s0 for H % 256 == 0
            bt.sg = *reinterpret_cast<const uint64_t *>(sg + o);
            bt.su = *reinterpret_cast<const uint64_t *>(su + o);
        } else {
            bt.sg = 0;
            bt.su = 0;
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const int o = 2 * s0 + b < (int)nbr ? 2 * s0 + b : 0;
                bt.sg |= (uint64_t)sg[o] << (8 * b);
                bt.su |= (uint64_t)su[o] << (8 * b);
            }
        }
    };
    MfmaBatch cur;

    // Slots routed to e, found 512 at a time: eight independent id loads, then ballots.
    uint64_t mk[8];
    int chunk = 0, next_chunk = 0;
    const int lBK = l_B * l_K;
    auto refill = [&]() {
        int idv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int sl = next_chunk + 64 * u + lane;
            idv[u] = sl < lBK ? l_ids[sl] : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) mk[u] = __builtin_amdgcn_ballot_w64(idv[u] == e);
        chunk = next_chunk;
        next_chunk += 512;
    };
    refill();
    zero_words(a);
    if (e == 0 && half == 0) {   // NaN rows for slots whose id is outside [0, E)
        for (int base = 0; base < BK; base += 64) {
            const int sl = base + lane;
            const int id = sl < BK ? a.ids[sl] : 0;
            uint64_t m = __builtin_amdgcn_ballot_w64(sl < BK && (unsigned)id >= (unsigned)a.E);
            while (m) {
                const int s0 = base + (int)__builtin_ctzll(m);
                m &= m - 1;
                if (lane < 16) a.out[(size_t)s0 * I + (size_t)jb * 16 + lane] = 0x7FC0;
            }
        }
    }
    // The first batch only once the routing shows a slot for e (or the ids need more than one
    // scan): a wave whose expert no slot uses reads no weights.
    {
        uint64_t any = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) any |= mk[u];
        if (any == 0 && next_chunk >= BK) return;
    }
    load_batch(s_lo, cur, false);

    // One pass per up to 16 * NGMAX slots routed to e: the weight batches stream once per
    // pass and feed one 16-slot tile, or with NGMAX 2 two when more than 16 slots remain (the
    // second tile's columns are slots 16..31 of the pass), so an expert with up to 32 slots is
    // read once; NGMAX 1 streams an expert with more than 16 slots once per 16 (from the L2
    // when it still holds them) but needs fewer registers.  A (row, slot) sum is the same
    // sequence of matrix instructions in every case.
    constexpr int kPass = 16 * NGMAX;
    auto pass = [&](auto ng_c, int my_slot, int cnt) {
        constexpr int NG = decltype(ng_c)::value;
        int slot[NG];
        bool live[NG];
        const uint16_t *xr[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            slot[g] = __shfl(my_slot, 16 * g + r16);
            live[g] = 16 * g + r16 < cnt;
            // lanes of empty columns read column 0's token (their products are never stored)
            const int slot_any = live[g] ? slot[g] : __shfl(my_slot, 0);
            xr[g] = a.x + (size_t)(slot_any / a.K) * H;
        }
        f32x4 cg[NG], cu[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) cg[g] = cu[g] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s0 = s_lo; s0 < s_hi; s0 += kMfmaSteps) {
            // the batch's codes into the wave's LDS tile (LDS operations of one wave complete
            // in order, so the previous batch's reads are done)
#pragma unroll
            for (int j = 0; j < 8; ++j) wt[j >> 2][4 * (j & 3) + wrow][wslot] = cur.v[j];
            stile[threadIdx.x >> 6][0][lane] = cur.sg;        // this batch's scale bytes
            stile[threadIdx.x >> 6][1][lane] = cur.su;
            // keep the prefetch below after these reads of cur, so it can reuse cur's registers
            __builtin_amdgcn_sched_barrier(0);
            u32x4 x0[NG][kMfmaSteps], x1[NG][kMfmaSteps];
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int i = 0; i < kMfmaSteps; ++i) {
                    const int k = 64 * (s0 + i) + 16 * q;
                    const int kc = (s0 + i < s_hi && k < H) ? k : 64 * s_lo;
                    x0[g][i] = ld16(xr[g] + kc);
                    x1[g][i] = ld16(xr[g] + kc + 8);
                }
            // prefetch into the same registers (their codes are in LDS now): the next batch, this
            // wave's first batch again for a further pass, or else loads whose data is not used
            // (the codes from x, which the caches hold, the scale bytes this batch's again), so
            // that every batch issues the same loads and each wait counts exactly
            const bool more = s0 + kMfmaSteps < s_hi;
            load_batch(more ? s0 + kMfmaSteps : cnt == kPass ? s_lo : s0, cur, !more && cnt != kPass);
#pragma unroll
            for (int i = 0; i < kMfmaSteps; ++i) {
                const int k = 64 * (s0 + i) + 16 * q;
                const bool ok = s0 + i < s_hi && k < H;
                const int sh = 8 * (2 * i + (q >> 1));      // byte of block 2 (s0 + i) + q / 2
                const uint64_t sgb = stile[threadIdx.x >> 6][0][lane], sub = stile[threadIdx.x >> 6][1][lane];
                const uint32_t bg = (uint32_t)(sgb >> sh) & 0xFFu, bu = (uint32_t)(sub >> sh) & 0xFFu;
                const float fg = e8m0_operand(ok ? bg : 127u), fu = e8m0_operand(ok ? bu : 127u);
                const int sl = (4 * i + q) ^ r16;           // segment 4 i + q of row r16
                const u32x4 wgi = ok ? wt[0][r16][sl] : zero, wui = ok ? wt[1][r16][sl] : zero;
                uint32_t gw[8], uw[8];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    mx_word_bf16(wgi[d], fg, gw[2 * d], gw[2 * d + 1]);
                    mx_word_bf16(wui[d], fu, uw[2 * d], uw[2 * d + 1]);
                }
                const u32x4 g0 = {gw[0], gw[1], gw[2], gw[3]}, g1 = {gw[4], gw[5], gw[6], gw[7]};
                const u32x4 u0 = {uw[0], uw[1], uw[2], uw[3]}, u1 = {uw[4], uw[5], uw[6], uw[7]};
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const bool xo = ok && live[g];
                    const u32x4 xa = xo ? x0[g][i] : zero, xb = xo ? x1[g][i] : zero;
                    cg[g] = mfma_bf16(g0, xa, cg[g]);
                    cg[g] = mfma_bf16(g1, xb, cg[g]);
                    cu[g] = mfma_bf16(u0, xa, cu[g]);
                    cu[g] = mfma_bf16(u1, xb, cu[g]);
                }
            }
        }
        if constexpr (HS == 2) {
            // the pair's sums: the second wave's go through LDS, the first adds them to its own
            if (half == 1) {
#pragma unroll
                for (int g = 0; g < NG; ++g) { xch[g][0][lane] = cg[g]; xch[g][1][lane] = cu[g]; }
            }
            __syncthreads();
            if (half == 0) {
#pragma unroll
                for (int g = 0; g < NG; ++g) { cg[g] += xch[g][0][lane]; cu[g] += xch[g][1][lane]; }
            }
            __syncthreads();                          // xch free for the next pass
            if (half == 1) return;
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if (!live[g]) continue;
            uint32_t packed[2];
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                uint32_t h2 = 0;
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const float gv = cg[g][r + d], uv = cu[g][r + d];
                    const float en = expf(-__builtin_fabsf(gv));
                    const float sig = gv >= 0.f ? 1.f / (1.f + en) : en / (1.f + en);
                    h2 |= (uint32_t)to_bf16(gv * sig * uv) << (16 * d);
                }
                packed[r >> 1] = h2;
            }
            *reinterpret_cast<uint2 *>(a.out + (size_t)slot[g] * I + (size_t)jb * 16 + 4 * q) =
                make_uint2(packed[0], packed[1]);
        }
    };

    for (;;) {
        // the next up-to-kPass slots routed to e, in slot order, one per lane 0..kPass-1
        int my_slot = 0, cnt = 0;
        for (;;) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                while (mk[u] != 0 && cnt < kPass) {
                    const int s0 = chunk + 64 * u + (int)__builtin_ctzll(mk[u]);
                    mk[u] &= mk[u] - 1;
                    if (lane == cnt) my_slot = s0;
                    ++cnt;
                }
            }
            if (cnt == kPass || next_chunk >= BK) break;
            refill();
        }
        if (cnt == 0) break;
        if constexpr (NGMAX == 2) {
            if (cnt > 16)
                pass(std::integral_constant<int, 2>{}, my_slot, cnt);
            else
                pass(std::integral_constant<int, 1>{}, my_slot, cnt);
        } else {
            pass(std::integral_constant<int, 1>{}, my_slot, cnt);
        }
        if (cnt < kPass) break;
    }
}

// ---------------------------------------------------------------------------
// Gate/up, expert form on the matrix cores, weight codes streamed straight
// into LDS (form 4; rows of a multiple of 256 elements).  The work and the
// arithmetic are those of gate_up_mfma_kernel above -- one wave per (expert
// e, block of 16 intermediate rows), the 16 x T gate and up tiles of each
// group of T <= 16 slots on v_mfma_f32_16x16x32_bf16, weights converted
// exactly to BF16, x as stored, FP32 accumulation in the same order -- so
// the intermediate is bit-identical to that kernel's.  What differs is how
// the bytes arrive:
//   * the codes of a batch (2 steps of 64 elements: 16 gate and 16 up rows x
//     128 bytes) go from memory to the wave's LDS ring by buffer-to-LDS loads
//     (no register staging and no LDS stores), two batches ahead: a ring of
//     two slots, the load of batch n + 2 issued into the slot of batch n as
//     soon as n's operands are read from it;
//   * x and the rows' E8M0 bytes come by buffer loads one batch ahead, into
//     one of two register sets; the columns past the group's slots get an
//     offset past the end of x, so their loads return zero without touching
//     memory;
//   * every address offset is loop-invariant except a wave-uniform batch
//     offset, so a batch costs its loads, 4 LDS reads, 32 conversions and 8
//     matrix instructions.
// Each 16-byte segment s of row r sits in slot s ^ ((r >> 1) & 7) of the
// row's 8 LDS slots, so the operand reads (16 rows, one segment each) hit
// distinct banks.  When a group holds 16 slots (another may follow), its
// last batches load the rows' first two batches into the ring for the next
// group of the same expert; otherwise nothing is loaded past the rows' end.
// Waves drain their loads before exiting.
// ---------------------------------------------------------------------------
template <int WPB>
__global__ __launch_bounds__(64 * WPB) void gate_up_mfma_lds_kernel(WD_LEAD_PARAMS, LayerArgs a) {
    constexpr int kSeg = 8;                                // 16-byte segments per row per batch
    __shared__ u32x4 ring0[WPB][2][16][kSeg];              // slot 0: [wave][gate, up][row][slot]
    __shared__ u32x4 ring1[WPB][2][16][kSeg];              // slot 1
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int unit = lead_wave(l_remap, l_nblocks, l_wpb);
    if (unit >= l_nwaves) {                                // wave-uniform, before any load
        zero_words(a);
        return;
    }
    int e, jb;
    expert_unit(a, unit, e, jb);
    const int BK = a.B * a.K, H = a.H, I = a.I;
    const int r16 = lane & 15, q = lane >> 4;
    const int nb = H >> 7;                                 // batches per row (even: H % 256 == 0)
    const uint32_t nbr = (uint32_t)(H >> 5);

    // the tile's gate rows start at row0, its up rows at row0 + I (one resource covers both)
    const size_t row0 = (size_t)e * 2 * I + (size_t)jb * 16;
    const rsrc_t rw = make_rsrc(a.w + row0 * (size_t)H, (uint32_t)((I + 16) * H));
    const rsrc_t rs = make_rsrc(a.s + row0 * nbr, (uint32_t)(I + 16) * nbr);
    const rsrc_t rx = make_rsrc(a.x, (uint32_t)((size_t)a.B * H * 2));   // at most 0x7FFF0000 (host check)

    // buffer-to-LDS loads of one batch: instruction j covers rows 8 (j & 1) + l / 8 of the gate
    // (j < 2) or up (j >= 2) tile, lane l bringing segment (l % 8) ^ ((row >> 1) & 7)
    uint32_t doff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 8 * (j & 1) + (lane >> 3);
        const int sg = (lane & 7) ^ ((r >> 1) & 7);
        doff[j] = (uint32_t)(((j >> 1) * I + r) * H + 16 * sg);
    }
    auto issue = [&](u32x4 (*slot)[2][16][kSeg], int n) {
        const uint32_t so = (uint32_t)(128 * n);
#pragma unroll
        for (int j = 0; j < 4; ++j) ld16_lds(rw, &slot[wv][j >> 1][8 * (j & 1)][0], doff[j], so);
    };
    // the first two batches do not depend on the routing
    issue(ring0, 0);
    issue(ring1, 1 % nb);

    // Slots routed to e, found 512 at a time: eight independent id loads, then ballots.
    uint64_t mk[8];
    int chunk = 0, next_chunk = 0;
    const int lBK = l_B * l_K;
    auto refill = [&]() {
        int idv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int sl = next_chunk + 64 * u + lane;
            idv[u] = sl < lBK ? l_ids[sl] : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) mk[u] = __builtin_amdgcn_ballot_w64(idv[u] == e);
        chunk = next_chunk;
        next_chunk += 512;
    };
    refill();
    zero_words(a);
    if (e == 0) {              // NaN rows for slots whose id is outside [0, E)
        for (int base = 0; base < BK; base += 64) {
            const int sl = base + lane;
            const int id = sl < BK ? a.ids[sl] : 0;
            uint64_t m = __builtin_amdgcn_ballot_w64(sl < BK && (unsigned)id >= (unsigned)a.E);
            while (m) {
                const int s0 = base + (int)__builtin_ctzll(m);
                m &= m - 1;
                if (lane < 16) a.out[(size_t)s0 * I + (size_t)jb * 16 + lane] = 0x7FC0;
            }
        }
    }

    // per-lane offsets of the rows' E8M0 bytes (4 per batch) and, per group, of x
    const uint32_t sg_off = (uint32_t)r16 * nbr, su_off = (uint32_t)(I + r16) * nbr;
    struct XSet {
        u32x4 x[4];            // step i: x[2 i] = elements 64 i + 16 q .. + 7, x[2 i + 1] = + 8 .. + 15
        uint32_t sg, su;       // the lane's gate and up row's 4 E8M0 bytes of the batch
    };
    uint32_t xoff = 0;
    auto load_x = [&](XSet &st, int n) {
        const uint32_t so = (uint32_t)(256 * n);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            st.x[2 * i] = buf16(rx, xoff + 128 * i, so);
            st.x[2 * i + 1] = buf16(rx, xoff + 128 * i + 16, so);
        }
        st.sg = buf4(rs, sg_off, (uint32_t)(4 * n));
        st.su = buf4(rs, su_off, (uint32_t)(4 * n));
    };
    f32x4 cg, cu;
    // one batch: the weight operands of its two steps from the ring slot (segment 4 i + q of
    // row r16), then 8 matrix instructions
    auto read_ops = [&](u32x4 (*slot)[2][16][kSeg], u32x4 (&wg)[2], u32x4 (&wu)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int sl = (4 * i + q) ^ ((r16 >> 1) & 7);
            wg[i] = slot[wv][0][r16][sl];
            wu[i] = slot[wv][1][r16][sl];
        }
    };
    auto mma = [&](const XSet &st, const u32x4 (&wg)[2], const u32x4 (&wu)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int sh = 8 * (2 * i + (q >> 1));         // byte of block 4 n + 2 i + q / 2
            const float fg = e8m0_operand((st.sg >> sh) & 0xFFu), fu = e8m0_operand((st.su >> sh) & 0xFFu);
            uint32_t gw[8], uw[8];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                mx_word_bf16(wg[i][d], fg, gw[2 * d], gw[2 * d + 1]);
                mx_word_bf16(wu[i][d], fu, uw[2 * d], uw[2 * d + 1]);
            }
            const u32x4 g0 = {gw[0], gw[1], gw[2], gw[3]}, g1 = {gw[4], gw[5], gw[6], gw[7]};
            const u32x4 u0 = {uw[0], uw[1], uw[2], uw[3]}, u1 = {uw[4], uw[5], uw[6], uw[7]};
            cg = mfma_bf16(g0, st.x[2 * i], cg);
            cg = mfma_bf16(g1, st.x[2 * i + 1], cg);
            cu = mfma_bf16(u0, st.x[2 * i], cu);
            cu = mfma_bf16(u1, st.x[2 * i + 1], cu);
        }
    };

    XSet sa, sb;
    for (;;) {
        // the next up-to-16 slots routed to e, in slot order, one per lane 0..15
        int my_slot = 0, cnt = 0;
        for (;;) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                while (mk[u] != 0 && cnt < 16) {
                    const int s0 = chunk + 64 * u + (int)__builtin_ctzll(mk[u]);
                    mk[u] &= mk[u] - 1;
                    if (lane == cnt) my_slot = s0;
                    ++cnt;
                }
            }
            if (cnt == 16 || next_chunk >= BK) break;
            refill();
        }
        if (cnt == 0) break;
        const int slot = __shfl(my_slot, r16);
        const bool live = r16 < cnt;
        // columns past the group's slots: an offset past the end of x, so their loads return zero
        xoff = live ? (uint32_t)((slot / a.K) * H * 2 + 32 * q) : 0x7FFF0000u;

        cg = f32x4{0.f, 0.f, 0.f, 0.f};
        cu = cg;
        load_x(sa, 0);
        // nothing in flight when the loop starts: its waits then need only the steady-state counts
        wait_vmcnt<0>();
        // Vector-memory instructions are issued in the order x(n + 1) (6), codes(n + 2) (4),
        // x(n + 2) (6), codes(n + 3) (4) per pair of batches (the waits below are scheduling
        // barriers and keep that order).  So when batch n's codes are read, at least x(n),
        // codes(n + 1) and x(n + 1) -- 16 instructions -- were issued after them, and
        // vmcnt(16) waits for codes(n) and nothing younger (at a group's first batches more
        // was issued since, which only makes the wait exact sooner); batch n's compute then
        // waits for x(n) alone, with codes(n + 1) and (n + 2) still in flight.  Each slot is
        // refilled only after its reads have returned (lgkmcnt(0)).
        const bool more = cnt == 16;                       // another group of this expert may follow
        int n = 0;
        for (; n + 2 < nb; n += 2) {
            u32x4 wg[2], wu[2];
            load_x(sb, n + 1);
            wait_vmcnt<16>();
            read_ops(ring0, wg, wu);
            wait_lgkmcnt0();
            issue(ring0, n + 2);
            mma(sa, wg, wu);
            __builtin_amdgcn_sched_barrier(0);
            load_x(sa, n + 2);
            wait_vmcnt<16>();
            read_ops(ring1, wg, wu);
            wait_lgkmcnt0();
            issue(ring1, n + 3);
            mma(sb, wg, wu);
            __builtin_amdgcn_sched_barrier(0);
        }
        {   // the last two batches (nb is even)
            u32x4 wg[2], wu[2];
            load_x(sb, n + 1);
            wait_vmcnt<16>();
            read_ops(ring0, wg, wu);
            if (more) {
                // the ring takes the rows' first two batches for the next group
                wait_lgkmcnt0();
                issue(ring0, 0);
                mma(sa, wg, wu);
                __builtin_amdgcn_sched_barrier(0);
                load_x(sa, 0);                             // (reloaded with the next group's tokens)
                wait_vmcnt<16>();
                read_ops(ring1, wg, wu);
                wait_lgkmcnt0();
                issue(ring1, 1);
                mma(sb, wg, wu);
            } else {
                // nothing more to load: after codes(n + 1) only x(n + 1) (6) was issued
                mma(sa, wg, wu);
                wait_vmcnt<6>();
                read_ops(ring1, wg, wu);
                mma(sb, wg, wu);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (live) {
            uint32_t packed[2];
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                uint32_t h2 = 0;
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const float gv = cg[r + d], uv = cu[r + d];
                    const float en = expf(-__builtin_fabsf(gv));
                    const float sig = gv >= 0.f ? 1.f / (1.f + en) : en / (1.f + en);
                    h2 |= (uint32_t)to_bf16(gv * sig * uv) << (16 * d);
                }
                packed[r >> 1] = h2;
            }
            *reinterpret_cast<uint2 *>(a.out + (size_t)slot * I + (size_t)jb * 16 + 4 * q) =
                make_uint2(packed[0], packed[1]);
        }
        if (cnt < 16) break;
    }
    // the ring's last loads (never read) land before the wave's LDS is released
    __builtin_amdgcn_s_waitcnt(0);
}

// ---------------------------------------------------------------------------
// Down: one wave per (token b, block of R output dims).
//
// The K routed rows Wd[e_k, h, 0:I] of one output dim are cut into 16-element
// chunks and the K * I / 16 chunks are dealt to the lanes (chunk c = l + 64 i),
// so each lane streams from one or more experts and every lane is busy for
// any I that is a multiple of 32.  Lane-held act chunks (packed BF16) and the
// chunk's router weight are loaded once per wave and reused for all R dims.
// Per chunk the lane forms p = sum deq * act in FP32 and folds the router
// weight in with one FMA, acc += w_k * p.
// ---------------------------------------------------------------------------
template <int CPL, int R, bool TAIL, int MATH, bool NT>
__global__ __launch_bounds__(256) void down_kernel(WD_LEAD_PARAMS, LayerArgs a) {
    const int lane = threadIdx.x & 63;
    const int t = lead_wave(l_remap, l_nblocks, l_wpb);
    if (t >= l_nwaves) return;

    int b, hb;
    if (l_order == 1) { b = t % l_B; hb = t / l_B; }        // t = hb * B + b
    else { hb = t % l_nrowblk; b = t / l_nrowblk; }         // t = b * nrowblk + hb
    const int I = l_I, K = l_K, H = a.H;
    const int NCI = I >> 4;                                  // chunks per expert row
    const int NC = K * NCI;
    const size_t nbr = (size_t)(I >> 5);

    size_t wbase[CPL];      // byte offset of (e_k, h = 0, chunk) in Wd
    size_t sbase[CPL];      // byte offset of its E8M0 byte in Sd
    float wk[CPL];
    u32x4 av0[CPL], av1[CPL];
    bool bad = false;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        const bool ok = !TAIL || c < NC;
        const int cc = ok ? c : 0;
        const int kk = (int)(((uint64_t)cc * l_nci_magic) >> 22);   // cc / NCI (checked on the host)
        const int ci = cc - kk * NCI;
        int e = l_ids[b * K + kk];
        bad |= ok && (unsigned)e >= (unsigned)a.E;
        if ((unsigned)e >= (unsigned)a.E) e = 0;
        wbase[i] = (size_t)e * H * I + (size_t)ci * 16;
        sbase[i] = (size_t)e * H * nbr + (size_t)(ci >> 1);
        wk[i] = a.tw[b * K + kk];
        const uint16_t *ap = a.act_in + ((size_t)b * K + kk) * I + (size_t)ci * 16;
        av0[i] = ld16(ap);
        av1[i] = ld16(ap + 8);
    }

    float res[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const size_t h = (size_t)hb * R + r;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const u32x4 q = ldw<NT>(a.w + wbase[i] + h * I);
            const float f = e8m0_operand(a.s[sbase[i] + h * nbr]);
            const float p = MATH == kMathF32 ? dot16_bf16(q, f, av0[i], av1[i], 0.f)
                                             : dot16_dot2(q, f, av0[i], av1[i], 0.f);
            const float acc2 = __builtin_fmaf(wk[i], p, acc);
            acc = (!TAIL || (lane + 64 * i) < NC) ? acc2 : acc;
        }
        if (bad) acc = __builtin_nanf("");
        res[r] = wave_sum(acc);
    }
    float mine = res[0];
#pragma unroll
    for (int r = 1; r < R; ++r) mine = lane == r ? res[r] : mine;
    if (lane < R) a.out[(size_t)b * H + (size_t)hb * R + lane] = to_bf16(mine);
}

// ---------------------------------------------------------------------------
// Down, expert form on the matrix cores: one workgroup of W waves per block of
// 16 output dims h, serving every token of the batch.
//
// The experts that at least one slot is routed to are handed to the waves
// from a shared counter, experts with more than one group of slots first, so
// a wave that drew a heavy expert takes fewer (with 16 waves, or several token
// ranges, they are dealt in turn instead: the n-th routed expert to wave
// n mod W).  For each of its experts
// a wave forms, G slots at a time (slot order), the tile
// P[h][c] = sum_i Wd[e][h][i] * act[slot c][i] with v_mfma_f32_16x16x32_bf16
// (weight codes converted exactly to BF16, act as stored, FP32 accumulation;
// A = the 16 weight rows, B = the slots' act rows) and keeps each slot's 16
// values in LDS: the expert's dot products are done once for all its slots.
// At the end each output folds its token's router weights in, one FMA per
// slot in expert order (equal experts in slot order),
// y = fma(w_slot, P[h][slot], y), the token form's routing-weight fold, and
// writes out[b][h] = BF16(y).  A token's result depends on its own slots only
// (not on the other tokens, the wave that served an expert, or its top-k
// order).  Each output is owned by one workgroup, or with the expert split
// (esplit 2) by the two workgroups of its block, one per class of experts, that
// meet in one scratch cell per output (one atomic exchange each; see the end of
// the kernel).  Every Wd byte is read once per call, except for an expert used
// by several token ranges.
//
// At the start the workgroup copies its slots' ids and router weights to LDS,
// counts the slots per expert (LDS atomics, one thread per slot) and computes
// each slot's fold rank; every wave then finds each routed expert's place in
// the deal and the start of its run of slot entries (a wave prefix sum of the
// counts, 64 experts per step) and files its experts' slots into their runs.  A wave's
// work is then a sequence of tasks (expert, group of up to
// G slots, batch of 4 64-element steps).  The loads of a task (the 16 rows'
// codes, coalesced as in the matrix-core gate/up; the rows' E8M0 bytes; the
// group's act, coalesced, two slots per instruction) go to one of three
// register sets (two with 16 waves) that many tasks ahead of the compute; a
// task's compute first copies its set into the wave's LDS tiles (codes
// XOR-swizzled by row, act rows padded to start 4 banks apart), refills the
// set, then reads its operands from LDS.  The workgroup's router weights are
// copied to LDS once at the start (a load per slot group, scalar or vector,
// would put a cache round trip in front of every group).  The task state
// is wave-uniform (scalar registers), and every refill issues the same loads
// in one straight block, so each wait names exactly the set it needs.
// With tsplit = S > 1 the batch's tokens are cut into S ranges of
// ceil(B / S) and each 16-output block gets S workgroups, one per range
// (workgroup g: range g / (H / 16), block g % (H / 16)); each output is still
// owned by one workgroup.  An expert used by tokens of several ranges is read
// once per range, from the L2 after the first: with H / 16 a multiple of 8 the
// S workgroups of a block sit on the same XCD.  This fills the CUs that H / 16
// workgroups leave idle.
// Limits per token range: MAXS slots (each slot's 16 products, its id, router
// weight, fold rank and run entry are kept in LDS) and MAXS / 8 tokens; 512
// slots with 16 waves (147 KB of LDS), 512 or 1,024 with 8 (119 or 156 KB).
// E <= 1024.
// ---------------------------------------------------------------------------
constexpr int kDnMfmaMaxB = 64;
constexpr int kDnMfmaMaxSlots = 512;
constexpr int kDnMfmaMaxBWide = 128;                    // the 8-wave variant with room for 1,024 slots
constexpr int kDnMfmaMaxSlotsWide = 1024;
constexpr int kDnMfmaMaxE = 1024;

template <int G>
struct DownSet {
    u32x4 v[4];        // codes: instruction j holds rows 4 j + l / 16, 16-byte slot l % 16 = segment (l % 16) ^ row
    uint64_t sc;       // the E8M0 bytes of the lane's row l % 16 for the batch's 8 blocks
    u32x4 x[G / 2];    // act: instruction j holds group slot 2 j + l / 32, elements 8 (l % 32) .. + 7 of the batch
};

struct DownCursor {    // position in a wave's task sequence
    int x, grp, sb;    // index in the wave's expert list, group of the expert's slots, batch
    int e, start, cnt; // that expert, its first entry in the wave's slot list, its slot count
};

// Leading scalar arguments (preloaded into SGPRs at dispatch, as WD_LEAD_PARAMS): what a
// workgroup needs to find its token range and load the range's ids and router weights.
#define WD_DOWN_LEAD_PARAMS                                                                         \
    const int32_t *__restrict__ l_ids, const float *__restrict__ l_tw, int l_nrowblk, int l_esplit, int l_tsplit, \
        int l_B, int l_K, int l_E

template <int W, int G, bool SC8, int MAXS>
__global__ __launch_bounds__(64 * W) void down_mfma_kernel(WD_DOWN_LEAD_PARAMS, LayerArgs a) {
    static_assert(MAXS == kDnMfmaMaxSlots || (MAXS == kDnMfmaMaxSlotsWide && W == 8), "slot capacity");
    constexpr int kMaxB = MAXS == kDnMfmaMaxSlots ? kDnMfmaMaxB : kDnMfmaMaxBWide;
    constexpr int kXRow = 33;                          // u32x4 per act row in LDS: 256 bf16 + 16 bytes of padding
    constexpr int kMaxExp = (kDnMfmaMaxE + W - 1) / W; // experts one wave can be given
    __shared__ u32x4 tile[W][16][16];                  // per wave: 16 rows x 256 bytes of codes, swizzled
    __shared__ u32x4 xtile[W][G][kXRow];               // per wave: the group's act for the batch
    __shared__ f32x4 pv[MAXS][4];           // per slot - sl0: P[0..15] of its expert's rows
    __shared__ int16_t lslot[MAXS];         // slots of the workgroup's experts, one run per expert
    __shared__ uint32_t lexp[W][kMaxExp];              // per wave: e | first entry << 10 | count << 20
    __shared__ float lw[MAXS];              // router weights of the workgroup's slots, by slot - sl0
    __shared__ int16_t lord[MAXS];          // per token of the range: its slots in fold order
    __shared__ uint16_t lid[MAXS];          // ids of the workgroup's slots, by slot - sl0 (E for bad ones)
    __shared__ uint32_t lcnt[kDnMfmaMaxE];             // slots of the range per expert it serves
    __shared__ uint32_t lcur[kDnMfmaMaxE];             // owning wave << 16 | next free entry of its run
    __shared__ uint8_t loth[kDnMfmaMaxE];              // experts some slot of another range is routed to
    __shared__ uint32_t lq[kDnMfmaMaxE];               // dynamic deal: e | first entry << 10 | count << 20, in deal order
    __shared__ int lnext;                              // dynamic deal: the next expert to hand out
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // wave-uniform: the task state stays scalar
    const int hb = (int)blockIdx.x % l_nrowblk;
    const int rg = (int)blockIdx.x / l_nrowblk;
    const int part = rg & (l_esplit - 1);              // expert split: this workgroup's experts are e % esplit == part
    const int tpr = (l_B + l_tsplit - 1) / l_tsplit;   // tokens per range
    const int tb0 = rg / l_esplit * tpr;               // this workgroup's tokens: [tb0, tb1)
    const int tb1 = min(l_B, tb0 + tpr);
    if (tb0 >= tb1) return;                            // workgroup-uniform: a range past the batch
    const int E = l_E, K = l_K;
    const int sl0 = tb0 * K, sl1 = tb1 * K;            // its slots
    const int nsl = sl1 - sl0;
    // the range's ids and router weights, every load issued before anything waits (the leading
    // arguments address them); they go to LDS once the tables below are cleared
    constexpr int kIt = (MAXS + 64 * W - 1) / (64 * W);
    int idr[kIt];
    float twr[kIt];
#pragma unroll
    for (int j = 0; j < kIt; ++j) {
        const int t = (int)threadIdx.x + 64 * W * j;
        idr[j] = t < nsl ? l_ids[sl0 + t] : 0;
        twr[j] = t < nsl ? l_tw[sl0 + t] : 0.f;
    }
    const int H = a.H, I = a.I;
    const int r16 = lane & 15, q = lane >> 4;
    const int wrow = lane >> 4, wslot = lane & 15;
    u32x4(*wt)[16] = tile[wv];
    u32x4(*xt)[kXRow] = xtile[wv];
    const int nbr = I >> 5;
    const int s_hi = (I + 63) >> 6;                    // 64-element steps
    const int s_full = I >> 6;                         // steps with all 64 elements inside the row
    const int nsb = (s_hi + kMfmaSteps - 1) / kMfmaSteps;   // batches per expert
    const u32x4 zero = {0u, 0u, 0u, 0u};

    for (int t = (int)threadIdx.x; t < E; t += 64 * W) {
        lcnt[t] = 0;
        lcur[t] = 0xFFFFFFFFu;
        loth[t] = 0;
    }
    if (threadIdx.x == 0) {
        lnext = W;                                     // experts 0 .. W-1 of the deal go to waves 0 .. W-1
    }
    // the range's ids and router weights into LDS
    {
#pragma unroll
        for (int j = 0; j < kIt; ++j) {
            const int t = (int)threadIdx.x + 64 * W * j;
            if (t < nsl) {
                lid[t] = (uint16_t)((unsigned)idr[j] < (unsigned)E ? (unsigned)idr[j] : (unsigned)E);
                lw[t] = twr[j];
            }
        }
    }
    __syncthreads();                                   // lcnt, lcur, loth cleared; lid, lw written
    for (int t = (int)threadIdx.x; t < nsl; t += 64 * W) {
        // fold order of the slot within its token: by expert, equal experts by slot (ids
        // outside [0, E) last)
        const int tl = t / K, k = t - tl * K;
        const uint16_t *tid = lid + tl * K;
        const unsigned ek = tid[k];
        int rank = 0;
        for (int k2 = 0; k2 < K; ++k2) {
            const unsigned e2 = tid[k2];
            rank += e2 < ek || (e2 == ek && k2 < k);
        }
        // slots whose expert this workgroup does not serve (another class of the expert split, or
        // an id outside [0, E)) are marked and skipped by the fold; an id outside [0, E) also
        // makes its token's outputs NaN
        const bool valid = ek < (unsigned)E;
        const bool mine = valid && (int)(ek & (unsigned)(a.esplit - 1)) == part;
        lord[tl * K + rank] = (int16_t)(k | (mine ? 0 : 0x4000) | (valid ? 0 : 0x2000));
        if (mine) atomicAdd(&lcnt[ek], 1u);           // the range's slots per expert
    }
    if (a.tsplit > 1) {
        const int BK = a.B * K;
        for (int t = (int)threadIdx.x; t < BK; t += 64 * W) {
            const int id = t >= sl0 && t < sl1 ? -1 : a.ids[t];
            if ((unsigned)id < (unsigned)E) loth[id] = 1;
        }
    }
    __syncthreads();                                   // lcnt, loth, lord complete

    // The routed experts this workgroup serves are dealt to the waves in turn (the n-th to wave
    // n % W) in expert order, experts that other token ranges use as well first, then the rest:
    // the workgroups of the other ranges of this output block stream the shared rows at about
    // the same time, so the later reads find them in the L2.  Each expert owns a run of lslot
    // entries, runs in expert order; every wave computes all run starts and keeps its own
    // experts' (e, first entry, count) in lexp and lcur (wave << 16 | first entry), then files
    // its experts' slots into their runs.  (Neither the order of experts nor the order of slots
    // within a run changes a result: each slot's products depend on its own act column only and
    // are kept per slot, and the fold takes them per token in expert order.)
    // With 8 waves and one token range the deal is dynamic: experts with more than one group
    // first, then the rest, each wave taking the next one from a shared counter when it moves on,
    // so a wave given a heavy expert takes fewer, and a wave that streams slower than the others
    // (the memory system serves them unevenly) is not left with a fixed share.  (Which wave
    // serves an expert changes no result.)
    const bool dyn = W < 16 && a.tsplit == 1;   // 16 waves: static
    // The deal order: first the experts of the first kind (dynamic deal: more than one group of
    // slots; several token ranges: used by another range too), then the rest, each kind in expert
    // order.  One pass counts the first kind; a second gives every routed expert its place n in
    // the deal and its run start (runs in expert order, a prefix sum of the counts 64 experts at
    // a time).  n's wave keeps the expert in lcur, and in its own list at n / W (static deal) or
    // in lq at n (dynamic).
    const bool two_kinds = dyn || a.tsplit > 1;
    auto first_kind = [&](int e, int c) { return dyn ? c > G : loth[e] != 0; };
    int nx = 0, nused = 0;
    {
        int n0 = 0;                                    // experts of the first kind
        if (two_kinds)
            for (int base = 0; base < E; base += 64) {
                const int e = base + lane;
                const int c = e < E ? (int)lcnt[e] : 0;
                n0 += __builtin_popcountll(__builtin_amdgcn_ballot_w64(c > 0 && first_kind(e < E ? e : 0, c)));
            }
        int gs = 0, s0 = 0, s1 = 0;                    // entries, and experts of each kind, so far
        for (int base = 0; base < E; base += 64) {
            const int e = base + lane;
            const int c = e < E ? (int)lcnt[e] : 0;
            const bool used = c > 0;
            const bool k0 = two_kinds && used && first_kind(e < E ? e : 0, c);
            const int cu = used ? c : 0;
            const int first = gs + wave_incl_scan(cu) - cu;
            const uint64_t m0 = __builtin_amdgcn_ballot_w64(k0), m1 = __builtin_amdgcn_ballot_w64(used && !k0);
            const int r0 = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m0 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m0, 0u));
            const int r1 = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m1 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m1, 0u));
            const int n = k0 ? s0 + r0 : n0 + s1 + r1;
            if (used && n % W == wv) {
                const uint32_t entry = (uint32_t)e | (uint32_t)first << 10 | (uint32_t)cu << 20;
                lcur[e] = (uint32_t)wv << 16 | (uint32_t)first;
                if (dyn)
                    lq[n] = entry;
                else
                    lexp[wv][n / W] = entry;
            }
            s0 += __builtin_popcountll(m0);
            s1 += __builtin_popcountll(m1);
            gs = __builtin_amdgcn_readlane(first + cu, 63);   // entries of the experts so far
        }
        nused = s0 + s1;
        nx = nused > wv ? (nused - wv + W - 1) / W : 0;    // this wave's experts in the static deal
    }
    if (dyn) nx = INT_MAX;                             // known once the deal runs out
    // The task sequence, compiled twice: with the static deal (each wave's list fixed by the scan)
    // and with the dynamic one, so the loop of each carries only its own bookkeeping.
    auto tasks = [&](auto dyn_c) {
        constexpr bool D = decltype(dyn_c)::value;
        // ---- task sequence ----
        auto set_cursor = [&](DownCursor &cu, uint32_t v) {
            cu.e = (int)(v & 1023u);
            cu.start = (int)((v >> 10) & 1023u);
            cu.cnt = (int)(v >> 20);
        };
        // the compute side reads the wave's list; with the dynamic deal, a ring of the experts the
        // load side (at most three tasks ahead) has taken
        auto fetch = [&](DownCursor &cu) {                 // the expert at list index x
            if (cu.x < nx) set_cursor(cu, (uint32_t)__builtin_amdgcn_readfirstlane((int)lexp[wv][D ? cu.x & 7 : cu.x]));
        };
        auto fetch_ld = [&](DownCursor &cu) {              // the load side: the static list, or the next expert dealt
            if constexpr (!D) {
                fetch(cu);
            } else if (cu.x < nx) {
                int n = wv;
                if (cu.x > 0) {
                    if (lane == 0) n = atomicAdd(&lnext, 1);
                    n = __builtin_amdgcn_readfirstlane(n);
                }
                if (n < nused) {
                    const uint32_t v = (uint32_t)__builtin_amdgcn_readfirstlane((int)lq[n]);
                    if (lane == 0) lexp[wv][cu.x & 7] = v;
                    set_cursor(cu, v);
                } else {
                    nx = cu.x;                             // the deal ran out: the wave's last expert stays named
                }
            }
        };
        auto advance = [&](DownCursor &cu, bool load_side) {
            if (++cu.sb < nsb) return;
            cu.sb = 0;
            if (++cu.grp * G < cu.cnt) return;
            cu.grp = 0;
            ++cu.x;
            if (load_side)
                fetch_ld(cu);
            else
                fetch(cu);
        };

        // per-lane offsets that do not change from task to task
        int coff[4];                                       // code instruction j: row 4 j + l / 16, segment (l % 16) ^ row
    #pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * j + wrow;
            coff[j] = r * I + 16 * (wslot ^ r);
        }
        const int soff = r16 * nbr;                        // the lane's row's E8M0 bytes

        // ---- load side: three tasks ahead ----
        DownCursor ld{0, 0, 0, 0, 0, 0};
        fetch_ld(ld);
        DownCursor cp = ld;
        int xo[G / 2];                                     // act row offset (elements) of instruction j for this lane
    #pragma unroll
        for (int j = 0; j < G / 2; ++j) xo[j] = 0;
        // Every call issues the same loads, in one straight block, so the wait before a set is
        // used counts exactly the younger sets' loads.  Past the end of the sequence the cursor
        // keeps naming the last expert (and expert 0 for a wave with none), so the loads stay
        // in bounds; their data is never used.
        // an in-bounds address in act (at least 64 bytes) for the code loads past the end of the
        // wave's tasks, whose data is not used
        const uint8_t *adum = reinterpret_cast<const uint8_t *>(a.act_in) + 16 * (lane & 3);
        auto issue_w = [&](DownSet<G> &st) {              // the task's weight codes and E8M0 bytes
            const int e = ld.e;
            const int s0 = ld.sb * kMfmaSteps;
            const bool dummy = ld.x >= nx;                 // past the end: keep the loads, not the HBM reads
            const uint8_t *pw = a.w + ((size_t)e * H + (size_t)hb * 16) * (size_t)I + 64 * s0;
            const int lim = I - 64 * s0;                   // bytes of each row left from this batch on
    #pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int seg = 16 * (wslot ^ (4 * j + wrow));
                const uint8_t *p = dummy ? adum : pw + (seg < lim ? coff[j] : coff[j] - seg - 64 * s0);   // past I: the row's start, zeroed when read
                // with one token range non-temporal, as in the matrix-core gate/up (the cached act
                // rows and tables stay); with several, the other ranges' workgroups read the same
                // rows from the L2
                if constexpr (D)
                    st.v[j] = ldw<true>(p);
                else
                    st.v[j] = ld16(p);
            }
            const uint8_t *ps = a.s + ((size_t)e * H + (size_t)hb * 16) * (size_t)nbr + soff;
            if constexpr (SC8) {       // rows of a multiple of 8 E8M0 bytes (I % 256 == 0): one 8-byte load
                st.sc = *reinterpret_cast<const uint64_t *>(ps + (2 * s0 + 8 <= nbr ? 2 * s0 : 0));
            } else {
                st.sc = 0;
    #pragma unroll
                for (int b = 0; b < 8; ++b) st.sc |= (uint64_t)ps[2 * s0 + b < nbr ? 2 * s0 + b : 0] << (8 * b);
            }
        };
        auto rows_x = [&]() {                             // at a new group: this lane's act rows
            if (ld.sb == 0) {
                const int gn = min(G, ld.cnt - ld.grp * G);
                const int base = ld.start + ld.grp * G;
    #pragma unroll
                for (int j = 0; j < G / 2; ++j) {
                    const int col = 2 * j + (lane >> 5);
                    xo[j] = col < gn ? (int)lslot[base + col] * I : 0;
                }
            }
        };
        auto issue_x = [&](DownSet<G> &st) {              // the task's act, then the cursor moves on
            const int kx = 64 * (ld.sb * kMfmaSteps) + 8 * (lane & 31);
            const int kxc = kx < I ? kx : 0;
    #pragma unroll
            for (int j = 0; j < G / 2; ++j) st.x[j] = ld16(a.act_in + xo[j] + kxc);
            advance(ld, true);
        };
        auto issue = [&](DownSet<G> &st) {
            rows_x();
            issue_w(st);
            issue_x(st);
        };

        // ---- compute side ----
        int slot = 0;
        bool live = false;
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
        const int xr = r16 < G ? r16 : 0;
        // One task: its data into the wave's LDS tiles, the set refilled with the task three
        // ahead, then (for a real task) the 4 steps on the matrix cores and, at a group's last
        // batch, the fold.  Past the end of the sequence only the first two run, so the loop
        // below has no exit between its three calls and each set keeps its registers.
        auto process = [&](DownSet<G> &st) {
            const bool real = cp.x < nx;
            if (real && cp.sb == 0) {
                const int gn = min(G, cp.cnt - cp.grp * G);
                live = r16 < gn;
                // every lane reads a slot of the group (lanes past its end: the first)
                slot = (int)lslot[cp.start + cp.grp * G + (live ? r16 : 0)];
                c = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            // the task's data into the wave's LDS tiles (the wave's reads of the previous task are
            // complete: LDS operations of one wave execute in order)
    #pragma unroll
            for (int j = 0; j < 4; ++j) wt[4 * j + wrow][wslot] = st.v[j];
    #pragma unroll
            for (int j = 0; j < G / 2; ++j) xt[2 * j + (lane >> 5)][lane & 31] = st.x[j];
            const uint64_t scb = st.sc;
            const int s0 = cp.sb * kMfmaSteps;
            issue(st);                                     // refill the set with the task three ahead
            if (!real) return;
            // Columns past the group's slots hold stale act; each result column depends only
            // on its own act column, and those columns are never folded.
            if (s0 + kMfmaSteps <= s_full) {               // all 4 steps inside the row
                // with registers to spare, every LDS read of the task first, so their latencies overlap
                constexpr int kPre = W < 16 ? kMfmaSteps : 1;
                u32x4 wqs[kPre], xas[kPre], xbs[kPre];
                if constexpr (W < 16) {
    #pragma unroll
                    for (int i = 0; i < kMfmaSteps; ++i) {
                        wqs[i] = wt[r16][(4 * i + q) ^ r16];
                        xas[i] = xt[xr][8 * i + 2 * q];
                        xbs[i] = xt[xr][8 * i + 2 * q + 1];
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
    #pragma unroll
                for (int i = 0; i < kMfmaSteps; ++i) {
                    const float f = e8m0_operand((uint32_t)(scb >> (8 * (2 * i + (q >> 1)))) & 0xFFu);
                    const int ip = W < 16 ? i : 0;
                    if constexpr (W >= 16) {
                        wqs[0] = wt[r16][(4 * i + q) ^ r16];    // segment 4 i + q of row r16
                        xas[0] = xt[xr][8 * i + 2 * q];         // elements 64 i + 16 q .. + 7
                        xbs[0] = xt[xr][8 * i + 2 * q + 1];     // .. + 8 .. + 15
                    }
                    const u32x4 wq = wqs[ip], xa = xas[ip], xb = xbs[ip];
                    uint32_t ww[8];
    #pragma unroll
                    for (int d = 0; d < 4; ++d) mx_word_bf16(wq[d], f, ww[2 * d], ww[2 * d + 1]);
                    const u32x4 w0 = {ww[0], ww[1], ww[2], ww[3]}, w1 = {ww[4], ww[5], ww[6], ww[7]};
                    c = mfma_bf16(w0, xa, c);
                    c = mfma_bf16(w1, xb, c);
                }
            } else {
    #pragma unroll
                for (int i = 0; i < kMfmaSteps; ++i) {
                    const int k = 64 * (s0 + i) + 16 * q;
                    const bool ok = s0 + i < s_hi && k < I;
                    const uint32_t bs = (uint32_t)(scb >> (8 * (2 * i + (q >> 1)))) & 0xFFu;
                    const float f = e8m0_operand(ok ? bs : 127u);
                    const u32x4 wq = ok ? wt[r16][(4 * i + q) ^ r16] : zero;
                    const u32x4 xa = ok ? xt[xr][8 * i + 2 * q] : zero;
                    const u32x4 xb = ok ? xt[xr][8 * i + 2 * q + 1] : zero;
                    uint32_t ww[8];
    #pragma unroll
                    for (int d = 0; d < 4; ++d) mx_word_bf16(wq[d], f, ww[2 * d], ww[2 * d + 1]);
                    const u32x4 w0 = {ww[0], ww[1], ww[2], ww[3]}, w1 = {ww[4], ww[5], ww[6], ww[7]};
                    c = mfma_bf16(w0, xa, c);
                    c = mfma_bf16(w1, xb, c);
                }
            }
            // lane (column r16, quad q) holds P[4 q + j][r16]: the slot's rows 4 q .. 4 q + 3
            if (cp.sb == nsb - 1 && live) pv[slot - sl0][q] = c;
            advance(cp, false);
        };

        DownSet<G> sa, sb, sc;
        // with 8 waves the first task's weights are in flight while the wave files its slots (its act
        // rows need them); with 16 (128 registers) the slots are filed first
        if constexpr (W < 16) issue_w(sa);
        // this wave's slots into their experts' runs (lcur of another wave's expert reads either the
        // cleared value or that wave's; neither names this wave).  With 8 waves (registers to spare)
        // each step's LDS operations are issued for all of the range's slots before the next step
        // waits for them.
        if constexpr (W >= 16) {
            for (int t = lane; t < nsl; t += 64) {
                const unsigned e = lid[t];
                if (e < (unsigned)E && lcur[e] >> 16 == (uint32_t)wv)
                    lslot[atomicAdd(&lcur[e], 1u) & 0xFFFFu] = (int16_t)(sl0 + t);
            }
        } else {
            constexpr int kC = MAXS / 64;
            unsigned ev[kC];
    #pragma unroll
            for (int j = 0; j < kC; ++j) ev[j] = 64 * j + lane < nsl ? (unsigned)lid[64 * j + lane] : (unsigned)E;
            bool own[kC];
    #pragma unroll
            for (int j = 0; j < kC; ++j) own[j] = ev[j] < (unsigned)E && lcur[ev[j] < (unsigned)E ? ev[j] : 0] >> 16 == (uint32_t)wv;
            uint32_t pos[kC];
    #pragma unroll
            for (int j = 0; j < kC; ++j) pos[j] = own[j] ? atomicAdd(&lcur[ev[j]], 1u) & 0xFFFFu : 0u;
    #pragma unroll
            for (int j = 0; j < kC; ++j)
                if (own[j]) lslot[pos[j]] = (int16_t)(sl0 + 64 * j + lane);
        }
        // dynamic deal: every wave's runs filed and its deal entries written before any wave takes an
        // expert another wave filed (workgroup-uniform condition)
        if constexpr (D) __syncthreads();

        if constexpr (W < 16) {
            rows_x();
            issue_x(sa);
        } else {
            issue(sa);
        }
        issue(sb);
        if constexpr (W < 16) issue(sc);
        while (cp.x < nx) {
            process(sa);
            process(sb);
            if constexpr (W < 16) process(sc);     // 16 waves: two sets (register budget 128)
        }
    };
    if constexpr (W < 16) {
        if (dyn)
            tasks(std::true_type{});
        else
            tasks(std::false_type{});
    } else {
        tasks(std::false_type{});
    }

    __syncthreads();
    // the fold: thread t owns output (token tb0 + t / 16, row t % 16) of the block
    constexpr int kPer = (kMaxB * 16 + 64 * W - 1) / (64 * W);
    const int nt = (tb1 - tb0) * 16;
    float yv[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int t = (int)threadIdx.x + 64 * W * j;
        float y = 0.f;
        if (t < nt) {
            const int bl = t >> 4, r = t & 15;
            bool bad = false;
            // the token's slots in fold order, 8 at a time: each group's table reads are issued
            // together (one LDS round trip per step instead of two per slot)
            for (int i0 = 0; i0 < K; i0 += 8) {
                int o[8];
                float wv[8], pvv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) o[j] = i0 + j < K ? (int)lord[bl * K + i0 + j] : 0x4000;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int sl = bl * K + (o[j] & 0xFF);
                    wv[j] = lw[sl];
                    pvv[j] = pv[sl][r >> 2][r & 3];
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    bad |= (o[j] & 0x2000) != 0;       // an id outside [0, E)
                    if (!(o[j] & 0x4000))              // one of this workgroup's experts
                        y = __builtin_fmaf(wv[j], pvv[j], y);
                }
            }
            if (bad) y = __builtin_nanf("");
        }
        yv[j] = y;
    }
    if (a.esplit == 1) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int t = (int)threadIdx.x + 64 * W * j;
            if (t < nt) a.out[(size_t)(tb0 + (t >> 4)) * H + (size_t)hb * 16 + (t & 15)] = to_bf16(yv[j]);
        }
        return;
    }
    // Expert split (two workgroups per block, all tokens each): each output's two partial sums
    // meet in its scratch cell.  A thread swaps its sum, tagged, into the cell with one atomic
    // exchange; whichever of the two comes second gets the other's sum back, adds them in class
    // order (part 0 + part 1), writes the output and clears the cell for the next call.  Nobody
    // waits and no barrier or counter is involved.  A token's result still depends on its own
    // slots only.  The two workgroups may sit on different XCDs: the exchange is an agent-scope
    // atomic, performed at the coherence point, and no cache is written back or invalidated.
    uint64_t *cell = a.dcell + (size_t)hb * ((size_t)a.B * 16);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int t = (int)threadIdx.x + 64 * W * j;
        if (t < nt) {
            const uint64_t mine = (uint64_t)__builtin_bit_cast(uint32_t, yv[j]) | 1ull << 32;
            const uint64_t got = __hip_atomic_exchange(cell + t, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (got >> 32) {                           // the other class's sum was there: this is the second
                const float o = __builtin_bit_cast(float, (uint32_t)got);
                const float y = part == 0 ? yv[j] + o : o + yv[j];
                a.out[(size_t)(tb0 + (t >> 4)) * H + (size_t)hb * 16 + (t & 15)] = to_bf16(y);
                __hip_atomic_store(cell + t, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Router: top-k gating ahead of the layer.  One wave per token; lane l holds
// logits l + 64 r (r < RPL).  K rounds: each finds the largest remaining logit
// (wave max) and, among lanes holding that value, the lowest expert index
// (wave min), then retires it.  Lane k keeps the k-th choice.  Weights are the
// softmax over the chosen logits, exp(l_k - l_0) / sum_j exp(l_j - l_0), in
// FP32.  Logits must be finite.
// ---------------------------------------------------------------------------
template <int RPL>
__global__ __launch_bounds__(256) void route_kernel(const float *logits, int B, int E, int K, int32_t *ids,
                                                    float *w) {
    const int lane = threadIdx.x & 63;
    const int b = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)));
    if (b >= B) return;
    float v[RPL];
    bool live[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const int e = lane + 64 * r;
        live[r] = e < E;
        v[r] = live[r] ? logits[(size_t)b * E + e] : 0.f;
    }
    int my_id = 0;
    float my_l = 0.f;
    for (int k = 0; k < K; ++k) {
        float bv = -__builtin_inff();
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int r = 0; r < RPL; ++r)       // ascending index within the lane: strict > keeps the lowest
            if (live[r] && (bi == 0x7FFFFFFF || v[r] > bv)) { bv = v[r]; bi = lane + 64 * r; }
        const float m = wave_max(bv);
        const int idx = wave_min(bi != 0x7FFFFFFF && bv == m ? bi : 0x7FFFFFFF);
#pragma unroll
        for (int r = 0; r < RPL; ++r)
            if (lane + 64 * r == idx) live[r] = false;
        if (lane == k) { my_id = idx; my_l = m; }
    }
    const float l0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_l), 0));
    const float ez = lane < K ? expf(my_l - l0) : 0.f;
    const float z = wave_sum(ez);
    if (lane < K) {
        ids[(size_t)b * K + lane] = my_id;
        w[(size_t)b * K + lane] = ez / z;
    }
}

// ---------------------------------------------------------------------------
// Measurement helpers.
// ---------------------------------------------------------------------------

// For E8M0 byte s = blockIdx.x and code c = threadIdx.x: the conversion of
// the four codes c, c+1, c+2, c+3 (mod 256) packed in one word, bytes 0..3,
// exactly as the layer kernels perform it (same operand construction, same
// instructions).  out[((s * 256) + c) * 4 + j] holds the FP32 conversion of
// byte j; out[65536 * 4 + ((s * 256) + c) * 4 + j] the BF16 conversion,
// widened to FP32.
__global__ __launch_bounds__(256) void dequant_probe_kernel(float *out) {
    const uint32_t s = blockIdx.x, c = threadIdx.x;
    const uint32_t word = (c & 255u) | (((c + 1) & 255u) << 8) | (((c + 2) & 255u) << 16) | (((c + 3) & 255u) << 24);
    const float f = e8m0_operand(s);
    const f32x2 lo = mx_pair<false>(word, f);
    const f32x2 hi = mx_pair<true>(word, f);
    float *o = out + ((size_t)s * 256 + c) * 4;
    o[0] = lo.x; o[1] = lo.y; o[2] = hi.x; o[3] = hi.y;
    const uint32_t blo = mx_pair_bf16<false>(word, f), bhi = mx_pair_bf16<true>(word, f);
    float *p = o + 65536 * 4;
    p[0] = bf16_lo(blo); p[1] = bf16_hi(blo); p[2] = bf16_lo(bhi); p[3] = bf16_hi(bhi);
}

// Reads n16 16-byte words in a grid-stride loop with U independent loads in
// flight per lane.  Each lane folds its words into an XOR; the sink is written
// only if that fold equals `never` (a value the caller chooses so it does not
// occur), which keeps every load live without a reduction.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *buf, size_t n16, uint32_t *sink, uint32_t never) {
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = buf[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += stride) {
        const u32x4 v = buf[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (acc == never) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void stream_copy_kernel(u32x4 *dst, const u32x4 *src, size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

__global__ void sleep_kernel(int units) {
    for (int i = 0; i < units; ++i) __builtin_amdgcn_s_sleep(127);
}

}  // namespace wd
