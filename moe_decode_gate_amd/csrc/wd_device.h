// Device helpers for the gfx950 MoE decode kernels: MXFP8 element conversion,
// BF16 unpack/round, 64-lane wave reduction, XCD-aware workgroup numbering.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wd {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;      // CDNA wavefront width
constexpr int kChunk = 16;     // elements per lane per 16-byte code load
constexpr int kXcds = 8;       // MI355X: 8 accelerator complex dies, each with its own L2

// ---- loads ---------------------------------------------------------------

__device__ __forceinline__ u32x4 ld16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

// Buffer resource (V#) for raw buffer loads over `bytes` bytes from `base`:
// stride 0, 32-bit data format (required by gfx9-family buffer loads).  A
// load whose offset is at or past `bytes` returns zero and touches no memory.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS (gfx950): lane l's bytes
// land at lds + 16 l; `voff` is the lane's byte offset, `soff` a wave-uniform
// one.
__device__ __forceinline__ void ld16_lds(rsrc_t r, void *lds, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3))) *)lds, 16, voff, soff, 0, 0);
}

// Waits on the wave's own counters (gfx9 s_waitcnt encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8; a field at its maximum does not
// wait).  Needed around buffer-to-LDS loads: the compiler models such a load
// as writing 16 bytes at the pointer it is given, not the 16 bytes per lane
// it writes, so it neither waits for the data before later LDS reads of the
// other lanes' bytes nor for earlier reads before the load overwrites them.
// Scheduling barriers on both sides keep the compiler from moving memory
// instructions across the wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    __builtin_amdgcn_sched_barrier(0);
}

// Wave-uniform 32-bit load through the scalar data cache (s_load): the
// pointer is read as constant memory, which the inputs of a launch are.
__device__ __forceinline__ int32_t sload(const int32_t *p) {
    return *(const __attribute__((address_space(4))) int32_t *)p;
}

__device__ __forceinline__ u32x4 buf16(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t buf4(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// 16-byte weight load; NT marks it non-temporal (streamed once, not kept in
// the caches), which pays off when no other wave re-reads the row.
template <bool NT>
__device__ __forceinline__ u32x4 ldw(const void *p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    else return *reinterpret_cast<const u32x4 *>(p);
}

// ---- MXFP8 ----------------------------------------------------------------

// E8M0 block exponent byte -> the FP32 scale operand of the scaled FP8
// conversion: the byte is placed in the FP32 exponent field, i.e. the value
// 2^(s-127) for s in [1, 254].  (Bytes 0 and 255 land on FP32 zero / infinity;
// what the hardware does with them is measured by the exhaustive probe.)
__device__ __forceinline__ float e8m0_operand(uint32_t s) {
    return __builtin_bit_cast(float, s << 23);
}

// Two E4M3 codes (byte pair 0-1 when hi == false, 2-3 when hi == true) times
// the block scale, to FP32, with gfx950's v_cvt_scalef32_pk_f32_fp8.
template <bool HI>
__device__ __forceinline__ f32x2 mx_pair(uint32_t word, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(word, scale, HI);
}

// Two E4M3 codes times the block scale, to a packed BF16 pair (element of the
// lower byte in the low half) with v_cvt_scalef32_pk_bf16_fp8.  Exact whenever
// the product is a normal BF16 number: an E4M3 value has at most 4
// significant bits and BF16 keeps 8 and the FP32 exponent range.
template <bool HI>
__device__ __forceinline__ uint32_t mx_pair_bf16(uint32_t word, float scale) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, scale, HI));
}

// ---- BF16 -----------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// FP32 -> BF16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// ---- 16-element dot products ----------------------------------------------

// acc + sum_{i<16} deq(codes[i], scale) * v[i]: codes packed 4 per word (byte
// 0 is the lowest-index element), v in FP32; one FMA per element, in index
// order.
__device__ __forceinline__ float dot16_f32(u32x4 q, float scale, const float *v, float acc) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        f32x2 lo = mx_pair<false>(q[d], scale);
        f32x2 hi = mx_pair<true>(q[d], scale);
        acc = __builtin_fmaf(lo.x, v[4 * d + 0], acc);
        acc = __builtin_fmaf(lo.y, v[4 * d + 1], acc);
        acc = __builtin_fmaf(hi.x, v[4 * d + 2], acc);
        acc = __builtin_fmaf(hi.y, v[4 * d + 3], acc);
    }
    return acc;
}

// Same with the 16 activations given as packed BF16 pairs (a0: elements 0-7,
// a1: elements 8-15; the low half of each word is the lower index).
__device__ __forceinline__ float dot16_bf16(u32x4 q, float scale, u32x4 a0, u32x4 a1, float acc) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        f32x2 lo = mx_pair<false>(q[d], scale);
        f32x2 hi = mx_pair<true>(q[d], scale);
        const uint32_t p0 = d < 2 ? a0[2 * d] : a1[2 * d - 4];
        const uint32_t p1 = d < 2 ? a0[2 * d + 1] : a1[2 * d - 3];
        acc = __builtin_fmaf(lo.x, bf16_lo(p0), acc);
        acc = __builtin_fmaf(lo.y, bf16_hi(p0), acc);
        acc = __builtin_fmaf(hi.x, bf16_lo(p1), acc);
        acc = __builtin_fmaf(hi.y, bf16_hi(p1), acc);
    }
    return acc;
}

// Same dot product with v_dot2_f32_bf16: weights converted to BF16 pairs
// (exact, see mx_pair_bf16), activations used as stored (BF16 pairs), two
// products (exact in FP32) added into the FP32 accumulator per instruction.
__device__ __forceinline__ float dot2(uint32_t w, uint32_t a, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, a), acc, false);
}

__device__ __forceinline__ float dot16_dot2(u32x4 q, float scale, u32x4 a0, u32x4 a1, float acc) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t p0 = d < 2 ? a0[2 * d] : a1[2 * d - 4];       // elements 4d, 4d+1
        const uint32_t p1 = d < 2 ? a0[2 * d + 1] : a1[2 * d - 3];   // elements 4d+2, 4d+3
        acc = dot2(mx_pair_bf16<false>(q[d], scale), p0, acc);
        acc = dot2(mx_pair_bf16<true>(q[d], scale), p1, acc);
    }
    return acc;
}

// Four codes of one word converted to two BF16 pairs (elements 0-1, 2-3).
__device__ __forceinline__ void mx_word_bf16(uint32_t word, float scale, uint32_t &lo, uint32_t &hi) {
    lo = mx_pair_bf16<false>(word, scale);
    hi = mx_pair_bf16<true>(word, scale);
}

// acc + sum of 16 products of pre-converted BF16 weight pairs w[0..7] with the
// activation pairs (a0, a1); same pairing and order as dot16_dot2.
__device__ __forceinline__ float dot16_pre(const uint32_t *w, u32x4 a0, u32x4 a1, float acc) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = dot2(w[j], j < 4 ? a0[j] : a1[j - 4], acc);
    return acc;
}

// Math modes of the layer kernels.
enum Math { kMathF32 = 1, kMathDot2 = 2 };

// ---- 64-lane reduction ----------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_upd(float v) {
    // lanes of rows outside ROW_MASK receive 0 (the `old` operand)
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                                                 0xF, false));
}

// Sum over the 64 lanes of a wave, returned to every lane (bit-identical).
// Within each row of 16 lanes, a butterfly: DPP quad_perm xor-1 and xor-2,
// then half-row mirror and row mirror, after which every lane of row r holds
// the row sum S_r.  Across rows, the GFX9 row broadcasts: row_bcast:15 adds
// S_0 into row 1 and S_2 into row 3, row_bcast:31 adds row 1 (S_0 + S_1) into
// row 3, so lane 63 holds (S_2 + S_3) + (S_0 + S_1); v_readlane hands it to
// all lanes.  No LDS, no barrier.  Must run with all 64 lanes active.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_mov<0xB1>(v);          // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);          // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);         // row_half_mirror
    v += dpp_mov<0x140>(v);         // row_mirror
    v += dpp_upd<0x142, 0xA>(v);    // row_bcast:15 into rows 1 and 3
    v += dpp_upd<0x143, 0xC>(v);    // row_bcast:31 into rows 2 and 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Maximum / minimum over the 64 lanes of a wave, returned to every lane;
// same exchange pattern as wave_sum.  Must run with all 64 lanes active.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_upd_i(int v, int old) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ float wave_max(float v) {
    auto step = [](float a, int b) { return __builtin_fmaxf(a, __builtin_bit_cast(float, b)); };
    const int ninf = __builtin_bit_cast(int, -__builtin_inff());
    v = step(v, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v = step(v, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v = step(v, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    v = step(v, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    v = step(v, dpp_upd_i<0x142, 0xA>(__builtin_bit_cast(int, v), ninf));
    v = step(v, dpp_upd_i<0x143, 0xC>(__builtin_bit_cast(int, v), ninf));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ int wave_min(int v) {
    auto step = [](int a, int b) { return a < b ? a : b; };
    const int big = 0x7FFFFFFF;
    v = step(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));
    v = step(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));
    v = step(v, __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false));
    v = step(v, __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false));
    v = step(v, dpp_upd_i<0x142, 0xA>(v, big));
    v = step(v, dpp_upd_i<0x143, 0xC>(v, big));
    return __builtin_amdgcn_readlane(v, 63);
}

// Inclusive prefix sum over the 64 lanes of a wave: lane l gets v_0 + ... + v_l.
// Within each row of 16 lanes, row_shr 1, 2, 4 and 8 (a lane whose source lies
// before its row's start adds 0); across rows, row_bcast:15 adds the last lane
// of row 0 into row 1 and of row 2 into row 3, then row_bcast:31 adds lane 31
// (rows 0 and 1 in all) into rows 2 and 3.  Integer, so exact.  Must run with
// all 64 lanes active.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1 and 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2 and 3
    return v;
}

// Sum over each group of LPR consecutive lanes (LPR = 16, 32 or 64), returned
// to every lane of the group (bit-identical within a group).  The in-row
// butterfly is the one of wave_sum; for 32-lane groups row_bcast:15 adds row
// 0 into row 1 and row 2 into row 3 and v_readlane of lanes 31 and 63 hands
// the two totals back to their groups.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(LPR == 16 || LPR == 32 || LPR == 64, "group of 16, 32 or 64 lanes");
    if constexpr (LPR == 64) {
        return wave_sum(v);
    } else {
        v += dpp_mov<0xB1>(v);          // quad_perm [1,0,3,2]
        v += dpp_mov<0x4E>(v);          // quad_perm [2,3,0,1]
        v += dpp_mov<0x141>(v);         // row_half_mirror
        v += dpp_mov<0x140>(v);         // row_mirror
        if constexpr (LPR == 32) {
            v += dpp_upd<0x142, 0xA>(v);    // row_bcast:15 into rows 1 and 3
            const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
            const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
            v = (threadIdx.x & 32) ? hi : lo;
        }
        return v;
    }
}

// ---- workgroup numbering ----------------------------------------------------

// Workgroups are handed to the XCDs round-robin (workgroup g runs on XCD
// g % 8).  Renumber so XCD x processes one contiguous range of logical
// workgroups, in order: work adjacent in the logical order then shares an L2.
// A bijection on [0, n) for any n.
__device__ __forceinline__ int xcd_logical(int g, int n) {
    const int x = g % kXcds, q = g / kXcds;
    const int base = n / kXcds, rem = n % kXcds;
    return x * base + (x < rem ? x : rem) + q;
}

}  // namespace wd
