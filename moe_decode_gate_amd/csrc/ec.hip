// Expert-centric MoE decode layer for gfx950: the conventional pipeline
// (align/pad -> gather -> grouped gate/up GEMM -> grouped down GEMM with
// scatter -> combine) that warp decode is compared with.  Entry points and
// workspace layout are declared in include/ec.h.
//
// Both projections run on the MX-scaled FP8 matrix instruction
// v_mfma_scale_f32_16x16x128_f8f6f4: A is a 16 x 128 block of E4M3 codes
// (activation rows), B a 128 x 16 block (16 weight rows), each with one E8M0
// scale per row per 32 K-elements, accumulated in FP32.  Operand layout, as
// measured on MI355X: lane l holds row (A) or column (B) l % 16; its first 16
// bytes are K = 16*(l/16) + 0..15, its last 16 bytes K = 64 + 16*(l/16) + 0..15;
// the scale operand of lane r + 16*q is the E8M0 byte of row/column r for the
// K-block [32q, 32q + 32); result lane l holds column l % 16, rows 4*(l/16) + 0..3.

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <atomic>
#include <climits>
#include <cstdint>
#include <cstring>

#include "ec.h"
#include "wd_device.h"

namespace ec {

using wd::u32x4;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;          // rows per tile (M of the matrix instruction)
constexpr int kStepK = 128;        // K per matrix instruction
constexpr int kBatch = 2;          // K steps whose loads are issued together (down)
constexpr int kMaxE = 1024, kMaxPairs = 4096, kMaxH = 8192, kMaxI = 8192;
constexpr int kAlignThreads = 1024;
constexpr int kGemmThreads = 256;  // down: 4 waves
constexpr int kGuWaves = 8;        // gate/up: 8 waves splitting K
constexpr int kGuThreads = 64 * kGuWaves;
constexpr int kGuCols = 32;        // intermediate columns per gate/up workgroup (one MX block)
constexpr int kDnCols = 64;        // output columns per down workgroup (16 per wave)

// ---- MXFP8 rounding ------------------------------------------------------

// E8M0 scale byte of a 32-block with largest magnitude amax: the FP32 exponent
// field of amax minus 8 (E4M3's largest binade is 2^8), clamped to [0, 254].
// amax = 0 and subnormal amax give 0.
__device__ __forceinline__ uint32_t scale_byte(float amax) {
    const int eb = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
    return (uint32_t)min(max(eb - 8, 0), 254);
}

// 2^(127 - s) as FP32, s <= 253: multiplying by it divides by the block scale exactly.
__device__ __forceinline__ float inv_scale(uint32_t s) { return __uint_as_float((254u - s) << 23); }

// FP32 -> E4M3 ("FN") code, round to nearest even, saturating at +-448.
// Below 2^-6 the format steps by 2^-9; above, 3 mantissa bits are kept.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const uint32_t b = __float_as_uint(v);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t a = b & 0x7FFFFFFFu;
    uint32_t c;
    if (a > 0x7F800000u) c = 0x7Fu;                                   // NaN
    else if (a >= 0x43E00000u) c = 0x7Eu;                             // >= 448
    else if (a < 0x3C800000u) c = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.f);
    else c = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);  // rebias 127 -> 7
    return sign | c;
}

// Quantize 32 FP32 values (one MX block) to 8 words of E4M3 codes; returns the scale byte.
__device__ __forceinline__ uint32_t quantize32(const float *v, uint32_t *codes) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const uint32_t s = scale_byte(amax);
    const float f = inv_scale(s);
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) word |= e4m3_code(v[4 * w + j] * f) << (8 * j);
        codes[w] = word;
    }
    return s;
}

// 32 BF16 values (64 bytes at p) to FP32.
__device__ __forceinline__ void load_bf16x32(const uint16_t *p, float *v) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const u32x4 d = wd::ld16(p + 8 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[8 * q + 2 * i] = wd::bf16_lo(d[i]);
            v[8 * q + 2 * i + 1] = wd::bf16_hi(d[i]);
        }
    }
}

__device__ __forceinline__ v8i make_operand(u32x4 lo, u32x4 hi) {
    v8i r;
    r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
    r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
    return r;
}

__device__ __forceinline__ v4f mfma_mx(v8i a, v8i b, v4f c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// One lane's share of a K step of a row of MXFP8 data (codes row, scales row,
// length n): the two 16-byte halves and the scale byte the lane supplies.
// Segments past n read as zero codes with scale byte 127.
struct Frag { u32x4 lo, hi; int s; };

__device__ __forceinline__ Frag load_frag(const uint8_t *codes, const uint8_t *scales, int n, int k0, int g) {
    Frag f;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int klo = k0 + 16 * g, khi = k0 + 64 + 16 * g, ks = k0 + 32 * g;
    f.lo = klo < n ? wd::ld16(codes + klo) : z;
    f.hi = khi < n ? wd::ld16(codes + khi) : z;
    f.s = ks < n ? (int)scales[ks / 32] : 127;
    return f;
}

// The codes of one K step without branches: both halves loaded at offsets
// clamped into the row, then zeroed past n (a branch around a load tends to
// end in a wait for it, which would serialise the batch).
struct Codes { u32x4 lo, hi; };

__device__ __forceinline__ Codes load_codes(const uint8_t *codes, int n, int k0, int g) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int klo = k0 + 16 * g, khi = k0 + 64 + 16 * g;
    Codes c;
    c.lo = wd::ld16(codes + (klo < n ? klo : 0));
    c.hi = wd::ld16(codes + (khi < n ? khi : 0));
    c.lo = klo < n ? c.lo : z;
    c.hi = khi < n ? c.hi : z;
    return c;
}

// E8M0 bytes of blocks blk0 .. blk0+7 of a row of nb blocks (two K steps), byte
// 127 past the row: one 8-byte load when the row starts on a 4-byte boundary and
// holds all eight, else byte by byte.  Step i's byte for lane group g is byte 4i + g.
__device__ __forceinline__ uint64_t load_scales8(const uint8_t *srow, int nb, int blk0) {
    if ((nb & 3) == 0 && blk0 + 8 <= nb) return *reinterpret_cast<const uint64_t *>(srow + blk0);
    uint64_t v = 0;
    for (int c = 0; c < 8; ++c) v |= (uint64_t)(blk0 + c < nb ? srow[blk0 + c] : 127u) << (8 * c);
    return v;
}

__device__ __forceinline__ int scale_of(uint64_t v, int i, int g) { return (int)((v >> (8 * (4 * i + g))) & 0xFFu); }

// ---- stage 1: align / pad ----------------------------------------------------

struct AlignArgs {
    const int32_t *ids;
    int32_t *header, *tile_expert, *row_pair;
    int pairs, E, max_tiles;
};

// One workgroup.  Tiles past the ones in use get expert -1 and their rows
// pair -2, so later stages find the end of the list with the load they make anyway.
__global__ void __launch_bounds__(kAlignThreads) align_kernel(AlignArgs a) {
    __shared__ int cnt[kMaxE], fill[kMaxE], base[kMaxE];
    __shared__ int wave_tot[kAlignThreads / 64];
    const int t = threadIdx.x;
    for (int e = t; e < a.E; e += kAlignThreads) { cnt[e] = 0; fill[e] = 0; }
    __syncthreads();
    for (int p = t; p < a.pairs; p += kAlignThreads) {
        const int e = a.ids[p];
        if (e >= 0 && e < a.E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    // exclusive scan of tiles per expert (E <= 1024: one expert per thread)
    const int tiles = t < a.E ? (cnt[t] + kTile - 1) / kTile : 0;
    int incl = tiles;
    const int lane = t & 63, wv = t >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
    }
    if (lane == 63) wave_tot[wv] = incl;
    __syncthreads();
    int off = 0, total = 0;
    for (int w = 0; w < kAlignThreads / 64; ++w) {
        off += w < wv ? wave_tot[w] : 0;
        total += wave_tot[w];
    }
    if (t < a.E) {
        const int b = off + incl - tiles;
        base[t] = b;
        for (int i = 0; i < tiles; ++i) a.tile_expert[b + i] = t;
        for (int r = cnt[t]; r < tiles * kTile; ++r) a.row_pair[b * kTile + r] = -1;
    }
    for (int i = total + t; i < a.max_tiles; i += kAlignThreads) a.tile_expert[i] = -1;
    for (int i = total * kTile + t; i < a.max_tiles * kTile; i += kAlignThreads) a.row_pair[i] = -2;
    if (t == 0) a.header[0] = total;
    __syncthreads();
    for (int p = t; p < a.pairs; p += kAlignThreads) {
        const int e = a.ids[p];
        if (e >= 0 && e < a.E) a.row_pair[base[e] * kTile + atomicAdd(&fill[e], 1)] = p;
    }
}

// ---- stage 2: gather + quantize x ------------------------------------------

struct GatherArgs {
    const uint16_t *x;
    const int32_t *row_pair;
    uint8_t *xq, *xs;
    int K, H, max_rows;
};

// One wave per row; each lane quantizes whole 32-blocks.  Padding rows get
// zero codes and scale byte 0.
__global__ void __launch_bounds__(256) gather_kernel(GatherArgs a) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= a.max_rows) return;
    const int p = a.row_pair[row];
    if (p == -2) return;                                   // past the tiles in use
    const int nb = a.H / 32;
    uint8_t *q = a.xq + (size_t)row * a.H;
    uint8_t *s = a.xs + (size_t)row * nb;
    for (int blk = lane; blk < nb; blk += 64) {
        uint32_t codes[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        uint32_t sb = 0;
        if (p >= 0) {
            float v[32];
            load_bf16x32(a.x + (size_t)(p / a.K) * a.H + 32 * blk, v);
            sb = quantize32(v, codes);
        }
        u32x4 c0 = {codes[0], codes[1], codes[2], codes[3]}, c1 = {codes[4], codes[5], codes[6], codes[7]};
        *reinterpret_cast<u32x4 *>(q + 32 * blk) = c0;
        *reinterpret_cast<u32x4 *>(q + 32 * blk + 16) = c1;
        s[blk] = (uint8_t)sb;
    }
}

// ---- stage 3: grouped gate/up GEMM + SiLU(g) * u + MXFP8 -------------------

struct GateUpArgs {
    const uint8_t *xq, *xs, *w, *ws;   // gathered x; gate/up codes [E][2I][H], scales [E][2I][H/32]
    const int32_t *tile_expert;
    uint8_t *aq, *as;                   // MXFP8 intermediate [rows][I], [rows][I/32]
    uint16_t *act;                      // optional BF16 intermediate [rows][I]
    int H, I, nblocks, ncolblk;
};

// Workgroup = (tile, 32 columns: the gate rows and the up rows of one MX
// block of the intermediate).  The eight waves split the K steps into
// contiguous ranges; their partial tiles are summed through LDS in wave
// order, and the epilogue rounds the block to BF16 and then to MXFP8.
__global__ void __launch_bounds__(kGuThreads) gate_up_kernel(GateUpArgs a) {
    __shared__ float part[kGuWaves][4][4][64];
    const int lb = wd::xcd_logical(blockIdx.x, a.nblocks);
    const int tile = lb / a.ncolblk, cb = lb % a.ncolblk;
    const int e = a.tile_expert[tile];
    if (e < 0) return;
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int H = a.H, I = a.I, nbh = H / 32;
    const size_t xrow = (size_t)tile * kTile + r;
    const uint8_t *xc = a.xq + xrow * H, *xsr = a.xs + xrow * nbh;
    // result tiles: gate columns +0 / +16, up columns +0 / +16 of this block
    const uint8_t *wc[4], *wsr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const size_t wrow = (size_t)e * 2 * I + (t >= 2 ? I : 0) + (size_t)cb * kGuCols + 16 * (t & 1) + r;
        wc[t] = a.w + wrow * H;
        wsr[t] = a.ws + wrow * nbh;
    }
    v4f c[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) c[t] = v4f{0.f, 0.f, 0.f, 0.f};
    // wave wv takes an even-length contiguous range of K steps, two at a time, so one
    // 8-byte load brings a row's scale bytes for both
    const int nks = (H + kStepK - 1) / kStepK;
    const int per = 2 * ((nks + 2 * kGuWaves - 1) / (2 * kGuWaves));
    const int s_hi = min(nks, (wv + 1) * per);
    for (int s0 = wv * per; s0 < s_hi; s0 += 2) {
        const uint64_t sx = load_scales8(xsr, nbh, 4 * s0);
        uint64_t sw[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) sw[t] = load_scales8(wsr[t], nbh, 4 * s0);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int k0 = (s0 + i) * kStepK;          // past H: codes read as zero
            const Codes fx = load_codes(xc, H, k0, g);
            Codes fw[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) fw[t] = load_codes(wc[t], H, k0, g);
            const v8i ax = make_operand(fx.lo, fx.hi);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                c[t] = mfma_mx(ax, make_operand(fw[t].lo, fw[t].hi), c[t], scale_of(sx, i, g), scale_of(sw[t], i, g));
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) part[wv][t][q][lane] = c[t][q];
    __syncthreads();
    // thread -> row m, column j of the block; its value sits in result lane
    // n + 16 * (m / 4), element m % 4, of tile j / 16 (gate) and 2 + j / 16 (up)
    const int m = threadIdx.x >> 5, j = threadIdx.x & 31;
    const int nt = j >> 4, l = (j & 15) + 16 * (m >> 2), q = m & 3;
    float gsum = part[0][nt][q][l], usum = part[0][2 + nt][q][l];
#pragma unroll
    for (int w = 1; w < kGuWaves; ++w) { gsum += part[w][nt][q][l]; usum += part[w][2 + nt][q][l]; }
    const float en = expf(-fabsf(gsum));
    const float sig = gsum >= 0.f ? 1.f / (1.f + en) : en / (1.f + en);
    const uint16_t ab = wd::to_bf16(gsum * sig * usum);
    const float av = __uint_as_float((uint32_t)ab << 16);
    // the block's 32 values are lanes [0, 32) or [32, 64) of this wave
    float amax = fabsf(av);
#pragma unroll
    for (int d = 16; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 32));
    const uint32_t sb = scale_byte(amax);
    const size_t row = (size_t)tile * kTile + m;
    a.aq[row * I + (size_t)cb * kGuCols + j] = (uint8_t)e4m3_code(av * inv_scale(sb));
    if (j == 0) a.as[row * (I / 32) + cb] = (uint8_t)sb;
    if (a.act) a.act[row * I + (size_t)cb * kGuCols + j] = ab;
}

// ---- stage 4: grouped down GEMM + scatter -----------------------------------

struct DownArgs {
    const uint8_t *aq, *as;             // MXFP8 intermediate
    const uint8_t *w, *ws;              // down codes [E][H][I], scales [E][H][I/32]
    const int32_t *tile_expert, *row_pair;
    uint16_t *out_pair;                 // [B*K][H] BF16
    int H, I, nblocks, ncolblk;
};

// Workgroup = (tile, 64 output columns), one 16-column result tile per wave
// over the whole I; both operands are loaded straight into the matrix
// instruction's layout.
__global__ void __launch_bounds__(kGemmThreads) down_kernel(DownArgs a) {
    const int lb = wd::xcd_logical(blockIdx.x, a.nblocks);
    const int tile = lb / a.ncolblk, cb = lb % a.ncolblk;
    const int e = a.tile_expert[tile];
    if (e < 0) return;
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int I = a.I, H = a.H, nbi = I / 32;
    const int col0 = cb * kDnCols + 16 * wv;
    if (col0 >= H) return;
    const u32x4 pairs = wd::ld16(a.row_pair + (size_t)tile * kTile + 4 * g);   // rows 4g .. 4g+3
    const size_t arow = (size_t)tile * kTile + r;
    const uint8_t *ac = a.aq + arow * I, *asr = a.as + arow * nbi;
    const size_t wrow = (size_t)e * H + col0 + r;
    const uint8_t *wc = a.w + wrow * I, *wsr = a.ws + wrow * nbi;
    v4f c = {0.f, 0.f, 0.f, 0.f};
    const int nks = (I + kStepK - 1) / kStepK;
    static_assert(kBatch % 2 == 0, "scale bytes come two K steps per load");
    for (int s0 = 0; s0 < nks; s0 += kBatch) {
        Codes fa[kBatch], fw[kBatch];
        uint64_t sa[kBatch / 2], sw[kBatch / 2];
#pragma unroll
        for (int i = 0; i < kBatch / 2; ++i) {
            sa[i] = load_scales8(asr, nbi, 4 * (s0 + 2 * i));
            sw[i] = load_scales8(wsr, nbi, 4 * (s0 + 2 * i));
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            fa[i] = load_codes(ac, I, (s0 + i) * kStepK, g);
            fw[i] = load_codes(wc, I, (s0 + i) * kStepK, g);
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            c = mfma_mx(make_operand(fa[i].lo, fa[i].hi), make_operand(fw[i].lo, fw[i].hi), c,
                        scale_of(sa[i / 2], i % 2, g), scale_of(sw[i / 2], i % 2, g));
    }
    // scatter: result rows 4g + q of column col0 + r
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int p = (int)pairs[q];
        if (p >= 0) a.out_pair[(size_t)p * H + col0 + r] = wd::to_bf16(c[q]);
    }
}

// ---- stage 5: combine ---------------------------------------------------------

struct CombineArgs {
    const uint16_t *out_pair;
    const int32_t *ids;
    const float *w;
    uint16_t *out;
    int B, K, E, H;
};

// One thread per (token, 8 consecutive columns): FP32 sum over the token's
// slots in slot order, rounded to BF16.  A token with an invalid id gets NaN.
__global__ void __launch_bounds__(256) combine_kernel(CombineArgs a) {
    const int per_tok = a.H / 8;
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= a.B * per_tok) return;
    const int b = t / per_tok, h0 = 8 * (t % per_tok);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    bool bad = false;
    for (int k = 0; k < a.K; ++k) {
        const int e = a.ids[b * a.K + k];
        if (e < 0 || e >= a.E) { bad = true; continue; }
        const float wk = a.w[b * a.K + k];
        const u32x4 d = wd::ld16(a.out_pair + ((size_t)b * a.K + k) * a.H + h0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(wk, wd::bf16_lo(d[i]), acc[2 * i]);
            acc[2 * i + 1] = fmaf(wk, wd::bf16_hi(d[i]), acc[2 * i + 1]);
        }
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = bad ? 0x7FC0u : wd::to_bf16(acc[2 * i]);
        const uint32_t hi = bad ? 0x7FC0u : wd::to_bf16(acc[2 * i + 1]);
        o[i] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4 *>(a.out + (size_t)b * a.H + h0) = o;
}

// ---- diagnostic: the MX matrix instruction on given operands -----------------

// Block i: C_i = A_i * B_i^T, A_i and B_i [16][128] E4M3 codes with E8M0 scales
// [16][4] (one per 32 along K), one matrix instruction per block.
__global__ void __launch_bounds__(64) mma_probe_kernel(const uint8_t *a, const uint8_t *b, const uint8_t *sa,
                                                       const uint8_t *sb, float *out) {
    const size_t i = blockIdx.x;
    const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
    const Frag fa = load_frag(a + (i * kTile + r) * kStepK, sa + (i * kTile + r) * 4, kStepK, 0, g);
    const Frag fb = load_frag(b + (i * kTile + r) * kStepK, sb + (i * kTile + r) * 4, kStepK, 0, g);
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    const v4f c = mfma_mx(make_operand(fa.lo, fa.hi), make_operand(fb.lo, fb.hi), zero, fa.s, fb.s);
#pragma unroll
    for (int q = 0; q < 4; ++q) out[(i * kTile + 4 * g + q) * kTile + r] = c[q];
}

}  // namespace ec

// ---- host ------------------------------------------------------------------

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) { (void)hipGetLastError(); return WD_ERR_DEVICE; }
    if (dev >= kMaxDevices) return WD_ERR_DEVICE;
    int st = g_arch[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) { (void)hipGetLastError(); return WD_ERR_DEVICE; }
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        g_arch[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? WD_OK : WD_ERR_DEVICE;
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

int check_dims(int B, int K, int E, int H, int I) {
    if (B < 0 || K < 1 || E < 1 || K > E || H < 32 || I < 32 || H % 32 || I % 32) return WD_ERR_DIMS;
    if (E > ec::kMaxE || H > ec::kMaxH || I > ec::kMaxI || (long long)B * K > ec::kMaxPairs)
        return WD_ERR_UNSUPPORTED;
    return WD_OK;
}

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// Region offsets; returns the tile bound.
int layout(int B, int K, int E, int H, int I, size_t *off) {
    const long long pairs = (long long)B * K;
    const long long used = pairs < E ? pairs : E;
    const long long tiles = (pairs + 15 * used) / ec::kTile;
    const size_t rows = (size_t)tiles * ec::kTile;
    size_t o = 0;
    off[EC_WS_HEADER] = o;      o += round256(64 * sizeof(int32_t));
    off[EC_WS_TILE_EXPERT] = o; o += round256((size_t)tiles * sizeof(int32_t));
    off[EC_WS_ROW_PAIR] = o;    o += round256(rows * sizeof(int32_t));
    off[EC_WS_XQ] = o;          o += round256(rows * H);
    off[EC_WS_XS] = o;          o += round256(rows * (H / 32));
    off[EC_WS_ACT] = o;         o += round256(rows * I * sizeof(uint16_t));
    off[EC_WS_AQ] = o;          o += round256(rows * I + rows * (I / 32));
    off[EC_WS_OUT_PAIR] = o;    o += round256((size_t)pairs * H * sizeof(uint16_t));
    off[EC_WS_TOTAL] = o;
    return (int)tiles;
}

template <class Kern, class Args>
int launch(Kern k, int blocks, int threads, size_t lds, const Args &args, const ec_launch &c, int stage,
           hipStream_t s) {
    hipEvent_t e0 = (hipEvent_t)c.start_event[stage - 1], e1 = (hipEvent_t)c.stop_event[stage - 1];
    if (e0 || e1)
        hipExtLaunchKernelGGL(k, dim3(blocks), dim3(threads), lds, s, e0, e1, 0, args);
    else
        hipLaunchKernelGGL(k, dim3(blocks), dim3(threads), lds, s, args);
    return hipGetLastError() == hipSuccess ? WD_OK : WD_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t ec_workspace_bytes(int B, int K, int E, int H, int I) {
    if (check_dims(B, K, E, H, I) != WD_OK || B == 0) return 0;
    size_t off[EC_WS_REGIONS];
    layout(B, K, E, H, I, off);
    return off[EC_WS_TOTAL];
}

int ec_workspace_layout(int B, int K, int E, int H, int I, size_t *offsets) {
    if (!offsets) return WD_ERR_NULL;
    const int rc = check_dims(B, K, E, H, I);
    if (rc != WD_OK) return rc;
    layout(B, K, E, H, I, offsets);
    return WD_OK;
}

int ec_moe_decode_ex(const uint16_t *x, const int32_t *ids, const float *w,
                     const uint8_t *wgu, const uint8_t *sgu, const uint8_t *wdn, const uint8_t *sd,
                     void *workspace, size_t workspace_bytes, uint16_t *out,
                     int B, int K, int E, int H, int I, const ec_launch *cfg, void *stream) {
    const ec_launch c = cfg ? *cfg : ec_launch{};
    if (c.last_stage < 0 || c.last_stage > 5) return WD_ERR_UNSUPPORTED;
    const int last = c.last_stage == 0 ? 5 : c.last_stage;
    int rc = check_dims(B, K, E, H, I);
    if (rc != WD_OK) return rc;
    if (B == 0) return WD_OK;
    if (!x || !ids || !w || !wgu || !sgu || !wdn || !sd || !workspace || (last == 5 && !out)) return WD_ERR_NULL;
    if (!aligned(x, 16) || !aligned(ids, 4) || !aligned(w, 4) || !aligned(wgu, 16) || !aligned(wdn, 16) ||
        !aligned(workspace, 256) || (out && !aligned(out, 16)))
        return WD_ERR_ALIGN;
    size_t off[EC_WS_REGIONS];
    const int tiles = layout(B, K, E, H, I, off);
    if (workspace_bytes < off[EC_WS_TOTAL]) return WD_ERR_WORKSPACE;
    if ((rc = check_device()) != WD_OK) return rc;

    hipStream_t s = (hipStream_t)stream;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    int32_t *header = reinterpret_cast<int32_t *>(ws + off[EC_WS_HEADER]);
    int32_t *tile_expert = reinterpret_cast<int32_t *>(ws + off[EC_WS_TILE_EXPERT]);
    int32_t *row_pair = reinterpret_cast<int32_t *>(ws + off[EC_WS_ROW_PAIR]);
    uint8_t *xq = ws + off[EC_WS_XQ], *xs = ws + off[EC_WS_XS];
    uint16_t *act = reinterpret_cast<uint16_t *>(ws + off[EC_WS_ACT]);
    uint8_t *aq = ws + off[EC_WS_AQ];
    uint16_t *out_pair = reinterpret_cast<uint16_t *>(ws + off[EC_WS_OUT_PAIR]);
    const int rows = tiles * ec::kTile;

    ec::AlignArgs aa{ids, header, tile_expert, row_pair, B * K, E, tiles};
    if ((rc = launch(ec::align_kernel, 1, ec::kAlignThreads, 0, aa, c, 1, s)) != WD_OK || last == 1) return rc;

    ec::GatherArgs ga{x, row_pair, xq, xs, K, H, rows};
    if ((rc = launch(ec::gather_kernel, (rows + 3) / 4, 256, 0, ga, c, 2, s)) != WD_OK || last == 2) return rc;

    const int gu_cols = I / ec::kGuCols;
    ec::GateUpArgs gua{xq, xs, wgu, sgu, tile_expert, aq, aq + (size_t)rows * I,
                       c.keep_intermediate ? act : nullptr, H, I, tiles * gu_cols, gu_cols};
    if ((rc = launch(ec::gate_up_kernel, tiles * gu_cols, ec::kGuThreads, 0, gua, c, 3, s)) != WD_OK ||
        last == 3)
        return rc;

    const int dn_cols = (H + ec::kDnCols - 1) / ec::kDnCols;
    ec::DownArgs da{aq, aq + (size_t)rows * I, wdn, sd, tile_expert, row_pair, out_pair, H, I, tiles * dn_cols,
                    dn_cols};
    if ((rc = launch(ec::down_kernel, tiles * dn_cols, ec::kGemmThreads, 0, da, c, 4, s)) != WD_OK || last == 4)
        return rc;

    ec::CombineArgs ca{out_pair, ids, w, out, B, K, E, H};
    return launch(ec::combine_kernel, (B * (H / 8) + 255) / 256, 256, 0, ca, c, 5, s);
}

int ec_mma_probe(const uint8_t *a, const uint8_t *b, const uint8_t *sa, const uint8_t *sb, float *out, int n,
                 void *stream) {
    if (n < 0 || n > 65536) return WD_ERR_UNSUPPORTED;
    if (n == 0) return WD_OK;
    if (!a || !b || !sa || !sb || !out) return WD_ERR_NULL;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(out, 4)) return WD_ERR_ALIGN;
    int rc = check_device();
    if (rc != WD_OK) return rc;
    hipLaunchKernelGGL(ec::mma_probe_kernel, dim3(n), dim3(64), 0, (hipStream_t)stream, a, b, sa, sb, out);
    return hipGetLastError() == hipSuccess ? WD_OK : WD_ERR_LAUNCH;
}

int ec_moe_decode(const uint16_t *x, const int32_t *ids, const float *w,
                  const uint8_t *wgu, const uint8_t *sgu, const uint8_t *wdn, const uint8_t *sd,
                  void *workspace, size_t workspace_bytes, uint16_t *out,
                  int B, int K, int E, int H, int I, void *stream) {
    return ec_moe_decode_ex(x, ids, w, wgu, sgu, wdn, sd, workspace, workspace_bytes, out, B, K, E, H, I,
                            nullptr, stream);
}

}  // extern "C"
