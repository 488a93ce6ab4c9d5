// Host side of the MoE decode library: argument checks, launch configuration
// and the C entry points declared in include/wd.h.
//
// Every check runs before the first HIP call, so a rejected call touches no
// device.  Compute entry points enqueue on the caller's stream and return
// without synchronising, allocating or freeing.

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <atomic>
#include <type_traits>
#include <climits>
#include <cstdint>
#include <cstring>

#include "wd.h"
#include "wd_kernels.h"

namespace {

using wd::LayerArgs;

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other

// The current device must be a gfx950 GPU.  Queried once per device.
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
    if (B < 0 || K < 1 || E < 1 || H < 32 || I < 32 || H % 32 || I % 32) return WD_ERR_DIMS;
    if (H > 8192 || (long long)K * I > 16384) return WD_ERR_UNSUPPORTED;
    if ((long long)B * K * I >= INT_MAX || (long long)B * H >= INT_MAX) return WD_ERR_UNSUPPORTED;
    return WD_OK;
}

// Token ranges the matrix-core down needs at least for B tokens of K slots: the smallest
// S in {1, 2, 4} whose ranges of ceil(B / S) tokens fit the 1,024-slot variant (128 tokens,
// 1,024 slots each); 0 when none does.
int down_min_ranges(int B, int K) {
    for (int S : {1, 2, 4}) {
        const long long tpr = (B + S - 1) / S;
        if (tpr <= wd::kDnMfmaMaxBWide && tpr * K <= wd::kDnMfmaMaxSlotsWide) return S;
    }
    return 0;
}

// A token range of tpr tokens needs the 1,024-slot variant (8 waves) past 64 tokens or 512 slots.
bool down_big_range(int tpr, int K) {
    return tpr > wd::kDnMfmaMaxB || (long long)tpr * K > wd::kDnMfmaMaxSlots;
}

// Resolve a launch configuration: fill unset fields with the defaults for
// this batch size, then validate.  Defaults come from sweeps of every
// configuration on MI355X at the 128-expert / top-8 / H 2048 / I 768 layer
// for B in {1, 2, 4, 8, 16, 32, 64}:
//   gate/up, B <= 4: one row per 64-lane wave, BF16-pair dot products,
//          non-temporal weight loads (no row is read twice), hardware order;
//   gate/up, B 5..17 (and form 1 above): 32 lanes per row, 4 rows per lane group (8 per wave),
//          row-block-major order with XCD-contiguous numbering, so the tokens
//          that share an expert row read it from the same L2 while resident;
//   gate/up, B >= 18 (B >= 4 when H >= 4096): the expert form on the matrix
//          cores (one wave per expert row block, and none for an expert no slot
//          uses; Qwen-3 layer 55.3 against 57.0 us at B = 18 with its weight
//          codes non-temporal, the token form ahead at B = 16, 51.7 against
//          53.1; before that: 58.6 against 61.5 us at B = 20, 70 against 85 at
//          B = 32, 75 against 136 at B = 64, the token form ahead at B = 16, 52.9
//          against 55.0; on the 4096 / 1536 layer with Zipf routing, with the H
//          split, 59.8 against 65.0 us at B = 4, 74.4 against 79.8 at B = 6, the
//          token form ahead at B = 2, 33 against 40),
//          register-staged (form 3; the form that
//          streams its codes into LDS measured no faster: 70.9 against 71.7 us
//          at B = 32, and slower on the 4096 / 1536 layer, 137 against 121 us
//          at B = 8);
//   down, B <= 2: one row per wave, BF16-pair dot products, non-temporal;
//   down, B 3..5: 4 rows per wave, FP32 math; B 6..55: 8 rows per wave;
//   down, B 24..512 (B * K <= 4096): the expert form on the matrix cores, one
//          16-wave workgroup per 16 outputs and token range, the batch cut in
//          two ranges when H / 16 workgroups would leave CUs idle (equal at
//          B = 24, 42 against 46 us at B = 28, 44 against 49 at B = 32, 58
//          against 83 at B = 64; at B = 16 the token form wins, 32 against 32.3);
//          with scratch for the expert split from B = 13 (Qwen-3 layer, split
//          against the token form: B = 13 27.8 against 30.0 us, B = 16 30.5
//          against 32.0, B = 20 33.7 against 35.3; B = 12 26.7 against 23.2);
//          past 64 tokens one 8-wave workgroup per range of up to 128 tokens and
//          1,024 slots, in 1, 2 or 4 ranges (B = 128 68 us, 256 102, 512 190,
//          where the token form took 139, 246 and 443).
// The token-form down keeps K * I / 1024 act chunks per lane in registers; past
// 6 (K * I > 6144) its FP32-math variants need more than 200 VGPRs (one or two
// waves per SIMD), so there it takes the BF16-pair math, 2 B rows per wave at
// B <= 2 (the 128-expert / top-8 / H 4096 / I 1536 layer: 10.0 against 12.4 us
// at B = 1, 16.1 against 17.5 at B = 2) and, from B = 3, the matrix-core form
// (26.5 against 30.7 us at B = 3, 35.0 against 44.9 at B = 5, 43 against 49 at
// B = 8, where the FP32 math took 225 us; the token form ahead at B = 2, 16.5
// against 21.0).
// form4_ok: the gate/up kernel that streams codes into LDS applies (rows of a multiple of 256
// elements, 4-byte-aligned scale bytes, x within one 2 GB buffer resource).
// have_scratch: the down kernel was given scratch for its expert split.
int resolve(const wd_launch *in, int B, int K, int E, int H, int I, bool down, wd_launch *out,
            bool form4_ok = false, bool have_scratch = false) {
    wd_launch c = in ? *in : wd_launch{};
    const bool batch = down ? B >= 3 : B >= 5;
    const bool wide = (long long)K * I > 6144;      // down: more than 6 act chunks per lane
    // B >= 24: gate/up in the expert form on the matrix cores, whose weight stream
    // is read once per expert however many tokens share it
    const bool untuned = c.rows_per_wave == 0 && c.lanes_per_row == 0 && c.math == 0 && c.weight_loads == 0;
    if (c.form == 0) {
        const bool mfma = down ? untuned && c.waves_per_block == 0 && B >= (wide ? 3 : have_scratch ? 13 : 24) &&
                                     down_min_ranges(B, K) > 0 && E <= wd::kDnMfmaMaxE
                               : untuned && (B >= 18 || (H >= 4096 && B >= 4));
        c.form = mfma ? 3 : 1;
    }
    if (c.form >= 3 && c.rows_per_wave == 0) c.rows_per_wave = 1;   // one 16-row block per wave
    if (c.rows_per_wave == 0)
        c.rows_per_wave = !batch ? (down && wide ? 2 * B : 1) : down ? (B >= 6 ? 8 : 4) : c.form == 2 ? 2 : 4;
    if (down && c.form == 3) {
        // two token ranges when one workgroup per 16 outputs would leave CUs idle, with 16
        // waves (Qwen-3 layer, B = 32: 44 us against 56 with 8); one range with 8 waves, which
        // take slots in groups of 8 where 16 waves take them in groups of 4, each group
        // streaming the expert's rows once (4096 / 1536 layer, Zipf routing: B = 8 43 against
        // 45 us, B = 32 98 against 118)
        // With scratch for the partial sums, the two workgroups of a block split the experts
        // instead (even / odd ids, all tokens each): every Wd row is read once, and each
        // workgroup streams about half the routed experts where a token range streams the
        // union of its tokens' experts, about two thirds of them at B = 32.
        // A range past 64 tokens or 512 slots takes the 8-wave variant with room for 128 tokens
        // and 1,024 slots; past 128 tokens or 1,024 slots the batch is cut into the fewest
        // ranges of that size (each range streams the experts its tokens use; the ranges of a
        // block sit on one XCD, so a second read of shared rows can come from the L2).
        const int smin = down_min_ranges(B, K);
        const bool few_blocks = H / 16 < 256 && B >= 2;
        if (c.expert_split == 0)
            c.expert_split = (have_scratch && few_blocks && smin == 1 && (c.token_split == 0 || c.token_split == 1))
                                 ? 2 : 1;
        if (c.token_split == 0)
            c.token_split = smin > 1 ? smin
                                     : (few_blocks && c.expert_split == 1 && !down_big_range(B, K)) ? 2 : 1;
        if (c.waves_per_block == 0)
            c.waves_per_block = (c.token_split > 1 && !down_big_range((B + c.token_split - 1) / c.token_split, K))
                                    ? 16 : 8;
    }
    // gate/up on the matrix cores: the H axis split over a pair of waves (needs whole 256-element
    // batches in each half).  Default from H = 4096, where a wave's 16 or more weight batches made
    // the last waves of a launch a long tail (128-expert / H 4096 / I 1536 layer, Zipf routing:
    // B = 8 96 -> 85 us, B = 16 141 -> 125, B = 32 187 -> 171); at H = 2048 (8 batches per wave)
    // the pair's fixed costs outweigh it (Qwen-3 layer: B = 32 70 -> 72 us, B = 64 77 -> 82)
    if (c.h_split == 0)
        c.h_split = (!down && c.form == 3 && H >= 4096 && H % 512 == 0 &&
                     (c.waves_per_block == 0 || c.waves_per_block == 2)) ? 2 : 1;
    if (c.h_split != 1 && c.h_split != 2) return WD_ERR_UNSUPPORTED;
    if (c.h_split == 2) {
        if (down || c.form != 3 || H % 512 != 0) return WD_ERR_UNSUPPORTED;
        if (c.waves_per_block == 0) c.waves_per_block = 2;
        if (c.waves_per_block != 2) return WD_ERR_UNSUPPORTED;
    }
    if (c.waves_per_block == 0)
        c.waves_per_block = down ? (B == 1 ? 2 : 1) : (batch || c.form == 4 ? 4 : 1);
    // gate/up expert forms: expert-major order (consecutive waves stream consecutive row blocks
    // of one expert) with the hardware's round-robin workgroup placement, which deals every
    // expert's row blocks over all 8 XCDs, so the XCDs stay balanced whichever experts the batch
    // routes to.  Measured at B = 32 / 64 (us): Qwen-3 layer 71.7 / 77.0 (XCD-contiguous: 71.5 /
    // 76.3; row-block-major: 73.8 / 81.5); 4096 / 1536 layer with Zipf routing, B = 8 / 32:
    // 121 / 218 (XCD-contiguous: 132 / 228; row-block-major: 117 / 214).
    const bool expert_form = !down && c.form >= 2;
    if (c.order == 0) c.order = expert_form ? 2 : 1;
    if (c.xcd_remap == 0) c.xcd_remap = ((!down && !batch) || expert_form) ? 2 : 1;
    if (c.math == 0) c.math = (down && batch && !wide && c.form != 3) ? wd::kMathF32 : wd::kMathDot2;
    if (c.weight_loads == 0) {
        // non-temporal where it measured faster and the variant is compiled
        const bool nt_ok = c.math == wd::kMathDot2 && c.form == 1 &&
                           (down ? c.rows_per_wave <= 2
                                 : (c.lanes_per_row == 0 || c.lanes_per_row == 64 || c.lanes_per_row == 32));
        // gate/up's token form non-temporal up to 16 tokens, where few tokens share an expert row
        // (Qwen-3 layer B = 8 31.4 -> 28.8 us, B = 16 51.5 -> 50.8; at B = 32, where rows are
        // shared, 84.9 -> 96.0); the token-form down at one or two rows per wave (one token; the
        // 128-expert / H 4096 / I 1536 layer at B = 1: step 28.9 -> 28.3 us; cached B = 4 9.29
        // against 9.56 us)
        c.weight_loads = ((!batch || (!down && B <= 16)) && nt_ok) ? 2 : 1;
    }
    // 32 lanes per row hold at most 8 chunks each (H <= 4096); longer rows take 64
    if (c.lanes_per_row == 0)
        c.lanes_per_row =
            (!down && batch && c.form == 1 && c.math == wd::kMathDot2 && H <= 4096) ? 32 : 64;
    if (c.rows_per_wave != 1 && c.rows_per_wave != 2 && c.rows_per_wave != 4 && c.rows_per_wave != 8)
        return WD_ERR_UNSUPPORTED;
    // down on the matrix cores: one workgroup of 8 or 16 waves per block of 16 outputs
    if (down && c.form == 3) {
        if (c.waves_per_block != 8 && c.waves_per_block != 16) return WD_ERR_UNSUPPORTED;
    } else if (c.waves_per_block < 1 || c.waves_per_block > 4) {
        return WD_ERR_UNSUPPORTED;
    }
    if (c.order != 1 && c.order != 2 && !(c.order == 3 && !down && c.form >= 2)) return WD_ERR_UNSUPPORTED;
    if (c.xcd_remap != 1 && c.xcd_remap != 2) return WD_ERR_UNSUPPORTED;
    if (c.math != wd::kMathF32 && c.math != wd::kMathDot2) return WD_ERR_UNSUPPORTED;
    if (c.lanes_per_row != 16 && c.lanes_per_row != 32 && c.lanes_per_row != 64) return WD_ERR_UNSUPPORTED;
    if (c.form < 1 || c.form > 4) return WD_ERR_UNSUPPORTED;
    if (c.form == 4 && (down || !form4_ok || (c.waves_per_block != 2 && c.waves_per_block != 4)))
        return WD_ERR_UNSUPPORTED;
    if (c.weight_loads != 1 && c.weight_loads != 2) return WD_ERR_UNSUPPORTED;
    if (down && (c.lanes_per_row != 64 || c.form == 2)) return WD_ERR_UNSUPPORTED;
    if (c.form == 2 && (c.lanes_per_row != 64 || c.math != wd::kMathDot2 || c.weight_loads != 1))
        return WD_ERR_UNSUPPORTED;
    // matrix-core expert form: fixed 16-row blocks and lane layout, BF16 operands; the knob stays 1
    // (form 3 loads its codes non-temporally in any case)
    if (c.form >= 3 && (c.rows_per_wave != 1 || c.lanes_per_row != 64 || c.math != wd::kMathDot2 ||
                        c.weight_loads != 1))
        return WD_ERR_UNSUPPORTED;
    // token ranges per 16-output block: the matrix-core down only
    if (c.token_split == 0) c.token_split = 1;
    if (c.token_split != 1 && c.token_split != 2 && c.token_split != 4) return WD_ERR_UNSUPPORTED;
    if (c.token_split != 1 && !(down && c.form == 3)) return WD_ERR_UNSUPPORTED;
    if (c.lds_bytes < 0 || c.lds_bytes > 65536) return WD_ERR_UNSUPPORTED;
    // slots per pass of the matrix-core gate/up over an expert's rows: 16 or 32.  Default 32
    // from B = 16: an expert with 17..32 slots is streamed once instead of twice (4096 / 1536
    // layer, Zipf routing: B = 16 164 -> 156 us, B = 32 218 -> 198 us; Qwen-3 layer B = 24..64
    // within 1%, where no expert has more than 16 slots); below, 16 (fewer registers; B = 8..12
    // 1-2% faster)
    if (c.slots_per_pass == 0) c.slots_per_pass = (!down && c.form == 3 && B >= 16) ? 32 : 16;
    if (c.slots_per_pass != 16 && c.slots_per_pass != 32) return WD_ERR_UNSUPPORTED;
    if (c.slots_per_pass == 32 && !(!down && c.form == 3)) return WD_ERR_UNSUPPORTED;
    // the expert split: the matrix-core down only, with scratch, not combined with token ranges
    if (c.expert_split == 0) c.expert_split = 1;
    if (c.expert_split != 1 && c.expert_split != 2) return WD_ERR_UNSUPPORTED;
    if (c.expert_split == 2 && !(down && c.form == 3 && have_scratch && c.token_split == 1)) return WD_ERR_UNSUPPORTED;
    *out = c;
    return WD_OK;
}

int launched() {
    return hipGetLastError() == hipSuccess ? WD_OK : WD_ERR_LAUNCH;
}

// ---- runtime -> compile-time dispatch ------------------------------------

// The kernels launched through launch(): leading scalar arguments (WD_LEAD_PARAMS), then LayerArgs.
typedef void (*KernelFn)(const int32_t *, int, int, int, int, int, int, int, int, uint32_t, int, LayerArgs);

template <int... V>
struct Ints {};

// Calls f(std::integral_constant<int, v>) for the v in the list equal to the
// runtime value, or returns nullptr.
template <int V0, int... Vs, class F>
KernelFn dispatch(int v, Ints<V0, Vs...>, F f) {
    if (v == V0) return f(std::integral_constant<int, V0>{});
    if constexpr (sizeof...(Vs) > 0) return dispatch(v, Ints<Vs...>{}, f);
    else return nullptr;
}

// Which variants are compiled.  Token-form gate/up: every chunk count, row
// count and tail; FP32 math only with 64 lanes per row and cached loads,
// non-temporal loads with 32 or 64 lanes per row.  Expert form: register use
// limits R * CPL to 8.  Down: non-temporal loads only at one row per wave.
template <int CPL, int R, int LPR, int M, int NT>
constexpr bool gate_up_compiled() {
    if (R == 8) return false;
    if (M == wd::kMathF32) return LPR == 64 && NT == 0;
    return NT == 0 || LPR == 64 || LPR == 32;
}
template <int CPL, int R>
constexpr bool gate_up_expert_compiled() { return R <= 4 && R * CPL <= 8; }
template <int CPL, int R, int M, int NT>
constexpr bool down_compiled() { return NT == 0 || (R <= 2 && M == wd::kMathDot2); }

KernelFn gate_up_fn(int cpl, int R, int lpr, int tail, int math, int nt) {
    return dispatch(cpl, Ints<1, 2, 4, 8>{}, [&](auto C) {
        return dispatch(R, Ints<1, 2, 4>{}, [&](auto Rv) {
            return dispatch(lpr, Ints<16, 32, 64>{}, [&](auto L) {
                return dispatch(tail, Ints<0, 1>{}, [&](auto T) {
                    return dispatch(math, Ints<wd::kMathF32, wd::kMathDot2>{}, [&](auto M) {
                        return dispatch(nt, Ints<0, 1>{}, [&](auto N) -> KernelFn {
                            if constexpr (gate_up_compiled<C, Rv, L, M, N>())
                                return wd::gate_up_kernel<C, Rv, L, T != 0, M, N != 0>;
                            else
                                return nullptr;
                        });
                    });
                });
            });
        });
    });
}

KernelFn gate_up_expert_fn(int cpl, int R, int tail) {
    return dispatch(cpl, Ints<1, 2, 4, 8>{}, [&](auto C) {
        return dispatch(R, Ints<1, 2, 4>{}, [&](auto Rv) {
            return dispatch(tail, Ints<0, 1>{}, [&](auto T) -> KernelFn {
                if constexpr (gate_up_expert_compiled<C, Rv>())
                    return wd::gate_up_expert_kernel<C, Rv, T != 0>;
                else
                    return nullptr;
            });
        });
    });
}

KernelFn down_fn(int cpl, int R, int tail, int math, int nt) {
    return dispatch(cpl, Ints<1, 2, 3, 4, 6, 8, 12, 16>{}, [&](auto C) {
        return dispatch(R, Ints<1, 2, 4, 8>{}, [&](auto Rv) {
            return dispatch(tail, Ints<0, 1>{}, [&](auto T) {
                return dispatch(math, Ints<wd::kMathF32, wd::kMathDot2>{}, [&](auto M) {
                    return dispatch(nt, Ints<0, 1>{}, [&](auto N) -> KernelFn {
                        if constexpr (down_compiled<C, Rv, M, N>())
                            return wd::down_kernel<C, Rv, T != 0, M, N != 0>;
                        else
                            return nullptr;
                    });
                });
            });
        });
    });
}

KernelFn gate_up_mfma_fn(bool sc8, int ngmax, int hs) {
    return dispatch(sc8 ? 1 : 0, Ints<0, 1>{}, [&](auto S) {
        return dispatch(ngmax, Ints<1, 2>{}, [&](auto N) {
            return dispatch(hs, Ints<1, 2>{}, [&](auto Hs) -> KernelFn {
                return wd::gate_up_mfma_kernel<S != 0, N, Hs>;
            });
        });
    });
}

// Smallest compiled chunks-per-lane >= need.
int round_cpl_gate_up(int need) {
    for (int c : {1, 2, 4, 8}) if (c >= need) return c;
    return -1;
}
int round_cpl_down(int need) {
    for (int c : {1, 2, 3, 4, 6, 8, 12, 16}) if (c >= need) return c;
    return -1;
}

int launch(KernelFn fn, LayerArgs a, const wd_launch &c, hipStream_t s) {
    const int blocks = (a.nwaves + c.waves_per_block - 1) / c.waves_per_block;
    a.nblocks = blocks;
    a.wpb = c.waves_per_block;
    const unsigned lds = (unsigned)c.lds_bytes;
    // the leading arguments repeat the fields a wave needs before its first routing-id load
    if (c.start_event || c.stop_event)
        hipExtLaunchKernelGGL(fn, dim3(blocks), dim3(64 * c.waves_per_block), lds, s,
                              (hipEvent_t)c.start_event, (hipEvent_t)c.stop_event, 0, a.ids, a.nwaves, a.nblocks,
                              a.wpb, a.remap, a.order, a.B, a.K, a.nrowblk, a.nci_magic, a.I, a);
    else
        hipLaunchKernelGGL(fn, dim3(blocks), dim3(64 * c.waves_per_block), lds, s, a.ids, a.nwaves, a.nblocks,
                           a.wpb, a.remap, a.order, a.B, a.K, a.nrowblk, a.nci_magic, a.I, a);
    return launched();
}

int gate_up_impl(const uint16_t *x, const int32_t *ids, const uint8_t *w_gu, const uint8_t *s_gu,
                 uint16_t *act, int B, int K, int E, int H, int I, const wd_launch *cfg,
                 void *stream, bool checked_device, void *zero_ptr = nullptr, int zero_n = 0) {
    int rc = check_dims(B, K, E, H, I);
    if (rc) return rc;
    if (!w_gu || !s_gu) return WD_ERR_NULL;
    if (B > 0 && (!x || !ids || !act)) return WD_ERR_NULL;
    if (!aligned(w_gu, 16) || (B > 0 && (!aligned(x, 16) || !aligned(act, 16) || !aligned(ids, 4))))
        return WD_ERR_ALIGN;
    wd_launch c;
    const bool form4_ok = H % 256 == 0 && aligned(s_gu, 4) && (long long)B * H * 2 <= 0x7FFF0000LL;
    if ((rc = resolve(cfg, B, K, E, H, I, false, &c, form4_ok))) return rc;
    const int lpr = c.lanes_per_row;
    const int cpl = round_cpl_gate_up((H / 16 + lpr - 1) / lpr);
    if (cpl < 0) return WD_ERR_UNSUPPORTED;
    const int rows_per_wave = c.form >= 3 ? 16 : (64 / lpr) * c.rows_per_wave;
    if (I % rows_per_wave) return WD_ERR_UNSUPPORTED;
    const bool tail = (H / 16) % (lpr * cpl) != 0;
    // rows of a multiple of 8 E8M0 bytes: every batch's 8 bytes lie inside its row, one load
    const bool sc8 = (H / 32) % 8 == 0 && aligned(s_gu, 4);
    KernelFn fn = c.form == 4   ? (c.waves_per_block == 2 ? wd::gate_up_mfma_lds_kernel<2>
                                                          : wd::gate_up_mfma_lds_kernel<4>)
                  : c.form == 3 ? gate_up_mfma_fn(sc8, c.slots_per_pass == 32 ? 2 : 1, c.h_split)
                  : c.form == 2 ? gate_up_expert_fn(cpl, c.rows_per_wave, tail)
                                : gate_up_fn(cpl, c.rows_per_wave, lpr, tail, c.math, c.weight_loads == 2);
    if (!fn) return WD_ERR_UNSUPPORTED;
    if (B == 0) return WD_OK;
    if (!checked_device && (rc = check_device())) return rc;
    LayerArgs a{};
    a.x = x; a.ids = ids; a.w = w_gu; a.s = s_gu; a.out = act;
    a.B = B; a.K = K; a.E = E; a.H = H; a.I = I;
    a.nrowblk = I / rows_per_wave;
    a.nwaves = (c.form == 1 ? B * K : E) * a.nrowblk * (c.form == 3 ? c.h_split : 1);
    a.order = c.order; a.remap = c.xcd_remap;
    a.zero_ptr = static_cast<uint4 *>(zero_ptr); a.zero_n = zero_ptr ? zero_n : 0;
    return launch(fn, a, c, (hipStream_t)stream);
}

// Bytes of the down kernel's expert-split scratch: one 8-byte cell per output,
// [H/16][B][16].
size_t down_scratch_bytes(int B, int H) { return (size_t)B * H * 8; }
size_t round256(size_t n) { return (n + 255) / 256 * 256; }

int down_impl(const uint16_t *act, const int32_t *ids, const float *tw, const uint8_t *w_d,
              const uint8_t *s_d, uint16_t *out, int B, int K, int E, int H, int I,
              const wd_launch *cfg, void *stream, bool checked_device,
              void *scratch_in, size_t scratch_bytes_in);

// Both kernels of one layer step on `stream`, act[B,K,I] at the start of `ws`; when `ws` also
// holds the down kernel's expert-split scratch after it, the gate/up kernel's workgroups clear
// that scratch first (the down kernel leaves it zero again).  Arguments already checked.
int layer(const uint16_t *x, const int32_t *ids, const float *tw, const uint8_t *w_gu, const uint8_t *s_gu,
          const uint8_t *w_d, const uint8_t *s_d, void *ws, size_t ws_bytes, uint16_t *out,
          int B, int K, int E, int H, int I, void *stream) {
    uint16_t *act = static_cast<uint16_t *>(ws);
    const size_t act_bytes = round256((size_t)B * K * I * 2u);
    uint8_t *scr = nullptr;
    size_t scr_bytes = 0;
    if (ws_bytes >= act_bytes + down_scratch_bytes(B, H) && aligned(ws, 256)) {
        scr = static_cast<uint8_t *>(ws) + act_bytes;
        scr_bytes = ws_bytes - act_bytes;
    }
    int rc = gate_up_impl(x, ids, w_gu, s_gu, act, B, K, E, H, I, nullptr, stream, true, scr,
                          (int)(down_scratch_bytes(B, H) / 16));
    if (rc) return rc;
    return down_impl(act, ids, tw, w_d, s_d, out, B, K, E, H, I, nullptr, stream, true, scr, scr_bytes);
}

int down_impl(const uint16_t *act, const int32_t *ids, const float *tw, const uint8_t *w_d,
              const uint8_t *s_d, uint16_t *out, int B, int K, int E, int H, int I,
              const wd_launch *cfg, void *stream, bool checked_device,
              void *scratch_in, size_t scratch_bytes_in) {
    int rc = check_dims(B, K, E, H, I);
    if (rc) return rc;
    if (!w_d || !s_d) return WD_ERR_NULL;
    if (B > 0 && (!act || !ids || !tw || !out)) return WD_ERR_NULL;
    if (!aligned(w_d, 16) ||
        (B > 0 && (!aligned(act, 16) || !aligned(ids, 4) || !aligned(tw, 4) || !aligned(out, 2))))
        return WD_ERR_ALIGN;
    // scratch for the expert split: the caller's (wd_launch.down_scratch) or the layer workspace's
    void *scr = scratch_in;
    size_t scr_bytes = scratch_bytes_in;
    if (cfg && cfg->down_scratch) { scr = cfg->down_scratch; scr_bytes = cfg->down_scratch_bytes; }
    const bool have_scratch = scr && aligned(scr, 256) && B > 0 && scr_bytes >= down_scratch_bytes(B, H);
    wd_launch c;
    if ((rc = resolve(cfg, B, K, E, H, I, true, &c, false, have_scratch))) return rc;
    if (c.form == 3) {
        // every slot's id held in registers (8 per lane), per-wave accumulators for 64 tokens,
        // expert ids packed in 10 bits
        // every wave keeps the ids of its token range's slots in registers: a range of up to 64
        // tokens and 512 slots, or with the 8-wave 1,024-slot variant up to 128 and 1,024
        const int tpr = (B + c.token_split - 1) / c.token_split;
        if (tpr > wd::kDnMfmaMaxBWide || (long long)tpr * K > wd::kDnMfmaMaxSlotsWide || E > wd::kDnMfmaMaxE)
            return WD_ERR_UNSUPPORTED;
        const bool big = down_big_range(tpr, K);
        if (big && c.waves_per_block != 8) return WD_ERR_UNSUPPORTED;
        // rows of a multiple of 8 E8M0 bytes: every batch's 8 bytes lie inside its row, one load
        const bool sc8 = (I / 32) % 8 == 0 && aligned(s_d, 4);
        // 8 waves: groups of 8 slots; 16 waves (register budget of four waves per SIMD): 4
        constexpr int S = wd::kDnMfmaMaxSlots, SW = wd::kDnMfmaMaxSlotsWide;
        void (*fn)(const int32_t *, const float *, int, int, int, int, int, int, LayerArgs) =
            c.waves_per_block == 16 ? (sc8 ? wd::down_mfma_kernel<16, 4, true, S> : wd::down_mfma_kernel<16, 4, false, S>)
            : big                   ? (sc8 ? wd::down_mfma_kernel<8, 8, true, SW> : wd::down_mfma_kernel<8, 8, false, SW>)
                                    : (sc8 ? wd::down_mfma_kernel<8, 8, true, S> : wd::down_mfma_kernel<8, 8, false, S>);
        if (B == 0) return WD_OK;
        if (!checked_device && (rc = check_device())) return rc;
        LayerArgs a{};
        a.act_in = act; a.ids = ids; a.tw = tw; a.w = w_d; a.s = s_d; a.out = out;
        a.B = B; a.K = K; a.E = E; a.H = H; a.I = I;
        a.nrowblk = H / 16;
        a.tsplit = c.token_split;
        a.esplit = c.expert_split;
        if (c.expert_split > 1) a.dcell = static_cast<uint64_t *>(scr);
        const int blocks = a.nrowblk * c.token_split * c.expert_split;
        a.nwaves = blocks * c.waves_per_block;
        a.nblocks = blocks;
        a.wpb = c.waves_per_block;
        const hipStream_t st = (hipStream_t)stream;
        const unsigned lds = (unsigned)c.lds_bytes;
        // the leading arguments repeat what a workgroup needs to load its range's ids and weights
        if (c.start_event || c.stop_event)
            hipExtLaunchKernelGGL(fn, dim3(blocks), dim3(64 * c.waves_per_block), lds, st,
                                  (hipEvent_t)c.start_event, (hipEvent_t)c.stop_event, 0, a.ids, a.tw, a.nrowblk,
                                  a.esplit, a.tsplit, a.B, a.K, a.E, a);
        else
            hipLaunchKernelGGL(fn, dim3(blocks), dim3(64 * c.waves_per_block), lds, st, a.ids, a.tw, a.nrowblk,
                               a.esplit, a.tsplit, a.B, a.K, a.E, a);
        return launched();
    }
    const int nc = K * (I / 16);
    const int cpl = round_cpl_down((nc + 63) / 64);
    if (cpl < 0) return WD_ERR_UNSUPPORTED;
    if (H % c.rows_per_wave) return WD_ERR_UNSUPPORTED;
    // Chunk -> slot division by multiply and shift: with magic = floor(2^22 / nci) + 1,
    // (cc * magic) >> 22 == cc / nci for every cc < 1024 whenever nci <= 1024 (the
    // rounding excess cc * (magic - 2^22 / nci) / 2^22 < 2^-12 cannot reach the next
    // integer, whose distance is at least 1 / nci >= 2^-10).  check_dims bounds
    // K * I <= 16384, so nc = K * I / 16 <= 1024 and nci <= 1024.
    const uint32_t nci = (uint32_t)(I / 16);
    const uint32_t magic = (uint32_t)((1u << 22) / nci + 1);
    const bool tail = nc % (64 * cpl) != 0;
    KernelFn fn = down_fn(cpl, c.rows_per_wave, tail, c.math, c.weight_loads == 2);
    if (!fn) return WD_ERR_UNSUPPORTED;
    if (B == 0) return WD_OK;
    if (!checked_device && (rc = check_device())) return rc;
    LayerArgs a{};
    a.act_in = act; a.ids = ids; a.tw = tw; a.w = w_d; a.s = s_d; a.out = out;
    a.B = B; a.K = K; a.E = E; a.H = H; a.I = I;
    a.nrowblk = H / c.rows_per_wave;
    a.nwaves = B * a.nrowblk;
    a.order = c.order; a.remap = c.xcd_remap;
    a.nci_magic = magic;
    return launch(fn, a, c, (hipStream_t)stream);
}

}  // namespace

extern "C" {

int wd_gate_up(const uint16_t *x, const int32_t *topk_ids, const uint8_t *w_gu, const uint8_t *s_gu,
               uint16_t *act, int B, int K, int E, int H, int I, void *stream) {
    return gate_up_impl(x, topk_ids, w_gu, s_gu, act, B, K, E, H, I, nullptr, stream, false);
}

int wd_gate_up_ex(const uint16_t *x, const int32_t *topk_ids, const uint8_t *w_gu, const uint8_t *s_gu,
                  uint16_t *act, int B, int K, int E, int H, int I, const wd_launch *cfg, void *stream) {
    return gate_up_impl(x, topk_ids, w_gu, s_gu, act, B, K, E, H, I, cfg, stream, false);
}

int wd_down(const uint16_t *act, const int32_t *topk_ids, const float *topk_w, const uint8_t *w_d,
            const uint8_t *s_d, uint16_t *out, int B, int K, int E, int H, int I, void *stream) {
    return down_impl(act, topk_ids, topk_w, w_d, s_d, out, B, K, E, H, I, nullptr, stream, false, nullptr, 0);
}

int wd_down_ex(const uint16_t *act, const int32_t *topk_ids, const float *topk_w, const uint8_t *w_d,
               const uint8_t *s_d, uint16_t *out, int B, int K, int E, int H, int I,
               const wd_launch *cfg, void *stream) {
    return down_impl(act, topk_ids, topk_w, w_d, s_d, out, B, K, E, H, I, cfg, stream, false, nullptr, 0);
}

size_t wd_workspace_bytes(int B, int K, int I) {
    if (B < 0 || K < 1 || I < 32 || I % 32) return 0;
    return (size_t)B * (size_t)K * (size_t)I * 2u;
}

size_t wd_down_scratch_bytes(int B, int H) {
    if (B < 1 || H < 32 || H % 32) return 0;
    return down_scratch_bytes(B, H);
}

size_t wd_layer_workspace_bytes(int B, int K, int H, int I) {
    const size_t act = wd_workspace_bytes(B, K, I);
    if (B < 1 || act == 0 || H < 32 || H % 32) return act;
    return round256(act) + down_scratch_bytes(B, H);
}

int wd_moe_decode(const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
                  const uint8_t *w_gu, const uint8_t *s_gu, const uint8_t *w_d, const uint8_t *s_d,
                  void *workspace, size_t workspace_bytes, uint16_t *out,
                  int B, int K, int E, int H, int I, void *stream) {
    int rc = check_dims(B, K, E, H, I);
    if (rc) return rc;
    if (!w_gu || !s_gu || !w_d || !s_d) return WD_ERR_NULL;
    if (B > 0 && (!x || !topk_ids || !topk_w || !out || !workspace)) return WD_ERR_NULL;
    if (B > 0 && !aligned(workspace, 16)) return WD_ERR_ALIGN;
    if (workspace_bytes < wd_workspace_bytes(B, K, I)) return WD_ERR_WORKSPACE;
    uint16_t *act = static_cast<uint16_t *>(workspace);
    // Check both halves' arguments before launching either.
    if (!aligned(w_gu, 16) || !aligned(w_d, 16) ||
        (B > 0 && (!aligned(x, 16) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(out, 2))))
        return WD_ERR_ALIGN;
    if (B == 0) return WD_OK;
    if ((rc = check_device())) return rc;
    return layer(x, topk_ids, topk_w, w_gu, s_gu, w_d, s_d, workspace, workspace_bytes, out, B, K, E, H, I, stream);
}

}  // extern "C"

// ---- the entry point that allocates nothing ---------------------------------
//
// wd_moe_decode_noalloc keeps the intermediate act[B,K,I] in this file-scope
// device array instead of a caller workspace.  Each GPU the library runs on
// holds its own copy for the life of the process.  In host code the name
// `scratch` is only a host-side stand-in: its device address is looked up with
// hipGetSymbolAddress once per device (with that device current) and only that
// address is handed to the kernels.
static __device__ __align__(256) uint8_t scratch[WD_NOALLOC_SCRATCH_BYTES];

namespace {

std::atomic<void *> g_scratch[kMaxDevices];   // device address of `scratch`, per device

// Device address of the current device's scratch array (nullptr on failure).
void *scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) { (void)hipGetLastError(); return nullptr; }
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        // two threads racing here both store the same address
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" {

int wd_moe_decode_noalloc(const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
                          const uint8_t *w_gu, const uint8_t *s_gu, const uint8_t *w_d, const uint8_t *s_d,
                          uint16_t *out, int B, int K, int E, int H, int I, void *stream) {
    int rc = check_dims(B, K, E, H, I);
    if (rc) return rc;
    if (!w_gu || !s_gu || !w_d || !s_d) return WD_ERR_NULL;
    if (B > 0 && (!x || !topk_ids || !topk_w || !out)) return WD_ERR_NULL;
    if (wd_workspace_bytes(B, K, I) > (size_t)WD_NOALLOC_SCRATCH_BYTES) return WD_ERR_SCRATCH;
    if (!aligned(w_gu, 16) || !aligned(w_d, 16) ||
        (B > 0 && (!aligned(x, 16) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(out, 2))))
        return WD_ERR_ALIGN;
    if (B == 0) return WD_OK;
    if ((rc = check_device())) return rc;
    void *ws = scratch_ptr();
    if (!ws) return WD_ERR_DEVICE;
    // act at the start; the down kernel's expert-split scratch after it when it fits (its
    // cells cleared by the gate/up kernel); gate/up writes every act element the down kernel
    // reads, so nothing else is cleared
    return layer(x, topk_ids, topk_w, w_gu, s_gu, w_d, s_d, ws, (size_t)WD_NOALLOC_SCRATCH_BYTES, out,
                 B, K, E, H, I, stream);
}

const char *wd_status_string(int status) {
    switch (status) {
        case WD_OK: return "ok";
        case WD_ERR_NULL: return "null pointer argument";
        case WD_ERR_DIMS: return "bad dimensions (need B >= 0, K >= 1, E >= 1, H and I positive multiples of 32)";
        case WD_ERR_ALIGN: return "misaligned pointer (16 bytes for x, weights, act, workspace; 4 for ids and weights; 2 for out)";
        case WD_ERR_WORKSPACE: return "workspace smaller than wd_workspace_bytes(B, K, I)";
        case WD_ERR_DEVICE: return "no HIP device, or the current device is not gfx950";
        case WD_ERR_LAUNCH: return "kernel launch failed";
        case WD_ERR_UNSUPPORTED: return "unsupported sizes or launch configuration (H <= 8192, K*I <= 16384)";
        case WD_ERR_SCRATCH:
            return "act[B,K,I] (B*K*I*2 bytes) exceeds the no-allocation scratch (WD_NOALLOC_SCRATCH_BYTES = 4 MiB)";
    }
    return "unknown status";
}

int wd_route(const float *logits, int B, int E, int K, int32_t *topk_ids, float *topk_w, void *stream) {
    if (B < 0 || E < 1 || K < 1 || K > E) return WD_ERR_DIMS;
    if (E > 1024 || K > 64) return WD_ERR_UNSUPPORTED;
    if (B > 0 && (!logits || !topk_ids || !topk_w)) return WD_ERR_NULL;
    if (B > 0 && (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4))) return WD_ERR_ALIGN;
    if (B == 0) return WD_OK;
    int rc = check_device();
    if (rc) return rc;
    const int rpl = (E + 63) / 64;
    void (*fn)(const float *, int, int, int, int32_t *, float *) =
        rpl <= 1 ? wd::route_kernel<1> : rpl <= 2 ? wd::route_kernel<2> : rpl <= 4 ? wd::route_kernel<4>
        : rpl <= 8 ? wd::route_kernel<8> : wd::route_kernel<16>;
    const int wpb = 4;
    hipLaunchKernelGGL(fn, dim3((B + wpb - 1) / wpb), dim3(64 * wpb), 0, (hipStream_t)stream,
                       logits, B, E, K, topk_ids, topk_w);
    return launched();
}

int wd_dequant_probe(float *out, void *stream) {
    if (!out) return WD_ERR_NULL;
    if (!aligned(out, 16)) return WD_ERR_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    hipLaunchKernelGGL(wd::dequant_probe_kernel, dim3(256), dim3(256), 0, (hipStream_t)stream, out);
    return launched();
}

int wd_stream_blocks(void) { return 256 * 32; }

int wd_stream_read(const void *buf, size_t bytes, uint32_t *sink, int blocks, int unroll, void *start_event,
                   void *stop_event, void *stream) {
    if (!buf || !sink) return WD_ERR_NULL;
    if (bytes % 16 || !aligned(buf, 16) || !aligned(sink, 4)) return WD_ERR_ALIGN;
    if (blocks <= 0) blocks = wd_stream_blocks();
    if (blocks > wd_stream_blocks()) return WD_ERR_UNSUPPORTED;
    void (*fn)(const wd::u32x4 *, size_t, uint32_t *, uint32_t) = nullptr;
    switch (unroll) {
        case 1: fn = wd::stream_read_kernel<1>; break;
        case 2: fn = wd::stream_read_kernel<2>; break;
        case 4: fn = wd::stream_read_kernel<4>; break;
        case 8: fn = wd::stream_read_kernel<8>; break;
        default: return WD_ERR_UNSUPPORTED;
    }
    int rc = check_device();
    if (rc) return rc;
    const wd::u32x4 *b16 = static_cast<const wd::u32x4 *>(buf);
    if (start_event || stop_event)
        hipExtLaunchKernelGGL(fn, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (hipEvent_t)start_event,
                              (hipEvent_t)stop_event, 0, b16, bytes / 16, sink, 0x9E3779B9u);
    else
        hipLaunchKernelGGL(fn, dim3(blocks), dim3(256), 0, (hipStream_t)stream, b16, bytes / 16, sink, 0x9E3779B9u);
    return launched();
}

int wd_stream_copy(void *dst, const void *src, size_t bytes, int blocks, void *stream) {
    if (!dst || !src) return WD_ERR_NULL;
    if (bytes % 16 || !aligned(dst, 16) || !aligned(src, 16)) return WD_ERR_ALIGN;
    if (blocks <= 0) blocks = wd_stream_blocks();
    if (blocks > wd_stream_blocks()) return WD_ERR_UNSUPPORTED;
    int rc = check_device();
    if (rc) return rc;
    hipLaunchKernelGGL(wd::stream_copy_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<wd::u32x4 *>(dst), static_cast<const wd::u32x4 *>(src), bytes / 16);
    return launched();
}

int wd_gpu_sleep(int sleep_units, void *stream) {
    if (sleep_units < 0 || sleep_units > (1 << 20)) return WD_ERR_UNSUPPORTED;
    int rc = check_device();
    if (rc) return rc;
    hipLaunchKernelGGL(wd::sleep_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, sleep_units);
    return launched();
}

}  // extern "C"
