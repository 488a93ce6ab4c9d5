/*
 * wd.h — C ABI of the MI355X (gfx950) small-batch MoE decode layer in its
 * output-neuron-centric ("warp decode") form.
 *
 * The layer (warp-decode write-ups: "Better MoE model inference with warp
 * decode", TL;DR and Key claims, section "How the two kernels work"; the
 * Chinese summary "Cursor推出MoE推理加速方法Warp Decode", section 技术原理):
 *
 *     y[b] = sum_k topk_w[b,k] * Down_e( SiLU(Gate_e x[b]) (.) Up_e x[b] ),
 *            e = topk_ids[b,k],
 *
 * computed by two kernels: a gate/up kernel that writes the SiLU-gated
 * intermediate once as BF16, and a down kernel that folds the router weight
 * into its FP32 accumulator, so no per-expert output, padding, gather,
 * scatter or combine buffer exists.
 *
 * Data formats and layouts (all tensors dense, row-major, reduction axis
 * innermost):
 *   x        [B, H]        BF16 bit patterns (uint16)
 *   topk_ids [B, K]        int32 expert ids, each in [0, E); duplicates allowed
 *   topk_w   [B, K]        fp32 router weights, used as given (not renormalised)
 *   w_gu     [E, 2I, H]    MXFP8 element codes, OCP E4M3 "FN" (uint8);
 *                          rows [0, I) are the gate projection, rows [I, 2I)
 *                          the up projection
 *   s_gu     [E, 2I, H/32] OCP E8M0 block exponents (uint8), value 2^(s-127),
 *                          one per 32 consecutive elements of a row
 *   w_d      [E, H, I]     MXFP8 codes of the down projection
 *   s_d      [E, H, I/32]  E8M0 exponents of the down projection
 *   act      [B, K, I]     BF16 intermediate SiLU(g) * u, rounded to nearest even
 *   out      [B, H]        BF16 output, rounded to nearest even from FP32
 *
 * Arithmetic: MXFP8 weights are converted as they are read, to FP32 or to BF16
 * (whichever the kernel multiplies in; exact for every normal value),
 * activations stay BF16 in memory, all products and sums are FP32 (FMA, BF16
 * pair dot products or the BF16 matrix cores).  The summation order is fixed
 * by the kernel and its launch configuration, so repeated calls with the same
 * inputs give bit-identical results; under one configuration a token's
 * outputs do not depend on the other tokens' values or order (the defaults
 * pick the configuration from the batch size, so they can change with it).
 *
 * Ownership: the caller owns every buffer (device memory) and the stream; the
 * compute entry points allocate, free and synchronise nothing, so they may be
 * recorded into a HIP graph.  Work is enqueued on `stream` (a hipStream_t;
 * NULL is the default stream) and the call returns without waiting.
 *
 * Errors: every entry point returns WD_OK (0) or a negative status.  Argument
 * checks run on the host before any HIP call; nothing is launched when a check
 * fails.  A fault inside a kernel surfaces at the caller's next synchronising
 * HIP call.  An expert id outside [0, E) is not a host-checked precondition
 * (ids live in device memory); the kernels never read out of bounds for it:
 * its slot's intermediate row is written as NaN and every output of its token
 * becomes NaN.
 *
 * Size limits of this library: H and I multiples of 32, H <= 8192,
 * K * I <= 16384, B * K * I < 2^31.  B = 0 is accepted and launches nothing
 * (activation/output/routing pointers may then be NULL).
 */
#ifndef WD_H
#define WD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum wd_status {
    WD_OK = 0,
    WD_ERR_NULL = -1,        /* a required pointer is NULL */
    WD_ERR_DIMS = -2,        /* B < 0, K < 1, E < 1, H or I not a positive multiple of 32 */
    WD_ERR_ALIGN = -3,       /* x, w_gu, w_d, act, workspace not 16-byte aligned; ids, w not 4-byte; out not 2-byte */
    WD_ERR_WORKSPACE = -4,   /* workspace smaller than wd_workspace_bytes() */
    WD_ERR_DEVICE = -5,      /* no HIP device, or the current device is not gfx950 */
    WD_ERR_LAUNCH = -6,      /* the kernel launch was rejected by the HIP runtime */
    WD_ERR_UNSUPPORTED = -7, /* sizes beyond the library's limits, or a bad launch configuration */
    WD_ERR_SCRATCH = -8      /* wd_moe_decode_noalloc: act[B,K,I] larger than WD_NOALLOC_SCRATCH_BYTES */
};

/* Size of the device-resident scratch array that wd_moe_decode_noalloc uses
 * for act[B,K,I] (B * K * I * 2 bytes must fit): 4 MiB, e.g. 341 tokens of
 * the 128-expert / top-8 / I 768 layer, 128 tokens at K * I = 16384. */
#define WD_NOALLOC_SCRATCH_BYTES (4u << 20)

/* Launch configuration (tuning and timing).  Any integer field left 0 takes
 * the library default for the call's sizes.
 *   rows_per_wave    1, 2, 4 (or 8 for down): rows each lane group computes in
 *                    turn (a wave computes rows_per_wave * 64 / lanes_per_row
 *                    rows)
 *   waves_per_block  1..4: waves per workgroup (down on the matrix cores:
 *                    8 or 16)
 *   order            token forms: 1 = row-block major (the waves of all tokens
 *                    and slots for one block of rows are adjacent, so tokens
 *                    that share an expert re-read its rows while they are in
 *                    cache); 2 = token/slot major (one slot's rows are
 *                    adjacent).  Gate/up expert forms (2, 3, 4): 1 = row-block
 *                    major with a per-expert skew of the row block; 2 = expert
 *                    major (the default, with xcd_remap 2); 3 = row-block
 *                    major without the skew
 *   xcd_remap        1 = renumber workgroups so that each of the 8 XCDs gets
 *                    one contiguous range of the work order; 2 = keep the
 *                    hardware's round-robin numbering (the default for
 *                    gate/up below 5 tokens and for its expert forms)
 *   math             1 = MXFP8 pairs converted to FP32, FMA accumulation;
 *                    2 = MXFP8 pairs converted to BF16 (exact for normal
 *                    values), two products per v_dot2_f32_bf16 into the FP32
 *                    accumulator.  Both are FP32 accumulation of exact products.
 *   lanes_per_row    gate/up only: 16, 32 or 64 lanes share one row's dot
 *                    products, so a wave works on 64 / lanes_per_row rows at
 *                    once (down: 64); each lane holds at most 8 chunks of 16
 *                    elements, so 16 lanes take H <= 2048 and 32 lanes
 *                    H <= 4096 (the default uses 64 above that)
 *   form             gate/up only: 1 = one wave per (token, slot, row block);
 *                    2 = one wave per (expert, row block) serving every slot
 *                    routed to that expert, each weight row read and
 *                    converted once (requires lanes_per_row 64, math 2,
 *                    weight_loads 1); both forms give bit-identical results
 *                    for lanes_per_row 64 and math 2;
 *                    3 = one wave per (expert, block of 16 rows) on the BF16
 *                    matrix cores (v_mfma_f32_16x16x32_bf16): weights
 *                    converted exactly to BF16, x as stored, FP32
 *                    accumulation in the matrix core's summation order
 *                    (rows_per_wave 1, lanes_per_row 64, math 2,
 *                    weight_loads 1; waves_per_block and order apply as for
 *                    the other forms);
 *                    4 = form 3's work and arithmetic (bit-identical
 *                    results) with the codes loaded straight from memory
 *                    into a two-batch LDS ring per wave and x one batch
 *                    ahead in registers; needs H a multiple of 256, s_gu
 *                    4-byte aligned, B * H * 2 <= 0x7FFF0000 and 2 or 4
 *                    waves per workgroup (default 4).
 *                    Default: 3 when B >= 18 (B >= 4 when H >= 4096) and
 *                    none of rows_per_wave, lanes_per_row, math,
 *                    weight_loads is set, else 1.
 *                    down: 1 = one wave per (token, block of output dims);
 *                    3 = one workgroup of 8 or 16 waves (waves_per_block)
 *                    per block of 16 output dims serving every token (of
 *                    its token range, see token_split): the routed experts
 *                    are dealt to the waves in turn, each wave forms the
 *                    16 x slots tile of its experts on the BF16 matrix cores
 *                    (weights converted exactly, act as stored, FP32
 *                    accumulation) and keeps each slot's 16 values in LDS;
 *                    each output then folds its token's router weights in,
 *                    one FMA per slot in expert order (rows_per_wave 1,
 *                    lanes_per_row 64, math 2, weight_loads 1; E <= 1024;
 *                    each token range at most 128 tokens and 1,024 slots
 *                    with 8 waves, 64 tokens and 512 slots with 16).
 *                    Default: 3 when E <= 1024, none of rows_per_wave,
 *                    lanes_per_row, math, weight_loads, waves_per_block is
 *                    set, B >= 24 (B >= 13 with down_scratch; B >= 3 when
 *                    K * I > 6144) and the batch
 *                    fits 4 ranges (B <= 512, ceil(B / 4) * K <= 1024), else
 *                    1.  With form 3 the defaults are: when one range holds
 *                    the batch (B <= 128, B * K <= 1024), the expert split
 *                    (8 waves) if scratch is given and H / 16 < 256, else two
 *                    ranges of 16 waves if H / 16 < 256 and B <= 64, B * K <=
 *                    512, else one range of 8 waves; a larger batch takes the
 *                    fewest ranges (2 or 4) that hold it, 16 waves when each
 *                    range has at most 64 tokens and 512 slots, else 8.
 *   weight_loads     token forms: 1 = cached weight loads; 2 = non-temporal
 *                    (the rows are streamed past the caches; gate/up: 32 or 64
 *                    lanes per row; down: one or two rows per wave).  0 =
 *                    default: 2 for gate/up up to 16 tokens and for the down
 *                    at one or two rows per wave (one token), else 1.
 *                    Forms 3 and 4 take 1 (form 3 always loads its weight
 *                    codes non-temporally: each pass reads an expert's rows
 *                    once)
 *   token_split      down, form 3 only: 1, 2 or 4 workgroups per block of 16
 *                    output dims, each serving its own contiguous range of
 *                    ceil(B / token_split) tokens (an expert shared by
 *                    several ranges is read once per range; the output does
 *                    not depend on it bit for bit).  0 = default: the fewest
 *                    ranges that hold the batch when one does not, else 2
 *                    when H / 16 < 256 (fewer blocks than the 256 CUs), the
 *                    expert split is off and the batch has at most 64 tokens
 *                    and 512 slots, else 1.
 *   lds_bytes        extra LDS per workgroup requested at launch (0..65536),
 *                    unused by the kernel: fewer workgroups then share a CU
 *                    (an occupancy knob for tuning)
 *   expert_split     down, form 3 only: 2 = two workgroups per block of 16
 *                    output dims, one for the experts with even ids and one
 *                    for odd, all tokens each; each workgroup keeps its
 *                    class's partial sums in FP32, the two hand them over
 *                    through one scratch cell per output (an atomic
 *                    exchange), and whichever comes second adds them (class
 *                    0 + class 1) and writes the output, so every Wd row is
 *                    read once.  Needs
 *                    down_scratch (not combined with token_split > 1).
 *                    1 = off.  0 = default: 2 when down_scratch is given and
 *                    the token ranges would otherwise be used (H / 16 < 256,
 *                    B >= 2), else 1.
 *   down_scratch,    down: device memory for the expert split, at least
 *   down_scratch_bytes  wd_down_scratch_bytes(B, H) bytes, 256-byte aligned:
 *                    one 8-byte cell per output.  The cells the call uses
 *                    (the first wd_down_scratch_bytes(B, H) bytes) must be
 *                    zero before the first call; every call leaves them
 *                    zero.  Calls that overlap in time must not share it.
 *   slots_per_pass   gate/up, form 3 only: 16 = each pass over an expert's 16-row
 *                    block serves up to 16 of its slots (an expert with more
 *                    slots is streamed once per 16); 32 = up to 32 slots per pass
 *                    (two 16-slot tiles per weight batch; more registers, so
 *                    fewer resident waves).  Bit-identical results.  0 = default
 *                    (32 for form 3 from B = 16, else 16).
 *   h_split          gate/up, form 3 only: 1 = one wave per (expert, 16 rows) streams
 *                    the whole H axis; 2 = a workgroup of two waves per (expert, 16
 *                    rows), each streaming half of the H axis, the second handing its
 *                    FP32 sums to the first, which adds them (first half + second half)
 *                    and writes the results: half as many weight batches per wave, so
 *                    the last waves of a launch finish sooner.  Needs H a multiple of
 *                    512; waves_per_block must be 0 or 2.  0 = default: 2 from
 *                    H = 4096 (H a multiple of 512, waves_per_block 0 or 2), else 1.
 *   start_event,     optional hipEvent_t handles (created by the caller); when
 *   stop_event       set, the kernel's own dispatch records its start and end
 *                    time into them (hipExtLaunchKernelGGL), so the elapsed
 *                    time is the kernel's execution alone
 */
typedef struct wd_launch {
    int rows_per_wave;
    int waves_per_block;
    int order;
    int xcd_remap;
    void *start_event;
    void *stop_event;
    int math;
    int lanes_per_row;
    int form;
    int weight_loads;
    int token_split;
    int lds_bytes;
    int expert_split;
    void *down_scratch;
    size_t down_scratch_bytes;
    int slots_per_pass;
    int h_split;
} wd_launch;

/* Gate/up kernel (the summary's moe_gate_up_3d_batched; Key claims, section
 * "How the two kernels work"; the Chinese summary's "Gate/Up Kernel"):
 * act[b,k,j] = BF16(SiLU(g) * u) with g, u the dot products of x[b] with gate
 * row j and up row I+j of expert e = topk_ids[b,k], MXFP8 converted exactly
 * as it is read, FP32 accumulation, x read once for both.  Below 18 tokens
 * (4 when H >= 4096; the default token form) one 64-lane wave serves each
 * (token, slot, block of rows) and reduces across its lanes: no LDS, no
 * barrier.  From there on the default is the expert form on the matrix cores
 * (wd_launch.form 3; form 4 is an equivalent variant): one wave per
 * (expert, 16 rows), from H = 4096 a pair of waves each over half of the H
 * axis (wd_launch.h_split), reads each weight row once for all slots routed
 * to that expert, stages its codes in its own LDS region and computes the
 * same sums on v_mfma_f32_16x16x32_bf16 in another order. */
int wd_gate_up(const uint16_t *x, const int32_t *topk_ids,
               const uint8_t *w_gu, const uint8_t *s_gu, uint16_t *act,
               int B, int K, int E, int H, int I, void *stream);
int wd_gate_up_ex(const uint16_t *x, const int32_t *topk_ids,
                  const uint8_t *w_gu, const uint8_t *s_gu, uint16_t *act,
                  int B, int K, int E, int H, int I, const wd_launch *cfg, void *stream);

/* Down kernel (moe_down_3d_batched; same sections; the Chinese summary's
 * "Down Kernel"): out[b,h] = BF16(sum_k topk_w[b,k] * Wd[e_k,h,:] . act[b,k,:])
 * with the router weight folded into the FP32 accumulator.  In the token
 * form (the default below 24 tokens, 13 with expert-split scratch, 3 when
 * K * I > 6144) one wave per (token b, output dims)
 * walks the K routed experts' rows, reduces across its 64 lanes with DPP row
 * operations and one lane read (no LDS) and writes out[b,h].  From B = 24
 * (B = 13 with expert-split scratch, B = 3 when K * I > 6144; up to 512
 * tokens in at most 4 ranges of 128
 * tokens and 1,024 slots) the default is
 * the expert form on the matrix cores (wd_launch.form 3): one workgroup per
 * 16 output dims and token range reads each Wd row block once per range for
 * all the range's tokens routed to its expert, keeps each slot's products in
 * LDS and folds the router weights in per token after a workgroup barrier. */
int wd_down(const uint16_t *act, const int32_t *topk_ids, const float *topk_w,
            const uint8_t *w_d, const uint8_t *s_d, uint16_t *out,
            int B, int K, int E, int H, int I, void *stream);
int wd_down_ex(const uint16_t *act, const int32_t *topk_ids, const float *topk_w,
               const uint8_t *w_d, const uint8_t *s_d, uint16_t *out,
               int B, int K, int E, int H, int I, const wd_launch *cfg, void *stream);

/* Whole layer: wd_gate_up into `workspace` (used as act[B,K,I]), then wd_down,
 * both on `stream`.  workspace_bytes must be >= wd_workspace_bytes(B, K, I).
 * With workspace_bytes >= wd_layer_workspace_bytes(B, K, H, I) (and the
 * workspace 256-byte aligned) the rest of the workspace serves the down
 * kernel's expert split (see wd_launch.expert_split); its cells are
 * cleared by this call's gate/up kernel, so the workspace needs no
 * preparation. */
int wd_moe_decode(const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
                  const uint8_t *w_gu, const uint8_t *s_gu,
                  const uint8_t *w_d, const uint8_t *s_d,
                  void *workspace, size_t workspace_bytes, uint16_t *out,
                  int B, int K, int E, int H, int I, void *stream);

/* Whole layer without any allocation, for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same kernels, launch defaults and
 * results (bit for bit) as wd_moe_decode; act[B,K,I] lives in a static device
 * array of WD_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends (its address is looked up once per device, on the
 * first call with that device current).  The caller passes inputs and `out`
 * as for wd_moe_decode.  Calls no hipMalloc, hipFree or allocating library
 * routine.  Returns WD_ERR_SCRATCH, launching nothing, when B * K * I * 2 >
 * WD_NOALLOC_SCRATCH_BYTES.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (different streams, or several host
 * threads without ordering) race on it and must be serialised by the caller;
 * calls in order on one stream are safe.  Nothing in the array needs to start
 * at zero (gate/up writes every act element the down kernel reads, and clears
 * the down kernel's expert-split cells when the array holds them after act). */
int wd_moe_decode_noalloc(const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
                          const uint8_t *w_gu, const uint8_t *s_gu,
                          const uint8_t *w_d, const uint8_t *s_d, uint16_t *out,
                          int B, int K, int E, int H, int I, void *stream);

/* Router (top-k gating ahead of the layer; the pages name it as routing each
 * token to 8 of 128 experts: the Chinese summary's 传统路径的困境 section, the
 * English summary's Method section).  For each token b: topk_ids[b, 0..K) = the experts with the K
 * largest logits[b, :] (larger first; equal logits: lower expert index
 * first), topk_w[b, k] = softmax over the chosen logits,
 * exp(l_k - l_0) / sum_j exp(l_j - l_0), in FP32.  logits [B, E] fp32, row
 * major, finite; 1 <= K <= min(E, 64), E <= 1024.  One wave per token. */
int wd_route(const float *logits, int B, int E, int K, int32_t *topk_ids, float *topk_w, void *stream);

/* Bytes of the intermediate act[B,K,I] (BF16); 0 for invalid sizes. */
size_t wd_workspace_bytes(int B, int K, int I);

/* Bytes of the down kernel's expert-split scratch (wd_launch.down_scratch):
 * one 8-byte cell per output, B * H * 8; 0 for invalid sizes. */
size_t wd_down_scratch_bytes(int B, int H);

/* Workspace of wd_moe_decode that also holds the expert-split scratch:
 * act[B,K,I] rounded up to 256 bytes plus wd_down_scratch_bytes(B, H). */
size_t wd_layer_workspace_bytes(int B, int K, int H, int I);

/* Static string naming a status code (never NULL). */
const char *wd_status_string(int status);

/* ---- measurement helpers (not on the layer's path) --------------------- */

/* Exhaustive MXFP8 conversion probe: for every E8M0 byte s and code c, the
 * codes c, c+1, c+2, c+3 (mod 256) are packed into one word (byte j holds
 * c+j) and converted exactly as the layer kernels do.
 * out[(s * 256 + c) * 4 + j] receives the FP32 conversion (math mode 1) of
 * byte j and out[262144 + (s * 256 + c) * 4 + j] the BF16 conversion (math
 * mode 2) widened to FP32: 524,288 floats, device memory, 16-byte aligned. */
int wd_dequant_probe(float *out, void *stream);

/* Contiguous-read bandwidth kernel: reads `bytes` (a multiple of 16) from
 * `buf` with 16-byte loads in a grid-stride loop, `unroll` (1, 2, 4 or 8)
 * independent loads in flight per lane, and keeps every load live through a
 * conditional write to sink[0 .. blocks).  blocks <= 0 picks a default; sink
 * must hold wd_stream_blocks() uint32.  start_event / stop_event (hipEvent_t,
 * may be NULL) receive the kernel's own start and end, as in wd_launch. */
int wd_stream_read(const void *buf, size_t bytes, uint32_t *sink, int blocks, int unroll, void *start_event,
                   void *stop_event, void *stream);
int wd_stream_blocks(void);

/* Contiguous copy with 16-byte loads and stores (bytes a multiple of 16). */
int wd_stream_copy(void *dst, const void *src, size_t bytes, int blocks, void *stream);

/* Enqueue one wave that sleeps for about `sleep_units` * 8192 shader clocks
 * (bounded to 2^20 units).  Used to let the host queue work ahead of the GPU
 * before event-timed regions. */
int wd_gpu_sleep(int sleep_units, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* WD_H */
