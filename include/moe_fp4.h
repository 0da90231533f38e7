/*
 * moe_fp4.h - C ABI of the MI355X (gfx950) library for the routed
 * mixture-of-experts FFN over block-scaled FP4 expert weights.
 *
 * The method (sources cited by title and section):
 *  [Q] "Running a 133 GB MoE model on an 8 GB GPU at 11 tokens/s by streaming
 *      experts from NVMe" (aiwithghost.com)
 *  [D] "Running the 510 GB DeepSeek-V4.1-Flash on an 8 GB GPU, and three bugs
 *      that never raise an error" (dev.to)
 *
 * One MoE layer: a router picks k of E experts per token from fp32 logits
 * (softmax, top-k, weights renormalised over the chosen k; [Q] "Why this
 * model, of all models": top-10 of 512; [D] "Bytes per token decide
 * everything": 6 of 384). Each chosen expert is a SwiGLU FFN
 * y = down(silu(gate x) * (up x)) whose three matrices are stored as 4-bit
 * e2m1 codes with one scale per group of G codes ([Q] "The engine", item 4:
 * NVFP4; [D] "Three bugs", item 2: ue8m0 scales). The layer output is the
 * weighted sum of the chosen experts' outputs (plus an optional dense bf16
 * shared expert). Decode runs one token; prefill runs the whole prompt
 * through the layer at once with tokens grouped by expert ([Q] "The engine",
 * item 5).
 *
 * Conventions for every entry point:
 *  - All buffers are DEVICE memory owned by the caller unless stated. The
 *    library never allocates, never synchronises, never reads device data on
 *    the host and never copies to the host; every call only enqueues work on
 *    `stream` (a hipStream_t; NULL = the default stream) and returns.
 *  - Return value: MOE_OK (0) or a negative MOE_ERR_* code. Arguments are
 *    validated on the host before anything is launched; on error nothing is
 *    launched and moe_last_error() describes the problem (thread-local).
 *  - A shape the library has no tuned kernel for returns
 *    MOE_ERR_UNSUPPORTED; there is no slow or silent fallback.
 *  - Faults inside kernels surface at the caller's next synchronisation.
 *  - Workspace `ws`: device memory of at least moe_workspace_bytes() bytes,
 *    256-byte aligned. Its contents on entry do not matter and nothing in it
 *    carries over from one call to the next (its first 4096 bytes are
 *    reserved and never written). Calls that share one workspace must not
 *    run concurrently.
 *  - The library keeps no mutable global state and is reentrant.
 */
#ifndef MOE_FP4_H
#define MOE_FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Expert weight formats. Both use e2m1 codes (OCP MX FP4: magnitudes 0, 0.5,
 * 1, 1.5, 2, 3, 4, 6 and a sign bit); they differ in the scale. */
#define MOE_FMT_NVFP4 1 /* one E4M3 (OCP FP8 E4M3FN) scale per 16 codes */
#define MOE_FMT_MXFP4 2 /* one UE8M0 (power-of-two) scale per 32 codes  */

#define MOE_OK 0
#define MOE_ERR_ARG (-1)         /* null / misaligned pointer, bad size or shape */
#define MOE_ERR_UNSUPPORTED (-2) /* valid, but no tuned kernel for this shape */
#define MOE_ERR_HIP (-3)         /* a HIP launch failed */
#define MOE_ERR_WORKSPACE (-4)   /* workspace missing or too small */

#define MOE_MODE_ROUTE 0
#define MOE_MODE_DECODE 1
#define MOE_MODE_PREFILL 2

#define MOE_OUT_F32 0
#define MOE_OUT_BF16 1

/* Layer shape. H = hidden size, I = expert intermediate size, E = experts,
 * k = experts per token, format = MOE_FMT_*. H and I must be multiples of
 * the format's group size G (16 or 32). */
typedef struct moe_desc {
    int32_t H, I, E, k, format;
} moe_desc;

/* Dense bf16 shared expert (bit patterns, row-major): gate [I][H], up [I][H],
 * down [H][I]. It is added to the layer output unweighted. */
typedef struct moe_shared {
    const uint16_t *gate;
    const uint16_t *up;
    const uint16_t *down;
} moe_shared;

/* Optional debug outputs of moe_expert_prefill (any member may be NULL).
 * Rows in "grouped order" are indexed by position p in perm (rows of one
 * expert are contiguous, see moe_expert_prefill). */
typedef struct moe_prefill_debug {
    uint16_t *x_bf16;   /* [T][H] x~ = bf16(x), NVFP4 layers */
    uint8_t *x_codes;   /* [T][H/2] x~ e2m1 codes, MXFP4 layers (element 2i in the low nibble) */
    uint8_t *x_scales;  /* [T][H/32] x~ UE8M0 scale bytes, MXFP4 layers */
    float *h_pre;       /* [T*k][I] silu(g)*u before rounding, grouped order */
    float *h_q;         /* [T*k][I] h~ (the rounded h, as fp32), grouped order */
    int32_t *perm;      /* [T*k] assignment id t*k+j at each grouped position */
    int32_t *off;       /* [E+1] first grouped position of each expert; off[E] = T*k */
    /* Controls of the NVFP4 GEMM launch's bounded wait (down tiles wait for
     * their gate/up tiles; a wait that ends unmet writes NaN over the tile's
     * outputs). 0 and 0: the library's behaviour. */
    int32_t tile_wait_polls;  /* > 0: poll limit instead of the library's (about 0.4 s) */
    int32_t tile_wait_unmet;  /* nonzero: every wait asks for one more gate/up tile than exists */
} moe_prefill_debug;

/* ---------------------------------------------------------------------- */
/* Expert block layout                                                     */
/* ---------------------------------------------------------------------- */

/* Bytes of one expert block: 3*H*I/2 code bytes + 3*H*I/G scale bytes.
 * Region order gate | up | down | gate_scale | up_scale | down_scale, as the
 * expert repack of [Q] "The engine", item 1 (2,764,800 B for the Qwen shape,
 * H=2560, I=640, NVFP4; 18,800,640 B = 17.93 MiB for the DeepSeek shape,
 * H=4096, I=2880, MXFP4, [D] "Bytes per token decide everything").
 * gate/up are [I][H] and down is [H][I]; every matrix is row-major with the
 * 4-bit codes packed along the row (element 2c in the low nibble of byte c of
 * the row); scales are row-major [rows][cols/G] bytes. Returns 0 for an
 * invalid descriptor. */
size_t moe_block_bytes(const moe_desc *d);

/* Byte offsets of the six regions (off[0..5]) and the block size (off[6]).
 * Returns MOE_OK or MOE_ERR_ARG. Host memory. */
int moe_block_layout(const moe_desc *d, int64_t off[7]);

/* Workspace bytes needed by one call of the given mode for T tokens. */
size_t moe_workspace_bytes(const moe_desc *d, int32_t T, int32_t mode);

/* ---------------------------------------------------------------------- */
/* Router                                                                  */
/* ---------------------------------------------------------------------- */

/* For each token t < T: logits[t][e] = sum_h Wr[e][h] * x[t][h] (fp32
 * accumulate); S = the k experts with the largest logits (ties: lower expert
 * index first), written to idx[t][0..k) in that order; w[t][j] =
 * softmax(logits[t])[S_j] / sum over S, i.e. the softmax weights
 * renormalised over the chosen k ([Q] "Where the time actually goes": the
 * router's chosen experts). Nothing is read back to the host.
 *   x          [T][H] fp32, 16-B aligned
 *   Wr         [E][H] fp32, 16-B aligned
 *   idx        [T][k] int32 (out);  w [T][k] fp32 (out)
 *   logits_out [T][E] fp32 (out) or NULL
 * Errors: MOE_ERR_ARG for an invalid descriptor (k > E, sizes not positive
 * or not multiples of G), a null or misaligned pointer, T < 1;
 * MOE_ERR_UNSUPPORTED unless H % 256 == 0, H <= 8192, E <= 1024 and k <= 32;
 * MOE_ERR_WORKSPACE for a workspace below moe_workspace_bytes(d, T,
 * MOE_MODE_ROUTE). */
int moe_route(const moe_desc *d, const float *x, int32_t T, const float *Wr, int32_t *idx, float *w,
              float *logits_out, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------- */
/* Decode: one token                                                       */
/* ---------------------------------------------------------------------- */

/* The single-token expert computation of one MoE layer ([Q] "The engine",
 * item 4: a single-token SwiGLU expert kernel over NVFP4 weights, decoding
 * the e2m1 codes on the fly; [Q] "Why this model, of all models": gate, up
 * and down matrices per expert, and a shared expert kept in bf16):
 * y = sum_{j<k} w[j] * expert_{idx[j]}(x)  (+ shared(x) if shared != NULL)
 * where expert_e(x) = down_e( silu(gate_e x) * (up_e x) ), silu(z) =
 * z / (1 + exp(-z)), weights decoded on the fly from the block at
 * expert_ptrs[e] (format per d->format), fp32 activations and fp32
 * accumulation. The combine runs in increasing j (then the shared
 * expert), so results are bit-identical from run to run.
 *   x           [H] fp32, 16-B aligned
 *   expert_ptrs DEVICE array of E pointers (8-B aligned), each to one
 *               256-B-aligned expert block (resident layers:
 *               base + e * moe_block_bytes)
 *   idx [k] int32, w [k] fp32: the routing (e.g. from moe_route)
 *   shared      host struct of device pointers, or NULL
 *   y           [H] fp32 (out)
 * Requires H % 512 == 0, H <= 4096, 16 <= I <= 4096 (a multiple of G), and
 * k <= 32; other shapes return MOE_ERR_UNSUPPORTED. */
int moe_expert_decode(const moe_desc *d, const float *x, const void *const *expert_ptrs, const int32_t *idx,
                      const float *w, const moe_shared *shared, float *y, void *ws, size_t ws_bytes, void *stream);

/* One decode layer in one call: moe_route (T = 1) followed by
 * moe_expert_decode, with the same results (bit-identical chosen experts,
 * weights and y), in three launches instead of four: the router GEMV shares
 * a launch with the shared expert's gate/up (neither depends on the
 * routing), and the top-k is recomputed at the start of every routed
 * gate/up workgroup. idx_out [k] int32 and w_out [k] fp32 receive the
 * routing. Requirements: those of moe_route and of moe_expert_decode;
 * workspace: moe_workspace_bytes(d, 1, MOE_MODE_DECODE). */
int moe_layer_decode(const moe_desc *d, const float *x, const float *Wr, const void *const *expert_ptrs,
                     const moe_shared *shared, float *y, int32_t *idx_out, float *w_out, void *ws, size_t ws_bytes,
                     void *stream);

/* ---------------------------------------------------------------------- */
/* Decode without a workspace                                              */
/* ---------------------------------------------------------------------- */

/* Bytes of the static scratch array behind moe_layer_decode_noalloc. Every
 * shape moe_layer_decode supports needs at most 549,120 bytes. */
#define MOE_NOALLOC_SCRATCH_BYTES 1048576

/* moe_layer_decode for callers that cannot allocate memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation. Same arguments minus the workspace, same kernels, bit-identical
 * results. The workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on until the process ends; its address on the current device is looked up
 * on the first call there (hipGetSymbolAddress). No call allocates or frees
 * memory. Nothing in the array carries over from one call to the next, but
 * all calls on one GPU share it: calls that may overlap on one GPU (other
 * streams, other host threads) race and must not be issued; calls ordered on
 * one stream are fine. Errors: those of moe_layer_decode (apart from the
 * workspace ones); MOE_ERR_WORKSPACE if a layer would need more than
 * MOE_NOALLOC_SCRATCH_BYTES; MOE_ERR_HIP if the lookup fails. */
int moe_layer_decode_noalloc(const moe_desc *d, const float *x, const float *Wr, const void *const *expert_ptrs,
                             const moe_shared *shared, float *y, int32_t *idx_out, float *w_out, void *stream);

/* ---------------------------------------------------------------------- */
/* Prefill: T tokens grouped by expert                                     */
/* ---------------------------------------------------------------------- */

/* out[t] = sum_{j<k} w[t][j] * down_e( Q( silu(gate_e x~_t) * (up_e x~_t) ) ),
 * e = idx[t][j], for every token at once ([Q] "The engine", item 5: the
 * whole prompt through each layer). Assignments a = t*k + j are grouped by
 * expert with a stable counting sort (count, exclusive prefix scan, scatter;
 * within an expert in increasing a) and each expert's rows are multiplied
 * as one ragged GEMM. Activation rounding points:
 *   NVFP4: x~ = bf16(x) and h~ = bf16(h) (round to nearest even); the
 *          weights are dequantised to bf16 exactly; bf16 MFMA, fp32 accumulate.
 *   MXFP4: x~ and h~ are converted to MXFP4 per 32 consecutive elements
 *          (OCP MX: shared exponent floor(log2 max|v|) - 2, e2m1 codes by
 *          round-to-nearest-even with saturation); scaled FP4 MFMA, fp32
 *          accumulate.
 * The combine runs in increasing j in fp32; out is fp32 [T][H] or, with
 * out_dtype = MOE_OUT_BF16, bf16 [T][H] rounded from that fp32 sum.
 *   x [T][H] fp32; idx, w [T][k]; expert_ptrs as for decode; dbg optional.
 * Requires H % 256 == 0 and I % 128 == 0 (NVFP4) or H % 512 == 0 and
 * I % 64 == 0 (MXFP4), H and I <= 16384, E <= 1024, k <= 32. */
int moe_expert_prefill(const moe_desc *d, const float *x, int32_t T, const void *const *expert_ptrs,
                       const int32_t *idx, const float *w, void *out, int32_t out_dtype, void *ws,
                       size_t ws_bytes, const moe_prefill_debug *dbg, void *stream);

/* ---------------------------------------------------------------------- */
/* FP8 beside the MoE path                                                 */
/* ---------------------------------------------------------------------- */

#define MOE_SCALE_FLOOR 0 /* OCP MX: X = floor(log2 amax) - 8; quotients above 448 saturate */
#define MOE_SCALE_CEIL 1  /* smallest X with amax <= 448 * 2^X; never saturates */

/* Activation quantiser: FP8 E4M3 codes with one UE8M0 (power-of-two) scale
 * per block of `block` consecutive values of a row ([D] "Three bugs", item
 * 2: DeepSeek's activation quantiser, ue8m0 scales, FP8 out, checked
 * bit-exact at 1, 17, 300 and 1024 rows; OCP MX: MXFP8 uses blocks of 32).
 *   x       fp32 [rows][cols], 16-byte aligned
 *   block   32 or 128; cols a positive multiple of block
 *   rule    MOE_SCALE_FLOOR or MOE_SCALE_CEIL (shared exponent X of a block
 *           from its largest magnitude amax, clamped to [-127, 127])
 *   codes   out: uint8 [rows][cols], 4-byte aligned: E4M3 (OCP E4M3FN) of
 *           v / 2^X rounded to nearest even, magnitudes clamped to 448;
 *           negative values that round to zero give 0x80
 *   scales  out: uint8 [rows][cols/block]: X + 127 (0 for an all-zero block)
 * rows == 0 enqueues nothing and returns MOE_OK. No workspace. Inputs must be
 * finite. Errors: MOE_ERR_ARG (pointers, sizes, block, rule). */
int moe_act_quant_fp8(const float *x, int32_t rows, int32_t cols, int32_t block, int32_t rule, uint8_t *codes,
                      uint8_t *scales, void *stream);

/* Row-scaled FP8 matrix-vector product ([Q] "The engine", item 4: the FP8
 * row-scaled matrix-vector kernel; [Q] "Why this model, of all models": the
 * large dense matrices stored in FP8 with one scale per row):  y[r] = row_scale[r] * sum_c e4m3(W[r][c]) * x[c],
 * accumulated in fp32.
 *   W          uint8 E4M3 codes [rows][cols], row-major, 16-byte aligned
 *   row_scale  fp32 [rows];  x  fp32 [cols], 16-byte aligned;  y  fp32 [rows]
 * cols must be 512 * d with d in 1..8, 10, 12 or 16 (MOE_ERR_UNSUPPORTED
 * otherwise); rows >= 0 (0 enqueues nothing). No workspace. */
int moe_gemv_fp8(const uint8_t *W, const float *row_scale, const float *x, int32_t rows, int32_t cols, float *y,
                 void *stream);

/* ---------------------------------------------------------------------- */
/* Speculative expert prefetch                                             */
/* ---------------------------------------------------------------------- */

/* ([Q] "The engine", item 3: guess the next layer's experts and read them
 * while the GPU is busy; [D] "Making it faster": predicting the next layer's
 * experts.) Reads the whole blocks of experts idx[0..n) (device int32; an
 * index outside [0, E) is skipped) through expert_ptrs so that they sit in
 * the GPU's last-level cache when a following launch needs them. The guess is
 * the caller's: typically moe_route with the next layer's router on this
 * layer's input, on a second stream. The read is made observable: sink
 * (device, 4-byte aligned, at least moe_prefetch_sink_bytes(d, n) bytes)
 * receives, for expert j and 64 KiB chunk c of its block, the XOR of the
 * chunk's 32-bit words at sink[j * nchunks + c] (0 for a skipped index).
 * n in 1..1024. Errors: MOE_ERR_ARG. */
size_t moe_prefetch_sink_bytes(const moe_desc *d, int32_t n);
int moe_expert_prefetch(const moe_desc *d, const void *const *expert_ptrs, const int32_t *idx, int32_t n,
                        uint32_t *sink, size_t sink_bytes, void *stream);

/* ---------------------------------------------------------------------- */
/* Expert tier: pinned host blocks with an HBM slot cache                  */
/* ---------------------------------------------------------------------- */

/* ([Q] "The engine", items 2-3: an LRU cache of experts in front of the slow
 * tier, GPU slots, and copies into them overlapped with compute; [D] "Making
 * it faster".) Every expert block of `layers` layers lives in pinned host
 * memory; n_slots HBM slots hold the most recently routed ones. The tier owns
 * the per-layer pointer tables the decode entry points take
 * (expert_ptrs = table + layer * E): each entry points at the expert's HBM
 * slot or, for experts not in HBM, at its pinned host block, which the
 * kernels then read in place over PCIe (no copy, no host synchronisation).
 *
 * Unlike the compute entry points, the tier is a resource-owning object: it
 * creates one copy stream and a few events, allocates a small pinned staging
 * array and host-side state, and moe_tier_create synchronises once (initial
 * table). Every decode launch that reads the table must be on the
 * compute_stream given to moe_tier_update (the tier orders its table writes
 * with those launches); not for use under graph capture. */
typedef struct moe_tier moe_tier;
typedef struct {
    int64_t resident;   /* experts whose table entry points at their HBM slot */
    int64_t pending;    /* experts being copied (entry switches at the next update) */
    int64_t hits;       /* routed (layer, slot) uses found resident, over all updates */
    int64_t misses;     /* routed uses read from host memory */
    int64_t promotions; /* blocks copied into slots */
    int64_t evictions;  /* experts moved back to their host blocks */
} moe_tier_stats;

/*   host_blocks  pinned host memory (hipHostMalloc or equivalent, mapped at the
 *                same address on the device): layers * E blocks of
 *                moe_block_bytes(d), layer-major, 256-byte aligned
 *   slots        device memory for n_slots blocks (NULL if n_slots == 0)
 *   table        device memory for layers * E pointers, 8-byte aligned;
 *                filled by the tier (all entries start at the host blocks)
 * Errors: MOE_ERR_ARG (sizes, alignment, memory not pinned / not on the
 * device), MOE_ERR_HIP. */
int moe_tier_create(const moe_desc *d, int32_t layers, void *host_blocks, void *slots, int32_t n_slots, void **table,
                    moe_tier **out);

/* Waits for the tier's own copies, then frees its streams, events and state
 * (not the caller's buffers). Work the caller enqueued that reads the table
 * must be finished first. */
int moe_tier_destroy(moe_tier *t);

/* After a decode step: idx_host [layers][k] is that step's routing (host
 * memory, e.g. read back asynchronously by the caller; indices outside
 * [0, E) are ignored). Enqueued on compute_stream, in this order: the table
 * entries of the previous update's newcomers switch to their slots (after
 * their copies, by event); up to max_promote experts of this step that are
 * not in HBM take a free slot or the slot of the least recently used expert
 * that this step did not use, whose entry first returns to its host block;
 * then, on the tier's copy stream, once the compute stream has passed those
 * entries, the newcomers' blocks are copied into their slots (overlapping the
 * compute stream). Nothing here waits on the host except for a staging
 * buffer four updates old. */
int moe_tier_update(moe_tier *t, const int32_t *idx_host, int32_t max_promote, void *compute_stream);

/* Counters and residency (host state, no device access). */
int moe_tier_get_stats(const moe_tier *t, moe_tier_stats *out);

/* Slot of (layer, expert) if its table entry points at HBM, else -1. */
int32_t moe_tier_slot_of(const moe_tier *t, int32_t layer, int32_t expert);

/* ---------------------------------------------------------------------- */
/* Test support and errors                                                 */
/* ---------------------------------------------------------------------- */

/* Dequantise one expert block to fp32 gate [I][H], up [I][H], down [H][I]
 * (each weight is e2m1(code) * scale, exact in fp32). For bit-exact checks
 * of the decode used by every kernel. */
int moe_dequant_block(const moe_desc *d, const void *block, float *gate, float *up, float *down, void *stream);

/* Static description of a status code. */
const char *moe_status_string(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP4_H */
