/*
 * nhm.h -- C ABI of libnhm: the NemotronH Mamba2 mixer with FP8 W8A8 projections
 * on AMD Instinct MI355X (gfx950).
 *
 * Sources (pull-request pages of one C++ LLM inference project, cited by number):
 *   [PR1288] "feat(#810 A2-Q1): NemotronH's 23 Mamba2 blocks reach the device on the
 *            FP8 W8A8 seam (#517)"
 *   [PR1289] the same change re-filed as #1289 (conversation and commit log)
 *   [PR988]  "spec(#810 A2-Q): split the quantized arms into A2-Q1 and A2-Q2, because
 *            their blockers differ (#517)"
 *   [PR950]  "feat(#810 A2-R): NemotronH's dense weights reach the device, and the
 *            attention block that reads them is model-local (#517)"
 *   [PR972]  "refactor(VT-FP8-SHARED-SEAM): the FP8 W8A8 linear path becomes a seam a
 *            second model can reach (#940)"
 *
 * Conventions that hold for every entry point:
 *   - Pointers marked (device) address GPU memory; (host) address host memory.
 *     The caller owns every buffer. The library allocates nothing (but the fixed scratch of
 *     nhm_mixer_decode_noalloc), keeps no cache and no state between calls (but the
 *     diagnostic dispatch counters), never synchronizes the device, and only enqueues work
 *     on the given stream (a hipStream_t; NULL = the default stream). All calls are
 *     therefore legal inside HIP graph capture.
 *   - Shapes, null pointers, alignment and geometry are validated on the host before
 *     anything is enqueued. A failed check returns a status and enqueues nothing; no
 *     C++ exception crosses the ABI. nhm_last_error() then describes the failure.
 *   - A failed kernel launch returns NHM_ERR_HIP.
 *   - Values that live only on the device (slot indices, cu_seqlens, has_initial)
 *     cannot be checked without a synchronization; their contract is stated per call
 *     and violating it is undefined behaviour.
 *   - bf16 tensors are passed as uint16_t bit patterns, e4m3 tensors as uint8_t
 *     codes (OCP FP8 E4M3FN: largest finite 448, no infinities).
 *   - Workspaces ("ws") are caller-allocated device memory (256-byte aligned) for the
 *     intermediates of one call; their contents on entry are ignored and on return
 *     hold the intermediates listed in nhm_ws_layout. One workspace must not be used
 *     by two calls that can run at the same time (e.g. on two streams).
 */
#ifndef NHM_H
#define NHM_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define NHM_API __attribute__((visibility("default")))
#else
#define NHM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */

typedef enum nhm_status {
    NHM_OK = 0,
    NHM_ERR_NULL = 1,        /* a required pointer is NULL                         */
    NHM_ERR_SHAPE = 2,       /* a size or leading dimension is out of range        */
    NHM_ERR_ALIGN = 3,       /* a pointer or leading dimension is misaligned       */
    NHM_ERR_UNSUPPORTED = 4, /* a geometry or option this build does not implement */
    NHM_ERR_WORKSPACE = 5,   /* ws is NULL or smaller than the call needs          */
    NHM_ERR_HIP = 6          /* the HIP runtime reported an error                  */
} nhm_status;

typedef enum nhm_dtype {
    NHM_BF16 = 0,            /* bfloat16 bit patterns (uint16_t)                   */
    NHM_E4M3 = 1,            /* OCP FP8 E4M3FN codes (uint8_t)                      */
    NHM_F32 = 2,             /* IEEE binary32 (float): GEMM output, SSM state       */
    /* Not types: they make every 32-bit int a value of the enum, so that any integer a
     * caller passes is well defined on the library side and reaches validation
     * (NHM_ERR_UNSUPPORTED). */
    NHM_DTYPE_RANGE_MIN_ = -2147483647 - 1,
    NHM_DTYPE_RANGE_MAX_ = 2147483647
} nhm_dtype;

/* Static name of a status code. Never NULL. */
NHM_API const char* nhm_status_str(nhm_status s);

/* Detail of the last failure on the calling thread ("" if none). The string stays
 * valid until the next libnhm call on the same thread. */
NHM_API const char* nhm_last_error(void);

/* Name of the GPU architecture the library was built for ("gfx950"). */
NHM_API const char* nhm_build_arch(void);

/* Path-taken counters ([PR1289] commit log: the device path is told from the host path by
 * its own dispatch counters -- state-update rows, chunk-scan calls, conv calls): for each
 * kernel the library launches, the launches and the rows they covered (tokens; chunks for the
 * chunked-scan kernels) since the counters were last reset. Host-side and atomic, the only
 * state the library keeps; a launch recorded into a HIP graph counts once, at capture, not
 * per replay. Fills out[0 .. min(max, count) - 1] (host; out may be NULL), zeroes the counters
 * when reset != 0, and returns the number of counters. Names are static strings. */
typedef struct nhm_dispatch_counter {
    const char* kernel;
    uint64_t launches;
    uint64_t rows;
} nhm_dispatch_counter;
NHM_API int32_t nhm_dispatch_counters(nhm_dispatch_counter* out, int32_t max, int32_t reset);

/* ---------------------------------------------------------------- geometry */

/* Mixer geometry. [PR1288] opening section (2688 -> 10304 in_proj, 4096 -> 2688
 * out_proj); [PR950] "Review repairs" F2 (64 heads; three f32 per-head SSM
 * tensors). Supported by the kernels: head_dim == 64, d_state == 128,
 * conv_width == 4, n_heads % n_groups == 0, n_heads % 8 == 0 (in_proj rows are
 * read 16 bytes at a time), hidden % 16 == 0, 0 < rms_eps
 * (an eps of 0 is refused: [PR950] "Not dense_attn::AttnBlock (#941)" reports a
 * missing rms eps key silently becoming 0). */
typedef struct nhm_geometry {
    int32_t hidden;      /* model width H (2688)                        */
    int32_t n_heads;     /* SSM heads (64)                              */
    int32_t head_dim;    /* P, channels per head (64)                   */
    int32_t d_state;     /* N, state width per head channel (128)       */
    int32_t n_groups;    /* G, groups sharing B and C; norm groups (8)  */
    int32_t conv_width;  /* causal conv taps (4)                        */
    float rms_eps;       /* gated RMSNorm epsilon (1e-5), > 0           */
} nhm_geometry;

/* Split indices of one in_proj row and of the conv output ([PR1289] commit log;
 * [PR1288] "What it does"). An in_proj row is z, then xBC, then dt: three adjacent
 * column ranges of widths I, conv_dim and n_heads. The conv output row is x, then B,
 * then C. */
typedef struct nhm_layout {
    int32_t d_inner;          /* I = n_heads * head_dim                      */
    int32_t conv_dim;         /* I + 2 * n_groups * d_state                  */
    int32_t d_in_proj;        /* I + conv_dim + n_heads                      */
    int32_t z_off, z_width;   /* within an in_proj row                       */
    int32_t xbc_off, xbc_width;
    int32_t dt_off, dt_width;
    int32_t x_off, x_width;   /* within an xBC row                           */
    int32_t b_off, b_width;
    int32_t c_off, c_width;
    int32_t heads_per_group;  /* head h reads B/C group h / heads_per_group  */
    int32_t norm_group;       /* channels per RMSNorm group = I / n_groups   */
} nhm_layout;

/* Fills *out (host) from *g (host). The kernels index with the same numbers.
 * Errors: NHM_ERR_NULL, NHM_ERR_UNSUPPORTED (geometry outside the list above). */
NHM_API nhm_status nhm_mixer_layout(const nhm_geometry* g, nhm_layout* out);

/* ---------------------------------------------------------------- FP8 W8A8 linear */

/* One FP8 W8A8 projection: e4m3 weight in the [out, in] torch-Linear orientation
 * (row-major [n, k]; [PR950] "Review repairs" F2: the GEMM consumers refuse any
 * other orientation), its f32 weight scale, and the static per-tensor f32 activation
 * scale ("input_scale"). All three pointers are device memory. The weight scale is one
 * f32 per output channel, or, with w_scale_per_tensor = 1, one f32 for the whole
 * projection: the form the checkpoint carries, two f32 scalars per FP8 projection
 * ([PR950] "Review repairs" F2, weight_scale beside input_scale). A zero-initialised
 * field keeps the per-channel form. */
typedef struct nhm_fp8_weight {
    const uint8_t* w;         /* (device) e4m3 [n, k], row stride k, 16-B aligned */
    const float* w_scale;     /* (device) f32 [n], or f32 [1] when per tensor     */
    const float* a_scale;     /* (device) f32 [1]                                 */
    int64_t n;                /* output features                                  */
    int64_t k;                /* input features, k % 16 == 0                      */
    int32_t w_scale_per_tensor; /* 0: per output channel; 1: one scale; other values
                                   are refused (NHM_ERR_UNSUPPORTED)                */
} nhm_fp8_weight;

/* Static per-tensor activation quant: q[r, c] = E4M3(f32(x[r, c]) / scale[0]),
 * the f32 quotient correctly rounded, the code rounded half to even and saturated
 * at +-448 (NaN -> 0x7F with the sign kept).
 * [PR988] "The Thor finding, measured" (the quant op is its own kernel, kQuantFp8Static);
 * [PR1288] "The comparison is not bit-comparable, and that is the point" (W8A8
 * applies input_scale to the activation).
 *   x      (device) bf16 [rows, ld_x], ld_x >= cols
 *   scale  (device) f32 [1]
 *   q      (device) e4m3 [rows, ld_q], ld_q >= cols; must not overlap x
 * rows == 0 or cols == 0 is a valid no-op.
 * Errors: NHM_ERR_NULL, NHM_ERR_SHAPE (negative sizes, ld < cols), NHM_ERR_ALIGN
 * (x not 2-byte aligned), NHM_ERR_HIP. */
NHM_API nhm_status nhm_fp8_quantize_static(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                   const float* scale, uint8_t* q, int64_t ld_q, void* stream);

/* Per-output-channel dequant of an e4m3 weight to bf16 ([PR950] "What runs where, and
 * why the line falls there": the one standalone device dequant is per-channel FP8 ->
 * bf16), the building block of the W8A16 reference the pages compare the W8A8 arm
 * against ([PR1288] "The comparison is not bit-comparable, and that is the point": the
 * host arm is W8A16, its input_scale carried and not applied). A debug and
 * counterfactual op, not on the W8A8 path:
 *   out[r, c] = bf16( val(w[r, c]) * w_scale[r] ), the product in f32, rounded once
 *   (half to even); NaN codes give NaN.
 *   w       (device) e4m3 [n, ld_w], 16-byte aligned, ld_w % 16 == 0
 *   w_scale (device) f32 [n]
 *   out     (device) bf16 [n, ld_out], 16-byte aligned, ld_out % 8 == 0; must not overlap w
 * k must be a multiple of 16 and ld_w, ld_out >= k. n == 0 or k == 0 is a valid no-op.
 * Errors: NHM_ERR_NULL, NHM_ERR_SHAPE, NHM_ERR_ALIGN, NHM_ERR_HIP. */
NHM_API nhm_status nhm_fp8_dequant_channel_bf16(const uint8_t* w, const float* w_scale, int64_t n, int64_t k,
                                        int64_t ld_w, uint16_t* out, int64_t ld_out, void* stream);

/* Workspace bytes for nhm_fp8_linear on this shape and input type: the activation codes
 * of a bf16 input (required), then, for the narrow shapes that split k (see below), room
 * for the f32 partials (optional: a workspace without it runs those shapes unsplit). */
NHM_API size_t nhm_fp8_linear_workspace_bytes(int64_t m, int64_t n, int64_t k, nhm_dtype a_type);

/* out[i, j] = bf16( (sum_k val(a_q[i, k]) * val(w[j, k])) * a_scale * w_scale[j] ),
 * accumulated in f32. a_q is a itself when a_type == NHM_E4M3 (a pre-quantized
 * activation: [PR972] "Correspondence with dense_nvfp4_gemm.h", the
 * QuantizedActivation overload), else nhm_fp8_quantize_static(a, w->a_scale).
 * [PR988] "The Thor finding, measured" (e4m3 x e4m3, f32 compute and scale, bf16 D).
 *   a      (device) [m, ld_a] of a_type, 16-B aligned, ld_a >= k, ld_a % 8 == 0
 *          (bf16) or % 16 == 0 (e4m3)
 *   w      (host struct of device pointers)
 *   out    (device) bf16 [m, ld_out], ld_out >= n; must not overlap a (rows that
 *          are 8-byte aligned are stored 4 features at a time)
 *   ws     (device, 256-byte aligned) nhm_fp8_linear_workspace_bytes(m, n, k, a_type)
 *          bytes; the bf16 input's codes (m * k bytes, rounded up to 256) are required,
 *          the rest only enables the split-k path; with an e4m3 input ws may be NULL
 * m == 0 is a valid no-op. m <= 16 (k <= 16384, weight under 2 GiB) runs the
 * weight-streaming GEMV, which sums the products exactly in f32 (the codes are
 * converted to bf16, exact for every e4m3 value, and summed by the bf16 MFMA).
 * Larger m runs the tiled e4m3 MFMA GEMM, whose 128-product reductions are coarser
 * than f32: measured on MI355X, within ~2^-17 of sum |a w| per 128 products (the
 * result still lies within 2^-8 |out| + 2^-16 sum |a w| of the exact one).
 * Where 16 < m <= 640 leaves the 64 x 128 tiles on at most 32 workgroups (narrow n, long
 * k) and the workspace holds the partials, k is split over 2-8 workgroups per tile and
 * their f32 partial sums are added in split order by a second kernel, then scaled and
 * rounded once.
 * Results are deterministic (no atomics).
 * Every kernel addresses its operands with 32-bit offsets: a weight (n * k) or an activation
 * (m * ld_a, or m * k for a bf16 input's codes) of 2 GiB or more is NHM_ERR_UNSUPPORTED,
 * refused before anything is enqueued.
 * Errors: NHM_ERR_NULL, NHM_ERR_SHAPE, NHM_ERR_ALIGN, NHM_ERR_UNSUPPORTED, NHM_ERR_WORKSPACE,
 * NHM_ERR_HIP. */
NHM_API nhm_status nhm_fp8_linear(const void* a, nhm_dtype a_type, int64_t m, int64_t ld_a,
                          const nhm_fp8_weight* w, uint16_t* out, int64_t ld_out,
                          void* ws, size_t ws_bytes, void* stream);

/* nhm_fp8_linear with a choice of output type: out_type NHM_BF16 is nhm_fp8_linear;
 * NHM_F32 stores the unrounded f32 result (sum_k val(a_q[i, k]) * val(w[j, k])) * a_scale
 * * w_scale[j] instead of its bf16 rounding. [PR988] "The Thor finding, measured": the
 * pages' fp8 GEMM plan takes the output dtype as part of its key, and both D = bf16 and
 * D = f32 plans are probed available for the same six shapes.
 *   out    (device) [m, ld_out] of out_type, ld_out >= n, aligned to its element size;
 *          must not overlap a (16-byte aligned rows with ld_out % 4 == 0 are stored four
 *          features at a time)
 * Every other argument, the accumulation and the errors are those of nhm_fp8_linear;
 * an out_type other than NHM_BF16 or NHM_F32 is NHM_ERR_UNSUPPORTED. */
NHM_API nhm_status nhm_fp8_linear_ex(const void* a, nhm_dtype a_type, int64_t m, int64_t ld_a,
                             const nhm_fp8_weight* w, void* out, nhm_dtype out_type, int64_t ld_out,
                             void* ws, size_t ws_bytes, void* stream);

/* nhm_fp8_linear_ex with every product summed in f32 on every path: the codes are converted
 * to bf16 (exact for every e4m3 value) and summed by the bf16 MFMA, as the GEMV does for
 * m <= 16, instead of the e4m3 MFMA's 128-product reductions. [PR988] "The Thor finding,
 * measured": the pages' fp8 GEMM plan computes in f32 (CUBLAS_COMPUTE_32F). The result is
 * within ~2^-24 of sum |a w| of the exact sum (measured), at up to twice the MFMA time of
 * nhm_fp8_linear_ex for m > 16 (the bf16 MFMA runs at half the e4m3 rate). Arguments,
 * workspace and errors are those of nhm_fp8_linear_ex. */
NHM_API nhm_status nhm_fp8_linear_exact(const void* a, nhm_dtype a_type, int64_t m, int64_t ld_a,
                                const nhm_fp8_weight* w, void* out, nhm_dtype out_type, int64_t ld_out,
                                void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- the mixer block */

/* All parameters of one mixer block (device pointers; the struct itself is host).
 * [PR1288] "What it does": in_proj (FP8 W8A8) -> split z | xBC | dt ->
 * CausalConv1dFwd(silu) -> split x | B | C -> Mamba2ChunkScan ->
 * RmsNormGatedGroup(n_groups) -> out_proj (FP8 W8A8). */
typedef struct nhm_mixer_params {
    nhm_geometry g;
    nhm_fp8_weight in_proj;   /* n = d_in_proj, k = hidden   */
    nhm_fp8_weight out_proj;  /* n = hidden,    k = d_inner  */
    const uint16_t* conv_w;   /* bf16 [conv_dim, conv_width] */
    const uint16_t* conv_b;   /* bf16 [conv_dim]             */
    const uint16_t* norm_w;   /* bf16 [d_inner]              */
    const float* A_log;       /* f32 [n_heads]; A = -exp(A_log) */
    const float* D;           /* f32 [n_heads] skip weight   */
    const float* dt_bias;     /* f32 [n_heads]; dt = softplus(dt_raw + dt_bias) */
} nhm_mixer_params;

/* Byte offsets of the intermediates a call leaves in its workspace (for
 * inspection; SIZE_MAX when that call does not keep one), and the total size. */
typedef struct nhm_ws_layout {
    size_t total;      /* bytes the call needs                                  */
    size_t q_in;       /* e4m3 [tokens, hidden]      quantized block input      */
    size_t zxbcdt;     /* bf16 [tokens, d_in_proj]   in_proj output             */
    size_t xbc_conv;   /* bf16 [tokens, conv_dim]    conv + SiLU output         */
    size_t y;          /* bf16 [tokens, d_inner]     SSM output incl. D skip    */
    size_t norm;       /* bf16 [tokens, d_inner]     gated RMSNorm output       */
    size_t q_out;      /* e4m3 [tokens, d_inner]     quantized out_proj input   */
} nhm_ws_layout;

/* Workspace layout of nhm_mixer_decode for `batch` rows.
 * Errors: NHM_ERR_NULL, NHM_ERR_UNSUPPORTED, NHM_ERR_SHAPE (batch < 0). */
NHM_API nhm_status nhm_mixer_decode_ws_layout(const nhm_geometry* g, int32_t batch, nhm_ws_layout* out);

/* One decode token for each of `batch` sequences whose recurrent state lives in
 * pool rows addressed by slot ([PR1288] "What it does": the paged arm hands the
 * mixer gathered recurrent rows and it advances them IN PLACE; decode always
 * continues from the stored rows, has_initial = true).
 *   hidden    (device) bf16 [batch, g.hidden], row stride g.hidden
 *   slot_idx  (device) int32 [batch]: pool row of each sequence. Contract: every
 *             non-negative entry is < n_slots and distinct; a negative entry marks
 *             a padded row, whose output row is zero and which touches no state.
 *   ssm_pool  (device) f32 [n_slots, n_heads, head_dim, d_state], updated in place
 *   conv_pool (device) bf16 [n_slots, conv_width-1, conv_dim], the previous
 *             conv_width-1 pre-conv xBC rows, oldest first; updated in place
 *   out       (device) bf16 [batch, g.hidden]; must not overlap hidden
 *   ws        (device) >= nhm_mixer_decode_ws_layout(g, batch).total bytes
 * Both projections run as the exact-f32 GEMV of nhm_fp8_linear, 16 rows at a time
 * (a weight or activation of 2 GiB or more is NHM_ERR_UNSUPPORTED, as in nhm_fp8_linear).
 * batch == 0 is a valid no-op.
 * Errors: NHM_ERR_NULL, NHM_ERR_SHAPE, NHM_ERR_ALIGN, NHM_ERR_UNSUPPORTED,
 * NHM_ERR_WORKSPACE, NHM_ERR_HIP. */
NHM_API nhm_status nhm_mixer_decode(const nhm_mixer_params* p, const uint16_t* hidden, int32_t batch,
                            const int32_t* slot_idx, float* ssm_pool, uint16_t* conv_pool,
                            int32_t n_slots, uint16_t* out, void* ws, size_t ws_bytes,
                            void* stream);

/* nhm_mixer_decode_ex with the block input pre-quantized and the block output's codes emitted,
 * so that stacked blocks pass e4m3 codes along instead of re-quantizing each block's input in
 * a launch of its own ([PR972] "Correspondence with dense_nvfp4_gemm.h": the GEMM seam takes a
 * pre-quantized activation; [PR1288] "What it does": each block's in_proj quantizes its input
 * with its static input_scale).
 *   hidden    (device) bf16 [batch, hidden] or NULL when hidden_q is given
 *   hidden_q  (device) e4m3 [batch, hidden], 16-byte aligned, or NULL: the codes
 *             E4M3(hidden / *p->in_proj.a_scale) (e.g. the previous block's out_q under this
 *             block's in_proj a_scale); used instead of quantizing hidden
 *   out_q     (device) e4m3 [batch, hidden], 16-byte aligned, or NULL: receives
 *             E4M3(out / *out_q_scale) of the bf16 block output (written by the out_proj
 *             epilogue up to 32 rows, by a quant launch above)
 *   out_q_scale (device) f32 [1]; required with out_q (the next block's in_proj a_scale)
 * out, the pools and everything else are those of nhm_mixer_decode_ex; with hidden_q given,
 * the workspace's q_in region is left as it was. Errors: those of nhm_mixer_decode_ex. */
NHM_API nhm_status nhm_mixer_decode_q(const nhm_mixer_params* p, const uint16_t* hidden, const uint8_t* hidden_q,
                              int32_t batch, const int32_t* slot_idx, void* ssm_pool, nhm_dtype ssm_type,
                              uint16_t* conv_pool, int32_t n_slots, uint16_t* out, uint8_t* out_q,
                              const float* out_q_scale, void* ws, size_t ws_bytes, void* stream);

/* nhm_mixer_decode_ex without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The intermediates go to a scratch array that the library holds in device memory, 16 MiB per
 * GPU it runs on, kept until the process ends; the call itself allocates nothing. A call
 * whose workspace (nhm_mixer_decode_ws_layout(g, batch).total) exceeds 16 MiB is refused with
 * NHM_ERR_WORKSPACE before anything is enqueued: batch <= 299 at the NemotronH geometry
 * (16.76 MB at 299 rows). Every call on one GPU from one process shares that GPU's scratch (another
 * process holds its own copy): calls that can overlap there (on two streams, from two
 * threads) race and must not be issued. The scratch keeps the last call's intermediates;
 * nothing in it needs to start at zero. The stream must belong to the current device (else NHM_ERR_UNSUPPORTED);
 * the first call on a device resolves that device's scratch address. Every other argument,
 * the results and the remaining errors are those of nhm_mixer_decode_ex. */
NHM_API nhm_status nhm_mixer_decode_noalloc(const nhm_mixer_params* p, const uint16_t* hidden, int32_t batch,
                                    const int32_t* slot_idx, void* ssm_pool, nhm_dtype ssm_type,
                                    uint16_t* conv_pool, int32_t n_slots, uint16_t* out, void* stream);

/* Workspace layout of nhm_mixer_prefill for up to n_tokens tokens in up to n_seqs
 * sequences with SSD chunk length `chunk`. total also covers scratch the layout does not
 * name: the chunk plan, per-chunk decays and states, and the projections' split-k partials.
 * Errors: NHM_ERR_NULL, NHM_ERR_UNSUPPORTED, NHM_ERR_SHAPE. */
NHM_API nhm_status nhm_mixer_prefill_ws_layout(const nhm_geometry* g, int64_t n_tokens, int32_t n_seqs,
                                       int32_t chunk, nhm_ws_layout* out);

/* Varlen prefill of n_seqs packed sequences: sequence i owns tokens
 * cu_seqlens[i] .. cu_seqlens[i+1]-1 of `hidden`. The Mamba2 chunk scan runs with
 * chunks of `chunk` tokens that start at each sequence's first token.
 *   hidden      (device) bf16 [n_tokens, g.hidden]
 *   cu_seqlens  (device) int32 [n_seqs+1]. Contract: cu_seqlens[0] == 0,
 *               non-decreasing, cu_seqlens[n_seqs] == n_tokens.
 *   slot_idx    (device) int32 [n_seqs]. Contract: distinct, in [0, n_slots).
 *   has_initial (device) int32 [n_seqs]: 0 starts sequence i from zero SSM state and
 *               a zero conv window; non-zero continues from pool row slot_idx[i].
 *   chunk       SSD chunk length; this build supports 128.
 *   ssm_pool, conv_pool: as for nhm_mixer_decode. The final state and window of
 *               every sequence are written to its row in place (an empty fresh
 *               sequence leaves a zero row).
 *   out         (device) bf16 [n_tokens, g.hidden]; must not overlap hidden
 *   ws          (device) >= nhm_mixer_prefill_ws_layout(g, n_tokens, n_seqs, chunk).total
 *               bytes
 * in_proj sums every product in f32 (nhm_fp8_linear_exact): its outputs feed dt, which
 * every later token's decay exponentiates, and the re-quantized out_proj input, whose e4m3
 * decisions amplify one-step differences upstream. out_proj follows nhm_fp8_linear (above
 * 16 tokens the e4m3 MFMA GEMM; its error goes to the output unamplified).
 * n_tokens == 0 with n_seqs == 0 is a valid no-op. The scan runs one block per
 * (chunk, head): (n_tokens / chunk + n_seqs) * g.n_heads above 2^31 - 1 is
 * NHM_ERR_UNSUPPORTED, and so is a projection operand of 2 GiB or more (as in
 * nhm_fp8_linear).
 * Errors: NHM_ERR_NULL, NHM_ERR_SHAPE, NHM_ERR_ALIGN, NHM_ERR_UNSUPPORTED,
 * NHM_ERR_WORKSPACE, NHM_ERR_HIP. */
NHM_API nhm_status nhm_mixer_prefill(const nhm_mixer_params* p, const uint16_t* hidden, int64_t n_tokens,
                             const int32_t* cu_seqlens, int32_t n_seqs, const int32_t* slot_idx,
                             const int32_t* has_initial, int32_t chunk, float* ssm_pool,
                             uint16_t* conv_pool, int32_t n_slots, uint16_t* out, void* ws,
                             size_t ws_bytes, void* stream);

/* nhm_mixer_decode and nhm_mixer_prefill with a choice of SSM state dtype. ssm_type
 * NHM_F32 is the calls above. NHM_BF16: ssm_pool is bf16 [n_slots, n_heads, head_dim,
 * d_state] (the state of a checkpoint whose SSM cache dtype is not f32). [PR1288] "What it
 * does": the gather widens the stored rows into an f32 working buffer and the result is
 * narrowed back to the cache dtype, a different computation from the f32 pool (the two
 * round differently). Here each touched row is widened to f32 when read (exact), the
 * call runs exactly as with the f32 pool (outputs come from the f32 state), and the
 * final state is rounded to bf16 (nearest even) when written back. The conv pool,
 * every other argument and the errors are those of the calls above; an ssm_type other
 * than NHM_F32 or NHM_BF16 is NHM_ERR_UNSUPPORTED. */
NHM_API nhm_status nhm_mixer_decode_ex(const nhm_mixer_params* p, const uint16_t* hidden, int32_t batch,
                               const int32_t* slot_idx, void* ssm_pool, nhm_dtype ssm_type,
                               uint16_t* conv_pool, int32_t n_slots, uint16_t* out, void* ws,
                               size_t ws_bytes, void* stream);
NHM_API nhm_status nhm_mixer_prefill_ex(const nhm_mixer_params* p, const uint16_t* hidden, int64_t n_tokens,
                                const int32_t* cu_seqlens, int32_t n_seqs, const int32_t* slot_idx,
                                const int32_t* has_initial, int32_t chunk, void* ssm_pool,
                                nhm_dtype ssm_type, uint16_t* conv_pool, int32_t n_slots, uint16_t* out,
                                void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NHM_H */
