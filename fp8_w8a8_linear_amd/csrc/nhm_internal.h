// Host-side declarations shared by the libnhm translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/nhm.h"

namespace nhm {

// Records a failure detail for nhm_last_error() and returns the status.
nhm_status fail(nhm_status s, const char* fmt, ...);

// Returns NHM_ERR_HIP (with the runtime's message) if the last launch failed.
nhm_status check_launch(const char* what);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Path-taken counters (nhm_dispatch_counters): one per kernel the library launches, counting
// launches and the rows (tokens, or chunks for the scan kernels) they covered. Host-side,
// atomic; a launch recorded into a HIP graph counts once, at capture.
enum class Kern : int {
    kQuantVec8, kQuantScalar, kDequantChannel, kGemv, kRing192x128, kRing192x128Exact, kRing256x128,
    kRing256x128Exact, kRing256x256, kRing256x256Exact, kPanel64x128, kPanel64x128Exact, kTile128,
    kTile128Exact, kSplitkReduce, kDecodeSsm, kGnormQuant, kClear, kConvFwd, kSsdState, kSsdPass, kSsdOut, kCount
};
void count_launch(Kern k, int64_t rows);

// ---- activation quant (quant.hip)
void launch_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, const float* scale,
                     uint8_t* q, int64_t ld_q, hipStream_t st);

// n 32-bit words set to zero (quant.hip)
void launch_clear(uint32_t* p, int n, hipStream_t st);

// per-channel e4m3 -> bf16 weight dequant (quant.hip); cols a multiple of 16, 16-byte rows
void launch_dequant_channel(const uint8_t* w, int64_t rows, int64_t cols, int64_t ld_w, const float* w_scale,
                            uint16_t* out, int64_t ld_out, hipStream_t st);

// ---- weight-streaming GEMV for m <= 16 (gemv.hip)

// out[m, n] = bf16(sum_k a[m,k] w[n,k] * a_scale * w_scale[n]); a is e4m3 [m, lda], stored to
// out[m * ld_out + n]; with out_f32 the unrounded f32 result goes to out_f32[m * ld_out + n]
// instead. out_q (bf16 output only): also E4M3(out / *q_scale) at out_q[m * ld_q + n].
// clear (optional): clear_n 32-bit words set to zero by the launch (side work of workgroup 0).
// ws_step: 1 for a weight scale per output channel, 0 for one scale (w_scale[0]) for all.
nhm_status launch_gemv(const uint8_t* a, int64_t lda, int m, const uint8_t* w, const float* w_scale,
                       const float* a_scale, int64_t n, int64_t k, uint16_t* out, int64_t ld_out, hipStream_t st,
                       float* out_f32 = nullptr, uint8_t* out_q = nullptr, int64_t ld_q = 0,
                       const float* q_scale = nullptr, uint32_t* clear = nullptr, int clear_n = 0, int ws_step = 1);

// ---- tiled MFMA GEMM for larger m (gemm.hip)
// part (16-byte aligned, part_bytes >= gemm_part_bytes(m, n, k)): scratch for the split-k
// partials of the shapes that take a split (m <= 640 with too few ring tiles); without it
// those shapes run unsplit.
size_t gemm_part_bytes(int64_t m, int64_t n, int64_t k);
// exact: every product summed in f32 (codes converted to bf16, bf16 MFMA) instead of the e4m3
// MFMA's coarser 128-product reductions.
nhm_status launch_gemm(const uint8_t* a, int64_t lda, int64_t m, const uint8_t* w, const float* w_scale,
                       const float* a_scale, int64_t n, int64_t k, uint16_t* out, int64_t ld_out,
                       hipStream_t st, float* out_f32 = nullptr, float* part = nullptr, size_t part_bytes = 0,
                       bool exact = false, int ws_step = 1);

// ---- decode SSM state update (decode.hip)
// The kernel also runs the causal conv + SiLU of the channels it reads (the head's x, the
// group's B and C) from the pre-conv projection and the carried window, stores them to
// xbc_conv, and shifts the windows of the head's x channels; the B and C channels' windows
// (read by every head of the group) are shifted by the gated-norm kernel that follows.
struct DecodeSsmArgs {
    const int32_t* slot_idx;
    float* ssm_pool;           // f32 state pool, or nullptr with ssm_pool_bf16
    uint16_t* ssm_pool_bf16;   // bf16 state pool (widened on load, rounded on store), or nullptr
    const uint16_t* zxbcdt;    // [m, d_in_proj]
    uint16_t* xbc_conv;        // [m, conv_dim] conv + SiLU output
    uint16_t* conv_pool;       // [S, W-1, conv_dim]
    const uint16_t* conv_w;    // [conv_dim, W]
    const uint16_t* conv_b;    // [conv_dim]
    const float* A_log;
    const float* D;
    const float* dt_bias;
    uint16_t* y;               // [m, d_inner]
    int32_t n_heads, n_groups, d_in_proj, conv_dim, d_inner, xbc_off, dt_off, b_off, c_off;
    // fused gated norm (cnt != nullptr): the last of a group's head workgroups to finish also
    // computes the group's gated RMSNorm and its e4m3 codes and shifts the group's B and C conv
    // windows; cnt holds one counter per (row, group), zero at launch
    uint32_t* cnt = nullptr;
    const uint16_t* norm_w = nullptr;   // [d_inner]
    const float* out_a_scale = nullptr;
    float eps = 0.f;
    int32_t z_off = 0;
    uint16_t* norm = nullptr;           // [m, d_inner]
    uint8_t* q_out = nullptr;           // [m, d_inner]
};
nhm_status launch_decode_ssm(const DecodeSsmArgs& a, int m, hipStream_t st);

// ---- gated group RMSNorm + out_proj quant (norm.hip)
struct GnormArgs {
    int64_t T;
    int32_t n_groups, d_inner, d_in_proj, z_off;
    float eps;
    const uint16_t* y;         // [T, d_inner]
    const uint16_t* zxbcdt;    // [T, d_in_proj] (z columns)
    const uint16_t* norm_w;    // [d_inner]
    const float* out_a_scale;  // [1]
    uint16_t* norm;            // [T, d_inner] bf16 norm output (nullptr: not kept)
    uint8_t* q_out;            // [T, d_inner]
    // decode: shift the B and C channels' conv windows of each token's slot (slot_idx ==
    // nullptr: none). Row 2 takes the pre-conv value from zxbcdt.
    const int32_t* slot_idx = nullptr;
    uint16_t* conv_pool = nullptr;   // [S, W-1, conv_dim]
    int32_t conv_dim = 0, xbc_off = 0, b_off = 0, c_off = 0, d_state = 0;
};
nhm_status launch_gnorm_quant(const GnormArgs& a, hipStream_t st);

// ---- prefill pieces (prefill.hip)
struct PrefillArgs {
    int64_t T;
    int32_t n_seqs, chunk, max_chunks, n_heads, n_groups, d_in_proj, conv_dim, d_inner;
    int32_t z_off, xbc_off, dt_off, b_off, c_off;
    float eps;
    const int32_t* cu_seqlens;
    const int32_t* slot_idx;
    const int32_t* has_initial;
    float* ssm_pool;           // f32 state pool, or nullptr with ssm_pool_bf16
    uint16_t* ssm_pool_bf16;   // bf16 state pool (widened on load, rounded on store), or nullptr
    uint16_t* conv_pool;
    const uint16_t* conv_w;
    const uint16_t* conv_b;
    const float* A_log;
    const float* D;
    const float* dt_bias;
    const uint16_t* norm_w;
    const float* out_a_scale;
    uint16_t* zxbcdt;         // [T, d_in_proj]
    uint16_t* xbc_conv;       // [T, conv_dim]
    int32_t* chunk_info;      // [max_chunks, 4]: seq, tok0, len, index in seq
    int32_t* seq_chunk0;      // [n_seqs + 1]
    float* chunk_cs;          // [max_chunks, n_heads, chunk]  cumulative log-decay
    float* chunk_dt;          // [max_chunks, n_heads, chunk]
    float* chunk_state;       // [max_chunks, n_heads, 64, 128]
    uint16_t* y;              // [T, d_inner]
    uint16_t* norm;           // [T, d_inner] (nullptr: not kept)
    uint8_t* q_out;           // [T, d_inner]
};
// conv + chunk plan in one launch, then the chunked scan and the gated norm + quant, in
// stream order.
nhm_status launch_prefill_mid(const PrefillArgs& a, hipStream_t st);

// SSD chunk kernels on the bf16 MFMA (ssd.hip): per (chunk, head) dt, cumulative
// log-decay and the chunk's own state; then, after the state pass, the outputs.
void launch_ssd_state(const PrefillArgs& a, hipStream_t st);
void launch_ssd_out(const PrefillArgs& a, hipStream_t st);

}  // namespace nhm
