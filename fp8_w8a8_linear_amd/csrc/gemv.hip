// Weight-streaming FP8 W8A8 GEMV for m <= 16 rows (decode).
//
// The problem is HBM-bound: every weight byte is read exactly once and the
// activations (m x k e4m3, a few KB) stay in L2/L1. The contraction runs on the MFMA
// with 16 weight rows as the A operand and the (zero-padded) 16 activation rows as
// the B operand; the e4m3 codes are converted to bf16 in registers (exact) and summed
// by the bf16 MFMA, which accumulates in full f32.
//
// Decomposition: one workgroup owns 16 output features and the whole k range; its
// waves take the 128-wide k-steps round-robin (neighbouring waves read neighbouring
// 128-byte pieces of each row) and issue all their weight loads before the first
// MFMA, so a wave keeps its whole share in flight. The per-wave partial tiles are
// summed through LDS in wave order -- deterministic, and no communication between
// workgroups (an agent-scope fence would write back the L2 of every XCD).
#include "nhm_device.h"
#include "nhm_internal.h"

namespace nhm {

constexpr int kGemvMaxSteps = 8;       // k-steps per wave held in registers

struct GemvArgs {
    const uint8_t* a; int64_t lda; int m;
    const uint8_t* w; const float* w_scale; const float* a_scale; int64_t n, k;
    uint16_t* out; int64_t ld_out; bool vec_out;   // vec_out: rows aligned for 4-element stores
    float* out_f32;                                 // non-null: f32 output [m, ld_out] instead of out
    int ksteps;
    int rows;                                       // features per workgroup: 16, or a multiple of 4 below
    ConvEpilogue conv;
};

constexpr int kStreamAux = 2;   // non-temporal: weight rows are read exactly once

template <int kWaves, int kSteps, bool kConv>
__global__ __launch_bounds__(kWaves * 64) void gemv_kernel(const GemvArgs g) {
    __shared__ v4f s_red[kWaves][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * g.rows;
    const int64_t row = n0 + (lane & 15);       // A operand row (feature); rows past g.rows load zeros
    const int64_t nend = n0 + g.rows < g.n ? n0 + g.rows : g.n;   // this workgroup's features end
    const int col = lane & 15;                  // B operand column (token)
    const int kq = (lane >> 4) * 32;
    const int64_t nbase = n0 + 4 * (lane >> 4);

    // Everything up to the MFMAs is straight-line code: loads past the operands go to an
    // out-of-range buffer offset (zeros) and indexes are clamped, so the compiler can wait
    // for each k-step's loads alone instead of for all outstanding loads at a branch join.
    // First the small operands of the epilogue (so that waiting for them later does not
    // wait for the weight stream), then the weight stream, k-step by k-step.
    const float sa = *g.a_scale;
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = sa * g.w_scale[nbase + r < g.n ? nbase + r : g.n - 1];
    int slot = -1;
    int64_t ch = -1;
    uint4 cw0{}, cw1{};
    uint2 cb{};
    if constexpr (kConv) {
        const ConvEpilogue& c = g.conv;
        ch = nbase - c.xbc_off;
        const int64_t chc = ch < 0 ? 0 : (ch > c.conv_dim - 4 ? c.conv_dim - 4 : ch);
        slot = c.slot_idx[col < g.m ? col : 0];
        cw0 = *reinterpret_cast<const uint4*>(c.conv_w + chc * 4);      // taps of channels ch, ch+1
        cw1 = *reinterpret_cast<const uint4*>(c.conv_w + chc * 4 + 8);  // channels ch+2, ch+3
        cb = *reinterpret_cast<const uint2*>(c.conv_b + chc);
        if (ch >= c.conv_dim || col >= g.m) ch = -1;
    }

    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc((void*)g.w, (short)0, (int)(g.n * g.k), 0x00020000);
    const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc((void*)g.a, (short)0, (int)(g.m * g.lda), 0x00020000);
    const uint32_t wrow = row < nend ? (uint32_t)(row * g.k) : kGemvOut;
    const uint32_t arow = col < g.m ? (uint32_t)(col * g.lda) : kGemvOut;
    // weight and activation pieces of each k-step are issued together
    v8i wa[kSteps], xb[kSteps];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        const int kb = (wave + i * kWaves) * 128 + kq;
        wa[i] = bload32<kStreamAux>(wrs, kb < g.k ? wrow + kb : kGemvOut, kb + 16 < g.k ? wrow + kb + 16 : kGemvOut);
        xb[i] = bload32<0>(ars, kb < g.k ? arow + kb : kGemvOut, kb + 16 < g.k ? arow + kb + 16 : kGemvOut);
    }
    // the carried conv window of this token's sequence (slot row 0 stands in for a padded row)
    uint2 w0{}, w1{}, w2{};
    if constexpr (kConv) {
        const ConvEpilogue& c = g.conv;
        const int64_t chc = ch < 0 ? 0 : ch;
        const uint16_t* win = c.conv_pool + (int64_t)(slot < 0 ? 0 : slot) * 3 * c.conv_dim + chc;
        w0 = *reinterpret_cast<const uint2*>(win);
        w1 = *reinterpret_cast<const uint2*>(win + c.conv_dim);
        w2 = *reinterpret_cast<const uint2*>(win + 2 * c.conv_dim);
    }
    // keep every load above issued before the first MFMA (the scheduler would otherwise sink
    // later steps' loads below earlier steps' MFMAs, serialising the stream)
    __builtin_amdgcn_sched_barrier(0);

    // Exact f32 accumulation: each 128-k step runs as four bf16 MFMAs on the converted codes
    // (sub-step j takes bytes 8j .. 8j+7 of the lane's 32, the same bytes of both operands).
    // The e4m3 MFMA would be 4x fewer instructions but sums coarser than f32; this kernel is
    // bound by the weight stream, and the conversions and MFMAs of a step run while later
    // steps are still streaming in. Steps past k hold zeros and add nothing.
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kSteps; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc = mfma_bf16(e4m3x8_to_bf16(wa[i][2 * j], wa[i][2 * j + 1]), e4m3x8_to_bf16(xb[i][2 * j], xb[i][2 * j + 1]),
                            acc);

    if (wave > 0) s_red[wave][lane] = acc;
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < kWaves; ++w) acc += s_red[w][lane];

    // acc[r] = D[feature nbase + r][token col]
    if (col >= g.m) return;
    if (g.out_f32) {   // (never with the conv epilogue)
        float* of = g.out_f32 + (int64_t)col * g.ld_out + nbase;
        if (g.vec_out && nbase + 3 < nend) {
            *reinterpret_cast<float4*>(of) = make_float4(acc[0] * sc[0], acc[1] * sc[1], acc[2] * sc[2], acc[3] * sc[3]);
        } else {
            for (int r = 0; r < 4; ++r)
                if (nbase + r < nend) of[r] = acc[r] * sc[r];
        }
        return;
    }
    uint32_t hb[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) hb[r] = f32_to_bf16(acc[r] * sc[r]);
    uint16_t* o = g.out + (int64_t)col * g.ld_out + nbase;
    if (g.vec_out && nbase + 3 < nend) {
        *reinterpret_cast<uint2*>(o) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
    } else {
        for (int r = 0; r < 4; ++r)
            if (nbase + r < nend) o[r] = (uint16_t)hb[r];
    }

    if constexpr (kConv) {
        // causal depthwise conv (width 4) + SiLU on the xBC features, window shift in place
        const ConvEpilogue& c = g.conv;
        if (ch < 0) return;
        uint16_t* xo = c.xbc_conv + (int64_t)col * c.conv_dim + ch;
        if (slot < 0) {
            *reinterpret_cast<uint2*>(xo) = make_uint2(0u, 0u);
            return;
        }
        uint16_t* win = c.conv_pool + (int64_t)slot * 3 * c.conv_dim + ch;
        const uint32_t u0[4] = {w0.x & 0xffffu, w0.x >> 16, w0.y & 0xffffu, w0.y >> 16};
        const uint32_t u1[4] = {w1.x & 0xffffu, w1.x >> 16, w1.y & 0xffffu, w1.y >> 16};
        const uint32_t u2[4] = {w2.x & 0xffffu, w2.x >> 16, w2.y & 0xffffu, w2.y >> 16};
        const uint32_t wt[8] = {cw0.x, cw0.y, cw0.z, cw0.w, cw1.x, cw1.y, cw1.z, cw1.w};
        const uint32_t bb[4] = {cb.x & 0xffffu, cb.x >> 16, cb.y & 0xffffu, cb.y >> 16};
        uint32_t ob[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // taps of channel ch+r: bf16 [4] = words wt[2r] (taps 0,1) and wt[2r+1] (taps 2,3)
            float pre = bf16_to_f32(bb[r]);
            pre = fmaf(bf16_to_f32(wt[2 * r] & 0xffffu), bf16_to_f32(u0[r]), pre);
            pre = fmaf(bf16_to_f32(wt[2 * r] >> 16), bf16_to_f32(u1[r]), pre);
            pre = fmaf(bf16_to_f32(wt[2 * r + 1] & 0xffffu), bf16_to_f32(u2[r]), pre);
            pre = fmaf(bf16_to_f32(wt[2 * r + 1] >> 16), bf16_to_f32(hb[r]), pre);
            ob[r] = f32_to_bf16(silu(pre));
        }
        *reinterpret_cast<uint2*>(xo) = make_uint2(ob[0] | (ob[1] << 16), ob[2] | (ob[3] << 16));
        *reinterpret_cast<uint2*>(win) = w1;
        *reinterpret_cast<uint2*>(win + c.conv_dim) = w2;
        *reinterpret_cast<uint2*>(win + 2 * c.conv_dim) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
    }
}

nhm_status launch_gemv(const uint8_t* a, int64_t lda, int m, const uint8_t* w, const float* w_scale,
                       const float* a_scale, int64_t n, int64_t k, uint16_t* out, int64_t ld_out,
                       const ConvEpilogue* conv, hipStream_t st, float* out_f32) {
    GemvArgs g;
    g.a = a; g.lda = lda; g.m = m;
    g.w = w; g.w_scale = w_scale; g.a_scale = a_scale; g.n = n; g.k = k;
    g.out = out; g.ld_out = ld_out;
    g.out_f32 = conv ? nullptr : out_f32;
    g.vec_out = out_f32 ? ld_out % 4 == 0 && reinterpret_cast<uintptr_t>(out_f32) % 16 == 0
                        : ld_out % 4 == 0 && reinterpret_cast<uintptr_t>(out) % 8 == 0;
    g.ksteps = (int)((k + 127) / 128);
    g.conv = conv ? *conv : ConvEpilogue{};
    if (g.ksteps > 16 * kGemvMaxSteps)
        return fail(NHM_ERR_UNSUPPORTED, "gemv: k %lld exceeds %d", (long long)k, 16 * 128 * kGemvMaxSteps);
    if (n * k >= (int64_t(1) << 31) || (int64_t)m * lda >= (int64_t(1) << 31))
        return fail(NHM_ERR_UNSUPPORTED, "gemv: operands of 2 GiB or more");
    // 4 waves up to 23 k-steps (k < 2944), then 8, then 16; each wave holds its steps in
    // registers, their count rounded up to 2, 4, 6 or 8
    const int waves = g.ksteps < 24 ? 4 : (g.ksteps <= 8 * kGemvMaxSteps ? 8 : 16);
    const int per = (g.ksteps + waves - 1) / waves;
    const int steps = per <= 2 ? 2 : per <= 4 ? 4 : per <= 6 ? 6 : 8;
    // 16 features per workgroup; where that leaves CUs idle (n < 16 x 256), fewer features
    // per workgroup, a multiple of 4 (whole 4-feature stores), so that the workgroups cover
    // more CUs: each CU streams its share of the weight at a rate bounded by the requests it
    // can keep in flight, so the weight is delivered faster over more CUs (the spare MFMA rows
    // load zeros). The conv epilogue keeps 16.
    g.rows = 16;
    if (!conv && n < 16 * 256) {
        const int64_t per = (n + 255) / 256;
        g.rows = per <= 4 ? 4 : (int)((per + 3) / 4 * 4);
    }
    const dim3 grid((unsigned)((n + g.rows - 1) / g.rows));
#define NHM_GEMV_LAUNCH(W, S)                                                  \
    do {                                                                       \
        if (conv) gemv_kernel<W, S, true><<<grid, dim3(W * 64), 0, st>>>(g);  \
        else gemv_kernel<W, S, false><<<grid, dim3(W * 64), 0, st>>>(g);      \
    } while (0)
#define NHM_GEMV_STEPS(W)                         \
    do {                                          \
        if (steps == 2) NHM_GEMV_LAUNCH(W, 2);    \
        else if (steps == 4) NHM_GEMV_LAUNCH(W, 4); \
        else if (steps == 6) NHM_GEMV_LAUNCH(W, 6); \
        else NHM_GEMV_LAUNCH(W, 8);               \
    } while (0)
    if (waves == 4) NHM_GEMV_STEPS(4);
    else if (waves == 8) NHM_GEMV_STEPS(8);
    else NHM_GEMV_STEPS(16);
#undef NHM_GEMV_STEPS
#undef NHM_GEMV_LAUNCH
    return check_launch("gemv");
}

}  // namespace nhm
