// Gated group RMSNorm fused with the static e4m3 quant of the out_proj input
// ([PR1288] "What it does": RmsNormGatedGroup(n_groups) -> out_proj (FP8 W8A8)).
//
// One wave per (token, group): v = y * silu(z); o = bf16(v / sqrt(mean(v^2) + eps) * w);
// q = E4M3(o / s_out). The gate is applied before the mean square; groups are
// contiguous runs of d_inner / n_groups channels. HBM-bound: reads y and z (bf16),
// writes o (bf16) and q (e4m3), 8 channels per lane per 16-byte load.
#include "nhm_device.h"
#include "nhm_internal.h"

namespace nhm {

// kIt > 0: groups of up to kIt * 512 channels; v = y * silu(z) is kept in registers
// between the mean square and the output, so y and z are read once and the gate is
// evaluated once per element. kIt == 0: any group width, two passes over y and z.
template <int kIt>
__global__ __launch_bounds__(256) void gnorm_quant_kernel(const GnormArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pair >= a.T * a.n_groups) return;
    const int64_t tok = pair / a.n_groups;
    const int g = (int)(pair % a.n_groups);
    const int gw = a.d_inner / a.n_groups;
    const uint16_t* yr = a.y + tok * a.d_inner + (int64_t)g * gw;
    const uint16_t* zr = a.zxbcdt + tok * a.d_in_proj + a.z_off + (int64_t)g * gw;
    const float so = *a.out_a_scale;
    // decode: this token's slot's conv windows of group g's B (lanes 0-31) and C (32-63)
    // channels, four per lane, shifted by one row (the decode state kernel, which reads them,
    // has finished; the x channels' windows it shifts itself). Loads go out with y and z.
    int wslot = -1;
    int64_t wc = 0;
    uint2 r1{}, r2{};
    uint32_t cur[4] = {0u, 0u, 0u, 0u};
    if (a.slot_idx) {
        wslot = a.slot_idx[tok];
        wc = lane < 32 ? a.b_off + (int64_t)g * a.d_state + 4 * lane : a.c_off + (int64_t)g * a.d_state + 4 * (lane - 32);
        const uint16_t* win = a.conv_pool + (int64_t)(wslot < 0 ? 0 : wslot) * 3 * a.conv_dim + wc;
        r1 = *reinterpret_cast<const uint2*>(win + a.conv_dim);
        r2 = *reinterpret_cast<const uint2*>(win + 2 * a.conv_dim);
        const uint16_t* pc = a.zxbcdt + tok * a.d_in_proj + a.xbc_off + wc;
#pragma unroll
        for (int j = 0; j < 4; ++j) cur[j] = pc[j];
    }
    // emit(c, v, r, nw): nw holds norm_w[c .. c + 7] (loaded with y and z where possible)
    auto emit = [&](int c, const float (&v)[8], float r, const uint4 nw) {
        const bool fast = fast_scale(so);    // the quant's reciprocal form (exact; see quant_bf16x8_fast)
        const float rso = __fdiv_rn(1.0f, so);
        float w[8];
        unpack8(nw, w);
        uint32_t ob[4];   // bf16 pairs
#pragma unroll
        for (int j = 0; j < 4; ++j) ob[j] = f32x2_to_bf16x2(v[2 * j] * r * w[2 * j], v[2 * j + 1] * r * w[2 * j + 1]);
        const int64_t o = tok * a.d_inner + (int64_t)g * gw + c;
        if (a.norm) *reinterpret_cast<uint4*>(a.norm + o) = make_uint4(ob[0], ob[1], ob[2], ob[3]);
        const uint4 ov = make_uint4(ob[0], ob[1], ob[2], ob[3]);
        uint2 code;
        if (fast && __builtin_amdgcn_ballot_w64(bf16x8_special(ov) != 0u) == 0) code = quant_bf16x8_fast(ov, so, rso);
        else code = quant_bf16x8(ov, so);
        *reinterpret_cast<uint2*>(a.q_out + o) = code;
    };
    float ss = 0.f;
    if constexpr (kIt > 0) {
        float v[kIt][8];
        uint4 yv[kIt], zv[kIt], wv[kIt];
#pragma unroll
        for (int it = 0; it < kIt; ++it) {                 // all loads first (norm weights too)
            const int c = lane * 8 + it * 512;
            const int cc = c < gw ? c : 0;                 // in bounds; masked below
            yv[it] = *reinterpret_cast<const uint4*>(yr + cc);
            zv[it] = *reinterpret_cast<const uint4*>(zr + cc);
            wv[it] = *reinterpret_cast<const uint4*>(a.norm_w + (int64_t)g * gw + cc);
        }
        // the scale's scalar load goes out with them, not after the reduction
        asm volatile("" ::"s"(so) : "memory");
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            float y[8], z[8];
            unpack8(yv[it], y);
            unpack8(zv[it], z);
            const bool in = lane * 8 + it * 512 < gw;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                v[it][j] = in ? y[j] * silu(z[j]) : 0.f;
                ss += v[it][j] * v[it][j];
            }
        }
        ss = wave_sum(ss);
        const float r = 1.0f / sqrtf(ss / (float)gw + a.eps);
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int c = lane * 8 + it * 512;
            if (c < gw) emit(c, v[it], r, wv[it]);
        }
    } else {
        for (int c = lane * 8; c < gw; c += 64 * 8) {
            float y[8], z[8];
            unpack8(*reinterpret_cast<const uint4*>(yr + c), y);
            unpack8(*reinterpret_cast<const uint4*>(zr + c), z);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float v = y[j] * silu(z[j]);
                ss += v * v;
            }
        }
        ss = wave_sum(ss);
        const float r = 1.0f / sqrtf(ss / (float)gw + a.eps);
        for (int c = lane * 8; c < gw; c += 64 * 8) {
            float y[8], z[8], v[8];
            unpack8(*reinterpret_cast<const uint4*>(yr + c), y);
            unpack8(*reinterpret_cast<const uint4*>(zr + c), z);
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = y[j] * silu(z[j]);
            emit(c, v, r, *reinterpret_cast<const uint4*>(a.norm_w + (int64_t)g * gw + c));
        }
    }
    if (wslot >= 0) {
        uint16_t* win = a.conv_pool + (int64_t)wslot * 3 * a.conv_dim + wc;
        *reinterpret_cast<uint2*>(win) = r1;
        *reinterpret_cast<uint2*>(win + a.conv_dim) = r2;
        *reinterpret_cast<uint2*>(win + 2 * a.conv_dim) = make_uint2(cur[0] | (cur[1] << 16), cur[2] | (cur[3] << 16));
    }
}

nhm_status launch_gnorm_quant(const GnormArgs& a, hipStream_t st) {
    if (a.T <= 0) return NHM_OK;
    const dim3 grid((unsigned)((a.T * a.n_groups + 3) / 4));
    const int gw = a.d_inner / a.n_groups;
    if (gw <= 512) gnorm_quant_kernel<1><<<grid, 256, 0, st>>>(a);
    else if (gw <= 1024) gnorm_quant_kernel<2><<<grid, 256, 0, st>>>(a);
    else if (gw <= 2048) gnorm_quant_kernel<4><<<grid, 256, 0, st>>>(a);
    else gnorm_quant_kernel<0><<<grid, 256, 0, st>>>(a);
    count_launch(Kern::kGnormQuant, a.T);
    return check_launch("gnorm_quant");
}

}  // namespace nhm
