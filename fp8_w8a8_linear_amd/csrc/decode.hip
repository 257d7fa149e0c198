// Decode step after in_proj: the state update of one token, the gated group
// RMSNorm and the e4m3 quant of the out_proj input, in one kernel.
//
// One workgroup per (sequence b, group g) owns the group's heads_per_group heads:
//   for each head h, f32 state rows [head_dim=64][d_state=128] of pool row slot_idx[b]:
//     h <- dA * h + (dt * x) (x) B,   y = h . C + D * x          (in place)
//   then over the group's heads_per_group * 64 channels:
//     v = y * silu(z),  o = bf16(v / sqrt(mean(v^2) + eps) * w),  q = E4M3(o / s_out)
// ([PR1288] "What it does": the paged arm advances the gathered recurrent rows in
// place; Mamba2ChunkScan -> RmsNormGatedGroup(n_groups) -> out_proj (FP8 W8A8)).
// Owning the whole group lets the norm run from LDS with no second launch and no
// communication between workgroups. HBM-bound: each workgroup streams its heads'
// state once in and once out (512 KB at 8 heads), all loads issued up front, every
// 32 consecutive lanes covering one 512-byte state row.
#include "nhm_device.h"
#include "nhm_internal.h"

namespace nhm {

constexpr int kP = 64, kN = 128;
constexpr int kMaxHpg = 8;                 // heads per group held by one workgroup
constexpr int kRowsPerThread = kP / 4;     // 16 float4 of state per thread

__global__ __launch_bounds__(kMaxHpg * 128) void decode_ssm_kernel(const DecodeSsmArgs a) {
    const int b = blockIdx.x, g = blockIdx.y;
    const int t = threadIdx.x;
    const int hpg = a.n_heads / a.n_groups;
    const int gw = hpg * kP;                   // channels of the group
    const int hh = t >> 7;                     // head within the group
    const int tl = t & 127;
    const int h = g * hpg + hh;
    const int slot = a.slot_idx[b];
    __shared__ float s_x[kMaxHpg * kP], s_B[kN], s_C[kN], s_y[kMaxHpg * kP];
    __shared__ float s_dt[kMaxHpg], s_dA[kMaxHpg], s_red[kMaxHpg * 2];

    v4f hv[kRowsPerThread];
    v4f* st = nullptr;
    if (slot >= 0) {
        // element e = 4 * (tl + 128 i): p = tl / 32 + 4 i, n = 4 * (tl % 32) .. + 3
        st = reinterpret_cast<v4f*>(a.ssm_pool + (((int64_t)slot * a.n_heads + h) * kP) * kN);
#pragma unroll
        for (int i = 0; i < kRowsPerThread; ++i) hv[i] = __builtin_nontemporal_load(st + tl + 128 * i);
        const uint16_t* xr = a.xbc_conv + (int64_t)b * a.conv_dim;
        if (t < gw) s_x[t] = bf16_to_f32(xr[g * gw + t]);
        for (int e = t; e < 2 * kN; e += blockDim.x) {
            if (e < kN) s_B[e] = bf16_to_f32(xr[a.b_off + g * kN + e]);
            else s_C[e - kN] = bf16_to_f32(xr[a.c_off + g * kN + e - kN]);
        }
        if (t < hpg) {
            const int hd = g * hpg + t;
            const float dt = softplus(bf16_to_f32(a.zxbcdt[(int64_t)b * a.d_in_proj + a.dt_off + hd]) + a.dt_bias[hd]);
            s_dt[t] = dt;
            s_dA[t] = __expf(dt * -__expf(a.A_log[hd]));
        }
    }
    __syncthreads();
    if (slot >= 0) {
        const float dt = s_dt[hh], dA = s_dA[hh];
        const int n0 = 4 * (tl & 31);
        const float b0 = s_B[n0], b1 = s_B[n0 + 1], b2 = s_B[n0 + 2], b3 = s_B[n0 + 3];
        const float c0 = s_C[n0], c1 = s_C[n0 + 1], c2 = s_C[n0 + 2], c3 = s_C[n0 + 3];
        float yp[kRowsPerThread];
#pragma unroll
        for (int i = 0; i < kRowsPerThread; ++i) {
            const int p = (tl >> 5) + 4 * i;
            const float u = dt * s_x[hh * kP + p];
            v4f v = hv[i];
            v[0] = fmaf(dA, v[0], u * b0);
            v[1] = fmaf(dA, v[1], u * b1);
            v[2] = fmaf(dA, v[2], u * b2);
            v[3] = fmaf(dA, v[3], u * b3);
            __builtin_nontemporal_store(v, st + tl + 128 * i);
            yp[i] = v[0] * c0 + v[1] * c1 + v[2] * c2 + v[3] * c3;
        }
        // reduce over the 32 lanes that share p
#pragma unroll
        for (int i = 0; i < kRowsPerThread; ++i) {
#pragma unroll
            for (int o = 16; o >= 1; o >>= 1) yp[i] += __shfl_xor(yp[i], o, kWave);
        }
        if ((tl & 31) == 0) {
            const float Dh = a.D[h];
#pragma unroll
            for (int i = 0; i < kRowsPerThread; ++i) {
                const int p = (tl >> 5) + 4 * i;
                s_y[hh * kP + p] = bf16_to_f32(f32_to_bf16(yp[i] + Dh * s_x[hh * kP + p]));
            }
        }
    } else if (t < gw) {
        s_y[t] = 0.f;                       // padded row: zero output, no state touched
    }
    __syncthreads();

    // ---- gated group RMSNorm + e4m3 quant over the group's gw channels (one per thread)
    const int64_t ch = (int64_t)b * a.d_inner + (int64_t)g * gw + t;
    float v = 0.f;
    if (t < gw) {
        const float yv = s_y[t];
        a.y[ch] = (uint16_t)f32_to_bf16(yv);
        v = yv * silu(bf16_to_f32(a.zxbcdt[(int64_t)b * a.d_in_proj + a.z_off + (int64_t)g * gw + t]));
    }
    float ss = wave_sum(v * v);
    if ((t & 63) == 0) s_red[t >> 6] = ss;
    __syncthreads();
    if (t < gw) {
        float tot = 0.f;
        for (int w = 0; w < (gw + 63) / 64; ++w) tot += s_red[w];
        const float r = 1.0f / sqrtf(tot / (float)gw + a.eps);
        const uint32_t ob = f32_to_bf16(v * r * bf16_to_f32(a.norm_w[(int64_t)g * gw + t]));
        a.norm[ch] = (uint16_t)ob;
        a.q_out[ch] = (uint8_t)quant_bf16(ob, *a.out_a_scale);
    }
}

nhm_status launch_decode_ssm(const DecodeSsmArgs& a, int m, hipStream_t st) {
    const int hpg = a.n_heads / a.n_groups;
    if (hpg > kMaxHpg) return fail(NHM_ERR_UNSUPPORTED, "decode: %d heads per group (at most %d)", hpg, kMaxHpg);
    decode_ssm_kernel<<<dim3(m, a.n_groups), dim3(hpg * 128), 0, st>>>(a);
    return check_launch("decode_ssm");
}

}  // namespace nhm
