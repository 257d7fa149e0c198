// Decode-step recurrence: one workgroup per (sequence, head) runs the causal conv + SiLU of
// the head's x channels and its group's B and C channels, then advances that head's
// f32 state rows [head_dim=64][d_state=128] of pool row slot_idx[b] in place,
//     h <- dA * h + (dt * x) (x) B,     y = h . C + D * x,
// and stores y as bf16 ([PR1288] "What it does": the paged arm advances the
// gathered recurrent rows in place). HBM-bound: the state is read and written once
// (64 KB per workgroup), streamed as 16-byte vectors with every half-wave covering
// one whole 512-byte state row.
#include "nhm_device.h"
#include "nhm_internal.h"

namespace nhm {

constexpr int kP = 64, kN = 128;
typedef uint32_t v2u __attribute__((ext_vector_type(2)));   // four bf16 state values

// kBf16: the pool holds bf16 state (the cache dtype of a checkpoint whose SSM cache is not
// f32): each row is widened to f32 on load (exact), advanced and read out in f32, and
// rounded to bf16 (nearest even) on store -- the f32 working row of the f32 pool, narrowed
// back to the cache dtype at the end of the step.
// causal depthwise conv (width 4) + SiLU of one channel: taps (bf16 pairs: taps 0,1 | 2,3)
// against the window rows u0 (oldest) .. u2 and the current pre-conv value u3; bf16 bits out
__device__ __forceinline__ uint32_t conv4_silu(uint32_t bias, uint2 taps, uint32_t u0, uint32_t u1, uint32_t u2,
                                               uint32_t u3) {
    float pre = bf16_to_f32(bias);
    pre = fmaf(bf16_to_f32(taps.x & 0xffffu), bf16_to_f32(u0), pre);
    pre = fmaf(bf16_to_f32(taps.x >> 16), bf16_to_f32(u1), pre);
    pre = fmaf(bf16_to_f32(taps.y & 0xffffu), bf16_to_f32(u2), pre);
    pre = fmaf(bf16_to_f32(taps.y >> 16), bf16_to_f32(u3), pre);
    return f32_to_bf16(silu(pre));
}

// kBf16: the pool holds bf16 state (the cache dtype of a checkpoint whose SSM cache is not
// f32): each row is widened to f32 on load (exact), advanced and read out in f32, and
// rounded to bf16 (nearest even) on store -- the f32 working row of the f32 pool, narrowed
// back to the cache dtype at the end of the step.
template <bool kBf16>
__global__ __launch_bounds__(256) void decode_ssm_kernel(const DecodeSsmArgs a) {
    const int b = blockIdx.x, h = blockIdx.y;
    const int t = threadIdx.x;
    const int hpg = a.n_heads / a.n_groups;
    const int g = h / hpg;
    const int slot = a.slot_idx[b];
    __shared__ float sx[kP], sB[kN], sC[kN];

    // The small operands first, branch-free (clamped indexes; row b of the workspace exists for
    // a padded row too, and slot row 0 stands in for its window), then the state stream: loads
    // complete in issue order, so the conv and the staging of x, B and C wait for these alone,
    // not for the state. Thread t convolves xBC channel cx (x of this head; used by t < 64) and
    // cb (B of group g for t < 128, else C).
    const int cx = h * kP + (t & (kP - 1));
    const int cb = t < kN ? a.b_off + g * kN + t : a.c_off + g * kN + t - kN;
    const uint16_t* pre = a.zxbcdt + (int64_t)b * a.d_in_proj + a.xbc_off;
    const uint32_t xcur = pre[cx], bcur = pre[cb];
    const uint2 xtap = *reinterpret_cast<const uint2*>(a.conv_w + (int64_t)cx * 4);
    const uint2 btap = *reinterpret_cast<const uint2*>(a.conv_w + (int64_t)cb * 4);
    const uint32_t xbias = a.conv_b[cx], bbias = a.conv_b[cb];
    const uint32_t dtu = a.zxbcdt[(int64_t)b * a.d_in_proj + a.dt_off + h];
    const float A_log = a.A_log[h], dt_bias = a.dt_bias[h], Dh = a.D[h];
    uint16_t* win = a.conv_pool + (int64_t)(slot < 0 ? 0 : slot) * 3 * a.conv_dim;
    const uint32_t x0 = win[cx], x1 = win[a.conv_dim + cx], x2 = win[2 * a.conv_dim + cx];
    const uint32_t b0 = win[cb], b1 = win[a.conv_dim + cb], b2 = win[2 * a.conv_dim + cb];
    asm volatile("" ::: "memory");   // keep the loads above ahead of the state stream

    uint16_t* yrow = a.y + (int64_t)b * a.d_inner + h * kP;
    uint16_t* xco = a.xbc_conv + (int64_t)b * a.conv_dim;
    const bool bc_owner = h % hpg == 0;   // one head per group stores the group's B and C
    if (slot < 0) {                       // padded row: zero outputs, no state or window touched
        if (t < kP) {
            yrow[t] = 0;
            xco[cx] = 0;
        }
        if (bc_owner) xco[cb] = 0;
        return;
    }

    // element e = 4 * (t + 256 i): p = t / 32 + 8 i, n = 4 * (t % 32) .. + 3
    const int64_t row0 = (((int64_t)slot * a.n_heads + h) * kP) * kN;
    v4f* st = reinterpret_cast<v4f*>(a.ssm_pool + (kBf16 ? 0 : row0));
    v2u* st16 = reinterpret_cast<v2u*>(a.ssm_pool_bf16 + (kBf16 ? row0 : 0));
    v4f hv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if constexpr (kBf16) {
            const v2u u = __builtin_nontemporal_load(st16 + t + 256 * i);
            hv[i] = v4f{bf16_to_f32(u[0] & 0xffffu), bf16_to_f32(u[0] >> 16), bf16_to_f32(u[1] & 0xffffu), bf16_to_f32(u[1] >> 16)};
        } else {
            hv[i] = __builtin_nontemporal_load(st + t + 256 * i);
        }
    }

    const uint32_t xo = conv4_silu(xbias, xtap, x0, x1, x2, xcur);
    const uint32_t bo = conv4_silu(bbias, btap, b0, b1, b2, bcur);
    if (t < kP) sx[t] = bf16_to_f32(xo);
    if (t < kN) sB[t] = bf16_to_f32(bo);
    else sC[t - kN] = bf16_to_f32(bo);
    if (t < kP) {                         // the conv output and this head's x windows, shifted
        xco[cx] = (uint16_t)xo;
        win[cx] = (uint16_t)x1;
        win[a.conv_dim + cx] = (uint16_t)x2;
        win[2 * a.conv_dim + cx] = (uint16_t)xcur;
    }
    if (bc_owner) xco[cb] = (uint16_t)bo;
    const float dt = softplus(bf16_to_f32(dtu) + dt_bias);
    const float dA = __expf(dt * -__expf(A_log));
    __syncthreads();

    const int n0 = 4 * (t & 31);
    const float b0f = sB[n0], b1f = sB[n0 + 1], b2f = sB[n0 + 2], b3f = sB[n0 + 3];
    const float c0 = sC[n0], c1 = sC[n0 + 1], c2 = sC[n0 + 2], c3 = sC[n0 + 3];
    float yp[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int p = (t >> 5) + 8 * i;
        const float u = dt * sx[p];
        v4f v = hv[i];
        v[0] = fmaf(dA, v[0], u * b0f);
        v[1] = fmaf(dA, v[1], u * b1f);
        v[2] = fmaf(dA, v[2], u * b2f);
        v[3] = fmaf(dA, v[3], u * b3f);
        if constexpr (kBf16)
            __builtin_nontemporal_store(v2u{f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3])}, st16 + t + 256 * i);
        else
            __builtin_nontemporal_store(v, st + t + 256 * i);
        yp[i] = v[0] * c0 + v[1] * c1 + v[2] * c2 + v[3] * c3;
    }
    // reduce over the 32 lanes that share p
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) yp[i] += __shfl_xor(yp[i], o, kWave);
    }
    if ((t & 31) == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int p = (t >> 5) + 8 * i;
            yrow[p] = (uint16_t)f32_to_bf16(yp[i] + Dh * sx[p]);
        }
    }
}

nhm_status launch_decode_ssm(const DecodeSsmArgs& a, int m, hipStream_t st) {
    if (a.ssm_pool_bf16)
        decode_ssm_kernel<true><<<dim3(m, a.n_heads), dim3(256), 0, st>>>(a);
    else
        decode_ssm_kernel<false><<<dim3(m, a.n_heads), dim3(256), 0, st>>>(a);
    count_launch(Kern::kDecodeSsm, m);
    return check_launch("decode_ssm");
}

}  // namespace nhm
