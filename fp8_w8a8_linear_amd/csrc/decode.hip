// Decode-step recurrence: one workgroup per (sequence, head) runs the causal conv + SiLU of
// the head's x channels and its group's B and C channels, then advances that head's
// f32 state rows [head_dim=64][d_state=128] of pool row slot_idx[b] in place,
//     h <- dA * h + (dt * x) (x) B,     y = h . C + D * x,
// and stores y as bf16 ([PR1288] "What it does": the paged arm advances the
// gathered recurrent rows in place). HBM-bound: the state is read and written once
// (64 KB per workgroup), streamed as 16-byte vectors with every half-wave covering
// one whole 512-byte state row.
//
// Fused gated norm: the heads of a norm group are the group's workgroups of one row, and the
// last of them to finish also computes the group's gated RMSNorm, the e4m3 codes of its
// output (the out_proj input) and the shift of the group's B and C conv windows, which every
// head's workgroup reads. The hand-off uses no fences: each workgroup writes its y through
// the caches to the device-coherent level (sc0 sc1 stores), waits for those stores, and counts
// itself in with a relaxed device-scope atomic; the workgroup that counts last reads the
// group's y past the caches (sc0 sc1 loads). Measured on MI355X in an SSM-update-shaped probe
// (512 workgroups streaming 32 KB each), this hand-off adds ~2 us per launch against ~16 us
// for an acquire-release counter, whose fences write back and invalidate each XCD's L2;
// ~1,000 graph-replayed launches read no stale value.
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
__device__ __forceinline__ void store_state(v4f* st, v2u* st16, int i, const v4f& v) {
    if constexpr (kBf16)
        __builtin_nontemporal_store(v2u{f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3])}, st16 + i);
    else
        __builtin_nontemporal_store(v, st + i);
}

// The cache policy of the y hand-off: stores written through to, and loads served from, the
// device-coherent level (sc0 sc1).
constexpr int kCoherent = 0x11;

template <bool kBf16, bool kFused>
__global__ __launch_bounds__(256) void decode_ssm_kernel(const DecodeSsmArgs a) {
    const int b = blockIdx.x, h = blockIdx.y;
    const int t = threadIdx.x;
    const int hpg = a.n_heads / a.n_groups;
    const int g = h / hpg;
    const int gw = hpg * kP;              // channels of a norm group (fused: at most 512)
    const int slot = a.slot_idx[b];
    __shared__ float sx[kP], sB[kN], sC[kN];
    __shared__ uint32_t s_y[kP / 2];
    __shared__ float s_ss[4];
    __shared__ uint32_t s_old;

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
    // fused: the group's gate values and norm weights, two channels per thread (the workgroup
    // that finishes the group uses them; loaded by all, ahead of the state stream)
    uint32_t zz = 0u, nw = 0u;
    if constexpr (kFused) {
        if (2 * t < gw) {
            zz = *reinterpret_cast<const uint32_t*>(a.zxbcdt + (int64_t)b * a.d_in_proj + a.z_off + g * gw + 2 * t);
            nw = *reinterpret_cast<const uint32_t*>(a.norm_w + g * gw + 2 * t);
        }
    }
    asm volatile("" ::: "memory");   // keep the loads above ahead of the state stream

    uint16_t* yrow = a.y + (int64_t)b * a.d_inner + h * kP;
    uint16_t* xco = a.xbc_conv + (int64_t)b * a.conv_dim;
    const bool bc_owner = h % hpg == 0;   // one head per group stores the group's B and C
    if (slot < 0) {                       // padded row: zero outputs, no state or window touched
        if (t < kP) {
            yrow[t] = 0;
            xco[cx] = 0;
        }
        if (bc_owner) {
            xco[cb] = 0;
            if constexpr (kFused) {       // the group's norm output and codes (no hand-off)
                const int64_t o = (int64_t)b * a.d_inner + g * gw;
                for (int c = 2 * t; c < gw; c += 512) {
                    *reinterpret_cast<uint32_t*>(a.norm + o + c) = 0u;
                    *reinterpret_cast<uint16_t*>(a.q_out + o + c) = 0;
                }
            }
        }
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
    // every state load is issued before the conv below, whose arithmetic waits for the small
    // loads (scheduled among the state loads, it held the state stream back by their round trip)
    __builtin_amdgcn_sched_barrier(0);

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
        v4f& v = hv[i];
        v[0] = fmaf(dA, v[0], u * b0f);
        v[1] = fmaf(dA, v[1], u * b1f);
        v[2] = fmaf(dA, v[2], u * b2f);
        v[3] = fmaf(dA, v[3], u * b3f);
        if constexpr (!kFused) store_state<kBf16>(st, st16, t + 256 * i, v);
        yp[i] = v[0] * c0 + v[1] * c1 + v[2] * c2 + v[3] * c3;
    }
    // reduce over the 32 lanes that share p (the sums land in the half's last lane)
#pragma unroll
    for (int i = 0; i < 8; ++i) yp[i] = half_sum(yp[i]);
    if constexpr (!kFused) {
        if ((t & 31) == 31) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int p = (t >> 5) + 8 * i;
                yrow[p] = (uint16_t)f32_to_bf16(yp[i] + Dh * sx[p]);
            }
        }
        return;
    } else {
        if ((t & 31) == 31) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int p = (t >> 5) + 8 * i;
                reinterpret_cast<uint16_t*>(s_y)[p] = (uint16_t)f32_to_bf16(yp[i] + Dh * sx[p]);
            }
        }
        __syncthreads();
        // y written through to the device-coherent level and waited for, then counted in; the
        // state stores go out behind the count, while its round trip is in flight
        const __amdgpu_buffer_rsrc_t yrs =
            __builtin_amdgcn_make_buffer_rsrc((void*)a.y, (short)0, (int)((int64_t)gridDim.x * a.d_inner * 2), 0x00020000);
        if (t < kP / 2) __builtin_amdgcn_raw_buffer_store_b32(s_y[t], yrs, (uint32_t)(((int64_t)b * a.d_inner + h * kP + 2 * t) * 2), 0, kCoherent);
        wait_vmcnt<0>();
        __syncthreads();
        uint32_t old = 0u;
        if (t == 0) old = __hip_atomic_fetch_add(a.cnt + (int64_t)b * a.n_groups + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < 8; ++i) store_state<kBf16>(st, st16, t + 256 * i, hv[i]);
        if (t == 0) s_old = old;
        __syncthreads();
        if (s_old % (uint32_t)hpg != (uint32_t)(hpg - 1)) return;

        // Last of the group: gated RMSNorm over the group's gw channels (two per thread), the
        // codes E4M3(o / s_out) of the bf16 output, and the shift of the group's B and C windows
        // (thread t holds channel cb's window rows and current value).
        const int64_t o = (int64_t)b * a.d_inner + g * gw;
        float v0 = 0.f, v1 = 0.f, ss = 0.f;
        if (2 * t < gw) {
            const uint32_t yy = __builtin_amdgcn_raw_buffer_load_b32(yrs, (uint32_t)((o + 2 * t) * 2), 0, kCoherent);
            v0 = bf16_to_f32(yy & 0xffffu) * silu(bf16_to_f32(zz & 0xffffu));
            v1 = bf16_to_f32(yy >> 16) * silu(bf16_to_f32(zz >> 16));
            ss = v0 * v0 + v1 * v1;
        }
        ss = wave_sum(ss);
        if ((t & 63) == 0) s_ss[t >> 6] = ss;
        __syncthreads();
        ss = s_ss[0] + s_ss[1] + s_ss[2] + s_ss[3];
        const float r = 1.0f / sqrtf(ss / (float)gw + a.eps);
        if (2 * t < gw) {
            const uint32_t ob = f32x2_to_bf16x2(v0 * r * bf16_to_f32(nw & 0xffffu), v1 * r * bf16_to_f32(nw >> 16));
            *reinterpret_cast<uint32_t*>(a.norm + o + 2 * t) = ob;
            const float so = *a.out_a_scale;
            *reinterpret_cast<uint16_t*>(a.q_out + o + 2 * t) =
                (uint16_t)(quant_bf16(ob & 0xffffu, so) | (quant_bf16(ob >> 16, so) << 8));
        }
        win[cb] = (uint16_t)b1;
        win[a.conv_dim + cb] = (uint16_t)b2;
        win[2 * a.conv_dim + cb] = (uint16_t)bcur;
    }
}

nhm_status launch_decode_ssm(const DecodeSsmArgs& a, int m, hipStream_t st) {
    const dim3 grid(m, a.n_heads);
    if (a.cnt) {
        if (a.ssm_pool_bf16) decode_ssm_kernel<true, true><<<grid, dim3(256), 0, st>>>(a);
        else decode_ssm_kernel<false, true><<<grid, dim3(256), 0, st>>>(a);
    } else {
        if (a.ssm_pool_bf16) decode_ssm_kernel<true, false><<<grid, dim3(256), 0, st>>>(a);
        else decode_ssm_kernel<false, false><<<grid, dim3(256), 0, st>>>(a);
    }
    count_launch(Kern::kDecodeSsm, m);
    return check_launch("decode_ssm");
}

}  // namespace nhm
