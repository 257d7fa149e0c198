// Weight-streaming FP8 W8A8 GEMV for m <= 16 rows (decode).
//
// The problem is HBM-bound: every weight byte is read exactly once and the
// activations (m x k e4m3, a few KB) stay in L2/L1. The contraction still runs on
// the 16x16x128 e4m3 MFMA: the 16 weight rows of a wave are the A operand, the
// (zero-padded) 16 activation rows the B operand, so the VALU never converts fp8.
//
// Decomposition: a workgroup of 4 waves owns 64 output features (16 per wave) and
// one slice of the k-steps (128 k each). All weight loads of the slice are issued
// before the first MFMA so each wave keeps its whole slice in flight. When k is
// split across workgroups, each workgroup stores an f32 partial and the last one
// to arrive (atomic counter) sums the partials in split order -- deterministic,
// no float atomics -- and runs the epilogue. The counter is reset to 0 by that
// last workgroup.
#include "nhm_device.h"
#include "nhm_internal.h"

namespace nhm {

constexpr int kGemvRows = 64;          // output features per workgroup
constexpr int kGemvMaxSteps = 8;       // k-steps per workgroup (registers)

GemvPlan gemv_plan(int64_t n, int64_t k) {
    GemvPlan p;
    p.row_blocks = (int)((n + kGemvRows - 1) / kGemvRows);
    p.ksteps = (int)((k + 127) / 128);
    // about 640 workgroups (2.5 per CU), at least 4 and at most 8 k-steps each
    long target = ((long)p.ksteps * p.row_blocks + 639) / 640;
    int sps = (int)(target < 4 ? 4 : target);
    if (sps > kGemvMaxSteps) sps = kGemvMaxSteps;
    if (sps > p.ksteps) sps = p.ksteps;
    if (sps < 1) sps = 1;
    p.ksplit = (p.ksteps + sps - 1) / sps;
    p.steps_per_split = (p.ksteps + p.ksplit - 1) / p.ksplit;
    return p;
}

size_t gemv_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    const GemvPlan p = gemv_plan(n, k);
    size_t bytes = align_up((size_t)p.row_blocks * sizeof(unsigned), 256);
    if (p.ksplit > 1) bytes += align_up((size_t)p.ksplit * (size_t)n * (size_t)m * sizeof(float), 256);
    return bytes;
}

// 32 bytes of row `row` starting at byte `kb`, zero beyond k or for rows >= nrows.
// Weight rows are streamed once: non-temporal loads keep them out of the caches.
template <bool kStream>
__device__ __forceinline__ v8i load32(const uint8_t* base, int64_t ld, int64_t row, int64_t nrows, int64_t kb,
                                      int64_t k) {
    v8i v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (row < nrows) {
        const uint8_t* p = base + row * ld + kb;
        if (kb + 16 <= k) {
            const v4u lo = kStream ? __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p))
                                   : *reinterpret_cast<const v4u*>(p);
            v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
        }
        if (kb + 32 <= k) {
            const v4u hi = kStream ? __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p + 16))
                                   : *reinterpret_cast<const v4u*>(p + 16);
            v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
        }
    }
    return v;
}

struct GemvArgs {
    const uint8_t* a; int64_t lda; int m;
    const uint8_t* w; const float* w_scale; const float* a_scale; int64_t n, k;
    uint16_t* out; int64_t ld_out; bool vec_out;   // vec_out: 8-byte aligned rows
    float* partial; unsigned* counters;
    int ksplit, steps_per_split, ksteps;
    ConvEpilogue conv;
};

template <bool kConv>
__global__ __launch_bounds__(256) void gemv_kernel(const GemvArgs g) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rb = blockIdx.x, split = blockIdx.y;
    const int64_t row = (int64_t)rb * kGemvRows + wave * 16 + (lane & 15);   // A operand row
    const int col = lane & 15;                                                // B operand column (token)
    const int s0 = split * g.steps_per_split;
    int ns = g.ksteps - s0;
    if (ns > g.steps_per_split) ns = g.steps_per_split;
    const int64_t kq = (lane >> 4) * 32;

    v8i wa[kGemvMaxSteps], xb[kGemvMaxSteps];
#pragma unroll
    for (int i = 0; i < kGemvMaxSteps; ++i)
        if (i < ns) wa[i] = load32<true>(g.w, g.k, row, g.n, (int64_t)(s0 + i) * 128 + kq, g.k);
#pragma unroll
    for (int i = 0; i < kGemvMaxSteps; ++i)
        if (i < ns) xb[i] = load32<false>(g.a, g.lda, col, g.m, (int64_t)(s0 + i) * 128 + kq, g.k);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kGemvMaxSteps; ++i)
        if (i < ns) acc = mfma_e4m3(wa[i], xb[i], acc);

    // acc[r] = D[feature rbase + r][token col]
    const int64_t nbase = (int64_t)rb * kGemvRows + wave * 16 + 4 * (lane >> 4);
    if (g.ksplit > 1) {
        __shared__ int s_last;
        if (col < g.m) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (nbase + r < g.n) g.partial[((int64_t)split * g.n + nbase + r) * g.m + col] = acc[r];
        }
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0) s_last = atomicAdd(&g.counters[rb], 1u) == (unsigned)(g.ksplit - 1);
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        v4f tot = {0.f, 0.f, 0.f, 0.f};
        for (int sp = 0; sp < g.ksplit; ++sp) {
            if (sp == split) {
                tot += acc;
            } else if (col < g.m) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (nbase + r < g.n)
                        tot[r] += (g.partial[((int64_t)sp * g.n + nbase + r) * g.m + col]);
            }
        }
        acc = tot;
        if (threadIdx.x == 0) g.counters[rb] = 0u;
    }
    if (col >= g.m) return;

    const float sa = *g.a_scale;
    uint32_t hb[4];
    float val[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t nn = nbase + r;
        val[r] = nn < g.n ? acc[r] * sa * g.w_scale[nn] : 0.f;
        hb[r] = f32_to_bf16(val[r]);
    }
    uint16_t* o = g.out + (int64_t)col * g.ld_out + nbase;
    if (g.vec_out && nbase + 3 < g.n) {
        *reinterpret_cast<uint2*>(o) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
    } else {
        for (int r = 0; r < 4; ++r)
            if (nbase + r < g.n) o[r] = (uint16_t)hb[r];
    }

    if constexpr (kConv) {
        // causal depthwise conv (width 4) + SiLU on the xBC features, window shift in place
        const ConvEpilogue& c = g.conv;
        const int64_t ch = nbase - c.xbc_off;
        if (ch < 0 || ch >= c.conv_dim) return;
        const int slot = c.slot_idx[col];
        uint16_t* xo = c.xbc_conv + (int64_t)col * c.conv_dim + ch;
        if (slot < 0) {
            *reinterpret_cast<uint2*>(xo) = make_uint2(0u, 0u);
            return;
        }
        uint16_t* win = c.conv_pool + (int64_t)slot * 3 * c.conv_dim + ch;
        const uint2 w0 = *reinterpret_cast<const uint2*>(win);
        const uint2 w1 = *reinterpret_cast<const uint2*>(win + c.conv_dim);
        const uint2 w2 = *reinterpret_cast<const uint2*>(win + 2 * c.conv_dim);
        const uint4 cw0 = *reinterpret_cast<const uint4*>(c.conv_w + ch * 4);      // channels ch, ch+1
        const uint4 cw1 = *reinterpret_cast<const uint4*>(c.conv_w + ch * 4 + 8);  // channels ch+2, ch+3
        const uint2 cb = *reinterpret_cast<const uint2*>(c.conv_b + ch);
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
                       const ConvEpilogue* conv, void* ws, hipStream_t st) {
    const GemvPlan p = gemv_plan(n, k);
    GemvArgs g;
    g.a = a; g.lda = lda; g.m = m;
    g.w = w; g.w_scale = w_scale; g.a_scale = a_scale; g.n = n; g.k = k;
    g.out = out; g.ld_out = ld_out;
    g.vec_out = ld_out % 4 == 0 && reinterpret_cast<uintptr_t>(out) % 8 == 0;
    g.counters = reinterpret_cast<unsigned*>(ws);
    g.partial = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                         align_up((size_t)p.row_blocks * sizeof(unsigned), 256));
    g.ksplit = p.ksplit; g.steps_per_split = p.steps_per_split; g.ksteps = p.ksteps;
    if (conv) g.conv = *conv; else g.conv = ConvEpilogue{};
    const dim3 grid(p.row_blocks, p.ksplit);
    if (conv)
        gemv_kernel<true><<<grid, dim3(256), 0, st>>>(g);
    else
        gemv_kernel<false><<<grid, dim3(256), 0, st>>>(g);
    return check_launch("gemv");
}

}  // namespace nhm
