// Weight-streaming FP8 W8A8 GEMV for m <= 16 rows (decode).
//
// The problem is HBM-bound: every weight byte is read exactly once and the
// activations (m x k, a few KB) stay on chip. The contraction still runs on the
// 16x16x128 e4m3 MFMA: 16 weight rows are the A operand, the (zero-padded) 16
// activation rows the B operand, so the VALU never converts fp8.
//
// Decomposition: one workgroup owns kRows output features (8, 16 or 32) and the
// whole k range; its waves take the 128-wide k-steps round-robin and issue all
// their weight loads before anything else, so a wave keeps its whole share in
// flight. A bf16 activation is quantized by every workgroup into LDS while those
// loads are in flight (the static per-tensor quant, fused: no separate launch).
// The per-wave partial tiles are summed through LDS in wave order --
// deterministic, and no communication between workgroups (an agent-scope fence
// would write back the L2 of every XCD).
#include "nhm_device.h"
#include "nhm_internal.h"

namespace nhm {

constexpr int kGemvMaxSteps = 8;       // k-steps per wave held in registers
constexpr int kLdsPad = 16;            // bytes of padding per staged activation row

// 32 bytes of row `row` starting at byte `kb`, zero beyond k.
// Weight rows are streamed once: non-temporal loads keep them out of the caches.
template <bool kStream>
__device__ __forceinline__ v8i load32(const uint8_t* p, int64_t kb, int64_t k) {
    v8i v = {0, 0, 0, 0, 0, 0, 0, 0};
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
    return v;
}

struct GemvArgs {
    const void* a; int64_t lda; int m;          // e4m3 [m, lda], or bf16 [m, lda] when quantized here
    const uint8_t* w; const float* w_scale; const float* a_scale; int64_t n, k;
    uint16_t* out; int64_t ld_out; bool vec_out;   // vec_out: 8-byte aligned rows
    int ksteps;
    uint8_t* q_copy;      // kQuantIn: if set, workgroup 0 also stores the e4m3 activation [m, k] here
    ConvEpilogue conv;
};

// Causal depthwise conv (width 4) + SiLU for 4 consecutive xBC channels of one
// token, given their bf16 projection outputs hb; shifts the window in place.
__device__ __forceinline__ void conv_epilogue(const ConvEpilogue& c, int col, int64_t ch, const uint32_t (&hb)[4]) {
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

template <int kRows, int kWaves, bool kQuantIn, bool kConv>
__global__ __launch_bounds__(kWaves * 64) void gemv_kernel(const GemvArgs g) {
    constexpr int kTiles = (kRows + 15) / 16;
    extern __shared__ __attribute__((aligned(16))) uint8_t s_act[];   // [m][k + pad] e4m3 (kQuantIn)
    __shared__ v4f s_red[kWaves][kTiles][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * kRows;
    const int col = lane & 15;                  // B operand column (token)
    const int64_t kq = (lane >> 4) * 32;

    // ---- weight stream: every load of this wave's share goes out first
    v8i wa[kTiles][kGemvMaxSteps];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        const int r16 = t * 16 + (lane & 15);
        const int64_t row = n0 + r16;
        const bool ok = r16 < kRows && row < g.n;
        const uint8_t* wr = g.w + row * g.k + kq;
#pragma unroll
        for (int i = 0; i < kGemvMaxSteps; ++i) {
            const int s = wave + i * kWaves;
            if (s < g.ksteps) wa[t][i] = ok ? load32<true>(wr + (int64_t)s * 128, (int64_t)s * 128 + kq, g.k)
                                            : v8i{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }

    // ---- activation operand
    v8i xb[kGemvMaxSteps];
    const int64_t lds_ld = g.k + kLdsPad;
    if constexpr (kQuantIn) {
        const uint16_t* a = static_cast<const uint16_t*>(g.a);
        const float s = *g.a_scale;
        const int64_t per_row = g.k / 8;
        for (int64_t e = threadIdx.x; e < g.m * per_row; e += kWaves * 64) {
            const int64_t r = e / per_row, c8 = e - r * per_row;
            const uint4 in = *reinterpret_cast<const uint4*>(a + r * g.lda + c8 * 8);
            const uint32_t w4[4] = {in.x, in.y, in.z, in.w};
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                lo |= quant_bf16(w4[j] & 0xffffu, s) << (16 * j);
                lo |= quant_bf16(w4[j] >> 16, s) << (16 * j + 8);
                hi |= quant_bf16(w4[j + 2] & 0xffffu, s) << (16 * j);
                hi |= quant_bf16(w4[j + 2] >> 16, s) << (16 * j + 8);
            }
            *reinterpret_cast<uint2*>(s_act + r * lds_ld + c8 * 8) = make_uint2(lo, hi);
            if (g.q_copy && blockIdx.x == 0) *reinterpret_cast<uint2*>(g.q_copy + r * g.k + c8 * 8) = make_uint2(lo, hi);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kGemvMaxSteps; ++i) {
            const int s = wave + i * kWaves;
            if (s < g.ksteps) {
                const int64_t kb = (int64_t)s * 128 + kq;
                xb[i] = col < g.m ? load32<false>(s_act + col * lds_ld + kb, kb, g.k) : v8i{0, 0, 0, 0, 0, 0, 0, 0};
            }
        }
    } else {
        const uint8_t* ar = static_cast<const uint8_t*>(g.a) + (int64_t)col * g.lda + kq;
#pragma unroll
        for (int i = 0; i < kGemvMaxSteps; ++i) {
            const int s = wave + i * kWaves;
            if (s < g.ksteps)
                xb[i] = col < g.m ? load32<false>(ar + (int64_t)s * 128, (int64_t)s * 128 + kq, g.k)
                                  : v8i{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }

    v4f acc[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kGemvMaxSteps; ++i)
            if (wave + i * kWaves < g.ksteps) acc[t] = mfma_e4m3(wa[t][i], xb[i], acc[t]);
    }

    // ---- sum the waves' partial tiles in wave order; wave t finishes tile t
#pragma unroll
    for (int t = 0; t < kTiles; ++t) s_red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave >= kTiles) return;
    const int t = wave;
    v4f tot = s_red[0][t][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) tot += s_red[w][t][lane];

    // tot[r] = D[feature nbase + r][token col]
    if (col >= g.m) return;
    const int64_t nbase = n0 + t * 16 + 4 * (lane >> 4);
    if (4 * (lane >> 4) + t * 16 >= kRows) return;
    const float sa = *g.a_scale;
    uint32_t hb[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t nn = nbase + r;
        hb[r] = f32_to_bf16(nn < g.n ? tot[r] * sa * g.w_scale[nn] : 0.f);
    }
    uint16_t* o = g.out + (int64_t)col * g.ld_out + nbase;
    if (g.vec_out && nbase + 3 < g.n) {
        *reinterpret_cast<uint2*>(o) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
    } else {
        for (int r = 0; r < 4; ++r)
            if (nbase + r < g.n) o[r] = (uint16_t)hb[r];
    }
    if constexpr (kConv) {
        const int64_t ch = nbase - g.conv.xbc_off;
        if (ch >= 0 && ch < g.conv.conv_dim) conv_epilogue(g.conv, col, ch, hb);
    }
}

template <int kRows, int kWaves, bool kQuantIn>
static void launch_rows(const GemvArgs& g, bool conv, hipStream_t st) {
    const dim3 grid((unsigned)((g.n + kRows - 1) / kRows));
    const size_t lds = kQuantIn ? (size_t)g.m * (size_t)(g.k + kLdsPad) : 0;
    if (conv) gemv_kernel<kRows, kWaves, kQuantIn, true><<<grid, dim3(kWaves * 64), lds, st>>>(g);
    else gemv_kernel<kRows, kWaves, kQuantIn, false><<<grid, dim3(kWaves * 64), lds, st>>>(g);
}

template <bool kQuantIn>
static void launch_sel(const GemvArgs& g, int rows, int waves, bool conv, hipStream_t st) {
    if (rows == 32) {
        if (waves == 4) launch_rows<32, 4, kQuantIn>(g, conv, st);
        else if (waves == 8) launch_rows<32, 8, kQuantIn>(g, conv, st);
        else launch_rows<32, 16, kQuantIn>(g, conv, st);
    } else if (rows == 16) {
        if (waves == 4) launch_rows<16, 4, kQuantIn>(g, conv, st);
        else if (waves == 8) launch_rows<16, 8, kQuantIn>(g, conv, st);
        else launch_rows<16, 16, kQuantIn>(g, conv, st);
    } else {
        if (waves == 4) launch_rows<8, 4, kQuantIn>(g, conv, st);
        else if (waves == 8) launch_rows<8, 8, kQuantIn>(g, conv, st);
        else launch_rows<8, 16, kQuantIn>(g, conv, st);
    }
}

bool gemv_supports(int64_t m, int64_t k, bool bf16_in) {
    if (m < 1 || m > 16 || k > 16 * 128 * kGemvMaxSteps) return false;
    return !bf16_in || (size_t)m * (size_t)(k + kLdsPad) <= 64 * 1024;
}

nhm_status launch_gemv(const void* a, bool bf16_in, int64_t lda, int m, const uint8_t* w, const float* w_scale,
                       const float* a_scale, int64_t n, int64_t k, uint16_t* out, int64_t ld_out,
                       const ConvEpilogue* conv, uint8_t* q_copy, hipStream_t st) {
    if (!gemv_supports(m, k, bf16_in)) return fail(NHM_ERR_UNSUPPORTED, "gemv: m %d, k %lld", m, (long long)k);
    GemvArgs g;
    g.a = a; g.lda = lda; g.m = m;
    g.w = w; g.w_scale = w_scale; g.a_scale = a_scale; g.n = n; g.k = k;
    g.out = out; g.ld_out = ld_out;
    g.vec_out = ld_out % 4 == 0 && reinterpret_cast<uintptr_t>(out) % 8 == 0;
    g.ksteps = (int)((k + 127) / 128);
    g.conv = conv ? *conv : ConvEpilogue{};
    g.q_copy = q_copy;
    // waves: enough that each holds at most kGemvMaxSteps k-steps
    const int waves = g.ksteps <= 4 * kGemvMaxSteps ? 4 : (g.ksteps <= 8 * kGemvMaxSteps ? 8 : 16);
    // rows per workgroup: large tiles amortize the activation staging, but keep >= ~300 workgroups
    const int rows = n >= 32 * 300 ? 32 : (n >= 16 * 300 ? 16 : 8);
    if (bf16_in) launch_sel<true>(g, rows, waves, conv != nullptr, st);
    else launch_sel<false>(g, rows, waves, conv != nullptr, st);
    return check_launch("gemv");
}

}  // namespace nhm
