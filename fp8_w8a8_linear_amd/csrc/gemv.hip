// Weight-streaming FP8 W8A8 GEMV for m <= 16 rows (decode).
//
// The problem is HBM-bound: every weight byte is read exactly once and the
// activations (m x k e4m3, a few KB) stay in L2/L1. The contraction runs on the MFMA
// with 16 weight rows as the A operand and the (zero-padded) 16 activation rows as
// the B operand; the e4m3 codes are converted to bf16 in registers (exact) and summed
// by the bf16 MFMA, which accumulates in full f32.
//
// Weight loads. In the 8-wave configuration (one row tile per workgroup, 2944 <= k <= 8192:
// out_proj among them), each load instruction brings whole 128-byte lines -- 8 weight rows x 128
// bytes of one k-step -- and every k-step passes through a per-wave LDS buffer to reach the
// MFMA's operand layout (row = lane % 16). Otherwise (in_proj's three tiles; the 16-wave
// configurations, whose 128-register budget the buffer's traffic would overflow) each
// instruction brings 16 rows x 64 bytes straight into the operand registers. Measured on MI355X at m = 8:
// out_proj 2688 x 4096 5.26 -> 4.58 us with whole lines; in_proj 10304 x 2688 8.48 us straight,
// 9.1-9.4 us with whole lines and the transpose (its extra LDS round trips per step do not
// hide behind one wave per SIMD), both bit-identical.
//
// Decomposition: one workgroup owns up to 48 output features (one to three 16-row MFMA
// tiles, as many as keep the busiest CU's operand bytes lowest) and the whole k range; its
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
    // non-null (bf16 output only): also the e4m3 codes of the bf16 output, E4M3(out / *q_scale),
    // at out_q[m * ld_q + n] -- the next projection's pre-quantized input
    uint8_t* out_q; int64_t ld_q; const float* q_scale; bool vec_q;
    int ksteps;
    uint32_t* clear; int clear_n;                   // words zeroed by workgroup 0 (side work)
    int ws_step;                                    // weight scale index step: 1 per channel, 0 per tensor
    // workgroup b owns features [b base + min(b, extra), ...) -- base + 1 of them for b < extra,
    // base for the others (at most 16 x kTiles)
    int base, extra;
};

// Cache policy of the weight stream: the default. The non-temporal hint (nt) made the in_proj
// GEMV at m = 8 slower, 9.24 against 8.37 us per launch (sc0 alone 8.39, sc1 9.76, nt with
// either 9.23), although each weight row is read once per call.
constexpr int kStreamAux = 0;

template <int kWaves, int kSteps, int kTiles, bool kLines>
__global__ __launch_bounds__(kWaves * 64) void gemv_kernel(const GemvArgs g) {
    __shared__ v4f s_red[kWaves][kTiles][64];   // every wave's partial of every row tile
    // kLines: this wave's transpose buffer, one k-step of the 16 kTiles rows
    __shared__ __attribute__((aligned(16))) uint8_t s_tr[kLines ? kWaves : 1][kLines ? 16 * kTiles * 128 : 16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int b = blockIdx.x;
    if (b == 0 && g.clear) {
        for (int i = threadIdx.x; i < g.clear_n; i += kWaves * 64) g.clear[i] = 0u;
    }
    const int64_t n0 = (int64_t)b * g.base + (b < g.extra ? b : g.extra);
    const int64_t nend = n0 + g.base + (b < g.extra ? 1 : 0);   // this workgroup's features end
    const int col = lane & 15;                  // B operand column (token)
    const int kq = (lane >> 4) * 32;
    // MFMA row tile t covers features n0 + 16 t .. + 15 (A operand row lane % 16; rows at or
    // past nend load zeros); its result lane holds features n0 + 16 t + 4 (lane / 16) .. + 3 of
    // token col. Wave t < kTiles finishes row tile t: its result lane's features start at nb.
    const int64_t nb = n0 + 16 * (wave < kTiles ? wave : 0) + 4 * (lane >> 4);

    // Everything up to the MFMAs is straight-line code: loads past the operands go to an
    // out-of-range buffer offset (zeros) and indexes are clamped, so the compiler can wait
    // for each k-step's loads alone instead of for all outstanding loads at a branch join.
    // First the scales of the epilogue (so that waiting for them later does not wait for the
    // weight stream), then the weight stream, k-step by k-step.
    const float sa = *g.a_scale;
    const float sq = g.out_q ? *g.q_scale : 1.0f;
    // the weight scales of this wave's row tile, one 16-byte load with no branch around it: per
    // channel, this lane's four consecutive features (zeros past n); per tensor, the one scale in
    // the first word of a one-word range. They are applied in the epilogue; using them here (the
    // product with sa under a branch) made the wave wait for this load before its weight stream.
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.w_scale, (short)0, g.ws_step != 0 ? (int)(g.n * 4) : 4, 0x00020000);
    const v4u sraw = __builtin_amdgcn_raw_buffer_load_b128(srs, g.ws_step != 0 ? (uint32_t)(nb * 4) : 0u, 0, 0);

    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc((void*)g.w, (short)0, (int)(g.n * g.k), 0x00020000);
    const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc((void*)g.a, (short)0, (int)(g.m * g.lda), 0x00020000);
    uint32_t wrow[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        const int64_t row = n0 + 16 * t + (lane & 15);
        wrow[t] = row < nend ? (uint32_t)(row * g.k) : kGemvOut;
    }
    const uint32_t arow = col < g.m ? (uint32_t)(col * g.lda) : kGemvOut;
    // kLines: unit u of a tile's k-step is rows 8u .. 8u + 7 of the tile, lane l on row 8u + l / 8,
    // loading the 16-byte chunk that swz128 places at slot l % 8 of that row
    const int lr = lane >> 3, slot = lane & 7;
    uint32_t urow[2 * kTiles];
    int uch[2 * kTiles];
    if constexpr (kLines) {
#pragma unroll
        for (int u = 0; u < 2 * kTiles; ++u) {
            const int r8 = 8 * u + lr;
            urow[u] = n0 + r8 < nend ? (uint32_t)((n0 + r8) * g.k) : kGemvOut;
            uch[u] = 16 * (slot ^ (r8 & 7) ^ ((r8 >> 3) & 1));
        }
    }
    // weight and activation pieces of each k-step are issued together
    v8i wa[kSteps][kTiles], xb[kSteps];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        const int kb = (wave + i * kWaves) * 128 + kq;
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
            if constexpr (kLines) {
                const int k0 = kb - kq + uch[2 * t], k1 = kb - kq + uch[2 * t + 1];
                wa[i][t] = bload32<kStreamAux>(wrs, k0 < g.k ? urow[2 * t] + k0 : kGemvOut,
                                               k1 < g.k ? urow[2 * t + 1] + k1 : kGemvOut);
            } else {
                wa[i][t] = bload32<kStreamAux>(wrs, kb < g.k ? wrow[t] + kb : kGemvOut,
                                               kb + 16 < g.k ? wrow[t] + kb + 16 : kGemvOut);
            }
        }
        xb[i] = bload32<0>(ars, kb < g.k ? arow + kb : kGemvOut, kb + 16 < g.k ? arow + kb + 16 : kGemvOut);
    }
    // keep every load above issued before the first MFMA (the scheduler would otherwise sink
    // later steps' loads below earlier steps' MFMAs, serialising the stream)
    __builtin_amdgcn_sched_barrier(0);

    // Exact f32 accumulation: each 128-k step runs as four bf16 MFMAs per row tile on the
    // converted codes (sub-step j takes bytes 8j .. 8j+7 of the lane's 32, the same bytes of
    // both operands; the activation piece is converted once for all row tiles). The e4m3 MFMA
    // would be 4x fewer instructions but sums coarser than f32; this kernel is bound by the
    // weight stream, and the conversions and MFMAs of a step run while later steps are still
    // streaming in. Steps past k hold zeros and add nothing.
    v4f acc[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        if constexpr (kLines) {   // step i's rows, written as loaded, read back in operand layout
            uint8_t* const tb = s_tr[wave];
#pragma unroll
            for (int t = 0; t < kTiles; ++t) {
                *reinterpret_cast<uint4*>(tb + (16 * t + lr) * 128 + slot * 16) =
                    make_uint4(wa[i][t][0], wa[i][t][1], wa[i][t][2], wa[i][t][3]);
                *reinterpret_cast<uint4*>(tb + (16 * t + 8 + lr) * 128 + slot * 16) =
                    make_uint4(wa[i][t][4], wa[i][t][5], wa[i][t][6], wa[i][t][7]);
            }
#pragma unroll
            for (int t = 0; t < kTiles; ++t) {
                const uint4 w0 = *reinterpret_cast<const uint4*>(tb + swz128(16 * t + col, 2 * (lane >> 4)));
                const uint4 w1 = *reinterpret_cast<const uint4*>(tb + swz128(16 * t + col, 2 * (lane >> 4) + 1));
                wa[i][t] = v8i{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8 xs = e4m3x8_to_bf16(xb[i][2 * j], xb[i][2 * j + 1]);
#pragma unroll
            for (int t = 0; t < kTiles; ++t)
                acc[t] = mfma_bf16(e4m3x8_to_bf16(wa[i][t][2 * j], wa[i][t][2 * j + 1]), xs, acc[t]);
        }
    }

    // The partial tiles go through LDS; wave t sums row tile t over the waves in wave order
    // (deterministic) and stores it, so the row tiles' epilogues run side by side.
#pragma unroll
    for (int t = 0; t < kTiles; ++t) s_red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave >= kTiles) return;
    v4f d = s_red[0][wave][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) d += s_red[w][wave][lane];

    // d[r] = D[feature nb + r][token col]
    if (col >= g.m || nb >= nend) return;
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = sa * __uint_as_float(g.ws_step != 0 ? sraw[r] : sraw[0]);
    {
        if (g.out_f32) {
            float* of = g.out_f32 + (int64_t)col * g.ld_out + nb;
            if (g.vec_out && (nb & 3) == 0 && nb + 3 < nend) {
                *reinterpret_cast<float4*>(of) = make_float4(d[0] * sc[0], d[1] * sc[1], d[2] * sc[2], d[3] * sc[3]);
            } else {
                for (int r = 0; r < 4; ++r)
                    if (nb + r < nend) of[r] = d[r] * sc[r];
            }
            return;
        }
        uint32_t hb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) hb[r] = f32_to_bf16(d[r] * sc[r]);
        uint16_t* o = g.out + (int64_t)col * g.ld_out + nb;
        if (g.vec_out && (nb & 3) == 0 && nb + 3 < nend) {
            *reinterpret_cast<uint2*>(o) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
        } else {
            for (int r = 0; r < 4; ++r)
                if (nb + r < nend) o[r] = (uint16_t)hb[r];
        }
        if (g.out_q) {   // the static quant of the bf16 values just stored (IEEE quotient)
            const uint32_t c4 = quant_bf16x4(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), sq);
            uint8_t* oq = g.out_q + (int64_t)col * g.ld_q + nb;
            if (g.vec_q && (nb & 3) == 0 && nb + 3 < nend) {
                *reinterpret_cast<uint32_t*>(oq) = c4;
            } else {
                for (int r = 0; r < 4; ++r)
                    if (nb + r < nend) oq[r] = (uint8_t)(c4 >> (8 * r));
            }
        }
    }
}

nhm_status launch_gemv(const uint8_t* a, int64_t lda, int m, const uint8_t* w, const float* w_scale,
                       const float* a_scale, int64_t n, int64_t k, uint16_t* out, int64_t ld_out, hipStream_t st,
                       float* out_f32, uint8_t* out_q, int64_t ld_q, const float* q_scale, uint32_t* clear,
                       int clear_n, int ws_step) {
    GemvArgs g;
    g.ws_step = ws_step;
    g.clear = clear_n > 0 ? clear : nullptr;
    g.clear_n = clear_n;
    g.out_q = out_f32 ? nullptr : out_q;
    g.ld_q = ld_q;
    g.q_scale = q_scale;
    g.vec_q = ld_q % 4 == 0 && reinterpret_cast<uintptr_t>(out_q) % 4 == 0;
    g.a = a; g.lda = lda; g.m = m;
    g.w = w; g.w_scale = w_scale; g.a_scale = a_scale; g.n = n; g.k = k;
    g.out = out; g.ld_out = ld_out;
    g.out_f32 = out_f32;
    g.vec_out = out_f32 ? ld_out % 4 == 0 && reinterpret_cast<uintptr_t>(out_f32) % 16 == 0
                        : ld_out % 4 == 0 && reinterpret_cast<uintptr_t>(out) % 8 == 0;
    g.ksteps = (int)((k + 127) / 128);
    if (g.ksteps > 16 * kGemvMaxSteps)
        return fail(NHM_ERR_UNSUPPORTED, "gemv: k %lld exceeds %d", (long long)k, 16 * 128 * kGemvMaxSteps);
    if (n * k >= (int64_t(1) << 31) || (int64_t)m * lda >= (int64_t(1) << 31))
        return fail(NHM_ERR_UNSUPPORTED, "gemv: operands of 2 GiB or more");
    // 4 waves up to 23 k-steps (k < 2944), then 8, then 16; each wave holds its steps in
    // registers, their count rounded up to 2, 4, 6 or 8
    const int waves = g.ksteps < 24 ? 4 : (g.ksteps <= 8 * kGemvMaxSteps ? 8 : 16);
    const int per = (g.ksteps + waves - 1) / waves;
    const int steps = per <= 2 ? 2 : per <= 4 ? 4 : per <= 6 ? 6 : 8;
    // Features per workgroup: up to 16 per MFMA row tile, 3 tiles (48) where each wave holds
    // few enough k-steps (4 waves), else 1. Each CU streams its share at a rate bounded by the
    // requests it keeps in flight, so the split minimises the operand bytes the busiest CU pulls,
    // (features + tokens) x k -- every workgroup reads its weight rows and the whole activation:
    // the features are dealt evenly over one workgroup per CU (256; in_proj at m = 8: 40-41
    // features each, against 44 on 235 CUs with whole multiples of 4), or over as many as the
    // tile limit needs, and never fewer than 4 per workgroup. The spare MFMA rows of a tile load
    // zeros; features that do not start a 4-aligned run are stored one at a time.
    const int max_rows = waves == 4 ? 48 : 16;
    int64_t wgs = (n + 3) / 4 < 256 ? (n + 3) / 4 : 256;
    if ((n + wgs - 1) / wgs > max_rows) wgs = (n + max_rows - 1) / max_rows;
    g.base = (int)(n / wgs);
    g.extra = (int)(n % wgs);
    const int tiles = (g.base + (g.extra ? 1 : 0) + 15) / 16;
    const dim3 grid((unsigned)wgs);
#define NHM_GEMV_LAUNCH(W, S, T) gemv_kernel<W, S, T, (W == 8)><<<grid, dim3(W * 64), 0, st>>>(g)
#define NHM_GEMV_STEPS(W, T)                         \
    do {                                             \
        if (steps == 2) NHM_GEMV_LAUNCH(W, 2, T);    \
        else if (steps == 4) NHM_GEMV_LAUNCH(W, 4, T); \
        else if (steps == 6) NHM_GEMV_LAUNCH(W, 6, T); \
        else NHM_GEMV_LAUNCH(W, 8, T);               \
    } while (0)
    if (waves == 4) {
        if (tiles == 1) NHM_GEMV_STEPS(4, 1);
        else if (tiles == 2) NHM_GEMV_STEPS(4, 2);
        else NHM_GEMV_STEPS(4, 3);
    } else if (waves == 8) {
        NHM_GEMV_STEPS(8, 1);
    } else {
        NHM_GEMV_STEPS(16, 1);
    }
#undef NHM_GEMV_STEPS
#undef NHM_GEMV_LAUNCH
    count_launch(Kern::kGemv, m);
    return check_launch("gemv");
}

}  // namespace nhm
