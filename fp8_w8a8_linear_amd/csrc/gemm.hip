// FP8 W8A8 GEMM on the gfx950 e4m3 MFMA (prefill-sized m).
//
// out[i, j] = bf16( (sum_k a[i, k] * w[j, k]) * a_scale * w_scale[j] ), f32 accumulate.
// Both operands are k-contiguous ([m, k] activations, [n, k] weights in the
// [out, in] orientation). In the MFMA 16x16x128 a lane supplies row (lane % 16) of
// each operand and 32 bytes of the 128-deep k-step; any assignment of k to lanes
// works as long as both operands use the same one.
//
// Three kernels:
//  * panel kernel (m up to 640 where the ring tiles are too few to fill the chip; 64 x 128
//    tiles, or narrower weight panels where those fill the chip better): a workgroup owns a
//    panel of up to BN weight rows and a BM-row tile of the activations. Each of its 4 waves streams
//    its own WN weight rows straight from memory into MFMA registers, two or four k-steps
//    ahead; only the activation tile, which all 4 waves share, is staged in LDS
//    (three buffers: the operands of step k+1 are read while the MFMAs of step k
//    run, one barrier per step). Workgroups that share a weight panel are placed on
//    one XCD so the panel is fetched into that XCD's L2 once. Loads go through
//    buffer descriptors, whose range check returns zeros past the operand's end,
//    so ragged edges and padded steps need no branches in the loop.
//  * ring tile kernels, 256 x 256 or 256 x 128 with 64-byte k-slices and 192 x 128 with
//    128-byte ones (enough tiles to fill the chip): both operand tiles stream into an LDS ring
//    of k-slices (4 to 6 stages, as many as fit 160 KB) by direct-to-LDS buffer loads (no register round trip; the range check
//    zero-fills ragged rows and k), eight waves on the 32x32x64 MFMA read the operands of
//    the next stage while the MFMAs of the current one run, and the bf16 result leaves
//    through LDS so that every store writes whole output rows. Each CU receives operands
//    at a rate bounded by the requests it keeps in flight, so the operand bytes a CU must
//    pull set the time: wide tiles (fewer bytes per MAC) at large m, and at m <= 640 the
//    tile shape whose busiest CU pulls the fewest bytes; and whole 128-byte line requests
//    carry twice the bytes of 64-byte ones per request in flight, where the LDS has room for
//    128-byte slices.
//  * 128 x 128 tile kernel (remaining shapes): both operands staged through
//    double-buffered LDS, four waves of 64 x 64.
#include <stdint.h>

#include "nhm_device.h"
#include "nhm_internal.h"

namespace nhm {

struct GemmArgs {
    const uint8_t* a; int64_t lda; int64_t m;
    const uint8_t* w; const float* w_scale; const float* a_scale; int64_t n, k;
    uint16_t* out; int64_t ld_out; bool vec_out;   // vec_out: rows aligned for 4-element stores
    float* out_f32;                                 // non-null: f32 output [m, ld_out] instead of out
    // split k (ring tile kernel): blocks [s * tiles, (s + 1) * tiles) sum the s-th of ksplit
    // contiguous k ranges into part [ksplit, m, n] (raw f32 sums), which splitk_reduce_kernel
    // adds up in split order, scales and rounds
    int ksplit = 1;
    float* part = nullptr;
    int ws_step = 1;    // weight scale index step: 1 per channel, 0 per tensor
    int panel_rows = 0; // panel kernel: weight rows per panel (0: all of its waves' rows)
};

// Row r of a 128-byte-wide LDS tile holds its 16-byte chunk c at slot c ^ (r & 7):
// the 16 lanes that read one chunk column of 16 consecutive rows hit all banks.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ v8i cat8(const uint4& lo, const uint4& hi) {
    v8i v;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    return v;
}

// Stores one 16 x 16 MFMA result tile (lane: 4 consecutive n of one m row), scaled.
// full: the whole wave tile is inside [m, n] and rows are 8-byte aligned (wave-uniform).
__device__ __forceinline__ void store_tile(uint16_t* out, int64_t ld_out, int64_t mm, int64_t nb, int64_t m, int64_t n,
                                           const v4f& acc, const float (&sc)[4], bool full) {
    uint32_t hb[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) hb[r] = f32_to_bf16(acc[r] * sc[r]);
    if (full) {
        *reinterpret_cast<uint2*>(out + mm * ld_out + nb) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
    } else if (mm < m) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (nb + r < n) out[mm * ld_out + nb + r] = (uint16_t)hb[r];
    }
}

// The same tile as f32 (acc * scale, no rounding); full: 16-byte aligned rows.
__device__ __forceinline__ void store_tile_f32(float* out, int64_t ld_out, int64_t mm, int64_t nb, int64_t m, int64_t n,
                                               const v4f& acc, const float (&sc)[4], bool full) {
    const float4 v = make_float4(acc[0] * sc[0], acc[1] * sc[1], acc[2] * sc[2], acc[3] * sc[3]);
    if (full) {
        *reinterpret_cast<float4*>(out + mm * ld_out + nb) = v;
    } else if (mm < m) {
        const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (nb + r < n) out[mm * ld_out + nb + r] = e[r];
    }
}

// One 128-deep k-step of a 16 x 16 tile. kExact == false: the e4m3 MFMA, whose 128-product
// reductions are coarser than f32. kExact: every product summed in f32 -- the lane's 32 code
// bytes of each operand are split into four runs of eight (the same bytes of both operands
// per run, so the four runs cover each product once), converted to bf16 (exact for every
// e4m3 value) and summed by four bf16 MFMAs.
template <bool kExact>
__device__ __forceinline__ v4f mfma16_step(const v8i& a, const v8i& b, const v4f& c) {
    if constexpr (!kExact) {
        return mfma_e4m3(a, b, c);
    } else {
        v4f r = c;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            r = mfma_bf16(e4m3x8_to_bf16(a[2 * j], a[2 * j + 1]), e4m3x8_to_bf16(b[2 * j], b[2 * j + 1]), r);
        return r;
    }
}

// ---------------------------------------------------------------- panel kernel

__device__ __forceinline__ uint4 bload(const __amdgpu_buffer_rsrc_t& r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
constexpr uint32_t kOutOfRange = 0x80000000u;   // past every buffer range used here (< 2^31 bytes)

// D: weight k-steps in flight per wave (and activation tiles in registers).
template <int BM, int WN, bool kExact, int D>
__global__ __launch_bounds__(256) void panel_kernel(const GemmArgs g) {
    constexpr int BN = 4 * WN, TN = WN / 16, TM = BM / 16;
    constexpr int U = D % 2 == 0 ? D : 2 * D;   // loop unroll: step kt's registers are slot kt % D
    constexpr int LA = BM * 8 / 256;   // 16-byte chunks of the activation tile per thread
    static_assert(WN % 16 == 0 && BM % 32 == 0, "tile shape");
    __shared__ __attribute__((aligned(16))) uint8_t sA[3][BM * 128];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, q = lane >> 4, r16 = lane & 15;
    // Tile order: blocks are dealt to the 8 XCDs round robin (block b runs on XCD b % 8),
    // so consecutive blocks of one XCD walk the m-tiles of one weight panel.
    // A panel holds PW <= BN weight rows; the waves' rows past its end load nothing (out of
    // range) and store nothing.
    const int PW = g.panel_rows > 0 ? g.panel_rows : BN;
    const int npan = (int)((g.n + PW - 1) / PW), nmt = (int)((g.m + BM - 1) / BM);
    const int loc = blockIdx.x >> 3;
    const int pan = (loc / nmt) * 8 + (blockIdx.x & 7), mt = loc % nmt;
    if (pan >= npan) return;
    const int64_t pend = min((int64_t)(pan + 1) * PW, g.n);
    const int64_t m0 = (int64_t)mt * BM, nw0 = (int64_t)pan * PW + wave * WN;
    const int nk = (int)((g.k + 127) / 128);
    const int ns = (nk + U - 1) / U * U;   // steps, padded to the unroll (padding steps read zeros)

    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc((void*)g.w, (short)0, (int)(g.n * g.k), 0x00020000);
    const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc((void*)g.a, (short)0, (int)(g.m * g.lda), 0x00020000);
    // this lane's k bytes of a step: [16 q, 16 q + 16) and [64 + 16 q, 80 + 16 q)
    uint32_t woff[TN];
    float wsc[TN][4];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        const int64_t row = nw0 + i * 16 + r16;
        woff[i] = row < pend ? (uint32_t)(row * g.k + 16 * q) : kOutOfRange;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t c = nw0 + i * 16 + 4 * q + r;
            wsc[i][r] = g.w_scale[(c < g.n ? c : g.n - 1) * g.ws_step];
        }
    }
    uint32_t aoff[LA];
#pragma unroll
    for (int p = 0; p < LA; ++p) {
        const int row = (t + p * 256) >> 3, c = t & 7;
        aoff[p] = m0 + row < g.m ? (uint32_t)((m0 + row) * g.lda + 16 * c) : kOutOfRange;
    }
    auto wload = [&](int s, uint4 (&dst)[TN][2]) {
        const int64_t kb = (int64_t)s * 128 + 16 * q;
#pragma unroll
        for (int i = 0; i < TN; ++i) {
            dst[i][0] = bload(wrs, kb < g.k ? woff[i] + (uint32_t)s * 128 : kOutOfRange);
            dst[i][1] = bload(wrs, kb + 64 < g.k ? woff[i] + (uint32_t)s * 128 + 64 : kOutOfRange);
        }
    };
    auto aload = [&](int s, uint4 (&dst)[LA]) {
        const int64_t kb = (int64_t)s * 128 + 16 * (t & 7);
#pragma unroll
        for (int p = 0; p < LA; ++p) dst[p] = bload(ars, kb < g.k ? aoff[p] + (uint32_t)s * 128 : kOutOfRange);
    };
    auto astore = [&](int b, const uint4 (&src)[LA]) {
#pragma unroll
        for (int p = 0; p < LA; ++p) *reinterpret_cast<uint4*>(&sA[b][swz((t + p * 256) >> 3, t & 7)]) = src[p];
    };
    auto opread = [&](int b, v8i (&dst)[TM]) {
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int row = j * 16 + r16;
            dst[j] = cat8(*reinterpret_cast<const uint4*>(&sA[b][swz(row, q)]),
                          *reinterpret_cast<const uint4*>(&sA[b][swz(row, q + 4)]));
        }
    };

    v4f acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // Prologue: activation tiles 0 and 1 into LDS buffers 0 and 1, their successors 2 .. D+1
    // and the weight steps 0 .. D-1 in registers, the operands of step 0 read.
    uint4 wr[D][TN][2];
    uint4 ar[D][LA];
    v8i bop[2][TM];
    {
        uint4 t0[LA], t1[LA];
        aload(0, t0);
        aload(1, t1);
#pragma unroll
        for (int s = 0; s < D; ++s) wload(s, wr[s]);
#pragma unroll
        for (int s = 2; s < D + 2; ++s) aload(s, ar[s % D]);
        astore(0, t0);
        astore(1, t1);
        __syncthreads();
        opread(0, bop[0]);
    }
    // Step kt: operands of kt in bop[kt & 1]; LDS buffer b1 holds tile kt+1, b2 receives kt+2
    // (its previous tile, kt-1, was read two steps ago, before the last barrier).
    int b1 = 1, b2 = 2;
    for (int kt0 = 0; kt0 < ns; kt0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kt = kt0 + u;
            opread(b1, bop[(u + 1) & 1]);
#pragma unroll
            for (int j = 0; j < TM; ++j)
#pragma unroll
                for (int i = 0; i < TN; ++i)
                    acc[i][j] = mfma16_step<kExact>(cat8(wr[u % D][i][0], wr[u % D][i][1]), bop[u & 1][j], acc[i][j]);
            wload(kt + D, wr[u % D]);
            astore(b2, ar[(u + 2) % D]);
            aload(kt + 2 + D, ar[(u + 2) % D]);
            __syncthreads();
            const int b0 = 3 - b1 - b2;
            b1 = b2;
            b2 = b0;
        }
    }

    const float sa = *g.a_scale;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        const bool full = g.vec_out && m0 + BM <= g.m && nw0 + 16 * (i + 1) <= pend;
        float sc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = sa * wsc[i][r];
#pragma unroll
        for (int j = 0; j < TM; ++j)
            if (g.out_f32)
                store_tile_f32(g.out_f32, g.ld_out, m0 + j * 16 + r16, nw0 + i * 16 + 4 * q, g.m, pend, acc[i][j], sc, full);
            else
                store_tile(g.out, g.ld_out, m0 + j * 16 + r16, nw0 + i * 16 + 4 * q, g.m, pend, acc[i][j], sc, full);
    }
}

// ---------------------------------------------------------------- tile kernel

constexpr int kTile = 128;   // n, m and k extent of a workgroup tile

// Loads this thread's four 16-byte chunks of a 128 x 128 operand tile through a buffer
// descriptor (operands under 2 GiB): its range check zero-fills rows and k past the end,
// so there are no branches around the loads.
__device__ __forceinline__ void load_tile(uint4 (&r)[4], const __amdgpu_buffer_rsrc_t& rs, int64_t ld, int64_t row0,
                                          int64_t nrows, int64_t k0, int64_t k) {
    const int t = threadIdx.x;
    const int64_t kb = k0 + (t & 7) * 16;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int64_t row = row0 + p * 32 + (t >> 3);
        r[p] = bload(rs, row < nrows && kb < k ? (uint32_t)(row * ld + kb) : kOutOfRange);
    }
}

__device__ __forceinline__ void stage_tile(uint8_t* s, const uint4 (&r)[4]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int p = 0; p < 4; ++p) *reinterpret_cast<uint4*>(s + swz(p * 32 + (t >> 3), t & 7)) = r[p];
}

__device__ __forceinline__ v8i lds_operand(const uint8_t* s, int row, int q) {
    return cat8(*reinterpret_cast<const uint4*>(s + swz(row, 2 * q)), *reinterpret_cast<const uint4*>(s + swz(row, 2 * q + 1)));
}

template <bool kExact>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs g) {
    __shared__ __attribute__((aligned(16))) uint8_t sW[2][kTile * kTile];
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][kTile * kTile];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wn = wave >> 1, wm = wave & 1;
    const int q = lane >> 4, r16 = lane & 15;
    const int64_t n0 = (int64_t)blockIdx.x * kTile, m0 = (int64_t)blockIdx.y * kTile;
    const int nk = (int)((g.k + kTile - 1) / kTile);

    float wsc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t c = n0 + wn * 64 + i * 16 + 4 * q + r;
            wsc[i][r] = g.w_scale[(c < g.n ? c : g.n - 1) * g.ws_step];
        }

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc((void*)g.w, (short)0, (int)(g.n * g.k), 0x00020000);
    const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc((void*)g.a, (short)0, (int)(g.m * g.lda), 0x00020000);
    uint4 rw[4], ra[4];
    load_tile(rw, wrs, g.k, n0, g.n, 0, g.k);
    load_tile(ra, ars, g.lda, m0, g.m, 0, g.k);
    stage_tile(sW[0], rw);
    stage_tile(sA[0], ra);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            load_tile(rw, wrs, g.k, n0, g.n, (int64_t)(kt + 1) * kTile, g.k);
            load_tile(ra, ars, g.lda, m0, g.m, (int64_t)(kt + 1) * kTile, g.k);
        }
        v8i av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = lds_operand(sW[cur], wn * 64 + i * 16 + r16, q);
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = lds_operand(sA[cur], wm * 64 + j * 16 + r16, q);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16_step<kExact>(av[i], bv[j], acc[i][j]);
        if (kt + 1 < nk) {
            stage_tile(sW[cur ^ 1], rw);
            stage_tile(sA[cur ^ 1], ra);
        }
        __syncthreads();
    }

    const float sa = *g.a_scale;
    const bool full = g.vec_out && m0 + wm * 64 + 64 <= g.m && n0 + wn * 64 + 64 <= g.n;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float sc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = sa * wsc[i][r];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (g.out_f32)
                store_tile_f32(g.out_f32, g.ld_out, m0 + wm * 64 + j * 16 + r16, n0 + wn * 64 + i * 16 + 4 * q, g.m, g.n,
                               acc[i][j], sc, full);
            else
                store_tile(g.out, g.ld_out, m0 + wm * 64 + j * 16 + r16, n0 + wn * 64 + i * 16 + 4 * q, g.m, g.n,
                           acc[i][j], sc, full);
    }
}

// ---------------------------------------------------------------- 256 x 256 tile kernel

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWT = 256;               // workgroup tile extent in n (and in m for the square tile)
constexpr int kWK = 64;                // k bytes per ring stage (one 32x32x64 MFMA deep)

// Ring geometry of a TN (n) x TM (m) tile with 64-byte k-slices: a stage holds TN weight rows
// then TM activation rows of 64 bytes; as many stages as fit the 160 KB LDS (5 x 32 KB for
// 256 x 256, 6 x 24 KB for 256 x 128). The eight waves are 2 (n) x 4 (m), each TN / 2 x
// TM / 4. A stage is (TN + TM) / 16 DMA blocks of 16 rows (1 KB each, block b at b KB of the
// stage); each wave issues kLoads of them per stage.
template <int TN, int TM>
struct RingShape {
    static constexpr int kStage = (TN + TM) * kWK;
    static constexpr int kRing = (160 * 1024) / kStage;
    static constexpr int kNI = TN / 64;           // 32-row weight blocks per wave (wave tile n = TN / 2)
    static constexpr int kJX = TM / 128;          // 32-row activation blocks per wave (wave tile m = TM / 4)
    static constexpr int kBlocks = (TN + TM) / 16;
    static constexpr int kLoads = (kBlocks + 7) / 8;   // DMA instructions per wave per stage
};

__device__ __forceinline__ v16f mfma32_e4m3(const v8i& a, const v8i& b, const v16f& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 32x32x16 bf16 MFMA, f32 accumulate: lane l supplies row (l % 32) of A and column (l % 32) of
// B as 8 consecutive k of the 16-k step chosen by l / 32; the accumulator layout is that of
// the 32x32x64 e4m3 MFMA.
__device__ __forceinline__ v16f mfma32_bf16(const bf16x8& a, const bf16x8& b, const v16f& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One 64-deep k-step of a wave's NI x NJ grid of 32 x 32 tiles (weight fragments w, activation
// fragments a; 32 code bytes per lane each). kExact == false: one e4m3 MFMA per tile. kExact:
// every product summed in f32 -- run j of four takes bytes 8 j .. 8 j + 7 of every fragment
// (the same k bytes of both operands), converts them to bf16 (exact for every e4m3 value; each
// fragment once per run, not once per tile) and feeds one bf16 MFMA per tile; the tiles are
// innermost, so consecutive MFMAs go to different accumulators.
template <bool kExact, int NI, int NJ>
__device__ __forceinline__ void mfma32_grid(v16f (&acc)[NI][NJ], const v8i (&w)[NI], const v8i (&a)[NJ]) {
    if constexpr (!kExact) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int jx = 0; jx < NJ; ++jx) acc[i][jx] = mfma32_e4m3(w[i], a[jx], acc[i][jx]);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x8 wb[NI], ab[NJ];
#pragma unroll
            for (int i = 0; i < NI; ++i) wb[i] = e4m3x8_to_bf16(w[i][2 * j], w[i][2 * j + 1]);
#pragma unroll
            for (int jx = 0; jx < NJ; ++jx) ab[jx] = e4m3x8_to_bf16(a[jx][2 * j], a[jx][2 * j + 1]);
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int jx = 0; jx < NJ; ++jx) acc[i][jx] = mfma32_bf16(wb[i], ab[jx], acc[i][jx]);
        }
    }
}

// Two floats to packed bf16 by the hardware conversion: round half to even, equal to
// f32_to_bf16 on every non-NaN input (checked over all 2^32 bit patterns); NaN stays NaN.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// 64-byte LDS rows; the 16-byte chunk c of row r sits at slot c ^ (((r >> 1) ^ (r >> 2)) & 3),
// so 16 consecutive rows read at one chunk (a 64-lane b128 read serves 16 lanes per pass)
// cover all 16 slots of the 256-byte bank window, and 8 consecutive rows all 8 of 128 bytes.
__device__ __forceinline__ int swz64(int row, int c) { return row * 64 + ((c ^ (((row >> 1) ^ (row >> 2)) & 3)) << 4); }

// Buffer descriptor over [base, base + bytes) (bytes clamped to 2^31 - 1) with range checking.
__device__ __forceinline__ i32x4 buffer_desc(const void* base, int64_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = (int)(uint32_t)b;
    r[1] = (int)((uint32_t)(b >> 32) & 0xffffu);
    r[2] = (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff);
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from byte offset voff of the buffer into LDS at lds + 16 * lane (an
// offset past the range writes zeros). Issued as asm so that the compiler's wait insertion
// does not hold every later LDS read behind it; the kernel waits for these loads itself.
__device__ __forceinline__ void dma16(const i32x4& rs, const uint8_t* lds, uint32_t voff) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)lds;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(rs)
                 : "memory", "m0");
}

__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Block -> (tile origin m0, n0; k split ks) of a ring kernel. Blocks go to the 8 XCDs round
// robin; each XCD takes a contiguous share of the tiles in an order that walks 8 m-tiles per
// n-tile, so the ~32 tiles an XCD holds at once share 8 activation and 4 weight panels
// through its L2. With a k split, blocks [s * tiles, (s + 1) * tiles) take split s.
template <int TN, int TM>
__device__ __forceinline__ void ring_tile(const GemmArgs& g, int64_t& m0, int64_t& n0, int& ks) {
    const int ntn = (int)((g.n + TN - 1) / TN), ntm = (int)((g.m + TM - 1) / TM);
    const int total = ntn * ntm;
    const int bid = (int)(blockIdx.x % (unsigned)total);
    ks = (int)(blockIdx.x / (unsigned)total);
    const int x = bid & 7, loc = bid >> 3;
    const int j = x * (total >> 3) + min(x, total & 7) + loc;
    constexpr int kGroupM = 8;
    const int grp = j / (kGroupM * ntn), within = j - grp * kGroupM * ntn;
    const int gms = min(kGroupM, ntm - grp * kGroupM);
    m0 = (int64_t)(grp * kGroupM + within % gms) * TM;
    n0 = (int64_t)(within / gms) * TN;
}

// The end of a ring kernel (all of its loads retired): split k stores this split's raw sums
// to the partial buffer; f32 output goes straight from the accumulators; bf16 output is
// scaled, staged through the ring as TM rows of 512 bytes and stored row by row.
template <int TN, int TM>
__device__ __forceinline__ void ring_epilogue(const GemmArgs& g, v16f (&acc)[TN / 64][TM / 128], int64_t m0,
                                              int64_t n0, int ks, uint8_t* smem, int t, int wn, int wm, int r32,
                                              int q) {
    constexpr int kNI = TN / 64, kJX = TM / 128;
    // acc[i][jx] register r: n = 32 i + 8 (r / 4) + 4 q + r % 4, m = 32 jx + lane % 32 (wave
    // tile relative). The scaled bf16 tile is staged in LDS as [m][n] with 512-byte rows, the
    // 16-byte chunk cn of row ml at slot cn ^ (ml & 15) with its two 8-byte halves swapped when
    // bit 3 xor bit 4 of ml is set: the 8-byte writes of 32 rows at one n land in 32 distinct
    // slots of the 256-byte bank window. Each half-wave then stores one whole 512-byte row.
    if (g.part) {
        // split k: this split's raw sums, f32 [m, n] slice ks of the partial buffer
        float* pt = g.part + (int64_t)ks * g.m * g.n;
        const float one[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
        for (int i = 0; i < kNI; ++i)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int64_t nb = n0 + wn * (TN / 2) + i * 32 + gq * 8 + q * 4;
#pragma unroll
                for (int jx = 0; jx < kJX; ++jx) {
                    const int64_t mm = m0 + wm * (TM / 4) + jx * 32 + r32;
                    const v4f a4 = {acc[i][jx][4 * gq], acc[i][jx][4 * gq + 1], acc[i][jx][4 * gq + 2], acc[i][jx][4 * gq + 3]};
                    store_tile_f32(pt, g.n, mm, nb, g.m, g.n, a4, one, (g.n & 3) == 0 && mm < g.m && nb + 3 < g.n);
                }
            }
        return;
    }
    const float sa = *g.a_scale;
    if (g.out_f32) {
        // f32 output: each lane stores its four consecutive n of one m row straight from the
        // accumulators (16 bytes per lane; the output is twice the bf16 size, no LDS staging)
#pragma unroll
        for (int i = 0; i < kNI; ++i)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int64_t nb = n0 + wn * (TN / 2) + i * 32 + gq * 8 + q * 4;
                float sc[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) sc[r] = sa * g.w_scale[(nb + r < g.n ? nb + r : g.n - 1) * g.ws_step];
#pragma unroll
                for (int jx = 0; jx < kJX; ++jx) {
                    const int64_t mm = m0 + wm * (TM / 4) + jx * 32 + r32;
                    const v4f a4 = {acc[i][jx][4 * gq], acc[i][jx][4 * gq + 1], acc[i][jx][4 * gq + 2], acc[i][jx][4 * gq + 3]};
                    store_tile_f32(g.out_f32, g.ld_out, mm, nb, g.m, g.n, a4, sc, g.vec_out && mm < g.m && nb + 3 < g.n);
                }
            }
        return;
    }
    __syncthreads();   // every wave is done reading the ring
#pragma unroll
    for (int i = 0; i < kNI; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int nl = wn * (TN / 2) + i * 32 + gq * 8;
            const int64_t nb = n0 + nl + q * 4;
            float sc[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[r] = sa * g.w_scale[(nb + r < g.n ? nb + r : g.n - 1) * g.ws_step];
#pragma unroll
            for (int jx = 0; jx < kJX; ++jx) {
                const int ml = wm * (TM / 4) + jx * 32 + r32;
                const int hs = ((ml >> 3) ^ (ml >> 4)) & 1;
                *reinterpret_cast<uint2*>(smem + ml * 512 + (((nl >> 3) ^ (ml & 15)) << 4) + ((q ^ hs) << 3)) =
                    make_uint2(pk_bf16(acc[i][jx][4 * gq] * sc[0], acc[i][jx][4 * gq + 1] * sc[1]),
                               pk_bf16(acc[i][jx][4 * gq + 2] * sc[2], acc[i][jx][4 * gq + 3] * sc[3]));
            }
        }
    __syncthreads();
    const bool vec = (g.ld_out & 7) == 0 && (reinterpret_cast<uintptr_t>(g.out) & 15) == 0;
    const bool full = vec && m0 + TM <= g.m && n0 + TN <= g.n;
#pragma unroll 4
    for (int it = 0; it < TM * 256 / 8 / 512; ++it) {    // TM rows x 32 chunk slots of 16 bytes
        const int e = t + it * 512, ml = e >> 5, cn = e & 31;
        if (cn >= TN / 8) continue;                          // past the tile's n extent
        uint4 v = lds16(smem + ml * 512 + ((cn ^ (ml & 15)) << 4));
        if (((ml >> 3) ^ (ml >> 4)) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
        const int64_t mm = m0 + ml, nn = n0 + cn * 8;
        uint16_t* o = g.out + mm * g.ld_out + nn;
        if (full) {
            *reinterpret_cast<uint4*>(o) = v;
        } else if (mm < g.m) {
            if (vec && nn + 8 <= g.n) {
                *reinterpret_cast<uint4*>(o) = v;
            } else {
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    if (nn + c < g.n) o[c] = (uint16_t)(w4[c >> 1] >> (16 * (c & 1)));
            }
        }
    }
}

// Operands under 2^31 bytes (buffer offsets). Grid = number of TN x TM tiles, 512 threads.
template <int TN, int TM, bool kExact>
__global__ __launch_bounds__(512) void tile256_kernel(const GemmArgs g) {
    using RS = RingShape<TN, TM>;
    constexpr int kStage = RS::kStage, kRing = RS::kRing, kNI = RS::kNI, kJX = RS::kJX, kLoads = RS::kLoads;
    constexpr int kWStageT = TN * kWK;              // the weight rows' part of a stage
    static_assert(TN == 256 && (TM == 256 || TM == 128), "tile shape");
    static_assert(kRing >= 4 && (kRing - 2) * kLoads < 64, "ring depth and the vmcnt field");
    __shared__ __attribute__((aligned(16))) uint8_t smem[kRing * kStage];
    // the epilogue stages the bf16 tile in the ring as TM rows of 512 bytes (TN <= 256)
    static_assert(kRing * kStage >= TM * 512, "the epilogue stages the whole bf16 tile in the ring");
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wn = wave >> 2, wm = wave & 3;        // wave tile: n TN / 2 x m TM / 4
    const int r32 = lane & 31, q = lane >> 5;

    int64_t m0, n0;
    int ks;
    ring_tile<TN, TM>(g, m0, n0, ks);

    // DMA: wave w fills weight rows 32 w .. 32 w + 31 and activation rows (TM / 8) w ..
    // (TM / 8) (w + 1) - 1 of a stage. 16 rows per instruction;
    // lane l lands in slot l of the instruction's 1 KB: row 16 i + l / 4, chunk slot l % 4,
    // which holds the logical chunk kc / 16 under the swizzle (the swizzle depends on the row
    // modulo 16 only).
    const i32x4 wrs = buffer_desc(g.w, g.n * g.k), ars = buffer_desc(g.a, g.m * g.lda);
    const int lr = lane >> 2;
    const int kc = ((lane & 3) ^ (((lr >> 1) ^ (lr >> 2)) & 3)) * 16;
    uint32_t dbase[kLoads];    // this lane's source offset of each of the wave's blocks (k = 0)
    int dlds[kLoads];          // the block's byte offset in a stage
    bool dw[kLoads];           // weight block (else activation)
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int blk = i < 2 ? wave * 2 + i : RS::kBlocks - TM / 16 + wave * kJX + (i - 2);
        dw[i] = blk < TN / 16;
        dlds[i] = blk * 1024;
        if (dw[i]) {
            const int row = blk * 16 + lr;
            dbase[i] = n0 + row < g.n ? (uint32_t)((n0 + row) * g.k + kc) : kOutOfRange;
        } else {
            const int row = (blk - TN / 16) * 16 + lr;
            dbase[i] = m0 + row < g.m ? (uint32_t)((m0 + row) * g.lda + kc) : kOutOfRange;
        }
    }
    // this block's k stages: s_beg .. s_beg + nk - 1 (all of k without a split)
    const int nk_all = (int)((g.k + kWK - 1) / kWK);
    const int kper = (nk_all + g.ksplit - 1) / g.ksplit;
    const int s_beg = ks * kper;
    const int nk = min(kper, nk_all - s_beg);   // >= 1: the launcher leaves no split empty
    auto issue = [&](int s) {   // stage s (past k its loads are out of range, zeros; past this
                                // split's range they are loaded and never read)
        const uint32_t k0 = (uint32_t)(s_beg + s) * kWK;
        const bool kin = (int64_t)k0 + kc < g.k;
        uint8_t* sb = smem + (s % kRing) * kStage;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) dma16(dw[i] ? wrs : ars, sb + dlds[i], kin ? dbase[i] + k0 : kOutOfRange);
    };
    auto read_ops = [&](int s, v8i (&wop)[kNI], v8i (&aop)[kJX]) {
        const uint8_t* sw = smem + (s % kRing) * kStage;
        const uint8_t* sa = sw + kWStageT;
#pragma unroll
        for (int i = 0; i < kNI; ++i) {
            const int row = wn * (TN / 2) + i * 32 + r32;
            wop[i] = cat8(lds16(sw + swz64(row, 2 * q)), lds16(sw + swz64(row, 2 * q + 1)));
        }
#pragma unroll
        for (int jx = 0; jx < kJX; ++jx) {
            const int row = wm * (TM / 4) + jx * 32 + r32;
            aop[jx] = cat8(lds16(sa + swz64(row, 2 * q)), lds16(sa + swz64(row, 2 * q + 1)));
        }
    };

    v16f acc[kNI][kJX];
#pragma unroll
    for (int i = 0; i < kNI; ++i)
#pragma unroll
        for (int jx = 0; jx < kJX; ++jx)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][jx][r] = 0.f;

    // Step kt: wait for stage kt + 1 (this thread's loads), barrier (all of them landed, and
    // every wave is past step kt - 1, so the slot of stage kt - 1 is free), refill that slot
    // with stage kt + kRing - 1, then read the operands of stage kt + 1 while the MFMAs of
    // stage kt (read one step earlier) run.
    auto step = [&](int kt, const v8i (&cw)[kNI], const v8i (&ca)[kJX], v8i (&nw)[kNI], v8i (&na)[kJX]) {
        wait_vmcnt<(kRing - 3) * kLoads>();
        __syncthreads();
        issue(kt + kRing - 1);
        if (kt + 1 < nk) read_ops(kt + 1, nw, na);
        __builtin_amdgcn_sched_barrier(0);   // the reads go out before the MFMAs
        mfma32_grid<kExact>(acc, cw, ca);
        __builtin_amdgcn_sched_barrier(0);   // and the MFMAs before the next barrier
    };
#pragma unroll
    for (int s = 0; s < kRing - 1; ++s) issue(s);
    if constexpr (kExact && TM == 256) {
        // Exact sums on the 256 x 256 tile: the 128 accumulators, one stage's operands and the
        // converted runs fill a wave's 256 registers, so each stage's operands are read in the
        // step that uses them instead of one step ahead (holding both spilled, and every spill
        // reload waited for all the DMA loads in flight). Step kt: wait for stage kt, barrier
        // (it has landed for every wave, and every wave is past step kt - 1, whose slot is
        // refilled with stage kt + kRing - 1), read, convert and multiply.
        for (int kt = 0; kt < nk; ++kt) {
            wait_vmcnt<(kRing - 2) * kLoads>();
            __syncthreads();
            issue(kt + kRing - 1);
            v8i w0[kNI], a0[kJX];
            read_ops(kt, w0, a0);
            mfma32_grid<true>(acc, w0, a0);
        }
    } else {
        v8i w0[kNI], a0[kJX], w1[kNI], a1[kJX];
        wait_vmcnt<(kRing - 2) * kLoads>();
        __syncthreads();
        read_ops(0, w0, a0);
        int kt = 0;
        for (; kt + 1 < nk; kt += 2) {
            step(kt, w0, a0, w1, a1);
            step(kt + 1, w1, a1, w0, a0);
        }
        if (kt < nk) step(kt, w0, a0, w1, a1);
    }
    wait_vmcnt<0>();   // the ring's trailing loads (past k) before the ring is reused

    ring_epilogue<TN, TM>(g, acc, m0, n0, ks, smem, t, wn, wm, r32, q);
}


// The ring tile kernel with 128-byte k-stages: a stage holds 128 bytes of k for each of the
// TN + TM rows, so every DMA request is a whole 128-byte line (the 64-byte stages issue half
// lines) and a CU's requests in flight carry twice the bytes. A DMA block is 8 rows (1 KB);
// each stage runs two MFMA k-steps. 192 x 128 only: four 40 KB stages fit the LDS.
template <int TN, int TM, bool kExact>
__global__ __launch_bounds__(512) void ring128_kernel(const GemmArgs g) {
    constexpr int kK = 128;                              // k bytes per stage
    constexpr int kStage = (TN + TM) * kK;
    constexpr int kRing = (160 * 1024) / kStage;
    constexpr int kNI = TN / 64, kJX = TM / 128;
    constexpr int kBlocks = (TN + TM) / 8;
    constexpr int kLoads = kBlocks / 8;                  // DMA instructions per wave per stage
    static_assert(TN == 192 && TM == 128, "tile shape");
    static_assert(kBlocks % 8 == 0 && kRing >= 4 && (kRing - 2) * kLoads < 64, "ring depth and the vmcnt field");
    __shared__ __attribute__((aligned(16))) uint8_t smem[kRing * kStage];
    static_assert(kRing * kStage >= TM * 512, "the epilogue stages the whole bf16 tile in the ring");
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wn = wave >> 2, wm = wave & 3;        // wave tile: n TN / 2 x m TM / 4
    const int r32 = lane & 31, q = lane >> 5;
    int64_t m0, n0;
    int ks;
    ring_tile<TN, TM>(g, m0, n0, ks);

    // DMA: wave w takes the 8-row blocks w + 8 i of a stage (weight blocks first); lane l lands
    // in slot l of the instruction's 1 KB: row 8 b + l / 8, slot l % 8, which holds the logical
    // chunk kc / 16 under swz128 (the block's parity is bit 3 of its rows).
    const i32x4 wrs = buffer_desc(g.w, g.n * g.k), ars = buffer_desc(g.a, g.m * g.lda);
    const int lr = lane >> 3;
    uint32_t dbase[kLoads];
    int dlds[kLoads], dkc[kLoads];
    bool dw[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int blk = wave + 8 * i;
        dw[i] = blk < TN / 8;
        dlds[i] = blk * 1024;
        const int row = (dw[i] ? blk : blk - TN / 8) * 8 + lr;    // within the weight or activation rows
        const int kc = ((lane & 7) ^ (row & 7) ^ ((row >> 3) & 1)) * 16;
        dkc[i] = kc;
        if (dw[i])
            dbase[i] = n0 + row < g.n ? (uint32_t)((n0 + row) * g.k + kc) : kOutOfRange;
        else
            dbase[i] = m0 + row < g.m ? (uint32_t)((m0 + row) * g.lda + kc) : kOutOfRange;
    }
    const int nk_all = (int)((g.k + kK - 1) / kK);
    const int kper = (nk_all + g.ksplit - 1) / g.ksplit;
    const int s_beg = ks * kper;
    const int nk = min(kper, nk_all - s_beg);   // >= 1: the launcher leaves no split empty
    auto issue = [&](int s) {   // stage s (past k: zeros; past this split's range: loaded, never read)
        const uint32_t k0 = (uint32_t)(s_beg + s) * kK;
        uint8_t* sb = smem + (s % kRing) * kStage;
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
            dma16(dw[i] ? wrs : ars, sb + dlds[i], (int64_t)k0 + dkc[i] < g.k ? dbase[i] + k0 : kOutOfRange);
    };
    auto read_ops = [&](int s, int h, v8i (&wop)[kNI], v8i (&aop)[kJX]) {   // k-step h of stage s
        const uint8_t* sw = smem + (s % kRing) * kStage;
        const uint8_t* sa = sw + TN * kK;
        const int c0 = 4 * h + 2 * q;
#pragma unroll
        for (int i = 0; i < kNI; ++i) {
            const int row = wn * (TN / 2) + i * 32 + r32;
            wop[i] = cat8(lds16(sw + swz128(row, c0)), lds16(sw + swz128(row, c0 + 1)));
        }
#pragma unroll
        for (int jx = 0; jx < kJX; ++jx) {
            const int row = wm * (TM / 4) + jx * 32 + r32;
            aop[jx] = cat8(lds16(sa + swz128(row, c0)), lds16(sa + swz128(row, c0 + 1)));
        }
    };

    v16f acc[kNI][kJX];
#pragma unroll
    for (int i = 0; i < kNI; ++i)
#pragma unroll
        for (int jx = 0; jx < kJX; ++jx)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][jx][r] = 0.f;
    auto mfmas = [&](const v8i (&cw)[kNI], const v8i (&ca)[kJX]) { mfma32_grid<kExact>(acc, cw, ca); };

    // Stage s: its second k-step's operands are read (the stage has landed) while the first
    // k-step's MFMAs run; then wait for stage s + 1 (this thread's loads), barrier (all of them
    // landed, and every wave is done reading stage s - 1, whose slot is refilled with stage
    // s + kRing - 1), read stage s + 1's first k-step and run the second k-step's MFMAs.
#pragma unroll
    for (int s = 0; s < kRing - 1; ++s) issue(s);
    v8i w0[kNI], a0[kJX], w1[kNI], a1[kJX];
    wait_vmcnt<(kRing - 2) * kLoads>();
    __syncthreads();
    read_ops(0, 0, w0, a0);
    for (int s = 0; s < nk; ++s) {
        read_ops(s, 1, w1, a1);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(w0, a0);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(kRing - 3) * kLoads>();
        __syncthreads();
        issue(s + kRing - 1);
        if (s + 1 < nk) read_ops(s + 1, 0, w0, a0);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(w1, a1);
        __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<0>();   // the ring's trailing loads (past k) before the ring is reused
    ring_epilogue<TN, TM>(g, acc, m0, n0, ks, smem, t, wn, wm, r32, q);
}

// Split-k epilogue: out[m, n] = (sum over s of part[s, m, n], in split order) * a_scale *
// w_scale[n], rounded once (bf16) or stored as f32. Four consecutive outputs per thread.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const GemmArgs g) {
    const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    const int64_t mn = g.m * g.n;
    if (e0 >= mn) return;
    const float sa = *g.a_scale;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if ((g.n & 3) == 0) {   // the four share a row; 16-byte partial loads
        for (int s = 0; s < g.ksplit; ++s) {
            const float4 p = *reinterpret_cast<const float4*>(g.part + (int64_t)s * mn + e0);
            v[0] += p.x; v[1] += p.y; v[2] += p.z; v[3] += p.w;
        }
        const int64_t mm = e0 / g.n, nn = e0 - mm * g.n;
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = v[r] * (sa * g.w_scale[(nn + r) * g.ws_step]);
        if (g.out_f32) {
            float* d = g.out_f32 + mm * g.ld_out + nn;
            if (g.vec_out) {
                *reinterpret_cast<float4*>(d) = make_float4(o[0], o[1], o[2], o[3]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) d[r] = o[r];
            }
        } else {
            uint16_t* d = g.out + mm * g.ld_out + nn;
            if (g.vec_out) {
                *reinterpret_cast<uint2*>(d) = make_uint2(pk_bf16(o[0], o[1]), pk_bf16(o[2], o[3]));
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) d[r] = (uint16_t)f32_to_bf16(o[r]);
            }
        }
        return;
    }
    for (int r = 0; r < 4 && e0 + r < mn; ++r) {
        const int64_t e = e0 + r, mm = e / g.n, nn = e - mm * g.n;
        float acc = 0.f;
        for (int s = 0; s < g.ksplit; ++s) acc += g.part[(int64_t)s * mn + e];
        const float o = acc * (sa * g.w_scale[nn * g.ws_step]);
        if (g.out_f32) g.out_f32[mm * g.ld_out + nn] = o;
        else g.out[mm * g.ld_out + nn] = (uint16_t)f32_to_bf16(o);
    }
}

// ---------------------------------------------------------------- dispatch

// Rows per weight panel: each workgroup pulls its BM activation rows and its panel's weight
// rows over all of k, and a CU's operand delivery rate is bounded, so the busiest CU's bytes,
// (rounds of 256 workgroups) x (BM + rows), set the time. Narrower panels (a multiple of 4
// rows, at least 64) are taken where they leave fewer such bytes: at 512 x 2688 x 4096, 84-row
// panels fill the chip with 256 workgroups of 148 rows instead of 168 of 192.
static int panel_rows(int64_t m, int64_t n, int BM, int BN) {
    const int64_t nmt = (m + BM - 1) / BM;
    auto cost = [&](int pw) {
        const int64_t wgs = 8 * nmt * (((n + pw - 1) / pw + 7) / 8);
        return ((wgs + 255) / 256) * (BM + pw);
    };
    int best = BN;
    for (int pw = BN - 4; pw >= 64; pw -= 4)
        if (cost(pw) < cost(best)) best = pw;
    return best;
}

// Prefetch depth: four k-steps in flight per wave on the e4m3 MFMA where k is a whole number
// of four-step groups (at 512 x 2688 x 4096 23.6 -> 23.1 us, 128 x 2688 x 4096 19.5 -> 18.0;
// where four-step padding was needed, as at k = 2688, it lost), else two; exact sums keep two,
// as their conversions leave no registers for more.
template <int BM, int WN, bool kExact>
static void launch_panel(GemmArgs g, hipStream_t st) {
    g.panel_rows = panel_rows(g.m, g.n, BM, 4 * WN);
    const int64_t npan = (g.n + g.panel_rows - 1) / g.panel_rows, nmt = (g.m + BM - 1) / BM;
    const dim3 grid((unsigned)(8 * nmt * ((npan + 7) / 8)));
    if constexpr (!kExact) {
        if ((g.k + 127) / 128 % 4 == 0) {   // k-steps: a whole number of four-step groups
            panel_kernel<BM, WN, false, 4><<<grid, dim3(256), 0, st>>>(g);
            count_launch(Kern::kPanel64x128, g.m);
            return;
        }
    }
    panel_kernel<BM, WN, kExact, 2><<<grid, dim3(256), 0, st>>>(g);
    count_launch(kExact ? Kern::kPanel64x128Exact : Kern::kPanel64x128, g.m);
}

// Measured on MI355X at m = 512 (in_proj 10304 x 2688, out_proj 2688 x 4096): the
// 192 x 128 ring tile (216 workgroups of 860 KB) takes in_proj to 25.4 us with 64-byte
// k-slices and 23.5 us with 128-byte ones (384 x 10300 x 2608: 34.3 vs 28.6 us), against 28.6
// for 256 x 128 (164 of 1 MB) and 30.4 for a 128 x 192 panel kernel (two k-steps of register
// prefetch); earlier panel versions took it from 37 to 33 us; where those
// tiles give too few workgroups to fill the chip (out_proj: 56), 64 x 128 tiles
// (168 workgroups) take it from 34 to 21 us. The 256 x 256 kernel leads from about
// 160 of its tiles (m = 1024 for in_proj, m = 4096 for out_proj: 45 vs 54 us and
// 60 vs 74 us; at m = 15,360 477 vs 652 us and 187 vs 253 us) and trails below
// (123 tiles at m = 641: 43 vs 36 us).
// Split k for m <= 640 where the ring tiles are too few to fill the chip (the panel kernel's
// case): the 192 x 128 ring tile over S k ranges puts fewer operand bytes on the busiest CU
// than a 64 x 128 panel over all of k, at the price of the f32 partials and the reduction.
// Costs in bytes of one CU's operand delivery (~37 GB/s); the partials' cost is fitted to
// three measured shapes (split against panel: 512 x 2688 x 4096 25.3 vs 20.9 us, 64 x 4096 x
// 4096 16.2 vs 19.3 us, 200 x 10304 x 2688 25.9 vs 26.4 us): ~6 us fixed (230 KB) plus
// ~0.35 us per MB of partials (bytes / 77) -- the tiles write them in one burst at their end.
// The estimate still missed 128 x 2688 x 4096 (split 20.7 vs panel 19.7 us, 42 panel
// workgroups), so a split is taken only where the panel kernel would run at most 32 workgroups
// (7/8 of the chip idle). Returns the S that minimises the estimate there, else 1.
static int split_k(int64_t m, int64_t n, int64_t k) {
    if (m > 640 || m <= 0 || n <= 0 || k <= 0) return 1;
    const int64_t half_tiles = ((n + kWT - 1) / kWT) * ((m + 127) / 128);
    const int64_t t192 = ((n + 191) / 192) * ((m + 127) / 128);
    if (half_tiles >= 160 || t192 >= 160) return 1;
    constexpr int64_t kSK = 128;   // k bytes per stage of the split kernel (ring128_kernel)
    const int64_t nk = (k + kSK - 1) / kSK;
    const int64_t panel_wgs = 8 * ((m + 63) / 64) * (((n + 127) / 128 + 7) / 8);
    if (panel_wgs > 32) return 1;
    int64_t best = (panel_wgs + 255) / 256 * (64 + 128) * k;
    int split = 1;
    for (int S = 2; S <= 8; ++S) {
        const int64_t kper = (nk + S - 1) / S;
        if (kper * (S - 1) >= nk) continue;   // a split would be empty
        const int64_t cost = (t192 * S + 255) / 256 * ((192 + 128) * kper * kSK + 4 * 192 * 128) +
                             S * m * n * 4 / 77 + 230000;
        if (cost < best) { best = cost; split = S; }
    }
    return split;
}

size_t gemm_part_bytes(int64_t m, int64_t n, int64_t k) {
    const int S = split_k(m, n, k);
    return S > 1 ? (size_t)S * (size_t)m * (size_t)n * sizeof(float) : 0;
}

template <bool kExact>
static nhm_status dispatch_gemm(GemmArgs g, hipStream_t st, float* part, size_t part_bytes) {
    const int64_t m = g.m, n = g.n, k = g.k, lda = g.lda;
    // buffer descriptors address the operands with 32-bit offsets
    const bool offsets_fit = n * k < (int64_t(1) << 31) && m * lda < (int64_t(1) << 31);
    // m <= 640: a ring tile when it gives >= 160 workgroups; of 256 x 128 and 192 x 128 the one
    // whose busiest CU pulls the fewest operand bytes, (workgroups per CU) x (tile n + tile m) x k
    // (each CU's delivery rate is bounded by the requests it keeps in flight)
    const int64_t half_tiles = ((n + kWT - 1) / kWT) * ((m + 127) / 128);
    const int64_t t192 = ((n + 191) / 192) * ((m + 127) / 128);
    if (m <= 640 && offsets_fit && (half_tiles >= 160 || t192 >= 160)) {
        const int64_t c256 = half_tiles >= 160 ? ((half_tiles + 255) / 256) * (256 + 128) : INT64_MAX;
        const int64_t c192 = t192 >= 160 ? ((t192 + 255) / 256) * (192 + 128) : INT64_MAX;
        if (c192 < c256) {
            ring128_kernel<192, 128, kExact><<<dim3((unsigned)t192), dim3(512), 0, st>>>(g);
            count_launch(kExact ? Kern::kRing192x128Exact : Kern::kRing192x128, m);
            return check_launch("gemm (192 x 128)");
        }
        tile256_kernel<256, 128, kExact><<<dim3((unsigned)half_tiles), dim3(512), 0, st>>>(g);
        count_launch(kExact ? Kern::kRing256x128Exact : Kern::kRing256x128, m);
        return check_launch("gemm (256 x 128)");
    }
    if (m <= 640 && offsets_fit) {   // too few ring tiles to fill the chip
        const int S = split_k(m, n, k);
        if (S > 1 && part && part_bytes >= gemm_part_bytes(m, n, k) && (reinterpret_cast<uintptr_t>(part) & 15) == 0) {
            g.ksplit = S;
            g.part = part;
            ring128_kernel<192, 128, kExact><<<dim3((unsigned)(t192 * S)), dim3(512), 0, st>>>(g);
            count_launch(kExact ? Kern::kRing192x128Exact : Kern::kRing192x128, m);
            nhm_status s = check_launch("gemm (192 x 128, split k)");
            if (s != NHM_OK) return s;
            splitk_reduce_kernel<<<dim3((unsigned)((m * n + 1023) / 1024)), dim3(256), 0, st>>>(g);
            count_launch(Kern::kSplitkReduce, m);
            return check_launch("gemm split-k reduce");
        }
        launch_panel<64, 32, kExact>(g, st);
        return check_launch("gemm (panel)");
    }
    const int64_t wide_tiles = ((n + kWT - 1) / kWT) * ((m + kWT - 1) / kWT);
    if (offsets_fit && wide_tiles >= 160) {
        tile256_kernel<256, 256, kExact><<<dim3((unsigned)wide_tiles), dim3(512), 0, st>>>(g);
        count_launch(kExact ? Kern::kRing256x256Exact : Kern::kRing256x256, m);
        return check_launch("gemm (256 x 256)");
    }
    if (!offsets_fit)   // refused by the callers' host checks before anything is enqueued
        return fail(NHM_ERR_UNSUPPORTED, "gemm: an operand of 2 GiB or more");
    const dim3 grid((unsigned)((n + kTile - 1) / kTile), (unsigned)((m + kTile - 1) / kTile));
    gemm_kernel<kExact><<<grid, dim3(256), 0, st>>>(g);
    count_launch(kExact ? Kern::kTile128Exact : Kern::kTile128, m);
    return check_launch("gemm");
}

nhm_status launch_gemm(const uint8_t* a, int64_t lda, int64_t m, const uint8_t* w, const float* w_scale,
                       const float* a_scale, int64_t n, int64_t k, uint16_t* out, int64_t ld_out,
                       hipStream_t st, float* out_f32, float* part, size_t part_bytes, bool exact, int ws_step) {
    GemmArgs g{a, lda, m, w, w_scale, a_scale, n, k, out, ld_out,
               out_f32 ? ld_out % 4 == 0 && reinterpret_cast<uintptr_t>(out_f32) % 16 == 0
                       : ld_out % 4 == 0 && reinterpret_cast<uintptr_t>(out) % 8 == 0,
               out_f32};
    g.ws_step = ws_step;
    return exact ? dispatch_gemm<true>(g, st, part, part_bytes) : dispatch_gemm<false>(g, st, part, part_bytes);
}

}  // namespace nhm
