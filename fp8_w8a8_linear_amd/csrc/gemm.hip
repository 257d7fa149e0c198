// Tiled FP8 W8A8 GEMM on the gfx950 e4m3 MFMA (prefill-sized m).
//
// out[i, j] = bf16( (sum_k a[i, k] * w[j, k]) * a_scale * w_scale[j] ), f32 accumulate.
// Both operands are k-contiguous ([m, k] activations, [n, k] weights in the
// [out, in] orientation), so a lane's 32-byte MFMA operand is one contiguous run.
//
// Workgroup tile 128 (n) x 128 (m) x 128 (k), 4 waves in a 2 x 2 grid, each wave a
// 64 x 64 block = 4 x 4 MFMA 16x16x128 tiles. Operand tiles are staged through
// LDS (double-buffered, 64 KB): global loads of tile t+1 are in flight while the
// MFMAs consume tile t. Rows of a staged tile are 128 bytes; the 16-byte chunk c
// of row r is stored at chunk c ^ (r & 7), so the 16 lanes that read one chunk
// column from 16 consecutive rows spread over all LDS banks.
#include "nhm_device.h"
#include "nhm_internal.h"

namespace nhm {

constexpr int kTile = 128;   // n, m and k extent of a workgroup tile

struct GemmArgs {
    const uint8_t* a; int64_t lda; int64_t m;
    const uint8_t* w; const float* w_scale; const float* a_scale; int64_t n, k;
    uint16_t* out; int64_t ld_out; bool vec_out;   // vec_out: 8-byte aligned rows
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kTile + ((chunk ^ (row & 7)) << 4); }

// Loads this thread's four 16-byte chunks of a 128 x 128 operand tile.
__device__ __forceinline__ void load_tile(uint4 (&r)[4], const uint8_t* base, int64_t ld, int64_t row0,
                                          int64_t nrows, int64_t k0, int64_t k) {
    const int t = threadIdx.x;
    const int chunk = t & 7;
    const int64_t kb = k0 + chunk * 16;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int64_t row = row0 + p * 32 + (t >> 3);
        if (row < nrows && kb < k)
            r[p] = *reinterpret_cast<const uint4*>(base + row * ld + kb);
        else
            r[p] = make_uint4(0u, 0u, 0u, 0u);
    }
}

__device__ __forceinline__ void store_tile(uint8_t* s, const uint4 (&r)[4]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int p = 0; p < 4; ++p)
        *reinterpret_cast<uint4*>(s + swz(p * 32 + (t >> 3), t & 7)) = r[p];
}

__device__ __forceinline__ v8i lds_operand(const uint8_t* s, int row, int q) {
    const uint4 lo = *reinterpret_cast<const uint4*>(s + swz(row, 2 * q));
    const uint4 hi = *reinterpret_cast<const uint4*>(s + swz(row, 2 * q + 1));
    v8i v;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    return v;
}

__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs g) {
    __shared__ __attribute__((aligned(16))) uint8_t sW[2][kTile * kTile];
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][kTile * kTile];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wn = wave >> 1, wm = wave & 1;
    const int64_t n0 = (int64_t)blockIdx.x * kTile, m0 = (int64_t)blockIdx.y * kTile;
    const int nk = (int)((g.k + kTile - 1) / kTile);

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    uint4 rw[4], ra[4];
    load_tile(rw, g.w, g.k, n0, g.n, 0, g.k);
    load_tile(ra, g.a, g.lda, m0, g.m, 0, g.k);
    store_tile(sW[0], rw);
    store_tile(sA[0], ra);
    __syncthreads();

    const int q = lane >> 4, r16 = lane & 15;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            load_tile(rw, g.w, g.k, n0, g.n, (int64_t)(kt + 1) * kTile, g.k);
            load_tile(ra, g.a, g.lda, m0, g.m, (int64_t)(kt + 1) * kTile, g.k);
        }
        v8i av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = lds_operand(sW[cur], wn * 64 + i * 16 + r16, q);
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = lds_operand(sA[cur], wm * 64 + j * 16 + r16, q);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma_e4m3(av[i], bv[j], acc[i][j]);
        if (kt + 1 < nk) {
            store_tile(sW[cur ^ 1], rw);
            store_tile(sA[cur ^ 1], ra);
        }
        __syncthreads();
    }

    const float sa = *g.a_scale;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t nb = n0 + wn * 64 + i * 16 + 4 * q;
        float sc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = nb + r < g.n ? sa * g.w_scale[nb + r] : 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t mm = m0 + wm * 64 + j * 16 + r16;
            if (mm >= g.m) continue;
            uint32_t hb[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) hb[r] = f32_to_bf16(acc[i][j][r] * sc[r]);
            uint16_t* o = g.out + mm * g.ld_out + nb;
            if (g.vec_out && nb + 3 < g.n) {
                *reinterpret_cast<uint2*>(o) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
            } else {
                for (int r = 0; r < 4; ++r)
                    if (nb + r < g.n) o[r] = (uint16_t)hb[r];
            }
        }
    }
}

nhm_status launch_gemm(const uint8_t* a, int64_t lda, int64_t m, const uint8_t* w, const float* w_scale,
                       const float* a_scale, int64_t n, int64_t k, uint16_t* out, int64_t ld_out,
                       hipStream_t st) {
    GemmArgs g{a, lda, m, w, w_scale, a_scale, n, k, out, ld_out,
               ld_out % 4 == 0 && reinterpret_cast<uintptr_t>(out) % 8 == 0};
    const dim3 grid((unsigned)((n + kTile - 1) / kTile), (unsigned)((m + kTile - 1) / kTile));
    gemm_kernel<<<grid, dim3(256), 0, st>>>(g);
    return check_launch("gemm");
}

}  // namespace nhm
