// Static per-tensor activation quant, bf16 -> e4m3 (the kQuantFp8Static op of
// [PR988] "The Thor finding, measured"). HBM-bound: 2 bytes in, 1 byte out per
// element, so the kernel only has to keep loads wide and coalesced.
#include "nhm_device.h"
#include "nhm_internal.h"

namespace nhm {

// Eight elements per thread: one 16-byte load, one 8-byte store. The first element's load
// goes out before the scale is read (at decode sizes each thread has one element, and the two
// round trips overlap); row indexes use 32-bit division when the element count allows.
__global__ __launch_bounds__(256) void quant_vec8_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                        int64_t vec_per_row, int64_t ld_x,
                                                        const float* __restrict__ scale,
                                                        uint8_t* __restrict__ q, int64_t ld_q) {
    const int64_t total = rows * vec_per_row;
    const bool narrow = total < (int64_t(1) << 31);
    auto split = [&](int64_t i, int64_t& r, int64_t& v) {
        if (narrow) {
            const uint32_t rr = (uint32_t)i / (uint32_t)vec_per_row;
            r = rr;
            v = (uint32_t)i - rr * (uint32_t)vec_per_row;
        } else {
            r = i / vec_per_row;
            v = i - r * vec_per_row;
        }
    };
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    int64_t r, v;
    split(i, r, v);
    uint4 in = *reinterpret_cast<const uint4*>(x + r * ld_x + v * 8);
    asm volatile("" ::: "memory");   // the first load ahead of the scale
    const float s = *scale;
    // the scale is uniform: one branch picks the reciprocal form or the IEEE division
    const bool fast = fast_scale(s);
    const float rs = __fdiv_rn(1.0f, s);
    for (;;) {
        uint2 code;
        if (fast && __builtin_amdgcn_ballot_w64(bf16x8_special(in) != 0u) == 0) code = quant_bf16x8_fast(in, s, rs);
        else code = quant_bf16x8(in, s);
        *reinterpret_cast<uint2*>(q + r * ld_q + v * 8) = code;
        i += (int64_t)gridDim.x * blockDim.x;
        if (i >= total) break;
        split(i, r, v);
        in = *reinterpret_cast<const uint4*>(x + r * ld_x + v * 8);
    }
}

__global__ __launch_bounds__(256) void quant_scalar_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                          int64_t cols, int64_t ld_x,
                                                          const float* __restrict__ scale,
                                                          uint8_t* __restrict__ q, int64_t ld_q) {
    const float s = *scale;
    const int64_t total = rows * cols;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / cols, c = i - r * cols;
        q[r * ld_q + c] = (uint8_t)quant_bf16(x[r * ld_x + c], s);
    }
}

void launch_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, const float* scale,
                     uint8_t* q, int64_t ld_q, hipStream_t st) {
    if (rows <= 0 || cols <= 0) return;
    const bool vec = cols % 8 == 0 && ld_x % 8 == 0 && ld_q % 8 == 0 &&
                     reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(q) % 8 == 0;
    const int64_t work = vec ? rows * (cols / 8) : rows * cols;
    int64_t blocks = (work + 255) / 256;
    if (blocks > 256 * 16) blocks = 256 * 16;
    if (vec)
        quant_vec8_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(x, rows, cols / 8, ld_x, scale, q, ld_q);
    else
        quant_scalar_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(x, rows, cols, ld_x, scale, q, ld_q);
    count_launch(vec ? Kern::kQuantVec8 : Kern::kQuantScalar, rows);
}

}  // namespace nhm

namespace nhm {

// Per-output-channel FP8 -> bf16 weight dequant (the standalone device dequant of the
// W8A16 arm): out[r, c] = bf16(val(w[r, c]) * w_scale[r]), the product in f32 and rounded
// once to bf16 (half to even). HBM-bound: 1 byte in, 2 bytes out per element; each thread
// takes 16 codes (one 16-byte load, two 16-byte stores). The codes convert to bf16
// exactly (every e4m3 value is a bf16 value; NaN codes stay NaN).
__global__ __launch_bounds__(256) void dequant_channel_kernel(const uint8_t* __restrict__ w, int64_t rows,
                                                             int64_t vec_per_row, int64_t ld_w,
                                                             const float* __restrict__ w_scale,
                                                             uint16_t* __restrict__ out, int64_t ld_out) {
    const int64_t total = rows * vec_per_row;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / vec_per_row, v = i - r * vec_per_row;
        const uint4 codes = *reinterpret_cast<const uint4*>(w + r * ld_w + v * 16);
        const float s = w_scale[r];
        const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
        uint32_t o[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bf16x8 b = e4m3x8_to_bf16(cw[2 * h], cw[2 * h + 1]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[4 * h + j] = f32x2_to_bf16x2((float)b[2 * j] * s, (float)b[2 * j + 1] * s);
        }
        uint4* dst = reinterpret_cast<uint4*>(out + r * ld_out + v * 16);
        dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
}

void launch_dequant_channel(const uint8_t* w, int64_t rows, int64_t cols, int64_t ld_w, const float* w_scale,
                            uint16_t* out, int64_t ld_out, hipStream_t st) {
    if (rows <= 0 || cols <= 0) return;
    const int64_t work = rows * (cols / 16);
    int64_t blocks = (work + 255) / 256;
    if (blocks > 256 * 16) blocks = 256 * 16;
    dequant_channel_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(w, rows, cols / 16, ld_w, w_scale, out,
                                                                        ld_out);
    count_launch(Kern::kDequantChannel, rows);
}

// n 32-bit words set to zero (in place of a memset node, which a captured graph should not hold)
__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* p, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

void launch_clear(uint32_t* p, int n, hipStream_t st) {
    if (n <= 0) return;
    const int blocks = (n + 255) / 256 < 64 ? (n + 255) / 256 : 64;
    clear_words_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(p, n);
    count_launch(Kern::kClear, n);
}

}  // namespace nhm
