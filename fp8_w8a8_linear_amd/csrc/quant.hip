// Static per-tensor activation quant, bf16 -> e4m3 (the kQuantFp8Static op of
// [PR988] "The Thor finding, measured"). HBM-bound: 2 bytes in, 1 byte out per
// element, so the kernel only has to keep loads wide and coalesced.
#include "nhm_device.h"
#include "nhm_internal.h"

namespace nhm {

// Eight elements per thread: one 16-byte load, one 8-byte store.
__global__ __launch_bounds__(256) void quant_vec8_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                        int64_t vec_per_row, int64_t ld_x,
                                                        const float* __restrict__ scale,
                                                        uint8_t* __restrict__ q, int64_t ld_q) {
    const float s = *scale;
    const int64_t total = rows * vec_per_row;
    // the scale is uniform: one branch picks the reciprocal form or the IEEE division
    const bool fast = fast_scale(s);
    const float rs = __fdiv_rn(1.0f, s);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / vec_per_row, v = i - r * vec_per_row;
        const uint4 in = *reinterpret_cast<const uint4*>(x + r * ld_x + v * 8);
        uint2 code;
        if (fast && __builtin_amdgcn_ballot_w64(bf16x8_special(in) != 0u) == 0) code = quant_bf16x8_fast(in, s, rs);
        else code = quant_bf16x8(in, s);
        *reinterpret_cast<uint2*>(q + r * ld_q + v * 8) = code;
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
}

}  // namespace nhm
