// Device-side number formats and small helpers shared by the libnhm kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nhm {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bfloat16 bits, round half to even (the hardware conversion; checked equal to
// the integer rounding (u + 0x7fff + lsb) >> 16 on every non-NaN float); NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// Two floats to a dword of two bf16 (a in the low half), each as f32_to_bf16, in one instruction.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// float -> OCP FP8 E4M3FN code: round half to even, saturating at +-448 (infinities
// included), NaN -> 0x7F with the sign kept, zero results keep the sign bit. The value is
// clamped to [-448, 448] and converted by the hardware (round half to even); NaN is
// selected separately. Checked on all 2^32 float bit patterns against the integer form:
// for |v| in [2^-6, 448) the code is the float's biased exponent and top three mantissa
// bits rounded half to even on the 20 bits below them and re-biased from 127 to 7, below
// 2^-6 it counts multiples of 2^-9.
__device__ __forceinline__ uint32_t e4m3_nan(float v, uint32_t code) {
    const uint32_t u = __float_as_uint(v);
    return (u & 0x7fffffffu) > 0x7f800000u ? (((u >> 24) & 0x80u) | 0x7fu) : code;
}
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const float c = __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
    return e4m3_nan(v, (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xffu);
}
// Four values to four codes (bytes in argument order), each as e4m3_code.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, -448.0f, 448.0f),
                                                            __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f), 0, false);
    r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(c, -448.0f, 448.0f),
                                                  __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f), (int)r, true);
    return e4m3_nan(a, r & 0xffu) | (e4m3_nan(b, (r >> 8) & 0xffu) << 8) | (e4m3_nan(c, (r >> 16) & 0xffu) << 16) |
           (e4m3_nan(d, r >> 24) << 24);
}

// The eight bf16 values of a 16-byte load, in memory order.
__device__ __forceinline__ void unpack8(const uint4 v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = bf16_to_f32(w[j] & 0xffffu);
        f[2 * j + 1] = bf16_to_f32(w[j] >> 16);
    }
}

// E4M3(x / s) for positive scales in [2^-80, 2^100], without a division per element.
// With r = 1/s rounded to nearest (one IEEE division per thread), q0 = RN(x r) is corrected
// once by the exact residual: q = RN(q0 - RN(q0 s - x) r) -- Markstein's correction step
// for division by a known reciprocal (P. Markstein, "Computation of elementary functions on
// the IBM RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990), whose residual
// q0 s - x one fused multiply-add computes exactly. This equals the IEEE quotient
// RN(x / s) bit for bit, signed zeros included: checked on the host's IEEE f32 arithmetic
// (tests/c/recip_div_check.c) over every bf16 significand (both signs) against every f32
// scale significand in [1, 2) (2^31 pairs; exponents only scale both sides inside this
// range), and over all 65,536 bf16 patterns at scales spread over 2^-80 .. 2^99. The product is clamped to
// +-2^100 so that the residual stays finite when x r overflows (such quotients saturate to
// +-448 either way). NaN inputs take 0x7F with their own sign, as the IEEE quotient of a
// NaN is that NaN. Other scales (negative, tiny, huge, NaN) use the IEEE division.
__device__ __forceinline__ bool fast_scale(float s) { return s >= 0x1p-80f && s <= 0x1p100f; }
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
    const float q0 = __builtin_amdgcn_fmed3f(x * r, -0x1p100f, 0x1p100f);
    return fmaf(fmaf(q0, s, -x), -r, q0);
}
// Eight bf16 values (a 16-byte load, memory order) to eight e4m3 codes (8 bytes, memory
// order) with the quotient of div_by_scale (fast_scale(s) must hold, r = 1/s). Finite
// inputs only: where bf16x8_special() holds for any input of the wave, the caller takes
// quant_bf16x8 instead (NaN codes), behind one wave-uniform branch.
__device__ __forceinline__ uint2 quant_bf16x8_fast(const uint4 v, float s, float r) {
    float x[8], q[8];
    unpack8(v, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = __builtin_amdgcn_fmed3f(div_by_scale(x[j], s, r), -448.0f, 448.0f);
    uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], (int)lo, true);
    uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
    hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], (int)hi, true);
    return make_uint2(lo, hi);
}
// Non-zero when one of eight bf16 values has an exponent field of all ones (inf or NaN):
// (h & 0x7f80) + 0x80 carries into the sign position of its half.
__device__ __forceinline__ uint32_t bf16x8_special(const uint4 v) {
    return (((v.x & 0x7f807f80u) + 0x00800080u) | ((v.y & 0x7f807f80u) + 0x00800080u) |
            ((v.z & 0x7f807f80u) + 0x00800080u) | ((v.w & 0x7f807f80u) + 0x00800080u)) & 0x80008000u;
}
// Exact float value of an e4m3 code (finite codes; the GEMMs never decode in software).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    const uint32_t e = (c >> 3) & 0xfu, m = c & 7u;
    float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
    return (c & 0x80u) ? -mag : mag;
}

// The static activation quant of one bf16 value: E4M3(f32(x) / s), IEEE division.
__device__ __forceinline__ uint32_t quant_bf16(uint32_t xb, float s) {
    return e4m3_code(__fdiv_rn(bf16_to_f32(xb), s));
}
// Four bf16 values (two dwords, memory order) to four codes, each as quant_bf16.
__device__ __forceinline__ uint32_t quant_bf16x4(uint32_t w0, uint32_t w1, float s) {
    return e4m3x4(__fdiv_rn(bf16_to_f32(w0 & 0xffffu), s), __fdiv_rn(bf16_to_f32(w0 >> 16), s),
                  __fdiv_rn(bf16_to_f32(w1 & 0xffffu), s), __fdiv_rn(bf16_to_f32(w1 >> 16), s));
}
// Eight bf16 values to eight codes as quant_bf16 (IEEE division; any scale).
__device__ __forceinline__ uint2 quant_bf16x8(const uint4 v, float s) {
    return make_uint2(quant_bf16x4(v.x, v.y, s), quant_bf16x4(v.z, v.w, s));
}

// x * sigmoid(x) with the hardware reciprocal (about 1 ulp) instead of an IEEE division
__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

__device__ __forceinline__ float softplus(float u) { return u > 20.0f ? u : log1pf(__expf(u)); }

// Sum over the 64 lanes of a wave; every lane receives the total.
// Lane sums by DPP (VALU lane moves within rows of 16 lanes, and row_bcast across rows)
// instead of LDS-crossbar permutes, which take an LDS round trip per step.
// dpp_take: lane i's view of another lane's v under the DPP control; 0 where the row or bank
// mask leaves lane i out or the source lies outside its row.
template <int kCtrl, int kRowMask = 0xF, int kBankMask = 0xF>
__device__ __forceinline__ float dpp_take(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, kRowMask, kBankMask, false));
}

// Sums over each 32-lane half: four in-row steps (quad xor 1 and xor 2, then each row's halves
// and quarters mirrored onto each other) leave every lane with its row's sum; row 1 (3) then adds
// lane 15 of row 0 (2). Lanes 31 and 63 hold their halves' sums (other lanes partial sums).
__device__ __forceinline__ float half_sum(float v) {
    v += dpp_take<0xB1>(v);      // quad_perm [1, 0, 3, 2]
    v += dpp_take<0x4E>(v);      // quad_perm [2, 3, 0, 1]
    v += dpp_take<0x141>(v);     // row_half_mirror
    v += dpp_take<0x140>(v);     // row_mirror
    return v + dpp_take<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
}

// The sum over the wave, in every lane: row_bcast:31 adds lane 31 into rows 2 and 3, and lane
// 63's total is read out.
__device__ __forceinline__ float wave_sum(float v) {
    v = half_sum(v);
    v += dpp_take<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Inclusive prefix sum over the wave's 64 lanes: within each row the sums of the last 4 lanes
// (shifts by 1, 2, 3 of the original values), then shifts by 4 (lanes 4-15) and 8 (lanes 8-15)
// of those partial sums; then row_bcast carries row 0's (2's) total into row 1 (3), and lane
// 31's into rows 2 and 3.
__device__ __forceinline__ float wave_prefix_sum(float v) {
    const float v0 = v;
    v += dpp_take<0x111>(v0);              // row_shr:1
    v += dpp_take<0x112>(v0);              // row_shr:2
    v += dpp_take<0x113>(v0);              // row_shr:3
    v += dpp_take<0x114, 0xF, 0xE>(v);     // row_shr:4, lanes 4-15 of each row
    v += dpp_take<0x118, 0xF, 0xC>(v);     // row_shr:8, lanes 8-15 of each row
    v += dpp_take<0x142, 0xA>(v);          // row_bcast:15 into rows 1 and 3
    return v + dpp_take<0x143, 0xC>(v);    // row_bcast:31 into rows 2 and 3
}

// 16x16x128 e4m3 MFMA, f32 accumulate (gfx950). Lane l supplies row (l % 16) of A
// and column (l % 16) of B, each as 32 consecutive k-bytes of the 128-k step chosen
// by l / 16; the accumulator lane l, register r holds D[4*(l/16)+r][l%16].
__device__ __forceinline__ v4f mfma_e4m3(const v8i& a, const v8i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// The e4m3 MFMA sums its 128 products in a narrower adder than f32: measured on MI355X,
// up to ~2^-17 of sum |a b| per instruction (and 32x32x64 the same). Where exact f32
// accumulation is wanted, the codes go through the bf16 MFMA instead: every e4m3 value
// is exact in bf16, and the bf16 16x16x32 MFMA sums its 32 exact products to within
// ~0.2 * 2^-24 of sum |a b| (measured).

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// 16x16x32 bf16 MFMA, f32 accumulate: lane l supplies row (l % 16) of A and column
// (l % 16) of B, 8 consecutive k of the 32-k step chosen by l / 16.
__device__ __forceinline__ v4f mfma_bf16(const bf16x8& a, const bf16x8& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32 bytes of an operand row through a buffer descriptor: the descriptor's range check
// returns zeros for offsets past the operand, so rows >= nrows and k beyond the end
// need no branches (the caller passes kGemvOut for them).
constexpr uint32_t kGemvOut = 0x80000000u;
template <int kAux>
__device__ __forceinline__ v8i bload32(const __amdgpu_buffer_rsrc_t& r, uint32_t lo_off, uint32_t hi_off) {
    const v4u lo = __builtin_amdgcn_raw_buffer_load_b128(r, lo_off, 0, kAux);
    const v4u hi = __builtin_amdgcn_raw_buffer_load_b128(r, hi_off, 0, kAux);
    v8i v;
    v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
    v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
    return v;
}
// Eight e4m3 codes (two dwords, memory order) as exact bf16 values (hardware convert, scale 1).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
    const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    // whole-register bit casts (no element extraction): each pair is one dword, low half first
    const uint4 u = make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                               __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
    return __builtin_bit_cast(bf16x8, u);
}

// s_waitcnt with vmcnt <= n (n < 64), expcnt and lgkmcnt left alone
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// 128-byte LDS rows: chunk c of row r sits at slot c ^ (r & 7) ^ ((r >> 3) & 1). A b128 read
// serves 16 lanes per pass; 16 consecutive rows read at one chunk land on 16 distinct 16-byte
// units of the 256-byte bank window (rows of one parity differ in the slot's low bits, the two
// parities sit 64 bytes apart, and bit 3 of the row flips the slot's lowest bit).
__device__ __forceinline__ int swz128(int row, int c) { return row * 128 + ((c ^ (row & 7) ^ ((row >> 3) & 1)) << 4); }

}  // namespace nhm
