// Mamba2 chunked scan (SSD) on the gfx950 bf16 MFMA, one workgroup per (chunk, head).
//
// With cs_t = sum_{s<=t} dt_s * A inside a chunk of Q = 128 tokens (Dao & Gu 2024,
// "Transformers are SSMs", the state-space-duality split):
//   state kernel : S_c[p][n] = sum_s (exp(cs_end - cs_s) dt_s x_s[p]) B_s[n]
//   output kernel: G[t][s]  = (C_t . B_s) exp(cs_t - cs_s) dt_s   for s <= t
//                  y_t[p]   = sum_s G[t][s] x_s[p] + exp(cs_t) sum_n C_t[n] H_in[p][n] + D x_t[p]
// x, B and C are bf16 already (conv outputs) and enter the MFMA exactly. The
// decay-weighted operands (w_s x_s, G, H_in) are f32; each is split into
// bf16 hi + lo (hi = rne(v), lo = rne(v - hi): ~16 significant bits together, with
// the hardware's packed f32 -> bf16 conversion) and contracted twice, keeping the
// f32 state well inside its 1e-3 bound where a single bf16 operand would not.
// Accumulation is f32.
//
// MFMA 16x16x32 bf16: lane l supplies row (l % 16) of A and column (l % 16) of B,
// each as 8 k-values chosen by l / 16 (any assignment shared by A and B gives the
// same dot products); the accumulator lane l, register r holds D[4*(l/16)+r][l%16].
// Operands must be k-contiguous per lane. C and B rows ([token][state]) and H_in
// ([p][n]) are; x and B^T (k = token) are transposed while staging into LDS, with
// consecutive lanes on consecutive tokens so the 2-byte LDS writes do not conflict.
#include "nhm_device.h"
#include "nhm_internal.h"

namespace nhm {

constexpr int kHP = 64;    // head_dim
constexpr int kDS = 128;   // d_state
constexpr int kQ = 128;    // chunk length
constexpr int kLd = 136;   // LDS row stride in bf16 (272 bytes: 16-byte aligned rows)
constexpr int kThreads = 512;

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// v = hi + lo, hi = rne_bf16(v), lo = rne_bf16(v - hi)
__device__ __forceinline__ void split_bf16(float v, __bf16& hi, __bf16& lo) {
    hi = (__bf16)v;
    lo = (__bf16)(v - (float)hi);
}

__device__ __forceinline__ uint16_t bits(__bf16 v) { return __builtin_bit_cast(uint16_t, v); }

// dt_s = softplus(dt_raw + bias) (zero beyond L) and the inclusive scan cs_s of dt_s * A
// over the chunk, in s_dt / s_cs, for the raw value u that thread s < Q loaded; also
// stored for the other kernels. Threads 0..127 are waves 0 and 1: each scans its 64
// values with DPP lane moves, then wave 1 adds wave 0's total. Ends with a barrier.
// u: the token's raw dt (bf16 widened); dt_bias, a_log: the head's parameters, loaded by the
// caller ahead of its bulk loads.
__device__ __forceinline__ void chunk_decay(const PrefillArgs& a, int c, int h, int L, float u, float dt_bias,
                                            float a_log, float* s_dt, float* s_cs) {
    const int t = threadIdx.x;
    __shared__ float s_w0;
    float dt = 0.f, v = 0.f;
    if (t < kQ) {
        dt = t < L ? softplus(u + dt_bias) : 0.f;
        v = wave_prefix_sum(dt * -__expf(a_log));
        if (t == 63) s_w0 = v;
    }
    __syncthreads();
    if (t < kQ) {
        if (t >= 64) v += s_w0;
        s_dt[t] = dt;
        s_cs[t] = v;
        a.chunk_cs[((int64_t)c * a.n_heads + h) * kQ + t] = v;
        a.chunk_dt[((int64_t)c * a.n_heads + h) * kQ + t] = dt;
    }
    __syncthreads();
}

// ---------------------------------------------------------------- chunk states

// Block -> (chunk, head) for the 1-D grid of max_chunks x n_heads blocks: the heads of a
// chunk are consecutive blocks, so they share the chunk's dt rows (one line holds every
// head's dt of a token) and B / C rows while those are in L2. Blocks go to the 8 XCDs round
// robin; with n_heads % 8 == 0 XCD x takes the contiguous heads x n_heads/8 .. + n_heads/8 - 1,
// whole groups when n_groups divides 8, so a group's B and C are fetched into one L2.
__device__ __forceinline__ void chunk_head(const PrefillArgs& a, int& c, int& h) {
    const int b = blockIdx.x, r = b % a.n_heads;
    c = b / a.n_heads;
    h = (a.n_heads & 7) ? r : (r & 7) * (a.n_heads >> 3) + (r >> 3);
}


// S_c = (w x)^T B with w_s = exp(cs_end - cs_s) dt_s. x^T and B^T are staged as they are
// (bf16, exact) with w in LDS; a wave forms its A operand w_s x_s[p] in f32 and splits it
// into bf16 hi + lo in registers. Wave w owns p-tile w % 4 and n-tiles 4 (w / 4) .. + 3, so
// each operand is formed once and serves four MFMA pairs. 53 KB of LDS: three workgroups
// share a CU.
__global__ __launch_bounds__(kThreads, 6) void ssd_state_kernel(const PrefillArgs a) {
    const int t = threadIdx.x;
    int c, h;
    chunk_head(a, c, h);
    const int4 info = reinterpret_cast<const int4*>(a.chunk_info)[c];
    if (info.x < 0) return;
    const int64_t tok0 = info.y;
    const int L = info.z;
    const int g = h / (a.n_heads / a.n_groups);
    __shared__ float s_cs[kQ], s_dt[kQ];
    __shared__ __attribute__((aligned(16))) float s_w[kQ];                // w_s, zero beyond L
    __shared__ __attribute__((aligned(16))) uint16_t s_xt[kHP * kLd];   // x^T [p][s]
    __shared__ __attribute__((aligned(16))) uint16_t s_bt[kDS * kLd];   // B^T [n][s]

    // All global loads first (rows past the chunk's end read its last row and are zeroed
    // when stored), then the decay scan, then the LDS stores. The scan's dt goes out first:
    // loads complete in issue order, so the scan waits for it alone and runs while the
    // staging loads are in flight.
    const int tr = t < L ? t : L - 1;
    const float u = bf16_to_f32(a.zxbcdt[(tok0 + tr) * a.d_in_proj + a.dt_off + h]);
    const float dt_bias = a.dt_bias[h], a_log = a.A_log[h];
    asm volatile("" ::: "memory");
    constexpr int kXI = kQ * (kHP / 8) / kThreads, kBI = kQ * (kDS / 8) / kThreads;
    uint4 xv[kXI], bv[kBI];
#pragma unroll
    for (int i = 0; i < kXI; ++i) {
        const int e = t + i * kThreads, s = e & (kQ - 1), p8 = e >> 7;
        xv[i] = *reinterpret_cast<const uint4*>(a.xbc_conv + (tok0 + (s < L ? s : L - 1)) * a.conv_dim + h * kHP + p8 * 8);
    }
#pragma unroll
    for (int i = 0; i < kBI; ++i) {
        const int e = t + i * kThreads, s = e & (kQ - 1), n8 = e >> 7;
        bv[i] = *reinterpret_cast<const uint4*>(a.xbc_conv + (tok0 + (s < L ? s : L - 1)) * a.conv_dim + a.b_off + g * kDS + n8 * 8);
    }
    chunk_decay(a, c, h, L, u, dt_bias, a_log, s_dt, s_cs);
    const float cs_end = s_cs[L - 1];
    if (t < kQ) s_w[t] = t < L ? __expf(cs_end - s_cs[t]) * s_dt[t] : 0.f;
#pragma unroll
    for (int i = 0; i < kXI; ++i) {
        const int e = t + i * kThreads, s = e & (kQ - 1), p8 = e >> 7;
        const uint4 v = s < L ? xv[i] : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s_xt[(p8 * 8 + 2 * j) * kLd + s] = (uint16_t)(w[j] & 0xffffu);
            s_xt[(p8 * 8 + 2 * j + 1) * kLd + s] = (uint16_t)(w[j] >> 16);
        }
    }
#pragma unroll
    for (int i = 0; i < kBI; ++i) {
        const int e = t + i * kThreads, s = e & (kQ - 1), n8 = e >> 7;
        const uint4 v = s < L ? bv[i] : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s_bt[(n8 * 8 + 2 * j) * kLd + s] = (uint16_t)(w[j] & 0xffffu);
            s_bt[(n8 * 8 + 2 * j + 1) * kLd + s] = (uint16_t)(w[j] >> 16);
        }
    }
    __syncthreads();

    const int lane = t & 63, wave = t >> 6, r16 = lane & 15, q = lane >> 4;
    const int pt = wave & 3, nt0 = (wave >> 2) * 4;
    const int nks = (L + 31) / 32;
    v4f acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < nks; ++ks) {
        const int koff = ks * 32 + q * 8;
        // A operand: w_s x_s[p] for p = 16 pt + r16 and the eight s at koff, split hi + lo
        const uint4 xr = *reinterpret_cast<const uint4*>(&s_xt[(16 * pt + r16) * kLd + koff]);
        const float4 w0 = *reinterpret_cast<const float4*>(&s_w[koff]);
        const float4 w1 = *reinterpret_cast<const float4*>(&s_w[koff + 4]);
        float f[8];
        unpack8(xr, f);
        const float ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        bf16x8 ah, al;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            __bf16 hi, lo;
            split_bf16(f[j] * ws[j], hi, lo);
            ah[j] = hi;
            al[j] = lo;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8 b = lds8(&s_bt[(16 * (nt0 + j) + r16) * kLd + koff]);
            acc[j] = mfma_bf16(ah, b, acc[j]);
            acc[j] = mfma_bf16(al, b, acc[j]);
        }
    }
    float* out = a.chunk_state + ((int64_t)c * a.n_heads + h) * kHP * kDS;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) out[(16 * pt + 4 * q + r) * kDS + 16 * (nt0 + j) + r16] = acc[j][r];
}

// ---------------------------------------------------------------- chunk outputs

// One workgroup of 8 waves per (chunk, head); wave w computes the output rows of
// t-tile w. B and x^T are staged once per workgroup for G.x; H_in (split hi | lo),
// loaded into registers at the start, then takes B's place in LDS for C.H_in^T, so a
// workgroup holds 53 KB and three share a CU. The C rows of a wave's t-tile are read
// from L2 into registers and serve as the B operand of C.B^T and the A operand of
// C.H_in^T. G never leaves registers: C.B^T is computed transposed (B as the A operand).
// B's rows are staged in a permuted order -- token 32 k + 8 q + 4 h + r of a 32-token block
// at row 32 k + 16 h + 4 q + r -- so that the accumulator lane (r16, q) of the two 16-row
// tiles h = 0, 1 of block k holds G for row t and the eight consecutive tokens
// 32 k + 8 q .. + 7: an A operand of G.x whose B operand, x^T for the same eight tokens, is
// one 16-byte LDS read. The result leaves through LDS (f32 rows, B's bytes once more), so each
// thread adds D x for eight channels of one token and stores them as one 16-byte piece.
__global__ __launch_bounds__(kThreads, 6) void ssd_out_kernel(const PrefillArgs a) {   // 6 waves per SIMD: 3 workgroups per CU
    const int t = threadIdx.x;
    int c, h;
    chunk_head(a, c, h);
    const int4 info = reinterpret_cast<const int4*>(a.chunk_info)[c];
    if (info.x < 0) return;
    const int64_t tok0 = info.y;
    const int L = info.z;
    const int g = h / (a.n_heads / a.n_groups);
    __shared__ float s_cs[kQ], s_dt[kQ];
    __shared__ __attribute__((aligned(16))) uint16_t s_xt[kHP * kLd];      // x^T [p][s]
    // B [s][n] for G x; afterwards the same bytes hold H_in hi and lo [p][n] for C H_in^T
    __shared__ __attribute__((aligned(16))) uint16_t s_b[kQ * kLd];
    static_assert(2 * kHP * kLd <= kQ * kLd, "H_in hi and lo fit where B was");
    uint16_t* const s_hh = s_b;
    uint16_t* const s_hl = s_b + kHP * kLd;

    const int lane = t & 63, wave = t >> 6, r16 = lane & 15, q = lane >> 4;
    const int ti = wave;
    const int trow = 16 * ti + r16;                   // this lane's row t
    const bool tok = trow < L;

    // Every global load of the staging, and this wave's C rows, is issued before the first
    // LDS store (a load-store loop would pay one memory latency per iteration). Rows past
    // the chunk's end are read from its last row (always in bounds) and zeroed.
    constexpr int kXI = kQ * (kHP / 8) / kThreads, kBI = kQ * (kDS / 8) / kThreads, kHI = kHP * kDS / 4 / kThreads;
    // the small cumulative-decay and dt rows first (loads complete in issue order: the staging
    // below then waits for each operand as it arrives, not for everything)
    const float* cs_in = a.chunk_cs + ((int64_t)c * a.n_heads + h) * kQ;
    const float* dt_in = a.chunk_dt + ((int64_t)c * a.n_heads + h) * kQ;
    const int tq = t & (kQ - 1);
    const float csv = cs_in[tq], dtv = dt_in[tq];
    asm volatile("" ::: "memory");
    uint4 xv[kXI], bv[kBI];
    float4 hv[kHI];
#pragma unroll
    for (int i = 0; i < kXI; ++i) {
        const int e = t + i * kThreads, s = e & (kQ - 1), p8 = e >> 7;
        xv[i] = *reinterpret_cast<const uint4*>(a.xbc_conv + (tok0 + (s < L ? s : L - 1)) * a.conv_dim + h * kHP + p8 * 8);
    }
#pragma unroll
    for (int i = 0; i < kBI; ++i) {
        const int e = t + i * kThreads, s = e >> 4, n8 = e & 15;
        bv[i] = *reinterpret_cast<const uint4*>(a.xbc_conv + (tok0 + (s < L ? s : L - 1)) * a.conv_dim + a.b_off + g * kDS + n8 * 8);
    }
    const float4* hin = reinterpret_cast<const float4*>(a.chunk_state + ((int64_t)c * a.n_heads + h) * kHP * kDS);
#pragma unroll
    for (int i = 0; i < kHI; ++i) hv[i] = hin[t + i * kThreads];
    const uint16_t* crow = a.xbc_conv + (tok0 + (tok ? trow : L - 1)) * a.conv_dim + a.c_off + g * kDS + q * 8;
    bf16x8 cop[kDS / 32];                             // C[t][k-step]
#pragma unroll
    for (int kn = 0; kn < kDS / 32; ++kn) cop[kn] = *reinterpret_cast<const bf16x8*>(crow + kn * 32);
    if (t < kQ) {
        s_cs[t] = csv;
        s_dt[t] = dtv;
    }
#pragma unroll
    for (int i = 0; i < kXI; ++i) {
        const int e = t + i * kThreads, s = e & (kQ - 1), p8 = e >> 7;
        const uint4 v = s < L ? xv[i] : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s_xt[(p8 * 8 + 2 * j) * kLd + s] = (uint16_t)(w[j] & 0xffffu);
            s_xt[(p8 * 8 + 2 * j + 1) * kLd + s] = (uint16_t)(w[j] >> 16);
        }
    }
#pragma unroll
    for (int i = 0; i < kBI; ++i) {
        const int e = t + i * kThreads, s = e >> 4, n8 = e & 15, u = s & 31;
        const int row = (s & ~31) + 16 * ((u >> 2) & 1) + 4 * (u >> 3) + (u & 3);
        *reinterpret_cast<uint4*>(&s_b[row * kLd + n8 * 8]) = s < L ? bv[i] : make_uint4(0u, 0u, 0u, 0u);
    }
    if (!tok) {
#pragma unroll
        for (int kn = 0; kn < kDS / 32; ++kn) cop[kn] = bf16x8{};
    }
    __syncthreads();
    const bool live = 16 * ti < L;                    // wave-uniform: this t-tile has rows
    const float cs_t = s_cs[trow];

    v4f acc1[4], acc2[4];
#pragma unroll
    for (int pj = 0; pj < 4; ++pj) acc1[pj] = acc2[pj] = v4f{0.f, 0.f, 0.f, 0.f};

    if (live) {
        // y1 = G x over the 32-token blocks kk with 32 kk <= 16 ti + 15 (both 16-row tiles of
        // a block hold tokens up to its end, so neither is skipped)
        const int nkk = (16 * ti + 15) / 32 + 1;
        for (int kk = 0; kk < nkk; ++kk) {
            float gv[8];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int sj = 2 * kk + half;               // LDS row tile
                v4f cb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kn = 0; kn < kDS / 32; ++kn)
                    cb = mfma_bf16(lds8(&s_b[(16 * sj + r16) * kLd + kn * 32 + q * 8]), cop[kn], cb);
                // cb[r] = (C.B^T)[t = trow][token sc]
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int sc = 32 * kk + 8 * q + 4 * half + r;
                    gv[4 * half + r] = (sc <= trow && tok) ? cb[r] * __expf(cs_t - s_cs[sc]) * s_dt[sc] : 0.f;
                }
            }
            bf16x8 gh, gl;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                __bf16 hi, lo;
                split_bf16(gv[j], hi, lo);
                gh[j] = hi;
                gl[j] = lo;
            }
            // B operand: x[s][p] for the same eight tokens, p = 16 pj + r16
#pragma unroll
            for (int pj = 0; pj < 4; ++pj) {
                const bf16x8 xb = lds8(&s_xt[(16 * pj + r16) * kLd + 32 * kk + 8 * q]);
                acc1[pj] = mfma_bf16(gh, xb, acc1[pj]);
                acc1[pj] = mfma_bf16(gl, xb, acc1[pj]);
            }
        }
    }
    __syncthreads();   // every wave is done with B
#pragma unroll
    for (int i = 0; i < kHI; ++i) {
        const int e = t + i * kThreads, p = e >> 5, n4 = (e & 31) * 4;
        const float4 v = hv[i];
        __bf16 hi[4], lo[4];
        split_bf16(v.x, hi[0], lo[0]);
        split_bf16(v.y, hi[1], lo[1]);
        split_bf16(v.z, hi[2], lo[2]);
        split_bf16(v.w, hi[3], lo[3]);
        *reinterpret_cast<uint2*>(&s_hh[p * kLd + n4]) =
            make_uint2(bits(hi[0]) | ((uint32_t)bits(hi[1]) << 16), bits(hi[2]) | ((uint32_t)bits(hi[3]) << 16));
        *reinterpret_cast<uint2*>(&s_hl[p * kLd + n4]) =
            make_uint2(bits(lo[0]) | ((uint32_t)bits(lo[1]) << 16), bits(lo[2]) | ((uint32_t)bits(lo[3]) << 16));
    }
    __syncthreads();
    // this thread's x for D x: token rows t / 8 and 64 + t / 8, channels 8 (t % 8) .. + 7 of the
    // head (rows past L read row L - 1 and are not stored)
    const int yc = 8 * (t & 7);
    uint4 xd[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = (t >> 3) + 64 * i;
        xd[i] = *reinterpret_cast<const uint4*>(a.xbc_conv + (tok0 + (row < L ? row : L - 1)) * a.conv_dim + h * kHP + yc);
    }
    if (live) {   // y2 = C H_in^T
#pragma unroll
        for (int pj = 0; pj < 4; ++pj) {
#pragma unroll
            for (int kn = 0; kn < kDS / 32; ++kn) {
                const int off = (16 * pj + r16) * kLd + kn * 32 + q * 8;
                acc2[pj] = mfma_bf16(cop[kn], lds8(&s_hh[off]), acc2[pj]);
                acc2[pj] = mfma_bf16(cop[kn], lds8(&s_hl[off]), acc2[pj]);
            }
        }
    }
    __syncthreads();   // every wave is done with H_in
    // acc[r] = Y[t = 16 ti + 4 q + r][p = 16 pj + r16]: G x + exp(cs_t) C H_in^T as f32 rows of
    // kYs floats in B's bytes
    constexpr int kYs = kHP + 4;
    static_assert(kQ * kYs * 4 <= kQ * kLd * 2, "the f32 result rows fit where B was");
    float* const s_y = reinterpret_cast<float*>(s_b);
    if (live) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tr = 16 * ti + 4 * q + r;
            const float e = __expf(s_cs[tr]);
#pragma unroll
            for (int pj = 0; pj < 4; ++pj) s_y[tr * kYs + 16 * pj + r16] = acc1[pj][r] + e * acc2[pj][r];
        }
    }
    __syncthreads();
    const float Dh = a.D[h];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = (t >> 3) + 64 * i;
        if (row >= L) continue;
        const float4 y0 = *reinterpret_cast<const float4*>(&s_y[row * kYs + yc]);
        const float4 y1 = *reinterpret_cast<const float4*>(&s_y[row * kYs + yc + 4]);
        float xf[8];
        unpack8(xd[i], xf);
        const float yv[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = f32_to_bf16(yv[2 * j] + Dh * xf[2 * j]) | (f32_to_bf16(yv[2 * j + 1] + Dh * xf[2 * j + 1]) << 16);
        *reinterpret_cast<uint4*>(a.y + (tok0 + row) * a.d_inner + h * kHP + yc) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

void launch_ssd_state(const PrefillArgs& a, hipStream_t st) {
    ssd_state_kernel<<<dim3((unsigned)(a.max_chunks * a.n_heads)), kThreads, 0, st>>>(a);
    count_launch(Kern::kSsdState, a.max_chunks);
}

void launch_ssd_out(const PrefillArgs& a, hipStream_t st) {
    ssd_out_kernel<<<dim3((unsigned)(a.max_chunks * a.n_heads)), kThreads, 0, st>>>(a);
    count_launch(Kern::kSsdOut, a.max_chunks);
}

}  // namespace nhm
