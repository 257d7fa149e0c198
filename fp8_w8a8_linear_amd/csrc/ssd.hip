// Mamba2 chunked scan (SSD) on the gfx950 bf16 MFMA, one workgroup per (chunk, head).
//
// With cs_t = sum_{s<=t} dt_s * A inside a chunk of Q = 128 tokens (Dao & Gu 2024,
// "Transformers are SSMs", the state-space-duality split):
//   state kernel : S_c[p][n] = sum_s (exp(cs_end - cs_s) dt_s x_s[p]) B_s[n]
//   output kernel: G[t][s]  = (C_t . B_s) exp(cs_t - cs_s) dt_s   for s <= t
//                  y_t[p]   = sum_s G[t][s] x_s[p] + exp(cs_t) sum_n C_t[n] H_in[p][n] + D x_t[p]
// x, B and C are bf16 already (conv outputs) and enter the MFMA exactly. The
// decay-weighted operands (w_s x_s, G, H_in) are f32; each is split into
// bf16 hi + lo (hi = rne(v), lo = rne(v - hi), ~16 significant bits together) and
// contracted twice, keeping the f32 state well inside its 1e-3 bound where a
// single bf16 operand would not. Accumulation is f32.
//
// MFMA 16x16x32 bf16: lane l supplies row (l % 16) of A and column (l % 16) of B,
// each as the 8 k-values 8*(l/16) .. +7 of the 32-k step (any assignment shared
// by A and B gives the same dot products); the accumulator lane l, register r
// holds D[4*(l/16)+r][l%16]. Both operands must be k-contiguous in LDS: C and B
// are staged as stored ([token][state]); x and B^T are transposed while staging.
#include "nhm_device.h"
#include "nhm_internal.h"

namespace nhm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kHP = 64;    // head_dim
constexpr int kDS = 128;   // d_state
constexpr int kQ = 128;    // chunk length
constexpr int kLd = 136;   // LDS row stride in bf16 (272 bytes: 16-byte aligned, rows 8 apart spread over the banks)

__device__ __forceinline__ v4f mfma_bf16(const bf16x8& a, const bf16x8& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// v = hi + lo with hi = rne_bf16(v), lo = rne_bf16(v - hi)
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
    const uint32_t h = f32_to_bf16(v);
    hi = (uint16_t)h;
    lo = (uint16_t)f32_to_bf16(v - bf16_to_f32(h));
}

// dt_s = softplus(dt_raw + bias) and the inclusive scan cs_s of dt_s * A over the
// chunk (zero dt beyond L), in s_dt / s_cs; also stored for the other kernels.
__device__ __forceinline__ void chunk_decay(const PrefillArgs& a, int c, int h, int64_t tok0, int L, float* s_dt,
                                            float* s_cs) {
    const int t = threadIdx.x;
    const float A = -__expf(a.A_log[h]);
    if (t < kQ) {
        float dt = 0.f;
        if (t < L) dt = softplus(bf16_to_f32(a.zxbcdt[(tok0 + t) * a.d_in_proj + a.dt_off + h]) + a.dt_bias[h]);
        s_dt[t] = dt;
        s_cs[t] = dt * A;
    }
    __syncthreads();
    for (int o = 1; o < kQ; o <<= 1) {
        float add = 0.f;
        if (t < kQ && t >= o) add = s_cs[t - o];
        __syncthreads();
        if (t < kQ) s_cs[t] += add;
        __syncthreads();
    }
    if (t < kQ) {
        a.chunk_cs[((int64_t)c * a.n_heads + h) * kQ + t] = s_cs[t];
        a.chunk_dt[((int64_t)c * a.n_heads + h) * kQ + t] = s_dt[t];
    }
}

// ---------------------------------------------------------------- chunk states

__global__ __launch_bounds__(256) void ssd_state_kernel(const PrefillArgs a) {
    const int c = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    const int4 info = reinterpret_cast<const int4*>(a.chunk_info)[c];
    if (info.x < 0) return;
    const int64_t tok0 = info.y;
    const int L = info.z;
    const int g = h / (a.n_heads / a.n_groups);
    __shared__ float s_cs[kQ], s_dt[kQ];
    __shared__ __attribute__((aligned(16))) uint16_t s_xh[kHP * kLd];   // (w_s x_s)^T hi  [p][s]
    __shared__ __attribute__((aligned(16))) uint16_t s_xl[kHP * kLd];   // (w_s x_s)^T lo
    __shared__ __attribute__((aligned(16))) uint16_t s_bt[kDS * kLd];   // B^T [n][s]

    chunk_decay(a, c, h, tok0, L, s_dt, s_cs);
    __syncthreads();
    const float cs_end = s_cs[L - 1];
    for (int e = t; e < kQ * (kHP / 8); e += 256) {
        const int s = e >> 3, p8 = e & 7;
        float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (s < L) {
            unpack8(*reinterpret_cast<const uint4*>(a.xbc_conv + (tok0 + s) * a.conv_dim + h * kHP + p8 * 8), f);
            const float ws = __expf(cs_end - s_cs[s]) * s_dt[s];
#pragma unroll
            for (int j = 0; j < 8; ++j) f[j] *= ws;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) split_bf16(f[j], s_xh[(p8 * 8 + j) * kLd + s], s_xl[(p8 * 8 + j) * kLd + s]);
    }
    for (int e = t; e < kQ * (kDS / 8); e += 256) {
        const int s = e >> 4, n8 = e & 15;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (s < L) v = *reinterpret_cast<const uint4*>(a.xbc_conv + (tok0 + s) * a.conv_dim + a.b_off + g * kDS + n8 * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s_bt[(n8 * 8 + 2 * j) * kLd + s] = (uint16_t)(w[j] & 0xffffu);
            s_bt[(n8 * 8 + 2 * j + 1) * kLd + s] = (uint16_t)(w[j] >> 16);
        }
    }
    __syncthreads();

    // S[p][n]: 4 p-tiles x 8 n-tiles; wave w owns n-tiles 2w, 2w+1
    const int lane = t & 63, wave = t >> 6, r16 = lane & 15, q = lane >> 4;
    const int nks = (L + 31) / 32;
    v4f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][0] = acc[i][1] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < nks; ++ks) {
        const int koff = ks * 32 + q * 8;
        const bf16x8 b0 = lds8(&s_bt[(16 * (2 * wave) + r16) * kLd + koff]);
        const bf16x8 b1 = lds8(&s_bt[(16 * (2 * wave + 1) + r16) * kLd + koff]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x8 ah = lds8(&s_xh[(16 * i + r16) * kLd + koff]);
            const bf16x8 al = lds8(&s_xl[(16 * i + r16) * kLd + koff]);
            acc[i][0] = mfma_bf16(ah, b0, acc[i][0]);
            acc[i][0] = mfma_bf16(al, b0, acc[i][0]);
            acc[i][1] = mfma_bf16(ah, b1, acc[i][1]);
            acc[i][1] = mfma_bf16(al, b1, acc[i][1]);
        }
    }
    float* out = a.chunk_state + ((int64_t)c * a.n_heads + h) * kHP * kDS;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                out[(16 * i + 4 * q + r) * kDS + 16 * (2 * wave + jj) + r16] = acc[i][jj][r];
}

// ---------------------------------------------------------------- chunk outputs

__global__ __launch_bounds__(256) void ssd_out_kernel(const PrefillArgs a) {
    const int c = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    const int4 info = reinterpret_cast<const int4*>(a.chunk_info)[c];
    if (info.x < 0) return;
    const int64_t tok0 = info.y;
    const int L = info.z;
    const int g = h / (a.n_heads / a.n_groups);
    __shared__ float s_cs[kQ], s_dt[kQ];
    __shared__ __attribute__((aligned(16))) uint16_t s_c[kQ * kLd];        // C [t][n]
    __shared__ __attribute__((aligned(16))) uint16_t s_bh[kQ * kLd];       // B [s][n]; then H_in hi | lo [p][n]
    __shared__ __attribute__((aligned(16))) uint16_t s_xt[kHP * kLd];      // x^T [p][s]
    __shared__ __attribute__((aligned(16))) uint16_t s_gh[kQ * kLd];       // G hi [t][s]
    __shared__ __attribute__((aligned(16))) uint16_t s_gl[kQ * kLd];       // G lo [t][s]

    const float* cs_in = a.chunk_cs + ((int64_t)c * a.n_heads + h) * kQ;
    const float* dt_in = a.chunk_dt + ((int64_t)c * a.n_heads + h) * kQ;
    if (t < kQ) {
        s_cs[t] = cs_in[t];
        s_dt[t] = dt_in[t];
    }
    for (int e = t; e < kQ * (kDS / 8); e += 256) {
        const int s = e >> 4, n8 = e & 15;
        uint4 cv = make_uint4(0u, 0u, 0u, 0u), bv = cv;
        if (s < L) {
            const uint16_t* row = a.xbc_conv + (tok0 + s) * a.conv_dim + g * kDS + n8 * 8;
            bv = *reinterpret_cast<const uint4*>(row + a.b_off);
            cv = *reinterpret_cast<const uint4*>(row + a.c_off);
        }
        *reinterpret_cast<uint4*>(&s_bh[s * kLd + n8 * 8]) = bv;
        *reinterpret_cast<uint4*>(&s_c[s * kLd + n8 * 8]) = cv;
    }
    for (int e = t; e < kQ * (kHP / 8); e += 256) {
        const int s = e >> 3, p8 = e & 7;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (s < L) v = *reinterpret_cast<const uint4*>(a.xbc_conv + (tok0 + s) * a.conv_dim + h * kHP + p8 * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s_xt[(p8 * 8 + 2 * j) * kLd + s] = (uint16_t)(w[j] & 0xffffu);
            s_xt[(p8 * 8 + 2 * j + 1) * kLd + s] = (uint16_t)(w[j] >> 16);
        }
    }
    __syncthreads();

    const int lane = t & 63, wave = t >> 6, r16 = lane & 15, q = lane >> 4;
    // t-tiles {wave, 7 - wave}: equal shares of the lower triangle
    const int tt[2] = {wave, 7 - wave};

    // ---- G = (C B^T) * decay * dt on the lower triangle (plus the zero tile right of
    // the diagonal that the 32-wide k-steps of the next contraction reach)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int ti = tt[u];
        const int sj_end = ti + 1 < 7 ? ti + 1 : 7;
        for (int sj = 0; sj <= sj_end; ++sj) {
            v4f acc = {0.f, 0.f, 0.f, 0.f};
            if (sj <= ti) {
#pragma unroll
                for (int kn = 0; kn < kDS / 32; ++kn) {
                    const int koff = kn * 32 + q * 8;
                    acc = mfma_bf16(lds8(&s_c[(16 * ti + r16) * kLd + koff]), lds8(&s_bh[(16 * sj + r16) * kLd + koff]), acc);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = 16 * ti + 4 * q + r, sc = 16 * sj + r16;
                const float v = (sc <= tr && tr < L) ? acc[r] * __expf(s_cs[tr] - s_cs[sc]) * s_dt[sc] : 0.f;
                split_bf16(v, s_gh[tr * kLd + sc], s_gl[tr * kLd + sc]);
            }
        }
    }
    __syncthreads();

    // ---- H_in (the state entering this chunk, f32 [p][n]) -> hi | lo in place of B
    uint16_t* s_hh = s_bh;
    uint16_t* s_hl = s_bh + kHP * kLd;
    {
        const float4* hin = reinterpret_cast<const float4*>(a.chunk_state + ((int64_t)c * a.n_heads + h) * kHP * kDS);
        for (int e = t; e < kHP * kDS / 4; e += 256) {
            const int p = e >> 5, n4 = (e & 31) * 4;
            const float4 v = hin[e];
            uint16_t hi[4], lo[4];
            split_bf16(v.x, hi[0], lo[0]);
            split_bf16(v.y, hi[1], lo[1]);
            split_bf16(v.z, hi[2], lo[2]);
            split_bf16(v.w, hi[3], lo[3]);
            *reinterpret_cast<uint2*>(&s_hh[p * kLd + n4]) =
                make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
            *reinterpret_cast<uint2*>(&s_hl[p * kLd + n4]) =
                make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
        }
    }
    __syncthreads();

    // ---- y tiles: t-tiles {wave, 7 - wave} x 4 p-tiles
    const float Dh = a.D[h];
    const int nks_l = (L + 31) / 32;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int ti = tt[u];
        if (16 * ti >= L) continue;
        int nks = (16 * ti + 15) / 32 + 1;
        if (nks > nks_l) nks = nks_l;
        for (int pj = 0; pj < 4; ++pj) {
            v4f acc1 = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
            for (int ks = 0; ks < nks; ++ks) {
                const int koff = ks * 32 + q * 8;
                const bf16x8 xb = lds8(&s_xt[(16 * pj + r16) * kLd + koff]);
                acc1 = mfma_bf16(lds8(&s_gh[(16 * ti + r16) * kLd + koff]), xb, acc1);
                acc1 = mfma_bf16(lds8(&s_gl[(16 * ti + r16) * kLd + koff]), xb, acc1);
            }
#pragma unroll
            for (int kn = 0; kn < kDS / 32; ++kn) {
                const int koff = kn * 32 + q * 8;
                const bf16x8 ca = lds8(&s_c[(16 * ti + r16) * kLd + koff]);
                acc2 = mfma_bf16(ca, lds8(&s_hh[(16 * pj + r16) * kLd + koff]), acc2);
                acc2 = mfma_bf16(ca, lds8(&s_hl[(16 * pj + r16) * kLd + koff]), acc2);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = 16 * ti + 4 * q + r, pc = 16 * pj + r16;
                if (tr >= L) continue;
                const float xv = bf16_to_f32(s_xt[pc * kLd + tr]);
                const float yv = acc1[r] + __expf(s_cs[tr]) * acc2[r] + Dh * xv;
                a.y[(tok0 + tr) * a.d_inner + h * kHP + pc] = (uint16_t)f32_to_bf16(yv);
            }
        }
    }
}

void launch_ssd_state(const PrefillArgs& a, hipStream_t st) {
    ssd_state_kernel<<<dim3(a.max_chunks, a.n_heads), 256, 0, st>>>(a);
}

void launch_ssd_out(const PrefillArgs& a, hipStream_t st) {
    ssd_out_kernel<<<dim3(a.max_chunks, a.n_heads), 256, 0, st>>>(a);
}

}  // namespace nhm
