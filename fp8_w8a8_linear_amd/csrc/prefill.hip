// Prefill kernels between the two projections: varlen causal conv and the Mamba2
// chunked scan (state-space duality split).
//
// [PR1288] "What it does": in_proj -> split z | xBC | dt -> CausalConv1dFwd(silu)
// -> split x | B | C -> Mamba2ChunkScan -> RmsNormGatedGroup(n_groups) -> out_proj.
// The splits are column offsets into the projection rows; nothing is copied. The
// gated norm (norm.hip) follows the scan.
//
// Chunked scan (Dao & Gu 2024, "Transformers are SSMs", the SSD algorithm): chunks
// of Q tokens start at each sequence's first token. With cs_t the cumulative
// log-decay inside a chunk (sum of dt_s * A over s <= t),
//   state kernel : S_c = sum_s exp(cs_end - cs_s) dt_s x_s (x) B_s
//   pass kernel  : H_in(c) = state entering chunk c; H_in(c+1) = exp(cs_end) H_in(c) + S_c,
//                  seeded from the pool row (or zero) and written back in place
//   output kernel: y_t = sum_{s<=t} (C_t . B_s) exp(cs_t - cs_s) dt_s x_s
//                        + exp(cs_t) C_t . H_in(c) + D x_t
// All three run in f32 on the VALU with LDS-staged operands.
#include "nhm_device.h"
#include "nhm_internal.h"

namespace nhm {

constexpr int kHP = 64;    // head_dim
constexpr int kDS = 128;   // d_state
constexpr int kQ = 128;    // chunk length

// ---------------------------------------------------------------- chunk plan

// Chunk c -> (sequence, first token, length, index within the sequence);
// seq_chunk0[i] = first chunk of sequence i, seq_chunk0[n] = number of chunks.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ cu, int n, int Q,
                                                    int max_chunks, int32_t* __restrict__ info,
                                                    int32_t* __restrict__ seq_chunk0) {
    __shared__ int s_scan[1024];
    const int t = threadIdx.x;
    int carry = 0;
    for (int base = 0; base < n; base += 1024) {
        const int i = base + t;
        const int v = i < n ? (cu[i + 1] - cu[i] + Q - 1) / Q : 0;
        s_scan[t] = v;
        __syncthreads();
        for (int o = 1; o < 1024; o <<= 1) {
            const int add = t >= o ? s_scan[t - o] : 0;
            __syncthreads();
            s_scan[t] += add;
            __syncthreads();
        }
        if (i < n) seq_chunk0[i] = carry + s_scan[t] - v;
        carry += s_scan[1023];
        __syncthreads();
    }
    if (t == 0) seq_chunk0[n] = carry;
    __syncthreads();
    const int total = carry;
    for (int c = t; c < max_chunks; c += 1024) {
        int4 r = make_int4(-1, 0, 0, 0);
        if (c < total) {
            int lo = 0, hi = n - 1;            // last i with seq_chunk0[i] <= c
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (seq_chunk0[mid] <= c) lo = mid; else hi = mid - 1;
            }
            const int idx = c - seq_chunk0[lo];
            const int tok0 = cu[lo] + idx * Q;
            const int len = min(Q, cu[lo + 1] - tok0);
            r = make_int4(lo, tok0, len, idx);
        }
        reinterpret_cast<int4*>(info)[c] = r;
    }
}

// ---------------------------------------------------------------- causal conv

constexpr int kConvRun = 8;   // tokens per thread

__device__ __forceinline__ int seq_of(const int32_t* cu, int n, int64_t tok) {
    int lo = 0, hi = n - 1;               // last i with cu[i] <= tok
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= tok) lo = mid; else hi = mid - 1;
    }
    return lo;
}


// Window row r (0 = oldest) of sequence i before the call: the pool row or zero.
__device__ __forceinline__ uint4 init_row(const PrefillArgs& a, int i, int r, int c8) {
    if (!a.has_initial[i]) return make_uint4(0u, 0u, 0u, 0u);
    return *reinterpret_cast<const uint4*>(a.conv_pool + ((int64_t)a.slot_idx[i] * 3 + r) * a.conv_dim + c8 * 8);
}

// One thread: 8 channels x kConvRun consecutive tokens. The three previous rows
// come from the same sequence or, before its first token, from its initial window.
__global__ __launch_bounds__(256) void conv_fwd_kernel(const PrefillArgs a) {
    const int c8 = blockIdx.x * 256 + threadIdx.x;
    if (c8 * 8 >= a.conv_dim) return;
    const int64_t t0 = (int64_t)blockIdx.y * kConvRun;
    if (t0 >= a.T) return;
    const uint16_t* src = a.zxbcdt + a.xbc_off + c8 * 8;
    float w[8][4], bias[8];
    {
        const uint4* wp = reinterpret_cast<const uint4*>(a.conv_w + (int64_t)c8 * 8 * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {          // channels 2j, 2j+1
            float f[8];
            unpack8(wp[j], f);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                w[2 * j][k] = f[k];
                w[2 * j + 1][k] = f[4 + k];
            }
        }
        unpack8(*reinterpret_cast<const uint4*>(a.conv_b + c8 * 8), bias);
    }
    int i = seq_of(a.cu_seqlens, a.n_seqs, t0);
    int64_t s0 = a.cu_seqlens[i];
    float u[3][8];
#pragma unroll
    for (int j = 1; j <= 3; ++j) {
        const int64_t tok = t0 - j;
        uint4 v = tok >= s0 ? *reinterpret_cast<const uint4*>(src + tok * a.d_in_proj)
                            : init_row(a, i, (int)(3 + tok - s0), c8);
        unpack8(v, u[3 - j]);
    }
    for (int r = 0; r < kConvRun; ++r) {
        const int64_t tok = t0 + r;
        if (tok >= a.T) break;
        if (i < a.n_seqs - 1 && tok >= a.cu_seqlens[i + 1]) {   // the next non-empty sequence starts here
            while (i < a.n_seqs - 1 && tok >= a.cu_seqlens[i + 1]) ++i;
#pragma unroll
            for (int j = 0; j < 3; ++j) unpack8(init_row(a, i, j, c8), u[j]);
        }
        float x[8];
        unpack8(*reinterpret_cast<const uint4*>(src + tok * a.d_in_proj), x);
        uint32_t ob[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float pre = bias[c];
            pre = fmaf(w[c][0], u[0][c], pre);
            pre = fmaf(w[c][1], u[1][c], pre);
            pre = fmaf(w[c][2], u[2][c], pre);
            pre = fmaf(w[c][3], x[c], pre);
            ob[c] = f32_to_bf16(silu(pre));
            u[0][c] = u[1][c];
            u[1][c] = u[2][c];
            u[2][c] = x[c];
        }
        *reinterpret_cast<uint4*>(a.xbc_conv + tok * a.conv_dim + c8 * 8) =
            make_uint4(ob[0] | (ob[1] << 16), ob[2] | (ob[3] << 16), ob[4] | (ob[5] << 16), ob[6] | (ob[7] << 16));
    }
}

// New window of sequence i: the last three rows of [initial window; its tokens].
// Runs after conv_fwd_kernel has read every initial window.
__global__ __launch_bounds__(256) void conv_store_kernel(const PrefillArgs a) {
    const int c8 = blockIdx.x * 256 + threadIdx.x;
    const int i = blockIdx.y;
    if (c8 * 8 >= a.conv_dim) return;
    const int64_t s0 = a.cu_seqlens[i];
    const int64_t L = a.cu_seqlens[i + 1] - s0;
    uint4 v[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        const int64_t idx = L + r;             // position in [window (3 rows); tokens]
        v[r] = idx < 3 ? init_row(a, i, (int)idx, c8)
                       : *reinterpret_cast<const uint4*>(a.zxbcdt + (s0 + idx - 3) * a.d_in_proj + a.xbc_off + c8 * 8);
    }
    uint4* dst = reinterpret_cast<uint4*>(a.conv_pool + (int64_t)a.slot_idx[i] * 3 * a.conv_dim + c8 * 8);
#pragma unroll
    for (int r = 0; r < 3; ++r) dst[(int64_t)r * a.conv_dim / 8] = v[r];
}

// ---------------------------------------------------------------- SSD: chunk states

// One workgroup per (chunk, head): dt, cumulative log-decay and the chunk's own
// state contribution S_c[p][n] (zero initial state).
__global__ __launch_bounds__(256) void ssd_state_kernel(const PrefillArgs a) {
    const int c = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    const int4 info = reinterpret_cast<const int4*>(a.chunk_info)[c];
    if (info.x < 0) return;
    const int64_t tok0 = info.y;
    const int L = info.z;
    const int g = h / (a.n_heads / a.n_groups);
    __shared__ float s_cs[kQ], s_dt[kQ];
    __shared__ __attribute__((aligned(16))) float s_x[kQ][kHP];   // w_s * x_s
    __shared__ __attribute__((aligned(16))) float s_b[kQ][kDS];

    const float A = -__expf(a.A_log[h]);
    if (t < kQ) {
        float dt = 0.f;
        if (t < L) dt = softplus(bf16_to_f32(a.zxbcdt[(tok0 + t) * a.d_in_proj + a.dt_off + h]) + a.dt_bias[h]);
        s_dt[t] = dt;
        s_cs[t] = dt * A;
    }
    __syncthreads();
    for (int o = 1; o < kQ; o <<= 1) {        // inclusive scan of dt*A over the chunk
        float add = 0.f;
        if (t < kQ && t >= o) add = s_cs[t - o];
        __syncthreads();
        if (t < kQ) s_cs[t] += add;
        __syncthreads();
    }
    const float cs_end = s_cs[L - 1];
    float* cs_out = a.chunk_cs + ((int64_t)c * a.n_heads + h) * kQ;
    float* dt_out = a.chunk_dt + ((int64_t)c * a.n_heads + h) * kQ;
    if (t < kQ) {
        cs_out[t] = s_cs[t];
        dt_out[t] = s_dt[t];
    }
    // stage w_s x_s and B_s (zero rows beyond L)
    for (int e = t; e < kQ * kHP / 8; e += 256) {
        const int s = e / (kHP / 8), p8 = e % (kHP / 8);
        float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (s < L) {
            unpack8(*reinterpret_cast<const uint4*>(a.xbc_conv + (tok0 + s) * a.conv_dim + h * kHP + p8 * 8), f);
            const float ws = __expf(cs_end - s_cs[s]) * s_dt[s];
#pragma unroll
            for (int j = 0; j < 8; ++j) f[j] *= ws;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) s_x[s][p8 * 8 + j] = f[j];
    }
    for (int e = t; e < kQ * kDS / 8; e += 256) {
        const int s = e / (kDS / 8), n8 = e % (kDS / 8);
        float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (s < L) unpack8(*reinterpret_cast<const uint4*>(a.xbc_conv + (tok0 + s) * a.conv_dim + a.b_off + g * kDS + n8 * 8), f);
#pragma unroll
        for (int j = 0; j < 8; ++j) s_b[s][n8 * 8 + j] = f[j];
    }
    __syncthreads();
    // thread: p = 4*(t/16) .. +3, n = 8*(t%16) .. +7
    const int p0 = 4 * (t >> 4), n0 = 8 * (t & 15);
    float acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
    for (int s = 0; s < L; ++s) {
        const float4 xv = *reinterpret_cast<const float4*>(&s_x[s][p0]);
        const float4 b0 = *reinterpret_cast<const float4*>(&s_b[s][n0]);
        const float4 b1 = *reinterpret_cast<const float4*>(&s_b[s][n0 + 4]);
        const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
        const float bs[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(xs[i], bs[j], acc[i][j]);
    }
    float* out = a.chunk_state + ((int64_t)c * a.n_heads + h) * kHP * kDS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float4* o = reinterpret_cast<float4*>(out + (p0 + i) * kDS + n0);
        o[0] = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        o[1] = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
    }
}

// ---------------------------------------------------------------- SSD: state passing

// One workgroup per (sequence, head, block of 8 state rows). Walks the sequence's
// chunks in order, replacing each S_c by the state entering chunk c, and leaves the
// final state in the pool row (read first, written last by this workgroup only).
__global__ __launch_bounds__(256) void ssd_pass_kernel(const PrefillArgs a) {
    const int i = blockIdx.x, h = blockIdx.y, pb = blockIdx.z, t = threadIdx.x;
    const int c0 = min(a.seq_chunk0[i], a.max_chunks), c1 = min(a.seq_chunk0[i + 1], a.max_chunks);
    const int64_t off = (int64_t)pb * 8 * kDS + 4 * t;
    float4* pool = reinterpret_cast<float4*>(a.ssm_pool + ((int64_t)a.slot_idx[i] * a.n_heads + h) * kHP * kDS + off);
    float4 H = a.has_initial[i] ? *pool : make_float4(0.f, 0.f, 0.f, 0.f);
    const int64_t hstride = (int64_t)kHP * kDS;
    float4 S = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c0 < c1) S = *reinterpret_cast<const float4*>(a.chunk_state + ((int64_t)c0 * a.n_heads + h) * hstride + off);
    for (int c = c0; c < c1; ++c) {
        float4 Snext = S;
        if (c + 1 < c1)
            Snext = *reinterpret_cast<const float4*>(a.chunk_state + ((int64_t)(c + 1) * a.n_heads + h) * hstride + off);
        const int L = a.chunk_info[4 * c + 2];
        const float dec = __expf(a.chunk_cs[((int64_t)c * a.n_heads + h) * kQ + L - 1]);
        *reinterpret_cast<float4*>(a.chunk_state + ((int64_t)c * a.n_heads + h) * hstride + off) = H;
        H.x = fmaf(dec, H.x, S.x);
        H.y = fmaf(dec, H.y, S.y);
        H.z = fmaf(dec, H.z, S.z);
        H.w = fmaf(dec, H.w, S.w);
        S = Snext;
    }
    *pool = H;
}

// ---------------------------------------------------------------- SSD: chunk outputs

// LDS swizzles of the output kernel. Threads of a wave read rows that are 4 or 8
// apart; XOR-ing the 16-byte chunk index with the row's block index spreads
// those rows over the banks.
__device__ __forceinline__ int sw_bf(int row, int col) {      // bf16 [128][128]
    return row * kDS + ((((col >> 3) ^ (row >> 3)) & 15) << 3) + (col & 7);
}
__device__ __forceinline__ int sw_g(int row, int col) {       // f32 [128][128]
    return row * kQ + ((((col >> 2) ^ (row >> 3)) & 31) << 2) + (col & 3);
}
__device__ __forceinline__ int sw_h(int row, int col) {       // f32 [64][128]
    return row * kDS + ((((col >> 2) ^ (row >> 2)) & 31) << 2) + (col & 3);
}

// One workgroup per (chunk, head): y for the chunk's tokens.
__global__ __launch_bounds__(256) void ssd_out_kernel(const PrefillArgs a) {
    const int c = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    const int4 info = reinterpret_cast<const int4*>(a.chunk_info)[c];
    if (info.x < 0) return;
    const int64_t tok0 = info.y;
    const int L = info.z;
    const int g = h / (a.n_heads / a.n_groups);
    __shared__ __attribute__((aligned(16))) uint16_t s_c[kQ * kDS];       // C_t, bf16 (sw_bf)
    __shared__ __attribute__((aligned(16))) float s_bh[kQ * kDS / 2];     // B_s bf16 (sw_bf), then H_in f32 (sw_h)
    __shared__ __attribute__((aligned(16))) float s_g[kQ * kQ];           // decayed, masked C.B * dt (sw_g)
    __shared__ __attribute__((aligned(16))) uint16_t s_x[kQ][kHP];
    __shared__ float s_cs[kQ], s_dt[kQ];
    uint16_t* s_b = reinterpret_cast<uint16_t*>(s_bh);

    const float* cs_in = a.chunk_cs + ((int64_t)c * a.n_heads + h) * kQ;
    const float* dt_in = a.chunk_dt + ((int64_t)c * a.n_heads + h) * kQ;
    if (t < kQ) {
        s_cs[t] = t < L ? cs_in[t] : 0.f;
        s_dt[t] = t < L ? dt_in[t] : 0.f;
    }
    for (int e = t; e < kQ * kDS / 8; e += 256) {
        const int s = e / (kDS / 8), n8 = e % (kDS / 8);
        uint4 cv = make_uint4(0u, 0u, 0u, 0u), bv = cv;
        if (s < L) {
            const uint16_t* row = a.xbc_conv + (tok0 + s) * a.conv_dim + g * kDS + n8 * 8;
            bv = *reinterpret_cast<const uint4*>(row + a.b_off);
            cv = *reinterpret_cast<const uint4*>(row + a.c_off);
        }
        *reinterpret_cast<uint4*>(&s_b[sw_bf(s, n8 * 8)]) = bv;
        *reinterpret_cast<uint4*>(&s_c[sw_bf(s, n8 * 8)]) = cv;
    }
    for (int e = t; e < kQ * kHP / 8; e += 256) {
        const int s = e / (kHP / 8), p8 = e % (kHP / 8);
        uint4 xv = make_uint4(0u, 0u, 0u, 0u);
        if (s < L) xv = *reinterpret_cast<const uint4*>(a.xbc_conv + (tok0 + s) * a.conv_dim + h * kHP + p8 * 8);
        *reinterpret_cast<uint4*>(&s_x[s][p8 * 8]) = xv;
    }
    __syncthreads();

    // G[t][s] for t in 8*(t/16).., s in 8*(t%16)..
    {
        const int tb = 8 * (t >> 4), sb = 8 * (t & 15);
        float acc[8][8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
        if (sb <= tb + 7) {
            for (int n2 = 0; n2 < kDS / 2; ++n2) {      // two state columns per step
                uint32_t cw[8], bw[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) cw[i] = *reinterpret_cast<const uint32_t*>(&s_c[sw_bf(tb + i, 2 * n2)]);
#pragma unroll
                for (int j = 0; j < 8; ++j) bw[j] = *reinterpret_cast<const uint32_t*>(&s_b[sw_bf(sb + j, 2 * n2)]);
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    float cf[8], bf[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) cf[i] = bf16_to_f32(k ? cw[i] >> 16 : cw[i] & 0xffffu);
#pragma unroll
                    for (int j = 0; j < 8; ++j) bf[j] = bf16_to_f32(k ? bw[j] >> 16 : bw[j] & 0xffffu);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
#pragma unroll
                        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(cf[i], bf[j], acc[i][j]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tt = tb + i;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int ss = sb + j;
                s_g[sw_g(tt, ss)] = (ss <= tt) ? acc[i][j] * __expf(s_cs[tt] - s_cs[ss]) * s_dt[ss] : 0.f;
            }
        }
    }
    __syncthreads();
    // H_in(c) replaces B in LDS
    {
        const float4* hin = reinterpret_cast<const float4*>(a.chunk_state + ((int64_t)c * a.n_heads + h) * kHP * kDS);
        for (int e = t; e < kHP * kDS / 4; e += 256)
            *reinterpret_cast<float4*>(&s_bh[sw_h(e / (kDS / 4), (e % (kDS / 4)) * 4)]) = hin[e];
    }
    __syncthreads();

    // y[t][p] for t in 8*(t/16).., p in 4*(t%16)..
    const int tb = 8 * (t >> 4), p0 = 4 * (t & 15);
    float acc1[8][4], acc2[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc1[i][j] = acc2[i][j] = 0.f;
    const int smax = min(tb + 8, L);
    for (int s = 0; s < smax; s += 4) {
        float gv[8][4];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 v = *reinterpret_cast<const float4*>(&s_g[sw_g(tb + i, s)]);
            gv[i][0] = v.x; gv[i][1] = v.y; gv[i][2] = v.z; gv[i][3] = v.w;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint2 xv = *reinterpret_cast<const uint2*>(&s_x[s + k][p0]);
            const float xs[4] = {bf16_to_f32(xv.x & 0xffffu), bf16_to_f32(xv.x >> 16), bf16_to_f32(xv.y & 0xffffu),
                                 bf16_to_f32(xv.y >> 16)};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc1[i][j] = fmaf(gv[i][k], xs[j], acc1[i][j]);
        }
    }
    for (int n8 = 0; n8 < kDS / 8; ++n8) {
        float cf[8][8];
#pragma unroll
        for (int i = 0; i < 8; ++i) unpack8(*reinterpret_cast<const uint4*>(&s_c[sw_bf(tb + i, n8 * 8)]), cf[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 h0 = *reinterpret_cast<const float4*>(&s_bh[sw_h(p0 + j, n8 * 8)]);
            const float4 h1 = *reinterpret_cast<const float4*>(&s_bh[sw_h(p0 + j, n8 * 8 + 4)]);
            const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int k = 0; k < 8; ++k) acc2[i][j] = fmaf(cf[i][k], hv[k], acc2[i][j]);
        }
    }
    const float Dh = a.D[h];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int tt = tb + i;
        if (tt >= L) break;
        const float e = __expf(s_cs[tt]);
        const uint2 xv = *reinterpret_cast<const uint2*>(&s_x[tt][p0]);
        const float xs[4] = {bf16_to_f32(xv.x & 0xffffu), bf16_to_f32(xv.x >> 16), bf16_to_f32(xv.y & 0xffffu),
                             bf16_to_f32(xv.y >> 16)};
        uint32_t ob[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) ob[j] = f32_to_bf16(acc1[i][j] + e * acc2[i][j] + Dh * xs[j]);
        *reinterpret_cast<uint2*>(a.y + (tok0 + tt) * a.d_inner + h * kHP + p0) =
            make_uint2(ob[0] | (ob[1] << 16), ob[2] | (ob[3] << 16));
    }
}

// ---------------------------------------------------------------- launcher

nhm_status launch_prefill_mid(const PrefillArgs& a, hipStream_t st) {
    plan_kernel<<<1, 1024, 0, st>>>(a.cu_seqlens, a.n_seqs, a.chunk, a.max_chunks, a.chunk_info, a.seq_chunk0);
    const int c8_blocks = (a.conv_dim / 8 + 255) / 256;
    if (a.T > 0)
        conv_fwd_kernel<<<dim3(c8_blocks, (unsigned)((a.T + kConvRun - 1) / kConvRun)), 256, 0, st>>>(a);
    if (a.n_seqs > 0) conv_store_kernel<<<dim3(c8_blocks, a.n_seqs), 256, 0, st>>>(a);
    if (a.max_chunks > 0) ssd_state_kernel<<<dim3(a.max_chunks, a.n_heads), 256, 0, st>>>(a);
    if (a.n_seqs > 0) ssd_pass_kernel<<<dim3(a.n_seqs, a.n_heads, kHP / 8), 256, 0, st>>>(a);
    if (a.max_chunks > 0) ssd_out_kernel<<<dim3(a.max_chunks, a.n_heads), 256, 0, st>>>(a);
    nhm_status s = check_launch("prefill");
    if (s != NHM_OK || a.T == 0) return s;
    GnormArgs ga{a.T, a.n_groups, a.d_inner, a.d_in_proj, a.z_off, a.eps, a.y, a.zxbcdt, a.norm_w, a.out_a_scale,
                 a.norm, a.q_out};
    return launch_gnorm_quant(ga, st);
}

}  // namespace nhm
