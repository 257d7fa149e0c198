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
// The state and output kernels (ssd.hip) run the contractions on the bf16 MFMA;
// the pass kernel below is a sequential f32 walk over the chunks of a sequence.
#include "nhm_device.h"
#include "nhm_internal.h"

namespace nhm {

constexpr int kHP = 64;    // head_dim
constexpr int kDS = 128;   // d_state
constexpr int kQ = 128;    // chunk length

// ---------------------------------------------------------------- chunk plan

// Chunk c -> (sequence, first token, length, index within the sequence);
// seq_chunk0[i] = first chunk of sequence i, seq_chunk0[n] = number of chunks.
// Run by one 256-thread block (the conv kernel's last block column, which the conv work
// does not use; nothing in the conv reads the plan).
__device__ __forceinline__ void plan_block(const int32_t* __restrict__ cu, int n, int Q, int max_chunks,
                                           int32_t* __restrict__ info, int32_t* __restrict__ seq_chunk0) {
    constexpr int kB = 256;
    __shared__ int s_scan[kB];
    const int t = threadIdx.x;
    int carry = 0;
    for (int base = 0; base < n; base += kB) {
        const int i = base + t;
        const int v = i < n ? (cu[i + 1] - cu[i] + Q - 1) / Q : 0;
        s_scan[t] = v;
        __syncthreads();
        for (int o = 1; o < kB; o <<= 1) {
            const int add = t >= o ? s_scan[t - o] : 0;
            __syncthreads();
            s_scan[t] += add;
            __syncthreads();
        }
        if (i < n) seq_chunk0[i] = carry + s_scan[t] - v;
        carry += s_scan[kB - 1];
        __syncthreads();
    }
    if (t == 0) seq_chunk0[n] = carry;
    __syncthreads();
    const int total = carry;
    for (int c = t; c < max_chunks; c += kB) {
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
// One launch for two independent jobs (neither reads what the other writes): block 0
// computes the chunk plan, the rest run the conv (channel blocks fastest).
__global__ __launch_bounds__(256) void conv_fwd_kernel(const PrefillArgs a, int c8_blocks) {
    const int64_t b = blockIdx.x;
    if (b == 0) {
        plan_block(a.cu_seqlens, a.n_seqs, a.chunk, a.max_chunks, a.chunk_info, a.seq_chunk0);
        return;
    }
    const int64_t cbk = b - 1;
    const int c8 = (int)(cbk % c8_blocks) * 256 + threadIdx.x;
    if (c8 * 8 >= a.conv_dim) return;
    const int64_t t0 = (cbk / c8_blocks) * kConvRun;
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
    // The run's rows are loaded before any is used (rows past T read row T - 1, unused): the
    // compiler cannot move a load above an earlier iteration's store, so loads inside the loop
    // would wait one memory latency per token.
    uint4 xr[kConvRun];
#pragma unroll
    for (int r = 0; r < kConvRun; ++r) {
        const int64_t tok = t0 + r < a.T ? t0 + r : a.T - 1;
        xr[r] = *reinterpret_cast<const uint4*>(src + tok * a.d_in_proj);
    }
    float u[3][8];
#pragma unroll
    for (int j = 1; j <= 3; ++j) {
        const int64_t tok = t0 - j;
        uint4 v = tok >= s0 ? *reinterpret_cast<const uint4*>(src + tok * a.d_in_proj)
                            : init_row(a, i, (int)(3 + tok - s0), c8);
        unpack8(v, u[3 - j]);
    }
    // the start of the next sequence, held in a register (a load in the loop would wait behind
    // the previous token's store)
    int64_t next = i < a.n_seqs - 1 ? a.cu_seqlens[i + 1] : INT64_MAX;
#pragma unroll
    for (int r = 0; r < kConvRun; ++r) {
        const int64_t tok = t0 + r;
        if (tok >= a.T) break;
        if (tok >= next) {   // the next non-empty sequence starts here
            while (i < a.n_seqs - 1 && tok >= a.cu_seqlens[i + 1]) ++i;
            next = i < a.n_seqs - 1 ? a.cu_seqlens[i + 1] : INT64_MAX;
#pragma unroll
            for (int j = 0; j < 3; ++j) unpack8(init_row(a, i, j, c8), u[j]);
        }
        float x[8];
        unpack8(xr[r], x);
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
// The carried window of sequence i after the call: the last 3 rows of [old window; tokens],
// 8 channels (c8 .. c8+7) per call. Runs after every conv read of the old window.
__device__ __forceinline__ void store_window(const PrefillArgs& a, int i, int c8) {
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

// One workgroup per (sequence, head, block of 8 state rows). Walks the sequence's
// chunks in order, replacing each S_c by the state entering chunk c, and leaves the
// final state in the pool row (read first, written last by this workgroup only).
// The first workgroups of each sequence also store its carried conv window (the conv
// kernel, which reads the old window, has finished by now).
// kBf16: a bf16 state pool, widened on the first read and rounded (nearest even) on the
// final write; the pass itself runs in f32.
template <bool kBf16>
__global__ __launch_bounds__(256) void ssd_pass_kernel(const PrefillArgs a) {
    const int i = blockIdx.x, h = blockIdx.y, pb = blockIdx.z, t = threadIdx.x;
    {
        const int c8 = (h * (kHP / 8) + pb) * 256 + t;      // 8-channel group of the window
        if (c8 * 8 < a.conv_dim) store_window(a, i, c8);
    }
    const int c0 = min(a.seq_chunk0[i], a.max_chunks), c1 = min(a.seq_chunk0[i + 1], a.max_chunks);
    const int64_t off = (int64_t)pb * 8 * kDS + 4 * t;
    const int64_t prow = ((int64_t)a.slot_idx[i] * a.n_heads + h) * kHP * kDS + off;
    float4* pool = reinterpret_cast<float4*>(a.ssm_pool + (kBf16 ? 0 : prow));
    uint2* pool16 = reinterpret_cast<uint2*>(a.ssm_pool_bf16 + (kBf16 ? prow : 0));
    float4 H = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.has_initial[i]) {
        if constexpr (kBf16) {
            const uint2 u = *pool16;
            H = make_float4(bf16_to_f32(u.x & 0xffffu), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xffffu),
                            bf16_to_f32(u.y >> 16));
        } else {
            H = *pool;
        }
    }
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
    if constexpr (kBf16)
        *pool16 = make_uint2(f32x2_to_bf16x2(H.x, H.y), f32x2_to_bf16x2(H.z, H.w));
    else
        *pool = H;
}

// ---------------------------------------------------------------- launcher

nhm_status launch_prefill_mid(const PrefillArgs& a, hipStream_t st) {
    const int c8_blocks = (a.conv_dim / 8 + 255) / 256;
    const int64_t tblocks = (a.T + kConvRun - 1) / kConvRun;
    conv_fwd_kernel<<<dim3((unsigned)(1 + c8_blocks * tblocks)), 256, 0, st>>>(a, c8_blocks);
    count_launch(Kern::kConvFwd, a.T);
    if (a.max_chunks > 0) launch_ssd_state(a, st);
    if (a.n_seqs > 0) {
        if (a.ssm_pool_bf16)
            ssd_pass_kernel<true><<<dim3(a.n_seqs, a.n_heads, kHP / 8), 256, 0, st>>>(a);
        else
            ssd_pass_kernel<false><<<dim3(a.n_seqs, a.n_heads, kHP / 8), 256, 0, st>>>(a);
        count_launch(Kern::kSsdPass, a.max_chunks);
    }
    if (a.max_chunks > 0) launch_ssd_out(a, st);
    nhm_status s = check_launch("prefill");
    if (s != NHM_OK || a.T == 0) return s;
    GnormArgs ga{a.T, a.n_groups, a.d_inner, a.d_in_proj, a.z_off, a.eps, a.y, a.zxbcdt, a.norm_w, a.out_a_scale,
                 a.norm, a.q_out};
    return launch_gnorm_quant(ga, st);
}

}  // namespace nhm
