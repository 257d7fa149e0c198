// libnhm C ABI: host-side validation, workspace layout and the launch order of
// the mixer block. Nothing here allocates, caches or synchronizes.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>

#include "nhm_device.h"
#include "nhm_internal.h"

namespace nhm {

static thread_local char g_err[512] = "";

nhm_status fail(nhm_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

static const char* const kKernNames[(int)Kern::kCount] = {
    "quant_vec8", "quant_scalar", "dequant_channel", "gemv", "gemm_ring192x128", "gemm_ring192x128_exact",
    "gemm_ring256x128", "gemm_ring256x128_exact", "gemm_ring256x256", "gemm_ring256x256_exact", "gemm_panel64x128",
    "gemm_panel64x128_exact", "gemm_tile128", "gemm_tile128_exact", "gemm_splitk_reduce", "decode_ssm",
    "gnorm_quant", "clear", "conv_fwd", "ssd_state", "ssd_pass", "ssd_out"};
static std::atomic<uint64_t> g_launches[(int)Kern::kCount];
static std::atomic<uint64_t> g_rows[(int)Kern::kCount];

void count_launch(Kern k, int64_t rows) {
    g_launches[(int)k].fetch_add(1, std::memory_order_relaxed);
    g_rows[(int)k].fetch_add((uint64_t)(rows > 0 ? rows : 0), std::memory_order_relaxed);
}

nhm_status check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(NHM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return NHM_OK;
}

static bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

static nhm_status check_geometry(const nhm_geometry* g) {
    if (!g) return fail(NHM_ERR_NULL, "geometry is NULL");
    if (g->hidden <= 0 || g->n_heads <= 0 || g->n_groups <= 0)
        return fail(NHM_ERR_UNSUPPORTED, "hidden, n_heads and n_groups must be positive");
    if (g->head_dim != 64 || g->d_state != 128 || g->conv_width != 4)
        return fail(NHM_ERR_UNSUPPORTED, "kernels implement head_dim 64, d_state 128, conv_width 4 (got %d, %d, %d)",
                    g->head_dim, g->d_state, g->conv_width);
    if (g->n_heads % g->n_groups != 0)
        return fail(NHM_ERR_UNSUPPORTED, "n_heads %d is not a multiple of n_groups %d", g->n_heads, g->n_groups);
    // in_proj rows are d_in_proj = 64 n_heads + conv_dim + n_heads bf16 wide and are read
    // 16 bytes at a time, which needs d_in_proj % 8 == 0, i.e. n_heads % 8 == 0
    if (g->n_heads % 8 != 0)
        return fail(NHM_ERR_UNSUPPORTED, "n_heads %d must be a multiple of 8 (16-byte in_proj rows)", g->n_heads);
    if (g->hidden % 16 != 0 || g->hidden > 16384)
        return fail(NHM_ERR_UNSUPPORTED, "hidden %d must be a multiple of 16 and at most 16384", g->hidden);
    if (!(g->rms_eps > 0.f) || !isfinite(g->rms_eps))
        return fail(NHM_ERR_UNSUPPORTED, "rms_eps must be finite and > 0 (got %g)", (double)g->rms_eps);
    return NHM_OK;
}

static void fill_layout(const nhm_geometry* g, nhm_layout* l) {
    const int32_t inner = g->n_heads * g->head_dim;
    const int32_t gs = g->n_groups * g->d_state;
    l->d_inner = inner;
    l->conv_dim = inner + 2 * gs;
    l->d_in_proj = inner + l->conv_dim + g->n_heads;
    l->z_off = 0;
    l->z_width = inner;
    l->xbc_off = inner;
    l->xbc_width = l->conv_dim;
    l->dt_off = inner + l->conv_dim;
    l->dt_width = g->n_heads;
    l->x_off = 0;
    l->x_width = inner;
    l->b_off = inner;
    l->b_width = gs;
    l->c_off = inner + gs;
    l->c_width = gs;
    l->heads_per_group = g->n_heads / g->n_groups;
    l->norm_group = inner / g->n_groups;
}

static nhm_status check_weight(const nhm_fp8_weight* w, int64_t n, int64_t k, const char* name) {
    if (!w->w || !w->w_scale || !w->a_scale) return fail(NHM_ERR_NULL, "%s: NULL weight, w_scale or a_scale", name);
    if (w->n != n || w->k != k)
        return fail(NHM_ERR_SHAPE, "%s: weight is [%lld, %lld], expected [%lld, %lld] ([out, in])", name,
                    (long long)w->n, (long long)w->k, (long long)n, (long long)k);
    if (!aligned(w->w, 16) || !aligned(w->w_scale, 4) || !aligned(w->a_scale, 4))
        return fail(NHM_ERR_ALIGN, "%s: weight must be 16-byte aligned, scales 4-byte aligned", name);
    if (w->w_scale_per_tensor != 0 && w->w_scale_per_tensor != 1)
        return fail(NHM_ERR_UNSUPPORTED, "%s: w_scale_per_tensor %d: 0 (per channel) or 1 (per tensor)", name,
                    (int)w->w_scale_per_tensor);
    return NHM_OK;
}

// Index step of the weight scale: per channel (w_scale[n]) or one scale for every channel.
static int ws_step(const nhm_fp8_weight& w) { return w.w_scale_per_tensor ? 0 : 1; }

// ---------------------------------------------------------------- workspace layouts

// bytes of the e4m3 copy of a bf16 activation (the only workspace nhm_fp8_linear needs)
// The weight-streaming GEMV serves m <= 16 (k up to 16384, weights under 2 GiB: its buffer
// descriptors take 32-bit offsets); the tiled GEMM the rest.
static bool use_gemv(int64_t m, int64_t n, int64_t k) { return m <= 16 && k <= 16384 && n * k < (int64_t(1) << 31); }

// Every kernel addresses its operands through buffer descriptors with 32-bit offsets: an
// operand of 2 GiB or more is refused on the host before anything is enqueued.
static nhm_status check_offsets(int64_t m, int64_t lda, int64_t n, int64_t k, const char* what) {
    if (n * k >= (int64_t(1) << 31) || m * lda >= (int64_t(1) << 31))
        return fail(NHM_ERR_UNSUPPORTED, "%s: an operand of 2 GiB or more ([%lld, %lld] weight, %lld x %lld activation)",
                    what, (long long)n, (long long)k, (long long)m, (long long)lda);
    return NHM_OK;
}

// Split-k partials of one projection: none where the GEMV runs.
static size_t proj_part_bytes(int64_t m, int64_t n, int64_t k) { return use_gemv(m, n, k) ? 0 : gemm_part_bytes(m, n, k); }

// The linear's workspace: the activation codes of a bf16 input (required), then the split-k
// partials of the shapes that take a split (optional: without them those shapes run unsplit).
static size_t linear_codes_ws(int64_t m, int64_t k, nhm_dtype t) {
    return t == NHM_BF16 ? align_up((size_t)m * (size_t)k, 256) : 0;
}
static size_t linear_ws(int64_t m, int64_t n, int64_t k, nhm_dtype t) {
    return linear_codes_ws(m, k, t) + align_up(proj_part_bytes(m, n, k), 256);
}

struct MixerWs {
    nhm_ws_layout pub;
    size_t chunk_info, seq_chunk0, chunk_cs, chunk_dt, chunk_state;
    size_t part, part_bytes;   // split-k partials of the projections (prefill)
    size_t cnt;                // decode: the fused norm's hand-off counters, one per (row, group)
    int max_chunks;
};

// The decode state kernel computes the gated norm itself (the last of a group's head workgroups
// takes the group) where a group is at most 512 channels, one pair per thread.
static bool decode_fused_norm(const nhm_geometry* g) { return (g->n_heads / g->n_groups) * g->head_dim <= 512; }

static MixerWs decode_ws(const nhm_geometry* g, int32_t batch) {
    nhm_layout l;
    fill_layout(g, &l);
    MixerWs w{};
    const size_t B = (size_t)batch;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes, 256); return o; };
    w.pub.q_in = take(B * g->hidden);
    w.pub.zxbcdt = take(B * l.d_in_proj * 2);
    w.pub.xbc_conv = take(B * l.conv_dim * 2);
    w.pub.y = take(B * l.d_inner * 2);
    w.pub.norm = take(B * l.d_inner * 2);
    w.pub.q_out = take(B * l.d_inner);
    // above 32 rows both projections run as GEMMs (split-k partials where a narrow shape asks)
    w.part_bytes = batch > 32 ? std::max(proj_part_bytes(batch, l.d_in_proj, g->hidden),
                                         proj_part_bytes(batch, g->hidden, l.d_inner))
                              : 0;
    w.part = take(w.part_bytes);
    w.cnt = take(decode_fused_norm(g) ? B * g->n_groups * sizeof(uint32_t) : 0);
    w.pub.total = off;
    return w;
}

static MixerWs prefill_ws(const nhm_geometry* g, int64_t T, int32_t n, int32_t chunk) {
    nhm_layout l;
    fill_layout(g, &l);
    MixerWs w{};
    const size_t Ts = (size_t)T;
    w.max_chunks = (int)(T / chunk + n);
    const size_t C = (size_t)w.max_chunks;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes, 256); return o; };
    w.pub.q_in = take(Ts * g->hidden);
    w.pub.zxbcdt = take(Ts * l.d_in_proj * 2);
    w.pub.xbc_conv = take(Ts * l.conv_dim * 2);
    w.chunk_info = take(C * 4 * sizeof(int32_t));
    w.seq_chunk0 = take(((size_t)n + 1) * sizeof(int32_t));
    w.chunk_cs = take(C * g->n_heads * chunk * sizeof(float));
    w.chunk_dt = take(C * g->n_heads * chunk * sizeof(float));
    w.chunk_state = take(C * g->n_heads * g->head_dim * g->d_state * sizeof(float));
    w.pub.y = take(Ts * l.d_inner * 2);
    w.pub.norm = take(Ts * l.d_inner * 2);
    w.pub.q_out = take(Ts * l.d_inner);
    w.part_bytes = std::max(proj_part_bytes(T, l.d_in_proj, g->hidden), proj_part_bytes(T, g->hidden, l.d_inner));
    w.part = take(w.part_bytes);
    w.pub.total = off;
    return w;
}


// One projection on an e4m3 activation [m, lda]; out_f32 non-null: f32 output instead of out.
// part / part_bytes: scratch for the GEMM's split-k partials (nullptr: no split).
// exact: every product summed in f32 on the tiled path too (the GEMV always is).
// out_q: also the e4m3 codes of the bf16 output under *q_scale (GEMV path only; callers of the
// tiled path quantize its output themselves).
static nhm_status project(const uint8_t* a, int64_t lda, int64_t m, const nhm_fp8_weight& w, uint16_t* out,
                          int64_t ld_out, hipStream_t st, float* out_f32 = nullptr, float* part = nullptr,
                          size_t part_bytes = 0, bool exact = false, uint8_t* out_q = nullptr, int64_t ld_q = 0,
                          const float* q_scale = nullptr) {
    if (use_gemv(m, w.n, w.k))
        return launch_gemv(a, lda, (int)m, w.w, w.w_scale, w.a_scale, w.n, w.k, out, ld_out, st, out_f32, out_q, ld_q,
                           q_scale, nullptr, 0, ws_step(w));
    return launch_gemm(a, lda, m, w.w, w.w_scale, w.a_scale, w.n, w.k, out, ld_out, st, out_f32, part, part_bytes,
                       exact, ws_step(w));
}

static nhm_status check_params(const nhm_mixer_params* p, nhm_layout* l) {
    if (!p) return fail(NHM_ERR_NULL, "params is NULL");
    nhm_status s = check_geometry(&p->g);
    if (s != NHM_OK) return s;
    fill_layout(&p->g, l);
    if ((s = check_weight(&p->in_proj, l->d_in_proj, p->g.hidden, "in_proj")) != NHM_OK) return s;
    if ((s = check_weight(&p->out_proj, p->g.hidden, l->d_inner, "out_proj")) != NHM_OK) return s;
    if (!p->conv_w || !p->conv_b || !p->norm_w || !p->A_log || !p->D || !p->dt_bias)
        return fail(NHM_ERR_NULL, "a block parameter pointer is NULL");
    if (!aligned(p->conv_w, 16) || !aligned(p->conv_b, 16) || !aligned(p->norm_w, 16) || !aligned(p->A_log, 4) ||
        !aligned(p->D, 4) || !aligned(p->dt_bias, 4))
        return fail(NHM_ERR_ALIGN, "conv_w, conv_b and norm_w must be 16-byte aligned, f32 params 4-byte aligned");
    return NHM_OK;
}

}  // namespace nhm

using namespace nhm;

extern "C" {

const char* nhm_status_str(nhm_status s) {
    switch (s) {
        case NHM_OK: return "NHM_OK";
        case NHM_ERR_NULL: return "NHM_ERR_NULL";
        case NHM_ERR_SHAPE: return "NHM_ERR_SHAPE";
        case NHM_ERR_ALIGN: return "NHM_ERR_ALIGN";
        case NHM_ERR_UNSUPPORTED: return "NHM_ERR_UNSUPPORTED";
        case NHM_ERR_WORKSPACE: return "NHM_ERR_WORKSPACE";
        case NHM_ERR_HIP: return "NHM_ERR_HIP";
    }
    return "NHM_ERR_UNKNOWN";
}

const char* nhm_last_error(void) { return g_err; }

const char* nhm_build_arch(void) { return "gfx950"; }

int32_t nhm_dispatch_counters(nhm_dispatch_counter* out, int32_t max, int32_t reset) {
    const int32_t n = (int32_t)Kern::kCount;
    for (int32_t i = 0; i < n; ++i) {
        const uint64_t l = reset ? g_launches[i].exchange(0, std::memory_order_relaxed)
                                 : g_launches[i].load(std::memory_order_relaxed);
        const uint64_t r = reset ? g_rows[i].exchange(0, std::memory_order_relaxed) : g_rows[i].load(std::memory_order_relaxed);
        if (out && i < max) out[i] = nhm_dispatch_counter{kKernNames[i], l, r};
    }
    return n;
}

nhm_status nhm_mixer_layout(const nhm_geometry* g, nhm_layout* out) {
    g_err[0] = 0;
    if (!out) return fail(NHM_ERR_NULL, "layout output is NULL");
    nhm_status s = check_geometry(g);
    if (s != NHM_OK) return s;
    fill_layout(g, out);
    return NHM_OK;
}

nhm_status nhm_fp8_quantize_static(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, const float* scale,
                                   uint8_t* q, int64_t ld_q, void* stream) {
    g_err[0] = 0;
    if (rows < 0 || cols < 0) return fail(NHM_ERR_SHAPE, "negative rows/cols (%lld, %lld)", (long long)rows, (long long)cols);
    if (rows == 0 || cols == 0) return NHM_OK;
    if (!x || !scale || !q) return fail(NHM_ERR_NULL, "x, scale or q is NULL");
    if (ld_x < cols || ld_q < cols)
        return fail(NHM_ERR_SHAPE, "leading dimensions (%lld, %lld) smaller than cols %lld", (long long)ld_x,
                    (long long)ld_q, (long long)cols);
    if (!aligned(x, 2) || !aligned(scale, 4)) return fail(NHM_ERR_ALIGN, "x must be 2-byte, scale 4-byte aligned");
    launch_quantize(x, rows, cols, ld_x, scale, q, ld_q, (hipStream_t)stream);
    return check_launch("quantize_static");
}

nhm_status nhm_fp8_dequant_channel_bf16(const uint8_t* w, const float* w_scale, int64_t n, int64_t k, int64_t ld_w,
                                        uint16_t* out, int64_t ld_out, void* stream) {
    g_err[0] = 0;
    if (n < 0 || k < 0) return fail(NHM_ERR_SHAPE, "negative n/k (%lld, %lld)", (long long)n, (long long)k);
    if (n == 0 || k == 0) return NHM_OK;
    if (!w || !w_scale || !out) return fail(NHM_ERR_NULL, "w, w_scale or out is NULL");
    if (k % 16 != 0 || ld_w < k || ld_out < k)
        return fail(NHM_ERR_SHAPE, "k %lld must be a multiple of 16 and ld_w %lld, ld_out %lld >= k", (long long)k,
                    (long long)ld_w, (long long)ld_out);
    if (!aligned(w, 16) || !aligned(out, 16) || !aligned(w_scale, 4) || ld_w % 16 != 0 || ld_out % 8 != 0)
        return fail(NHM_ERR_ALIGN, "w and out must be 16-byte aligned with 16-byte row strides");
    launch_dequant_channel(w, n, k, ld_w, w_scale, out, ld_out, (hipStream_t)stream);
    return check_launch("dequant_channel_bf16");
}

size_t nhm_fp8_linear_workspace_bytes(int64_t m, int64_t n, int64_t k, nhm_dtype a_type) {
    if (m <= 0 || n <= 0 || k <= 0) return 0;
    return linear_ws(m, n, k, a_type);
}

nhm_status nhm_fp8_linear(const void* a, nhm_dtype a_type, int64_t m, int64_t ld_a, const nhm_fp8_weight* w,
                          uint16_t* out, int64_t ld_out, void* ws, size_t ws_bytes, void* stream) {
    return nhm_fp8_linear_ex(a, a_type, m, ld_a, w, out, NHM_BF16, ld_out, ws, ws_bytes, stream);
}

static nhm_status linear_call(const void* a, nhm_dtype a_type, int64_t m, int64_t ld_a, const nhm_fp8_weight* w,
                              void* out, nhm_dtype out_type, int64_t ld_out, void* ws, size_t ws_bytes, void* stream,
                              bool exact) {
    g_err[0] = 0;
    if (out_type != NHM_BF16 && out_type != NHM_F32)
        return fail(NHM_ERR_UNSUPPORTED, "output dtype %d: bf16 or f32", (int)out_type);
    if (!w) return fail(NHM_ERR_NULL, "weight is NULL");
    if (a_type != NHM_BF16 && a_type != NHM_E4M3) return fail(NHM_ERR_UNSUPPORTED, "unknown activation dtype %d", (int)a_type);
    if (m < 0) return fail(NHM_ERR_SHAPE, "negative m");
    if (w->n <= 0 || w->k <= 0 || w->k % 16 != 0)
        return fail(NHM_ERR_SHAPE, "weight [%lld, %lld]: n and k must be positive, k a multiple of 16", (long long)w->n,
                    (long long)w->k);
    nhm_status s = check_weight(w, w->n, w->k, "weight");
    if (s != NHM_OK) return s;
    if (m == 0) return NHM_OK;
    if (!a || !out) return fail(NHM_ERR_NULL, "a or out is NULL");
    if (ld_a < w->k || ld_out < w->n)
        return fail(NHM_ERR_SHAPE, "ld_a %lld < k %lld or ld_out %lld < n %lld", (long long)ld_a, (long long)w->k,
                    (long long)ld_out, (long long)w->n);
    if (!aligned(a, 16) || (a_type == NHM_BF16 ? ld_a % 8 : ld_a % 16) != 0)
        return fail(NHM_ERR_ALIGN, "a must be 16-byte aligned with 16-byte row stride");
    if (!aligned(out, out_type == NHM_F32 ? 4 : 2))
        return fail(NHM_ERR_ALIGN, "out must be aligned to its element size");
    const size_t need = linear_codes_ws(m, w->k, a_type);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(NHM_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    if (ws && !aligned(ws, 256)) return fail(NHM_ERR_ALIGN, "ws must be 256-byte aligned");
    if ((s = check_offsets(m, a_type == NHM_BF16 ? w->k : ld_a, w->n, w->k, "linear")) != NHM_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    const uint8_t* aq = static_cast<const uint8_t*>(a);
    int64_t lda = ld_a;
    char* wsb = static_cast<char*>(ws);
    if (a_type == NHM_BF16) {
        uint8_t* q = reinterpret_cast<uint8_t*>(wsb);
        launch_quantize(static_cast<const uint16_t*>(a), m, w->k, ld_a, w->a_scale, q, w->k, st);
        if ((s = check_launch("quantize_static")) != NHM_OK) return s;
        aq = q;
        lda = w->k;
    }
    // the split-k partials after the codes, where the workspace holds them
    const size_t pb = proj_part_bytes(m, w->n, w->k);
    float* part = pb > 0 && ws && ws_bytes >= need + pb ? reinterpret_cast<float*>(wsb + need) : nullptr;
    if (out_type == NHM_F32)
        return project(aq, lda, m, *w, nullptr, ld_out, st, static_cast<float*>(out), part, part ? pb : 0, exact);
    return project(aq, lda, m, *w, static_cast<uint16_t*>(out), ld_out, st, nullptr, part, part ? pb : 0, exact);
}

nhm_status nhm_fp8_linear_ex(const void* a, nhm_dtype a_type, int64_t m, int64_t ld_a, const nhm_fp8_weight* w,
                             void* out, nhm_dtype out_type, int64_t ld_out, void* ws, size_t ws_bytes, void* stream) {
    return linear_call(a, a_type, m, ld_a, w, out, out_type, ld_out, ws, ws_bytes, stream, false);
}

nhm_status nhm_fp8_linear_exact(const void* a, nhm_dtype a_type, int64_t m, int64_t ld_a, const nhm_fp8_weight* w,
                                void* out, nhm_dtype out_type, int64_t ld_out, void* ws, size_t ws_bytes,
                                void* stream) {
    return linear_call(a, a_type, m, ld_a, w, out, out_type, ld_out, ws, ws_bytes, stream, true);
}

nhm_status nhm_mixer_decode_ws_layout(const nhm_geometry* g, int32_t batch, nhm_ws_layout* out) {
    g_err[0] = 0;
    if (!out) return fail(NHM_ERR_NULL, "layout output is NULL");
    nhm_status s = check_geometry(g);
    if (s != NHM_OK) return s;
    if (batch < 0) return fail(NHM_ERR_SHAPE, "negative batch");
    *out = decode_ws(g, batch).pub;
    return NHM_OK;
}

nhm_status nhm_mixer_prefill_ws_layout(const nhm_geometry* g, int64_t n_tokens, int32_t n_seqs, int32_t chunk,
                                       nhm_ws_layout* out) {
    g_err[0] = 0;
    if (!out) return fail(NHM_ERR_NULL, "layout output is NULL");
    nhm_status s = check_geometry(g);
    if (s != NHM_OK) return s;
    if (chunk != 128) return fail(NHM_ERR_UNSUPPORTED, "chunk %d: this build implements chunk 128", chunk);
    if (n_tokens < 0 || n_seqs < 0 || n_tokens > INT32_MAX)
        return fail(NHM_ERR_SHAPE, "n_tokens %lld / n_seqs %d out of range", (long long)n_tokens, n_seqs);
    *out = prefill_ws(g, n_tokens, n_seqs, chunk).pub;
    return NHM_OK;
}

nhm_status nhm_mixer_decode(const nhm_mixer_params* p, const uint16_t* hidden, int32_t batch, const int32_t* slot_idx,
                            float* ssm_pool, uint16_t* conv_pool, int32_t n_slots, uint16_t* out, void* ws,
                            size_t ws_bytes, void* stream) {
    return nhm_mixer_decode_ex(p, hidden, batch, slot_idx, ssm_pool, NHM_F32, conv_pool, n_slots, out, ws, ws_bytes,
                               stream);
}

}  // extern "C"

namespace nhm {

// ---------------------------------------------------------------- decode scratch without allocation
// nhm_mixer_decode_noalloc keeps its workspace in this file-scope device array instead of a
// caller's buffer. Each GPU the library runs on holds its own copy, at its own address, until
// the process ends; host code reaches it only through the address hipGetSymbolAddress returns
// on that device (the array's name is a host-side stand-in, not a device address).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_addr[kMaxDevices];

// The scratch address on the device the call's work runs on: resolved once per device, on
// that device's first call (the current device, which must be the stream's).
static nhm_status device_scratch(hipStream_t st, void** out) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(NHM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    }
    if (st) {
        int sd = -1;
        e = hipStreamGetDevice(st, &sd);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(NHM_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
        }
        if (sd != cur)
            return fail(NHM_ERR_UNSUPPORTED, "the stream belongs to device %d but device %d is current", sd, cur);
    }
    if (cur < 0 || cur >= kMaxDevices) return fail(NHM_ERR_UNSUPPORTED, "device %d: at most %d devices", cur, kMaxDevices);
    void* p = g_scratch_addr[cur].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(NHM_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", cur, hipGetErrorString(e));
        }
        g_scratch_addr[cur].store(p, std::memory_order_release);
    }
    *out = p;
    return NHM_OK;
}

// nhm_mixer_decode_ex; noalloc: the workspace is this library's device scratch (ws ignored).
// hidden_q (optional): the block input's e4m3 codes under in_proj's activation scale, used
// instead of quantizing hidden (which may then be NULL). out_q (optional): the codes of the
// bf16 block output under *out_q_scale.
static nhm_status decode_call(const nhm_mixer_params* p, const uint16_t* hidden, const uint8_t* hidden_q,
                              int32_t batch, const int32_t* slot_idx, void* ssm_pool, nhm_dtype ssm_type,
                              uint16_t* conv_pool, int32_t n_slots, uint16_t* out, uint8_t* out_q,
                              const float* out_q_scale, void* ws, size_t ws_bytes, void* stream, bool noalloc) {
    g_err[0] = 0;
    if (ssm_type != NHM_F32 && ssm_type != NHM_BF16)
        return fail(NHM_ERR_UNSUPPORTED, "SSM state dtype %d: f32 or bf16", (int)ssm_type);
    nhm_layout l;
    nhm_status s = check_params(p, &l);
    if (s != NHM_OK) return s;
    if (batch < 0) return fail(NHM_ERR_SHAPE, "negative batch");
    if (batch == 0) return NHM_OK;
    if (n_slots <= 0) return fail(NHM_ERR_SHAPE, "n_slots must be positive");
    if ((!hidden && !hidden_q) || !slot_idx || !ssm_pool || !conv_pool || !out || (!noalloc && !ws))
        return fail(NHM_ERR_NULL, "hidden (or its codes), slot_idx, pools, out or ws is NULL");
    if (out_q && !out_q_scale) return fail(NHM_ERR_NULL, "out_q needs out_q_scale");
    if ((hidden && !aligned(hidden, 16)) || !aligned(out, 16) || !aligned(ssm_pool, 16) || !aligned(conv_pool, 16) ||
        !aligned(slot_idx, 4) || (!noalloc && !aligned(ws, 256)) || (hidden_q && !aligned(hidden_q, 16)) ||
        (out_q && !aligned(out_q, 16)) || (out_q_scale && !aligned(out_q_scale, 4)))
        return fail(NHM_ERR_ALIGN, "hidden, its codes, out, out_q and pools must be 16-byte aligned, ws 256-byte aligned");
    const MixerWs w = decode_ws(&p->g, batch);
    if (noalloc && w.pub.total > kNoAllocScratchBytes)
        return fail(NHM_ERR_WORKSPACE, "batch %d needs %zu bytes of scratch; the library's per-device scratch holds %zu",
                    batch, w.pub.total, kNoAllocScratchBytes);
    if (!noalloc && ws_bytes < w.pub.total)
        return fail(NHM_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.pub.total, ws_bytes);
    if ((s = check_offsets(batch, p->g.hidden, l.d_in_proj, p->g.hidden, "decode in_proj")) != NHM_OK ||
        (s = check_offsets(batch, l.d_inner, p->g.hidden, l.d_inner, "decode out_proj")) != NHM_OK)
        return s;
    hipStream_t st = (hipStream_t)stream;
    if (noalloc && (s = device_scratch(st, &ws)) != NHM_OK) return s;
    char* wsb = static_cast<char*>(ws);
    const int64_t H = p->g.hidden;
    const uint8_t* q_in = reinterpret_cast<uint8_t*>(wsb + w.pub.q_in);
    uint16_t* zx = reinterpret_cast<uint16_t*>(wsb + w.pub.zxbcdt);
    uint16_t* xc = reinterpret_cast<uint16_t*>(wsb + w.pub.xbc_conv);
    uint8_t* q_out = reinterpret_cast<uint8_t*>(wsb + w.pub.q_out);

    if (hidden_q) {
        q_in = hidden_q;   // pre-quantized by the caller (e.g. the previous block's out_q)
    } else {
        launch_quantize(hidden, batch, H, H, p->in_proj.a_scale, const_cast<uint8_t*>(q_in), H, st);
        if ((s = check_launch("decode quant")) != NHM_OK) return s;
    }
    // in_proj: up to 32 rows on the GEMV, 16 rows a launch, whose first launch also zeroes the
    // fused norm's hand-off counters; above 32 rows one GEMM that reads the weight once, with
    // every product summed in f32 as on the GEMV (its sums feed dt, which every later decay
    // exponentiates). Measured on MI355X, 10304 x 2688: 32 rows 15.6 us as two GEMV launches
    // against 21.2 us for the GEMM; 48 rows 23.3 against 22.1; 64 rows 30.6 against 20.2.
    const bool fused = decode_fused_norm(&p->g);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(wsb + w.cnt);
    if (!use_gemv(16, l.d_in_proj, H))
        return fail(NHM_ERR_UNSUPPORTED, "decode in_proj %d x %lld outside the GEMV", l.d_in_proj, (long long)H);
    if (batch > 32) {
        if (fused) launch_clear(cnt, batch * p->g.n_groups, st);
        if ((s = project(q_in, H, batch, p->in_proj, zx, l.d_in_proj, st, nullptr,
                         reinterpret_cast<float*>(wsb + w.part), w.part_bytes, true)) != NHM_OK)
            return s;
    }
    for (int32_t r0 = 0; batch <= 32 && r0 < batch; r0 += 16) {
        const int mg = batch - r0 < 16 ? batch - r0 : 16;
        s = launch_gemv(q_in + (int64_t)r0 * H, H, mg, p->in_proj.w, p->in_proj.w_scale, p->in_proj.a_scale,
                        l.d_in_proj, H, zx + (int64_t)r0 * l.d_in_proj, l.d_in_proj, st, nullptr, nullptr, 0, nullptr,
                        fused && r0 == 0 ? cnt : nullptr, fused && r0 == 0 ? batch * p->g.n_groups : 0,
                        ws_step(p->in_proj));
        if (s != NHM_OK) return s;
    }
    DecodeSsmArgs da;
    da.slot_idx = slot_idx;
    da.ssm_pool = ssm_type == NHM_F32 ? static_cast<float*>(ssm_pool) : nullptr;
    da.ssm_pool_bf16 = ssm_type == NHM_BF16 ? static_cast<uint16_t*>(ssm_pool) : nullptr;
    da.zxbcdt = zx;
    da.xbc_conv = xc;
    da.conv_pool = conv_pool;
    da.conv_w = p->conv_w;
    da.conv_b = p->conv_b;
    da.A_log = p->A_log;
    da.D = p->D;
    da.dt_bias = p->dt_bias;
    da.y = reinterpret_cast<uint16_t*>(wsb + w.pub.y);
    da.n_heads = p->g.n_heads;
    da.n_groups = p->g.n_groups;
    da.d_in_proj = l.d_in_proj;
    da.conv_dim = l.conv_dim;
    da.d_inner = l.d_inner;
    da.xbc_off = l.xbc_off;
    da.dt_off = l.dt_off;
    da.b_off = l.b_off;
    da.c_off = l.c_off;
    if (fused) {
        da.cnt = cnt;
        da.norm_w = p->norm_w;
        da.out_a_scale = p->out_proj.a_scale;
        da.eps = p->g.rms_eps;
        da.z_off = l.z_off;
        da.norm = reinterpret_cast<uint16_t*>(wsb + w.pub.norm);
        da.q_out = q_out;
    }
    if ((s = launch_decode_ssm(da, batch, st)) != NHM_OK) return s;
    GnormArgs ga{batch, p->g.n_groups, l.d_inner, l.d_in_proj, l.z_off, p->g.rms_eps, da.y, zx, p->norm_w,
                 p->out_proj.a_scale, reinterpret_cast<uint16_t*>(wsb + w.pub.norm), q_out};
    ga.slot_idx = slot_idx;   // the B and C conv windows are shifted here (see DecodeSsmArgs)
    ga.conv_pool = conv_pool;
    ga.conv_dim = l.conv_dim;
    ga.xbc_off = l.xbc_off;
    ga.b_off = l.b_off;
    ga.c_off = l.c_off;
    ga.d_state = p->g.d_state;
    if (!fused && (s = launch_gnorm_quant(ga, st)) != NHM_OK) return s;
    // out_proj above 32 rows in one GEMM call (which splits k for these narrow shapes), reading
    // the weight once instead of once per 16 rows: one block at B = 64 104.9 -> 98.0 us; at
    // B = 32 two GEMV launches stay ahead (60.0 against 61.6 us). in_proj stays on the GEMV per
    // 16 rows: its exact f32 sums feed dt, which every later decay exponentiates (the GEMM's
    // coarser sums would need the dt recompute the prefill runs).
    if (batch > 32) {
        if ((s = project(q_out, l.d_inner, batch, p->out_proj, out, H, st, nullptr,
                         reinterpret_cast<float*>(wsb + w.part), w.part_bytes)) != NHM_OK)
            return s;
        if (out_q) {   // the tiled path has no code epilogue
            launch_quantize(out, batch, H, H, out_q_scale, out_q, H, st);
            return check_launch("decode out_q");
        }
        return NHM_OK;
    }
    // up to 32 rows: the GEMV, which also writes the codes of its bf16 output when asked
    for (int32_t r0 = 0; r0 < batch; r0 += 16) {
        const int mg = batch - r0 < 16 ? batch - r0 : 16;
        s = project(q_out + (int64_t)r0 * l.d_inner, l.d_inner, mg, p->out_proj, out + (int64_t)r0 * H, H, st, nullptr,
                    nullptr, 0, false, out_q ? out_q + (int64_t)r0 * H : nullptr, H, out_q_scale);
        if (s != NHM_OK) return s;
    }
    return NHM_OK;
}

}  // namespace nhm

extern "C" {

nhm_status nhm_mixer_decode_ex(const nhm_mixer_params* p, const uint16_t* hidden, int32_t batch,
                               const int32_t* slot_idx, void* ssm_pool, nhm_dtype ssm_type, uint16_t* conv_pool,
                               int32_t n_slots, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
    return decode_call(p, hidden, nullptr, batch, slot_idx, ssm_pool, ssm_type, conv_pool, n_slots, out, nullptr,
                       nullptr, ws, ws_bytes, stream, false);
}

nhm_status nhm_mixer_decode_q(const nhm_mixer_params* p, const uint16_t* hidden, const uint8_t* hidden_q, int32_t batch,
                              const int32_t* slot_idx, void* ssm_pool, nhm_dtype ssm_type, uint16_t* conv_pool,
                              int32_t n_slots, uint16_t* out, uint8_t* out_q, const float* out_q_scale, void* ws,
                              size_t ws_bytes, void* stream) {
    return decode_call(p, hidden, hidden_q, batch, slot_idx, ssm_pool, ssm_type, conv_pool, n_slots, out, out_q,
                       out_q_scale, ws, ws_bytes, stream, false);
}

nhm_status nhm_mixer_decode_noalloc(const nhm_mixer_params* p, const uint16_t* hidden, int32_t batch,
                                    const int32_t* slot_idx, void* ssm_pool, nhm_dtype ssm_type, uint16_t* conv_pool,
                                    int32_t n_slots, uint16_t* out, void* stream) {
    return decode_call(p, hidden, nullptr, batch, slot_idx, ssm_pool, ssm_type, conv_pool, n_slots, out, nullptr,
                       nullptr, nullptr, 0, stream, true);
}

nhm_status nhm_mixer_prefill(const nhm_mixer_params* p, const uint16_t* hidden, int64_t n_tokens,
                             const int32_t* cu_seqlens, int32_t n_seqs, const int32_t* slot_idx,
                             const int32_t* has_initial, int32_t chunk, float* ssm_pool, uint16_t* conv_pool,
                             int32_t n_slots, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
    return nhm_mixer_prefill_ex(p, hidden, n_tokens, cu_seqlens, n_seqs, slot_idx, has_initial, chunk, ssm_pool,
                                NHM_F32, conv_pool, n_slots, out, ws, ws_bytes, stream);
}

nhm_status nhm_mixer_prefill_ex(const nhm_mixer_params* p, const uint16_t* hidden, int64_t n_tokens,
                                const int32_t* cu_seqlens, int32_t n_seqs, const int32_t* slot_idx,
                                const int32_t* has_initial, int32_t chunk, void* ssm_pool, nhm_dtype ssm_type,
                                uint16_t* conv_pool, int32_t n_slots, uint16_t* out, void* ws, size_t ws_bytes,
                                void* stream) {
    g_err[0] = 0;
    if (ssm_type != NHM_F32 && ssm_type != NHM_BF16)
        return fail(NHM_ERR_UNSUPPORTED, "SSM state dtype %d: f32 or bf16", (int)ssm_type);
    nhm_layout l;
    nhm_status s = check_params(p, &l);
    if (s != NHM_OK) return s;
    if (chunk != 128) return fail(NHM_ERR_UNSUPPORTED, "chunk %d: this build implements chunk 128", chunk);
    if (n_tokens < 0 || n_seqs < 0 || n_tokens > INT32_MAX)
        return fail(NHM_ERR_SHAPE, "n_tokens %lld / n_seqs %d out of range", (long long)n_tokens, n_seqs);
    if (n_seqs == 0) {
        if (n_tokens != 0) return fail(NHM_ERR_SHAPE, "%lld tokens but no sequences", (long long)n_tokens);
        return NHM_OK;
    }
    if (n_slots <= 0) return fail(NHM_ERR_SHAPE, "n_slots must be positive");
    if (n_seqs > n_slots) return fail(NHM_ERR_SHAPE, "%d sequences need distinct slots, pool has %d", n_seqs, n_slots);
    if (!cu_seqlens || !slot_idx || !has_initial || !ssm_pool || !conv_pool || !ws || (n_tokens > 0 && (!hidden || !out)))
        return fail(NHM_ERR_NULL, "a required pointer is NULL");
    if ((hidden && !aligned(hidden, 16)) || (out && !aligned(out, 16)) || !aligned(ssm_pool, 16) ||
        !aligned(conv_pool, 16) || !aligned(cu_seqlens, 4) || !aligned(slot_idx, 4) || !aligned(has_initial, 4) ||
        !aligned(ws, 256))
        return fail(NHM_ERR_ALIGN, "hidden, out and pools must be 16-byte aligned, ws 256-byte aligned");
    const MixerWs w = prefill_ws(&p->g, n_tokens, n_seqs, chunk);
    if (ws_bytes < w.pub.total)
        return fail(NHM_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.pub.total, ws_bytes);
    if ((int64_t)w.max_chunks * p->g.n_heads > INT32_MAX)   // one scan block per (chunk, head)
        return fail(NHM_ERR_UNSUPPORTED, "%d chunks x %d heads exceed the scan's grid", w.max_chunks, p->g.n_heads);
    if ((s = check_offsets(n_tokens, p->g.hidden, l.d_in_proj, p->g.hidden, "prefill in_proj")) != NHM_OK ||
        (s = check_offsets(n_tokens, l.d_inner, p->g.hidden, l.d_inner, "prefill out_proj")) != NHM_OK)
        return s;
    hipStream_t st = (hipStream_t)stream;
    char* wsb = static_cast<char*>(ws);
    const int64_t H = p->g.hidden;
    uint8_t* q_in = reinterpret_cast<uint8_t*>(wsb + w.pub.q_in);
    uint16_t* zx = reinterpret_cast<uint16_t*>(wsb + w.pub.zxbcdt);
    if (n_tokens > 0) {
        launch_quantize(hidden, n_tokens, H, H, p->in_proj.a_scale, q_in, H, st);
        if ((s = check_launch("prefill quant")) != NHM_OK) return s;
        // every product summed in f32: the e4m3 MFMA's coarser 128-product sums move about 1 %
        // of the bf16 projection outputs by one step, and those steps reach the a9 codes through
        // dt (exponentiated by every later token's decay), x, B, C and the gate
        if ((s = project(q_in, H, n_tokens, p->in_proj, zx, l.d_in_proj, st, nullptr,
                         reinterpret_cast<float*>(wsb + w.part), w.part_bytes, true)) != NHM_OK)
            return s;
    }
    PrefillArgs a;
    a.T = n_tokens;
    a.n_seqs = n_seqs;
    a.chunk = chunk;
    a.max_chunks = w.max_chunks;
    a.n_heads = p->g.n_heads;
    a.n_groups = p->g.n_groups;
    a.d_in_proj = l.d_in_proj;
    a.conv_dim = l.conv_dim;
    a.d_inner = l.d_inner;
    a.z_off = l.z_off;
    a.xbc_off = l.xbc_off;
    a.dt_off = l.dt_off;
    a.b_off = l.b_off;
    a.c_off = l.c_off;
    a.eps = p->g.rms_eps;
    a.cu_seqlens = cu_seqlens;
    a.slot_idx = slot_idx;
    a.has_initial = has_initial;
    a.ssm_pool = ssm_type == NHM_F32 ? static_cast<float*>(ssm_pool) : nullptr;
    a.ssm_pool_bf16 = ssm_type == NHM_BF16 ? static_cast<uint16_t*>(ssm_pool) : nullptr;
    a.conv_pool = conv_pool;
    a.conv_w = p->conv_w;
    a.conv_b = p->conv_b;
    a.A_log = p->A_log;
    a.D = p->D;
    a.dt_bias = p->dt_bias;
    a.norm_w = p->norm_w;
    a.out_a_scale = p->out_proj.a_scale;
    a.zxbcdt = zx;
    a.xbc_conv = reinterpret_cast<uint16_t*>(wsb + w.pub.xbc_conv);
    a.chunk_info = reinterpret_cast<int32_t*>(wsb + w.chunk_info);
    a.seq_chunk0 = reinterpret_cast<int32_t*>(wsb + w.seq_chunk0);
    a.chunk_cs = reinterpret_cast<float*>(wsb + w.chunk_cs);
    a.chunk_dt = reinterpret_cast<float*>(wsb + w.chunk_dt);
    a.chunk_state = reinterpret_cast<float*>(wsb + w.chunk_state);
    a.y = reinterpret_cast<uint16_t*>(wsb + w.pub.y);
    a.norm = reinterpret_cast<uint16_t*>(wsb + w.pub.norm);
    a.q_out = reinterpret_cast<uint8_t*>(wsb + w.pub.q_out);
    if ((s = launch_prefill_mid(a, st)) != NHM_OK) return s;
    if (n_tokens > 0)
        return project(a.q_out, l.d_inner, n_tokens, p->out_proj, out, H, st, nullptr,
                       reinterpret_cast<float*>(wsb + w.part), w.part_bytes);
    return NHM_OK;
}

}  // extern "C"
