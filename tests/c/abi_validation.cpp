// Host-only driver for an AddressSanitizer / UndefinedBehaviorSanitizer build of the C ABI's
// validation (csrc/api.hip compiled for the host only). Every call below either fails
// validation before anything is enqueued or is a pure host query, so no GPU is needed; the
// kernel launchers of the other translation units are replaced by stubs that abort if reached.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../fp8_w8a8_linear_amd/csrc/nhm_internal.h"   // the launchers' declarations

namespace nhm {
[[noreturn]] static void reached(const char* f) {
    fprintf(stderr, "kernel launcher %s reached from a call that should have failed validation\n", f);
    abort();
}
void launch_quantize(const uint16_t*, int64_t, int64_t, int64_t, const float*, uint8_t*, int64_t, hipStream_t) {
    reached("launch_quantize");
}
void launch_dequant_channel(const uint8_t*, int64_t, int64_t, int64_t, const float*, uint16_t*, int64_t, hipStream_t) {
    reached("launch_dequant_channel");
}
nhm_status launch_gemv(const uint8_t*, int64_t, int, const uint8_t*, const float*, const float*, int64_t, int64_t,
                       uint16_t*, int64_t, hipStream_t, float*, uint8_t*, int64_t, const float*, uint32_t*, int, int) {
    reached("launch_gemv");
}
// The workspace queries size the split-k partials with this; the driver checks only that
// they succeed, so the stub reports none.
size_t gemm_part_bytes(int64_t, int64_t, int64_t) { return 0; }
nhm_status launch_gemm(const uint8_t*, int64_t, int64_t, const uint8_t*, const float*, const float*, int64_t, int64_t,
                       uint16_t*, int64_t, hipStream_t, float*, float*, size_t, bool, int) {
    reached("launch_gemm");
}
nhm_status launch_decode_ssm(const DecodeSsmArgs&, int, hipStream_t) { reached("launch_decode_ssm"); }
void launch_clear(uint32_t*, int, hipStream_t) { reached("launch_clear"); }
nhm_status launch_gnorm_quant(const GnormArgs&, hipStream_t) { reached("launch_gnorm_quant"); }
nhm_status launch_prefill_mid(const PrefillArgs&, hipStream_t) { reached("launch_prefill_mid"); }
}  // namespace nhm

static int failures = 0;
#define EXPECT(call, want)                                                                        \
    do {                                                                                          \
        const int got_ = (int)(call);                                                             \
        if (got_ != (int)(want)) {                                                                \
            fprintf(stderr, "line %d: %s -> %d, expected %d (%s)\n", __LINE__, #call, got_, (int)(want), \
                    nhm_last_error());                                                            \
            ++failures;                                                                           \
        }                                                                                         \
    } while (0)

static void* P(uintptr_t v) { return reinterpret_cast<void*>(v); }

int main() {
    nhm_geometry g = {2688, 64, 64, 128, 8, 4, 1e-5f};
    nhm_layout l;
    EXPECT(nhm_mixer_layout(&g, &l), NHM_OK);
    EXPECT(l.d_in_proj, 10304);
    EXPECT(nhm_mixer_layout(nullptr, &l), NHM_ERR_NULL);
    EXPECT(nhm_mixer_layout(&g, nullptr), NHM_ERR_NULL);
    nhm_geometry bad = g;
    bad.rms_eps = 0.f;
    EXPECT(nhm_mixer_layout(&bad, &l), NHM_ERR_UNSUPPORTED);
    bad = g;
    bad.n_heads = 12;
    bad.n_groups = 4;
    EXPECT(nhm_mixer_layout(&bad, &l), NHM_ERR_UNSUPPORTED);
    for (int i = 0; i < 7; ++i) EXPECT(strlen(nhm_status_str((nhm_status)i)) > 0, 1);
    EXPECT(strcmp(nhm_build_arch(), "gfx950"), 0);

    nhm_ws_layout wl;
    EXPECT(nhm_mixer_decode_ws_layout(&g, 8, &wl), NHM_OK);
    EXPECT(nhm_mixer_decode_ws_layout(&g, -1, &wl), NHM_ERR_SHAPE);
    EXPECT(nhm_mixer_prefill_ws_layout(&g, 15360, 4, 128, &wl), NHM_OK);
    EXPECT(nhm_mixer_prefill_ws_layout(&g, 512, 1, 64, &wl), NHM_ERR_UNSUPPORTED);
    EXPECT(nhm_mixer_prefill_ws_layout(&g, -5, 1, 128, &wl), NHM_ERR_SHAPE);

    // quant and dequant
    EXPECT(nhm_fp8_quantize_static(nullptr, 0, 8, 8, nullptr, nullptr, 8, nullptr), NHM_OK);
    EXPECT(nhm_fp8_quantize_static(nullptr, 2, 8, 8, (float*)P(0x100), (uint8_t*)P(0x200), 8, nullptr), NHM_ERR_NULL);
    EXPECT(nhm_fp8_quantize_static((uint16_t*)P(0x101), 2, 8, 8, (float*)P(0x100), (uint8_t*)P(0x200), 8, nullptr),
           NHM_ERR_ALIGN);
    EXPECT(nhm_fp8_dequant_channel_bf16((uint8_t*)P(0x1000), (float*)P(0x2000), 4, 24, 32, (uint16_t*)P(0x3000), 32,
                                        nullptr),
           NHM_ERR_SHAPE);

    // linear
    nhm_fp8_weight w = {(const uint8_t*)P(0x1000), (const float*)P(0x2000), (const float*)P(0x3000), 64, 128};
    const size_t need = nhm_fp8_linear_workspace_bytes(32, 64, 128, NHM_BF16);
    EXPECT(need >= 32 * 128, 1);
    EXPECT(nhm_fp8_linear(P(0x10000), NHM_BF16, 32, 128, &w, (uint16_t*)P(0x20000), 64, P(0x40000), need - 1, nullptr),
           NHM_ERR_WORKSPACE);
    EXPECT(nhm_fp8_linear(P(0x10002), NHM_BF16, 32, 128, &w, (uint16_t*)P(0x20000), 64, P(0x40000), need, nullptr),
           NHM_ERR_ALIGN);
    EXPECT(nhm_fp8_linear(P(0x10000), (nhm_dtype)7, 32, 128, &w, (uint16_t*)P(0x20000), 64, P(0x40000), need, nullptr),
           NHM_ERR_UNSUPPORTED);
    EXPECT(nhm_fp8_linear(nullptr, NHM_BF16, 0, 128, &w, nullptr, 64, nullptr, 0, nullptr), NHM_OK);
    nhm_fp8_weight big = {(const uint8_t*)P(0x1000), (const float*)P(0x2000), (const float*)P(0x3000), 1 << 19, 4096};
    EXPECT(nhm_fp8_linear(P(0x10000), NHM_E4M3, 32, 4096, &big, (uint16_t*)P(0x20000), 1 << 19, nullptr, 0, nullptr),
           NHM_ERR_UNSUPPORTED);
    EXPECT(nhm_fp8_linear_ex(P(0x10000), NHM_BF16, 32, 128, &w, P(0x20002), NHM_F32, 64, P(0x40000), need, nullptr),
           NHM_ERR_ALIGN);

    // mixer
    nhm_mixer_params p;
    memset(&p, 0, sizeof(p));
    p.g = g;
    p.in_proj = {(const uint8_t*)P(0x1000), (const float*)P(0x2000), (const float*)P(0x3000), 10304, 2688};
    p.out_proj = {(const uint8_t*)P(0x1000), (const float*)P(0x2000), (const float*)P(0x3000), 2688, 4096};
    p.conv_w = (const uint16_t*)P(0x5000);
    p.conv_b = (const uint16_t*)P(0x6000);
    p.norm_w = (const uint16_t*)P(0x7000);
    p.A_log = (const float*)P(0x8000);
    p.D = (const float*)P(0x9000);
    p.dt_bias = (const float*)P(0xA000);
    nhm_ws_layout dl;
    EXPECT(nhm_mixer_decode_ws_layout(&g, 8, &dl), NHM_OK);
    uint16_t* H = (uint16_t*)P(0x100000);
    const int32_t* SL = (const int32_t*)P(0x200000);
    float* SP = (float*)P(0x300000);
    uint16_t* CP = (uint16_t*)P(0x400000);
    uint16_t* O = (uint16_t*)P(0x500000);
    void* WS = P(0x600000);
    EXPECT(nhm_mixer_decode(&p, H, 0, SL, SP, CP, 64, O, WS, dl.total, nullptr), NHM_OK);
    EXPECT(nhm_mixer_decode(&p, nullptr, 8, SL, SP, CP, 64, O, WS, dl.total, nullptr), NHM_ERR_NULL);
    EXPECT(nhm_mixer_decode(&p, H, 8, SL, SP, CP, 64, O, WS, dl.total - 1, nullptr), NHM_ERR_WORKSPACE);
    EXPECT(nhm_mixer_decode(&p, H + 4, 8, SL, SP, CP, 64, O, WS, dl.total, nullptr), NHM_ERR_ALIGN);
    EXPECT(nhm_mixer_decode(&p, H, 8, SL, SP, CP, 0, O, WS, dl.total, nullptr), NHM_ERR_SHAPE);
    EXPECT(nhm_mixer_decode_ex(&p, H, 8, SL, SP, NHM_E4M3, CP, 64, O, WS, dl.total, nullptr), NHM_ERR_UNSUPPORTED);
    nhm_mixer_params pw = p;
    pw.in_proj.k = 4096;
    EXPECT(nhm_mixer_decode(&pw, H, 8, SL, SP, CP, 64, O, WS, dl.total, nullptr), NHM_ERR_SHAPE);
    // the no-allocation decode: refused before any device call (its scratch holds batch <= 299)
    EXPECT(nhm_mixer_decode_noalloc(&p, H, 0, SL, SP, NHM_F32, CP, 64, O, nullptr), NHM_OK);
    EXPECT(nhm_mixer_decode_noalloc(&p, H, 300, SL, SP, NHM_F32, CP, 512, O, nullptr), NHM_ERR_WORKSPACE);
    EXPECT(nhm_mixer_decode_noalloc(&p, nullptr, 8, SL, SP, NHM_F32, CP, 64, O, nullptr), NHM_ERR_NULL);
    EXPECT(nhm_mixer_decode_noalloc(&p, H + 4, 8, SL, SP, NHM_F32, CP, 64, O, nullptr), NHM_ERR_ALIGN);
    EXPECT(nhm_mixer_decode_noalloc(&p, H, 8, SL, SP, (nhm_dtype)5, CP, 64, O, nullptr), NHM_ERR_UNSUPPORTED);
    nhm_ws_layout pl;
    EXPECT(nhm_mixer_prefill_ws_layout(&g, 512, 1, 128, &pl), NHM_OK);
    const int32_t* CU = (const int32_t*)P(0x700000);
    const int32_t* HI = (const int32_t*)P(0x800000);
    EXPECT(nhm_mixer_prefill(&p, H, 0, CU, 0, SL, HI, 128, SP, CP, 4, O, WS, pl.total, nullptr), NHM_OK);
    EXPECT(nhm_mixer_prefill(&p, H, 5, CU, 0, SL, HI, 128, SP, CP, 4, O, WS, pl.total, nullptr), NHM_ERR_SHAPE);
    EXPECT(nhm_mixer_prefill(&p, H, 512, CU, 1, SL, HI, 64, SP, CP, 4, O, WS, pl.total, nullptr), NHM_ERR_UNSUPPORTED);
    EXPECT(nhm_mixer_prefill(&p, H, 512, nullptr, 1, SL, HI, 128, SP, CP, 4, O, WS, pl.total, nullptr), NHM_ERR_NULL);
    EXPECT(nhm_mixer_prefill(&p, H, 512, CU, 1, SL, HI, 128, SP, CP, 4, O, WS, pl.total - 1, nullptr),
           NHM_ERR_WORKSPACE);
    EXPECT(nhm_mixer_prefill(&p, H, 512, CU, 5, SL, HI, 128, SP, CP, 4, O, WS, pl.total, nullptr), NHM_ERR_SHAPE);
    // a long error message through the formatter (the detail buffer is bounded)
    nhm_geometry huge = g;
    huge.hidden = 16400;
    EXPECT(nhm_mixer_layout(&huge, &l), NHM_ERR_UNSUPPORTED);
    EXPECT(strlen(nhm_last_error()) > 0, 1);
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("abi validation ok\n");
    return 0;
}
