// Drives libmla_decode's host code (argument checks, split plan, workspace
// layout) through its C entry points with the HIP stand-ins of
// hip_stubs.cpp.  Built with AddressSanitizer and UBSan by
// tests/test_host_sanitized.py; exits non-zero on the first wrong return code
// and prints "ALL OK" at the end.
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mla_decode.h"

extern int g_launches;
static int g_fail = 0;

#define EXPECT(cond, ...)                                   \
    do {                                                    \
        if (!(cond)) {                                      \
            printf("FAIL %s:%d: ", __FILE__, __LINE__);     \
            printf(__VA_ARGS__);                            \
            printf(" (%s)\n", mla_last_error());            \
            g_fail = 1;                                     \
        }                                                   \
    } while (0)

static const uintptr_t FAKE = 1u << 20;   // aligned, never dereferenced by the stand-ins

static mla_decode_params_t base(int B, int H, int K, int L, int act, int wdt) {
    mla_decode_params_t p;
    memset(&p, 0, sizeof p);
    p.B = B; p.H = H; p.K = K;
    p.d_nope = 128; p.d_rope = 64; p.d_v = 128; p.kv_rank = 512;
    p.max_cache_len = L; p.rope_table_len = L;
    p.dtype_act = act; p.dtype_w = wdt; p.dtype_out = MLA_DTYPE_F32;
    p.num_cus = 256;
    p.softmax_scale = 0.1f;
    const void* f = (const void*)FAKE;
    p.q_nope = f; p.q_pe = f; p.w_uk = f; p.w_uv = f; p.kv_cache = f; p.pe_cache = f;
    p.topk_indices = (const int32_t*)f; p.cache_lens = (const int32_t*)f; p.rope_table = (const float*)f;
    p.out = (void*)f;
    p.q_nope_stride_b = (int64_t)H * 128; p.q_nope_stride_h = 128;
    p.q_pe_stride_b = (int64_t)H * 64; p.q_pe_stride_h = 64;
    p.w_uk_stride_h = p.w_uv_stride_h = 128 * 512;
    p.kv_stride_b = (int64_t)L * 512; p.kv_stride_t = 512;
    p.pe_stride_b = (int64_t)L * 64; p.pe_stride_t = 64;
    p.idx_stride_b = K;
    p.out_stride_b = (int64_t)H * 128; p.out_stride_h = 128;
    return p;
}

// The argument checks: each case breaks one field of an otherwise valid call.
static void bad_arguments() {
    struct Case { const char* name; int code; } names[] = {
        {"d_nope", 2}, {"kv_rank", 2}, {"dtype_act", 2}, {"B", 1}, {"K", 1}, {"q_nope", 1},
        {"kv_cache_misaligned", 1}, {"kv_stride_t", 1}, {"pe_stride_t", 1}, {"idx_stride_b", 1},
        {"q_pe_stride_h", 1}, {"w_uk_stride_h", 1}, {"softmax_scale", 1}, {"num_splits", 1}, {"flags", 1},
        {"max_cache_len", 1}, {"workspace_size", 3}, {"B_huge", 1}, {"H_huge", 1}, {"K_huge_stride", 1},
        {"cache_span", 2}, {"q_stride_huge", 2}, {"lse_misaligned", 1}, {"append_one_side", 1},
        {"append_stride", 1}, {"neg_stride", 1}, {"nan_scale", 1}, {"num_cus_neg", 1},
    };
    for (auto& c : names) {
        mla_decode_params_t p = base(2, 128, 16, 64, MLA_DTYPE_BF16, MLA_DTYPE_BF16);
        static char ws[1 << 22];
        p.workspace = ws; p.workspace_size = sizeof ws;
        const char* n = c.name;
        if (!strcmp(n, "d_nope")) p.d_nope = 64;
        else if (!strcmp(n, "kv_rank")) p.kv_rank = 256;
        else if (!strcmp(n, "dtype_act")) p.dtype_act = 5;
        else if (!strcmp(n, "B")) p.B = 0;
        else if (!strcmp(n, "K")) p.K = 0;
        else if (!strcmp(n, "q_nope")) p.q_nope = NULL;
        else if (!strcmp(n, "kv_cache_misaligned")) p.kv_cache = (const void*)(FAKE + 2);
        else if (!strcmp(n, "kv_stride_t")) p.kv_stride_t = 513;
        else if (!strcmp(n, "pe_stride_t")) p.pe_stride_t = 32;
        else if (!strcmp(n, "idx_stride_b")) p.idx_stride_b = 8;
        else if (!strcmp(n, "q_pe_stride_h")) p.q_pe_stride_h = 68;
        else if (!strcmp(n, "w_uk_stride_h")) p.w_uk_stride_h = 128 * 512 + 4;
        else if (!strcmp(n, "softmax_scale")) p.softmax_scale = -1.f;
        else if (!strcmp(n, "num_splits")) p.num_splits = 65;
        else if (!strcmp(n, "flags")) p.flags = 2;
        else if (!strcmp(n, "max_cache_len")) p.max_cache_len = 0;
        else if (!strcmp(n, "workspace_size")) p.workspace_size = 0;
        else if (!strcmp(n, "B_huge")) p.B = INT_MAX;
        else if (!strcmp(n, "H_huge")) p.H = INT_MAX;
        else if (!strcmp(n, "K_huge_stride")) { p.K = INT_MAX; p.idx_stride_b = 16; }
        else if (!strcmp(n, "cache_span")) { p.max_cache_len = 1 << 19; p.kv_stride_t = 4096; }
        else if (!strcmp(n, "q_stride_huge")) p.q_nope_stride_b = (int64_t)1 << 40;
        else if (!strcmp(n, "lse_misaligned")) p.lse_out = (float*)(FAKE + 2);
        else if (!strcmp(n, "append_one_side")) p.kv_new = (const void*)FAKE;
        else if (!strcmp(n, "append_stride")) {
            p.kv_new = (const void*)FAKE; p.pe_new = (const void*)FAKE;
            p.kv_new_stride_b = 500; p.pe_new_stride_b = 64;
        }
        else if (!strcmp(n, "neg_stride")) p.out_stride_b = -1;
        else if (!strcmp(n, "nan_scale")) p.softmax_scale = __builtin_nanf("");
        else if (!strcmp(n, "num_cus_neg")) p.num_cus = -1;
        const int before = g_launches;
        const int rc = mla_decode_attn(&p, NULL);
        EXPECT(rc == c.code, "case %s: rc %d, want %d", n, rc, c.code);
        EXPECT(g_launches == before, "case %s launched", n);
        EXPECT(mla_last_error()[0] != 0, "case %s: no message", n);
    }
    EXPECT(mla_decode_attn(NULL, NULL) == MLA_ERR_INVALID_ARG, "null params");
}

// Valid calls over a sweep of sizes, dtypes, split counts and modes, each
// with a heap workspace of exactly the size the library asks for (so that a
// region past its end is a heap overflow), and the same call one byte short.
static void valid_calls() {
    const int Bs[] = {1, 3, 128, 300};
    const int Hs[] = {1, 16, 128, 129, 256};
    const int Ks[] = {1, 65, 2048};
    const int splits[] = {0, 1, 2, 7, 64};
    int n = 0;
    for (int B : Bs)
        for (int H : Hs)
            for (int K : Ks)
                for (int act = 0; act < 2; ++act)
                    for (int S : splits) {
                        if (act == MLA_DTYPE_F32 && S > 1) continue;
                        const int L = K < 64 ? 64 : K;
                        mla_decode_params_t p = base(B, H, K, L, act, 1 - act);
                        p.num_splits = S;
                        p.flags = (n % 3 == 0) ? MLA_FLAG_VALIDATE : 0;
                        if (n % 4 == 1) {
                            p.kv_new = (const void*)FAKE; p.pe_new = (const void*)FAKE;
                            p.kv_new_stride_b = 512; p.pe_new_stride_b = 64;
                        }
                        const size_t need = mla_decode_workspace_size(B, H, K, act, 1 - act, 256, S);
                        EXPECT(need > 0, "workspace size B=%d H=%d K=%d act=%d S=%d", B, H, K, act, S);
                        if (!need) continue;
                        void* ws = malloc(need);
                        p.workspace = ws;
                        p.workspace_size = need - 1;
                        EXPECT(mla_decode_attn(&p, NULL) == MLA_ERR_WORKSPACE, "one byte short accepted");
                        p.workspace_size = need;
                        const int before = g_launches;
                        const int rc = mla_decode_attn(&p, NULL);
                        EXPECT(rc == MLA_OK, "B=%d H=%d K=%d act=%d S=%d: rc %d", B, H, K, act, S, rc);
                        EXPECT(g_launches == before + MLA_NUM_KERNELS, "launch count");
                        free(ws);
                        ++n;
                    }
    printf("%d valid calls\n", n);
}

// The planner and the workspace sizing over a wide range, including sizes
// whose products overflow 32 bits.
static void planner() {
    const int Bs[] = {1, 2, 7, 8, 31, 32, 64, 128, 255, 256, 1000, 1 << 20};
    const int Hs[] = {1, 31, 32, 33, 128, 129, 4096};
    const int Ks[] = {1, 32, 63, 64, 2048, 20000, 1 << 19};
    for (int B : Bs)
        for (int H : Hs)
            for (int K : Ks)
                for (int cus = 1; cus <= 1024; cus *= 4) {
                    const int S = mla_decode_num_splits(B, H, K, MLA_DTYPE_BF16, cus);
                    EXPECT(S >= 1 && S <= 64, "splits %d for B=%d H=%d K=%d cus=%d", S, B, H, K, cus);
                    const size_t ws = mla_decode_workspace_size(B, H, K, MLA_DTYPE_BF16, MLA_DTYPE_F32, cus, 0);
                    EXPECT(ws > (size_t)B * H * 576 * 2, "workspace %zu for B=%d H=%d K=%d", ws, B, H, K);
                }
    EXPECT(mla_decode_num_splits(0, 128, 2048, MLA_DTYPE_BF16, 256) < 1, "B=0 planned");
    EXPECT(mla_decode_workspace_size(4, 128, 2048, 7, 1, 256, 0) == 0, "bad dtype sized");
    EXPECT(mla_decode_workspace_size(4, 16, 64, 0, 0, 256, 2) == 0, "fp32 split sized");
}

static void other_entry_points() {
    mla_topk_params_t t;
    memset(&t, 0, sizeof t);
    t.B = 4; t.k = 64; t.max_len = 1000; t.scores = (const float*)FAKE; t.score_stride = 1000;
    t.cache_lens = (const int32_t*)FAKE; t.topk_indices = (int32_t*)FAKE; t.idx_stride = 64;
    EXPECT(mla_topk(&t, NULL) == MLA_OK, "topk valid");
    t.max_len = (1 << 19) + 1;
    EXPECT(mla_topk(&t, NULL) == MLA_ERR_INVALID_ARG, "topk max_len");
    t.max_len = 1000; t.idx_stride = 63;
    EXPECT(mla_topk(&t, NULL) == MLA_ERR_INVALID_ARG, "topk stride");
    EXPECT(mla_topk(NULL, NULL) == MLA_ERR_INVALID_ARG, "topk null");

    mla_rope_apply_params_t r;
    memset(&r, 0, sizeof r);
    r.N = 8; r.H = 4; r.dtype = MLA_DTYPE_BF16; r.interleaved = 0; r.table_len = 4096;
    r.x = (const void*)FAKE; r.x_stride_n = 256; r.x_stride_h = 64;
    r.y = (void*)(FAKE * 4); r.y_stride_n = 256; r.y_stride_h = 64;
    r.positions = (const int32_t*)FAKE; r.rope_table = (const float*)FAKE;
    EXPECT(mla_rope_apply(&r, NULL) == MLA_OK, "rope valid");
    r.N = 1 << 24; r.H = 16; r.x_stride_n = r.y_stride_n = 1024;
    EXPECT(mla_rope_apply(&r, NULL) == MLA_ERR_INVALID_ARG, "rope N*H");
    r.N = INT_MAX; r.H = INT_MAX;
    EXPECT(mla_rope_apply(&r, NULL) == MLA_ERR_INVALID_ARG, "rope huge");
    EXPECT(mla_rope_apply(NULL, NULL) == MLA_ERR_INVALID_ARG, "rope null");

    mla_rope_cfg_t c = {64, 16384, 4096, 0, 10000.0, 40.0, 32.0, 1.0, 1.0};
    EXPECT(mla_rope_freqs(&c, (float*)FAKE, NULL) == MLA_OK, "freqs valid");
    c.rope_dim = 32;
    EXPECT(mla_rope_freqs(&c, (float*)FAKE, NULL) == MLA_ERR_UNSUPPORTED, "freqs dim");
    c.rope_dim = 64; c.theta = 0.5;
    EXPECT(mla_rope_freqs(&c, (float*)FAKE, NULL) == MLA_ERR_INVALID_ARG, "freqs theta");
    c.theta = 10000.0;
    EXPECT(mla_softmax_scale(192, &c) > 0.13 && mla_softmax_scale(192, &c) < 0.14, "scale");
    EXPECT(mla_softmax_scale(0, &c) < 0, "scale dim");
    EXPECT(mla_decode_params_size() == sizeof(mla_decode_params_t), "params size");
}

int main() {
    bad_arguments();
    valid_calls();
    planner();
    other_entry_points();
    if (g_fail) return 1;
    printf("ALL OK\n");
    return 0;
}
