// Host side of libmla_decode: argument checks, launch planning, workspace
// layout and the kernel launches of one decode call.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "mla_internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Largest cache length the selection bitmap supports (LDS holds L_max/8 bytes).
constexpr int kMaxCacheLen = 1 << 19;
constexpr int kMaxBatch = 1 << 20;
constexpr int kMaxHeads = 1 << 12;
constexpr int kMaxSplits = 64;
constexpr int kMaxRopeRows = 1 << 24;
constexpr long long kMaxRopeVectors = 1ll << 27;   // 4 threads each: the grid stays below 2^31

int query_num_cus(int* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    *out = n;
    return 0;
}

// Split-KV plan.  The attention grid is B * hgroups * splits workgroups of
// one per CU (the kernel uses all of a CU's registers); splits fill the
// chip when B * hgroups is below the CU count, each keeping at least two
// tiles of work.
bool make_plan(int B, int H, int K, int dtype_act, int num_cus, int forced_splits, mla::Plan* pl) {
    if (B < 1 || H < 1 || K < 1 || num_cus < 1) return false;
    pl->bf16_path = dtype_act == MLA_DTYPE_BF16;
    if (!pl->bf16_path) {
        pl->nhg = 0; pl->heads_per_wg = 1; pl->hgroups = H; pl->splits = 1; pl->tile_rows = 256;
        return forced_splits <= 1;
    }
    pl->nhg = 4;                                    // 128 heads per attention workgroup
    pl->heads_per_wg = 128;
    pl->hgroups = (H + 127) / 128;
    pl->tile_rows = 32;
    int S;
    if (forced_splits > 0) {
        S = forced_splits;
    } else {
        const int base = B * pl->hgroups;
        S = base >= num_cus ? 1 : num_cus / base;
        const int max_by_rows = (K + 2 * pl->tile_rows - 1) / (2 * pl->tile_rows);
        if (S > max_by_rows) S = max_by_rows;
        if (S > kMaxSplits) S = kMaxSplits;
        if ((int64_t)S * H > 65536) S = 65536 / H;   // bounds the split partials: S * H KB per sequence
        if (S < 1) S = 1;
    }
    if (S > kMaxSplits) return false;
    pl->splits = S;
    return true;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

namespace mla {

int set_error(int code, const char* msg) {
    snprintf(g_err, sizeof g_err, "%s", msg);
    return code;
}

size_t workspace_layout(int B, int H, int K, bool bf16_path, int splits, void* base, Work* w) {
    const size_t act = bf16_path ? 2 : 4;
    size_t off = 0;
    char* p = (char*)base;
    Work ww{};
    ww.qt = p + off;       off = align256(off + (size_t)B * H * 576 * act);
    ww.qlo = p + off;      off = align256(off + (bf16_path ? (size_t)B * H * 64 * 2 : 0));
    ww.list = (int32_t*)(p + off);  off = align256(off + (size_t)B * K * 4);
    ww.counts = (int32_t*)(p + off); off = align256(off + (size_t)B * 4);
    ww.status = (uint32_t*)(p + off); off = align256(off + 4);
    ww.opart = p + off;
    off = align256(off + (bf16_path ? (size_t)B * splits * H * 512 * 2 : (size_t)B * H * 512 * 4));
    ww.lsepart = (float*)(p + off);
    off = align256(off + (size_t)B * (bf16_path ? splits : 1) * H * 4);
    ww.bytes = off;
    if (w) *w = ww;
    return off;
}

}  // namespace mla

extern "C" {

const char* mla_last_error(void) { return g_err; }

int mla_topk(const mla_topk_params_t* p, void* stream) {
    g_err[0] = 0;
    if (!p) return fail(MLA_ERR_INVALID_ARG, "mla_topk: null params");
    if (!p->scores || !p->cache_lens || !p->topk_indices)
        return fail(MLA_ERR_INVALID_ARG, "mla_topk: null pointer");
    if (p->B < 1 || p->B > kMaxBatch || p->k < 1 || p->max_len < 1 || p->max_len > kMaxCacheLen || p->reserved != 0)
        return fail(MLA_ERR_INVALID_ARG, "mla_topk: sizes out of range (B=%d k=%d max_len=%d)", p->B, p->k, p->max_len);
    if (p->score_stride < p->max_len || p->idx_stride < p->k)
        return fail(MLA_ERR_INVALID_ARG, "mla_topk: a stride is smaller than its row");
    if (mla::launch_topk(p->B, p->k, p->max_len, p->scores, p->score_stride, p->cache_lens, p->topk_indices,
                         p->idx_stride, (hipStream_t)stream) != hipSuccess)
        return fail(MLA_ERR_HIP, "mla_topk: launch failed");
    return MLA_OK;
}

int mla_rope_apply(const mla_rope_apply_params_t* p, void* stream) {
    g_err[0] = 0;
    if (!p) return fail(MLA_ERR_INVALID_ARG, "mla_rope_apply: null params");
    if (!p->x || !p->y || !p->positions || !p->rope_table)
        return fail(MLA_ERR_INVALID_ARG, "mla_rope_apply: null pointer");
    if (p->N < 1 || p->N > kMaxRopeRows || p->H < 1 || p->H > kMaxHeads || p->table_len < 1 || p->reserved != 0)
        return fail(MLA_ERR_INVALID_ARG, "mla_rope_apply: sizes out of range (N=%d H=%d table_len=%d)", p->N, p->H,
                    p->table_len);
    if (p->dtype != MLA_DTYPE_BF16 && p->dtype != MLA_DTYPE_F32)
        return fail(MLA_ERR_INVALID_ARG, "mla_rope_apply: dtype must be MLA_DTYPE_BF16 or MLA_DTYPE_F32");
    if (p->interleaved != 0 && p->interleaved != 1)
        return fail(MLA_ERR_INVALID_ARG, "mla_rope_apply: interleaved must be 0 or 1");
    if ((long long)p->N * p->H > kMaxRopeVectors)
        return fail(MLA_ERR_INVALID_ARG, "mla_rope_apply: N*H exceeds %lld", kMaxRopeVectors);
    // 64 features per vector; the vectors of one row must not overlap
    auto strides_ok = [&](long long sn, long long sh) {
        if (sh < 64 || sn < 0 || sn % 8 != 0 || sh % 8 != 0) return false;
        if (p->N > 1 && sn < (long long)(p->H - 1) * sh + 64) return false;
        return true;
    };
    if (!strides_ok(p->x_stride_n, p->x_stride_h) || !strides_ok(p->y_stride_n, p->y_stride_h))
        return fail(MLA_ERR_INVALID_ARG,
                    "mla_rope_apply: strides must be multiples of 8 with stride_h >= 64 and stride_n >= "
                    "(H-1)*stride_h + 64");
    if (!aligned16(p->x) || !aligned16(p->y) || !aligned16(p->rope_table))
        return fail(MLA_ERR_INVALID_ARG, "mla_rope_apply: x, y and rope_table must be 16-byte aligned");
    if (p->x == p->y && (p->x_stride_n != p->y_stride_n || p->x_stride_h != p->y_stride_h))
        return fail(MLA_ERR_INVALID_ARG, "mla_rope_apply: in place (x == y) needs equal strides");
    if (mla::launch_rope_apply(p->N, p->H, p->dtype == MLA_DTYPE_BF16, p->interleaved == 1, p->table_len, p->x,
                               p->x_stride_n, p->x_stride_h, p->y, p->y_stride_n, p->y_stride_h, p->positions,
                               p->rope_table, (hipStream_t)stream) != hipSuccess)
        return fail(MLA_ERR_HIP, "mla_rope_apply: launch failed");
    return MLA_OK;
}

size_t mla_decode_params_size(void) { return sizeof(mla_decode_params_t); }

double mla_softmax_scale(int qk_head_dim, const mla_rope_cfg_t* cfg) {
    if (!cfg || qk_head_dim < 1) return -1.0;
    double s = 1.0 / sqrt((double)qk_head_dim);
    if (cfg->max_seq_len > cfg->original_seq_len) {
        const double m = 0.1 * cfg->mscale * log(cfg->factor) + 1.0;
        s = s * m * m;
    }
    return s;
}

int mla_rope_freqs(const mla_rope_cfg_t* cfg, float* table, void* stream) {
    g_err[0] = 0;
    if (!cfg || !table) return fail(MLA_ERR_INVALID_ARG, "mla_rope_freqs: null cfg or table");
    if (cfg->rope_dim != 64) return fail(MLA_ERR_UNSUPPORTED, "mla_rope_freqs: rope_dim must be 64");
    if (cfg->max_seq_len < 1 || cfg->original_seq_len < 1 || cfg->reserved != 0)
        return fail(MLA_ERR_INVALID_ARG, "mla_rope_freqs: bad lengths");
    if (!(cfg->theta > 1.0) || !(cfg->factor > 0.0) || !(cfg->beta_fast > 0.0) || !(cfg->beta_slow > 0.0))
        return fail(MLA_ERR_INVALID_ARG, "mla_rope_freqs: theta must exceed 1; factor and betas positive");
    if (mla::launch_rope_freqs(*cfg, table, (hipStream_t)stream) != hipSuccess)
        return fail(MLA_ERR_HIP, "mla_rope_freqs: launch failed");
    return MLA_OK;
}

int mla_decode_num_splits(int B, int H, int K, int dtype_act, int num_cus) {
    if (num_cus == 0 && query_num_cus(&num_cus) != 0) return -1;
    mla::Plan pl;
    if ((dtype_act != MLA_DTYPE_BF16 && dtype_act != MLA_DTYPE_F32) || !make_plan(B, H, K, dtype_act, num_cus, 0, &pl))
        return -1;
    return pl.splits;
}

size_t mla_decode_workspace_size(int B, int H, int K, int dtype_act, int dtype_w, int num_cus, int num_splits) {
    if (B < 1 || B > kMaxBatch || H < 1 || H > kMaxHeads || K < 1) return 0;
    if ((dtype_act != MLA_DTYPE_BF16 && dtype_act != MLA_DTYPE_F32) ||
        (dtype_w != MLA_DTYPE_BF16 && dtype_w != MLA_DTYPE_F32))
        return 0;
    if (num_cus == 0 && query_num_cus(&num_cus) != 0) return 0;
    mla::Plan pl;
    if (!make_plan(B, H, K, dtype_act, num_cus, num_splits, &pl)) return 0;
    return mla::workspace_layout(B, H, K, pl.bf16_path, pl.splits, nullptr, nullptr);
}

int mla_decode_attn(mla_decode_params_t* p, void* stream) {
    g_err[0] = 0;
    if (!p) return fail(MLA_ERR_INVALID_ARG, "null params");
    p->validate_status = 0;
    if (p->d_nope != 128 || p->d_rope != 64 || p->d_v != 128 || p->kv_rank != 512)
        return fail(MLA_ERR_UNSUPPORTED, "dims must be d_nope=128, d_rope=64, d_v=128, kv_rank=512");
    auto okdt = [](int d) { return d == MLA_DTYPE_BF16 || d == MLA_DTYPE_F32; };
    if (!okdt(p->dtype_act) || !okdt(p->dtype_w) || !okdt(p->dtype_out))
        return fail(MLA_ERR_UNSUPPORTED, "unknown dtype");
    if (p->B < 1 || p->B > kMaxBatch || p->H < 1 || p->H > kMaxHeads || p->K < 1)
        return fail(MLA_ERR_INVALID_ARG, "sizes out of range: B=%d H=%d K=%d", p->B, p->H, p->K);
    if (p->max_cache_len < 1 || p->max_cache_len > kMaxCacheLen)
        return fail(MLA_ERR_INVALID_ARG, "max_cache_len must be in [1, %d]", kMaxCacheLen);
    if (p->rope_table_len < 1) return fail(MLA_ERR_INVALID_ARG, "rope_table_len must be >= 1");
    if (!(p->softmax_scale > 0.f) || !isfinite(p->softmax_scale))
        return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be positive and finite");
    if (p->num_splits < 0 || p->num_splits > kMaxSplits || p->num_cus < 0)
        return fail(MLA_ERR_INVALID_ARG, "num_splits must be in [0, %d], num_cus >= 0", kMaxSplits);
    if (p->flags & ~MLA_FLAG_VALIDATE) return fail(MLA_ERR_INVALID_ARG, "unknown flags");
    const void* ptrs[] = {p->q_nope, p->q_pe, p->w_uk, p->w_uv, p->kv_cache, p->pe_cache,
                          p->topk_indices, p->cache_lens, p->rope_table, p->out, p->workspace};
    const char* names[] = {"q_nope", "q_pe", "w_uk", "w_uv", "kv_cache", "pe_cache",
                           "topk_indices", "cache_lens", "rope_table", "out", "workspace"};
    for (int i = 0; i < 11; ++i) {
        if (!ptrs[i]) return fail(MLA_ERR_INVALID_ARG, "%s is null", names[i]);
        if (!aligned16(ptrs[i])) return fail(MLA_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
    }
    if (p->lse_out && ((uintptr_t)p->lse_out & 3u)) return fail(MLA_ERR_INVALID_ARG, "lse_out misaligned");
    if ((p->kv_new == nullptr) != (p->pe_new == nullptr))
        return fail(MLA_ERR_INVALID_ARG, "kv_new and pe_new must both be set (fused append) or both be null");
    if (p->kv_new) {
        if (!aligned16(p->kv_new) || !aligned16(p->pe_new))
            return fail(MLA_ERR_INVALID_ARG, "kv_new and pe_new must be 16-byte aligned");
        if (p->kv_new_stride_b < 0 || (p->kv_new_stride_b & 7) || p->pe_new_stride_b < 0 || (p->pe_new_stride_b & 7))
            return fail(MLA_ERR_INVALID_ARG, "kv_new/pe_new strides must be non-negative multiples of 8");
        if (p->B > 1 && (p->kv_new_stride_b < 512 || p->pe_new_stride_b < 64))
            return fail(MLA_ERR_INVALID_ARG, "kv_new/pe_new batch stride smaller than its row");
    }
    const int64_t vec_strides[] = {p->q_nope_stride_b, p->q_nope_stride_h, p->q_pe_stride_b, p->q_pe_stride_h,
                                   p->w_uk_stride_h, p->w_uv_stride_h, p->kv_stride_b, p->kv_stride_t,
                                   p->pe_stride_b, p->pe_stride_t};
    for (int64_t st : vec_strides)
        if (st < 0 || (st & 7)) return fail(MLA_ERR_INVALID_ARG, "q/weight/cache strides must be non-negative multiples of 8");
    const int64_t other[] = {p->idx_stride_b, p->out_stride_b, p->out_stride_h};
    for (int64_t st : other)
        if (st < 0) return fail(MLA_ERR_INVALID_ARG, "negative stride");
    if (p->kv_stride_t < 512 || p->pe_stride_t < 64 || p->q_nope_stride_h < 128 || p->q_pe_stride_h < 64 ||
        p->w_uk_stride_h < 128 * 512 || p->w_uv_stride_h < 128 * 512 || p->idx_stride_b < p->K ||
        p->out_stride_h < 128)
        return fail(MLA_ERR_INVALID_ARG, "a stride is smaller than the row it steps over");
    // the attention kernel addresses one sequence's cache rows with 32-bit byte offsets
    if ((int64_t)(p->max_cache_len - 1) * p->kv_stride_t * 2 + 1024 > INT32_MAX ||
        (int64_t)(p->max_cache_len - 1) * p->pe_stride_t * 2 + 128 > INT32_MAX)
        return fail(MLA_ERR_UNSUPPORTED, "one sequence's cache rows span more than 2 GiB");
    // the absorption copies 128 sequences' queries at a time with 32-bit byte offsets
    if ((int64_t)127 * p->q_nope_stride_b * 2 + 256 > INT32_MAX)
        return fail(MLA_ERR_UNSUPPORTED, "q_nope batch stride too large");

    int num_cus = p->num_cus;
    if (num_cus == 0 && query_num_cus(&num_cus) != 0) return fail(MLA_ERR_HIP, "cannot query the device");
    mla::Plan plan;
    if (!make_plan(p->B, p->H, p->K, p->dtype_act, num_cus, p->num_splits, &plan))
        return fail(MLA_ERR_INVALID_ARG, "no launch plan (fp32 activations take num_splits 0 or 1)");
    mla::Work w;
    const size_t need = mla::workspace_layout(p->B, p->H, p->K, plan.bf16_path, plan.splits, p->workspace, &w);
    if (p->workspace_size < need)
        return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", p->workspace_size, need);

    hipStream_t s = (hipStream_t)stream;
    const bool validate = (p->flags & MLA_FLAG_VALIDATE) != 0;
    hipEvent_t* ev = (hipEvent_t*)p->profile_events;
    if (validate && hipMemsetAsync(w.status, 0, 4, s) != hipSuccess)
        return fail(MLA_ERR_HIP, "hipMemsetAsync failed");
    hipError_t e;
    if (ev && hipEventRecord(ev[0], s) != hipSuccess) return fail(MLA_ERR_HIP, "hipEventRecord failed");
    if ((e = mla::launch_prep(*p, plan, w, validate, s)) != hipSuccess)
        return fail(MLA_ERR_HIP, "prep launch: %s", hipGetErrorString(e));
    if (ev && (hipEventRecord(ev[1], s) != hipSuccess || hipEventRecord(ev[2], s) != hipSuccess))
        return fail(MLA_ERR_HIP, "hipEventRecord failed");
    if ((e = mla::launch_attn(*p, plan, w, s)) != hipSuccess)
        return fail(MLA_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
    if (ev && (hipEventRecord(ev[3], s) != hipSuccess || hipEventRecord(ev[4], s) != hipSuccess))
        return fail(MLA_ERR_HIP, "hipEventRecord failed");
    if ((e = mla::launch_merge(*p, plan, w, s)) != hipSuccess)
        return fail(MLA_ERR_HIP, "merge launch: %s", hipGetErrorString(e));
    if (ev && hipEventRecord(ev[5], s) != hipSuccess) return fail(MLA_ERR_HIP, "hipEventRecord failed");
    if (validate) {
        uint32_t st = 0;
        if (hipMemcpyAsync(&st, w.status, 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess)
            return fail(MLA_ERR_HIP, "validation readback failed");
        p->validate_status = st;
        if (st) return fail(MLA_ERR_INVALID_INDEX, "invalid selection or cache length (status 0x%x)", st);
    }
    return MLA_OK;
}

}  // extern "C"
