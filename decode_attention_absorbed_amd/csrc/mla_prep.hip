// Rotation table and the per-call preparation kernel of the MLA decode step.
//
// Sources (atlas pages on DeepSeek-V3.2-Exp sparse latent attention):
//   rotation table:  "Transformer blocks / RoPE coefficients", excerpt rope
//   query rotation:  "Rotated query part", excerpt apply-rope (interleaved pairs)
//   absorption:      "Rotated query part", excerpt mla-decode (q_nope . W_UK[h])
//   selection:       "Rotated query part", excerpt mla-decode (index mask; one
//                    set per sequence, shared by every head)
#include <math.h>

#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

// ---------------------------------------------------------------------------
// (cos, sin)(t * theta'_i), angles in double precision.
// theta_i = theta^(-2i/d); with interpolation (T_max > T_0) theta'_i =
// theta_i/factor * ramp_i + theta_i * (1 - ramp_i), ramp linear in i between
// the YaRN correction dimensions floor(D(beta_fast)) and ceil(D(beta_slow)).
// ---------------------------------------------------------------------------
struct RopeArgs {
    int T, d, T0;
    double theta, factor, beta_fast, beta_slow;
    float* table;
};

__device__ double correction_dim(double beta, int d, int T0, double theta) {
    return d * log((double)T0 / (2.0 * M_PI * beta)) / (2.0 * log(theta));
}

__global__ __launch_bounds__(256) void rope_freqs_kernel(RopeArgs a) {
    const int half = a.d / 2;
    const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (long long)a.T * half) return;
    const int t = (int)(e / half), i = (int)(e % half);
    double f = pow(a.theta, -(2.0 * i) / a.d);
    if (a.T > a.T0) {
        double lo = floor(correction_dim(a.beta_fast, a.d, a.T0, a.theta));
        double hi = ceil(correction_dim(a.beta_slow, a.d, a.T0, a.theta));
        lo = fmax(lo, 0.0);
        hi = fmin(hi, (double)(a.d - 1));
        if (hi == lo) hi += 0.001;
        double ramp = fmin(fmax((i - lo) / (hi - lo), 0.0), 1.0);
        f = f / a.factor * ramp + f * (1.0 - ramp);
    }
    const double ang = (double)t * f;
    a.table[2 * e] = (float)cos(ang);
    a.table[2 * e + 1] = (float)sin(ang);
}

hipError_t launch_rope_freqs(const mla_rope_cfg_t& cfg, float* table, hipStream_t s) {
    RopeArgs a{cfg.max_seq_len, cfg.rope_dim, cfg.original_seq_len, cfg.theta, cfg.factor,
               cfg.beta_fast, cfg.beta_slow, table};
    const long long n = (long long)cfg.max_seq_len * (cfg.rope_dim / 2);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(rope_freqs_kernel, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Preparation kernel.  Blocks [0, n_absorb) compute the absorbed content
// query q_abs = q_nope . W_UK[h] into Q~[b, h, 0:512]; blocks
// [n_absorb, n_absorb + B) handle one sequence each: compact the selection
// and rotate the rotary query into Q~[b, h, 512:576].
// ---------------------------------------------------------------------------
struct PrepArgs {
    int B, H, K, Lmax, Trope, n_absorb, validate;
    const void* q_nope; long long qn_sb, qn_sh;
    const void* q_pe;   long long qp_sb, qp_sh;
    const void* w_uk;   long long wk_sh;
    const int32_t* idx; long long idx_sb;
    const int32_t* cache_lens;
    const float* rope_table;
    void* qt;
    int32_t* list;
    int32_t* counts;
    uint32_t* status;
};

// Block-wide exclusive scan of one int per thread (256 threads).
__device__ int block_exclusive_scan(int v, int* total, int* lds_wave) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int inc = v;
    for (int o = 1; o < 64; o <<= 1) {
        int n = __shfl_up(inc, o);
        if (lane >= o) inc += n;
    }
    if (lane == 63) lds_wave[wave] = inc;
    __syncthreads();
    int base = 0, tot = 0;
    for (int w = 0; w < 4; ++w) {
        int x = lds_wave[w];
        if (w < wave) base += x;
        tot += x;
    }
    *total = tot;
    return base + inc - v;
}

// Selection compaction for sequence b: every position listed in the index
// row (minus -1 slots and entries outside [0, L_b)), once, ascending.
// Dynamic LDS holds a bitmap of ceil(L_max / 32) words.
template <typename QtT, typename ActT>
__device__ void prep_sequence(const PrepArgs& a, int b, uint32_t* bm) {
    __shared__ int lds_wave[4];
    __shared__ uint32_t lds_status;
    const int tid = threadIdx.x;
    const int L = a.cache_lens[b];
    uint32_t status = 0;
    if (L < 1 || L > a.Lmax || L > a.Trope) status |= BAD_CACHE_LEN;
    const int Lc = L < 0 ? 0 : (L > a.Lmax ? a.Lmax : L);
    const int nwords = (Lc + 31) >> 5;
    if (tid == 0) lds_status = 0;
    for (int w = tid; w < nwords; w += 256) bm[w] = 0u;
    __syncthreads();
    const int32_t* row = a.idx + (long long)b * a.idx_sb;
    for (int j = tid; j < a.K; j += 256) {
        const int v = row[j];
        if (v == -1) continue;
        if (v < 0 || v >= L) { status |= BAD_INDEX_RANGE; continue; }
        if (v >= Lc) continue;                        // cache length already flagged
        const uint32_t bit = 1u << (v & 31);
        const uint32_t old = atomicOr(&bm[v >> 5], bit);
        if (old & bit) status |= BAD_DUPLICATE;
    }
    __syncthreads();
    const int wpt = (nwords + 255) / 256;
    const int w0 = min(tid * wpt, nwords), w1 = min(w0 + wpt, nwords);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(bm[w]);
    int total;
    int off = block_exclusive_scan(cnt, &total, lds_wave);
    int32_t* out = a.list + (long long)b * a.K;
    for (int w = w0; w < w1; ++w) {
        uint32_t bits = bm[w];
        while (bits) {
            const int pos = (w << 5) + __ffs(bits) - 1;
            out[off++] = pos;
            bits &= bits - 1;
        }
    }
    if (tid == 0) {
        a.counts[b] = total;
        if (total == 0) status |= BAD_EMPTY;
    }
    // Rotary query at p_b = L_b - 1: pairs (2i, 2i+1) are one complex number.
    const int p = min(max(L - 1, 0), a.Trope - 1);
    const float* cs = a.rope_table + (long long)p * D_ROPE;
    for (int e = tid; e < a.H * (D_ROPE / 2); e += 256) {
        const int h = e >> 5, i = e & 31;
        const ActT* q = (const ActT*)a.q_pe + b * a.qp_sb + h * a.qp_sh;
        const float x0 = to_f32(q[2 * i]), x1 = to_f32(q[2 * i + 1]);
        const float c = cs[2 * i], s = cs[2 * i + 1];
        QtT* dst = (QtT*)a.qt + ((long long)b * a.H + h) * ROW + RANK;
        dst[2 * i] = from_f32<QtT>(x0 * c - x1 * s);
        dst[2 * i + 1] = from_f32<QtT>(x0 * s + x1 * c);
    }
    if (status) atomicOr(&lds_status, status);
    __syncthreads();
    if (tid == 0 && lds_status && a.validate) atomicOr(a.status, lds_status);
}

// q_abs for head h, latent columns [256*half, 256*half + 256), every
// sequence, with bf16 MFMA: M = sequences (32 per block), N = latent
// columns, K = the 128 content features.  Wave w owns 64 columns.  fp32
// weights are split into bf16 hi + lo parts (two MFMAs each), so they enter
// with ~16 significant bits instead of 8.
template <typename WT>
__device__ void absorb_bf16(const PrepArgs& a, int h, int half) {
    constexpr int NP = sizeof(WT) == 4 ? 2 : 1;       // weight parts
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const int c0 = 256 * half + 64 * wave;
    const WT* W = (const WT*)a.w_uk + h * a.wk_sh;
    // B operand: B[k = d][n = c] = W_UK[h][d][c]; lane holds d = 16kb + 8g + j.
    bf16x8 bw[NP][2][8];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int c = c0 + 32 * nb + l32;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int d = 16 * kb + 8 * g + j;
                const float wv = to_f32(W[d * RANK + c]);
                const bf16 hi = (bf16)wv;
                bw[0][nb][kb][j] = hi;
                if constexpr (NP == 2) bw[NP - 1][nb][kb][j] = (bf16)(wv - (float)hi);
            }
        }
    }
    for (int b0 = 0; b0 < a.B; b0 += 32) {
        const int bA = b0 + l32;
        bf16x8 aq[8];
        if (bA < a.B) {
            const bf16* q = (const bf16*)a.q_nope + bA * a.qn_sb + h * a.qn_sh;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) aq[kb] = *(const bf16x8*)(q + 16 * kb + 8 * g);
        } else {
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) aq[kb] = bf16x8{};
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            f32x16 acc = {};
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) acc = mfma32(aq[kb], bw[pp][nb][kb], acc);
            const int c = c0 + 32 * nb + l32;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int bo = b0 + 8 * (i >> 2) + 4 * g + (i & 3);
                if (bo < a.B) ((bf16*)a.qt)[((long long)bo * a.H + h) * ROW + c] = f2bf(acc[i]);
            }
        }
    }
}

// fp32 variant: thread t owns latent column 256*half + t.
template <typename WT>
__device__ void absorb_f32(const PrepArgs& a, int h, int half) {
    const int c = 256 * half + threadIdx.x;
    const WT* W = (const WT*)a.w_uk + h * a.wk_sh;
    float wc[D_NOPE];
#pragma unroll
    for (int d = 0; d < D_NOPE; ++d) wc[d] = to_f32(W[d * RANK + c]);
    for (int b = 0; b < a.B; ++b) {
        const float* q = (const float*)a.q_nope + b * a.qn_sb + h * a.qn_sh;
        float acc = 0.f;
#pragma unroll
        for (int d = 0; d < D_NOPE; ++d) acc = fmaf(q[d], wc[d], acc);
        ((float*)a.qt)[((long long)b * a.H + h) * ROW + c] = acc;
    }
}

template <typename ActT, typename WT>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
    extern __shared__ uint32_t dyn_lds[];
    const int bid = blockIdx.x;
    if (bid < a.n_absorb) {
        const int h = bid >> 1, half = bid & 1;
        if constexpr (sizeof(ActT) == 2) absorb_bf16<WT>(a, h, half);
        else absorb_f32<WT>(a, h, half);
    } else {
        prep_sequence<ActT, ActT>(a, bid - a.n_absorb, dyn_lds);
    }
}

hipError_t launch_prep(const mla_decode_params_t& p, const Plan& plan, const Work& w, bool validate,
                       hipStream_t s) {
    PrepArgs a{};
    a.B = p.B; a.H = p.H; a.K = p.K; a.Lmax = p.max_cache_len; a.Trope = p.rope_table_len;
    a.n_absorb = 2 * p.H; a.validate = validate ? 1 : 0;
    a.q_nope = p.q_nope; a.qn_sb = p.q_nope_stride_b; a.qn_sh = p.q_nope_stride_h;
    a.q_pe = p.q_pe; a.qp_sb = p.q_pe_stride_b; a.qp_sh = p.q_pe_stride_h;
    a.w_uk = p.w_uk; a.wk_sh = p.w_uk_stride_h;
    a.idx = p.topk_indices; a.idx_sb = p.idx_stride_b;
    a.cache_lens = p.cache_lens; a.rope_table = p.rope_table;
    a.qt = w.qt; a.list = w.list; a.counts = w.counts; a.status = w.status;
    const size_t lds = (size_t)((p.max_cache_len + 31) / 32) * 4;
    const dim3 grid(a.n_absorb + p.B), block(256);
    const bool wf = p.dtype_w == MLA_DTYPE_F32;
    if (lds > 48 * 1024) {
        const void* fns[] = {(const void*)prep_kernel<bf16, float>, (const void*)prep_kernel<bf16, bf16>,
                             (const void*)prep_kernel<float, float>, (const void*)prep_kernel<float, bf16>};
        for (const void* f : fns) {
            hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
    }
    if (plan.bf16_path) {
        if (wf) hipLaunchKernelGGL((prep_kernel<bf16, float>), grid, block, lds, s, a);
        else hipLaunchKernelGGL((prep_kernel<bf16, bf16>), grid, block, lds, s, a);
    } else {
        if (wf) hipLaunchKernelGGL((prep_kernel<float, float>), grid, block, lds, s, a);
        else hipLaunchKernelGGL((prep_kernel<float, bf16>), grid, block, lds, s, a);
    }
    return hipGetLastError();
}

}  // namespace mla
