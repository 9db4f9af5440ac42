// Merge of split-KV partials and the W_UV up-projection, plus the fp32
// attention used when the activations are fp32.
//
// Sources (atlas pages on DeepSeek-V3.2-Exp sparse latent attention):
//   page "Rotated query part", excerpt mla-decode: softmax over the selected
//   scores, the weighted latent sum and the per-head W_UV up-projection
//   (x . W_UV[h]^T over the 512 latent columns, 128 outputs per head).
//   Merging independently normalised partials by their log-sum-exp is the
//   standard split-softmax identity; the pages do not partition the keys.
#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

// ---------------------------------------------------------------------------
// bf16 path: out[b, h, :] = W_UV[h] . sum_s w_{b,s} o_s[b, h, :]
//   w_{b,s} = 2^(lse_s - M) / sum_s' 2^(lse_s' - M),  M = max_s lse_s.
// Workgroup (head h, output half dh) covers every sequence with 8 waves (two
// per SIMD, so that one wave's loads overlap the other's work).  bf16 MFMA
// with M = sequences (32 per step), N = 64 outputs, K = 512 latent columns
// split over the 8 waves (64 each) and reduced through LDS.
// ---------------------------------------------------------------------------
struct MergeArgs {
    int B, H, S;
    const bf16* opart;
    const float* lsepart;
    const void* w_uv; long long wv_sh;
    void* out; long long out_sb, out_sh;
    float* lse_out;
};

constexpr int MW = 8;            // waves per merge workgroup
constexpr int MKB = RANK / (16 * MW);   // K steps (16 latent columns) per wave

template <typename WT, typename OutT>
__global__ __launch_bounds__(64 * MW) void merge_kernel(MergeArgs a) {
    __shared__ float red[MW * 2 * 16 * 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    // the two output halves of one head sit 8 ids apart (same XCD, shared L2)
    const int id = blockIdx.x;
    const int xcd = id & 7, k8 = id >> 3;
    const int dh = k8 & 1, h = (k8 >> 1) * 8 + xcd;
    if (h >= a.H) return;
    const int col0 = (RANK / MW) * wave;

    // The partials are consumed in units of (32 sequences, 2 splits); unit
    // u + 1 is loaded while unit u is processed, across the reduction of a
    // finished batch too, so the memory system never idles between batches.
    // Splits are combined with a running maximum (rescaling what was summed
    // when the maximum grows).
    const int G = (a.S + 1) / 2;                     // split pairs per sequence
    const int U = ((a.B + 31) / 32) * G;
    auto load_unit = [&](int u, bf16x8 (&v)[2][MKB], float (&ls)[2]) {
        const int bA = 32 * (u / G) + l32, s0 = 2 * (u % G);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int s = s0 + t;
            const bool ok = bA < a.B && s < a.S;
            const long long row = ((long long)h * a.B + bA) * a.S + s;   // head-major partials
            ls[t] = ok ? a.lsepart[row] : -INFINITY;
            const bf16* src = a.opart + row * RANK + col0 + 8 * g;
#pragma unroll
            for (int kb = 0; kb < MKB; ++kb) v[t][kb] = ok ? *(const bf16x8*)(src + 16 * kb) : bf16x8{};
        }
    };
    bf16x8 vc[2][MKB], vn[2][MKB];
    float lc[2], ln[2];
    load_unit(0, vc, lc);           // first partials in flight together with the weights
    // fp32 weights enter as bf16 hi + lo parts (two MFMAs each).
    constexpr int NP = sizeof(WT) == 4 ? 2 : 1;
    const WT* W = (const WT*)a.w_uv + h * a.wv_sh;
    bf16x8 bw[NP][2][MKB];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int d = 64 * dh + 32 * nb + l32;
#pragma unroll
        for (int kb = 0; kb < MKB; ++kb) {
            const WT* src = W + d * RANK + col0 + 16 * kb + 8 * g;
            if constexpr (NP == 2) {
                const f32x4 x0 = *(const f32x4*)src, x1 = *(const f32x4*)(src + 4);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float wv = j < 4 ? x0[j] : x1[j - 4];
                    const bf16 hi = (bf16)wv;
                    bw[0][nb][kb][j] = hi;
                    bw[NP - 1][nb][kb][j] = (bf16)(wv - (float)hi);
                }
            } else {
                bw[0][nb][kb] = load8_bf16<WT>(src);
            }
        }
    }

    float M = -INFINITY, Wsum = 0.f;
    float xs[MKB][8];
#pragma unroll
    for (int kb = 0; kb < MKB; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) xs[kb][j] = 0.f;
    for (int u = 0; u < U; ++u) {
        if (u + 1 < U) load_unit(u + 1, vn, ln);
        // fold the current unit's two splits into the running sums
        const float Mn = fmaxf(M, fmaxf(lc[0], lc[1]));
        const float sc = M == Mn ? 1.f : exp2f(M - Mn);
        const float w0 = exp2f(lc[0] - Mn), w1 = exp2f(lc[1] - Mn);
        Wsum = Wsum * sc + w0 + w1;
#pragma unroll
        for (int kb = 0; kb < MKB; ++kb)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                xs[kb][j] = fmaf(w1, (float)vc[1][kb][j], fmaf(w0, (float)vc[0][kb][j], xs[kb][j] * sc));
        M = Mn;
        if (u % G == G - 1) {
            // batch of 32 sequences complete: A operand = merged latent (bf16,
            // zero past the batch), MFMAs with every lane active, reduction
            // over the 8 waves' column ranges, output
            const int b0 = 32 * (u / G), bA = b0 + l32;
            const float invW = 1.f / Wsum;
            bf16x8 av[MKB];
#pragma unroll
            for (int kb = 0; kb < MKB; ++kb)
#pragma unroll
                for (int j = 0; j < 8; ++j) av[kb][j] = bA < a.B ? f2bf(xs[kb][j] * invW) : (bf16)0.f;
            f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int kb = 0; kb < MKB; ++kb)
#pragma unroll
                    for (int pp = 0; pp < NP; ++pp) acc[nb] = mfma32(av[kb], bw[pp][nb][kb], acc[nb]);
            if (dh == 0 && wave == 0 && g == 0 && bA < a.B && a.lse_out)
                a.lse_out[(long long)bA * a.H + h] = LN2 * (M + log2f(Wsum));
            __syncthreads();                        // previous batch's reads of red[] done
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int i = 0; i < 16; ++i) red[((wave * 2 + nb) * 16 + i) * 64 + lane] = acc[nb][i];
            __syncthreads();
            // 32 sequences x 64 outputs; D element (row 8(i/4) + 4gg + i%4,
            // column 32 nb + n) sits at red[w][nb][i][32 gg + n]
#pragma unroll
            for (int k = 0; k < 2048 / (64 * MW); ++k) {
                const int e = tid + 64 * MW * k;
                const int dl = e & 63, bl = e >> 6;
                const int nb = dl >> 5, n = dl & 31;
                const int i = 4 * (bl >> 3) + (bl & 3), gg = (bl >> 2) & 1;
                const int lnn = gg * 32 + n;
                float v = 0.f;
#pragma unroll
                for (int w = 0; w < MW; ++w) v += red[((w * 2 + nb) * 16 + i) * 64 + lnn];
                const int bo = b0 + bl;
                if (bo < a.B)
                    ((OutT*)a.out)[bo * a.out_sb + h * a.out_sh + 64 * dh + dl] = from_f32<OutT>(v);
            }
            M = -INFINITY;
            Wsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < MKB; ++kb)
#pragma unroll
                for (int j = 0; j < 8; ++j) xs[kb][j] = 0.f;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            lc[t] = ln[t];
#pragma unroll
            for (int kb = 0; kb < MKB; ++kb) vc[t][kb] = vn[t][kb];
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 path.  attn_f32: one workgroup per (sequence, head); scores, softmax
// and the weighted latent sum in fp32 over the compacted selection, 256 rows
// at a time with an online rescale between chunks.  Writes the normalised
// latent sum (fp32) and the log2-domain sum-exp.
// ---------------------------------------------------------------------------
struct AttnF32Args {
    int B, H, K;
    float scale;
    const float* qt;
    const int32_t* list;
    const int32_t* counts;
    const float* kv; long long kv_sb, kv_st;
    const float* pe; long long pe_sb, pe_st;
    float* olat;
    float* lse2;
};

__global__ __launch_bounds__(256) void attn_f32_kernel(AttnF32Args a) {
    __shared__ float qs[ROW];
    __shared__ float ps[256];
    __shared__ float wred[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x / a.H, h = blockIdx.x % a.H;
    const float* q = a.qt + ((long long)b * a.H + h) * ROW;
    for (int i = tid; i < ROW; i += 256) qs[i] = q[i];
    __syncthreads();
    const int cnt = a.counts[b];
    const int32_t* list = a.list + (long long)b * a.K;
    float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
    for (int base = 0; base < cnt; base += 256) {
        const int j = base + tid;
        float sc = -INFINITY;
        if (j < cnt) {
            const long long t = list[j] - 1;   // entries are 1-based
            const float* c = a.kv + b * a.kv_sb + t * a.kv_st;
            const float* r = a.pe + b * a.pe_sb + t * a.pe_st;
            float acc = 0.f;
            for (int k = 0; k < RANK; ++k) acc = fmaf(qs[k], c[k], acc);
            for (int k = 0; k < D_ROPE; ++k) acc = fmaf(qs[RANK + k], r[k], acc);
            sc = acc * a.scale;
        }
        float cm = wave_max(sc);
        if (lane == 0) wred[wave] = cm;
        __syncthreads();
        cm = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
        __syncthreads();
        const float mn = fmaxf(m, cm);
        const float alpha = m == -INFINITY ? 0.f : expf(m - mn);
        const float p = j < cnt ? expf(sc - mn) : 0.f;
        ps[tid] = p;
        float psum = wave_sum(p);
        if (lane == 0) wred[wave] = psum;
        __syncthreads();
        psum = wred[0] + wred[1] + wred[2] + wred[3];
        l = l * alpha + psum;
        o0 *= alpha;
        o1 *= alpha;
        m = mn;
        const int nrow = min(256, cnt - base);
        for (int r = 0; r < nrow; ++r) {
            const long long t = list[base + r] - 1;
            const float* c = a.kv + b * a.kv_sb + t * a.kv_st;
            const float pr = ps[r];
            o0 = fmaf(pr, c[tid], o0);
            o1 = fmaf(pr, c[tid + 256], o1);
        }
        __syncthreads();
    }
    const float inv = l > 0.f ? 1.f / l : NAN;
    float* dst = a.olat + ((long long)b * a.H + h) * RANK;
    dst[tid] = o0 * inv;
    dst[tid + 256] = o1 * inv;
    if (tid == 0) a.lse2[(long long)b * a.H + h] = (m + logf(l)) * LOG2E;
}

// fp32 up-projection: one thread per (sequence, head, output feature).
template <typename WT, typename OutT>
__global__ __launch_bounds__(256) void uproj_f32_kernel(MergeArgs a, const float* olat) {
    const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
    if (e >= (long long)a.B * a.H * D_V) return;
    const int d = (int)(e % D_V), h = (int)((e / D_V) % a.H), b = (int)(e / D_V / a.H);
    const float* x = olat + ((long long)b * a.H + h) * RANK;
    const WT* w = (const WT*)a.w_uv + h * a.wv_sh + (long long)d * RANK;
    float acc = 0.f;
    for (int c = 0; c < RANK; ++c) acc = fmaf(x[c], to_f32(w[c]), acc);
    ((OutT*)a.out)[b * a.out_sb + h * a.out_sh + d] = from_f32<OutT>(acc);
    if (d == 0 && a.lse_out) a.lse_out[(long long)b * a.H + h] = a.lsepart[(long long)b * a.H + h] * LN2;
}

hipError_t launch_attn_f32(const mla_decode_params_t& p, const Work& w, hipStream_t s) {
    AttnF32Args a{};
    a.B = p.B; a.H = p.H; a.K = p.K; a.scale = p.softmax_scale;
    a.qt = (const float*)w.qt; a.list = w.list; a.counts = w.counts;
    a.kv = (const float*)p.kv_cache; a.kv_sb = p.kv_stride_b; a.kv_st = p.kv_stride_t;
    a.pe = (const float*)p.pe_cache; a.pe_sb = p.pe_stride_b; a.pe_st = p.pe_stride_t;
    a.olat = (float*)w.opart; a.lse2 = w.lsepart;
    hipLaunchKernelGGL(attn_f32_kernel, dim3(p.B * p.H), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_merge(const mla_decode_params_t& p, const Plan& plan, const Work& w, hipStream_t s) {
    MergeArgs a{};
    a.B = p.B; a.H = p.H; a.S = plan.splits;
    a.opart = (const bf16*)w.opart; a.lsepart = w.lsepart;
    a.w_uv = p.w_uv; a.wv_sh = p.w_uv_stride_h;
    a.out = p.out; a.out_sb = p.out_stride_b; a.out_sh = p.out_stride_h;
    a.lse_out = p.lse_out;
    const bool wf = p.dtype_w == MLA_DTYPE_F32, of = p.dtype_out == MLA_DTYPE_F32;
    if (plan.bf16_path) {
        const dim3 grid(((p.H + 7) / 8) * 16), block(64 * MW);
        if (wf && of) hipLaunchKernelGGL((merge_kernel<float, float>), grid, block, 0, s, a);
        else if (wf) hipLaunchKernelGGL((merge_kernel<float, bf16>), grid, block, 0, s, a);
        else if (of) hipLaunchKernelGGL((merge_kernel<bf16, float>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((merge_kernel<bf16, bf16>), grid, block, 0, s, a);
    } else {
        const long long n = (long long)p.B * p.H * D_V;
        const dim3 grid((unsigned)((n + 255) / 256)), block(256);
        const float* olat = (const float*)w.opart;
        if (wf && of) hipLaunchKernelGGL((uproj_f32_kernel<float, float>), grid, block, 0, s, a, olat);
        else if (wf) hipLaunchKernelGGL((uproj_f32_kernel<float, bf16>), grid, block, 0, s, a, olat);
        else if (of) hipLaunchKernelGGL((uproj_f32_kernel<bf16, float>), grid, block, 0, s, a, olat);
        else hipLaunchKernelGGL((uproj_f32_kernel<bf16, bf16>), grid, block, 0, s, a, olat);
    }
    return hipGetLastError();
}

}  // namespace mla
