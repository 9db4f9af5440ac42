// Split-KV sparse attention over the latent cache (bf16 MFMA, fp32 accumulation).
//
// Computes, for one sequence b, one split s of its selected positions and a
// group of 32*NHG heads, the partial softmax-weighted latent sum
//   o[h, :] = sum_t exp2(x[h,t] - m[h]) C[b,t,:],  l[h] = sum_t exp2(x[h,t] - m[h]),
//   x[h,t] = scale * log2(e) * (Q~[b,h,:] . [C[b,t,:] ; R[b,t,:]])
// and writes o / l (bf16) and m + log2(l).  The scores are the latent plus
// rotary dot products of the MQA decode branch; positions outside the
// selection never enter (their additive mask is -inf, exp2 gives 0).
// Source: atlas page "Rotated query part" (also "Query content heads",
// "Attention weights"), excerpt mla-decode; split-KV partitioning and the
// online softmax are this library's, not the pages'.
//
// Workgroup: 4 waves (one per SIMD), 32*NHG heads, tiles of R = 32*RG
// gathered rows staged in LDS by direct global->LDS copies.
//   QK^T: wave (hg, rg) computes S^T[32 rows][32 heads] = K_tile . Q^T with
//         v_mfma_f32_32x32x16_bf16 (M = rows, N = heads, K = 576); its 32
//         heads of Q~ stay in registers for the whole split.
//   softmax: per head (one lane column), in-lane max over 16 rows plus one
//         cross-half shuffle; lazy rescaling (the running max only moves when
//         a score exceeds it by 2^8).
//   PV:   wave w owns latent columns [128w, 128w+128) for every head of the
//         workgroup: O^T[c][h] += V^T[c][t] . P^T[t][h], V^T read with
//         ds_read_b64_tr_b16, P^T shared through LDS.
#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

struct AttnArgs {
    int B, H, K, S, HG;
    float scale_log2;
    const bf16* qt;
    const int32_t* list;
    const int32_t* counts;
    const bf16* kv; long long kv_sb, kv_st;
    const bf16* pe; long long pe_sb, pe_st;
    bf16* opart;
    float* lsepart;
};

template <int NHG> struct AttnCfg {
    static constexpr int RG = (NHG == 4) ? 1 : 2;     // row groups of 32 in a tile
    static constexpr int R = 32 * RG;                  // rows per tile
    static constexpr int RW = R / 4;                   // rows staged by each wave
    static constexpr int NK = RW / 8;                  // rotary copies per wave per tile
    static constexpr int HW = 32 * NHG;                // heads per workgroup
    static constexpr int NQK = NHG * RG;               // waves with a QK role
    static constexpr int LAT = R * RANK * 2;           // latent region of a stage (row stride 1 KB)
    static constexpr int STAGE = R * ROW * 2;          // latent + rotary regions
    static constexpr int PST = R + 8;                  // P^T row stride (elements)
    static constexpr int P_BYTES = HW * PST * 2;
    static constexpr int OFF_P = 2 * STAGE;
    static constexpr int OFF_XMAX = OFF_P + P_BYTES;          // [RG][HW] float
    static constexpr int OFF_L = OFF_XMAX + RG * HW * 4;      // [RG][HW] float
    static constexpr int OFF_M = OFF_L + RG * HW * 4;         // [HW] float
    static constexpr int OFF_FLAG = OFF_M + HW * 4;           // int
    static constexpr int LDS = OFF_FLAG + 16;
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Tile layout in LDS.  Latent region: row r at r * 1024 bytes, its 16-byte
// chunk c (8 latent features) at slot c ^ swz(r), swz(r) = ((r&3)<<2)|((r>>2)&3).
// 16 consecutive rows read at one chunk (QK^T operand) hit 16 different bank
// groups, and the 4x4 row/chunk blocks of the transposed PV reads do too.
// Rotary region: row r at r * 128 bytes, chunk c' (0..7) at slot c' ^ ((r>>1)&7).
__device__ __forceinline__ int lat_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int lat_off(int r, int chunk) { return r * 1024 + ((chunk ^ lat_swz(r)) << 4); }
__device__ __forceinline__ int rot_off(int r, int chunk) { return r * 128 + ((chunk ^ ((r >> 1) & 7)) << 4); }

// Largest exponent (log2) a probability may reach relative to the
// reference maximum before the split is recomputed with the exact maximum.
constexpr float P_EXP_LIMIT = 64.f;

struct SplitCtx {
    int b, s, h0, start, end, ntiles;
    const int32_t* list;
    const char* kvb;    // sequence base of the latent cache (bytes)
    const char* peb;    // sequence base of the rotary-key cache (bytes)
};

// One pass over the split.  With KNOWN = false the reference maximum of each
// head is the maximum of the first tile; probabilities of later tiles are
// exp2(x - m_ref), which may exceed 1 (fp32 and bf16 share the 8-bit
// exponent), so the accumulators never need rescaling.  The pass reports
// whether any head's true maximum exceeded m_ref by more than P_EXP_LIMIT;
// the caller then runs the pass again with KNOWN = true and m_ref = that
// exact maximum, where every probability is <= 1.
template <int NHG, bool KNOWN>
__device__ __forceinline__ bool attn_pass(const AttnArgs& a, const SplitCtx& sc, char* smem,
                                          const bf16x8 (&qreg)[ROW / 16], float& m_ref) {
    using C = AttnCfg<NHG>;
    constexpr int R = C::R, RG = C::RG, RW = C::RW, NK = C::NK;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const bool qk = wave < C::NQK;
    const int hg = wave % NHG, rg = wave / NHG;
    const int start = sc.start, end = sc.end, ntiles = sc.ntiles;

    auto load_idx = [&](int it, int* idx) {
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            const int pos = start + it * R + wave * RW + 8 * k + (lane >> 3);
            idx[k] = pos < end ? sc.list[pos] : 0;
        }
    };
    // One 1 KB latent copy per row (lane l moves chunk l ^ swz(r), which lands
    // in slot l) and one rotary copy per 8 rows.
    auto stage_tile = [&](int it, int buf, const int* idx) {
        char* lat = smem + buf * C::STAGE;
        char* rot = lat + C::LAT;
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const int r = wave * RW + j;
            if (start + it * R + r < end) {
                const long long t = __builtin_amdgcn_readlane(idx[j >> 3], 8 * (j & 7));
                const char* rowp = sc.kvb + t * a.kv_st * 2;
                const uint32_t off = (uint32_t)(lane ^ lat_swz(r)) << 4;
                global_to_lds16(rowp + off, (MLA_LDS void*)(lat + r * 1024));
            }
        }
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            const int r = wave * RW + 8 * k + (lane >> 3);
            if (start + it * R + r < end) {
                const long long t = idx[k];
                const char* src = sc.peb + t * a.pe_st * 2 + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
                global_to_lds16(src, (MLA_LDS void*)(rot + (wave * RW + 8 * k) * 128));
            }
        }
    };

    float m_true = KNOWN ? m_ref : -INFINITY;
    float lsum = 0.f;
    f32x16 o[NHG][4];
#pragma unroll
    for (int nb = 0; nb < NHG; ++nb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) o[nb][cb] = f32x16{};

    float* xmax = (float*)(smem + C::OFF_XMAX);
    bf16* pbuf = (bf16*)(smem + C::OFF_P);

    int idx_next[NK];
    __syncthreads();
    if (ntiles > 0) {
        load_idx(0, idx_next);
        stage_tile(0, 0, idx_next);
        if (ntiles > 1) load_idx(1, idx_next);
    }

    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1;
        wait_vmcnt<0>();
        __syncthreads();                                   // tile `it` resident; P buffer free
        if (it + 1 < ntiles) {
            stage_tile(it + 1, buf ^ 1, idx_next);
            if (it + 2 < ntiles) load_idx(it + 2, idx_next);
        }
        __builtin_amdgcn_sched_barrier(0);
        const char* lat = smem + buf * C::STAGE;
        const char* rot = lat + C::LAT;

        f32x16 acc = {};
        float mt = -INFINITY;
        if (qk) {
            const int row = rg * 32 + l32;
#pragma unroll
            for (int kb = 0; kb < RANK / 16; kb += 4) {
                bf16x8 kv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) kv[u] = *(const bf16x8*)(lat + lat_off(row, 2 * (kb + u) + g));
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = mfma32(kv[u], qreg[kb + u], acc);
                __builtin_amdgcn_sched_barrier(0);
            }
            {
                bf16x8 kv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) kv[u] = *(const bf16x8*)(rot + rot_off(row, 2 * u + g));
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = mfma32(kv[u], qreg[RANK / 16 + u], acc);
            }
            const int rem = end - (start + it * R + rg * 32);   // valid rows of this chunk
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int t = 8 * (i >> 2) + 4 * g + (i & 3);
                acc[i] = t < rem ? acc[i] * a.scale_log2 : -INFINITY;
                mt = fmaxf(mt, acc[i]);
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            if constexpr (RG == 2) {
                if (g == 0) xmax[rg * C::HW + hg * 32 + l32] = mt;
            }
        }
        if constexpr (RG == 2) {
            __syncthreads();
            if (qk) mt = fmaxf(mt, xmax[(1 - rg) * C::HW + hg * 32 + l32]);
        }
        if (qk) {
            // Reference maximum: the first tile's, floored to an integer so that
            // exp2(x - m_ref) differs from exp2(x) by a power of two only and
            // its bf16 rounding does not depend on where the splits fall.
            if (!KNOWN && it == 0) m_ref = floorf(mt);
            m_true = fmaxf(m_true, mt);
            float ps = 0.f;
            bf16* prow = pbuf + (hg * 32 + l32) * C::PST + rg * 32 + 4 * g;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x4 pk;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = exp2f(fminf(acc[4 * j + r] - m_ref, P_EXP_LIMIT));
                    ps += p;
                    pk[r] = f2bf(p);
                }
                *(bf16x4*)(prow + 8 * j) = pk;
            }
            lsum += ps;
        }
        __syncthreads();                                   // P^T visible
        __builtin_amdgcn_sched_barrier(0);

        // ---- PV: O^T[c][h] += V^T[c][t] P^T[t][h] ----
        const int blk = lane >> 4, L = lane & 15;
#pragma unroll
        for (int kt = 0; kt < R / 16; ++kt) {
            bf16x8 av[4];
            const int r0 = 16 * kt + 8 * (blk >> 1) + (L >> 2);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const int col = 128 * wave + 32 * cb + 16 * (blk & 1) + 4 * (L & 3);
                const int chunk = col >> 3, within = (col & 7) * 2;
                const bf16x4 lo = lds_read_tr16((const MLA_LDS void*)(lat + lat_off(r0, chunk) + within));
                const bf16x4 hi = lds_read_tr16((const MLA_LDS void*)(lat + lat_off(r0 + 4, chunk) + within));
                av[cb] = cat(lo, hi);
            }
#pragma unroll
            for (int nb = 0; nb < NHG; ++nb) {
                const bf16x8 pv = *(const bf16x8*)(pbuf + (nb * 32 + l32) * C::PST + 16 * kt + 8 * g);
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) o[nb][cb] = mfma32(av[cb], pv, o[nb][cb]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- overflow check, then combine row groups, normalise, write ----
    float* lred = (float*)(smem + C::OFF_L);
    float* mfin = (float*)(smem + C::OFF_M);
    int* flag = (int*)(smem + C::OFF_FLAG);
    __syncthreads();
    if (tid == 0) *flag = 0;
    __syncthreads();
    if (qk) {
        if (!KNOWN && m_true > m_ref + P_EXP_LIMIT) *flag = 1;
        const float lt = lsum + __shfl_xor(lsum, 32);
        if (g == 0) {
            lred[rg * C::HW + hg * 32 + l32] = lt;
            if (rg == 0) mfin[hg * 32 + l32] = m_ref;
        }
    }
    __syncthreads();
    if (!KNOWN && *flag) {
        m_ref = floorf(m_true);
        return true;
    }
    const long long pbase = ((long long)sc.b * a.S + sc.s) * a.H;
#pragma unroll
    for (int nb = 0; nb < NHG; ++nb) {
        const int hl = nb * 32 + l32, h = sc.h0 + hl;
        float l = lred[hl];
        if constexpr (RG == 2) l += lred[C::HW + hl];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        if (h < a.H) {
            bf16* dst = a.opart + (pbase + h) * RANK + 128 * wave;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    bf16x4 v;
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = f2bf(o[nb][cb][4 * j + r] * inv);
                    *(bf16x4*)(dst + 32 * cb + 8 * j + 4 * g) = v;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (wave == 0 && g == 0) a.lsepart[pbase + h] = l > 0.f ? mfin[hl] + log2f(l) : -INFINITY;
        }
    }
    return false;
}

template <int NHG>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void attn_kernel(AttnArgs a) {
    using C = AttnCfg<NHG>;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;

    // XCD-aware mapping: workgroups of the same (sequence, split) and
    // different head groups get ids 8 apart, i.e. the same XCD and L2.
    const int id = blockIdx.x;
    const int xcd = id & 7, k8 = id >> 3;
    const int hgi = k8 % a.HG, q8 = k8 / a.HG;
    const int bs = q8 * 8 + xcd;
    if (bs >= a.B * a.S) return;

    SplitCtx sc;
    sc.b = bs / a.S;
    sc.s = bs % a.S;
    sc.h0 = hgi * C::HW;
    const int cnt = a.counts[sc.b];
    int rps = (cnt + a.S - 1) / a.S;
    rps = (rps + 7) & ~7;
    sc.start = min(sc.s * rps, cnt);
    sc.end = min(sc.start + rps, cnt);
    sc.ntiles = (sc.end - sc.start + C::R - 1) / C::R;
    sc.list = a.list + (long long)sc.b * a.K;
    sc.kvb = (const char*)(a.kv + (long long)sc.b * a.kv_sb);
    sc.peb = (const char*)(a.pe + (long long)sc.b * a.pe_sb);

    // Zero both stages so rows past the end of the split read as zeros.
    for (int i = tid * 16; i < 2 * C::STAGE; i += 256 * 16) *(u32x4*)(smem + i) = u32x4{0, 0, 0, 0};

    // This wave's 32 heads of Q~ stay in registers (QK^T B operand).
    bf16x8 qreg[ROW / 16];
    {
        const int hg = wave % NHG;
        const int h = sc.h0 + hg * 32 + l32;
        if (wave < C::NQK && h < a.H) {
            const bf16* q = a.qt + ((long long)sc.b * a.H + h) * ROW + 8 * g;
#pragma unroll
            for (int kb = 0; kb < ROW / 16; ++kb) qreg[kb] = *(const bf16x8*)(q + 16 * kb);
        } else {
#pragma unroll
            for (int kb = 0; kb < ROW / 16; ++kb) qreg[kb] = bf16x8{};
        }
    }
    float m_ref = 0.f;
    if (attn_pass<NHG, false>(a, sc, smem, qreg, m_ref)) attn_pass<NHG, true>(a, sc, smem, qreg, m_ref);
}

hipError_t launch_attn_f32(const mla_decode_params_t& p, const Work& w, hipStream_t s);

int attn_grid(const Plan& plan, int B) {
    return ((B * plan.splits + 7) / 8) * 8 * plan.hgroups;
}

hipError_t launch_attn(const mla_decode_params_t& p, const Plan& plan, const Work& w, hipStream_t s) {
    if (!plan.bf16_path) return launch_attn_f32(p, w, s);
    AttnArgs a{};
    a.B = p.B; a.H = p.H; a.K = p.K; a.S = plan.splits; a.HG = plan.hgroups;
    a.scale_log2 = p.softmax_scale * LOG2E;
    a.qt = (const bf16*)w.qt; a.list = w.list; a.counts = w.counts;
    a.kv = (const bf16*)p.kv_cache; a.kv_sb = p.kv_stride_b; a.kv_st = p.kv_stride_t;
    a.pe = (const bf16*)p.pe_cache; a.pe_sb = p.pe_stride_b; a.pe_st = p.pe_stride_t;
    a.opart = (bf16*)w.opart; a.lsepart = w.lsepart;
    const dim3 grid(attn_grid(plan, p.B)), block(256);
    switch (plan.nhg) {
        case 4: hipLaunchKernelGGL(attn_kernel<4>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(attn_kernel<2>, grid, block, 0, s, a); break;
        case 1: hipLaunchKernelGGL(attn_kernel<1>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mla
