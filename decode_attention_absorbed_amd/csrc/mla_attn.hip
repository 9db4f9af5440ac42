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

// ---------------------------------------------------------------------------
// Workgroup shape: 4 waves, 64 heads, tiles of 32 gathered rows, a ring of
// four LDS stages (tiles t..t+3: PV reads t, QK reads t+1, t+2 and t+3 are
// in flight).
// ---------------------------------------------------------------------------
constexpr int HW = 64;                 // heads per workgroup
constexpr int R = 32;                  // rows per tile
constexpr int NST = 4;                 // LDS stages
constexpr int LAT = R * RANK * 2;      // latent region of a stage: row r at r * 1 KB
constexpr int STAGE = R * ROW * 2;     // + rotary region: row r at LAT + r * 128
constexpr int PST = R + 8;             // P^T row stride (elements): 80 bytes
constexpr int PBYTES = HW * PST * 2;
constexpr int OFF_P = NST * STAGE;                 // two P^T buffers
constexpr int OFF_IDX = OFF_P + 2 * PBYTES;        // [NST][4 waves][8] int: row indices
constexpr int OFF_XMAX = OFF_IDX + NST * 4 * 8 * 4;  // [2][HW] float
constexpr int OFF_L = OFF_XMAX + 2 * HW * 4;       // [2][HW] float
constexpr int OFF_M = OFF_L + 2 * HW * 4;          // [HW] float
constexpr int OFF_FLAG = OFF_M + HW * 4;
constexpr int LDS_BYTES = OFF_FLAG + 16;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

// Tile layout in LDS.  Latent region: row r at r * 1024 bytes, its 16-byte
// chunk c (8 latent features) at slot c ^ swz(r), swz(r) = ((r&3)<<2)|((r>>2)&3).
// 16 consecutive rows read at one chunk (QK^T operand) hit 16 different bank
// groups, and the 4 row x 4 chunk blocks of the transposed PV reads do too.
// Rotary region: row r at r * 128 bytes, chunk c' (0..7) at slot c' ^ ((r>>1)&7).
__device__ __forceinline__ int lat_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Largest exponent (log2) a probability may reach relative to the
// reference maximum before the split is recomputed with the exact maximum.
constexpr float P_EXP_LIMIT = 64.f;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// s_waitcnt vmcnt(n) for the counts the copy pipeline produces.
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
        case 21: wait_vmcnt<21>(); break;
        case 20: wait_vmcnt<20>(); break;
        case 19: wait_vmcnt<19>(); break;
        case 18: wait_vmcnt<18>(); break;
        case 11: wait_vmcnt<11>(); break;
        case 10: wait_vmcnt<10>(); break;
        case 9: wait_vmcnt<9>(); break;
        default: wait_vmcnt<0>(); break;
    }
}

struct SplitCtx {
    int b, s, h0, start, end, ntiles;
    const int32_t* list;
    const char* kvb;    // sequence base of the latent cache (bytes)
    const char* peb;    // sequence base of the rotary-key cache (bytes)
};

// Per-lane LDS offsets, relative to a stage or a P^T buffer.
struct LaneOffsets {
    int qk_off[4];      // QK operand: latent chunk 16j + 4k + lane/16 at qk_off[k] + 256 j
    int qk_rot[2];      // QK operand: rotary chunk 4k + lane/16
    int tr_row[2][2];   // PV transposed reads [kt][rd]: row base with the column part
    int tr_y[2][2];     //   and the swizzle bits that permute the 32-column blocks
    int p_wr;           // P^T element written by this lane (+ 16 nb * PST)
    int p_rd;           // P^T operand read by this lane (+ 32 nb * PST + 16 kt)
};

// Softmax state of this wave's 32 heads (2 groups of 16) and the O^T
// accumulators of its 128 latent columns x 64 heads.
struct PassState {
    float m_ref[2], m_true[2], lsum[2];
    f32x16 o[2][4];
};

__device__ __forceinline__ LaneOffsets lane_offsets() {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 5, l32 = lane & 31, q4 = lane >> 4, l16 = lane & 15;
    const int hg = wave & 1, rg = wave >> 1;
    LaneOffsets lo;
    const int qrow = rg * 16 + l16;
#pragma unroll
    for (int k = 0; k < 4; ++k) lo.qk_off[k] = qrow * 1024 + (((4 * k + q4) ^ lat_swz(qrow)) << 4);
#pragma unroll
    for (int k = 0; k < 2; ++k) lo.qk_rot[k] = LAT + qrow * 128 + (((4 * k + q4) ^ ((qrow >> 1) & 7)) << 4);
    const int blk = lane >> 4, L = lane & 15;
    const int c0 = 2 * (blk & 1) + ((L & 3) >> 1);
    const int within = (L & 1) * 8;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
            const int r = 16 * kt + 8 * (blk >> 1) + 4 * rd + (L >> 2);
            const int sw = lat_swz(r);
            lo.tr_row[kt][rd] = r * 1024 + ((16 * wave + (c0 ^ (sw & 3))) << 4) + within;
            lo.tr_y[kt][rd] = sw >> 2;
        }
    lo.p_wr = (hg * 32 + l16) * PST + rg * 16 + 4 * q4;
    lo.p_rd = l32 * PST + 8 * g;
    return lo;
}

// Row indices of tile T for this wave: lanes 0..7 copy 4 bytes each into the
// ring slot (positions past the end repeat the last row, so every tile costs
// the same number of copies).
__device__ __forceinline__ void fetch_idx(const SplitCtx& sc, int T, int* __restrict__ slot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane < 8) {
        const int pos = min(sc.start + T * R + wave * 8 + lane, sc.end - 1);
        __builtin_amdgcn_global_load_lds(sc.list + pos, (MLA_LDS void*)slot, 4, 0, 0);
    }
}

// Copy this wave's 8 rows of a tile into a stage: 8 latent copies of 1 KB
// (lane l moves chunk l ^ swz(r), which lands in slot l) and one copy of
// their 8 rotary parts.
__device__ __forceinline__ void issue_tile(const AttnArgs& a, const SplitCtx& sc, char* __restrict__ stage,
                                           const int* __restrict__ slot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const u32x4 i0 = *(const u32x4*)slot;
    const u32x4 i1 = *(const u32x4*)(slot + 4);
    const int idx_rot = slot[lane >> 3];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = wave * 8 + j;
        const long long t = (long long)__builtin_amdgcn_readfirstlane(j < 4 ? i0[j & 3] : i1[j & 3]);
        const char* src = sc.kvb + t * a.kv_st * 2 + ((lane ^ lat_swz(r)) << 4);
        global_to_lds16(src, (MLA_LDS void*)(stage + r * 1024));
    }
    const int r = wave * 8 + (lane >> 3);
    const char* src = sc.peb + (long long)idx_rot * a.pe_st * 2 + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
    global_to_lds16(src, (MLA_LDS void*)(stage + LAT + wave * 8 * 128));
}

// QK^T of one tile for this wave's 16 rows x 32 heads; operands read two
// steps ahead of the MFMAs.
__device__ __forceinline__ void qk_tile(const char* __restrict__ st, const LaneOffsets& lo,
                                        const bf16x8 (&qreg)[ROW / 32][2], f32x4 (&acc)[2]) {
    auto off = [&](int ks) { return ks < 16 ? lo.qk_off[ks & 3] + 256 * (ks >> 2) : lo.qk_rot[ks - 16]; };
    acc[0] = f32x4{};
    acc[1] = f32x4{};
    bf16x8 kv[3];
    kv[0] = *(const bf16x8*)(st + off(0));
    kv[1] = *(const bf16x8*)(st + off(1));
#pragma unroll
    for (int ks = 0; ks < ROW / 32; ++ks) {
        if (ks + 2 < ROW / 32) kv[(ks + 2) % 3] = *(const bf16x8*)(st + off(ks + 2));
        acc[0] = mfma16(kv[ks % 3], qreg[ks][0], acc[0]);
        acc[1] = mfma16(kv[ks % 3], qreg[ks][1], acc[1]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One softmax element (head group nb, row i of this lane's 4): scale, mask
// rows past the end, exponentiate against the reference maximum.
__device__ __forceinline__ void soft_elem(PassState& ps, const f32x4 (&acc)[2], int nb, int i, int rem,
                                          float scale_log2, bf16x4& pk) {
    const float x = i < rem ? acc[nb][i] * scale_log2 : -INFINITY;
    ps.m_true[nb] = fmaxf(ps.m_true[nb], x);
    const float p = exp2f(fminf(x - ps.m_ref[nb], P_EXP_LIMIT));
    ps.lsum[nb] += p;
    pk[i] = f2bf(p);
}

// PV of one tile (O^T += V^T . P^T) with, when has_next, the softmax of the
// next tile interleaved (acc in, P^T of the next tile out).
__device__ __forceinline__ void pv_tile(const char* __restrict__ st, const bf16* __restrict__ p_in,
                                        bf16* __restrict__ p_out, const LaneOffsets& lo, PassState& ps,
                                        const f32x4 (&acc)[2], bool has_next, int rem_next, float scale_log2) {
    const bf16* pb = p_in + lo.p_rd;
    auto tr = [&](int kt, int cb) {
        const bf16x4 lo0 = lds_read_tr16((const MLA_LDS void*)(st + lo.tr_row[kt][0] + ((cb ^ lo.tr_y[kt][0]) << 6)));
        const bf16x4 hi0 = lds_read_tr16((const MLA_LDS void*)(st + lo.tr_row[kt][1] + ((cb ^ lo.tr_y[kt][1]) << 6)));
        return cat(lo0, hi0);
    };
    bf16x8 pvb[2][2], av[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) pvb[0][nb] = *(const bf16x8*)(pb + 32 * nb * PST);
    av[0] = tr(0, 0);
    bf16x4 pk[2];
#pragma unroll
    for (int step = 0; step < 8; ++step) {
        const int kt = step >> 2, cb = step & 3;
        if (step + 1 < 8) av[(step + 1) & 1] = tr((step + 1) >> 2, (step + 1) & 3);
        if (step == 1) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) pvb[1][nb] = *(const bf16x8*)(pb + 32 * nb * PST + 16);
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) ps.o[nb][cb] = mfma32(av[step & 1], pvb[kt][nb], ps.o[nb][cb]);
        if (has_next && step >= 4) {
            // two softmax elements per step from step 4 on (the QK results
            // are complete by then)
            const int e0 = 2 * (step - 4);
#pragma unroll
            for (int e = e0; e < e0 + 2; ++e) soft_elem(ps, acc, e >> 2, e & 3, rem_next, scale_log2, pk[e >> 2]);
            if ((e0 + 2) % 4 == 0) *(bf16x4*)(p_out + lo.p_wr + 16 * (e0 >> 2) * PST) = pk[e0 >> 2];
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One main-loop iteration's work after the barrier: copy tile it+3 and the
// indices of tile it+6, QK^T of tile it+1, PV of tile it with the softmax
// of tile it+1.  Distinct restrict-qualified pointers tell the compiler
// that the reads never touch the stage or slot being filled, so it does not
// wait for the copies in flight.
__device__ __forceinline__ void main_step(const AttnArgs& a, const SplitCtx& sc, int it, const LaneOffsets& lo,
                                          const bf16x8 (&qreg)[ROW / 32][2], PassState& ps,
                                          char* __restrict__ dma_stage, const int* __restrict__ dma_slot,
                                          int* __restrict__ idx_slot, const char* __restrict__ qk_stage,
                                          const char* __restrict__ pv_stage, const bf16* __restrict__ p_in,
                                          bf16* __restrict__ p_out) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q4 = lane >> 4, rg = wave >> 1;
    const int nt = sc.ntiles;
    if (it + 3 < nt) issue_tile(a, sc, dma_stage, dma_slot);
    if (it + 6 < nt) fetch_idx(sc, it + 6, idx_slot);
    const bool has_next = it + 1 < nt;
    f32x4 acc[2] = {f32x4{}, f32x4{}};
    if (has_next) qk_tile(qk_stage, lo, qreg, acc);
    const int rem_next = sc.end - (sc.start + (it + 1) * R + rg * 16 + 4 * q4);
    pv_tile(pv_stage, p_in, p_out, lo, ps, acc, has_next, rem_next, a.scale_log2);
}

// One pass over the split (see attn_kernel).  Returns true when the pass
// must be repeated with the exact maximum (then m_ref holds it).
//
// Copy pipeline, per wave and tile T: 9 global->LDS copies issued in
// iteration T-3 and the 4-byte index copy issued in iteration T-6.
// Iteration t waits until tile t+1 has landed, so 11 later copies of this
// wave may still be in flight.
__device__ __forceinline__ bool attn_pass(const AttnArgs& a, const SplitCtx& sc, char* smem,
                                          const bf16x8 (&qreg)[ROW / 32][2], float (&m_ref)[2], bool known) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31, q4 = lane >> 4, l16 = lane & 15;
    const int hg = wave & 1, rg = wave >> 1;
    const int start = sc.start, end = sc.end, nt = sc.ntiles;
    int* idx_ring = (int*)(smem + OFF_IDX) + wave * 8;      // + slot * 32
    auto stage = [&](int T) { return smem + (T % NST) * STAGE; };
    auto pbuf = [&](int T) { return (bf16*)(smem + OFF_P + (T & 1) * PBYTES); };
    auto slot = [&](int T) { return idx_ring + (T % NST) * 32; };

    const LaneOffsets lo = lane_offsets();
    PassState ps;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        ps.m_ref[nb] = m_ref[nb];
        ps.m_true[nb] = known ? m_ref[nb] : -INFINITY;
        ps.lsum[nb] = 0.f;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) ps.o[nb][cb] = f32x16{};
    }
    float* xmax = (float*)(smem + OFF_XMAX);

    // ---- prologue: indices for tiles 0..5, copies for tiles 0..2 ----
    __syncthreads();                               // LDS zeroing / previous pass done
    if (nt > 0) {
#pragma unroll
        for (int T = 0; T < 3; ++T)
            if (T < nt) fetch_idx(sc, T, slot(T));
        wait_vmcnt<0>();
#pragma unroll
        for (int T = 0; T < 3; ++T) {
            if (T < nt) issue_tile(a, sc, stage(T), slot(T));
            if (T + 3 < nt) fetch_idx(sc, T + 3, slot(T + 3));
        }
        const int after0 = (nt > 3) + 9 * (nt > 1) + (nt > 4) + 9 * (nt > 2) + (nt > 5);
        wait_vm(after0);
        __syncthreads();                           // tile 0 visible
        f32x4 acc[2];
        qk_tile(stage(0), lo, qreg, acc);
        // reference maximum from the first tile, shared by both row halves
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            float mt = -INFINITY;
            const int rem = end - (start + rg * 16 + 4 * q4);
#pragma unroll
            for (int i = 0; i < 4; ++i) mt = fmaxf(mt, i < rem ? acc[nb][i] * a.scale_log2 : -INFINITY);
            mt = fmaxf(mt, __shfl_xor(mt, 16));
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            if (q4 == 0) xmax[rg * HW + hg * 32 + 16 * nb + l16] = mt;
        }
        __syncthreads();
        if (!known) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int h = hg * 32 + 16 * nb + l16;
                ps.m_ref[nb] = floorf(fmaxf(xmax[h], xmax[HW + h]));
            }
        }
        const int rem = end - (start + rg * 16 + 4 * q4);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            bf16x4 pk;
#pragma unroll
            for (int i = 0; i < 4; ++i) soft_elem(ps, acc, nb, i, rem, a.scale_log2, pk);
            *(bf16x4*)(pbuf(0) + lo.p_wr + 16 * nb * PST) = pk;
        }
    }

    // ---- main loop ----
    for (int it = 0; it < nt; ++it) {
        const int left = nt - it;
        wait_vm(left >= 6 ? 11 : left == 5 ? 10 : left >= 3 ? 9 : 0);
        __syncthreads();        // tile it+1 resident, P(it) visible, stage (it-1)%4 free
        main_step(a, sc, it, lo, qreg, ps, stage(it + 3), slot(it + 3), slot(it + 6), stage(it + 1), stage(it),
                  pbuf(it), pbuf(it + 1));
    }

    // ---- overflow check, then combine row halves, normalise, write ----
    float* lred = (float*)(smem + OFF_L);
    float* mfin = (float*)(smem + OFF_M);
    int* flag = (int*)(smem + OFF_FLAG);
    __syncthreads();
    if (tid == 0) *flag = 0;
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        if (!known && ps.m_true[nb] > ps.m_ref[nb] + P_EXP_LIMIT) *flag = 1;
        float lt = ps.lsum[nb];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        float m = ps.m_true[nb];
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        const int h = hg * 32 + 16 * nb + l16;
        if (q4 == 0) {
            lred[rg * HW + h] = lt;
            xmax[rg * HW + h] = m;
            if (rg == 0) mfin[h] = ps.m_ref[nb];
        }
    }
    __syncthreads();
    if (!known && *flag) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int h = hg * 32 + 16 * nb + l16;
            m_ref[nb] = floorf(fmaxf(xmax[h], xmax[HW + h]));
        }
        return true;
    }
    const long long pbase = ((long long)sc.b * a.S + sc.s) * a.H;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int hl = nb * 32 + l32, h = sc.h0 + hl;
        const float l = lred[hl] + lred[HW + hl];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        if (h < a.H) {
            bf16* dst = a.opart + (pbase + h) * RANK + 128 * wave;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    bf16x4 v;
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = f2bf(ps.o[nb][cb][4 * j + r] * inv);
                    *(bf16x4*)(dst + 32 * cb + 8 * j + 4 * g) = v;
                }
            }
            if (wave == 0 && g == 0) a.lsepart[pbase + h] = l > 0.f ? mfin[hl] + log2f(l) : -INFINITY;
        }
    }
    return false;
}

// Split-KV attention workgroup: 4 waves, 64 heads, 32-row tiles, 4-stage
// LDS ring.  Per wave: QK role (hg = wave & 1, rg = wave >> 1): S^T[16 rows]
// [32 heads] of each tile with v_mfma_f32_16x16x32_bf16, Q~ for 32 heads held
// in registers.  PV role: O^T[128 latent columns][64 heads], columns
// [128 wave, 128 wave + 128), with v_mfma_f32_32x32x16_bf16, V^T read with
// ds_read_b64_tr_b16 and P^T from LDS.  The reference maximum of each head is
// the (floored) maximum of the split's first tile; later probabilities are
// exp2(x - m_ref) and may exceed 1 (fp32 and bf16 share the 8-bit exponent),
// so the accumulators are never rescaled.  If a head's true maximum exceeds
// m_ref by more than P_EXP_LIMIT the split is run again with the exact
// maximum as reference.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void attn_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

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
    sc.h0 = hgi * HW;
    const int cnt = a.counts[sc.b];
    int rps = (cnt + a.S - 1) / a.S;
    rps = (rps + 7) & ~7;
    sc.start = min(sc.s * rps, cnt);
    sc.end = min(sc.start + rps, cnt);
    sc.ntiles = (sc.end - sc.start + R - 1) / R;
    sc.list = a.list + (long long)sc.b * a.K;
    sc.kvb = (const char*)(a.kv + (long long)sc.b * a.kv_sb);
    sc.peb = (const char*)(a.pe + (long long)sc.b * a.pe_sb);

    // This wave's 32 heads of Q~ (QK^T B operand): qreg[ks][nb] holds
    // features 32 ks + 8 (lane/16) .. +7 of head 32 hg + 16 nb + lane%16.
    bf16x8 qreg[ROW / 32][2];
    {
        const int hg = wave & 1, q4 = lane >> 4, l16 = lane & 15;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int h = sc.h0 + hg * 32 + 16 * nb + l16;
            if (h < a.H) {
                const bf16* q = a.qt + ((long long)sc.b * a.H + h) * ROW + 8 * q4;
#pragma unroll
                for (int ks = 0; ks < ROW / 32; ++ks) qreg[ks][nb] = *(const bf16x8*)(q + 32 * ks);
            } else {
#pragma unroll
                for (int ks = 0; ks < ROW / 32; ++ks) qreg[ks][nb] = bf16x8{};
            }
        }
    }
    float m_ref[2] = {0.f, 0.f};
    for (int pass = 0; pass < 2; ++pass)
        if (!attn_pass(a, sc, smem, qreg, m_ref, pass == 1)) break;
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
    hipLaunchKernelGGL(attn_kernel, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace mla
