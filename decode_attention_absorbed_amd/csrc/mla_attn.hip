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
    uint32_t kv_win, pe_win;   // bytes of one sequence's rows: (L_max - 1) * row stride + row
    bf16* opart;
    float* lsepart;
};

// ---------------------------------------------------------------------------
// Workgroup shape: 4 waves (one per SIMD), 128 heads, tiles of 32 gathered
// rows, a ring of three LDS stages (PV reads tile t, QK reads tile t+1, the
// copies of tile t+2 are in flight).  Every selected row is gathered once
// per (sequence, split), and the staged tile feeds all 128 heads.
// ---------------------------------------------------------------------------
constexpr int HW = 128;                // heads per workgroup
constexpr int R = 32;                  // rows per tile
constexpr int NST = 3;                 // LDS stages
constexpr int LAT = R * RANK * 2;      // latent region of a stage: row r at r * 1 KB
constexpr int STAGE = R * ROW * 2;     // + rotary region: row r at LAT + r * 128
constexpr int PST = R + 8;             // P^T row stride (elements): 80 bytes
constexpr int PBYTES = HW * PST * 2;
constexpr int NSLOT = 3;               // index ring slots
constexpr int OFF_P = NST * STAGE;                 // two P^T buffers
constexpr int OFF_IDX = OFF_P + 2 * PBYTES;        // [NSLOT][4 waves][8] int: row indices
constexpr int OFF_L = OFF_IDX + NSLOT * 4 * 8 * 4; // [HW] float
constexpr int OFF_M = OFF_L + HW * 4;              // [HW] float
constexpr int OFF_FLAG = OFF_M + HW * 4;
constexpr int QK_REG = 29;                         // Q~ feature blocks 0..28 live in registers,
constexpr int QK_LDS = ROW / 16 - QK_REG;          // blocks 29..35 in LDS: [block][head][16]
constexpr int OFF_Q = OFF_FLAG + 16;
constexpr int LDS_BYTES = OFF_Q + QK_LDS * HW * 32;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

// Tile layout in LDS.  Latent region: row r at r * 1024 bytes, its 16-byte
// chunk c (8 latent features) at slot c ^ swz(r), swz(r) = ((r&3)<<2)|((r>>2)&3).
// 16 consecutive rows read at one chunk (QK^T operand) hit 16 different bank
// groups, and the 4 row x 4 chunk blocks of the transposed PV reads do too.
// Rotary region: row r at r * 128 bytes, chunk c' (0..7) at slot c' ^ ((r>>1)&7).
__device__ __forceinline__ int lat_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// The wave index, known to the compiler as wave-uniform (an SGPR).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }


// Largest exponent (log2) a probability may reach relative to the
// reference maximum before the split is recomputed with the exact maximum.
constexpr float P_EXP_LIMIT = 64.f;

// s_waitcnt vmcnt(n) for the counts the copy pipeline produces.
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
        case 11: wait_vmcnt<11>(); break;
        case 10: wait_vmcnt<10>(); break;
        case 9: wait_vmcnt<9>(); break;
        case 1: wait_vmcnt<1>(); break;
        default: wait_vmcnt<0>(); break;
    }
}

// Workgroup barrier for the main loop.  It waits for this wave's LDS
// operations only: the global->LDS copies still in flight target stages no
// one reads before a later, explicit vmcnt wait (__syncthreads would drain
// them).  The asm memory clobber keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

struct SplitCtx {
    int b, s, h0, start, end, ntiles;
    rsrc_t list;        // the sequence's compacted row list
    rsrc_t kv;          // the sequence's rows of the latent cache
    rsrc_t pe;          // the sequence's rows of the rotary-key cache
};

// Per-lane LDS offsets.  The swizzles are XORs on address bits that the
// bases leave zero, so every operand address is a base XOR a constant.
//   QK latent chunk 16j + 2k + lane/32 of row lane%32:  (qk ^ (k << 5)) + 256 j
//   QK rotary chunk 2k + lane/32:                       rot ^ (k << 5)
//   PV transposed read rd of rows 16 kt.., block cb:    (tr[rd] ^ (cb << 6)) + 16384 kt
//   Q~ block 29 + i (LDS part):                         q + 4096 i
struct LaneOffsets {
    int qk, rot, tr[2];
    int p_wr;           // P^T elements written by this lane (+ 8 j)
    int p_rd;           // P^T operand read by this lane (+ 32 nb * PST + 16 kt)
    int q;
};

// Softmax state of this wave's 32 heads and the O^T accumulators of its
// 128 latent columns x 128 heads.
struct PassState {
    float m_ref, m_true, lsum;
    f32x16 o[4][4];     // [nb: 32-head block][cb: 32-column block]
};

__device__ __forceinline__ LaneOffsets lane_offsets() {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 5, l32 = lane & 31;
    LaneOffsets lo;
    // chunk (2k + g) ^ sw of row l32 = (k ^ (sw >> 1)) << 1 | (g ^ (sw & 1))
    const int sw = lat_swz(l32);
    lo.qk = l32 * 1024 + ((g ^ (sw & 1)) << 4) + ((sw >> 1) << 5);
    const int u = (l32 >> 1) & 7;
    lo.rot = LAT + l32 * 128 + ((g ^ (u & 1)) << 4) + ((u >> 1) << 5);
    // transposed reads: 16-lane block blk reads rows 8 (blk >> 1) + 4 rd + L/4
    // (+ 16 kt); their swizzle has low bits (2 (blk >> 1) + rd) & 3 and high
    // bits L/4, the same for both kt
    const int blk = lane >> 4, L = lane & 15;
    const int c0 = 2 * (blk & 1) + ((L & 3) >> 1);
    const int within = (L & 1) * 8;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
        const int r = 8 * (blk >> 1) + 4 * rd + (L >> 2);
        const int s = lat_swz(r);
        lo.tr[rd] = r * 1024 + ((16 * wave + (c0 ^ (s & 3))) << 4) + within + ((s >> 2) << 6);
    }
    lo.p_wr = (wave * 32 + l32) * PST + 4 * g;
    lo.p_rd = l32 * PST + 8 * g;
    lo.q = OFF_Q + (wave * 32 + l32) * 32 + 16 * g;
    return lo;
}

// Keeps the compiler from hoisting per-read address arithmetic out of the
// tile loop (which would hold one register per distinct address) or turning
// lane-dependent loop terms into induction variables that live in VGPRs
// across the whole kernel.
__device__ __forceinline__ void opaque(int& x) { asm volatile("" : "+v"(x)); }


// Row indices of tile T for this wave: lanes 0..7 copy 4 bytes each into the
// ring slot (positions past the end repeat the last row, so every tile costs
// the same number of copies).
__device__ __forceinline__ void fetch_idx(const SplitCtx& sc, int T, int* __restrict__ slot) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    if (lane < 8) {
        int lp = wave * 8 + lane;
        opaque(lp);
        const int pos = min(sc.start + T * R + lp, sc.end - 1);
        buffer_to_lds4(sc.list, (uint32_t)pos * 4u, (MLA_LDS void*)slot);
    }
}

// Copy this wave's 8 rows of a tile into a stage: 8 latent copies of 1 KB
// (lane l moves chunk l ^ swz(r), which lands in slot l) and one copy of
// their 8 rotary parts.
__device__ __forceinline__ void issue_tile(const AttnArgs& a, const SplitCtx& sc, char* __restrict__ stage,
                                           const int* __restrict__ slot) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const u32x4 i0 = *(const u32x4*)slot;
    const u32x4 i1 = *(const u32x4*)(slot + 4);
    const int idx_rot = slot[lane >> 3];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = wave * 8 + j;
        const uint32_t t = __builtin_amdgcn_readfirstlane(j < 4 ? i0[j & 3] : i1[j & 3]);
        buffer_to_lds16(sc.kv, t * (uint32_t)a.kv_st * 2u + ((lane ^ lat_swz(r)) << 4),
                        (MLA_LDS void*)(stage + r * 1024));
    }
    const int r = wave * 8 + (lane >> 3);
    buffer_to_lds16(sc.pe, (uint32_t)idx_rot * (uint32_t)a.pe_st * 2u + (((lane & 7) ^ ((r >> 1) & 7)) << 4),
                    (MLA_LDS void*)(stage + LAT + wave * 8 * 128));
}

// v_mfma_f32_32x32x16_bf16 with the accumulator pinned to VGPRs.  The 256
// AGPRs hold the PV accumulators; if the compiler also placed this chain's
// accumulator there it would have to move PV accumulators out and back every
// tile.  The compiler does not track MFMA hazards across inline asm, so the
// wait states are explicit: "s_nop 1" covers a VALU write of an operand just
// before the MFMA, and qk_settle pads 21 wait states between the last MFMA
// (16 passes) and any other read of its result.
__device__ __forceinline__ void qk_mfma_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_mfma(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_settle(f32x16& acc) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(acc));
}

// QK^T of one tile for this wave's 32 heads: S^T[32 rows][32 heads]; tile
// operands are read two steps ahead of the MFMAs.
__device__ __forceinline__ void qk_tile(const char* __restrict__ st, const char* __restrict__ smem_q,
                                        LaneOffsets lo, const bf16x8 (&qreg)[QK_REG], f32x16& acc) {
    opaque(lo.qk);
    opaque(lo.rot);
    auto off = [&](int ks) { return ks < 32 ? (lo.qk ^ ((ks & 7) << 5)) + 256 * (ks >> 3) : lo.rot ^ ((ks - 32) << 5); };
    bf16x8 kv[3], qv[3];
    auto load = [&](int ks) {
        kv[ks % 3] = *(const bf16x8*)(st + off(ks));
        if (ks >= QK_REG) qv[ks % 3] = *(const bf16x8*)(smem_q + lo.q + 4096 * (ks - QK_REG));
    };
    load(0);
    load(1);
#pragma unroll
    for (int ks = 0; ks < ROW / 16; ++ks) {
        if (ks + 2 < ROW / 16) load(ks + 2);
        const bf16x8 q = ks < QK_REG ? qreg[ks < QK_REG ? ks : 0] : qv[ks % 3];
        if (ks == 0) qk_mfma_first(acc, kv[0], q);
        else qk_mfma(acc, kv[ks % 3], q);
    }
    qk_settle(acc);
}

// Softmax of 4 consecutive rows (8j + 4g .. +3) of this lane's head:
// scale, mask rows past the end, exponentiate against the reference maximum.
__device__ __forceinline__ bf16x4 soft4(PassState& ps, const f32x16& acc, int j, int rem, float scale_log2) {
    bf16x4 pk;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float x = 8 * j + r < rem ? acc[4 * j + r] * scale_log2 : -INFINITY;
        ps.m_true = fmaxf(ps.m_true, x);
        const float p = __builtin_amdgcn_exp2f(fminf(x - ps.m_ref, P_EXP_LIMIT));
        ps.lsum += p;
        pk[r] = f2bf(p);
    }
    return pk;
}

// PV of one tile (O^T += V^T . P^T) with, when has_next, the softmax of the
// next tile interleaved (acc in, P^T of the next tile out).
__device__ __forceinline__ void pv_tile(const char* __restrict__ st, const bf16* __restrict__ p_in,
                                        bf16* __restrict__ p_out, LaneOffsets lo, PassState& ps,
                                        const f32x16& acc, bool has_next, int rem_next, float scale_log2) {
    opaque(lo.tr[0]);
    opaque(lo.tr[1]);
    const bf16* pb = p_in + lo.p_rd;
    auto tr = [&](int kt, int cb) {
        const bf16x4 lo0 = lds_read_tr16((const MLA_LDS void*)(st + (lo.tr[0] ^ (cb << 6)) + 16384 * kt));
        const bf16x4 hi0 = lds_read_tr16((const MLA_LDS void*)(st + (lo.tr[1] ^ (cb << 6)) + 16384 * kt));
        return cat(lo0, hi0);
    };
    bf16x8 av[2], pvb[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) pvb[nb] = *(const bf16x8*)(pb + 32 * nb * PST);
    av[0] = tr(0, 0);
#pragma unroll
    for (int step = 0; step < 8; ++step) {
        const int cb = step & 3;
        if (step + 1 < 8) av[(step + 1) & 1] = tr((step + 1) >> 2, (step + 1) & 3);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            ps.o[nb][cb] = mfma32(av[step & 1], pvb[nb], ps.o[nb][cb]);
            if (step == 3) pvb[nb] = *(const bf16x8*)(pb + 32 * nb * PST + 16);   // P^T rows 16..31
        }
        // the softmax of the next tile, one group of 4 rows per step from
        // step 4 on (the QK^T results are complete by then)
        if (has_next && step >= 4) {
            const int j = step - 4;
            *(bf16x4*)(p_out + lo.p_wr + 8 * j) = soft4(ps, acc, j, rem_next, scale_log2);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One main-loop iteration's work after the barrier: copy tile it+2 and the
// indices of tile it+4, QK^T of tile it+1, PV of tile it with the softmax
// of tile it+1.  Distinct restrict-qualified pointers tell the compiler
// that the reads never touch the stage or slot being filled, so it does not
// wait for the copies in flight.
__device__ __forceinline__ void main_step(const AttnArgs& a, const SplitCtx& sc, int it, const LaneOffsets& lo,
                                          const char* __restrict__ smem_q, const bf16x8 (&qreg)[QK_REG], PassState& ps,
                                          char* __restrict__ dma_stage, const int* __restrict__ dma_slot,
                                          int* __restrict__ idx_slot, const char* __restrict__ qk_stage,
                                          const char* __restrict__ pv_stage, const bf16* __restrict__ p_in,
                                          bf16* __restrict__ p_out) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 5;
    const int nt = sc.ntiles;
    if (it + 2 < nt) issue_tile(a, sc, dma_stage, dma_slot);
    if (it + 4 < nt) fetch_idx(sc, it + 4, idx_slot);
    const bool has_next = it + 1 < nt;
    f32x16 acc;
    if (has_next) qk_tile(qk_stage, smem_q, lo, qreg, acc);
    int g4 = 4 * g;
    opaque(g4);
    const int rem_next = sc.end - sc.start - (it + 1) * R - g4;
    pv_tile(pv_stage, p_in, p_out, lo, ps, acc, has_next, rem_next, a.scale_log2);
}

// One pass over the split (see attn_kernel).  Returns true when the pass
// must be repeated with the exact maximum (then m_ref holds it).
//
// Copy pipeline, per wave and tile T: 9 global->LDS copies issued in
// iteration T-2 and the 4-byte index copy issued in iteration T-4.
// Iteration t waits until tile t+1 has landed; only the index copy issued
// after it may still be in flight.
__device__ __forceinline__ bool attn_pass(const AttnArgs& a, const SplitCtx& sc, char* smem,
                                          float& m_ref, bool known) {
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int g = lane >> 5, l32 = lane & 31;
    __syncthreads();                               // previous pass done
    // This wave's 32 heads of Q~ (QK^T B operand): feature block ks (16
    // features) holds features 16 ks + 8 (lane/32) .. +7 of head 32 wave +
    // lane%32; blocks below QK_REG stay in registers, the rest go to LDS.
    bf16x8 qreg[QK_REG];
    {
        const int h = sc.h0 + wave * 32 + l32;
        const bool ok = h < a.H;
        const bf16* q = a.qt + ((long long)sc.b * a.H + (ok ? h : 0)) * ROW + 8 * g;
#pragma unroll
        for (int ks = 0; ks < QK_REG; ++ks) qreg[ks] = ok ? *(const bf16x8*)(q + 16 * ks) : bf16x8{};
        char* qd = smem + OFF_Q + (wave * 32 + l32) * 32 + 16 * g;
#pragma unroll
        for (int i = 0; i < QK_LDS; ++i)
            *(bf16x8*)(qd + 4096 * i) = ok ? *(const bf16x8*)(q + 16 * (QK_REG + i)) : bf16x8{};
    }

    const int start = sc.start, end = sc.end, nt = sc.ntiles;
    int* idx_ring = (int*)(smem + OFF_IDX) + wave * 8;      // + slot * 32
    auto stage = [&](int T) { return smem + (T % NST) * STAGE; };
    auto pbuf = [&](int T) { return (bf16*)(smem + OFF_P + (T & 1) * PBYTES); };
    auto slot = [&](int T) { return idx_ring + (T % NSLOT) * 32; };

    const LaneOffsets lo = lane_offsets();
    PassState ps;
    ps.m_ref = m_ref;
    ps.m_true = known ? m_ref : -INFINITY;
    ps.lsum = 0.f;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) ps.o[nb][cb] = f32x16{};

    // ---- prologue: indices for tiles 0..3, copies for tiles 0 and 1 ----
    if (nt > 0) {
        fetch_idx(sc, 0, slot(0));
        if (nt > 1) fetch_idx(sc, 1, slot(1));
        wait_vmcnt<0>();
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            if (T < nt) issue_tile(a, sc, stage(T), slot(T));
            if (T + 2 < nt) fetch_idx(sc, T + 2, slot(T + 2));
        }
        wait_vm((nt > 2) + 9 * (nt > 1) + (nt > 3));
        __syncthreads();                           // tile 0 visible
        f32x16 acc;
        qk_tile(stage(0), smem, lo, qreg, acc);
        // reference maximum: the first tile's, floored to an integer so that
        // exp2(x - m_ref) differs from exp2(x) by a power of two only and its
        // bf16 rounding does not depend on where the splits fall
        const int rem = end - (start + 4 * g);
        if (!known) {
            float mt = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = 8 * (i >> 2) + (i & 3);
                mt = fmaxf(mt, row < rem ? acc[i] * a.scale_log2 : -INFINITY);
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            ps.m_ref = floorf(mt);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) *(bf16x4*)(pbuf(0) + lo.p_wr + 8 * j) = soft4(ps, acc, j, rem, a.scale_log2);
    }

    // ---- main loop ----
    for (int it = 0; it < nt; ++it) {
        wait_vm(it + 3 < nt ? 1 : 0);
        lds_barrier();          // tile it+1 resident, P(it) visible, stage (it-1)%3 free
        main_step(a, sc, it, lo, smem, qreg, ps, stage(it + 2), slot(it + 2), slot(it + 4), stage(it + 1), stage(it),
                  pbuf(it), pbuf(it + 1));
    }

    // ---- overflow check, then normalise and write ----
    float* lred = (float*)(smem + OFF_L);
    float* mfin = (float*)(smem + OFF_M);
    int* flag = (int*)(smem + OFF_FLAG);
    __syncthreads();
    if (tid == 0) *flag = 0;
    __syncthreads();
    if (!known && ps.m_true > ps.m_ref + P_EXP_LIMIT) *flag = 1;
    const float lt = ps.lsum + __shfl_xor(ps.lsum, 32);
    const float mx = fmaxf(ps.m_true, __shfl_xor(ps.m_true, 32));
    if (g == 0) {
        lred[wave * 32 + l32] = lt;
        mfin[wave * 32 + l32] = ps.m_ref;
    }
    __syncthreads();
    if (!known && *flag) {
        m_ref = floorf(mx);
        return true;
    }
    const long long pbase = ((long long)sc.b * a.S + sc.s) * a.H;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int hl = nb * 32 + l32, h = sc.h0 + hl;
        const float l = lred[hl];
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

// Split-KV attention workgroup: 4 waves, 128 heads, 32-row tiles.  Wave w:
// QK role: S^T[32 rows][heads 32w..32w+31] of each tile with
// v_mfma_f32_32x32x16_bf16 (M = rows, N = heads, K = 576), its heads of Q~
// held in registers.  PV role: O^T[latent columns 128w..128w+127][128 heads]
// with v_mfma_f32_32x32x16_bf16 (M = columns, N = heads, K = rows), V^T read
// with ds_read_b64_tr_b16 and P^T from LDS.  The reference maximum of each
// head is the (floored) maximum of the split's first tile; later
// probabilities are exp2(x - m_ref) and may exceed 1 (fp32 and bf16 share
// the 8-bit exponent), so the accumulators are never rescaled.  If a head's
// true maximum exceeds m_ref by more than P_EXP_LIMIT the split is run again
// with the exact maximum as reference.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void attn_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
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
    sc.h0 = hgi * HW;
    const int cnt = a.counts[sc.b];
    int rps = (cnt + a.S - 1) / a.S;
    rps = (rps + 7) & ~7;
    sc.start = min(sc.s * rps, cnt);
    sc.end = min(sc.start + rps, cnt);
    sc.ntiles = (sc.end - sc.start + R - 1) / R;
    sc.list = make_rsrc(a.list + (long long)sc.b * a.K, (uint32_t)a.K * 4u);
    sc.kv = make_rsrc(a.kv + (long long)sc.b * a.kv_sb, a.kv_win);
    sc.pe = make_rsrc(a.pe + (long long)sc.b * a.pe_sb, a.pe_win);

    float m_ref = 0.f;
    for (int pass = 0; pass < 2; ++pass)
        if (!attn_pass(a, sc, smem, m_ref, pass == 1)) break;
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
    a.kv_win = (uint32_t)((long long)(p.max_cache_len - 1) * p.kv_stride_t * 2 + RANK * 2);
    a.pe_win = (uint32_t)((long long)(p.max_cache_len - 1) * p.pe_stride_t * 2 + 64 * 2);
    a.opart = (bf16*)w.opart; a.lsepart = w.lsepart;
    const dim3 grid(attn_grid(plan, p.B)), block(256);
    hipLaunchKernelGGL(attn_kernel, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace mla
