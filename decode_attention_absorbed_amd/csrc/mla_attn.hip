// Split-KV sparse attention over the latent cache (bf16 MFMA, fp32 accumulation).
//
// Computes, for one sequence b, one split s of its selected positions and a
// group of 128 heads, the partial softmax-weighted latent sum
//   o[h, :] = sum_t exp2(x[h,t] - m[h]) C[b,t,:],  l[h] = sum_t exp2(x[h,t] - m[h]),
//   x[h,t] = scale * log2(e) * (Q~[b,h,:] . [C[b,t,:] ; R[b,t,:]])
// and writes o / l (bf16) and m + log2(l).  The scores are the latent plus
// rotary dot products of the MQA decode branch; positions outside the
// selection never enter (their additive mask is -inf, exp2 gives 0).
// Source: atlas page "Rotated query part" (also "Query content heads",
// "Attention weights"), excerpt mla-decode; the split-KV partition and the
// softmax bookkeeping are this library's, not the pages'.
//
// Workgroup: 4 waves (one per SIMD), 128 heads, tiles of 32 selected rows
// copied into a 4-stage LDS ring by buffer->LDS DMA, each wave copying 8
// rows.  Every selected row is read from HBM once per (sequence, split).
// Wave w owns heads 32w..32w+31 from scores to output:
//   QK^T: S^T[32 rows][32 heads] = K_tile . Q~^T, v_mfma_f32_32x32x16_bf16
//         (M = rows, N = heads, K = 576).  The wave's Q~ is held in
//         registers (33 of 36 feature blocks) and LDS (3 blocks).
//   softmax: in registers; each lane holds 16 rows of one head.
//   PV:   O^T[512 columns][32 heads] += V^T . P^T, v_mfma_f32_32x32x16_bf16
//         (M = columns, N = heads, K = rows).  P^T comes straight from the
//         QK^T accumulator: the rows of the contraction are ordered to match
//         the accumulator layout, and V^T is read in that order with
//         ds_read_b64_tr_b16.  O^T lives in the 256 AGPRs.
// No wave waits for another's softmax, so QK^T and PV read the same stage
// and three tiles are in flight while one is consumed.
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

constexpr int HW = 128;                // heads per workgroup
constexpr int R = 32;                  // rows per tile
constexpr int NST = 4;                 // LDS stages
constexpr int LAT = R * RANK * 2;      // latent region of a stage: row r at r * 1 KB
constexpr int STAGE = R * ROW * 2;     // + rotary region: row r at LAT + r * 128
constexpr int NSLOT = 4;               // index ring slots
constexpr int OFF_IDX = NST * STAGE;               // [NSLOT][4 waves][8] int: row indices
constexpr int OFF_FLAG = OFF_IDX + NSLOT * 4 * 8 * 4;
constexpr int QK_REG = 33;                         // Q~ feature blocks 0..32 live in registers,
constexpr int QK_LDS = ROW / 16 - QK_REG;          // blocks 33..35 in LDS: [block][head][16]
constexpr int OFF_Q = OFF_FLAG + 16;
constexpr int QK_DEPTH = 4;                        // QK^T operand reads run this many steps ahead
constexpr int PV_DEPTH = 4;                        // PV operand reads run this many steps ahead
constexpr int LDS_BYTES = OFF_Q + QK_LDS * HW * 32;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

// Tile layout in LDS.  Latent region: row r at r * 1024 bytes, its 16-byte
// chunk c (8 latent features) at slot c ^ swz(r), with the 5-bit swizzle
// swz(r) = ((r&3)<<2) | ((r>>2)&3) | (r&16), a bijection on the 32 rows of a
// tile.  The LDS serves 32 lanes per cycle: the QK^T operand read (32 rows at
// one chunk) then touches 32 distinct 16-byte slots, and each half of a
// transposed PV read (4 rows x 4 chunks) 16 distinct slots.
// Rotary region: row r at r * 128 bytes, chunk c' (0..7) at slot c' ^ ((r>>1)&7).
__device__ __forceinline__ int lat_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3) | (r & 16); }

// The wave index, known to the compiler as wave-uniform (an SGPR).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Largest exponent (log2) a probability may reach relative to the
// reference maximum before the split is recomputed with the exact maximum.
constexpr float P_EXP_LIMIT = 64.f;

// s_waitcnt vmcnt(n) for the counts the copy pipeline produces (n is
// rounded down to one of them, which only waits longer).
__device__ __forceinline__ void wait_vm(int n) {
    if (n >= 53) wait_vmcnt<53>();
    else if (n >= 52) wait_vmcnt<52>();
    else if (n >= 51) wait_vmcnt<51>();
    else if (n >= 42) wait_vmcnt<42>();
    else if (n >= 33) wait_vmcnt<33>();
    else if (n >= 20) wait_vmcnt<20>();
    else if (n >= 19) wait_vmcnt<19>();
    else if (n >= 18) wait_vmcnt<18>();
    else if (n >= 9) wait_vmcnt<9>();
    else wait_vmcnt<0>();
}

// Workgroup barrier for the main loop.  It waits for this wave's LDS
// operations only: the buffer->LDS copies still in flight target stages no
// one reads before a later, explicit vmcnt wait (__syncthreads would drain
// them).  The asm memory clobber keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

// Keeps the compiler from hoisting per-read address arithmetic out of the
// tile loop (which would hold one register per distinct address) or turning
// lane-dependent loop terms into induction variables that live in VGPRs
// across the whole kernel.
__device__ __forceinline__ void opaque(int& x) { asm volatile("" : "+v"(x)); }

struct SplitCtx {
    int b, s, h0, start, end, ntiles;
    rsrc_t list;        // the sequence's compacted row list
    rsrc_t kv;          // the sequence's rows of the latent cache
    rsrc_t pe;          // the sequence's rows of the rotary-key cache
};

// Per-lane LDS offsets.  The swizzles are XORs on address bits that the
// bases leave zero, so every operand address is a base XOR a constant.
//   QK latent chunk 16j + 2k + lane/32 of row lane%32:  qk ^ (k << 5) ^ (j << 8)
//   QK rotary chunk 2k + lane/32:                       rot ^ (k << 5)
//   PV read rd of column block cb (32 columns), rows 16 kt + 8 rd + 4 (lane/32) + 0..3:
//                                                       (tr[rd] ^ ((cb & 3) << 6)) + 256 ((cb >> 2) ^ kt) + 16384 kt
//   Q~ block 33 + i (LDS part):                         q + 4096 i
struct LaneOffsets {
    int qk, rot, tr[2], q;
};

__device__ __forceinline__ LaneOffsets lane_offsets() {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 5, l32 = lane & 31;
    LaneOffsets lo;
    // chunk (16j + 2k + g) ^ sw of row l32: bit 0 is g ^ (sw & 1), bits 1-3
    // are k ^ ((sw >> 1) & 7), bits 4-5 are j ^ (sw >> 4)
    const int sw = lat_swz(l32);
    lo.qk = l32 * 1024 + ((g ^ (sw & 1)) << 4) + (((sw >> 1) & 7) << 5) + ((sw >> 4) << 8);
    const int u = (l32 >> 1) & 7;
    lo.rot = LAT + l32 * 128 + ((g ^ (u & 1)) << 4) + ((u >> 1) << 5);
    // Transposed reads: in 16-lane block blk, lane 4j + qq addresses row
    // 16 kt + 8 rd + 4 (blk >> 1) + j, columns 16 (blk & 1) + 4 qq .. +3 of the
    // column block; lane i of the block receives column 16 (blk & 1) + i of
    // the rows 16 kt + 8 rd + 4 (blk >> 1) + 0..3.  The row's swizzle has bits
    // 2-3 = j, bits 0-1 = (2 rd + (blk >> 1)) & 3 and bit 4 = kt.
    const int blk = lane >> 4, L = lane & 15, j = L >> 2, qq = L & 3;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
        const int lowsw = (2 * rd + (blk >> 1)) & 3;
        lo.tr[rd] = (8 * rd + 4 * (blk >> 1) + j) * 1024 + (((2 * (blk & 1) + (qq >> 1)) ^ lowsw) << 4) +
                    (qq & 1) * 8 + (j << 6);
    }
    lo.q = OFF_Q + (wave * 32 + l32) * 32 + 16 * g;
    return lo;
}

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

// Row indices of one tile for this wave, read from its ring slot.
struct TileRows {
    u32x4 i0, i1;       // rows 8 wave + 0..7 (latent copies)
    int rot;            // row 8 wave + lane/8 (rotary copy)
};

__device__ __forceinline__ TileRows read_rows(const int* __restrict__ slot) {
    const int lane = threadIdx.x & 63;
    TileRows tr;
    tr.i0 = *(const u32x4*)slot;
    tr.i1 = *(const u32x4*)(slot + 4);
    tr.rot = slot[lane >> 3];
    return tr;
}

// Copy row j (0..7) of this wave's 8 rows of a tile into a stage: 1 KB, lane
// l moves chunk l ^ swz(r), which lands in slot l.
__device__ __forceinline__ void issue_row(const AttnArgs& a, const SplitCtx& sc, char* __restrict__ stage,
                                          const TileRows& tr, int j) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int r = wave * 8 + j;
    const uint32_t t = __builtin_amdgcn_readfirstlane(j < 4 ? tr.i0[j & 3] : tr.i1[j & 3]);
    buffer_to_lds16(sc.kv, t * (uint32_t)a.kv_st * 2u + ((lane ^ lat_swz(r)) << 4), (MLA_LDS void*)(stage + r * 1024));
}

// Copy the rotary parts (128 bytes each) of this wave's 8 rows.
__device__ __forceinline__ void issue_rot(const AttnArgs& a, const SplitCtx& sc, char* __restrict__ stage,
                                          const TileRows& tr) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int r = wave * 8 + (lane >> 3);
    buffer_to_lds16(sc.pe, (uint32_t)tr.rot * (uint32_t)a.pe_st * 2u + (((lane & 7) ^ ((r >> 1) & 7)) << 4),
                    (MLA_LDS void*)(stage + LAT + wave * 8 * 128));
}

// All 9 copies of this wave's part of a tile (prologue).
__device__ __forceinline__ void issue_tile(const AttnArgs& a, const SplitCtx& sc, char* __restrict__ stage,
                                           const int* __restrict__ slot) {
    const TileRows tr = read_rows(slot);
#pragma unroll
    for (int j = 0; j < 8; ++j) issue_row(a, sc, stage, tr, j);
    issue_rot(a, sc, stage, tr);
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

// QK^T of one tile for this wave's 32 heads: S^T[32 rows][32 heads] in acc
// (lane l: head l%32, rows 8(i/4) + 4(l/32) + i%4 for i = 0..15); tile
// operands are read two steps ahead of the MFMAs.  hook(ks) runs after the
// MFMA of step ks: the copies for a later tile are spread over the chain so
// that a stalled copy issue never leaves the matrix unit idle for long.
template <typename Hook>
__device__ __forceinline__ void qk_tile(const char* __restrict__ st, const char* __restrict__ smem_q,
                                        LaneOffsets lo, const bf16x8 (&qreg)[QK_REG], f32x16& acc, Hook&& hook) {
    opaque(lo.qk);
    opaque(lo.rot);
    constexpr int NK = ROW / 16, D = QK_DEPTH;
    auto off = [&](int ks) { return ks < 32 ? lo.qk ^ (((ks & 7) << 5) | ((ks >> 3) << 8)) : lo.rot ^ ((ks - 32) << 5); };
    bf16x8 kv[D + 1], qv[D + 1];
    auto load = [&](int ks) {
        kv[ks % (D + 1)] = *(const bf16x8*)(st + off(ks));
        if (ks >= QK_REG) qv[ks % (D + 1)] = *(const bf16x8*)(smem_q + lo.q + 4096 * (ks - QK_REG));
    };
#pragma unroll
    for (int ks = 0; ks < D; ++ks) load(ks);
    // two interleaved chains (even and odd feature blocks): a single
    // dependent chain runs at the MFMA latency, two at its throughput
    f32x16 acc1;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
        if (ks + D < NK) load(ks + D);
        const bf16x8 q = ks < QK_REG ? qreg[ks < QK_REG ? ks : 0] : qv[ks % (D + 1)];
        const bf16x8 k = kv[ks % (D + 1)];
        if (ks == 0) qk_mfma_first(acc, k, q);
        else if (ks == 1) qk_mfma_first(acc1, k, q);
        else if (ks & 1) qk_mfma(acc1, k, q);
        else qk_mfma(acc, k, q);
        hook(ks);
        __builtin_amdgcn_sched_barrier(0);
    }
    qk_settle(acc);
    qk_settle(acc1);
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] += acc1[i];
}

// Softmax state of this lane's head (half of its rows: the other half is in
// lane ^ 32) and the O^T accumulators of the wave's 32 heads.
struct PassState {
    float m_ref, m_true, lsum;
    f32x16 o[16];       // [cb]: columns 32cb + 8(i/4) + 4(lane/32) + i%4 of head lane%32
};

// Probabilities of accumulator entries 8kt .. 8kt+7 (rows 16kt + 8(e/4) +
// 4(lane/32) + e%4): scale, mask rows past the end, exponentiate against the
// reference maximum; returned as the PV B operand of K step kt.
__device__ __forceinline__ bf16x8 soft8(PassState& ps, const f32x16& acc, int kt, int rem, float scale_log2) {
    bf16x8 pk;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int i = 8 * kt + e;
        const float x = 8 * (i >> 2) + (i & 3) < rem ? acc[i] * scale_log2 : -INFINITY;
        ps.m_true = fmaxf(ps.m_true, x);
        const float p = __builtin_amdgcn_exp2f(fminf(x - ps.m_ref, P_EXP_LIMIT));
        ps.lsum += p;
        pk[e] = f2bf(p);
    }
    return pk;
}

// PV of one tile: O^T[cb] += V^T(kt, cb) . P^T(kt) for 16 column blocks and
// two K steps of 16 rows.  The K index k = 8 (lane/32) + e of step kt is row
// 16kt + 8(e/4) + 4(lane/32) + e%4, matching soft8's operand; the A operand
// (columns x those rows) is two transposed reads of 4 rows each.  The second
// K step's probabilities are computed while the first step's MFMAs run.
__device__ __forceinline__ void pv_tile(const char* __restrict__ st, LaneOffsets lo, PassState& ps,
                                        const f32x16& acc, int rem, float scale_log2) {
    opaque(lo.tr[0]);
    opaque(lo.tr[1]);
    auto tr = [&](int kt, int cb) {
        const int o = 256 * ((cb >> 2) ^ kt) + 16384 * kt;
        const bf16x4 r0 = lds_read_tr16((const MLA_LDS void*)(st + (lo.tr[0] ^ ((cb & 3) << 6)) + o));
        const bf16x4 r1 = lds_read_tr16((const MLA_LDS void*)(st + (lo.tr[1] ^ ((cb & 3) << 6)) + o));
        return cat(r0, r1);
    };
    constexpr int D = PV_DEPTH;
    bf16x8 av[D + 1];
#pragma unroll
    for (int st2 = 0; st2 < D; ++st2) av[st2] = tr(st2 >> 4, st2 & 15);
    bf16x8 p0 = soft8(ps, acc, 0, rem, scale_log2);
    bf16x8 p1;
#pragma unroll
    for (int step = 0; step < 32; ++step) {
        const int kt = step >> 4, cb = step & 15;
        if (step + D < 32) av[(step + D) % (D + 1)] = tr((step + D) >> 4, (step + D) & 15);
        ps.o[cb] = mfma32(av[step % (D + 1)], kt == 0 ? p0 : p1, ps.o[cb]);
        if (step == 3) p1 = soft8(ps, acc, 1, rem, scale_log2);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One pass over the split (see attn_kernel).  Returns true when the pass
// must be repeated with the exact maximum (then m_ref holds it).
//
// Copy pipeline, per wave: iteration j fetches the indices of tile j+6 and
// copies tile j+3 (9 copies, spread over the QK^T chain) into the stage tile
// j-1 left; the prologue plays iterations -3..-1.  Iteration it waits until tile it has landed:
// the copies issued after it (indices of it+4 and it+5, tiles it+1 and
// it+2) may still be in flight.
__device__ __forceinline__ bool attn_pass(const AttnArgs& a, const SplitCtx& sc, char* smem,
                                          float& m_ref, bool known) {
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int g = lane >> 5, l32 = lane & 31;
    const int nt = sc.ntiles;
    int* flag = (int*)(smem + OFF_FLAG);
    __syncthreads();                               // previous pass done
    if (tid == 0) *flag = 0;

    int* idx_ring = (int*)(smem + OFF_IDX) + wave * 8;      // + slot * 32
    auto stage = [&](int T) { return smem + (T % NST) * STAGE; };
    auto slot = [&](int T) { return idx_ring + (T % NSLOT) * 32; };

    const LaneOffsets lo = lane_offsets();
    PassState ps;
    ps.m_ref = m_ref;
    ps.m_true = known ? m_ref : -INFINITY;
    ps.lsum = 0.f;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) ps.o[cb] = f32x16{};

    // ---- prologue ----
    // Order of the copies (so that tile 0 does not wait behind Q~): indices
    // of tiles 0..2; Q~ blocks 33..35 into LDS; indices of tile 3 and tile 0;
    // Q~ blocks 0..32 into registers; indices 4 and tile 1; indices 5 and
    // tile 2.  Q~ of this wave's 32 heads (QK^T B operand): block ks holds
    // features 16 ks + 8 (lane/32) .. +7 of head h0 + 32 wave + lane%32;
    // heads past H read as zero (outside the buffer window).
    const rsrc_t qsrc = make_rsrc(a.qt + (long long)sc.b * a.H * ROW, (uint32_t)a.H * ROW * 2u);
    bf16x8 qreg[QK_REG];
    if (nt > 0) {
#pragma unroll
        for (int T = 0; T < 3; ++T)
            if (T < nt) fetch_idx(sc, T, slot(T));
        wait_vmcnt<0>();
    }
    {
        // LDS part: lane l fills bytes 16 l of the wave's 1 KB row of block i,
        // i.e. head 32 wave + l/2, features 16 (QK_REG + i) + 8 (l & 1)
        const uint32_t hq = (uint32_t)(sc.h0 + wave * 32 + (lane >> 1));
#pragma unroll
        for (int i = 0; i < QK_LDS; ++i)
            buffer_to_lds16(qsrc, hq * (ROW * 2) + (16 * (QK_REG + i) + 8 * (lane & 1)) * 2,
                            (MLA_LDS void*)(smem + OFF_Q + 4096 * i + 1024 * wave));
    }
    if (nt > 0) {
        if (3 < nt) fetch_idx(sc, 3, slot(3));
        issue_tile(a, sc, stage(0), slot(0));
    }
    {
        const uint32_t h = (uint32_t)(sc.h0 + wave * 32 + l32);
#pragma unroll
        for (int ks = 0; ks < QK_REG; ++ks)
            qreg[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qsrc, h * (ROW * 2) + (16 * ks + 8 * g) * 2, 0, 0));
    }
    if (nt > 0) {
#pragma unroll
        for (int T = 1; T < 3; ++T) {
            if (T + 3 < nt) fetch_idx(sc, T + 3, slot(T + 3));
            if (T < nt) issue_tile(a, sc, stage(T), slot(T));
        }
    }

    // ---- main loop ----
    for (int it = 0; it < nt; ++it) {
        // copies issued after tile it: indices of it+4 and it+5, tiles it+1
        // and it+2, and (first iteration only) the Q~ register loads
        wait_vm((it + 4 < nt) + 9 * (it + 1 < nt) + (it + 5 < nt) + 9 * (it + 2 < nt) + (it == 0 ? QK_REG : 0));
        lds_barrier();          // tile it resident and visible; stage (it-1)%4 free
        const bool do_fetch = it + 6 < nt, do_issue = it + 3 < nt;
        TileRows rows;
        if (do_issue) rows = read_rows(slot(it + 3));
        char* dst = stage(it + 3);
        f32x16 acc;
        qk_tile(stage(it), smem, lo, qreg, acc, [&](int ks) {
            if (ks == 1 && do_fetch) fetch_idx(sc, it + 6, slot(it + 6));
            if (do_issue) {
                if (ks >= 2 && ks <= 30 && (ks - 2) % 4 == 0) issue_row(a, sc, dst, rows, (ks - 2) / 4);
                if (ks == 34) issue_rot(a, sc, dst, rows);
            }
        });
        int g4 = 4 * g;
        opaque(g4);
        const int rem = sc.end - sc.start - it * R - g4;
        if (it == 0 && !known) {
            // reference maximum: the first tile's, floored to an integer so
            // that exp2(x - m_ref) differs from exp2(x) by a power of two only
            // and its bf16 rounding does not depend on where the splits fall
            float mt = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                mt = fmaxf(mt, 8 * (i >> 2) + (i & 3) < rem ? acc[i] * a.scale_log2 : -INFINITY);
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            ps.m_ref = floorf(mt);
        }
        pv_tile(stage(it), lo, ps, acc, rem, a.scale_log2);
    }

    // ---- overflow check, then normalise and write ----
    __syncthreads();
    const float mx = fmaxf(ps.m_true, __shfl_xor(ps.m_true, 32));
    if (!known && mx > ps.m_ref + P_EXP_LIMIT) *flag = 1;
    __syncthreads();
    if (!known && *flag) {
        m_ref = floorf(mx);
        return true;
    }
    const float l = ps.lsum + __shfl_xor(ps.lsum, 32);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    // Stage the wave's 32 normalised bf16 rows in the (now idle) tile area,
    // 1 KB per head with 16-byte chunk c at slot c ^ head, then write each
    // head's row with one fully coalesced 1 KB store.
    char* orow = smem + wave * 32768;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            bf16x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = f2bf(ps.o[cb][4 * q4 + r] * inv);
            *(bf16x4*)(orow + l32 * 1024 + (((4 * cb + q4) ^ l32) << 4) + 8 * g) = v;
        }
    }
    const long long prow0 = ((long long)sc.b * a.S + sc.s) * a.H + sc.h0 + wave * 32;
    if (g == 0 && sc.h0 + wave * 32 + l32 < a.H) a.lsepart[prow0 + l32] = l > 0.f ? ps.m_ref + log2f(l) : -INFINITY;
    __builtin_amdgcn_s_waitcnt(0xC07F);            // this wave's LDS writes done (only it reads them)
#pragma unroll 4
    for (int hr = 0; hr < 32; ++hr) {
        if (sc.h0 + wave * 32 + hr >= a.H) break;
        const u32x4 v = *(const u32x4*)(orow + hr * 1024 + ((lane ^ hr) << 4));
        *(u32x4*)(a.opart + (prow0 + hr) * RANK + 8 * lane) = v;
    }
    return false;
}

// Split-KV attention workgroup (see the top of this file).  The reference
// maximum of each head is the (floored) maximum of the split's first tile;
// later probabilities are exp2(x - m_ref) and may exceed 1 (fp32 and bf16
// share the 8-bit exponent), so the accumulators are never rescaled.  If a
// head's true maximum exceeds m_ref by more than P_EXP_LIMIT the split is
// run again with the exact maximum as reference.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void attn_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];

    // XCD-aware mapping: workgroups with ids 8 apart run on the same XCD and
    // share its L2.  The head groups of one (sequence, split) and, when there
    // are at least 8 sequences, all splits of a sequence stay on one XCD
    // (they read the same Q~ and the same cache rows).
    const int id = blockIdx.x;
    const int xcd = id & 7, k8 = id >> 3;
    const int hgi = k8 % a.HG, r8 = k8 / a.HG;
    int bsq, ssp;
    if (a.B >= 8) {
        ssp = r8 % a.S;
        bsq = (r8 / a.S) * 8 + xcd;
    } else {
        const int bs = r8 * 8 + xcd;
        bsq = bs / a.S;
        ssp = bs % a.S;
    }
    if (bsq >= a.B) return;

    SplitCtx sc;
    sc.b = bsq;
    sc.s = ssp;
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
    // B >= 8: 8 * ceil(B / 8) sequences x splits x head groups; otherwise the
    // (sequence, split) pairs rounded up to a multiple of 8, x head groups
    if (B >= 8) return ((B + 7) / 8) * 8 * plan.splits * plan.hgroups;
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
