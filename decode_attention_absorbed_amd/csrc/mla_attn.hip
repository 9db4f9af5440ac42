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
//
// With one wave per SIMD a wave issues at most one instruction every few
// cycles, so the tile loop is written to keep its instruction count well
// under the MFMA time (72 MFMAs of 32 cycles per tile): every LDS operand
// address is a per-lane base plus an immediate offset, the copies of a tile
// cost the same number of instructions whether its rows exist or not (rows
// past the split read outside the buffer window and land as zeros), so the
// copy wait is one constant count, and only the first and the last tile
// take a (uniform) branch.
#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

struct AttnArgs {
    int B, H, K, S, HG;
    float scale_log2;
    const bf16* qt;
    const bf16* qlo;           // low bf16 parts of the rotary queries: [B][H][64]
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

// Latent region of a stage.  Tile row m (the MFMA row index) is stored
// unswizzled, 1 KB at row_start(m), and the row starts are shifted against
// each other within the 256-byte bank window:
//   shift(m) = 64 (m & 3) + 16 ((m >> 2) & 3),
//   row_start(m) = 1024 (2 (shift(m) / 16) + m / 16) + shift(m),
// i.e. the rows sit in order of increasing shift, two per shift value, so
// the whole region is only 240 bytes larger than 32 KB.  The LDS serves 16
// lanes of a 16-byte read or 32 lanes of an 8-byte read per cycle:
//   QK^T operand read (lanes 0..15 = rows 0..15 at one chunk): 16 distinct
//     shifts, 16 distinct 16-byte slots;
//   transposed PV read (lanes 0..31 = rows 4q..4q+3, 64 bytes each): shifts
//     64 j + 16 (q & 3), j = 0..3, four disjoint 64-byte windows.
// A step's offset within a row (32 bytes per QK^T step, 64 bytes per PV
// column block) is then an immediate on a per-lane base.
__host__ __device__ constexpr int row_shift(int m) { return 64 * (m & 3) + 16 * ((m >> 2) & 3); }
__host__ __device__ constexpr int row_start(int m) { return 1024 * (2 * (row_shift(m) >> 4) + (m >> 4)) + row_shift(m); }
constexpr int LATB = 33024;            // >= row_start(31) + 1024 = 33008, 256-aligned
static_assert(row_start(31) + 1024 <= LATB, "latent region");
// Rotary region: row m at LATB + 128 m, its 16-byte chunk c' (0..7) at slot
// c' ^ ((m >> 1) & 7); 16 consecutive rows at one chunk hit 16 distinct slots.
constexpr int STAGE = LATB + R * 128;
constexpr int NSLOT = 4;               // index ring slots
constexpr int OFF_IDX = NST * STAGE;                // [NSLOT][4 waves][8] int: row indices (1-based)
constexpr int OFF_FLAG = OFF_IDX + NSLOT * 4 * 8 * 4;
constexpr int QK_REG = 33;                          // Q~ feature blocks 0..32 live in registers,
constexpr int QK_LDS = ROW / 16 - QK_REG;           // blocks 33..35 in LDS: [block][head][16]
constexpr int OFF_Q = OFF_FLAG + 16;
constexpr int LDS_BYTES = OFF_Q + QK_LDS * HW * 32;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
static_assert(STAGE % 256 == 0 && OFF_Q % 16 == 0, "alignment");
// Copies per wave per tile: one index fetch, 8 latent rows, one rotary copy.
constexpr int COPIES_PER_TILE = 10;
constexpr int Q_EARLY = 16;                          // Q~ register blocks loaded before tile 0's copies

// threadIdx.x through an empty asm statement, read once per pass: values
// derived from it (lane offsets, addresses) are then computed inside the
// pass instead of being hoisted out of the pass loop, where they would stay
// live across the whole tile loop and spill.
__device__ __forceinline__ int tid_opaque() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// Largest exponent (log2) a probability may reach relative to the
// reference maximum before the split is recomputed with the exact maximum.
constexpr float P_EXP_LIMIT = 64.f;

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
// tile loop (which would hold one register per distinct address).
__device__ __forceinline__ void opaque(int& x) { asm volatile("" : "+v"(x)); }

struct SplitCtx {
    int b, s, h0, start, end, ntiles;
    rsrc_t list;        // this split's part of the compacted row list
    rsrc_t kv;          // the sequence's rows of the latent cache
    rsrc_t pe;          // the sequence's rows of the rotary-key cache
};

// Per-lane constants.
//   qk:  QK^T latent operand of step ks (< 32): qk + stage + 32 ks
//   rot: QK^T rotary operand of step 32 + k:    (rot ^ (k << 5)) + stage
//   tr:  PV read rd (rows 16 kt + 8 rd + 4 (lane/32) + 0..3) of column
//        block cb:                              tr[rd] + stage + 1024 kt + 64 cb
//   q:   Q~ block 33 + i (LDS part):            q + 4096 i
//   lat: byte offset in a latent row for this lane's copy, minus one row
//        stride (the row list is 1-based)
//   rcp: the same for the rotary copy
struct LaneOffsets {
    int qk, rot, tr[2], q;
    uint32_t lat, rcp;
};

__device__ __forceinline__ LaneOffsets lane_offsets(const AttnArgs& a, int lane, int wave) {
    const int g = lane >> 5, l32 = lane & 31;
    LaneOffsets lo;
    lo.qk = row_start(l32) + 16 * g;
    // chunk 2k + g of rotary row l32 sits at slot (2k + g) ^ u: bit 0 is
    // g ^ (u & 1), bits 1-2 are k ^ (u >> 1)
    const int u = (l32 >> 1) & 7;
    lo.rot = LATB + l32 * 128 + ((g ^ (u & 1)) << 4) + ((u >> 1) << 5);
    // Transposed reads: in 16-lane block blk, lane 4j + qq addresses row
    // 8 rd + 4 (blk >> 1) + j (+16 kt), columns 16 (blk & 1) + 4 qq .. +3 of
    // the column block; lane i of the block receives column 16 (blk & 1) + i
    // of the rows 8 rd + 4 (blk >> 1) + 0..3.
    const int blk = lane >> 4, L = lane & 15, j = L >> 2, qq = L & 3;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
        lo.tr[rd] = row_start(8 * rd + 4 * (blk >> 1) + j) + 32 * (blk & 1) + 8 * qq;
    lo.q = OFF_Q + (wave * 32 + l32) * 32 + 16 * g;
    lo.lat = (uint32_t)lane * 16u - (uint32_t)a.kv_st * 2u;
    // rotary copy: lane l fills slot l & 7 of row 8 wave + l/8, i.e. chunk
    // (l & 7) ^ ((row >> 1) & 7) of that row
    const int rrow = wave * 8 + (lane >> 3);
    lo.rcp = (uint32_t)(((lane & 7) ^ ((rrow >> 1) & 7)) << 4) - (uint32_t)a.pe_st * 2u;
    return lo;
}

// Row indices of tile T for this wave: lanes 0..7 copy 4 bytes each into the
// ring slot.  The list descriptor's window is the split's rows, so positions
// past its end read 0 ("no row").
__device__ __forceinline__ void fetch_idx(const SplitCtx& sc, int T, int* __restrict__ slot, int lane, int wave) {
    if (lane < 8) buffer_to_lds4(sc.list, (uint32_t)(T * R + wave * 8 + lane) * 4u, (MLA_LDS void*)slot);
}

// Row indices of one tile for this wave, read from its ring slot.
struct TileRows {
    u32x4 i0, i1;       // rows 8 wave + 0..7 (latent copies)
    uint32_t rot;       // row 8 wave + lane/8 (rotary copy)
};

__device__ __forceinline__ TileRows read_rows(const int* __restrict__ slot, int lane) {
    TileRows tr;
    tr.i0 = *(const u32x4*)slot;
    tr.i1 = *(const u32x4*)(slot + 4);
    tr.rot = (uint32_t)slot[lane >> 3];
    return tr;
}

// Copy row j (0..7) of this wave's 8 rows of a tile into a stage: 1 KB, lane
// l moves bytes 16 l..16 l+15.  Row index t is 1-based; t = 0 gives an offset
// far outside the buffer window, and the copy writes zeros.
__device__ __forceinline__ void issue_row(const AttnArgs& a, const SplitCtx& sc, const LaneOffsets& lo,
                                          MLA_LDS char* __restrict__ dst, const TileRows& tr, int j) {
    const uint32_t t = __builtin_amdgcn_readfirstlane(j < 4 ? tr.i0[j & 3] : tr.i1[j & 3]);
    buffer_to_lds16(sc.kv, lo.lat + t * ((uint32_t)a.kv_st * 2u), (MLA_LDS void*)dst);
}

// Copy the rotary parts (128 bytes each) of this wave's 8 rows.
__device__ __forceinline__ void issue_rot(const AttnArgs& a, const SplitCtx& sc, const LaneOffsets& lo,
                                          MLA_LDS char* __restrict__ stage, const TileRows& tr, int wave) {
    buffer_to_lds16(sc.pe, lo.rcp + tr.rot * ((uint32_t)a.pe_st * 2u), (MLA_LDS void*)(stage + LATB + wave * 1024));
}

// All 9 copies of this wave's part of a tile (prologue).
__device__ __forceinline__ void issue_tile(const AttnArgs& a, const SplitCtx& sc, const LaneOffsets& lo,
                                           const int (&mst)[8], MLA_LDS char* stage, const int* __restrict__ slot,
                                           int lane, int wave) {
    const TileRows tr = read_rows(slot, lane);
#pragma unroll
    for (int j = 0; j < 8; ++j) issue_row(a, sc, lo, stage + mst[j], tr, j);
    issue_rot(a, sc, lo, stage, tr, wave);
}

// v_mfma_f32_32x32x16_bf16 with the accumulator pinned to VGPRs.  The 256
// AGPRs hold the PV accumulators; if the compiler also placed this chain's
// accumulator there it would have to move PV accumulators out and back every
// tile.  Operands come from LDS reads or registers loaded before the loop
// (no VALU write precedes them), and consecutive MFMAs of the chain use the
// same accumulator, which the hardware forwards.  The compiler does not
// track MFMA hazards across inline asm, so qk_settle pads 21 wait states
// between the last MFMA and any other read of its result.
__device__ __forceinline__ void qk_mfma_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_mfma(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_settle(f32x16& acc) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(acc));
}

// max(m, x[o..o+7]) as four v_max3_f32 (two calls cover the 16 entries).
// fmaxf on values the compiler cannot prove canonical (results of the
// inline-asm MFMAs) costs an extra NaN-quieting max per operand.
template <int o>
__device__ __forceinline__ float max9_raw(float m, const f32x16& x) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3\n\t"
        "v_max3_f32 %0, %0, %4, %5\n\t"
        "v_max3_f32 %0, %0, %6, %7\n\t"
        "v_max3_f32 %0, %0, %8, %9"
        : "=&v"(r)
        : "v"(m), "v"(x[o]), "v"(x[o + 1]), "v"(x[o + 2]), "v"(x[o + 3]), "v"(x[o + 4]), "v"(x[o + 5]),
          "v"(x[o + 6]), "v"(x[o + 7]));
    return r;
}

// Softmax state of this lane's head (half of its rows: the other half is in
// lane ^ 32) and the O^T accumulators of the wave's 32 heads.
struct PassState {
    float m_ref;        // reference maximum (log2 units)
    float mraw;         // largest raw score (before scaling) seen
    float lsum;
    f32x16 o[16];       // [cb]: columns 32cb + 8(i/4) + 4(lane/32) + i%4 of head lane%32
};

// Probability of accumulator entry i, exponentiated against the reference
// maximum.  One per MFMA step at most: v_exp_f32 runs at a quarter of the
// VALU rate, and a step whose other work outlasts its MFMA delays the next
// one.  Pairs (2j, 2j + 1) are added to the running sum as lsum + (pa + pb)
// and packed into the PV B operand together.
__device__ __forceinline__ float soft1(const f32x16& acc, int i, float m_ref, float scale_log2) {
    return __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i], scale_log2, -m_ref));
}
__device__ __forceinline__ void soft_pair(float pa, float pb, float& lsum, bf16x8& pk, int e) {
    lsum += pa + pb;
    pk[e] = f2bf(pa);
    pk[e + 1] = f2bf(pb);
    asm volatile("" : "+v"(pk));       // pack here, not all four pairs at the first use
}

// The tile loop's MFMA schedule.  Tile it is one run of 72 steps, one MFMA
// each:
//   steps  0.. 7  PV of tile it-1, K step 1 (its rows 16..31), column blocks 0..7
//   steps  8..47  QK^T of tile it: latent feature blocks 0..31, then the 4
//                 rotary blocks against the high and the low query parts
//   steps 48..55  PV of tile it-1, K step 1, column blocks 8..15
//   steps 56..71  PV of tile it, K step 0 (rows 0..15), column blocks 0..15
// so that no MFMA waits for the softmax: the probabilities of tile it's rows
// 0..15 are computed during steps 48..55, which do not need them, and those
// of rows 16..31 during steps 56..71 (they are used at the next tile's steps
// 0..7 and 48..55).  The copies of tile it+2 are issued during the QK^T
// chain, whose steps carry only their operand reads.  PV: O^T[cb] +=
// V^T(kt, cb) . P^T(kt); the K index k = 8 (lane/32) + e of step kt is row
// 16kt + 8(e/4) + 4(lane/32) + e%4, matching the packed probabilities, and
// the A operand (columns x those rows) is two transposed reads of 4 rows each.
// QK^T: S^T[32 rows][32 heads] in acc (lane l: head l%32, rows 8(i/4) +
// 4(l/32) + i%4 for i = 0..15).
// PV operands: PV step p (0..31 in a tile: p = s for s < 8, s - 40 for s
// >= 48) is read PV_AHEAD PV steps earlier into ring slot p % RING (32 =
// 8 RING, so the slots line up from tile to tile); the reads for the next
// tile's PV steps 0..2 (its PV of this tile, K step 1) are issued during
// steps 69..71.  QK^T operands: feature block ks is read QK_AHEAD steps
// earlier into slot ks % (QK_AHEAD + 1) of a ring that lives within the
// tile (its first reads are issued during steps 3..7).
constexpr int RING = 4;
constexpr int PV_AHEAD = RING - 1;
constexpr int QK_AHEAD = 5;
// The QK^T chain: the 32 latent feature blocks, then each of the 4 rotary
// blocks twice, against the high and then the low bf16 part of the rotary
// query (q^ = hi + lo to 16 significant bits: its rounding to bf16 would
// otherwise move every score by up to 2^-9 of the rotary term).
constexpr int NLO = 4;
constexpr int PRO_LATE = (QK_REG - Q_EARLY) + NLO + COPIES_PER_TILE;   // prologue ops issued after tile 0's copies
constexpr int NQK = ROW / 16 + NLO;                  // 40 MFMAs
constexpr int QK_END = 8 + NQK;                      // first step after the chain
constexpr int NSTEP = 32 + NQK;                      // 72
static_assert(32 % RING == 0, "ring alignment");
// Chain step j: feature block and whether it takes the low rotary part.
__host__ __device__ constexpr int chain_block(int j) { return j < 32 ? j : 32 + (j - 32) / 2; }
__host__ __device__ constexpr bool chain_lo(int j) { return j >= 32 && ((j - 32) & 1) != 0; }
// K operands of the chain live in a ring of QK_AHEAD + 1 slots indexed by
// block.  Block b + KRING, loaded QK_AHEAD chain steps before its first use,
// replaces block b only after b's last use: for latent blocks that is
// KRING > QK_AHEAD; a rotary block (first used at 32 + 2 (b - 32), twice)
// lands KRING - QK_AHEAD >= 1 steps after the last use of the block KRING
// before it, and no rotary block has a successor KRING blocks later.
constexpr int KRING = QK_AHEAD + 1;
static_assert(KRING > QK_AHEAD && KRING >= NLO, "operand ring");
// Steps after which the copies of tile it+2 are issued: the index fetch of
// tile it+4, then the 8 latent rows CP_GAP steps apart, then the rotary
// keys, all within the QK^T chain, whose steps issue little else (the PV
// steps after it carry the softmax).
constexpr int CP_IDX = 9, CP_ROW = 11, CP_GAP = 4, CP_ROT = CP_ROW + 8 * CP_GAP;
static_assert(CP_ROT < QK_END, "copies within the QK^T chain");

// A operand of PV step (kt, cb) of the tile in stage st.
__device__ __forceinline__ bf16x8 pv_operand(const char* __restrict__ st, int t0, int t1, int kt, int cb) {
    const int o = 1024 * kt + 64 * cb;
    const bf16x4 r0 = lds_read_tr16((const MLA_LDS void*)(st + t0 + o));
    const bf16x4 r1 = lds_read_tr16((const MLA_LDS void*)(st + t1 + o));
    return cat(r0, r1);
}

// One tile (it) of the loop.  cur: its stage; prv: the previous tile's
// stage.  All LDS reads go through the restrict pointers cur, prv (stages)
// and smem_q (the Q~ blocks): the copies the hook issues write another stage
// (the copy pipeline's own waits order them against these reads), and the
// restrict scopes tell the compiler so, which keeps it from draining all
// copies before the first transposed PV read.  hook(s) runs after the MFMA
// of step s.
template <typename Hook>
__device__ __forceinline__ void tile_iter(const char* __restrict__ cur, const char* __restrict__ prv,
                                          const char* __restrict__ smem_q, const LaneOffsets& lo,
                                          const bf16x8 (&qreg)[QK_REG], const bf16x8 (&qlo)[NLO], PassState& ps,
                                          bf16x8 (&ring)[RING], bf16x8& ptail, float scale_log2, int rem, bool first,
                                          int g, Hook&& hook) {
    int qb = lo.qk, rb = lo.rot, t0 = lo.tr[0], t1 = lo.tr[1], qo = lo.q;
    opaque(qb);
    opaque(rb);
    opaque(t0);
    opaque(t1);
    opaque(qo);
    auto pv_load = [&](int p) -> bf16x8 {
        if (p >= 32) return pv_operand(cur, t0, t1, 1, p - 32);        // next tile's tail
        if (p < 16) return pv_operand(prv, t0, t1, 1, p);               // tail: previous tile, K step 1
        return pv_operand(cur, t0, t1, 0, p - 16);                      // head: this tile, K step 0
    };
    auto qk_load = [&](int ks) -> bf16x8 {
        const int addr = ks < 32 ? qb + 32 * ks : (ks == 32 ? rb : rb ^ ((ks - 32) << 5));
        return *(const bf16x8*)(cur + addr);
    };
    bf16x8 kv[KRING];
    bf16x8 qv[QK_LDS];
    f32x16 acc;
    bf16x8 p0 = {}, p1 = {};
    float px = 0.f;                    // first entry of the pair being exponentiated
#pragma clang loop unroll(full)
    for (int s = 0; s < NSTEP; ++s) {
        const bool is_qk = s >= 8 && s < QK_END;
        const int pvs = s < 8 ? s : s - NQK;                            // PV step index (PV steps only)
        if (!is_qk) ring[(pvs + PV_AHEAD) % RING] = pv_load(pvs + PV_AHEAD);
        {
            // operand of chain step jl, read QK_AHEAD steps ahead (once per block)
            const int jl = s - 8 + QK_AHEAD;
            if (jl >= 0 && jl < NQK && !chain_lo(jl)) {
                const int kl = chain_block(jl);
                kv[kl % KRING] = qk_load(kl);
                if (kl >= QK_REG) qv[kl - QK_REG] = *(const bf16x8*)(smem_q + qo + 4096 * (kl - QK_REG));
            }
        }
        if (!is_qk) {
            const bf16x8 av = ring[pvs % RING];
            const int cb = pvs & 15;
            ps.o[cb] = mfma32(av, pvs < 16 ? ptail : p0, ps.o[cb]);
        } else {
            const int j = s - 8, ks = chain_block(j);
            const bf16x8 q = chain_lo(j) ? qlo[ks - 32 >= 0 ? ks - 32 : 0]
                                         : (ks < QK_REG ? qreg[ks < QK_REG ? ks : 0] : qv[ks >= QK_REG ? ks - QK_REG : 0]);
            const bf16x8 k = kv[ks % KRING];
            if (j == 0) qk_mfma_first(acc, k, q);
            else qk_mfma(acc, k, q);
        }
        if (s == QK_END - 1) {
            qk_settle(acc);
            if (rem < R) {
                // last tile, partly filled: rows past the end score -inf
                const int rl = rem - 4 * g;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (8 * (i >> 2) + (i & 3) >= rl) acc[i] = -INFINITY;
            }
            if (first) {
                // reference maximum: the first tile's, floored to an integer
                // so that exp2(x - m_ref) differs from exp2(x) by a power of
                // two only and its bf16 rounding does not depend on where
                // the splits fall
                float mt = -INFINITY;
#pragma unroll
                for (int i = 0; i < 16; ++i) mt = fmaxf(mt, acc[i]);
                mt = fmaxf(mt, __shfl_xor(mt, 32)) * scale_log2;
                ps.m_ref = floorf(mt);
            }
        }
        // softmax of rows 0..15 one entry per step (steps S0..S0+7, done
        // before their first PV use at step S0 + 8); rows 16..31 one entry
        // every other step (S1, S1 + 2, .., S1 + 14), the raw maximum in two
        // halves between them
        constexpr int S0 = QK_END, S1 = QK_END + 8;
        static_assert(S1 + 15 < NSTEP, "softmax steps");
        if (s >= S0 && s < S0 + 8) {
            const int j = s - S0;
            const float x = soft1(acc, j, ps.m_ref, scale_log2);
            if (j & 1) soft_pair(px, x, ps.lsum, p0, j - 1);
            else px = x;
        }
        if (s >= S1 && s < S1 + 16 && ((s - S1) & 1) == 0) {
            const int j = (s - S1) >> 1;
            const float x = soft1(acc, 8 + j, ps.m_ref, scale_log2);
            if (j & 1) soft_pair(px, x, ps.lsum, p1, j - 1);
            else px = x;
        }
        if (s == S1 + 1) ps.mraw = max9_raw<0>(ps.mraw, acc);
        if (s == S1 + 3) ps.mraw = max9_raw<8>(ps.mraw, acc);
        hook(s);
        __builtin_amdgcn_sched_barrier(0);
    }
    ptail = p1;
}

// The last tile's K step 1 (steps 0..7 and 48..55 of a following tile that
// does not exist).  Its first PV_AHEAD operands are already in the ring.
__device__ __forceinline__ void pv_last(const char* __restrict__ prv, const LaneOffsets& lo, PassState& ps,
                                        bf16x8 (&ring)[RING], const bf16x8& ptail) {
    int t0 = lo.tr[0], t1 = lo.tr[1];
    opaque(t0);
    opaque(t1);
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) {
        if (cb + PV_AHEAD < 16) ring[(cb + PV_AHEAD) % RING] = pv_operand(prv, t0, t1, 1, cb + PV_AHEAD);
        ps.o[cb] = mfma32(ring[cb % RING], ptail, ps.o[cb]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One pass over the split (see attn_kernel).  Returns true when the pass
// must be repeated with the exact maximum (then m_ref holds it).
//
// Copy pipeline, per wave: iteration j fetches the indices of tile j+4 and
// copies tile j+2 (9 copies, spread over the QK^T chain) into the stage that
// tile j-2 left (its last reads were the previous iteration's PV, K step
// 1); the prologue plays iterations -2..-1.  Tiles past the split are copied
// as well (from row 0 = "no row": zeros, no memory traffic), so every
// iteration issues COPIES_PER_TILE copies and iteration it waits with one
// constant count: the copies issued after tile it's (the index fetch of
// tile it+3 and tile it+1) may still be in flight.
__device__ __forceinline__ bool attn_pass(const AttnArgs& a, const SplitCtx& sc, char* smem,
                                          float& m_ref, bool known) {
    const int tid = tid_opaque(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const int nt = sc.ntiles;
    int* flag = (int*)(smem + OFF_FLAG);
    __syncthreads();                               // previous pass done
    if (tid == 0) *flag = 0;

    int* idx_ring = (int*)(smem + OFF_IDX) + wave * 8;      // + slot * 32
    auto stage = [&](int T) { return (T & (NST - 1)) * STAGE; };
    MLA_LDS char* const lsm = (MLA_LDS char*)smem;
    auto lstage = [&](int T) { return lsm + stage(T); };
    auto slot = [&](int T) { return idx_ring + (T % NSLOT) * 32; };

    const LaneOffsets lo = lane_offsets(a, lane, wave);
    int mst[8];                                    // row_start of this wave's 8 rows
#pragma unroll
    for (int j = 0; j < 8; ++j) mst[j] = __builtin_amdgcn_readfirstlane(row_start(wave * 8 + j));
    PassState ps;
    ps.m_ref = m_ref;
    ps.mraw = -INFINITY;
    ps.lsum = 0.f;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) ps.o[cb] = f32x16{};

    // The first tile's steps 0..7 and 48..55 multiply the stage before stage
    // 0 (stage NST-1) by zero probabilities: clear its latent region so that
    // whatever it held cannot turn into NaN.
    for (int i = tid; i < LATB / 16; i += 256) *(u32x4*)(smem + (NST - 1) * STAGE + 16 * i) = u32x4{};

    // ---- prologue ----
    // Copy order: indices of tiles 0..1; Q~ (blocks 33..35 into LDS, blocks
    // 0..32 into registers), which needs no index and is the largest
    // transfer; then, once the indices have landed, indices 2 and tile 0,
    // indices 3 and tile 1.  Q~ of this wave's 32 heads (QK^T B operand):
    // block ks holds features 16 ks + 8 (lane/32) .. +7 of head h0 + 32 wave
    // + lane%32; heads past H read as zero (outside the buffer window).
    const rsrc_t qsrc = make_rsrc(a.qt + (long long)sc.b * a.H * ROW, (uint32_t)a.H * ROW * 2u);
    bf16x8 qreg[QK_REG];
    bf16x8 qlo[NLO];
    {
        // also for an empty split (nt = 0): its index window reads zeros, so
        // the copies write zero rows and nothing reads them; a conditional
        // prologue would make the compiler wait for all its loads where the
        // two paths join
#pragma unroll
        for (int T = 0; T < 2; ++T) fetch_idx(sc, T, slot(T), lane, wave);
        const uint32_t h = (uint32_t)(sc.h0 + wave * 32 + l32);
        {
            // LDS part: lane l fills bytes 16 l of the wave's 1 KB row of
            // block i, i.e. head 32 wave + l/2, features 16 (QK_REG + i) + 8 (l & 1)
            const uint32_t hq = (uint32_t)(sc.h0 + wave * 32 + (lane >> 1));
#pragma unroll
            for (int i = 0; i < QK_LDS; ++i)
                buffer_to_lds16(qsrc, hq * (ROW * 2) + (16 * (QK_REG + i) + 8 * (lane & 1)) * 2,
                                (MLA_LDS void*)(smem + OFF_Q + 4096 * i + 1024 * wave));
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int ks = 0; ks < Q_EARLY; ++ks)
            qreg[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                      qsrc, h * (ROW * 2) + (16 * ks + 8 * g) * 2, 0, 0));
        asm volatile("" ::: "memory");
        wait_vmcnt<QK_LDS + Q_EARLY>();            // the two index fetches (issued first) landed
        fetch_idx(sc, 2, slot(2), lane, wave);
        issue_tile(a, sc, lo, mst, lstage(0), slot(0), lane, wave);
        asm volatile("" ::: "memory");
        // the rest of Q~ and its low rotary parts load under tile 0's copies
        // and first MFMA steps (each register block is first used at QK^T
        // step 8 + its index)
#pragma unroll
        for (int ks = Q_EARLY; ks < QK_REG; ++ks)
            qreg[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                      qsrc, h * (ROW * 2) + (16 * ks + 8 * g) * 2, 0, 0));
        // low parts of the rotary query: [H][64] per sequence
        const rsrc_t lsrc = make_rsrc(a.qlo + (long long)sc.b * a.H * D_ROPE, (uint32_t)a.H * D_ROPE * 2u);
#pragma unroll
        for (int i = 0; i < NLO; ++i)
            qlo[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                    lsrc, h * (D_ROPE * 2) + (16 * i + 8 * g) * 2, 0, 0));
        asm volatile("" ::: "memory");
        fetch_idx(sc, 3, slot(3), lane, wave);
        issue_tile(a, sc, lo, mst, lstage(1), slot(1), lane, wave);
    }

    // ---- main loop ----
    lds_barrier();                                 // the cleared stage visible
    bf16x8 ring[RING];
    bf16x8 ptail = {};
    {
        int t0 = lo.tr[0], t1 = lo.tr[1];
        opaque(t0);
        opaque(t1);
#pragma unroll
        for (int s = 0; s < PV_AHEAD; ++s) ring[s] = pv_operand(smem + stage(NST - 1), t0, t1, 1, s);
    }
    const int nrows = sc.end - sc.start;
    auto tile = [&](int it, bool first) {
        lds_barrier();          // tile it resident and visible; stage (it-2)%4 free
        const TileRows rows = read_rows(slot(it + 2), lane);
        const int dsto = stage(it + 2);
        int* const fslot = slot(it + 4);
        tile_iter(smem + stage(it), smem + stage(it + NST - 1), smem, lo, qreg, qlo, ps, ring, ptail, a.scale_log2,
                  nrows - it * R, first, g, [&](int st_) {
            // copies of tile it+2 spread over the QK^T chain; each copy's LDS
            // address is formed at its own step (an opaque stage offset), not
            // all nine at the first one
            auto dst = [&]() {
                int o = dsto;
                asm volatile("" : "+s"(o));
                return lsm + o;
            };
            if (st_ == CP_IDX) fetch_idx(sc, it + 4, fslot, lane, wave);
            if (st_ >= CP_ROW && st_ < CP_ROW + 8 * CP_GAP && (st_ - CP_ROW) % CP_GAP == 0)
                issue_row(a, sc, lo, dst() + mst[(st_ - CP_ROW) / CP_GAP], rows, (st_ - CP_ROW) / CP_GAP);
            if (st_ == CP_ROT) issue_rot(a, sc, lo, dst(), rows, wave);
        });
    };
    // Tile 0 is peeled off the loop.  The later Q~ blocks and the low parts
    // may still be in flight when it starts, so the compiler places a wait
    // for each register block at its first use; inside a shared loop body
    // those waits would run on every tile and, late in the QK^T chain, hold
    // a steady-state tile until the next tile's first copies had landed.
    // After tile 0 (or the explicit wait of an empty split) no register load
    // is pending, and the loop below carries only its one copy wait.
    if (nt > 0) {
        wait_vmcnt<PRO_LATE>();    // the later Q~ blocks, the low parts and tile 1 may still be in flight
        tile(0, !known);
    } else {
        wait_vmcnt<0>();
    }
    for (int it = 1; it < nt; ++it) {
        wait_vmcnt<COPIES_PER_TILE>();   // the copies issued during the previous tile may be in flight
        tile(it, false);
    }
    if (nt > 0) pv_last(smem + stage(nt - 1), lo, ps, ring, ptail);

    // ---- overflow check, then normalise and write ----
    __syncthreads();            // also drains the copies of the tiles past the split
    const float mx = fmaxf(ps.mraw, __shfl_xor(ps.mraw, 32)) * a.scale_log2;
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
    // partials are head-major, [H][B][S] rows: head h's rows for consecutive
    // sequences are contiguous, so each merge workgroup (one head) streams
    // one contiguous region
    const long long hstride = (long long)a.B * a.S;
    const long long prow0 = (long long)(sc.h0 + wave * 32) * hstride + (long long)sc.b * a.S + sc.s;
    if (g == 0 && sc.h0 + wave * 32 + l32 < a.H)
        a.lsepart[prow0 + l32 * hstride] = l > 0.f ? ps.m_ref + log2f(l) : -INFINITY;
    __builtin_amdgcn_s_waitcnt(0xC07F);            // this wave's LDS writes done (only it reads them)
#pragma unroll 4
    for (int hr = 0; hr < 32; ++hr) {
        if (sc.h0 + wave * 32 + hr >= a.H) break;
        const u32x4 v = *(const u32x4*)(orow + hr * 1024 + ((lane ^ hr) << 4));
        *(u32x4*)(a.opart + (prow0 + hr * hstride) * RANK + 8 * lane) = v;
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
    sc.list = make_rsrc(a.list + (long long)sc.b * a.K + sc.start, (uint32_t)(sc.end - sc.start) * 4u);
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
    a.qt = (const bf16*)w.qt; a.qlo = (const bf16*)w.qlo; a.list = w.list; a.counts = w.counts;
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
