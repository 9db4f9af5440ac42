// Merge of split-KV partials and the W_UV up-projection, plus the fp32
// attention used when the activations are fp32.
//
// Sources (atlas pages on DeepSeek-V3.2-Exp sparse latent attention):
//   page "Rotated query part", excerpt mla-decode: softmax over the selected
//   scores, the weighted latent sum and the per-head W_UV up-projection
//   (x . W_UV[h]^T over the 512 latent columns, 128 outputs per head).
//   Merging independently normalised partials by their log-sum-exp is the
//   standard split-softmax identity; the pages do not partition the keys.
#include <algorithm>

#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

// ---------------------------------------------------------------------------
// bf16 path: out[b, h, :] = sum_s w_{b,s} (W_UV[h] . o_s[b, h, :])
//   w_{b,s} = 2^(lse_s - M) / sum_s' 2^(lse_s' - M),  M = max_s lse_s.
// The projection is linear, so each split's bf16 partial is projected as it
// is stored (no re-rounding of a merged latent) and the fp32 projections are
// combined.  Workgroup (head h, output half dh) covers every sequence (or,
// below 128 heads, the 32-sequence batches of its share) with 8
// waves (two per SIMD, so that one wave's loads overlap the other's work).
// bf16 MFMA with M = 64 outputs (two blocks), N = sequences (32 per step),
// K = 512 latent columns split over the 8 waves (64 each) and reduced
// through LDS.
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
    // Cross-wave reduction buffers, used by alternate batches: a batch's
    // writes never meet the previous batch's reads, so one barrier per batch
    // suffices.  Layout [wave][nb][output m][sequence n], rows padded to 33
    // words: the writes (32 sequences of one output per half-wave) and the
    // reads (32 consecutive outputs of one sequence) both spread over the banks.
    constexpr int RS = 33;
    constexpr int SLAB = 32 * RS;
    __shared__ float red2[2][MW * 2 * SLAB];
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
    // With few heads the grid's second dimension splits the 32-sequence
    // batches between workgroups (each re-reads its weights, from L2 after
    // the first), so that more CUs share the partials.
    const int G = (a.S + 1) / 2;                     // split pairs per sequence
    const int NBT = (a.B + 31) / 32;                 // 32-sequence batches
    const int BPG = (NBT + (int)gridDim.y - 1) / (int)gridDim.y;
    const int bt0 = (int)blockIdx.y * BPG;           // this workgroup's first batch
    const int nbt = min(BPG, NBT - bt0);
    if (nbt <= 0) return;
    const int U = nbt * G;
    auto load_unit = [&](int u, bf16x8 (&v)[2][MKB], float (&ls)[2]) {
        const int bA = 32 * (bt0 + u / G) + l32, s0 = 2 * (u % G);
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

    // Each split's partial is projected on its own (A = W_UV rows, B = the
    // partial's latent columns, so a lane's result column is its sequence
    // and the split weights are per-lane scalars) and the projections are
    // combined in fp32.  Lanes past the batch hold zero partials and an LSE
    // of -inf; their columns are never stored.  The last unit of a batch
    // folds 1 / sum of weights into its coefficients.
    float M = -INFINITY, Wsum = 0.f;
    f32x16 acc[2] = {f32x16{}, f32x16{}};
    for (int u = 0; u < U; ++u) {
        if (u + 1 < U) load_unit(u + 1, vn, ln);
        const float Mn = fmaxf(M, fmaxf(lc[0], lc[1]));
        const float sc = M == Mn ? 1.f : exp2f(M - Mn);
        float w0 = exp2f(lc[0] - Mn), w1 = exp2f(lc[1] - Mn);
        Wsum = Wsum * sc + w0 + w1;
        M = Mn;
        const bool last = u % G == G - 1;
        float cs = sc;
        if (last) {
            const float invW = 1.f / Wsum;
            cs *= invW; w0 *= invW; w1 *= invW;
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            f32x16 p0 = f32x16{}, p1 = f32x16{};
#pragma unroll
            for (int kb = 0; kb < MKB; ++kb)
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) {
                    p0 = mfma32(bw[pp][nb][kb], vc[0][kb], p0);
                    p1 = mfma32(bw[pp][nb][kb], vc[1][kb], p1);
                }
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[nb][i] = fmaf(w1, p1[i], fmaf(w0, p0[i], acc[nb][i] * cs));
        }
        if (last) {
            const int b0 = 32 * (bt0 + u / G), bA = b0 + l32;
            if (dh == 0 && wave == 0 && g == 0 && bA < a.B && a.lse_out)
                a.lse_out[(long long)bA * a.H + h] = LN2 * (M + log2f(Wsum));
            float* red = red2[(u / G) & 1];
            // result element (output 8(i/4) + 4g + i%4 of block nb, sequence l32)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    red[(wave * 2 + nb) * SLAB + (8 * (i >> 2) + 4 * g + (i & 3)) * RS + l32] = acc[nb][i];
            __syncthreads();
#pragma unroll
            for (int k = 0; k < 2048 / (64 * MW); ++k) {
                const int e = tid + 64 * MW * k;
                const int dl = e & 63, bl = e >> 6;
                const int nb = dl >> 5, m = dl & 31;
                float v = 0.f;
#pragma unroll
                for (int w = 0; w < MW; ++w) v += red[(w * 2 + nb) * SLAB + m * RS + bl];
                const int bo = b0 + bl;
                if (bo < a.B)
                    ((OutT*)a.out)[bo * a.out_sb + h * a.out_sh + 64 * dh + dl] = from_f32<OutT>(v);
            }
            M = -INFINITY;
            Wsum = 0.f;
            acc[0] = f32x16{};
            acc[1] = f32x16{};
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
// Tiled form of the same merge, used for batches of fewer than 128 sequences
// with at most 8 splits, where it runs faster than the form above (fewer
// sequence tiles, more split pairs per tile).  The workgroup's 64 W_UV rows (head h,
// output half dh) go to LDS once, as bf16 high and low parts for fp32
// weights.  Wave w takes 32-sequence tiles st = w / 2 (+ 4 j) and latent
// half kh = w % 2, and computes both 32-output blocks of its tile over its
// 256 columns, with the partial rows streamed from memory MT_PD steps ahead;
// the two halves of a tile are added through LDS once per tile.  MFMA step
// ks (0..15), lane group g: latent columns 256 kh + 16 ks + 8 g + j (j < 8),
// the same for A (W rows, M = outputs) and B (partial rows, N = sequences).
// LDS holds the weights in operand order, [part][output block][half][step]
// [lane] x 16 bytes, so each step's read is lane-contiguous.
// ---------------------------------------------------------------------------
constexpr int MT_PD = 6;                 // partial steps in flight per wave
constexpr int MT_XB = 4 * 2 * 16 * 64;   // exchange floats: 4 tiles x 2 blocks x 16 x 64 lanes

template <typename WT, typename OutT>
__global__ __launch_bounds__(64 * MW) void merge_tile_kernel(MergeArgs a) {
    constexpr int NP = sizeof(WT) == 4 ? 2 : 1;
    __shared__ __attribute__((aligned(16))) bf16 wl[NP * 64 * RANK];
    __shared__ __attribute__((aligned(16))) float xb[MT_XB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    // the two output halves of one head sit 8 ids apart (same XCD, shared L2)
    const int id = blockIdx.x;
    const int xcd = id & 7, k8 = id >> 3;
    const int dh = k8 & 1, h = (k8 >> 1) * 8 + xcd;
    if (h >= a.H) return;
    const int st0 = wave >> 1, kh = wave & 1;
    const int NST = (a.B + 31) / 32;                 // sequence tiles
    const int NI = (NST + 3) / 4;                    // tile rounds, the same for every wave
    const int G = (a.S + 1) / 2;                     // split pairs per sequence

    const rsrc_t prs = make_rsrc(a.opart + (long long)h * a.B * a.S * RANK, (uint32_t)((long long)a.B * a.S * RANK * 2));
    bf16x8 ring[MT_PD][2];
    uint32_t voff[2];
    float lse_n[2];
    // item (round r, pair gp) of this wave: its first MT_PD steps and two
    // LSEs.  Lanes past the batch read the last sequence's rows (never
    // stored); a missing second split reads the last split, LSE -inf.
    auto issue_item = [&](int r, int gp) {
        const int bc = min(32 * (st0 + 4 * r) + l32, a.B - 1);
        const int s0 = 2 * gp, s1 = min(2 * gp + 1, a.S - 1);
        voff[0] = (uint32_t)(((long long)bc * a.S + s0) * RANK + 256 * kh + 8 * g) * 2u;
        voff[1] = (uint32_t)(((long long)bc * a.S + s1) * RANK + 256 * kh + 8 * g) * 2u;
        lse_n[0] = a.lsepart[((long long)h * a.B + bc) * a.S + s0];
        lse_n[1] = a.lsepart[((long long)h * a.B + bc) * a.S + s1];
#pragma unroll
        for (int k = 0; k < MT_PD; ++k)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                ring[k][u] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(prs, voff[u] + 32 * k, 0, 0));
    };
    const bool has0 = st0 < NST;
    if (has0) issue_item(0, 0);                      // in flight together with the weights

    // weights: lane = row m (0..63), wave = 16-byte chunks 8 w .. 8 w + 7;
    // chunk q (columns 8 q .. + 7) is half q / 32, step (q % 32) / 2, group q % 2
    {
        const int m = lane, cq = 8 * wave;
        const WT* wsrc = (const WT*)a.w_uv + h * a.wv_sh + (long long)(64 * dh + m) * RANK + 8 * cq;
        bf16* dst = wl + 8 * (2048 * (m >> 5) + (m & 31));
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int q = cq + k;
            const int slot = 1024 * (q >> 5) + 64 * ((q & 31) >> 1) + 32 * (q & 1);
            if constexpr (NP == 2) {
                const f32x4 x0 = *(const f32x4*)(wsrc + 8 * k), x1 = *(const f32x4*)(wsrc + 8 * k + 4);
                bf16x8 hi, lo;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float wv = e < 4 ? x0[e] : x1[e - 4];
                    hi[e] = (bf16)wv;
                    lo[e] = (bf16)(wv - (float)hi[e]);
                }
                *(bf16x8*)(dst + 8 * slot) = hi;
                *(bf16x8*)(dst + 64 * RANK + 8 * slot) = lo;
            } else {
                *(bf16x8*)(dst + 8 * slot) = load8_bf16<WT>(wsrc + 8 * k);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);              // this wave's LDS writes done
    asm volatile("s_barrier" ::: "memory");          // every wave's weights visible (loads stay in flight)

    const bool vec_out = ((uintptr_t)a.out & 15) == 0 && (a.out_sb & 3) == 0 && (a.out_sh & 3) == 0;
    // operand of block ot, part pp, step ks: wop + 8 (4096 pp + 2048 ot + 64 ks)
    const bf16* wop = wl + 8 * (1024 * kh + lane);
    float* xw = xb + st0 * (2 * 16 * 64) + lane;     // this tile pair's exchange area
    for (int r = 0; r < NI; ++r) {
        const int st = st0 + 4 * r;
        const bool has = st < NST;
        float M = -INFINITY, Wsum = 0.f;
        f32x16 acc[2] = {f32x16{}, f32x16{}};
        for (int gp = 0; has && gp < G; ++gp) {
            const bool last = gp == G - 1;
            const uint32_t v0 = voff[0], v1 = voff[1];
            float l0 = lse_n[0], l1 = 2 * gp + 1 < a.S ? lse_n[1] : -INFINITY;
            f32x16 p[2][2];
#pragma unroll
            for (int ot = 0; ot < 2; ++ot) { p[ot][0] = f32x16{}; p[ot][1] = f32x16{}; }
            // weight operands are read one step ahead
            bf16x8 wc[2][NP];
#pragma unroll
            for (int ot = 0; ot < 2; ++ot)
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) wc[ot][pp] = *(const bf16x8*)(wop + 8 * (4096 * pp + 2048 * ot));
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) {
                bf16x8 wn[2][NP];
                if (ks + 1 < 16) {
#pragma unroll
                    for (int ot = 0; ot < 2; ++ot)
#pragma unroll
                        for (int pp = 0; pp < NP; ++pp)
                            wn[ot][pp] = *(const bf16x8*)(wop + 8 * (4096 * pp + 2048 * ot + 64 * (ks + 1)));
                }
#pragma unroll
                for (int ot = 0; ot < 2; ++ot)
#pragma unroll
                    for (int pp = 0; pp < NP; ++pp) {
                        p[ot][0] = mfma32(wc[ot][pp], ring[ks % MT_PD][0], p[ot][0]);
                        p[ot][1] = mfma32(wc[ot][pp], ring[ks % MT_PD][1], p[ot][1]);
                    }
                if (ks + MT_PD < 16) {
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        ring[ks % MT_PD][u] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                                      prs, (u ? v1 : v0) + 32 * (ks + MT_PD), 0, 0));
                }
                if (ks + 1 < 16) {
#pragma unroll
                    for (int ot = 0; ot < 2; ++ot)
#pragma unroll
                        for (int pp = 0; pp < NP; ++pp) wc[ot][pp] = wn[ot][pp];
                }
                __builtin_amdgcn_sched_barrier(0);   // keep each step's reads with its MFMAs
            }
            // the next item streams during the combine
            if (!last) issue_item(r, gp + 1);
            else if (st + 4 < NST) issue_item(r + 1, 0);
            const float Mn = fmaxf(M, fmaxf(l0, l1));
            const float sc = M == Mn ? 1.f : exp2f(M - Mn);
            float w0 = exp2f(l0 - Mn), w1 = exp2f(l1 - Mn);
            Wsum = Wsum * sc + w0 + w1;
            M = Mn;
            float cs = sc;
            if (last) {
                const float invW = 1.f / Wsum;
                cs *= invW; w0 *= invW; w1 *= invW;
            }
#pragma unroll
            for (int ot = 0; ot < 2; ++ot)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[ot][i] = fmaf(w1, p[ot][1][i], fmaf(w0, p[ot][0][i], acc[ot][i] * cs));
        }
        // the upper latent half hands its sums to the lower one
        if (has && kh == 1) {
#pragma unroll
            for (int ot = 0; ot < 2; ++ot)
#pragma unroll
                for (int i = 0; i < 16; ++i) xw[(ot * 16 + i) * 64] = acc[ot][i];
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        asm volatile("s_barrier" ::: "memory");
        if (has && kh == 0) {
            // lane: sequence 32 st + l32, outputs 32 ot + 8 i4 + 4 g .. + 3
            const int bl = 32 * st + l32;
            if (bl < a.B) {
                OutT* o = (OutT*)a.out + (long long)bl * a.out_sb + (long long)h * a.out_sh + 64 * dh + 4 * g;
#pragma unroll
                for (int ot = 0; ot < 2; ++ot)
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4) {
                        float v[4];
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) v[rr] = acc[ot][4 * i4 + rr] + xw[(ot * 16 + 4 * i4 + rr) * 64];
                        OutT* oo = o + 32 * ot + 8 * i4;
                        if (vec_out) {
                            if constexpr (sizeof(OutT) == 4) *(f32x4*)oo = f32x4{v[0], v[1], v[2], v[3]};
                            else *(bf16x4*)oo = bf16x4{f2bf(v[0]), f2bf(v[1]), f2bf(v[2]), f2bf(v[3])};
                        } else {
#pragma unroll
                            for (int rr = 0; rr < 4; ++rr) oo[rr] = from_f32<OutT>(v[rr]);
                        }
                    }
                if (dh == 0 && g == 0 && a.lse_out) a.lse_out[(long long)bl * a.H + h] = LN2 * (M + log2f(Wsum));
            }
        }
        if (r + 1 < NI) {
            __builtin_amdgcn_s_waitcnt(0xC07F);
            asm volatile("s_barrier" ::: "memory");  // exchange area read before the next round writes it
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 path (fp32 activations, parity at 1e-5).  attn_f32: one workgroup per
// (sequence, group of HG heads), 256 threads, over the compacted selection in
// tiles of 16 rows.  Each tile's rows (latent and rotary parts, 576 floats)
// are read once into LDS and shared by the group's heads.  The score of
// (head, row) is formed by TPS = 16 / HG threads, each over a contiguous
// 576 / TPS features in order, and their partial sums are added with lane
// shuffles; the threads of a head reduce the tile's maximum and sum the same
// way (online softmax, rescaling when the maximum grows), and thread tid
// accumulates latent columns tid and tid + 256 of all HG heads.  Writes the
// normalised latent sum (fp32) and the log2-domain sum-exp.  HG = 16 reads
// each row once per 16 heads; HG = 4 runs four times as many workgroups, for
// batches too small to occupy the chip otherwise.
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

constexpr int F32_TR = 16;              // selected rows per tile
constexpr int F32_RS = ROW + 4;         // LDS row stride (floats): rows 4 banks apart, 16-byte aligned
constexpr int F32_C4 = ROW / 4;         // 16-byte chunks per row

template <int HG>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnF32Args a) {
    constexpr int TR = F32_TR, TPS = 256 / (HG * TR), CPT = F32_C4 / TPS;
    static_assert(HG * TR * TPS == 256 && F32_C4 % TPS == 0, "thread mapping");
    static_assert(TPS * TR <= 64, "a head's threads share one wave (its reductions are lane shuffles)");
    __shared__ __attribute__((aligned(16))) float qs[HG * F32_RS];
    __shared__ __attribute__((aligned(16))) float ks[TR * F32_RS];
    __shared__ float ps[HG][TR];
    __shared__ float al[HG];
    __shared__ float fin[2][HG];
    const int tid = threadIdx.x;
    const int ng = (a.H + HG - 1) / HG;
    const int b = blockIdx.x / ng, h0 = (blockIdx.x % ng) * HG;
    const int nh = min(HG, a.H - h0);
    // Q~ of the group's heads; heads past H are zero (never written out)
    for (int i = tid; i < HG * F32_C4; i += 256) {
        const int hh = i / F32_C4, c4 = i % F32_C4;
        f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
        if (hh < nh) v = *(const f32x4*)(a.qt + ((long long)b * a.H + h0 + hh) * ROW + 4 * c4);
        *(f32x4*)(qs + hh * F32_RS + 4 * c4) = v;
    }
    const int cnt = a.counts[b];
    const int32_t* list = a.list + (long long)b * a.K;
    const float* kvb = a.kv + b * a.kv_sb;
    const float* peb = a.pe + b * a.pe_sb;
    // score of head sh, tile row sr, features [CPT q, CPT (q + 1)) in chunks
    const int q = tid % TPS, sr = (tid / TPS) % TR, sh = tid / (TPS * TR);
    float m = -INFINITY, l = 0.f;                   // softmax state of head sh (same in all its threads)
    float o[HG][2];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) o[hh][0] = o[hh][1] = 0.f;
    // The tile's rows: 16 x 144 chunks of 16 bytes, 9 per thread.  The next
    // tile's loads are issued before this tile's scores and stay in flight
    // (in registers) until the tile after has been consumed.  Rows past the
    // selection repeat its last row and are stored as zeros: loads without a
    // condition are not waited for where they are issued.
    constexpr int NLD = TR * F32_C4 / 256;
    f32x4 v[NLD];
    auto fetch = [&](int base) {
        int t[NLD];
#pragma unroll
        for (int j = 0; j < NLD; ++j) t[j] = list[min(base + (tid + 256 * j) / F32_C4, cnt - 1)] - 1;   // 1-based
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int c4 = (tid + 256 * j) % F32_C4;
            v[j] = c4 < RANK / 4 ? *(const f32x4*)(kvb + (long long)t[j] * a.kv_st + 4 * c4)
                                 : *(const f32x4*)(peb + (long long)t[j] * a.pe_st + 4 * (c4 - RANK / 4));
        }
    };
    if (cnt > 0) fetch(0);
    for (int base = 0; base < cnt; base += TR) {
        const int nr = min(TR, cnt - base);
        __syncthreads();                            // the previous tile's reads of ks, ps, al are done
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int i = tid + 256 * j, r = i / F32_C4, c4 = i % F32_C4;
            *(f32x4*)(ks + r * F32_RS + 4 * c4) = r < nr ? v[j] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();
        if (base + TR < cnt) fetch(base + TR);
        float acc = 0.f;
        const float* qrow = qs + sh * F32_RS + 4 * CPT * q;
        const float* krow = ks + sr * F32_RS + 4 * CPT * q;
#pragma unroll 8
        for (int c4 = 0; c4 < CPT; ++c4) {
            const f32x4 qv = *(const f32x4*)(qrow + 4 * c4), kv = *(const f32x4*)(krow + 4 * c4);
            acc = fmaf(qv[0], kv[0], acc);
            acc = fmaf(qv[1], kv[1], acc);
            acc = fmaf(qv[2], kv[2], acc);
            acc = fmaf(qv[3], kv[3], acc);
        }
#pragma unroll
        for (int d = 1; d < TPS; d <<= 1) acc += __shfl_xor(acc, d);
        const float sc = sr < nr ? acc * a.scale : -INFINITY;
        float tm = sc;
#pragma unroll
        for (int d = TPS; d < TPS * TR; d <<= 1) tm = fmaxf(tm, __shfl_xor(tm, d));
        const float mn = fmaxf(m, tm);
        const float alpha = m == -INFINITY ? 0.f : expf(m - mn);
        const float p = sr < nr ? expf(sc - mn) : 0.f;
        float ts = p;
#pragma unroll
        for (int d = TPS; d < TPS * TR; d <<= 1) ts += __shfl_xor(ts, d);
        l = l * alpha + ts;
        m = mn;
        if (q == 0) ps[sh][sr] = p;
        if (q == 0 && sr == 0) al[sh] = alpha;
        __syncthreads();
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
            const float x = al[hh];
            o[hh][0] *= x;
            o[hh][1] *= x;
        }
#pragma unroll 4
        for (int r = 0; r < nr; ++r) {
            const float v0 = ks[r * F32_RS + tid], v1 = ks[r * F32_RS + tid + 256];
#pragma unroll
            for (int hh = 0; hh < HG; ++hh) {
                const float pr = ps[hh][r];
                o[hh][0] = fmaf(pr, v0, o[hh][0]);
                o[hh][1] = fmaf(pr, v1, o[hh][1]);
            }
        }
    }
    if (q == 0 && sr == 0) {
        fin[0][sh] = l;
        fin[1][sh] = m;
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
        if (hh >= nh) break;
        const float lh = fin[0][hh];
        const float inv = lh > 0.f ? 1.f / lh : NAN;
        float* dst = a.olat + ((long long)b * a.H + h0 + hh) * RANK;
        dst[tid] = o[hh][0] * inv;
        dst[tid + 256] = o[hh][1] * inv;
    }
    if (tid < nh) a.lse2[(long long)b * a.H + h0 + tid] = (fin[1][tid] + logf(fin[0][tid])) * LOG2E;
}

// fp32 up-projection: one workgroup per (head, half of the 128 outputs,
// group of 8 sequences) with the group's latent sums in LDS; thread t forms
// output 64 (half) + t / 4 over latent columns 128 (t % 4) .. + 127 for
// every sequence of the group, and the four quarters are added with lane
// shuffles.  Each weight row is read once per group.
constexpr int F32_UB = 8;               // sequences per up-projection workgroup

template <typename WT>
__device__ __forceinline__ f32x4 load4_f32(const WT* p);
template <> __device__ __forceinline__ f32x4 load4_f32<float>(const float* p) { return *(const f32x4*)p; }
template <> __device__ __forceinline__ f32x4 load4_f32<bf16>(const bf16* p) {
    const bf16x4 v = *(const bf16x4*)p;
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

template <typename WT, typename OutT>
__global__ __launch_bounds__(256) void uproj_f32_kernel(MergeArgs a, const float* olat) {
    __shared__ __attribute__((aligned(16))) float xs[F32_UB][RANK];
    const int tid = threadIdx.x;
    const int nbg = (a.B + F32_UB - 1) / F32_UB;
    const int h = blockIdx.x / (2 * nbg), dh = (blockIdx.x / nbg) & 1, b0 = (blockIdx.x % nbg) * F32_UB;
    const int nb = min(F32_UB, a.B - b0);
    for (int i = tid; i < F32_UB * RANK / 4; i += 256) {
        const int s = i / (RANK / 4), c4 = i % (RANK / 4);
        f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
        if (s < nb) v = *(const f32x4*)(olat + ((long long)(b0 + s) * a.H + h) * RANK + 4 * c4);
        *(f32x4*)(xs[s] + 4 * c4) = v;
    }
    __syncthreads();
    const int d = 64 * dh + (tid >> 2), c0 = (RANK / 4) * (tid & 3);
    const WT* w = (const WT*)a.w_uv + h * a.wv_sh + (long long)d * RANK + c0;
    float acc[F32_UB];
#pragma unroll
    for (int s = 0; s < F32_UB; ++s) acc[s] = 0.f;
#pragma unroll 16
    for (int c = 0; c < RANK / 4; c += 4) {
        const f32x4 wv = load4_f32<WT>(w + c);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int s = 0; s < F32_UB; ++s) acc[s] = fmaf(xs[s][c0 + c + j], wv[j], acc[s]);
    }
#pragma unroll
    for (int s = 0; s < F32_UB; ++s) {
        acc[s] += __shfl_xor(acc[s], 1);
        acc[s] += __shfl_xor(acc[s], 2);
    }
    if ((tid & 3) == 0) {
#pragma unroll
        for (int s = 0; s < F32_UB; ++s) {
            if (s >= nb) break;
            const int bb = b0 + s;
            ((OutT*)a.out)[bb * a.out_sb + h * a.out_sh + d] = from_f32<OutT>(acc[s]);
            if (d == 0 && a.lse_out) a.lse_out[(long long)bb * a.H + h] = a.lsepart[(long long)bb * a.H + h] * LN2;
        }
    }
}

hipError_t launch_attn_f32(const mla_decode_params_t& p, const Work& w, hipStream_t s) {
    AttnF32Args a{};
    a.B = p.B; a.H = p.H; a.K = p.K; a.scale = p.softmax_scale;
    a.qt = (const float*)w.qt; a.list = w.list; a.counts = w.counts;
    a.kv = (const float*)p.kv_cache; a.kv_sb = p.kv_stride_b; a.kv_st = p.kv_stride_t;
    a.pe = (const float*)p.pe_cache; a.pe_sb = p.pe_stride_b; a.pe_st = p.pe_stride_t;
    a.olat = (float*)w.opart; a.lse2 = w.lsepart;
    // 16 heads per workgroup when that gives enough workgroups, else 4
    const int g16 = p.B * ((p.H + 15) / 16);
    if (g16 >= 64) hipLaunchKernelGGL(attn_f32_kernel<16>, dim3(g16), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(attn_f32_kernel<4>, dim3(p.B * ((p.H + 3) / 4)), dim3(256), 0, s, a);
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
        if (p.B < 128 && plan.splits <= 8) {
            if (wf && of) hipLaunchKernelGGL((merge_tile_kernel<float, float>), grid, block, 0, s, a);
            else if (wf) hipLaunchKernelGGL((merge_tile_kernel<float, bf16>), grid, block, 0, s, a);
            else if (of) hipLaunchKernelGGL((merge_tile_kernel<bf16, float>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((merge_tile_kernel<bf16, bf16>), grid, block, 0, s, a);
        } else {
            // fewer than 256 workgroups (under 128 heads): split the batches
            const int nbt = (p.B + 31) / 32;
            const dim3 gridm(grid.x, (unsigned)std::max(1, std::min(nbt, 256 / (int)grid.x)));
            if (wf && of) hipLaunchKernelGGL((merge_kernel<float, float>), gridm, block, 0, s, a);
            else if (wf) hipLaunchKernelGGL((merge_kernel<float, bf16>), gridm, block, 0, s, a);
            else if (of) hipLaunchKernelGGL((merge_kernel<bf16, float>), gridm, block, 0, s, a);
            else hipLaunchKernelGGL((merge_kernel<bf16, bf16>), gridm, block, 0, s, a);
        }
    } else {
        const dim3 grid((unsigned)(p.H * 2 * ((p.B + F32_UB - 1) / F32_UB))), block(256);
        const float* olat = (const float*)w.opart;
        if (wf && of) hipLaunchKernelGGL((uproj_f32_kernel<float, float>), grid, block, 0, s, a, olat);
        else if (wf) hipLaunchKernelGGL((uproj_f32_kernel<float, bf16>), grid, block, 0, s, a, olat);
        else if (of) hipLaunchKernelGGL((uproj_f32_kernel<bf16, float>), grid, block, 0, s, a, olat);
        else hipLaunchKernelGGL((uproj_f32_kernel<bf16, bf16>), grid, block, 0, s, a, olat);
    }
    return hipGetLastError();
}

}  // namespace mla
