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
// bf16 path: out[b, h, :] = sum_s w_{b,s} (W_UV[h] . o_s[b, h, :])
//   w_{b,s} = 2^(lse_s - M) / sum_s' 2^(lse_s' - M),  M = max_s lse_s.
// The projection is linear, so each split's bf16 partial is projected as it
// is stored (no re-rounding of a merged latent) and the fp32 projections are
// combined.  Workgroup (head h, output half dh) covers every sequence with 8
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
            const int b0 = 32 * (u / G), bA = b0 + l32;
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
        if (p.B < 128 && plan.splits <= 8) {
            if (wf && of) hipLaunchKernelGGL((merge_tile_kernel<float, float>), grid, block, 0, s, a);
            else if (wf) hipLaunchKernelGGL((merge_tile_kernel<float, bf16>), grid, block, 0, s, a);
            else if (of) hipLaunchKernelGGL((merge_tile_kernel<bf16, float>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((merge_tile_kernel<bf16, bf16>), grid, block, 0, s, a);
        } else {
            if (wf && of) hipLaunchKernelGGL((merge_kernel<float, float>), grid, block, 0, s, a);
            else if (wf) hipLaunchKernelGGL((merge_kernel<float, bf16>), grid, block, 0, s, a);
            else if (of) hipLaunchKernelGGL((merge_kernel<bf16, float>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((merge_kernel<bf16, bf16>), grid, block, 0, s, a);
        }
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
