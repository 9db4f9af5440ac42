// Top-k selection: the step that turns the indexer's per-position scores
// into the index rows the decode step consumes.
//
// For sequence b with L_b cached positions, the positions of the
// k_b = min(k, L_b) largest scores among scores[b][0 .. L_b), ascending,
// then -1 in the remaining slots of the row.  Source: page "Rotated query
// part", excerpt mla-decode (topk_indices = indexer(...) feeds the index
// mask; one set per sequence, shared by all heads).  The indexer's scoring
// is not on the pages; this kernel is its selection step only.  Ordering:
// IEEE order of the scores with -0 equal to +0 and NaN below everything
// (-inf included); among equal scores at the threshold the lowest positions
// are taken.
//
// One workgroup (16 waves) per sequence.  Scores become order-preserving
// 32-bit keys, and the threshold key T (the k_b-th largest) and how many
// keys equal to T are taken are found by histogram passes: each builds an
// LDS histogram of the keys still in play and locates the bin holding the
// k-th largest with a block-wide scan.
//
// topk_reg_kernel (launches whose rows have at most 32768 positions) keeps
// each thread's 16 or 32 contiguous keys in registers.  Its first pass
// buckets the scores by a monotone linear map of their value over the row's
// finite range (2048 even buckets), so that rows of similar values spread
// over many buckets (same-address LDS atomics within one instruction
// serialise).  The keys of the threshold bucket are gathered into an LDS
// list; up to 64 of them are ranked by one wave directly, more go through a
// radix select over three digits (bits 31..21, 20..10, 9..0).  The output
// is one block-wide scan of the per-thread (above T, equal to T) counts;
// selections of up to 4096 positions are compacted in LDS and written with
// coalesced stores.
//
// topk_kernel (longer rows) runs the radix select directly: its first digit
// spans the sign, the exponent and two mantissa bits, and the keys that fall
// in the first pass's threshold bin are gathered into a short LDS list (when
// there are at most 2048 of them), so that the later passes visit only
// those.  It keeps a row's keys in LDS when they fit and otherwise re-reads
// the scores each pass (they stay in L2); its output pass gives each wave a
// contiguous range of positions, visited 64 at a time and compacted with
// ballots.  Either way the positions come out ascending.
#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_LDS_KEYS = 32768;          // 128 KB of keys in LDS
constexpr int TK_BINS = 2048;               // widest digit: 11 bits
constexpr int TK_CAND = TK_BINS;            // candidate list (aliases the second histogram copy)

struct TopkArgs {
    int B, k, max_len;
    const float* scores; long long score_stride;
    const int32_t* cache_lens;
    int32_t* out; long long out_stride;
};

// Order-preserving key: larger score -> larger key; +-0 -> one key; NaN -> 0
// (below the key of -inf, 0x007FFFFF).
__device__ __forceinline__ uint32_t score_key(float f) {
    if (f != f) return 0u;
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0u) u = 0u;                  // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-wide inclusive prefix sum with DPP moves (no LDS round trips):
// within each row of 16 lanes add the values 1, 2, 4 and 8 lanes below
// (zero past the row start), then carry row 0's total into row 1 and row
// 2's into row 3 (lane 15 broadcast), then the total of rows 0-1 into rows
// 2 and 3 (lane 31 broadcast).
__device__ __forceinline__ int wave_scan_add(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
    return v;
}

// Largest value over the wave, in every lane: the same scan with max
// (identity -inf), then lane 63's result.
__device__ __forceinline__ float wave_max_dpp(float x) {
    const int ninf = __float_as_int(-INFINITY);
    int v = __float_as_int(x);
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(ninf, v, 0x111, 0xf, 0xf, false))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(ninf, v, 0x112, 0xf, 0xf, false))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(ninf, v, 0x114, 0xf, 0xf, false))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(ninf, v, 0x118, 0xf, 0xf, false))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(ninf, v, 0x142, 0xa, 0xf, false))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(ninf, v, 0x143, 0xc, 0xf, false))));
    return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(TopkArgs a) {
    __shared__ uint32_t keys[TK_LDS_KEYS];
    __shared__ int hist[2][TK_BINS];
    __shared__ int wsum[TK_WAVES];
    __shared__ int wcnt[2][TK_WAVES];
    __shared__ int sel_digit, sel_above, sel_count, ncand;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* row = a.scores + (long long)b * a.score_stride;
    int32_t* out = a.out + (long long)b * a.out_stride;
    const int L = min(max(a.cache_lens[b], 0), a.max_len);
    const int kb = min(a.k, L);

    if (kb == L) {
        // every position is selected
        for (int i = tid; i < a.k; i += TK_THREADS) out[i] = i < L ? i : -1;
        return;
    }
    const bool in_lds = L <= TK_LDS_KEYS;
    // Visit keys i = i0 + j * step (j < 8) for i0 = first, first + 8 step, ...:
    // the eight reads of a round are issued before any is used.
    auto visit8 = [&](int first, int step, auto&& f) {
        for (int i0 = first; i0 < L; i0 += 8 * step) {
            uint32_t kk[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = i0 + j * step;
                kk[j] = i < L ? (in_lds ? keys[i] : score_key(row[i])) : 0u;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) f(kk[j], i0 + j * step);
        }
    };
    if (in_lds) {
        for (int i0 = tid; i0 < L; i0 += 8 * TK_THREADS) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = i0 + j * TK_THREADS;
                v[j] = i < L ? row[i] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = i0 + j * TK_THREADS;
                if (i < L) keys[i] = score_key(v[j]);
            }
        }
    }
    if (tid == 0) ncand = 0;
    uint32_t* cand = (uint32_t*)&hist[1][0];

    // radix select: after each pass, prefix holds the leading bits of T
    // (pmask marks them), and krem the number of keys equal to that prefix
    // still to take (keys above the prefix are all taken)
    uint32_t prefix = 0u, pmask = 0u;
    int krem = kb;
    bool use_cand = false;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nb = pass == 2 ? 1024 : 2048;
        const int ncopy = pass == 0 ? 2 : 1;
        for (int i = tid; i < ncopy * TK_BINS; i += TK_THREADS) (&hist[0][0])[i] = 0;
        __syncthreads();
        if (pass == 0) {
            int* h = hist[wave & 1];
            visit8(tid, TK_THREADS, [&](uint32_t key, int i) {
                if (i < L) atomicAdd(&h[key >> 21], 1);
            });
        } else if (use_cand) {
            for (int i = tid; i < ncand; i += TK_THREADS) {
                const uint32_t key = cand[i];
                if ((key & pmask) == prefix) atomicAdd(&hist[0][(key >> shift) & (nb - 1)], 1);
            }
        } else {
            visit8(tid, TK_THREADS, [&](uint32_t key, int i) {
                if (i < L && (key & pmask) == prefix) atomicAdd(&hist[0][(key >> shift) & (nb - 1)], 1);
            });
        }
        __syncthreads();
        // thread t holds bins nb-1-2t and nb-2-2t (t < nb/2); an inclusive
        // scan over t gives the keys in higher bins
        int c0 = 0, c1 = 0;
        if (tid < nb / 2) {
            const int b0 = nb - 1 - 2 * tid;
            c0 = hist[0][b0] + (pass == 0 ? hist[1][b0] : 0);
            c1 = hist[0][b0 - 1] + (pass == 0 ? hist[1][b0 - 1] : 0);
        }
        int inc = c0 + c1;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int n = __shfl_up(inc, o);
            if (lane >= o) inc += n;
        }
        if (lane == 63) wsum[wave] = inc;
        __syncthreads();
        int above = inc - c0 - c1;
        for (int w = 0; w < wave; ++w) above += wsum[w];
        if (tid < nb / 2) {
            if (above < krem && above + c0 >= krem) {
                sel_digit = nb - 1 - 2 * tid; sel_above = above; sel_count = c0;
            } else if (above + c0 < krem && above + c0 + c1 >= krem) {
                sel_digit = nb - 2 - 2 * tid; sel_above = above + c0; sel_count = c1;
            }
        }
        __syncthreads();
        prefix |= (uint32_t)sel_digit << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
        krem -= sel_above;
        if (pass == 0 && sel_count <= TK_CAND) {
            // gather the keys of the threshold bin (the histogram copy it
            // overwrites was last read before the barrier above)
            use_cand = true;
            visit8(tid, TK_THREADS, [&](uint32_t key, int i) {
                const bool hit = i < L && (key >> 21) == (prefix >> 21);
                const uint64_t m = __ballot(hit);
                if (m) {
                    int base = 0;
                    if (lane == 0) base = atomicAdd(&ncand, __popcll(m));
                    base = __shfl(base, 0);
                    if (hit) cand[base + __popcll(m & ((1ull << lane) - 1ull))] = key;
                }
            });
            __syncthreads();
        }
    }
    const uint32_t T = prefix;                   // krem keys equal to T are taken

    // Output, ascending: wave w owns positions [w W, w W + W), visited 64 at a
    // time (lane l: position base + l), and compacts with ballots.
    const int W = (L + TK_THREADS - 1) / TK_THREADS * 64;
    const int wa = min(wave * W, L), wz = min(wa + W, L);
    int ngt = 0, neq = 0;
    for (int base = wa; base < wz; base += 64 * 8) {
        uint32_t kk[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = base + 64 * j + lane;
            kk[j] = i < wz ? (in_lds ? keys[i] : score_key(row[i])) : 0u;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = base + 64 * j + lane;
            ngt += __popcll(__ballot(i < wz && kk[j] > T));
            neq += __popcll(__ballot(i < wz && kk[j] == T));
        }
    }
    if (lane == 0) { wcnt[0][wave] = ngt; wcnt[1][wave] = neq; }
    __syncthreads();
    int eq_before = 0, sel_before = 0;
    for (int w = 0; w < wave; ++w) {
        const int e = wcnt[1][w];
        sel_before += wcnt[0][w] + min(e, max(0, krem - eq_before));
        eq_before += e;
    }
    int eq_left = min(neq, max(0, krem - eq_before));  // equal keys this wave takes
    int off = sel_before;
    for (int base = wa; base < wz; base += 64 * 8) {
        uint32_t kk[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = base + 64 * j + lane;
            kk[j] = i < wz ? (in_lds ? keys[i] : score_key(row[i])) : 0u;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = base + 64 * j + lane;
            const uint64_t gt = __ballot(i < wz && kk[j] > T);
            uint64_t eq = __ballot(i < wz && kk[j] == T);
            // keep the lowest eq_left lanes of eq
            const int ne = __popcll(eq);
            if (ne > eq_left) {
                uint64_t m = eq;
                for (int d = ne - eq_left; d > 0; --d) m &= ~(1ull << (63 - __clzll(m)));   // drop the highest
                eq = m;
            }
            eq_left -= __popcll(eq);
            const uint64_t take = gt | eq;
            if ((take >> lane) & 1ull) out[off + __popcll(take & ((1ull << lane) - 1ull))] = i;
            off += __popcll(take);
        }
    }
    for (int i = kb + tid; i < a.k; i += TK_THREADS) out[i] = -1;
}

// ---------------------------------------------------------------------------
// Rows of at most 32 * 1024 positions: thread t keeps the keys of positions
// [C t, C t + C) in registers (C = 16 or 32), so the passes read no LDS for
// keys.  The histograms are four LDS copies (one per group of four waves);
// the candidate list is its own LDS array.  The output is one block-wide
// scan of each thread's (above T, equal to T) counts, after which every
// thread writes its selected positions in order.
// ---------------------------------------------------------------------------
constexpr int TK_COPIES = 4;

// Thread t holds bins nb-1-2t and nb-2-2t (summed over the copies); a
// block-wide inclusive scan over t counts the keys in higher bins.  The
// thread whose bins contain the krem-th largest key records the digit, the
// number of keys above it and the digit's own count in sel[0..2].
__device__ __forceinline__ void find_digit(const int (*hist)[TK_BINS], int nb, int krem, int* wsum, int* sel) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int c0 = 0, c1 = 0;
    if (tid < nb / 2) {
        const int b0 = nb - 1 - 2 * tid;
#pragma unroll
        for (int c = 0; c < TK_COPIES; ++c) { c0 += hist[c][b0]; c1 += hist[c][b0 - 1]; }
    }
    const int inc = wave_scan_add(c0 + c1);
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int above = inc - c0 - c1;
#pragma unroll
    for (int w = 0; w < TK_WAVES; ++w) above += w < wave ? wsum[w] : 0;   // independent reads
    if (tid < nb / 2) {
        if (above < krem && above + c0 >= krem) {
            sel[0] = nb - 1 - 2 * tid; sel[1] = above; sel[2] = c0;
        } else if (above + c0 < krem && above + c0 + c1 >= krem) {
            sel[0] = nb - 2 - 2 * tid; sel[1] = above + c0; sel[2] = c1;
        }
    }
}

// Bucket of a score for the first pass: a monotone (non-decreasing) map of
// the value onto TK_BINS evenly spaced buckets over [lo, lo + 2047 / scale]
// (lo, scale from the row's finite scores), so that rows of similar values
// spread over many buckets.  NaN and -inf go to bucket 0 and +inf to the top
// one; the exact order inside a bucket is settled on the keys.
__device__ __forceinline__ int score_bucket(float x, float lo, float scale) {
    if (!(x > -INFINITY)) return 0;                  // NaN, -inf
    if (x == INFINITY) return TK_BINS - 1;
    if (scale == 0.f) return 0;                      // one bucket (no spread, or a span past float range)
    const float t = (x - lo) * scale;                // finite and >= 0 for finite x >= lo
    return t >= (float)(TK_BINS - 1) ? TK_BINS - 1 : (int)t;
}

// Largest candidates at most this many are settled by one wave counting
// ranks; more go through the radix passes.
constexpr int TK_RANK_MAX = 64;
// Selections of at most this many positions are compacted in LDS and
// written with coalesced stores.
constexpr int TK_OUT_LDS = 4096;

template <int C>
__global__ __launch_bounds__(TK_THREADS) void topk_reg_kernel(TopkArgs a) {
    // two histogram sets: the bucket pass and radix pass 1 use set 0, radix
    // passes 0 and 2 set 1, each cleared before its next use
    __shared__ int hist[2][TK_COPIES][TK_BINS];
    __shared__ uint32_t cand[TK_CAND];
    __shared__ int32_t outl[TK_OUT_LDS];
    __shared__ int wsum[TK_WAVES];
    __shared__ float wmin[TK_WAVES], wmax[TK_WAVES];
    __shared__ int sel[3];
    __shared__ int ncand;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* row = a.scores + (long long)b * a.score_stride;
    int32_t* out = a.out + (long long)b * a.out_stride;
    const int L = min(max(a.cache_lens[b], 0), a.max_len);
    const int kb = min(a.k, L);
    if (kb == L) {
        for (int i = tid; i < a.k; i += TK_THREADS) out[i] = i < L ? i : -1;
        return;
    }
    // Thread t holds positions [C t, C t + C).  Positions at or past L get a
    // NaN score: the lowest key, and higher positions than every real key,
    // so they rank below all L real keys (ties go to the lowest position)
    // and are never taken, since k_b <= L.  No per-key "present" predicate
    // is then needed (such lane masks would pin C SGPR pairs).
    const int p0 = tid * C;
    const int nv = min(max(L - p0, 0), C);            // this thread's positions below L
    float sc[C];
    if (nv == C && ((uintptr_t)row & 15) == 0) {
#pragma unroll
        for (int q = 0; q < C / 4; ++q) {
            const f32x4 v = *(const f32x4*)(row + p0 + 4 * q);
#pragma unroll
            for (int e = 0; e < 4; ++e) sc[4 * q + e] = v[e];
        }
    } else {
#pragma unroll
        for (int j = 0; j < C; ++j) sc[j] = j < nv ? row[p0 + j] : __builtin_nanf("");
    }
    // cleared while the scores are in flight (16-byte stores)
    for (int i = tid; i < 2 * TK_COPIES * TK_BINS / 4; i += TK_THREADS) ((u32x4*)&hist[0][0][0])[i] = u32x4{};
    if (tid == 0) ncand = 0;
    uint32_t key[C];
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < C; ++j) {
        key[j] = score_key(sc[j]);
        const bool fin = sc[j] > -INFINITY && sc[j] < INFINITY;
        mn = fin ? fminf(mn, sc[j]) : mn;
        mx = fin ? fmaxf(mx, sc[j]) : mx;
    }
    // range of the finite scores
    mn = -wave_max_dpp(-mn);
    mx = wave_max_dpp(mx);
    if (lane == 0) { wmin[wave] = mn; wmax[wave] = mx; }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < TK_WAVES; ++w) { mn = fminf(mn, wmin[w]); mx = fmaxf(mx, wmax[w]); }
    // scale 0 (one bucket) when there is no spread or it does not fit a float
    const float span = mx - mn;
    const float scale = (span > 0.f && span < INFINITY) ? (float)(TK_BINS - 1) / span : 0.f;
    const float lo = mn < INFINITY ? mn : 0.f;

    // ---- pass B: bucket histogram, threshold bucket Bt ----
    int bk[C];
    {
        int* h = hist[0][wave & (TK_COPIES - 1)];
#pragma unroll
        for (int j = 0; j < C; ++j) {
            bk[j] = score_bucket(sc[j], lo, scale);
            atomicAdd(&h[bk[j]], 1);
        }
    }
    __syncthreads();
    find_digit(hist[0], TK_BINS, kb, wsum, sel);      // counts include the NaN padding (bucket 0)
    __syncthreads();
    const int Bt = sel[0];
    int krem = kb - sel[1];                           // keys of bucket Bt still to take
    const int nbt = sel[2];
    // set 0 again for radix pass 1 (its reads ended at the barrier above)
    for (int i = tid; i < TK_COPIES * TK_BINS / 4; i += TK_THREADS) ((u32x4*)&hist[0][0][0])[i] = u32x4{};
    bool use_cand = false;
    if (nbt <= TK_CAND) {
        // the keys of bucket Bt into cand: a wave scan of the per-thread
        // counts, one LDS atomic per wave for its base
        use_cand = true;
        int nh = 0;
#pragma unroll
        for (int j = 0; j < C; ++j) nh += bk[j] == Bt ? 1 : 0;
        const int inc = wave_scan_add(nh);
        int base = 0;
        if (lane == 63 && inc > 0) base = atomicAdd(&ncand, inc);
        base = __builtin_amdgcn_readlane(base, 63);
        int off = base + inc - nh;
        // bucket Bt is usually a few keys of the row: a key slot that no
        // lane of the wave keeps is skipped with a uniform branch
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const bool hit = bk[j] == Bt;
            if (__builtin_amdgcn_ballot_w64(hit)) {
                if (hit) cand[off] = key[j];
            }
            off += hit ? 1 : 0;
        }
    }
    __syncthreads();

    uint32_t T;
    if (use_cand && nbt <= TK_RANK_MAX) {
        // every wave: lane i holds candidate i and counts the candidates
        // above and equal to it (read lane by lane from registers); T is the
        // candidate whose rank covers krem, and the keys equal to T to take
        // are krem minus the candidates above T
        const uint32_t mine = lane < nbt ? cand[lane] : 0u;
        int gt = 0, eq = 0;
        for (int j = 0; j < nbt; ++j) {
            const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)mine, j);
            gt += c > mine ? 1 : 0;
            eq += c == mine ? 1 : 0;
        }
        const bool is_t = lane < nbt && gt < krem && gt + eq >= krem;
        const int tl = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(is_t));   // a lane holding T
        T = (uint32_t)__builtin_amdgcn_readlane((int)mine, tl);
        krem -= __builtin_amdgcn_readlane(gt, tl);
    } else {
        // radix select over the keys of bucket Bt, three digits, most
        // significant first (bits 31..21, 20..10, 9..0)
        uint32_t prefix = 0u, pmask = 0u;
#pragma unroll 1
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
            const int nb = pass == 2 ? 1024 : 2048;
            int (*hs)[TK_BINS] = hist[(pass & 1) ^ 1];
            int* h = hs[wave & (TK_COPIES - 1)];
            if (use_cand) {
                for (int i = tid; i < nbt; i += TK_THREADS) {
                    const uint32_t kk = cand[i];
                    if ((kk & pmask) == prefix) atomicAdd(&h[(kk >> shift) & (nb - 1)], 1);
                }
            } else {
#pragma unroll
                for (int j = 0; j < C; ++j)
                    if (bk[j] == Bt && (key[j] & pmask) == prefix)
                        atomicAdd(&h[(key[j] >> shift) & (nb - 1)], 1);
            }
            __syncthreads();
            find_digit(hs, nb, krem, wsum, sel);
            __syncthreads();
            prefix |= (uint32_t)sel[0] << shift;
            pmask |= (uint32_t)(nb - 1) << shift;
            krem -= sel[1];
            // set 1 again for pass 2 (its reads ended at the barrier above;
            // pass 1's barrier orders this before pass 2's atomics)
            if (pass == 0)
                for (int i = tid; i < TK_COPIES * TK_BINS; i += TK_THREADS) (&hist[1][0][0])[i] = 0;
        }
        T = prefix;
    }
    // krem keys equal to T are taken (the lowest positions)

    // counts above and equal to T, packed 16 + 16 bits (at most 32768 keys
    // with the padding: no carry out of the low half, and the high half
    // stays below 2^16)
    int ngt = 0, neq = 0;
#pragma unroll
    for (int j = 0; j < C; ++j) {
        ngt += key[j] > T ? 1 : 0;
        neq += key[j] == T ? 1 : 0;
    }
    const uint32_t v = (uint32_t)ngt | ((uint32_t)neq << 16);
    const uint32_t inc = (uint32_t)wave_scan_add((int)v);
    if (lane == 63) wsum[wave] = (int)inc;
    __syncthreads();
    uint32_t excl = inc - v;
#pragma unroll
    for (int w = 0; w < TK_WAVES; ++w) excl += w < wave ? (uint32_t)wsum[w] : 0u;
    const int gt_before = (int)(excl & 0xFFFFu), eq_before = (int)(excl >> 16);
    int eq_take = min(neq, max(0, krem - eq_before));  // equal keys this thread takes (lowest first)
    int off = gt_before + min(eq_before, krem);
    if (kb <= TK_OUT_LDS) {
        // compact in LDS (positions not taken go to the spare slot), then
        // write the row with coalesced stores
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const int eq = (key[j] == T && eq_take > 0) ? 1 : 0;
            const int take = (key[j] > T ? 1 : 0) | eq;
            eq_take -= eq;
            if (take) outl[off] = p0 + j;
            off += take;
        }
        __syncthreads();
        for (int i = tid; i < a.k; i += TK_THREADS) out[i] = i < kb ? outl[i] : -1;
    } else {
#pragma unroll
        for (int j = 0; j < C; ++j) {
            bool take = key[j] > T;
            if (key[j] == T && eq_take > 0) { take = true; --eq_take; }
            if (take) out[off++] = p0 + j;
        }
        for (int i = kb + tid; i < a.k; i += TK_THREADS) out[i] = -1;
    }
}

hipError_t launch_topk(int B, int k, int max_len, const float* scores, long long score_stride,
                       const int32_t* cache_lens, int32_t* out, long long out_stride, hipStream_t s) {
    TopkArgs a{B, k, max_len, scores, score_stride, cache_lens, out, out_stride};
    if (max_len <= 16 * TK_THREADS)
        hipLaunchKernelGGL(topk_reg_kernel<16>, dim3(B), dim3(TK_THREADS), 0, s, a);
    else if (max_len <= 32 * TK_THREADS)
        hipLaunchKernelGGL(topk_reg_kernel<32>, dim3(B), dim3(TK_THREADS), 0, s, a);
    else
        hipLaunchKernelGGL(topk_kernel, dim3(B), dim3(TK_THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace mla
