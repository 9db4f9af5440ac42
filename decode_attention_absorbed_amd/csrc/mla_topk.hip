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
// 32-bit keys; a radix select over four 8-bit digits, most significant
// first, finds the threshold key T and how many keys equal to T are taken
// (256-bin LDS histograms of the keys that share the prefix found so far,
// one per wave and then summed, so that the many keys of one digit value
// do not all collide on one LDS word).
// The keys live in LDS when the row fits (up to 32768 positions), otherwise
// every pass re-reads the row (it stays in L2).  The output pass gives each
// wave a contiguous range of positions, visits it 64 positions at a time
// and compacts with ballots, so the positions come out ascending.
#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

constexpr int TK_THREADS = 1024;
constexpr int TK_LDS_KEYS = 32768;          // 128 KB of keys in LDS

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

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(TopkArgs a) {
    __shared__ uint32_t keys[TK_LDS_KEYS];
    __shared__ int whist[TK_THREADS / 64][256];   // per-wave histograms (fewer colliding atomics)
    __shared__ int hist[256];
    __shared__ int wcnt[2][TK_THREADS / 64];
    __shared__ int sel_digit, sel_above;
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

    // radix select: after the pass at shift s, prefix holds the top 32 - s
    // bits of T, and krem the number of keys equal to that prefix still to
    // take (keys above the prefix are all taken)
    uint32_t prefix = 0u, pmask = 0u;
    int krem = kb;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < (TK_THREADS / 64) * 256; i += TK_THREADS) (&whist[0][0])[i] = 0;
        __syncthreads();
        visit8(tid, TK_THREADS, [&](uint32_t key, int i) {
            if (i < L && (key & pmask) == prefix) atomicAdd(&whist[wave][(key >> shift) & 255], 1);
        });
        __syncthreads();
        if (tid < 256) {
            int c = 0;
#pragma unroll
            for (int w = 0; w < TK_THREADS / 64; ++w) c += whist[w][tid];
            hist[tid] = c;
        }
        __syncthreads();
        if (tid < 64) {
            // suffix sums over the 256 bins, 4 bins per lane (lane 0 holds
            // the top bins 255..252)
            int c[4], s = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) { c[j] = hist[255 - (4 * tid + j)]; s += c[j]; }
            int inc = s;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int n = __shfl_up(inc, o);
                if (tid >= o) inc += n;
            }
            int above = inc - s;                 // keys in bins above this lane's four
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (above < krem && above + c[j] >= krem) {
                    sel_digit = 255 - (4 * tid + j);
                    sel_above = above;
                }
                above += c[j];
            }
        }
        __syncthreads();
        prefix |= (uint32_t)sel_digit << shift;
        pmask |= 255u << shift;
        krem -= sel_above;
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

hipError_t launch_topk(int B, int k, int max_len, const float* scores, long long score_stride,
                       const int32_t* cache_lens, int32_t* out, long long out_stride, hipStream_t s) {
    TopkArgs a{B, k, max_len, scores, score_stride, cache_lens, out, out_stride};
    hipLaunchKernelGGL(topk_kernel, dim3(B), dim3(TK_THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace mla
