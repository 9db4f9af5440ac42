// Rotation table and the per-call preparation kernel of the MLA decode step.
//
// Sources (atlas pages on DeepSeek-V3.2-Exp sparse latent attention):
//   rotation table:  "Transformer blocks / RoPE coefficients", excerpt rope
//   query rotation:  "Rotated query part", excerpt apply-rope (interleaved pairs)
//   absorption:      "Rotated query part", excerpt mla-decode (q_nope . W_UK[h])
//   selection:       "Rotated query part", excerpt mla-decode (index mask; one
//                    set per sequence, shared by every head)
#include <math.h>

#include <algorithm>

#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

// ---------------------------------------------------------------------------
// (cos, sin)(t * theta'_i), angles in double precision.
// theta_i = theta^(-2i/d); with interpolation (T_max > T_0) theta'_i =
// theta_i/factor * ramp_i + theta_i * (1 - ramp_i), ramp linear in i between
// the YaRN correction dimensions floor(D(beta_fast)) and ceil(D(beta_slow)).
// ---------------------------------------------------------------------------
struct RopeArgs {
    int T, d, T0;
    double theta, factor, beta_fast, beta_slow;
    float* table;
};

__device__ double correction_dim(double beta, int d, int T0, double theta) {
    return d * log((double)T0 / (2.0 * M_PI * beta)) / (2.0 * log(theta));
}

__global__ __launch_bounds__(256) void rope_freqs_kernel(RopeArgs a) {
    const int half = a.d / 2;
    const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (long long)a.T * half) return;
    const int t = (int)(e / half), i = (int)(e % half);
    double f = pow(a.theta, -(2.0 * i) / a.d);
    if (a.T > a.T0) {
        double lo = floor(correction_dim(a.beta_fast, a.d, a.T0, a.theta));
        double hi = ceil(correction_dim(a.beta_slow, a.d, a.T0, a.theta));
        lo = fmax(lo, 0.0);
        hi = fmin(hi, (double)(a.d - 1));
        if (hi == lo) hi += 0.001;
        double ramp = fmin(fmax((i - lo) / (hi - lo), 0.0), 1.0);
        f = f / a.factor * ramp + f * (1.0 - ramp);
    }
    const double ang = (double)t * f;
    a.table[2 * e] = (float)cos(ang);
    a.table[2 * e + 1] = (float)sin(ang);
}

hipError_t launch_rope_freqs(const mla_rope_cfg_t& cfg, float* table, hipStream_t s) {
    RopeArgs a{cfg.max_seq_len, cfg.rope_dim, cfg.original_seq_len, cfg.theta, cfg.factor,
               cfg.beta_fast, cfg.beta_slow, table};
    const long long n = (long long)cfg.max_seq_len * (cfg.rope_dim / 2);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(rope_freqs_kernel, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Preparation kernel.  Blocks [0, n_absorb) compute the absorbed content
// query q_abs = q_nope . W_UK[h] into Q~[b, h, 0:512] and, on the bf16
// path, the rotary query of their head into Q~[b, h, 512:576]; blocks
// [n_absorb, n_absorb + B) handle one sequence each: compact the selection
// (and, on the fp32 path, rotate the rotary query).
// ---------------------------------------------------------------------------
struct PrepArgs {
    int B, H, K, Lmax, Trope, n_absorb, n_sg, validate;   // n_sg: absorption blocks per head half
    const void* q_nope; long long qn_sb, qn_sh;
    const void* q_pe;   long long qp_sb, qp_sh;
    const void* w_uk;   long long wk_sh;
    const int32_t* idx; long long idx_sb;
    const int32_t* cache_lens;
    const float* rope_table;
    // fused append (kv_new == nullptr: off)
    const void* kv_new; long long kn_sb;
    const void* pe_new; long long pn_sb;
    void* kv_dst; long long kd_sb, kd_st;
    void* pe_dst; long long pd_sb, pd_st;
    void* qt;
    void* qlo;          // bf16 path: low parts of the rotated query [B][H][64]
    int32_t* list;
    int32_t* counts;
    uint32_t* status;
};

// Eight consecutive elements as fp32 (16 or 32 bytes, aligned), and back.
template <typename T> __device__ __forceinline__ void load8f(const T* p, float (&v)[8]);
template <> __device__ __forceinline__ void load8f<bf16>(const bf16* p, float (&v)[8]) {
    const bf16x8 x = *(const bf16x8*)p;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
}
template <> __device__ __forceinline__ void load8f<float>(const float* p, float (&v)[8]) {
    const f32x4 x0 = *(const f32x4*)p, x1 = *(const f32x4*)(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = x0[e]; v[4 + e] = x1[e]; }
}
template <typename T> __device__ __forceinline__ void store8f(T* p, const float (&v)[8]);
template <> __device__ __forceinline__ void store8f<bf16>(bf16* p, const float (&v)[8]) {
    bf16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = f2bf(v[e]);
    *(bf16x8*)p = x;
}
template <> __device__ __forceinline__ void store8f<float>(float* p, const float (&v)[8]) {
    f32x4 x0, x1;
#pragma unroll
    for (int e = 0; e < 4; ++e) { x0[e] = v[e]; x1[e] = v[4 + e]; }
    *(f32x4*)p = x0;
    *(f32x4*)(p + 4) = x1;
}

// The new token's row: kv_cache[b][p] = kv_new[b] (16-byte copies by the
// first threads) and pe_cache[b][p] = pe_new[b] rotated at p, interleaved
// pairs, by threads 128..135 (8 features = 4 pairs each; cs is table row p).
template <typename ActT>
__device__ void append_row(const PrepArgs& a, int b, int p, const float* cs) {
    const int tid = threadIdx.x;
    constexpr int PER = 16 / (int)sizeof(ActT);       // elements per 16 bytes
    if (tid < RANK / PER) {
        const ActT* src = (const ActT*)a.kv_new + b * a.kn_sb;
        ActT* dst = (ActT*)a.kv_dst + b * a.kd_sb + (long long)p * a.kd_st;
        *(u32x4*)(dst + tid * PER) = *(const u32x4*)(src + tid * PER);
    } else if (tid >= 128 && tid < 128 + D_ROPE / 8) {
        const int q = tid - 128;
        float v[8], o[8];
        load8f<ActT>((const ActT*)a.pe_new + b * a.pn_sb + 8 * q, v);
        const f32x4 c0 = *(const f32x4*)(cs + 8 * q), c1 = *(const f32x4*)(cs + 8 * q + 4);
        const float cc[4] = {c0[0], c0[2], c1[0], c1[2]}, ss[4] = {c0[1], c0[3], c1[1], c1[3]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            o[2 * j] = v[2 * j] * cc[j] - v[2 * j + 1] * ss[j];
            o[2 * j + 1] = v[2 * j] * ss[j] + v[2 * j + 1] * cc[j];
        }
        store8f<ActT>((ActT*)a.pe_dst + b * a.pd_sb + (long long)p * a.pd_st + 8 * q, o);
    }
}

// Longest compacted list built in LDS (it overwrites the 64 KB bitmap area).
constexpr int PREP_LIST_MAX = 16384;

// Block-wide exclusive scan of one int per thread (256 threads).
__device__ int block_exclusive_scan(int v, int* total, int* lds_wave) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int inc = v;
    for (int o = 1; o < 64; o <<= 1) {
        int n = __shfl_up(inc, o);
        if (lane >= o) inc += n;
    }
    if (lane == 63) lds_wave[wave] = inc;
    __syncthreads();
    int base = 0, tot = 0;
    for (int w = 0; w < 4; ++w) {
        int x = lds_wave[w];
        if (w < wave) base += x;
        tot += x;
    }
    *total = tot;
    return base + inc - v;
}

// Selection compaction for sequence b: every position listed in the index
// row (minus -1 slots and entries outside [0, L_b)), once, ascending.
// LDS holds a bitmap of ceil(L_max / 32) words.
// Rotary query of one (head, 32-feature half): x is the raw q_pe slice,
// t the (cos, sin) pairs of row p_b; writes Q~[b, h, 512 + f0 ..].
template <typename QtT>
__device__ __forceinline__ void rotate32(const PrepArgs& a, int b, int h, int f0, const float (&x)[32],
                                         const float (&t)[32]) {
    QtT* dst = (QtT*)a.qt + ((long long)b * a.H + h) * ROW + RANK + f0;
    float yf[32];
    QtT y[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float c = t[2 * i], sn = t[2 * i + 1];
        yf[2 * i] = x[2 * i] * c - x[2 * i + 1] * sn;
        yf[2 * i + 1] = x[2 * i] * sn + x[2 * i + 1] * c;
        y[2 * i] = from_f32<QtT>(yf[2 * i]);
        y[2 * i + 1] = from_f32<QtT>(yf[2 * i + 1]);
    }
    if constexpr (sizeof(QtT) == 2) {
        // high part into Q~, the remainder (rounded to bf16) beside it
        bf16* lo = (bf16*)a.qlo + ((long long)b * a.H + h) * D_ROPE + f0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            bf16x8 v, r;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                v[j] = y[8 * k + j];
                r[j] = f2bf(yf[8 * k + j] - (float)y[8 * k + j]);
            }
            *(bf16x8*)(dst + 8 * k) = v;
            *(bf16x8*)(lo + 8 * k) = r;
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) *(f32x4*)(dst + 4 * k) = f32x4{y[4 * k], y[4 * k + 1], y[4 * k + 2], y[4 * k + 3]};
    }
}

// Rotary query of 8 pairs (features f .. f + 15) of head h, sequence b, with
// the table row's (cos, sin) values tv: the bf16 result into
// Q~[b, h, 512 + f ..] and the remainder (fp32 value minus that bf16 value,
// rounded to bf16) into the low-part region.
__device__ __forceinline__ void rotate16_bf16(const PrepArgs& a, int b, int h, int f, const bf16x8 (&xv)[2],
                                              const f32x4 (&tv)[4]) {
    bf16x8 v[2], r[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float x0 = (float)xv[i >> 2][2 * (i & 3)], x1 = (float)xv[i >> 2][2 * (i & 3) + 1];
        const float c = tv[i >> 1][2 * (i & 1)], sn = tv[i >> 1][2 * (i & 1) + 1];
        const float y0 = x0 * c - x1 * sn, y1 = x0 * sn + x1 * c;
        const bf16 h0 = f2bf(y0), h1 = f2bf(y1);
        v[i >> 2][2 * (i & 3)] = h0;
        v[i >> 2][2 * (i & 3) + 1] = h1;
        r[i >> 2][2 * (i & 3)] = f2bf(y0 - (float)h0);
        r[i >> 2][2 * (i & 3) + 1] = f2bf(y1 - (float)h1);
    }
    bf16* dst = (bf16*)a.qt + ((long long)b * a.H + h) * ROW + RANK + f;
    bf16* lo = (bf16*)a.qlo + ((long long)b * a.H + h) * D_ROPE + f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        *(bf16x8*)(dst + 8 * k) = v[k];
        *(bf16x8*)(lo + 8 * k) = r[k];
    }
}

template <typename ActT>
__device__ __forceinline__ void load_qpe32(const PrepArgs& a, int b, int h, int f0, float (&x)[32]) {
    const ActT* q = (const ActT*)a.q_pe + b * a.qp_sb + h * a.qp_sh + f0;
    if constexpr (sizeof(ActT) == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const bf16x8 v = *(const bf16x8*)(q + 8 * k);
#pragma unroll
            for (int j = 0; j < 8; ++j) x[8 * k + j] = (float)v[j];
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const f32x4 v = *(const f32x4*)(q + 4 * k);
#pragma unroll
            for (int j = 0; j < 4; ++j) x[4 * k + j] = v[j];
        }
    }
}

// One sequence: the selection compaction (every position listed in the
// index row, minus -1 slots and entries outside [0, L_b), once, ascending)
// and, on the fp32 path, the rotary query at p_b = L_b - 1 (pairs
// (2i, 2i+1) are one complex number; the bf16 path rotates it in the
// absorption blocks).  LDS holds a bitmap of ceil(L_b / 32) words, then the compacted
// list before it is copied out with coalesced stores.  The loads that do
// not depend on each other (cache length, the first 2048 indices, the first
// q_pe slices) are issued together; the rotation table row, which needs
// L_b, is loaded while the selection runs.
template <typename QtT, typename ActT>
__device__ void prep_sequence(const PrepArgs& a, int b, uint32_t* bm) {
    __shared__ int lds_wave[4];
    __shared__ uint32_t lds_status;
    const int tid = threadIdx.x;
    const int32_t* row = a.idx + (long long)b * a.idx_sb;
    const bool vec = ((uintptr_t)row & 15) == 0;
    const int kv = vec ? (a.K & ~3) : 0;              // indices read four at a time
    // -- loads issued together --
    const int L = a.cache_lens[b];
    int4 iv[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int j = 4 * tid + 1024 * k;
        iv[k] = j < kv ? *(const int4*)(row + j) : int4{-1, -1, -1, -1};
    }
    // The bf16 path rotates the query in the absorption blocks (one head
    // each); the fp32 path does it here.
    constexpr bool ROT_HERE = sizeof(QtT) == 4;
    float x[32];
    const bool rot0 = ROT_HERE && tid < 2 * a.H;      // this thread's first (head, half)
    if (rot0) load_qpe32<ActT>(a, b, tid >> 1, 32 * (tid & 1), x);
    const int p = min(max(L - 1, 0), a.Trope - 1);
    const float* cs = a.rope_table + (long long)p * D_ROPE;
    float t[32];
    if (rot0) {
        const int f0 = 32 * (tid & 1);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const f32x4 v = *(const f32x4*)(cs + f0 + 4 * k);
            t[4 * k] = v[0]; t[4 * k + 1] = v[1]; t[4 * k + 2] = v[2]; t[4 * k + 3] = v[3];
        }
    }
    // -- fused append of the new row (before any position is read: the
    // attention kernel runs after this one) --
    if (a.kv_new && L >= 1 && L <= a.Lmax && L <= a.Trope) append_row<ActT>(a, b, L - 1, cs);
    // -- selection --
    uint32_t status = 0;
    if (L < 1 || L > a.Lmax || L > a.Trope) status |= BAD_CACHE_LEN;
    const int Lc = L < 0 ? 0 : (L > a.Lmax ? a.Lmax : L);
    const int nwords = (Lc + 31) >> 5;
    if (tid == 0) lds_status = 0;
    for (int w = tid; w < nwords; w += 256) bm[w] = 0u;
    __syncthreads();
    auto mark = [&](int v) {
        if (v == -1) return;
        if (v < 0 || v >= L) { status |= BAD_INDEX_RANGE; return; }
        if (v >= Lc) return;                          // cache length already flagged
        const uint32_t bit = 1u << (v & 31);
        if (a.validate) {
            const uint32_t old = atomicOr(&bm[v >> 5], bit);
            if (old & bit) status |= BAD_DUPLICATE;
        } else {
            __hip_atomic_fetch_or(&bm[v >> 5], bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    };
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        mark(iv[k].x); mark(iv[k].y); mark(iv[k].z); mark(iv[k].w);
    }
    for (int j = 4 * tid + 2048; j < kv; j += 1024) {
        const int4 v = *(const int4*)(row + j);
        mark(v.x); mark(v.y); mark(v.z); mark(v.w);
    }
    for (int j = kv + tid; j < a.K; j += 256) mark(row[j]);
    __syncthreads();
    const int wpt = (nwords + 255) / 256;
    const int w0 = min(tid * wpt, nwords), w1 = min(w0 + wpt, nwords);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(bm[w]);
    int total;
    int off = block_exclusive_scan(cnt, &total, lds_wave);
    int32_t* out = a.list + (long long)b * a.K;
    if (total <= PREP_LIST_MAX && wpt <= 2) {
        // each thread's (at most two) words into registers, then the list
        // is built in LDS over the bitmap and copied out coalesced
        uint32_t wd[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) wd[k] = w0 + k < w1 ? bm[w0 + k] : 0u;
        __syncthreads();                              // every word read before the list overwrites them
        int* ll = (int*)bm;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            uint32_t bits = wd[k];
            while (bits) {
                ll[off++] = ((w0 + k) << 5) + __ffs(bits);   // 1-based: 0 marks "no row"
                bits &= bits - 1;
            }
        }
        __syncthreads();
        for (int i = tid; i < total; i += 256) out[i] = ll[i];
    } else {
        for (int w = w0; w < w1; ++w) {
            uint32_t bits = bm[w];
            while (bits) {
                out[off++] = (w << 5) + __ffs(bits);  // 1-based: 0 marks "no row"
                bits &= bits - 1;
            }
        }
    }
    if (tid == 0) {
        a.counts[b] = total;
        if (total == 0) status |= BAD_EMPTY;
    }
    // -- rotary query --
    for (int e = tid; ROT_HERE && e < a.H * 2; e += 256) {
        const int h = e >> 1, f0 = 32 * (e & 1);
        if (e != tid) {
            load_qpe32<ActT>(a, b, h, f0, x);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const f32x4 v = *(const f32x4*)(cs + f0 + 4 * k);
                t[4 * k] = v[0]; t[4 * k + 1] = v[1]; t[4 * k + 2] = v[2]; t[4 * k + 3] = v[3];
            }
        }
        rotate32<QtT>(a, b, h, f0, x, t);
    }
    if (status) atomicOr(&lds_status, status);
    __syncthreads();
    if (tid == 0 && lds_status && a.validate) atomicOr(a.status, lds_status);
}

// q_abs for head h, latent columns [256*half, 256*half + 256), every
// sequence, with bf16 MFMA: M = latent columns, N = sequences (32 per
// step), K = the 128 content features.  Wave w owns 64 columns.  Its
// weight slice W_UK[h][0:128][64 columns] is read once per group of
// sequences (128, or 64 when the batch has at most 64) with 16-byte loads,
// in eight chunks of 16 feature rows, two chunks in flight (four with
// 64-sequence groups).  Each chunk, as it lands, is converted to bf16 (fp32
// weights split into a bf16 high part and a bf16 remainder, two MFMAs each,
// so they enter with ~16 significant bits), passed through a wave-private
// LDS region to be read back transposed (8 consecutive features of one
// column per lane, ds_read_b64_tr_b16), and multiplied into the
// accumulators of every sequence of the group, so the MFMA work runs under
// the later chunks' loads; the staging of each chunk is split into parts
// placed between the previous chunk's MFMA groups, where they issue while
// the matrix core works.  The group's queries q_nope[:, h, :] are copied
// into LDS once (buffer->LDS, issued before the weight loads) and shared by
// the 4 waves.
constexpr int ABS_WAVE_LDS = 64 * 64 * 2;             // a wave's staging region (32 of its 64 rows used)
constexpr int ABS_QROWS = 128;                        // sequences per group (query chunk in LDS)
constexpr int ABS_Q_OFF = 4 * ABS_WAVE_LDS;           // query chunk: [128][128] bf16, 256 B rows
constexpr int ABS_CHUNKS = D_NOPE / 16;               // weight chunks of 16 feature rows (one K step)

// s_barrier after this wave's LDS operations, without waiting for its
// loads in flight (__syncthreads() waits for those too).
__device__ __forceinline__ void lds_barrier_only() {
    __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

// The thread index through an empty asm statement: lane-derived addresses
// are then computed inside the sequence-group loop instead of being hoisted
// out of it, where they would each hold a register for the whole loop.
__device__ __forceinline__ int tid_opaque() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// Sequences [b0, b0 + QR) of head h, latent half `half` (QR = 128, or 64
// when the batch has at most 64 sequences: half the accumulators, which
// leaves room for four weight chunks in flight instead of two).
template <typename WT, int QR>
__device__ __forceinline__ void absorb_group(const PrepArgs& a, int h, int half, char* lds, int b0) {
    constexpr int NP = sizeof(WT) == 4 ? 2 : 1;       // weight parts
    constexpr int ABS_AHEAD = QR == 64 ? 4 : 2;       // weight chunks in flight
    const int tid = tid_opaque(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const int c0 = 256 * half + 64 * wave;
    const WT* W = (const WT*)a.w_uk + h * a.wk_sh + c0;
    char* wl = lds + wave * ABS_WAVE_LDS;             // row d, column c at d*128 + c*2 (swizzled)
    const char* ql = lds + ABS_Q_OFF;
    // Staging row d holds 64 columns = 8 chunks of 16 bytes; chunk q sits at
    // slot q ^ (d & 7) so that the transposed reads (4 rows x 16 columns per
    // 16 lanes) do not collide.
    auto waddr = [&](int d, int c) {
        return d * 128 + ((((c >> 3) ^ (d & 7))) << 4) + (c & 7) * 2;
    };
    // Query chunk in LDS: sequence row r (0..127) at r * 256, its 16-byte
    // chunk k (features 8k..8k+7) at slot k ^ (r & 15): the MFMA operand read
    // (32 rows at one chunk) then touches 16 distinct slots per 16 lanes.
    // Copy: instruction i of a wave moves rows 4 (4 wave + i) + l/16, lane l
    // filling slot l % 16, i.e. fetching chunk (l % 16) ^ (row & 15).
    auto copy_q = [&](int b0) {
        const int nrow = min(QR, a.B - b0);
        const rsrc_t qs = make_rsrc((const bf16*)a.q_nope + b0 * a.qn_sb + h * a.qn_sh,
                                    (uint32_t)((nrow - 1) * a.qn_sb * 2 + D_NOPE * 2));
#pragma unroll
        for (int i = 0; i < QR / 16; ++i) {
            const int r = 4 * (QR / 16 * wave + i) + (lane >> 4);
            const uint32_t off = (uint32_t)(r < nrow ? r * a.qn_sb * 2 : 0x7FFFFFFF) + (uint32_t)((((lane & 15) ^ (r & 15))) << 4);
            buffer_to_lds16(qs, off, (MLA_LDS void*)(lds + ABS_Q_OFF + (QR / 16 * wave + i) * 1024));
        }
    };
    // Load: lane l takes columns 4 (l % 16) .. +3 of rows d = l / 16 + 4 i;
    // loads [4c, 4c + 4) hold feature rows [16c, 16c + 16) (chunk c).
    const int cq = 4 * (lane & 15);
    float wv[D_NOPE / 4][4];
    auto load_chunk = [&](int c) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int i = 4 * c + ii, d = (lane >> 4) + 4 * i;
            if constexpr (sizeof(WT) == 4) {
                const f32x4 x = *(const f32x4*)(W + d * RANK + cq);
#pragma unroll
                for (int e = 0; e < 4; ++e) wv[i][e] = x[e];
            } else {
                const bf16x4 x = *(const bf16x4*)(W + d * RANK + cq);
#pragma unroll
                for (int e = 0; e < 4; ++e) wv[i][e] = (float)x[e];
            }
        }
    };
    // Weight operand (A) of the chunk's K step, column block nb: lane l holds
    // column 32 nb + l%32, features 8 (l/32) .. +7 of the chunk -- two
    // transposed reads of 4 rows each.  In a 16-lane block, lane 4j + q
    // addresses local row 8 (blk >> 1) + 4 rr + j, columns
    // 32 nb + 16 (blk & 1) + 4 q .. +3.
    const int blk = lane >> 4, L = lane & 15, jj = L >> 2, qq = L & 3;

    const int nrow = min(QR, a.B - b0);
    // Rotary query of this head's feature half (32 features) for the group's
    // sequences: thread t takes sequence b0 + t/2, features
    // 32 half + 16 (t & 1) .. +15.  The cache length is loaded first; q_pe
    // and the table row are loaded after the last weight chunk, land while the
    // absorbed results are stored, and the rotation follows the stores.
    const int rs = tid >> 1, rf = 32 * half + 16 * (tid & 1);
    const bool rot = rs < nrow;
    const int Lr = rot ? a.cache_lens[b0 + rs] : 1;
    bf16x8 rxv[2];
    f32x4 rtv[4];
    {
        // The query copies go out before the weight loads, so the wait for
        // the first weight chunk covers them too.
        copy_q(b0);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int c = 0; c < ABS_AHEAD; ++c) load_chunk(c);
        f32x16 acc[QR / 32][2];
#pragma unroll
        for (int bt = 0; bt < QR / 32; ++bt)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) acc[bt][nb] = f32x16{};
        // Chunk c's operand: its two bf16 parts (part pp at local rows
        // 16 pp .. 16 pp + 15 of the wave's LDS region), read back transposed.
        // The staging of a chunk is four parts: converting feature rows 0-7,
        // converting rows 8-15 (then chunk c + AHEAD's loads go out), the
        // LDS writes, the transposed reads.  A wave issues in order, so the
        // parts of chunk c + 1 are placed between chunk c's MFMA groups (one
        // group per 32 sequences), where they issue while the matrix core
        // works.  A wave's LDS accesses run in order, so a chunk's writes
        // follow the previous chunk's reads and its reads follow its writes.
        bf16x4 wp[NP][4];
        auto convert = [&](int c, int half8) {
#pragma unroll
            for (int ii = 2 * half8; ii < 2 * half8 + 2; ++ii) {
                const int i = 4 * c + ii;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bf16 hi = (bf16)wv[i][e];
                    wp[0][ii][e] = hi;
                    if constexpr (NP == 2) wp[NP - 1][ii][e] = (bf16)(wv[i][e] - (float)hi);
                }
            }
        };
        auto write_stage = [&]() {
#pragma unroll
            for (int pp = 0; pp < NP; ++pp)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) *(bf16x4*)(wl + waddr(16 * pp + (lane >> 4) + 4 * ii, cq)) = wp[pp][ii];
        };
        auto read_stage = [&](bf16x8 (&bw)[NP][2]) {
#pragma unroll
            for (int pp = 0; pp < NP; ++pp)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    bf16x4 r[2];
#pragma unroll
                    for (int rr = 0; rr < 2; ++rr) {
                        const int d = 16 * pp + 8 * (blk >> 1) + 4 * rr + jj;
                        const int cc = 32 * nb + 16 * (blk & 1) + 4 * qq;
                        r[rr] = lds_read_tr16((const MLA_LDS void*)(wl + waddr(d, cc)));
                    }
                    bw[pp][nb] = cat(r[0], r[1]);
                }
        };
        // part p of chunk c's staging (c < ABS_CHUNKS)
        auto stage_part = [&](int c, int p, bf16x8 (&bw)[NP][2]) {
            if (p == 0) convert(c, 0);
            if (p == 1) {
                convert(c, 1);
                if (c + ABS_AHEAD < ABS_CHUNKS) load_chunk(c + ABS_AHEAD);
            }
            if (p == 2) write_stage();
            if (p == 3) read_stage(bw);
        };
        bf16x8 bwc[NP][2];
        wait_vmcnt<4 * (ABS_AHEAD - 1)>();            // query copies and chunk 0 landed
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            stage_part(0, p, bwc);
            asm volatile("" ::: "memory");
        }
        lds_barrier_only();                           // every wave's query copies visible
        constexpr int NG = QR / 32;                   // MFMA groups per chunk
#pragma unroll
        for (int c = 0; c < ABS_CHUNKS; ++c) {
            const bool more = c + 1 < ABS_CHUNKS;
            // Every group runs, without a branch: query rows past the batch
            // hold the zeros their out-of-window copies wrote, and their
            // results are never stored.
            bf16x8 aq[NG];
#pragma unroll
            for (int bt = 0; bt < NG; ++bt) {
                const int r = 32 * bt + l32;
                aq[bt] = *(const bf16x8*)(ql + r * 256 + (((2 * c + g) ^ (r & 15)) << 4));
            }
            bf16x8 bwn[NP][2];
            if (NG < 4 && more) stage_part(c + 1, 0, bwn);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int bt = 0; bt < NG; ++bt) {
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int pp = 0; pp < NP; ++pp) acc[bt][nb] = mfma32(bwc[pp][nb], aq[bt], acc[bt][nb]);
                if (more) {
                    // four groups: parts 0, 1 and 2 after groups 0, 1 and 2,
                    // part 3 after group 2 as well (group 3 then runs under
                    // the transposed reads' latency); two groups: part 0
                    // before group 0, part 1 after it, parts 2 and 3 after
                    // group 1
#pragma unroll
                    for (int p = NG >= 4 ? 0 : 1; p < 4; ++p)
                        if ((NG >= 4 ? (p < 3 ? p : 2) : (p == 1 ? 0 : 1)) == bt) stage_part(c + 1, p, bwn);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (more) {
#pragma unroll
                for (int pp = 0; pp < NP; ++pp)
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) bwc[pp][nb] = bwn[pp][nb];
            }
        }
        // q_pe and the table row for the rotary query, landing while the
        // results below are stored
        if (rot) {
            const int p = min(max(Lr - 1, 0), a.Trope - 1);
            const float* cs = a.rope_table + (long long)p * D_ROPE + rf;
            const bf16* q = (const bf16*)a.q_pe + (long long)(b0 + rs) * a.qp_sb + h * a.qp_sh + rf;
#pragma unroll
            for (int k = 0; k < 4; ++k) rtv[k] = *(const f32x4*)(cs + 4 * k);
#pragma unroll
            for (int k = 0; k < 2; ++k) rxv[k] = *(const bf16x8*)(q + 8 * k);
        }
        // D[column][sequence] (M = 32 columns, N = 32 sequences): lane l holds
        // sequence 32 bt + l%32 and columns 8(i/4) + 4(l/32) + i%4 of block nb.
        // Each batch passes through the wave's LDS region as [32 sequences]
        // [64 columns] (16-byte chunk k of row r at slot k ^ (r & 7)) and is
        // read back so that 8 lanes write one sequence's 128 contiguous bytes.
#pragma unroll
        for (int bt = 0; bt < QR / 32; ++bt) {
            __builtin_amdgcn_sched_barrier(0);
            if (32 * bt < nrow) {
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4) {
                        bf16x4 v;
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) v[rr] = f2bf(acc[bt][nb][4 * i4 + rr]);
                        const int k = 4 * nb + i4;             // 16-byte chunk of the 64 columns
                        *(bf16x4*)(wl + l32 * 128 + ((k ^ (l32 & 7)) << 4) + 8 * g) = v;
                    }
                __builtin_amdgcn_s_waitcnt(0xC07F);
                asm volatile("" ::: "memory");
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = (lane >> 3) + 8 * j, k = lane & 7;
                    const bf16x8 v = *(const bf16x8*)(wl + r * 128 + ((k ^ (r & 7)) << 4));
                    const int bA = b0 + 32 * bt + r;
                    if (bA < a.B) *(bf16x8*)((bf16*)a.qt + ((long long)bA * a.H + h) * ROW + c0 + 8 * k) = v;
                }
                __builtin_amdgcn_s_waitcnt(0xC07F);           // reads done before the next batch overwrites
                asm volatile("" ::: "memory");
            }
        }
        if (rot) rotate16_bf16(a, b0 + rs, h, rf, rxv, rtv);
    }
}

// Block sg of the head half takes the sequence groups sg, sg + n_sg, ...
// (n_sg > 1 only with few heads, so that more CUs share the groups).
template <typename WT, int QR>
__device__ void absorb_bf16(const PrepArgs& a, int h, int half, int sg, char* lds) {
    for (int b0 = sg * QR; b0 < a.B; b0 += a.n_sg * QR) {
        if (b0 > sg * QR) __syncthreads();            // every wave done with the previous query chunk
        absorb_group<WT, QR>(a, h, half, lds, b0);
    }
}

// fp32 variant: thread t owns latent column 256*half + t.
template <typename WT>
__device__ void absorb_f32(const PrepArgs& a, int h, int half) {
    const int c = 256 * half + threadIdx.x;
    const WT* W = (const WT*)a.w_uk + h * a.wk_sh;
    float wc[D_NOPE];
#pragma unroll
    for (int d = 0; d < D_NOPE; ++d) wc[d] = to_f32(W[d * RANK + c]);
    for (int b = 0; b < a.B; ++b) {
        const float* q = (const float*)a.q_nope + b * a.qn_sb + h * a.qn_sh;
        float acc = 0.f;
#pragma unroll
        for (int d = 0; d < D_NOPE; ++d) acc = fmaf(q[d], wc[d], acc);
        ((float*)a.qt)[((long long)b * a.H + h) * ROW + c] = acc;
    }
}

// LDS of a prep block: the absorption's weight staging (4 waves) and query
// chunk, or the selection bitmap of up to 2^19 positions.  64 KB lets two
// blocks share a CU, so selection blocks run beside absorption blocks.
constexpr int PREP_LDS = ABS_Q_OFF + ABS_QROWS * D_NOPE * 2;
static_assert(PREP_LDS >= (1 << 19) / 8, "bitmap of the largest cache");

// Blocks [0, n_absorb) compute absorption slices: block bid takes head
// (bid % 2H) / 2, half bid % 2 and, when n_sg > 1, its share bid / 2H of the
// sequence groups; they come first, so that each CU gets one of them;
// blocks [n_absorb, n_absorb + B) prepare one sequence each.  Two blocks per CU (64 KB of LDS each) need at most 256 registers per
// lane: the bound makes the compiler fit the absorption's accumulators for
// 128 sequences within it.
template <typename ActT, typename WT, int QR>
__global__ __launch_bounds__(256, 2) void prep_kernel(PrepArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t plds[PREP_LDS / 4];
    const int bid = blockIdx.x;
    if (bid >= a.n_absorb) {
        prep_sequence<ActT, ActT>(a, bid - a.n_absorb, plds);
    } else {
        const int hb = bid % (2 * a.H), sg = bid / (2 * a.H);
        const int h = hb >> 1, half = hb & 1;
        if constexpr (sizeof(ActT) == 2) absorb_bf16<WT, QR>(a, h, half, sg, (char*)plds);
        else absorb_f32<WT>(a, h, half);
    }
}

hipError_t launch_prep(const mla_decode_params_t& p, const Plan& plan, const Work& w, bool validate,
                       hipStream_t s) {
    PrepArgs a{};
    a.B = p.B; a.H = p.H; a.K = p.K; a.Lmax = p.max_cache_len; a.Trope = p.rope_table_len;
    a.validate = validate ? 1 : 0;
    a.q_nope = p.q_nope; a.qn_sb = p.q_nope_stride_b; a.qn_sh = p.q_nope_stride_h;
    a.q_pe = p.q_pe; a.qp_sb = p.q_pe_stride_b; a.qp_sh = p.q_pe_stride_h;
    a.w_uk = p.w_uk; a.wk_sh = p.w_uk_stride_h;
    a.idx = p.topk_indices; a.idx_sb = p.idx_stride_b;
    a.cache_lens = p.cache_lens; a.rope_table = p.rope_table;
    a.kv_new = p.kv_new; a.kn_sb = p.kv_new_stride_b;
    a.pe_new = p.pe_new; a.pn_sb = p.pe_new_stride_b;
    a.kv_dst = const_cast<void*>(p.kv_cache); a.kd_sb = p.kv_stride_b; a.kd_st = p.kv_stride_t;
    a.pe_dst = const_cast<void*>(p.pe_cache); a.pd_sb = p.pe_stride_b; a.pd_st = p.pe_stride_t;
    a.qt = w.qt; a.qlo = w.qlo; a.list = w.list; a.counts = w.counts; a.status = w.status;
    const bool wf = p.dtype_w == MLA_DTYPE_F32;
    // bf16 path: with fewer than 128 heads the 64-sequence groups of one
    // head half are spread over up to 256 / 2H blocks
    const int groups64 = (p.B + 63) / 64;
    a.n_sg = plan.bf16_path && p.H < 128 ? std::max(1, std::min(groups64, 256 / (2 * p.H))) : 1;
    a.n_absorb = 2 * p.H * a.n_sg;
    const dim3 grid(a.n_absorb + p.B), block(256);
    if (plan.bf16_path) {
        const bool small = p.B <= 64 || a.n_sg > 1;
        if (wf && small) hipLaunchKernelGGL((prep_kernel<bf16, float, 64>), grid, block, 0, s, a);
        else if (wf) hipLaunchKernelGGL((prep_kernel<bf16, float, ABS_QROWS>), grid, block, 0, s, a);
        else if (small) hipLaunchKernelGGL((prep_kernel<bf16, bf16, 64>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((prep_kernel<bf16, bf16, ABS_QROWS>), grid, block, 0, s, a);
    } else {
        if (wf) hipLaunchKernelGGL((prep_kernel<float, float, ABS_QROWS>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((prep_kernel<float, bf16, ABS_QROWS>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace mla
