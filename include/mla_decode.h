/*
 * mla_decode.h -- C ABI of libmla_decode.so: the absorbed multi-head latent
 * attention (MLA) decode step of DeepSeek-V3.2-Exp with top-k sparse
 * selection, for AMD Instinct MI355X (gfx950).
 *
 * What one call computes (sources: the atlas pages on DeepSeek-V3.2-Exp's
 * sparse latent attention; excerpt names in brackets):
 *   For every sequence b and head h, with p_b = L_b - 1 the position of the
 *   single query token ("Attention weights": L = P + 1 keys in decode):
 *     q^    = rope(q_pe[b,h], p_b)                      [apply-rope, interleaved]
 *     q_abs = q_nope[b,h] . W_UK[h]          (512)      [mla-decode, absorption]
 *     s_t   = scale * (q_abs . C[b,t] + q^ . R[b,t])    [mla-decode, scores]
 *             for t in S_b, the top-k selection; -inf elsewhere [mla-decode, index mask]
 *     P     = softmax_t(s)                              [mla-decode]
 *     o     = sum_t P_t C[b,t]                   (512)  [mla-decode, latent sum]
 *     out   = W_UV[h] . o                        (128)  [mla-decode, up-projection]
 *   where C is the latent cache (kv_cache), R the rotated rope-key cache
 *   (pe_cache) and W_UK / W_UV the two halves of the per-head key-value
 *   up-projection ("Rotated query part", excerpt mla-decode: the weight is
 *   viewed as [heads, 256, 512], W_UK = rows 0..127, W_UV = rows 128..255,
 *   latent index contiguous).
 *
 * Beside the step: mla_topk (the selection step that produces topk_indices
 * from per-position scores), mla_rope_apply (RoPE at per-row positions, in
 * the interleaved or the half-split pair layout), and an optional fused
 * append of each sequence's new cache row inside mla_decode_attn (fields
 * kv_new / pe_new of mla_decode_params_t).
 *
 * Conventions
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library allocates no device memory and keeps no state between calls;
 *     scratch memory comes from the caller's workspace.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream).  No host synchronisation happens unless
 *     MLA_FLAG_VALIDATE is set.
 *   - Strides are in ELEMENTS of the tensor's dtype.  The innermost
 *     dimension is always contiguous.
 *   - Functions are thread-safe; mla_last_error() is per thread.
 *   - All argument checks finish before anything is enqueued: a call that
 *     returns an error has launched nothing.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- codes ------------------------------------------------------------ */
#define MLA_OK                 0
#define MLA_ERR_INVALID_ARG    1  /* null/misaligned pointer, bad stride or size */
#define MLA_ERR_UNSUPPORTED    2  /* dims other than 128/64/128/512, unknown dtype */
#define MLA_ERR_WORKSPACE      3  /* workspace missing or smaller than required */
#define MLA_ERR_INVALID_INDEX  4  /* validate mode: bad index set or cache length */
#define MLA_ERR_HIP            5  /* a HIP runtime call failed */

#define MLA_DTYPE_F32   0
#define MLA_DTYPE_BF16  1

#define MLA_FLAG_VALIDATE  1u     /* check indices/lengths on the device, then sync */

/* Bits reported through mla_decode_params_t.validate_status (validate mode). */
#define MLA_BAD_INDEX_RANGE  1u   /* an index outside [0, L_b) and not -1 */
#define MLA_BAD_DUPLICATE    2u   /* a position listed twice in one row */
#define MLA_BAD_EMPTY        4u   /* no selected position in a row */
#define MLA_BAD_CACHE_LEN    8u   /* L_b < 1, L_b > max_cache_len or L_b > rope_table_len */

/* Number of kernels one mla_decode_attn call enqueues (see profile_events). */
#define MLA_NUM_KERNELS 3

/* ---- rotary / YaRN configuration -------------------------------------- */
/* Field meanings follow the ModelArgs defaults on page "Transformer blocks /
 * RoPE coefficients" (excerpt model-args): max_seq_len 16384 (= 4096 * 4),
 * original_seq_len 4096, rope_theta 10000, rope_factor 40, beta_fast 32,
 * beta_slow 1, mscale 1; rope_dim is qk_rope_head_dim = 64. */
typedef struct mla_rope_cfg {
    int32_t rope_dim;          /* rotary features per head; must be 64 */
    int32_t max_seq_len;       /* T_max: rows of the table */
    int32_t original_seq_len;  /* T_0: interpolation applies when T_max > T_0 */
    int32_t reserved;          /* must be 0 */
    double  theta;             /* rope_theta */
    double  factor;            /* rope_factor */
    double  beta_fast;
    double  beta_slow;
    double  mscale;
} mla_rope_cfg_t;

/*
 * mla_rope_freqs -- the rotation table [page "Transformer blocks / RoPE
 * coefficients" and page "Rotated query part", excerpt rope].
 *   table: device float32 [cfg->max_seq_len][rope_dim/2][2], written with
 *          (cos, sin)(t * theta'_i) for position t and pair i, where
 *          theta_i = theta^(-2i/rope_dim) and, when max_seq_len >
 *          original_seq_len, theta'_i blends theta_i/factor and theta_i with
 *          YaRN's linear ramp over the pair index between the correction
 *          dimensions floor(D(beta_fast)) and ceil(D(beta_slow)),
 *          D(beta) = rope_dim * ln(T_0 / (2 pi beta)) / (2 ln theta).
 *          Angles are formed in double precision and stored as float.
 *   Enqueues one kernel on `stream`.  Returns MLA_OK, MLA_ERR_INVALID_ARG
 *   (null pointer, max_seq_len < 1, non-positive theta/factor) or
 *   MLA_ERR_UNSUPPORTED (rope_dim != 64).
 */
int mla_rope_freqs(const mla_rope_cfg_t* cfg, float* table, void* stream);

/*
 * mla_softmax_scale -- qk_head_dim^-1/2, multiplied by
 * (0.1 * mscale * ln(factor) + 1)^2 when max_seq_len > original_seq_len
 * [page "Query rotary features", excerpt mla-init].  Host only.
 * Returns a negative value on a null cfg or qk_head_dim < 1.
 */
double mla_softmax_scale(int qk_head_dim, const mla_rope_cfg_t* cfg);

/* ---- the decode step --------------------------------------------------- */
typedef struct mla_decode_params {
    /* sizes */
    int32_t B;                 /* sequences (one query token each), >= 1 */
    int32_t H;                 /* query heads, >= 1 */
    int32_t K;                 /* width of topk_indices rows, >= 1 */
    int32_t d_nope;            /* must be 128 (content features per head) */
    int32_t d_rope;            /* must be 64  (rotary features per head)  */
    int32_t d_v;               /* must be 128 (value features per head)   */
    int32_t kv_rank;           /* must be 512 (latent rank)               */
    int32_t max_cache_len;     /* L_max: rows allocated per sequence in the caches, 1..2^19 */
    int32_t rope_table_len;    /* rows of rope_table (its T_max) */
    /* dtypes: MLA_DTYPE_BF16 or MLA_DTYPE_F32 */
    int32_t dtype_act;         /* q_nope, q_pe, kv_cache, pe_cache */
    int32_t dtype_w;           /* w_uk, w_uv */
    int32_t dtype_out;         /* out */
    /* planning */
    int32_t num_cus;           /* compute units to plan for; 0 = current device */
    int32_t num_splits;        /* split-KV partitions per sequence; 0 = planner's choice */
    uint32_t flags;            /* MLA_FLAG_* */
    float   softmax_scale;     /* from mla_softmax_scale() */

    /* q_nope [B][H][128], q_pe [B][H][64] (q_pe raw: rotated inside);
     * strides are multiples of 8 (rows are read 16 bytes at a time) */
    const void* q_nope;  int64_t q_nope_stride_b, q_nope_stride_h;
    const void* q_pe;    int64_t q_pe_stride_b,   q_pe_stride_h;
    /* w_uk, w_uv [H][128][512], row stride 512, head stride given (a
     * multiple of 8); passing wkv_b viewed as [H][256][512] works with
     * w_uv = w_uk + 128*512 and both head strides 256*512. */
    const void* w_uk;    int64_t w_uk_stride_h;
    const void* w_uv;    int64_t w_uv_stride_h;
    /* kv_cache [B][max_cache_len][512], pe_cache [B][max_cache_len][64];
     * one fused [B][L_max][576] buffer works as pe_cache = kv_cache + 512
     * with both row strides 576. Row strides must be multiples of 8 and
     * the base pointers 16-byte aligned (bf16 rows are read 16 bytes at a time). */
    const void* kv_cache; int64_t kv_stride_b, kv_stride_t;
    const void* pe_cache; int64_t pe_stride_b, pe_stride_t;
    /* topk_indices [B][K] int32: positions in [0, L_b); -1 = unused slot.
     * One set per sequence, shared by every head; a position listed twice
     * counts once (set semantics of the index mask). */
    const int32_t* topk_indices; int64_t idx_stride_b;
    /* cache_lens [B] int32 on the device: L_b, keys present for sequence b
     * including the new token's own row (its query sits at p_b = L_b - 1). */
    const int32_t* cache_lens;
    /* rope_table from mla_rope_freqs(): [rope_table_len][32][2] float32 */
    const float* rope_table;

    /* outputs */
    void*  out;  int64_t out_stride_b, out_stride_h;  /* [B][H][128] in dtype_out */
    float* lse_out;            /* optional contiguous [B][H] float32 (element b*H + h): natural-log
                                * sum-exp of the scores; may be NULL */

    /* scratch: at least mla_decode_workspace_size(...) bytes, 256-byte aligned.
     * Its contents are undefined between calls (nothing needs clearing); two
     * calls whose work overlaps in time (different streams) must not share
     * one workspace. */
    void*  workspace;  size_t workspace_size;

    /* optional instrumentation: NULL, or 2*MLA_NUM_KERNELS hipEvent_t handles
     * recorded on `stream` before and after each enqueued kernel */
    void* const* profile_events;

    /* validate mode output: OR of MLA_BAD_* bits (0 when every row is valid) */
    uint32_t validate_status;
    uint32_t reserved0;

    /* optional fused append of the new token's row [page "Query rotary
     * features", excerpt mla-init: the joint down-projection emits the
     * latent and one shared rotary key].  Both NULL: the caches are only
     * read.  Both set: kv_new [B][512] (the latent, already normalised) and
     * pe_new [B][64] (the rotary key before rotation), dtype_act, 16-byte
     * aligned, batch strides in elements (multiples of 8).  Before any
     * cached position is read, row p_b = L_b - 1 of each sequence is written:
     * kv_cache[b][p_b] = kv_new[b] and pe_cache[b][p_b] = pe_new[b] rotated
     * at p_b (interleaved pairs, as the query).  The caches are then written
     * through kv_cache and pe_cache, which must be writable device memory;
     * a sequence whose L_b is invalid (see MLA_BAD_CACHE_LEN) is not
     * written. */
    const void* kv_new;  int64_t kv_new_stride_b;
    const void* pe_new;  int64_t pe_new_stride_b;
} mla_decode_params_t;

/*
 * mla_decode_num_splits -- the split-KV partition count the planner uses
 * for these sizes (host only; a pure function of its arguments).
 * num_cus = 0 queries the current device.  Returns < 1 on invalid sizes.
 */
int mla_decode_num_splits(int B, int H, int K, int dtype_act, int num_cus);

/*
 * mla_decode_workspace_size -- bytes of workspace one call needs for these
 * sizes, with num_splits = 0 meaning the planner's choice (same rule as
 * mla_decode_attn).  Host only.  Returns 0 on invalid sizes.
 */
size_t mla_decode_workspace_size(int B, int H, int K, int dtype_act, int dtype_w,
                                 int num_cus, int num_splits);

/*
 * mla_decode_attn -- one decode step for every sequence, as defined at the
 * top of this file [excerpt mla-decode on pages "Rotated query part",
 * "Query content heads" and "Attention weights"].
 *
 * Enqueues MLA_NUM_KERNELS kernels on `stream`:
 *   1. selection compaction (per sequence: drops -1 slots, duplicates and
 *      out-of-range entries, sorts the set ascending), query rotation at
 *      p_b, the W_UK absorption into Q~ = [q_abs ; q^], and, when kv_new
 *      is set, the write of each sequence's new row p_b into the caches;
 *   2. split-KV attention over the gathered 576-wide rows (bf16 MFMA,
 *      fp32 accumulation and online softmax) -- or fp32 arithmetic when
 *      dtype_act is F32;
 *   3. merge of the split partials and the W_UV up-projection.
 *
 * Returns MLA_OK; MLA_ERR_INVALID_ARG / _UNSUPPORTED / _WORKSPACE from the
 * host checks (nothing launched); MLA_ERR_HIP if a launch fails; and, with
 * MLA_FLAG_VALIDATE only, MLA_ERR_INVALID_INDEX after a stream sync when
 * p->validate_status is non-zero.  Without MLA_FLAG_VALIDATE a bad index
 * row or cache length is a precondition violation: the results for that
 * sequence are unspecified (an empty selection yields NaN), but no memory
 * outside the documented tensors is read or written.
 */
int mla_decode_attn(mla_decode_params_t* p, void* stream);

/* sizeof(mla_decode_params_t) as compiled into the library, so a binding
 * can check its own struct layout before the first call. */
size_t mla_decode_params_size(void);

/* Bytes of the scratch buffer mla_decode_attn_noalloc uses on each device. */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * mla_decode_attn_noalloc -- mla_decode_attn for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same computation, kernels, arguments and
 * return codes as mla_decode_attn, except that p->workspace and
 * p->workspace_size are ignored: the scratch memory is a buffer of
 * MLA_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs
 * on (in its code object, until the process ends).  The caller still owns
 * and passes every input and output.
 *   - Sizes whose mla_decode_workspace_size exceeds MLA_NOALLOC_SCRATCH_BYTES
 *     return MLA_ERR_WORKSPACE with nothing launched (the ragged batch of
 *     128 sequences x 128 heads x 2048 selected rows needs about 56 MB).
 *   - The first call on a device looks up that device's buffer address with
 *     hipGetSymbolAddress (with the device current); no call allocates.
 *   - Every call on one device shares its buffer and nothing in it needs
 *     clearing between calls.  Calls that overlap in time on one device
 *     (different streams or threads) race on the buffer: serialise them.
 */
int mla_decode_attn_noalloc(mla_decode_params_t* p, void* stream);

/* ---- top-k selection ---------------------------------------------------- */
typedef struct mla_topk_params {
    int32_t B;                 /* sequences, 1..2^20 */
    int32_t k;                 /* selection size and output row width, >= 1 */
    int32_t max_len;           /* positions per scores row, 1..2^19 */
    int32_t reserved;          /* must be 0 */
    /* scores [B][score_stride] float32 on the device, score_stride >= max_len */
    const float* scores;       int64_t score_stride;
    /* cache_lens [B] int32 on the device: L_b, clamped to [0, max_len] */
    const int32_t* cache_lens;
    /* topk_indices [B][idx_stride] int32 on the device (output), idx_stride >= k */
    int32_t* topk_indices;     int64_t idx_stride;
} mla_topk_params_t;

/*
 * mla_topk -- the indexer's selection step, which produces the index rows
 * mla_decode_attn consumes [page "Rotated query part", excerpt mla-decode:
 * topk_indices = indexer(...), then the index mask; the indexer's scoring
 * is not on the pages].  For every sequence b: the positions of the
 * k_b = min(k, L_b) largest of scores[b][0 .. L_b), written ascending to
 * topk_indices[b][0 .. k_b), then -1 up to k.  Scores compare in IEEE
 * order with -0 equal to +0 and NaN below every other value; among scores
 * equal to the k_b-th largest, the lowest positions are taken.
 * Enqueues one kernel on `stream`.  Returns MLA_OK, MLA_ERR_INVALID_ARG
 * (null pointer, sizes or strides out of range, reserved != 0) or
 * MLA_ERR_HIP (launch failure).
 */
int mla_topk(const mla_topk_params_t* p, void* stream);

/* ---- rotary embedding at per-row positions ------------------------------ */
typedef struct mla_rope_apply_params {
    int32_t N;                 /* rows (tokens or sequences), 1..2^24 */
    int32_t H;                 /* 64-wide vectors per row (heads), 1..4096; N*H <= 2^27 */
    int32_t dtype;             /* MLA_DTYPE_BF16 or MLA_DTYPE_F32, for x and y */
    int32_t interleaved;       /* 1: pairs (2i, 2i+1); 0: pairs (i, i+32) */
    int32_t table_len;         /* rows of rope_table */
    int32_t reserved;          /* must be 0 */
    /* x [N][H][64] on the device, element strides: row x_stride_n, vector
     * x_stride_h; both multiples of 8, x_stride_h >= 64 and
     * x_stride_n >= (H-1)*x_stride_h + 64; 16-byte aligned base */
    const void* x;             int64_t x_stride_n;  int64_t x_stride_h;
    /* y: same shape and rules (output); y == x with equal strides rotates in
     * place; any other overlap of x and y is undefined */
    void* y;                   int64_t y_stride_n;  int64_t y_stride_h;
    /* positions [N] int32 on the device: t_n for every vector of row n */
    const int32_t* positions;
    /* rope_table from mla_rope_freqs(): [table_len][32][2] float32, 16-byte aligned */
    const float* rope_table;
} mla_rope_apply_params_t;

/*
 * mla_rope_apply -- rotary embedding of every 64-wide vector x[n][h] at
 * position t_n [page "Rotated query part", excerpt apply-rope; table from
 * page "Transformer blocks / RoPE coefficients"]: the 32 feature pairs are
 * complex numbers z_i multiplied by cos(t theta'_i) + i sin(t theta'_i)
 * = rope_table[t][i].  interleaved = 1 pairs features (2i, 2i+1), the layout
 * of the attention path's rotary query and key; interleaved = 0 pairs
 * (i, i+32), the indexer's layout (the vector viewed as [2][32] and
 * transposed; real parts written to 0..31, imaginary parts to 32..63).
 * fp32 arithmetic; bf16 output rounds to nearest even.  A position outside
 * [0, table_len) is a precondition violation: that row's vectors are
 * written as NaN.  Enqueues one kernel on `stream`.  Returns MLA_OK,
 * MLA_ERR_INVALID_ARG (null pointer, sizes, strides or alignment out of
 * range, reserved != 0) or MLA_ERR_HIP (launch failure).
 */
int mla_rope_apply(const mla_rope_apply_params_t* p, void* stream);

/* Text of the last error on the calling thread ("" if none). */
const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_DECODE_H */
