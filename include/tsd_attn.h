/*
 * tsd_attn.h — C ABI of the MI355X (gfx950) tiled scaled-dot-product
 * attention forward library (libtsd_attn.so).
 *
 * Operation (VeriTile, "FlashAttention1.NaiveRefinement": the definitions
 * `fa1NaiveReference4D` / `fa1NaiveCausalReference4D` and the refinement
 * theorems for the FA-1 boundary + head-dim-tail kernels):
 *
 *   for every batch b < B, head h < H, query row i < S_q:
 *     s_j      = scale * sum_{d < D_qk} Q[b,h,i,d] * K[b,h,j,d]
 *     O[b,h,i,e] = sum_j softmax_j(s) * V[b,h,j,e]          (e < D_v)
 *     LSE[b,h,i] = ln sum_j exp(s_j)
 *   where j runs over 0 .. S_k-1, or over 0 .. min(i, S_k-1) when causal
 *   (key j visible to query i iff j <= i, top-left alignment).
 *
 * The key/query width D_qk may differ from the value width D_v (equation
 * "bqh,bkh,bkv->bqv", tiny.accy.kernel.library.attention).  The result is
 * computed tile by tile with an online softmax (running row max and sum);
 * in real arithmetic that equals the plain definition above exactly.
 */
#ifndef TSD_ATTN_H
#define TSD_ATTN_H

#include <stdint.h>

/* The library is built with hidden visibility; only these entry points are
 * exported. */
#if defined(__GNUC__) || defined(__clang__)
#define TSD_API __attribute__((visibility("default")))
#else
#define TSD_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Every check runs on the host before any HIP call; on an
 * error nothing is launched and no output byte is written. */
enum {
    TSD_OK = 0,
    TSD_ERR_NULL = 1,        /* Q, K, V or O is NULL (or plan output NULL)      */
    TSD_ERR_SHAPE = 2,       /* a dimension below 1 (the refinement theorems
                                require 0 < S_k; empty inputs are rejected)    */
    TSD_ERR_UNSUPPORTED = 3, /* D_qk or D_v above 128 (the block width: the
                                theorems need D <= block width), an unknown
                                dtype, a misaligned pointer, or a size beyond
                                the 32-bit in-slice / grid limits               */
    TSD_ERR_SCALE = 4,       /* scale is NaN or infinite                        */
    TSD_ERR_ALIAS = 5,       /* O or LSE overlaps Q, K, V, or each other (the
                                output region must be disjoint from the inputs) */
    TSD_ERR_HIP = 6,         /* the kernel launch itself failed                 */
    TSD_ERR_SCRATCH = 7      /* attn_fwd_splitkv_noalloc: the partial results
                                exceed TSD_NOALLOC_SCRATCH_BYTES                */
};

/* Storage dtypes of Q, K, V and O (all four share one).  Accumulation is
 * always f32; LSE is always f32. */
enum {
    TSD_F32 = 0,
    TSD_F16 = 1,
    TSD_BF16 = 2,
    TSD_FP8_E4M3 = 3     /* Q and K of attn_fwd_scaled only (OCP e4m3: 4 exponent
                            bits, 3 mantissa bits, no infinities)            */
};

/* Launch plan, as chosen by the planner for one call (pure host data). */
typedef struct tsd_plan {
    int32_t dtype;          /* TSD_F32 / TSD_F16 / TSD_BF16                     */
    int32_t causal;         /* 0 or 1                                           */
    int32_t block_m;        /* query rows per workgroup                         */
    int32_t block_n;        /* keys per K/V tile                                */
    int32_t dqk_block;      /* padded Q/K width the kernel runs at (>= D_qk)    */
    int32_t dv_block;       /* padded V/O width the kernel runs at (>= D_v)     */
    int32_t waves;          /* 64-lane waves per workgroup                      */
    int32_t threads;        /* threads per workgroup                            */
    int32_t lds_bytes;      /* LDS per workgroup                                */
    int32_t order;          /* 0: slice-major order; 1: slices grouped per XCD  */
    int64_t slices;         /* B * H                                            */
    int64_t q_blocks;       /* query blocks per slice = ceil(S_q / block_m)     */
    int64_t kv_blocks;      /* key tiles per slice    = ceil(S_k / block_n)     */
    int64_t grid;           /* workgroups launched = q_blocks * slices          */
    int64_t total_kv_steps; /* sum over workgroups of the key tiles visited     */
    int64_t vector_io;      /* 1: 16-byte global loads/stores; 0: per element   */
    int64_t key_split;      /* waves of a workgroup that split its key tiles    */
                            /* between them (f32 on small grids: 4), else 1     */
} tsd_plan;

/*
 * attn_fwd — enqueue the forward pass on `stream` and return.
 *
 *   Q   [B,H,S_q,D_qk], K [B,H,S_k,D_qk], V [B,H,S_k,D_v], O [B,H,S_q,D_v]:
 *       contiguous row-major device buffers of `dtype` (TSD_F32/F16/BF16),
 *       each aligned to its element size.
 *   LSE [B,H,S_q] contiguous f32 device buffer, natural log of the softmax
 *       denominator of the scaled scores; may be NULL (then not written).
 *   scale  any finite float (0 and negative allowed); multiplies the dot
 *       product.  Scores are formed in f32: a |scale * q.k| beyond the f32
 *       range (about 3.4e38) overflows.
 *   causal 0 or nonzero (top-left: key j visible to query i iff j <= i).
 *   stream a hipStream_t of the current device (NULL = its null stream);
 *       the kernels run on the current device, so every buffer must live
 *       there (or be accessible from it).
 *
 * Ownership: the caller allocates and frees every buffer; the library
 * allocates no device memory, keeps no pointer after returning, and never
 * synchronises.  It holds no global state and may be called from several
 * threads.  Only rows i < S_q and columns e < D_v of O, and only the B*H*S_q
 * entries of LSE, are written.  Returns a TSD_* status.
 */
TSD_API int attn_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE,
                     int64_t B, int64_t H, int64_t S_q, int64_t S_k,
                     int64_t D_qk, int64_t D_v, float scale, int causal, int dtype,
                     void *stream);

/*
 * attn_fwd_plan — fill `out` with the plan attn_fwd would use for these
 * sizes (no HIP call, no device access).  It is this library's form of the
 * launch description that tiny.accy.kernel.library.attention attaches to
 * its scaled-dot-product specialization (the `launch` / `schedule` entries:
 * a 3-D grid of thread blocks over the value, query and batch axes, whose
 * grid and block sizes that page's first unit test reads back): here a 1-D
 * grid of `grid` workgroups of `threads` threads, one per (query block of
 * `block_m` rows, slice), the slices being that page's batch axis (b, h).
 * Pointer alignment is not known here, so `vector_io` reports what aligned
 * buffers would get.  Returns the same shape/dtype statuses as attn_fwd
 * (TSD_ERR_NULL if out is NULL).
 */
TSD_API int attn_fwd_plan(int64_t B, int64_t H, int64_t S_q, int64_t S_k,
                          int64_t D_qk, int64_t D_v, int causal, int dtype,
                          tsd_plan *out);

/*
 * attn_fwd_plan_block — for workgroup `block` (0 <= block < plan->grid),
 * report the query block, the (batch*H + head) slice and the number of key
 * tiles it visits, exactly as the kernel derives them (host only): the
 * block-to-coordinates map of the schedule above (tiny.accy.kernel.library.
 * attention, the specialization's thread-block schedule), and the key-tile
 * count of the FA-1 kernels (VeriTile, "FlashAttention1.NaiveRefinement":
 * numKVBlocks tiles of Bk keys cover S_k, and a causal query block stops at
 * the tile of its last row).  Returns TSD_ERR_SHAPE if `block` is out of
 * range, TSD_ERR_NULL if `plan` is NULL.
 */
TSD_API int attn_fwd_plan_block(const tsd_plan *plan, int64_t S_q, int64_t S_k,
                                int64_t block, int64_t *q_block, int64_t *slice,
                                int64_t *kv_steps);

/*
 * ------------------------------------------------------------------------
 * Extended visibility, key chunks and the merge of partial results.
 *
 * These entry points run on the LDS-direct kernel only: dtype TSD_F16 or
 * TSD_BF16, Q/K/V (and a 16-bit O) 16-byte aligned, D_qk and D_v multiples
 * of 8 (else TSD_ERR_UNSUPPORTED).  Buffer ownership, threading and
 * synchronisation are as for attn_fwd.
 *
 * Grouped K/V heads (H_kv).  Q [B,H,S_q,D_qk], O [B,H,S_q,D_v] and LSE
 * [B,H,S_q] keep H heads; K [B,H_kv,S_k,D_qk] and V [B,H_kv,S_k,D_v] hold
 * H_kv heads, H a multiple of H_kv (else TSD_ERR_SHAPE), and query head h
 * reads K/V head h / (H / H_kv) (VeriTile proof coverage, attention_score:
 * program p of batch p / H reads K head (p mod H) / (H / H_KV)).  H_kv = H
 * is the usual layout; H_kv = 1 shares one K/V head among all heads.  The
 * H / H_kv query heads of a group are processed as one slice of their
 * stacked rows, so each K/V tile is read once for the whole group.
 *
 * Key visibility (tsd_mask).  Query row i of a slice sees exactly the keys
 *   j in [lo_i, hi_i),
 *   lo_i = max(kv_begin, i + causal_offset - window + 1)   (window > 0)
 *        = kv_begin                                          (window = 0)
 *   hi_i = min(kv_end, i + causal_offset + 1)                (causal)
 *        = kv_end                                            (not causal)
 * and the row's result is the definition above restricted to those keys.
 * A row that sees no key gets O = 0 and LSE = -infinity, the neutral
 * element of the merge below.  NULL means {0, 0, 0, S_k}: attn_fwd's own
 * visibility.
 *   - causal_offset moves the diagonal: S_k - S_q aligns it to the bottom
 *     right (VeriTile proof coverage, attention_llama: the causal case
 *     whose start_position shifts the key limit of every query block).
 *   - window keeps the `window` keys ending at the diagonal (VeriTile proof
 *     coverage, attention_fwd_triton3 case 1, the sliding-window keep
 *     predicate; its complement, the keys before the window, is the
 *     causal mask with causal_offset - window and no window).
 *   - [kv_begin, kv_end) restricts the keys (one chunk of a split key
 *     sequence: attention_fwd_triton3 case 4, the continuation that merges
 *     a chunk's result into the running one).
 * Invalid: kv_begin < 0, kv_end > S_k, kv_begin > kv_end, window < 0
 * (TSD_ERR_SHAPE); |causal_offset| or window above 2^30
 * (TSD_ERR_UNSUPPORTED).
 * K and V rows that no query row of the call sees (outside [kv_begin,
 * kv_end), after the last row's diagonal, before the first row's window)
 * may hold anything, NaN and infinity included: they never reach a result
 * (an unwritten cache tail after kv_end is fine).  Rows that some query row
 * sees are inputs like any other (a NaN there is not masked for the rows
 * that do not see it).
 */
typedef struct tsd_mask {
    int64_t causal_offset;  /* causal: key j visible to row i iff j <= i + causal_offset */
    int64_t window;         /* > 0: also j > i + causal_offset - window; 0: no window  */
    int64_t kv_begin;       /* first key of the range                                   */
    int64_t kv_end;         /* one past the last key of the range                       */
} tsd_mask;

/*
 * attn_fwd_ext — attn_fwd with the visibility of `mask` and H_kv K/V heads
 * (H_kv = H: the layout of attn_fwd).  Q [B,H,S_q,D_qk], K [B,H_kv,S_k,D_qk],
 * V [B,H_kv,S_k,D_v]; O [B,H,S_q,D_v] of `dtype`, LSE [B,H,S_q] f32 (may be
 * NULL).  Same statuses as attn_fwd, plus the mask, grouped-head and
 * fast-path conditions above.
 */
TSD_API int attn_fwd_ext(const void *Q, const void *K, const void *V, void *O, float *LSE,
                         int64_t B, int64_t H, int64_t H_kv, int64_t S_q, int64_t S_k,
                         int64_t D_qk, int64_t D_v, float scale, int causal, int dtype,
                         const tsd_mask *mask, void *stream);

/*
 * attn_fwd_partial — one partial result per key chunk (VeriTile proof
 * coverage, attention_fwd_triton3 case 3: a pass that writes O and a per-row
 * statistic for a later continuation).  Chunk s (0 <= s < n_splits) covers
 * the keys [kv_begin + s*split_len, kv_begin + (s+1)*split_len), cut to
 * [kv_begin, kv_end) and to each row's visibility; it writes
 *   O_parts   [n_splits,B,H,S_q,D_v] f32 (16-byte aligned): softmax over
 *             the chunk's visible keys times V (0 if none);
 *   LSE_parts [n_splits,B,H,S_q] f32 (required): ln of the chunk's sum of
 *             exp of the scaled scores (-infinity if none).
 * Q, K, V and H_kv as for attn_fwd_ext.  n_splits >= 1 and split_len >= 1
 * (TSD_ERR_SHAPE); kv_begin + n_splits * split_len must fit in int32
 * (TSD_ERR_UNSUPPORTED); a multiple of 64 keeps chunks on whole key tiles.
 * Merging the n_splits results with attn_merge gives attn_fwd_ext's result
 * up to rounding.
 */
TSD_API int attn_fwd_partial(const void *Q, const void *K, const void *V,
                             float *O_parts, float *LSE_parts,
                             int64_t B, int64_t H, int64_t H_kv, int64_t S_q, int64_t S_k,
                             int64_t D_qk, int64_t D_v, float scale, int causal, int dtype,
                             const tsd_mask *mask, int64_t n_splits, int64_t split_len,
                             void *stream);

/*
 * attn_merge — combine n_parts partial results of the same rows (VeriTile
 * proof coverage, attention_fwd_triton3 case 4, the continuation pass: the
 * running output is rescaled by the change of the row statistic and the
 * new chunk added).  For every row r:
 *   LSE[r] = ln sum_g exp(LSE_parts[g,r])
 *   O[r,:] = sum_g exp(LSE_parts[g,r] - LSE[r]) * O_parts[g,r,:]
 * (O = 0, LSE = -infinity when every part is -infinity).  O_parts
 * [n_parts,B,H,S_q,D_v] and LSE_parts [n_parts,B,H,S_q] are f32 (4-byte
 * aligned); O [B,H,S_q,D_v] of `dtype` (any of the three, element aligned);
 * LSE [B,H,S_q] f32 or NULL.  Any D_v in 1..128.  Outputs must not overlap
 * the parts (TSD_ERR_ALIAS).
 */
TSD_API int attn_merge(const float *O_parts, const float *LSE_parts, int64_t n_parts,
                       int64_t B, int64_t H, int64_t S_q, int64_t D_v,
                       void *O, float *LSE, int dtype, void *stream);

/*
 * attn_splitkv_plan — the chunking attn_fwd_splitkv uses (host only): the
 * launch description (tiny.accy.kernel.library.attention, the
 * specialization's `launch` entry) of a pass over key chunks whose partial
 * results a continuation merges (VeriTile proof coverage,
 * attention_fwd_triton3 cases 3 and 4).
 * n_splits <= 0 lets the library choose: enough chunks that one round of
 * workgroups covers the 256 compute units, chunks of at least 512 keys,
 * at most 256 chunks.  Reports the chunk count actually used (chunks are
 * whole 64-key tiles, so it may come out below the request; a request
 * above 256 is TSD_ERR_UNSUPPORTED), the chunk length in keys and the
 * workspace bytes attn_fwd_splitkv needs (0 when a single chunk is used:
 * then no workspace is touched).
 */
TSD_API int attn_splitkv_plan(int64_t B, int64_t H, int64_t H_kv, int64_t S_q, int64_t S_k,
                              int64_t D_qk, int64_t D_v, int causal, int dtype,
                              const tsd_mask *mask, int64_t n_splits,
                              int64_t *splits_out, int64_t *split_len_out,
                              int64_t *workspace_bytes);

/*
 * attn_fwd_splitkv — attn_fwd_ext computed as attn_fwd_partial over key
 * chunks followed by attn_merge, both enqueued on `stream`.  For launches
 * with few query blocks and many keys (long-context decoding, chunked
 * prefill) the chunks fill the chip that one workgroup per query block
 * cannot.  `workspace` (256-byte aligned, at least the planned bytes,
 * caller-owned, disjoint from every other buffer) holds the partial
 * results between the two launches; it may be NULL when the plan needs
 * none.  Too small a workspace: TSD_ERR_SHAPE.
 */
TSD_API int attn_fwd_splitkv(const void *Q, const void *K, const void *V, void *O, float *LSE,
                             int64_t B, int64_t H, int64_t H_kv, int64_t S_q, int64_t S_k,
                             int64_t D_qk, int64_t D_v, float scale, int causal, int dtype,
                             const tsd_mask *mask, int64_t n_splits,
                             void *workspace, int64_t workspace_bytes, void *stream);

/*
 * attn_fwd_splitkv_noalloc — attn_fwd_splitkv for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments without the
 * workspace.  The partial results are staged in a scratch array of
 * TSD_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs
 * on until the process ends (the device is the current one; a `stream` of
 * another device: TSD_ERR_UNSUPPORTED).  The call allocates nothing and
 * frees nothing.
 *   - A plan whose workspace (attn_splitkv_plan) exceeds the array:
 *     TSD_ERR_SCRATCH, nothing launched.  One chunk needs no scratch.
 *   - All calls on one device share its array.  Calls that overlap in time
 *     on one device (other streams, other host threads) race on it and give
 *     wrong results: serialise them (one stream, or events).  Each call
 *     writes every scratch entry it reads, so nothing carries over from an
 *     earlier call.
 * Other statuses, results and threading as for attn_fwd_splitkv.
 */
#define TSD_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)   /* 64 MiB */
TSD_API int attn_fwd_splitkv_noalloc(const void *Q, const void *K, const void *V, void *O,
                                     float *LSE, int64_t B, int64_t H, int64_t H_kv,
                                     int64_t S_q, int64_t S_k, int64_t D_qk, int64_t D_v,
                                     float scale, int causal, int dtype,
                                     const tsd_mask *mask, int64_t n_splits, void *stream);

/*
 * attn_fwd_scaled — base-2 attention with per-block Q and K scales
 * (VeriTile proof coverage, attention_forward_triton: the Q_scale value of
 * the program's query block and the K_scale value of each key block multiply
 * the scores, whose base-2 softmax weights V; `attentionRealBase2PerKeyScale`):
 *
 *   s_ij = Q_scale[b,h,i / q_block] * K_scale[b,h,j / k_block] * (Q_i . K_j)
 *   O_i  = sum_j 2^(s_ij) V_j / sum_j 2^(s_ij)       (j <= i when causal)
 *   LSE_i = ln sum_j 2^(s_ij)                        (natural log, as attn_fwd)
 *
 * The softmax scale and log2(e) belong in the block scales (a caller
 * quantising to fp8 passes absmax/448 * scale * log2(e) as Q_scale).
 *   Q [B,H,S_q,D_qk], K [B,H,S_k,D_qk] of `qk_dtype`: TSD_FP8_E4M3, or the
 *       same 16-bit dtype as V.  fp8 scores run on the fp8 MFMA.
 *   V [B,H,S_k,D_v], O [B,H,S_q,D_v] of `dtype` (TSD_F16 / TSD_BF16);
 *       LSE [B,H,S_q] f32 or NULL.
 *   Q_scale [B,H,ceil(S_q/q_block)] f32 and K_scale [B,H,ceil(S_k/k_block)]
 *       f32: any finite values, of either sign, zero included (the scales
 *       live in device memory and are not inspected on the host: NaN or
 *       infinite scales give unspecified results).
 *   q_block >= 1; k_block a multiple of 64 (the kernel's key tile).
 * Fast path only: every buffer but the scales 16-byte aligned, D_v a
 * multiple of 8, D_qk a multiple of 8 (16 for fp8); with fp8, D_qk in
 * 65..128, or D_qk and D_v both at most 64 (else TSD_ERR_UNSUPPORTED).
 * Statuses, ownership and threading as for attn_fwd.
 */
TSD_API int attn_fwd_scaled(const void *Q, const void *K, const void *V, void *O, float *LSE,
                            const float *Q_scale, const float *K_scale,
                            int64_t B, int64_t H, int64_t S_q, int64_t S_k,
                            int64_t D_qk, int64_t D_v, int64_t q_block, int64_t k_block,
                            int causal, int qk_dtype, int dtype, void *stream);

/* attn_status_string — static text for a status code (never NULL).  The
 * codes name the premise a call broke: the refinement theorems' 0 < S_k and
 * D <= block width (VeriTile, "FlashAttention1.NaiveRefinement"), the
 * disjoint output region of the coverage page's region premises (VeriTile
 * proof coverage), a finite scale, and this library's own limits. */
TSD_API const char *attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TSD_ATTN_H */
