// Host side of the C ABI: argument validation, the launch planner and the
// status strings.  Every check here runs before any HIP call, so an invalid
// call launches nothing and writes nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "launch.h"
#include "tsd_attn.h"

namespace {

constexpr int64_t kMaxHeadDim = 128;       // block width of the kernels
constexpr int64_t kMaxSliceBytes = (int64_t(1) << 31) - 1;

int elt_bytes(int dtype)
{
    switch (dtype) {
    case TSD_F32: return 4;
    case TSD_F16: return 2;
    case TSD_BF16: return 2;
    default: return 0;
    }
}

bool overlap(const void *a, uint64_t na, const void *b, uint64_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const uint64_t a0 = reinterpret_cast<uintptr_t>(a);
    const uint64_t b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

// Shape and dtype checks shared by attn_fwd and attn_fwd_plan.
int check_shape(int64_t B, int64_t H, int64_t S_q, int64_t S_k, int64_t D_qk, int64_t D_v,
                int dtype)
{
    if (B < 1 || H < 1 || S_q < 1 || S_k < 1 || D_qk < 1 || D_v < 1)
        return TSD_ERR_SHAPE;
    const int elt = elt_bytes(dtype);
    if (elt == 0) return TSD_ERR_UNSUPPORTED;
    if (D_qk > kMaxHeadDim || D_v > kMaxHeadDim) return TSD_ERR_UNSUPPORTED;
    // In-slice offsets are 32-bit in the kernels.
    if (S_q > kMaxSliceBytes / (D_qk * elt) || S_q > kMaxSliceBytes / (D_v * elt) ||
        S_k > kMaxSliceBytes / (D_qk * elt) || S_k > kMaxSliceBytes / (D_v * elt))
        return TSD_ERR_UNSUPPORTED;
    // Grid: q_blocks * B * H workgroups must fit an int32 block index.
    const int64_t q_blocks = (S_q + 127) / 128;
    if (B > INT32_MAX / H) return TSD_ERR_UNSUPPORTED;
    if (q_blocks > (int64_t(INT32_MAX) / 256) / (B * H)) return TSD_ERR_UNSUPPORTED;
    return TSD_OK;
}

void fill_plan(int64_t B, int64_t H, int64_t S_q, int64_t S_k, int64_t D_qk, int64_t D_v,
               int causal, int dtype, bool vector_io, tsd_plan *pl)
{
    const tsd::TileConfig cfg =
        tsd::tile_config(dtype, D_qk, D_v, vector_io, B * H, S_q, causal != 0);
    std::memset(pl, 0, sizeof(*pl));
    pl->dtype = dtype;
    pl->causal = causal ? 1 : 0;
    pl->block_m = cfg.block_m;
    pl->block_n = cfg.block_n;
    pl->dqk_block = cfg.dqk_block;
    pl->dv_block = cfg.dv_block;
    pl->waves = cfg.waves;
    pl->threads = cfg.threads;
    pl->lds_bytes = cfg.lds_bytes;
    pl->slices = B * H;
    pl->q_blocks = (S_q + cfg.block_m - 1) / cfg.block_m;
    pl->kv_blocks = (S_k + cfg.block_n - 1) / cfg.block_n;
    pl->grid = pl->q_blocks * pl->slices;
    pl->order = (pl->slices % 8 == 0) ? 1 : 0;
    pl->vector_io = vector_io ? 1 : 0;
    pl->key_split = cfg.split_keys ? cfg.waves : 1;
    int64_t steps = 0;
    for (int64_t qb = 0; qb < pl->q_blocks; ++qb)
        steps += tsd::kv_tiles_for((int32_t)qb, cfg.block_m, cfg.block_n, (int32_t)S_q,
                                   (int32_t)S_k, pl->causal != 0);
    pl->total_kv_steps = steps * pl->slices;
}

bool vector_dims_ok(int dtype, int64_t D_qk, int64_t D_v)
{
    const int per16 = 16 / elt_bytes(dtype);   // elements per 16-byte access
    return D_qk % per16 == 0 && D_v % per16 == 0;
}

// Kernel arguments common to every attention launch: sizes, the plan's
// grid mapping, the scale folded into Q, and the default key visibility
// (every key, plain causal).
tsd::KernelArgs base_args(const void *Q, const void *K, const void *V, void *O, float *LSE,
                          int64_t S_q, int64_t S_k, int64_t D_qk, int64_t D_v, float scale,
                          int dtype, bool vec, const tsd_plan &plan)
{
    tsd::KernelArgs a;
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.O = O;
    a.LSE = LSE;
    a.S_q = (int32_t)S_q;
    a.S_k = (int32_t)S_k;
    a.D_qk = (int32_t)D_qk;
    a.D_v = (int32_t)D_v;
    a.q_blocks = (int32_t)plan.q_blocks;
    a.slices = (int32_t)plan.slices;
    a.order = plan.order;
    a.per_xcd = (int32_t)(plan.slices / 8);
    // exp(x) = 2^(x log2 e): the log2(e) factor is folded into the scale.
    // A negative scale becomes a sign flip of Q (exact) with |scale|; a zero
    // scale makes every score 0, which is Q = 0 with any positive factor.
    const float log2e = 1.4426950408889634f;
    const uint32_t sign = dtype == TSD_F32 ? 0x80000000u : 0x80008000u;
    a.c = scale == 0.0f ? 1.0f : std::fabs(scale) * log2e;
    a.q_xor = scale < 0.0f ? sign : 0u;
    a.q_and = scale == 0.0f ? 0u : 0xffffffffu;
    a.vec = vec ? 1 : 0;
    a.kv_begin = 0;
    a.kv_end = (int32_t)S_k;
    a.coff = 0;
    a.window = 0;
    a.splits = 1;
    a.split_len = (int32_t)S_k;
    a.part_o_stride = 0;
    a.part_lse_stride = 0;
    a.q_per_head = (int32_t)S_q;
    a.Q_scale = nullptr;
    a.K_scale = nullptr;
    a.q_block = 1;
    a.q_scale_blocks = 0;
    a.k_tiles_per_block = 1;
    a.k_scale_blocks = 0;
    return a;
}

// Limits of the mask parameters: every per-row bound the kernel forms
// (i + offset - window + 1, i + offset + 1) stays inside int32.
constexpr int64_t kMaxMaskValue = int64_t(1) << 30;

// Validate a key mask (NULL = every key, no offset, no window) against S_k.
int check_mask(const tsd_mask *mask, int64_t S_k, tsd_mask *out)
{
    tsd_mask m = {0, 0, 0, S_k};
    if (mask) m = *mask;
    if (m.kv_begin < 0 || m.kv_end > S_k || m.kv_begin > m.kv_end || m.window < 0)
        return TSD_ERR_SHAPE;
    if (m.causal_offset > kMaxMaskValue || m.causal_offset < -kMaxMaskValue ||
        m.window > kMaxMaskValue)
        return TSD_ERR_UNSUPPORTED;
    *out = m;
    return TSD_OK;
}

// Sizes of an extended call.  Q, O and LSE have H heads, K and V H_kv;
// the kernels see one slice per K/V head whose rows are the query rows of
// its H / H_kv query heads (contiguous in Q, O and LSE), position = row
// modulo S_q.
struct ExtShape {
    int64_t B, H, H_kv, S_q, S_k, D_qk, D_v;
    int64_t group() const { return H / H_kv; }
    int64_t rows() const { return group() * S_q; }   // rows per kernel slice
};

// Checks shared by the extended entry points (which run on the LDS-direct
// kernel only): 16-bit dtype, 16-byte aligned Q/K/V, widths a multiple of 8.
int check_ext_inputs(const void *Q, const void *K, const void *V, const ExtShape &es,
                     float scale, int dtype)
{
    if (!Q || !K || !V) return TSD_ERR_NULL;
    if (es.B < 1 || es.H < 1 || es.H_kv < 1 || es.S_q < 1 || es.H % es.H_kv != 0)
        return TSD_ERR_SHAPE;
    if (es.S_q > INT32_MAX / es.group()) return TSD_ERR_UNSUPPORTED;   // rows() fits int32
    const int st = check_shape(es.B, es.H_kv, es.rows(), es.S_k, es.D_qk, es.D_v, dtype);
    if (st != TSD_OK) return st;
    if (!std::isfinite(scale)) return TSD_ERR_SCALE;
    if (dtype == TSD_F32) return TSD_ERR_UNSUPPORTED;
    if (!vector_dims_ok(dtype, es.D_qk, es.D_v)) return TSD_ERR_UNSUPPORTED;
    for (uintptr_t p : {(uintptr_t)Q, (uintptr_t)K, (uintptr_t)V})
        if (p % 16 != 0) return TSD_ERR_UNSUPPORTED;
    return TSD_OK;
}

// Byte sizes of the inputs (for the alias checks).
struct InputBytes {
    uint64_t q, k, v;
};
InputBytes input_bytes(const ExtShape &es, int dtype)
{
    const uint64_t elt = (uint64_t)elt_bytes(dtype);
    const uint64_t BH = (uint64_t)es.B * es.H, BHk = (uint64_t)es.B * es.H_kv;
    return InputBytes{BH * es.S_q * es.D_qk * elt, BHk * es.S_k * es.D_qk * elt,
                      BHk * es.S_k * es.D_v * elt};
}

bool overlaps_inputs(const void *p, uint64_t n, const void *Q, const void *K, const void *V,
                     const InputBytes &ib)
{
    return overlap(p, n, Q, ib.q) || overlap(p, n, K, ib.k) || overlap(p, n, V, ib.v);
}

// Launch the extended kernel over `splits` chunks of `split_len` keys
// starting at mask.kv_begin (splits = 1: the whole range).  out_f32: O and
// LSE are the chunked f32 partial buffers.
int launch_ext(const void *Q, const void *K, const void *V, void *O, float *LSE,
               const ExtShape &es, float scale, int causal, int dtype, const tsd_mask &mk,
               int64_t splits, int64_t split_len, bool out_f32, hipStream_t stream)
{
    const int64_t S_q = es.rows(), D_v = es.D_v;   // the kernel's view
    tsd_plan plan;
    fill_plan(es.B, es.H_kv, S_q, es.S_k, es.D_qk, D_v, causal, dtype, true, &plan);
    if (plan.grid > INT32_MAX / splits) return TSD_ERR_UNSUPPORTED;
    tsd::KernelArgs a =
        base_args(Q, K, V, O, LSE, S_q, es.S_k, es.D_qk, D_v, scale, dtype, true, plan);
    a.q_per_head = (int32_t)es.S_q;
    a.kv_begin = (int32_t)mk.kv_begin;
    a.kv_end = (int32_t)mk.kv_end;
    a.coff = (int32_t)mk.causal_offset;
    a.window = (int32_t)mk.window;
    a.splits = (int32_t)splits;
    a.split_len = (int32_t)split_len;
    if (out_f32) {
        a.part_o_stride = plan.slices * S_q * D_v;
        a.part_lse_stride = plan.slices * S_q;
    }
    const tsd::TileConfig cfg = tsd::tile_config(dtype, es.D_qk, D_v, true);
    const hipError_t err = tsd::launch_attn_ext(cfg, dtype, causal != 0, out_f32,
                                                plan.grid * splits, a, stream);
    return err == hipSuccess ? TSD_OK : TSD_ERR_HIP;
}

// Split count chosen when the caller passes n_splits <= 0: enough chunks
// that one round of workgroups covers the chip (256 CUs, one workgroup per
// CU for wide heads and three for narrow ones; measured on long-context
// prefill and decoding, more chunks only add merge traffic and re-reads of
// Q), with chunks of at least kMinSplitKeys keys so that the pipeline
// prologue and the merge stay small next to the chunk's own work.
constexpr int64_t kMinSplitKeys = 512;
constexpr int64_t kMaxSplits = 256;

int64_t auto_splits(const tsd_plan &plan, int64_t keys)
{
    const int64_t per_cu = plan.waves == 8 ? 1 : 3;
    const int64_t want = (256 * per_cu + plan.grid - 1) / plan.grid;
    int64_t cap = keys / kMinSplitKeys;
    if (cap < 1) cap = 1;
    if (cap > kMaxSplits) cap = kMaxSplits;
    return want < 1 ? 1 : (want > cap ? cap : want);
}

}  // namespace

extern "C" int attn_fwd_plan(int64_t B, int64_t H, int64_t S_q, int64_t S_k, int64_t D_qk,
                             int64_t D_v, int causal, int dtype, tsd_plan *out)
{
    if (!out) return TSD_ERR_NULL;
    const int st = check_shape(B, H, S_q, S_k, D_qk, D_v, dtype);
    if (st != TSD_OK) return st;
    fill_plan(B, H, S_q, S_k, D_qk, D_v, causal, dtype, vector_dims_ok(dtype, D_qk, D_v), out);
    return TSD_OK;
}

extern "C" int attn_fwd_plan_block(const tsd_plan *plan, int64_t S_q, int64_t S_k,
                                   int64_t block, int64_t *q_block, int64_t *slice,
                                   int64_t *kv_steps)
{
    if (!plan) return TSD_ERR_NULL;
    if (block < 0 || block >= plan->grid) return TSD_ERR_SHAPE;
    int32_t qb = 0, sl = 0;
    const int32_t per_xcd = (int32_t)(plan->slices / 8);
    tsd::map_block((int32_t)block, (int32_t)plan->q_blocks, (int32_t)plan->slices, plan->order,
                   per_xcd, plan->causal != 0, qb, sl);
    if (q_block) *q_block = qb;
    if (slice) *slice = sl;
    if (kv_steps)
        *kv_steps = tsd::kv_tiles_for(qb, plan->block_m, plan->block_n, (int32_t)S_q,
                                      (int32_t)S_k, plan->causal != 0);
    return TSD_OK;
}

extern "C" int attn_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE,
                        int64_t B, int64_t H, int64_t S_q, int64_t S_k, int64_t D_qk,
                        int64_t D_v, float scale, int causal, int dtype, void *stream)
{
    if (!Q || !K || !V || !O) return TSD_ERR_NULL;
    int st = check_shape(B, H, S_q, S_k, D_qk, D_v, dtype);
    if (st != TSD_OK) return st;
    if (!std::isfinite(scale)) return TSD_ERR_SCALE;

    const uint64_t elt = (uint64_t)elt_bytes(dtype);
    const uint64_t BH = (uint64_t)B * (uint64_t)H;
    const uint64_t q_bytes = BH * S_q * D_qk * elt;
    const uint64_t k_bytes = BH * S_k * D_qk * elt;
    const uint64_t v_bytes = BH * S_k * D_v * elt;
    const uint64_t o_bytes = BH * S_q * D_v * elt;
    const uint64_t l_bytes = LSE ? BH * S_q * sizeof(float) : 0;

    // Element alignment is required; 16-byte alignment enables vector I/O.
    const uintptr_t ptrs[4] = {(uintptr_t)Q, (uintptr_t)K, (uintptr_t)V, (uintptr_t)O};
    bool aligned16 = ((uintptr_t)LSE % 4) == 0;
    if (!aligned16) return TSD_ERR_UNSUPPORTED;
    for (uintptr_t p : ptrs) {
        if (p % elt != 0) return TSD_ERR_UNSUPPORTED;
        if (p % 16 != 0) aligned16 = false;
    }

    if (overlap(O, o_bytes, Q, q_bytes) || overlap(O, o_bytes, K, k_bytes) ||
        overlap(O, o_bytes, V, v_bytes) || overlap(LSE, l_bytes, Q, q_bytes) ||
        overlap(LSE, l_bytes, K, k_bytes) || overlap(LSE, l_bytes, V, v_bytes) ||
        overlap(LSE, l_bytes, O, o_bytes))
        return TSD_ERR_ALIAS;

    tsd_plan plan;
    const bool vec = aligned16 && vector_dims_ok(dtype, D_qk, D_v);
    fill_plan(B, H, S_q, S_k, D_qk, D_v, causal, dtype, vec, &plan);
    const tsd::KernelArgs a =
        base_args(Q, K, V, O, LSE, S_q, S_k, D_qk, D_v, scale, dtype, vec, plan);

    const tsd::TileConfig cfg = tsd::tile_config(dtype, D_qk, D_v, vec, B * H, S_q);
    hipError_t err = tsd::launch_attn(cfg, dtype, causal != 0, plan.grid, a,
                                      reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? TSD_OK : TSD_ERR_HIP;
}

extern "C" int attn_fwd_ext(const void *Q, const void *K, const void *V, void *O, float *LSE,
                            int64_t B, int64_t H, int64_t H_kv, int64_t S_q, int64_t S_k,
                            int64_t D_qk, int64_t D_v, float scale, int causal, int dtype,
                            const tsd_mask *mask, void *stream)
{
    const ExtShape es{B, H, H_kv, S_q, S_k, D_qk, D_v};
    int st = check_ext_inputs(Q, K, V, es, scale, dtype);
    if (st != TSD_OK) return st;
    if (!O) return TSD_ERR_NULL;
    tsd_mask mk;
    if ((st = check_mask(mask, S_k, &mk)) != TSD_OK) return st;
    if ((uintptr_t)O % 16 != 0 || (uintptr_t)LSE % 4 != 0) return TSD_ERR_UNSUPPORTED;
    const InputBytes ib = input_bytes(es, dtype);
    const uint64_t rows = (uint64_t)B * H * S_q;
    const uint64_t o_bytes = rows * D_v * 2, l_bytes = LSE ? rows * 4 : 0;
    if (overlaps_inputs(O, o_bytes, Q, K, V, ib) || overlaps_inputs(LSE, l_bytes, Q, K, V, ib) ||
        overlap(LSE, l_bytes, O, o_bytes))
        return TSD_ERR_ALIAS;
    return launch_ext(Q, K, V, O, LSE, es, scale, causal, dtype, mk, 1,
                      mk.kv_end - mk.kv_begin, false, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int attn_fwd_partial(const void *Q, const void *K, const void *V, float *O_parts,
                                float *LSE_parts, int64_t B, int64_t H, int64_t H_kv,
                                int64_t S_q, int64_t S_k, int64_t D_qk, int64_t D_v,
                                float scale, int causal, int dtype, const tsd_mask *mask,
                                int64_t n_splits, int64_t split_len, void *stream)
{
    const ExtShape es{B, H, H_kv, S_q, S_k, D_qk, D_v};
    int st = check_ext_inputs(Q, K, V, es, scale, dtype);
    if (st != TSD_OK) return st;
    if (!O_parts || !LSE_parts) return TSD_ERR_NULL;
    tsd_mask mk;
    if ((st = check_mask(mask, S_k, &mk)) != TSD_OK) return st;
    if (n_splits < 1 || split_len < 1) return TSD_ERR_SHAPE;
    // chunk bounds kv_begin + s * split_len stay inside int32
    if (split_len > INT32_MAX || n_splits > (INT32_MAX - mk.kv_begin) / split_len)
        return TSD_ERR_UNSUPPORTED;
    if (es.rows() > kMaxSliceBytes / (D_v * 4)) return TSD_ERR_UNSUPPORTED;   // f32 slice of O
    if ((uintptr_t)O_parts % 16 != 0 || (uintptr_t)LSE_parts % 4 != 0)
        return TSD_ERR_UNSUPPORTED;
    const InputBytes ib = input_bytes(es, dtype);
    const uint64_t rows = (uint64_t)B * H * S_q;
    const uint64_t o_bytes = (uint64_t)n_splits * rows * D_v * 4;
    const uint64_t l_bytes = (uint64_t)n_splits * rows * 4;
    if (overlaps_inputs(O_parts, o_bytes, Q, K, V, ib) ||
        overlaps_inputs(LSE_parts, l_bytes, Q, K, V, ib) ||
        overlap(LSE_parts, l_bytes, O_parts, o_bytes))
        return TSD_ERR_ALIAS;
    return launch_ext(Q, K, V, O_parts, LSE_parts, es, scale, causal, dtype, mk, n_splits,
                      split_len, true, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int attn_merge(const float *O_parts, const float *LSE_parts, int64_t n_parts,
                          int64_t B, int64_t H, int64_t S_q, int64_t D_v, void *O, float *LSE,
                          int dtype, void *stream)
{
    if (!O_parts || !LSE_parts || !O) return TSD_ERR_NULL;
    if (n_parts < 1 || B < 1 || H < 1 || S_q < 1 || D_v < 1) return TSD_ERR_SHAPE;
    const int elt = elt_bytes(dtype);
    if (elt == 0 || D_v > kMaxHeadDim || n_parts > INT32_MAX) return TSD_ERR_UNSUPPORTED;
    if (B > INT32_MAX / H || B * H > (INT64_MAX / 1024) / S_q) return TSD_ERR_UNSUPPORTED;
    const int64_t rows = B * H * S_q;
    if (n_parts > (INT64_MAX / 1024) / rows) return TSD_ERR_UNSUPPORTED;
    const int64_t groups = (D_v + 3) / 4;
    if ((rows * groups + 255) / 256 > INT32_MAX) return TSD_ERR_UNSUPPORTED;
    if ((uintptr_t)O_parts % 4 != 0 || (uintptr_t)LSE_parts % 4 != 0 ||
        (uintptr_t)O % elt != 0 || (uintptr_t)LSE % 4 != 0)
        return TSD_ERR_UNSUPPORTED;
    const uint64_t po = (uint64_t)n_parts * rows * D_v * 4, pl = (uint64_t)n_parts * rows * 4;
    const uint64_t o_bytes = (uint64_t)rows * D_v * elt, l_bytes = LSE ? (uint64_t)rows * 4 : 0;
    if (overlap(O, o_bytes, O_parts, po) || overlap(O, o_bytes, LSE_parts, pl) ||
        overlap(LSE, l_bytes, O_parts, po) || overlap(LSE, l_bytes, LSE_parts, pl) ||
        overlap(LSE, l_bytes, O, o_bytes))
        return TSD_ERR_ALIAS;
    tsd::MergeArgs a;
    a.O_parts = O_parts;
    a.LSE_parts = LSE_parts;
    a.O = O;
    a.LSE = LSE;
    a.rows = rows;
    a.part_o_stride = rows * D_v;
    a.part_lse_stride = rows;
    a.D_v = (int32_t)D_v;
    a.n_parts = (int32_t)n_parts;
    a.groups = (int32_t)groups;
    const bool vec = D_v % 4 == 0 && (uintptr_t)O_parts % 16 == 0 &&
                     (uintptr_t)O % (4 * elt) == 0;
    const hipError_t err =
        tsd::launch_merge(dtype, vec, a, reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? TSD_OK : TSD_ERR_HIP;
}

namespace {

// Workspace layout of attn_fwd_splitkv: the f32 partial O of every chunk,
// then (at a 256-byte boundary) the partial LSE.
int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

int splitkv_plan(const ExtShape &es, int causal, int dtype, const tsd_mask &mk,
                 int64_t n_splits, int64_t *splits_out, int64_t *split_len_out, int64_t *ws_out)
{
    tsd_plan plan;
    fill_plan(es.B, es.H_kv, es.rows(), es.S_k, es.D_qk, es.D_v, causal, dtype, true, &plan);
    const int64_t keys = mk.kv_end - mk.kv_begin;
    int64_t n = n_splits > 0 ? n_splits : auto_splits(plan, keys);
    if (n > kMaxSplits) return TSD_ERR_UNSUPPORTED;
    // chunks of whole key tiles; no chunk past the range
    int64_t len = keys > 0 ? (keys + n - 1) / n : 64;
    len = (len + 63) / 64 * 64;
    if (keys > 0) n = (keys + len - 1) / len;
    if (n > (INT32_MAX - mk.kv_begin) / len) return TSD_ERR_UNSUPPORTED;
    if (n > 1 && es.rows() > kMaxSliceBytes / (es.D_v * 4)) return TSD_ERR_UNSUPPORTED;
    const int64_t rows = es.B * es.H * es.S_q;
    *splits_out = n;
    *split_len_out = len;
    *ws_out = n > 1 ? round256(n * rows * es.D_v * 4) + round256(n * rows * 4) : 0;
    return TSD_OK;
}

}  // namespace

extern "C" int attn_splitkv_plan(int64_t B, int64_t H, int64_t H_kv, int64_t S_q, int64_t S_k,
                                 int64_t D_qk, int64_t D_v, int causal, int dtype,
                                 const tsd_mask *mask, int64_t n_splits, int64_t *splits_out,
                                 int64_t *split_len_out, int64_t *workspace_bytes)
{
    if (!splits_out || !split_len_out || !workspace_bytes) return TSD_ERR_NULL;
    const ExtShape es{B, H, H_kv, S_q, S_k, D_qk, D_v};
    if (B < 1 || H < 1 || H_kv < 1 || S_q < 1 || H % H_kv != 0) return TSD_ERR_SHAPE;
    if (es.S_q > INT32_MAX / es.group()) return TSD_ERR_UNSUPPORTED;   // rows() fits int32
    int st = check_shape(B, H_kv, es.rows(), S_k, D_qk, D_v, dtype);
    if (st != TSD_OK) return st;
    if (dtype == TSD_F32 || !vector_dims_ok(dtype, D_qk, D_v)) return TSD_ERR_UNSUPPORTED;
    tsd_mask mk;
    if ((st = check_mask(mask, S_k, &mk)) != TSD_OK) return st;
    return splitkv_plan(es, causal, dtype, mk, n_splits, splits_out, split_len_out,
                        workspace_bytes);
}

extern "C" int attn_fwd_splitkv(const void *Q, const void *K, const void *V, void *O,
                                float *LSE, int64_t B, int64_t H, int64_t H_kv, int64_t S_q,
                                int64_t S_k, int64_t D_qk, int64_t D_v, float scale,
                                int causal, int dtype, const tsd_mask *mask, int64_t n_splits,
                                void *workspace, int64_t workspace_bytes, void *stream)
{
    const ExtShape es{B, H, H_kv, S_q, S_k, D_qk, D_v};
    int st = check_ext_inputs(Q, K, V, es, scale, dtype);
    if (st != TSD_OK) return st;
    if (!O) return TSD_ERR_NULL;
    tsd_mask mk;
    if ((st = check_mask(mask, S_k, &mk)) != TSD_OK) return st;
    int64_t n = 0, len = 0, ws = 0;
    if ((st = splitkv_plan(es, causal, dtype, mk, n_splits, &n, &len, &ws)) != TSD_OK)
        return st;
    if (n == 1)
        return attn_fwd_ext(Q, K, V, O, LSE, B, H, H_kv, S_q, S_k, D_qk, D_v, scale, causal,
                            dtype, &mk, stream);
    if (!workspace) return TSD_ERR_NULL;
    if (workspace_bytes < ws) return TSD_ERR_SHAPE;
    if ((uintptr_t)workspace % 256 != 0) return TSD_ERR_UNSUPPORTED;
    if ((uintptr_t)O % 16 != 0 || (uintptr_t)LSE % 4 != 0) return TSD_ERR_UNSUPPORTED;
    const InputBytes ib = input_bytes(es, dtype);
    const uint64_t rows = (uint64_t)B * H * S_q;
    const uint64_t o_bytes = rows * D_v * 2, l_bytes = LSE ? rows * 4 : 0;
    if (overlaps_inputs(O, o_bytes, Q, K, V, ib) || overlaps_inputs(LSE, l_bytes, Q, K, V, ib) ||
        overlap(LSE, l_bytes, O, o_bytes) || overlaps_inputs(workspace, ws, Q, K, V, ib) ||
        overlap(workspace, ws, O, o_bytes) || overlap(workspace, ws, LSE, l_bytes))
        return TSD_ERR_ALIAS;
    float *o_parts = static_cast<float *>(workspace);
    float *l_parts = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) +
                                               round256((int64_t)(n * rows * D_v * 4)));
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    st = launch_ext(Q, K, V, o_parts, l_parts, es, scale, causal, dtype, mk, n, len, true, s);
    if (st != TSD_OK) return st;
    return attn_merge(o_parts, l_parts, n, B, H, S_q, D_v, O, LSE, dtype, stream);
}

// ------------------------------------------------------------------------
// attn_fwd_splitkv_noalloc: the split-KV path with its partial results in a
// fixed device array instead of a caller workspace.  The array is a
// file-scope __device__ object: the loader places one copy on every device
// the library runs on, each held until the process ends.  In host code its
// name stands for a host-side shadow, not a device address, so the device
// address of the current device's copy is looked up once per device with
// hipGetSymbolAddress and only that address is handed to kernels.
namespace {

__device__ __align__(256) uint8_t scratch[TSD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// Device address of the current device's scratch array.  The kernels run
// on the device of `stream`: a stream of another device would get an
// address it cannot use, so that is refused.
int scratch_address(hipStream_t stream, void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return TSD_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return TSD_ERR_UNSUPPORTED;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return TSD_ERR_HIP;
        if ((int)sdev != dev) return TSD_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TSD_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return TSD_OK;
}

}  // namespace

extern "C" int attn_fwd_splitkv_noalloc(const void *Q, const void *K, const void *V, void *O,
                                        float *LSE, int64_t B, int64_t H, int64_t H_kv,
                                        int64_t S_q, int64_t S_k, int64_t D_qk, int64_t D_v,
                                        float scale, int causal, int dtype,
                                        const tsd_mask *mask, int64_t n_splits, void *stream)
{
    const ExtShape es{B, H, H_kv, S_q, S_k, D_qk, D_v};
    int st = check_ext_inputs(Q, K, V, es, scale, dtype);
    if (st != TSD_OK) return st;
    if (!O) return TSD_ERR_NULL;
    tsd_mask mk;
    if ((st = check_mask(mask, S_k, &mk)) != TSD_OK) return st;
    int64_t n = 0, len = 0, ws = 0;
    if ((st = splitkv_plan(es, causal, dtype, mk, n_splits, &n, &len, &ws)) != TSD_OK)
        return st;
    if (n == 1)   // one chunk: no partial results, nothing staged
        return attn_fwd_ext(Q, K, V, O, LSE, B, H, H_kv, S_q, S_k, D_qk, D_v, scale, causal,
                            dtype, &mk, stream);
    if (ws > TSD_NOALLOC_SCRATCH_BYTES) return TSD_ERR_SCRATCH;
    if ((uintptr_t)O % 16 != 0 || (uintptr_t)LSE % 4 != 0) return TSD_ERR_UNSUPPORTED;
    void *work = nullptr;
    if ((st = scratch_address(reinterpret_cast<hipStream_t>(stream), &work)) != TSD_OK)
        return st;
    // The same chunking, so attn_fwd_splitkv takes the same plan and checks
    // the outputs against the scratch array like any workspace.  Every
    // partial entry is written before the merge reads it (chunks a row sees
    // nothing of get O = 0, LSE = -inf), so nothing left from an earlier
    // call is read.
    return attn_fwd_splitkv(Q, K, V, O, LSE, B, H, H_kv, S_q, S_k, D_qk, D_v, scale, causal,
                            dtype, &mk, n, work, TSD_NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" int attn_fwd_scaled(const void *Q, const void *K, const void *V, void *O, float *LSE,
                               const float *Q_scale, const float *K_scale, int64_t B,
                               int64_t H, int64_t S_q, int64_t S_k, int64_t D_qk, int64_t D_v,
                               int64_t q_block, int64_t k_block, int causal, int qk_dtype,
                               int dtype, void *stream)
{
    if (!Q || !K || !V || !O || !Q_scale || !K_scale) return TSD_ERR_NULL;
    if (B < 1 || H < 1 || S_q < 1 || S_k < 1 || D_qk < 1 || D_v < 1 || q_block < 1 ||
        k_block < 1)
        return TSD_ERR_SHAPE;
    if (dtype != TSD_BF16 && dtype != TSD_F16) return TSD_ERR_UNSUPPORTED;
    const bool qk8 = qk_dtype == TSD_FP8_E4M3;
    if (!qk8 && qk_dtype != dtype) return TSD_ERR_UNSUPPORTED;
    // V/O sizes and the grid as for attn_fwd; Q/K at their own element size
    int st = check_shape(B, H, S_q, S_k, D_qk, D_v, dtype);
    if (st != TSD_OK) return st;
    const int64_t qkb = qk8 ? 1 : 2;
    if (k_block % 64 != 0 || k_block > INT32_MAX || q_block > INT32_MAX)
        return TSD_ERR_UNSUPPORTED;
    if (D_v % 8 != 0 || D_qk % (16 / qkb) != 0) return TSD_ERR_UNSUPPORTED;
    const tsd::TileConfig cfg = tsd::tile_config(dtype, D_qk, D_v, true);
    if (qk8 && !(cfg.dqk_block == 128 || (cfg.dqk_block == 64 && cfg.dv_block == 64)))
        return TSD_ERR_UNSUPPORTED;
    for (uintptr_t p : {(uintptr_t)Q, (uintptr_t)K, (uintptr_t)V, (uintptr_t)O})
        if (p % 16 != 0) return TSD_ERR_UNSUPPORTED;
    if ((uintptr_t)LSE % 4 != 0 || (uintptr_t)Q_scale % 4 != 0 || (uintptr_t)K_scale % 4 != 0)
        return TSD_ERR_UNSUPPORTED;

    const uint64_t BH = (uint64_t)B * H;
    const int64_t nqb = (S_q + q_block - 1) / q_block, nkb = (S_k + k_block - 1) / k_block;
    const uint64_t q_bytes = BH * S_q * D_qk * qkb, k_bytes = BH * S_k * D_qk * qkb;
    const uint64_t v_bytes = BH * S_k * D_v * 2, o_bytes = BH * S_q * D_v * 2;
    const uint64_t l_bytes = LSE ? BH * S_q * 4 : 0;
    const uint64_t qs_bytes = BH * nqb * 4, ks_bytes = BH * nkb * 4;
    const void *ins[5] = {Q, K, V, Q_scale, K_scale};
    const uint64_t in_bytes[5] = {q_bytes, k_bytes, v_bytes, qs_bytes, ks_bytes};
    for (int i = 0; i < 5; ++i)
        if (overlap(O, o_bytes, ins[i], in_bytes[i]) || overlap(LSE, l_bytes, ins[i], in_bytes[i]))
            return TSD_ERR_ALIAS;
    if (overlap(LSE, l_bytes, O, o_bytes)) return TSD_ERR_ALIAS;

    tsd_plan plan;
    fill_plan(B, H, S_q, S_k, D_qk, D_v, causal, dtype, true, &plan);
    // the score scale lives in the block scales; Q enters unchanged
    tsd::KernelArgs a = base_args(Q, K, V, O, LSE, S_q, S_k, D_qk, D_v, 1.0f, dtype, true, plan);
    a.Q_scale = Q_scale;
    a.K_scale = K_scale;
    a.q_block = (int32_t)q_block;
    a.q_scale_blocks = (int32_t)nqb;
    a.k_tiles_per_block = (int32_t)(k_block / 64);
    a.k_scale_blocks = (int32_t)nkb;
    const hipError_t err = tsd::launch_attn_scaled(cfg, dtype, causal != 0, qk8, plan.grid, a,
                                                   reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? TSD_OK : TSD_ERR_HIP;
}

extern "C" const char *attn_status_string(int status)
{
    switch (status) {
    case TSD_OK: return "ok";
    case TSD_ERR_NULL: return "null pointer argument";
    case TSD_ERR_SHAPE: return "invalid shape: every dimension must be at least 1";
    case TSD_ERR_UNSUPPORTED:
        return "unsupported: head width above 128, unknown dtype, misaligned pointer, "
               "or size beyond the 32-bit limits";
    case TSD_ERR_SCALE: return "scale is not finite";
    case TSD_ERR_ALIAS: return "output buffer overlaps an input or the other output";
    case TSD_ERR_HIP: return "HIP kernel launch failed";
    case TSD_ERR_SCRATCH:
        return "the partial results need more than the library's fixed scratch array "
               "(TSD_NOALLOC_SCRATCH_BYTES); use attn_fwd_splitkv with a workspace";
    default: return "unknown status";
    }
}
