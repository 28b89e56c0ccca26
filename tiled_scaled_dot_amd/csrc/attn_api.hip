// Host side of the C ABI: argument validation, the launch planner and the
// status strings.  Every check here runs before any HIP call, so an invalid
// call launches nothing and writes nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

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
    const tsd::TileConfig cfg = tsd::tile_config(dtype, D_qk, D_v, vector_io);
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

    const tsd::TileConfig cfg = tsd::tile_config(dtype, D_qk, D_v, vec);
    hipError_t err = tsd::launch_attn(cfg, dtype, causal != 0, plan.grid, a,
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
    default: return "unknown status";
    }
}
