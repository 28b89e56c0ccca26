// gfx950 (CDNA4) kernels for the tiled scaled-dot-product attention forward.
//
// What is computed: O = softmax(Q K^T * scale) V and LSE = ln(sum exp) per
// (batch, head) slice, non-causal or causal, with S_q / S_k boundaries and a
// head-dim tail (VeriTile, "FlashAttention1.NaiveRefinement": the FA-1
// boundary + D-tail kernels refine the naive reference).  Each query row
// runs the reduction chain dot -> max -> shifted exp-sum -> weighted sum
// (tiny.accy.kernel.library.attention, the specialization's reductions),
// online over key tiles: the running max m and sum l are rescaled by
// exp(m_old - m_new) whenever m grows, which in real arithmetic gives the
// plain definition exactly.
//
// Kernels in this file:
//   * attn_fwd_fast16 — the main kernel: 16-bit inputs whose rows are
//     16-byte aligned; plus its extended (key ranges, offsets, windows, key
//     chunks, grouped heads), per-block scaled and fp8-score forms.
//   * attn_fwd_16 / attn_fwd_32 — generic kernels for any alignment and
//     head width (16-bit and f32 inputs), staged through VGPRs.
//   * attn_fwd_32s — f32 on small grids: 32 rows per workgroup, the four
//     waves splitting the key tiles, combined through LDS at the end.
//   * attn_merge_kernel — the merge of partial results over key chunks.
//
// Common work decomposition (one workgroup = one query block of one slice):
//   * Each wave owns 32 query rows and keeps them in VGPRs for the whole
//     key loop (the generic kernels: 4 waves, 128 rows per workgroup).
//   * Key/value tiles are staged through LDS with their global loads in
//     flight while earlier tiles are computed.
//   * Scores are formed transposed, S^T = K Q^T, on MFMA: the 32x32 result
//     puts one query per lane column, so each lane holds 16 keys of a single
//     query and the row max / sum are in-lane plus one swap with lane^32.
//   * The S^T accumulator layout is exactly the B operand layout of the
//     P V MFMA (O^T = V^T P^T), so P never leaves registers.  The A operand
//     needs 8 consecutive keys of one V column per lane: the generic
//     kernels write V to LDS d-major, the main kernel keeps the key-major
//     rows its LDS-direct loads land and reads them with ds_read_b64_tr_b16.
//   * Key rows read for the score MFMA are permuted (sigma below) so that
//     each lane's P values cover 8 consecutive keys, which makes every LDS
//     operand read a single 16-byte access.  Permuting keys is legal: the
//     key index is only summed over.
//   * 16-bit inputs: v_mfma_f32_32x32x16_{bf16,f16}; f32 inputs:
//     v_mfma_f32_32x32x2_f32.  Accumulation is always f32.
//   * exp is computed as exp2 with log2(e) folded into the scale.
#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

#include "launch.h"

// This file is compiled once per unit, each unit instantiating one family
// of kernels so that the units build in parallel: 0 = the plain kernels and
// the merge, 1 = the extended kernels, 2 = the per-block scaled kernels.
#ifndef TSD_UNIT
#define TSD_UNIT 0
#endif

namespace tsd {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;   // 4 waves
constexpr int kBlockM = 128;    // 4 waves x 32 query rows
constexpr float kLn2 = 0.69314718055994531f;

__device__ inline float neg_inf() { return -__builtin_inff(); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Swap-half reduction partner: lane l <-> lane l ^ 32.
__device__ inline float other_half(float x) { return __shfl_xor(x, 32); }

// Cross-half reductions with one v_permlane32_swap (gfx950).  The
// instruction exchanges the upper 32 lanes of its first operand with the
// lower 32 lanes of its second; with both operands = x, every lane l ends up
// holding {x[l], x[l^32]} across the two results (in an order that depends
// on the half), so max / sum of the pair is the reduction over lanes l and
// l^32 on every lane, bitwise identical within the pair.
__device__ inline void swap32(float x, float &a, float &b)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __builtin_bit_cast(float, (uint32_t)r[0]);
    b = __builtin_bit_cast(float, (uint32_t)r[1]);
}
// IEEE maximum (NaN-propagating): lowers to v_maximum3_f32 without the
// canonicalising copies fmaxf needs.
__device__ inline float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ inline float max_halves(float x)
{
    float a, b;
    swap32(x, a, b);
    return fmax_nan(a, b);
}
__device__ inline float sum_halves(float x)
{
    float a, b;
    swap32(x, a, b);
    return a + b;
}

// ---------------------------------------------------------------- MFMA
template <bool BF16>
__device__ inline f32x16 mma16(u32x4 a, u32x4 b, f32x16 c)
{
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// fp8 (e4m3) scores: 32x32 outputs over 64 dims.  Each lane passes two
// 16-byte chunks of its A row and of its B column; A and B share one lane
// layout, so any assignment of dims to chunks that both operands follow
// gives the full dot product.  The block scales of the instruction are left
// at 1 (E8M0 127).
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ inline f32x16 mma8(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x16 c)
{
    const i32x8 a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                     (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const i32x8 b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                     (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ inline f32x16 mma32(float a, float b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Two f32 -> one word of two 16-bit values (round to nearest even).
template <bool BF16>
__device__ inline uint32_t pack2(float lo, float hi)
{
    if constexpr (BF16) {
        bf16x2 v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        f16x2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
}

// ------------------------------------------------------- layout helpers
// MFMA 32x32 accumulator: lane l, register r holds row (r/4)*8 + 4*(l/32) + r%4
// and column l%32.  For the score MFMA the row is a key; sigma maps the MFMA
// row i to the key of the tile read into it so that lane half h, registers
// 8u..8u+7 hold keys 16u + 8h + 0..7.
__device__ inline int sigma(int i)
{
    return (i & 16) | (((i >> 2) & 1) << 3) | (((i >> 3) & 1) << 2) | (i & 3);
}

// XOR swizzle of 16-byte chunks within a row (LDS bank spreading).  For
// ds_read_b128 every group of 8 lanes must hit 8 different 16-byte bank
// groups; the reads here visit rows {sigma(0..7)}, {sigma(8..15)}, ... and
// the transposed-V writes visit rows {e, e+4, ..., e+28}; this XOR makes
// both patterns conflict-free.
__device__ inline int swz(int row)
{
    return (((row & 3) | ((row >> 1) & 4)) ^ ((row >> 2) & 7));
}

// ====================================================================
// 16-bit (bf16 / f16) kernel
// ====================================================================
template <int DQ, int DV>
struct Tile16 {
    static constexpr int BN = 64;                   // keys per tile
    static constexpr int KCH = DQ / 8;              // 16-byte chunks per K row
    static constexpr int VCH = BN / 8;              // 16-byte chunks per V^T row
    static constexpr int K_CHUNKS = BN * KCH;
    static constexpr int V_CHUNKS = DV * VCH;
    static constexpr int STAGE = K_CHUNKS + V_CHUNKS;   // chunks per LDS stage
    static constexpr int K_PER_T = K_CHUNKS / kThreads; // K chunks loaded per thread
    static constexpr int V_UNITS = (BN / 8) * (DV / 4); // (8 keys x 4 dims) units
    static constexpr int V_PER_T = (V_UNITS + kThreads - 1) / kThreads;
    static_assert(K_CHUNKS % kThreads == 0, "K tile must split evenly");
};

template <int DQ, int DV>
struct Regs16 {
    u32x4 k[Tile16<DQ, DV>::K_PER_T];
    u32x2 v[Tile16<DQ, DV>::V_PER_T][8];
};

template <int DQ, int DV>
__device__ inline void load_tile16(Regs16<DQ, DV> &r, const uint16_t *__restrict__ Ks,
                                   const uint16_t *__restrict__ Vs, int kbase,
                                   const KernelArgs &p, int tid)
{
    using T = Tile16<DQ, DV>;
#pragma unroll
    for (int it = 0; it < T::K_PER_T; ++it) {
        const int ci = tid + kThreads * it;
        const int row = ci / T::KCH, c = ci % T::KCH;
        const int key = kbase + row;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (p.vec) {
            if (key < p.S_k && c * 8 < p.D_qk)
                x = *reinterpret_cast<const u32x4 *>(Ks + (size_t)key * p.D_qk + c * 8);
        } else if (key < p.S_k) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int d = c * 8 + 2 * e;
                const uint32_t lo = d < p.D_qk ? Ks[(size_t)key * p.D_qk + d] : 0u;
                const uint32_t hi = d + 1 < p.D_qk ? Ks[(size_t)key * p.D_qk + d + 1] : 0u;
                w[e] = lo | (hi << 16);
            }
            x = u32x4{w[0], w[1], w[2], w[3]};
        }
        r.k[it] = x;
    }
#pragma unroll
    for (int it = 0; it < T::V_PER_T; ++it) {
        const int u = tid + kThreads * it;
        const int kg = u / (DV / 4), dq = u % (DV / 4);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int key = kbase + kg * 8 + j;
            const int d0 = dq * 4;
            u32x2 x = {0u, 0u};
            if (u < T::V_UNITS && key < p.S_k) {
                if (p.vec) {
                    if (d0 < p.D_v)
                        x = *reinterpret_cast<const u32x2 *>(Vs + (size_t)key * p.D_v + d0);
                } else {
                    uint32_t e4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        e4[e] = d0 + e < p.D_v ? Vs[(size_t)key * p.D_v + d0 + e] : 0u;
                    x = u32x2{e4[0] | (e4[1] << 16), e4[2] | (e4[3] << 16)};
                }
            }
            r.v[it][j] = x;
        }
    }
}

template <int DQ, int DV>
__device__ inline void store_tile16(const Regs16<DQ, DV> &r, u32x4 *__restrict__ stage, int tid)
{
    using T = Tile16<DQ, DV>;
#pragma unroll
    for (int it = 0; it < T::K_PER_T; ++it) {
        const int ci = tid + kThreads * it;
        const int row = ci / T::KCH, c = ci % T::KCH;
        stage[row * T::KCH + (c ^ swz(row))] = r.k[it];
    }
    u32x4 *vt = stage + T::K_CHUNKS;
#pragma unroll
    for (int it = 0; it < T::V_PER_T; ++it) {
        const int u = tid + kThreads * it;
        if (u < T::V_UNITS) {
            const int kg = u / (DV / 4), dq = u % (DV / 4);
            // r.v[it][j] holds dims 4dq..4dq+3 of key 8kg+j; V^T row 4dq+e
            // takes element e of each of the 8 keys.
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t w[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const uint32_t a = (e < 2) ? r.v[it][2 * m].x : r.v[it][2 * m].y;
                    const uint32_t b = (e < 2) ? r.v[it][2 * m + 1].x : r.v[it][2 * m + 1].y;
                    w[m] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u))
                                   : ((a & 0xffffu) | (b << 16));
                }
                const int d = dq * 4 + e;
                vt[d * T::VCH + (kg ^ swz(d))] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
    }
}

template <int DQ, int DV, bool CAUSAL, bool BF16>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(2, 2)))
attn_fwd_16(KernelArgs p)
{
    using T = Tile16<DQ, DV>;
    constexpr int BN = T::BN;
    __shared__ u32x4 lds[2 * T::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, l32 = lane & 31;

    int32_t qb, slice;
    map_block((int32_t)blockIdx.x, p.q_blocks, p.slices, p.order, p.per_xcd, CAUSAL, qb, slice);
    const int q0 = qb * kBlockM;
    const int qi = q0 + wave * 32 + l32;   // this lane's query row

    const uint16_t *Qs = static_cast<const uint16_t *>(p.Q) + (size_t)slice * p.S_q * p.D_qk;
    const uint16_t *Ks = static_cast<const uint16_t *>(p.K) + (size_t)slice * p.S_k * p.D_qk;
    const uint16_t *Vs = static_cast<const uint16_t *>(p.V) + (size_t)slice * p.S_k * p.D_v;

    // Q fragment: B operand of S^T = K Q^T.  Lane (l32, hh) holds query qi,
    // dims 16*st + 8*hh + 0..7 for step st.
    u32x4 qf[DQ / 16];
#pragma unroll
    for (int st = 0; st < DQ / 16; ++st) {
        const int d0 = st * 16 + hh * 8;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (qi < p.S_q) {
            if (p.vec) {
                if (d0 < p.D_qk)
                    x = *reinterpret_cast<const u32x4 *>(Qs + (size_t)qi * p.D_qk + d0);
            } else {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int d = d0 + 2 * e;
                    const uint32_t lo = d < p.D_qk ? Qs[(size_t)qi * p.D_qk + d] : 0u;
                    const uint32_t hi = d + 1 < p.D_qk ? Qs[(size_t)qi * p.D_qk + d + 1] : 0u;
                    w[e] = lo | (hi << 16);
                }
                x = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
        x = (x ^ p.q_xor) & p.q_and;
        // padded dims must stay exactly zero after the sign flip
        if (d0 >= p.D_qk) x = u32x4{0u, 0u, 0u, 0u};
        qf[st] = x;
    }

    const int ntiles = kv_tiles_for(qb, kBlockM, BN, p.S_q, p.S_k, CAUSAL);
    const float c = p.c;

    f32x16 o[DV / 32];
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) o[d] = f32x16{};
    float m = neg_inf();   // running max of the raw scores of this query
    float l = 0.0f;        // running sum of this lane's half of the keys

    Regs16<DQ, DV> rg;
    load_tile16<DQ, DV>(rg, Ks, Vs, 0, p, tid);
    store_tile16<DQ, DV>(rg, lds, tid);
    __syncthreads();

    const int krow0 = sigma(l32);   // key row (within a 32-key block) for this lane
    const int vrow0 = sigma(l32);   // V^T row (dim within a 32-dim block)

    for (int t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) load_tile16<DQ, DV>(rg, Ks, Vs, (t + 1) * BN, p, tid);

        const u32x4 *Kl = lds + (t & 1) * T::STAGE;
        const u32x4 *Vl = Kl + T::K_CHUNKS;
        const int kbase = t * BN;

        // ---- scores S^T (two 32-key blocks)
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x16{};
            const int row = kb * 32 + krow0;
#pragma unroll
            for (int st = 0; st < DQ / 16; ++st) {
                const u32x4 a = Kl[row * T::KCH + ((2 * st + hh) ^ swz(row))];
                s[kb] = mma16<BF16>(a, qf[st], s[kb]);
            }
        }

        // ---- masks: keys beyond S_k, and keys after the query when causal
        const bool need_mask = (kbase + BN > p.S_k) || (CAUSAL && kbase + BN - 1 > q0);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kbase + kb * 32 + (r >> 3) * 16 + hh * 8 + (r & 7);
                    bool ok = key < p.S_k;
                    if (CAUSAL) ok = ok && key <= qi;
                    s[kb][r] = ok ? s[kb][r] : neg_inf();
                }
        }

        // ---- running max (in-lane over 32 keys, then with the other half)
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = fmaxf(mx, other_half(mx));
        const float m_new = fmaxf(m, mx);
        const float alpha = fast_exp2((m - m_new) * c);
        const float mc = m_new * c;
        m = m_new;

        // ---- P = exp(s - m), row sum, pack to 16-bit B operands
        u32x4 pf[2][2];
        float rs = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                uint32_t w[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p0 = fast_exp2(__builtin_fmaf(s[kb][8 * u + 2 * j], c, -mc));
                    const float p1 = fast_exp2(__builtin_fmaf(s[kb][8 * u + 2 * j + 1], c, -mc));
                    rs += p0 + p1;
                    w[j] = pack2<BF16>(p0, p1);
                }
                pf[kb][u] = u32x4{w[0], w[1], w[2], w[3]};
            }
        l = l * alpha + rs;
#pragma unroll
        for (int d = 0; d < DV / 32; ++d) o[d] *= alpha;

        // ---- O^T += V^T P^T
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int d = 0; d < DV / 32; ++d) {
                    const int row = d * 32 + vrow0;
                    const u32x4 a = Vl[row * T::VCH + ((kb * 4 + u * 2 + hh) ^ swz(row))];
                    o[d] = mma16<BF16>(a, pf[kb][u], o[d]);
                }

        if (t + 1 < ntiles) store_tile16<DQ, DV>(rg, lds + ((t + 1) & 1) * T::STAGE, tid);
        __syncthreads();
    }

    // ---- epilogue: O = O_acc / l, LSE = m*scale + ln(l)
    const float lt = l + other_half(l);
    const float inv = 1.0f / lt;
    if (qi < p.S_q) {
        uint16_t *Os = static_cast<uint16_t *>(p.O) + ((size_t)slice * p.S_q + qi) * p.D_v;
#pragma unroll
        for (int d = 0; d < DV / 32; ++d)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int d0 = d * 32 + u * 16 + hh * 8;   // 8 consecutive dims
                uint32_t w[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    w[j] = pack2<BF16>(o[d][8 * u + 2 * j] * inv, o[d][8 * u + 2 * j + 1] * inv);
                if (p.vec) {
                    if (d0 < p.D_v) *reinterpret_cast<u32x4 *>(Os + d0) = u32x4{w[0], w[1], w[2], w[3]};
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (d0 + j < p.D_v) Os[d0 + j] = (uint16_t)(w[j >> 1] >> ((j & 1) * 16));
                }
            }
        if (p.LSE && hh == 0)
            p.LSE[(size_t)slice * p.S_q + qi] = (m * c + __builtin_amdgcn_logf(lt)) * kLn2;
    }
}

// ====================================================================
// f32 kernel (v_mfma_f32_32x32x2_f32)
// ====================================================================
template <int DQ, int DV>
struct Tile32 {
    static constexpr int BN = 32;
    static constexpr int KCH = DQ / 4;   // 16-byte chunks per K row
    static constexpr int VCH = DV / 4;   // 16-byte chunks per V row
    static constexpr int K_CHUNKS = BN * KCH;
    static constexpr int V_CHUNKS = BN * VCH;
    static constexpr int STAGE = K_CHUNKS + V_CHUNKS;
    static constexpr int K_PER_T = K_CHUNKS / kThreads;
    static constexpr int V_PER_T = V_CHUNKS / kThreads;
    static_assert(K_CHUNKS % kThreads == 0 && V_CHUNKS % kThreads == 0, "tile split");
};

template <int DQ, int DV>
struct Regs32 {
    u32x4 k[Tile32<DQ, DV>::K_PER_T];
    u32x4 v[Tile32<DQ, DV>::V_PER_T];
};

__device__ inline u32x4 load_f32x4(const float *__restrict__ base, int row, int nrows, int col,
                                   int ncols, int vec)
{
    u32x4 x = {0u, 0u, 0u, 0u};
    if (row < nrows) {
        if (vec) {
            if (col < ncols)
                x = *reinterpret_cast<const u32x4 *>(base + (size_t)row * ncols + col);
        } else {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = col + e < ncols
                           ? __builtin_bit_cast(uint32_t, base[(size_t)row * ncols + col + e])
                           : 0u;
            x = u32x4{w[0], w[1], w[2], w[3]};
        }
    }
    return x;
}

template <int DQ, int DV>
__device__ inline void load_tile32(Regs32<DQ, DV> &r, const float *__restrict__ Ks,
                                   const float *__restrict__ Vs, int kbase, const KernelArgs &p,
                                   int tid)
{
    using T = Tile32<DQ, DV>;
#pragma unroll
    for (int it = 0; it < T::K_PER_T; ++it) {
        const int ci = tid + kThreads * it;
        r.k[it] = load_f32x4(Ks, kbase + ci / T::KCH, p.S_k, (ci % T::KCH) * 4, p.D_qk, p.vec);
    }
#pragma unroll
    for (int it = 0; it < T::V_PER_T; ++it) {
        const int ci = tid + kThreads * it;
        r.v[it] = load_f32x4(Vs, kbase + ci / T::VCH, p.S_k, (ci % T::VCH) * 4, p.D_v, p.vec);
    }
}

template <int DQ, int DV>
__device__ inline void store_tile32(const Regs32<DQ, DV> &r, u32x4 *__restrict__ stage, int tid)
{
    using T = Tile32<DQ, DV>;
#pragma unroll
    for (int it = 0; it < T::K_PER_T; ++it) {
        const int ci = tid + kThreads * it;
        const int row = ci / T::KCH, c = ci % T::KCH;
        stage[row * T::KCH + (c ^ (row & 7))] = r.k[it];
    }
#pragma unroll
    for (int it = 0; it < T::V_PER_T; ++it) {
        const int ci = tid + kThreads * it;
        stage[T::K_CHUNKS + ci] = r.v[it];
    }
}

template <int DQ, int DV, bool CAUSAL>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(2, 2)))
attn_fwd_32(KernelArgs p)
{
    using T = Tile32<DQ, DV>;
    constexpr int BN = T::BN;
    __shared__ u32x4 lds[2 * T::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, l32 = lane & 31;

    int32_t qb, slice;
    map_block((int32_t)blockIdx.x, p.q_blocks, p.slices, p.order, p.per_xcd, CAUSAL, qb, slice);
    const int q0 = qb * kBlockM;
    const int qi = q0 + wave * 32 + l32;

    const float *Qs = static_cast<const float *>(p.Q) + (size_t)slice * p.S_q * p.D_qk;
    const float *Ks = static_cast<const float *>(p.K) + (size_t)slice * p.S_k * p.D_qk;
    const float *Vs = static_cast<const float *>(p.V) + (size_t)slice * p.S_k * p.D_v;

    // Q fragment: step 4u+j of the k=2 MFMA uses dim 8u + 4hh + j.
    float qf[DQ / 2];
#pragma unroll
    for (int u = 0; u < DQ / 8; ++u) {
        u32x4 x = load_f32x4(Qs, qi, p.S_q, u * 8 + hh * 4, p.D_qk, p.vec);
        x = (x ^ p.q_xor) & p.q_and;
        // Bit-cast the whole vector: hipcc mis-compiles a bit_cast of a single
        // ext-vector element (it reads element 0 for every index).
        const f32x4 xf = __builtin_bit_cast(f32x4, x);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            qf[4 * u + j] = (u * 8 + hh * 4 + j < p.D_qk) ? xf[j] : 0.0f;
    }

    const int ntiles = kv_tiles_for(qb, kBlockM, BN, p.S_q, p.S_k, CAUSAL);
    const float c = p.c;

    f32x16 o[DV / 32];
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) o[d] = f32x16{};
    float m = neg_inf();
    float l = 0.0f;

    Regs32<DQ, DV> rg;
    load_tile32<DQ, DV>(rg, Ks, Vs, 0, p, tid);
    store_tile32<DQ, DV>(rg, lds, tid);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) load_tile32<DQ, DV>(rg, Ks, Vs, (t + 1) * BN, p, tid);

        const u32x4 *Kl = lds + (t & 1) * T::STAGE;
        const float *Vl = reinterpret_cast<const float *>(Kl + T::K_CHUNKS);
        const int kbase = t * BN;

        // ---- S^T: lane (l32, hh) gets keys (r/4)*8 + 4hh + r%4 of query qi
        f32x16 s = f32x16{};
#pragma unroll
        for (int u = 0; u < DQ / 8; ++u) {
            const f32x4 a = __builtin_bit_cast(f32x4, Kl[l32 * T::KCH + ((2 * u + hh) ^ (l32 & 7))]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                s = mma32(a[j], qf[4 * u + j], s);
        }

        const bool need_mask = (kbase + BN > p.S_k) || (CAUSAL && kbase + BN - 1 > q0);
        if (need_mask) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kbase + (r >> 2) * 8 + hh * 4 + (r & 3);
                bool ok = key < p.S_k;
                if (CAUSAL) ok = ok && key <= qi;
                s[r] = ok ? s[r] : neg_inf();
            }
        }

        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = fmaxf(mx, other_half(mx));
        const float m_new = fmaxf(m, mx);
        const float alpha = fast_exp2((m - m_new) * c);
        const float mc = m_new * c;
        m = m_new;

        float pv[16];
        float rs = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            pv[r] = fast_exp2(__builtin_fmaf(s[r], c, -mc));
            rs += pv[r];
        }
        l = l * alpha + rs;
#pragma unroll
        for (int d = 0; d < DV / 32; ++d) o[d] *= alpha;

        // ---- O^T += V^T P^T; step r uses key (r/4)*8 + 4hh + r%4
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = (r >> 2) * 8 + hh * 4 + (r & 3);
#pragma unroll
            for (int d = 0; d < DV / 32; ++d)
                o[d] = mma32(Vl[key * DV + d * 32 + l32], pv[r], o[d]);
        }

        if (t + 1 < ntiles) store_tile32<DQ, DV>(rg, lds + ((t + 1) & 1) * T::STAGE, tid);
        __syncthreads();
    }

    const float lt = l + other_half(l);
    const float inv = 1.0f / lt;
    if (qi < p.S_q) {
        float *Os = static_cast<float *>(p.O) + ((size_t)slice * p.S_q + qi) * p.D_v;
#pragma unroll
        for (int d = 0; d < DV / 32; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = d * 32 + g * 8 + hh * 4;   // 4 consecutive dims
                f32x4 v4 = {o[d][4 * g] * inv, o[d][4 * g + 1] * inv, o[d][4 * g + 2] * inv,
                            o[d][4 * g + 3] * inv};
                if (p.vec) {
                    if (d0 < p.D_v) *reinterpret_cast<f32x4 *>(Os + d0) = v4;
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (d0 + j < p.D_v) Os[d0 + j] = v4[j];
                }
            }
        if (p.LSE && hh == 0)
            p.LSE[(size_t)slice * p.S_q + qi] = (m * c + __builtin_amdgcn_logf(lt)) * kLn2;
    }
}

// ====================================================================
// Fast 16-bit kernel (vector-aligned inputs, D_qk and D_v multiples of 8).
//
//   * 32 query rows per wave; 8 waves (256 rows) per workgroup and one
//     workgroup per CU for 128-wide heads, 4 waves and three workgroups per
//     CU for 64-wide heads (FastShape below).
//   * K and V tiles (64 keys) go HBM -> LDS directly with buffer loads
//     (buffer_load_dwordx4 ... lds): no VGPR staging, no LDS write
//     instructions.  The buffer range is the slice, so key rows >= S_k read
//     as zero; head-dim chunks >= D read as zero through an out-of-range
//     offset.  K and V sit in LDS rings (4 and 2 tiles for 128-wide heads,
//     4 and 4 with the causal mask, which synchronises every second tile):
//     a tile's K is read one iteration before its V, so K is fetched up to
//     KS-1 tiles ahead and V VS-1 tiles ahead.
//   * Each wave instruction fills 1 KB of LDS contiguously (lane i -> bytes
//     16i..16i+15); the swizzle is realised by choosing which global chunk
//     each lane fetches.
//   * V stays row-major in LDS; the A operand of O^T += V^T P^T is read with
//     ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives
//     element i%4 of the 8-byte chunks addressed by lanes i/4, 4+i/4, 8+i/4
//     and 12+i/4, so lanes pointing at 4 consecutive key rows hand every lane
//     4 keys of one head-dim column.
//   * The running max is only moved when some row's max grows by more than
//     2^kTau (wave-uniform decision); in between, P = 2^(s*c - m*c) may reach
//     2^kTau.  O/l is unchanged in real arithmetic, and the rescale of O and
//     l becomes rare.
//   * O and LSE are written with buffer stores; stores outside the slice are
//     dropped by the hardware range check.
// ====================================================================
// Launch shapes of the fast kernel, chosen per head width (measured on
// MI355X): with 128-wide heads a wave needs ~210 VGPRs, so two waves per
// SIMD (8-wave workgroups, one per CU); with 64-wide heads it fits in ~160,
// and three 4-wave workgroups per CU (three waves per SIMD) hide more
// latency.  K and V tiles sit in LDS ring buffers of kslots / vslots tiles;
// the main loop is unrolled by kslots so every ring slot is a compile-time
// offset (vslots divides kslots).
struct FastShape {
    int waves;    // waves per workgroup (rows per workgroup = 32 * waves)
    int kslots;   // K ring size (the unroll factor of the main loop)
    int vslots;   // V ring size
    int occ;      // waves per SIMD the kernel is compiled for
};
constexpr FastShape kShapeWide = {8, 4, 2, 2};
constexpr FastShape kShapeNarrow = {4, 2, 2, 3};
constexpr FastShape fast_shape(int dq, int dv)
{
    return (dq <= 64 && dv <= 64) ? kShapeNarrow : kShapeWide;
}
constexpr float kTau = 8.0f;
constexpr uint32_t kOutOfRange = 0x80000000u;   // above any slice size (< 2^31 bytes)
constexpr int kBufferConfig = 0x00020000;       // raw buffer, 32-bit data format

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int N>
using IC = std::integral_constant<int, N>;

// f(IC<B>{}), f(IC<B+1>{}), ..., f(IC<E-1>{})
template <int B, int E, typename F>
__host__ __device__ __attribute__((always_inline)) inline void static_for(F &&f)
{
    if constexpr (B < E) {
        f(IC<B>{});
        static_for<B + 1, E>(f);
    }
}

// Instruction interleaving of one main-loop iteration.  A wave issues in
// order, so the compiler's default order (a run of score MFMAs separated by
// LDS waits, then a run of exp/convert VALU) leaves the matrix and vector
// pipes taking turns.  These scheduling groups ask for each MFMA to be
// followed by a few VALU instructions and the next LDS reads, keeping
// operands a few reads ahead.  Masks: 0x8 MFMA, 0x2 VALU, 0x100 LDS read.
constexpr int kSchedValu = 3;    // VALU slots per MFMA (128-wide Q/K; 64-wide: one more)
constexpr int kSchedLead = 4;    // LDS operand reads issued ahead of their MFMA
constexpr int kSchedValu8 = 4;   // VALU slots per fp8 score MFMA, in units of kSchedValu
// Causal launches of the 8-wave shape synchronise every second key tile
// (four-tile V ring).
constexpr bool kBar2 = true;
template <int MASK, int N>
__device__ __attribute__((always_inline)) inline void sched_group()
{
    if constexpr (N > 0) __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
}
// NS score MFMAs (RS K reads and VS x VA VALU slots each: an fp8 score
// MFMA takes twice the cycles of a 16-bit one and reads two chunks; four
// times the VALU slots measured 3-4% faster than twice), then NP P V MFMAs
// (two transposed V reads and VA VALU slots each).  VA is 3 for 128-wide
// Q/K and 4 for 64-wide Q/K, whose tiles have half the score MFMAs for the
// same softmax work.
template <int NS, int NP, int RS = 1, int VS = 1, int VA = kSchedValu>
__device__ __attribute__((always_inline)) inline void schedule_iteration()
{
    {
        constexpr int LEAD = kSchedLead < NS * RS ? kSchedLead : NS * RS;
        sched_group<0x100, LEAD>();
        sched_group<0x002, 2 * VA>();
        static_for<0, NS>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            sched_group<0x008, 1>();
            sched_group<0x100, ((i + 1) * RS + LEAD <= NS * RS) ? RS : RS + 1>();
            sched_group<0x002, VA * VS>();
        });
        static_for<0, NP>([&](auto ic) __attribute__((always_inline)) {
            sched_group<0x008, 1>();
            sched_group<0x100, 2>();
            sched_group<0x002, VA>();
        });
    }
}

template <int DQ, int DV, int QKB = 2, bool BAR2 = false>
struct Fast16 {
    static constexpr FastShape SH = fast_shape(DQ, DV);
    static constexpr int NW = SH.waves, THREADS = 64 * SH.waves, BM = 32 * SH.waves;
    static constexpr int BN = 64;
    static constexpr int KROW = DQ * QKB, VROW = DV * 2; // bytes per row in LDS (QKB bytes
                                                         // per Q/K element: 2, or 1 for fp8)
    static constexpr int KCH = KROW / 16, VCH = DV / 8;  // 16-byte chunks per row
    static constexpr int KT = BN * KROW, VT = BN * VROW;
    // Ring buffers of KS K tiles and VS V tiles.  Iteration t reads K(t+1)
    // (scores of the next tile) and V(t); after its barrier it refills the
    // slots of K(t) and V(t-1) with K(t+KS) and V(t+VS-1).  BAR2 (a barrier
    // every second iteration) keeps four V tiles.
    static constexpr int KS = SH.kslots, VS = BAR2 ? 4 : SH.vslots, U = SH.kslots;
    static constexpr int K_SLOT0 = 0, V_SLOT0 = KS * KT;
    static constexpr int LDS_BYTES = KS * KT + VS * VT;
    // Waves that issue the tile loads: with two waves per SIMD (waves w and
    // w+4 share one), only the first of each pair.  It is the older one,
    // ahead in issue priority, and reaches the barrier ~600 clocks before
    // the second; this way the second starts its MFMAs right after the
    // barrier instead of issuing loads.
    static constexpr int DMA_WAVES = NW == 8 ? NW / 2 : NW;
    static constexpr int K_PER_W = KT / 1024 / DMA_WAVES;   // 1 KB loads per issuing wave
    static constexpr int V_PER_W = VT / 1024 / DMA_WAVES;
    static constexpr int LOADS = K_PER_W + V_PER_W;  // per issuing wave per tile
    static_assert(K_PER_W >= 1 && V_PER_W >= 1 && KT % (1024 * DMA_WAVES) == 0 &&
                      VT % (1024 * DMA_WAVES) == 0, "tile split");
    static_assert(VS >= 2 && KS >= VS && KS % VS == 0 && (KS == 2 || KS == 4), "ring sizes");
    // ds_read immediate offsets are 16-bit: every K slot and every V slot
    // must be reachable from one base register each.
    static_assert(KS * KT <= 65536 && VS * VT <= 65536, "ring too large for immediates");
};

// LDS swizzles for the fast kernel.  gfx950's LDS has 64 banks of 4 bytes
// (256 bytes per clock): a ds_read_b128 is serviced 16 lanes at a time and a
// ds_read_b64_tr_b16 32 lanes at a time, and each such group must touch all
// 64 banks to avoid conflicts.  16-byte chunk c of row r is stored at chunk
// c ^ f(r):
//   K (score A operand, 16 lanes read rows 0..15 of a block at one chunk):
//     f(r) = r % 16 for 256-byte rows, (r / 2) % 8 for 128-byte rows,
//     (r / 4) % 4 for 64-byte rows (fp8 keys of width 64);
//   V (transposed reads, 32 lanes read 64 bytes from each of 4 consecutive
//     rows): f(r) = 4 * (r % 4) for 256-byte rows, 4 * ((r / 2) % 2) for
//     128-byte rows.
template <int CHUNKS>
__device__ inline int kswz(int row)
{
    return CHUNKS == 16 ? (row & 15) : CHUNKS == 8 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}
template <int CHUNKS>
__device__ inline int vswz(int row) { return CHUNKS == 16 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2); }

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kBufferConfig);
}

// The same raw buffer descriptor as four scalar words, for inline asm.
__device__ inline u32x4 rsrc_words(const void *base, uint32_t bytes)
{
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b),
                 (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)),
                 (uint32_t)__builtin_amdgcn_readfirstlane(bytes), (uint32_t)kBufferConfig};
}

// The descriptor advanced by `off` bytes (off <= its range): base + off,
// range - off.  All words are wave-uniform.
__device__ __attribute__((always_inline)) inline u32x4 tile_rsrc(const u32x4 &r, uint32_t off)
{
    const uint64_t base = ((uint64_t)r.y << 32 | r.x) + off;
    return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base),
                 (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)),
                 (uint32_t)__builtin_amdgcn_readfirstlane(r.z - off), r.w};
}

// One wave instruction: 64 lanes x 16 bytes from the buffer (lane offset
// `voffset`, zero when out of range) into LDS bytes lds_addr + 16*lane.
// Issued through inline asm on purpose: the compiler's wait-count pass
// treats a transposed LDS read as aliasing every pending LDS-DMA load and
// would wait for the whole prefetch pipeline before it; the kernel keeps the
// vmcnt bookkeeping itself (wait_loads) and VMEM loads complete in order.
__device__ inline void dma16(uint32_t lds_addr, uint32_t voffset, u32x4 rsrc)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voffset), "s"(rsrc)
                 : "memory", "m0");
}

__device__ inline uint32_t lds_address(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)(p);
}

typedef const __attribute__((address_space(3))) uint8_t lds_u8;
__device__ inline lds_u8 *lds_ptr(uint32_t addr) { return (lds_u8 *)(uintptr_t)addr; }

template <int LOADS_LEFT>
__device__ inline void wait_loads()
{
    // s_waitcnt vmcnt(LOADS_LEFT), expcnt / lgkmcnt left at their maximum.
    static_assert(LOADS_LEFT >= 0 && LOADS_LEFT < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((LOADS_LEFT & 15) | ((LOADS_LEFT >> 4) << 14) | (7 << 4) |
                               (15 << 8));
}

// EXT: the key range [kv_begin, kv_end) (optionally cut into `splits`
// chunks, one per group of workgroups), a signed causal offset and a
// window; rows that see no key get O = 0 and LSE = -inf.  OUT_F32: O is
// written as f32 (partial results for a merge), chunk s at O + s *
// part_o_stride and LSE + s * part_lse_stride.
// SCALED: base-2 attention with per-block scales, score = Q_scale[query
// block] * K_scale[key block] * (q . k) and weights 2^score; QK8: Q and K
// are fp8 (e4m3) and the scores run on the fp8 MFMA (64 dims per
// instruction, twice the 16-bit rate).
template <int DQ, int DV, bool CAUSAL, bool BF16, bool EXT = false, bool OUT_F32 = false,
          bool SCALED = false, bool QK8 = false>
__global__ void __attribute__((amdgpu_flat_work_group_size(Fast16<DQ, DV>::THREADS,
                                                           Fast16<DQ, DV>::THREADS),
                               amdgpu_waves_per_eu(Fast16<DQ, DV>::SH.occ,
                                                   Fast16<DQ, DV>::SH.occ)))
attn_fwd_fast16(KernelArgs p)
{
    // Causal attention with the 8-wave shape synchronises every second key
    // tile (measured 1-3% faster there, 1% slower without the causal mask;
    // the per-block scaled kernels would spill).
    constexpr bool BAR2 = kBar2 && CAUSAL && !SCALED && fast_shape(DQ, DV).kslots == 4;
    using T = Fast16<DQ, DV, QK8 ? 1 : 2, BAR2>;
    constexpr int BN = T::BN;
    constexpr int QKB = QK8 ? 1 : 2;          // bytes per Q/K element
    constexpr int KREADS = T::KCH / 2;        // 16-byte K reads per lane per 32-key block
    static_assert(EXT || !OUT_F32, "f32 output only in the extended kernel");
    static_assert(!(SCALED && EXT), "per-block scales use the plain visibility");
    static_assert(SCALED || !QK8, "fp8 keys come with their block scales");
    static_assert(!QK8 || DQ % 64 == 0, "fp8 scores take 64 dims per MFMA");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5, l32 = lane & 31;

    int32_t qb, slice, split = 0;
    int32_t blk = (int32_t)blockIdx.x;
    if constexpr (EXT) {
        const int32_t per_split = p.q_blocks * p.slices;
        split = blk / per_split;
        blk -= split * per_split;
    }
    map_block(blk, p.q_blocks, p.slices, p.order, p.per_xcd, CAUSAL, qb, slice);
    const int q0 = qb * T::BM;
    const int qw = q0 + wave * 32;          // first query row of this wave
    const int qi = qw + l32;                // this lane's query row
    // this workgroup's key range: everything, or one chunk of [kv_begin, kv_end)
    int32_t klo = 0, khi = p.S_k;
    if constexpr (EXT) {
        klo = p.kv_begin + split * p.split_len;
        khi = min(p.kv_end, klo + p.split_len);
    }

    // key tiles of this workgroup: t_first .. t_first + ntiles - 1, holding
    // the keys [wg_lo, wg_hi) some row of it sees
    int t_first = 0, ntiles;
    int32_t wg_lo = 0, wg_hi = p.S_k;
    if constexpr (EXT) {
        const PosRange pr = row_positions(q0, min(q0 + T::BM, p.S_q), p.q_per_head);
        const KeyRange kr = wg_key_range(pr.lo, pr.hi + 1, klo, khi, CAUSAL, p.coff, p.window);
        wg_lo = kr.key_lo;
        wg_hi = kr.key_hi;
        t_first = kr.key_lo / BN;
        ntiles = kr.key_hi > kr.key_lo ? (kr.key_hi + BN - 1) / BN - t_first : 0;
    } else {
        ntiles = kv_tiles_for(qb, T::BM, BN, p.S_q, p.S_k, CAUSAL);
    }

    const uint32_t q_bytes = (uint32_t)p.S_q * p.D_qk * QKB;
    const uint32_t k_bytes = (uint32_t)p.S_k * p.D_qk * QKB;
    const uint32_t v_bytes = (uint32_t)p.S_k * p.D_v * 2;
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(static_cast<const uint8_t *>(p.Q) + (size_t)slice * q_bytes, q_bytes);
    // K and V are read through ranges that end at the workgroup's last
    // visible key (the slice's end in the plain kernel): the keys after it
    // that share its tile read as zero, so that whatever the caller keeps
    // there (an unwritten cache tail, NaN) never reaches a result.
    const uint32_t k_range = EXT ? (uint32_t)wg_hi * p.D_qk * QKB : k_bytes;
    const uint32_t v_range = EXT ? (uint32_t)wg_hi * p.D_v * 2 : v_bytes;
    const u32x4 rk = rsrc_words(static_cast<const uint8_t *>(p.K) + (size_t)slice * k_bytes, k_range);
    const u32x4 rv = rsrc_words(static_cast<const uint8_t *>(p.V) + (size_t)slice * v_bytes, v_range);

    // ---- per-lane source offsets of this wave's K/V load instructions
    // (waves past DMA_WAVES issue no loads; their offsets are those of wave 0)
    const bool dma_wave = T::DMA_WAVES == T::NW || wave < T::DMA_WAVES;
    const int dw = dma_wave ? wave : 0;
    uint32_t koff[T::K_PER_W], voff[T::V_PER_W];
#pragma unroll
    for (int j = 0; j < T::K_PER_W; ++j) {
        const int P = (dw * T::K_PER_W + j) * 64 + lane;   // chunk slot in the K tile
        const int row = P / T::KCH, c = (P % T::KCH) ^ kswz<T::KCH>(row);
        constexpr int EPC = 16 / QKB;   // elements per 16-byte chunk
        koff[j] = c * EPC < p.D_qk ? (uint32_t)(row * p.D_qk + c * EPC) * QKB : kOutOfRange;
    }
#pragma unroll
    for (int j = 0; j < T::V_PER_W; ++j) {
        const int P = (dw * T::V_PER_W + j) * 64 + lane;
        const int row = P / T::VCH, c = (P % T::VCH) ^ vswz<T::VCH>(row);
        voff[j] = c * 8 < p.D_v ? (uint32_t)(row * p.D_v + c * 8) * 2 : kOutOfRange;
    }
    const uint32_t lds_k0 = (uint32_t)__builtin_amdgcn_readfirstlane(
        lds_address(smem) + T::K_SLOT0 + (uint32_t)dw * T::K_PER_W * 1024);
    const uint32_t lds_v0 = (uint32_t)__builtin_amdgcn_readfirstlane(
        lds_address(smem) + T::V_SLOT0 + (uint32_t)dw * T::V_PER_W * 1024);
    // K(t) into K slot t % KS and V(t) into V slot t % VS; the slot is a
    // compile-time constant at every call.
    // The tile's offset moves the descriptor's base (and shrinks its range)
    // in scalar registers, so the per-lane offsets stay fixed and the range
    // check still drops rows past the slice.
    auto issue_k = [&](int t, auto slot_c) __attribute__((always_inline)) {
        constexpr uint32_t sl = decltype(slot_c)::value * T::KT;
        const u32x4 r = tile_rsrc(rk, (uint32_t)(t_first + t) * BN * p.D_qk * QKB);
        if (dma_wave) {
#pragma unroll
            for (int j = 0; j < T::K_PER_W; ++j) dma16(lds_k0 + sl + j * 1024, koff[j], r);
        }
    };
    auto issue_v = [&](int t, auto slot_c) __attribute__((always_inline)) {
        constexpr uint32_t sl = decltype(slot_c)::value * T::VT;
        const u32x4 r = tile_rsrc(rv, (uint32_t)(t_first + t) * BN * p.D_v * 2);
        if (dma_wave) {
#pragma unroll
            for (int j = 0; j < T::V_PER_W; ++j) dma16(lds_v0 + sl + j * 1024, voff[j], r);
        }
    };
    // Tile 0 into slot 0.  In the extended kernel the rows of the first
    // tile before the workgroup's first visible key read as zero as well
    // (the counterpart of the range end above).
    const int skip0 = EXT ? wg_lo - t_first * BN : 0;   // rows of tile 0 before wg_lo
    auto issue_k0 = [&]() __attribute__((always_inline)) {
        if (EXT && skip0 > 0) {
            const u32x4 r = tile_rsrc(rk, (uint32_t)t_first * BN * p.D_qk * QKB);
            if (dma_wave) {
#pragma unroll
                for (int j = 0; j < T::K_PER_W; ++j) {
                    const int row = ((dw * T::K_PER_W + j) * 64 + lane) / T::KCH;
                    dma16(lds_k0 + j * 1024, row < skip0 ? kOutOfRange : koff[j], r);
                }
            }
        } else {
            issue_k(0, IC<0>{});
        }
    };
    auto issue_v0 = [&]() __attribute__((always_inline)) {
        if (EXT && skip0 > 0) {
            const u32x4 r = tile_rsrc(rv, (uint32_t)t_first * BN * p.D_v * 2);
            if (dma_wave) {
#pragma unroll
                for (int j = 0; j < T::V_PER_W; ++j) {
                    const int row = ((dw * T::V_PER_W + j) * 64 + lane) / T::VCH;
                    dma16(lds_v0 + j * 1024, row < skip0 ? kOutOfRange : voff[j], r);
                }
            }
        } else {
            issue_v(0, IC<0>{});
        }
    };

    // Output of this slice (of chunk `split` when the output is partial).
    constexpr uint32_t o_elt = OUT_F32 ? 4u : 2u;
    const uint32_t o_bytes = (uint32_t)p.S_q * p.D_v * o_elt;
    auto out_rsrc = [&]() __attribute__((always_inline)) {
        uint8_t *base = static_cast<uint8_t *>(p.O) + (size_t)slice * o_bytes;
        if constexpr (OUT_F32) base += (size_t)split * p.part_o_stride * 4;
        return make_rsrc(base, o_bytes);
    };
    auto lse_at = [&](int row) __attribute__((always_inline)) -> float & {
        size_t idx = (size_t)slice * p.S_q + row;
        if constexpr (OUT_F32) idx += (size_t)split * p.part_lse_stride;
        return p.LSE[idx];
    };
    if constexpr (EXT) {
        if (ntiles == 0) {
            // no row of the workgroup sees a key: O = 0, LSE = -inf
            const __amdgpu_buffer_rsrc_t ro0 = out_rsrc();
            const bool ok = qi < p.S_q;
#pragma unroll
            for (int d = 0; d < DV / 32; ++d)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d0 = d * 32 + g4 * 8 + hh * 4;
                    const uint32_t off = (ok && d0 < p.D_v) ? (uint32_t)(qi * p.D_v + d0) * o_elt
                                                            : kOutOfRange;
                    if constexpr (OUT_F32)
                        __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, ro0, off, 0, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, ro0, off, 0, 0);
                }
            if (p.LSE && hh == 0 && ok) lse_at(qi) = neg_inf();
            return;
        }
    }

    static_assert(!BAR2 || (T::KS == 4 && T::VS == 4), "BAR2 needs four-tile rings");
    if constexpr (BAR2) {
        // K(0..2) and V(0..1): the tiles of iterations 0 and 1
        issue_k0();
        if (1 < ntiles) issue_k(1, IC<1>{});
        if (2 < ntiles) issue_k(2, IC<2>{});
        issue_v0();
        if (1 < ntiles) issue_v(1, IC<1>{});
    } else {
    // Prologue: K(0 .. KS-1) and V(0 .. VS-2) in the order the main loop
    // would have issued them (K(j) before V(j-1)), K(0) first.
    issue_k0();
    static_for<1, T::KS>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        if (j < ntiles) issue_k(j, IC<j>{});
        if constexpr (j == 1) issue_v0();
        else if constexpr (j - 1 < T::VS - 1)
            if (j - 1 < ntiles) issue_v(j - 1, IC<j - 1>{});
    });
    }

    // ---- per-row scale (SCALED): this lane's query block's Q scale, folded
    // into the exponent factor; a negative scale flips Q's sign, a zero one
    // zeroes Q (as the global scale does in the plain kernel).
    float c = p.c;
    uint32_t q_xor = p.q_xor, q_and = p.q_and;
    if constexpr (SCALED) {
        float qs = 1.0f;
        if (qi < p.S_q) qs = p.Q_scale[(size_t)slice * p.q_scale_blocks + qi / p.q_block];
        c = qs == 0.0f ? 1.0f : __builtin_fabsf(qs);
        q_xor = qs < 0.0f ? (QK8 ? 0x80808080u : 0x80008000u) : 0u;
        q_and = qs == 0.0f ? 0u : 0xffffffffu;
    }

    // ---- Q fragment (B operand of S^T = K Q^T): query qi, 16-byte chunk
    // 2j + hh of the row in register group j (16-bit: dims 16j + 8hh + 0..7,
    // one MFMA each; fp8: dims 32j + 16hh + 0..15, two groups per MFMA).
    constexpr int QCH = DQ * QKB / 32;   // 16-byte chunks per lane
    u32x4 qf[QCH];
#pragma unroll
    for (int j = 0; j < QCH; ++j) {
        const int d0 = (2 * j + hh) * (16 / QKB);
        const uint32_t off = d0 < p.D_qk ? (uint32_t)(qi * p.D_qk + d0) * QKB : kOutOfRange;
        u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
        x = (x ^ q_xor) & q_and;
        if (d0 >= p.D_qk) x = u32x4{0u, 0u, 0u, 0u};
        qf[j] = x;
    }

    // ---- per-lane LDS read addresses in stage 0, computed once
    // K (score A operand): row 32kb + sigma(l32), logical chunk 2st + hh.
    // The swizzle depends on the row only through bits the kb term does not
    // touch, so the kb offset is an immediate.
    uint32_t kro[KREADS];
    {
        const int krow = sigma(l32);
#pragma unroll
        for (int st = 0; st < KREADS; ++st)
            kro[st] = lds_address(smem) +
                      (uint32_t)(krow * T::KROW + ((2 * st + hh) ^ kswz<T::KCH>(krow)) * 16);
    }
    // V (transposed reads): group g = lane/16, i = lane%16, source lane
    // i = 4k + q points at key row R + k (R a multiple of 4: the swizzle only
    // sees k and the row's low bits), dims 32*dblk + 16*(g%2) + 4q.
    uint32_t vro[DV / 32];
    {
        const int vg = lane >> 4, vi = lane & 15, vk = vi >> 2, vq = vi & 3;
        const int row = hh * 8 + vk;   // + 32kb + 16u + 4sh, multiples of 8 and 4
#pragma unroll
        for (int d = 0; d < DV / 32; ++d) {
            const int chunk = (d * 4 + (vg & 1) * 2 + (vq >> 1)) ^ vswz<T::VCH>(row);
            vro[d] = lds_address(smem) +
                     (uint32_t)(T::V_SLOT0 + row * T::VROW + chunk * 16 + (vq & 1) * 8);
        }
    }

    f32x16 o[DV / 32];
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) o[d] = f32x16{};
    float m = neg_inf();   // running max of the raw scores of this query (SCALED:
                           // of the scores times their key block's scale)
    float l = 0.0f;        // running sum of this lane's half of the keys

    // S^T of the key tile staged at `so` (two 32-key blocks).
    auto scores = [&](uint32_t so, f32x16 (&out)[2]) __attribute__((always_inline)) {
        out[0] = f32x16{};
        out[1] = f32x16{};
        typedef const __attribute__((address_space(3))) u32x4 lds_u32x4;
        if constexpr (QK8) {
#pragma unroll
            for (int st = 0; st < DQ / 64; ++st) {
                const u32x4 a0 = *reinterpret_cast<lds_u32x4 *>(lds_ptr(kro[2 * st] + so));
                const u32x4 a1 = *reinterpret_cast<lds_u32x4 *>(lds_ptr(kro[2 * st + 1] + so));
                const u32x4 b0 = *reinterpret_cast<lds_u32x4 *>(
                    lds_ptr(kro[2 * st] + so) + 32 * T::KROW);
                const u32x4 b1 = *reinterpret_cast<lds_u32x4 *>(
                    lds_ptr(kro[2 * st + 1] + so) + 32 * T::KROW);
                out[0] = mma8(a0, a1, qf[2 * st], qf[2 * st + 1], out[0]);
                out[1] = mma8(b0, b1, qf[2 * st], qf[2 * st + 1], out[1]);
            }
        } else {
#pragma unroll
            for (int st = 0; st < DQ / 16; ++st) {
                const auto *k0 = reinterpret_cast<lds_u32x4 *>(lds_ptr(kro[st] + so));
                const auto *k1 = reinterpret_cast<lds_u32x4 *>(lds_ptr(kro[st] + so) + 32 * T::KROW);
                out[0] = mma16<BF16>(*k0, qf[st], out[0]);
                out[1] = mma16<BF16>(*k1, qf[st], out[1]);
            }
        }
    };
    auto lane_max = [](const f32x16 (&x)[2]) __attribute__((always_inline)) {
        float mx = x[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmax_nan(mx, x[kb][r]);
        return mx;
    };
    // O^T += V^T P^T for one 32-key block kb of the tile staged at `so`.
    auto pv_block = [&](uint32_t so, int kb, const u32x4 (&pb)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int d = 0; d < DV / 32; ++d) {
                uint32_t a[4];
#pragma unroll
                for (int sh = 0; sh < 2; ++sh) {
                    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(
                        lds_ptr(vro[d] + so) + (kb * 32 + u * 16 + sh * 4) * T::VROW));
                    const u32x2 xw = __builtin_bit_cast(u32x2, x);
                    a[2 * sh] = xw.x;
                    a[2 * sh + 1] = xw.y;
                }
                o[d] = mma16<BF16>(u32x4{a[0], a[1], a[2], a[3]}, pb[u], o[d]);
            }
    };
    // P = 2^(s c - m c) for one 32-key block, packed to 16 bits; the row sum
    // is taken over the f32 values so that LSE keeps f32 accuracy.
    auto probs = [&](const f32x16 &sb, float ct, float mc, u32x4 (&pb)[2], float &rs) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float p0 = fast_exp2(__builtin_fmaf(sb[8 * u + 2 * j], ct, -mc));
                const float p1 = fast_exp2(__builtin_fmaf(sb[8 * u + 2 * j + 1], ct, -mc));
                rs += p0 + p1;
                w[j] = pack2<BF16>(p0, p1);
            }
            pb[u] = u32x4{w[0], w[1], w[2], w[3]};
        }
    };

    // Visible keys of this lane, [lo_i, hi_i), and of the wave: a tile needs
    // no mask when it lies inside every row's range, and the wave is idle
    // on a tile outside every row's range.  Ranges follow the query
    // position, the row modulo the positions per head.
    int lo_i = 0, hi_i = 0, wave_lo_min = 0, wave_lo_max = 0, wave_hi_min = 0, wave_hi_max = 0;
    if constexpr (EXT) {
        const bool win = p.window > 0;
        const int pi = qi % p.q_per_head;
        lo_i = win ? max(klo, pi + p.coff - p.window + 1) : klo;
        hi_i = CAUSAL ? min(khi, pi + p.coff + 1) : khi;
        const PosRange pw = row_positions(qw, min(qw + 32, p.S_q), p.q_per_head);
        wave_lo_min = win ? max(klo, pw.lo + p.coff - p.window + 1) : klo;
        wave_lo_max = win ? max(klo, pw.hi + p.coff - p.window + 1) : klo;
        wave_hi_min = CAUSAL ? min(khi, pw.lo + p.coff + 1) : khi;
        wave_hi_max = CAUSAL ? min(khi, pw.hi + p.coff + 1) : khi;
        if (qw >= p.S_q) wave_hi_max = -1;   // no row of the wave exists: idle throughout
    }

    // ---- prologue: scores of tile 0.  K(0) was the first load issued; every
    // other prologue load may still be in flight when all of them exist.
    if constexpr (BAR2) {
        if (ntiles > 2) wait_loads<2 * T::K_PER_W + 2 * T::V_PER_W>();
        else wait_loads<0>();
    } else {
    if (ntiles >= T::KS) wait_loads<(T::KS - 1) * T::K_PER_W + (T::VS - 1) * T::V_PER_W>();
    else wait_loads<0>();
    }
    __syncthreads();
    f32x16 sc[2][2];     // scores of tiles t and t+1, alternating by parity
    float mxs[2];        // their row maxima (both lane halves)
    bool grows[2];       // some row's max exceeds m by more than 2^kTau (unmasked tiles)
    // SCALED: the key block scale of tile t (wave-uniform, a scalar load),
    // read one tile ahead of its use.  The scores of a tile whose key scale
    // is negative are formed with -Q (a sign flip of the Q fragment, exact),
    // so the scale applied to every tile's raw scores is |K_scale| > 0: the
    // max of the scaled scores is that scale times the max of the raw ones
    // and masked scores stay -inf.  A zero scale is raised to the smallest
    // normal float, which changes no result.
    float kss[2] = {1.0f, 1.0f};
    float ks_ahead = 0.0f;   // key scale of the tile after the next one
    bool q_neg = false;      // the Q fragment holds -Q
    auto key_scale = [&](int t) __attribute__((always_inline)) {
        const int tt = min(t, ntiles - 1);
        return p.K_scale[(size_t)slice * p.k_scale_blocks + tt / p.k_tiles_per_block];
    };
    auto key_mag = [](float ks) __attribute__((always_inline)) {
        return fmaxf(__builtin_fabsf(ks), 1.17549435e-38f);
    };
    // the sign of Q for the scores of a tile with key scale ks (wave-uniform)
    auto key_sign = [&](float ks) __attribute__((always_inline)) {
        const bool neg = ks < 0.0f;
        if (neg != q_neg) {
            constexpr uint32_t flip = QK8 ? 0x80808080u : 0x80008000u;
#pragma unroll
            for (int j = 0; j < QCH; ++j) qf[j] ^= flip;
            q_neg = neg;
        }
    };
    if constexpr (SCALED) {
        const float ks0 = key_scale(0);
        key_sign(ks0);
        kss[0] = key_mag(ks0);
        ks_ahead = key_scale(1);
    }
    scores(0, sc[0]);
    mxs[0] = max_halves(lane_max(sc[0]));
    if constexpr (SCALED) mxs[0] *= kss[0];
    grows[0] = true;     // m is still -inf

    // ---- one iteration of the main loop, software pipelined: iteration t
    // finishes tile t (softmax, P V) while the scores of tile t+1 are formed,
    // so every phase has MFMA and VALU work from the same wave to overlap.
    // u = t % KS is a compile-time constant, so ring slots are immediates and
    // the score registers alternate without copies.
    auto step = [&](int t, auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        constexpr uint32_t so = (uint32_t)(u % T::VS) * T::VT;          // V slot of tile t
        constexpr uint32_t so1 = (uint32_t)((u + 1) % T::KS) * T::KT;   // K slot of tile t+1
        f32x16(&s)[2] = sc[u & 1];
        f32x16(&sn)[2] = sc[(u + 1) & 1];
        const int kbase = (t_first + t) * BN;
        // some key of tile t is visible to some row of the wave
        bool active;
        if constexpr (EXT) active = kbase < wave_hi_max && kbase + BN > wave_lo_min;
        else active = !CAUSAL || kbase <= qw + 31;

        float mx = mxs[u & 1];
        bool grow_any = grows[u & 1];
        if constexpr (SCALED) {
            // tile t+1: its scale was read during the previous iteration
            key_sign(ks_ahead);
            kss[(u + 1) & 1] = key_mag(ks_ahead);
            ks_ahead = key_scale(t + 2);
        }
        if (active) {
            // masks: keys >= S_k; keys after the query when causal (in the
            // extended kernel: keys outside the row's [lo_i, hi_i))
            bool need_mask;
            if constexpr (EXT) need_mask = kbase < wave_lo_max || kbase + BN > wave_hi_min;
            else need_mask = (kbase + BN > p.S_k) || (CAUSAL && kbase + BN - 1 > qw);
            if (need_mask) {
                // Register r of block kb holds key kbase + hh*8 + kb*32 +
                // (r/8)*16 + r%8; it is kept when that key is < S_k and,
                // causal, <= the query: one per-lane limit against
                // compile-time offsets (two limits in the extended kernel).
                int lim, lim_lo = 0;
                if constexpr (EXT) {
                    lim = hi_i - 1 - kbase - hh * 8;
                    lim_lo = lo_i - kbase - hh * 8;
                } else {
                    lim = p.S_k - 1;
                    if (CAUSAL) lim = min(lim, qi);
                    lim -= kbase + hh * 8;
                }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = kb * 32 + (r >> 3) * 16 + (r & 7);
                        bool keep = off <= lim;
                        if constexpr (EXT) keep = keep && off >= lim_lo;
                        s[kb][r] = keep ? s[kb][r] : neg_inf();
                    }
                mx = max_halves(lane_max(s));
                if constexpr (SCALED) mx *= kss[u & 1];
                grow_any = __builtin_amdgcn_ballot_w64((mx - m) * c > kTau) != 0;
            }
            // running max; rescale only when a row's max grows by > 2^kTau
            if (grow_any) {
                const float m_new = fmaxf(m, mx);
                float alpha = fast_exp2((m - m_new) * c);
                if constexpr (EXT)
                    if (m_new == neg_inf()) alpha = 1.0f;   // row still without keys
                m = m_new;
                l *= alpha;
#pragma unroll
                for (int d = 0; d < DV / 32; ++d) o[d] *= alpha;
            }
        }

        // V(t) (the last load of iteration t-VS+1) must be resident; K(t+1)
        // was issued no later.  Loads issued after V(t): the groups of
        // iterations t-VS+2 .. t-1, all full while t+KS-1 < ntiles; near the
        // end wait for everything.  After the barrier every wave is done with
        // the slots of K(t) and V(t-1), which this iteration refills.
        if constexpr (BAR2) {
            // A barrier every second iteration: the leading wave of a SIMD
            // pair runs on into the next tile while the other finishes.  At
            // an even iteration t everything issued before (what iterations
            // t and t+1 read) must be resident; then the slots of K(t-1),
            // K(t), V(t-2) and V(t-1), which no wave reads from here to the
            // next barrier, take what iterations t+2 and t+3 read: K(t+3)
            // and V(t+2) right after the barrier, K(t+4) and V(t+3) one
            // iteration later, which halves the leading waves' load burst
            // after a barrier.
            if constexpr (u % 2 == 0) {
                wait_loads<0>();
                __syncthreads();
                if (t + 3 < ntiles) issue_k(t + 3, IC<(u + 3) % 4>{});
                if (t + 2 < ntiles) issue_v(t + 2, IC<(u + 2) % 4>{});
            } else {
                if (t + 3 < ntiles) issue_k(t + 3, IC<(u + 3) % 4>{});
                if (t + 2 < ntiles) issue_v(t + 2, IC<(u + 2) % 4>{});
            }
        } else {
        if (t + T::KS - 1 < ntiles) wait_loads<(T::VS - 2) * T::LOADS>();
        else wait_loads<0>();
        __syncthreads();
        if (t + T::KS < ntiles) issue_k(t + T::KS, IC<u % T::KS>{});
        if (t + T::VS - 1 < ntiles) issue_v(t + T::VS - 1, IC<(u + T::VS - 1) % T::VS>{});
        }
        if (!active) {
            // With a window a wave can be idle on tile t and busy on t+1:
            // then it still forms the scores of t+1 here.
            if constexpr (EXT) {
                const int kn = kbase + BN;
                if (t + 1 < ntiles && kn < wave_hi_max && kn + BN > wave_lo_min) {
                    scores(so1, sn);
                    mxs[(u + 1) & 1] = max_halves(lane_max(sn));
                    grows[(u + 1) & 1] = true;   // m is still -inf for this wave
                }
            }
            return;   // without a window, every later tile is idle too
        }

        float mc = m * c;
        if constexpr (EXT)
            if (m == neg_inf()) mc = 0.0f;   // row without keys so far: every P is 0
        float rs = 0.0f;
        u32x4 pb0[2], pb1[2];
        float ct = c;   // exponent factor of this tile's raw scores
        // (raised to the smallest normal float: a product that underflows
        // to 0 would turn the -inf of a masked score into NaN)
        if constexpr (SCALED) ct = fmaxf(c * kss[u & 1], 1.17549435e-38f);
        // phase A: scores of tile t+1 (garbage past the last tile, unused) || P of block 0
        scores(so1, sn);
        probs(s[0], ct, mc, pb0, rs);
        // phase B1: O += V P for block 0 || P of block 1
        pv_block(so, 0, pb0);
        probs(s[1], ct, mc, pb1, rs);
        // phase B2: O += V P for block 1 || lane max of the next scores
        pv_block(so, 1, pb1);
        // the next tile's row max and its rescale decision, decided here
        // beside the P V MFMAs (m no longer changes in this iteration)
        mxs[(u + 1) & 1] = max_halves(lane_max(sn));
        if constexpr (SCALED) mxs[(u + 1) & 1] *= kss[(u + 1) & 1];
        grows[(u + 1) & 1] = __builtin_amdgcn_ballot_w64((mxs[(u + 1) & 1] - m) * c > kTau) != 0;
        l += rs;
        if constexpr (QK8)
            schedule_iteration<2 * (DQ / 64), 4 * (DV / 32), 2, kSchedValu8>();
        else
            schedule_iteration<2 * (DQ / 16), 4 * (DV / 32), 1, 1,
                               DQ <= 64 ? kSchedValu + 1 : kSchedValu>();
    };

    for (int t0 = 0; t0 < ntiles; t0 += T::U) {
        step(t0, IC<0>{});
        if (t0 + 1 >= ntiles) break;
        step(t0 + 1, IC<1>{});
        if constexpr (T::U == 4) {
            if (t0 + 2 >= ntiles) break;
            step(t0 + 2, IC<2>{});
            if (t0 + 3 >= ntiles) break;
            step(t0 + 3, IC<3>{});
        }
    }

    // ---- epilogue: O = O_acc / l, LSE = m*scale + ln(l)
    const float lt = sum_halves(l);
    float inv = 1.0f / lt;
    if constexpr (EXT)
        if (!(lt > 0.0f)) inv = 0.0f;   // no visible key: O = 0
    const __amdgpu_buffer_rsrc_t ro = out_rsrc();
    const bool row_ok = qi < p.S_q;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = d * 32 + g4 * 8 + hh * 4;   // 4 consecutive dims
            const uint32_t off =
                (row_ok && d0 < p.D_v) ? (uint32_t)(qi * p.D_v + d0) * o_elt : kOutOfRange;
            if constexpr (OUT_F32) {
                const f32x4 v4 = {o[d][4 * g4] * inv, o[d][4 * g4 + 1] * inv,
                                  o[d][4 * g4 + 2] * inv, o[d][4 * g4 + 3] * inv};
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v4), ro, off, 0,
                                                       0);
            } else {
                const uint32_t w0 = pack2<BF16>(o[d][4 * g4] * inv, o[d][4 * g4 + 1] * inv);
                const uint32_t w1 = pack2<BF16>(o[d][4 * g4 + 2] * inv, o[d][4 * g4 + 3] * inv);
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, u32x2{w0, w1}),
                                                      ro, off, 0, 0);
            }
        }
    if (p.LSE && hh == 0 && row_ok) {
        float lse = (m * c + __builtin_amdgcn_logf(lt)) * kLn2;
        if constexpr (EXT)
            if (!(lt > 0.0f)) lse = neg_inf();
        lse_at(qi) = lse;
    }
}

// ====================================================================
// f32 kernel with the key tiles split over the waves, for small grids.
//
// When 128-row workgroups would leave most CUs idle (few slices, short
// sequences), a workgroup takes 32 query rows and its four waves (one per
// SIMD) split the key tiles: wave w takes tiles w, w+4, w+8, ..., each with
// its own online softmax over the keys it sees.  The four partial results
// (running max m_w, sum l_w, unnormalised O_w) are combined through LDS at
// the end, as chunks of keys are merged: M = max m_w, a_w = exp(m_w - M),
// O = sum a_w O_w / sum a_w l_w.
//
// A wave stages its own tiles in a private LDS region (K at 16-byte chunk
// c ^ (row % 8) of its row, V row-major), so the key loop has no barrier.
// One tile's worth of registers carries the loads in flight: K(t+4) is
// loaded while the softmax and P V of tile t run and stored after them; V(t)
// is loaded while the scores of t run and stored after them.
// ====================================================================
template <int DQ, int DV>
struct Split32 {
    static constexpr int BN = 32;                              // keys per tile
    static constexpr int KCH = DQ / 4, VCH = DV / 4;           // 16-byte chunks per row
    static constexpr int K_CHUNKS = BN * KCH, V_CHUNKS = BN * VCH;
    static constexpr int K_PER_L = K_CHUNKS / 64, V_PER_L = V_CHUNKS / 64;   // per lane
    static constexpr int WAVE_CHUNKS = K_CHUNKS + V_CHUNKS;   // LDS per wave
    // combination: O_w as [wave][row][OROW] floats, then m_w and l_w [wave][row]
    static constexpr int OROW = DV + 4;
    static constexpr int COMBINE_CHUNKS = (4 * 32 * OROW + 2 * 4 * 32) / 4;
    static constexpr int LDS_CHUNKS =
        4 * WAVE_CHUNKS > COMBINE_CHUNKS ? 4 * WAVE_CHUNKS : COMBINE_CHUNKS;
    static_assert(K_CHUNKS % 64 == 0 && V_CHUNKS % 64 == 0 && KCH % 8 == 0, "tile split");
};
constexpr int kSplitRows = 32;   // query rows per workgroup of the split kernel


template <int DQ, int DV, bool CAUSAL>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(1, 1)))
attn_fwd_32s(KernelArgs p)
{
    using T = Split32<DQ, DV>;
    constexpr int BN = T::BN;
    __shared__ u32x4 lds[T::LDS_CHUNKS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5, l32 = lane & 31;

    int32_t qb, slice;
    map_block((int32_t)blockIdx.x, p.q_blocks, p.slices, p.order, p.per_xcd, CAUSAL, qb, slice);
    // workgroup-uniform: keeps the buffer descriptors below in scalar registers
    qb = __builtin_amdgcn_readfirstlane(qb);
    slice = __builtin_amdgcn_readfirstlane(slice);
    const int q0 = qb * kSplitRows;
    const int qi = q0 + l32;

    // Buffer descriptors over this slice's Q, K and V: an offset past the
    // slice reads as zero, so rows past S_q / S_k and columns past D need no
    // branch (offsets are 32-bit: a slice is below 2^31 bytes).
    const uint32_t q_bytes = (uint32_t)p.S_q * p.D_qk * 4;
    const uint32_t k_bytes = (uint32_t)p.S_k * p.D_qk * 4;
    const uint32_t v_bytes = (uint32_t)p.S_k * p.D_v * 4;
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(static_cast<const uint8_t *>(p.Q) + (size_t)slice * q_bytes, q_bytes);
    const __amdgpu_buffer_rsrc_t rk =
        make_rsrc(static_cast<const uint8_t *>(p.K) + (size_t)slice * k_bytes, k_bytes);
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(static_cast<const uint8_t *>(p.V) + (size_t)slice * v_bytes, v_bytes);
    // Columns col .. col+3 of a row of a row-major f32 matrix with `ncols`
    // columns; zero past nrows rows or ncols columns: one 16-byte load when
    // the inputs are vector-aligned (ncols % 4 == 0), else four 4-byte loads.
    auto load4v = [&](__amdgpu_buffer_rsrc_t r, int row, int nrows, int col, int ncols)
        __attribute__((always_inline)) {
        const uint32_t off =
            (row < nrows && col < ncols) ? (uint32_t)(row * ncols + col) * 4 : kOutOfRange;
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    };
    auto load4s = [&](__amdgpu_buffer_rsrc_t r, int row, int nrows, int col, int ncols)
        __attribute__((always_inline)) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t off = (row < nrows && col + e < ncols)
                                     ? (uint32_t)(row * ncols + col + e) * 4
                                     : kOutOfRange;
            w[e] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
        }
        return u32x4{w[0], w[1], w[2], w[3]};
    };

    // Q fragment: step 4u+j of the k=2 MFMA uses dim 8u + 4hh + j.
    float qf[DQ / 2];
#pragma unroll
    for (int u = 0; u < DQ / 8; ++u) {
        u32x4 x = p.vec ? load4v(rq, qi, p.S_q, u * 8 + hh * 4, p.D_qk)
                        : load4s(rq, qi, p.S_q, u * 8 + hh * 4, p.D_qk);
        x = (x ^ p.q_xor) & p.q_and;
        const f32x4 xf = __builtin_bit_cast(f32x4, x);   // whole-vector bit cast
#pragma unroll
        for (int j = 0; j < 4; ++j) qf[4 * u + j] = xf[j];
    }

    const int ntiles = kv_tiles_for(qb, kSplitRows, BN, p.S_q, p.S_k, CAUSAL);
    const float c = p.c;

    f32x16 o[DV / 32];
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) o[d] = f32x16{};
    float m = neg_inf();
    float l = 0.0f;

    u32x4 *Kw = lds + wave * T::WAVE_CHUNKS;   // this wave's K tile, then its V tile
    const float *Vw = reinterpret_cast<const float *>(Kw + T::K_CHUNKS);

    // The key loop, for 16-byte (VEC) or 4-byte global loads.  Per tile t:
    // the scores of t, during which V(t) goes from registers to LDS and
    // K(t+4) is loaded into registers, one chunk per group of four MFMAs;
    // the softmax; then P V, during which K(t+4) goes to LDS and V(t+4) is
    // loaded, one chunk per key.  So the MFMA pipe is fed throughout except
    // for the softmax.  LDS reads and writes of one wave execute in order,
    // so a region is rewritten only after the reads of the tile before have
    // been served.
    auto key_loop = [&](auto vec_c) __attribute__((always_inline)) {
        constexpr bool VEC = decltype(vec_c)::value != 0;
        auto load4 = [&](__amdgpu_buffer_rsrc_t r, int row, int col, int ncols)
            __attribute__((always_inline)) {
            if constexpr (VEC) return load4v(r, row, p.S_k, col, ncols);
            else return load4s(r, row, p.S_k, col, ncols);
        };
        u32x4 rk4[T::K_PER_L], rv4[T::V_PER_L];   // one tile of K and of V in flight
        auto load_k = [&](int t, int i) __attribute__((always_inline)) {
            const int ci = lane + 64 * i;
            rk4[i] = load4(rk, t * BN + ci / T::KCH, (ci % T::KCH) * 4, p.D_qk);
        };
        auto store_k = [&](int i) __attribute__((always_inline)) {
            const int ci = lane + 64 * i;
            const int row = ci / T::KCH, cc = ci % T::KCH;
            Kw[row * T::KCH + (cc ^ (row & 7))] = rk4[i];
        };
        auto load_v = [&](int t, int i) __attribute__((always_inline)) {
            const int ci = lane + 64 * i;
            rv4[i] = load4(rv, t * BN + ci / T::VCH, (ci % T::VCH) * 4, p.D_v);
        };
        auto store_v = [&](int i) __attribute__((always_inline)) {
            Kw[T::K_CHUNKS + lane + 64 * i] = rv4[i];
        };

        if (wave < ntiles) {
#pragma unroll
            for (int i = 0; i < T::K_PER_L; ++i) load_k(wave, i);
#pragma unroll
            for (int i = 0; i < T::K_PER_L; ++i) store_k(i);
#pragma unroll
            for (int i = 0; i < T::V_PER_L; ++i) load_v(wave, i);
        }
        for (int t = wave; t < ntiles; t += 4) {
            const int kbase = t * BN;
            // The loads and stores for tile t+4 run unconditionally: past
            // the last tile of the wave they move rows that are never read
            // (or zeros, past S_k), and keep the loop free of branches.

            // ---- S^T: lane (l32, hh) gets keys (r/4)*8 + 4hh + r%4 of query
            // qi.  K chunks are read three groups ahead of their MFMAs;
            // scheduling barriers keep the compiler from sinking the reads
            // (and the chunk moves) back next to their use.
            f32x16 s = f32x16{};
            {
                constexpr int NU = DQ / 8;
                f32x4 ka[4];
                auto kread = [&](int u) __attribute__((always_inline)) {
                    return __builtin_bit_cast(f32x4,
                                              Kw[l32 * T::KCH + ((2 * u + hh) ^ (l32 & 7))]);
                };
#pragma unroll
                for (int u = 0; u < 3; ++u) ka[u] = kread(u);
#pragma unroll
                for (int u = 0; u < NU; ++u) {
                    if (u + 3 < NU) ka[(u + 3) & 3] = kread(u + 3);
#pragma unroll
                    for (int i = u; i < T::V_PER_L; i += NU) store_v(i);   // V(t)
#pragma unroll
                    for (int i = u; i < T::K_PER_L; i += NU) load_k(t + 4, i);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < 4; ++j) s = mma32(ka[u & 3][j], qf[4 * u + j], s);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }

            const bool need_mask = (kbase + BN > p.S_k) || (CAUSAL && kbase + BN - 1 > q0);
            if (need_mask) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kbase + (r >> 2) * 8 + hh * 4 + (r & 3);
                    bool ok = key < p.S_k;
                    if (CAUSAL) ok = ok && key <= qi;
                    s[r] = ok ? s[r] : neg_inf();
                }
            }

            // Every tile a wave visits holds a key visible to each of its
            // rows (key kbase <= the first row when causal, kbase < S_k), so
            // m is finite from the first tile on.  The running max only moves
            // when some row's max grows by more than 2^kTau in the exponent
            // (always on the first tile), so O and l are rescaled rarely and
            // P stays below 2^kTau.
            float mx = s[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
            mx = fmaxf(mx, other_half(mx));
            if (__builtin_amdgcn_ballot_w64((mx - m) * c > kTau) != 0) {
                const float m_new = fmaxf(m, mx);
                const float alpha = fast_exp2((m - m_new) * c);
                m = m_new;
                l *= alpha;
#pragma unroll
                for (int d = 0; d < DV / 32; ++d) o[d] *= alpha;
            }
            const float mc = m * c;

            float pv[16];
            float rs = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                pv[r] = fast_exp2(__builtin_fmaf(s[r], c, -mc));
                rs += pv[r];
            }
            l += rs;

            // ---- O^T += V^T P^T; step r uses key (r/4)*8 + 4hh + r%4; V is
            // read two keys ahead
            {
                float va[3][DV / 32];
                auto vread = [&](int r, float (&dst)[DV / 32]) __attribute__((always_inline)) {
                    const int key = (r >> 2) * 8 + hh * 4 + (r & 3);
#pragma unroll
                    for (int d = 0; d < DV / 32; ++d) dst[d] = Vw[key * DV + d * 32 + l32];
                };
                vread(0, va[0]);
                vread(1, va[1]);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if (r + 2 < 16) vread(r + 2, va[(r + 2) % 3]);
#pragma unroll
                    for (int i = r; i < T::K_PER_L; i += 16) store_k(i);       // K(t+4)
#pragma unroll
                    for (int i = r; i < T::V_PER_L; i += 16) load_v(t + 4, i);  // V(t+4)
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int d = 0; d < DV / 32; ++d) o[d] = mma32(va[r % 3][d], pv[r], o[d]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };
    if (p.vec) key_loop(IC<1>{});
    else key_loop(IC<0>{});

    // ---- combination of the four waves' partial results
    __syncthreads();   // every wave is done with its K / V region
    float *cmb = reinterpret_cast<float *>(lds);
    float *cm = cmb + 4 * 32 * T::OROW;   // m_w per row
    float *cl = cm + 4 * 32;              // l_w per row (both lane halves)
    const float lt = l + other_half(l);
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = d * 32 + g * 8 + hh * 4;
            *reinterpret_cast<f32x4 *>(cmb + (wave * 32 + l32) * T::OROW + d0) =
                f32x4{o[d][4 * g], o[d][4 * g + 1], o[d][4 * g + 2], o[d][4 * g + 3]};
        }
    if (hh == 0) {
        cm[wave * 32 + l32] = m;   // -inf for a wave without tiles (its l and O are 0)
        cl[wave * 32 + l32] = lt;
    }
    __syncthreads();

    // thread (row r, part) writes columns 4 * (part + 8 i) .. +3 of row q0 + r
    const int r = tid >> 3, part = tid & 7;
    float mw[4], mmax = neg_inf();
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        mw[w] = cm[w * 32 + r];
        mmax = fmaxf(mmax, mw[w]);
    }
    float aw[4], lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        aw[w] = fast_exp2((mw[w] - mmax) * c);   // 0 for a wave without tiles
        lsum += aw[w] * cl[w * 32 + r];
    }
    const float inv = 1.0f / lsum;
    const int row = q0 + r;
    if (row < p.S_q) {
        float *Os = static_cast<float *>(p.O) + ((size_t)slice * p.S_q + row) * p.D_v;
#pragma unroll
        for (int i = 0; i < DV / 32; ++i) {
            const int d0 = 4 * (part + 8 * i);
            f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int w = 0; w < 4; ++w)
                acc += aw[w] * *reinterpret_cast<const f32x4 *>(cmb + (w * 32 + r) * T::OROW + d0);
            acc *= inv;
            if (p.vec) {
                if (d0 < p.D_v) *reinterpret_cast<f32x4 *>(Os + d0) = acc;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (d0 + j < p.D_v) Os[d0 + j] = acc[j];
            }
        }
        if (p.LSE && part == 0)
            p.LSE[(size_t)slice * p.S_q + row] = (mmax * c + __builtin_amdgcn_logf(lsum)) * kLn2;
    }
}

int pad_dim(int64_t d) { return d <= 64 ? 64 : 128; }
int pad_split(int64_t d) { return d <= 64 ? 64 : d <= 96 ? 96 : 128; }

template <typename Kern>
hipError_t launch(Kern kern, int64_t grid, const KernelArgs &args, hipStream_t stream,
                  int threads = kThreads)
{
    hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(threads), 0, stream, args);
    return hipGetLastError();
}

template <int DQ, int DV>
hipError_t dispatch_fast(int dtype, bool causal, int64_t grid, const KernelArgs &a,
                         hipStream_t s)
{
    constexpr int threads = Fast16<DQ, DV>::THREADS;
    if (dtype == TSD_BF16)
        return causal ? launch(attn_fwd_fast16<DQ, DV, true, true>, grid, a, s, threads)
                      : launch(attn_fwd_fast16<DQ, DV, false, true>, grid, a, s, threads);
    return causal ? launch(attn_fwd_fast16<DQ, DV, true, false>, grid, a, s, threads)
                  : launch(attn_fwd_fast16<DQ, DV, false, false>, grid, a, s, threads);
}

template <int DQ, int DV>
hipError_t dispatch_fast_ext(int dtype, bool causal, bool out_f32, int64_t grid,
                             const KernelArgs &a, hipStream_t s)
{
    constexpr int threads = Fast16<DQ, DV>::THREADS;
    if (out_f32) {
        if (dtype == TSD_BF16)
            return causal
                       ? launch(attn_fwd_fast16<DQ, DV, true, true, true, true>, grid, a, s, threads)
                       : launch(attn_fwd_fast16<DQ, DV, false, true, true, true>, grid, a, s, threads);
        return causal
                   ? launch(attn_fwd_fast16<DQ, DV, true, false, true, true>, grid, a, s, threads)
                   : launch(attn_fwd_fast16<DQ, DV, false, false, true, true>, grid, a, s, threads);
    }
    if (dtype == TSD_BF16)
        return causal
                   ? launch(attn_fwd_fast16<DQ, DV, true, true, true, false>, grid, a, s, threads)
                   : launch(attn_fwd_fast16<DQ, DV, false, true, true, false>, grid, a, s, threads);
    return causal
               ? launch(attn_fwd_fast16<DQ, DV, true, false, true, false>, grid, a, s, threads)
               : launch(attn_fwd_fast16<DQ, DV, false, false, true, false>, grid, a, s, threads);
}

template <int DQ, int DV>
hipError_t dispatch_fast_scaled(int dtype, bool causal, bool qk8, int64_t grid,
                                const KernelArgs &a, hipStream_t s)
{
    constexpr int threads = Fast16<DQ, DV>::THREADS;
    // fp8 keys: a K tile of 64 x DQ bytes must give each wave at least one
    // 1 KB load (DQ = 128, or DQ = 64 with the 4-wave shape)
    if constexpr (DQ == 128 || (DQ == 64 && DV == 64)) {
        if (qk8) {
            if (dtype == TSD_BF16)
                return causal ? launch(attn_fwd_fast16<DQ, DV, true, true, false, false, true, true>,
                                       grid, a, s, threads)
                              : launch(attn_fwd_fast16<DQ, DV, false, true, false, false, true, true>,
                                       grid, a, s, threads);
            return causal ? launch(attn_fwd_fast16<DQ, DV, true, false, false, false, true, true>,
                                   grid, a, s, threads)
                          : launch(attn_fwd_fast16<DQ, DV, false, false, false, false, true, true>,
                                   grid, a, s, threads);
        }
    }
    if (qk8) return hipErrorInvalidValue;
    if (dtype == TSD_BF16)
        return causal ? launch(attn_fwd_fast16<DQ, DV, true, true, false, false, true, false>, grid,
                               a, s, threads)
                      : launch(attn_fwd_fast16<DQ, DV, false, true, false, false, true, false>,
                               grid, a, s, threads);
    return causal ? launch(attn_fwd_fast16<DQ, DV, true, false, false, false, true, false>, grid, a,
                           s, threads)
                  : launch(attn_fwd_fast16<DQ, DV, false, false, false, false, true, false>, grid,
                           a, s, threads);
}

// ====================================================================
// Merge of partial results over key chunks (the continuation pass):
// for each query row, LSE = ln sum_g exp(LSE_g) and O = sum_g
// exp(LSE_g - LSE) O_g.  A chunk with LSE_g = -inf (no visible key)
// contributes nothing; a row whose chunks are all empty gets O = 0 and
// LSE = -inf.  One thread per (row, 4 consecutive output columns): every
// thread reads the row's n LSE values (shared by the row's threads through
// the cache) and its own 4 columns of each chunk, so each byte of the
// partial outputs is read once.  Bound by HBM bandwidth.
// ====================================================================
constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 8;

template <int ODT, bool VEC>
__global__ void __launch_bounds__(kMergeThreads) attn_merge_kernel(MergeArgs p)
{
    const int64_t g = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
    const int64_t row = g / p.groups;
    if (row >= p.rows) return;
    const int d0 = (int)(g - row * p.groups) * 4;
    constexpr float kLog2e = 1.4426950408889634f;

    // One pass in batches of kMergeBatch chunks, all loads of a batch issued
    // before any is used: a running max m, the sum of exp(LSE_g - m) and the
    // weighted O, rescaled when m grows.
    float m = neg_inf(), sum = 0.0f;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j0 = 0; j0 < p.n_parts; j0 += kMergeBatch) {
        float lv[kMergeBatch];
        f32x4 ov[kMergeBatch];
#pragma unroll
        for (int b = 0; b < kMergeBatch; ++b) {
            const int j = j0 + b;
            lv[b] = neg_inf();
            ov[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (j < p.n_parts) {
                lv[b] = p.LSE_parts[j * p.part_lse_stride + row];
                const float *src = p.O_parts + j * p.part_o_stride + row * p.D_v + d0;
                if constexpr (VEC) {
                    ov[b] = *reinterpret_cast<const f32x4 *>(src);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (d0 + e < p.D_v) ov[b][e] = src[e];
                }
            }
        }
        float bm = m;
#pragma unroll
        for (int b = 0; b < kMergeBatch; ++b) bm = fmaxf(bm, lv[b]);
        if (bm == neg_inf()) continue;   // no chunk so far sees a key
        const float r = fast_exp2((m - bm) * kLog2e);   // 0 while m is -inf
        sum *= r;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= r;
#pragma unroll
        for (int b = 0; b < kMergeBatch; ++b) {
            const float w = fast_exp2((lv[b] - bm) * kLog2e);   // 0 for an empty chunk
            sum += w;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, ov[b][e], acc[e]);
        }
        m = bm;
    }
    float lse = neg_inf();
    if (m != neg_inf()) {
        const float inv = 1.0f / sum;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= inv;
        lse = m + __builtin_amdgcn_logf(sum) * kLn2;
    }
    if (p.LSE && d0 == 0) p.LSE[row] = lse;
    if constexpr (ODT == TSD_F32) {
        float *dst = static_cast<float *>(p.O) + row * p.D_v + d0;
        if constexpr (VEC) {
            *reinterpret_cast<f32x4 *>(dst) = f32x4{acc[0], acc[1], acc[2], acc[3]};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (d0 + e < p.D_v) dst[e] = acc[e];
        }
    } else {
        constexpr bool BF = ODT == TSD_BF16;
        uint16_t *dst = static_cast<uint16_t *>(p.O) + row * p.D_v + d0;
        if constexpr (VEC) {
            *reinterpret_cast<u32x2 *>(dst) =
                u32x2{pack2<BF>(acc[0], acc[1]), pack2<BF>(acc[2], acc[3])};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (d0 + e < p.D_v) dst[e] = (uint16_t)(pack2<BF>(acc[e], 0.0f) & 0xffffu);
        }
    }
}

template <int DQ, int DV>
hipError_t dispatch_split(bool causal, int64_t grid, const KernelArgs &a, hipStream_t s)
{
    return causal ? launch(attn_fwd_32s<DQ, DV, true>, grid, a, s)
                  : launch(attn_fwd_32s<DQ, DV, false>, grid, a, s);
}

template <int DQ, int DV>
hipError_t dispatch_causal(int dtype, bool causal, int64_t grid, const KernelArgs &a,
                           hipStream_t s)
{
    if (dtype == TSD_F32)
        return causal ? launch(attn_fwd_32<DQ, DV, true>, grid, a, s)
                      : launch(attn_fwd_32<DQ, DV, false>, grid, a, s);
    if (dtype == TSD_BF16)
        return causal ? launch(attn_fwd_16<DQ, DV, true, true>, grid, a, s)
                      : launch(attn_fwd_16<DQ, DV, false, true>, grid, a, s);
    return causal ? launch(attn_fwd_16<DQ, DV, true, false>, grid, a, s)
                  : launch(attn_fwd_16<DQ, DV, false, false>, grid, a, s);
}

}  // namespace

#if TSD_UNIT == 0
// f32 grids below this many 128-row blocks take the key-split kernel.
constexpr int64_t kSplitBelow = 512;
TileConfig tile_config(int dtype, int64_t D_qk, int64_t D_v, bool vec, int64_t slices,
                       int64_t S_q, bool causal)
{
    TileConfig t;
    t.dqk_block = pad_dim(D_qk);
    t.dv_block = pad_dim(D_v);
    t.fast = dtype != TSD_F32 && vec;
    // f32: the 128-row kernel runs two workgroups per CU; when it would
    // launch fewer than two per CU, the key-split kernel (32 rows per
    // workgroup) spreads the work over four times as many.
    t.split_keys = dtype == TSD_F32 && slices > 0 &&
                   slices * ((S_q + kBlockM - 1) / kBlockM) < kSplitBelow;
    if (t.fast) {
        const FastShape sh = fast_shape(t.dqk_block, t.dv_block);
        t.block_m = 32 * sh.waves;
        t.waves = sh.waves;
        t.threads = 64 * sh.waves;
        t.block_n = 64;
        const int vslots = (kBar2 && causal && sh.kslots == 4) ? 4 : sh.vslots;
        t.lds_bytes = (sh.kslots * t.dqk_block + vslots * t.dv_block) * 64 * 2;
    } else if (t.split_keys) {
        // widths padded to 64, 96 or 128 (MFMA work grows with the padding)
        t.dqk_block = pad_split(D_qk);
        t.dv_block = pad_split(D_v);
        t.block_m = kSplitRows;
        t.waves = kThreads / 64;
        t.threads = kThreads;
        t.block_n = 32;
        t.lds_bytes = 0;
        static_for<0, 9>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            constexpr int dq = 64 + 32 * (i / 3), dv = 64 + 32 * (i % 3);
            if (t.dqk_block == dq && t.dv_block == dv) t.lds_bytes = 16 * Split32<dq, dv>::LDS_CHUNKS;
        });
    } else if (dtype == TSD_F32) {
        t.block_m = kBlockM;
        t.waves = kThreads / 64;
        t.threads = kThreads;
        t.block_n = 32;
        t.lds_bytes = 2 * (32 * t.dqk_block + 32 * t.dv_block) * 4;
    } else {
        t.block_m = kBlockM;
        t.waves = kThreads / 64;
        t.threads = kThreads;
        t.block_n = 64;
        t.lds_bytes = 2 * (64 * t.dqk_block + t.dv_block * 64) * 2;
    }
    return t;
}

#endif

#if TSD_UNIT == 1
hipError_t launch_attn_ext(const TileConfig &cfg, int dtype, bool causal, bool out_f32,
                           int64_t grid, const KernelArgs &args, hipStream_t stream)
{
    if (!cfg.fast) return hipErrorInvalidValue;
    switch ((cfg.dqk_block == 128 ? 2 : 0) + (cfg.dv_block == 128 ? 1 : 0)) {
    case 0: return dispatch_fast_ext<64, 64>(dtype, causal, out_f32, grid, args, stream);
    case 1: return dispatch_fast_ext<64, 128>(dtype, causal, out_f32, grid, args, stream);
    case 2: return dispatch_fast_ext<128, 64>(dtype, causal, out_f32, grid, args, stream);
    default: return dispatch_fast_ext<128, 128>(dtype, causal, out_f32, grid, args, stream);
    }
}

#endif

#if TSD_UNIT == 2
hipError_t launch_attn_scaled(const TileConfig &cfg, int dtype, bool causal, bool qk8,
                              int64_t grid, const KernelArgs &args, hipStream_t stream)
{
    if (!cfg.fast) return hipErrorInvalidValue;
    switch ((cfg.dqk_block == 128 ? 2 : 0) + (cfg.dv_block == 128 ? 1 : 0)) {
    case 0: return dispatch_fast_scaled<64, 64>(dtype, causal, qk8, grid, args, stream);
    case 1: return dispatch_fast_scaled<64, 128>(dtype, causal, false, grid, args, stream);
    case 2: return dispatch_fast_scaled<128, 64>(dtype, causal, qk8, grid, args, stream);
    default: return dispatch_fast_scaled<128, 128>(dtype, causal, qk8, grid, args, stream);
    }
}

#endif

#if TSD_UNIT == 0
hipError_t launch_merge(int dtype, bool vec, const MergeArgs &args, hipStream_t stream)
{
    const int64_t threads = args.rows * args.groups;
    const int64_t grid = (threads + kMergeThreads - 1) / kMergeThreads;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(kMergeThreads), 0, stream, args);
        return hipGetLastError();
    };
    if (dtype == TSD_F32)
        return vec ? go(attn_merge_kernel<TSD_F32, true>) : go(attn_merge_kernel<TSD_F32, false>);
    if (dtype == TSD_BF16)
        return vec ? go(attn_merge_kernel<TSD_BF16, true>) : go(attn_merge_kernel<TSD_BF16, false>);
    return vec ? go(attn_merge_kernel<TSD_F16, true>) : go(attn_merge_kernel<TSD_F16, false>);
}

hipError_t launch_attn(const TileConfig &cfg, int dtype, bool causal, int64_t grid,
                       const KernelArgs &args, hipStream_t stream)
{
    const int key = (cfg.dqk_block == 128 ? 2 : 0) + (cfg.dv_block == 128 ? 1 : 0);
    if (cfg.split_keys) {
        hipError_t err = hipErrorInvalidValue;
        static_for<0, 9>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            constexpr int dq = 64 + 32 * (i / 3), dv = 64 + 32 * (i % 3);
            if (cfg.dqk_block == dq && cfg.dv_block == dv)
                err = dispatch_split<dq, dv>(causal, grid, args, stream);
        });
        return err;
    }
    if (cfg.fast) {
        switch (key) {
        case 0: return dispatch_fast<64, 64>(dtype, causal, grid, args, stream);
        case 1: return dispatch_fast<64, 128>(dtype, causal, grid, args, stream);
        case 2: return dispatch_fast<128, 64>(dtype, causal, grid, args, stream);
        default: return dispatch_fast<128, 128>(dtype, causal, grid, args, stream);
        }
    }
    switch (key) {
    case 0: return dispatch_causal<64, 64>(dtype, causal, grid, args, stream);
    case 1: return dispatch_causal<64, 128>(dtype, causal, grid, args, stream);
    case 2: return dispatch_causal<128, 64>(dtype, causal, grid, args, stream);
    default: return dispatch_causal<128, 128>(dtype, causal, grid, args, stream);
    }
}

#endif

}  // namespace tsd
