// Internal interface between the host-side planner (attn_api.hip) and the
// gfx950 kernels (attn_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsd_attn.h"

namespace tsd {

// Kernel arguments (passed by value).  Pointers address slice 0; the kernel
// adds the slice offset itself.
struct KernelArgs {
    const void *Q;
    const void *K;
    const void *V;
    void *O;
    float *LSE;        // may be null
    int32_t S_q, S_k, D_qk, D_v;
    int32_t q_blocks;  // per slice
    int32_t slices;    // B * H
    int32_t order;     // block order, see map_block
    int32_t per_xcd;   // slices per XCD when order == 1
    float c;           // |scale| * log2(e); 1 when scale == 0
    uint32_t q_xor;    // XOR applied to every Q storage word (sign flip)
    uint32_t q_and;    // AND applied to every Q storage word (0 zeroes Q)
    int32_t vec;       // 1: 16-byte global accesses are legal
    // Key visibility of the extended kernels (see KeyRange); the plain
    // kernels use kv_begin = 0, kv_end = S_k, coff = 0, window = 0.
    int32_t kv_begin, kv_end;   // key range [kv_begin, kv_end)
    int32_t coff;               // causal: key j visible iff j <= i + coff
    int32_t window;             // > 0: also j > i + coff - window
    int32_t splits;             // key range cut into `splits` chunks ...
    int32_t split_len;          // ... of split_len keys (a multiple of 64)
    int64_t part_o_stride;      // elements between consecutive chunks' O (f32 output)
    int64_t part_lse_stride;    // elements between consecutive chunks' LSE
    int32_t q_per_head;         // row r of a slice is query position r % q_per_head (grouped
                                // heads: a slice holds the rows of every query head that
                                // shares its K/V head); S_q when each slice is one head
    // Per-block scales of the scaled kernels (null otherwise): Q_scale
    // [slices][q_scale_blocks], one per q_block rows; K_scale
    // [slices][k_scale_blocks], one per k_tiles_per_block 64-key tiles.
    const float *Q_scale;
    const float *K_scale;
    int32_t q_block, q_scale_blocks, k_tiles_per_block, k_scale_blocks;
};

// Keys a workgroup of query positions [q0, q_end) sees inside the key range
// [klo, khi): position i sees [max(klo, i + coff - window + 1) (window > 0),
// min(khi, i + coff + 1) (causal)); the workgroup's span is the union,
// [key_lo, key_hi) (empty when key_hi <= key_lo).
struct KeyRange {
    int32_t key_lo, key_hi;
};
__host__ __device__ inline KeyRange wg_key_range(int32_t q0, int32_t q_end, int32_t klo,
                                                 int32_t khi, bool causal, int32_t coff,
                                                 int32_t window)
{
    int64_t lo = klo, hi = khi;
    if (window > 0 && (int64_t)q0 + coff - window + 1 > lo) lo = (int64_t)q0 + coff - window + 1;
    if (causal && (int64_t)q_end - 1 + coff + 1 < hi) hi = (int64_t)q_end - 1 + coff + 1;
    if (hi < lo) hi = lo;
    return KeyRange{(int32_t)lo, (int32_t)hi};
}

// Query positions (inclusive) of rows [r0, r1) of a slice whose rows are
// heads x positions, qph positions per head: where the rows run into the
// next head the range is every position.
struct PosRange {
    int32_t lo, hi;
};
__host__ __device__ inline PosRange row_positions(int32_t r0, int32_t r1, int32_t qph)
{
    const int32_t p0 = r0 % qph, p1 = (r1 - 1) % qph;
    if (r1 - r0 >= qph || p1 < p0) return PosRange{0, qph - 1};
    return PosRange{p0, p1};
}

// Workgroup index -> (query block, slice).
//
// Query blocks are issued heaviest first when causal (the last query block
// visits the most key tiles).  With order == 1 the slices are grouped so
// that every workgroup of one slice lands on the same XCD: the dispatcher
// hands consecutive workgroup ids to the 8 XCDs in turn, so id % 8 selects
// the XCD and each XCD walks its own slices, keeping a slice's K/V tiles in
// that XCD's L2.
__host__ __device__ inline void map_block(int32_t block, int32_t q_blocks, int32_t slices,
                                          int32_t order, int32_t per_xcd, bool heaviest_first,
                                          int32_t &q_block, int32_t &slice)
{
    int32_t rank;
    if (order == 1) {
        const int32_t xcd = block & 7;
        const int32_t j = block >> 3;
        rank = j / per_xcd;
        slice = (j - rank * per_xcd) * 8 + xcd;
    } else {
        rank = block / slices;
        slice = block - rank * slices;
    }
    q_block = heaviest_first ? (q_blocks - 1 - rank) : rank;
}

// Key tiles visited by query block `q_block`: all tiles, or, when causal,
// those holding a key <= the block's last valid query.
__host__ __device__ inline int32_t kv_tiles_for(int32_t q_block, int32_t block_m, int32_t block_n,
                                                int32_t S_q, int32_t S_k, bool causal)
{
    int32_t kv_len = S_k;
    if (causal) {
        int32_t q_last = (q_block + 1) * block_m;
        if (q_last > S_q) q_last = S_q;
        if (q_last < kv_len) kv_len = q_last;   // keys 0 .. q_last-1
    }
    return (kv_len + block_n - 1) / block_n;
}

// Fill the kernel's tile configuration for a dtype (shared by the planner
// and the launcher so both agree).
struct TileConfig {
    int32_t block_m, block_n, waves, threads, dqk_block, dv_block, lds_bytes;
    bool fast;         // 16-byte aligned 16-bit inputs: the LDS-direct kernel
    bool split_keys;   // f32 on a small grid: 32 rows per workgroup, the
                       // waves splitting the key tiles
};

// `slices` and `S_q` size the grid (0: not known, no key split).
// `causal` only changes the reported LDS size (causal launches of the
// 8-wave shape keep four V tiles).
TileConfig tile_config(int dtype, int64_t D_qk, int64_t D_v, bool vec, int64_t slices = 0,
                       int64_t S_q = 0, bool causal = false);

// Launch the kernel that matches (dtype, dqk_block, dv_block, causal).
hipError_t launch_attn(const TileConfig &cfg, int dtype, bool causal, int64_t grid,
                       const KernelArgs &args, hipStream_t stream);

// The extended form of the LDS-direct kernel (key range, offset, window,
// key chunks; 16-bit or f32 output).  Grid: q_blocks * slices * splits.
hipError_t launch_attn_ext(const TileConfig &cfg, int dtype, bool causal, bool out_f32,
                           int64_t grid, const KernelArgs &args, hipStream_t stream);

// Arguments of the merge of partial results over key chunks.
struct MergeArgs {
    const float *O_parts;     // [n_parts][rows][D_v] f32, chunk j at j * part_o_stride
    const float *LSE_parts;   // [n_parts][rows] f32, chunk j at j * part_lse_stride
    void *O;                  // [rows][D_v] of the output dtype
    float *LSE;               // [rows] or null
    int64_t rows;             // B * H * S_q
    int64_t part_o_stride, part_lse_stride;
    int32_t D_v, n_parts;
    int32_t groups;           // ceil(D_v / 4) threads per row
};

// The per-block scaled form of the LDS-direct kernel (base-2 weights; Q and
// K in `dtype` or, with qk8, fp8 e4m3).  qk8 needs a Q/K block of 128, or 64
// with a V block of 64.
hipError_t launch_attn_scaled(const TileConfig &cfg, int dtype, bool causal, bool qk8,
                              int64_t grid, const KernelArgs &args, hipStream_t stream);

// vec: D_v % 4 == 0 and the buffers allow 16-byte (f32) / 8-byte (16-bit) access.
hipError_t launch_merge(int dtype, bool vec, const MergeArgs &args, hipStream_t stream);

}  // namespace tsd
