// Internal launchers of the MoE layer kernels (host side).  Not part of the
// C ABI: api.cpp sequences these on the caller's stream.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

enum DType { DT_F32 = 0, DT_BF16 = 1 };
enum Epi { EPI_STORE = 0, EPI_SWIGLU = 1 };
// Tile shapes of the grouped GEMM: SMALL streams weights for a few rows
// per expert (decode-sized batches); LARGE (128 x 256, both operands through
// LDS) and WIDE (128 x 512, weights fed to registers) are the prefill tiles.
// All bf16 prefill tiles are 128 rows, so one tile table serves both.
// WIDE16 is the register-fed tile at 16 x 256 (FP8 decode; bf16 decode runs
// SMALL).  ROUTER is the LDS tile at 128 x 192 for the router logits, in
// 128-byte row pieces and two stages (unpacked fp32-out store only): 384
// experts fill two N tiles exactly.  NARROW is SMALL at 16 x 256, for
// batches so small that the 512-wide tiles would leave most CUs idle.
enum TileCfg { TILE_SMALL = 0, TILE_LARGE = 1, TILE_WIDE = 2, TILE_WIDE16 = 3, TILE_ROUTER = 4, TILE_NARROW = 5 };

int tile_bm(TileCfg cfg);         // rows per M tile
int tile_bn_out(TileCfg cfg, Epi epi);  // output columns per N tile

// One K segment: C += A[:, 0:K] * B[:, 0:K]^T.  A rows have stride lda,
// B (weights, [N, K] row-major) rows have stride ldb; Bu is the up
// projection paired with B for the SwiGLU epilogue.  Strides in elements.
struct GemmSeg {
    const void* A;
    const void* B;
    const void* Bu;
    int64_t lda, ldb;
    int32_t K;
    int32_t pad_;
};

// A family of tiles sharing operands: the routed experts (B offset by
// expert * b_estride) or one dense matrix (the shared experts, a latent
// map, the router).  Row p of the group reads A row rowmap ? rowmap[p] : p
// and writes C row p.
// FP8 weights (launch_gemm_f8): bs / bsu hold the E8M0 exponents of B / Bu
// per 128 x 128 block, [N/128, K/128] per matrix, s_estride bytes apart per
// expert; b_estride is then in bytes (one per element).
struct GemmGroup {
    GemmSeg seg[3];
    int32_t nseg;
    int32_t N;
    int64_t b_estride;
    const int32_t* rowmap;
    void* C;
    int64_t ldc;
    const uint8_t* bs;
    const uint8_t* bsu;
    int64_t s_estride;
};

// One M tile of a grouped GEMM.  `first` and `count` describe the run of
// consecutive tiles that share weights (all tiles of one routed expert, or
// up to 8 tiles of the shared rows); the GEMM walks each run M-tile-fastest
// so those tiles stream every weight slice together.  run_row0 / run_rows
// are the run's rows (tile i of the run: rows run_row0 + i bm ..), so that a
// workgroup finds its tile from any entry of the run with one table load.
struct TileInfo {
    int32_t group, expert, row0, rows;
    int32_t first, count, run_row0, run_rows;
};

// XCD-aware slot map of a tile-table launch.  Blocks go to the eight XCDs
// round robin (block b runs on XCD b % 8).  The active (M tile, N tile)
// pairs are numbered 0 .. total-1, the first total_r of them routed, the
// rest shared-expert pairs; each XCD walks one contiguous stretch of the
// routed pairs, ceil(total_r / 8) long, and then one stretch of the shared
// pairs, ceil((total - total_r) / 8) long.  Returns block b's pair, or -1
// for a block without work.  Every pair has exactly one block as long as
// the grid holds job_blocks(tiles, ntn) blocks for tiles * ntn >= total.
__host__ __device__ inline int xcd_slot_pair(int b, int total_r, int total) {
    const int per = (total_r + 7) >> 3, per_s = (total - total_r + 7) >> 3;
    const int slot = b >> 3, xcd = b & 7;
    if (slot < per) {
        const int lin = xcd * per + slot;
        return lin < total_r ? lin : -1;
    }
    const int k = slot - per, lin = total_r + xcd * per_s + k;
    return (k < per_s && lin < total) ? lin : -1;
}

// Grid of a tile-table launch for up to max_tiles M tiles of ntn N tiles:
// the routed and shared stretches take 8 * (ceil(routed / 8) + ceil(shared
// / 8)) blocks, at most the pairs plus 14, so round the pairs up to a
// multiple of 8 and add 16 (blocks past the active pairs return at once).
inline unsigned job_blocks(int max_tiles, int ntn) {
    const unsigned blocks = static_cast<unsigned>(max_tiles) * static_cast<unsigned>(ntn);
    return ((blocks + 7u) & ~7u) + 16u;
}

struct GemmArgs {
    GemmGroup g[2];
    const TileInfo* tiles;   // device tile table (grouped) or NULL (dense)
    const int32_t* ntiles;   // device counts (grouped): [0] valid tiles, [1] of them routed (group 0)
    int32_t M;               // dense: rows of group 0
    int32_t nsplit;          // split-K ways; output split s at C + s*split_stride
    int64_t split_stride;
    int32_t ntn;             // N tiles per M tile (set by launch_gemm)
};

// Launch C = epi(A * B^T) for element type `dt`; `out_f32` selects an fp32
// output (the router logits) instead of the element type.  `max_tiles` is
// the grid's M extent (upper bound of the device tile count when grouped).
// `packed`: every B is in the fragment-block layout of moe_pack_weights
// (bf16 only); WIDE tiles need it and fall back to LARGE without it.
hipError_t launch_gemm(const GemmArgs& args, DType dt, bool out_f32, Epi epi,
                       TileCfg cfg, int max_tiles, int max_n, bool packed,
                       hipStream_t stream);

// C = epi(A * B^T) with bf16 A and C; group 0 with block-scaled FP8 B
// (16 x 64 fragment blocks of MOE_LAYOUT_FRAG16 for FP8; N and K multiples
// of 128, K <= 8192), group 1 with packed bf16 B; one K segment per group.
// cfg: TILE_WIDE (128-row tiles) or TILE_WIDE16 (16-row tiles).
hipError_t launch_gemm_f8(const GemmArgs& args, Epi epi, TileCfg cfg, int max_tiles, int max_n,
                          hipStream_t stream);

// Row-major [rows, cols] uint8 FP8 matrices -> 16 x 64 blocks of 1 KiB:
// lane l of a block holds columns 8 (l/16) .. + 7 and 32 + 8 (l/16) .. + 7
// of row l % 16.
hipError_t launch_pack_frag16_fp8(const uint8_t* src, uint8_t* dst, int64_t count, int rows, int cols,
                                  hipStream_t stream);

// Row-major [rows, cols] bf16 matrices (count of them, consecutive) -> the
// fragment-block layout: block (rows/16) x (cols/32) of 1 KiB each.
hipError_t launch_pack_frag16(const uint16_t* src, uint16_t* dst, int64_t count, int rows, int cols,
                              hipStream_t stream);

// Quantile Balancing bias from the router logits (nsplit partial planes of
// [T, ldz]): theta_e = n-th largest sigmoid(z[., e]), b_e = mean(theta) -
// theta_e.  theta: E floats of scratch.  T <= kQuantileMaxT (LDS).
constexpr int kQuantileMaxT = 32768;
hipError_t launch_quantile_bias(const float* z, int nsplit, int64_t split_stride, int ldz, int T, int E, int n,
                                float* theta, float* b, hipStream_t stream);

// b[e] += gamma * sgn(mean(counts) - counts[e]) for e < E (E <= 1024).
hipError_t launch_bias_update(const int32_t* counts, int E, float gamma, float* b, hipStream_t stream);

// Router logits z [T, ldz] = x W_r^T for T <= kRouterGemvMaxT tokens (x bf16,
// or fp32 when x_f32), fp32 FMAs on the fp32 weight; one plane (nsplit 1).
constexpr int kRouterGemvMaxT = 32;
hipError_t launch_router_gemv(const void* x, bool x_f32, const float* W, int T, int d, int E, int ldz, float* z,
                              hipStream_t stream);

// W_r (fp32) -> three bf16 planes with hi + mid + lo == W_r exactly.
hipError_t launch_split3(const float* W, int64_t n, uint16_t* hi,
                         uint16_t* mid, uint16_t* lo, hipStream_t stream);

// Sigmoid, biased top-K (limited to the topk_group best of n_group expert
// groups when n_group > 1), renormalise and scale; z holds nsplit partial
// logit planes of [T, ldz].  counts (nullable, E <= 1024) gets the number of
// selections of each expert.
hipError_t launch_topk_gate(const float* z, int nsplit, int64_t split_stride,
                            int ldz, const float* b, int T, int E, int K,
                            int n_group, int topk_group, float scale,
                            int32_t* idx, float* w, int32_t* counts,
                            hipStream_t stream);

hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n,
                           hipStream_t stream);

// Histogram, scan and stable permutation; also the tile table for the
// grouped GEMMs (routed tiles of bm rows, then shared tiles if
// shared_rows > 0) and ntiles[0..1] = (all tiles, routed tiles).  Experts
// e0 .. e0 + E - 1 of idx are dispatched, as local experts 0 .. E - 1; an
// assignment to any other id (another slice's expert) gets pos = -1.
hipError_t launch_dispatch(const int32_t* idx, int T, int E, int e0, int K, int bm,
                           int shared_rows, uint64_t* masks,
                           int32_t* chunk_base, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_token,
                           int32_t* pos, TileInfo* tiles, int32_t* ntiles,
                           hipStream_t stream);

// out[t] = (Yshared ? Yshared[t] : 0) + sum_k w[t,k] * Y[pos[t,k]], over
// the slots with pos >= 0
hipError_t launch_combine(DType dt, const void* Y, int64_t ldy,
                          const void* Yshared, const int32_t* pos,
                          const float* w, int T, int K, int N, void* out,
                          int64_t ldo, hipStream_t stream);

}  // namespace moe
