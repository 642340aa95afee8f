// Token dispatch of the MoE layer: per-expert histogram, exclusive scan and
// a stable permutation of the (token, slot) assignments into
// expert-contiguous order (each expert's tokens ascending), plus the tile
// table the grouped GEMMs walk.  The pages call this step
// dispatch_and_combine without defining it (llm-arch-kb "Kimi K2 MoE",
// section 3 code) and draw it as "run the selected expert FFNs" (K3 essay
// flowchart); the histogram / scan / stable-permute form is this library's.
//
// Determinism without ordering atomics: tokens are cut into chunks of 64
// (one wave).  For every (chunk, expert) a 64-bit mask records which tokens
// of the chunk chose the expert (an OR, whose result does not depend on
// order).  The rank of token t inside expert e is then
//   offsets[e] + sum_{c' < c} popcount(mask[c'][e]) + popcount(mask[c][e] & lanes_below(t)).
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kMaxE = 1024;

// grid: ceil(nch / 4) blocks of 4 waves; wave w owns chunk 4*block + w.
// Expert ids are taken relative to e0; ids outside [e0, e0 + E) are not
// this dispatch's (an expert-parallel slice) and are skipped.
__global__ __launch_bounds__(256) void k_dispatch_masks(const int32_t* __restrict__ idx, int T, int E, int e0, int K,
                                                        int nch, uint64_t* __restrict__ masks) {
    __shared__ unsigned long long sm[4][kMaxE];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = blockIdx.x * 4 + w;
    for (int e = lane; e < E; e += 64) sm[w][e] = 0ull;
    __syncthreads();
    const int t = c * 64 + lane;
    if (c < nch && t < T)
        for (int k = 0; k < K; ++k) {
            const unsigned e = static_cast<unsigned>(idx[static_cast<int64_t>(t) * K + k] - e0);
            if (e < static_cast<unsigned>(E)) atomicOr(&sm[w][e], 1ull << lane);
        }
    __syncthreads();
    if (c < nch)
        for (int e = lane; e < E; e += 64) masks[static_cast<int64_t>(c) * E + e] = sm[w][e];
}

// Block-wide exclusive scan over 1024 threads (16 waves).
__device__ int block_exclusive_scan(int x, int* total, int* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63) sh[w] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int i = 0; i < 16; ++i) {
            const int v = sh[i];
            sh[i] = run;
            run += v;
        }
        sh[16] = run;
    }
    __syncthreads();
    const int res = sh[w] + incl - x;
    *total = sh[16];
    __syncthreads();
    return res;
}

// Per-expert running bases over the chunks: one wave per expert.  Lane l
// takes the chunks [l * cpl, (l + 1) * cpl), sums their token counts, the
// wave scans the lane sums, and each lane writes the exclusive base of its
// chunks in order; lane 63 holds the expert's total.
// grid: ceil(E / 4) blocks of 4 waves; wave w owns expert 4 * block + w.
__global__ __launch_bounds__(256) void k_dispatch_chunk_scan(const uint64_t* __restrict__ masks, int nch, int E,
                                                             int32_t* __restrict__ chunk_base,
                                                             int32_t* __restrict__ counts) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    const int cpl = (nch + 63) / 64;
    const int c0 = lane * cpl, c1 = min(nch, c0 + cpl);
    int mine = 0;
    for (int c = c0; c < c1; ++c) mine += __popcll(masks[static_cast<int64_t>(c) * E + e]);
    int incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    int base = incl - mine;
    for (int c = c0; c < c1; ++c) {
        chunk_base[static_cast<int64_t>(c) * E + e] = base;
        base += __popcll(masks[static_cast<int64_t>(c) * E + e]);
    }
    if (lane == 63) counts[e] = incl;
}

// One block of 1024 threads; thread e owns expert e (its count from
// k_dispatch_chunk_scan).
__global__ __launch_bounds__(1024) void k_dispatch_scan(int E, int bm, int shared_rows,
                                                        int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                        TileInfo* __restrict__ tiles, int32_t* __restrict__ ntiles) {
    __shared__ int sh[17];
    const int e = threadIdx.x;
    const int cnt = e < E ? counts[e] : 0;
    int total = 0, ttotal = 0;
    const int off = block_exclusive_scan(cnt, &total, sh);
    const int nt = (cnt + bm - 1) / bm;
    const int toff = block_exclusive_scan(nt, &ttotal, sh);
    if (e < E) {
        offsets[e] = off;
        for (int j = 0; j < nt; ++j) {
            TileInfo ti;
            ti.group = 0;
            ti.expert = e;
            ti.row0 = off + j * bm;
            ti.rows = min(bm, cnt - j * bm);
            ti.first = toff;
            ti.count = nt;
            ti.run_row0 = off;
            ti.run_rows = cnt;
            tiles[toff + j] = ti;
        }
    }
    if (e == 0) offsets[E] = total;
    const int nsh = shared_rows > 0 ? (shared_rows + bm - 1) / bm : 0;
    constexpr int kSharedRun = 8;  // shared-row tiles walked together
    for (int j = threadIdx.x; j < nsh; j += blockDim.x) {
        TileInfo ti;
        ti.group = 1;
        ti.expert = 0;
        ti.row0 = j * bm;
        ti.rows = min(bm, shared_rows - j * bm);
        ti.first = ttotal + (j / kSharedRun) * kSharedRun;
        ti.count = min(kSharedRun, nsh - (j / kSharedRun) * kSharedRun);
        ti.run_row0 = (j / kSharedRun) * kSharedRun * bm;
        ti.run_rows = min(kSharedRun * bm, shared_rows - ti.run_row0);
        tiles[ttotal + j] = ti;
    }
    if (threadIdx.x == 0) {
        ntiles[0] = ttotal + nsh;
        ntiles[1] = ttotal;
    }
}

__global__ __launch_bounds__(1024) void k_fill_counts_zero(int32_t* __restrict__ counts, int E) {
    if (static_cast<int>(threadIdx.x) < E) counts[threadIdx.x] = 0;
}

__global__ __launch_bounds__(256) void k_dispatch_scatter(const int32_t* __restrict__ idx, int T, int E, int e0, int K,
                                                          int nch, const uint64_t* __restrict__ masks,
                                                          const int32_t* __restrict__ chunk_base,
                                                          const int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_token,
                                                          int32_t* __restrict__ pos) {
    const int lane = threadIdx.x & 63;
    const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int t = c * 64 + lane;
    if (c >= nch || t >= T) return;
    const uint64_t below = (1ull << lane) - 1ull;
    for (int k = 0; k < K; ++k) {
        const int64_t a = static_cast<int64_t>(t) * K + k;
        const int e = idx[a] - e0;
        if (static_cast<unsigned>(e) >= static_cast<unsigned>(E)) {  // another slice's expert
            pos[a] = -1;
            continue;
        }
        const int64_t ce = static_cast<int64_t>(c) * E + e;
        const int p = offsets[e] + chunk_base[ce] + __popcll(masks[ce] & below);
        sorted_token[p] = t;
        pos[a] = p;
    }
}

// The combine reads every row of Y and Ysh exactly once: non-temporal
// loads keep those 2 GB (prefill) from displacing cached lines on the way.
// At T = 16384 this measured 0.43 ms against 0.48 ms.
__device__ __forceinline__ void unpack8_once(const bf16_t* p, float (&o)[8]) {
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(v[i] << 16);
        o[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack8_once(const float* p, float (&o)[8]) { unpack8(p, o); }

template <typename T>
__global__ __launch_bounds__(256) void k_combine(const T* __restrict__ Y, int64_t ldy, const T* __restrict__ Ysh,
                                                 const int32_t* __restrict__ pos, const float* __restrict__ w, int K,
                                                 int N, T* __restrict__ out, int64_t ldo) {
    const int t = blockIdx.x;
    for (int c = threadIdx.x; c < N / 8; c += 256) {
        float acc[8];
        if (Ysh) {
            unpack8_once(Ysh + static_cast<int64_t>(t) * ldy + c * 8, acc);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        }
        for (int k = 0; k < K; ++k) {
            const int p = pos[static_cast<int64_t>(t) * K + k];
            if (p < 0) continue;  // an expert of another slice
            const float wk = w[static_cast<int64_t>(t) * K + k];
            float y[8];
            unpack8_once(Y + static_cast<int64_t>(p) * ldy + c * 8, y);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += wk * y[e];
        }
        pack8(out + static_cast<int64_t>(t) * ldo + c * 8, acc);
    }
}

}  // namespace

hipError_t launch_dispatch(const int32_t* idx, int T, int E, int e0, int K, int bm, int shared_rows, uint64_t* masks,
                           int32_t* chunk_base, int32_t* counts, int32_t* offsets, int32_t* sorted_token, int32_t* pos,
                           TileInfo* tiles, int32_t* ntiles, hipStream_t stream) {
    const int nch = (T + 63) / 64;
    const dim3 g4((nch + 3) / 4);
    if (nch > 0) {
        hipLaunchKernelGGL(k_dispatch_masks, g4, dim3(256), 0, stream, idx, T, E, e0, K, nch, masks);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (nch > 0) {
        hipLaunchKernelGGL(k_dispatch_chunk_scan, dim3((E + 3) / 4), dim3(256), 0, stream, masks, nch, E, chunk_base,
                           counts);
    } else {
        hipLaunchKernelGGL(k_fill_counts_zero, dim3(1), dim3(1024), 0, stream, counts, E);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_dispatch_scan, dim3(1), dim3(1024), 0, stream, E, bm, shared_rows, counts, offsets, tiles,
                       ntiles);
    err = hipGetLastError();
    if (err != hipSuccess || nch == 0) return err;
    hipLaunchKernelGGL(k_dispatch_scatter, g4, dim3(256), 0, stream, idx, T, E, e0, K, nch, masks, chunk_base,
                       offsets, sorted_token, pos);
    return hipGetLastError();
}

hipError_t launch_combine(DType dt, const void* Y, int64_t ldy, const void* Yshared, const int32_t* pos, const float* w,
                          int T, int K, int N, void* out, int64_t ldo, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    if (dt == DT_F32)
        hipLaunchKernelGGL(k_combine<float>, dim3(T), dim3(256), 0, stream, static_cast<const float*>(Y), ldy,
                           static_cast<const float*>(Yshared), pos, w, K, N, static_cast<float*>(out), ldo);
    else
        hipLaunchKernelGGL(k_combine<bf16_t>, dim3(T), dim3(256), 0, stream, static_cast<const bf16_t*>(Y), ldy,
                           static_cast<const bf16_t*>(Yshared), pos, w, K, N, static_cast<bf16_t*>(out), ldo);
    return hipGetLastError();
}

}  // namespace moe
