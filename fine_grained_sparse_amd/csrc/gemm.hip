// Grouped GEMM on gfx950 MFMA for the MoE layer: C = epi(A * B^T) over a
// table of tiles.
//   - routed experts: each tile is up to BM consecutive rows of the
//     expert-sorted assignment space; A rows are gathered through a row map
//     (sorted position -> token) while they are loaded, B is that expert's
//     [N, K] weight matrix;
//   - dense groups (shared experts, latent maps, router): plain row tiles.
// The SwiGLU epilogue computes H = silu(A Wg^T) * (A Wu^T) with the gate and
// up columns held by the same lanes (the expert form of the llm-arch-kb
// "Kimi K2 MoE" entry, section 2: three matrices per expert).
//
// Three kernels:
//   k_gemm       fp32 operands (small parity workloads): register-staged
//                16 x 256 tiles, four v_mfma_f32_16x16x4_f32 per fragment.
//   k_gemm_big   bf16, both operands DMA'd into an LDS ring
//                (global_load_lds_dwordx4): 16 x 512 and 16 x 256 decode
//                tiles, 128 x 256 prefill tiles on row-major weights,
//                128 x 192 router-logit tiles.
//   k_gemm_wide  bf16 activations on packed weights: 128 x 512 prefill tiles,
//                A through LDS, each wave's weight fragments straight into
//                registers; its FP8 form also at 16 x 256 (decode).
// One 64-byte K slab feeds one v_mfma_f32_16x16x32_bf16 per 16x16 block; a
// lane supplies row lane % 16 and the 16-byte K chunk lane / 16 of it.
#include "common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace moe {

int tile_bm(TileCfg cfg);
int tile_bn_out(TileCfg cfg, Epi epi);

namespace {

constexpr int kStageRowBytes = 128;
constexpr int kLdsRowBytes = 144;  // 16 bytes of padding against bank conflicts

__device__ __forceinline__ const GemmSeg& seg_of(const GemmGroup& G, int s) {
    return s == 0 ? G.seg[0] : (s == 1 ? G.seg[1] : G.seg[2]);
}

template <typename T, typename TC, int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(256) void k_gemm(const GemmArgs a) {
    constexpr int ES = sizeof(T);
    constexpr int BKE = kStageRowBytes / ES;  // K elements per stage
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int MB = TM / 16, NB = TN / 16;
    constexpr int BNO = EPI == EPI_SWIGLU ? BN / 2 : BN;
    constexpr int A_CH = BM * 8, B_CH = BN * 8;  // 16-byte chunks per stage
    constexpr int LA = (A_CH + 255) / 256, LB = B_CH / 256;
    constexpr int STAGE = (BM + BN) * kLdsRowBytes;
    constexpr int EP_STRIDE = BNO + 4;
    constexpr int LDS_BYTES = (2 * STAGE > BM * EP_STRIDE * 4) ? 2 * STAGE : BM * EP_STRIDE * 4;
    static_assert(WM * WN == 4, "four waves");
    static_assert(B_CH % 256 == 0, "B tile chunks");
    static_assert(EPI != EPI_SWIGLU || NB % 2 == 0, "gate/up pairs per wave");
    __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid / WN, wn = wid % WN;

    // ---- which tile: linear block id -> (M tile, N tile), N fastest, so
    // the workgroups that share an A tile are launched together and the
    // M tiles of one expert read each weight tile on the same XCD when the
    // N-tile count is a multiple of the eight XCDs.
    int gi = 0, expert = 0, row0, rows;
    const int mt = static_cast<int>(blockIdx.x) / a.ntn;
    const int nt_n = static_cast<int>(blockIdx.x) % a.ntn;
    if (a.tiles) {
        if (mt >= *a.ntiles) return;
        const TileInfo ti = a.tiles[mt];
        gi = ti.group;
        expert = ti.expert;
        row0 = ti.row0;
        rows = ti.rows;
    } else {
        row0 = mt * BM;
        rows = min(BM, a.M - row0);
        if (rows <= 0) return;
    }
    const GemmGroup& G = gi ? a.g[1] : a.g[0];
    const int N = G.N;
    const int n0 = nt_n * BNO;
    if (n0 >= N) return;

    // ---- split-K range over the concatenated segments
    int nk = 0;
    for (int s = 0; s < G.nseg; ++s) nk += seg_of(G, s).K / BKE;
    const int chunk = (nk + a.nsplit - 1) / a.nsplit;
    const int kt0 = min(nk, static_cast<int>(blockIdx.z) * chunk);
    const int kt1 = min(nk, kt0 + chunk);

    // ---- per-thread source rows
    int arow[LA];
    int achunk[LA];
    bool aval[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int c = tid + i * 256;
        aval[i] = c < A_CH;
        const int r = aval[i] ? (c >> 3) : 0;
        const int p = row0 + (r < rows ? r : 0);
        arow[i] = G.rowmap ? G.rowmap[p] : p;
        achunk[i] = c & 7;
    }
    int bn_[LB];
    bool bup[LB];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int c = tid + i * 256;
        const int q = c >> 3;
        int n;
        if (EPI == EPI_SWIGLU) {
            const int blk = q / TN, rq = q % TN, half = TN / 2;
            n = n0 + blk * half + (rq % half);
            bup[i] = rq >= half;
        } else {
            n = n0 + q;
            bup[i] = false;
        }
        bn_[i] = n < N ? n : N - 1;
    }

    // ---- global load cursor (segment s, step kk within it)
    int cs = 0, ck = kt0;
    while (cs + 1 < G.nseg && ck >= seg_of(G, cs).K / BKE) {
        ck -= seg_of(G, cs).K / BKE;
        ++cs;
    }
    const char* ap[LA];
    const char* bp[LB];
    auto set_ptrs = [&](int s) {
        const GemmSeg& S = seg_of(G, s);
        const int64_t eoff = s == 0 ? static_cast<int64_t>(expert) * G.b_estride : 0;
#pragma unroll
        for (int i = 0; i < LA; ++i)
            ap[i] = static_cast<const char*>(S.A) + (static_cast<int64_t>(arow[i]) * S.lda) * ES + achunk[i] * 16;
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            const void* base = bup[i] ? S.Bu : S.B;
            bp[i] = static_cast<const char*>(base) + (eoff + static_cast<int64_t>(bn_[i]) * S.ldb) * ES + ((tid + i * 256) & 7) * 16;
        }
    };
    set_ptrs(cs);

    uint4 ra[LA], rb[LB];
    auto gload = [&]() {
        const int64_t off = static_cast<int64_t>(ck) * kStageRowBytes;
#pragma unroll
        for (int i = 0; i < LA; ++i)
            if (aval[i]) ra[i] = ldg16(ap[i] + off);
#pragma unroll
        for (int i = 0; i < LB; ++i) rb[i] = ldg16(bp[i] + off);
        ++ck;
        if (cs + 1 < G.nseg && ck == seg_of(G, cs).K / BKE) {
            ++cs;
            ck = 0;
            set_ptrs(cs);
        }
    };
    auto lstore = [&](int stage) {
        char* As = lds + stage * STAGE;
        char* Bs = As + BM * kLdsRowBytes;
#pragma unroll
        for (int i = 0; i < LA; ++i)
            if (aval[i]) {
                const int c = tid + i * 256;
                *reinterpret_cast<uint4*>(As + (c >> 3) * kLdsRowBytes + (c & 7) * 16) = ra[i];
            }
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            const int c = tid + i * 256;
            *reinterpret_cast<uint4*>(Bs + (c >> 3) * kLdsRowBytes + (c & 7) * 16) = rb[i];
        }
    };

    f32x4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int frow = lane & 15;
    const int fcol = (lane >> 4) * 16;
    if (kt0 < kt1) {
        gload();
        lstore(0);
        __syncthreads();
        for (int kt = kt0; kt < kt1; ++kt) {
            const int cur = (kt - kt0) & 1;
            const bool more = kt + 1 < kt1;
            if (more) gload();
            const char* As = lds + cur * STAGE;
            const char* Bs = As + BM * kLdsRowBytes;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                uint4 fa[MB], fb[NB];
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    fa[i] = *reinterpret_cast<const uint4*>(As + (wm * TM + i * 16 + frow) * kLdsRowBytes + s * 64 + fcol);
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    fb[j] = *reinterpret_cast<const uint4*>(Bs + (wn * TN + j * 16 + frow) * kLdsRowBytes + s * 64 + fcol);
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int j = 0; j < NB; ++j) acc[i][j] = Mfma<T>::run(fa[i], fb[j], acc[i][j]);
            }
            if (more) lstore(cur ^ 1);
            __syncthreads();
        }
    }

    // ---- epilogue: accumulators -> LDS tile (fp32) -> coalesced stores.
    // MFMA 16x16 output layout: lane l holds rows 4*(l/16)+r, column l%16.
    float* ep = reinterpret_cast<float*>(lds);
    if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB / 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = wm * TM + i * 16 + (lane >> 4) * 4 + r;
                    const int col = wn * (TN / 2) + j * 16 + (lane & 15);
                    const float g = acc[i][j][r], u = acc[i][j + NB / 2][r];
                    ep[row * EP_STRIDE + col] = g / (1.0f + expf(-g)) * u;
                }
    } else {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = wm * TM + i * 16 + (lane >> 4) * 4 + r;
                    const int col = wn * TN + j * 16 + (lane & 15);
                    ep[row * EP_STRIDE + col] = acc[i][j][r];
                }
    }
    __syncthreads();
    constexpr int CPR = BNO / 8;
    TC* C = static_cast<TC*>(G.C) + static_cast<int64_t>(blockIdx.z) * a.split_stride;
    for (int c = tid; c < BM * CPR; c += 256) {
        const int r = c / CPR, cc = c % CPR;
        const int col = n0 + cc * 8;
        if (r >= rows || col >= N) continue;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = ep[r * EP_STRIDE + cc * 8 + e];
        TC* dst = C + static_cast<int64_t>(row0 + r) * G.ldc + col;
        if (col + 8 <= N) {
            pack8(dst, v);
        } else {
            for (int e = 0; e < N - col; ++e) dst[e] = Elem<TC>::from_f32(v[e]);
        }
    }
}

// ---------------------------------------------------------------------------
// Prefill-sized tiles: 128 x 256 (B rows) per workgroup, 64 x 128 per wave,
// so each wave issues 32 MFMAs per 64-byte K slab.
//
// Operands go from global memory straight into LDS with gfx950's
// global_load_lds_dwordx4: a wave's instruction moves 64 x 16 B into one
// contiguous 1 KiB LDS block (lane i at byte 16 i; the LDS address comes
// from M0).  Three LDS stages: while stage k is read by the MFMA loop, the
// loads of stages k+1 and k+2 are in flight, so about two compute steps of
// memory latency are hidden with one workgroup (4 waves, one per SIMD) per
// CU and no registers holding tiles in flight.
// A stage holds 128 bytes (64 bf16) of every tile row; a 1 KiB block holds
// 8 rows.  The 16-byte chunks of row r sit XOR-swizzled (logical chunk c at
// position c ^ (r & 7)) so the fragment reads of 16 consecutive rows do not
// collide in LDS banks; lane i of a block therefore loads logical chunk
// (i & 7) ^ (i >> 3) of row i >> 3.
// The DMA is issued from inline assembly: the compiler then does not treat
// it as a pending LDS write (which would make it wait for every load in
// flight before each LDS read).  Completion is ordered explicitly: each
// wave waits until only the newer stage's loads are outstanding, then the
// workgroup barrier publishes every wave's blocks.
//
// Workgroup -> tile: the device tile count gives the number of active
// (M tile, N tile) pairs; XCD x (= block id mod 8) takes the x-th
// contiguous share of them in the logical order below, so the M tiles of
// one expert that share each weight slice run side by side on one XCD and
// fetch the slice from HBM once.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// The same wait as a hard scheduling fence: no instruction moves across it.
// Needed wherever it guards registers written by untracked loads, which the
// compiler would otherwise read (an MFMA) or reuse (after their last use)
// on its side of the wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt_fenced() {
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<N>();
    __builtin_amdgcn_sched_barrier(0);
}

// 16 FP8 E4M3FN codes (two 8-code K chunks) -> two bf16 fragments of 8,
// each code times `scale` (a power of two: the product is exact).
__device__ __forceinline__ void fp8x16_to_bf16(uint4 q, float scale, uint4& lo, uint4& hi) {
#define MOE_CVT(w, upper) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, upper))
    lo = make_uint4(MOE_CVT(q.x, false), MOE_CVT(q.x, true), MOE_CVT(q.y, false), MOE_CVT(q.y, true));
    hi = make_uint4(MOE_CVT(q.z, false), MOE_CVT(q.z, true), MOE_CVT(q.w, false), MOE_CVT(q.w, true));
#undef MOE_CVT
}

// Scheduling hint for a region holding NM MFMAs and about NV VALU
// instructions: alternate one MFMA with a share of the VALU work, so the
// VALU instructions issue while the matrix pipe is busy.
template <int NM, int NV>
__device__ __forceinline__ void interleave() {
#pragma unroll
    for (int k = 0; k < NM; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, (NV + NM - 1) / NM, 0);
    }
}

// 16 bytes per lane from base + voff (base wave-uniform), issued as inline
// assembly: the compiler does not count it, so the caller waits for it with
// an explicit vmcnt that also counts the A DMA loads in flight.  (Counted by
// the compiler, its waits would leave out those DMA loads and hold each MFMA
// until loads issued after its operand had landed too.)
__device__ __forceinline__ uint4 gload16_untracked(const char* base, uint32_t voff) {
    uint4 v;
    asm volatile("global_load_dwordx4 %0, %1, %2" : "=v"(v) : "v"(voff), "s"(base));
    return v;
}

__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(src) : "memory", "m0");
}
// A 16-byte load with the non-temporal hint, for data read once (the FP8
// decode tiles' weight codes: 1.91-1.96 -> 1.77 ms for the K2 up launch).
__device__ __forceinline__ uint4 gload16_once(const char* p) {
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// The same with the non-temporal hint, for data read once: the decode
// tiles' packed expert weights (each routed expert's slice is streamed by
// one 16-row tile).  Keeping them from displacing cached lines measured
// 3% off the K2 decode layer (5.39 vs 5.54 ms).
__device__ __forceinline__ void lds_dma16_once(const void* src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds_addr), "v"(src) : "memory", "m0");
}

// LDS swizzle of a row's 16-byte chunks (position = chunk ^ swz(row)).
// ds_read_b128 serves 8 lanes per cycle: 8 consecutive rows at one logical
// chunk must land on 8 different 16-byte bank groups of a 128-byte line.
// 128-byte rows: chunk ^ (row & 7).  64-byte rows (two per line): the line
// half is row & 1, so the chunk is flipped by (row >> 1) & 3.
template <int ROWB>
__device__ __forceinline__ int swz(int row) {
    return ROWB == 128 ? (row & 7) : ((row >> 1) & 3);
}

// Which (M tile, N tile) pair a block computes.  Blocks go to the eight
// XCDs round robin (block b runs on XCD b % 8), so block b takes logical
// slot (b % 8) * per + b / 8: each XCD walks one contiguous stretch of the
// logical order.  That order is: runs of tiles that share weights (one
// expert, or up to 8 dense row tiles), inside a run N tile by N tile with
// the M tile fastest.  A run of `cnt` tiles starting at tile `first`
// occupies slots [first*ntn, (first+cnt)*ntn), so slot / ntn names a tile of
// the run that owns the slot.  With a tile table the routed slots and the
// shared-expert slots (the table's tail) are split across the XCDs
// separately, each XCD walking a stretch of either: the shared tiles re-read
// one weight matrix per run and would otherwise all land on the last XCD.
// The grid holds 8 * (per_routed + per_shared) blocks or more (launch
// grids carry 16 spare blocks).  Returns false for blocks without work.
struct Job {
    int gi, expert, row0, rows, n0;
};

// With a tile table, BM is the table's rows per tile (the planner builds the
// table for the kernels that walk it), and the job comes from one load of
// the entry at slot / ntn, whose run fields place every tile of its run;
// the two tile counts come in one load.
template <int BM, int BNO>
__device__ __forceinline__ bool pick_job(const GemmArgs& a, Job& jb) {
    int total, total_r;  // active (M, N) tile pairs, and the routed ones among them
    if (a.tiles) {
        const int2 nt = *reinterpret_cast<const int2*>(a.ntiles);
        total = nt.x * a.ntn;
        total_r = nt.y * a.ntn;
    } else {
        total = total_r = ((a.M + BM - 1) / BM) * a.ntn;
    }
    const int lin = xcd_slot_pair(static_cast<int>(blockIdx.x), total_r, total);
    if (lin < 0) return false;
    if (a.tiles) {
        const TileInfo t0 = a.tiles[lin / a.ntn];
        const int u = lin - t0.first * a.ntn, i = u % t0.count;
        jb.gi = t0.group;
        jb.expert = t0.expert;
        jb.row0 = t0.run_row0 + i * BM;
        jb.rows = min(BM, t0.run_rows - i * BM);
        jb.n0 = (u / t0.count) * BNO;
    } else {
        const int mtiles = total / a.ntn;
        const int first = (lin / a.ntn) & ~7, cnt = min(8, mtiles - first);
        const int u = lin - first * a.ntn;
        jb.gi = 0;
        jb.expert = 0;
        jb.row0 = (first + u % cnt) * BM;
        jb.rows = min(BM, a.M - jb.row0);
        if (jb.rows <= 0) return false;
        jb.n0 = (u / cnt) * BNO;
    }
    return jb.n0 < (jb.gi ? a.g[1].N : a.g[0].N);
}

// Accumulators -> C.  Wave (wm, wn) holds output block rows wm*TM + 16 i +
// 4 (lane / 16) + r, columns wn*TN + 16 j + lane % 16 (for SwiGLU, block
// columns j < NB/2 are the gate and j + NB/2 the matching up columns, and
// the output column is wn*TN/2 + 16 j + lane % 16).  The fp32 tile goes
// through LDS in column passes of WP and leaves as 16-byte row stores.
template <typename TC, int EPI, int BM, int BNO, int TM, int TN, int MB, int NB, int WP, int NT>
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[MB][NB], char* lds, int wm, int wn, const GemmGroup& G,
                                           TC* C, int row0, int rows, int n0) {
    constexpr int NP = BNO / WP, EP_STRIDE = WP + 4, CPR = WP / 8;
    static_assert(BNO % WP == 0 && WP % 8 == 0, "epilogue passes");
    const int tid = threadIdx.x, lane = tid & 63;
    const int N = G.N;
    float* ep = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
        __syncthreads();
        if (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB / 2; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = wm * TM + i * 16 + (lane >> 4) * 4 + r;
                        const int col = wn * (TN / 2) + j * 16 + (lane & 15) - pass * WP;
                        if (col >= 0 && col < WP) {
                            const float g = acc[i][j][r], u = acc[i][j + NB / 2][r];
                            ep[row * EP_STRIDE + col] = g / (1.0f + expf(-g)) * u;
                        }
                    }
        } else {
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = wm * TM + i * 16 + (lane >> 4) * 4 + r;
                        const int col = wn * TN + j * 16 + (lane & 15) - pass * WP;
                        if (col >= 0 && col < WP) ep[row * EP_STRIDE + col] = acc[i][j][r];
                    }
        }
        __syncthreads();
        for (int c = tid; c < BM * CPR; c += NT) {
            const int r = c / CPR, cc = c % CPR;
            const int col = n0 + pass * WP + cc * 8;
            if (r >= rows || col >= N) continue;
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = ep[r * EP_STRIDE + cc * 8 + e];
            TC* dst = C + static_cast<int64_t>(row0 + r) * G.ldc + col;
            if (col + 8 <= N) {
                pack8(dst, v);
            } else {
                for (int e = 0; e < N - col; ++e) dst[e] = Elem<TC>::from_f32(v[e]);
            }
        }
    }
}

// Workgroups per CU the LDS ring allows (two when a ring fits in 80 KiB).
template <int BM, int BN, int NST, int ROWB>
constexpr int big_occupancy() {
    return NST * (BM + BN) * ROWB <= 81920 ? 2 : 1;
}

template <typename TC, int BM, int BN, int WM, int WN, int NST, int ROWB, int EPI, bool PK>
__global__ __launch_bounds__(64 * WM * WN, (big_occupancy<BM, BN, NST, ROWB>())) void k_gemm_big(const GemmArgs a) {
    using T = bf16_t;
    constexpr int ES = 2;
    static_assert(ROWB == 64 || ROWB == 128, "bytes of a row per stage");
    constexpr int BKE = ROWB / ES;
    constexpr int SLABS = ROWB / 64;           // 64-byte K slabs per stage
    constexpr int CHUNKS = ROWB / 16;          // 16-byte chunks per row
    constexpr int RPB = 1024 / ROWB;           // rows per 1 KiB block
    constexpr int NW = WM * WN;               // waves per workgroup
    constexpr int NT = 64 * NW;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int MB = TM / 16, NB = TN / 16;
    constexpr int BNO = EPI == EPI_SWIGLU ? BN / 2 : BN;
    constexpr int NA = BM / RPB, NBB = BN / RPB;  // 1 KiB blocks of A and of B per stage
    // A blocks are split across the waves, or (fewer A blocks than waves,
    // small row tiles) loaded by every wave: the copies carry identical
    // bytes to identical LDS addresses.  B blocks are split across waves.
    constexpr bool A_ALL = NA < NW;
    constexpr int LPA = A_ALL ? NA : NA / NW;
    constexpr int LPW = LPA + NBB / NW;  // 1 KiB blocks per wave per stage
    constexpr int STAGE = (BM + BN) * ROWB;
    // epilogue passes: the fp32 tile goes through LDS in NP column slices
    constexpr int NP = (BM * (BNO + 4) * 4 <= NST * STAGE) ? 1
                       : (BM * (BNO / 2 + 4) * 4 <= NST * STAGE) ? 2
                       : (BM * (BNO / 4 + 4) * 4 <= NST * STAGE) ? 4 : 8;
    constexpr int WP = BNO / NP;
    constexpr int EP_STRIDE = WP + 4;
    constexpr int LDS_BYTES = (NST * STAGE > BM * EP_STRIDE * 4) ? NST * STAGE : BM * EP_STRIDE * 4;
    static_assert((NW == 4 || NW == 8) && BM % RPB == 0 && NBB % NW == 0 && (A_ALL || NA % NW == 0), "tile shape");
    static_assert(EPI != EPI_SWIGLU || (NB % 2 == 0 && (TN / 2) % RPB == 0), "gate/up pairs per wave");
    static_assert(NST >= 2 && LPW * (NST - 2) < 64, "pipeline depth");
    __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid / WN, wn = wid % WN;

    Job jb;
    if (!pick_job<BM, BNO>(a, jb)) return;
    const int expert = jb.expert, row0 = jb.row0, rows = jb.rows, n0 = jb.n0;
    const GemmGroup& G = jb.gi ? a.g[1] : a.g[0];
    const int N = G.N;

    int nk = 0;
    for (int s = 0; s < G.nseg; ++s) nk += seg_of(G, s).K / BKE;
    const int chunk = (nk + a.nsplit - 1) / a.nsplit;
    const int kt0 = min(nk, static_cast<int>(blockIdx.z) * chunk);
    const int kt1 = min(nk, kt0 + chunk);
    const int nkt = kt1 - kt0;

    // ---- this lane's source row in each block the wave loads.  Block q
    // covers tile rows RPB q .. RPB q + RPB-1 (A rows first, then B rows);
    // lane i fills LDS position (row i / CHUNKS, chunk i % CHUNKS), which
    // holds logical chunk (i % CHUNKS) ^ swz(row).  blk(j) is the j-th block
    // of this wave.  Packed weights (PK): B block q' = q - NA is the
    // 16-row x 32-K fragment block (row block q' / SLABS, slab q' % SLABS),
    // 1 KiB stored contiguously in lane order; srow holds its row block.
    const int lrow = lane / CHUNKS;
    const int lchunk16 = ((lane % CHUNKS) ^ swz<ROWB>(lrow)) * 16;
    auto blk = [&](int j) { return j < LPA ? (A_ALL ? j : wid + NW * j) : NA + wid + NW * (j - LPA); };
    int srow[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int r = blk(j) * RPB + lrow;
        if (j < LPA) {
            const int p = row0 + (r < rows ? r : 0);
            srow[j] = G.rowmap ? G.rowmap[p] : p;
        } else if (PK) {
            const int rb = (blk(j) - NA) / SLABS;  // row block inside the B tile
            int nb;
            if (EPI == EPI_SWIGLU) {
                const int per = TN / 16, half = TN / 32;
                nb = n0 / 16 + (rb / per) * half + (rb % per) % half;
            } else {
                nb = n0 / 16 + rb;
            }
            srow[j] = nb < N / 16 ? nb : N / 16 - 1;
        } else {
            const int qb = r - BM;
            int n;
            if (EPI == EPI_SWIGLU) {
                const int blk = qb / TN, rq = qb % TN, half = TN / 2;
                n = n0 + blk * half + (rq % half);
            } else {
                n = n0 + qb;
            }
            srow[j] = n < N ? n : N - 1;
        }
    }
    // whether block q reads A, the gate or the up matrix depends on q alone
    auto blk_is_a = [&](int j) { return j < LPA; };
    auto blk_is_up = [&](int j) {
        if (PK) return EPI == EPI_SWIGLU && ((blk(j) - NA) / SLABS) % (TN / 16) >= TN / 32;
        return EPI == EPI_SWIGLU && (((blk(j) * RPB - BM) % TN) >= TN / 2);
    };
    auto blk_slab = [&](int j) { return (blk(j) - NA) % SLABS; };
    int cs = 0, ck = kt0;
    while (cs + 1 < G.nseg && ck >= seg_of(G, cs).K / BKE) {
        ck -= seg_of(G, cs).K / BKE;
        ++cs;
    }
    const char *pA, *pB, *pBu;
    int64_t lda, ldb;  // packed weights: ldb = bytes per row block (K / 32 fragment blocks)
    auto set_seg = [&](int s) {
        const GemmSeg& S = seg_of(G, s);
        const int64_t eoff = s == 0 ? static_cast<int64_t>(expert) * G.b_estride * ES : 0;
        const int bl = PK ? lane * 16 : lchunk16;
        pA = static_cast<const char*>(S.A) + lchunk16;
        pB = static_cast<const char*>(S.B) + eoff + bl;
        pBu = static_cast<const char*>(S.Bu) + eoff + bl;
        lda = S.lda * ES;
        ldb = PK ? static_cast<int64_t>(S.K) * 32 : S.ldb * ES;
    };
    set_seg(cs);
    const uint32_t lds_base = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(lds)));
    auto issue = [&](int buf) {
        const int64_t off = static_cast<int64_t>(ck) * ROWB;
        const uint32_t dst = lds_base + buf * STAGE;
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const bool isa = blk_is_a(j);
            const char* base = isa ? pA : (blk_is_up(j) ? pBu : pB);
            const int64_t koff = (PK && !isa) ? (static_cast<int64_t>(ck) * SLABS + blk_slab(j)) * 1024 : off;
            const char* src = base + static_cast<int64_t>(srow[j]) * (isa ? lda : ldb) + koff;
            if (PK && BM == 16 && !isa)
                lds_dma16_once(src, dst + blk(j) * 1024);
            else
                lds_dma16(src, dst + blk(j) * 1024);
        }
        ++ck;
        if (cs + 1 < G.nseg && ck == seg_of(G, cs).K / BKE) {
            ++cs;
            ck = 0;
            set_seg(cs);
        }
    };

    f32x4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // fragment offsets inside a 16-row group for each 64-byte slab:
    // row (lane & 15), logical chunk 4*slab + (lane >> 4), swizzled by row
    const int frow = lane & 15;
    const int fo0 = frow * ROWB + ((((lane >> 4) + 0) ^ swz<ROWB>(frow)) << 4);
    const int fo1 = frow * ROWB + ((((lane >> 4) + 4) ^ swz<ROWB>(frow)) << 4);

#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        if (s < nkt) issue(s);
    for (int it = 0; it < nkt; ++it) {
        if (it + NST - 2 < nkt)
            wait_vmcnt<LPW * (NST - 2)>();  // the NST-2 newer stages may still be in flight
        else
            wait_vmcnt<0>();
        __syncthreads();  // every wave's blocks of stage `it` have landed
        if (it + NST - 1 < nkt) issue((it + NST - 1) % NST);  // reuses the stage read at it-1
        const char* As = lds + (it % NST) * STAGE;
        const char* Bs = As + BM * ROWB;
#pragma unroll
        for (int sl = 0; sl < SLABS; ++sl) {
            const int fo = sl ? fo1 : fo0;
            uint4 fa[MB], fb[NB];
#pragma unroll
            for (int i = 0; i < MB; ++i)
                fa[i] = *reinterpret_cast<const uint4*>(As + (wm * TM + i * 16) * ROWB + fo);
#pragma unroll
            for (int j = 0; j < NB; ++j)
                fb[j] = PK ? *reinterpret_cast<const uint4*>(Bs + ((wn * TN / 16 + j) * SLABS + sl) * 1024 + lane * 16)
                           : *reinterpret_cast<const uint4*>(Bs + (wn * TN + j * 16) * ROWB + fo);
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j) acc[i][j] = Mfma<T>::run(fa[i], fb[j], acc[i][j]);
        }
    }

    // ---- epilogue
    TC* C = static_cast<TC*>(G.C) + static_cast<int64_t>(blockIdx.z) * a.split_stride;
    store_tile<TC, EPI, BM, BNO, TM, TN, MB, NB, WP, NT>(acc, lds, wm, wn, G, C, row0, rows, n0);
}

// Register-fed tile for packed weights: BM A rows x BN B rows per
// workgroup of four waves (BN = 512; 256 for the 16-row kernel); wave w owns
// B rows [w BN/4, (w + 1) BN/4), a BM x BN/4 output block held in 16x16
// accumulators.  Only A is shared
// between the waves, so only A goes through LDS (DMA into a ring of four
// 64-K slots).  Each wave loads its own weight fragments from global memory
// straight into registers one stage ahead, a fragment being reloaded with
// the next stage as soon as its last use in this stage has issued.  In the
// packed layouts a fragment block is one contiguous KiB in lane order, so
// each of these loads reads eight whole 128-byte lines: the vector memory
// path on gfx950 is limited by the lines an instruction touches, and a
// row-major fragment (16 rows x 64 bytes) touches twice as many.
//
// bf16 weights (F8 false): a 1 KiB block is one 16 x 32 fragment, two loads
// per 16-row block per stage.  FP8 weights (F8 true; OCP E4M3FN codes with
// one E8M0 exponent per 128 x 128 block): a 1 KiB block is 16 rows x 64
// columns, lane l holding columns 8 (l/16) .. + 7 of both 32-column halves
// of row l % 16, so one load per 16-row block brings both slabs of a stage;
// v_cvt_scalef32_pk_bf16_fp8 turns the codes into bf16 scaled by the
// block's power of two (exact: 3 mantissa bits fit in bf16's 7), and the
// MFMAs are the bf16 ones.  Lane l keeps the exponent of K block l of its
// row block (K <= 8192) and a stage reads its own with readlane.
//
// NSEG K segments (1, or 2 for a sum of two products; FP8: 1).  Per stage
// and lane the memory operations are, in issue order: the first slab's B
// loads of the next stage among the first slab's MFMAs (bf16: NB; FP8: the
// NB loads of both slabs), NAB A DMA loads for stage it + NST (after the
// barrier between the slabs), the second slab's NB B loads among its MFMAs
// (bf16 only).  Every stage issues the same loads (past the last stage they
// re-read it), so the loads younger than A(it + 1) at its wait are a
// compile-time count (the first stages, after a prologue of A(0..NST-1) and
// B(0), have their own).
template <int BM>
constexpr int wide_lds_bytes() {  // the A ring: four 64-K stages of BM rows
    return 4 * BM * 128;
}

// Results of a register-fed tile straight to C (no LDS).  The MFMAs there
// take the weight fragment as their first operand, so acc[i][j] holds rows
// 16 i + lane % 16 and the four consecutive columns 16 j + 4 (lane / 16) ..
// + 3 of the wave's block (for SwiGLU, blocks j < NB/2 are the gate and j +
// NB/2 the matching up columns).  bf16: blocks go in pairs (j0, j0 + 1);
// lanes l and l ^ 16 trade one 8-byte half (ds_swizzle, xor 16), after which
// each lane holds 8 consecutive columns of one row and stores 16 bytes, and
// the four lanes of a row cover 64 contiguous bytes.  fp32: 16 bytes per
// block and lane.  Rows past `rows` and columns past N are not stored.
template <typename TC, int EPI, int MB, int NB, int TN>
__device__ __forceinline__ void store_direct(const f32x4 (&acc)[MB][NB], const GemmGroup& G, TC* C, int row0,
                                             int rows, int n0, int wid) {
    const int lane = threadIdx.x & 63;
    const int N = G.N, q = lane >> 4;
    constexpr int NJ = EPI == EPI_SWIGLU ? NB / 2 : NB;  // output blocks per row
    const int cb = n0 + wid * (EPI == EPI_SWIGLU ? TN / 2 : TN);
    // silu(g) * u with the hardware exp2 and reciprocal (about 1 ulp each,
    // against the 8 significant bits the bf16 result keeps): an IEEE
    // division and the library exp cost some 20 VALU instructions per
    // output, and this epilogue writes 32768 of them per workgroup.
    auto val = [&](int i, int j, int e) {
        if (EPI == EPI_SWIGLU) {
            const float g = acc[i][j][e], u = acc[i][j + NB / 2][e];
            return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
        }
        return acc[i][j][e];
    };
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        const int r = i * 16 + (lane & 15);
        TC* dst = C + static_cast<int64_t>(row0 + (r < rows ? r : 0)) * G.ldc;
        if constexpr (sizeof(TC) == 4) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int col = cb + j * 16 + 4 * q;
                if (r < rows && col < N)
                    *reinterpret_cast<float4*>(dst + col) = make_float4(val(i, j, 0), val(i, j, 1), val(i, j, 2),
                                                                        val(i, j, 3));
            }
        } else {
            static_assert(NJ % 2 == 0, "block pairs");
#pragma unroll
            for (int jp = 0; jp < NJ / 2; ++jp) {
                const int j0 = 2 * jp, j1 = j0 + 1;
                uint32_t p0[2], p1[2];  // bf16 pairs: columns 4q .. 4q+3 of blocks j0, j1
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    p0[h] = f32_to_bf16(val(i, j0, 2 * h)) |
                            (static_cast<uint32_t>(f32_to_bf16(val(i, j0, 2 * h + 1))) << 16);
                    p1[h] = f32_to_bf16(val(i, j1, 2 * h)) |
                            (static_cast<uint32_t>(f32_to_bf16(val(i, j1, 2 * h + 1))) << 16);
                }
                // even q keeps block j0 and receives its neighbour's j0 columns;
                // odd q keeps block j1 and receives its neighbour's j1 columns
                const bool odd = q & 1;
                uint32_t rcv[2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    rcv[h] = static_cast<uint32_t>(
                        __builtin_amdgcn_ds_swizzle(static_cast<int>(odd ? p0[h] : p1[h]), 0x401F));
                const int col = odd ? cb + j1 * 16 + 4 * (q - 1) : cb + j0 * 16 + 4 * q;
                const uint4 v = odd ? make_uint4(rcv[0], rcv[1], p1[0], p1[1]) : make_uint4(p0[0], p0[1], rcv[0], rcv[1]);
                if (r < rows && col < N) *reinterpret_cast<uint4*>(dst + col) = v;
            }
        }
    }
}

// B rows per N tile of the register-fed tile: 512, and 256 for the 16-row
// (FP8 decode) kernel, where twice the workgroups each stream half the
// bytes (K2 FP8 layer 0.211-0.215 -> 0.204-0.205 ms at 1 token, 2.83 ->
// 2.76-2.79 ms at 256).  The ragged bodies of the 128-row kernel (32, 64
// rows) keep its 512.
constexpr int wide_bn(int bm) { return bm == 16 ? 256 : 512; }

template <typename TC, int EPI, int NSEG, int BM, bool F8>
__device__ __forceinline__ void wide_tile(const GemmArgs& a, const Job& jb, char* lds) {
    using T = bf16_t;
    static_assert(BM % 16 == 0 && BM <= 128 && (BM * 128 / 1024 < 4 || BM * 128 / 1024 % 4 == 0), "row tiles");
    static_assert(!F8 || NSEG == 1, "FP8 weights: one K segment");
    constexpr int ES = 2, BN = wide_bn(BM), NW = 4, TN = BN / NW;
    constexpr int WES = F8 ? 1 : 2;            // bytes per weight element
    constexpr int MB = BM / 16, NB = TN / 16;
    constexpr int ROWB = 128, BKE = ROWB / ES;  // a stage is 64 K = two 32-K slabs
    constexpr int NST = 4;                     // A slots: stages it .. it+3 (it+4 after the barrier)
    constexpr int STAGE = BM * ROWB;
    constexpr int BNO = EPI == EPI_SWIGLU ? BN / 2 : BN;
    // A blocks of 1 KiB (8 rows) per stage, split across the waves; with
    // fewer blocks than waves every wave loads all of them (identical bytes
    // to identical LDS addresses)
    constexpr int NBLK = STAGE / 1024;
    constexpr bool A_ALL = NBLK < NW;
    constexpr int NAB = A_ALL ? NBLK : NBLK / NW;  // A DMA loads per wave per stage
    constexpr int NBL = F8 ? NB : 2 * NB;         // B loads per wave per stage
    constexpr int LOADS = NAB + NBL;               // vector loads per lane per stage
    constexpr int B2 = F8 ? 0 : NB;                // B loads after the A DMA of a stage
    // A(it + 1) is waited for between the slabs of stage it.  Loads younger
    // than it: once A(it + 1) came from stage it + 1 - NST, that stage's
    // later B loads, NST - 2 whole stages and the first-slab B loads of
    // stage it; before that (A from the prologue: A(0..NST-1), B(0)), the
    // later prologue loads, the stages so far and the first slab.
    constexpr int kWaitA = B2 + NB + (NST - 2) * LOADS;
    constexpr int kY0 = NAB * (NST - 2) + NBL + NB, kY1 = NAB * (NST - 3) + NBL + NB + LOADS;
    constexpr int kWait0 = kY0 < kWaitA ? kY0 : kWaitA, kWait1 = kY1 < kWaitA ? kY1 : kWaitA;
    static_assert(kWaitA < 64 && (NSEG == 1 || NSEG == 2) && NST == 4, "vmcnt range; shape");
    static_assert(NST * STAGE <= wide_lds_bytes<BM>(), "LDS");

    const GemmGroup& G = jb.gi ? a.g[1] : a.g[0];
    const int N = G.N, row0 = jb.row0, rows = jb.rows, n0 = jb.n0;
    const int nk0 = G.seg[0].K / BKE;
    const int nkt = nk0 + (NSEG == 2 ? G.seg[1].K / BKE : 0);  // >= 1

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);

    // A: block q of a stage holds tile rows 8q .. 8q+7 (128 bytes each, the
    // 16-byte chunk c of row r at position c ^ (r & 7)); lane i fills row
    // 8q + i/8, position i%8.  This wave loads blocks ablk(j).
    const int achunk = ((lane & 7) ^ (lane >> 3)) << 4;
    int arow[NAB];
    auto ablk = [&](int j) { return A_ALL ? j : wid + NW * j; };
#pragma unroll
    for (int j = 0; j < NAB; ++j) {
        const int r = ablk(j) * 8 + (lane >> 3);
        const int p = row0 + (r < rows ? r : 0);
        arow[j] = G.rowmap ? G.rowmap[p] : p;
    }
    // Everything the loop needs from the group, held in registers: the DMA
    // asm clobbers memory, so fields read through G inside the loop would be
    // reloaded (scalar loads, which also blunt the LDS wait counts) every
    // stage.
    const char* const sA0 = static_cast<const char*>(G.seg[0].A);
    const char* const sA1 = static_cast<const char*>(G.seg[NSEG - 1].A);
    const int64_t lda0 = G.seg[0].lda * ES, lda1 = G.seg[NSEG - 1].lda * ES;
    const int64_t eoff = static_cast<int64_t>(jb.expert) * G.b_estride * WES;  // segment 0 only
    const char* const sB0 = static_cast<const char*>(G.seg[0].B) + eoff;
    const char* const sU0 = EPI == EPI_SWIGLU ? static_cast<const char*>(G.seg[0].Bu) + eoff : sB0;
    const char* const sB1 = static_cast<const char*>(G.seg[NSEG - 1].B);
    const char* const sU1 = EPI == EPI_SWIGLU ? static_cast<const char*>(G.seg[NSEG - 1].Bu) : sB1;
    // fragment blocks per row block: K/32 (bf16) or K/64 (FP8)
    const uint32_t kb0 = static_cast<uint32_t>(G.seg[0].K / (F8 ? 64 : 32));
    const uint32_t kb1 = static_cast<uint32_t>(G.seg[NSEG - 1].K / 32);

    const char* asrc[NAB];  // segment 0 row addresses
#pragma unroll
    for (int j = 0; j < NAB; ++j) asrc[j] = sA0 + static_cast<int64_t>(arow[j]) * lda0 + achunk;
    const uint32_t lds_base = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(lds)));
    auto issue_a = [&](int kt, int slot) {
        const uint32_t dst = lds_base + slot * STAGE;
        if (NSEG == 1) {
#pragma unroll
            for (int j = 0; j < NAB; ++j) lds_dma16(asrc[j] + kt * ROWB, dst + ablk(j) * 1024);
        } else {
            const bool s1 = kt >= nk0;
            const char* base = (s1 ? sA1 : sA0) + (kt - (s1 ? nk0 : 0)) * ROWB + achunk;
            const int64_t lda = s1 ? lda1 : lda0;
#pragma unroll
            for (int j = 0; j < NAB; ++j) lds_dma16(base + arow[j] * lda, dst + ablk(j) * 1024);
        }
    };

    // B: fragment j of this wave is row block rb[j] (16 rows); for SwiGLU,
    // j < NB/2 are gate row blocks and j + NB/2 the same blocks of the up
    // matrix.  Fragment block (row block r, column block k) of a [rows, K]
    // matrix sits at byte (r kb + k) 1024; lane l reads its 16 bytes at 16 l.
    int rb[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int nb = EPI == EPI_SWIGLU ? (n0 + wid * (TN / 2)) / 16 + j % (NB / 2) : (n0 + wid * TN) / 16 + j;
        rb[j] = nb < N / 16 ? nb : N / 16 - 1;
    }
    auto load_b = [&](int kt, int sl, int j) {
        const bool s1 = NSEG == 2 && kt >= nk0;
        const bool up = EPI == EPI_SWIGLU && j >= NB / 2;
        const char* m = s1 ? (up ? sU1 : sB1) : (up ? sU0 : sB0);
        const uint32_t kblk = F8 ? static_cast<uint32_t>(kt) : static_cast<uint32_t>((kt - (s1 ? nk0 : 0)) * 2 + sl);
        const uint32_t blk = static_cast<uint32_t>(rb[j]) * (s1 ? kb1 : kb0) + kblk;
        // decode tiles (16 rows) stream each expert's FP8 codes once, with
        // the non-temporal hint and compiler-counted waits (exact explicit
        // waits measured the same there); everything else is untracked
        if constexpr (F8 && BM == 16) return gload16_once(m + blk * 1024u + lane * 16);
        return gload16_untracked(m + blk * 1024u, lane * 16);
    };
    // FP8 block scales: lane l holds the exponent of K block l of this
    // wave's 128-row block (gate and up), placed as the exponent field of
    // the float 2^(s - 127); the wave's rows never straddle a 128-row block
    // (n0 is a multiple of 128, the wave's B rows an aligned range of 32 to
    // 128 rows).  Exponent 0 gives the bits of +0.0, which the scaled
    // conversion reads as 2^-127 like any E8M0 scale (the parity test of
    // extreme block scales pins both ends of the range).
    uint32_t scg = 0, scu = 0;
    if constexpr (F8) {
        const int kbl = G.seg[0].K / 128;
        const int r128 = min((EPI == EPI_SWIGLU ? n0 + wid * (TN / 2) : n0 + wid * TN) / 128, N / 128 - 1);
        const int64_t so = static_cast<int64_t>(jb.expert) * G.s_estride + static_cast<int64_t>(r128) * kbl;
        scg = lane < kbl ? static_cast<uint32_t>(G.bs[so + lane]) << 23 : 0u;
        scu = EPI == EPI_SWIGLU ? (lane < kbl ? static_cast<uint32_t>(G.bsu[so + lane]) << 23 : 0u) : scg;
    }

    f32x4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // A fragment of a slab: row (lane & 15), logical chunk 4 slab + lane/16
    const int frow = lane & 15;
    const int fo0 = frow * ROWB + ((((lane >> 4) + 0) ^ (frow & 7)) << 4);
    const int fo1 = frow * ROWB + ((((lane >> 4) + 4) ^ (frow & 7)) << 4);

    // B fragments of the current stage, refilled with the next: bf16, both
    // slabs; FP8, the raw codes of both slabs in fb[0]
    uint4 fb[F8 ? 1 : 2][NB];
    uint4 fa0[MB];  // A fragments of the first slab of the current stage
    auto read_a = [&](uint4 (&fa)[MB], int stage, int fo) {
        const char* As = lds + (stage % NST) * STAGE;
#pragma unroll
        for (int i = 0; i < MB; ++i) fa[i] = *reinterpret_cast<const uint4*>(As + i * 16 * ROWB + fo);
    };
    // One K stage.  The order below is the schedule (the scheduler would
    // otherwise sink the B loads to their next use and expose their
    // latency): a B fragment is reloaded with the next stage right after its
    // last use here; the second slab's A fragments are read early in the
    // first slab; the barrier sits between the slabs, after which the slot
    // of this stage (read by every wave) takes A(it + NST) and the next
    // stage's first A fragments are read while the second slab computes.
    // The weight loads (bf16 fragments; FP8 codes at 128 rows) are issued
    // untracked (like the A DMA), so the waits for them are explicit and
    // exact.  A fragment's load is LOADS - 1 loads older than the point of
    // its first use, save the first stage's first slab, whose loads come
    // from the prologue (2 NB - 1 for bf16, NB - 1 for FP8 codes, which
    // carry both slabs).  Waits counted by the compiler would leave out the
    // A DMA loads and hold each fragment until NAB loads issued after it
    // had landed too (K2 FP8 prefill: 12.24 -> 11.90 ms from exact waits).
    //
    // FP8 at 128 rows converts one fragment ahead of the MFMAs: fragment
    // j + 1 of the first slab while fragment j's MFMAs run, and fragment 0
    // of the next stage in the second slab, each conversion interleaved
    // with the MFMAs of its slot.  (Converted right before its own MFMAs,
    // a fragment's conversions left the matrix pipe idle while they
    // issued.)  Code j of stage it + 1 is loaded right after code j of
    // stage it is converted, so the loads keep their order and their
    // waits keep their counts.
    constexpr bool PIPE = F8 && BM != 16;
    uint4 fq0 = make_uint4(0u, 0u, 0u, 0u);  // PIPE: stage's first-slab fragment 0
    uint4 fh[PIPE ? NB : 1];                 // PIPE: stage's second-slab fragments
    auto scale = [&](int stage, int j) {
        const uint32_t v = (EPI == EPI_SWIGLU && j >= NB / 2) ? scu : scg;
        return __uint_as_float(__builtin_amdgcn_readlane(v, stage >> 1));
    };
    auto convert = [&](int stage, int j, uint4& lo, uint4& hi, int kload) {
        fp8x16_to_bf16(fb[0][j], scale(stage, j), lo, hi);
        asm volatile("" ::"v"(hi.x), "v"(hi.y), "v"(hi.z), "v"(hi.w) : "memory");
        fb[0][j] = load_b(kload, 0, j);
    };
    auto step = [&](int it, auto wait_next, auto first) {
        const int kb = min(it + 1, nkt - 1);
        uint4 fa1[MB];
        uint4 f1[F8 && !PIPE ? NB : 1];  // FP8 at 16 rows: the second slab's converted fragments
        float sg = 0.f, su = 0.f;
        if constexpr (F8 && !PIPE) {
            sg = __uint_as_float(__builtin_amdgcn_readlane(scg, it >> 1));
            su = EPI == EPI_SWIGLU ? __uint_as_float(__builtin_amdgcn_readlane(scu, it >> 1)) : sg;
        }
        uint4 fq[PIPE ? NB : 1];
        fq[0] = fq0;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if constexpr (PIPE) {
                if (j + 1 < NB) {
                    wait_vmcnt_fenced<decltype(first)::value ? NB - 1 : LOADS - 1>();
                    convert(it, j + 1, fq[j + 1], fh[j + 1], kb);
                }
#pragma unroll
                for (int i = 0; i < MB; ++i) acc[i][j] = Mfma<T>::run(fq[j], fa0[i], acc[i][j]);
                if (j + 1 < NB) interleave<MB, 8>();
            } else if constexpr (F8) {
                uint4 f0;
                fp8x16_to_bf16(fb[0][j], (EPI == EPI_SWIGLU && j >= NB / 2) ? su : sg, f0, f1[j]);
                // Both halves are converted before the codes' registers take the
                // next stage's load (the empty asm uses the second half here, and
                // its memory clobber keeps the load below it).  Left to itself the
                // compiler converts the second half in the second slab, keeps the
                // old codes in other registers and copies the new ones back at the
                // loop's end -- a copy that must wait for every load in flight
                // (vmcnt(0)) once per stage.
                asm volatile("" ::"v"(f1[j].x), "v"(f1[j].y), "v"(f1[j].z), "v"(f1[j].w) : "memory");
                fb[0][j] = load_b(kb, 0, j);
#pragma unroll
                for (int i = 0; i < MB; ++i) acc[i][j] = Mfma<T>::run(f0, fa0[i], acc[i][j]);
            } else {
                wait_vmcnt_fenced<decltype(first)::value ? 2 * NB - 1 : LOADS - 1>();
#pragma unroll
                for (int i = 0; i < MB; ++i) acc[i][j] = Mfma<T>::run(fb[0][j], fa0[i], acc[i][j]);
                fb[0][j] = load_b(kb, 0, j);
            }
            if (j == 1) read_a(fa1, it, fo1);
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_next();      // this wave's A(it + 1) has landed
        __syncthreads();  // ... every wave's; every wave is done reading slot it % NST
        issue_a(min(it + NST, nkt - 1), it % NST);
        read_a(fa0, it + 1, fo0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if constexpr (PIPE) {
                if (j == 1) {
                    wait_vmcnt_fenced<LOADS - 1>();
                    convert(kb, 0, fq0, fh[0], min(it + 2, nkt - 1));
                }
#pragma unroll
                for (int i = 0; i < MB; ++i) acc[i][j] = Mfma<T>::run(fh[j], fa1[i], acc[i][j]);
                if (j == 1) interleave<MB, 8>();
            } else if constexpr (F8) {
#pragma unroll
                for (int i = 0; i < MB; ++i) acc[i][j] = Mfma<T>::run(f1[j], fa1[i], acc[i][j]);
            } else {
                wait_vmcnt_fenced<LOADS - 1>();
#pragma unroll
                for (int i = 0; i < MB; ++i) acc[i][j] = Mfma<T>::run(fb[1][j], fa1[i], acc[i][j]);
                fb[1][j] = load_b(kb, 1, j);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

#pragma unroll
    for (int p = 0; p < NST; ++p) issue_a(min(p, nkt - 1), p);
#pragma unroll
    for (int sl = 0; sl < (F8 ? 1 : 2); ++sl)
#pragma unroll
        for (int j = 0; j < NB; ++j) fb[sl][j] = load_b(0, sl, j);
    wait_vmcnt<(NST - 1) * NAB + NBL>();  // A(0): younger are A(1..NST-1) and B(0)
    __syncthreads();
    read_a(fa0, 0, fo0);
    if constexpr (PIPE) {
        wait_vmcnt_fenced<NB - 1>();  // code 0 of stage 0: younger are codes 1 .. NB - 1
        convert(0, 0, fq0, fh[0], min(1, nkt - 1));
    }
    step(0, [] { wait_vmcnt<kWait0>(); }, std::true_type{});
    for (int it = 1; it < nkt; ++it)
        step(it, [it] {
            if (it >= NST - 2)
                wait_vmcnt<kWaitA>();
            else
                wait_vmcnt<kWait1>();
        }, std::false_type{});
    wait_vmcnt_fenced<0>();  // every load has landed before its registers are reused
    // The last stage's weight loads (re-reading that stage) are never used;
    // this empty use keeps their registers allocated up to the wait, so
    // nothing else is placed in them while they are in flight.
#pragma unroll
    for (int sl = 0; sl < (F8 ? 1 : 2); ++sl)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            asm volatile("" ::"v"(fb[sl][j].x), "v"(fb[sl][j].y), "v"(fb[sl][j].z), "v"(fb[sl][j].w));
    store_direct<TC, EPI, MB, NB, TN>(acc, G, static_cast<TC*>(G.C), row0, rows, n0, wid);
}

// F8: group 0 (routed experts) has FP8 weights, group 1 (the shared
// experts, riding in the same launch) bf16 ones; a tile takes its group's
// path.
template <typename TC, int EPI, int NSEG, int BM, bool F8>
__device__ __forceinline__ void wide_group(const GemmArgs& a, const Job& jb, char* lds) {
    if constexpr (F8) {
        if (jb.gi) {
            wide_tile<TC, EPI, 1, BM, false>(a, jb, lds);
            return;
        }
    }
    wide_tile<TC, EPI, NSEG, BM, F8>(a, jb, lds);
}

// A 128-row tile holding fewer rows (the ragged last tile of an expert)
// runs the body of the next multiple of 32 rows: fewer MFMAs and less A
// traffic, the same weight traffic.
template <typename TC, int EPI, int NSEG, int BM, bool F8>
__global__ __launch_bounds__(256, BM >= 64 ? 1 : 2) void k_gemm_wide(const GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) char lds[wide_lds_bytes<BM>()];
    constexpr int BNO = EPI == EPI_SWIGLU ? wide_bn(BM) / 2 : wide_bn(BM);
    Job jb;
    if (!pick_job<BM, BNO>(a, jb)) return;
    if constexpr (BM == 128) {
        if (jb.rows <= 32) {
            wide_group<TC, EPI, NSEG, 32, F8>(a, jb, lds);
            return;
        }
        if (jb.rows <= 64) {
            wide_group<TC, EPI, NSEG, 64, F8>(a, jb, lds);
            return;
        }
        if (jb.rows <= 96) {
            wide_group<TC, EPI, NSEG, 96, F8>(a, jb, lds);
            return;
        }
    }
    wide_group<TC, EPI, NSEG, BM, F8>(a, jb, lds);
}

// fp32 operands: register-staged 16 x 256 tiles
constexpr int kF32BN = 256;
// decode tile (few rows per expert): 16 x 512.  bf16 output (expert and
// dense GEMMs): a ring of four slots of 64-byte row pieces, three stages
// (99 KiB) in flight.  A workgroup walks its whole K in sequence, and with
// few workgroups per CU (small batches) the latency of each stage is the
// cost: against two slots of 128-byte pieces (one 66 KiB stage in flight),
// K2 layer 0.36 -> 0.32 ms at 1 token, 5.37 -> 5.19-5.28 ms at 256, 5.43 ->
// 5.17-5.30 ms at 384; K3 shapes 4-5% at 32-256 tokens.  fp32 output (the
// router logits of up to 64 tokens): two slots of 128-byte pieces, 7%
// faster there than four.
constexpr int kSmBM = 16, kSmBN = 512, kSmWM = 1, kSmWN = 4;
constexpr int kSmNST = 4, kSmROWB = 64, kSmNST32 = 2, kSmROWB32 = 128;
// 256-wide form: twice the workgroups, each streaming half the bytes, for
// launches of too few 512-wide workgroups to fill the chip (each walks its
// whole K in sequence).  K2 layer at 1 token: up 0.167 -> 0.098 ms, the
// layer 0.30-0.32 -> 0.24 ms; at 2-4 tokens the 512-wide tiles already
// make 136-264 workgroups and measured the same or 3% better.  The router
// logits of up to 64 tokens always take it (E = 384 fills 1.5 of them
// instead of 0.75 of one; 0.046 -> 0.039 ms at 1 token).
constexpr int kNarBN = 256;
// prefill tile: BM x BN (B rows), waves WM x WN, NST LDS stages
constexpr int kBigBM = 128, kBigBN = 256, kBigWM = 2, kBigWN = 2, kBigNST = 3, kBigROWB = 64;
// router logits tile: 128 x 192 (E = 384 is two whole N tiles, where 256
// left half of the second one idle), both operands DMA'd in 128-byte row
// pieces through a two-stage ring of 80 KiB, two workgroups per CU.  Against
// 64-byte pieces in three stages: 0.40 -> 0.32 ms at 16384 tokens, 0.147 ->
// 0.134 ms at 4096, K3's 896 experts 0.27 -> 0.23 ms.
constexpr int kRtBN = 192, kRtNST = 2, kRtROWB = 128;
// prefill expert tile with register-fed weights: 128 x 512
constexpr int kWideBM = 128, kWideBN = wide_bn(kWideBM), kWide16BN = wide_bn(16);

}  // namespace

static_assert(kSmBM == 16, "fp32 small tiles share the 16-row M tiling");
static_assert(kBigBM == kWideBM, "prefill tiles share the tile table's 128-row M tiling");
int tile_bm(TileCfg cfg) {
    return (cfg == TILE_SMALL || cfg == TILE_WIDE16 || cfg == TILE_NARROW) ? kSmBM : kBigBM;
}
int tile_bn_out(TileCfg cfg, Epi epi) {  // bf16 kernels (sizing heuristics only)
    // B rows per N tile (gate + up rows for SwiGLU)
    const int bn = cfg == TILE_SMALL ? kSmBN
                   : cfg == TILE_NARROW ? kNarBN
                   : cfg == TILE_WIDE ? kWideBN
                   : cfg == TILE_WIDE16 ? kWide16BN
                   : cfg == TILE_ROUTER ? kRtBN : kBigBN;
    return epi == EPI_SWIGLU ? bn / 2 : bn;
}

namespace {

// What the wide kernel handles: packed weights, one or two K segments per
// group (multiples of 64), no split K, fragment-block byte offsets in 31 bits.
bool wide_fits(const GemmArgs& a) {
    if (a.nsplit != 1) return false;
    for (int g = 0; g < 2; ++g) {
        const GemmGroup& G = a.g[g];
        if (G.N == 0) continue;
        if (G.nseg < 1 || G.nseg > 2 || G.N % 16 != 0) return false;
        for (int s = 0; s < G.nseg; ++s)
            if (G.seg[s].K < 64 || G.seg[s].K % 64 != 0 ||
                static_cast<int64_t>(G.N) * G.seg[s].K * 2 >= (int64_t{1} << 31))
                return false;
    }
    return true;
}

int max_nseg(const GemmArgs& a) {
    return a.g[0].nseg > a.g[1].nseg ? a.g[0].nseg : a.g[1].nseg;
}

template <typename T, typename TC, int EPI>
hipError_t launch_t(const GemmArgs& args, TileCfg cfg, int max_tiles, int max_n, bool packed, hipStream_t stream) {
    if constexpr (sizeof(T) == 4) {
        if (packed || cfg != TILE_SMALL) return hipErrorInvalidValue;  // fp32 runs the small tiles only
    }
    if (cfg == TILE_ROUTER && (packed || EPI != EPI_STORE)) return hipErrorInvalidValue;
    if (cfg == TILE_WIDE && !(packed && wide_fits(args))) cfg = TILE_LARGE;
    if (cfg == TILE_WIDE16) cfg = TILE_SMALL;  // bf16 decode: the LDS tile streams slightly faster
    if (cfg == TILE_SMALL && sizeof(TC) == 4) cfg = TILE_NARROW;  // the router logits (fp32 out)
    const bool wide = cfg == TILE_WIDE;
    // output columns per N tile of the kernel actually launched
    const int bn = sizeof(T) == 4 ? kF32BN
                   : cfg == TILE_SMALL ? kSmBN
                   : cfg == TILE_NARROW ? kNarBN
                   : wide ? kWideBN
                   : cfg == TILE_ROUTER ? kRtBN : kBigBN;
    const int bno = EPI == EPI_SWIGLU ? bn / 2 : bn;
    GemmArgs a = args;
    a.ntn = (max_n + bno - 1) / bno;
    const dim3 grid(job_blocks(max_tiles, a.ntn), 1, a.nsplit);
    if constexpr (sizeof(T) == 4) {
        hipLaunchKernelGGL((k_gemm<T, TC, 16, kF32BN, 1, 4, EPI>), grid, dim3(256), 0, stream, a);
    } else {
        if (cfg == TILE_WIDE) {
            if (max_nseg(a) == 1)
                hipLaunchKernelGGL((k_gemm_wide<TC, EPI, 1, kWideBM, false>), grid, dim3(256), 0, stream, a);
            else
                hipLaunchKernelGGL((k_gemm_wide<TC, EPI, 2, kWideBM, false>), grid, dim3(256), 0, stream, a);
        } else if (cfg == TILE_SMALL || cfg == TILE_NARROW) {
            constexpr int nst = sizeof(TC) == 4 ? kSmNST32 : kSmNST, rowb = sizeof(TC) == 4 ? kSmROWB32 : kSmROWB;
            if (cfg == TILE_NARROW) {
                if (packed)
                    hipLaunchKernelGGL((k_gemm_big<TC, kSmBM, kNarBN, kSmWM, kSmWN, nst, rowb, EPI, true>), grid,
                                       dim3(64 * kSmWM * kSmWN), 0, stream, a);
                else
                    hipLaunchKernelGGL((k_gemm_big<TC, kSmBM, kNarBN, kSmWM, kSmWN, nst, rowb, EPI, false>), grid,
                                       dim3(64 * kSmWM * kSmWN), 0, stream, a);
            } else if constexpr (sizeof(TC) == 2) {
                if (packed)
                    hipLaunchKernelGGL((k_gemm_big<TC, kSmBM, kSmBN, kSmWM, kSmWN, nst, rowb, EPI, true>), grid,
                                       dim3(64 * kSmWM * kSmWN), 0, stream, a);
                else
                    hipLaunchKernelGGL((k_gemm_big<TC, kSmBM, kSmBN, kSmWM, kSmWN, nst, rowb, EPI, false>), grid,
                                       dim3(64 * kSmWM * kSmWN), 0, stream, a);
            }
        } else if (cfg == TILE_ROUTER) {
            if constexpr (EPI == EPI_STORE)
                hipLaunchKernelGGL((k_gemm_big<TC, kBigBM, kRtBN, kBigWM, kBigWN, kRtNST, kRtROWB, EPI, false>), grid,
                                   dim3(64 * kBigWM * kBigWN), 0, stream, a);
        } else {
            if (packed)
                hipLaunchKernelGGL((k_gemm_big<TC, kBigBM, kBigBN, kBigWM, kBigWN, kBigNST, kBigROWB, EPI, true>), grid,
                                   dim3(64 * kBigWM * kBigWN), 0, stream, a);
            else
                hipLaunchKernelGGL((k_gemm_big<TC, kBigBM, kBigBN, kBigWM, kBigWN, kBigNST, kBigROWB, EPI, false>),
                                   grid, dim3(64 * kBigWM * kBigWN), 0, stream, a);
        }
    }
    return hipGetLastError();
}

// What the FP8 form of the wide kernel handles: one K segment per group;
// group 0 with block scales, rows and K in whole 128 x 128 scale blocks,
// the scale row of a 128-row block in one wave (K <= 8192), byte offsets
// in 31 bits; group 1 (bf16) as wide_fits.
bool wide_f8_fits(const GemmArgs& a, Epi epi) {
    if (a.nsplit != 1 || !wide_fits(a)) return false;
    const GemmGroup& G = a.g[0];
    const int K = G.seg[0].K;
    if (G.N == 0 || G.nseg != 1 || (a.g[1].N != 0 && a.g[1].nseg != 1)) return false;
    if (!G.bs || (epi == EPI_SWIGLU && !G.bsu)) return false;
    if (G.N % 128 || K < 128 || K % 128 || K > 64 * 128) return false;
    return static_cast<int64_t>(G.N) * K < (int64_t{1} << 31);
}

template <int EPI>
hipError_t launch_f8_t(const GemmArgs& args, TileCfg cfg, int max_tiles, int max_n, hipStream_t stream) {
    if ((cfg != TILE_WIDE && cfg != TILE_WIDE16) || !wide_f8_fits(args, static_cast<Epi>(EPI)))
        return hipErrorInvalidValue;
    const int bn = cfg == TILE_WIDE ? kWideBN : kWide16BN;
    const int bno = EPI == EPI_SWIGLU ? bn / 2 : bn;
    GemmArgs a = args;
    a.ntn = (max_n + bno - 1) / bno;
    const dim3 grid(job_blocks(max_tiles, a.ntn), 1, 1);
    if (cfg == TILE_WIDE)
        hipLaunchKernelGGL((k_gemm_wide<bf16_t, EPI, 1, kWideBM, true>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((k_gemm_wide<bf16_t, EPI, 1, kSmBM, true>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_f8(const GemmArgs& args, Epi epi, TileCfg cfg, int max_tiles, int max_n,
                          hipStream_t stream) {
    if (max_tiles <= 0 || max_n <= 0) return hipSuccess;
    if (epi == EPI_SWIGLU) return launch_f8_t<EPI_SWIGLU>(args, cfg, max_tiles, max_n, stream);
    return launch_f8_t<EPI_STORE>(args, cfg, max_tiles, max_n, stream);
}

hipError_t launch_gemm(const GemmArgs& args, DType dt, bool out_f32, Epi epi, TileCfg cfg, int max_tiles,
                       int max_n, bool packed, hipStream_t stream) {
    if (max_tiles <= 0 || max_n <= 0) return hipSuccess;
    if (dt == DT_F32) {
        if (epi == EPI_SWIGLU) return launch_t<float, float, EPI_SWIGLU>(args, cfg, max_tiles, max_n, packed, stream);
        return launch_t<float, float, EPI_STORE>(args, cfg, max_tiles, max_n, packed, stream);
    }
    if (out_f32) {
        if (packed) return hipErrorInvalidValue;  // fp32 output: the router, on row-major planes
        return launch_t<bf16_t, float, EPI_STORE>(args, cfg, max_tiles, max_n, false, stream);
    }
    if (epi == EPI_SWIGLU) return launch_t<bf16_t, bf16_t, EPI_SWIGLU>(args, cfg, max_tiles, max_n, packed, stream);
    return launch_t<bf16_t, bf16_t, EPI_STORE>(args, cfg, max_tiles, max_n, packed, stream);
}

}  // namespace moe
