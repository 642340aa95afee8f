// C ABI of the MoE layer forward (include/moe.h): argument validation,
// workspace layout and the launch sequence on the caller's stream.
//
// moe_forward enqueues, in order:
//   [bf16] split W_r into three exact bf16 planes
//   router GEMM (split-K partial logits) -> sigmoid / biased top-K / weights
//   dispatch: chunk masks -> scan + tile table -> stable scatter
//   [latent] x_lat = x W_lat_down^T
//   routed + shared up projection with the SwiGLU epilogue  (one launch)
//   routed + shared down projection                          (one launch)
//   K2 form: out = Y_shared + sum_k w_k Y[pos_k]             (combine)
//   latent:  R = sum_k w_k Y[pos_k];  out = [Hs | R] [Ws_down | W_lat_up]^T
// Nothing is read back to the host: the grouped GEMM grids are sized by
// the worst case and tiles past the device-side tile count exit at once.
// Weight GEMMs at prefill sizes use the register-fed WIDE tile when the
// weights are packed (MOE_LAYOUT_FRAG16), the LDS tile otherwise.
// FP8 routed experts (w_dtype MOE_FP8_E4M3): the up and down projections
// run the FP8 form of the WIDE tile (WIDE16 at decode sizes), whose shared
// (bf16) tiles take the bf16 path inside the same launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "../../include/moe.h"
#include "launch.hpp"

using namespace moe;

namespace {

constexpr int64_t kAlign = 256;
constexpr int kRouterGemvT = 32;  // router logits by k_router_gemv up to this many tokens
static_assert(kRouterGemvT <= kRouterGemvMaxT, "the kernel's token capacity");
int64_t up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Plan {
    int T, d, E, K, F, ns, Fs, dl, din, Fsh;  // Fsh = n_shared * F_shared
    int ng, tg;                               // expert groups, groups kept (1, 1: plain top-K)
    float scale;
    int64_t A;                                // assignments T*K
    DType dt;
    bool packed;                              // weights in MOE_LAYOUT_FRAG16
    bool f8;                                  // routed experts in block-scaled FP8
    int64_t es;                               // element size
    // router
    bool gemv;                                // logits by k_router_gemv (a few tokens)
    TileCfg rcfg;
    int nsplit, ldz, rtiles;
    // experts
    TileCfg ecfg;
    int bm, max_tiles, nch;
    TileCfg dcfg;                             // dense GEMMs (latent maps)
    // workspace offsets (bytes); -1 = absent
    int64_t o_planes, o_z, o_idx, o_w, o_counts, o_offsets, o_masks, o_cbase, o_sorted, o_pos, o_tiles,
        o_ntiles, o_xlat, o_H, o_Hs, o_Y, o_R, o_theta, total;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_desc(const moe_layer_desc* D, bool forward) {
    if (!D) return MOE_ERR_NULL;
    if (D->act_dtype != MOE_F32 && D->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (forward) {
        if (D->w_dtype == MOE_FP8_E4M3) {  // bf16 activations, packed weights
            if (D->act_dtype != MOE_BF16 || D->w_layout != MOE_LAYOUT_FRAG16) return MOE_ERR_UNSUPPORTED;
        } else {
            if (D->w_dtype != D->act_dtype) return MOE_ERR_UNSUPPORTED;
            if (D->w_layout != MOE_LAYOUT_ROWS && !(D->w_layout == MOE_LAYOUT_FRAG16 && D->w_dtype == MOE_BF16))
                return MOE_ERR_UNSUPPORTED;
        }
    }
    if (D->T < 0 || D->E < 1 || D->E > 1024 || D->K < 1 || D->K > 16 || D->K > D->E) return MOE_ERR_SHAPE;
    if (D->d <= 0 || D->d % 64) return MOE_ERR_SHAPE;
    if (static_cast<int64_t>(D->T) * D->K >= (int64_t{1} << 31)) return MOE_ERR_SHAPE;
    if (D->n_group > 1) {  // group-limited choice
        if (D->n_group > 64 || D->E % D->n_group || D->E / D->n_group < 2) return MOE_ERR_SHAPE;
        if (D->topk_group < 1 || D->topk_group > D->n_group) return MOE_ERR_SHAPE;
    } else if (D->n_group < 0) {
        return MOE_ERR_SHAPE;
    }
    if (static_cast<int64_t>(D->T) * D->d >= (int64_t{1} << 40)) return MOE_ERR_SHAPE;
    if (forward) {
        if (D->F <= 0 || D->F % 64) return MOE_ERR_SHAPE;
        if (D->n_shared < 0 || D->n_shared > 8) return MOE_ERR_SHAPE;
        if (D->n_shared > 0 && (D->F_shared <= 0 || D->F_shared % 64)) return MOE_ERR_SHAPE;
        if (D->d_latent < 0 || D->d_latent % 64) return MOE_ERR_SHAPE;
        if (D->w_dtype == MOE_FP8_E4M3) {  // whole 128 x 128 scale blocks; K <= 8192 per GEMM
            const int64_t din = D->d_latent ? D->d_latent : D->d;
            if (din % 128 || D->F % 128 || din > 8192 || D->F > 8192) return MOE_ERR_SHAPE;
        }
    }
    return MOE_OK;
}

// E_total > 0: an expert-parallel slice (moe_forward_slice) of D->E experts
// out of E_total, whose routing comes from the caller: no router buffers,
// and the tiles are chosen for the rows the slice expects, A E / E_total
// (the grids and buffers still hold all A assignments).
Plan make_plan(const moe_layer_desc* D, bool forward, int E_total = 0) {
    Plan p{};
    p.T = D->T;
    p.d = D->d;
    p.E = D->E;
    p.K = D->K;
    p.scale = D->scale;
    p.ng = D->n_group > 1 ? D->n_group : 1;
    p.tg = D->n_group > 1 ? D->topk_group : 1;
    p.F = forward ? D->F : 0;
    p.ns = forward ? D->n_shared : 0;
    p.Fs = p.ns ? D->F_shared : 0;
    p.Fsh = p.ns * p.Fs;
    p.dl = forward ? D->d_latent : 0;
    p.din = p.dl ? p.dl : p.d;
    p.A = static_cast<int64_t>(p.T) * p.K;
    p.dt = D->act_dtype == MOE_BF16 ? DT_BF16 : DT_F32;
    p.es = p.dt == DT_BF16 ? 2 : 4;

    // Router: 16-row tiles (16 x 256) for tiny batches, else 128 x 192 (each M tile
    // streams the W_r planes once, so fewer, taller tiles read less); split
    // K until about 512 workgroups (two per CU) are in flight, keeping at
    // least 8 K steps each.  Each split writes, and the gate reads back, a
    // partial plane of logits.  (fp32 activations only serve small parity
    // workloads: small tiles)
    const bool slice = E_total > 0;
    p.rcfg = (p.T <= 64 || p.dt == DT_F32) ? TILE_SMALL : TILE_ROUTER;
    const int64_t rbm = tile_bm(p.rcfg), rbn = tile_bn_out(p.rcfg, EPI_STORE);
    p.rtiles = static_cast<int>(cdiv(p.T, rbm));
    const int64_t wgs = std::max<int64_t>(1, p.rtiles * cdiv(p.E, rbn));
    const int64_t ksteps = p.dt == DT_BF16 ? 3 * (p.d / 64) : p.d / 32;
    int64_t ns = cdiv(512, wgs);
    ns = std::min<int64_t>(ns, std::max<int64_t>(1, ksteps / 8));
    p.nsplit = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(16, ns)));
    p.ldz = static_cast<int>(up(p.E, 8));
    // up to kRouterGemvT tokens the logits are T dot products per expert
    // read straight from the fp32 W_r (one pass, no planes, no split)
    p.gemv = p.T <= kRouterGemvT;
    if (p.gemv) p.nsplit = 1;

    // Experts: 128-row M tiles once experts average 10 rows or more (the
    // register-fed WIDE tile on packed weights, the LDS tile otherwise),
    // 16-row tiles below.  A 16-row tile streams its expert's weights once
    // per 16 rows, a 128-row tile once per 128, so the small tiles lose as
    // soon as experts hold a few of them.  Measured on K2 shapes (bf16,
    // 16-row vs 128-row tiles): 5.78 vs 5.86 ms at 10.7 rows per expert,
    // 6.91 vs 5.92 at 16, 13.1 vs 6.1 at 43; FP8 3.19 vs 3.13 at 10.7,
    // 8.28 vs 3.37 at 43; K3 shapes 10.7 vs 10.6 at 9.1, 22.1 vs 10.5 at 37.
    p.packed = forward && D->w_layout == MOE_LAYOUT_FRAG16;
    p.f8 = forward && D->w_dtype == MOE_FP8_E4M3;
    const TileCfg big = p.packed ? TILE_WIDE : TILE_LARGE;
    const int64_t arows = slice ? cdiv(p.A * p.E, E_total) : p.A;  // expected routed rows
    p.ecfg = (arows >= 10ll * p.E && p.dt == DT_BF16) ? big : (p.f8 ? TILE_WIDE16 : TILE_SMALL);
    // ... at 16 x 256 when the 512-wide 16-row tiles would make fewer than
    // 128 workgroups (at most one tile per assignment, plus the shared rows'
    // tiles, times the N tiles of the wider of the two expert GEMMs)
    if (p.ecfg == TILE_SMALL && p.dt == DT_BF16) {
        const int64_t mt = std::min<int64_t>(arows, p.E) + (p.ns ? cdiv(p.T, 16) : 0);
        const int64_t nt = std::max<int64_t>(cdiv(std::max(p.F, p.Fsh), 256), cdiv(p.din, 512));
        if (mt * nt < 128) p.ecfg = TILE_NARROW;
    }
    p.bm = tile_bm(p.ecfg);
    // dense maps of the latent form: 128-row tiles from 512 tokens (K3
    // shapes: 12.5 -> 10.3 ms at 768 tokens with the expert switch above;
    // below 512 the two measured the same within run-to-run noise)
    p.dcfg = (p.T >= 512 && p.dt == DT_BF16) ? big : TILE_SMALL;
    p.nch = static_cast<int>(cdiv(p.T, 64));
    p.max_tiles = static_cast<int>(cdiv(p.A, p.bm) + p.E + (p.ns ? cdiv(p.T, p.bm) : 0));

    int64_t off = 0;
    auto take = [&](int64_t bytes) {
        const int64_t o = off;
        off = up(off + std::max<int64_t>(bytes, 1), kAlign);
        return o;
    };
    const int64_t T = p.T, E = p.E;
    p.o_planes = p.o_z = p.o_idx = p.o_w = -1;
    if (!slice) {
        p.o_planes = (p.dt == DT_BF16 && !p.gemv) ? take(3 * E * p.d * 2) : -1;
        p.o_z = take(static_cast<int64_t>(p.nsplit) * T * p.ldz * 4);
        p.o_idx = take(p.A * 4);
        p.o_w = take(p.A * 4);
    }
    p.o_counts = take(E * 4);
    p.o_theta = take(E * 4);
    p.o_offsets = p.o_masks = p.o_cbase = p.o_sorted = p.o_pos = p.o_tiles = p.o_ntiles = -1;
    p.o_xlat = p.o_H = p.o_Hs = p.o_Y = p.o_R = -1;
    if (forward) {
        p.o_offsets = take((E + 1) * 4);
        p.o_masks = take(static_cast<int64_t>(p.nch) * E * 8);
        p.o_cbase = take(static_cast<int64_t>(p.nch) * E * 4);
        p.o_sorted = take(p.A * 4);
        p.o_pos = take(p.A * 4);
        p.o_tiles = take(static_cast<int64_t>(p.max_tiles) * sizeof(TileInfo));
        p.o_ntiles = take(8);
        if (p.dl) p.o_xlat = take(T * p.dl * p.es);
        p.o_H = take(p.A * p.F * p.es);
        if (p.ns) p.o_Hs = take(T * p.Fsh * p.es);
        const int64_t yrows = p.A + ((p.ns && !p.dl) ? T : 0);
        p.o_Y = take(yrows * p.din * p.es);
        if (p.dl) p.o_R = take(T * p.dl * p.es);
    }
    p.total = off;
    return p;
}

template <typename P>
P* at(void* ws, int64_t off) {
    return off < 0 ? nullptr : reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

#define MOE_HIP(x)                                   \
    do {                                             \
        if ((x) != hipSuccess) return MOE_ERR_HIP;   \
    } while (0)

GemmArgs gemm_args() {
    GemmArgs a{};
    a.nsplit = 1;
    return a;
}

// Router logits into the split-K partial planes of the workspace.
moe_status run_logits(const Plan& p, const void* x, const float* W_r, void* ws, hipStream_t s) {
    float* z = at<float>(ws, p.o_z);
    if (p.gemv) {
        MOE_HIP(launch_router_gemv(x, p.dt == DT_F32, W_r, p.T, p.d, p.E, p.ldz, z, s));
        return MOE_OK;
    }
    GemmArgs g = gemm_args();
    GemmGroup& G = g.g[0];
    if (p.dt == DT_BF16) {
        uint16_t* hi = at<uint16_t>(ws, p.o_planes);
        uint16_t* mid = hi + static_cast<int64_t>(p.E) * p.d;
        uint16_t* lo = mid + static_cast<int64_t>(p.E) * p.d;
        MOE_HIP(launch_split3(W_r, static_cast<int64_t>(p.E) * p.d, hi, mid, lo, s));
        const uint16_t* planes[3] = {hi, mid, lo};
        for (int i = 0; i < 3; ++i) G.seg[i] = GemmSeg{x, planes[i], nullptr, p.d, p.d, p.d, 0};
        G.nseg = 3;
    } else {
        G.seg[0] = GemmSeg{x, W_r, nullptr, p.d, p.d, p.d, 0};
        G.nseg = 1;
    }
    G.N = p.E;
    G.C = z;
    G.ldc = p.ldz;
    g.M = p.T;
    g.nsplit = p.nsplit;
    g.split_stride = static_cast<int64_t>(p.T) * p.ldz;
    MOE_HIP(launch_gemm(g, p.dt, true, EPI_STORE, p.rcfg, p.rtiles, p.E, false, s));
    return MOE_OK;
}

int64_t split_stride(const Plan& p) { return static_cast<int64_t>(p.T) * p.ldz; }

// Router: logits, then the top-K gate.
moe_status run_router(const Plan& p, const void* x, const float* W_r, const float* b, int32_t* idx, float* w,
                      int32_t* counts, void* ws, hipStream_t s) {
    moe_status st = run_logits(p, x, W_r, ws, s);
    if (st != MOE_OK) return st;
    MOE_HIP(launch_topk_gate(at<float>(ws, p.o_z), p.nsplit, split_stride(p), p.ldz, b, p.T, p.E, p.K, p.ng, p.tg,
                             p.scale, idx, w, counts, s));
    return MOE_OK;
}

// FP8 form of a grouped projection: g.g[0] the routed experts (FP8 weights
// with block scales bs / bsu), g.g[1] the shared experts (bf16), one launch.
hipError_t launch_f8(const Plan& p, GemmArgs g, const uint8_t* bs, const uint8_t* bsu, Epi epi, int max_n,
                     hipStream_t s) {
    g.g[0].bs = bs;
    g.g[0].bsu = bsu;
    g.g[0].s_estride = static_cast<int64_t>(g.g[0].N / 128) * (g.g[0].seg[0].K / 128);
    return launch_gemm_f8(g, epi, p.ecfg, p.max_tiles, max_n, s);
}

hipError_t record(void* const* ev, int i, hipStream_t s) {
    if (!ev || !ev[i]) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(ev[i]), s);
}

// Everything after the router: dispatch of the experts e0 .. e0 + p.E - 1
// of idx, the latent down-map, the up and down projections and the combine.
moe_status run_experts(const Plan& p, const void* x, const int32_t* idx, const float* w, int e0,
                       const moe_expert_weights* W, void* out, int32_t* u_counts, int32_t* u_offsets,
                       int32_t* u_sorted, void* ws, hipStream_t s, void* const* ev) {
    int32_t* counts = u_counts ? u_counts : at<int32_t>(ws, p.o_counts);
    int32_t* offsets = u_offsets ? u_offsets : at<int32_t>(ws, p.o_offsets);
    int32_t* sorted = u_sorted ? u_sorted : at<int32_t>(ws, p.o_sorted);
    int32_t* pos = at<int32_t>(ws, p.o_pos);
    TileInfo* tiles = at<TileInfo>(ws, p.o_tiles);
    int32_t* ntiles = at<int32_t>(ws, p.o_ntiles);
    char* H = at<char>(ws, p.o_H);
    char* Hs = at<char>(ws, p.o_Hs);
    char* Y = at<char>(ws, p.o_Y);
    char* xlat = at<char>(ws, p.o_xlat);
    char* R = at<char>(ws, p.o_R);
    const bool latent = p.dl > 0;

    // shared tiles ride in the routed launches (rows = tokens)
    MOE_HIP(launch_dispatch(idx, p.T, p.E, e0, p.K, p.bm, p.ns ? p.T : 0, at<uint64_t>(ws, p.o_masks),
                            at<int32_t>(ws, p.o_cbase), counts, offsets, sorted, pos, tiles, ntiles, s));
    MOE_HIP(record(ev, MOE_EV_DISPATCH, s));

    const void* xin = x;
    if (latent) {  // x_lat = x W_lat_down^T   [T, d_latent]
        GemmArgs g = gemm_args();
        g.g[0].seg[0] = GemmSeg{x, W->W_lat_down, nullptr, p.d, p.d, p.d, 0};
        g.g[0].nseg = 1;
        g.g[0].N = p.dl;
        g.g[0].C = xlat;
        g.g[0].ldc = p.dl;
        g.M = p.T;
        MOE_HIP(launch_gemm(g, p.dt, false, EPI_STORE, p.dcfg, static_cast<int>(cdiv(p.T, tile_bm(p.dcfg))), p.dl,
                            p.packed, s));
        xin = xlat;
    }
    MOE_HIP(record(ev, MOE_EV_LATENT, s));

    // up projection + SwiGLU: routed (gathered rows) and shared (all tokens)
    {
        GemmArgs g = gemm_args();
        GemmGroup& R0 = g.g[0];
        R0.seg[0] = GemmSeg{xin, W->W_gate, W->W_up, p.din, p.din, p.din, 0};
        R0.nseg = 1;
        R0.N = p.F;
        R0.b_estride = static_cast<int64_t>(p.F) * p.din;
        R0.rowmap = sorted;
        R0.C = H;
        R0.ldc = p.F;
        GemmGroup& S1 = g.g[1];
        S1.seg[0] = GemmSeg{x, W->Ws_gate, W->Ws_up, p.d, p.d, p.d, 0};
        S1.nseg = 1;
        S1.N = p.Fsh;
        S1.C = Hs;
        S1.ldc = p.Fsh;
        g.tiles = tiles;
        g.ntiles = ntiles;
        if (p.f8)
            MOE_HIP(launch_f8(p, g, W->W_gate_scale, W->W_up_scale, EPI_SWIGLU, std::max(p.F, p.Fsh), s));
        else
            MOE_HIP(launch_gemm(g, p.dt, false, EPI_SWIGLU, p.ecfg, p.max_tiles, std::max(p.F, p.Fsh), p.packed, s));
    }
    MOE_HIP(record(ev, MOE_EV_UP, s));
    // down projection: routed -> Y[sorted rows]; shared (K2 form) -> Y[A + t]
    {
        GemmArgs g = gemm_args();
        GemmGroup& R0 = g.g[0];
        R0.seg[0] = GemmSeg{H, W->W_down, nullptr, p.F, p.F, p.F, 0};
        R0.nseg = 1;
        R0.N = p.din;
        R0.b_estride = static_cast<int64_t>(p.din) * p.F;
        R0.C = Y;
        R0.ldc = p.din;
        GemmGroup& S1 = g.g[1];
        if (p.ns && !latent) {
            S1.seg[0] = GemmSeg{Hs, W->Ws_down, nullptr, p.Fsh, p.Fsh, p.Fsh, 0};
            S1.nseg = 1;
            S1.N = p.d;
            S1.C = Y + p.A * p.d * p.es;
            S1.ldc = p.d;
        } else {
            S1.N = 0;  // shared tiles (latent form) do nothing here
            S1.nseg = 0;
        }
        g.tiles = tiles;
        g.ntiles = ntiles;
        if (p.f8)
            MOE_HIP(launch_f8(p, g, W->W_down_scale, nullptr, EPI_STORE, p.din, s));
        else
            MOE_HIP(launch_gemm(g, p.dt, false, EPI_STORE, p.ecfg, p.max_tiles, p.din, p.packed, s));
    }
    MOE_HIP(record(ev, MOE_EV_DOWN, s));
    if (!latent) {
        const void* ysh = p.ns ? static_cast<const void*>(Y + p.A * p.d * p.es) : nullptr;
        MOE_HIP(launch_combine(p.dt, Y, p.d, ysh, pos, w, p.T, p.K, p.d, out, p.d, s));
        MOE_HIP(record(ev, MOE_EV_END, s));
        return MOE_OK;
    }
    // latent form: R = sum_k w Y[pos];  out = Hs Ws_down^T + R W_lat_up^T
    MOE_HIP(launch_combine(p.dt, Y, p.dl, nullptr, pos, w, p.T, p.K, p.dl, R, p.dl, s));
    GemmArgs g = gemm_args();
    GemmGroup& G = g.g[0];
    int ns = 0;
    if (p.ns) G.seg[ns++] = GemmSeg{Hs, W->Ws_down, nullptr, p.Fsh, p.Fsh, p.Fsh, 0};
    G.seg[ns++] = GemmSeg{R, W->W_lat_up, nullptr, p.dl, p.dl, p.dl, 0};
    G.nseg = ns;
    G.N = p.d;
    G.C = out;
    G.ldc = p.d;
    g.M = p.T;
    MOE_HIP(launch_gemm(g, p.dt, false, EPI_STORE, p.dcfg, static_cast<int>(cdiv(p.T, tile_bm(p.dcfg))), p.d,
                        p.packed, s));
    MOE_HIP(record(ev, MOE_EV_END, s));
    return MOE_OK;
}

moe_status run_forward(const Plan& p, const void* x, const float* W_r, const float* b, const moe_expert_weights* W,
                       void* out, int32_t* u_idx, float* u_w, int32_t* u_counts, int32_t* u_offsets,
                       int32_t* u_sorted, void* ws, hipStream_t s, void* const* ev) {
    int32_t* idx = u_idx ? u_idx : at<int32_t>(ws, p.o_idx);
    float* w = u_w ? u_w : at<float>(ws, p.o_w);
    MOE_HIP(record(ev, MOE_EV_START, s));
    moe_status st = run_router(p, x, W_r, b, idx, w, nullptr, ws, s);
    if (st != MOE_OK) return st;
    MOE_HIP(record(ev, MOE_EV_ROUTER, s));
    return run_experts(p, x, idx, w, 0, W, out, u_counts, u_offsets, u_sorted, ws, s, ev);
}

// The checks of a slice: the descriptor as a whole layer of E_total experts
// (K, shapes, dtypes), then the slice inside it.
moe_status check_slice(const moe_layer_desc* desc, int e0, int E_total) {
    if (!desc) return MOE_ERR_NULL;
    if (E_total < 1 || E_total > 1024 || e0 < 0 || desc->E < 1 || e0 > E_total - desc->E) return MOE_ERR_SHAPE;
    moe_layer_desc whole = *desc;
    whole.E = E_total;
    whole.n_group = 1;  // the routing comes from the caller
    whole.topk_group = 1;
    return check_desc(&whole, true);
}

// The weight pointers every forward needs, with their alignment.
moe_status check_weights(const moe_layer_desc* desc, const moe_expert_weights* W) {
    if (!W->W_gate || !W->W_up || !W->W_down) return MOE_ERR_NULL;
    if (desc->w_dtype == MOE_FP8_E4M3 && (!W->W_gate_scale || !W->W_up_scale || !W->W_down_scale))
        return MOE_ERR_NULL;
    if (desc->n_shared > 0 && (!W->Ws_gate || !W->Ws_up || !W->Ws_down)) return MOE_ERR_NULL;
    if (desc->d_latent > 0 && (!W->W_lat_down || !W->W_lat_up)) return MOE_ERR_NULL;
    const void* need[] = {W->W_gate, W->W_up, W->W_down};
    for (const void* q : need)
        if (!aligned16(q)) return MOE_ERR_ALIGN;
    if (desc->n_shared > 0 && (!aligned16(W->Ws_gate) || !aligned16(W->Ws_up) || !aligned16(W->Ws_down)))
        return MOE_ERR_ALIGN;
    if (desc->d_latent > 0 && (!aligned16(W->W_lat_down) || !aligned16(W->W_lat_up))) return MOE_ERR_ALIGN;
    return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_layer_desc* desc, int for_forward) {
    if (check_desc(desc, for_forward != 0) != MOE_OK) return 0;
    return static_cast<size_t>(make_plan(desc, for_forward != 0).total);
}

const char* moe_status_str(moe_status st) {
    switch (st) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "a size is out of range";
        case MOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_size()";
        case MOE_ERR_UNSUPPORTED: return "unsupported dtype combination";
        case MOE_ERR_HIP: return "a HIP launch failed";
        case MOE_ERR_SCRATCH: return "the layer needs more than the fixed scratch of moe_forward_noalloc";
    }
    return "unknown status";
}

moe_status moe_router(const moe_layer_desc* desc, const void* x, const float* W_r, const float* b, int32_t* topk_idx,
                      float* topk_w, int32_t* expert_counts, void* workspace, size_t workspace_bytes, void* stream) {
    moe_status st = check_desc(desc, false);
    if (st != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (desc->T == 0) {  // no tokens: empty tensors may come as NULL pointers
        if (expert_counts && !aligned16(expert_counts)) return MOE_ERR_ALIGN;
        if (expert_counts) MOE_HIP(launch_fill_i32(expert_counts, 0, desc->E, s));
        return MOE_OK;
    }
    if (!x || !W_r || !b || !topk_idx || !topk_w || !workspace) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(W_r) || !aligned16(b) || !aligned16(topk_idx) || !aligned16(topk_w) ||
        !aligned16(workspace) || (expert_counts && !aligned16(expert_counts)))
        return MOE_ERR_ALIGN;
    const Plan p = make_plan(desc, false);
    if (workspace_bytes < static_cast<size_t>(p.total)) return MOE_ERR_WORKSPACE;
    return run_router(p, x, W_r, b, topk_idx, topk_w, expert_counts, workspace, s);
}

moe_status moe_forward(const moe_layer_desc* desc, const void* x, const float* W_r, const float* b,
                       const moe_expert_weights* weights, void* out, int32_t* topk_idx, float* topk_w,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_token, void* workspace,
                       size_t workspace_bytes, void* stream, void* const* stage_events) {
    moe_status st = check_desc(desc, true);
    if (st != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (desc->T == 0) {  // no tokens: empty tensors may come as NULL pointers
        if ((expert_counts && !aligned16(expert_counts)) || (expert_offsets && !aligned16(expert_offsets)))
            return MOE_ERR_ALIGN;
        for (int i = 0; i < MOE_NUM_STAGE_EVENTS; ++i) MOE_HIP(record(stage_events, i, s));
        if (expert_counts) MOE_HIP(launch_fill_i32(expert_counts, 0, desc->E, s));
        if (expert_offsets) MOE_HIP(launch_fill_i32(expert_offsets, 0, desc->E + 1, s));
        return MOE_OK;
    }
    if (!x || !W_r || !b || !weights || !out || !workspace) return MOE_ERR_NULL;
    const moe_expert_weights* W = weights;
    st = check_weights(desc, W);
    if (st != MOE_OK) return st;
    const void* need[] = {x, W_r, b, out, workspace};
    for (const void* q : need)
        if (!aligned16(q)) return MOE_ERR_ALIGN;
    const void* opt[] = {topk_idx, topk_w, expert_counts, expert_offsets, sorted_token};
    for (const void* q : opt)
        if (q && !aligned16(q)) return MOE_ERR_ALIGN;
    const Plan p = make_plan(desc, true);
    if (workspace_bytes < static_cast<size_t>(p.total)) return MOE_ERR_WORKSPACE;
    return run_forward(p, x, W_r, b, W, out, topk_idx, topk_w, expert_counts, expert_offsets, sorted_token,
                       workspace, s, stage_events);
}

size_t moe_slice_workspace_size(const moe_layer_desc* desc, int32_t e0, int32_t E_total) {
    if (check_slice(desc, e0, E_total) != MOE_OK) return 0;
    return static_cast<size_t>(make_plan(desc, true, E_total).total);
}

moe_status moe_forward_slice(const moe_layer_desc* desc, const moe_expert_weights* weights, const void* x,
                             const int32_t* topk_idx, const float* topk_w, int32_t e0, int32_t E_total, void* out,
                             int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_token,
                             void* workspace, size_t workspace_bytes, void* stream) {
    moe_status st = check_slice(desc, e0, E_total);
    if (st != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((expert_counts && !aligned16(expert_counts)) || (expert_offsets && !aligned16(expert_offsets)) ||
        (sorted_token && !aligned16(sorted_token)))
        return MOE_ERR_ALIGN;
    if (desc->T == 0) {  // no tokens: empty tensors may come as NULL pointers
        if (expert_counts) MOE_HIP(launch_fill_i32(expert_counts, 0, desc->E, s));
        if (expert_offsets) MOE_HIP(launch_fill_i32(expert_offsets, 0, desc->E + 1, s));
        return MOE_OK;
    }
    if (!x || !topk_idx || !topk_w || !weights || !out || !workspace) return MOE_ERR_NULL;
    st = check_weights(desc, weights);
    if (st != MOE_OK) return st;
    const void* need[] = {x, topk_idx, topk_w, out, workspace};
    for (const void* q : need)
        if (!aligned16(q)) return MOE_ERR_ALIGN;
    const Plan p = make_plan(desc, true, E_total);
    if (workspace_bytes < static_cast<size_t>(p.total)) return MOE_ERR_WORKSPACE;
    return run_experts(p, x, topk_idx, topk_w, e0, weights, out, expert_counts, expert_offsets, sorted_token,
                       workspace, s, nullptr);
}

moe_status moe_bias_quantile(const moe_layer_desc* desc, const void* x, const float* W_r, float* b,
                             void* workspace, size_t workspace_bytes, void* stream) {
    moe_status st = check_desc(desc, false);
    if (st != MOE_OK) return st;
    if (desc->T < 1 || desc->T > kQuantileMaxT) return MOE_ERR_SHAPE;
    if (!x || !W_r || !b || !workspace) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(W_r) || !aligned16(b) || !aligned16(workspace)) return MOE_ERR_ALIGN;
    const Plan p = make_plan(desc, false);
    if (workspace_bytes < static_cast<size_t>(p.total)) return MOE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = run_logits(p, x, W_r, workspace, s);
    if (st != MOE_OK) return st;
    const int64_t n = std::max<int64_t>(1, static_cast<int64_t>(p.T) * p.K / p.E);
    MOE_HIP(launch_quantile_bias(at<float>(workspace, p.o_z), p.nsplit, split_stride(p), p.ldz, p.T, p.E,
                                 static_cast<int>(n), at<float>(workspace, p.o_theta), b, s));
    return MOE_OK;
}

moe_status moe_bias_update(const moe_layer_desc* desc, const int32_t* expert_counts, float* b, float gamma,
                           void* stream) {
    if (!desc) return MOE_ERR_NULL;
    if (desc->E < 1 || desc->E > 1024) return MOE_ERR_SHAPE;
    if (!expert_counts || !b) return MOE_ERR_NULL;
    if (!aligned16(expert_counts) || !aligned16(b)) return MOE_ERR_ALIGN;
    MOE_HIP(launch_bias_update(expert_counts, desc->E, gamma, b, static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

moe_status moe_pack_weights(const moe_layer_desc* desc, const moe_expert_weights* src,
                            const moe_expert_weights* dst, void* stream) {
    if (!desc || !src || !dst) return MOE_ERR_NULL;
    moe_layer_desc D = *desc;
    if (D.w_dtype != MOE_BF16 && D.w_dtype != MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
    // shapes as for the forward over the packed result (src is row-major)
    D.w_layout = MOE_LAYOUT_FRAG16;
    const moe_status st = check_desc(&D, true);
    if (st != MOE_OK) return st;
    const int din = D.d_latent ? D.d_latent : D.d, Fsh = D.n_shared * D.F_shared;
    const bool f8 = D.w_dtype == MOE_FP8_E4M3;  // routed matrices: one byte per element
    struct Mat {
        const void* s;
        const void* d;
        int64_t count;
        int rows, cols;
        bool f8;
    };
    const Mat mats[] = {
        {src->W_gate, dst->W_gate, D.E, D.F, din, f8},     {src->W_up, dst->W_up, D.E, D.F, din, f8},
        {src->W_down, dst->W_down, D.E, din, D.F, f8},     {src->Ws_gate, dst->Ws_gate, 1, Fsh, D.d, false},
        {src->Ws_up, dst->Ws_up, 1, Fsh, D.d, false},      {src->Ws_down, dst->Ws_down, 1, D.d, Fsh, false},
        {src->W_lat_down, dst->W_lat_down, 1, D.d_latent, D.d, false},
        {src->W_lat_up, dst->W_lat_up, 1, D.d, D.d_latent, false},
    };
    for (const Mat& m : mats) {  // validate everything before enqueueing
        if (!m.s) continue;
        if (!m.d) return MOE_ERR_NULL;
        if (!aligned16(m.s) || !aligned16(m.d)) return MOE_ERR_ALIGN;
        if (m.rows <= 0 || m.cols <= 0) return MOE_ERR_SHAPE;
        const uintptr_t bytes = static_cast<uintptr_t>(m.count) * m.rows * m.cols * (m.f8 ? 1 : 2);
        const uintptr_t a = reinterpret_cast<uintptr_t>(m.s), b = reinterpret_cast<uintptr_t>(m.d);
        if (a < b + bytes && b < a + bytes) return MOE_ERR_SHAPE;  // overlapping buffers
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (const Mat& m : mats) {
        if (!m.s) continue;
        if (m.f8)
            MOE_HIP(launch_pack_frag16_fp8(static_cast<const uint8_t*>(m.s), static_cast<uint8_t*>(const_cast<void*>(m.d)),
                                           m.count, m.rows, m.cols, s));
        else
            MOE_HIP(launch_pack_frag16(static_cast<const uint16_t*>(m.s), static_cast<uint16_t*>(const_cast<void*>(m.d)),
                                       m.count, m.rows, m.cols, s));
    }
    return MOE_OK;
}

}  // extern "C"
