// Router kernels of the MoE layer (OpenModelAtlas "Kimi K2 · Router": the
// four steps z = x W_r, s = sigmoid(z), top-K of s + b, renormalised and
// scaled weights; the MoEGate excerpt computes the logits in fp32 and, with
// more than one expert group, limits the choice to the best groups).
//
// The logits of up to 32 tokens are fp32 dot products (k_router_gemv);
// above that they come from the grouped GEMM (gemm.hip).  For bf16
// activations the fp32 router weight is then split exactly into three bf16
// planes, W_r = hi + mid + lo (Henry, Tang & Heinecke 2019, "Leveraging the
// bfloat16 Artificial Intelligence Datatype for Higher-Precision
// Computations"): every bf16 x bf16 product is exact in the fp32 MFMA
// accumulator, so three bf16 MFMA passes give an fp32-accumulated product
// of the exact inputs at 16/3 times the fp32 MFMA rate.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

// hi = rne(w); mid = rne(w - hi); lo = rne(w - hi - mid).  Each difference
// is exact in fp32 (its operands agree to within a factor of two), and
// after two 8-bit captures at most 8 significant bits remain, so lo holds
// the rest exactly: hi + mid + lo == w for finite normal w.
__device__ __forceinline__ void split3_one(float w, bf16_t& h, bf16_t& m, bf16_t& l) {
    h = f32_to_bf16(w);
    const float r1 = w - bf16_to_f32(h);
    m = f32_to_bf16(r1);
    l = f32_to_bf16(r1 - bf16_to_f32(m));
}

// Four consecutive weights per thread: one 16-byte load, three 8-byte
// stores (2-byte stores of one weight per thread took twice as long); the
// last n % 4 weights one by one.
__global__ __launch_bounds__(256) void k_split3(const float* __restrict__ W, int64_t n, bf16_t* __restrict__ hi,
                                                bf16_t* __restrict__ mid, bf16_t* __restrict__ lo) {
    const int64_t n4 = n / 4, stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n4; i += stride) {
        const float4 w = reinterpret_cast<const float4*>(W)[i];
        const float v[4] = {w.x, w.y, w.z, w.w};
        uint32_t ph[2], pm[2], pl[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            bf16_t h0, m0, l0, h1, m1, l1;
            split3_one(v[2 * q], h0, m0, l0);
            split3_one(v[2 * q + 1], h1, m1, l1);
            ph[q] = h0 | (static_cast<uint32_t>(h1) << 16);
            pm[q] = m0 | (static_cast<uint32_t>(m1) << 16);
            pl[q] = l0 | (static_cast<uint32_t>(l1) << 16);
        }
        reinterpret_cast<uint2*>(hi)[i] = make_uint2(ph[0], ph[1]);
        reinterpret_cast<uint2*>(mid)[i] = make_uint2(pm[0], pm[1]);
        reinterpret_cast<uint2*>(lo)[i] = make_uint2(pl[0], pl[1]);
    }
    for (int64_t i = 4 * n4 + blockIdx.x * 256ll + threadIdx.x; i < n; i += stride)
        split3_one(W[i], hi[i], mid[i], lo[i]);
}

// Router logits of a few tokens straight from the fp32 weight (T <=
// kRouterGemvMaxT): one workgroup per expert reads its row of W_r once, 16
// bytes per lane, and forms the T dot products with fp32 FMAs; the lanes'
// partial sums are then added in a fixed tree (the wave's butterfly, then
// the four waves in pairs), so the result does not depend on timing.
// Each product of a bf16 (or fp32) activation and the fp32 weight is exact
// inside the FMA, as in the three-plane form, and the sums are fp32.  At
// these sizes the planes and a split-K GEMM cost more, in launches and in a
// chip left mostly idle, than the arithmetic.
__device__ __forceinline__ void load4(const bf16_t* p, float (&o)[4]) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    o[0] = __uint_as_float(v.x << 16);
    o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16);
    o[3] = __uint_as_float(v.y & 0xffff0000u);
}
__device__ __forceinline__ void load4(const float* p, float (&o)[4]) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    o[0] = v.x;
    o[1] = v.y;
    o[2] = v.z;
    o[3] = v.w;
}

// TM: the kernel's token capacity (a power of two >= T); rows past T - 1
// repeat row T - 1 and are not written, so every load of a chunk is issued
// before its FMAs, with no branch between them.
template <typename TX, int TM>
__global__ __launch_bounds__(256) void k_router_gemv(const TX* __restrict__ x, const float* __restrict__ W, int T,
                                                     int d, int ldz, float* __restrict__ z) {
    __shared__ float red[4][TM];
    const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const float* w = W + static_cast<int64_t>(e) * d;
    const TX* xr[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) xr[t] = x + static_cast<int64_t>(t < T ? t : T - 1) * d;
    float acc[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[t] = 0.f;
    for (int c = tid * 4; c < d; c += 1024) {
        const float4 wv = *reinterpret_cast<const float4*>(w + c);
        float xv[TM][4];
#pragma unroll
        for (int t = 0; t < TM; ++t) load4(xr[t] + c, xv[t]);
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            acc[t] = fmaf(xv[t][0], wv.x, acc[t]);
            acc[t] = fmaf(xv[t][1], wv.y, acc[t]);
            acc[t] = fmaf(xv[t][2], wv.z, acc[t]);
            acc[t] = fmaf(xv[t][3], wv.w, acc[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        float v = acc[t];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0) red[wid][t] = v;
    }
    __syncthreads();
    if (tid < T) z[static_cast<int64_t>(tid) * ldz + e] = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
}

__global__ __launch_bounds__(256) void k_fill_i32(int32_t* p, int32_t v, int64_t n) {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) p[i] = v;
}

// (value, index) order of the selection: larger biased score first, the
// lower expert index on equal scores, as one unsigned 64-bit key.  The top
// half is the score's bits made monotone (negative floats flipped, positive
// ones offset by the sign bit; -0 is first made +0, since the two compare
// equal), the bottom half the complement of the index, so that of two equal
// scores the lower index has the larger key.  Every valid pair's key is
// above 0 (-inf maps to 0x007fffff in the top half).
__device__ __forceinline__ uint64_t sel_key(float v, int e) {
    uint32_t u = __float_as_uint(v + 0.0f);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<uint64_t>(u) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(e));
}

// One wave per token.  Lane l holds experts l, l+64, l+128, ... (J of
// them), so inside a lane the expert index rises with j.  K rounds of a
// wave-wide (value, index) arg-max pick the set; slot order is then the
// ascending expert id (rank of each pick among the picks).
// Group-limited choice (router card, MoEGate excerpt, noaux_tc branch):
// the E experts form n_group contiguous groups of `per`; a group scores the
// sum of its two largest biased scores; the topk_group best groups are kept
// (ties toward the lower group index); every expert of a dropped group
// takes the value 0.0 (the excerpt's masked_fill), the others keep theirs.
// n_group <= 64: lane g ends up holding group g's score.
template <int J>
__device__ __forceinline__ void limit_to_groups(float (&v)[J], int lane, int E, int n_group, int per,
                                                int topk_group) {
    float gscore = -INFINITY;
    for (int g = 0; g < n_group; ++g) {
        float m1 = -INFINITY, m2 = -INFINITY;  // two largest of this lane's members of g
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int e = j * 64 + lane;
            if (e < E && e / per == g) {
                if (v[j] > m1) {
                    m2 = m1;
                    m1 = v[j];
                } else if (v[j] > m2) {
                    m2 = v[j];
                }
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {  // merge the lanes' pairs
            const float o1 = __shfl_xor(m1, off), o2 = __shfl_xor(m2, off);
            const float n2 = fmaxf(fminf(m1, o1), fmaxf(m2, o2));
            m1 = fmaxf(m1, o1);
            m2 = n2;
        }
        if (lane == g) gscore = m1 + m2;
    }
    bool kept = false;
    for (int k = 0; k < topk_group; ++k) {
        const bool cand = lane < n_group && !kept;
        float bv = cand ? gscore : -INFINITY;
        int bg = cand ? lane : 0x7fffffff;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int og = __shfl_xor(bg, off);
            if (ov > bv || (ov == bv && og < bg)) {
                bv = ov;
                bg = og;
            }
        }
        if (lane == bg) kept = true;
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int e = j * 64 + lane;
        const int g = (e < E ? e : E - 1) / per;
        const bool keep = __shfl(kept ? 1 : 0, g) != 0;
        if (e < E && !keep) v[j] = 0.0f;
    }
}

constexpr int kMaxSplit = 16;  // split-K partial planes the gate sums (the router plan caps at 16)

template <int J>
__global__ __launch_bounds__(256) void k_topk_gate(const float* __restrict__ z, int nsplit, int64_t split_stride,
                                                   int ldz, const float* __restrict__ b, int T, int E, int K,
                                                   int n_group, int topk_group, float scale,
                                                   int32_t* __restrict__ idx, float* __restrict__ w,
                                                   int32_t* __restrict__ counts) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    // the per-expert counts start at zero here; k_expert_counts, launched
    // after this kernel, adds them up
    if (counts && blockIdx.x == 0)
        for (int e = threadIdx.x; e < E; e += 256) counts[e] = 0;
    if (t >= T) return;
    float v[J], s[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int e = j * 64 + lane;
        if (e < E) {
            // every split-K partial is loaded before the first add (a loop of
            // dependent load-adds waited out one memory latency per plane);
            // the adds keep plane order
            float part[kMaxSplit];
#pragma unroll
            for (int p = 0; p < kMaxSplit; ++p)
                part[p] = p < nsplit ? z[p * split_stride + static_cast<int64_t>(t) * ldz + e] : 0.f;
            float zz = 0.f;
#pragma unroll
            for (int p = 0; p < kMaxSplit; ++p)
                if (p < nsplit) zz += part[p];
            s[j] = 1.0f / (1.0f + expf(-zz));  // step 2: per-expert sigmoid
            v[j] = s[j] + b[e];                // step 3: the bias only chooses
            // A NaN score would never win a comparison and leave the arg-max
            // on its out-of-range sentinel; rank it below every number so the
            // K picks are always valid, distinct expert ids.
            if (!(v[j] == v[j])) v[j] = -INFINITY;
        } else {
            s[j] = 0.f;
            v[j] = -INFINITY;
        }
    }
    if (n_group > 1) limit_to_groups<J>(v, lane, E, n_group, E / n_group, topk_group);
    uint64_t key[J];
#pragma unroll
    for (int j = 0; j < J; ++j) key[j] = j * 64 + lane < E ? sel_key(v[j], j * 64 + lane) : 0ull;
    uint32_t taken = 0;
    int my_e = 0;
    float my_s = 0.f, den = 0.f;
    for (int k = 0; k < K; ++k) {
        // this lane's best untaken expert, then the wave-wide largest key;
        // the winning lane's own best is the winner, so its score comes
        // from that lane with one shuffle
        uint64_t bk = 0;
        float bs = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            if (!((taken >> j) & 1u) && key[j] > bk) {
                bk = key[j];
                bs = s[j];
            }
        }
        uint64_t wk = bk;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const uint32_t ohi = __shfl_xor(static_cast<uint32_t>(wk >> 32), off);
            const uint32_t olo = __shfl_xor(static_cast<uint32_t>(wk), off);
            const uint64_t ok = (static_cast<uint64_t>(ohi) << 32) | olo;
            wk = ok > wk ? ok : wk;
        }
        const int be = static_cast<int>(~static_cast<uint32_t>(wk));
        bs = __shfl(bs, be & 63);
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (lane == k) {
            my_e = be;
            my_s = bs;
        }
        den += bs;  // sum of the unbiased scores of the set, in pick order
    }
    // step 4: renormalise over the set (+1e-20 as in the MoEGate excerpt)
    // and apply the routed scaling factor
    den += 1e-20f;
    int rank = 0;
    for (int j = 0; j < K; ++j) rank += __shfl(my_e, j) < my_e ? 1 : 0;
    if (lane < K) {
        idx[static_cast<int64_t>(t) * K + rank] = my_e;
        w[static_cast<int64_t>(t) * K + rank] = (my_s / den) * scale;
    }
}

// Per-expert counts of the n = T K selections in idx: each block counts its
// share in LDS, then adds its nonzero bins to counts (zeroed by the gate's
// first block).  Integer adds, so the result does not depend on their
// order; the global adds of one address number at most the blocks (64),
// where one add per selection (T K of them, a hot expert's thousands to
// one address) serialised in L2.
constexpr int kCountsMaxE = 1024;
__global__ __launch_bounds__(1024) void k_expert_counts(const int32_t* __restrict__ idx, int64_t n, int E,
                                                        int32_t* __restrict__ counts) {
    __shared__ int h[kCountsMaxE];
    for (int e = threadIdx.x; e < E; e += 1024) h[e] = 0;
    __syncthreads();
    for (int64_t i = blockIdx.x * 1024ll + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 1024) {
        const unsigned e = static_cast<unsigned>(idx[i]);
        if (e < static_cast<unsigned>(E)) atomicAdd(&h[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 1024)
        if (h[e]) atomicAdd(counts + e, h[e]);
}

// Aux-loss-free bias update after a batch (llm-arch-kb "Kimi K2 MoE": the
// selection bias follows DeepSeek V3's schedule, gamma = 1e-3, sign only):
// b_e += gamma * sgn(mean count - c_e), the comparison taken exactly as
// sum(c) - E c_e.  One block; thread e owns expert e (E <= 1024).
__global__ __launch_bounds__(1024) void k_bias_update(const int32_t* __restrict__ counts, int E, float gamma,
                                                      float* __restrict__ b) {
    __shared__ long long part[16];
    const int e = threadIdx.x, lane = e & 63, w = e >> 6;
    long long c = e < E ? counts[e] : 0;
    long long sum = c;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane == 0) part[w] = sum;
    __syncthreads();
    long long total = 0;
    for (int i = 0; i < 16; ++i) total += part[i];
    if (e < E) {
        const long long diff = total - static_cast<long long>(E) * c;
        const float sg = diff > 0 ? 1.0f : (diff < 0 ? -1.0f : 0.0f);
        b[e] = b[e] + gamma * sg;  // gamma * sg is exact: one rounding
    }
}

// Quantile Balancing (lilting.ch K3 essay, load-balancing paragraph; read
// as: theta_e = the n-th largest router score of expert e over the batch,
// b_e = mean(theta) - theta_e).  Block e gathers sigmoid(z[., e]) into LDS
// (summing the split-K partial planes) and selects the n-th largest by a
// most-significant-digit radix select over the fp32 bit patterns, 8 bits a
// pass: scores are >= 0, so bit order is value order and the result is the
// exact order statistic.
__global__ __launch_bounds__(256) void k_quantile_theta(const float* __restrict__ z, int nsplit,
                                                        int64_t split_stride, int ldz, int T, int n,
                                                        float* __restrict__ theta) {
    extern __shared__ uint32_t vals[];  // T fp32 bit patterns
    __shared__ uint32_t hist[256];
    __shared__ uint32_t pick_prefix;
    __shared__ int pick_rem;
    const int e = blockIdx.x, tid = threadIdx.x;
    for (int t = tid; t < T; t += 256) {
        float zz = 0.f;
        for (int p = 0; p < nsplit; ++p) zz += z[p * split_stride + static_cast<int64_t>(t) * ldz + e];
        float sc = 1.0f / (1.0f + expf(-zz));
        if (!(sc == sc)) sc = 0.0f;
        vals[t] = __float_as_uint(sc);
    }
    uint32_t prefix = 0, mask = 0;
    int rem = n;  // rank (1-based, from the top) still to find among the matching values
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        hist[tid] = 0;
        __syncthreads();
        for (int t = tid; t < T; t += 256) {
            const uint32_t u = vals[t];
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid == 0) {
            int acc = 0, dgt = 255;
            for (; dgt > 0; --dgt) {
                if (acc + static_cast<int>(hist[dgt]) >= rem) break;
                acc += static_cast<int>(hist[dgt]);
            }
            pick_prefix = prefix | (static_cast<uint32_t>(dgt) << shift);
            pick_rem = rem - acc;
        }
        __syncthreads();
        prefix = pick_prefix;
        rem = pick_rem;
        mask |= 255u << shift;
    }
    if (tid == 0) theta[e] = __uint_as_float(prefix);
}

// b_e = mean(theta) - theta_e; one block, thread e owns expert e.
__global__ __launch_bounds__(1024) void k_bias_center(const float* __restrict__ theta, int E, float* __restrict__ b) {
    __shared__ float part[16];
    const int e = threadIdx.x, lane = e & 63, w = e >> 6;
    const float th = e < E ? theta[e] : 0.f;
    float sum = th;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane == 0) part[w] = sum;
    __syncthreads();
    float total = 0.f;
    for (int i = 0; i < 16; ++i) total += part[i];
    if (e < E) b[e] = total / static_cast<float>(E) - th;
}

}  // namespace

hipError_t launch_quantile_bias(const float* z, int nsplit, int64_t split_stride, int ldz, int T, int E, int n,
                                float* theta, float* b, hipStream_t stream) {
    if (T <= 0 || E <= 0 || E > 1024 || n < 1 || n > T || T > kQuantileMaxT) return hipErrorInvalidValue;
    const size_t lds = static_cast<size_t>(T) * 4;
    if (lds > 48 * 1024) {  // more dynamic LDS than the default allowance (gfx950 has 160 KiB)
        const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_quantile_theta),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(k_quantile_theta, dim3(E), dim3(256), lds, stream, z, nsplit, split_stride, ldz, T, n,
                       theta);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_bias_center, dim3(1), dim3(1024), 0, stream, theta, E, b);
    return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t* counts, int E, float gamma, float* b, hipStream_t stream) {
    if (E <= 0) return hipSuccess;
    if (E > 1024) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_bias_update, dim3(1), dim3(1024), 0, stream, counts, E, gamma, b);
    return hipGetLastError();
}

hipError_t launch_split3(const float* W, int64_t n, uint16_t* hi, uint16_t* mid, uint16_t* lo, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(k_split3, dim3(static_cast<unsigned>(blocks < 8192 ? blocks : 8192)), dim3(256), 0, stream, W,
                       n, hi, mid, lo);
    return hipGetLastError();
}

hipError_t launch_router_gemv(const void* x, bool x_f32, const float* W, int T, int d, int E, int ldz, float* z,
                              hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    if (T > kRouterGemvMaxT || d <= 0 || d % 4 || E <= 0 || ldz < E) return hipErrorInvalidValue;
#define MOE_GEMV(TM)                                                                                      \
    do {                                                                                                  \
        if (x_f32)                                                                                        \
            hipLaunchKernelGGL((k_router_gemv<float, TM>), dim3(E), dim3(256), 0, stream,                 \
                               static_cast<const float*>(x), W, T, d, ldz, z);                            \
        else                                                                                              \
            hipLaunchKernelGGL((k_router_gemv<bf16_t, TM>), dim3(E), dim3(256), 0, stream,                \
                               static_cast<const bf16_t*>(x), W, T, d, ldz, z);                           \
    } while (0)
    if (T <= 1)
        MOE_GEMV(1);
    else if (T <= 2)
        MOE_GEMV(2);
    else if (T <= 4)
        MOE_GEMV(4);
    else if (T <= 8)
        MOE_GEMV(8);
    else if (T <= 16)
        MOE_GEMV(16);
    else
        MOE_GEMV(32);
#undef MOE_GEMV
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(k_fill_i32, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream, p,
                       v, n);
    return hipGetLastError();
}

hipError_t launch_topk_gate(const float* z, int nsplit, int64_t split_stride, int ldz, const float* b, int T, int E,
                            int K, int n_group, int topk_group, float scale, int32_t* idx, float* w, int32_t* counts,
                            hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    if (n_group < 1 || n_group > 64 || E % n_group || topk_group < 1 || topk_group > n_group ||
        (n_group > 1 && E / n_group < 2) || nsplit < 1 || nsplit > kMaxSplit)
        return hipErrorInvalidValue;
    const dim3 grid((T + 3) / 4), block(256);
    const int J = (E + 63) / 64;
#define MOE_TOPK(JJ)                                                                                           \
    hipLaunchKernelGGL(k_topk_gate<JJ>, grid, block, 0, stream, z, nsplit, split_stride, ldz, b, T, E, K, n_group, \
                       topk_group, scale, idx, w, counts)
    if (J <= 1)
        MOE_TOPK(1);
    else if (J <= 2)
        MOE_TOPK(2);
    else if (J <= 4)
        MOE_TOPK(4);
    else if (J <= 6)
        MOE_TOPK(6);
    else if (J <= 8)
        MOE_TOPK(8);
    else if (J <= 14)
        MOE_TOPK(14);
    else
        MOE_TOPK(16);
#undef MOE_TOPK
    if (counts) {
        if (E > kCountsMaxE) return hipErrorInvalidValue;
        const int64_t n = static_cast<int64_t>(T) * K;
        const int64_t blocks = std::min<int64_t>(64, (n + 16383) / 16384);
        hipLaunchKernelGGL(k_expert_counts, dim3(static_cast<unsigned>(blocks)), dim3(1024), 0, stream, idx, n, E,
                           counts);
    }
    return hipGetLastError();
}

}  // namespace moe
