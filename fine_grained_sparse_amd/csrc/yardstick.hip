// Yardsticks for the roofline fractions the bench reports (libyardstick.so;
// not part of the layer or its C ABI).  Each kernel is timed by the caller
// with events on `stream`:
//   ys_stream_read  reads a buffer once, 16 bytes per lane, 8 or 16 loads in
//                   flight per lane (plain or non-temporal loads): the HBM
//                   read rate the chip delivers to a pure stream;
//   ys_mfma_loop    chains of v_mfma_f32_16x16x32_bf16 on register operands,
//                   16 independent accumulators per wave, one wave per SIMD
//                   when launched with one workgroup per CU: the bf16 MFMA
//                   rate without any memory traffic.  It also records the
//                   shader clock it ran at: clock64 (shader cycles) and
//                   wall_clock64 (a fixed-rate counter) at the start and end
//                   of each workgroup's loop.
// Operands of the MFMA loop are pseudo-random bf16 values in [1, 2) with
// random signs, so the multipliers toggle as they do on real data.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 512;
constexpr int kMfmaThreads = 256;
constexpr int kAcc = 16;

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <bool NT, int U>
__global__ __launch_bounds__(kReadThreads) void k_stream_read(const u32x4* __restrict__ p, int64_t n,
                                                              uint32_t* __restrict__ sink) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kReadThreads;
    int64_t i = static_cast<int64_t>(blockIdx.x) * kReadThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (U - 1) * stride < n; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) v[j] = load16<NT>(p + i + j * stride);
#pragma unroll
        for (int j = 0; j < U; ++j) acc ^= v[j];
    }
    for (; i < n; i += stride) acc ^= load16<NT>(p + i);
    sink[static_cast<int64_t>(blockIdx.x) * kReadThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__device__ __forceinline__ uint32_t mix(uint32_t x) {  // a 32-bit integer hash (xorshift-multiply)
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

__device__ __forceinline__ bf16x8 operand(uint32_t seed) {
    u32x4 w;
    for (int j = 0; j < 4; ++j) {  // two bf16 per word: sign random, exponent of 1.0, mantissa random
        const uint32_t h = mix(seed * 4u + j);
        w[j] = (h & 0x807f807fu) | 0x3f803f80u;
    }
    return __builtin_bit_cast(bf16x8, w);
}

__global__ __launch_bounds__(kMfmaThreads) void k_mfma_loop(int iters, float* __restrict__ sink,
                                                            uint64_t* __restrict__ clocks) {
    const uint32_t gid = blockIdx.x * kMfmaThreads + threadIdx.x;
    bf16x8 a[4], b[4];
    for (int j = 0; j < 4; ++j) {
        a[j] = operand(gid * 8u + j);
        b[j] = operand(gid * 8u + 4u + j);
    }
    f32x4 acc[kAcc];
#pragma unroll
    for (int j = 0; j < kAcc; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    const uint64_t c0 = clock64(), w0 = wall_clock64();
    // Each accumulator is updated in place (inline assembly: the builtin lets
    // the register allocator route half of them through copies, which adds
    // dependent moves between the MFMAs).
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kAcc; ++j)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                         : "+a"(acc[j])
                         : "v"(a[j & 3]), "v"(b[(j >> 2) & 3]));
    }
    // the compiler does not see the MFMA results' latency through the asm:
    // wait it out before the accumulators are read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    const uint64_t c1 = clock64(), w1 = wall_clock64();
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kAcc; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    sink[gid] = s;
    if (threadIdx.x == 0) {
        clocks[4 * blockIdx.x + 0] = c0;
        clocks[4 * blockIdx.x + 1] = c1;
        clocks[4 * blockIdx.x + 2] = w0;
        clocks[4 * blockIdx.x + 3] = w1;
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

// Flops one ys_mfma_loop workgroup executes per iteration.
int64_t ys_mfma_flops_per_block_iter(void) { return int64_t{kMfmaThreads / 64} * kAcc * 16 * 16 * 32 * 2; }

// Read `bytes` (a multiple of 16) of `buf` once with `blocks` workgroups of
// 512 lanes, `inflight` (8 or 16) loads in flight per lane; sink receives
// blocks * 512 words.  Returns a hipError_t.
int ys_stream_read(const void* buf, int64_t bytes, int nontemporal, int inflight, int blocks, uint32_t* sink,
                   void* stream) {
    if (!buf || !sink || bytes <= 0 || bytes % 16 || blocks < 1 || blocks > (1 << 20)) return hipErrorInvalidValue;
    if (!aligned16(buf) || (inflight != 8 && inflight != 16)) return hipErrorInvalidValue;
    const auto* p = static_cast<const u32x4*>(buf);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 g(blocks), b(kReadThreads);
    const int64_t n = bytes / 16;
    if (nontemporal && inflight == 16)
        hipLaunchKernelGGL((k_stream_read<true, 16>), g, b, 0, s, p, n, sink);
    else if (nontemporal)
        hipLaunchKernelGGL((k_stream_read<true, 8>), g, b, 0, s, p, n, sink);
    else if (inflight == 16)
        hipLaunchKernelGGL((k_stream_read<false, 16>), g, b, 0, s, p, n, sink);
    else
        hipLaunchKernelGGL((k_stream_read<false, 8>), g, b, 0, s, p, n, sink);
    return hipGetLastError();
}

// `iters` iterations of the MFMA loop on `blocks` workgroups of 256 lanes;
// sink receives blocks * 256 floats, clocks blocks * 4 counters (clock64
// start, end; wall_clock64 start, end).  Returns a hipError_t.
int ys_mfma_loop(int iters, int blocks, float* sink, uint64_t* clocks, void* stream) {
    if (!sink || !clocks || iters < 1 || blocks < 1 || blocks > (1 << 16)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_mfma_loop, dim3(blocks), dim3(kMfmaThreads), 0, static_cast<hipStream_t>(stream), iters,
                       sink, clocks);
    return hipGetLastError();
}

// Rate of wall_clock64 on the current device, in kHz (0 on error).
int ys_wall_clock_khz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return khz;
}

}  // extern "C"
