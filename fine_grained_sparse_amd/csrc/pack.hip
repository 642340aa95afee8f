// Weight repacking into the fragment-block layout (MOE_LAYOUT_FRAG16 in
// include/moe.h): a [rows, cols] bf16 matrix becomes (rows/16) x (cols/32)
// blocks of 1 KiB, each holding the B operand of one 16x16x32 MFMA in lane
// order (lane l: row l % 16, columns 8 (l / 16) .. + 7); an FP8 matrix
// becomes (rows/16) x (cols/64) blocks of 1 KiB, each holding the codes of
// two such operands (both 32-column halves) in lane order.  A pure
// permutation, run once when the weights are loaded.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

// One thread per 16-byte output piece (lane l of block b of matrix m).
__global__ __launch_bounds__(256) void k_pack_frag16(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                     int64_t pieces, int rows, int cols) {
    const int64_t per = static_cast<int64_t>(rows) * cols / 8;  // pieces per matrix
    const int kb = cols / 32;                                   // blocks along a row block
    for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < pieces; q += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t m = q / per, rem = q % per;
        const int64_t blk = rem / 64;
        const int l = static_cast<int>(rem % 64);
        const int64_t i = blk / kb, j = blk % kb;
        const int64_t row = i * 16 + (l & 15), col = j * 32 + (l >> 4) * 8;
        const uint4 v = *reinterpret_cast<const uint4*>(src + m * per * 8 + row * cols + col);
        *reinterpret_cast<uint4*>(dst + q * 8) = v;
    }
}

// FP8: one thread per 16-byte output piece, built from two 8-byte pieces
// of a source row (columns 8 g .. 8 g + 7 and 32 + 8 g .. 32 + 8 g + 7 of
// the block's 64, g = l / 16).
__global__ __launch_bounds__(256) void k_pack_frag16_fp8(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                         int64_t pieces, int rows, int cols) {
    const int64_t per = static_cast<int64_t>(rows) * cols / 16;  // pieces per matrix
    const int kb = cols / 64;                                    // blocks along a row block
    for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < pieces; q += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t m = q / per, rem = q % per;
        const int64_t blk = rem / 64;
        const int l = static_cast<int>(rem % 64);
        const int64_t i = blk / kb, j = blk % kb;
        const int64_t row = i * 16 + (l & 15), col = j * 64 + (l >> 4) * 8;
        const uint8_t* s = src + m * per * 16 + row * cols + col;
        const uint2 lo = *reinterpret_cast<const uint2*>(s);
        const uint2 hi = *reinterpret_cast<const uint2*>(s + 32);
        *reinterpret_cast<uint4*>(dst + q * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
}

}  // namespace

hipError_t launch_pack_frag16_fp8(const uint8_t* src, uint8_t* dst, int64_t count, int rows, int cols,
                                  hipStream_t stream) {
    if (count <= 0 || rows <= 0 || cols <= 0) return hipSuccess;
    if (rows % 16 || cols % 64) return hipErrorInvalidValue;
    const int64_t pieces = count * rows * cols / 16;
    const int64_t blocks = (pieces + 255) / 256;
    hipLaunchKernelGGL(k_pack_frag16_fp8, dim3(static_cast<unsigned>(blocks < 16384 ? blocks : 16384)), dim3(256),
                       0, stream, src, dst, pieces, rows, cols);
    return hipGetLastError();
}

hipError_t launch_pack_frag16(const uint16_t* src, uint16_t* dst, int64_t count, int rows, int cols,
                              hipStream_t stream) {
    if (count <= 0 || rows <= 0 || cols <= 0) return hipSuccess;
    if (rows % 16 || cols % 32) return hipErrorInvalidValue;
    const int64_t pieces = count * rows * cols / 8;
    const int64_t blocks = (pieces + 255) / 256;
    hipLaunchKernelGGL(k_pack_frag16, dim3(static_cast<unsigned>(blocks < 16384 ? blocks : 16384)), dim3(256), 0,
                       stream, src, dst, pieces, rows, cols);
    return hipGetLastError();
}

}  // namespace moe
