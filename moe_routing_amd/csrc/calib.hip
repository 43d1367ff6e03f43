// Calibration kernel for bench.py, built into its own library (libtk_calib.so),
// not part of the routing C ABI: a streaming device copy, the repository's
// reference for what a plain HBM copy reaches on this GPU.  16-byte
// nontemporal loads and stores; each wave moves one contiguous KiB (one load
// and one store per lane) and ends, so the waves in flight cover a compact,
// advancing window of the buffers.  Measured over 1 GiB against 2, 4, 8 and
// 16 loads per lane and against persistent grid-striding waves, this form was
// the fastest: about 6.55 TB/s of read + write against 5.1-6.2.
#include "tk_internal.h"

namespace {

constexpr int kCopyLoads = 1;

__global__ __launch_bounds__(tk::kBlock) void stream_copy_kernel(const uint16_t* __restrict__ src,
                                                                 uint16_t* __restrict__ dst, int64_t n16)
{
    const int lane = threadIdx.x & (tk::kWave - 1);
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * tk::kWavesPerBlock +
                         tk::uniform(threadIdx.x / tk::kWave);
    const int64_t base = wave * kCopyLoads * tk::kWave;
    tk::u32x4 d[kCopyLoads];
#pragma unroll
    for (int i = 0; i < kCopyLoads; ++i) {
        const int64_t p = base + i * tk::kWave + lane;
        d[i] = p < n16 ? tk::load_stream(src + p * 8) : tk::u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kCopyLoads; ++i) {
        const int64_t p = base + i * tk::kWave + lane;
        if (p < n16) tk::store_stream(dst + p * 8, d[i]);
    }
}

}  // namespace

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned) on `stream`.
// Returns 0, -1 for bad arguments, -3 if the launch fails.
TK_EXPORT int tk_calib_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream)
{
    if (bytes == 0) return 0;
    if (src == nullptr || dst == nullptr || bytes % 16 != 0 || !tk::aligned16(src) || !tk::aligned16(dst))
        return -1;
    const int64_t n16 = static_cast<int64_t>(bytes / 16);
    const int64_t waves = (n16 + kCopyLoads * tk::kWave - 1) / (kCopyLoads * tk::kWave);
    const int64_t blocks = (waves + tk::kWavesPerBlock - 1) / tk::kWavesPerBlock;
    if (blocks > INT32_MAX) return -1;
    const hipError_t e = tk::launch(stream_copy_kernel, dim3(static_cast<unsigned>(blocks)),
                                    dim3(tk::kBlock), 0, stream, static_cast<const uint16_t*>(src),
                                    static_cast<uint16_t*>(dst), n16);
    return e == hipSuccess ? 0 : -3;
}
