// tk_quant: the quantisation granularities of TileKernels' quant/ module
// ("刚刚！DeepSeek开源高性能GPU算子库TileKernels", item quant/: per-token,
// per-block and per-channel FP8; "剛剛，DeepSeek開始頻繁更新：Tile Kernels、
// DeepEP V2", feature list: FP8 / FP4 conversion) on a bf16 matrix
// (rows, cols), row-major:
//
//   TK_QUANT_FP8_1X128       per-token 1x128 blocks, scale = RN(max(amax,1e-4)/448)
//                            (the codec of tk_expand_quant)
//   TK_QUANT_FP8_1X128_POW2  same blocks, scale = the smallest power of two
//                            with 448*scale >= max(amax, 1e-4)
//   TK_QUANT_FP8_128X128     one scale per 128x128 tile (weights)
//   TK_QUANT_FP8_PER_CHANNEL one scale per column over all rows
//   TK_QUANT_FP4_1X32        E2M1 codes (two per byte, even column in the low
//                            nibble), 1x32 blocks, scale 2^(floor(log2 amax)-2)
//
// Kernels:
//  - 1x128 (and pow2): the matrix as one flat run of values (no block
//    straddles a row); one wave per 2048 values, 8 per lane and piece (16-byte
//    loads, 1 KB contiguous per wave instruction), a 128-value block per 16
//    lanes (amax by a 4-step DPP butterfly), 8 bytes of codes per lane.
//  - 128x128: one 256-thread workgroup per tile; each thread holds an 8x8
//    patch (eight 16-byte row loads), the tile amax is a DPP wave max then an
//    LDS step over the four waves.
//  - per-channel: workgroups of 256 columns x 8 row groups.  Pass 1 takes
//    column maxima over chunks of 128 rows (16 rows per thread, 8 streaming
//    loads in flight, row groups combined in LDS) into the workspace; a small
//    pass takes the maximum over the chunks (exact in any order) per column
//    and forms the scale and its reciprocal; the last pass quantises 64 rows
//    per workgroup with them.
//  - FP4: the matrix as one flat run of values (no block straddles a row);
//    one wave per 2048 values, one 32-value block per lane quad (16-byte
//    loads, the wave reading 1 KB contiguous per instruction; one 32-bit
//    word of codes per lane); E2M1 codes from a compile-time table in LDS
//    indexed by the quotient's clamped bf16 magnitude.
// Codes are written with streaming stores; the E4M3 quotient is the shared
// Markstein-corrected one, exact for power-of-two scales.
#include "e2m1_table.h"
#include "tk_internal.h"

namespace {

constexpr int kPcRowsPerChunk = 128;   // rows per partial-maximum chunk (per-channel)
constexpr int kPcRowsPerBlock = 64;    // rows per quantising block (per-channel)

__device__ __forceinline__ float pow2_scale_e4m3(float amax)
{
    amax = fmaxf(amax, 1e-4f);
    int x;
    const float m = __builtin_frexpf(amax, &x);
    return __builtin_ldexpf(1.0f, m <= 0.875f ? x - 9 : x - 8);
}

// eight bf16 (one 16-byte word) -> fp32
__device__ __forceinline__ void unpack8(tk::u32x4 w, float* v)
{
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = tk::bf16_lo(ws[i]);
        v[2 * i + 1] = tk::bf16_hi(ws[i]);
    }
}

// ------------------------------------------------------------------ 1x128
// The matrix as one flat run of rows * cols values (cols % 128 == 0, so no
// block straddles a row; a block's codes sit at flat and its scale at
// flat / 128).  A wave takes 2048 consecutive values in four 512-value
// pieces; in each piece lane l holds values 8l..8l+7 (one 16-byte load, the
// wave reading 1 KB contiguous), 16 lanes make a 128-value block (DPP max),
// and each lane stores its 8 codes as one 8-byte word.
constexpr int kQPerWave = 2048;

template <bool POW2>
__global__ __launch_bounds__(tk::kBlock) void quant_1x128_kernel(
    const uint16_t* __restrict__ x, int64_t n, uint8_t* __restrict__ q, float* __restrict__ scales)
{
    const int lane = threadIdx.x & (tk::kWave - 1);
    const int64_t base = (static_cast<int64_t>(blockIdx.x) * tk::kWavesPerBlock +
                          tk::uniform(threadIdx.x / tk::kWave)) * kQPerWave;
    if (base >= n) return;
    tk::u32x4 w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t f = base + j * 512 + lane * 8;
        w[j] = f < n ? tk::load_stream(x + f) : tk::u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t f = base + j * 512 + lane * 8;   // n % 128 == 0: 16-lane runs wholly in or out
        float v[8];
        unpack8(w[j], v);
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
        amax = fmaxf(amax, tk::dpp_f32<tk::kQuadXor1>(amax));
        amax = fmaxf(amax, tk::dpp_f32<tk::kQuadXor2>(amax));
        amax = fmaxf(amax, tk::dpp_f32<tk::kHalfMirror>(amax));
        amax = fmaxf(amax, tk::dpp_f32<tk::kMirror>(amax));
        const float scale = POW2 ? pow2_scale_e4m3(amax) : fmaxf(amax, 1e-4f) / 448.0f;
        const float inv = 1.0f / scale;
        uint2 c;
        c.x = tk::pack_fp8x4(tk::fp8_quotient(v[0], scale, inv), tk::fp8_quotient(v[1], scale, inv),
                             tk::fp8_quotient(v[2], scale, inv), tk::fp8_quotient(v[3], scale, inv));
        c.y = tk::pack_fp8x4(tk::fp8_quotient(v[4], scale, inv), tk::fp8_quotient(v[5], scale, inv),
                             tk::fp8_quotient(v[6], scale, inv), tk::fp8_quotient(v[7], scale, inv));
        if (f < n) {
            __builtin_nontemporal_store(c.x, reinterpret_cast<uint32_t*>(q + f));
            __builtin_nontemporal_store(c.y, reinterpret_cast<uint32_t*>(q + f + 4));
            if ((lane & 15) == 0) scales[f / 128] = scale;
        }
    }
}

// ---------------------------------------------------------------- 128x128
__global__ __launch_bounds__(tk::kBlock) void quant_128x128_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int cols, uint8_t* __restrict__ q,
    float* __restrict__ scales)
{
    __shared__ float wave_max[tk::kWavesPerBlock];
    const int tiles_c = cols / 128;
    const int64_t tr = blockIdx.x / tiles_c;
    const int tc = static_cast<int>(blockIdx.x - tr * tiles_c);
    // thread -> 8 rows x 8 columns of the tile
    const int cg = threadIdx.x & 15, rg = threadIdx.x >> 4;
    const int col = tc * 128 + cg * 8;
    const int64_t r0 = tr * 128 + rg * 8;
    float v[8][8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        tk::u32x4 w = tk::u32x4{0u, 0u, 0u, 0u};
        if (r0 + i < rows) w = tk::load_stream(x + static_cast<size_t>(r0 + i) * cols + col);
        unpack8(w, v[i]);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
    }
    amax = tk::max_wave_f32(amax);
    if ((threadIdx.x & (tk::kWave - 1)) == 0) wave_max[threadIdx.x / tk::kWave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
    const float scale = fmaxf(amax, 1e-4f) / 448.0f;
    const float inv = 1.0f / scale;
    if (threadIdx.x == 0) scales[tr * tiles_c + tc] = scale;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (r0 + i >= rows) break;
        uint2 o;
        o.x = tk::pack_fp8x4(tk::fp8_quotient(v[i][0], scale, inv), tk::fp8_quotient(v[i][1], scale, inv),
                             tk::fp8_quotient(v[i][2], scale, inv), tk::fp8_quotient(v[i][3], scale, inv));
        o.y = tk::pack_fp8x4(tk::fp8_quotient(v[i][4], scale, inv), tk::fp8_quotient(v[i][5], scale, inv),
                             tk::fp8_quotient(v[i][6], scale, inv), tk::fp8_quotient(v[i][7], scale, inv));
        *reinterpret_cast<uint2*>(q + static_cast<size_t>(r0 + i) * cols + col) = o;
    }
}

// ------------------------------------------------------------ per-channel
// A workgroup covers 256 columns (32 groups of 8) and kPcRowsPerChunk rows
// (8 row groups); maxima over its rows are combined in LDS.
constexpr int kPcCols = 256;
constexpr int kPcRowGroups = tk::kBlock / (kPcCols / 8);   // 8

// partial[chunk][c] = max |x[r, c]| over the chunk's rows
__global__ __launch_bounds__(tk::kBlock) void quant_pc_partial_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int cols, float* __restrict__ partial)
{
    __shared__ float red[kPcRowGroups][kPcCols];
    const int cgi = threadIdx.x & 31, rg = threadIdx.x >> 5;
    const int col = blockIdx.x * kPcCols + cgi * 8;
    const bool active = col < cols;
    const int64_t chunk = blockIdx.y;
    const int rows_per_group = kPcRowsPerChunk / kPcRowGroups;   // 16
    const int64_t r0 = chunk * kPcRowsPerChunk + rg * rows_per_group;
    float m[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = 0.f;
#pragma unroll
    for (int i0 = 0; i0 < rows_per_group; i0 += 8) {
        tk::u32x4 w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            w[i] = tk::u32x4{0u, 0u, 0u, 0u};
            if (active && r0 + i0 + i < rows) w[i] = tk::load_stream(x + static_cast<size_t>(r0 + i0 + i) * cols + col);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float v[8];
            unpack8(w[i], v);
#pragma unroll
            for (int j = 0; j < 8; ++j) m[j] = fmaxf(m[j], fabsf(v[j]));
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) red[rg][cgi * 8 + j] = m[j];
    __syncthreads();
    if (rg == 0 && active) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
#pragma unroll
            for (int g = 1; g < kPcRowGroups; ++g) m[j] = fmaxf(m[j], red[g][cgi * 8 + j]);
        }
        float* p = partial + static_cast<size_t>(chunk) * cols + col;
        *reinterpret_cast<float4*>(p) = make_float4(m[0], m[1], m[2], m[3]);
        *reinterpret_cast<float4*>(p + 4) = make_float4(m[4], m[5], m[6], m[7]);
    }
}

// Per column: the maximum over all chunks, the scale (written to scales) and
// its reciprocal (workspace, after the chunk maxima).  A workgroup takes 32
// columns; its 8 thread groups split the chunks (group g: chunks g, g+8, ...,
// eight loads in flight per batch, each a coalesced 128-byte row piece) and
// combine in LDS.
constexpr int kPsCols = 32;
constexpr int kPsGroups = tk::kBlock / kPsCols;   // 8

__global__ __launch_bounds__(tk::kBlock) void quant_pc_scale_kernel(
    const float* __restrict__ partial, int cols, int n_chunks, float* __restrict__ scales,
    float* __restrict__ inv_out)
{
    __shared__ float red[kPsGroups][kPsCols];
    const int cl = threadIdx.x % kPsCols, g = threadIdx.x / kPsCols;
    const int c = blockIdx.x * kPsCols + cl;
    float m = 0.f;
    if (c < cols) {
        for (int b = g; b < n_chunks; b += kPsGroups * 8) {
            float t[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int ch = b + u * kPsGroups;
                t[u] = ch < n_chunks ? partial[static_cast<size_t>(ch) * cols + c] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) m = fmaxf(m, t[u]);
        }
    }
    red[g][cl] = m;
    __syncthreads();
    if (g != 0 || c >= cols) return;
#pragma unroll
    for (int k = 1; k < kPsGroups; ++k) m = fmaxf(m, red[k][cl]);
    const float s = fmaxf(m, 1e-4f) / 448.0f;
    scales[c] = s;
    inv_out[c] = 1.0f / s;
}

// the codes of kPcRowsPerBlock rows from the per-column scales and reciprocals
__global__ __launch_bounds__(tk::kBlock) void quant_pc_apply_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int cols, const float* __restrict__ scales,
    const float* __restrict__ inv_in, uint8_t* __restrict__ q)
{
    const int cgi = threadIdx.x & 31, rg = threadIdx.x >> 5;
    const int col = blockIdx.x * kPcCols + cgi * 8;
    if (col >= cols) return;
    const int rows_per_group = kPcRowsPerBlock / kPcRowGroups;   // 8
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kPcRowsPerBlock + rg * rows_per_group;
    tk::u32x4 w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        w[i] = tk::u32x4{0u, 0u, 0u, 0u};
        if (i < rows_per_group && r0 + i < rows) w[i] = tk::load_stream(x + static_cast<size_t>(r0 + i) * cols + col);
    }
    const float4 sa = *reinterpret_cast<const float4*>(scales + col);
    const float4 sb = *reinterpret_cast<const float4*>(scales + col + 4);
    const float4 ia = *reinterpret_cast<const float4*>(inv_in + col);
    const float4 ib = *reinterpret_cast<const float4*>(inv_in + col + 4);
    const float s[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
    const float inv[8] = {ia.x, ia.y, ia.z, ia.w, ib.x, ib.y, ib.z, ib.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (i >= rows_per_group || r0 + i >= rows) break;
        float v[8];
        unpack8(w[i], v);
        uint2 o;
        o.x = tk::pack_fp8x4(tk::fp8_quotient(v[0], s[0], inv[0]), tk::fp8_quotient(v[1], s[1], inv[1]),
                             tk::fp8_quotient(v[2], s[2], inv[2]), tk::fp8_quotient(v[3], s[3], inv[3]));
        o.y = tk::pack_fp8x4(tk::fp8_quotient(v[4], s[4], inv[4]), tk::fp8_quotient(v[5], s[5], inv[5]),
                             tk::fp8_quotient(v[6], s[6], inv[6]), tk::fp8_quotient(v[7], s[7], inv[7]));
        *reinterpret_cast<uint2*>(q + static_cast<size_t>(r0 + i) * cols + col) = o;
    }
}

// ------------------------------------------------------------------- FP4
// E2M1 codes by table (e2m1_table.h): a quotient x * 2^j of a bf16 input by
// the block's exact power-of-two reciprocal keeps at most 8 significant bits,
// so its code is a 640-entry byte table indexed by its clamped bf16 magnitude
// -- four instructions and one LDS byte read where rounding by arithmetic took
// about a dozen.  The table is built at compile time.
__device__ const tk::E2m1Table kE2m1Dev = tk::make_e2m1_table();
static_assert(tk::kE2m1N % 4 == 0, "the table is copied in 4-byte words");

// The matrix is taken as one flat run of rows * cols values: cols % 32 == 0,
// so no block straddles a row, and a block's codes and scale sit at flat / 2
// and flat / 32 of the row-major outputs.  A wave takes 2048 consecutive
// values in four 512-value pieces; in each piece lane l holds values
// 8l..8l+7 (one 16-byte load, the wave reading 1 KB contiguous), a lane quad
// is one 32-value block (DPP max), and each lane stores its 8 codes as one
// 32-bit word.
constexpr int kFp4PerWave = 2048;

__global__ __launch_bounds__(tk::kBlock) void quant_fp4_kernel(
    const uint16_t* __restrict__ x, int64_t n, uint8_t* __restrict__ q, float* __restrict__ scales)
{
    __shared__ __align__(4) uint8_t table[tk::kE2m1N];
    const int lane = threadIdx.x & (tk::kWave - 1);
    const int64_t base = (static_cast<int64_t>(blockIdx.x) * tk::kWavesPerBlock +
                          tk::uniform(threadIdx.x / tk::kWave)) * kFp4PerWave;
    tk::u32x4 w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t f = base + j * 512 + lane * 8;
        w[j] = f < n ? tk::load_stream(x + f) : tk::u32x4{0u, 0u, 0u, 0u};
    }
    for (int i = threadIdx.x; i < static_cast<int>(tk::kE2m1N / 4); i += tk::kBlock)
        reinterpret_cast<uint32_t*>(table)[i] = reinterpret_cast<const uint32_t*>(kE2m1Dev.code)[i];
    __syncthreads();
    if (base >= n) return;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t f = base + j * 512 + lane * 8;   // n % 32 == 0: quads are wholly in or out
        float v[8];
        unpack8(w[j], v);
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
        amax = fmaxf(amax, tk::dpp_f32<tk::kQuadXor1>(amax));
        amax = fmaxf(amax, tk::dpp_f32<tk::kQuadXor2>(amax));
        amax = fmaxf(amax, 1e-4f);
        int e;
        __builtin_frexpf(amax, &e);
        const float scale = __builtin_ldexpf(1.0f, e - 3);     // 2^(floor(log2 amax) - 2)
        const float inv = __builtin_ldexpf(1.0f, 3 - e);       // exact
        uint32_t p = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) p |= tk::e2m1_lookup(__float_as_uint(v[i] * inv), table) << (4 * i);
        if (f < n) {
            __builtin_nontemporal_store(p, reinterpret_cast<uint32_t*>(q + f / 2));
            if ((lane & 3) == 0) scales[f / 32] = scale;
        }
    }
}

unsigned blocks_for(int64_t waves) { return static_cast<unsigned>((waves + tk::kWavesPerBlock - 1) / tk::kWavesPerBlock); }

}  // namespace

TK_EXPORT size_t tk_quant_workspace_bytes(int64_t rows, int32_t cols, int32_t mode)
{
    if (mode != TK_QUANT_FP8_PER_CHANNEL || rows <= 0 || cols <= 0) return 0;
    const int64_t n_chunks = (rows + kPcRowsPerChunk - 1) / kPcRowsPerChunk;
    // the chunk maxima, then one row of reciprocal scales
    return static_cast<size_t>(n_chunks + 1) * static_cast<size_t>(cols) * sizeof(float);
}

TK_EXPORT tk_status tk_quant(const void* x_bf16, int64_t rows, int32_t cols, int32_t mode,
                             void* out, float* scales, void* workspace, size_t workspace_bytes,
                             hipStream_t stream)
{
    using tk::fail;
    if (rows < 0) return fail(TK_ERR_ARG, "tk_quant: rows < 0");
    int align = 0;
    switch (mode) {
    case TK_QUANT_FP8_1X128: case TK_QUANT_FP8_1X128_POW2: case TK_QUANT_FP8_128X128: align = 128; break;
    case TK_QUANT_FP8_PER_CHANNEL: align = 8; break;
    case TK_QUANT_FP4_1X32: align = 32; break;
    default: return fail(TK_ERR_ARG, "tk_quant: unknown mode %d", mode);
    }
    if (cols <= 0 || cols % align != 0)
        return fail(TK_ERR_ARG, "tk_quant: cols=%d must be a positive multiple of %d for mode %d",
                    cols, align, mode);
    if (rows == 0) return tk::ok();
    if (x_bf16 == nullptr || out == nullptr || scales == nullptr)
        return fail(TK_ERR_ARG, "tk_quant: NULL tensor pointer");
    if (!tk::aligned16(x_bf16) || !tk::aligned16(out) || !tk::aligned16(scales))
        return fail(TK_ERR_ARG, "tk_quant: x, out and scales must be 16-byte aligned");
    const auto* x = static_cast<const uint16_t*>(x_bf16);
    auto* q = static_cast<uint8_t*>(out);
    const dim3 block(tk::kBlock);
    hipError_t e = hipSuccess;
    if (mode == TK_QUANT_FP8_1X128 || mode == TK_QUANT_FP8_1X128_POW2) {
        const int64_t n = rows * cols;
        const int64_t waves = (n + kQPerWave - 1) / kQPerWave;
        if ((waves + tk::kWavesPerBlock - 1) / tk::kWavesPerBlock > INT32_MAX)
            return fail(TK_ERR_UNSUPPORTED, "tk_quant: too many values");
        const dim3 grid(blocks_for(waves));
        e = mode == TK_QUANT_FP8_1X128_POW2
            ? tk::launch(quant_1x128_kernel<true>, grid, block, 0, stream, x, n, q, scales)
            : tk::launch(quant_1x128_kernel<false>, grid, block, 0, stream, x, n, q, scales);
    } else if (mode == TK_QUANT_FP8_128X128) {
        const int64_t tiles = (rows + 127) / 128 * (cols / 128);
        if (tiles > INT32_MAX) return fail(TK_ERR_UNSUPPORTED, "tk_quant: too many tiles");
        e = tk::launch(quant_128x128_kernel, dim3(static_cast<unsigned>(tiles)), block, 0, stream,
                       x, rows, cols, q, scales);
    } else if (mode == TK_QUANT_FP8_PER_CHANNEL) {
        const size_t need = tk_quant_workspace_bytes(rows, cols, mode);
        if (workspace == nullptr || workspace_bytes < need || !tk::aligned16(workspace))
            return fail(TK_ERR_ARG, "tk_quant: per-channel needs a 16-byte aligned workspace of "
                        "%zu bytes (got %zu)", need, workspace_bytes);
        const int64_t n_chunks = (rows + kPcRowsPerChunk - 1) / kPcRowsPerChunk;
        const int64_t n_blocks = (rows + kPcRowsPerBlock - 1) / kPcRowsPerBlock;
        if (n_chunks > 65535 || n_blocks > 65535)
            return fail(TK_ERR_UNSUPPORTED, "tk_quant: too many rows for per-channel");
        const unsigned gx = static_cast<unsigned>((cols + kPcCols - 1) / kPcCols);
        auto* partial = static_cast<float*>(workspace);
        float* inv = partial + static_cast<size_t>(n_chunks) * cols;
        e = tk::launch(quant_pc_partial_kernel, dim3(gx, static_cast<unsigned>(n_chunks)), block, 0,
                       stream, x, rows, cols, partial);
        if (e != hipSuccess) return tk::launched(e, "tk_quant (per-channel maxima)");
        e = tk::launch(quant_pc_scale_kernel, dim3(static_cast<unsigned>((cols + kPsCols - 1) / kPsCols)),
                       block, 0, stream, partial, cols, static_cast<int>(n_chunks), scales, inv);
        if (e != hipSuccess) return tk::launched(e, "tk_quant (per-channel scales)");
        e = tk::launch(quant_pc_apply_kernel, dim3(gx, static_cast<unsigned>(n_blocks)), block, 0,
                       stream, x, rows, cols, scales, inv, q);
    } else {
        const int64_t n = rows * cols;
        const int64_t waves = (n + kFp4PerWave - 1) / kFp4PerWave;
        if ((waves + tk::kWavesPerBlock - 1) / tk::kWavesPerBlock > INT32_MAX)
            return fail(TK_ERR_UNSUPPORTED, "tk_quant: too many values for FP4");
        e = tk::launch(quant_fp4_kernel, dim3(blocks_for(waves)), block, 0, stream, x, n, q, scales);
    }
    return tk::launched(e, "tk_quant");
}
