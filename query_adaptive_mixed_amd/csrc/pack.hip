// Packing int8 codes into four residual 2-bit slice planes, and the debug
// probe that reads codes back through the product kernels' own assembly.
//
// One stored copy, a base with refinements, any depth read from it without
// repacking ("FoQLens", table "Progress"); one stored copy of residual slices
// read at 2, 4, 6 or 8 bits (FoQLens landing page, "The mechanism").
#include "qam_common.h"

namespace qam {

// One thread per (block, tile, lane, word): reads the 16 codes that word j of
// lane L covers and writes the matching word of all four planes.
__global__ __launch_bounds__(256) void pack_kernel(const int8_t* __restrict__ W, const float* __restrict__ scales,
                                                   int64_t N, int64_t K, uint8_t* __restrict__ out) {
    const int64_t total = N * K / 16;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (tid < N) reinterpret_cast<float*>(out + N * K)[tid] = scales[tid];
    if (tid >= total) return;
    const int j = (int)(tid & 3);
    const int L = (int)((tid >> 2) & 63);
    const int64_t bt = tid >> 8;              // block * n_tiles + tile
    const int64_t n_tiles = K / kTileCols;
    const int64_t b = bt / n_tiles;
    const int64_t t = bt - b * n_tiles;
    const int64_t row = b * kRows + 16 * j + (L & 15);
    const int64_t col0 = t * kTileCols + 16 * (L >> 4);
    const uint4 v = *reinterpret_cast<const uint4*>(W + row * K + col0);
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};   // word u holds columns 4u .. 4u+3
    const int64_t plane_bytes = N * K / 4;
    const int64_t off = b * 16 * K + t * kTileBytes + L * 16 + 4 * j;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int s = 3 - p;
        uint32_t word = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t byte = (wd[u] >> (8 * i)) & 0xFFu;
                const uint32_t digit = (byte >> (2 * s)) & 3u;
                word |= digit << ((8 * i + 2 * s - 2 * u) & 31);
            }
        }
        *reinterpret_cast<uint32_t*>(out + p * plane_bytes + off) = word;
    }
}

template <int NS>
__device__ __forceinline__ void unpack_lane(const uint8_t* __restrict__ planes, int64_t plane_bytes, int64_t off,
                                            uint32_t (&code)[4][4]) {
    uint32_t w[NS][4];
#pragma unroll
    for (int p = 0; p < NS; ++p) {
        const uint4 v = *reinterpret_cast<const uint4*>(planes + p * plane_bytes + off);
        w[p][0] = v.x; w[p][1] = v.y; w[p][2] = v.z; w[p][3] = v.w;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t col[NS];
#pragma unroll
        for (int p = 0; p < NS; ++p) col[p] = w[p][j];
        code[j][0] = assemble<NS, 0>(col);
        code[j][1] = assemble<NS, 1>(col);
        code[j][2] = assemble<NS, 2>(col);
        code[j][3] = assemble<NS, 3>(col);
    }
}

// One thread per (block, tile, lane): the 64 codes that lane covers.
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* __restrict__ planes, int64_t N, int64_t K,
                                                     const uint8_t* __restrict__ level, int8_t* __restrict__ codes) {
    const int64_t n_tiles = K / kTileCols;
    const int64_t total = (N / kRows) * n_tiles * kLanes;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (tid >= total) return;
    const int L = (int)(tid & 63);
    const int64_t bt = tid >> 6;
    const int64_t b = bt / n_tiles;
    const int64_t t = bt - b * n_tiles;
    const int64_t plane_bytes = N * K / 4;
    const int64_t off = b * 16 * K + t * kTileBytes + L * 16;
    uint32_t code[4][4] = {};
    switch (level[b] < 4 ? level[b] : 4) {
        case 1: unpack_lane<1>(planes, plane_bytes, off, code); break;
        case 2: unpack_lane<2>(planes, plane_bytes, off, code); break;
        case 3: unpack_lane<3>(planes, plane_bytes, off, code); break;
        case 4: unpack_lane<4>(planes, plane_bytes, off, code); break;
        default: break;   // ZERO (rung 0): nothing read, codes 0
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t row = b * kRows + 16 * j + (L & 15);
        const int64_t col0 = t * kTileCols + 16 * (L >> 4);
        uint4 v;
        v.x = code[j][0]; v.y = code[j][1]; v.z = code[j][2]; v.w = code[j][3];
        *reinterpret_cast<uint4*>(codes + row * K + col0) = v;
    }
}

static int check_shape(int64_t N, int64_t K, const char* who) {
    if (N <= 0 || K <= 0 || N % kRows || K % kTileCols || K > QAM_MAX_K)
        QAM_FAIL(QAM_ERR_SHAPE, "%s: N=%lld K=%lld must be positive multiples of 64 with K <= %d", who,
                 (long long)N, (long long)K, QAM_MAX_K);
    return QAM_OK;
}

}  // namespace qam

using namespace qam;

extern "C" int qam_pack_slices(const int8_t* W, const float* scales, int64_t N, int64_t K, void* out,
                               size_t out_bytes, qam_packed* desc_out, hipStream_t s) {
    clear_error();
    if (!W || !scales || !out || !desc_out) QAM_FAIL(QAM_ERR_NULL, "pack_slices: null pointer");
    if (int rc = check_shape(N, K, "pack_slices")) return rc;
    if (out_bytes < qam_packed_bytes(N, K))
        QAM_FAIL(QAM_ERR_ARG, "pack_slices: out_bytes %zu < %zu", out_bytes, qam_packed_bytes(N, K));
    if (!aligned(out, 256)) QAM_FAIL(QAM_ERR_ALIGN, "pack_slices: out must be 256-byte aligned");
    if (!aligned(W, 16) || !aligned(scales, 4)) QAM_FAIL(QAM_ERR_ALIGN, "pack_slices: W must be 16-byte aligned");
    const char* o = static_cast<const char*>(out);
    const char* w = reinterpret_cast<const char*>(W);
    if (o < w + N * K && w < o + qam_packed_bytes(N, K)) QAM_FAIL(QAM_ERR_ARG, "pack_slices: out overlaps W");
    const int64_t threads = N * K / 16;
    const int64_t grid = (threads + 255) / 256;
    if (grid > 0x7FFFFFFF) QAM_FAIL(QAM_ERR_SHAPE, "pack_slices: matrix too large");
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)grid), dim3(256), 0, s, W, scales, N, K,
                       static_cast<uint8_t*>(out));
    QAM_HIP_CHECK(hipGetLastError());
    if (int rc = qam_describe_packed(out, N, K, desc_out)) return rc;
    set_variant("pack_slices");
    return QAM_OK;
}

extern "C" int qam_unpack_codes(const qam_packed* packed, const uint8_t* level_map, int8_t* codes_out,
                                hipStream_t s) {
    clear_error();
    if (!packed || !level_map || !codes_out || !packed->planes) QAM_FAIL(QAM_ERR_NULL, "unpack_codes: null pointer");
    if (int rc = check_shape(packed->N, packed->K, "unpack_codes")) return rc;
    if (!aligned(codes_out, 16)) QAM_FAIL(QAM_ERR_ALIGN, "unpack_codes: codes_out must be 16-byte aligned");
    const int64_t threads = packed->n_blocks * (packed->K / kTileCols) * kLanes;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint8_t*>(packed->planes), packed->N, packed->K, level_map, codes_out);
    QAM_HIP_CHECK(hipGetLastError());
    set_variant("unpack_codes");
    return QAM_OK;
}
