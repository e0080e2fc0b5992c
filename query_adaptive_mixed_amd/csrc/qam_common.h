// Internal helpers shared by the libqam translation units.
//
// Layout of one packed matrix (see include/qam.h for the full statement):
// plane p = 0..3 holds digit s = 3 - p of every int8 code; plane bytes are
// N*K/4; block b owns 16*K bytes of each plane; tile t (64 columns) owns 1 KiB;
// lane L owns 16 bytes = words j = 0..3 covering row 16j + (L & 15) and
// columns 16(L >> 4) + 4u + i, with digit (u, i) of slice s at bit
// (8i + 2s - 2u) mod 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "qam.h"

namespace qam {

constexpr int kRows = QAM_ROWS_PER_BLOCK;   // rows per block
constexpr int kTileCols = 64;               // columns per tile
constexpr int kTileBytes = 1024;            // bytes per tile per plane
constexpr int kLanes = 64;                  // wavefront width on gfx950

// ---------------------------------------------------------------- host errors
void set_error(const char* fmt, ...);
void clear_error();
void set_variant(const std::string& v);

#define QAM_FAIL(code, ...)            \
    do {                               \
        ::qam::set_error(__VA_ARGS__); \
        return (code);                 \
    } while (0)

#define QAM_HIP_CHECK(expr)                                                              \
    do {                                                                                 \
        hipError_t _e = (expr);                                                          \
        if (_e != hipSuccess)                                                            \
            QAM_FAIL(QAM_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(_e));        \
    } while (0)

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---------------------------------------------------------------- device side
// Mask of the bits of slice s that belong to group u, before rotation:
// bits (8i + 2s - 2u) mod 32 for i = 0..3.
__host__ __device__ constexpr uint32_t rotr_const(uint32_t x, int r) {
    return r == 0 ? x : ((x >> r) | (x << (32 - r)));
}
__host__ __device__ constexpr uint32_t slice_mask(int s, int u) {
    return rotr_const(0x03030303u << (2 * s), 2 * u);
}

__device__ __forceinline__ uint32_t rotl32(uint32_t x, int r) {
    // r in 1..31; v_alignbit_b32 with both halves equal is a rotate
    return __builtin_amdgcn_alignbit(x, x, 32 - r);
}

// Four int8 codes (columns 4u .. 4u+3 of one row, byte i = column i) read at
// NS slices, from the NS plane words w[0..NS-1] (plane 0 first).  Bits of the
// slices not read stay zero, so the byte is the code truncated to 2*NS bits.
template <int NS, int U>
__device__ __forceinline__ uint32_t assemble(const uint32_t* w) {
    uint32_t acc = w[0] & slice_mask(3, U);
#pragma unroll
    for (int p = 1; p < NS; ++p) acc |= w[p] & slice_mask(3 - p, U);
    if constexpr (U == 0) return acc;
    else return rotl32(acc, 2 * U);
}

}  // namespace qam
