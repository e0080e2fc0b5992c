// Internal interface of the qmatvec kernels, shared by the translation units
// that launch them (single and grouped products, the decode driver).
#pragma once

#include "qam_common.h"

namespace qam {

// ---------------------------------------------------------------- device helpers

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 global_u32x4;

// Weight loads must be global (not flat) memory operations: a flat load also
// counts against the LDS wait counter, so every wait for the limb words in LDS
// would drain the whole prefetch ring with it.
__device__ __forceinline__ u32x4 load_plane(const uint8_t* p) {
    return __builtin_nontemporal_load((global_u32x4*)(p));
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x2 global_u32x2;
typedef __attribute__((address_space(4))) const uint32_t const_u32;

// Raw bits of four x values: fp32 (16 bytes) or bf16 (8 bytes, in .x/.y).
// Converting later, when the values are staged, keeps the wait off this load.
template <bool XBF16>
__device__ __forceinline__ u32x4 load_x4_raw(const void* x, int64_t idx) {
    if constexpr (XBF16) {
        const u32x2 h = *(global_u32x2*)(static_cast<const uint16_t*>(x) + idx);
        return u32x4{h.x, h.y, 0u, 0u};
    } else {
        return *(global_u32x4*)(static_cast<const float*>(x) + idx);
    }
}

template <bool XBF16>
__device__ __forceinline__ float4 x4_value(u32x4 raw) {
    if constexpr (XBF16)
        return make_float4(__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xFFFF0000u),
                           __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xFFFF0000u));
    return make_float4(__uint_as_float(raw.x), __uint_as_float(raw.y), __uint_as_float(raw.z), __uint_as_float(raw.w));
}

// The level byte of block b through the scalar cache: the aligned dword that
// holds it (same page as the byte, so never a fault), waited on with the
// scalar counter rather than the vector one.
__device__ __forceinline__ int level_of(const uint8_t* level, int b) {
    const uintptr_t addr = reinterpret_cast<uintptr_t>(level + b);
    const uint32_t word = *(const_u32*)(addr & ~(uintptr_t)3);
    return (int)((word >> (8 * (addr & 3))) & 0xFFu);
}

// Activations are held as three signed int8 limbs of a 24-bit fixed point
// per sub-chunk: v = rint(x * 2^(kFrac - e)), |v| <= 2^22.
constexpr int kLimbs = 3;
constexpr int kFrac = 22;

// Balanced base-256 digits of the fixed-point value of one element, as three
// signed bytes (byte l = digit l; the top byte is unused).
__device__ __forceinline__ uint32_t limbs_of(float v, int sh) {
    const int q = (int)rintf(ldexpf(v, sh));            // |q| <= 2^22
    return ((uint32_t)q + 0x808080u) ^ 0x808080u;
}

// The same digits when 2^sh is a normal float (sh <= 126, the usual case):
// fma(v, 2^sh, 1.5 * 2^23) rounds v * 2^sh to the nearest integer q (ties to
// even, as rintf) because the sum's ulp is 1 for |q| <= 2^22, and the float's
// bits are 0x4B400000 + q.
__device__ __forceinline__ uint32_t limbs_fast(float v, float scale) {
    const uint32_t bits = __float_as_uint(__builtin_fmaf(v, scale, 12582912.0f));
    return (bits + (0x808080u - 0x4B400000u)) ^ 0x808080u;
}

// Limb words of four consecutive elements (digit words w0..w3): word l holds
// digit l of the four elements, element i in byte i.
__device__ __forceinline__ int4 limb_words(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
    // byte selectors of v_perm_b32: 0-3 pick the second operand's bytes, 4-7 the first's
    const uint32_t lo = __builtin_amdgcn_perm(w1, w0, 0x05010400u);   // w0.0 w1.0 w0.1 w1.1
    const uint32_t hi = __builtin_amdgcn_perm(w3, w2, 0x05010400u);   // w2.0 w3.0 w2.1 w3.1
    const uint32_t lo2 = __builtin_amdgcn_perm(w1, w0, 0x00000602u);  // w0.2 w1.2
    const uint32_t hi2 = __builtin_amdgcn_perm(w3, w2, 0x00000602u);  // w2.2 w3.2
    int4 out;
    out.x = (int)__builtin_amdgcn_perm(hi, lo, 0x05040100u);
    out.y = (int)__builtin_amdgcn_perm(hi, lo, 0x07060302u);
    out.z = (int)__builtin_amdgcn_perm(hi2, lo2, 0x05040100u);
    out.w = 0;
    return out;
}

// ---------------------------------------------------------------- launch descriptors

// One matrix of a launch.
struct Item {
    const uint8_t* planes;
    const float* scales;
    const void* x;             // [B][K]
    float* y;                  // [B][N]
    const uint8_t* level;      // [n_blocks] (written by grouped launches that build the map)
    const double* coords;      // [n_blocks][2] block coordinates (grouped launches that build the map)
    double* partials;          // [n_chunks][B][N] (split K only)
    uint32_t* counters;        // [n_blocks]       (split K only)
    int64_t plane_bytes;       // N*K/4
    int64_t N, K;
    int n_blocks;
    int n_tiles;               // K / 64
    int tpc;                   // tiles per chunk
    int n_chunks;
    int n_quads;               // workgroups per chunk (one per block)
    int wg_begin;              // first workgroup of this item in a grouped launch
    int fixed_level;           // >= 0: every block at this rung, `level` not read (uniform maps)
    int rms;                   // 1: y uses x / sqrt(mean(x^2) + eps)
    int out_mode;              // QAM_OUT_STORE / _ADD / _GLU
    double eps;
};

struct Common {
    const Item* items;         // grouped launches: the descriptor table
    const int* wg_item;        // grouped launches: item index of every workgroup
    int B;
    int x_bf16;
    int KS;                    // waves per (block, chunk), 1..8 (batch 1, single launches)
};

// Chunking of one matrix: tiles per chunk, chunks, workgroups per chunk and
// the fp64 partial bytes a split of K needs.
struct Plan {
    int tpc, n_chunks, n_quads;
    size_t partial_bytes;
};

int tpc_align_for(int64_t B);
int stage_tiles_for(int64_t B);
size_t lds_bytes_for(int64_t B);
// Chunk length goal for a launch of `block_tiles` block x tile pairs aiming at
// `target_waves` wavefronts (<= 0: the library default).
int chunk_goal(int64_t block_tiles, int64_t target_waves);
// align: chunk lengths are rounded up to a multiple of it (<= 0: a whole
// number of prefetch rings for batch B).
Plan make_plan(int64_t N, int64_t K, int64_t B, int goal, int align = 0);
Item make_item(const void* x, const qam_packed* packed, const uint8_t* level_map, float* y, const Plan& p);
int check_item(const void* x, int x_dtype, int64_t B, const qam_packed* packed, const uint8_t* level_map, float* y,
               const char* who, int out_mode);
// Matrix-core route of qam_qmatvec (batches up to 32, per-request maps).
size_t qam_mfma_workspace_bytes(int64_t N, int64_t K, int64_t B);
int qmatvec_mfma(const void* x, int x_dtype, int64_t B, const qam_packed* packed, const uint8_t* level_map,
                 int per_request_maps, float* y, void* workspace, size_t workspace_bytes, hipStream_t s);
size_t mfma_group_bytes(const qam_gemv_item* items, int n_items, int64_t B);
int mfma_group_init(const qam_gemv_item* items, int n_items, int64_t B, int x_dtype, int per_request_maps,
                    void* dev_mem, size_t dev_bytes, qam_group* out, hipStream_t s);
int mfma_group_run(const qam_group* g, hipStream_t s);
bool mfma_route(int64_t B, int per_request_maps);
// Enqueues one single-matrix product launch (grid = n_chunks * n_quads
// workgroups of c.KS wavefronts; c.KS > 1 only for B == 1).
void launch_single(int64_t B, const Item& it, const Common& c, int64_t grid, hipStream_t s);

}  // namespace qam
