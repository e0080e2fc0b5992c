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

// ---------------------------------------------------------------- x in fixed point
//
// The products are exact integer arithmetic on a fixed-point x.  For a chunk
// of columns of one request with largest |x| in [2^(e-1), 2^e):
//   q1 = rint(x 2^(22-e)),   r1 = x - q1 2^(e-22)     (|q1| <= 2^22, r1 exact)
//   q2 = rint(r1 2^(45-e)),  r2 = r1 - q2 2^(e-45)    (|q2| <= 2^22, r2 exact)
// so x = q1 2^(e-22) + q2 2^(e-45) + r2 with |r2| <= 2^(e-46).  Each q is held
// as three signed int8 limbs (balanced base-256 digits): six B-operand columns
// per request, hi limbs 0..2 then lo limbs 0..2.  An element with
// |r2| > 2^-15 |x| (possible only when |x| < 2^(e-31)) is "uncovered": its r2
// times its code is added to the row sum in fp64 afterwards, so every element
// enters the sum with relative error at most 2^-15 and every output meets
// |y - y_exact| <= 2^-15 sum|w||x| + fl32 rounding, for any finite x.
// A chunk whose largest |x| is below 2^-82 is first scaled by 2^100 (exact),
// so that every constant below is a normal float; the digits are unchanged.
constexpr int kLimbCols = 6;       // B-operand columns per request
constexpr int kHiShift = 22;       // q1 = x 2^(22-e)
constexpr int kLoShift = 45;       // q2 = r1 2^(45-e)
constexpr int kCoarseShift = 29;   // coarse lo digit: q2c = r1 2^(29-e), |q2c| <= 64
constexpr int kSmallExp = -81;     // below this exponent the chunk is prescaled
constexpr int kPrescale = 100;     // by 2^100

__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

struct XSplit {
    float pre;                     // 1 or 2^100
    float scale_hi, step_hi;       // 2^(22-e'), 2^(e'-22)
    float scale_lo, step_lo;       // 2^(45-e'), 2^(e'-45)
    float scale_c, step_c;         // 2^(29-e'), 2^(e'-29): the coarse lo digit
};

__device__ __forceinline__ XSplit xsplit_of(int e) {
    XSplit s;
    const bool small = e < kSmallExp;
    const int ep = small ? e + kPrescale : e;
    s.pre = small ? pow2f(kPrescale) : 1.0f;
    s.scale_hi = pow2f(kHiShift - ep);
    s.step_hi = pow2f(ep - kHiShift);
    s.scale_lo = pow2f(kLoShift - ep);
    s.step_lo = pow2f(ep - kLoShift);
    s.scale_c = pow2f(kCoarseShift - ep);
    s.step_c = pow2f(ep - kCoarseShift);
    return s;
}

// fma(v, 2^k, 1.5 * 2^23) rounds v 2^k to the nearest integer q (ties to even)
// for |v 2^k| <= 2^22, and its bits are 0x4B400000 + q; the limb word holds
// q's balanced base-256 digits in bytes 0..2 (byte 3 unused).
__device__ __forceinline__ uint32_t limb_word_of(float t) {
    return (__float_as_uint(t) + (0x808080u - 0x4B400000u)) ^ 0x808080u;
}

// One element: its hi and lo limb words, its residual r2 (in the prescaled
// unit) and whether it is uncovered.
__device__ __forceinline__ void split_elem(float v, const XSplit& s, uint32_t& w_hi, uint32_t& w_lo, float& r2,
                                           bool& unc) {
    constexpr float kMagic = 12582912.0f;   // 1.5 * 2^23
    v = v * s.pre;
    const float t1 = __builtin_fmaf(v, s.scale_hi, kMagic);
    w_hi = limb_word_of(t1);
    const float r1 = __builtin_fmaf(-(t1 - kMagic), s.step_hi, v);
    const float t2 = __builtin_fmaf(r1, s.scale_lo, kMagic);
    w_lo = limb_word_of(t2);
    r2 = __builtin_fmaf(-(t2 - kMagic), s.step_lo, r1);
    unc = fabsf(r2) > fabsf(v) * 0x1p-15f;
}

// The coarse split of one element (the pre-pass route's common case): the
// same hi part, then ONE lo digit q2c = rint(r1 2^(29-e)) (|q2c| <= 64, so a
// single balanced int8 digit), r2c = r1 - q2c 2^(e-29) exact, |r2c| <= 2^(e-30).
// w_lo holds q2c in byte 2 and zeros in bytes 0 and 1, so that the six-column
// arithmetic below reads it as the lo part 65536 q2c 2^(e-45) = q2c 2^(e-29).
// An element with |r2c| > 2^-15 |x| (possible only when |x| < 2^(e-15)) is
// uncovered.
__device__ __forceinline__ void split_coarse(float v, const XSplit& s, uint32_t& w_hi, uint32_t& w_lo, float& r2,
                                             bool& unc) {
    constexpr float kMagic = 12582912.0f;   // 1.5 * 2^23
    v = v * s.pre;
    const float t1 = __builtin_fmaf(v, s.scale_hi, kMagic);
    w_hi = limb_word_of(t1);
    const float r1 = __builtin_fmaf(-(t1 - kMagic), s.step_hi, v);
    const float tc = __builtin_fmaf(r1, s.scale_c, kMagic);
    w_lo = limb_word_of(tc) << 16;
    r2 = __builtin_fmaf(-(tc - kMagic), s.step_c, r1);
    unc = fabsf(r2) > fabsf(v) * 0x1p-15f;
}

// Whether the coarse split leaves one element uncovered (the count decides a
// chunk's columns before any is written).
__device__ __forceinline__ bool coarse_uncovered(float v, const XSplit& s) {
    uint32_t wh, wl;
    float r2;
    bool unc;
    split_coarse(v, s, wh, wl, r2, unc);
    return unc;
}

// The fp64 value of one request's six column sums (hi limbs s[0..2], lo
// limbs s[3..5]) for a chunk of exponent e.
__device__ __forceinline__ double limb_value(int64_t h0, int64_t h1, int64_t h2, int64_t l0, int64_t l1, int64_t l2,
                                             int e) {
    const double hi = (double)(h2 * 65536 + h1 * 256 + h0);
    const double lo = (double)(l2 * 65536 + l1 * 256 + l0);
    return ldexp(hi, e - kHiShift) + ldexp(lo, e - kLoShift);
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

// The int8 code of row `row` (0..63) of block b, column k, read from planes
// first .. ns-1 (the code at depth 2 ns less the code at depth 2 first): one
// 4-byte load per plane from the packed layout.  For the exact corrections of
// uncovered elements (a slow path taken for them alone).
__device__ __forceinline__ int code_at(const uint8_t* planes, int64_t pb, int64_t K, int b, int row, int64_t k,
                                       int first, int ns) {
    const int64_t t = k >> 6;
    const int kc = (int)(k & 63);
    const int lane = (row & 15) + 16 * (kc >> 4);
    const int u = (kc >> 2) & 3, i = kc & 3;
    const uint8_t* base = planes + (int64_t)b * 16 * K + t * 1024 + lane * 16 + 4 * (row >> 4);
    uint32_t acc = 0;
    for (int p = first; p < ns; ++p) {
        const uint32_t w = *(const uint32_t*)(base + p * pb);
        const uint32_t m = 0x03030303u << (2 * (3 - p));                 // slice 3 - p, before rotation
        const uint32_t mk = u == 0 ? m : ((m >> (2 * u)) | (m << (32 - 2 * u)));
        acc |= w & mk;
    }
    if (u != 0) acc = (acc << (2 * u)) | (acc >> (32 - 2 * u));
    return (int)(int8_t)(uint8_t)(acc >> (8 * i));
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
    const int* run_if;         // single launches: when set and *run_if == 0, every workgroup exits at once
};

struct Common {
    const Item* items;         // grouped launches: the descriptor table
    const int* wg_item;        // grouped launches: item index of every workgroup
    uint32_t* status;          // the call's status word (QAM_STATUS_*), or null
    int B;
    int x_bf16;
    int KS;                    // waves per (block, chunk), 1..8
};

// Chunking of one matrix: tiles per chunk, chunks, workgroups per chunk and
// the fp64 partial bytes a split of K needs.
struct Plan {
    int tpc, n_chunks, n_quads;
    size_t partial_bytes;
};

int tpc_align();
size_t lds_bytes_staged();
// Chunk length goal for a launch of `block_tiles` block x tile pairs aiming at
// `target_waves` wavefronts, at most `cap` tiles (cap <= 0: no cap).
int chunk_goal(int64_t block_tiles, int64_t target_waves, int cap);
// The staged-limb route's goal under a group's tuning (null: defaults).
int staged_goal(int64_t block_tiles, const qam_tuning* t);
// align: chunk lengths are rounded up to a multiple of it (<= 0: a whole
// number of prefetch rings).
Plan make_plan(int64_t N, int64_t K, int goal, int align = 0);
Item make_item(const void* x, const qam_packed* packed, const uint8_t* level_map, float* y, const Plan& p);
int check_item(const void* x, int x_dtype, int64_t B, const qam_packed* packed, const uint8_t* level_map, float* y,
               const char* who, int out_mode);
int check_workspace(void* workspace, size_t workspace_bytes, size_t need, const char* who);
// The status word inside a counter region (a workspace, a group's or a
// decoder's device memory).
uint32_t* status_word(void* counter_region);
// Matrix-core route of qam_qmatvec (batches of 2 to 32, per-request maps).
bool mfma_route(int64_t B);
size_t qam_mfma_workspace_bytes(int64_t N, int64_t K, int64_t B);
int qmatvec_mfma(const void* x, int x_dtype, int64_t B, const qam_packed* packed, const uint8_t* level_map,
                 int per_request_maps, float* y, void* workspace, size_t workspace_bytes, hipStream_t s);
// A transform the pre-pass route's pre-pass applies to fp32 x before
// splitting it (the product itself reads only the limbs), so that a chain of
// products needs no separate elementwise launches:
//   kXStrided  row r of x starts at r ld;
//   kXAddNorm  x is a residual h: v = h + add (fp32), written back into res
//              (res may be x itself), then the RMS-normalised
//              x' = fl32(v / sqrt(mean_k v^2 + eps)) (fp64), written to side;
//              the row is taken in one column chunk;
//   kXGated    x is a gate|up product's output, rows interleaved 32 gate / 32
//              up per 64-row block, row stride ld:
//              x'_j = fl32(silu(g_j) u_j) (fp64), written to side.
// add, res and side rows have stride K.  The output y may be add, or x in
// kXGated: the pre-pass has read them before the product writes y.
enum XMode { kXPlain = 0, kXStrided = 1, kXAddNorm = 2, kXGated = 3 };
struct XIn {
    int mode = kXPlain;
    int64_t ld = 0;
    const float* add = nullptr;
    float* res = nullptr;
    float* side = nullptr;
    double eps = 0.0;
};
// qam_qmatvec's pre-pass route with a shared map and an input transform
// (x fp32; B in [2, 32]); workspace: at least qam_mfma_workspace_bytes.
int qmatvec_mfma_in(const float* x, int64_t B, const qam_packed* packed, const uint8_t* level_map, float* y,
                    const XIn& in, void* workspace, size_t workspace_bytes, hipStream_t s);
size_t mfma_group_bytes(const qam_gemv_item* items, int n_items, int64_t B, const qam_tuning* t);
int mfma_group_init(const qam_gemv_item* items, int n_items, int64_t B, int x_dtype, int per_request_maps,
                    const qam_tuning* t, void* dev_mem, size_t dev_bytes, qam_group* out, hipStream_t s);
int mfma_group_run(const qam_group* g, hipStream_t s);
// Enqueues one single-matrix product launch of the staged-limb route (grid =
// n_chunks * n_quads workgroups of c.KS wavefronts).
void launch_single(const Item& it, const Common& c, int64_t grid, hipStream_t s);

}  // namespace qam
