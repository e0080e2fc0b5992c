// Internal interface of the qmatvec kernels, shared by the translation units
// that launch them (single and grouped products, the decode driver).
#pragma once

#include "qam_common.h"

namespace qam {

// One matrix of a launch.
struct Item {
    const uint8_t* planes;
    const float* scales;
    const void* x;             // [B][K]
    float* y;                  // [B][N]
    const uint8_t* level;      // [n_blocks]
    double* partials;          // [n_chunks][B][N] (split K only)
    uint32_t* counters;        // [n_blocks]       (split K only)
    int64_t plane_bytes;       // N*K/4
    int64_t N, K;
    int n_blocks;
    int n_tiles;               // K / 64
    int tpc;                   // tiles per chunk
    int n_chunks;
    int n_quads;               // ceil(n_blocks / 4)
    int wg_begin;              // first workgroup of this item in a grouped launch
    int rms;                   // 1: y uses x / sqrt(mean(x^2) + eps)
    int out_mode;              // QAM_OUT_STORE / _ADD / _GLU
    double eps;
};

struct Common {
    const Item* items;         // grouped launches: the descriptor table
    const int* wg_item;        // grouped launches: item index of every workgroup
    int B;
    int x_bf16;
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
// Enqueues one single-matrix product launch (grid = n_chunks * n_quads).
void launch_single(int64_t B, const Item& it, const Common& c, int64_t grid, hipStream_t s);

}  // namespace qam
