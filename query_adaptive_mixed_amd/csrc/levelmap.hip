// Level maps from the lens rules of the FoQLens landing page
// (vovanda.github.io/FoQLens), section "The mechanism", which repeat the rule
// list of "FoQZones, the mechanism" on foqlens.sawking.tech with the per-lens
// radius R_i = r_i f / (1 - f).  The rules and the readings taken where the
// pages are open are stated in lens_rules.h, with the device code this file
// and the grouped product share.  Here: the host checks, rules 1-3 on the
// host, and a kernel that runs rules 4-6 with a group of lanes per block (one
// lane per lens).
//
// The file is compiled with -ffp-contract=off: every product and sum is a
// separate correctly rounded IEEE operation, as is sqrt (an FMA-corrected
// Newton sequence) and division, so the map matches the same rules evaluated
// in IEEE fp64 on a CPU bit for bit.
#include <math.h>

#include <algorithm>
#include <vector>

#include "lens_rules.h"

namespace qam {

constexpr int kMapsPerLaunch = 8;

// The bits of every rung of a ladder, by value for the byte-sum kernel.
struct LadderBits {
    uint32_t v[QAM_MAX_RUNGS];
};

// Up to kMapsPerLaunch maps of one launch over a shared lens table.
struct LensArgs {
    LensTable t;
    MapParams maps[kMapsPerLaunch];
    int glass;
    int lanes_log2;                // log2 of the lanes per block: >= log2(n_lenses), <= 6
    int64_t out_stride;            // bytes between the maps of one launch
};

// grid.y = map of the launch.  Each block is taken by a group of 2^lanes_log2
// lanes of one wavefront, lane j of the group computing lens j's lift (rule
// 4); the lifts are then combined in lens order (rule 5) through lane
// shuffles, so the sum is the same left-to-right fp64 sum as one thread
// walking the lenses, and the group's first lane writes the level (rule 6).
__global__ __launch_bounds__(256) void levelmap_kernel(const double* __restrict__ coords, int64_t n_blocks,
                                                       LensArgs a, uint8_t* __restrict__ out) {
    const MapParams& p = a.maps[blockIdx.y];
    uint8_t* o = out + (int64_t)blockIdx.y * a.out_stride;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t b_raw = t >> a.lanes_log2;
    const int j = (int)(t & ((1 << a.lanes_log2) - 1));
    const bool live = b_raw < n_blocks;
    const int64_t b = live ? b_raw : n_blocks - 1;   // past the end: a valid block, nothing written
    if (p.n <= 0 || p.n_lenses == 0) {               // uniform over the launch's map
        if (live && j == 0) o[b] = (uint8_t)a.glass;
        return;
    }
    double lift = 0.0;
    if (j < p.n_lenses) {
        const int i = p.first + j;
        lift = lens_lift(coords[2 * b], coords[2 * b + 1], a.t.cx[i], a.t.cy[i], a.t.R[i], p.stops[0]);
    }
    const int base = (int)(threadIdx.x & 63) & ~((1 << a.lanes_log2) - 1);
    const int rung = lens_rung(lift, base, p, a.glass);
    if (live && j == 0) o[b] = (uint8_t)rung;
}

int lens_check_map(const qam_lens* lenses, int n_lenses, const qam_lens_params* params, int n_rungs, int glass,
                   MapParams& mp, const char* who) {
    if (n_lenses < 0 || n_lenses > QAM_MAX_LENSES)
        QAM_FAIL(QAM_ERR_ARG, "%s: n_lenses=%d outside [0, %d]", who, n_lenses, QAM_MAX_LENSES);
    if (n_lenses > 0 && !lenses) QAM_FAIL(QAM_ERR_NULL, "%s: null lenses", who);
    const double f = params->f, g = params->g;
    if (!(f >= 0.0 && f <= 1.0)) QAM_FAIL(QAM_ERR_ARG, "%s: f outside [0, 1]", who);
    if (params->radius_mode != QAM_RADIUS_LENS && params->radius_mode != QAM_RADIUS_ZONE)
        QAM_FAIL(QAM_ERR_ARG, "%s: unknown radius_mode %d", who, params->radius_mode);
    if (params->radius_mode == QAM_RADIUS_ZONE && !(params->width >= 0.0 && isfinite(params->width)))
        QAM_FAIL(QAM_ERR_ARG, "%s: zone radius needs a finite width >= 0", who);
    if (!(g >= 0.0 && g <= 1.0)) QAM_FAIL(QAM_ERR_ARG, "%s: g outside [0, 1]", who);
    if (params->combine != QAM_COMBINE_SUM && params->combine != QAM_COMBINE_MAX)
        QAM_FAIL(QAM_ERR_ARG, "%s: combine must be SUM or MAX", who);
    const int m = n_rungs - 1;
    const int kappa = glass + (int)floor(g * (double)(m - glass));   // rule 2
    const int n = kappa - glass;
    mp = MapParams{};
    mp.n = n;
    if (params->n_stops != 0) {   // rule 3, given
        if (params->n_stops != n)
            QAM_FAIL(QAM_ERR_ARG, "%s: %d stops given, kappa - glass = %d", who, params->n_stops, n);
        for (int j = 0; j < n; ++j) {
            if (!(params->stops[j] > 0.0) || !isfinite(params->stops[j]))
                QAM_FAIL(QAM_ERR_ARG, "%s: stop %d not positive and finite", who, j);
            if (j > 0 && !(params->stops[j] < params->stops[j - 1]))
                QAM_FAIL(QAM_ERR_ARG, "%s: stops not strictly decreasing", who);
            mp.stops[j] = params->stops[j];
        }
    } else {                      // rule 3, default spacing
        for (int j = 0; j < n; ++j) mp.stops[j] = (double)(n - j) / (double)n;
    }
    for (int i = 0; i < n_lenses; ++i)
        if (!isfinite(lenses[i].cx) || !isfinite(lenses[i].cy) || !(lenses[i].r >= 0.0) || !isfinite(lenses[i].r))
            QAM_FAIL(QAM_ERR_ARG, "%s: lens %d has a non-finite centre or a bad size", who, i);
    mp.combine = params->combine;
    mp.n_lenses = n_lenses;
    return QAM_OK;
}

double lens_radius(const qam_lens_params& p, double r, double f) {
    if (p.radius_mode == QAM_RADIUS_ZONE) return f * p.width;   // R = f D, every lens alike
    return f == 1.0 ? INFINITY : (r * f) / (1.0 - f);
}

int lens_check_ladder(const uint8_t* ladder_bits, int n_rungs, int glass, const char* who) {
    if (n_rungs < 2 || n_rungs > QAM_MAX_RUNGS)
        QAM_FAIL(QAM_ERR_LADDER, "%s: n_rungs=%d outside [2, %d]", who, n_rungs, QAM_MAX_RUNGS);
    if (ladder_bits[0] != 0) QAM_FAIL(QAM_ERR_LADDER, "%s: ladder must start at ZERO", who);
    for (int i = 1; i < n_rungs; ++i)
        if (ladder_bits[i] <= ladder_bits[i - 1]) QAM_FAIL(QAM_ERR_LADDER, "%s: ladder not increasing", who);
    if (glass < 0 || glass >= n_rungs) QAM_FAIL(QAM_ERR_ARG, "%s: glass=%d not a rung", who, glass);
    return QAM_OK;
}

int lens_check_product_ladder(const uint8_t* ladder_bits, int n_rungs, int glass, const char* who) {
    static const uint8_t kProduct[5] = {0, 2, 4, 6, 8};
    if (n_rungs != 5) QAM_FAIL(QAM_ERR_LADDER, "%s: the product ladder {0,2,4,6,8} has 5 rungs, got %d", who, n_rungs);
    for (int i = 0; i < 5; ++i)
        if (ladder_bits[i] != kProduct[i]) QAM_FAIL(QAM_ERR_LADDER, "%s: ladder must be {0,2,4,6,8}", who);
    return lens_check_ladder(ladder_bits, n_rungs, glass, who);
}

// Lanes per block: the least power of two holding the launch's lens count.
static int lanes_log2_for(int n_lenses) {
    int l = 0;
    while ((1 << l) < n_lenses) ++l;
    return l;
}

static void launch_maps(const double* coords, int64_t n_blocks, const LensArgs& a, int cnt, uint8_t* out,
                        hipStream_t s) {
    const int64_t threads = n_blocks << a.lanes_log2;
    const dim3 grid((unsigned)((threads + 255) / 256), (unsigned)cnt);
    hipLaunchKernelGGL(levelmap_kernel, grid, dim3(256), 0, s, coords, n_blocks, a, out);
}

// Rule 7 bytes of a map, summed exactly: sum_b w_b bits(level_b) into *acc
// (int64 adds, so the order does not matter).
__global__ __launch_bounds__(256) void map_bits_kernel(const uint8_t* __restrict__ level,
                                                       const int64_t* __restrict__ w, int64_t n_blocks,
                                                       LadderBits bits, unsigned long long* acc) {
    unsigned long long sum = 0;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < n_blocks; b += (int64_t)gridDim.x * blockDim.x)
        sum += (unsigned long long)w[b] * bits.v[level[b]];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    if ((threadIdx.x & 63) == 0 && sum) atomicAdd(acc, sum);
}

}  // namespace qam

using namespace qam;

extern "C" int qam_build_level_maps(const double* coords, int64_t n_blocks, const qam_lens* lenses, int n_lenses,
                                    const qam_lens_params* params, const uint8_t* ladder_bits, int n_rungs,
                                    int glass, int n_maps, uint8_t* level_out, hipStream_t s) {
    clear_error();
    if (n_blocks < 0) QAM_FAIL(QAM_ERR_SHAPE, "build_level_maps: n_blocks < 0");
    if (!params || !ladder_bits) QAM_FAIL(QAM_ERR_NULL, "build_level_maps: null params/ladder");
    if (n_maps < 1 || n_maps > QAM_MAX_BATCH_MFMA)
        QAM_FAIL(QAM_ERR_ARG, "build_level_maps: n_maps=%d outside [1, %d]", n_maps, QAM_MAX_BATCH_MFMA);
    if (n_blocks > 0 && (!coords || !level_out)) QAM_FAIL(QAM_ERR_NULL, "build_level_maps: null coords/output");
    if (int rc = lens_check_product_ladder(ladder_bits, n_rungs, glass, "build_level_maps")) return rc;
    if (n_lenses < 0 || n_lenses > QAM_MAX_LENSES)
        QAM_FAIL(QAM_ERR_ARG, "build_level_maps: n_lenses=%d outside [0, %d]", n_lenses, QAM_MAX_LENSES);
    std::vector<MapParams> mps((size_t)n_maps);
    for (int k = 0; k < n_maps; ++k)
        if (int rc = lens_check_map(n_lenses ? lenses + (int64_t)k * n_lenses : nullptr, n_lenses, params + k, n_rungs,
                               glass, mps[(size_t)k], "build_level_maps"))
            return rc;
    if (n_blocks == 0) return QAM_OK;
    if (n_blocks > (INT64_C(1) << 31) >> lanes_log2_for(n_lenses))
        QAM_FAIL(QAM_ERR_SHAPE, "build_level_maps: %lld blocks of %d lenses exceed one launch", (long long)n_blocks,
                 n_lenses);
    // as many maps per launch as the lens table (and the map slots) hold
    const int per = std::max(1, std::min(kMapsPerLaunch, n_lenses ? QAM_MAX_LENSES / n_lenses : kMapsPerLaunch));
    for (int k0 = 0; k0 < n_maps; k0 += per) {
        const int cnt = std::min(per, n_maps - k0);
        LensArgs a = {};
        for (int k = 0; k < cnt; ++k) {
            a.maps[k] = mps[(size_t)(k0 + k)];
            a.maps[k].first = k * n_lenses;
            for (int i = 0; i < n_lenses; ++i) {
                const qam_lens& l = lenses[(int64_t)(k0 + k) * n_lenses + i];
                a.t.cx[k * n_lenses + i] = l.cx;
                a.t.cy[k * n_lenses + i] = l.cy;
                a.t.R[k * n_lenses + i] = lens_radius(params[k0 + k], l.r, params[k0 + k].f);
            }
        }
        a.glass = glass;
        a.lanes_log2 = lanes_log2_for(n_lenses);
        a.out_stride = n_blocks;
        launch_maps(coords, n_blocks, a, cnt, level_out + (int64_t)k0 * n_blocks, s);
        QAM_HIP_CHECK(hipGetLastError());
    }
    set_variant("levelmap_fp64");
    return QAM_OK;
}

static int build_map(const double* coords, int64_t n_blocks, const qam_lens* lenses, int n_lenses,
                     const qam_lens_params* params, const uint8_t* ladder_bits, int n_rungs, int glass,
                     uint8_t* level_out, hipStream_t s, bool product, const char* who) {
    clear_error();
    if (n_blocks < 0) QAM_FAIL(QAM_ERR_SHAPE, "%s: n_blocks < 0", who);
    if (!params || !ladder_bits) QAM_FAIL(QAM_ERR_NULL, "%s: null params/ladder", who);
    if (n_blocks > 0 && (!coords || !level_out)) QAM_FAIL(QAM_ERR_NULL, "%s: null coords/output", who);
    if (int rc = product ? lens_check_product_ladder(ladder_bits, n_rungs, glass, who)
                         : lens_check_ladder(ladder_bits, n_rungs, glass, who))
        return rc;
    MapParams mp;
    if (int rc = lens_check_map(lenses, n_lenses, params, n_rungs, glass, mp, who)) return rc;
    if (n_blocks == 0) return QAM_OK;
    if (n_blocks > (INT64_C(1) << 31) >> lanes_log2_for(n_lenses))
        QAM_FAIL(QAM_ERR_SHAPE, "%s: %lld blocks of %d lenses exceed one launch", who, (long long)n_blocks, n_lenses);
    LensArgs a = {};
    a.maps[0] = mp;
    for (int i = 0; i < n_lenses; ++i) {
        a.t.cx[i] = lenses[i].cx;
        a.t.cy[i] = lenses[i].cy;
        a.t.R[i] = lens_radius(*params, lenses[i].r, params->f);
    }
    a.glass = glass;
    a.lanes_log2 = lanes_log2_for(n_lenses);
    a.out_stride = n_blocks;
    launch_maps(coords, n_blocks, a, 1, level_out, s);
    QAM_HIP_CHECK(hipGetLastError());
    set_variant("levelmap_fp64");
    return QAM_OK;
}

extern "C" int qam_build_level_map(const double* coords, int64_t n_blocks, const qam_lens* lenses, int n_lenses,
                                   const qam_lens_params* params, const uint8_t* ladder_bits, int n_rungs,
                                   int glass, uint8_t* level_out, hipStream_t s) {
    return build_map(coords, n_blocks, lenses, n_lenses, params, ladder_bits, n_rungs, glass, level_out, s, true,
                     "build_level_map");
}

extern "C" int qam_build_rung_map(const double* coords, int64_t n_blocks, const qam_lens* lenses, int n_lenses,
                                  const qam_lens_params* params, const uint8_t* ladder_bits, int n_rungs, int glass,
                                  uint8_t* rung_out, hipStream_t s) {
    return build_map(coords, n_blocks, lenses, n_lenses, params, ladder_bits, n_rungs, glass, rung_out, s, false,
                     "build_rung_map");
}

// The largest squared distance between two blocks, exactly (a max of fp64
// values, order-free), into *acc as its bit pattern (non-negative doubles
// order as their bits).  One thread per block i against every block j > i.
__global__ __launch_bounds__(256) void width_kernel(const double* __restrict__ coords, int64_t n,
                                                    unsigned long long* acc) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    double best = 0.0;
    if (i < n) {
        const double xi = coords[2 * i], yi = coords[2 * i + 1];
        for (int64_t j = i + 1; j < n; ++j) {
            const double dx = coords[2 * j] - xi;
            const double dy = coords[2 * j + 1] - yi;
            const double d2 = dx * dx + dy * dy;
            best = d2 > best ? d2 : best;
        }
    }
    unsigned long long u = __builtin_bit_cast(unsigned long long, best);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long v = __shfl_xor(u, o);
        u = v > u ? v : u;
    }
    if ((threadIdx.x & 63) == 0 && u) atomicMax(acc, u);
}

extern "C" int qam_field_width(const double* coords, int64_t n_blocks, void* workspace, size_t workspace_bytes,
                               double* width_out, hipStream_t s) {
    clear_error();
    if (!coords || !workspace || !width_out) QAM_FAIL(QAM_ERR_NULL, "field_width: null pointer");
    if (n_blocks < 1 || n_blocks > QAM_MAX_FIELD_BLOCKS)
        QAM_FAIL(QAM_ERR_SHAPE, "field_width: n_blocks=%lld outside [1, %d]", (long long)n_blocks, QAM_MAX_FIELD_BLOCKS);
    if (workspace_bytes < 256) QAM_FAIL(QAM_ERR_WORKSPACE, "field_width: workspace %zu < 256 bytes", workspace_bytes);
    if (!aligned(workspace, 256) || !aligned(coords, 8))
        QAM_FAIL(QAM_ERR_ALIGN, "field_width: workspace 256-byte and coords 8-byte aligned");
    unsigned long long* acc = static_cast<unsigned long long*>(workspace);
    unsigned long long host = 0;
    QAM_HIP_CHECK(hipMemsetAsync(acc, 0, sizeof(unsigned long long), s));
    hipLaunchKernelGGL(width_kernel, dim3((unsigned)((n_blocks + 255) / 256)), dim3(256), 0, s, coords, n_blocks, acc);
    QAM_HIP_CHECK(hipGetLastError());
    QAM_HIP_CHECK(hipMemcpyAsync(&host, acc, sizeof(host), hipMemcpyDeviceToHost, s));
    QAM_HIP_CHECK(hipStreamSynchronize(s));
    const double d2 = __builtin_bit_cast(double, host);
    if (!isfinite(d2)) QAM_FAIL(QAM_ERR_ARG, "field_width: coordinates not finite");
    *width_out = sqrt(d2);
    set_variant("field_width_fp64");
    return QAM_OK;
}

extern "C" int qam_fit_focus_area(const double* coords, int64_t n_blocks, const int64_t* block_weights,
                                  const qam_lens* lenses, int n_lenses, const qam_lens_params* params,
                                  const uint8_t* ladder_bits, int n_rungs, int glass, int64_t budget_bytes, int iters,
                                  uint8_t* level_out, void* workspace, size_t workspace_bytes, double* f_out,
                                  int64_t* bytes_out, hipStream_t s) {
    clear_error();
    if (!params || !ladder_bits || !f_out || !bytes_out) QAM_FAIL(QAM_ERR_NULL, "fit_focus_area: null pointer");
    if (n_blocks < 1) QAM_FAIL(QAM_ERR_SHAPE, "fit_focus_area: n_blocks < 1");
    if (!coords || !block_weights || !level_out || !workspace) QAM_FAIL(QAM_ERR_NULL, "fit_focus_area: null pointer");
    if (iters < 0 || iters > 60) QAM_FAIL(QAM_ERR_ARG, "fit_focus_area: iters=%d outside [0, 60]", iters);
    if (budget_bytes < 0) QAM_FAIL(QAM_ERR_ARG, "fit_focus_area: negative budget");
    if (workspace_bytes < 256) QAM_FAIL(QAM_ERR_WORKSPACE, "fit_focus_area: workspace %zu < 256 bytes", workspace_bytes);
    if (!aligned(workspace, 256) || !aligned(block_weights, 8) || !aligned(coords, 8))
        QAM_FAIL(QAM_ERR_ALIGN, "fit_focus_area: workspace 256-byte, weights and coords 8-byte aligned");
    if (int rc = lens_check_product_ladder(ladder_bits, n_rungs, glass, "fit_focus_area")) return rc;
    if (n_blocks > (INT64_C(1) << 31) >> lanes_log2_for(n_lenses))
        QAM_FAIL(QAM_ERR_SHAPE, "fit_focus_area: %lld blocks of %d lenses exceed one launch", (long long)n_blocks,
                 n_lenses);
    qam_lens_params p = *params;
    LensArgs a = {};
    LadderBits lb = {};
    for (int i = 0; i < n_rungs; ++i) lb.v[i] = ladder_bits[i];
    unsigned long long* acc = static_cast<unsigned long long*>(workspace);
    unsigned long long host = 0;
    // the map at f and its byte count (host-synchronous)
    auto at = [&](double f, int64_t& bytes) -> int {
        p.f = f;
        if (int rc = lens_check_map(lenses, n_lenses, &p, n_rungs, glass, a.maps[0], "fit_focus_area")) return rc;
        for (int i = 0; i < n_lenses; ++i) {
            a.t.cx[i] = lenses[i].cx;
            a.t.cy[i] = lenses[i].cy;
            a.t.R[i] = lens_radius(p, lenses[i].r, f);
        }
        a.glass = glass;
        a.lanes_log2 = lanes_log2_for(n_lenses);
        a.out_stride = n_blocks;
        launch_maps(coords, n_blocks, a, 1, level_out, s);
        QAM_HIP_CHECK(hipGetLastError());
        QAM_HIP_CHECK(hipMemsetAsync(acc, 0, sizeof(unsigned long long), s));
        const int64_t grid = std::min<int64_t>(1024, (n_blocks + 255) / 256);
        hipLaunchKernelGGL(map_bits_kernel, dim3((unsigned)grid), dim3(256), 0, s, level_out, block_weights, n_blocks,
                           lb, acc);
        QAM_HIP_CHECK(hipGetLastError());
        QAM_HIP_CHECK(hipMemcpyAsync(&host, acc, sizeof(unsigned long long), hipMemcpyDeviceToHost, s));
        QAM_HIP_CHECK(hipStreamSynchronize(s));
        if (host % 8) QAM_FAIL(QAM_ERR_ARG, "fit_focus_area: weight bits not a whole number of bytes");
        bytes = (int64_t)(host / 8);
        return QAM_OK;
    };
    int rc = QAM_OK;
    double f = 1.0;
    int64_t b = 0;
    do {
        if ((rc = at(1.0, b))) break;
        if (b <= budget_bytes) break;
        f = 0.0;
        if ((rc = at(0.0, b))) break;
        if (b > budget_bytes) break;
        double lo = 0.0, hi = 1.0;
        for (int k = 0; k < iters; ++k) {
            const double mid = 0.5 * (lo + hi);
            int64_t bm = 0;
            if ((rc = at(mid, bm))) break;
            if (bm <= budget_bytes) lo = mid;
            else hi = mid;
        }
        if (rc) break;
        f = lo;
        rc = at(lo, b);   // the returned map is the one at f
    } while (false);
    if (rc) return rc;
    *f_out = f;
    *bytes_out = b;
    set_variant("fit_focus_area");
    return QAM_OK;
}
