// Level map from the lens rules: one thread per block, fp64.
//
// Rules 1-6 of the FoQLens landing page (vovanda.github.io/FoQLens), section
// "The mechanism", which repeat the rule list of "FoQZones, the mechanism" on
// foqlens.sawking.tech with the per-lens radius R_i = r_i f / (1 - f):
//   1 radius   R_i = r_i f / (1 - f)
//   2 ceiling  kappa = gamma + floor(g (m - gamma))
//   3 stops    s_kappa < ... < s_(gamma+1), ring ends in radii
//   4 lift     rho_i = d(b, c_i) / R_i,  L_i = max(0, 1 - rho_i / s_last)
//   5 combine  L = min(1, sum L_i)  or  max L_i
//   6 level    rho* = s_last (1 - L); the ring rho* falls into; else the glass
// Readings where the pages are open: Euclidean distance on the block field,
// s_last = s_(gamma+1), default stops evenly spaced with the outermost at 1,
// half-open rings (level = gamma + #{j : rho* < s_(gamma+j)}), R = +inf at
// f = 1, and a radius of 0 lifting only a block at distance 0.
//
// The file is compiled with -ffp-contract=off: every product and sum is a
// separate correctly rounded IEEE operation, as is sqrt (an FMA-corrected
// Newton sequence) and division, so the map matches the same rules evaluated
// in IEEE fp64 on a CPU bit for bit.
#include <math.h>

#include <algorithm>
#include <vector>

#include "qam_common.h"

namespace qam {

constexpr int kMapsPerLaunch = 8;

// One map's rule parameters (its lenses are [first, first + n_lenses) of the
// launch's lens table).
struct MapParams {
    double stops[QAM_MAX_STOPS];
    double f, g;
    int combine;
    int n_stops;     // 0: default spacing
    int first;
    int n_lenses;
};

struct LensArgs {
    double cx[QAM_MAX_LENSES];
    double cy[QAM_MAX_LENSES];
    double r[QAM_MAX_LENSES];
    MapParams maps[kMapsPerLaunch];
    int n_rungs;
    int glass;
    int64_t out_stride;   // bytes between the maps of one launch
};

// grid.y = map of the launch; one thread per block of that map.
__global__ __launch_bounds__(256) void levelmap_kernel(const double* __restrict__ coords, int64_t n_blocks,
                                                       LensArgs a, uint8_t* __restrict__ out) {
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n_blocks) return;
    const MapParams& p = a.maps[blockIdx.y];
    uint8_t* o = out + (int64_t)blockIdx.y * a.out_stride;
    const int m = a.n_rungs - 1;
    // rule 2: ceiling
    const int kappa = a.glass + (int)floor(p.g * (double)(m - a.glass));
    const int n = kappa - a.glass;
    if (n <= 0 || p.n_lenses == 0) {
        o[b] = (uint8_t)a.glass;
        return;
    }
    // rule 3: stops, s[j-1] = s_(gamma+j)
    double s[QAM_MAX_STOPS];
#pragma unroll
    for (int j = 0; j < QAM_MAX_STOPS; ++j) {
        if (p.n_stops) s[j] = p.stops[j];
        else s[j] = (double)(n - j) / (double)n;
    }
    const double s_last = s[0];
    const double bx = coords[2 * b];
    const double by = coords[2 * b + 1];
    double acc = 0.0;
    for (int i = p.first; i < p.first + p.n_lenses; ++i) {
        // rule 1: radius
        const double R = (p.f == 1.0) ? INFINITY : (a.r[i] * p.f) / (1.0 - p.f);
        // rule 4: distance in radii, then the lift
        const double dx = bx - a.cx[i];
        const double dy = by - a.cy[i];
        const double dist = sqrt(dx * dx + dy * dy);
        double rho;
        if (R == 0.0) rho = (dist == 0.0) ? 0.0 : INFINITY;
        else rho = dist / R;
        const double t = 1.0 - rho / s_last;
        const double lift = t > 0.0 ? t : 0.0;
        // rule 5: combine (sum in lens order, or max)
        if (p.combine == QAM_COMBINE_SUM) acc = acc + lift;
        else acc = acc > lift ? acc : lift;
    }
    const double L = (p.combine == QAM_COMBINE_SUM) ? (acc < 1.0 ? acc : 1.0) : acc;
    // rule 6: the ring rho* falls into
    const double rho_star = s_last * (1.0 - L);
    int count = 0;
#pragma unroll
    for (int j = 0; j < QAM_MAX_STOPS; ++j)
        if (j < n && rho_star < s[j]) ++count;
    o[b] = (uint8_t)(a.glass + count);
}

// Host checks of one map's parameters and lenses (error text names `who`).
static int check_map(const qam_lens* lenses, int n_lenses, const qam_lens_params* params, int n_rungs, int glass,
                     MapParams& mp, const char* who) {
    if (n_lenses < 0 || n_lenses > QAM_MAX_LENSES)
        QAM_FAIL(QAM_ERR_ARG, "%s: n_lenses=%d outside [0, %d]", who, n_lenses, QAM_MAX_LENSES);
    if (n_lenses > 0 && !lenses) QAM_FAIL(QAM_ERR_NULL, "%s: null lenses", who);
    const double f = params->f, g = params->g;
    if (!(f >= 0.0 && f <= 1.0)) QAM_FAIL(QAM_ERR_ARG, "%s: f outside [0, 1]", who);
    if (!(g >= 0.0 && g <= 1.0)) QAM_FAIL(QAM_ERR_ARG, "%s: g outside [0, 1]", who);
    if (params->combine != QAM_COMBINE_SUM && params->combine != QAM_COMBINE_MAX)
        QAM_FAIL(QAM_ERR_ARG, "%s: combine must be SUM or MAX", who);
    const int m = n_rungs - 1;
    const int kappa = glass + (int)floor(g * (double)(m - glass));
    const int n = kappa - glass;
    mp = MapParams{};
    if (params->n_stops != 0) {
        if (params->n_stops != n)
            QAM_FAIL(QAM_ERR_ARG, "%s: %d stops given, kappa - glass = %d", who, params->n_stops, n);
        for (int j = 0; j < n; ++j) {
            if (!(params->stops[j] > 0.0) || !isfinite(params->stops[j]))
                QAM_FAIL(QAM_ERR_ARG, "%s: stop %d not positive and finite", who, j);
            if (j > 0 && !(params->stops[j] < params->stops[j - 1]))
                QAM_FAIL(QAM_ERR_ARG, "%s: stops not strictly decreasing", who);
            mp.stops[j] = params->stops[j];
        }
    }
    for (int i = 0; i < n_lenses; ++i)
        if (!isfinite(lenses[i].cx) || !isfinite(lenses[i].cy) || !(lenses[i].r >= 0.0) || !isfinite(lenses[i].r))
            QAM_FAIL(QAM_ERR_ARG, "%s: lens %d has a non-finite centre or a bad size", who, i);
    mp.f = f;
    mp.g = g;
    mp.combine = params->combine;
    mp.n_stops = params->n_stops;
    mp.n_lenses = n_lenses;
    return QAM_OK;
}

static int check_ladder(const uint8_t* ladder_bits, int n_rungs, int glass, const char* who) {
    if (n_rungs < 2 || n_rungs > QAM_MAX_RUNGS)
        QAM_FAIL(QAM_ERR_LADDER, "%s: n_rungs=%d outside [2, %d]", who, n_rungs, QAM_MAX_RUNGS);
    if (ladder_bits[0] != 0) QAM_FAIL(QAM_ERR_LADDER, "%s: ladder must start at ZERO", who);
    for (int i = 1; i < n_rungs; ++i)
        if (ladder_bits[i] <= ladder_bits[i - 1]) QAM_FAIL(QAM_ERR_LADDER, "%s: ladder not increasing", who);
    if (glass < 0 || glass >= n_rungs) QAM_FAIL(QAM_ERR_ARG, "%s: glass=%d not a rung", who, glass);
    return QAM_OK;
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
    if (int rc = check_ladder(ladder_bits, n_rungs, glass, "build_level_maps")) return rc;
    if (n_lenses < 0 || n_lenses > QAM_MAX_LENSES)
        QAM_FAIL(QAM_ERR_ARG, "build_level_maps: n_lenses=%d outside [0, %d]", n_lenses, QAM_MAX_LENSES);
    std::vector<MapParams> mps((size_t)n_maps);
    for (int k = 0; k < n_maps; ++k)
        if (int rc = check_map(n_lenses ? lenses + (int64_t)k * n_lenses : nullptr, n_lenses, params + k, n_rungs,
                               glass, mps[(size_t)k], "build_level_maps"))
            return rc;
    if (n_blocks == 0) return QAM_OK;
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
                a.cx[k * n_lenses + i] = l.cx;
                a.cy[k * n_lenses + i] = l.cy;
                a.r[k * n_lenses + i] = l.r;
            }
        }
        a.n_rungs = n_rungs;
        a.glass = glass;
        a.out_stride = n_blocks;
        const dim3 grid((unsigned)((n_blocks + 255) / 256), (unsigned)cnt);
        hipLaunchKernelGGL(levelmap_kernel, grid, dim3(256), 0, s, coords, n_blocks, a, level_out + (int64_t)k0 * n_blocks);
        QAM_HIP_CHECK(hipGetLastError());
    }
    set_variant("levelmap_fp64");
    return QAM_OK;
}

extern "C" int qam_build_level_map(const double* coords, int64_t n_blocks, const qam_lens* lenses, int n_lenses,
                                   const qam_lens_params* params, const uint8_t* ladder_bits, int n_rungs,
                                   int glass, uint8_t* level_out, hipStream_t s) {
    clear_error();
    if (n_blocks < 0) QAM_FAIL(QAM_ERR_SHAPE, "build_level_map: n_blocks < 0");
    if (!params || !ladder_bits) QAM_FAIL(QAM_ERR_NULL, "build_level_map: null params/ladder");
    if (n_blocks > 0 && (!coords || !level_out)) QAM_FAIL(QAM_ERR_NULL, "build_level_map: null coords/output");
    if (int rc = check_ladder(ladder_bits, n_rungs, glass, "build_level_map")) return rc;
    MapParams mp;
    if (int rc = check_map(lenses, n_lenses, params, n_rungs, glass, mp, "build_level_map")) return rc;
    if (n_blocks == 0) return QAM_OK;
    LensArgs a = {};
    a.maps[0] = mp;
    for (int i = 0; i < n_lenses; ++i) {
        a.cx[i] = lenses[i].cx;
        a.cy[i] = lenses[i].cy;
        a.r[i] = lenses[i].r;
    }
    a.n_rungs = n_rungs;
    a.glass = glass;
    a.out_stride = n_blocks;
    const int64_t grid = (n_blocks + 255) / 256;
    hipLaunchKernelGGL(levelmap_kernel, dim3((unsigned)grid, 1), dim3(256), 0, s, coords, n_blocks, a, level_out);
    QAM_HIP_CHECK(hipGetLastError());
    set_variant("levelmap_fp64");
    return QAM_OK;
}
