// The lens rules of the FoQLens landing page (vovanda.github.io/FoQLens),
// section "The mechanism", as the kernels run them: rules 1-3 depend on the
// map and the lens only, so the host evaluates them (the same IEEE fp64
// operations in the same order as the rules, hence the same values) and the
// kernels run rules 4-6 per block.  Shared by the level-map kernel and the
// grouped product that builds its map in the same launch, so both give the
// same rung for a block bit for bit.
//
// Rules, with the readings taken where the pages are open:
//   1 radius   R_i = r_i f / (1 - f), +inf at f = 1 (the lens rule); or the
//              zone rule R = f D of "FoQLens", "FoQZones, the mechanism", with
//              D the width of the field, the same R for every lens
//   2 ceiling  kappa = gamma + floor(g (m - gamma)); n = kappa - gamma
//   3 stops    s_(gamma+1) > ... > s_kappa, default (n - j) / n, j = 0..n-1
//   4 lift     rho_i = d(b, c_i) / R_i (Euclidean d; R = 0 lifts only a block
//              at distance 0), L_i = max(0, 1 - rho_i / s_last), s_last = s_(gamma+1)
//   5 combine  L = min(1, sum L_i) in lens order, or max L_i
//   6 level    rho* = s_last (1 - L); gamma + #{j : rho* < s_(gamma+j)}
// Every file including this is compiled with -ffp-contract=off: no product
// and sum is fused, and sqrt and division are correctly rounded.
#pragma once

#include "qam_common.h"

namespace qam {

// One map's rules 2-3 and its lenses' place in the lens table.
struct MapParams {
    double stops[QAM_MAX_STOPS];   // s_(gamma+1) > ... > s_kappa, n of them
    int n;                         // kappa - gamma (0: every block at the glass)
    int combine;                   // QAM_COMBINE_SUM / QAM_COMBINE_MAX
    int first;                     // the map's lenses: [first, first + n_lenses)
    int n_lenses;
};

// Lens centres and rule-1 radii.
struct LensTable {
    double cx[QAM_MAX_LENSES];
    double cy[QAM_MAX_LENSES];
    double R[QAM_MAX_LENSES];
};

// One map as a kernel argument: its rules, lenses and glass rung.
struct LensMap {
    LensTable t;
    MapParams p;
    int glass;
};

// Rule 4 for one lens at block coordinates (bx, by).
__device__ __forceinline__ double lens_lift(double bx, double by, double cx, double cy, double R, double s_last) {
    const double dx = bx - cx;
    const double dy = by - cy;
    const double dist = sqrt(dx * dx + dy * dy);
    double rho;
    if (R == 0.0) rho = (dist == 0.0) ? 0.0 : INFINITY;
    else rho = dist / R;
    const double t = 1.0 - rho / s_last;
    return t > 0.0 ? t : 0.0;
}

// Rules 5-6 for a block whose lens k lift sits on lane base + k of the
// wavefront (k < p.n_lenses).  Every lane of the wavefront must call this
// with the same p (the lifts travel by lane shuffles); each gets the rung of
// its own group.  The sum runs in lens order, left to right.
__device__ __forceinline__ int lens_rung(double lift, int base, const MapParams& p, int glass) {
    double acc = 0.0;
    for (int k = 0; k < p.n_lenses; ++k) {
        const double v = __shfl(lift, base + k, 64);
        if (p.combine == QAM_COMBINE_SUM) acc = acc + v;
        else acc = acc > v ? acc : v;
    }
    const double L = (p.combine == QAM_COMBINE_SUM) ? (acc < 1.0 ? acc : 1.0) : acc;
    const double rho_star = p.stops[0] * (1.0 - L);
    int count = 0;
    for (int k = 0; k < p.n; ++k)
        if (rho_star < p.stops[k]) ++count;
    return glass + count;
}

// Lane `lane`'s fp64 value, into scalar registers (lane uniform).
__device__ __forceinline__ double read_lane_f64(double v, int lane) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// The rung of block b (coordinates coords[2b], coords[2b + 1]) under map m,
// computed by one whole wavefront, lane L taking lens L; rules 5-6 as in
// lens_rung (the same operations in the same order), the lifts read lane by
// lane in lens order.  Wave-uniform.
__device__ __forceinline__ int lens_block_rung(const double* coords, int64_t b, int L, const LensMap& m) {
    const MapParams& p = m.p;
    if (p.n <= 0 || p.n_lenses == 0) return m.glass;
    double lift = 0.0;
    if (L < p.n_lenses) {
        const int i = p.first + L;
        lift = lens_lift(coords[2 * b], coords[2 * b + 1], m.t.cx[i], m.t.cy[i], m.t.R[i], p.stops[0]);
    }
    double acc = 0.0;
    for (int k = 0; k < p.n_lenses; ++k) {
        const double v = read_lane_f64(lift, k);
        if (p.combine == QAM_COMBINE_SUM) acc = acc + v;
        else acc = acc > v ? acc : v;
    }
    const double Lb = (p.combine == QAM_COMBINE_SUM) ? (acc < 1.0 ? acc : 1.0) : acc;
    const double rho_star = p.stops[0] * (1.0 - Lb);
    int count = 0;
    for (int k = 0; k < p.n; ++k)
        if (rho_star < p.stops[k]) ++count;
    return m.glass + count;
}

// ---------------------------------------------------------------- host side
// Ladder checks of a map call (error text names `who`): any ladder, or the
// product's ladder {0,2,4,6,8} (rung index = slices read).
int lens_check_ladder(const uint8_t* ladder_bits, int n_rungs, int glass, const char* who);
int lens_check_product_ladder(const uint8_t* ladder_bits, int n_rungs, int glass, const char* who);
// Checks of one map's parameters and lenses; fills mp's rules 2-3, combine
// and lens count (mp.first = 0).
int lens_check_map(const qam_lens* lenses, int n_lenses, const qam_lens_params* params, int n_rungs, int glass,
                   MapParams& mp, const char* who);
// Rule 1 at focus area f: (r f) / (1 - f), +inf at f = 1; in zone mode f D.
double lens_radius(const qam_lens_params& p, double r, double f);

}  // namespace qam
