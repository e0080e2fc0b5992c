"""CPU oracle (int64 / fp64) for the mixed-depth weight-read hot path.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  No product code may
import this module; it exists to check the HIP library.

Sources (the pages this follows; cited by title and section):

* [FoQLens] "FoQLens" (foqlens.sawking.tech), table "Progress" (one stored
  stack, 2/4/6/8 bits read from one copy; a kernel that reads each block of
  rows at its own depth inside the pass) and section "FoQZones, the
  mechanism" (ladder, base G, distance, rules 1-7).
* [Lens] "FoQLens" landing page (vovanda.github.io/FoQLens), sections
  "The mechanism" (rules 1-7 with the per-lens radius R_i = r_i f/(1-f),
  the three controls glass / focus_area / focus_strength, the ladder
  ZERO, D2, D4, D6, D8 read from one stored copy of residual slices) and the
  field description (blocks of 64 output rows).
* [PoD] "Precision on Demand: Escalating Weight Bits at Uncertain Decoding
  Steps in a Small Local Model" (arXiv:2611.14418 v1), abstract (store 8-bit
  weights, decode with their top 4 bits, redo a step at 8 bits when gated;
  cost counted in weight bytes read per token).

Where the pages leave a step open, the reading taken here is stated in the
function's docstring.  Nothing here is blocked, fused or reordered: each
function is the plain definition or the rules in the pages' order.
"""

from __future__ import annotations

import numpy as np

# [Lens] "The mechanism": the ladder of this storage is ZERO, D2, D4, D6, D8.
LADDER_BITS = (0, 2, 4, 6, 8)

ROWS_PER_BLOCK = 64  # [Lens] field description: blocks of 64 output rows


# --------------------------------------------------------------------------
# Truncation: reading an int8 code at depth d
# --------------------------------------------------------------------------

def truncate(q, d: int) -> np.ndarray:
    """Code read at depth ``d`` bits from stored int8 codes ``q``.

    [PoD] abstract: decoding "with their top 4 bits" of stored 8-bit weights;
    [FoQLens] "Progress": 2, 4, 6 or 8 bits are read from one stored copy.
    Reading (the plainest one for a two's-complement byte): keep the top ``d``
    bits of the byte and zero the rest, i.e. floor truncation
    ``c_d = (q >> (8-d)) << (8-d)`` with an arithmetic shift.  ``d = 0``
    (the ZERO rung) reads nothing and gives 0.  ``d = 8`` returns ``q``.
    """
    if d not in LADDER_BITS:
        raise ValueError(f"depth {d} is not on the ladder {LADDER_BITS}")
    q = np.asarray(q).astype(np.int64)
    if d == 0:
        return np.zeros_like(q)
    sh = 8 - d
    return (q >> sh) << sh


def slice_digits(q) -> np.ndarray:
    """The four 2-bit residual digits of each int8 code.

    [Lens] "The mechanism": one stored copy of residual slices read at 2, 4,
    6 or 8 bits.  Digit ``s`` (``s = 3`` the top one, carrying the sign) is
    ``(u >> 2s) & 3`` with ``u`` the code's byte.  Returns an int64 array of
    shape ``q.shape + (4,)`` indexed by ``s``.
    """
    u = np.asarray(q).astype(np.int64) & 0xFF
    return np.stack([(u >> (2 * s)) & 3 for s in range(4)], axis=-1)


def residual_code(digits, d: int) -> np.ndarray:
    """Rebuild the depth-``d`` code from residual digits (base + refinements).

    The top digit is a signed base (two's complement, values -2..1) worth 64;
    each further slice adds a refinement worth 16, 4, 1.  Reading depth ``d``
    sums the base and the first ``d/2 - 1`` refinements.
    """
    if d not in LADDER_BITS:
        raise ValueError(f"depth {d} is not on the ladder {LADDER_BITS}")
    digits = np.asarray(digits).astype(np.int64)
    if d == 0:
        return np.zeros(digits.shape[:-1], dtype=np.int64)
    top = digits[..., 3]
    out = 64 * (top - 4 * (top >= 2))
    weights = {2: 16, 1: 4, 0: 1}
    for s in (2, 1, 0):
        if (3 - s) < d // 2:
            out = out + weights[s] * digits[..., s]
    return out


# --------------------------------------------------------------------------
# Lens rules: the per-block level map
# --------------------------------------------------------------------------

def ceiling(g: float, m: int, glass: int) -> int:
    """Rule 2 ([FoQLens] "FoQZones, the mechanism"; [Lens] "The mechanism"):
    kappa = gamma + floor(g (m - gamma)); g = 0 gives the glass, g = 1 the top rung."""
    return int(glass + np.floor(np.float64(g) * np.float64(m - glass)))


def profile_stops(n: int, stops=None) -> np.ndarray:
    """Rule 3: ring stops s_(gamma+1) > ... > s_kappa, in radii.

    Returned as an fp64 array ``s`` with ``s[j-1] = s_(gamma+j)``, j = 1..n.
    The pages give only the ordering ("where each ring ends, in radii; above
    1, past the edge").  Reading taken: by default the stops are evenly spaced
    with the outermost at 1, ``s_(gamma+j) = (n - j + 1) / n`` (one fp64
    division each); explicit stops must be strictly decreasing and positive.
    """
    if n <= 0:
        return np.zeros(0, dtype=np.float64)
    if stops is None:
        return np.array([np.float64(n - j + 1) / np.float64(n) for j in range(1, n + 1)],
                        dtype=np.float64)
    s = np.asarray(stops, dtype=np.float64)
    if s.shape != (n,):
        raise ValueError(f"need {n} stops, got {s.shape}")
    if not (np.all(s > 0) and np.all(np.diff(s) < 0)):
        raise ValueError("stops must be positive and strictly decreasing")
    return s


def lens_radius(r, f: float) -> np.ndarray:
    """Rule 1 ([Lens] "The mechanism"): R_i = r_i f / (1 - f).

    Evaluated as ``(r * f) / (1 - f)`` in fp64.  Reading taken for the end
    f = 1 (a division by zero): the radius is +inf, every block lies at
    distance 0 in radii.  f = 0 gives R = 0: only a block exactly at the
    centre is inside.
    """
    r = np.asarray(r, dtype=np.float64)
    f = np.float64(f)
    if f == 1.0:
        return np.full(r.shape, np.inf)
    return (r * f) / (np.float64(1.0) - f)


def zone_radius(f: float, width: float) -> np.float64:
    """Rule 1 of the zone form ([FoQLens] "FoQZones, the mechanism"): the
    zone radius is R = f D, with D the width of the network; f = 0 leaves
    only the centre, f = 1 takes the whole network.  One fp64 product, the
    same R for every zone."""
    return np.float64(f) * np.float64(width)


def field_width(coords) -> np.float64:
    """D for the zone radius: the width of the network, read as the largest
    Euclidean distance between two blocks of the field (its diameter), so
    that at f = 1 a zone around any block reaches every block.  The largest
    squared distance dx*dx + dy*dy over all pairs (fp64, elementwise, no
    fused multiply-add), then one correctly rounded square root."""
    c = np.asarray(coords, dtype=np.float64).reshape(-1, 2)
    best = np.float64(0.0)
    for i in range(c.shape[0] - 1):
        dx = c[i + 1:, 0] - c[i, 0]
        dy = c[i + 1:, 1] - c[i, 1]
        best = max(best, np.max(dx * dx + dy * dy))
    return np.sqrt(best)


def level_map(coords, centres, radii, f: float, g: float, combine: str,
              n_rungs: int, glass: int, stops=None, radius: str = "lens", width=None) -> np.ndarray:
    """Per-block rung index from the lens rules (rules 1-6).

    [Lens] "The mechanism" and [FoQLens] "FoQZones, the mechanism":

    1. radius R_i = r_i f / (1 - f)
    2. ceiling kappa = gamma + floor(g (m - gamma))
    3. profile stops s_kappa < ... < s_(gamma+1)
    4. lift rho_i(b) = d(b, c_i) / R_i, L_i(b) = max(0, 1 - rho_i(b) / s_last)
    5. combine L(b) = min(1, sum_i L_i) or max_i L_i
    6. level: rho* = s_last (1 - L(b)); the ring rho* falls into; outside
       every lens, G.

    Readings taken where the pages are open: the distance d(a, b) is
    Euclidean on the 2-D block coordinates; s_last is s_(gamma+1), the last
    stop listed; rings are half-open, so a rho* exactly on a stop falls to
    the lower level and the level is gamma + #{j : rho* < s_(gamma+j)}; a
    lens of radius 0 lifts only a block at distance 0 (rho = 0) and leaves
    every other block at rho = +inf.

    All arithmetic is fp64, elementwise, in the order written (no fused
    multiply-add); numpy's sqrt and division are correctly rounded.

    With ``radius='zone'`` rule 1 is the zone form R = f D of [FoQLens]
    "FoQZones, the mechanism" (``width`` = D, see ``field_width``) for every
    centre, the per-lens r_i unused; rules 2-6 are the same.

    Parameters: ``coords`` [n_blocks, 2] fp64; ``centres`` [n_lenses, 2];
    ``radii`` [n_lenses] (the per-lens r_i); ``combine`` 'sum' or 'max';
    ``n_rungs`` = m + 1 (ladder length, rung 0 = ZERO); ``glass`` = gamma.
    Returns uint8 rung indices [n_blocks].
    """
    coords = np.asarray(coords, dtype=np.float64).reshape(-1, 2)
    centres = np.asarray(centres, dtype=np.float64).reshape(-1, 2)
    radii = np.asarray(radii, dtype=np.float64).reshape(-1)
    if combine not in ("sum", "max"):
        raise ValueError("combine must be 'sum' or 'max'")
    m = n_rungs - 1
    if not (0 <= glass <= m):
        raise ValueError("glass must be a rung index")
    if not (0.0 <= f <= 1.0 and 0.0 <= g <= 1.0):
        raise ValueError("f and g must lie in [0, 1]")
    nb = coords.shape[0]
    kappa = ceiling(g, m, glass)
    n = kappa - glass
    if n == 0 or centres.shape[0] == 0:
        return np.full(nb, glass, dtype=np.uint8)
    s = profile_stops(n, stops)
    s_last = s[0]
    if radius == "lens":
        R = lens_radius(radii, f)
    elif radius == "zone":
        R = np.full(centres.shape[0], zone_radius(f, width))
    else:
        raise ValueError("radius must be 'lens' or 'zone'")
    acc = np.zeros(nb, dtype=np.float64)
    for i in range(centres.shape[0]):
        dx = coords[:, 0] - centres[i, 0]
        dy = coords[:, 1] - centres[i, 1]
        dist = np.sqrt(dx * dx + dy * dy)
        if R[i] == 0.0:
            rho = np.where(dist == 0.0, 0.0, np.inf)
        else:
            rho = dist / R[i]
        lift = np.maximum(np.float64(0.0), np.float64(1.0) - rho / s_last)
        if combine == "sum":
            acc = acc + lift
        else:
            acc = np.maximum(acc, lift)
    L = np.minimum(np.float64(1.0), acc) if combine == "sum" else acc
    rho_star = s_last * (np.float64(1.0) - L)
    count = np.zeros(nb, dtype=np.int64)
    for j in range(n):
        count += (rho_star < s[j]).astype(np.int64)
    return (glass + count).astype(np.uint8)


# --------------------------------------------------------------------------
# Memory: rule 7 and the bytes-read cost
# --------------------------------------------------------------------------

def mean_bits(level, block_weights, ladder_bits=LADDER_BITS) -> float:
    """Rule 7 ([Lens] / [FoQLens]): bits = sum_b w_b bits(b) / sum_b w_b (fp64)."""
    level = np.asarray(level).astype(np.int64)
    w = np.asarray(block_weights).astype(np.float64)
    bits = np.asarray(ladder_bits, dtype=np.float64)[level]
    return float(np.sum(w * bits) / np.sum(w))


def weight_bytes(level, block_weights, ladder_bits=LADDER_BITS) -> int:
    """Weight bytes read for one pass: sum_b w_b bits(b) / 8 ([PoD]: cost is
    counted in weight bytes read per token).  Exact integer."""
    level = np.asarray(level).astype(np.int64)
    w = np.asarray(block_weights).astype(np.int64)
    bits = np.asarray(ladder_bits, dtype=np.int64)[level]
    total_bits = int(np.sum(w * bits))
    if total_bits % 8:
        raise ValueError("weight bits are not a whole number of bytes")
    return total_bits // 8


# --------------------------------------------------------------------------
# The mixed-depth matrix-vector / matrix product
# --------------------------------------------------------------------------

def _block_codes(W, level, ladder_bits):
    """Per-row truncated codes (int64) for a [N, K] int8 matrix."""
    W = np.asarray(W)
    N = W.shape[0]
    if N % ROWS_PER_BLOCK:
        raise ValueError("N must be a multiple of 64")
    level = np.asarray(level).astype(np.int64)
    out = np.empty(W.shape, dtype=np.int64)
    for b in range(N // ROWS_PER_BLOCK):
        rows = slice(b * ROWS_PER_BLOCK, (b + 1) * ROWS_PER_BLOCK)
        out[rows] = truncate(W[rows], ladder_bits[int(level[b])])
    return out


def qmatvec_ref(W, scales, x, level, ladder_bits=LADDER_BITS, per_request=False):
    """y[r, n] = scale[n] * sum_k c[n, k] x[r, k] in fp64.

    [FoQLens] "Progress": each block of 64 rows is read to its own depth from
    the stored bytes inside the pass; c is the row's code truncated to its
    block's depth (``truncate``); a ZERO block reads nothing and gives 0.
    ``level`` is [n_blocks] (shared by every request) or, with
    ``per_request``, [B, n_blocks].  ``x`` is [B, K] (or [K]).
    Returns fp64 [B, N].  Blocks are processed one at a time so memory stays
    bounded; each uses one fp64 matrix product.
    """
    W = np.asarray(W)
    N, K = W.shape
    x = np.asarray(x, dtype=np.float64).reshape(-1, K)
    B = x.shape[0]
    sc = np.asarray(scales, dtype=np.float64).reshape(N)
    level = np.asarray(level).astype(np.int64)
    if per_request:
        level = level.reshape(B, N // ROWS_PER_BLOCK)
    else:
        level = np.broadcast_to(level.reshape(1, -1), (B, N // ROWS_PER_BLOCK))
    y = np.zeros((B, N), dtype=np.float64)
    for b in range(N // ROWS_PER_BLOCK):
        rows = slice(b * ROWS_PER_BLOCK, (b + 1) * ROWS_PER_BLOCK)
        for d_idx in np.unique(level[:, b]):
            reqs = np.nonzero(level[:, b] == d_idx)[0]
            d = ladder_bits[int(d_idx)]
            if d == 0:
                continue
            c = truncate(W[rows], d).astype(np.float64)
            y[np.ix_(reqs, np.arange(rows.start, rows.stop))] = (x[reqs] @ c.T) * sc[rows]
    return y


def qmatvec_tolerance(W, scales, x, level, ladder_bits=LADDER_BITS, per_request=False,
                      rel=1e-4):
    """Per-output bound rel * sum_k |scale[n] c[n, k]| |x[r, k]| (fp64, [B, N]).

    The accuracy contract for fp32 outputs: |y - y_ref| <= 1e-4 sum|w||x| per
    row, with w = scale * c taken at the block's read depth (so a ZERO block
    must give exactly 0).
    """
    W = np.asarray(W)
    N, K = W.shape
    x = np.abs(np.asarray(x, dtype=np.float64).reshape(-1, K))
    B = x.shape[0]
    sc = np.abs(np.asarray(scales, dtype=np.float64).reshape(N))
    level = np.asarray(level).astype(np.int64)
    if per_request:
        level = level.reshape(B, N // ROWS_PER_BLOCK)
    else:
        level = np.broadcast_to(level.reshape(1, -1), (B, N // ROWS_PER_BLOCK))
    t = np.zeros((B, N), dtype=np.float64)
    for b in range(N // ROWS_PER_BLOCK):
        rows = slice(b * ROWS_PER_BLOCK, (b + 1) * ROWS_PER_BLOCK)
        for d_idx in np.unique(level[:, b]):
            reqs = np.nonzero(level[:, b] == d_idx)[0]
            d = ladder_bits[int(d_idx)]
            if d == 0:
                continue
            c = np.abs(truncate(W[rows], d)).astype(np.float64)
            t[np.ix_(reqs, np.arange(rows.start, rows.stop))] = (x[reqs] @ c.T) * sc[rows]
    return rel * t


def fit_focus_area(coords, centres, radii, g: float, combine: str, n_rungs: int, glass: int,
                   block_weights, budget_bytes: int, iters: int = 40, ladder_bits=LADDER_BITS, stops=None,
                   radius: str = "lens", width=None):
    """The byte-budget regulator: the largest focus area f in [0, 1] whose
    lens map reads at most ``budget_bytes`` of weights.

    [Lens] "The mechanism": memory is what the lenses cost (rule 7, bytes
    sum_b w_b bits(b) / 8), and focus_area is the control that widens every
    lens.  The pages set no budget rule; the reading taken: bytes never
    decrease as f grows (a wider lens lifts no block less), so f is found by
    bisection on [0, 1], ``iters`` halvings, keeping the end that fits.  If
    f = 1 fits, f = 1; if not even f = 0 fits, f = 0 (and the returned
    bytes exceed the budget).  Exact integers decide every step.  The same
    holds for zones, R = f D ([FoQLens] "FoQZones, the mechanism": the
    budget sets the zone radius), with ``radius='zone'`` and ``width`` = D.

    Returns (f, bytes at f, level map at f).
    """
    def at(f):
        lv = level_map(coords, centres, radii, f, g, combine, n_rungs, glass, stops, radius, width)
        return weight_bytes(lv, block_weights, ladder_bits), lv

    b1, lv1 = at(1.0)
    if b1 <= budget_bytes:
        return 1.0, b1, lv1
    b0, lv0 = at(0.0)
    if b0 > budget_bytes:
        return 0.0, b0, lv0
    lo, hi = 0.0, 1.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        b, _ = at(mid)
        if b <= budget_bytes:
            lo = mid
        else:
            hi = mid
    b, lv = at(lo)
    return lo, b, lv


# --------------------------------------------------------------------------
# Layer decides: per-block levels from the layer's own base read
# --------------------------------------------------------------------------

def layer_scores(y_base, scales, K: int) -> np.ndarray:
    """Reduced draft scores, one per (request, block): fp64 [B, n_blocks].

    [FoQLens] "FoQZones, the mechanism", the variant in which the layer
    decides: the "draft" score of a unit is the squared norm of its output
    read at the base depth times the square of its quantisation step,
    s_c = |y_c(base)|^2 Delta_c^2, and the reduced score divides in the
    step once more and the block's weights, s^_c = s_c Delta_c^2 / w_c.

    Readings where the page is open: the unit c is a block of 64 output
    rows; y_c(base) are its 64 outputs of the product at the base depth;
    Delta_c^2 is the mean over the block's rows of the squared row scale
    (the step of the stored 8-bit codes); w_c is the number of weights in
    the block, 64 K.  Sums run over the block's rows in order, in fp64
    (squares of fp32 values are exact there), and the reduced score is
    ((|y_c|^2 Delta_c^2) Delta_c^2) / w_c, evaluated left to right.
    """
    y = np.asarray(y_base, dtype=np.float32).astype(np.float64)
    y = y.reshape(-1, y.shape[-1])
    B, N = y.shape
    if N % ROWS_PER_BLOCK:
        raise ValueError("N must be a multiple of 64")
    nb = N // ROWS_PER_BLOCK
    sc = np.asarray(scales, dtype=np.float32).astype(np.float64).reshape(nb, ROWS_PER_BLOCK)
    yb = y.reshape(B, nb, ROWS_PER_BLOCK)
    energy = np.zeros((B, nb))
    step2 = np.zeros(nb)
    for i in range(ROWS_PER_BLOCK):          # row by row, in order
        energy = energy + yb[:, :, i] * yb[:, :, i]
        step2 = step2 + sc[:, i] * sc[:, i]
    step2 = step2 / ROWS_PER_BLOCK
    w = np.float64(ROWS_PER_BLOCK * K)
    draft = energy * step2[None, :]
    return (draft * step2[None, :]) / w


def layer_levels_threshold(shat, n_rungs: int, glass: int, g: float, lam: float) -> np.ndarray:
    """Rung per block from its reduced score: uint8, the shape of ``shat``.

    [FoQLens] "FoQZones, the mechanism", layer-decides variant:
    level = gamma + #{j >= 1 : s^ >= lambda 16^j}, capped at the ceiling
    kappa = gamma + floor(g (m - gamma)) (``ceiling``), m = n_rungs - 1.
    The page leaves lambda open: it is the caller's parameter.  With the
    cap, j runs over 1 .. kappa - gamma; 16^j is exact in fp64.  A NaN score
    meets no threshold and stays at the glass.
    """
    shat = np.asarray(shat, dtype=np.float64)
    kappa = ceiling(g, n_rungs - 1, glass)
    level = np.full(shat.shape, glass, dtype=np.int64)
    for j in range(1, kappa - glass + 1):
        level = level + (shat >= np.float64(lam) * np.float64(16.0 ** j))
    return level.astype(np.uint8)


def layer_levels_share(shat, n_rungs: int, glass: int, g: float, share: float) -> np.ndarray:
    """Rung per block by share: uint8, the shape of ``shat`` ([B, n_blocks]).

    [FoQLens] "FoQZones, the mechanism", layer-decides variant, "by share":
    the top f of the layer by reduced score rise and the rest stays at the
    base.  Readings: per request, the floor(f n_blocks) blocks of largest
    score rise to the ceiling kappa (``ceiling``); equal scores are ordered
    by block index, the lower first; a NaN score ranks below every number
    and never rises.
    """
    shat = np.asarray(shat, dtype=np.float64)
    sh = shat.reshape(-1, shat.shape[-1])
    B, nb = sh.shape
    kappa = ceiling(g, n_rungs - 1, glass)
    k = int(np.floor(np.float64(share) * np.float64(nb)))
    level = np.full((B, nb), glass, dtype=np.uint8)
    for r in range(B):
        numbers = [c for c in range(nb) if not np.isnan(sh[r, c])]
        order = sorted(numbers, key=lambda c: (-sh[r, c], c))
        for c in order[:k]:
            level[r, c] = kappa
    return level.reshape(shat.shape)


# --------------------------------------------------------------------------
# Escalation: top-4-bit decode with a gated 8-bit re-run
# --------------------------------------------------------------------------

def escalation_schedule(scores, rate: float) -> np.ndarray:
    """Which steps are re-run at 8 bits ([PoD] abstract).

    The pass reads every block at 4 bits; a step is redone at 8 bits when its
    low-precision output looks uncertain.  Reading taken for a fixed rate:
    escalate exactly ``round(rate * T)`` steps, those with the largest
    uncertainty score (ties to the earlier step).  Returns a bool mask [T].
    """
    scores = np.asarray(scores, dtype=np.float64).reshape(-1)
    T = scores.shape[0]
    n_esc = int(np.floor(rate * T + 0.5))
    order = sorted(range(T), key=lambda t: (-scores[t], t))
    mask = np.zeros(T, dtype=bool)
    mask[order[:n_esc]] = True
    return mask


def uncertainty(logits):
    """Entropy and top-two margin of the low pass's output distribution
    ([PoD] abstract: a step is redone at 8 bits when the low-precision output
    distribution looks uncertain, entropy above a threshold or a small
    top-two margin).

    Readings taken where the abstract is open: the distribution is the
    softmax of the logits, p_i = exp(z_i) / sum_j exp(z_j), evaluated in fp64
    as exp(z_i - max z) / sum; the entropy is in nats, H = -sum_i p_i ln p_i
    with 0 ln 0 = 0 (a logit of -inf is a token of probability 0); the
    margin is between the two largest probabilities, p_(1) - p_(2), the top
    two taken by value, ties to the lower index.  Logits holding a NaN or a
    +inf, or all -inf, give no distribution: entropy and margin are NaN.

    Returns dict(entropy, margin, top1, top2, p1, p2).
    """
    z = np.asarray(logits, dtype=np.float64).reshape(-1)
    V = z.shape[0]
    if V < 2:
        raise ValueError("need at least two logits")
    order = np.lexsort((np.arange(V), -z))         # by value, descending; ties to the lower index
    top1, top2 = int(order[0]), int(order[1])
    if np.any(np.isnan(z)) or np.any(z == np.inf) or np.all(z == -np.inf):
        nan = float("nan")
        return dict(entropy=nan, margin=nan, top1=top1, top2=top2, p1=nan, p2=nan)
    m = z.max()
    e = np.exp(z - m)
    p = e / np.sum(e)
    plogp = np.zeros(V)
    nz = p > 0.0
    plogp[nz] = p[nz] * np.log(p[nz])
    H = -np.sum(plogp)
    return dict(entropy=float(H), margin=float(p[top1] - p[top2]), top1=top1, top2=top2,
                p1=float(p[top1]), p2=float(p[top2]))


def gate(logits, tau_entropy: float, tau_margin: float) -> bool:
    """The escalation gate ([PoD] abstract): redo the step when the entropy
    exceeds ``tau_entropy`` or the top-two margin falls below ``tau_margin``
    (+inf / -inf switch either test off).  No distribution (NaN) escalates."""
    u = uncertainty(logits)
    H, mg = u["entropy"], u["margin"]
    if np.isnan(H):
        return True
    return bool(H > tau_entropy or mg < tau_margin)


def escalation_byte_ratio(mask, low_bits: int = 4, high_bits: int = 8) -> float:
    """Weight bytes read by the gated schedule over the all-high schedule.

    Every step reads all weights at ``low_bits``; an escalated step reads them
    again at ``high_bits`` ([PoD]: cost counted in weight bytes read per
    token).  For a uniform map the ratio is
    (T low + n_esc high) / (T high).
    """
    mask = np.asarray(mask, dtype=bool)
    T = mask.shape[0]
    return float((T * low_bits + int(mask.sum()) * high_bits) / (T * high_bits))


def speculative_decode(draft_next, target_next, first_token: int, n_tokens: int, k: int):
    """Greedy draft-and-verify decoding ([PoD] abstract: speculation verified
    at 8 bits reaches the 8-bit output at similar bytes).

    Readings taken where the abstract is open: greedy decoding; a step's next
    token depends on the current token alone (``draft_next(t)`` and
    ``target_next(t)`` give the draft's and the target's next token after
    ``t``).  A round drafts ``k`` tokens with the draft, d_1 = draft(cur),
    d_i = draft(d_{i-1}); the target gives t_0 = target(cur) and
    t_i = target(d_i) (in the method one batched pass over the k + 1
    inputs); the round keeps d_1 .. d_j for the longest run with
    t_{i-1} = d_i, then emits t_j.  The emitted sequence is the target's
    greedy sequence whatever the draft does.

    Returns (the first ``n_tokens`` emitted tokens, stats) with stats
    rounds, draft_steps, drafted, accepted, emitted (the last round's surplus
    counted in ``emitted`` but not returned).
    """
    if k < 1:
        raise ValueError("k must be at least 1")
    out = []
    st = dict(rounds=0, draft_steps=0, drafted=0, accepted=0, emitted=0)
    cur = int(first_token)
    while len(out) < n_tokens:
        drafts = []
        t = cur
        for _ in range(k):
            t = int(draft_next(t))
            drafts.append(t)
        targets = [int(target_next(x)) for x in [cur] + drafts]
        j = 0
        while j < k and targets[j] == drafts[j]:
            j += 1
        emitted = drafts[:j] + [targets[j]]
        out.extend(emitted)
        cur = emitted[-1]
        st["rounds"] += 1
        st["draft_steps"] += k
        st["drafted"] += k
        st["accepted"] += j
        st["emitted"] += j + 1
    return out[:n_tokens], st


def speculation_byte_ratio(stats, n_tokens: int, draft_bits: int = 4, verify_bits: int = 8) -> float:
    """Weight bytes per emitted token over those of one full-depth step.

    Each draft step reads every weight at ``draft_bits``, each verify pass
    reads every weight once at ``verify_bits`` for all its positions
    ([PoD]: cost counted in weight bytes read per token).  Per token:
    (draft_steps draft_bits + rounds verify_bits) / (n_tokens verify_bits).
    """
    return float((stats["draft_steps"] * draft_bits + stats["rounds"] * verify_bits) / (n_tokens * verify_bits))


# --------------------------------------------------------------------------
# Glue around the chained decode step (shape stand-ins, not the method)
# --------------------------------------------------------------------------

def rmsnorm_ref(x, eps: float = 1e-6) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) per row, fp64, no learned weight."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def silu_mul_ref(gate, up) -> np.ndarray:
    """silu(gate) * up = gate / (1 + exp(-gate)) * up, fp64."""
    gate = np.asarray(gate, dtype=np.float64)
    up = np.asarray(up, dtype=np.float64)
    return gate / (1.0 + np.exp(-gate)) * up
