"""CPU oracle for the dynamic any-precision MoE FFN layer (float64, NumPy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library or its
Python binding and imports nothing from them.

Each function states the plain definition it computes and the passage of the
pages it follows.  Pages, by title:
  [DPA]  "DPA-MoE: A Runtime Precision Control Framework for MoE Inference"
         (abstract; news summary "DPA-MoE enables dynamic precision routing
         for expert selection").
  [DUO]  "DuoRate: Two-Rate Per-Expert Precision Allocation for
         Mixture-of-Experts Serving" (abstract).
  [MAT]  "MatMoE: Matryoshka Mixture-of-Experts with Dynamic Mixed-Precision
         Quantization for Efficient Inference" (abstract and the review's
         sections Core Contribution, Methodological Rigor, Strengths,
         Limitations).

Readings taken where the pages are silent are listed next to the function
that takes them.  Parity status: every function here is pinned by tests
under tests/ (closed forms, brute force, library special cases); none is
"parity unpinned".
"""
from __future__ import annotations

from fractions import Fraction
import math

import numpy as np

# ---------------------------------------------------------------------------
# stored checkpoint -> integer codes


def plane_word_and_bit(n, c, N: int, K: int):
    """Position of the bit of (row n, column c) inside one plane of an N x K
    matrix: (word index within the plane, bit index within the word).

    Layout (the stored format; [MAT] Core Contribution, bitplane storage):
    rows in tiles of 16, columns in 128-column blocks of four 32-column
    chunks; within a tile, block-major, then chunk, then row.  Works
    elementwise on NumPy integer arrays."""
    tile = n // 16
    r = n % 16
    kb = c // 128
    j = (c % 128) // 32
    bit = c % 32
    word = tile * (16 * K // 32) + 64 * kb + 16 * j + r
    return word, bit


def unpack_codes(planes: np.ndarray, b_max: int, N: int, K: int) -> np.ndarray:
    """Unsigned codes q[e, n, c] = sum_p bit_p * 2^(b_max-1-p), plane 0 being
    the most significant bit ([MAT] Core Contribution: bitplane storage;
    [DPA] prefix-decodable chunks).  planes: uint32 [E, b_max, words]."""
    planes = np.asarray(planes)
    E = planes.shape[0]
    n = np.arange(N)[:, None]
    c = np.arange(K)[None, :]
    word, bit = plane_word_and_bit(n, c, N, K)
    q = np.zeros((E, N, K), dtype=np.int64)
    for p in range(b_max):
        w = planes[:, p, :].astype(np.int64)[:, word]          # [E, N, K]
        q += ((w >> bit) & 1) << (b_max - 1 - p)
    return q


def unpack_scale_zero(sz: np.ndarray, N: int, G: int):
    """sz float32 [E, N/16, G, 2, 16] (tile, quant group, {scale, zero}, row
    in tile) -> (scale, zero) float64 [E, N, G]."""
    sz = np.asarray(sz, dtype=np.float64).reshape(-1, N // 16, G, 2, 16)
    E = sz.shape[0]
    scale = np.empty((E, N, G))
    zero = np.empty((E, N, G))
    for n in range(N):
        scale[:, n, :] = sz[:, n // 16, :, 0, n % 16]
        zero[:, n, :] = sz[:, n // 16, :, 1, n % 16]
    return scale, zero


# ---------------------------------------------------------------------------
# floor-and-compensation dequantisation


def fc_constant(delta: int) -> float:
    """Compensation added after dropping `delta` low bits: (2^delta - 1)/2, the
    mean of a residual uniform on {0, ..., 2^delta - 1} ([MAT] Core
    Contribution, floor-and-compensation paragraph; the constant is printed
    there without its opening parenthesis)."""
    return (2.0 ** delta - 1.0) / 2.0


def fc_codes(q: np.ndarray, b: int, b_max: int) -> np.ndarray:
    """Code read from the first b planes with F&C: keep the top b bits of q
    (floor of q / 2^delta), put them back in place and add the compensation
    ([MAT] abstract item (2) and Core Contribution, F&C paragraph)."""
    delta = b_max - b
    qb = np.asarray(q, dtype=np.int64) >> delta
    return (qb << delta).astype(np.float64) + fc_constant(delta)


def floor_codes(q: np.ndarray, b: int, b_max: int) -> np.ndarray:
    """Negative control: truncation without compensation (the plain floor that
    the MatMoE review, Methodological Rigor, reports as collapsing)."""
    delta = b_max - b
    return ((np.asarray(q, dtype=np.int64) >> delta) << delta).astype(np.float64)


def dequant(q: np.ndarray, scale: np.ndarray, zero: np.ndarray, b: int, b_max: int,
            g: int, compensate: bool = True) -> np.ndarray:
    """w_hat = (code_b - z) * s, with (s, z) of group floor(c/g) of the row,
    shared by every read width ([DPA] SharedScale; [MAT] Core Contribution,
    shared quantisation parameters).  q [.., N, K]; scale, zero [.., N, K/g].
    Exact in float64 (code_b - z is a multiple of 1/2 below 16 in size)."""
    codes = fc_codes(q, b, b_max) if compensate else floor_codes(q, b, b_max)
    s = np.repeat(np.asarray(scale, dtype=np.float64), g, axis=-1)
    z = np.repeat(np.asarray(zero, dtype=np.float64), g, axis=-1)
    return (codes - z) * s


# ---------------------------------------------------------------------------
# router


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def router_logits(x_bf16: np.ndarray, w_router: np.ndarray, logit_bias=None) -> np.ndarray:
    """l[t, e] = sum_i W_r[e, i] x[t, i] (+ bias_e), float64 ([DPA] abstract:
    routing each token to a small set of experts; [MAT] routing scores)."""
    x = bf16_to_f64(x_bf16)
    l = x @ np.asarray(w_router, dtype=np.float64).T
    if logit_bias is not None:
        l = l + np.asarray(logit_bias, dtype=np.float64)[None, :]
    return l


def softmax(l: np.ndarray) -> np.ndarray:
    """p = exp(l - max) / sum exp(l - max) along the expert axis."""
    m = l.max(axis=-1, keepdims=True)
    e = np.exp(l - m)
    return e / e.sum(axis=-1, keepdims=True)


def topk(l: np.ndarray, k: int):
    """Top-k experts per token ordered by (logit descending, index ascending).
    Returns idx [T, k] and the gap l_(k) - l_(k+1) per token (inf if k == E),
    used to flag near-ties."""
    T, E = l.shape
    idx = np.empty((T, k), dtype=np.int64)
    gap = np.full(T, np.inf)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-l[t, e], e))
        idx[t] = order[:k]
        if k < E:
            gap[t] = l[t, order[k - 1]] - l[t, order[k]]
    return idx, gap


def route(x_bf16, w_router, logit_bias, k: int, renorm: bool = False):
    """Gate scores of the chosen experts: softmax over all experts, then the
    top k; renormalised over the k only if asked (reading: the pages say
    "gate scores"/"routing score" without fixing renormalisation)."""
    l = router_logits(x_bf16, w_router, logit_bias)
    p = softmax(l)
    idx, gap = topk(l, k)
    gate = np.take_along_axis(p, idx, axis=1)
    if renorm:
        gate = gate / gate.sum(axis=1, keepdims=True)
    return idx, gate, gap, l


# ---------------------------------------------------------------------------
# bit allocation


def n_star(P: int, b_lo: int, b_max: int, target) -> int:
    """Budget in high-precision pairs: floor(P (b* - B_lo) / (B_max - B_lo)),
    exact rational arithmetic on the float32 value of b*, clamped to [0, P]
    (reading: the budget is never exceeded)."""
    t = Fraction(float(np.float32(target)))
    if b_max == b_lo:
        return 0
    v = Fraction(P) * (t - b_lo) / (b_max - b_lo)
    return max(0, min(P, math.floor(v)))


def allocate_bits(gates: np.ndarray, b_lo: int, b_max: int, target):
    """Threshold allocation over the live routed pairs of the batch ([MAT]
    abstract item (3); Core Contribution: pairs whose routing score exceeds a
    threshold run at high precision, the rest low, the threshold set to hit a
    target average bit-width; [DPA] post-routing allocation from live gate
    scores).

    Plain definition by sorting: with scores sorted s_(1) >= ... >= s_(P),
    start from n = n*, and while 0 < n < P and s_(n) == s_(n+1) step n down
    (a threshold can not split equal scores).  The n highest pairs read B_max,
    the rest B_lo.  Returns (bits [P] int, n, n*)."""
    g = np.asarray(gates, dtype=np.float64).ravel()
    P = g.size
    ns = n_star(P, b_lo, b_max, target)
    s = np.sort(g)[::-1]
    n = ns
    while 0 < n < P and s[n - 1] == s[n]:
        n -= 1
    bits = np.full(P, b_lo, dtype=np.int64)
    if n == P:
        bits[:] = b_max
    elif n > 0:
        bits[g > s[n]] = b_max
    return bits, n, ns


def threshold_interval(gates: np.ndarray, n: int):
    """The thresholds tau with #{g > tau} == n form [s_(n+1), s_(n)); returns
    that half-open interval (None for an open end)."""
    s = np.sort(np.asarray(gates, dtype=np.float64).ravel())[::-1]
    P = s.size
    lo = s[n] if n < P else None
    hi = s[n - 1] if n > 0 else None
    return lo, hi


def calibrate_threshold(calib_gates: np.ndarray, b_lo: int, b_max: int, target) -> float:
    """Threshold set on a calibration set of routing scores ([MAT] Core
    Contribution: the threshold is calibrated on a score distribution to hit
    the target average bit-width; Methodological Rigor: the average is met in
    expectation).  Plain definition: the allocation rule of allocate_bits on
    the calibration scores gives n high pairs; the threshold is the lowest
    value whose strict upper set is those n, i.e. s_(n+1) of the sorted
    scores (-inf when n is every score)."""
    g = np.asarray(calib_gates, dtype=np.float64).ravel()
    _, n, _ = allocate_bits(g, b_lo, b_max, target)
    s = np.sort(g)[::-1]
    return float(s[n]) if n < g.size else -math.inf


def bits_from_threshold(gates: np.ndarray, tau: float, b_lo: int, b_max: int) -> np.ndarray:
    """Widths from a fixed threshold: B_max where the score exceeds tau
    (strictly, R8), B_lo elsewhere ([MAT] Core Contribution)."""
    g = np.asarray(gates, dtype=np.float64).ravel()
    return np.where(g > tau, b_max, b_lo).astype(np.int64)


# ---------------------------------------------------------------------------
# expert FFN


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits),
    ties to even."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.round(m * 256.0), e - 8)


def rmsnorm_bf16(h: np.ndarray, eps: float) -> np.ndarray:
    """Layer input of the residual stack from the fp32 residual h [T][d]:
    each row scaled by r = fp32(1 / sqrt(mean of its squares + eps)), the
    product rounded to fp32, then to bf16 (returned as float64 values).

    Not from the pages: they define one MoE layer, not a stack.  Reading: a
    48-layer stack of these SwiGLU layers carries its residual through a
    root-mean-square normalisation before each layer, as the Qwen3-MoE
    models the stack is shaped after do (unit weight, eps 1e-6); without it
    the residual overflows fp32 within a few layers.  The mean of squares is
    taken in float64 (each square of an fp32 value is exact there)."""
    h = np.asarray(h, dtype=np.float32)
    ms = np.sum(h.astype(np.float64) ** 2, axis=-1) / h.shape[-1] + float(eps)
    r = (1.0 / np.sqrt(ms)).astype(np.float32)
    return round_bf16((h * r[..., None]).astype(np.float32))


def silu(v: np.ndarray) -> np.ndarray:
    return v / (1.0 + np.exp(-v))


def expert_ffn(x: np.ndarray, w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """SwiGLU expert: g = W_gate x, u = W_up x, h = silu(g) u rounded to
    bfloat16 (reading: activations between the projections are bf16, as the
    layer's inputs are), o = W_down h.  w13 [2f, d] (gate rows first), w2 [d, f]."""
    f = w13.shape[0] // 2
    gu = w13 @ x
    h = round_bf16(silu(gu[:f]) * gu[f:])
    return w2 @ h


class DequantCache:
    """Dequantised matrices of one bank, computed on demand per (expert, bits)."""

    def __init__(self, planes13, sz13, planes2, sz2, d: int, f: int, g: int, b_max: int):
        self.p13, self.sz13, self.p2, self.sz2 = planes13, sz13, planes2, sz2
        self.d, self.f, self.g, self.b_max = d, f, g, b_max
        self._q = {}
        self._w = {}

    def codes(self, e: int):
        if e not in self._q:
            d, f, g, B = self.d, self.f, self.g, self.b_max
            q13 = unpack_codes(self.p13[e:e + 1], B, 2 * f, d)[0]
            q2 = unpack_codes(self.p2[e:e + 1], B, d, f)[0]
            s13, z13 = unpack_scale_zero(self.sz13[e:e + 1], 2 * f, d // g)
            s2, z2 = unpack_scale_zero(self.sz2[e:e + 1], d, f // g)
            self._q[e] = (q13, s13[0], z13[0], q2, s2[0], z2[0])
        return self._q[e]

    def weights(self, e: int, b: int):
        key = (e, b)
        if key not in self._w:
            q13, s13, z13, q2, s2, z2 = self.codes(e)
            self._w[key] = (dequant(q13, s13, z13, b, self.b_max, self.g),
                            dequant(q2, s2, z2, b, self.b_max, self.g))
        return self._w[key]


def bank_cache(bank) -> DequantCache:
    return DequantCache(bank.w13_planes, bank.w13_sz, bank.w2_planes, bank.w2_sz,
                        bank.d, bank.f, bank.g, bank.b_max)


def combine(x_bf16, idx, gate, bits, routed: DequantCache, shared: DequantCache = None,
            n_shared: int = 0, tokens=None) -> np.ndarray:
    """y[t] = sum_j gate[t, j] * FFN_{idx[t, j]}^(bits[t, j])(x_t)
    + sum_s FFN_shared_s^(b_max)(x_t); float64.  `tokens` restricts the
    rows computed (others stay zero)."""
    x = bf16_to_f64(x_bf16)
    T, k = idx.shape
    d = x.shape[1]
    bits = np.asarray(bits).reshape(T, k)
    y = np.zeros((T, d))
    rows = range(T) if tokens is None else tokens
    for t in rows:
        for j in range(k):
            w13, w2 = routed.weights(int(idx[t, j]), int(bits[t, j]))
            y[t] += gate[t, j] * expert_ffn(x[t], w13, w2)
        for s in range(n_shared):
            w13, w2 = shared.weights(s, shared.b_max)
            y[t] += expert_ffn(x[t], w13, w2)
    return y


def layer(x_bf16, w_router, logit_bias, k: int, b_lo: int, b_max: int, target,
          routed: DequantCache, shared: DequantCache = None, n_shared: int = 0,
          renorm: bool = False, tokens=None) -> dict:
    """One full layer step: route, allocate, per-pair FFN, combine."""
    idx, gate, gap, logits = route(x_bf16, w_router, logit_bias, k, renorm)
    bits, n, ns = allocate_bits(gate, b_lo, b_max, target)
    y = combine(x_bf16, idx, gate, bits, routed, shared, n_shared, tokens)
    return dict(idx=idx, gate=gate, gap=gap, logits=logits, bits=bits, n_hi=n, n_star=ns, y=y)


# ---------------------------------------------------------------------------
# DuoRate: per-expert read widths from a baked distortion tensor, a
# label-free prefill profile and a Lagrangian rate-distortion solve under the
# decode rate ([DUO] abstract).


def distortion_tensor(cache: DequantCache, experts=None) -> np.ndarray:
    """The baked distortion tensor: Delta[e, b-1, c] = sum over the rows n of
    the gate/up matrix W13 of (W_hat^(B)[n, c] - W_hat^(b)[n, c])^2, the
    squared change of input column c's weights when expert e is read at b
    planes instead of the stored uniform tier of B planes ([DUO] abstract:
    one uniform stored tier of a prefix-readable stream, a baked distortion
    tensor).  Reading: the stored tier is the reference (the checkpoint holds
    no other weights), and the tensor covers the expert's input projection,
    whose input is the layer input a prefill can profile.  float64
    [E, B, d]; rows of width B are zero."""
    E = cache.p13.shape[0]
    experts = range(E) if experts is None else experts
    B = cache.b_max
    out = np.zeros((E, B, cache.d))
    for e in experts:
        full = cache.weights(e, B)[0]
        for b in range(1, B + 1):
            diff = full - cache.weights(e, b)[0]
            out[e, b - 1] = np.sum(diff * diff, axis=0)
    return out


def prefill_profile(x_bf16: np.ndarray, idx: np.ndarray, E: int):
    """Label-free workload profile of a prefill batch ([DUO] abstract: it
    profiles the workload's own prefill without labels): per expert the
    number of routed pairs n[e] and the summed input energy
    a[e, c] = sum over pairs (t, j) with idx[t, j] = e of x[t, c]^2."""
    x = bf16_to_f64(x_bf16)
    idx = np.asarray(idx)
    a = np.zeros((E, x.shape[1]))
    n = np.zeros(E, dtype=np.int64)
    for t in range(idx.shape[0]):
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            a[e] += x[t] * x[t]
            n[e] += 1
    return a, n


def expert_distortion(delta: np.ndarray, a: np.ndarray, n: np.ndarray) -> np.ndarray:
    """Per-token distortion of expert e read at b planes on this workload:
    Dbar[e, b-1] = <Delta[e, b-1], a[e]> / n[e] (one dot product per expert
    and width, [DUO] abstract), the expected squared error of the expert's
    gate/up pre-activations per routed token (diagonal approximation: input
    channels treated as uncorrelated).  0 for an expert the prefill never
    routes to."""
    E, B, _ = delta.shape
    D = np.zeros((E, B))
    for e in range(E):
        if n[e] > 0:
            for b in range(B):
                D[e, b] = float(np.dot(delta[e, b], a[e])) / float(n[e])
    return D


def rate_budget(n: np.ndarray, target) -> int:
    """Budget of the decode rate in summed bits: floor(b* x sum_e n_e), exact
    on the float32 value of the target."""
    N = int(np.sum(n))
    return math.floor(Fraction(float(np.float32(target))) * N)


def lagrangian_widths(D: np.ndarray, lam: float, b_lo: int, b_max: int) -> np.ndarray:
    """Per-expert decision at multiplier lam: b_e = argmin over widths
    b in [b_lo, b_max] of Dbar[e, b-1] + lam * b, evaluated as
    fl(Dbar + fl(lam * b)) in float64, ties to the smaller width.  The
    routing frequency does not appear: in the decode functional
    sum_e p_e (Dbar_e(b_e) + lam b_e) it is a common factor of each
    expert's own terms ([DUO] abstract: it cancels from every per-expert
    decision)."""
    E = D.shape[0]
    out = np.empty(E, dtype=np.int64)
    for e in range(E):
        best, bw = None, b_lo
        for b in range(b_lo, b_max + 1):
            c = float(D[e, b - 1]) + float(lam) * float(b)
            if best is None or c < best:
                best, bw = c, b
        out[e] = bw
    return out


def duorate_widths(D: np.ndarray, n: np.ndarray, b_lo: int, b_max: int, target):
    """Lagrangian rate-distortion allocation under the decode functional
    ([DUO] abstract: solved by a bisection).  The decode rate of widths b_e
    is sum_e n_e b_e over sum_e n_e (bits read per routed pair, in
    expectation over the profiled routing).  lam* is the smallest
    non-negative float64 whose widths meet the budget, found by bisection
    over the bit patterns of non-negative doubles (monotone in value), with
    the upper end lam_hi = 2 max_e Dbar[e, b_lo - 1] + 1, where every expert
    takes b_lo.  Returns (widths [E], lam*)."""
    budget = rate_budget(n, target)
    n = np.asarray(n, dtype=np.int64)

    def rate_ok(lam):
        return int(np.sum(n * lagrangian_widths(D, lam, b_lo, b_max))) <= budget

    lam_hi = 2.0 * float(np.max(D[:, b_lo - 1])) + 1.0
    lo = 0
    hi = int(np.float64(lam_hi).view(np.uint64))
    while lo < hi:
        mid = (lo + hi) // 2
        if rate_ok(float(np.uint64(mid).view(np.float64))):
            hi = mid
        else:
            lo = mid + 1
    lam = float(np.uint64(lo).view(np.float64))
    return lagrangian_widths(D, lam, b_lo, b_max), lam


def pair_bits_from_expert_widths(idx: np.ndarray, widths: np.ndarray) -> np.ndarray:
    """Per-pair read widths of a decode batch: each pair reads its expert's
    DuoRate width, b[t, j] = widths[idx[t, j]]."""
    return np.asarray(widths)[np.asarray(idx)].ravel()


# ---------------------------------------------------------------------------
# DPA-MoE: residual-aware chunk allocation over more than two widths
# ([DPA] abstract: per-expert reconstruction residuals profiled offline;
# chunks allocated at inference time from live router gate scores).  The
# abstract gives no rule; the reading taken here is a proposal, stated in
# each function.


def expert_residuals(cache: DequantCache, experts=None) -> np.ndarray:
    """Offline per-expert reconstruction residual at every width:
    r[e, b-1] = ||W_hat^(B) - W_hat^(b)||_F^2 summed over both matrices of
    expert e (gate/up and down), the stored uniform tier being the reference
    (the checkpoint holds no other weights).  float64 [E, B]; r[:, B-1] = 0."""
    E = cache.p13.shape[0]
    experts = range(E) if experts is None else experts
    B = cache.b_max
    out = np.zeros((E, B))
    for e in experts:
        f13, f2 = cache.weights(e, B)
        for b in range(1, B + 1):
            w13, w2 = cache.weights(e, b)
            out[e, b - 1] = float(np.sum((f13 - w13) ** 2)) + float(np.sum((f2 - w2) ** 2))
    return out


def chunk_scores(gates: np.ndarray, idx: np.ndarray, resid: np.ndarray, b_lo: int, b_max: int) -> np.ndarray:
    """Score of reading chunk (plane) k of pair p, k = b_lo+1 .. b_max:
    float32(g_p^2 * (r[e, k-2] - r[e, k-1])), the gate-weighted residual
    the k-th plane removes (reading: a pair's output enters the layer output
    scaled by its gate, so its squared error is scaled by g^2).  The product
    is formed in float64 (g^2 of a float32 gate is exact there) and rounded
    once to float32.  Returns [P, b_max - b_lo]."""
    g = np.asarray(gates, dtype=np.float32).ravel().astype(np.float64)
    e = np.asarray(idx).ravel()
    P = g.size
    out = np.empty((P, b_max - b_lo), dtype=np.float32)
    for p in range(P):
        for k in range(b_lo + 1, b_max + 1):
            gain = float(resid[e[p], k - 2]) - float(resid[e[p], k - 1])
            out[p, k - b_lo - 1] = np.float32((g[p] * g[p]) * gain)
    return out


def chunk_budget(P: int, b_lo: int, target) -> int:
    """Extra planes beyond b_lo for P pairs: floor(P (b* - b_lo)), exact on
    the float32 value of the target, clamped at 0."""
    return max(0, math.floor(Fraction(P) * (Fraction(float(np.float32(target))) - b_lo)))


def dpa_allocate(gates: np.ndarray, idx: np.ndarray, resid: np.ndarray, b_lo: int, b_max: int, target):
    """Residual-aware allocation: every pair reads b_lo planes; the extra
    planes go to the candidate chunks of highest score, as many as the budget
    allows, never splitting equal scores (the rule of allocate_bits, applied
    to the P (b_max - b_lo) candidate chunks).  A pair's width is b_lo plus
    the number of its chunks chosen.  Plain definition by sorting.  Returns
    (bits [P], chunks chosen, budget)."""
    s = chunk_scores(gates, idx, resid, b_lo, b_max)
    P = s.shape[0]
    flat = s.astype(np.float64).ravel()
    budget = min(chunk_budget(P, b_lo, target), flat.size)
    srt = np.sort(flat)[::-1]
    n = budget
    while 0 < n < flat.size and srt[n - 1] == srt[n]:
        n -= 1
    if n == flat.size:
        chosen = np.ones_like(flat, dtype=bool)
    elif n == 0:
        chosen = np.zeros_like(flat, dtype=bool)
    else:
        chosen = flat > srt[n]
    bits = b_lo + chosen.reshape(s.shape).sum(axis=1)
    return bits.astype(np.int64), int(chosen.sum()), budget


# ---------------------------------------------------------------------------
# per-expert maximum width (ragged plane counts)


class RaggedDequantCache(DequantCache):
    """Dequantised matrices of a bank whose expert e stores its own number
    of planes B_e = prefix[e+1] - prefix[e] (MatMoE review, Core
    Contribution: each expert's maximum bit-width is chosen offline under a
    memory budget; the choice itself is not made here).  The planes of all
    experts are one array of planes, expert e's at rows prefix[e] ..
    prefix[e+1]-1; the codes of expert e are B_e-bit and its (s, z) belong to
    that precision.  A pair of width b reads min(b, B_e) planes (reading: an
    expert can not be read wider than it is stored), with floor and
    compensation relative to B_e."""

    def __init__(self, planes13, sz13, planes2, sz2, prefix, d: int, f: int, g: int):
        self.prefix = [int(v) for v in prefix]
        super().__init__(planes13, sz13, planes2, sz2, d, f, g, max(
            self.prefix[e + 1] - self.prefix[e] for e in range(len(self.prefix) - 1)))

    def b_of(self, e: int) -> int:
        return self.prefix[e + 1] - self.prefix[e]

    def codes(self, e: int):
        if e not in self._q:
            d, f, g = self.d, self.f, self.g
            Be = self.b_of(e)
            p0, p1 = self.prefix[e], self.prefix[e + 1]
            q13 = unpack_codes(np.asarray(self.p13)[None, p0:p1], Be, 2 * f, d)[0]
            q2 = unpack_codes(np.asarray(self.p2)[None, p0:p1], Be, d, f)[0]
            s13, z13 = unpack_scale_zero(self.sz13[e:e + 1], 2 * f, d // g)
            s2, z2 = unpack_scale_zero(self.sz2[e:e + 1], d, f // g)
            self._q[e] = (q13, s13[0], z13[0], q2, s2[0], z2[0])
        return self._q[e]

    def weights(self, e: int, b: int):
        Be = self.b_of(e)
        b = min(int(b), Be)
        key = (e, b)
        if key not in self._w:
            q13, s13, z13, q2, s2, z2 = self.codes(e)
            self._w[key] = (dequant(q13, s13, z13, b, Be, self.g), dequant(q2, s2, z2, b, Be, self.g))
        return self._w[key]


def ragged_bank_cache(bank) -> RaggedDequantCache:
    return RaggedDequantCache(bank.w13_planes, bank.w13_sz, bank.w2_planes, bank.w2_sz, bank.plane_prefix,
                              bank.d, bank.f, bank.g)
