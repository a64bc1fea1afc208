"""Seeded synthetic workloads and the offline checkpoint encoder.

This module is the one piece shared by the CPU oracle's tests and the GPU
path: it draws every random input (router weights, activations, expert
weights) from numbered NumPy streams and encodes expert weights into the
stored bitplane checkpoint.  It contains no step of the layer computation
(no dequantisation, routing, allocation or FFN arithmetic).

Encoding follows the storage idea of the MatMoE review (Core Contribution:
bitplane storage, shared quantisation parameters valid at every prefix) and
the DPA-MoE abstract (prefix-decodable chunks, one encoded checkpoint for all
budgets).  The learned quantiser of those pages is out of reach without
trained weights; round-to-nearest min-max per group stands in for it.

Storage layout of one matrix of one expert, N rows x K columns, B planes
(plane 0 = most significant bit of the unsigned code q):

* planes: uint32 words, plane-major, so the first b planes of a matrix are one
  contiguous prefix.  Inside a plane the rows are cut into 16-row tiles; a
  tile holds 16 * K/32 words.  Columns are cut into 128-column "k-blocks",
  each split into four 32-column chunks j = 0..3.  The word holding row
  n = 16*tile + r, k-block kb, chunk j sits at

      tile * (16*K/32) + 64*kb + (16*j + r),

  and bit i of that word is column 128*kb + 32*j + i.  A 64-lane wave reads
  one k-block of one tile as 256 contiguous bytes, lane 16*j + r holding the
  32 columns that lane needs for the matrix-core operand.
* scale/zero: float32 laid out [N/16][K/g][2][16] per expert (tile, quant
  group, {scale, zero}, row in tile): the 16 scales of a tile's quant group
  are contiguous, followed by the 16 zero points.
"""
from __future__ import annotations

import dataclasses
from fractions import Fraction
from typing import Optional

import numpy as np

# Order in which SeedSequence(seed).spawn streams are assigned.
STREAMS = ("router", "x", "w13", "w2", "shared", "lognorm", "perm", "steps")


@dataclasses.dataclass(frozen=True)
class MoeConfig:
    name: str
    d: int                 # hidden size (K of gate/up, N of down)
    f: int                 # expert intermediate size
    E: int                 # routed experts
    k: int                 # experts per token
    T: int                 # tokens in the batch
    g: int = 128           # quantisation group along K
    b_max: int = 4         # stored planes
    b_lo: int = 2          # low read width
    target: float = 3.0    # target average bits over routed pairs
    seed: int = 0
    router_lognorm: float = 0.0   # sigma of per-row LogNormal router scaling (0 = off)
    zipf_bias: bool = False       # Zipf(1.1)-skewed expert load via a logit bias
    n_shared: int = 0             # always-on shared experts (read at b_max)
    f_shared: int = 0
    renorm_topk: bool = False
    ragged: bool = False          # per-expert maximum width B_e in {2, 3, 4} (ragged plane counts)

    @property
    def P(self) -> int:
        return self.T * self.k


def config(i: int, **overrides) -> MoeConfig:
    """The five workloads: 1 tiny, 2 Qwen3-30B-A3B-shaped decode,
    3 DeepSeekMoE-16B-shaped decode, 4 Qwen-shaped prefill, 5 layer of the
    48-layer Qwen-shaped stack."""
    base = {
        1: dict(name="tiny", d=256, f=128, E=8, k=2, T=16, g=64, b_lo=2, target=3.0, seed=0),
        2: dict(name="qwen3-30b-a3b-decode", d=2048, f=768, E=128, k=8, T=32, g=128,
                b_lo=2, target=3.0, seed=1, router_lognorm=0.5),
        3: dict(name="deepseekmoe-16b-decode", d=2048, f=1408, E=64, k=6, T=16, g=128,
                b_lo=2, target=2.5, seed=2, n_shared=2, f_shared=1408),
        4: dict(name="qwen3-30b-a3b-prefill", d=2048, f=768, E=128, k=8, T=4096, g=128,
                b_lo=2, target=3.0, seed=3, router_lognorm=0.5, zipf_bias=True),
        5: dict(name="qwen3-30b-a3b-stack48", d=2048, f=768, E=128, k=8, T=64, g=128,
                b_lo=2, target=3.0, seed=4, router_lognorm=0.5),
    }[i]
    base.update(overrides)
    return MoeConfig(**base)


# ---------------------------------------------------------------------------
# bf16 helpers (input conversion only)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# offline encoder


def quantize_rtn(w: np.ndarray, g: int, b_max: int):
    """Round-to-nearest min-max quantiser per group of g along the last axis.

    Returns q (uint8, [.., N, K]), scale and zero (float32, [.., N, K/g]);
    zero is integer-valued in [0, 2^b_max - 1]."""
    w = np.asarray(w, dtype=np.float32)
    *lead, N, K = w.shape
    assert K % g == 0
    levels = (1 << b_max) - 1
    wg = w.reshape(*lead, N, K // g, g)
    mn = wg.min(axis=-1)
    mx = wg.max(axis=-1)
    s = ((mx - mn) / np.float32(levels)).astype(np.float32)
    s = np.where(s > 0, s, np.float32(1e-8)).astype(np.float32)
    z = np.clip(np.rint(-mn / s), 0, levels).astype(np.float32)
    q = np.clip(np.rint(wg / s[..., None]) + z[..., None], 0, levels).astype(np.uint8)
    return q.reshape(*lead, N, K), s, z


def pack_planes(q: np.ndarray, b_max: int) -> np.ndarray:
    """Encode codes q [E, N, K] into the tiled MSB-first bitplane words
    [E, b_max, N/16 * 16*K/32] (uint32)."""
    q = np.asarray(q, dtype=np.uint8)
    E, N, K = q.shape
    assert N % 16 == 0 and K % 128 == 0
    nkb = K // 128
    tiles = N // 16
    out = np.empty((E, b_max, tiles * 16 * K // 32), dtype=np.uint32)
    for p in range(b_max):
        bits = ((q >> (b_max - 1 - p)) & 1).astype(np.uint8)          # [E, N, K]
        bits = bits.reshape(E, tiles, 16, nkb, 4, 32)                   # [E, tiles, r, kb, j, i]
        words = np.packbits(bits, axis=-1, bitorder="little")          # [E, tiles, r, kb, j, 4 bytes]
        words = np.ascontiguousarray(words).view("<u4")[..., 0]         # [E, tiles, r, kb, j]
        words = words.transpose(0, 1, 3, 4, 2)                          # [E, tiles, kb, j, r]
        out[:, p] = words.reshape(E, -1)
    return out


def pack_scale_zero(s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """[E, N, K/g] scale and zero -> float32 [E, N/16, K/g, 2, 16]."""
    E, N, G = s.shape
    sz = np.stack([s, z], axis=0).astype(np.float32)                   # [2,E,N,G]
    sz = sz.reshape(2, E, N // 16, 16, G).transpose(1, 2, 4, 0, 3)      # [E,tiles,G,2,16]
    return np.ascontiguousarray(sz)


@dataclasses.dataclass
class ExpertBank:
    """Encoded bank of experts (numpy, host).  W13 rows 0..f-1 are the gate
    projection, rows f..2f-1 the up projection; W2 is the down projection."""
    n_experts: int
    d: int
    f: int
    g: int
    b_max: int
    w13_planes: np.ndarray   # uint32 [E, b_max, words]
    w13_sz: np.ndarray       # float32 [E, 2f/16, d/g, 2, 16]
    w2_planes: np.ndarray    # uint32 [E, b_max, words]
    w2_sz: np.ndarray        # float32 [E, d/16, f/g, 2, 16]
    # codes kept for tests that need the encoder's own view
    q13: Optional[np.ndarray] = None
    q2: Optional[np.ndarray] = None
    s13: Optional[np.ndarray] = None
    z13: Optional[np.ndarray] = None
    s2: Optional[np.ndarray] = None
    z2: Optional[np.ndarray] = None

    def stored_bytes(self) -> int:
        return (self.w13_planes.nbytes + self.w13_sz.nbytes
                + self.w2_planes.nbytes + self.w2_sz.nbytes)


def encode_bank(w13: np.ndarray, w2: np.ndarray, g: int, b_max: int,
                keep_codes: bool = True) -> ExpertBank:
    E, twof, d = w13.shape
    f = twof // 2
    q13, s13, z13 = quantize_rtn(w13, g, b_max)
    q2, s2, z2 = quantize_rtn(w2, g, b_max)
    bank = ExpertBank(E, d, f, g, b_max,
                      pack_planes(q13, b_max), pack_scale_zero(s13, z13),
                      pack_planes(q2, b_max), pack_scale_zero(s2, z2))
    if keep_codes:
        bank.q13, bank.q2, bank.s13, bank.z13, bank.s2, bank.z2 = q13, q2, s13, z13, s2, z2
    return bank


# ---------------------------------------------------------------------------
# workload generation


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return dict(zip(STREAMS, (np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(len(STREAMS)))))


def _gen_bank(rng: np.random.Generator, E: int, d: int, f: int, g: int, b_max: int,
              keep_codes: bool, which: str) -> tuple:
    """Draw N(0, 0.02) weights one expert at a time and quantise them."""
    out_q, out_s, out_z = [], [], []
    for _ in range(E):
        if which == "w13":
            w = rng.standard_normal((2 * f, d), dtype=np.float32) * np.float32(0.02)
        else:
            w = rng.standard_normal((d, f), dtype=np.float32) * np.float32(0.02)
        q, s, z = quantize_rtn(w, g, b_max)
        out_q.append(q); out_s.append(s); out_z.append(z)
    return np.stack(out_q), np.stack(out_s), np.stack(out_z)


@dataclasses.dataclass
class Workload:
    cfg: MoeConfig
    x_bf16: np.ndarray            # uint16 [T, d]
    w_router: np.ndarray          # float32 [E, d]
    logit_bias: Optional[np.ndarray]  # float32 [E] or None
    routed: ExpertBank
    shared: Optional[ExpertBank]

    def x_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.x_bf16)


def make_workload(cfg: MoeConfig, keep_codes: bool = True, T: Optional[int] = None,
                  n_experts_drawn: Optional[int] = None) -> Workload:
    """Build the seeded synthetic layer of `cfg`.

    n_experts_drawn < E draws only that many distinct experts and repeats them
    cyclically to fill the bank (used to keep very large banks cheap to build
    where only byte volume matters); None draws every expert."""
    T = cfg.T if T is None else T
    st = _streams(cfg.seed)
    d, f, E = cfg.d, cfg.f, cfg.E
    w_router = st["router"].standard_normal((E, d), dtype=np.float32) * np.float32(0.02)
    if cfg.router_lognorm > 0:
        rowscale = np.exp(st["lognorm"].normal(0.0, cfg.router_lognorm, size=E)).astype(np.float32)
        w_router = (w_router * rowscale[:, None]).astype(np.float32)
    x = f32_to_bf16_bits(st["x"].standard_normal((T, d), dtype=np.float32))
    logit_bias = None
    if cfg.zipf_bias:
        ranks = np.arange(1, E + 1, dtype=np.float64)
        p = ranks ** -1.1
        p /= p.sum()
        perm = st["perm"].permutation(E)
        logit_bias = (0.6 * np.log(p[perm])).astype(np.float32)
    nd = E if n_experts_drawn is None else min(E, n_experts_drawn)
    q13, s13, z13 = _gen_bank(st["w13"], nd, d, f, cfg.g, cfg.b_max, keep_codes, "w13")
    q2, s2, z2 = _gen_bank(st["w2"], nd, d, f, cfg.g, cfg.b_max, keep_codes, "w2")
    if nd < E:
        rep = np.arange(E) % nd
        q13, s13, z13, q2, s2, z2 = (a[rep] for a in (q13, s13, z13, q2, s2, z2))
    routed = ExpertBank(E, d, f, cfg.g, cfg.b_max,
                        pack_planes(q13, cfg.b_max), pack_scale_zero(s13, z13),
                        pack_planes(q2, cfg.b_max), pack_scale_zero(s2, z2))
    if keep_codes:
        routed.q13, routed.q2, routed.s13, routed.z13, routed.s2, routed.z2 = q13, q2, s13, z13, s2, z2
    shared = None
    if cfg.n_shared:
        fs = cfg.f_shared
        sq13, ss13, sz13 = _gen_bank(st["shared"], cfg.n_shared, d, fs, cfg.g, cfg.b_max, keep_codes, "w13")
        sq2, ss2, sz2 = _gen_bank(st["shared"], cfg.n_shared, d, fs, cfg.g, cfg.b_max, keep_codes, "w2")
        shared = ExpertBank(cfg.n_shared, d, fs, cfg.g, cfg.b_max,
                            pack_planes(sq13, cfg.b_max), pack_scale_zero(ss13, sz13),
                            pack_planes(sq2, cfg.b_max), pack_scale_zero(ss2, sz2))
        if keep_codes:
            shared.q13, shared.q2, shared.s13, shared.z13, shared.s2, shared.z2 = sq13, sq2, ss13, sz13, ss2, sz2
    return Workload(cfg, x, w_router, logit_bias, routed, shared)


@dataclasses.dataclass
class RaggedBank:
    """Encoded bank whose expert e stores its own number of planes B_e
    (plane_prefix[e+1] - plane_prefix[e]): the planes of every expert are one
    array of planes (uint32 [sum B_e, words]), expert e's in rows
    plane_prefix[e] .. plane_prefix[e+1]-1, its codes B_e-bit and its
    (scale, zero) those of B_e-bit quantisation; b_max is the largest B_e."""
    n_experts: int
    d: int
    f: int
    g: int
    b_max: int
    plane_prefix: np.ndarray  # int32 [E+1]
    w13_planes: np.ndarray    # uint32 [sum B_e, 2f/16 * 16 d/32]
    w13_sz: np.ndarray        # float32 [E, 2f/16, d/g, 2, 16]
    w2_planes: np.ndarray     # uint32 [sum B_e, d/16 * 16 f/32]
    w2_sz: np.ndarray         # float32 [E, d/16, f/g, 2, 16]
    q13: Optional[list] = None
    q2: Optional[list] = None

    def stored_bytes(self) -> int:
        return (self.w13_planes.nbytes + self.w13_sz.nbytes + self.w2_planes.nbytes + self.w2_sz.nbytes)


def expert_max_widths(cfg: MoeConfig) -> np.ndarray:
    """Seeded per-expert maximum widths B_e in {2, 3, 4} (a quarter at 2,
    a third at 3, the rest at 4), standing in for the offline choice under a
    memory budget (stream SeedSequence([seed, 77]))."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 77])))
    u = rng.random(cfg.E)
    return np.where(u < 0.25, 2, np.where(u < 0.25 + 1 / 3, 3, 4)).astype(np.int32)


def make_ragged_workload(cfg: MoeConfig, keep_codes: bool = True, widths: Optional[np.ndarray] = None) -> Workload:
    """The workload of `cfg` with a ragged routed bank: the same seeded
    weights as make_workload, expert e quantised to B_e bits
    (expert_max_widths, or `widths`) and stored as B_e planes."""
    st = _streams(cfg.seed)
    d, f, E, g = cfg.d, cfg.f, cfg.E, cfg.g
    # router and activations exactly as make_workload draws them
    w_router = st["router"].standard_normal((E, d), dtype=np.float32) * np.float32(0.02)
    if cfg.router_lognorm > 0:
        rowscale = np.exp(st["lognorm"].normal(0.0, cfg.router_lognorm, size=E)).astype(np.float32)
        w_router = (w_router * rowscale[:, None]).astype(np.float32)
    x = f32_to_bf16_bits(st["x"].standard_normal((cfg.T, d), dtype=np.float32))
    widths = expert_max_widths(cfg) if widths is None else np.asarray(widths, dtype=np.int32)
    p13, p2, s13l, s2l, q13l, q2l = [], [], [], [], [], []
    # redraw the same N(0, 0.02) weights expert by expert (streams w13 and w2 in order)
    for e in range(E):
        w13 = st["w13"].standard_normal((2 * f, d), dtype=np.float32) * np.float32(0.02)
        q, s_, z = quantize_rtn(w13, g, int(widths[e]))
        p13.append(pack_planes(q[None], int(widths[e]))[0])
        s13l.append((s_, z))
        if keep_codes:
            q13l.append(q)
    for e in range(E):
        w2 = st["w2"].standard_normal((d, f), dtype=np.float32) * np.float32(0.02)
        q, s_, z = quantize_rtn(w2, g, int(widths[e]))
        p2.append(pack_planes(q[None], int(widths[e]))[0])
        s2l.append((s_, z))
        if keep_codes:
            q2l.append(q)
    prefix = np.concatenate([[0], np.cumsum(widths)]).astype(np.int32)
    sz13 = pack_scale_zero(np.stack([a for a, _ in s13l]), np.stack([b for _, b in s13l]))
    sz2 = pack_scale_zero(np.stack([a for a, _ in s2l]), np.stack([b for _, b in s2l]))
    bank = RaggedBank(E, d, f, g, int(widths.max()), prefix, np.ascontiguousarray(np.concatenate(p13)), sz13,
                      np.ascontiguousarray(np.concatenate(p2)), sz2)
    if keep_codes:
        bank.q13, bank.q2 = q13l, q2l
    return Workload(cfg, x, w_router, None, bank, None)


def step_activations(cfg: MoeConfig, step: int, T: Optional[int] = None) -> np.ndarray:
    """Fresh bf16 activations for decode step `step` (stream [seed, 1000+step])."""
    T = cfg.T if T is None else T
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 1000 + step])))
    return f32_to_bf16_bits(rng.standard_normal((T, cfg.d), dtype=np.float32))


def target_as_fraction(target: float) -> Fraction:
    """The float32 value of a target average bit-width, as an exact rational."""
    return Fraction(float(np.float32(target)))


# ---------------------------------------------------------------------------
# stack layer (48-layer workload): codes drawn uniformly, group parameters
# drawn to the statistics of round-to-nearest on N(0, 0.02) groups of 128.


def make_stack_layer(cfg: MoeConfig, layer: int) -> tuple:
    """Returns (w_router, routed bank) for layer `layer` of the stack.

    Drawing and quantising 600M Gaussian weights per layer on the host is too
    slow for 48 layers, so codes are drawn uniformly over [0, 2^b_max) as raw
    plane bits and (scale, zero) per group are drawn around the values RTN
    gives for N(0, 0.02) groups of 128 (range ~ 0.02 * 5.2, zero ~ 7.5)."""
    ss = np.random.SeedSequence([cfg.seed, layer])
    c = ss.spawn(4)
    rr, rp, rs, rl = (np.random.Generator(np.random.PCG64(x)) for x in c)
    d, f, E, g, B = cfg.d, cfg.f, cfg.E, cfg.g, cfg.b_max
    w_router = rr.standard_normal((E, d), dtype=np.float32) * np.float32(0.02)
    if cfg.router_lognorm > 0:
        rowscale = np.exp(rl.normal(0.0, cfg.router_lognorm, size=E)).astype(np.float32)
        w_router = (w_router * rowscale[:, None]).astype(np.float32)

    def planes(N, K):
        return rp.integers(0, 1 << 32, size=(E, B, N * K // 32), dtype=np.uint32)

    def sz(N, K):
        G = K // g
        s = (np.float32(0.02 * 5.2 / 15) * (1 + 0.1 * rs.standard_normal((E, N // 16, G, 16)))).astype(np.float32)
        z = rs.integers(6, 10, size=(E, N // 16, G, 16)).astype(np.float32)
        return np.ascontiguousarray(np.stack([s, z], axis=3))

    bank = ExpertBank(E, d, f, g, B, planes(2 * f, d), sz(2 * f, d), planes(d, f), sz(d, f))
    return w_router, bank
