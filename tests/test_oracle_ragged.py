"""Pins of the oracle's per-expert maximum width (ragged plane counts;
MatMoE review, Core Contribution: each expert's maximum bit-width is chosen
offline, 2/3/4 bits).  Closed forms from the encoder's own codes, the F&C
table of a 3-bit store written by hand, and the reduction to the uniform
bank when every expert stores 4 planes."""
import numpy as np
import pytest

from dynamic_any_precision_amd import workloads as wl
import oracle as orc


@pytest.fixture(scope="module")
def ragged():
    return wl.make_ragged_workload(wl.config(1, ragged=True))


def test_widths_and_prefix(ragged):
    b = ragged.routed
    widths = np.diff(b.plane_prefix)
    assert set(widths.tolist()) <= {2, 3, 4} and len(set(widths.tolist())) > 1
    assert b.w13_planes.shape[0] == widths.sum() == b.w2_planes.shape[0]


def test_ragged_unpack_equals_encoder_codes(ragged):
    b = ragged.routed
    cache = orc.ragged_bank_cache(b)
    for e in range(b.n_experts):
        Be = cache.b_of(e)
        q13, s13, z13, q2, s2, z2 = cache.codes(e)
        assert np.array_equal(q13, b.q13[e]) and np.array_equal(q2, b.q2[e])
        assert q13.max() < (1 << Be) and q2.max() < (1 << Be)


def test_full_read_is_full_dequant_at_the_expert_width(ragged):
    b = ragged.routed
    cache = orc.ragged_bank_cache(b)
    g = b.g
    for e in range(b.n_experts):
        Be = cache.b_of(e)
        w13, _ = cache.weights(e, Be)
        s, z = orc.unpack_scale_zero(b.w13_sz[e:e + 1], 2 * b.f, b.d // g)
        ref = (b.q13[e].astype(np.float64) - np.repeat(z[0], g, -1)) * np.repeat(s[0], g, -1)
        assert np.array_equal(w13, ref)
        # wider requests read the stored width
        assert np.array_equal(cache.weights(e, 4)[0], w13)


def test_fc_relative_to_a_three_bit_store():
    # codes 0..7 of a 3-bit store: width 2 keeps 2 bits (2 floor(q/2) + 0.5),
    # width 1 keeps 1 bit (4 floor(q/4) + 1.5); written out by hand
    w2 = [0.5, 0.5, 2.5, 2.5, 4.5, 4.5, 6.5, 6.5]
    w1 = [1.5, 1.5, 1.5, 1.5, 5.5, 5.5, 5.5, 5.5]
    q = np.arange(8)
    assert orc.fc_codes(q, 2, 3).tolist() == w2
    assert orc.fc_codes(q, 1, 3).tolist() == w1
    assert orc.fc_codes(q, 3, 3).tolist() == q.tolist()


def test_uniform_widths_reduce_to_the_uniform_bank():
    cfg = wl.config(1)
    uni = wl.make_workload(cfg)
    rag = wl.make_ragged_workload(wl.config(1, ragged=True), widths=np.full(cfg.E, 4))
    assert np.array_equal(rag.x_bf16, uni.x_bf16) and np.array_equal(rag.w_router, uni.w_router)
    idx, gate, _, _ = orc.route(uni.x_bf16, uni.w_router, None, cfg.k)
    bits, _, _ = orc.allocate_bits(gate, 2, 4, 3.0)
    y_u = orc.combine(uni.x_bf16, idx, gate, bits, orc.bank_cache(uni.routed))
    y_r = orc.combine(rag.x_bf16, idx, gate, bits, orc.ragged_bank_cache(rag.routed))
    assert np.array_equal(y_u, y_r)


def test_pairs_wider_than_their_expert_read_its_width(ragged):
    cfg = ragged.cfg
    b = ragged.routed
    cache = orc.ragged_bank_cache(b)
    idx, gate, _, _ = orc.route(ragged.x_bf16, ragged.w_router, None, cfg.k)
    widths = np.diff(b.plane_prefix)
    full = np.full(cfg.P, 4)
    clamped = np.minimum(full, widths[idx.ravel()])
    assert np.array_equal(orc.combine(ragged.x_bf16, idx, gate, full, cache),
                          orc.combine(ragged.x_bf16, idx, gate, clamped, cache))
