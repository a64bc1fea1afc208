"""Host-side tests of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments with the documented status before touching
the GPU (so these run on a machine without one)."""
import ctypes

import numpy as np
import pytest

from dynamic_any_precision_amd import binding as bd
import oracle as orc

OK, NULL, SHAPE, ALIGN, RANGE, WS, UNSUP = 0, 1, 2, 3, 4, 5, 6


@pytest.fixture(scope="module")
def L():
    return bd.lib()


def test_library_exports_every_header_symbol(L):
    names = bd.header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in range(8):
        assert L.moe_status_string(s)


def _bank(**kw):
    base = dict(n_experts=8, d_model=256, d_ff=128, group=64, b_max=4,
                w13_planes=16, w13_sz=16, w2_planes=16, w2_sz=16)
    base.update(kw)
    return bd.ExpertBankC(**base)


def test_route_validation(L):
    fake = 256
    ws_ok = L.moe_route_workspace_bytes(4, 8)
    assert ws_ok > 0
    args = lambda **kw: dict(dict(x=fake, T=4, d=256, w=fake, E=8, bias=None, k=2, renorm=0, idx=fake,
                                  gate=fake, ws=fake, wsb=ws_ok, s=None), **kw)

    def call(**kw):
        a = args(**kw)
        return L.moe_route(a["x"], a["T"], a["d"], a["w"], a["E"], a["bias"], a["k"], a["renorm"], a["idx"],
                           a["gate"], a["ws"], a["wsb"], a["s"])
    assert call(T=0) == OK
    assert call(E=0) == RANGE
    assert call(E=300) == RANGE
    assert call(k=9, E=16) == RANGE
    assert call(k=3, E=2) == RANGE
    assert call(d=200) == SHAPE
    assert call(x=None) == NULL
    assert call(ws=None) == NULL
    assert call(x=fake + 2) == ALIGN
    assert call(wsb=ws_ok - 1) == WS


def test_alloc_validation_and_budget(L):
    assert L.moe_alloc_bits(None, 0, 2, 4, 3.0, None, None, None, None) == OK
    assert L.moe_alloc_bits(256, 8, 2, 4, 1.5, 256, None, None, None) == RANGE
    assert L.moe_alloc_bits(256, 8, 2, 4, 4.5, 256, None, None, None) == RANGE
    assert L.moe_alloc_bits(256, 8, 3, 2, 2.5, 256, None, None, None) == RANGE
    assert L.moe_alloc_bits(256, 8, 0, 4, 2.5, 256, None, None, None) == RANGE
    assert L.moe_alloc_bits(None, 8, 2, 4, 3.0, 256, None, None, None) == NULL
    assert L.moe_alloc_bits(256, 8, 2, 4, float("nan"), 256, None, None, None) == RANGE


@pytest.mark.parametrize("b_lo", [1, 2, 3])
def test_budget_matches_oracle_exact_rationals(L, b_lo):
    rng = np.random.default_rng(b_lo)
    for _ in range(400):
        P = int(rng.integers(1, 40000))
        t = float(np.float32(rng.uniform(b_lo, 4)))
        assert L.moe_budget_pairs(P, b_lo, 4, t) == orc.n_star(P, b_lo, 4, t), (P, t)
    for P in (1, 8, 96, 256, 512, 32768):
        for t in np.arange(b_lo, 4.0001, 0.25):
            assert L.moe_budget_pairs(P, b_lo, 4, float(t)) == orc.n_star(P, b_lo, 4, float(t))


def test_ffn_validation(L):
    fake = 256
    ws = L.moe_ffn_workspace_bytes(ctypes.byref(_bank()), None, 16, 2)
    assert ws > 0

    def call(bank=None, shared=None, T=16, k=2, x=fake, y=fake, wsp=fake, wsb=ws):
        b = _bank() if bank is None else bank
        return L.moe_anyprec_ffn(ctypes.byref(b), None if shared is None else ctypes.byref(shared), x, T, k,
                                 fake, fake, fake, y, 0, wsp, wsb, None)
    assert call(T=0) == OK
    assert call(bank=_bank(group=32)) == UNSUP
    assert call(bank=_bank(d_model=200)) == SHAPE
    assert call(bank=_bank(b_max=5)) == RANGE
    assert call(bank=_bank(w13_planes=None)) == NULL
    assert call(bank=_bank(w2_sz=fake + 4)) == ALIGN
    assert call(k=9) == RANGE
    assert call(x=None) == NULL
    assert call(x=fake + 2) == ALIGN
    assert call(wsp=fake + 16) == ALIGN
    assert call(wsb=ws - 1) == WS
    assert call(shared=_bank(n_experts=2, d_model=512)) == SHAPE
    assert call(shared=_bank(n_experts=2, b_max=3)) == SHAPE
    assert L.moe_ffn_workspace_bytes(ctypes.byref(_bank(group=32)), None, 16, 2) == 0


def test_workspace_grows_with_tokens(L):
    a = L.moe_ffn_workspace_bytes(ctypes.byref(_bank()), None, 16, 2)
    b = L.moe_ffn_workspace_bytes(ctypes.byref(_bank()), None, 64, 2)
    c = L.moe_ffn_workspace_bytes(ctypes.byref(_bank()), ctypes.byref(_bank(n_experts=2)), 64, 2)
    assert 0 < a < b < c


def test_other_entry_points_validate(L):
    fake = 256
    assert L.moe_dequant(ctypes.byref(_bank()), 8, 0, 4, fake, None) == RANGE
    assert L.moe_dequant(ctypes.byref(_bank()), 0, 2, 4, fake, None) == RANGE
    assert L.moe_dequant(ctypes.byref(_bank()), 0, 0, 0, fake, None) == RANGE
    assert L.moe_dequant(ctypes.byref(_bank()), 0, 0, 4, None, None) == NULL
    assert L.moe_residual_to_bf16(None, None, 0, None) == OK
    assert L.moe_residual_to_bf16(None, fake, 4, None) == NULL
    assert L.moe_residual_to_bf16(fake, fake, -1, None) == RANGE
    assert L.moe_bits_from_threshold(None, 0, 0.5, 2, 4, None, None) == OK
    assert L.moe_bits_from_threshold(fake, 4, 0.5, 2, 4, None, None) == NULL
    assert L.moe_bits_from_threshold(fake, -1, 0.5, 2, 4, fake, None) == RANGE
    assert L.moe_bits_from_threshold(fake, 4, float("nan"), 2, 4, fake, None) == RANGE
    assert L.moe_bits_from_threshold(fake, 4, 0.5, 3, 2, fake, None) == RANGE
    assert L.moe_bits_from_threshold(fake, 4, 0.5, 2, 5, fake, None) == RANGE
    assert L.moe_bits_from_threshold(fake, 4, 0.5, 0, 4, fake, None) == RANGE
    assert L.moe_rmsnorm_to_bf16(None, None, 0, 2048, 1e-6, None) == OK
    assert L.moe_rmsnorm_to_bf16(None, fake, 4, 2048, 1e-6, None) == NULL
    assert L.moe_rmsnorm_to_bf16(fake, fake, -1, 2048, 1e-6, None) == RANGE
    assert L.moe_rmsnorm_to_bf16(fake, fake, 4, 0, 1e-6, None) == RANGE
    assert L.moe_rmsnorm_to_bf16(fake, fake, 4, 2048, -1.0, None) == RANGE
    assert L.moe_rmsnorm_to_bf16(fake, fake, 4, 2048, float("nan"), None) == RANGE
    assert L.moe_rmsnorm_to_bf16(fake, fake, 4, 2048, float("inf"), None) == RANGE


def test_stream_read_validation(L):
    fake = 256
    assert L.moe_stream_read(None, 0, None, None) == OK
    assert L.moe_stream_read(fake, 24, fake, None) == RANGE
    assert L.moe_stream_read(fake, -16, fake, None) == RANGE
    assert L.moe_stream_read(None, 16, fake, None) == NULL
    assert L.moe_stream_read(fake, 16, None, None) == NULL
    assert L.moe_stream_read(fake + 8, 16, fake, None) == ALIGN
    assert L.moe_permute(fake, fake, 0, 2, 8, 4, fake, fake, fake, fake, 1 << 20, None) == OK
    assert L.moe_permute(fake, fake, 4, 2, 8, 5, fake, fake, fake, fake, 1 << 20, None) == RANGE
    assert L.moe_permute(fake, fake, 4, 2, 8, 4, fake, fake, fake, fake + 1, 1 << 20, None) == ALIGN
    assert L.moe_permute(fake, fake, 4, 2, 8, 4, fake, fake, fake, fake, 16, None) == WS


def test_layer_validation(L):
    fake = 256
    b = _bank()
    args = lambda **kw: [ctypes.byref(kw.get("bank", b)), None, kw.get("x", fake), kw.get("T", 4), kw.get("k", 2),
                         kw.get("wr", fake), None, 0, kw.get("b_lo", 2), kw.get("tgt", 3.0), fake, fake, fake,
                         kw.get("y", fake), 0, kw.get("ws", fake), kw.get("wsb", 1 << 30), None]
    assert L.moe_layer(*args(T=0)) == OK
    assert L.moe_layer(*args(x=None)) == NULL
    assert L.moe_layer(*args(wr=None)) == NULL
    assert L.moe_layer(*args(b_lo=0)) == RANGE
    assert L.moe_layer(*args(tgt=4.5)) == RANGE
    assert L.moe_layer(*args(tgt=1.5)) == RANGE
    assert L.moe_layer(*args(k=9)) == RANGE
    assert L.moe_layer(*args(ws=fake + 16)) == ALIGN
    need = L.moe_layer_workspace_bytes(ctypes.byref(b), None, 4, 2)
    assert need > L.moe_ffn_workspace_bytes(ctypes.byref(b), None, 4, 2)
    assert L.moe_layer(*args(wsb=need - 1)) == WS
