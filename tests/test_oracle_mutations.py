"""Planted mistakes in the oracle (on the CPU only): each plausible slip must
make at least one pin fail, which shows the pins are sharp enough."""
import types

import numpy as np
import pytest

import oracle
import oracle.formats
import oracle.moe
import oracle.pack
import oracle.route
import pins


def _ns(**over):
    ns = types.SimpleNamespace(**{k: getattr(oracle, k) for k in dir(oracle) if not k.startswith("_")})
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


def _fails(pin, O):
    with pytest.raises(AssertionError):
        pin(O)


def test_wrong_e2m1_entry(monkeypatch):
    bad = oracle.E2M1_VALUES.copy()
    bad[5] = 2.5                                   # 3.0 mistyped
    _fails(pins.pin_e2m1_grid, _ns(E2M1_VALUES=bad))


def test_e4m3_wrong_bias():
    bad = np.array([oracle.e4m3_decode(c) * 2 for c in range(256)])
    _fails(pins.pin_e4m3_table, _ns(E4M3_VALUES=bad))


def test_e2m1_ties_away_from_zero(monkeypatch):
    def enc(x):
        x = np.asarray(x, np.float64)
        shape = x.shape
        x = x.reshape(-1)
        mags = np.float64([0, .5, 1, 1.5, 2, 3, 4, 6])
        d = np.abs(np.abs(x)[:, None] - mags[None])
        # last minimum instead of the even one: ties go up
        m = (d.shape[1] - 1 - np.argmin(d[:, ::-1], axis=1)).astype(np.uint8)
        return (m | (((x < 0) & (m != 0)).astype(np.uint8) << 3)).astype(np.uint8).reshape(shape)
    _fails(pins.pin_e2m1_encode, _ns(e2m1_encode=enc))
    monkeypatch.setattr(oracle.pack, "e2m1_encode", enc)
    _fails(pins.pin_quant_fixture, oracle)


def test_nibble_order_swapped(monkeypatch):
    real = oracle.pack.quantize

    def swapped(W):
        p = real(W)
        v = p.values
        p.values = ((v >> 4) | (v << 4)).astype(np.uint8)
        return p
    _fails(pins.pin_quant_fixture, _ns(quantize=swapped))


def test_scale_without_six(monkeypatch):
    monkeypatch.setattr(oracle.pack, "e4m3_encode",
                        lambda x: oracle.formats.e4m3_encode(np.asarray(x) * 6))
    _fails(pins.pin_quant_fixture, oracle)


def test_support_ties_to_higher_position():
    def sup(W):
        N, K = W.shape
        a = np.abs(W.astype(np.float32)).reshape(N, K // 8, 8)[:, :, ::-1]
        order = 7 - np.argsort(-a, axis=2, kind="stable")
        keep = np.zeros_like(a, dtype=bool)
        np.put_along_axis(keep, order[:, :, :4], True, axis=2)
        return keep.reshape(N, K)
    _fails(pins.pin_support_bruteforce, _ns(support=sup))


def test_route_unstable():
    def rt(ids, E):
        off, perm, inv = oracle.route(ids, E)
        ids = np.asarray(ids)
        perm = np.argsort(ids * (len(ids) + 1) - np.arange(len(ids)), kind="stable").astype(np.int32)
        inv = np.empty_like(perm)
        inv[perm] = np.arange(len(perm))
        return off, perm, inv
    _fails(pins.pin_route_bruteforce, _ns(route=rt))


def test_gemm_transposed_operand(monkeypatch):
    def gg(xr, off, weight_of):
        return oracle.grouped_gemm(xr, off, lambda e: weight_of(e)[:, ::-1])
    _fails(pins.pin_gemm_exact, _ns(grouped_gemm=gg))


def test_gemm_dropped_global_scale(monkeypatch):
    real = oracle.pack.decode
    monkeypatch.setattr(oracle.pack, "decode", lambda p, include_global=True: real(p, False))
    _fails(pins.pin_quant_fixture, _ns(decode=oracle.pack.decode))


def test_unpermute_weight_index():
    def up(y, inv, w, T, k):
        if w is None:
            return oracle.unpermute(y, inv, None, T, k)
        w = np.asarray(w).reshape(k, T).T.reshape(-1) if T != k else w[::-1]
        return oracle.unpermute(y, inv, w, T, k)
    _fails(pins.pin_unpermute, _ns(unpermute=up))


def test_swiglu_halves_swapped():
    def sw(y1):
        n2 = y1.shape[1] // 2
        return oracle.silu(y1[:, n2:]) * y1[:, :n2]
    _fails(pins.pin_swiglu, _ns(swiglu=sw))


def test_silu_sign():
    _fails(pins.pin_swiglu, _ns(silu=lambda x: np.asarray(x) / (1 + np.exp(np.asarray(x)))))


# ---------------------------------------------------------------- paired 4:8

import oracle.paired  # noqa: E402


def test_paired_pattern_order(monkeypatch):
    # (0,3) and (1,2) numbered the other way round
    monkeypatch.setattr(oracle.paired, "PAIRS", ((0, 1), (0, 2), (1, 2), (0, 3), (1, 3), (2, 3)))
    _fails(pins.pin_paired_fixture, oracle)


def test_paired_pattern_nibbles_swapped():
    real = oracle.quantize_paired

    def q(W):
        p = real(W)
        p.patterns = ((p.patterns >> 4) | (p.patterns << 4)).astype(np.uint8)
        return p
    _fails(pins.pin_paired_fixture, _ns(quantize_paired=q))


def test_paired_ties_to_higher_pair():
    def pat(W):
        N, K = W.shape
        a = np.abs(np.asarray(W, np.float32)).reshape(N, K // 8, 4, 2)
        s = (a[..., 0] + a[..., 1])[..., ::-1]
        order = 3 - np.argsort(-s, axis=2, kind="stable")
        i, j = np.minimum(order[..., 0], order[..., 1]), np.maximum(order[..., 0], order[..., 1])
        lk = {c: n for n, c in enumerate(oracle.PAIRS)}
        return np.vectorize(lambda x, y: lk[(x, y)])(i, j).astype(np.uint8)
    _fails(pins.pin_paired_support_bruteforce, _ns(paired_pattern=pat))


def test_paired_max_instead_of_sum():
    def pat(W):
        N, K = W.shape
        a = np.abs(np.asarray(W, np.float32)).reshape(N, K // 8, 4, 2)
        s = np.maximum(a[..., 0], a[..., 1])
        order = np.argsort(-s, axis=2, kind="stable")
        i, j = np.minimum(order[..., 0], order[..., 1]), np.maximum(order[..., 0], order[..., 1])
        lk = {c: n for n, c in enumerate(oracle.PAIRS)}
        return np.vectorize(lambda x, y: lk[(x, y)])(i, j).astype(np.uint8)
    _fails(pins.pin_paired_support_bruteforce, _ns(paired_pattern=pat))


def test_paired_decode_pair_offset(monkeypatch):
    # pairs counted from the top of the group: pair i = positions 6-2i, 7-2i
    monkeypatch.setattr(oracle.paired, "pattern_mask",
                        lambda p: (3 << (6 - 2 * oracle.PAIRS[p][0])) | (3 << (6 - 2 * oracle.PAIRS[p][1])))
    _fails(pins.pin_paired_matches_48, oracle)
    _fails(pins.pin_paired_fixture, oracle)


# ---------------------------------------------------------------- the expert chain

import oracle.moe  # noqa: E402

_CHAIN_PINS = (pins.pin_chain_fixture, pins.pin_chain_bruteforce)


def _chain_fails(O):
    for pin in _CHAIN_PINS:
        _fails(pin, O)


def test_chain_h_not_rounded(monkeypatch):
    # the hidden activation kept in float64 instead of crossing as bf16
    monkeypatch.setattr(oracle.moe, "bf16_round", lambda v: np.asarray(v, np.float64))
    _chain_fails(oracle)


def test_chain_down_fed_gate_half():
    # the down GEMM fed Y1's gate half instead of h
    def chain(x, off, perm, inv, k, w_up, w_down, tw=None):
        xr = oracle.permute(np.asarray(x, np.float64), perm, k)
        y1 = oracle.grouped_gemm(xr, off, w_up)
        h = oracle.bf16_round(oracle.swiglu(y1))
        y2 = oracle.grouped_gemm(y1[:, :y1.shape[1] // 2], off, w_down)
        return y1, h, y2, oracle.unpermute(y2, inv, tw, x.shape[0], k)
    _chain_fails(_ns(moe_chain=chain))


def test_chain_weights_swapped():
    def chain(x, off, perm, inv, k, w_up, w_down, tw=None):
        return oracle.moe_chain(x, off, perm, inv, k, w_down, w_up, tw)
    # the fixture's projections have the same shape; the brute-force case
    # does not, so its run raises before any comparison
    _fails(pins.pin_chain_fixture, _ns(moe_chain=chain))
    with pytest.raises(Exception):
        pins.pin_chain_bruteforce(_ns(moe_chain=chain))


def test_chain_unweighted_combine():
    def chain(x, off, perm, inv, k, w_up, w_down, tw=None):
        ones = None if tw is None else np.ones_like(np.asarray(tw))
        return oracle.moe_chain(x, off, perm, inv, k, w_up, w_down, ones)
    _chain_fails(_ns(moe_chain=chain))


def test_chain_silu_on_up_half():
    # SwiGLU halves swapped inside the chain
    def chain(x, off, perm, inv, k, w_up, w_down, tw=None):
        xr = oracle.permute(np.asarray(x, np.float64), perm, k)
        y1 = oracle.grouped_gemm(xr, off, w_up)
        n2 = y1.shape[1] // 2
        h = oracle.bf16_round(oracle.silu(y1[:, n2:]) * y1[:, :n2])
        y2 = oracle.grouped_gemm(h, off, w_down)
        return y1, h, y2, oracle.unpermute(y2, inv, tw, x.shape[0], k)
    _chain_fails(_ns(moe_chain=chain))
