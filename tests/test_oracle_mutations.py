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


# ---------------------------------------------------------------- W4A4 activations

import oracle.w4a4  # noqa: E402

_ACT_PINS = (pins.pin_act_fixture, pins.pin_act_nearest)


def _quant_act(x, g_of, block=32):
    """The activation quantizer with the second-level scale from g_of(x) and
    scale blocks of `block` positions (layout of 32-blocks kept)."""
    x = np.asarray(x, np.float32)
    T, K = x.shape
    g = g_of(x)
    six_g = (np.float32(6) * g).astype(np.float32)
    ab = np.abs(x).reshape(T, K // block, block).max(axis=2)
    sc = oracle.e4m3_encode((ab / six_g[:, None]).astype(np.float32))
    sg = np.repeat((oracle.E4M3_VALUES[sc].astype(np.float32) * g[:, None]).astype(np.float32),
                   block, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(sg > 0, x / np.where(sg > 0, sg, 1), 0).astype(np.float32)
    c = oracle.e2m1_encode(q)
    step = 32 // block
    return oracle.PackedActivations((c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8),
                                    sc[:, ::step].astype(np.uint8), g.astype(np.float32))


def test_act_per_tensor_scale():
    # one second-level scale for the whole tensor instead of one per row
    def g_tensor(x):
        amax = np.float32(np.abs(x).max())
        g = np.float32(amax / np.float32(2688)) if amax > 0 else np.float32(1)
        return np.full(x.shape[0], g, np.float32)
    _fails(pins.pin_act_fixture, _ns(quantize_activations=lambda x: _quant_act(x, g_tensor)))


def _g_row(x):
    amax = np.abs(x).max(axis=1)
    return np.where(amax > 0, (amax / np.float32(2688)).astype(np.float32), np.float32(1))


def test_act_blocks_of_16():
    O = _ns(quantize_activations=lambda x: _quant_act(x, _g_row, block=16))
    for pin in _ACT_PINS:
        _fails(pin, O)


def test_act_scale_without_six(monkeypatch):
    monkeypatch.setattr(oracle.w4a4, "e4m3_encode",
                        lambda v: oracle.formats.e4m3_encode(np.asarray(v) * 6))
    for pin in _ACT_PINS:
        _fails(pin, oracle)


def test_act_nibbles_swapped():
    real = oracle.quantize_activations

    def q(x):
        p = real(x)
        p.codes = ((p.codes >> 4) | (p.codes << 4)).astype(np.uint8)
        return p
    O = _ns(quantize_activations=q)
    for pin in _ACT_PINS:
        _fails(pin, O)


def test_act_decode_without_row_scale():
    def dec(p, include_row_scale=True):
        return oracle.decode_activations(p, include_row_scale=False)
    _fails(pins.pin_act_fixture, _ns(decode_activations=dec))


def test_act_scale_truncated(monkeypatch):
    # block scales rounded down instead of to nearest
    def trunc(v):
        v = np.minimum(np.asarray(v, np.float64), 448)
        pos = oracle.E4M3_VALUES[:0x7F]
        return (np.searchsorted(pos, v, side="right") - 1).astype(np.uint8)
    monkeypatch.setattr(oracle.w4a4, "e4m3_encode", trunc)
    for pin in _ACT_PINS:
        _fails(pin, oracle)


def test_w4a4_gemm_unquantized_activations():
    # the GEMM fed the bf16 activations instead of their NVFP4 rounding
    def gemm(x_rows, W):
        return np.asarray(x_rows, np.float64) @ np.asarray(W, np.float64).T
    _fails(pins.pin_w4a4_gemm_exact, _ns(w4a4_expert_gemm=gemm))


def test_act_mutation_harness_is_faithful():
    # without a planted mistake the rewritten quantizer passes the pins, so
    # the failures above come from the mistakes alone
    O = _ns(quantize_activations=lambda x: _quant_act(x, _g_row))
    for pin in _ACT_PINS:
        pin(O)
