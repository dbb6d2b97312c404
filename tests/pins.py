"""Pins of the CPU oracle: checks against what the pages and the mathematics
fix, written so that each takes the oracle module as an argument.  The
`test_oracle_*` files run them on the real oracle; `test_oracle_mutations`
runs them on copies of the oracle with one planted mistake each and expects
a failure, which shows the pins would catch that mistake."""
from __future__ import annotations

import itertools
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# ---------------------------------------------------------------- formats

def pin_e2m1_grid(O):
    """All 16 E2M1 codes equal the OCP MX FP4 table (golden fixture)."""
    for code, val in _lines("e2m1_grid.txt"):
        want = float(val)
        got = O.E2M1_VALUES[int(code)]
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)


def pin_e4m3_table(O):
    """All 256 E4M3 codes equal torch's float8_e4m3fn cast (library cross
    check) and the fixture's selected points."""
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.E4M3_VALUES
    assert np.array_equal(np.isnan(lib), np.isnan(ours))
    ok = ~np.isnan(lib)
    assert np.array_equal(lib[ok], ours[ok])
    for code, val in _lines("e4m3_points.txt"):
        got = O.E4M3_VALUES[int(code, 16)]
        if val == "nan":
            assert math.isnan(got), code
        else:
            assert got == float(val), (code, got, val)


def pin_e4m3_encode(O, n=20000, seed=0):
    """Encoding = torch's RNE float32->float8_e4m3fn cast below 448 (library
    cross check) and saturation to 448 above it."""
    rng = np.random.default_rng(seed)
    x = np.concatenate([
        np.exp(rng.uniform(np.log(1e-4), np.log(500.0), n)).astype(np.float32),
        # exact midpoints between neighbouring codes (ties)
        ((O.E4M3_VALUES[1:0x7E] + O.E4M3_VALUES[2:0x7F]) / 2).astype(np.float32),
        np.float32([0.0, 448.0, 464.0, 1e6, 2.0 ** -10, 3 * 2.0 ** -11])])
    codes = O.e4m3_encode(x)
    below = x < 448
    ref = torch.from_numpy(x[below]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes[below], ref)
    assert (codes[~below] == 0x7E).all()


def pin_e2m1_encode(O, n=20000, seed=1):
    """Encoding picks a nearest grid value (brute force over all 8
    magnitudes), ties to the even code, saturation at 6, zero as +0, and the
    tie cases of round-half-to-even."""
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6,
            -0.25: 0, -0.75: 10, -1.25: 10, -1.75: 12, -2.5: 12, -3.5: 14, -5.0: 14,
            6.5: 7, 100.0: 7, -7.0: 15, 0.0: 0, -0.0: 0, 0.1: 0, -0.1: 0, 0.3: 1}
    xs = np.float32(list(ties))
    assert O.e2m1_encode(xs).tolist() == list(ties.values())
    rng = np.random.default_rng(seed)
    x = rng.uniform(-8, 8, n).astype(np.float32)
    c = O.e2m1_encode(x)
    mags = np.float64([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for xi, ci in zip(x.astype(np.float64), c):
        v = O.E2M1_VALUES[ci]
        best = np.min(np.abs(np.abs(xi) - mags))
        if abs(xi) <= 6:
            assert abs(abs(xi) - abs(v)) == best, (xi, ci)
        else:
            assert abs(v) == 6
        if v != 0:
            assert np.sign(v) == np.sign(xi)
        else:
            assert ci == 0


def pin_bf16_round(O, n=20000, seed=2):
    """bf16 rounding of fp32 inputs equals torch's RNE cast; explicit ties."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * np.exp(rng.uniform(-20, 20, n))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_round(x.astype(np.float64)), ref)
    assert O.bf16_round(1 + 2.0 ** -8) == 1.0                      # tie -> even
    assert O.bf16_round(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6        # tie -> even
    assert O.bf16_round(1 + 2.0 ** -8 + 2.0 ** -30) == 1 + 2.0 ** -7


# ---------------------------------------------------------------- packing

def _hex(tokens):
    return np.array([int(t, 16) for t in tokens], np.uint8)


def pin_quant_fixture(O):
    """The hand-derived 2 x 64 compression (tests/golden/quant_rows.txt)."""
    d = {ln[0]: ln[1:] for ln in _lines("quant_rows.txt")}
    W = np.array([[float(v) for v in d["w0"]], [float(v) for v in d["w1"]]], np.float32)
    p = O.quantize(W)
    assert float(p.g) == float(d["g"][0])
    for r in range(2):
        assert np.array_equal(p.masks[r], _hex(d[f"masks{r}"])), (r, p.masks[r])
        assert np.array_equal(p.values[r], _hex(d[f"values{r}"])), (r, p.values[r])
        assert np.array_equal(p.scales[r], _hex(d[f"scales{r}"])), (r, p.scales[r])
    # decoded values, derived by hand from the codes: q * s * g
    u, v = 0.109375, 36 * 2.0 ** -12
    want0 = ([6 * u, 0, 4 * u, 0, 0, 0, 2 * u, 0] + [u, -u, u, -u, 0, 0, 0, 0] +
             [0, 0, 0, 0, u, -u, 4 * u, -2 * u] + [0.5 * u, 0, -0.5 * u, 0, 0, 0, 0, 0] +
             [6 * v, 1.5 * v, 0, 0, 0, 0, -3 * v, 0.5 * v] + [0] * 24)
    dec = O.decode(p)
    assert np.array_equal(dec[0], np.float64(want0))
    assert np.array_equal(dec[1], -np.float64(want0))


def pin_support_bruteforce(O, seed=3):
    """The kept set of every group is the unique 4-subset whose members all
    beat every dropped position (|w| larger, or equal and lower position),
    found by enumerating all 70 subsets."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((6, 64)).astype(np.float32)
    W[0, :8] = 1.0          # all equal
    W[1, 8:16] = [2, -2, 1, 1, -1, 1, 0, 0]
    W[2, :8] = 0.0
    keep = O.support(W)
    a = np.abs(W)
    for n in range(W.shape[0]):
        for g in range(8):
            grp = a[n, 8 * g:8 * g + 8]
            winners = []
            for S in itertools.combinations(range(8), 4):
                rest = [j for j in range(8) if j not in S]
                if all(grp[i] > grp[j] or (grp[i] == grp[j] and i < j) for i in S for j in rest):
                    winners.append(S)
            assert len(winners) == 1
            got = tuple(np.nonzero(keep[n, 8 * g:8 * g + 8])[0])
            assert got == winners[0], (n, g, got, winners)


def pin_masks_and_layout(O, seed=4):
    """Every mask byte has popcount 4; a large random matrix realises all 70
    valid masks, the six paired patterns among them; packed size is 13/32
    byte per logical weight plus the fp32 global scale (golden layout)."""
    d = {ln[0]: ln[1:] for ln in _lines("layout.txt")}
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((256, 512)) * 0.02).astype(np.float32)
    p = O.quantize(W)
    pc = np.unpackbits(p.masks[..., None], axis=-1).sum(-1)
    assert (pc == 4).all()
    seen = set(np.unique(p.masks).tolist())
    assert len(seen) == int(d["valid_mask_count"][0])
    assert {int(x, 16) for x in d["paired_patterns"]} <= seen
    N, K = W.shape
    bpw = float(d["mask_bits_per_weight"][0])
    assert p.nbytes == N * K * bpw / 8 + 4
    assert p.values.nbytes + p.masks.nbytes + p.scales.nbytes == N * K // 32 * int(d["mask_bytes_per_32"][0])
    # the pages' paired format: 4-bit index instead of the 8-bit mask
    paired = ((4 * 4 + int(d["paired_index_bits"][0])) * 4 + 8) / 32
    assert paired == float(d["paired_bits_per_weight"][0])


def pin_quant_nearest(O, seed=5):
    """Every decoded kept weight is a nearest point of the scaled E2M1 grid
    (brute force over all grid values) to the input, unless it saturates;
    every block scale is a nearest E4M3 value to amax_32/(6g) (brute force
    over all 127 finite non-negative codes); dropped positions decode to 0."""
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((8, 128)) * 0.02).astype(np.float32)
    W[3, 40] = 0.5                                  # an outlier
    p = O.quantize(W)
    dec = O.decode(p, include_global=False)
    keep = O.support(W)
    g = np.float64(p.g)
    assert (dec[~keep] == 0).all()
    e4 = O.E4M3_VALUES[:0x7F]
    grid = np.float64([0, .5, 1, 1.5, 2, 3, 4, 6])
    grid = np.concatenate([-grid[::-1], grid])
    for n in range(W.shape[0]):
        for b in range(W.shape[1] // 32):
            blk = W[n, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.max(np.abs(blk))
            target = np.float32(np.float32(amax) / np.float32(np.float32(6) * p.g))
            s = O.E4M3_VALUES[p.scales[n, b]]
            assert abs(s - target) == np.min(np.abs(e4 - target)) or (target > 448 and s == 448)
            sg = np.float32(np.float32(s) * p.g)
            for i in range(32):
                if not keep[n, 32 * b + i]:
                    continue
                q = np.float64(np.float32(np.float32(blk[i]) / sg)) if sg > 0 else 0.0
                got = dec[n, 32 * b + i] / s if s else 0.0
                if abs(q) <= 6:
                    assert abs(q - got) == np.min(np.abs(grid - q)), (n, b, i, q, got)
                else:
                    assert got == np.sign(q) * 6


# ---------------------------------------------------------------- routing

def pin_route_bruteforce(O, seed=6):
    """Offsets and permutation equal a plain loop: for each expert in turn,
    the flat indices that chose it, in increasing order."""
    rng = np.random.default_rng(seed)
    for E, M in [(5, 40), (16, 300), (3, 1), (7, 7000)]:
        ids = rng.integers(0, E, M).astype(np.int32)
        if M > 10:
            ids[: M // 3] = 1                       # many duplicates
        off, perm, inv = O.route(ids, E)
        p, o = [], [0]
        for e in range(E):
            for i in range(M):
                if ids[i] == e:
                    p.append(i)
            o.append(len(p))
        assert off.tolist() == o
        assert perm.tolist() == p
        for r in range(M):
            assert inv[perm[r]] == r


# ---------------------------------------------------------------- GEMM

def _to_fraction(x):
    return Fraction(float(x))


def pin_gemm_exact(O, seed=7):
    """Grouped GEMM against exact rational arithmetic on tiny inputs: bf16
    tokens and decoded weights are dyadic, so Fraction sums are exact; the
    float64 oracle must lie within gamma_K * sum |x||w| of them."""
    rng = np.random.default_rng(seed)
    E, N, K, T, k = 3, 6, 64, 5, 2
    Ws = [O.quantize((rng.standard_normal((N, K)) * 0.02).astype(np.float32)) for _ in range(E)]
    dense = [O.decode(p) for p in Ws]
    x = torch.randn(T, K, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    x = x.to(torch.float64).numpy()
    ids = np.array([[0, 2], [2, 1], [0, 1], [2, 0], [1, 2]], np.int32).reshape(-1)
    off, perm, inv = O.route(ids, E)
    xr = O.permute(x, perm, k)
    Y = O.grouped_gemm(xr, off, lambda e: dense[e])
    u = 2.0 ** -53
    gamma = K * u / (1 - K * u)
    for r in range(T * k):
        e = ids[perm[r]]
        assert np.array_equal(xr[r], x[perm[r] // k])
        for n in range(N):
            exact = sum(_to_fraction(xr[r, kk]) * _to_fraction(dense[e][n, kk]) for kk in range(K))
            bound = gamma * float(sum(abs(_to_fraction(xr[r, kk]) * _to_fraction(dense[e][n, kk]))
                                      for kk in range(K)))
            assert abs(Fraction(float(Y[r, n])) - exact) <= Fraction(bound) + Fraction(1, 2 ** 1074), (r, n)


def pin_gemm_invariances(O, seed=8):
    """Permuting tokens permutes routed rows consistently; relabelling
    experts permutes offsets; scaling X by 2^p scales Y by 2^p exactly."""
    rng = np.random.default_rng(seed)
    E, N, K, T, k = 4, 16, 96, 9, 2
    Ws = [O.decode(O.quantize((rng.standard_normal((N, K)) * 0.02).astype(np.float32)))
          for _ in range(E)]
    x = np.float64(rng.standard_normal((T, K)).astype(np.float32))
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)

    def run(x, ids, Ws):
        off, perm, inv = O.route(ids.reshape(-1), len(Ws))
        Y = O.grouped_gemm(O.permute(x, perm, k), off, lambda e: Ws[e])
        return off, O.unpermute(Y, inv, None, x.shape[0], k)

    off, flat = run(x, ids, Ws)
    sigma = rng.permutation(T)
    off2, flat2 = run(x[sigma], ids[sigma], Ws)
    assert np.array_equal(off, off2)
    assert np.allclose(flat2.reshape(T, k, N), flat.reshape(T, k, N)[sigma], rtol=1e-12, atol=0)
    tau = rng.permutation(E)                       # expert e becomes tau[e]
    Wt = [None] * E
    for e in range(E):
        Wt[tau[e]] = Ws[e]
    off3, flat3 = run(x, tau[ids].astype(np.int32), Wt)
    counts = np.diff(off)
    assert np.array_equal(np.diff(off3)[tau], counts)
    assert np.allclose(flat3, flat, rtol=1e-12, atol=0)
    _, flat4 = run(x * 2.0 ** 5, ids, Ws)
    assert np.array_equal(flat4, flat * 2.0 ** 5)
    # each routed row equals the dense product with that token and expert
    for t in range(T):
        for j in range(k):
            want = np.array([sum(x[t, kk] * Ws[ids[t, j]][n, kk] for kk in range(K)) for n in range(N)])
            assert np.allclose(flat[t * k + j], want, rtol=1e-12, atol=1e-300)


# ---------------------------------------------------------------- combine and SwiGLU

def pin_unpermute(O, seed=9):
    """k = 1 with unit weights inverts dispatch exactly; the weighted combine
    equals a plain loop over (t, j)."""
    rng = np.random.default_rng(seed)
    T, E, N = 11, 4, 8
    x = rng.standard_normal((T, N))
    ids = rng.integers(0, E, T).astype(np.int32)
    off, perm, inv = O.route(ids, E)
    xr = O.permute(x, perm, 1)
    assert np.array_equal(O.unpermute(xr, inv, np.ones(T, np.float32), T, 1), x)
    assert np.array_equal(O.unpermute(xr, inv, None, T, 1), x)
    k = 3
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).reshape(-1).astype(np.int32)
    off, perm, inv = O.route(ids, E)
    Y = rng.standard_normal((T * k, N))
    w = rng.random(T * k).astype(np.float32)
    out = O.unpermute(Y, inv, w, T, k)
    for t in range(T):
        want = np.zeros(N)
        for j in range(k):
            r = list(perm).index(t * k + j)
            want = want + np.float64(w[t * k + j]) * Y[r]
        assert np.array_equal(out[t], want)


def pin_swiglu(O):
    """silu against torch's float64 silu and closed forms; gate = first half."""
    x = np.linspace(-30, 30, 2001)
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    assert np.allclose(O.silu(x), ref, rtol=1e-14, atol=1e-300)
    assert O.silu(0.0) == 0.0
    assert abs(O.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert O.silu(-800.0) == 0.0
    y1 = np.array([[0.0, 1.0, 2.0, 3.0]])          # gate [0, 1], up [2, 3]
    h = O.swiglu(y1)
    assert np.allclose(h, [[0.0, 3.0 / (1.0 + math.exp(-1.0))]], rtol=1e-15)



# ---------------------------------------------------------------- the expert chain

def _fixture_rows(d, prefix, n):
    return np.array([[float(v) for v in d[f"{prefix}{i}"]] for i in range(n)], np.float64)


def pin_chain_fixture(O):
    """The hand-derived chain (tests/golden/chain_rows.txt): routing, Y1, the
    bf16 hidden activation h, Y2 and the router-weighted combine of two tokens
    over two experts, every value derived by hand from the inputs."""
    d = {ln[0]: ln[1:] for ln in _lines("chain_rows.txt")}
    x = _fixture_rows(d, "x", 2)
    ids = np.array([int(v) for v in d["ids"]], np.int32)
    tw = np.array([float(v) for v in d["topk_weights"]], np.float32)
    up = [np.array([float(v) for v in d[f"up{e}"]], np.float64).reshape(4, 2) for e in range(2)]
    down = [np.array([float(v) for v in d[f"down{e}"]], np.float64).reshape(4, 2) for e in range(2)]
    off, perm, inv = O.route(ids, 2)
    assert off.tolist() == [0, 2, 4] and perm.tolist() == [1, 2, 0, 3] and inv.tolist() == [2, 0, 1, 3]
    y1, h, y2, out = O.moe_chain(x, off, perm, inv, 2, lambda e: up[e], lambda e: down[e], tw)
    assert np.array_equal(y1, _fixture_rows(d, "y1_r", 4)), y1
    assert np.array_equal(h, _fixture_rows(d, "h_r", 4)), h
    assert np.array_equal(y2, _fixture_rows(d, "y2_r", 4)), y2
    assert np.array_equal(out, _fixture_rows(d, "out", 2)), out


def _bf16_exact(v: Fraction) -> Fraction:
    """Round a rational to the nearest value with 8 significant bits, ties to
    even (exact; no floating point)."""
    if v == 0:
        return Fraction(0)
    s = -1 if v < 0 else 1
    a, e = abs(v), 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    q = a * 128
    n = math.floor(q)
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2):
        n += 1
    return s * Fraction(n, 128) * Fraction(2) ** e


def pin_chain_bruteforce(O, seed=13):
    """The chain on compressed experts against exact rational arithmetic in
    plain loops: Y1 and Y2 as exact sums, h as the exact bf16 rounding of
    silu(gate) * up (silu by math.exp), the combine as exact weighted sums.
    The oracle's float64 results must lie within their summation bounds, and
    h must equal the exact rounding except within 1e-12 of a rounding
    midpoint (where either neighbour is right)."""
    rng = np.random.default_rng(seed)
    E, T, k, K, N1, N2 = 3, 5, 2, 64, 64, 16
    up = [O.decode(O.quantize((rng.standard_normal((N1, K)) * 0.5).astype(np.float32)))
          for _ in range(E)]
    down = [O.decode(O.quantize((rng.standard_normal((N2, N1 // 2)) * 0.5).astype(np.float32)))
            for _ in range(E)]
    x = torch.randn(T, K, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    x = x.to(torch.float64).numpy()
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).reshape(-1).astype(np.int32)
    tw = rng.random(T * k).astype(np.float32)
    off, perm, inv = O.route(ids, E)
    y1, h, y2, out = O.moe_chain(x, off, perm, inv, k, lambda e: up[e], lambda e: down[e], tw)
    u = 2.0 ** -53
    y2_exact = {}
    for t in range(T):
        for j in range(k):
            i = t * k + j
            e = int(ids[i])
            r = int(inv[i])
            assert perm[r] == i
            xf = [Fraction(float(v)) for v in x[t]]
            y1e = [sum(xf[c] * Fraction(float(up[e][n, c])) for c in range(K)) for n in range(N1)]
            for n in range(N1):
                mag = sum(abs(xf[c] * Fraction(float(up[e][n, c]))) for c in range(K))
                assert abs(Fraction(float(y1[r, n])) - y1e[n]) <= Fraction(K * u) * mag + Fraction(1, 2 ** 1074)
            he = []
            for c in range(N1 // 2):
                g = float(y1e[c])
                v = Fraction(g / (1.0 + math.exp(-g))) * y1e[c + N1 // 2]
                want = _bf16_exact(v)
                got = Fraction(float(h[r, c]))
                if got != want:
                    # only a value at a rounding midpoint may go either way
                    lo, hi = sorted([got, want])
                    mid = (lo + hi) / 2
                    assert abs(v - mid) <= Fraction(1, 10 ** 12) * abs(v), (r, c, float(v), float(got))
                he.append(got)
            y2e = [sum(he[c] * Fraction(float(down[e][n, c])) for c in range(N1 // 2)) for n in range(N2)]
            for n in range(N2):
                mag = sum(abs(he[c] * Fraction(float(down[e][n, c]))) for c in range(N1 // 2))
                assert abs(Fraction(float(y2[r, n])) - y2e[n]) <= Fraction(N1 * u) * mag + Fraction(1, 2 ** 1074)
            y2_exact[i] = (y2e, [sum(abs(he[c] * Fraction(float(down[e][n, c]))) for c in range(N1 // 2))
                                 for n in range(N2)])
    for t in range(T):
        for n in range(N2):
            want = sum(Fraction(float(tw[t * k + j])) * y2_exact[t * k + j][0][n] for j in range(k))
            mag = sum(Fraction(float(tw[t * k + j])) * y2_exact[t * k + j][1][n] for j in range(k))
            assert abs(Fraction(float(out[t, n])) - want) <= Fraction((N1 + 2 * k) * u) * mag + Fraction(1, 2 ** 1074), (t, n)


# ---------------------------------------------------------------- paired 4:8

def pin_paired_fixture(O):
    """The hand-derived paired 2 x 32 compression and the pattern table
    (tests/golden/paired_rows.txt)."""
    lines = _lines("paired_rows.txt")
    d = {ln[0]: ln[1:] for ln in lines if ln[0] != "pattern"}
    for ln in lines:
        if ln[0] == "pattern":
            p, pos = int(ln[1]), [int(v) for v in ln[2:]]
            assert O.pattern_mask(p) == sum(1 << i for i in pos), (p, O.pattern_mask(p))
    w0 = np.array([float(v) for v in d["w0"]], np.float32)
    W = np.stack([w0, -w0])
    p = O.quantize_paired(W)
    assert float(p.g) == float(d["g"][0])
    for r in range(2):
        assert np.array_equal(p.values[r], _hex(d[f"values{r}"])), (r, p.values[r])
        assert np.array_equal(p.patterns[r], _hex(d["patterns0"])), (r, p.patterns[r])
        assert np.array_equal(p.scales[r], _hex(d["scales0"])), (r, p.scales[r])
    want = np.float64([float(v) for v in d["decoded0"]])
    dec = O.decode_paired(p)
    assert np.array_equal(dec[0], want)
    assert np.array_equal(dec[1], -want)
    # decoding without the global scale divides by g exactly
    assert np.array_equal(O.decode_paired(p, include_global=False)[0], want / float(p.g))


def pin_paired_support_bruteforce(O, seed=10):
    """Every group keeps the unique couple of pairs whose members both beat
    both dropped pairs (larger fp32 |w| sum, or equal and lower index), found
    by enumerating the six allowed patterns; that couple also has the largest
    exact total, and the keep-map is its pattern's mask."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((6, 96)).astype(np.float32)
    W[0, :8] = 1.0                                   # all four sums equal
    W[1, 8:16] = [2, 0, 0, 2, 1, 1, -2, 0]           # sums 2 2 2 2
    W[2, :8] = 0.0
    W[3, 16:24] = [0, 0, 1, 0, 0, 1, 0.5, 0.5]       # sums 0 1 1 1
    W[4, :] = np.round(W[4, :] * 2) / 2              # many equal sums
    pat = O.paired_pattern(W)
    keep = O.paired_support(W)
    a = np.abs(W)
    couples = [tuple(sorted(c)) for c in itertools.combinations(range(4), 2)]
    assert sorted(O.PAIRS) == couples and len(set(O.PAIRS)) == 6
    for n in range(W.shape[0]):
        for g in range(W.shape[1] // 8):
            grp = a[n, 8 * g:8 * g + 8]
            sums = [np.float32(grp[2 * i] + grp[2 * i + 1]) for i in range(4)]
            winners = [S for S in couples
                       if all(sums[i] > sums[j] or (sums[i] == sums[j] and i < j)
                              for i in S for j in range(4) if j not in S)]
            assert len(winners) == 1
            got = O.PAIRS[pat[n, g]]
            assert got == winners[0], (n, g, got, winners)
            best = max(Fraction(float(sums[i])) + Fraction(float(sums[j])) for i, j in couples)
            assert Fraction(float(sums[got[0]])) + Fraction(float(sums[got[1]])) == best
            kept = [i for i in range(8) if keep[n, 8 * g + i]]
            assert kept == [2 * got[0], 2 * got[0] + 1, 2 * got[1], 2 * got[1] + 1]


def pin_paired_layout(O, seed=11):
    """Pattern masks are exactly the six unions of two adjacent pairs (the
    golden set); a random matrix uses all six; packed size is the pages'
    2.75 bits per logical weight plus the fp32 global scale."""
    d = {ln[0]: ln[1:] for ln in _lines("layout.txt")}
    pairs = [0x03, 0x0C, 0x30, 0xC0]
    unions = {a | b for a, b in itertools.combinations(pairs, 2)}
    masks = {O.pattern_mask(p) for p in range(6)}
    assert masks == unions == {int(x, 16) for x in d["paired_patterns"]}
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    p = O.quantize_paired(W)
    nib = np.stack([p.patterns & 15, p.patterns >> 4], -1)
    assert set(np.unique(nib).tolist()) == set(range(6))
    N, K = W.shape
    assert p.nbytes * 8 == N * K * float(d["paired_bits_per_weight"][0]) + 32
    assert p.values.shape == (N, K // 4) and p.patterns.shape == (N, K // 16)
    assert p.scales.shape == (N, K // 32)


def pin_paired_matches_48(O, seed=12):
    """When the four largest |w| of every group form two adjacent pairs that
    also have the two largest pair sums, the paired and the 4:8 formats keep
    the same positions, so their decodes agree exactly; dropped positions
    decode to zero."""
    rng = np.random.default_rng(seed)
    N, K = 16, 256
    W = (rng.uniform(0, 0.1, (N, K)) * rng.choice([-1, 1], (N, K))).astype(np.float32)
    for n in range(N):
        for g in range(K // 8):
            for i in rng.choice(4, 2, replace=False):
                W[n, 8 * g + 2 * i:8 * g + 2 * i + 2] = rng.uniform(1, 2, 2) * rng.choice([-1, 1], 2)
    big = np.flatnonzero(np.abs(W[3, 40:48]) >= 1) + 40
    W[3, big] *= 20.0                                 # an outlier group
    pp = O.quantize_paired(W)
    p4 = O.quantize(W)
    assert np.array_equal(O.paired_support(W), O.support(W))
    d = O.decode_paired(pp)
    assert np.array_equal(d, O.decode(p4))
    assert (d[~O.paired_support(W)] == 0).all()
    assert np.array_equal(pp.scales, p4.scales) and pp.g == p4.g



# ---------------------------------------------------------------- W4A4 activations

def pin_act_fixture(O):
    """The hand-derived NVFP4 quantization of two activation rows
    (tests/golden/act_rows.txt): codes, scales, row scales and decoded values."""
    d = {ln[0]: ln[1:] for ln in _lines("act_rows.txt")}
    x = np.array([[float(v) for v in d["x0"]], [float(v) for v in d["x1"]]], np.float32)
    p = O.quantize_activations(x)
    assert p.g.tolist() == [float(v) for v in d["g"]], p.g
    for r in range(2):
        assert np.array_equal(p.scales[r], _hex(d[f"scales{r}"])), (r, p.scales[r])
        assert np.array_equal(p.codes[r], _hex(d[f"codes{r}"])), (r, p.codes[r])
        want = np.array([float(v) for v in d[f"decoded{r}"]])
        assert np.array_equal(O.decode_activations(p)[r], want), r
        assert np.array_equal(O.decode_activations(p, include_row_scale=False)[r],
                              want / float(p.g[r])), r


def _act_rows(rng, T=24, K=256):
    x = rng.standard_normal((T, K)).astype(np.float32)
    x *= np.exp(rng.uniform(-12, 12, (T, 1))).astype(np.float32)          # per-row range
    x[:, rng.choice(K, 5, replace=False)] *= 10                            # outlier channels
    x[3] = 0                                                               # zero row
    x[4, 32:64] = 0                                                        # zero block
    x[5, :] = np.float32(0.75) * np.sign(x[5])                             # all ties
    x[6, 7] = -x[6].__abs__().max() * 2                                    # negative row max
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()


def pin_act_nearest(O, seed=14):
    """On random bf16 rows: g is the fp32 amax/2688 (1 for a zero row); every
    block scale is torch's float32 -> float8_e4m3fn cast of amax_b/(6g) below
    448 and saturates to 448 above it; every code is a nearest E2M1 value of
    x/(s g) (brute force over the grid, ties to the even code, saturation
    at 6), with +0 for a zero result; zero rows and blocks decode to zero."""
    rng = np.random.default_rng(seed)
    x = _act_rows(rng)
    p = O.quantize_activations(x)
    T, K = x.shape
    amax = np.abs(x).max(axis=1)
    g = np.where(amax > 0, (amax / np.float32(2688)).astype(np.float32), np.float32(1))
    assert np.array_equal(p.g, g.astype(np.float32))
    six_g = (np.float32(6) * p.g).astype(np.float32)
    ab = np.abs(x).reshape(T, K // 32, 32).max(axis=2)
    r = (ab / six_g[:, None]).astype(np.float32)
    lib = torch.from_numpy(np.minimum(r, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(p.scales, np.where(r >= 448, 0x7E, lib))
    grid = np.float64([0, .5, 1, 1.5, 2, 3, 4, 6])
    codes = np.empty((T, K), np.uint8)
    codes[:, 0::2], codes[:, 1::2] = p.codes & 15, p.codes >> 4
    for t in range(T):
        for b in range(K // 32):
            sg = np.float32(np.float32(O.E4M3_VALUES[p.scales[t, b]]) * p.g[t])
            for i in range(32):
                c = int(codes[t, 32 * b + i])
                v = O.E2M1_VALUES[c]
                if sg == 0:
                    assert c == 0
                    continue
                q = float(np.float32(np.float32(x[t, 32 * b + i]) / sg))
                if abs(q) >= 6:
                    assert v == np.sign(q) * 6, (t, b, i, q, c)
                    continue
                d = np.abs(abs(q) - grid)
                best = np.flatnonzero(d == d.min())
                assert abs(v) == grid[best[0] if len(best) == 1 else best[0] + (best[0] % 2)], (t, b, i, q, c)
                assert (v == 0 and c == 0) or np.sign(v) == np.sign(q), (t, b, i, q, c)
    dec = O.decode_activations(p)
    assert not dec[3].any() and not dec[4, 32:64].any()


def pin_act_invariances(O, seed=15):
    """Rows are quantized on their own: permuting rows permutes the packed
    rows; scaling a row by 2^p (within range) keeps its codes and scales and
    scales g by 2^p; a row's largest magnitude decodes exactly (its block
    scale is 448 and its code 6)."""
    rng = np.random.default_rng(seed)
    x = _act_rows(rng, T=16, K=128)
    p = O.quantize_activations(x)
    sigma = rng.permutation(16)
    q = O.quantize_activations(x[sigma])
    assert np.array_equal(q.codes, p.codes[sigma]) and np.array_equal(q.scales, p.scales[sigma])
    assert np.array_equal(q.g, p.g[sigma])
    s = O.quantize_activations(x * np.float32(2.0 ** 7))
    nz = np.abs(x).max(axis=1) > 0
    assert np.array_equal(s.codes, p.codes) and np.array_equal(s.scales, p.scales)
    assert np.array_equal(s.g[nz], p.g[nz] * np.float32(2.0 ** 7))
    dec = O.decode_activations(p)
    for t in np.flatnonzero(nz):
        k = int(np.argmax(np.abs(x[t])))
        assert p.scales[t, k // 32] == 0x7E
        assert abs(dec[t, k]) == abs(np.float64(x[t, k])) or abs(dec[t, k]) == 6 * 448 * float(p.g[t])


def pin_w4a4_gemm_exact(O, seed=16):
    """The W4A4 expert GEMM against exact rational arithmetic: its operands
    are the dequantized activations (the pinned decode) and the dequantized
    weights, both dyadic; the float64 result lies within gamma_K * sum |x||w|
    of the exact sum."""
    rng = np.random.default_rng(seed)
    N, K, m = 5, 64, 8
    W = O.decode(O.quantize((rng.standard_normal((N, K)) * 0.02).astype(np.float32)))
    x = _act_rows(rng, T=m, K=K)
    y = O.w4a4_expert_gemm(x, W)
    xq = O.decode_activations(O.quantize_activations(x))
    u = 2.0 ** -53
    for r in range(m):
        for n in range(N):
            terms = [Fraction(float(xq[r, k])) * Fraction(float(W[n, k])) for k in range(K)]
            mag = sum(abs(t) for t in terms)
            assert abs(Fraction(float(y[r, n])) - sum(terms)) <= Fraction(K * u) * mag + Fraction(1, 2 ** 1074)


ALL_PINS = [pin_e2m1_grid, pin_e4m3_table, pin_e4m3_encode, pin_e2m1_encode,
            pin_bf16_round, pin_quant_fixture, pin_support_bruteforce,
            pin_masks_and_layout, pin_quant_nearest, pin_route_bruteforce,
            pin_gemm_exact, pin_gemm_invariances, pin_unpermute, pin_swiglu,
            pin_paired_fixture, pin_paired_support_bruteforce, pin_paired_layout,
            pin_paired_matches_48, pin_chain_fixture, pin_chain_bruteforce,
            pin_act_fixture, pin_act_nearest, pin_act_invariances, pin_w4a4_gemm_exact]
