"""The C-ABI library loads, exports every symbol include/moesq.h declares, and
rejects bad arguments on the host before touching the GPU.  No GPU: only
argument checks that return before any HIP call are exercised."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moesq.h")
LIB = os.path.join(ROOT, "sparse_fp4_expert_amd", "libmoesq.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moesq_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libmoesq.so is not built: run python -m sparse_fp4_expert_amd.build")
    return ctypes.CDLL(LIB)


@pytest.fixture(scope="module")
def m():
    from sparse_fp4_expert_amd import moesq
    return moesq


def test_exports_every_declared_symbol(lib, m):
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(m.EXPORTED) == names


def test_status_strings_and_version(m):
    assert m.version() >= 100
    for st in [m.OK, m.ERR_NULL, m.ERR_SHAPE, m.ERR_WORKSPACE, m.ERR_LAYOUT, m.ERR_HIP, m.ERR_ARG]:
        assert m._status_string(st).decode().startswith("MOESQ_")
    assert m._route_ws(64, 2, 8) == 0


def _desc(m, E=8, N=128, K=256, layout=0, null=False):
    p = None if null else 0x1000
    return m.WeightsDesc(p, p, p, p, E, N, K, layout)


def test_route_rejects(m):
    r = m._route
    assert r(None, 4, 2, 0, 0x10, 0x10, 0x10, None, 0, None) == m.ERR_SHAPE      # E = 0
    assert r(None, 4, 2, 2000, 0x10, 0x10, 0x10, None, 0, None) == m.ERR_SHAPE   # E too large
    assert r(None, 4, 9, 8, 0x10, 0x10, 0x10, None, 0, None) == m.ERR_SHAPE      # k > E
    assert r(None, -1, 2, 8, 0x10, 0x10, 0x10, None, 0, None) == m.ERR_SHAPE     # T < 0
    assert r(None, 4, 2, 8, 0x10, 0x10, 0x10, None, 0, None) == m.ERR_NULL       # ids NULL
    assert r(0x10, 4, 2, 8, None, 0x10, 0x10, None, 0, None) == m.ERR_NULL
    assert b"expert_offsets" in m._last_error()
    assert r(0x10, 1 << 30, 4, 8, 0x10, 0x10, 0x10, None, 0, None) == m.ERR_SHAPE  # T*k >= 2^31
    assert b"2^31" in m._last_error()


def test_permute_unpermute_reject(m):
    assert m._permute(0x10, 0x10, 4, 2, 12, 0x10, None) == m.ERR_SHAPE            # K % 8
    assert m._permute(None, 0x10, 4, 2, 16, 0x10, None) == m.ERR_NULL
    assert m._permute(None, None, 0, 2, 16, None, None) == m.OK                   # empty: no-op
    assert m._unpermute(0x10, 0x10, None, 4, 2, 12, 0x10, None) == m.ERR_SHAPE     # N % 8
    assert m._unpermute(0x10, None, None, 4, 2, 16, 0x10, None) == m.ERR_NULL
    assert m._unpermute(0x10, 0x10, None, 4, 0, 16, 0x10, None) == m.ERR_SHAPE     # k < 1


def test_spgemm_rejects(m):
    ref = ctypes.byref
    g = m._spgemm
    ok_off = 0x10
    assert g(0x10, ok_off, 4, None, 0, 0x10, None, 0, None) == m.ERR_NULL
    assert g(0x10, ok_off, 4, ref(_desc(m, layout=7)), 0, 0x10, None, 0, None) == m.ERR_LAYOUT
    assert g(0x10, ok_off, 4, ref(_desc(m, null=True)), 0, 0x10, None, 0, None) == m.ERR_NULL
    assert g(0x10, ok_off, 4, ref(_desc(m, K=48)), 0, 0x10, None, 0, None) == m.ERR_SHAPE
    assert g(0x10, ok_off, 4, ref(_desc(m, N=24)), 0, 0x10, None, 0, None) == m.ERR_SHAPE
    assert g(0x10, ok_off, 4, ref(_desc(m, E=0)), 0, 0x10, None, 0, None) == m.ERR_SHAPE
    assert g(0x10, ok_off, 4, ref(_desc(m, E=1025)), 0, 0x10, None, 0, None) == m.ERR_SHAPE
    assert g(0x10, ok_off, 4, ref(_desc(m, N=48)), 1, 0x10, None, 0, None) == m.ERR_SHAPE  # SwiGLU N%32
    big = _desc(m, N=1 << 16, K=1 << 17)                       # one expert's values = 2 GiB
    assert g(0x10, ok_off, 4, ref(big), 0, 0x10, None, 0, None) == m.ERR_SHAPE
    assert g(0x10, ok_off, 4, ref(_desc(m)), 5, 0x10, None, 0, None) == m.ERR_ARG          # epilogue
    # flat output order needs a gather permutation, which this call has not
    assert g(0x10, ok_off, 4, ref(_desc(m)), m.OUT_FLAT, 0x10, None, 0, None) == m.ERR_ARG
    assert b"MOESQ_OUT_FLAT" in m._last_error()
    assert g(0x10, ok_off, 4, ref(_desc(m)), m.OUT_FLAT | 5, 0x10, None, 0, None) == m.ERR_ARG
    assert g(0x10, None, 4, ref(_desc(m)), 0, 0x10, None, 0, None) == m.ERR_NULL
    assert g(0x10, ok_off, -1, ref(_desc(m)), 0, 0x10, None, 0, None) == m.ERR_SHAPE
    assert g(None, ok_off, 0, ref(_desc(m)), 0, None, None, 0, None) == m.OK                # M = 0
    assert g(None, ok_off, 4, ref(_desc(m)), 0, 0x10, None, 0, None) == m.ERR_NULL


def test_pack_and_decode_reject(m):
    assert m._pack(0x10, 1, 16, 48, 0x10, 0x10, 0x10, 0x10, None) == m.ERR_SHAPE
    assert m._pack(0x10, 0, 16, 64, 0x10, 0x10, 0x10, 0x10, None) == m.ERR_SHAPE
    assert m._pack(None, 1, 16, 64, 0x10, 0x10, 0x10, 0x10, None) == m.ERR_NULL
    d = _desc(m)
    assert m._decode(ctypes.byref(d), 8, 0x10, None) == m.ERR_ARG
    assert m._decode(ctypes.byref(d), -1, 0x10, None) == m.ERR_ARG
    assert m._decode(ctypes.byref(d), 0, None, None) == m.ERR_NULL
    assert m._decode(None, 0, 0x10, None) == m.ERR_NULL


def test_validate_rejects(m):
    v = m._validate
    ref = ctypes.byref
    assert v(0x10, 4, 2, 0, None, None, None, None) == m.ERR_SHAPE        # E = 0 with ids
    assert v(0x10, 4, 2, 2000, None, None, None, None) == m.ERR_SHAPE     # E too large
    assert v(None, -1, 2, 8, 0x10, None, None, None) == m.ERR_SHAPE       # T < 0 with offsets
    assert v(None, 4, 0, 8, 0x10, None, None, None) == m.ERR_SHAPE        # k < 1
    assert v(None, 0, 1, 1, None, ref(_desc(m, layout=7)), None, None) == m.ERR_LAYOUT
    assert v(None, 0, 1, 1, None, ref(_desc(m, null=True)), None, None) == m.ERR_NULL
    assert v(None, 0, 1, 1, None, ref(_desc(m, K=48)), None, None) == m.ERR_SHAPE


def test_spgemm_gather_rejects(m):
    g = m._spgemm_gather
    ref = ctypes.byref
    d = ref(_desc(m))
    assert g(0x10, 0x10, -1, 2, 0x10, d, 0, 0x10, None, 0, None) == m.ERR_SHAPE      # T < 0
    assert g(0x10, 0x10, 4, 0, 0x10, d, 0, 0x10, None, 0, None) == m.ERR_SHAPE       # k < 1
    assert g(0x10, 0x10, 1 << 30, 4, 0x10, d, 0, 0x10, None, 0, None) == m.ERR_SHAPE  # T*k >= 2^31
    assert g(0x10, None, 4, 2, 0x10, d, 0, 0x10, None, 0, None) == m.ERR_NULL        # perm NULL
    assert g(0x10, 0x10, 4, 2, None, d, 0, 0x10, None, 0, None) == m.ERR_NULL        # offsets NULL
    assert g(0x10, 0x10, 4, 2, 0x10, ref(_desc(m, layout=7)), 0, 0x10, None, 0, None) == m.ERR_LAYOUT
    assert g(0x10, 0x10, 4, 2, 0x10, d, 5, 0x10, None, 0, None) == m.ERR_ARG         # epilogue
    assert g(0x10, 0x10, 4, 2, 0x10, d, m.OUT_FLAT | 2, 0x10, None, 0, None) == m.ERR_ARG
    assert g(None, None, 0, 2, 0x10, d, 0, None, None, 0, None) == m.OK              # T = 0


def test_paired_rejects(m):
    ref = ctypes.byref
    pp = m._pack_paired
    assert pp(0x10, 1, 16, 48, 0x10, 0x10, 0x10, 0x10, None) == m.ERR_SHAPE      # K % 32
    assert pp(0x10, 0, 16, 64, 0x10, 0x10, 0x10, 0x10, None) == m.ERR_SHAPE      # E = 0
    assert pp(0x10, 1, 16, 64, 0x10, None, 0x10, 0x10, None) == m.ERR_NULL       # patterns NULL
    g = m._spgemm
    # canonical paired weights must be tiled before the GEMM
    assert g(0x10, 0x10, 4, ref(_desc(m, layout=m.LAYOUT_PAIRED)), 0, 0x10, None, 0,
             None) == m.ERR_LAYOUT
    assert b"tiled first" in m._last_error()
    # the paired tiled layout needs N % 32 and K % 64
    assert g(0x10, 0x10, 4, ref(_desc(m, N=48, layout=m.LAYOUT_PAIRED_TILED)), 0, 0x10, None, 0,
             None) == m.ERR_SHAPE
    assert g(0x10, 0x10, 4, ref(_desc(m, K=96, layout=m.LAYOUT_PAIRED_TILED)), 0, 0x10, None, 0,
             None) == m.ERR_SHAPE
    # tiling takes canonical or paired sources only
    assert m._tile(ref(_desc(m, layout=m.LAYOUT_PAIRED_TILED)), 0x10, 0x10, 0x10,
                   None) == m.ERR_LAYOUT
    assert m._tile(ref(_desc(m, N=48, layout=m.LAYOUT_PAIRED)), 0x10, 0x10, 0x10,
                   None) == m.ERR_SHAPE
    assert m._decode(ref(_desc(m, K=96, layout=m.LAYOUT_PAIRED_TILED)), 0, 0x10,
                     None) == m.ERR_SHAPE
    assert m._decode(ref(_desc(m, layout=4)), 0, 0x10, None) == m.ERR_LAYOUT


def test_stream_read_rejects(m):
    sr = m._stream_read
    assert sr(None, 16, 0x10, None) == m.ERR_NULL
    assert sr(0x10, 16, None, None) == m.ERR_NULL
    assert sr(0x10, 24, 0x10, None) == m.ERR_ARG      # bytes % 16
    assert sr(0x18, 16, 0x10, None) == m.ERR_ARG      # misaligned buffer
    assert sr(0x10, 0, 0x10, None) == m.OK            # nothing to read


def test_route_spgemm_rejects(m):
    ref = ctypes.byref
    f = m._route_spgemm
    d = ref(_desc(m))
    assert f(0x10, 0x10, 4, 2, None, 0, 0x10, 0x10, 0x10, 0x10, None) == m.ERR_NULL     # descriptor
    assert f(0x10, 0x10, -1, 2, d, 0, 0x10, 0x10, 0x10, 0x10, None) == m.ERR_SHAPE      # T < 0
    assert f(0x10, 0x10, 4, 0, d, 0, 0x10, 0x10, 0x10, 0x10, None) == m.ERR_SHAPE       # k < 1
    assert f(0x10, 0x10, 4, 9, ref(_desc(m, E=8)), 0, 0x10, 0x10, 0x10, 0x10,
             None) == m.ERR_SHAPE                                                       # k > E
    assert f(0x10, 0x10, 4, 2, d, 5, 0x10, 0x10, 0x10, 0x10, None) == m.ERR_ARG         # epilogue
    assert f(0x10, 0x10, 4, 2, d, 0, 0x10, None, 0x10, 0x10, None) == m.ERR_NULL        # offsets
    assert f(None, 0x10, 4, 2, d, 0, 0x10, 0x10, 0x10, 0x10, None) == m.ERR_NULL        # ids


# ---------------------------------------------------------------- binding size checks

def _fake_weights(m, E=8, N=128, K=256):
    """A weight descriptor stand-in on the CPU (the size checks run before any
    pointer is taken)."""
    import types
    return types.SimpleNamespace(E=E, N=N, K=K, desc=_desc(m, E, N, K))


def test_binding_rejects_mismatched_sizes(m):
    """Every mirror of a C call compares the tensors' element counts with the
    shape arguments before any pointer reaches the library, so a mismatched
    tensor raises ValueError instead of being read or written out of bounds."""
    import torch
    i32, bf, u8, f32 = torch.int32, torch.bfloat16, torch.uint8, torch.float32
    z = lambda *s, dt=i32: torch.zeros(*s, dtype=dt)          # noqa: E731
    w = _fake_weights(m)
    T, k, E, K, N = 4, 2, 8, 256, 128
    cases = [
        lambda: m.moesq_route(z(T * k + 1), T, k, E, z(E + 1), z(T * k), z(T * k)),
        lambda: m.moesq_route(z(T * k), T, k, E, z(E), z(T * k), z(T * k)),
        lambda: m.moesq_route(z(T * k), T, k, E, z(E + 1), z(T * k), z(T * k - 1)),
        lambda: m.moesq_permute(z(T, K + 8, dt=bf), z(T * k), T, k, K, z(T * k, K, dt=bf)),
        lambda: m.moesq_permute(z(T, K, dt=bf), z(T * k), T, k, K, z(T * k - 1, K, dt=bf)),
        lambda: m.moesq_grouped_spgemm(z(T * k, K - 32, dt=bf), z(E + 1), T * k, w, 0,
                                       z(T * k, N, dt=bf)),
        lambda: m.moesq_grouped_spgemm(z(T * k, K, dt=bf), z(E + 1), T * k, w, 0,
                                       z(T * k, N // 2, dt=bf)),          # plain epilogue: N cols
        lambda: m.moesq_grouped_spgemm(z(T * k, K, dt=bf), z(E + 1), T * k, w, m.EPI_SWIGLU,
                                       z(T * k, N, dt=bf)),               # SwiGLU: N/2 cols
        lambda: m.moesq_grouped_spgemm(z(T * k, K, dt=bf), z(E + 2), T * k, w, 0,
                                       z(T * k, N, dt=bf)),
        lambda: m.moesq_grouped_spgemm_gather(z(T + 1, K, dt=bf), z(T * k), T, k, z(E + 1), w, 0,
                                              z(T * k, N, dt=bf)),
        lambda: m.moesq_grouped_spgemm_gather(z(T, K, dt=bf), z(T), T, k, z(E + 1), w, 0,
                                              z(T * k, N, dt=bf)),
        lambda: m.moesq_route_grouped_spgemm(z(T * k), z(T, K, dt=bf), T, k, w, 0,
                                             z(T, N, dt=bf), z(E + 1), z(T * k), z(T * k)),
        lambda: m.moesq_route_grouped_spgemm(z(T * k), z(T, K, dt=bf), T, k, w, 0,
                                             z(T * k, N, dt=bf), z(E + 1), z(T * k), z(T)),
        lambda: m.moesq_unpermute(z(T * k, N, dt=bf), z(T * k), z(T * k, dt=f32), T, k, N,
                                  z(T * k, N, dt=bf)),                    # weighted: T rows
        lambda: m.moesq_unpermute(z(T * k, N, dt=bf), z(T * k), None, T, k, N,
                                  z(T, N, dt=bf)),                        # flat: T*k rows
        lambda: m.moesq_unpermute(z(T * k, N + 8, dt=bf), z(T * k), None, T, k, N,
                                  z(T * k, N, dt=bf)),
        lambda: m.moesq_pack_weights(z(1, 16, 64, dt=f32), 1, 16, 64, z(1, 16, 15, dt=u8),
                                     z(1, 16, 8, dt=u8), z(1, 16, 2, dt=u8), z(1, dt=f32)),
        lambda: m.moesq_pack_weights_paired(z(1, 16, 64, dt=f32), 1, 16, 64, z(1, 16, 16, dt=u8),
                                            z(1, 16, 8, dt=u8), z(1, 16, 2, dt=u8), z(1, dt=f32)),
        lambda: m.moesq_decode_weights(w, 0, z(N, K - 1, dt=bf)),
        # convenience wrappers: operand shapes against the weights
        lambda: m.grouped_spgemm(z(T * k, K + 64, dt=bf), z(E + 1), w),
        lambda: m.grouped_spgemm(z(T * k, K, dt=bf), z(E + 1), w, out=z(T * k + 1, N, dt=bf)),
        lambda: m.grouped_spgemm_gather(z(T, K // 2, dt=bf), z(T * k), k, z(E + 1), w),
        lambda: m.grouped_spgemm_gather(z(T, K, dt=bf), z(T * k), k, z(E + 1), w,
                                        out=z(T * k, N, dt=bf), epilogue=m.EPI_SWIGLU),
        lambda: m.route_grouped_spgemm(z(T * k), z(T, K - 32, dt=bf), k, w),
        lambda: m.unpermute(z(T * k + 2, N, dt=bf), z(T * k), None, T, k),
        lambda: m.route(z(T * k + 1), E, k),
        lambda: m.permute(z(T * K, dt=bf), z(T * k), k),
    ]
    for i, case in enumerate(cases):
        with pytest.raises(ValueError) as ei:
            case()
        msg = str(ei.value)
        assert "on the GPU" not in msg, (i, msg)


def test_w4a4_calls_reject(m):
    ref = ctypes.byref
    q = m._quant_act
    assert q(0x10, 4, 48, 0x10, 0x10, 0x10, None) == m.ERR_SHAPE        # K % 32
    assert q(0x10, -1, 64, 0x10, 0x10, 0x10, None) == m.ERR_SHAPE       # T < 0
    assert q(None, 4, 64, 0x10, 0x10, 0x10, None) == m.ERR_NULL
    assert q(0x10, 4, 64, 0x10, 0x10, None, None) == m.ERR_NULL          # row scales
    assert q(0x18, 4, 64, 0x10, 0x10, 0x10, None) == m.ERR_ARG           # misaligned x
    assert q(None, 0, 64, None, None, None, None) == m.OK                # nothing to do
    g = m._spgemm_act4
    d = ref(_desc(m))                                                    # E=8, N=128, K=256
    act = m.Act4Desc(0x10, 0x10, 0x10, 8, 256)
    assert g(None, None, 0, 1, 0x10, 8, d, 0, 0x10, None) == m.ERR_NULL  # no activation descriptor
    assert g(ref(m.Act4Desc(0x10, 0x10, 0x10, 8, 128)), None, 0, 1, 0x10, 8, d, 0, 0x10,
             None) == m.ERR_SHAPE                                        # K differs
    assert b"K differs" in m._last_error()
    assert g(ref(m.Act4Desc(0x10, 0x10, 0x10, 7, 256)), None, 0, 1, 0x10, 8, d, 0, 0x10,
             None) == m.ERR_SHAPE                                        # rows != M
    assert g(ref(act), 0x10, 4, 2, 0x10, 9, d, 0, 0x10, None) == m.ERR_SHAPE   # M != T*k
    assert g(ref(m.Act4Desc(None, 0x10, 0x10, 8, 256)), None, 0, 1, 0x10, 8, d, 0, 0x10,
             None) == m.ERR_NULL                                         # codes NULL
    assert g(ref(act), None, 0, 1, 0x10, 8, d, 5, 0x10, None) == m.ERR_ARG    # epilogue
    assert g(ref(act), None, 0, 1, 0x10, 8, d, m.OUT_FLAT, 0x10, None) == m.ERR_ARG  # flat needs perm
    assert g(ref(act), None, 0, 1, 0x10, 0, d, 0, None, None) == m.OK          # M = 0
