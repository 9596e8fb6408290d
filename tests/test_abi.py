"""C-ABI library on the CPU: it loads, exports every symbol the header declares, and its
host-side logic (sizes, argument checks, status strings) behaves; no kernel is launched."""
import ctypes
import os
import re

import pytest

import oracle
import weight_only_quantization_amd as hq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hq.LIB_PATH):
        from weight_only_quantization_amd import build
        build.build()
    return hq.load()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "hqq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hqq_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(hq.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_packed_bytes_match_oracle(lib):
    o = oracle.get()
    for nbits in (2, 3, 4):
        for rows, cols in [(1, 16), (3, 80), (16, 64), (7, 96), (1024, 1024), (11008, 4096)]:
            assert hq.hqq_packed_bytes(rows, cols, nbits) == o.packed_bytes(rows * cols, nbits)
    assert hq.hqq_packed_bytes(4, 4, 5) == 0 and hq.hqq_packed_bytes(0, 4, 4) == 0


def test_num_groups(lib):
    assert hq.hqq_num_groups(4096, 4096, 64) == 262144
    assert hq.hqq_num_groups(28672, 8192, 128) == 1835008
    assert hq.hqq_num_groups(3, 5, 4) == -1


def test_workspace_bytes(lib):
    assert hq.hqq_quantize_workspace_bytes(1024, 1024, 4, 64, 1, 20) > 0
    # 3-bit: axis 1 packs in the solve (two partial words per tile); axis 0 keeps one byte per code
    assert hq.hqq_quantize_workspace_bytes(64, 640, 3, 64, 1, 20) < hq.hqq_quantize_workspace_bytes(64, 640, 4, 64, 1, 20) + 4096
    assert hq.hqq_quantize_workspace_bytes(640, 64, 3, 64, 0, 20) >= 64 * 640
    assert hq.hqq_quantize_workspace_bytes(1024, 1024, 4, 48, 1, 20) == 0      # g does not divide
    assert hq.hqq_quantize_workspace_bytes(1024, 1024, 4, 64, 1, 65) == 0      # iters too large
    assert hq.hqq_quantize_workspace_bytes(1024, 1024, 5, 64, 1, 20) == 0      # nbits


FAKE = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: every case below fails validation


def quantize(lib, rows=64, cols=64, nbits=4, g=64, axis=1, iters=20, p=0.7, b=10.0, k=1.01, meta=0,
             W=FAKE, ws=FAKE, wsb=1 << 30, out=FAKE):
    return lib.hqq_quantize(W, rows, cols, nbits, g, axis, iters, p, b, k, out, out, out, meta, ws, wsb, None,
                            None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(nbits=5), hq.HQQ_ERR_INVALID_ARGUMENT),
    (dict(nbits=1), hq.HQQ_ERR_INVALID_ARGUMENT),
    (dict(axis=2), hq.HQQ_ERR_INVALID_ARGUMENT),
    (dict(g=48), hq.HQQ_ERR_INVALID_ARGUMENT),
    (dict(cols=96, g=48), hq.HQQ_ERR_UNSUPPORTED),
    (dict(rows=0), hq.HQQ_ERR_INVALID_ARGUMENT),
    (dict(iters=-1), hq.HQQ_ERR_INVALID_ARGUMENT),
    (dict(iters=65), hq.HQQ_ERR_INVALID_ARGUMENT),
    (dict(p=0.0), hq.HQQ_ERR_INVALID_ARGUMENT),
    (dict(p=1.5), hq.HQQ_ERR_INVALID_ARGUMENT),
    (dict(b=0.0), hq.HQQ_ERR_INVALID_ARGUMENT),
    (dict(k=-1.0), hq.HQQ_ERR_INVALID_ARGUMENT),
    (dict(meta=7), hq.HQQ_ERR_INVALID_ARGUMENT),
    (dict(W=None), hq.HQQ_ERR_INVALID_ARGUMENT),
    (dict(W=ctypes.c_void_p((1 << 20) + 2)), hq.HQQ_ERR_INVALID_ARGUMENT),
    (dict(ws=None), hq.HQQ_ERR_WORKSPACE),
    (dict(wsb=16), hq.HQQ_ERR_WORKSPACE),
    (dict(rows=16, cols=4, g=16, axis=0, nbits=4), hq.HQQ_ERR_UNSUPPORTED),
])
def test_quantize_rejects_before_launch(lib, kw, status):
    assert quantize(lib, **kw) == status
    assert hq.last_error() != ""


def test_dequantize_and_gemv_reject(lib):
    d = lib.hqq_dequantize
    assert d(FAKE, FAKE, FAKE, 2, 64, 64, 4, 64, 1, FAKE, None) == hq.HQQ_ERR_INVALID_ARGUMENT  # f64 meta
    assert d(None, FAKE, FAKE, 0, 64, 64, 4, 64, 1, FAKE, None) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert d(FAKE, FAKE, FAKE, 0, 64, 96, 4, 24, 1, FAKE, None) == hq.HQQ_ERR_UNSUPPORTED
    gv = lib.hqq_gemv_w4a16
    assert gv(FAKE, FAKE, FAKE, 64, 256, 32, FAKE, 1, FAKE, 0, None) == hq.HQQ_ERR_UNSUPPORTED
    assert gv(FAKE, FAKE, FAKE, 64, 200, 64, FAKE, 1, FAKE, 0, None) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert gv(FAKE, FAKE, FAKE, 24, 256, 64, FAKE, 1, FAKE, 0, None) == hq.HQQ_ERR_UNSUPPORTED
    assert gv(FAKE, FAKE, FAKE, 64, 256, 64, FAKE, 0, FAKE, 0, None) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert gv(FAKE, FAKE, FAKE, 64, 256, 64, FAKE, 1, FAKE, 9, None) == hq.HQQ_ERR_INVALID_ARGUMENT


def test_batched_products_reject(lib):
    """hqq_gemm_w4a16, hqq_gemm (every stored format) and hqq_gemm_w4a16_dx check shapes, formats and
    the workspace size before any launch."""
    ws = lib.hqq_gemm_workspace_bytes(256, 1024, 32)
    assert ws > 0 and lib.hqq_gemm_workspace_bytes(200, 1024, 32) == 0 and lib.hqq_gemm_workspace_bytes(256, 1000, 32) == 0
    g = lib.hqq_gemm
    ok = dict(N=256, K=1024, nbits=3, gs=64, axis=1, batch=32, ydt=0, wsb=ws)

    def call(**kw):
        a = dict(ok, **kw)
        return g(FAKE, FAKE, FAKE, a["N"], a["K"], a["nbits"], a["gs"], a["axis"], FAKE, a["batch"], FAKE, a["ydt"],
                 FAKE, a["wsb"], None)
    assert call(nbits=5) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(axis=2) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(gs=48) == hq.HQQ_ERR_INVALID_ARGUMENT          # does not divide K
    assert call(axis=0) == hq.HQQ_ERR_UNSUPPORTED              # axis 0 only at 4 bits
    assert call(nbits=4, gs=32) == hq.HQQ_ERR_UNSUPPORTED      # 4-bit axis 1: 64 or 128
    assert call(nbits=4, axis=0, gs=8, N=256) == hq.HQQ_ERR_UNSUPPORTED   # axis 0: 16..256
    assert call(nbits=4, axis=0, gs=64, N=96) == hq.HQQ_ERR_INVALID_ARGUMENT  # g must divide N
    assert call(nbits=2, gs=512) == hq.HQQ_ERR_UNSUPPORTED
    assert call(N=192) == hq.HQQ_ERR_UNSUPPORTED               # N % 128
    assert call(K=640) == hq.HQQ_ERR_UNSUPPORTED               # K % 256
    assert call(ydt=7) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(wsb=ws - 16) == hq.HQQ_ERR_WORKSPACE
    assert call(batch=0) == hq.HQQ_ERR_INVALID_ARGUMENT
    w4 = lib.hqq_gemm_w4a16
    assert w4(FAKE, FAKE, FAKE, 256, 1024, 32, FAKE, 32, FAKE, 0, FAKE, ws, None) == hq.HQQ_ERR_UNSUPPORTED
    assert w4(FAKE, FAKE, FAKE, 256, 1024, 64, FAKE, 32, FAKE, 0, FAKE, ws - 16, None) == hq.HQQ_ERR_WORKSPACE
    wdx = lib.hqq_gemm_dx_workspace_bytes(1024, 256, 32)
    assert wdx > 0 and lib.hqq_gemm_dx_workspace_bytes(1000, 256, 32) == 0
    dx = lib.hqq_gemm_w4a16_dx
    assert dx(FAKE, FAKE, FAKE, 1024, 200, 64, FAKE, 32, FAKE, 0, FAKE, wdx, None) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert dx(FAKE, FAKE, FAKE, 1024, 256, 64, FAKE, 32, FAKE, 0, FAKE, wdx - 16, None) == hq.HQQ_ERR_WORKSPACE
    gdx = lib.hqq_gemm_dx
    okd = dict(N=1024, K=256, nbits=3, gs=64, axis=1, batch=32, ydt=0, wsb=wdx)

    def call_dx(**kw):
        a = dict(okd, **kw)
        return gdx(FAKE, FAKE, FAKE, a["N"], a["K"], a["nbits"], a["gs"], a["axis"], FAKE, a["batch"], FAKE,
                   a["ydt"], FAKE, a["wsb"], None)
    assert call_dx(nbits=1) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call_dx(axis=0) == hq.HQQ_ERR_UNSUPPORTED           # axis 0 only at 4 bits
    assert call_dx(nbits=4, axis=0, gs=512) == hq.HQQ_ERR_UNSUPPORTED
    assert call_dx(gs=48) == hq.HQQ_ERR_INVALID_ARGUMENT      # does not divide K
    assert call_dx(nbits=4, gs=32) == hq.HQQ_ERR_UNSUPPORTED
    assert call_dx(nbits=2, gs=8) == hq.HQQ_ERR_UNSUPPORTED
    assert call_dx(K=192) == hq.HQQ_ERR_UNSUPPORTED           # K % 128
    assert call_dx(N=640) == hq.HQQ_ERR_UNSUPPORTED           # N % 256
    assert call_dx(ydt=5) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call_dx(wsb=wdx - 16) == hq.HQQ_ERR_WORKSPACE
    assert call_dx(batch=-1) == hq.HQQ_ERR_INVALID_ARGUMENT


def test_status_strings(lib):
    assert hq.status_string(0) == "HQQ_OK"
    assert hq.status_string(3) == "HQQ_ERR_WORKSPACE"
    assert hq.status_string(99) == "HQQ_ERR_UNKNOWN"


def test_quantize_v2_rejects_before_launch(lib):
    """hqq_quantize_v2 refuses an unknown axis or a shape its axis does not divide, a grid of 0 or more than
    HQQ_V2_MAX_CANDIDATES multipliers or one that is not finite and positive, a missing or
    small 3-bit workspace, and the shared argument errors, all before any launch."""
    grid = (ctypes.c_double * 17)(*([1.0] * 17))

    def call(**kw):
        a = dict(W_fp16=FAKE.value, rows=64, cols=128, nbits=4, group_size=64, axis=1, iters=20, p=0.7, beta0=10.0,
                 kappa=1.01, tiny_range=1e-4, scale_grid=ctypes.addressof(grid), n_candidates=3, packed=FAKE.value,
                 delta=FAKE.value, zero=FAKE.value, meta_dtype=0, choice_dev=None, stream=None, workspace=None,
                 workspace_bytes=0)
        a.update(kw)
        return lib.hqq_quantize_v2(ctypes.byref(hq.QuantV2Args(**a)))
    assert lib.hqq_quantize_v2(None) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(axis=2) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(axis=0, group_size=128) == hq.HQQ_ERR_INVALID_ARGUMENT  # 128 does not divide the 64 rows
    ws3 = lib.hqq_quantize_v2_workspace_bytes(64, 128, 3)
    assert ws3 >= 64 * 128 and lib.hqq_quantize_v2_workspace_bytes(64, 128, 4) == 0
    assert call(nbits=3) == hq.HQQ_ERR_WORKSPACE
    assert call(nbits=3, workspace=FAKE.value, workspace_bytes=ws3 - 1) == hq.HQQ_ERR_WORKSPACE
    assert call(nbits=3, workspace=FAKE.value + 8, workspace_bytes=ws3) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(nbits=5) == hq.HQQ_ERR_INVALID_ARGUMENT
    for n in (0, 17):
        assert call(n_candidates=n) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(scale_grid=None) == hq.HQQ_ERR_INVALID_ARGUMENT
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        grid[1] = bad
        assert call() == hq.HQQ_ERR_INVALID_ARGUMENT
    grid[1] = 1.0
    assert call(iters=65) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(p=0.0) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(tiny_range=-1.0) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(meta_dtype=7) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(packed=None) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(packed=FAKE.value + 8) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(group_size=48) != hq.HQQ_OK
    assert hq.last_error() != ""


def test_quantize_ex_rejects_before_launch(lib):
    """hqq_quantize_ex checks its own fields (stop rule, tiny range, flags) and then the same
    arguments as hqq_quantize, before any launch."""
    ws = lib.hqq_quantize_workspace_bytes(64, 128, 4, 64, 1, 20)

    def call(**kw):
        a = dict(W_fp16=FAKE.value, rows=64, cols=128, nbits=4, group_size=64, axis=1, iters=20, p=0.7, beta0=10.0,
                 kappa=1.01, packed=FAKE.value, delta=FAKE.value, zero=FAKE.value, meta_dtype=0,
                 workspace=FAKE.value, workspace_bytes=ws, stop_iter_dev=None, mae_trace_dev=None, stream=None,
                 stop_rule=0, tiny_range=1e-4, debug_flags=0)
        a.update(kw)
        return lib.hqq_quantize_ex(ctypes.byref(hq.QuantArgs(**a)))
    assert lib.hqq_quantize_ex(None) == hq.HQQ_ERR_INVALID_ARGUMENT
    for rule in (-1, 3, 7, 8):
        assert call(stop_rule=rule) == hq.HQQ_ERR_INVALID_ARGUMENT
    for t in (-1e-4, float("inf"), float("nan")):
        assert call(tiny_range=t) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(debug_flags=8) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(nbits=5) != hq.HQQ_OK                       # the shared checks of hqq_quantize follow
    assert call(workspace_bytes=ws - 8) == hq.HQQ_ERR_WORKSPACE
    assert call(p=0.0) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert hq.last_error() != ""


def test_probe_library_exports_and_checks():
    """libhqq_probe.so (include/hqq_probe.h) loads, exports what its header declares and refuses
    invalid arguments before any launch."""
    if not os.path.exists(hq.PROBE_LIB_PATH):
        from weight_only_quantization_amd import build
        build.build()
    plib = hq.load_probe()
    src = open(os.path.join(ROOT, "include", "hqq_probe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = sorted(set(re.findall(r"\b(hqq_probe_[a-z0-9_]+)\s*\(", src)))
    assert set(names) == set(hq.PROBE_EXPORTS), names
    for n in names:
        assert hasattr(plib, n), n
    assert plib.hqq_probe_copy(FAKE, FAKE, 24, 4, None) == 1          # not a multiple of 16
    assert plib.hqq_probe_copy(FAKE, FAKE, 4096, 5, None) == 1        # unroll
    assert plib.hqq_probe_copy(None, FAKE, 4096, 4, None) == 1
    p3 = (ctypes.c_void_p * 1)(FAKE.value)
    assert plib.hqq_probe_read(p3, (ctypes.c_size_t * 1)(4096), 0, FAKE, 4, None) == 1    # nbuf
    assert plib.hqq_probe_read(p3, (ctypes.c_size_t * 1)(4100), 1, FAKE, 4, None) == 1    # size
    assert plib.hqq_probe_read(p3, (ctypes.c_size_t * 1)(4096), 1, None, 4, None) == 1    # sink


def test_noalloc_rejects_before_any_device_call(lib):
    """hqq_quantize_noalloc checks the shape and its scratch need before it touches the device."""
    i64 = ctypes.c_int64
    def call(rows, cols, nbits, g, axis, iters):
        return lib.hqq_quantize_noalloc(FAKE, rows, cols, nbits, g, axis, iters, 0.7, 10.0, 1.01, FAKE, FAKE, FAKE,
                                        hq.HQQ_META_F16, None, None, None)
    # 4-bit g64 at 20 rounds over 65536x8192: 42 MB of per-round sums, beyond the array
    need = hq.hqq_quantize_workspace_bytes(65536, 8192, 4, 64, 1, 20)
    assert need > hq.HQQ_NOALLOC_SCRATCH_BYTES
    assert call(65536, 8192, 4, 64, 1, 20) == hq.HQQ_ERR_WORKSPACE
    assert "scratch" in hq.last_error()
    assert call(8192, 8192, 3, 64, 0, 20) == hq.HQQ_ERR_WORKSPACE      # 3-bit axis 0: a byte per code
    assert call(64, 64, 5, 64, 1, 20) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(64, 64, 4, 64, 1, 65) == hq.HQQ_ERR_INVALID_ARGUMENT
    assert call(64, 96, 4, 64, 1, 20) == hq.HQQ_ERR_INVALID_ARGUMENT    # 64 does not divide 96
