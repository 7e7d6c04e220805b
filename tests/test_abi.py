"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before any kernel launch (no GPU needed:
every call here fails validation, so nothing is enqueued)."""
import ctypes
import functools

import pytest

from group_circulant_linear_amd import eqlin

OK, EINVAL, ENOTSUP, EALIGN, EWORKSPACE = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    return eqlin.load_library()


def test_exports_every_header_symbol(lib):
    names = eqlin.header_symbols()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.eqlin_version() >= 100
    for s in range(6):
        assert lib.eqlin_status_str(s)
    assert lib.eqlin_status_str(99) == b"unknown status"
    assert lib.eqlin_last_hip_error() == 0


def test_size_queries(lib):
    # rows x ceil(groups / S) stage blocks of 256 bytes (S = 16 fp32, 32 f16),
    # forward set then the transposed set at a 256 B boundary
    assert lib.eqlin_prepared_transpose_offset(768, 768, 4, 0) == 192 * 12 * 256
    assert lib.eqlin_prepared_weight_bytes(768, 768, 4, 0) == 2 * 192 * 12 * 256
    assert lib.eqlin_prepared_weight_bytes(768, 3072, 4, 1) == 768 * 6 * 256 + 192 * 24 * 256
    off = lib.eqlin_prepared_transpose_offset(4, 4, 4, 0)
    assert off == 256 and lib.eqlin_prepared_weight_bytes(4, 4, 4, 0) == 512
    # 20 input groups -> 2 stage blocks per forward row (zero padded)
    assert lib.eqlin_prepared_transpose_offset(80, 12, 4, 0) == 3 * 2 * 256
    assert lib.eqlin_prepared_weight_bytes(768, 768, 3, 0) == 0
    assert lib.eqlin_prepared_weight_bytes(770, 768, 4, 0) == 0
    assert lib.eqlin_prepared_weight_bytes(12, 16, 4, 1) == 0      # odd C' with f16
    assert lib.eqlin_backward_workspace_bytes(0, 768, 768, 4, 0) == 0
    ws = lib.eqlin_backward_workspace_bytes(12608, 768, 768, 4, 0)
    assert ws > 0 and ws % (4 * 192 * 192 * 4) == 0
    # narrow fp32 layers read rows in chunks of 4 (here 50432 chunked rows, 112
    # per split: 451 splits, two per CU), each split still one D' x C' partial per plane
    assert lib.eqlin_backward_workspace_bytes(201728, 64, 64, 4, 0) == 451 * 4 * 16 * 16 * 4
    assert lib.eqlin_backward_workspace_bytes(201728, 64, 64, 4, 1) == 485 * 4 * 16 * 16 * 4   # f16: whole rows
    assert lib.eqlin_backward_workspace_bytes(1002, 64, 32, 4, 0) % (4 * 8 * 16 * 4) == 0


def test_size_queries_c8(lib):
    # C8: stage blocks of 8 planes x 64 bytes = 512 bytes; 96 groups -> 6 (fp32) / 3 (f16) blocks
    assert lib.eqlin_prepared_transpose_offset(768, 768, 8, 0) == 96 * 6 * 512
    assert lib.eqlin_prepared_weight_bytes(768, 768, 8, 0) == 2 * 96 * 6 * 512
    assert lib.eqlin_prepared_weight_bytes(768, 3072, 8, 1) == 384 * 3 * 512 + 96 * 12 * 512
    assert lib.eqlin_prepared_weight_bytes(8, 8, 8, 0) == 1024
    # odd group counts are fine with f16 when a group is 16 bytes
    assert lib.eqlin_prepared_weight_bytes(40, 24, 8, 1) == 3 * 512 + 5 * 512
    assert lib.eqlin_prepared_weight_bytes(36, 32, 8, 0) == 0      # C not a multiple of 8
    assert lib.eqlin_prepared_weight_bytes(48, 48, 6, 0) == 0      # only T = 4 and T = 8
    ws = lib.eqlin_backward_workspace_bytes(12608, 768, 768, 8, 0)
    assert ws > 0 and ws % (8 * 96 * 96 * 4) == 0


P4M = 108   # EQLIN_P4M


def test_size_queries_p4m(lib):
    # p4m has 8 planes per group channel like C8: identical layout sizes
    for C, D, dt in ((768, 768, 0), (768, 3072, 1), (40, 24, 1), (8, 8, 0)):
        assert lib.eqlin_prepared_weight_bytes(C, D, P4M, dt) == lib.eqlin_prepared_weight_bytes(C, D, 8, dt)
        assert lib.eqlin_prepared_transpose_offset(C, D, P4M, dt) == lib.eqlin_prepared_transpose_offset(C, D, 8, dt)
    assert lib.eqlin_backward_workspace_bytes(12608, 768, 768, P4M, 0) == \
        lib.eqlin_backward_workspace_bytes(12608, 768, 768, 8, 0)
    assert lib.eqlin_prepared_weight_bytes(36, 32, P4M, 0) == 0


FAKE = ctypes.c_void_p(0x1000)        # aligned, never dereferenced (validation fails first)
MISALIGNED = ctypes.c_void_p(0x1004)


def test_forward_validation(lib):
    f = lib.eqlin_forward
    assert f(FAKE, 8, 32, 32, 3, FAKE, FAKE, 0, None) == ENOTSUP
    assert f(FAKE, 8, 30, 32, 4, FAKE, FAKE, 0, None) == EINVAL
    assert f(FAKE, 8, 32, 0, 4, FAKE, FAKE, 0, None) == EINVAL
    assert f(FAKE, -1, 32, 32, 4, FAKE, FAKE, 0, None) == EINVAL
    assert f(FAKE, 8, 32, 32, 4, FAKE, FAKE, 7, None) == EINVAL
    assert f(None, 8, 32, 32, 4, FAKE, FAKE, 0, None) == EINVAL
    assert f(FAKE, 8, 32, 32, 4, None, FAKE, 0, None) == EINVAL
    assert f(MISALIGNED, 8, 32, 32, 4, FAKE, FAKE, 0, None) == EALIGN
    assert f(FAKE, 8, 32, 32, 4, FAKE, MISALIGNED, 0, None) == EALIGN
    assert f(FAKE, 8, 20, 32, 4, FAKE, FAKE, 1, None) == ENOTSUP   # C'=5 odd with f16
    assert f(FAKE, 8, 36, 32, 8, FAKE, FAKE, 0, None) == EINVAL    # C not a multiple of 8
    assert f(FAKE, 8, 48, 48, 6, FAKE, FAKE, 0, None) == ENOTSUP
    assert f(FAKE, 8, 36, 32, P4M, FAKE, FAKE, 0, None) == EINVAL   # C not a multiple of 8
    assert f(FAKE, 8, 48, 48, 107, FAKE, FAKE, 0, None) == ENOTSUP
    assert f(MISALIGNED, 8, 40, 32, 8, FAKE, FAKE, 1, None) == EALIGN
    assert f(None, 0, 32, 32, 4, None, None, 0, None) == OK        # empty batch: nothing enqueued


def test_prepare_validation(lib):
    p = lib.eqlin_prepare_weights
    need = lib.eqlin_prepared_weight_bytes(32, 32, 4, 0)
    assert p(FAKE, 32, 32, 4, 0, FAKE, need - 1, None) == EWORKSPACE
    assert p(None, 32, 32, 4, 0, FAKE, need, None) == EINVAL
    assert p(MISALIGNED, 32, 32, 4, 0, FAKE, need, None) == EALIGN
    assert p(FAKE, 32, 32, 5, 0, FAKE, need, None) == ENOTSUP


def test_backward_validation(lib):
    b = lib.eqlin_backward
    ws = lib.eqlin_backward_workspace_bytes(64, 32, 32, 4, 0)
    assert b(FAKE, FAKE, 64, 32, 32, 4, FAKE, None, None, FAKE, ws, 0, None) == EINVAL   # nothing requested
    assert b(FAKE, FAKE, 64, 32, 32, 4, FAKE, FAKE, FAKE, FAKE, ws - 1, 0, None) == EWORKSPACE
    assert b(FAKE, None, 64, 32, 32, 4, FAKE, None, FAKE, FAKE, ws, 0, None) == EINVAL   # dw without X
    assert b(FAKE, FAKE, 64, 32, 32, 4, FAKE, FAKE, FAKE, None, ws, 0, None) == EINVAL   # dw without workspace
    assert b(FAKE, FAKE, 64, 32, 32, 4, None, FAKE, None, None, 0, 0, None) == EINVAL    # dX without W_hat
    assert b(FAKE, FAKE, 64, 32, 32, 4, FAKE, MISALIGNED, FAKE, FAKE, ws, 0, None) == EALIGN
    assert b(FAKE, FAKE, 64, 32, 32, 2, FAKE, FAKE, FAKE, FAKE, ws, 0, None) == ENOTSUP
    d = lib.eqlin_backward_dw
    assert d(FAKE, FAKE, 64, 32, 32, 4, None, FAKE, ws, 0, None) == EINVAL
    assert d(FAKE, FAKE, 64, 32, 32, 4, FAKE, FAKE, 0, 0, None) == EWORKSPACE
    x = lib.eqlin_backward_dx
    assert x(FAKE, 64, 32, 32, 4, FAKE, None, 0, None) == EINVAL
    assert x(None, 0, 32, 32, 4, None, None, 0, None) == OK


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    w = torch.zeros(8, 8, 4)
    with pytest.raises(ValueError):
        eqlin.eqlin_prepare_weights(w)


def test_forward_ex_validation(lib):
    f = lib.eqlin_forward_ex
    assert f(FAKE, 8, 32, 32, 4, FAKE, None, 2, FAKE, 0, None) == EINVAL        # unknown activation
    assert f(FAKE, 8, 32, 32, 4, FAKE, ctypes.c_void_p(0x1001), 1, FAKE, 0, None) == EALIGN  # misaligned fp32 bias
    assert f(FAKE, 8, 32, 32, 3, FAKE, None, 1, FAKE, 0, None) == ENOTSUP
    assert f(None, 0, 32, 32, 4, None, None, 1, None, 0, None) == OK            # empty batch


def test_forward_residual_validation(lib):
    f = lib.eqlin_forward_residual
    assert f(FAKE, 8, 32, 32, 4, FAKE, None, 2, FAKE, FAKE, 0, None) == EINVAL        # unknown activation
    assert f(FAKE, 8, 32, 32, 4, FAKE, None, 1, ctypes.c_void_p(0x1008), FAKE, 0, None) == EALIGN  # residual
    assert f(FAKE, 8, 32, 32, 4, FAKE, None, 1, FAKE, None, 0, None) == EINVAL        # no output
    assert f(FAKE, 8, 32, 32, 3, FAKE, None, 1, FAKE, FAKE, 0, None) == ENOTSUP
    assert f(None, 0, 32, 32, 4, None, None, 1, None, None, 0, None) == OK            # empty batch


# ------------------------------------------------------------ p4 group convolution

def test_conv_size_queries(lib):
    # gathered groups C'K^2 padded to whole 16 (fp32) / 32 (f16) group blocks of 256 bytes
    # C = D = 256, K = 3, fp32: 64 * 9 = 576 groups = 36 blocks per row, 64 rows per set
    assert lib.eqconv_prepared_adjoint_offset(256, 256, 3, 0) == 64 * 36 * 256
    assert lib.eqconv_prepared_weight_bytes(256, 256, 3, 0) == 2 * 64 * 36 * 256
    # C' = 4, K = 3: 36 groups -> 3 fp32 blocks; D' = 8: 72 groups -> 5 blocks
    assert lib.eqconv_prepared_adjoint_offset(16, 32, 3, 0) == 8 * 3 * 256
    assert lib.eqconv_prepared_weight_bytes(16, 32, 3, 0) == 8 * 3 * 256 + 4 * 5 * 256
    # K = 1 is the linear layer's layout
    assert lib.eqconv_prepared_weight_bytes(768, 768, 1, 0) == lib.eqlin_prepared_weight_bytes(768, 768, 4, 0)
    # f16 needs C', D' multiples of 8; fp32 multiples of 4
    assert lib.eqconv_prepared_weight_bytes(16, 32, 3, 1) == 0
    assert lib.eqconv_prepared_weight_bytes(32, 32, 3, 1) > 0
    assert lib.eqconv_prepared_weight_bytes(24, 32, 3, 0) == 0
    for K in (0, 2, -1, 17):
        assert lib.eqconv_prepared_weight_bytes(16, 16, K, 0) == 0
    assert lib.eqconv_backward_workspace_bytes(-1, 8, 8, 16, 16, 3, 0) == 0
    ws0 = lib.eqconv_backward_workspace_bytes(0, 8, 8, 16, 16, 3, 0)
    assert ws0 == (4 * 48 * 4 * 4 + 255) // 256 * 256        # the gathered layer's dw only
    # plus whole split partials (4 planes x D' x gathered groups, fp32); no gathered copy of X
    ws = lib.eqconv_backward_workspace_bytes(2, 8, 8, 16, 16, 3, 0)
    assert ws > ws0 and (ws - ws0) % (4 * 4 * 48 * 4) == 0 and ws - ws0 < 128 * 48 * 4 * 4


def test_conv_validation(lib):
    st = lib.eqconv_forward
    # bad dtype, sizes, K, act
    assert st(FAKE, 1, 4, 4, 16, 16, 3, FAKE, None, 0, FAKE, 2, None) == EINVAL
    assert st(FAKE, -1, 4, 4, 16, 16, 3, FAKE, None, 0, FAKE, 0, None) == EINVAL
    assert st(FAKE, 1, -4, 4, 16, 16, 3, FAKE, None, 0, FAKE, 0, None) == EINVAL
    assert st(FAKE, 1, 4, 4, 18, 16, 3, FAKE, None, 0, FAKE, 0, None) == EINVAL
    assert st(FAKE, 1, 4, 4, 16, 16, 2, FAKE, None, 0, FAKE, 0, None) == EINVAL
    assert st(FAKE, 1, 4, 4, 16, 16, 17, FAKE, None, 0, FAKE, 0, None) == ENOTSUP
    assert st(FAKE, 1, 4, 4, 24, 16, 3, FAKE, None, 0, FAKE, 0, None) == ENOTSUP   # C' = 6
    assert st(FAKE, 1, 4, 4, 16, 16, 3, FAKE, None, 0, FAKE, 1, None) == ENOTSUP   # f16 needs C' % 8
    assert st(FAKE, 1, 4, 4, 16, 16, 3, FAKE, None, 7, FAKE, 0, None) == EINVAL
    # null and misaligned pointers
    assert st(None, 1, 4, 4, 16, 16, 3, FAKE, None, 0, FAKE, 0, None) == EINVAL
    assert st(FAKE, 1, 4, 4, 16, 16, 3, None, None, 0, FAKE, 0, None) == EINVAL
    assert st(MISALIGNED, 1, 4, 4, 16, 16, 3, FAKE, None, 0, FAKE, 0, None) == EALIGN
    assert st(FAKE, 1, 4, 4, 16, 16, 3, FAKE, ctypes.c_void_p(0x1001), 0, FAKE, 0, None) == EALIGN
    # an input map of 2^31 bytes or more
    assert st(FAKE, 1 << 12, 128, 128, 32, 16, 3, FAKE, None, 0, FAKE, 0, None) == ENOTSUP
    # empty batches are no-ops (nothing launched)
    assert st(None, 0, 4, 4, 16, 16, 3, None, None, 0, None, 0, None) == OK
    assert st(None, 3, 0, 4, 16, 16, 3, None, None, 0, None, 0, None) == OK
    # prepare
    pw = lib.eqconv_prepare_weights
    need = lib.eqconv_prepared_weight_bytes(16, 16, 3, 0)
    assert pw(FAKE, 16, 16, 3, 0, FAKE, need - 1, None) == EWORKSPACE
    assert pw(None, 16, 16, 3, 0, FAKE, need, None) == EINVAL
    assert pw(FAKE, 16, 16, 3, 0, MISALIGNED, need, None) == EALIGN
    assert pw(FAKE, 16, 16, 4, 0, FAKE, need, None) == EINVAL
    # backward
    bw = lib.eqconv_backward
    ws = lib.eqconv_backward_workspace_bytes(1, 4, 4, 16, 16, 3, 0)
    assert bw(FAKE, FAKE, 1, 4, 4, 16, 16, 3, FAKE, None, None, FAKE, ws, 0, None) == EINVAL   # nothing asked
    assert bw(FAKE, FAKE, 1, 4, 4, 16, 16, 3, FAKE, None, FAKE, FAKE, ws - 1, 0, None) == EWORKSPACE
    assert bw(FAKE, FAKE, 1, 4, 4, 16, 16, 3, FAKE, None, FAKE, None, ws, 0, None) == EINVAL
    assert bw(FAKE, None, 1, 4, 4, 16, 16, 3, FAKE, None, FAKE, FAKE, ws, 0, None) == EINVAL
    assert bw(FAKE, FAKE, 1, 4, 4, 16, 16, 3, FAKE, MISALIGNED, FAKE, FAKE, ws, 0, None) == EALIGN
    assert bw(None, FAKE, 1, 4, 4, 16, 16, 3, FAKE, FAKE, None, None, 0, 0, None) == EINVAL
    # validation of the dpsi half runs before the dX launch
    assert bw(FAKE, FAKE, 1, 4, 4, 16, 16, 3, FAKE, FAKE, FAKE, FAKE, ws - 1, 0, None) == EWORKSPACE
    # empty batch with dX only: no-op
    assert bw(None, None, 0, 4, 4, 16, 16, 3, None, FAKE, None, None, 0, 0, None) == OK
    # an X map of 2^31 bytes or more is refused for dpsi (dY small: C = 4 D)
    big = (1 << 12, 128, 128, 64, 16, 3)
    wsb = lib.eqconv_backward_workspace_bytes(*big, 0)
    assert bw(FAKE, FAKE, *big, FAKE, None, FAKE, FAKE, wsb, 0, None) == ENOTSUP


def _plan(lib, N, C, D, T, dt):
    tile, tiles, whole = ctypes.c_int(-1), ctypes.c_int64(-1), ctypes.c_int64(-1)
    st = lib.eqlin_forward_plan(N, C, D, T, dt, ctypes.byref(tile), ctypes.byref(tiles), ctypes.byref(whole))
    return st, tile.value, tiles.value, whole.value


def test_forward_plan_tiles_and_tail_split(lib, monkeypatch):
    # the host's tile choice and float32 tail split for the benchmark shapes
    # (no device work): tiles = ceil(N / rows) * ceil(D' / cols); the last
    # round over the 256 CUs runs as halves when it is at most half full
    monkeypatch.delenv("EQLIN_FWD_TILE", raising=False)
    monkeypatch.delenv("EQLIN_FWD_SPLIT", raising=False)
    assert _plan(lib, 12608, 768, 768, 4, 0) == (OK, 112211, 197 * 3, 512)       # ViT-B attention fp32
    assert _plan(lib, 8224, 1280, 5120, 4, 0) == (OK, 112211, 129 * 20, 2560)    # ViT-H fc1 fp32
    assert _plan(lib, 8224, 5120, 1280, 4, 0) == (OK, 112211, 129 * 5, 645)      # last round 133 > 128
    assert _plan(lib, 12608, 768, 3072, 4, 1) == (OK, 122241, 197 * 6, 1182)     # f16: 64 x 128, no split
    assert _plan(lib, 8224, 1280, 5120, 4, 1) == (OK, 212431, 65 * 10, 650)      # f16: 128 x 128
    assert _plan(lib, 12608, 768, 768, 8, 0) == (OK, 112211, 197 * 2, 394)       # C8: last round 138
    assert _plan(lib, 12608, 768, 768, 8, 1) == (OK, 122241, 197, 197)          # C8 f16: 64 x 128, weight DMA
    assert _plan(lib, 12608, 768, 768, 108, 1) == (OK, 122241, 197, 197)        # p4m f16: same table
    assert _plan(lib, 8224, 5120, 1280, 8, 1) == (OK, 2122111, 65 * 3, 195)     # C8 f16: 128 x 64 stream
    assert _plan(lib, 201728, 64, 64, 4, 0) == (OK, 112111, 3152, 3072)         # narrow fp32: 64 x 32
    assert _plan(lib, 201728, 64, 64, 4, 1) == (OK, 1121111, 3152, 3152)        # narrow f16: persistent 64 x 32
    assert _plan(lib, 201728, 64, 192, 4, 0)[1] == 112211                       # 48 output groups: 64 x 64
    assert _plan(lib, 0, 768, 768, 4, 0) == (OK, 112211, 0, 0)
    monkeypatch.setenv("EQLIN_FWD_SPLIT", "0")
    assert _plan(lib, 12608, 768, 768, 4, 0)[3] == 591
    monkeypatch.delenv("EQLIN_FWD_SPLIT")
    monkeypatch.setenv("EQLIN_FWD_TILE", "111211")                                # one wave row: never split
    assert _plan(lib, 12608, 768, 768, 4, 0) == (OK, 111211, 394 * 3, 1182)
    monkeypatch.setenv("EQLIN_FWD_TILE", "212421")
    assert _plan(lib, 12608, 768, 768, 4, 0) == (OK, 212421, 99 * 2, 198)
    monkeypatch.setenv("EQLIN_FWD_TILE", "122241")                                # weight DMA: never split
    assert _plan(lib, 8224, 5120, 1280, 4, 0) == (OK, 122241, 129 * 3, 387)
    monkeypatch.setenv("EQLIN_FWD_TILE", "112241")
    assert _plan(lib, 8224, 5120, 1280, 4, 0) == (OK, 112241, 129 * 5, 645)
    monkeypatch.setenv("EQLIN_FWD_TILE", "123456")                                # not compiled: ignored
    assert _plan(lib, 12608, 768, 768, 4, 0)[1] == 112211
    assert _plan(lib, 12608, 770, 768, 4, 0)[0] == EINVAL
    assert _plan(lib, 16, 12, 16, 4, 1)[0] == ENOTSUP                             # odd C' with f16
    st = lib.eqlin_forward_plan(12608, 768, 768, 4, 0, None, None, None)
    assert st == OK


def _ws(lib, N, C, D, T, dt):
    parts = ctypes.c_int(-1)
    nbytes = lib.eqlin_forward_workspace_bytes(N, C, D, T, dt, ctypes.byref(parts))
    return nbytes, parts.value


def test_forward_k_split_plan(lib, monkeypatch):
    # eqlin_forward_ws's K split of the last round (no device work): parts p
    # minimise ceil(tail p / 256) ceil(stages / p) / stages, at least 10%
    # below the other choice (half a tile with the tail split, else a whole
    # tile); workspace = 1024 bytes of counters + tail x p slots of
    # T x 64 x 64 float32 (the 64 x 64 tile) or T x 32 x 64 (32 x 64)
    monkeypatch.delenv("EQLIN_FWD_TILE", raising=False)
    monkeypatch.delenv("EQLIN_FWD_SPLIT", raising=False)
    slot = 4 * 64 * 64 * 4
    assert _ws(lib, 12608, 768, 768, 4, 0) == (1024 + 79 * 3 * slot, 3)        # ViT-B attention: 591 tiles, 12 stages
    assert _ws(lib, 12608, 3072, 768, 4, 0) == (1024 + 79 * 3 * slot, 3)       # ViT-B fc2: 48 stages
    assert _ws(lib, 12608, 768, 3072, 4, 0) == (1024 + 60 * 4 * slot, 4)       # ViT-B fc1: tail 60 of 2364
    assert _ws(lib, 8224, 1280, 5120, 4, 0) == (1024 + 20 * 4 * slot, 4)       # ViT-H fc1: tail 20 of 2580
    assert _ws(lib, 8224, 5120, 1280, 4, 0) == (1024 + 133 * 3 * slot, 3)      # ViT-H fc2: tail 133, no halves
    assert _ws(lib, 12608, 768, 768, 8, 0) == (0, 0)                            # order 8: never
    assert _ws(lib, 12608, 768, 768, 108, 0) == (0, 0)
    assert _ws(lib, 2171, 768, 768, 4, 0) == (1024 + 204 * 2 * slot // 2, 2)   # 204 tiles of 32 x 64
    assert _ws(lib, 12608, 768, 768, 4, 1) == (0, 0)                            # f16: never
    assert _ws(lib, 201728, 64, 64, 4, 0) == (0, 0)                             # one k stage
    assert _ws(lib, 16448, 768, 768, 4, 0) == (1024 + 3 * 4 * slot, 4)         # 771 tiles: tail 3
    assert _ws(lib, 0, 768, 768, 4, 0) == (0, 0)
    assert _ws(lib, 12608, 770, 768, 4, 0) == (0, 0)                            # invalid
    assert lib.eqlin_forward_workspace_bytes(12608, 768, 768, 4, 0, None) == 1024 + 79 * 3 * slot
    monkeypatch.setenv("EQLIN_FWD_SPLIT", "0")
    assert _ws(lib, 12608, 768, 768, 4, 0) == (0, 0)


def test_forward_k_split_plan_rule(lib, monkeypatch):
    # the plan against the rule the header and the launcher state, over a grid
    # of shapes on the forced 64 x 64 tile: with t tiles (r = t mod 256 in the
    # last round) of s k stages, parts p in 2..4 (p <= s) cost
    # ceil(r p / 256) ceil(s / p) / s tiles on the busiest CU; the plan takes
    # the cheapest p that is at least 10% below the other choice (half a tile
    # where the tail split applies: more than 256 tiles and r <= 128; else a
    # whole tile), and the workspace is 1024 bytes + r p slots of 64 KB
    monkeypatch.setenv("EQLIN_FWD_TILE", "112211")
    monkeypatch.delenv("EQLIN_FWD_SPLIT", raising=False)
    checked = 0
    for N in (64, 1000, 2176, 6400, 12608, 16448, 19000, 33000):
        for C in (64, 192, 768, 1280, 3072):
            for D in (256, 768, 1280):
                tiles = -(-N // 64) * -(-(D // 4) // 64)
                s = -(-(C // 4) // 16)
                r = tiles % 256
                want_p, cost = 0, (0.5 if tiles > 256 and 2 * r <= 256 else 1.0)
                bar = 0.9 * cost
                for p in range(2, 5):
                    if p > s or r == 0:
                        continue
                    c = -(-r * p // 256) * -(-s // p) / s
                    if c < bar and c < cost:
                        want_p, cost = p, c
                want = (1024 + r * want_p * 65536, want_p) if want_p else (0, 0)
                assert _ws(lib, N, C, D, 4, 0) == want, (N, C, D)
                checked += 1
    assert checked == 120


def test_forward_ws_validation(lib):
    X, W, Y = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)
    need = lib.eqlin_forward_workspace_bytes(12608, 768, 768, 4, 0, None)
    ws = ctypes.c_void_p(0x10000)
    f = lib.eqlin_forward_ws
    assert f(X, 12608, 768, 768, 4, W, None, 0, None, Y, ws, need - 1, 0, None) == EWORKSPACE
    assert f(X, 12608, 768, 768, 4, W, None, 0, None, Y, ctypes.c_void_p(0x10008), need, 0, None) == EALIGN
    assert f(X, 12608, 768, 768, 4, W, None, 3, None, Y, ws, need, 0, None) == EINVAL
    assert f(X, 12608, 770, 768, 4, W, None, 0, None, Y, ws, need, 0, None) == EINVAL
    assert f(X, 12608, 768, 768, 5, W, None, 0, None, Y, ws, need, 0, None) == ENOTSUP
    assert f(None, 12608, 768, 768, 4, W, None, 0, None, Y, ws, need, 0, None) == EINVAL
    assert f(X, 0, 768, 768, 4, W, None, 0, None, Y, ws, 0, 0, None) == OK       # empty batch: nothing to do


# ------------------------------------------------------------ refused launches

EHIP = 5
HIP_ERROR_INVALID_CONFIGURATION = 9


def test_refused_launch_returns_ehip(lib, monkeypatch):
    # A grid the device cannot take (more than 2^31 - 1 workgroups) is refused
    # by the launcher before anything of that launch is enqueued: the call
    # returns EQLIN_EHIP and records hipErrorInvalidConfiguration.  2^38 rows
    # of a 16-channel layer make 2^32 tiles of 64 rows.  The pointers are
    # never dereferenced (no kernel is launched), so this holds with or
    # without a GPU; only the one-workgroup-per-tile float32 tiles are used
    # (a persistent tile's grid is the resident count, which would launch).
    monkeypatch.delenv("EQLIN_FWD_TILE", raising=False)
    N = 1 << 38
    st, tile, tiles, _ = _plan(lib, N, 16, 16, 4, 0)
    assert st == OK and tile < 1000000 and tiles > 0x7fffffff
    assert lib.eqlin_forward(FAKE, N, 16, 16, 4, FAKE, FAKE, 0, None) == EHIP
    assert lib.eqlin_last_hip_error() == HIP_ERROR_INVALID_CONFIGURATION
    assert lib.eqlin_backward_dx(FAKE, N, 16, 16, 4, FAKE, FAKE, 0, None) == EHIP
    ws = lib.eqlin_backward_workspace_bytes(N, 16, 16, 4, 0)
    assert ws > 0
    assert lib.eqlin_backward(FAKE, FAKE, N, 16, 16, 4, FAKE, FAKE, FAKE, FAKE, ws, 0, None) == EHIP
    assert lib.eqlin_last_hip_error() == HIP_ERROR_INVALID_CONFIGURATION
    # the binding turns the status into an exception naming the HIP error
    with pytest.raises(eqlin.EqlinError, match="EQLIN_EHIP.*hipError 9"):
        eqlin._check("eqlin_forward", lib.eqlin_forward(FAKE, N, 16, 16, 4, FAKE, FAKE, 0, None))


# ------------------------------------------------------- binding output checks

class _RecordingLib:
    """Stands in for libeqlin.so: size queries answer 1, every other entry
    point records that it was called (and would have enqueued work)."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            if not name.endswith(("_bytes", "_offset")):
                self.calls.append(name)
            return 1 if name.endswith(("_bytes", "_offset")) else 0
        return fn


def test_binding_rejects_wrong_outputs_before_any_launch(monkeypatch):
    # the C ABI takes no output sizes: an output tensor of the wrong shape or
    # dtype must be refused in Python, before the library is called
    torch = pytest.importorskip("torch")
    fake = _RecordingLib()
    monkeypatch.setattr(eqlin, "load_library", lambda path=None: fake)
    monkeypatch.setattr(eqlin, "_fwd_ws_bytes", functools.lru_cache(maxsize=None)(eqlin._fwd_ws_bytes.__wrapped__))
    monkeypatch.setattr(eqlin, "_need_cuda", lambda t, name: None)
    monkeypatch.setattr(eqlin, "_stream", lambda t: 0)
    N, C, D = 16, 32, 48
    f32, f16 = torch.float32, torch.float16
    W = eqlin.Prepared(torch.zeros(64, dtype=torch.uint8), C, D, f32, 4)
    X, dY = torch.zeros(N, C), torch.zeros(N, D)
    cases = [
        lambda: eqlin.eqlin_forward(X, W, out=torch.zeros(N, D - 4)),
        lambda: eqlin.eqlin_forward(X, W, out=torch.zeros(N, D, dtype=f16)),
        lambda: eqlin.eqlin_forward_ex(X, W, None, "gelu", out=torch.zeros(N - 1, D)),
        lambda: eqlin.eqlin_forward_ex(X, W, None, "none", out=torch.zeros(N, D, dtype=f16)),
        lambda: eqlin.eqlin_backward(dY, X, W, dX_out=torch.zeros(N, C + 4)),
        lambda: eqlin.eqlin_backward(dY, X, W, dX_out=torch.zeros(N, C, dtype=f16)),
        lambda: eqlin.eqlin_backward(dY, X, W, dw_out=torch.zeros(D // 4, C // 4, 4, dtype=f16)),
        lambda: eqlin.eqlin_backward(dY, X, W, dw_out=torch.zeros(D // 4, C // 4)),
        lambda: eqlin.eqlin_backward_dx(dY, W, out=torch.zeros(N, D)),
        lambda: eqlin.eqlin_backward_dw(dY, X, out=torch.zeros(C // 4, D // 4, 4)),
        lambda: eqlin.eqlin_backward_dw(dY, X, out=torch.zeros(D // 4, C // 4, 4, dtype=torch.float64)),
    ]
    for i, case in enumerate(cases):
        with pytest.raises(ValueError):
            case()
        assert fake.calls == [], (i, fake.calls)
    # a caller's K-split workspace smaller than the layer's need (the stand-in
    # library reports 1 byte) or of another dtype is refused the same way
    for ws in (torch.zeros(0, dtype=torch.uint8), torch.zeros(4, dtype=torch.float32)):
        with pytest.raises(ValueError):
            eqlin.eqlin_forward(X, W, workspace=ws)
        assert fake.calls == []
    # correctly shaped outputs reach the library: the default forward through
    # eqlin_forward_ws with the binding's workspace, without one eqlin_forward
    eqlin.eqlin_forward(X, W, out=torch.zeros(N, D))
    eqlin.eqlin_forward(X, W, out=torch.zeros(N, D), workspace=None)
    eqlin.eqlin_backward(dY, X, W, dX_out=torch.zeros(N, C), dw_out=torch.zeros(D // 4, C // 4, 4))
    assert fake.calls == ["eqlin_forward_ws", "eqlin_forward", "eqlin_backward"]


def test_noalloc_backward_refuses_layers_beyond_its_scratch(lib):
    # eqlin_backward_noalloc keeps its dw split partials in a static 32 MiB
    # scratch; a layer one split of which (4 planes x D' x C' float32) does
    # not fit is refused before any launch.  The pointers are placeholders
    # that must never reach a kernel, so the size is checked here first: a
    # layer whose split fits would be launched.
    scratch = 32 << 20
    assert eqlin.NOALLOC_SCRATCH_BYTES == scratch
    C = D = 4 * 1456
    assert 4 * (C // 4) * (D // 4) * 4 > scratch            # 33.9 MB: one split does not fit
    assert lib.eqlin_backward_noalloc(FAKE, FAKE, 64, C, D, 4, FAKE, None, FAKE, 0, None) == EWORKSPACE


def test_binding_keeps_a_bounded_number_of_forward_workspaces(monkeypatch):
    # one zero-filled workspace per (device, stream), the least recently used
    # dropped past the cap; a stream's workspace is reused while it is large
    # enough and replaced (zero-filled) when a layer needs more
    torch = pytest.importorskip("torch")
    monkeypatch.setattr(eqlin, "_FWD_WS", __import__("collections").OrderedDict())
    streams = iter(range(1000, 2000))
    current = {"s": 0}
    monkeypatch.setattr(eqlin, "_stream", lambda t: current["s"])
    need = {"n": 64}
    monkeypatch.setattr(eqlin, "eqlin_forward_workspace_bytes", lambda *a, **k: (need["n"], 3))
    W = eqlin.Prepared(torch.zeros(1, dtype=torch.uint8), 32, 32, torch.float32, 4)
    X = torch.zeros(4, 32)
    current["s"] = next(streams)
    first = eqlin._forward_workspace(X, 4, W)
    assert first.numel() == 64 and int(first.sum()) == 0
    assert eqlin._forward_workspace(X, 4, W) is first
    need["n"] = 128
    bigger = eqlin._forward_workspace(X, 4, W)
    assert bigger is not first and bigger.numel() == 128 and int(bigger.sum()) == 0
    for _ in range(3 * eqlin._FWD_WS_MAX):
        current["s"] = next(streams)
        eqlin._forward_workspace(X, 4, W)
    assert len(eqlin._FWD_WS) == eqlin._FWD_WS_MAX
    need["n"] = 0
    assert eqlin._forward_workspace(X, 4, W) is None
