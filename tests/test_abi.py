"""The C ABI without a GPU: exports, validation before any device call, status strings."""
import ctypes
import os
import re

import pytest

import tile_overlapped_gemm_amd as tog
from libentwine import ensure_built

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "entwine.h")
FAKE = 0x10000  # a 16-byte aligned, never dereferenced "device" address


@pytest.fixture(scope="module")
def lib():
    return ensure_built()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(entwine_[a-z_]+)\s*\(", text)))


def test_header_declarations_are_exported(lib):
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), f"{n} declared in entwine.h but not exported"
    assert sorted(tog.EXPORTS) == names


def test_status_strings(lib):
    for code, name in [(0, "ENTWINE_OK"), (1, "ENTWINE_ERR_INVALID_ARGUMENT"),
                       (2, "ENTWINE_ERR_UNSUPPORTED"), (3, "ENTWINE_ERR_OUT_OF_MEMORY"),
                       (4, "ENTWINE_ERR_HIP"), (5, "ENTWINE_ERR_TIMEOUT")]:
        assert lib.entwine_status_string(code).decode() == name


def test_config_init(lib):
    c = tog.config()
    assert c.struct_size == ctypes.sizeof(tog.entwine_config)
    assert (c.block_m, c.tile_m, c.reducer_threads, c.peer_ready, c.release_group) == (0, 0, 0, 0, 1)


def call(M=512, N=256, K=128, P=4, rank=0, order=tog.ORDER_INTERLEAVED, budget=4, X=FAKE,
         W=FAKE * 2, out=FAKE * 3, peers="default", cfg=None):
    lib = tog.load()
    if peers == "default":
        peers = [None if r == rank else FAKE * (4 + r) for r in range(max(P, 1))]
    arr = (ctypes.c_void_p * max(P, 1))(*peers) if peers is not None else None
    if cfg is None:
        return lib.entwine_gemm_rs(X, W, arr, out, M, N, K, P, rank, order, budget, None)
    return lib.entwine_gemm_rs_ex(X, W, arr, out, M, N, K, P, rank, order, budget, None,
                                  ctypes.byref(cfg))


@pytest.mark.parametrize("kw,status", [
    (dict(M=510), tog.ENTWINE_ERR_INVALID_ARGUMENT),           # M % P != 0
    (dict(M=0), tog.ENTWINE_ERR_INVALID_ARGUMENT),
    (dict(N=-8), tog.ENTWINE_ERR_INVALID_ARGUMENT),
    (dict(N=250), tog.ENTWINE_ERR_INVALID_ARGUMENT),           # N % 8 != 0
    (dict(K=100), tog.ENTWINE_ERR_UNSUPPORTED),                # K % 64 != 0
    (dict(P=9, M=576), tog.ENTWINE_ERR_UNSUPPORTED),
    (dict(P=0), tog.ENTWINE_ERR_INVALID_ARGUMENT),
    (dict(rank=4), tog.ENTWINE_ERR_INVALID_ARGUMENT),
    (dict(rank=-1), tog.ENTWINE_ERR_INVALID_ARGUMENT),
    (dict(order=4), tog.ENTWINE_ERR_INVALID_ARGUMENT),
    (dict(order=-2), tog.ENTWINE_ERR_INVALID_ARGUMENT),
    (dict(budget=-2), tog.ENTWINE_ERR_INVALID_ARGUMENT),
    (dict(X=0), tog.ENTWINE_ERR_INVALID_ARGUMENT),
    (dict(out=0), tog.ENTWINE_ERR_INVALID_ARGUMENT),
    (dict(W=FAKE + 8), tog.ENTWINE_ERR_INVALID_ARGUMENT),      # misaligned
    (dict(peers=None), tog.ENTWINE_ERR_INVALID_ARGUMENT),
    (dict(peers=[None, 0, FAKE * 6, FAKE * 7]), tog.ENTWINE_ERR_INVALID_ARGUMENT),
    (dict(peers=[None, FAKE * 5 + 4, FAKE * 6, FAKE * 7]), tog.ENTWINE_ERR_INVALID_ARGUMENT),
    (dict(out=FAKE * 2), tog.ENTWINE_ERR_INVALID_ARGUMENT),    # out aliases W
    (dict(out=FAKE * 5), tog.ENTWINE_ERR_INVALID_ARGUMENT),    # out aliases a peer
    (dict(M=1 << 20, K=1 << 12), tog.ENTWINE_ERR_UNSUPPORTED),  # beyond 2^31 elements
    (dict(M=8, K=(1 << 21) + 64), tog.ENTWINE_ERR_UNSUPPORTED),  # K_local above 2^21
    (dict(M=8, N=(1 << 22) + 8), tog.ENTWINE_ERR_UNSUPPORTED),   # N above 2^22
])
def test_validation_before_any_device_call(lib, kw, status):
    assert call(**kw) == status
    assert lib.entwine_last_error_message().decode()


@pytest.mark.parametrize("field,value,status", [
    ("w_layout", 7, tog.ENTWINE_ERR_INVALID_ARGUMENT),
    ("w_layout", -1, tog.ENTWINE_ERR_INVALID_ARGUMENT),
    ("block_m", 64, tog.ENTWINE_ERR_UNSUPPORTED),
    ("tile_m", 32, tog.ENTWINE_ERR_UNSUPPORTED),
    ("reducer_threads", 384, tog.ENTWINE_ERR_INVALID_ARGUMENT),
    ("peer_dtype", 3, tog.ENTWINE_ERR_INVALID_ARGUMENT),
    ("peer_ready", 2, tog.ENTWINE_ERR_INVALID_ARGUMENT),
    ("release_group", -2, tog.ENTWINE_ERR_INVALID_ARGUMENT),
    ("task_slabs", 3, tog.ENTWINE_ERR_INVALID_ARGUMENT),
    ("publish_all", 2, tog.ENTWINE_ERR_INVALID_ARGUMENT),
    ("schedule", 4, tog.ENTWINE_ERR_INVALID_ARGUMENT),
    ("schedule", -1, tog.ENTWINE_ERR_INVALID_ARGUMENT),
    ("reducer_cus", -4, tog.ENTWINE_ERR_INVALID_ARGUMENT),
    ("push_outgoing", 2, tog.ENTWINE_ERR_INVALID_ARGUMENT),
    ("struct_size", 4, tog.ENTWINE_ERR_INVALID_ARGUMENT),
])
def test_config_validation(lib, field, value, status):
    cfg = tog.config(**{field: value})
    assert call(cfg=cfg) == status


def test_w_kn_builds(lib):
    """W [K_local][N] (the default) is built for the base pipeline of every
    block shape; the other pipelines are refused before any device call."""
    assert tog.config().w_layout == tog.W_KN
    for kw in (dict(block_m=256, block_n=256, gemm_variant=4),
               dict(block_m=256, block_n=256, gemm_variant=3)):
        assert call(cfg=tog.config(w_layout=tog.W_KN, **kw)) == tog.ENTWINE_ERR_UNSUPPORTED
        assert lib.entwine_last_error_message().decode()
    # the same choices with W [N][K_local] pass validation (and then fail at the
    # first device call in a process without a GPU)
    for kw in (dict(block_m=128, block_n=384), dict(block_m=256, block_n=256, gemm_variant=4)):
        assert call(cfg=tog.config(w_layout=tog.W_NK, **kw)) != tog.ENTWINE_ERR_UNSUPPORTED
    assert call(cfg=tog.config(w_layout=tog.W_KN, block_m=128, block_n=384)) != \
        tog.ENTWINE_ERR_UNSUPPORTED


def test_block_shapes(lib):
    """384-column blocks exist only with 128 rows; other widths are refused."""
    for bm, bn in ((256, 384), (128, 512), (384, 128)):
        assert call(cfg=tog.config(block_m=bm, block_n=bn)) == tog.ENTWINE_ERR_UNSUPPORTED
    assert tog.entwine_plan_shape(1000, 12288, 8, 128, 384, 128, 128) == (256, 32, 96)
    with pytest.raises(tog.EntwineError):
        tog.entwine_plan_shape(1000, 12288, 8, 256, 384, 128, 128)


def test_tuning_table_parsing(lib, tmp_path):
    good = tmp_path / "t.txt"
    good.write_text("# M N K P order budget bm bn threads\n4096 4096 1792 8 2 32 256 128 256\n")
    tog.entwine_load_tuning(str(good))
    good.write_text("4096 4096 1792 8 2 32 256 128 256 4 2\n")  # with slabs and schedule
    tog.entwine_load_tuning(str(good))
    bad = tmp_path / "b.txt"
    good.write_text("4096 4096 1792 8 2 32 256 256 256 1 1 4\n")  # with a GEMM pipeline
    tog.entwine_load_tuning(str(good))
    for text in ("4096 4096 1792 8 2\n", "4096 4096 1792 8 2 32 256 128 256 4 7\n",
                 "4096 4096 1792 8 2 32 256 256 256 1 1 5\n"):
        bad.write_text(text)
        with pytest.raises(tog.EntwineError):
            tog.entwine_load_tuning(str(bad))
    with pytest.raises(tog.EntwineError):
        tog.entwine_load_tuning(str(tmp_path / "missing.txt"))
    empty = tmp_path / "e.txt"
    empty.write_text("")
    tog.entwine_load_tuning(str(empty))


def test_plan_query_errors(lib):
    with pytest.raises(tog.EntwineError):
        tog.entwine_plan_shape(510, 256, 4, 128, 128, 128, 128)
    with pytest.raises(tog.EntwineError):
        tog.entwine_plan_shape(512, 256, 4, 96, 128, 128, 128)
    with pytest.raises(tog.EntwineError):
        tog.entwine_plan_blocks(512, 256, 4, 4, tog.ORDER_INTERLEAVED, 128, 128, 128, 128)


def chain_call(residual=FAKE * 8, gamma=FAKE * 9, eps=1e-5, h_out=FAKE * 3, y_out=FAKE * 10,
               M=512, N=256, K=128, P=4, rank=0):
    lib = tog.load()
    peers = [None if r == rank else FAKE * (4 + r) for r in range(P)]
    arr = (ctypes.c_void_p * P)(*peers)
    return lib.entwine_gemm_rs_rmsnorm(FAKE, FAKE * 2, arr, residual, gamma, eps, h_out, y_out,
                                       M, N, K, P, rank, tog.ORDER_INTERLEAVED, 4, None, None)


@pytest.mark.parametrize("kw", [
    dict(residual=0), dict(gamma=0), dict(y_out=0),
    dict(gamma=FAKE * 9 + 4),                         # misaligned
    dict(eps=-1.0), dict(eps=float("nan")), dict(eps=float("inf")),
    dict(y_out=FAKE * 3),                             # y aliases h
    dict(y_out=FAKE * 8),                             # y aliases the residual
    dict(residual=FAKE * 3 + 1024),                   # residual partly overlaps h
    dict(gamma=FAKE * 3 + 256),                       # gamma inside h
])
def test_chain_validation_before_any_device_call(lib, kw):
    assert chain_call(**kw) == tog.ENTWINE_ERR_INVALID_ARGUMENT
    assert lib.entwine_last_error_message().decode()


def test_trace_switch_and_read_without_a_traced_call(lib):
    """entwine_trace only sets a switch (no device call); reading with no traced
    call on the current device is an error, never a crash."""
    assert lib.entwine_trace(1) == tog.ENTWINE_OK
    assert lib.entwine_trace(0) == tog.ENTWINE_OK
    out = [ctypes.c_double(-1.0) for _ in range(4)]
    rc = lib.entwine_trace_read(*(ctypes.byref(x) for x in out))
    assert rc in (tog.ENTWINE_ERR_INVALID_ARGUMENT, tog.ENTWINE_ERR_HIP)
    assert lib.entwine_trace_read(None, None, None, None) in (tog.ENTWINE_ERR_INVALID_ARGUMENT,
                                                              tog.ENTWINE_ERR_HIP)
