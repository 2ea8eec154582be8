"""C-ABI contract checks that need no GPU: the library loads, exports every
symbol include/ssd.h declares, and rejects invalid arguments on the host before
any HIP call (so these calls are safe without a device)."""
import ctypes
import os
import re

import pytest

from mamba_ssd_layer_amd import _binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

INVALID, UNSUPPORTED = 1, 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.library_path()):
        import mamba_ssd_layer_amd.build as b
        b.build()
    return bd.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
        assert n in bd.SIGNATURES, f"binding lacks a signature for {n}"


def test_status_strings(lib):
    assert lib.ssd_status_string(0) == b"SSD_OK"
    assert lib.ssd_status_string(2) == b"SSD_ERR_UNSUPPORTED"
    assert lib.ssd_status_string(99) == b"SSD_ERR_UNKNOWN"


def test_chunk_slots(lib):
    assert lib.ssd_chunk_slots(8, 8 * 2048, 256, 0) == 64
    assert lib.ssd_chunk_slots(2, 2 * 300, 256, 0) == 4
    assert lib.ssd_chunk_slots(16, 34000, 256, 1) == (34000 + 255) // 256 + 16
    assert lib.ssd_chunk_slots(0, 0, 256, 1) == 0


def test_supported_set(lib):
    # the benchmark workloads
    assert lib.ssd_config_supported(1, 128, 256) == 1
    assert lib.ssd_config_supported(1, 256, 128) == 1
    assert lib.ssd_config_supported(0, 16, 64) == 1
    # every (N, Q) of the table in both dtypes, N = 256 at Q = 256 included
    for dt in (0, 1):
        assert all(lib.ssd_config_supported(dt, n, q) == 1 for n in (16, 32, 64, 128, 256) for q in (64, 128, 256))
    # outside the table
    assert lib.ssd_config_supported(0, 48, 64) == 0
    assert lib.ssd_config_supported(1, 128, 96) == 0
    assert lib.ssd_config_supported(5, 128, 64) == 0


FAKE = 0x100000  # 16-byte aligned, never dereferenced: validation fails first


def call_fwd(lib, **kw):
    a = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, b=1, T=256, H=4, P=64, N=128, G=1, Q=256,
             dtype=1, y=FAKE, fs=None)
    a.update(kw)
    return lib.ssd_chunked_fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["b"], a["T"], a["H"],
                               a["P"], a["N"], a["G"], a["Q"], a["dtype"], a["y"], a["fs"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(H=3, G=2), INVALID),          # H % G != 0
    (dict(G=0), INVALID),
    (dict(H=0), INVALID),
    (dict(b=-1), INVALID),
    (dict(T=-5), INVALID),
    (dict(dtype=7), INVALID),
    (dict(P=128), UNSUPPORTED),
    (dict(N=48), UNSUPPORTED),
    (dict(Q=100), UNSUPPORTED),
    (dict(Q=0), INVALID),
    (dict(N=128, Q=64, P=32, dtype=0), UNSUPPORTED),  # head dim other than 64, fp32
    (dict(x=FAKE + 4), INVALID),        # misaligned
    (dict(y=FAKE + 8), INVALID),
    (dict(fs=FAKE + 4), INVALID),
    (dict(dt=FAKE + 2), INVALID),
    (dict(x=None), INVALID),
    (dict(A=None), INVALID),
])
def test_fwd_rejects_invalid_arguments(lib, kw, code):
    assert call_fwd(lib, **kw) == code


@pytest.mark.parametrize("kw", [
    dict(b=1, T=1 << 41),          # more tokens than the index arithmetic allows
    dict(b=1 << 31, T=2),          # more sequences than the grids allow
    dict(b=1 << 20, T=1 << 21),    # b * T beyond 2^40
    dict(H=1 << 30, G=1),          # chunk slots x heads beyond a 32-bit grid
])
def test_fwd_rejects_oversized_problems(lib, kw):
    """Sizes past what the kernels index with their integer widths are refused on
    the host, before any allocation or launch."""
    assert call_fwd(lib, **kw) == INVALID


def test_varlen_rejects_invalid_arguments(lib):
    # null cu_seqlens with sequences
    assert lib.ssd_chunked_fwd_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, None, 2, 100, 4, 64, 128, 1,
                                      256, 1, FAKE, None, None) == INVALID
    # misaligned cu_seqlens
    assert lib.ssd_chunked_fwd_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, 2, 100, 4, 64, 128,
                                      1, 256, 1, FAKE, None, None) == INVALID
    assert lib.ssd_chunked_fwd_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1, 100, 4, 64, 128, 1,
                                      256, 1, FAKE, None, None) == INVALID


def call_ex(lib, **kw):
    a = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, cu=None, S=2, T=512, H=4, P=64, N=128, G=1,
             Q=256, dtype=1, h0=FAKE, D=None, xdt=0, y=FAKE, fs=FAKE)
    a.update(kw)
    return lib.ssd_chunked_fwd_ex(a["x"], a["dt"], a["A"], a["B"], a["C"], a["cu"], a["S"], a["T"],
                                  a["H"], a["P"], a["N"], a["G"], a["Q"], a["dtype"], a["h0"], a["D"],
                                  a["xdt"], a["y"], a["fs"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(h0=FAKE + 4), INVALID),       # misaligned initial state
    (dict(D=FAKE + 2), INVALID),        # misaligned skip weights
    (dict(xdt=2), INVALID),             # the input-scaling flag is 0 or 1
    (dict(S=3, T=512), INVALID),        # batched form: total_len not a multiple of nseqs
    (dict(S=0, T=10), INVALID),
    (dict(S=-1), INVALID),
    (dict(cu=FAKE + 2), INVALID),       # misaligned cu_seqlens
    (dict(N=48), UNSUPPORTED),
    (dict(H=3, G=2), INVALID),
])
def test_ex_rejects_invalid_arguments(lib, kw, code):
    assert call_ex(lib, **kw) == code


def call_decode(lib, **kw):
    a = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, b=4, H=8, P=64, N=128, G=2, dtype=1,
             D=None, xdt=0, st=FAKE, y=FAKE)
    a.update(kw)
    return lib.ssd_decode_step(a["x"], a["dt"], a["A"], a["B"], a["C"], a["b"], a["H"], a["P"],
                               a["N"], a["G"], a["dtype"], a["D"], a["xdt"], a["st"], a["y"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(st=FAKE + 8), INVALID),       # misaligned state
    (dict(D=FAKE + 1), INVALID),
    (dict(xdt=-1), INVALID),
    (dict(st=None), INVALID),
    (dict(y=None), INVALID),
    (dict(x=FAKE + 2), INVALID),
    (dict(b=-1), INVALID),
    (dict(H=6, G=4), INVALID),
    (dict(dtype=3), INVALID),
    (dict(P=32), UNSUPPORTED),
    (dict(N=100), UNSUPPORTED),
])
def test_decode_rejects_invalid_arguments(lib, kw, code):
    assert call_decode(lib, **kw) == code


def test_normalized_needs_denominator_buffer(lib):
    # x dt A B C cu S T H P N G Q dtype D xdt y fs denom stream
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, None, 2, 512, 4, 64, 128, 1, 256, 1, None, 0, FAKE, None, None, None]
    assert lib.ssd_chunked_fwd_normalized(*args) == INVALID          # denom missing
    args[18] = FAKE + 2
    assert lib.ssd_chunked_fwd_normalized(*args) == INVALID          # denom misaligned
    args[18] = FAKE
    args[10] = 48
    assert lib.ssd_chunked_fwd_normalized(*args) == UNSUPPORTED


def call_scan(lib, **kw):
    a = dict(x=FAKE, dl=FAKE, A=FAKE, B=FAKE, C=FAKE, b=2, T=512, D=256, N=128, dtype=1, y=FAKE, fs=None)
    a.update(kw)
    return lib.ssd_selective_scan(a["x"], a["dl"], a["A"], a["B"], a["C"], a["b"], a["T"], a["D"],
                                  a["N"], a["dtype"], a["y"], a["fs"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dl=FAKE + 2), INVALID),      # delta is fp32
    (dict(x=FAKE + 1), INVALID),       # bf16 elements
    (dict(dtype=0, B=FAKE + 2), INVALID),
    (dict(fs=FAKE + 2), INVALID),
    (dict(A=None), INVALID),
    (dict(y=None), INVALID),
    (dict(b=-1), INVALID),
    (dict(T=-1), INVALID),
    (dict(D=0), INVALID),
    (dict(dtype=3), INVALID),
    (dict(N=16), UNSUPPORTED),
    (dict(N=96), UNSUPPORTED),
    (dict(b=1 << 20, T=1 << 20), INVALID),  # indices past 2^40
])
def test_selective_scan_rejects_invalid_arguments(lib, kw, code):
    assert call_scan(lib, **kw) == code


def test_backward_rejects_invalid_arguments(lib):
    # x dt A B C cu S T H P N G Q dtype h0 D xdt dy dfinal dx ddt dA dB dC dD dinit stream
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, None, 2, 512, 4, 64, 128, 1, 256, 1, None, None, 0,
            FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None]

    def call(changes):
        a = list(base)
        for i, v in changes.items():
            a[i] = v
        return lib.ssd_chunked_bwd(*a)

    assert call({17: None}) == INVALID        # dy missing
    assert call({17: FAKE + 2}) == INVALID    # dy misaligned
    assert call({21: None}) == INVALID        # dA missing
    assert call({18: FAKE + 4}) == INVALID    # dfinal misaligned
    assert call({6: 3}) == INVALID            # batched: 512 not a multiple of 3
    assert call({10: 48}) == UNSUPPORTED
    assert call({16: 5}) == INVALID           # x_times_dt is 0 or 1


@pytest.mark.parametrize("route", ["packed", "batched_unaligned"])
def test_backward_padded_route_rejects_invalid_arguments(lib, route):
    """bf16 calls that take the padded route (packed sequences; a batched length
    that no chunk length divides) check their arguments before any HIP call."""
    # x dt A B C cu S T H P N G Q dtype h0 D xdt dy dfinal dx ddt dA dB dC dD dinit stream
    cu, T = (FAKE, 512) if route == "packed" else (None, 600)
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, cu, 2, T, 4, 64, 128, 1, 256, 1, None, None, 0,
            FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None]

    def call(changes):
        a = list(base)
        for i, v in changes.items():
            a[i] = v
        return lib.ssd_chunked_bwd(*a)

    assert call({17: None}) == INVALID        # dy missing
    assert call({17: FAKE + 2}) == INVALID    # dy misaligned
    assert call({21: None}) == INVALID        # dA missing
    assert call({22: FAKE + 2}) == INVALID    # dB misaligned
    assert call({18: FAKE + 4}) == INVALID    # dfinal misaligned
    assert call({25: FAKE + 4}) == INVALID    # dinitial_state misaligned
    assert call({16: 5}) == INVALID           # x_times_dt is 0 or 1
    assert call({10: 48}) == UNSUPPORTED


def test_intermediates_rejects_uneven_batch(lib):
    assert lib.ssd_chunked_fwd_intermediates(FAKE, FAKE, FAKE, FAKE, FAKE, None, 3, 100, 4, 64, 128,
                                             1, 256, 1, FAKE, None, None, None, None, None) == INVALID


def test_timing_read_rejects_bad_kernel(lib):
    ms = ctypes.c_double(0)
    n = ctypes.c_int64(0)
    assert lib.ssd_kernel_timing_read(9, ctypes.byref(ms), ctypes.byref(n), 0) == INVALID


def call_noalloc(lib, **kw):
    a = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, b=1, T=256, H=4, P=64, N=128, G=1, Q=256,
             dtype=1, y=FAKE, fs=None)
    a.update(kw)
    return lib.ssd_chunked_fwd_noalloc(a["x"], a["dt"], a["A"], a["B"], a["C"], a["b"], a["T"], a["H"],
                                       a["P"], a["N"], a["G"], a["Q"], a["dtype"], a["y"], a["fs"], None)


SCRATCH_LIMIT = 5


def test_noalloc_rejects_beyond_its_scratch(lib):
    """The entry point that allocates nothing refuses, on the host and before any
    HIP call, a problem whose workspace exceeds its static scratch, and
    validates its arguments as ssd_chunked_fwd does before that."""
    assert lib.ssd_status_string(SCRATCH_LIMIT) == b"SSD_ERR_SCRATCH_LIMIT"
    # 64K tokens of 32 heads, dstate 128, bf16, chunk 256: about twice the scratch
    assert call_noalloc(lib, b=1, T=65536, H=32) == SCRATCH_LIMIT
    assert call_noalloc(lib, b=8, T=2048, H=80) == SCRATCH_LIMIT
    for kw, code in ((dict(H=3, G=2), INVALID), (dict(N=48), UNSUPPORTED), (dict(x=FAKE + 4), INVALID),
                     (dict(b=-1), INVALID), (dict(H=32, T=65536, y=None), INVALID)):
        assert call_noalloc(lib, **kw) == code, kw


def test_workspace_layouts_selfcheck(lib):
    """Every workspace carving of every entry point (forward forms, the
    no-allocation forward, the normalised forward, the backward's routes) over
    a grid of shapes and options puts each non-null piece inside its allocation
    with no overlap, absent pieces null (dry: fake pointers, nothing launched)."""
    assert lib.ssd_workspace_selfcheck() == 0
