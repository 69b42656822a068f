"""The C ABI without a GPU: the library loads, exports every function that the
headers under include/ declare, and its host-side validation rejects bad
arguments with the documented status before anything is launched."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

nv4 = pytest.importorskip("nvfp4_w4a4_moe_amd")


def _declared_functions():
    names = []
    for h in HEADERS:
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "for", "sizeof")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(nv4.LIB_PATH):
        pytest.fail("libnv4moe.so is not built (run `python -c 'import __graft_entry__ as g; g.build()'`)")
    return nv4.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"nvfp4_quantize", "moe_permute", "nvfp4_grouped_gemm", "moe_combine"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == {"nv4_version", "nv4_status_string", "nv4_last_error", "nvfp4_quantize_workspace",
                          "nvfp4_quantize", "moe_permute_workspace", "moe_permute",
                          "nvfp4_grouped_gemm_workspace", "nvfp4_grouped_gemm", "moe_combine",
                          "nv4_to_bf16", "bf16_grouped_gemm", "nvfp4_quantize_sr",
                          "nv4_bench_copy", "nv4_bench_read", "nv4_bench_mfma_out_floats", "nv4_bench_mfma", "nv4_bench_mix",
                          "moe_permute_noalloc", "moe_permute_noalloc_max_workspace", "nv4_amax",
                          "nvfp4_decode_f16", "nv4_bench_lds", "nv4_bench_lds_out_words",
                          "nv4_bench_write"}


def test_binding_covers_every_symbol():
    assert set(_declared_functions()) <= set(nv4._SIGS)


def test_status_strings(lib):
    assert lib.nv4_version() >= 100
    for s in (0, -1, -2, -3, -4, -5):
        assert lib.nv4_status_string(s)


def _q(lib, **kw):
    d = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, kw.get("orows", 32), kw.get("oK", 64), 0, 1)
    return lib.nvfp4_quantize(ctypes.c_void_p(kw.get("x", 0x1000)), kw.get("xt", 0), kw.get("rows", 32),
                              kw.get("K", 64), kw.get("ldx", 64), kw.get("row_index"), kw.get("layout", 1),
                              kw.get("mode", 0),
                              kw.get("nseg", 1), None, None, None, None, ctypes.byref(d), kw.get("out_rows"),
                              ctypes.c_void_p(0x1000), 1 << 20, None, None)


def test_quantize_validation(lib):
    assert _q(lib, K=40, ldx=40, oK=40) == -2          # K % 16
    assert _q(lib, x=0x1008) == -2                      # x misaligned
    assert _q(lib, ldx=68) == -2                        # row stride (136 bytes) not a 16-byte multiple
    assert _q(lib, ldx=32) == -1                        # ldx < K
    assert _q(lib, orows=31) == -1                      # out shape mismatch
    assert _q(lib, layout=2, mode=2) == -3              # per-row scales only with rows layout
    assert _q(lib, layout=7) == -1
    assert _q(lib, xt=5) == -1
    assert _q(lib, layout=3, nseg=3, orows=3 * 64, oK=32 // 3) == -2   # batched needs rows/nseg % 16 == 0
    assert b"multiple of 16" in lib.nv4_last_error()
    # NV4_COLS without segment offsets
    assert _q(lib, layout=2, orows=64, oK=64) == -1
    # row gather is not offered for the batched transpose
    assert _q(lib, layout=3, nseg=2, orows=2 * 64, oK=16, row_index=ctypes.c_void_p(0x1000)) == -3
    d = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 32, 64, 0, 1)
    assert lib.nvfp4_quantize(ctypes.c_void_p(0x1000), 0, 32, 64, 64, None, 1, 0, 1, None, None, None, None,
                              ctypes.byref(d), None, None, 0, None, None) == -4      # no workspace
    # one scale per half of each matrix's rows: batched columns only, rows/nseg % 32 == 0
    assert _q(lib, mode=3, nseg=1) == -3
    assert _q(lib, layout=3, mode=3, nseg=2, orows=2 * 64, oK=16) == -2
    # rows-and-columns: tensor scale only, needs out_rows of the source shape
    assert _q(lib, layout=4, mode=1, nseg=2, orows=64, oK=128) == -3
    assert _q(lib, layout=4, orows=64, oK=128) == -1          # no out_rows


def test_permute_validation(lib):
    P = ctypes.c_void_p(0x1000)
    args = lambda T, E, k, ws=P, wsb=1 << 20, ids=P: (None, T, E, k, 0, ids, P, P, P, P, P, None, None, ws, wsb,
                                                      None, None)
    assert lib.moe_permute(*args(16, 0, 1)) == -1
    assert lib.moe_permute(*args(16, 2000, 2)) == -3
    assert lib.moe_permute(*args(16, 8, 9)) == -3
    assert lib.moe_permute(*args(16, 64, 33)) == -3
    assert lib.moe_permute(*args(-1, 8, 2)) == -1
    assert lib.moe_permute(*args(16, 8, 2, ids=None)) == -1
    assert lib.moe_permute(*args(16, 8, 2, wsb=1)) == -4
    assert lib.moe_permute_workspace(16384, 128, 8) >= 16384 * 8 * 4


def test_gemm_validation(lib):
    a = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 256, 2048, 0, 1)
    b = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 8 * 1536, 2048, 1, 8)
    P = ctypes.c_void_p(0x1000)
    g = lambda A, B, E=8, N=768, Mc=256, mode=0, epi=1, ldc=768: lib.nvfp4_grouped_gemm(
        ctypes.byref(A), ctypes.byref(B), P, E, Mc, N, None, mode, epi, P, 1, ldc, None, None, 0, None)
    assert g(a, b, N=700) == -1                 # B rows != E * 2N
    assert g(a, b, ldc=100) == -1
    assert g(a, b, Mc=257) == -1                # M_cap > rows of A
    assert g(a, b, mode=1) == -3                # SwiGLU with GROUP_K
    bk = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 8 * 1536, 2000, 1, 8)
    assert g(a, bk) == -2                       # K mismatch
    b7 = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 8 * 1536, 2048, 1, 7)
    assert g(a, b7) == -1                       # per-expert scales for 7 of 8 experts
    a_seg = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 256, 2048, 1, 8)
    assert g(a_seg, b) == -3
    assert g(a, b, E=0) == -1
    # one scale per projection: 2E segments only with the SwiGLU epilogue (gate, up)
    bn = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 8 * 768, 2048, 1, 16)
    assert g(a, bn, epi=0) == -1
    # one scale per K half: EPI_NONE, per-tensor A, (K/2) % 128 == 0
    bh2 = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 8 * 1536, 2048, 3, 8)
    assert g(a, bh2, epi=1) == -3
    bh = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 8 * 768, 2048, 3, 8)
    a_row = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 256, 2048, 2, 256)
    assert g(a_row, bh, epi=0) == -3
    a3 = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 256, 1536 + 64, 0, 1)
    bh3 = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 8 * 768, 1536 + 64, 3, 8)
    assert g(a3, bh3, epi=0) == -3            # K/2 = 800 is not a whole number of 128-wide stages
    assert b"K/2" in lib.nv4_last_error()
    # K % 16 is the contract; K % 64 != 0 needs the workspace for the repacked operands
    a40 = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 256, 40, 0, 1)
    b40 = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 8 * 1536, 40, 1, 8)
    assert g(a40, b40) == -2
    a80 = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 256, 80, 0, 1)
    b80 = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 8 * 1536, 80, 1, 8)
    assert g(a80, b80) == -4 and b"workspace" in lib.nv4_last_error()
    need = lib.nvfp4_grouped_gemm_workspace(ctypes.byref(a80), ctypes.byref(b80), 0)
    pad = lambda n: (n + 255) // 256 * 256
    assert need == pad(256 * 64) + pad(256 * 8) + pad(8 * 1536 * 64) + pad(8 * 1536 * 8)
    assert lib.nvfp4_grouped_gemm_workspace(ctypes.byref(a), ctypes.byref(b), 0) == 0
    assert lib.nvfp4_grouped_gemm_workspace(ctypes.byref(a), ctypes.byref(b), 1) == 256


def test_combine_validation(lib):
    P = ctypes.c_void_p(0x1000)
    assert lib.moe_combine(P, 1, 2048, P, P, 16, 8, 2046, P, 0, None) == -2
    assert lib.moe_combine(P, 1, 2000, P, P, 16, 8, 2048, P, 0, None) == -2
    assert lib.moe_combine(P, 3, 2048, P, P, 16, 8, 2048, P, 0, None) == -1
    assert lib.moe_combine(ctypes.c_void_p(0x1004), 1, 2048, P, P, 16, 8, 2048, P, 0, None) == -2


def test_to_bf16_validation(lib):
    P = ctypes.c_void_p(0x1000)
    q = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 64, 128, 0, 1)
    c = lambda x=P, q=None, rows=64, K=128, ldx=128, xr=64, ri=None, layout=1, nseg=1, off=None, po=None, out=P, \
        orow=64, ocol=128: lib.nv4_to_bf16(x, xr, ldx, None if q is None else ctypes.byref(q), rows, K, ri, layout,
                                           nseg, off, po, out, orow, ocol, None)
    assert c(x=None) == -1                       # neither source
    assert c(q=q) == -1                          # both sources
    assert c(K=120, ldx=120, ocol=120) == -2     # K % 16
    assert c(ldx=132) == -2                      # ldx % 8
    assert c(x=ctypes.c_void_p(0x1008)) == -2    # x misaligned
    assert c(orow=63) == -1                      # rows output shape
    assert c(xr=65) == -1                        # x rows != rows without a gather
    assert c(layout=2, nseg=4, orow=128, ocol=64 + 15 * 4 + 4) == -1      # COLS without offsets
    assert c(layout=2, nseg=4, off=P, po=P, orow=128, ocol=120) == -1      # COLS capacity
    assert c(layout=3, nseg=3, orow=3 * 128, ocol=21) == -1               # batched rows / nseg % 16
    assert c(layout=3, nseg=2, ri=P, orow=256, ocol=32) == -3             # no gather when batched
    assert c(layout=9) == -1
    assert b"layout" in lib.nv4_last_error()


def test_decode_f16_validation(lib):
    P = ctypes.c_void_p(0x1000)
    q = lambda rows=64, K=128, codes=0x1000: nv4.NV4Tensor(codes, 0x1000, 0x1000, rows, K, 0, 1)
    d = lambda t, out=P, ldo=128: lib.nvfp4_decode_f16(ctypes.byref(t), out, ldo, None)
    assert lib.nvfp4_decode_f16(None, P, 128, None) == -1      # no tensor
    assert d(q(K=120), ldo=120) == -2                           # K % 16
    assert d(q(), ldo=100) == -2                                # ldo < K
    assert d(q(), ldo=132) == -2                                # ldo % 8
    assert d(q(), out=ctypes.c_void_p(0x1008)) == -2            # out misaligned
    assert d(q(codes=0x1004)) == -2                             # codes misaligned
    assert d(q(), out=None) == -1                               # no output
    assert d(q(rows=0), out=None) == 0                          # nothing to decode


def test_bf16_gemm_validation(lib):
    P = ctypes.c_void_p(0x1000)
    g = lambda A=P, ar=256, B=P, br=8 * 1536, K=2048, E=8, Mc=256, N=768, ri=None, mode=0, epi=1, ldc=768: \
        lib.bf16_grouped_gemm(A, ar, B, br, K, P, E, Mc, N, ri, mode, epi, P, 1, ldc, None, None, 0, None)
    assert g(K=2040) == -2                       # K % 32
    assert g(A=ctypes.c_void_p(0x1008)) == -2    # A misaligned
    assert g(N=700) == -1                        # B rows != E * 2N
    assert g(ldc=100) == -1
    assert g(Mc=257) == -1                       # M_cap > rows of A
    assert g(mode=1) == -3                       # SwiGLU with GROUP_K
    assert g(mode=1, epi=0, ri=P, ldc=1536) == -3   # row index with GROUP_K
    assert g(ar=1 << 20, K=4096, ri=P) == -1     # A above 4 GiB
    assert g(E=0) == -1


def test_quantize_sr_validates_like_quantize(lib):
    d = nv4.NV4Tensor(0x1000, 0x1000, 0x1000, 32, 64, 0, 1)
    q = lambda K=64, ldx=64: lib.nvfp4_quantize_sr(ctypes.c_void_p(0x1000), 0, 32, K, ldx, None, 1, 0, 1, None, None,
                                                   None, None, ctypes.byref(d), None, ctypes.c_void_p(0x1000), 1 << 20,
                                                   None, ctypes.c_uint64(7), None)
    assert q(K=40, ldx=40) == -2
    assert q(ldx=32) == -1


def test_permute_noalloc_rejects_sizes_above_its_static_workspace(lib):
    """Checked on the host before the device is touched: a routing whose workspace
    would not fit the static array fails with NV4_EWORKSPACE and a clear message."""
    P = ctypes.c_void_p(0x1000)
    cap = lib.moe_permute_noalloc_max_workspace()
    assert cap == 16 << 20
    T = 4_000_000 // 8
    assert lib.moe_permute_workspace(T, 128, 8) > cap
    rc = lib.moe_permute_noalloc(None, T, 128, 8, 0, P, P, P, P, P, P, None, None, None, None)
    assert rc == -4 and b"moe_permute_noalloc" in lib.nv4_last_error()
    assert lib.moe_permute_noalloc(None, 16, 2000, 2, 0, P, P, P, P, P, P, None, None, None, None) == -3
