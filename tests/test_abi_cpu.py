"""C-ABI boundary checks that need no GPU: the library loads, exports every
function include/trellis.h declares, and rejects bad arguments on the host
before touching the HIP runtime (nothing is enqueued on error). No compute
call is made here; fake device addresses are only ever passed alongside an
argument the host checks reject.
"""
import ctypes as C
import os
import re
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))
LIB = os.path.join(ROOT, "dequant_gemm_trellis_amd", "libtrellis.so")


@pytest.fixture(scope="module")
def T():
    if not os.path.exists(LIB):
        import __graft_entry__

        __graft_entry__.build()
    from dequant_gemm_trellis_amd import trellis

    return trellis


def declared_functions():
    """Every function the headers under include/ declare."""
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(trellis_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("trellis_lut_upload", "trellis_gemv", "trellis_gemv_scatter", "trellis_prefill"):
        assert n in names


def test_library_exports_every_declared_symbol(T):
    lib = T.raw()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(T.EXPORTED)
    nm = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (trellis_\w+)$", nm, flags=re.M))
    assert exported == set(declared_functions())


def test_library_does_not_link_torch(T):
    """The library's own link dependencies (DT_NEEDED), independent of the
    environment's library search path."""
    r = subprocess.run(["readelf", "-d", LIB], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    needed = re.findall(r"\(NEEDED\)\s+Shared library: \[([^\]]+)\]", r.stdout)
    assert needed, r.stdout
    assert not [n for n in needed if "torch" in n or "c10" in n], needed


FAKE = 0x10000  # 16-byte aligned, never dereferenced (every call below fails validation)


def geom(T, axis=1, Tb=256, L=12, k=2, i=512, o=256, il=0):
    return T.Geometry(axis, Tb, L, k, i, o, il)


def call_gemv(T, g, x=FAKE, codes=FAKE, scales=FAKE, lut=FAKE, y=FAKE):
    return T.raw().trellis_gemv(C.c_void_p(x), C.c_void_p(codes), C.c_void_p(scales),
                                C.c_void_p(lut), C.byref(g) if g is not None else None,
                                C.c_void_p(y), C.c_void_p(0))


@pytest.mark.parametrize("field,value", [("axis", 2), ("axis", -1), ("T", 128), ("L", 11),
                                         ("k", 1), ("k", 5), ("in_features", 0),
                                         ("out_features", 0), ("in_features", 300),
                                         ("in_features", (1 << 19) + 256),
                                         ("out_features", (1 << 19) + 1)])
def test_gemv_rejects_bad_geometry(T, field, value):
    g = geom(T)
    setattr(g, field, value)
    assert call_gemv(T, g) == T.ERR_GEOMETRY


def test_gemv_rejects_wrong_axis(T):
    assert call_gemv(T, geom(T, axis=0, i=256, o=512)) == T.ERR_GEOMETRY


def test_gemv_rejects_null(T):
    assert call_gemv(T, None) == T.ERR_NULL
    for arg in ("x", "codes", "scales", "lut", "y"):
        assert call_gemv(T, geom(T), **{arg: 0}) == T.ERR_NULL, arg


@pytest.mark.parametrize("arg,addr", [("x", FAKE + 2), ("codes", FAKE + 4), ("lut", FAKE + 8),
                                      ("y", FAKE + 2), ("scales", FAKE + 2)])
def test_gemv_rejects_misaligned(T, arg, addr):
    assert call_gemv(T, geom(T), **{arg: addr}) == T.ERR_ALIGN


def call_dual(T, g, **kw):
    a = dict(x=FAKE, codes_a=FAKE, scales_a=FAKE, lut_a=FAKE, y_a=FAKE, codes_b=FAKE,
             scales_b=FAKE, lut_b=FAKE, y_b=FAKE + 4096)
    a.update(kw)
    order = ("x", "codes_a", "scales_a", "lut_a", "y_a", "codes_b", "scales_b", "lut_b", "y_b")
    return T.raw().trellis_gemv_dual(*[C.c_void_p(a[n]) for n in order],
                                     C.byref(g) if g is not None else None, C.c_void_p(0))


def test_gemv_dual_validation(T):
    g = geom(T)  # 256 output rows: y spans 512 bytes
    assert call_dual(T, None) == T.ERR_NULL
    assert call_dual(T, geom(T, axis=0, i=256, o=512)) == T.ERR_GEOMETRY
    assert call_dual(T, geom(T, k=5)) == T.ERR_GEOMETRY
    for arg in ("x", "codes_a", "scales_a", "lut_a", "y_a", "codes_b", "scales_b", "lut_b", "y_b"):
        assert call_dual(T, g, **{arg: 0}) == T.ERR_NULL, arg
    for arg, addr in (("x", FAKE + 2), ("codes_b", FAKE + 4), ("lut_b", FAKE + 8),
                      ("y_b", FAKE + 4096 + 2), ("scales_a", FAKE + 2)):
        assert call_dual(T, g, **{arg: addr}) == T.ERR_ALIGN, arg
    # the outputs must not overlap
    assert call_dual(T, g, y_b=FAKE) == T.ERR_OVERLAP
    assert call_dual(T, g, y_b=FAKE + 496) == T.ERR_OVERLAP
    assert call_dual(T, g, y_a=FAKE + 4096 + 256) == T.ERR_OVERLAP


def call_prefill_dual(T, g, M, **kw):
    a = dict(x=FAKE, codes_a=FAKE, scales_a=FAKE, lut_a=FAKE, y_a=FAKE, codes_b=FAKE,
             scales_b=FAKE, lut_b=FAKE, y_b=FAKE + (1 << 20))
    a.update(kw)
    names = ("codes_a", "scales_a", "lut_a", "y_a", "codes_b", "scales_b", "lut_b", "y_b")
    return T.raw().trellis_prefill_dual(C.c_void_p(a["x"]), M, *[C.c_void_p(a[n]) for n in names],
                                        C.byref(g) if g is not None else None, C.c_void_p(0))


def test_prefill_dual_validation(T):
    g = geom(T)  # 256 output rows: M rows of y span 512 M bytes
    assert call_prefill_dual(T, None, 8) == T.ERR_NULL
    assert call_prefill_dual(T, geom(T, axis=0, i=256, o=512), 8) == T.ERR_GEOMETRY
    assert call_prefill_dual(T, g, -1) == T.ERR_GEOMETRY
    assert call_prefill_dual(T, g, 33) == T.ERR_GEOMETRY
    for arg in ("x", "codes_a", "scales_a", "lut_a", "y_a", "codes_b", "scales_b", "lut_b", "y_b"):
        assert call_prefill_dual(T, g, 8, **{arg: 0}) == T.ERR_NULL, arg
    for arg, addr in (("x", FAKE + 2), ("codes_b", FAKE + 4), ("lut_a", FAKE + 8),
                      ("y_b", FAKE + (1 << 20) + 2), ("scales_b", FAKE + 2)):
        assert call_prefill_dual(T, g, 8, **{arg: addr}) == T.ERR_ALIGN, arg
    # the outputs must not overlap: 8 rows of y span 4096 bytes
    assert call_prefill_dual(T, g, 8, y_b=FAKE) == T.ERR_OVERLAP
    assert call_prefill_dual(T, g, 8, y_b=FAKE + 4096 - 16) == T.ERR_OVERLAP
    assert call_prefill_dual(T, g, 8, y_a=FAKE + (1 << 20) + 4096 - 16) == T.ERR_OVERLAP
    # M = 0 enqueues nothing once the arguments check out
    assert call_prefill_dual(T, g, 0) == T.OK


def test_scatter_validation(T):
    lib = T.raw()
    g = geom(T, axis=0, i=17408, o=5120, k=3)
    need = T.workspace_bytes(g, 1, T.OP_GEMV_SCATTER)
    assert need > 0 and need % 16 == 0

    def call(g, ws=FAKE, nbytes=need):
        return lib.trellis_gemv_scatter(C.c_void_p(FAKE), C.c_void_p(FAKE), C.c_void_p(FAKE),
                                        C.c_void_p(FAKE), C.byref(g), C.c_void_p(ws), nbytes,
                                        C.c_void_p(FAKE), C.c_void_p(0))

    assert call(g, nbytes=need - 4) == T.ERR_WORKSPACE
    assert call(g, ws=0) == T.ERR_WORKSPACE
    assert call(g, ws=FAKE + 4, nbytes=need) == T.ERR_ALIGN
    assert call(geom(T, axis=1, i=5120, o=17408)) == T.ERR_GEOMETRY
    assert call(geom(T, axis=0, i=17408, o=5000)) == T.ERR_GEOMETRY


def test_prefill_validation(T):
    lib = T.raw()

    def call(M, g, ws=0, nbytes=0, x=FAKE):
        return lib.trellis_prefill(C.c_void_p(x), M, C.c_void_p(FAKE), C.c_void_p(FAKE),
                                   C.c_void_p(FAKE), C.byref(g), C.c_void_p(ws), nbytes,
                                   C.c_void_p(FAKE), C.c_void_p(0))

    g1 = geom(T, axis=1, i=5120, o=17408)
    assert call(33, g1) == T.ERR_GEOMETRY
    assert call(-1, g1) == T.ERR_GEOMETRY
    assert call(0, g1, x=0) == T.OK  # M = 0: nothing to do, nothing enqueued
    g0 = geom(T, axis=0, i=17408, o=5120, k=4)
    need = T.workspace_bytes(g0, 32, T.OP_PREFILL)
    assert need > 0
    assert call(32, g0, ws=FAKE, nbytes=need - 1) == T.ERR_WORKSPACE
    assert call(32, g0) == T.ERR_WORKSPACE
    # axis 1: the workspace is optional; one given must hold the balanced plan
    g1 = geom(T, axis=1, i=5120, o=17408, k=3)
    need1 = T.workspace_bytes(g1, 32, T.OP_PREFILL)
    assert need1 > 0
    assert call(32, g1, ws=FAKE, nbytes=need1 - 1) == T.ERR_WORKSPACE
    assert call(32, g1, ws=FAKE + 4, nbytes=need1) == T.ERR_ALIGN


def test_workspace_bytes(T):
    g0 = geom(T, axis=0, i=17408, o=5120, k=3)
    # 40 tiles of 128 output columns, each tile's 544 32-row steps cut into
    # 256 // 40 = 6 bands of 8 ranges, one per wave: 240 workgroups of one
    # (band, tile) each, one M x 128 partial per workgroup; the scatter
    # (M = 1) sums its bands in the same launch, the partials as 8-byte
    # tagged words, the prefill in a reduce launch from float32 partials
    assert T.workspace_bytes(g0, 1, T.OP_GEMV_SCATTER) == 240 * 128 * 8
    assert T.workspace_bytes(g0, 32, T.OP_PREFILL) == 240 * 32 * 128 * 4
    # the prefill sums in the launch too up to M = 8
    assert T.workspace_bytes(g0, 8, T.OP_PREFILL) == 240 * 8 * 128 * 8
    assert T.workspace_bytes(g0, 9, T.OP_PREFILL) == 240 * 9 * 128 * 4
    # 136 tiles (5120 x 17408 stored): one band per tile would leave 120 of
    # 256 compute units idle, so the finer plan: 15 ranges per tile, one whole
    # band of 8 per tile, then 7 per tile packed 8 to a workgroup (a tile's 7
    # may span two workgroups): 136 + 2 * 136 partials
    up = geom(T, axis=0, i=5120, o=17408, k=3)
    assert T.workspace_bytes(up, 1, T.OP_GEMV_SCATTER) == 3 * 136 * 128 * 4
    # 2 tiles, ranges capped by the 32-row steps (37 rows: 2 steps): 4 ranges,
    # one wave per workgroup (whole bands: summed in the launch, tagged words)
    small = geom(T, axis=0, i=37, o=256, k=3)
    assert T.workspace_bytes(small, 1, T.OP_GEMV_SCATTER) == 4 * 128 * 8
    # the widest geometry still fits the no-allocation scatter's 2 MB: 4096
    # tiles of one range each, 4096 float32 partial rows of 128 (too many to
    # sum in the launch as tagged words)
    wide = geom(T, axis=0, i=100, o=1 << 19, k=2)
    assert T.workspace_bytes(wide, 1, T.OP_GEMV_SCATTER) == T.static_scratch_bytes()
    assert T.workspace_bytes(geom(T), 1, T.OP_GEMV) == 0
    # axis-1 prefill, 5120 -> 17408 on 256 compute units: 1088 16-row groups,
    # 4 whole ones per workgroup and 64 left over, each cut into 4 block
    # ranges: one part's tile per workgroup, 64 lanes x 4 tagged 8-byte words
    # per M tile
    g1 = geom(T, axis=1, i=5120, o=17408, k=3)
    assert T.workspace_bytes(g1, 32, T.OP_PREFILL) == 256 * 2 * 64 * 4 * 8
    assert T.workspace_bytes(g1, 16, T.OP_PREFILL) == 256 * 1 * 64 * 4 * 8
    # k = 2 with two M tiles keeps the plan without the split
    g2 = geom(T, axis=1, i=5120, o=17408, k=2)
    assert T.workspace_bytes(g2, 16, T.OP_PREFILL) == 256 * 1 * 64 * 4 * 8
    assert T.workspace_bytes(g2, 17, T.OP_PREFILL) == 0
    assert T.workspace_bytes(g1, 1, T.OP_PREFILL) == 0  # the GEMV
    # 16384 rows: four whole groups per workgroup, nothing left over
    assert T.workspace_bytes(geom(T, axis=1, i=5120, o=16384, k=2), 32, T.OP_PREFILL) == 0
    # 17000 rows: 39 groups left over do not divide 256 workgroups
    assert T.workspace_bytes(geom(T, axis=1, i=5120, o=17000, k=2), 32, T.OP_PREFILL) == 0
    with pytest.raises(T.TrellisError):
        T.workspace_bytes(geom(T), 2, T.OP_GEMV)
    with pytest.raises(T.TrellisError):
        T.workspace_bytes(geom(T, k=7), 1, T.OP_GEMV)
    with pytest.raises(T.TrellisError):
        T.workspace_bytes(geom(T), 1, 9)


def test_lut_upload_validation(T):
    lib = T.raw()
    good = np.zeros(4096, dtype=np.float32)

    def up(h, n, dev=FAKE):
        return lib.trellis_lut_upload(C.c_void_p(h.ctypes.data) if h is not None else None, n,
                                      C.c_void_p(dev), C.c_void_p(0))

    assert up(good, 4095) == T.ERR_LUT
    bad = good.copy()
    bad[17] = np.inf
    assert up(bad, 4096) == T.ERR_LUT
    bad[17] = np.nan
    assert up(bad, 4096) == T.ERR_LUT
    assert up(good, 4096, FAKE + 4) == T.ERR_ALIGN
    assert up(None, 4096) == T.ERR_NULL


def test_expand_validation(T):
    lib = T.raw()
    g = geom(T)
    assert lib.trellis_expand(C.c_void_p(FAKE), C.c_void_p(FAKE), C.c_void_p(FAKE), C.byref(g),
                              None, C.c_void_p(0)) == T.ERR_NULL
    assert lib.trellis_expand(C.c_void_p(FAKE), C.c_void_p(FAKE), C.c_void_p(FAKE), C.byref(g),
                              C.c_void_p(FAKE + 2), C.c_void_p(0)) == T.ERR_ALIGN


def test_strerror(T):
    for s in (T.OK, T.ERR_NULL, T.ERR_GEOMETRY, T.ERR_ALIGN, T.ERR_LUT, T.ERR_WORKSPACE,
              T.ERR_HIP, T.ERR_OVERLAP):
        assert T.strerror(s) and T.strerror(s) != T.strerror(-99)


@pytest.mark.parametrize("il", [1, 3, -2, 4])
def test_geometry_rejects_unknown_block_interleave(T, il):
    assert call_gemv(T, geom(T, il=il)) == T.ERR_GEOMETRY


def test_block_interleave_needs_even_block_count(T):
    # 768 inputs = 3 blocks per row: no pair layout
    assert call_gemv(T, geom(T, i=768, il=2)) == T.ERR_GEOMETRY
    with pytest.raises(T.TrellisError):
        T.workspace_bytes(geom(T, axis=0, i=300, o=768, il=2), 1, T.OP_GEMV_SCATTER)
    # an even count is accepted, and the layout does not change the workspace
    g0, g2 = geom(T, axis=0, i=300, o=1024), geom(T, axis=0, i=300, o=1024, il=2)
    assert T.workspace_bytes(g2, 1, T.OP_GEMV_SCATTER) == T.workspace_bytes(g0, 1, T.OP_GEMV_SCATTER)


def test_repack_validation(T):
    lib = T.raw()

    def rp(src, dst, g, to):
        return lib.trellis_repack(C.c_void_p(src) if src else None, C.c_void_p(dst) if dst else None,
                                  C.byref(g) if g is not None else None, to, C.c_void_p(0))

    g = geom(T, i=1024, o=256)          # 4 blocks per row, 2048 words at k = 2
    far = FAKE + (1 << 20)
    assert rp(FAKE, far, None, 2) == T.ERR_NULL
    assert rp(None, far, g, 2) == T.ERR_NULL
    assert rp(FAKE, None, g, 2) == T.ERR_NULL
    assert rp(FAKE + 4, far, g, 2) == T.ERR_ALIGN
    assert rp(FAKE, far + 8, g, 2) == T.ERR_ALIGN
    assert rp(FAKE, far, g, 1) == T.ERR_GEOMETRY
    assert rp(FAKE, far, geom(T, i=768, o=256), 2) == T.ERR_GEOMETRY   # odd block count
    assert rp(FAKE, far, geom(T, i=1024, o=256, il=5), 0) == T.ERR_GEOMETRY
    # 256 rows x 1024 columns x 2 bits = 65536 bytes: any closer start overlaps
    assert rp(FAKE, FAKE, g, 2) == T.ERR_OVERLAP
    assert rp(FAKE, FAKE + 65536 - 16, g, 2) == T.ERR_OVERLAP
    assert rp(FAKE + 65536 - 16, FAKE, g, 0) == T.ERR_OVERLAP


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU; a request for more exits with status 2
    and says why, before touching any device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_static_scatter_validation(T):
    """The no-allocation scatter checks its arguments like the regular one
    (no workspace argument; the static array's size is fixed)."""
    lib = T.raw()
    assert T.static_scratch_bytes() == 2 << 20

    def call(g, x=FAKE, codes=FAKE, scales=FAKE, lut=FAKE, y=FAKE):
        return lib.trellis_gemv_scatter_static(C.c_void_p(x), C.c_void_p(codes),
                                               C.c_void_p(scales), C.c_void_p(lut),
                                               C.byref(g) if g is not None else None,
                                               C.c_void_p(y), C.c_void_p(0))

    assert call(None) == T.ERR_NULL
    assert call(geom(T, axis=1)) == T.ERR_GEOMETRY
    assert call(geom(T, axis=0, k=5)) == T.ERR_GEOMETRY
    assert call(geom(T, axis=0), x=0) == T.ERR_NULL
    assert call(geom(T, axis=0), y=FAKE + 2) == T.ERR_ALIGN
    assert call(geom(T, axis=0), codes=FAKE + 4) == T.ERR_ALIGN


def test_gate_up_swiglu_validation(T):
    """The fused gate/up SwiGLU entry point checks geometry, batch size,
    pointers and alignment on the host; M = 0 is a no-op."""
    lib = T.raw()
    g = geom(T)
    far = FAKE + (1 << 20)

    def call(g, M, x=FAKE, cg=FAKE, sg=FAKE, lg=FAKE, cu=FAKE, su=FAKE, lu=FAKE, h=far):
        return lib.trellis_gate_up_swiglu(
            C.c_void_p(x), M, C.c_void_p(cg), C.c_void_p(sg), C.c_void_p(lg), C.c_void_p(cu),
            C.c_void_p(su), C.c_void_p(lu), C.byref(g) if g is not None else None, C.c_void_p(h),
            C.c_void_p(0))

    assert call(None, 4) == T.ERR_NULL
    assert call(geom(T, axis=0, i=256, o=512), 4) == T.ERR_GEOMETRY
    assert call(geom(T, k=5), 4) == T.ERR_GEOMETRY
    assert call(g, -1) == T.ERR_GEOMETRY
    assert call(g, 33) == T.ERR_GEOMETRY
    for arg in ("x", "cg", "sg", "lg", "cu", "su", "lu", "h"):
        assert call(g, 4, **{arg: 0}) == T.ERR_NULL, arg
    for arg, addr in (("x", FAKE + 2), ("cg", FAKE + 4), ("lu", FAKE + 8), ("h", far + 2),
                      ("su", FAKE + 2)):
        assert call(g, 4, **{arg: addr}) == T.ERR_ALIGN, arg
    assert call(g, 0) == T.OK


def test_gather_probe_validation(T):
    """The gather probe rejects a bad kind, round count or output buffer on the
    host, and reports how many values a launch reads."""
    lib = T.raw()
    n = T.gather_probe_out_floats()
    assert n > 0 and n % 512 == 0

    def call(kind, rounds, out=FAKE, floats=n):
        return lib.trellis_gather_probe(kind, rounds, C.c_void_p(out), floats, C.c_void_p(0))

    assert call(3, 10) == -2 and call(-1, 10) == -2
    assert call(0, -1) == -2 and call(0, (1 << 20) + 1) == -2
    assert call(0, 10, out=0) == -2
    assert call(1, 10, floats=n - 1) == -2
    assert lib.trellis_gather_probe_values(0, 10) == n * 32 * 10 * 2
    assert lib.trellis_gather_probe_values(1, 10) == n * 32 * 10
    assert lib.trellis_gather_probe_values(2, 3) == n * 32 * 3
    assert lib.trellis_gather_probe_values(5, 3) == 0
