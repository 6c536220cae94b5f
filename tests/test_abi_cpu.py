"""Host-side checks of the C ABI: the library loads, exports every function
that include/dq.h declares, and rejects bad arguments and out-of-order calls
before touching a device (no GPU needed)."""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dq.h")

dq = pytest.importorskip("compressed_hop_gradient_amd.dq")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*(dq_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dq.LIB_PATH):
        pytest.fail("libdq.so is not built; run __graft_entry__.build()")
    return dq.lib()


def test_header_declares_the_stage_calls():
    names = declared_functions()
    for n in ("dq_plan_create", "dq_stats", "dq_allocate", "dq_reorder", "dq_compress", "dq_hop",
              "dq_finalize", "dq_plan_destroy", "dq_get_info"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", dq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    # and the binding's signature table covers the header
    assert sorted(dq._SIGS) == declared_functions()


def _create(lib, d=256 * 64, n=4, topo=dq.RING, bits=5.0):
    h = C.c_void_p()
    rc = lib.dq_plan_create(d, n, topo, bits, C.byref(h))
    return rc, h


def test_create_validation(lib):
    assert _create(lib, d=0)[0] == dq.DQ_EINVAL
    assert _create(lib, d=255)[0] == dq.DQ_EINVAL
    assert _create(lib, d=256 * 3 + 1)[0] == dq.DQ_EINVAL
    assert _create(lib, n=0)[0] == dq.DQ_EINVAL
    assert _create(lib, n=6, topo=dq.BUTTERFLY)[0] == dq.DQ_EINVAL
    assert _create(lib, topo=7)[0] == dq.DQ_EINVAL
    assert _create(lib, bits=1.99)[0] == dq.DQ_EBUDGET
    assert _create(lib, bits=float("nan"))[0] == dq.DQ_EBUDGET
    assert lib.dq_plan_create(256, 1, 0, 5.0, None) == dq.DQ_ENULL
    for args in ((256, 1, dq.RING, 2.0), (256 * 1000, 8, dq.BUTTERFLY, 100.0), (256, 16, dq.RING, 5.0)):
        rc, h = _create(lib, *args)
        assert rc == dq.DQ_OK and h.value
        lib.dq_plan_destroy(h)
    lib.dq_plan_destroy(None)


def test_options(lib):
    rc, h = _create(lib)
    assert lib.dq_plan_set_u64(h, dq.OPT_SEED, 2 ** 64 - 1) == dq.DQ_OK
    assert lib.dq_plan_set_u64(h, dq.OPT_ROUND, 2 ** 32) == dq.DQ_EINVAL
    for mode in (dq.CORRELATED, dq.INDEPENDENT, dq.STRATIFIED):
        assert lib.dq_plan_set_u64(h, dq.OPT_ROUNDING, mode) == dq.DQ_OK
    assert lib.dq_plan_set_u64(h, dq.OPT_ROUNDING, 3) == dq.DQ_EINVAL
    assert lib.dq_plan_set_u64(h, dq.OPT_TIMING, 3) == dq.DQ_EINVAL
    for mode in (dq.ALLOC_THRESHOLD, dq.ALLOC_MEAN_CORRECTED, dq.ALLOC_UNIFORM):
        assert lib.dq_plan_set_u64(h, dq.OPT_ALLOC, mode) == dq.DQ_OK
    assert lib.dq_plan_set_u64(h, dq.OPT_ALLOC, 3) == dq.DQ_EINVAL
    assert lib.dq_plan_set_u64(h, dq.OPT_TIMING_KINDS, 1 << 4) == dq.DQ_OK
    assert lib.dq_plan_set_u64(h, dq.OPT_TIMING_KINDS, 0) == dq.DQ_EINVAL
    assert lib.dq_plan_set_u64(h, dq.OPT_TIMING_KINDS, 1 << 8) == dq.DQ_OK
    assert lib.dq_plan_set_u64(h, dq.OPT_TIMING_KINDS, 1 << len(dq.KERNEL_KINDS)) == dq.DQ_EINVAL
    assert lib.dq_plan_set_u64(h, 99, 0) == dq.DQ_EINVAL
    assert lib.dq_plan_set_u64(None, 0, 0) == dq.DQ_ENULL
    # level shape: (0, 1] and one level boundary per search bucket
    for eps in (1.0, 0.5, 0.3, 0.05, 0.03):
        assert lib.dq_plan_set_f64(h, dq.OPT_EPS, eps) == dq.DQ_OK
    for eps in (0.0, -0.5, 1.5, float("nan"), float("inf"), 0.02, 0.01):
        assert lib.dq_plan_set_f64(h, dq.OPT_EPS, eps) == dq.DQ_EINVAL
    assert lib.dq_plan_set_f64(h, 1, 0.5) == dq.DQ_EINVAL
    assert lib.dq_plan_set_f64(None, dq.OPT_EPS, 0.5) == dq.DQ_ENULL
    lib.dq_plan_destroy(h)


def test_workspace_and_region_sizes(lib):
    d, n = 256 * 5000, 8
    rc, h = _create(lib, d=d, n=n, topo=dq.BUTTERFLY)
    J = d // 256
    ws = lib.dq_workspace_bytes(h)
    lay = dq.dq_layout()
    assert lib.dq_workspace_layout(h, C.byref(lay)) == dq.DQ_OK
    assert lay.total == ws
    offs = [lay.sum, lay.sumsq, lay.widths, lay.perm, lay.inv, lay.mu_stream, lay.tables, lay.ctrl]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.sumsq - lay.sum >= 4 * J and lay.perm - lay.widths >= J
    # regions: worst case of any part of m is at most (J/m + 3) SGs of 276 bytes
    for m in (1, 2, 4, 8):
        b = lib.dq_region_bytes_max(h, m)
        assert b % 256 == 0 and b >= (J // m + 2) * 276
    assert lib.dq_region_bytes_max(h, 3) == 0 and lib.dq_region_bytes_max(h, 16) == 0
    assert lib.dq_arena_bytes(h) > 0
    # binding checks size and alignment only (no device access)
    assert lib.dq_plan_bind(h, C.c_void_p(4096), ws - 1) == dq.DQ_EWORKSPACE
    assert lib.dq_plan_bind(h, C.c_void_p(4096 + 16), ws) == dq.DQ_EWORKSPACE
    assert lib.dq_plan_bind(h, None, ws) == dq.DQ_ENULL
    lib.dq_plan_destroy(h)


def test_stage_order_enforced_on_host(lib):
    rc, h = _create(lib, n=4)
    ws = lib.dq_workspace_bytes(h)
    fake = C.c_void_p(1 << 20)  # never dereferenced: every call below fails its checks first
    assert lib.dq_allocate(h, None) == dq.DQ_EWORKSPACE
    assert lib.dq_plan_bind(h, fake, ws) == dq.DQ_OK
    assert lib.dq_allocate(h, None) == dq.DQ_ESTATE
    assert lib.dq_reorder(h, None) == dq.DQ_ESTATE
    assert lib.dq_stats(h, 1, fake, dq.BF16, None) == dq.DQ_ESTATE      # rank order
    assert lib.dq_stats(h, 4, fake, dq.BF16, None) == dq.DQ_EINVAL      # no such worker
    assert lib.dq_stats(h, 0, fake, dq.PACKED, None) == dq.DQ_EINVAL    # gradients only
    assert lib.dq_stats(h, 0, None, dq.BF16, None) == dq.DQ_ENULL
    assert lib.dq_compress(h, 0, 0, fake, dq.BF16, fake, None) == dq.DQ_ESTATE
    assert lib.dq_hop(h, 0, 1, fake, fake, dq.BF16, fake, None, None) == dq.DQ_ESTATE
    assert lib.dq_finalize(h, 0, fake, fake, None) == dq.DQ_ESTATE
    info = dq.dq_info()
    assert lib.dq_get_info(h, C.byref(info), None) == dq.DQ_ESTATE
    lib.dq_plan_destroy(h)


def test_final_parts_and_status_strings(lib):
    rc, h = _create(lib, n=8, topo=dq.RING)
    assert [lib.dq_final_part(h, w) for w in range(8)] == [1, 2, 3, 4, 5, 6, 7, 0]
    assert lib.dq_final_part(h, 8) == -1
    lib.dq_plan_destroy(h)
    rc, h = _create(lib, n=8, topo=dq.BUTTERFLY)
    assert [lib.dq_final_part(h, w) for w in range(8)] == list(range(8))
    lib.dq_plan_destroy(h)
    rc, h = _create(lib, n=1)
    assert lib.dq_final_part(h, 0) == 0
    lib.dq_plan_destroy(h)
    for s in range(-7, 1):
        assert lib.dq_status_string(s).decode() != "unknown status"
    assert lib.dq_version() >= 1


def test_package_has_no_cpu_fallback():
    """The binding must fail loudly when the library is missing."""
    src = open(os.path.join(ROOT, "compressed_hop_gradient_amd", "dq.py")).read()
    assert "oracle" not in src
    assert "raise RuntimeError" in src


def test_check_reciprocal_argument_checks(lib):
    fake = C.c_void_p(0x1000)
    assert lib.dq_check_reciprocal(0, 16, None, None) == dq.DQ_ENULL
    assert lib.dq_check_reciprocal(0xFFFFFFFF, 2, fake, None) == dq.DQ_EINVAL
    assert lib.dq_check_reciprocal(0xFFFFFFF0, 0, fake, None) == dq.DQ_OK   # nothing to do, no launch


def test_region_limit(lib):
    """The largest region a schedule writes must stay below 4 GB (32-bit
    offsets in the kernels): 276 bytes per super-group at worst."""
    J = 16_000_000                                    # 4.1e9 coordinates
    assert _create(lib, d=256 * J, n=1)[0] == dq.DQ_EINVAL        # the whole vector in one region
    for n, topo in ((2, dq.RING), (2, dq.BUTTERFLY), (8, dq.RING)):
        rc, h = _create(lib, d=256 * J, n=n, topo=topo)            # halves and eighths fit
        assert rc == dq.DQ_OK
        lib.dq_plan_destroy(h)
    assert _create(lib, d=256 * 2 * J, n=2, topo=dq.BUTTERFLY)[0] == dq.DQ_EINVAL


def test_header_compiles_as_c_and_host_calls_work(lib, tmp_path):
    """include/dq.h is a C header (C11, pedantic, warnings as errors), and a
    plain C program linked against the library gets the documented results
    from the host-only calls (tests/native/abi_c_check.c)."""
    import shutil
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = os.path.join(ROOT, "tests", "native", "abi_c_check.c")
    libdir = os.path.dirname(dq.LIB_PATH)
    exe = str(tmp_path / "abi_c_check")
    subprocess.run([cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    src, "-L", libdir, "-ldq", "-Wl,-rpath," + libdir, "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout


def test_streams_option(lib):
    rc, h = _create(lib)
    assert rc == dq.DQ_OK
    assert lib.dq_plan_set_u64(h, dq.OPT_STREAMS, 1) == dq.DQ_OK
    assert lib.dq_plan_set_u64(h, dq.OPT_STREAMS, 0) == dq.DQ_EINVAL
    assert lib.dq_plan_set_u64(h, dq.OPT_STREAMS, 3) == dq.DQ_EINVAL
    lib.dq_plan_destroy(h)


def test_max_width_option(lib):
    """DQ_OPT_MAX_WIDTH: 8 or 16; 16 adds the 16-bit tables to the workspace
    and 256 more region bytes per super-group, unbinds the plan, and is
    refused where a widest region would reach 4 GB."""
    J = 4096
    rc, h = _create(lib, 256 * J, 4, dq.RING, 5.0)
    ws8 = lib.dq_workspace_bytes(h)
    r8 = lib.dq_region_bytes_max(h, 4)
    for v in (0, 4, 12, 32):
        assert lib.dq_plan_set_u64(h, dq.OPT_MAX_WIDTH, v) == dq.DQ_EINVAL
    assert lib.dq_plan_set_u64(h, dq.OPT_MAX_WIDTH, 16) == dq.DQ_OK
    assert lib.dq_workspace_bytes(h) >= ws8 + 2 * 65536 * 4
    assert lib.dq_region_bytes_max(h, 4) - r8 >= (J // 4) * 256
    lay = dq.dq_layout()
    assert lib.dq_workspace_layout(h, C.byref(lay)) == dq.DQ_OK
    assert lay.tables16 > 0 and lay.tables16 + 4 * 65536 * 4 <= lay.total
    # the workspace size changed: the plan is unbound
    g = C.c_void_p(256)
    assert lib.dq_stats(h, 0, g, dq.F32, None) == dq.DQ_EWORKSPACE
    assert lib.dq_plan_set_u64(h, dq.OPT_MAX_WIDTH, 8) == dq.DQ_OK
    assert lib.dq_workspace_bytes(h) == ws8
    lib.dq_plan_destroy(h)
    # a ring of two workers with 1.5e7 super-groups per part fits at 8 bits, not at 16
    rc, h = _create(lib, 256 * 2 * 15_000_000, 2, dq.RING, 5.0)
    assert rc == dq.DQ_OK
    assert lib.dq_plan_set_u64(h, dq.OPT_MAX_WIDTH, 16) == dq.DQ_EINVAL
    lib.dq_plan_destroy(h)
