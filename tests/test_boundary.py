"""The C-ABI library: it loads, exports every function include/moe.h declares,
and rejects invalid arguments on the host before anything is enqueued.  CPU
only: no call here passes validation, so no kernel is ever launched."""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for fn in ("moe_route", "moe_bucket", "moe_expert_ffn_mxfp4", "moe_combine", "q8_0_matmul"):
        assert fn in names


def test_library_exports_every_declared_symbol():
    import router_top_bucket_amd as moe
    lib = moe.raw_library()
    out = subprocess.run(["nm", "-D", "--defined-only", moe.library_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared_functions():
        assert name in exported, f"{name} not exported"
        assert hasattr(lib, name)
    assert set(moe.ABI_FUNCTIONS) == set(_declared_functions())


def test_header_compiles_as_c():
    # the header is plain C: no HIP or torch types in the signatures
    r = subprocess.run(["gcc", "-std=c99", "-fsyntax-only", "-Wall", "-Werror", "-x", "c", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_status_strings():
    import router_top_bucket_amd as moe
    lib = moe.raw_library()
    assert lib.moe_status_str(0) == b"MOE_OK"
    assert lib.moe_status_str(-1).startswith(b"MOE_EINVAL")
    assert lib.moe_status_str(-2).startswith(b"MOE_EUNSUPPORTED")
    assert lib.moe_status_str(-3).startswith(b"MOE_EHIP")
    assert lib.moe_status_str(-4).startswith(b"MOE_ESCRATCH")


FAKE = 0x100000  # never dereferenced: every call below fails host validation


def test_route_validation():
    import router_top_bucket_amd as moe
    lib = moe.raw_library()
    EINVAL, EUNSUP = moe.MOE_EINVAL, moe.MOE_EUNSUPPORTED
    assert lib.moe_route(None, 0, None, None, 1, 0, 16, 2, None, None, None) == EINVAL  # NULL outputs
    assert lib.moe_route(None, 0, None, FAKE, -1, 0, 16, 2, FAKE, FAKE, None) == EINVAL  # M < 0
    assert lib.moe_route(None, 0, None, FAKE, 1, 0, 16, 0, FAKE, FAKE, None) == EINVAL  # k < 1
    assert lib.moe_route(None, 0, None, FAKE, 1, 0, 16, 17, FAKE, FAKE, None) == EINVAL  # k > E
    assert lib.moe_route(None, 7, None, FAKE, 1, 0, 16, 2, FAKE, FAKE, None) == EINVAL  # dtype
    assert lib.moe_route(FAKE, 0, FAKE, FAKE, 1, 100, 16, 2, FAKE, FAKE, None) == EINVAL  # d % 32
    assert lib.moe_route(None, 0, FAKE, FAKE, 1, 256, 16, 2, FAKE, FAKE, None) == EINVAL  # x NULL with router
    assert lib.moe_route(None, 0, None, FAKE, 1, 0, 5000, 2, FAKE, FAKE, None) == EUNSUP  # E too large
    assert lib.moe_route(None, 0, None, FAKE, 0, 0, 16, 2, FAKE, FAKE, None) == moe.MOE_OK  # M = 0: no-op


def test_bucket_validation():
    import router_top_bucket_amd as moe
    lib = moe.raw_library()
    EINVAL = moe.MOE_EINVAL
    assert lib.moe_bucket(None, 1, 2, 16, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == EINVAL
    assert lib.moe_bucket(FAKE, 1, 0, 16, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == EINVAL
    assert lib.moe_bucket(FAKE, 1, 2, 16, -1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == EINVAL
    assert lib.moe_bucket(FAKE, 1, 2, 16, 0, FAKE, FAKE, FAKE, FAKE, None, None) == EINVAL
    assert lib.moe_bucket(FAKE, 1, 2, 4095, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None) == moe.MOE_EUNSUPPORTED
    assert lib.moe_bucket(FAKE, 0, 2, 16, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == moe.MOE_OK


def _experts(**kw):
    import router_top_bucket_amd as moe
    v = dict(base=FAKE, stride=52224, d=256, f=128, n_routed=16, n_shared=0, layout=0)
    v.update(kw)
    return moe._Experts(v["base"], v["stride"], v["d"], v["f"], v["n_routed"], v["n_shared"], v["layout"])


def test_ffn_validation_and_workspace_query():
    import router_top_bucket_amd as moe
    lib = moe.raw_library()
    EINVAL = moe.MOE_EINVAL
    ok = _experts()
    assert lib.moe_workspace_bytes(1, 2, ctypes.byref(ok)) > 0
    for bad in (_experts(d=100), _experts(f=50), _experts(stride=1000), _experts(base=0), _experts(n_routed=0),
                _experts(base=FAKE + 4), _experts(layout=2), _experts(layout=-1)):
        assert lib.moe_workspace_bytes(1, 2, ctypes.byref(bad)) == 0
        assert lib.moe_expert_ffn_mxfp4(FAKE, 0, 1, 2, ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        1 << 20, None) == EINVAL
    # workspace too small
    need = lib.moe_workspace_bytes(4, 2, ctypes.byref(ok))
    assert lib.moe_expert_ffn_mxfp4(FAKE, 0, 4, 2, ctypes.byref(ok), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
                                    None) == EINVAL
    # k > E, NULL y, misaligned workspace
    assert lib.moe_expert_ffn_mxfp4(FAKE, 0, 1, 17, ctypes.byref(ok), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                    None) == EINVAL
    assert lib.moe_expert_ffn_mxfp4(FAKE, 0, 1, 2, ctypes.byref(ok), FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30,
                                    None) == EINVAL
    assert lib.moe_expert_ffn_mxfp4(FAKE, 0, 1, 2, ctypes.byref(ok), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16,
                                    1 << 30, None) == EINVAL
    assert lib.moe_expert_ffn_mxfp4(FAKE, 0, 0, 2, ctypes.byref(ok), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0,
                                    None) == moe.MOE_OK


def test_workspace_grows_with_rows():
    import router_top_bucket_amd as moe
    lib = moe.raw_library()
    kimi = _experts(stride=17547264, d=7168, f=1536, n_routed=896, n_shared=2)
    a = lib.moe_workspace_bytes(1, 16, ctypes.byref(kimi))
    b = lib.moe_workspace_bytes(16, 16, ctypes.byref(kimi))
    c = lib.moe_workspace_bytes(1533, 16, ctypes.byref(kimi))
    assert 0 < a < b < c
    # h for every slot in two bf16 parts, at least
    assert c >= 1533 * 18 * 1536 * 4


def test_combine_and_q8_0_validation():
    import router_top_bucket_amd as moe
    lib = moe.raw_library()
    EINVAL = moe.MOE_EINVAL
    assert lib.moe_combine(FAKE, FAKE, 1, 0, 0, 16, FAKE, None) == EINVAL
    assert lib.moe_combine(FAKE, FAKE, 1, 2, 0, 18, FAKE, None) == EINVAL  # d % 4
    assert lib.moe_combine(None, FAKE, 1, 2, 0, 16, FAKE, None) == EINVAL
    assert lib.moe_combine(FAKE, FAKE, 0, 2, 0, 16, FAKE, None) == moe.MOE_OK
    assert lib.q8_0_matmul(FAKE, 1, 100, FAKE, FAKE, 10, FAKE, None) == EINVAL  # K % 32
    assert lib.q8_0_matmul(FAKE, 9, 128, FAKE, FAKE, 10, FAKE, None) == moe.MOE_EUNSUPPORTED  # M > 8
    assert lib.q8_0_matmul(None, 1, 128, FAKE, FAKE, 10, FAKE, None) == EINVAL
    assert lib.q8_0_matmul(FAKE, 0, 128, FAKE, FAKE, 10, FAKE, None) == moe.MOE_OK


def test_binding_fails_loudly_without_library(tmp_path):
    # the product path has no fallback: a copy of the package without the
    # built library raises on import instead of computing anything elsewhere
    import shutil
    pkg = os.path.join(ROOT, "router_top_bucket_amd")
    dst = tmp_path / "router_top_bucket_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__"))
    code = ("import sys\n"
            "try:\n"
            "    import router_top_bucket_amd\n"
            "except ImportError as e:\n"
            "    print('RAISED', e)\n")
    r = subprocess.run(["python", "-c", code], cwd=str(tmp_path), capture_output=True, text=True)
    assert "RAISED" in r.stdout, r.stdout + r.stderr


def test_layer_validation():
    import router_top_bucket_amd as moe
    lib = moe.raw_library()
    EINVAL, EUNSUP = moe.MOE_EINVAL, moe.MOE_EUNSUPPORTED
    ok = _experts()
    ws = lib.moe_workspace_bytes(2, 2, ctypes.byref(ok))

    def call(x=FAKE, dt=0, wr=FAKE, lg=FAKE, M=2, k=2, ex=ok, out=FAKE, dev_error=FAKE, y=FAKE, wsp=FAKE,
             nbytes=ws):
        return lib.moe_layer_mxfp4(x, dt, wr, lg, M, k, ctypes.byref(ex), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   dev_error, y, out, wsp, nbytes, None)

    assert call(ex=_experts(d=100)) == EINVAL
    assert call(ex=_experts(base=0)) == EINVAL
    assert call(M=-1) == EINVAL
    assert call(k=0) == EINVAL
    assert call(k=17) == EINVAL  # k > E
    assert call(dt=5) == EINVAL
    assert call(lg=None) == EINVAL
    assert call(x=None) == EINVAL  # x is needed by the FFN even with given logits
    assert call(out=None) == EINVAL
    assert call(out=FAKE + 4) == EINVAL
    assert call(dev_error=None) == EINVAL
    assert call(y=None) == EINVAL
    assert call(nbytes=ws - 1) == EINVAL
    assert call(wsp=FAKE + 16) == EINVAL
    assert call(ex=_experts(n_routed=5000, n_shared=0)) == EUNSUP
    assert call(M=0) == moe.MOE_OK


def test_noalloc_layer_validation():
    """The no-allocation layer call checks what moe_layer_mxfp4 checks (no
    workspace argument), and refuses a call whose scratch need exceeds its
    static array, all on the host before anything is enqueued."""
    import router_top_bucket_amd as moe
    lib = moe.raw_library()
    EINVAL, EUNSUP = moe.MOE_EINVAL, moe.MOE_EUNSUPPORTED
    cap = lib.moe_noalloc_scratch_bytes()
    assert cap == 8 << 20
    ok = _experts()

    def call(x=FAKE, dt=0, wr=FAKE, lg=FAKE, M=2, k=2, ex=ok, out=FAKE, dev_error=FAKE, y=FAKE):
        return lib.moe_layer_mxfp4_noalloc(x, dt, wr, lg, M, k, ctypes.byref(ex), FAKE, FAKE, FAKE, FAKE, FAKE,
                                           FAKE, dev_error, y, out, None)

    assert call(ex=_experts(d=100)) == EINVAL
    assert call(M=-1) == EINVAL
    assert call(k=17) == EINVAL
    assert call(lg=None) == EINVAL
    assert call(out=FAKE + 4) == EINVAL
    assert call(y=None) == EINVAL
    assert call(ex=_experts(n_routed=5000, n_shared=0)) == EUNSUP
    assert call(M=0) == moe.MOE_OK
    # the Kimi shape: 75 rows fit the 8 MiB array, 76 do not
    kimi = _experts(d=7168, f=1536, n_routed=896, n_shared=2, stride=17547264)
    assert lib.moe_workspace_bytes(75, 16, ctypes.byref(kimi)) <= cap < lib.moe_workspace_bytes(76, 16,
                                                                                                 ctypes.byref(kimi))
    assert call(M=76, k=16, ex=kimi) == moe.MOE_ESCRATCH
    assert call(M=76, k=16, ex=kimi, out=None) == EINVAL  # argument errors come first


def test_cache_and_streamed_layer_validation():
    import router_top_bucket_amd as moe
    lib = moe.raw_library()
    EINVAL = moe.MOE_EINVAL

    def cfg(**kw):
        v = dict(device_pool=FAKE, n_slots=20, host_pool=FAKE, n_layers=2, n_routed=16, n_shared=1, d=256, f=128,
                 stride=52224, n_upload_streams=4, upload_groups=2, admit_min_rows=0, n_transient=2, layout=0)
        v.update(kw)
        return moe._CacheConfig(*[v[name] for name, _ in moe._CacheConfig._fields_])

    h = ctypes.c_void_p()
    assert lib.moe_cache_create(None, ctypes.byref(h)) == EINVAL
    for bad in (dict(device_pool=0), dict(host_pool=0), dict(n_layers=0), dict(d=100), dict(f=50),
                dict(stride=1000), dict(stride=52224 + 8), dict(device_pool=FAKE + 4), dict(n_upload_streams=0),
                dict(n_upload_streams=9), dict(upload_groups=0), dict(upload_groups=17), dict(admit_min_rows=-1),
                dict(n_transient=-1), dict(layout=2), dict(n_slots=2 * 1 + 2)):  # (last: no cached slot left)
        c = cfg(**bad)
        assert lib.moe_cache_create(ctypes.byref(c), ctypes.byref(h)) == EINVAL, bad
    assert lib.moe_cache_destroy(None) == EINVAL
    assert lib.moe_cache_get_stats(None, ctypes.byref(moe._CacheStats())) == EINVAL
    assert lib.moe_layer_streamed(None, 0, FAKE, 0, None, FAKE, 1, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, FAKE, 1 << 20, None) == EINVAL


def test_cache_simulate_validation():
    import router_top_bucket_amd as moe
    lib = moe.raw_library()
    EINVAL = moe.MOE_EINVAL
    assert lib.moe_cache_simulate(0, 16, 4, 0, 0, 0, None, None, None, None, None, None, None) == EINVAL
    assert lib.moe_cache_simulate(1, 16, 0, 0, 0, 0, None, None, None, None, None, None, None) == EINVAL
    assert lib.moe_cache_simulate(1, 16, 4, -1, 0, 0, None, None, None, None, None, None, None) == EINVAL
    assert lib.moe_cache_simulate(1, 16, 4, 0, 0, 1, None, None, None, None, None, None, None) == EINVAL
    assert lib.moe_cache_simulate(1, 16, 4, 0, 0, 0, None, None, None, None, None, None, None) == moe.MOE_OK


def test_verify_helpers_validation():
    import router_top_bucket_amd as moe
    lib = moe.raw_library()
    EINVAL = moe.MOE_EINVAL
    assert lib.q8_0_rows(FAKE, 1, 100, FAKE, FAKE, 10, FAKE, 0, None) == EINVAL       # K % 32
    assert lib.q8_0_rows(None, 1, 128, FAKE, FAKE, 10, FAKE, 0, None) == EINVAL
    assert lib.q8_0_rows(FAKE, 1, 128, FAKE, FAKE, 10, FAKE + 4, 0, None) == EINVAL   # X alignment
    assert lib.q8_0_rows(FAKE, 1, 128, FAKE, FAKE, 10, FAKE, 1, None) == EINVAL       # tiles need N % 16
    assert lib.q8_0_rows(FAKE, 1, 128, FAKE, FAKE, 16, FAKE, 2, None) == EINVAL       # layout
    assert lib.q8_0_rows(FAKE, 0, 128, FAKE, FAKE, 10, FAKE, 0, None) == moe.MOE_OK
    assert lib.moe_residual_bf16(None, FAKE, 10, None, None) == EINVAL
    assert lib.moe_residual_bf16(FAKE, None, 10, None, None) == EINVAL             # nothing to do
    assert lib.moe_residual_bf16(FAKE, FAKE, -1, None, None) == EINVAL
    assert lib.moe_residual_bf16(FAKE, FAKE, 0, None, None) == moe.MOE_OK
    assert lib.moe_rmsnorm(FAKE, 1, 0, 1e-6, FAKE, None, None) == EINVAL
    assert lib.moe_rmsnorm(FAKE, 1, 16, 1e-6, None, None, None) == EINVAL
    assert lib.moe_rmsnorm(FAKE, 1, 16, -1.0, FAKE, None, None) == EINVAL
    assert lib.moe_rmsnorm(FAKE + 4, 1, 16, 1e-6, FAKE, None, None) == EINVAL
    assert lib.moe_rmsnorm(FAKE, 0, 16, 1e-6, FAKE, None, None) == moe.MOE_OK
    assert lib.moe_argmax_rows(FAKE, 1, 0, FAKE, None) == EINVAL
    assert lib.moe_argmax_rows(FAKE + 4, 1, 8, FAKE, None) == EINVAL
    assert lib.moe_argmax_rows(FAKE, 0, 8, FAKE, None) == moe.MOE_OK
    assert lib.moe_fnv1a_rows(FAKE, 1, 8, FAKE + 4, None) == EINVAL
    assert lib.moe_fnv1a_rows(FAKE, 1, 0, FAKE, None) == EINVAL
    assert lib.moe_fnv1a_rows(FAKE, 0, 8, FAKE, None) == moe.MOE_OK


def test_pack_experts_validation():
    import router_top_bucket_amd as moe
    lib = moe.raw_library()
    EINVAL = moe.MOE_EINVAL
    B = FAKE * 16
    assert lib.moe_pack_experts(None, B, 1, 52224, 256, 128, 1, None) == EINVAL
    assert lib.moe_pack_experts(FAKE, B, 1, 52224, 256, 128, 2, None) == EINVAL     # layout
    assert lib.moe_pack_experts(FAKE, B, 1, 52224, 100, 128, 1, None) == EINVAL     # d % 32
    assert lib.moe_pack_experts(FAKE, B, 1, 1000, 256, 128, 1, None) == EINVAL      # stride too small
    assert lib.moe_pack_experts(FAKE, FAKE + 16, 1, 52224, 256, 128, 1, None) == EINVAL  # overlap
    assert lib.moe_pack_experts(FAKE + 8, B, 1, 52224, 256, 128, 1, None) == EINVAL  # alignment
    assert lib.moe_pack_experts(FAKE, B, 0, 52224, 256, 128, 1, None) == moe.MOE_OK


def test_q8_0_layout_and_pack_validation():
    import router_top_bucket_amd as moe
    lib = moe.raw_library()
    EINVAL = moe.MOE_EINVAL
    assert lib.q8_0_matmul_layout(FAKE, 1, 128, FAKE, FAKE, 10, FAKE, 1, None) == EINVAL  # tiles need N % 16
    assert lib.q8_0_matmul_layout(FAKE, 1, 128, FAKE, FAKE, 16, FAKE, 2, None) == EINVAL  # layout
    assert lib.q8_0_matmul_layout(FAKE, 0, 128, FAKE, FAKE, 16, FAKE, 1, None) == moe.MOE_OK
    B = FAKE * 16
    assert lib.q8_0_pack(FAKE, B, 10, 128, 1, None) == EINVAL          # N % 16
    assert lib.q8_0_pack(FAKE, B, 16, 100, 1, None) == EINVAL          # K % 32
    assert lib.q8_0_pack(FAKE, B, 16, 128, 3, None) == EINVAL          # layout
    assert lib.q8_0_pack(FAKE, FAKE + 64, 16, 128, 1, None) == EINVAL  # overlap
    assert lib.q8_0_pack(None, B, 16, 128, 1, None) == EINVAL
