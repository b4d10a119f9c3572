"""C-ABI checks that need no GPU: the library loads, exports what
include/moe.h declares, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

import sparse_moe_routed_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails validation first


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def header_abi_version():
    return int(re.search(r"#define\s+MOE_ABI_VERSION\s+(\d+)", open(HEADER).read()).group(1))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail("libmoe.so is not built: run `python -m sparse_moe_routed_amd.build`")
    return moe.lib()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert "moe_route" in names and "moe_forward" in names
    raw = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    # the binding describes exactly the declared functions
    assert sorted(moe._SIGS) == names


def test_version_and_status_strings(lib):
    assert moe.abi_version() == header_abi_version() == moe.ABI_VERSION
    assert moe.status_str(moe.OK) == "ok"
    for s in (moe.EINVAL, moe.EUNSUPPORTED, moe.EWORKSPACE, moe.EHIP, 99):
        assert moe.status_str(s)


def _dims(h=2688, f=1856, e=128, k=6):
    return moe.Dims(h, f, e, k)


def test_workspace_size(lib):
    d = _dims()
    sizes = [lib.moe_workspace_size(ctypes.byref(d), fmt, T)
             for fmt in (0, 1, 2) for T in (0, 1, 4, 64, 511, 512, 4096)]
    assert all(s > 0 and s % 256 == 0 for s in sizes)
    for fmt in (0, 1, 2):
        prev = 0
        for T in range(0, 3000, 37):
            s = lib.moe_workspace_size(ctypes.byref(d), fmt, T)
            assert s >= prev
            prev = s
    assert lib.moe_workspace_size(None, 0, 4) == 0
    assert lib.moe_workspace_size(ctypes.byref(d), 7, 4) == 0
    assert lib.moe_workspace_size(ctypes.byref(d), 0, -1) == 0
    assert lib.moe_workspace_size(ctypes.byref(_dims(h=100)), 0, 4) == 0
    # fp32 rows of the down projection dominate: T*k*H*4 bytes
    assert lib.moe_workspace_size(ctypes.byref(d), 0, 4096) > 4096 * 6 * 2688 * 4


def test_workspace_layout(lib):
    lay = moe.workspace_layout(moe.LayerDims(), "fp8", 64)
    assert lay["x_q"] > 0 and lay["act_q"] > 0 and lay["total"] > lay["out_rows"]
    lay = moe.workspace_layout(moe.LayerDims(), "bf16", 64)
    assert lay["x_q"] == -1 and lay["act_q"] == -1
    lay = moe.workspace_layout(moe.LayerDims(), "nvfp4", 64)
    assert lay["act_q"] == lay["act"]  # quantised in place
    offs = [lay[k] for k in ("counts", "offsets", "sorted_src", "inv", "act", "out_rows", "scales")]
    assert all(o % 256 == 0 for o in offs)


def test_route_validation(lib):
    d = _dims()
    r = moe.Router(FAKE.value, None)
    st = None
    need = lib.moe_route_workspace_size(ctypes.byref(d), 4)
    assert need >= 4 * 128 * 4 and need % 256 == 0

    def call(dims=d, T=4, x=FAKE, router=r, ids=FAKE, gates=FAKE, ws=FAKE, wsb=need):
        return lib.moe_route(dims if dims is None else ctypes.byref(dims), T, x,
                             router if router is None else ctypes.byref(router), ids, gates, ws,
                             wsb, st)

    assert call(dims=None) == moe.EINVAL
    assert call(T=-1) == moe.EINVAL
    assert call(x=None) == moe.EINVAL
    assert call(router=None) == moe.EINVAL
    assert call(router=moe.Router(None, None)) == moe.EINVAL
    assert call(ids=None) == moe.EINVAL
    assert call(dims=_dims(k=0)) == moe.EINVAL
    assert call(dims=_dims(e=8, k=9)) == moe.EINVAL
    assert call(dims=_dims(k=9)) == moe.EUNSUPPORTED
    assert call(dims=_dims(e=120)) == moe.EUNSUPPORTED
    assert call(dims=_dims(h=2690)) == moe.EUNSUPPORTED
    assert call(ws=None) == moe.EWORKSPACE
    assert call(wsb=64) == moe.EWORKSPACE
    assert call(ws=ctypes.c_void_p(FAKE.value + 4)) == moe.EWORKSPACE
    # rows move in 16-byte vectors, routing entries in 4-byte words
    assert call(x=ctypes.c_void_p(FAKE.value + 8)) == moe.EINVAL
    assert call(router=moe.Router(FAKE.value + 2, None)) == moe.EINVAL
    assert call(router=moe.Router(FAKE.value, FAKE.value + 2)) == moe.EINVAL
    assert call(ids=ctypes.c_void_p(FAKE.value + 2)) == moe.EINVAL
    assert call(gates=ctypes.c_void_p(FAKE.value + 1)) == moe.EINVAL
    # T == 0 is a no-op that touches nothing
    assert call(T=0, x=None, ids=None, gates=None, ws=None, wsb=0) == moe.OK
    assert lib.moe_router_pack(ctypes.byref(d), None, FAKE, st) == moe.EINVAL
    assert lib.moe_router_pack(None, FAKE, FAKE, st) == moe.EINVAL
    assert lib.moe_route_workspace_size(None, 4) == 0


def test_forward_validation(lib):
    d = _dims()
    ex = moe.Experts(0, FAKE.value, FAKE.value, None, None, None, None)
    need = lib.moe_workspace_size(ctypes.byref(d), 0, 4)

    def call(dims=d, T=4, x=FAKE, ids=FAKE, gates=FAKE, e=ex, y=FAKE, yd=1, ws=FAKE, wsb=need):
        return lib.moe_forward(dims if dims is None else ctypes.byref(dims), T, x, ids, gates,
                               e if e is None else ctypes.byref(e), y, yd, ws, wsb, None)

    assert call(dims=None) == moe.EINVAL
    assert call(e=None) == moe.EINVAL
    assert call(T=-3) == moe.EINVAL
    assert call(T=(1 << 20) + 1) == moe.EINVAL
    assert call(x=None) == moe.EINVAL
    assert call(ids=None) == moe.EINVAL
    assert call(gates=None) == moe.EINVAL
    assert call(y=None) == moe.EINVAL
    assert call(yd=5) == moe.EINVAL
    assert call(e=moe.Experts(9, FAKE.value, FAKE.value, None, None, None, None)) == moe.EINVAL
    assert call(e=moe.Experts(0, None, FAKE.value, None, None, None, None)) == moe.EINVAL
    # quantised formats need their scales (and block scales for nvfp4)
    assert call(e=moe.Experts(1, FAKE.value, FAKE.value, None, None, None, None)) == moe.EINVAL
    assert call(e=moe.Experts(2, FAKE.value, FAKE.value, None, None, FAKE.value, FAKE.value)) == moe.EINVAL
    assert call(dims=_dims(f=1850)) == moe.EUNSUPPORTED
    # workspace: missing, too small, misaligned
    assert call(ws=None) == moe.EWORKSPACE
    assert call(wsb=need - 1) == moe.EWORKSPACE
    assert call(ws=ctypes.c_void_p(FAKE.value + 16)) == moe.EWORKSPACE
    # alignment: token and output rows 16 bytes, ids / gates 4 bytes, weight
    # codes 16 bytes, scales and block scales 4 bytes
    off = lambda n: ctypes.c_void_p(FAKE.value + n)
    assert call(x=off(8)) == moe.EINVAL
    assert call(x=off(2)) == moe.EINVAL
    assert call(y=off(4)) == moe.EINVAL
    assert call(ids=off(2)) == moe.EINVAL
    assert call(gates=off(2)) == moe.EINVAL
    assert call(e=moe.Experts(0, FAKE.value + 8, FAKE.value, None, None, None, None)) == moe.EINVAL
    assert call(e=moe.Experts(0, FAKE.value, FAKE.value + 2, None, None, None, None)) == moe.EINVAL
    assert call(e=moe.Experts(1, FAKE.value, FAKE.value, None, None, FAKE.value + 2,
                              FAKE.value)) == moe.EINVAL
    assert call(e=moe.Experts(2, FAKE.value, FAKE.value, FAKE.value + 1, FAKE.value, FAKE.value,
                              FAKE.value)) == moe.EINVAL
    # T == 0: nothing to do, no workspace needed
    assert call(T=0, ws=None, wsb=0) == moe.OK
    # the timed variant needs at least one event per stage boundary
    evs = (ctypes.c_void_p * moe.N_TIMED_EVENTS)()
    for n, want in ((0, moe.EINVAL), (moe.N_STAGES, moe.EINVAL)):
        assert lib.moe_forward_timed(ctypes.byref(d), 4, FAKE, FAKE, FAKE, ctypes.byref(ex), FAKE,
                                     1, FAKE, need, None, evs, n) == want
    assert lib.moe_forward_timed(ctypes.byref(d), 4, FAKE, FAKE, FAKE, ctypes.byref(ex), FAKE,
                                 1, FAKE, need, None, None, moe.N_TIMED_EVENTS) == moe.EINVAL


def test_shared_validation(lib):
    sd = moe.Dims(2688, 3712, 1, 1)
    need = lib.moe_shared_workspace_size(ctypes.byref(sd), 0, 64)
    assert need > 0 and need % 256 == 0
    assert lib.moe_shared_workspace_size(ctypes.byref(_dims()), 0, 64) == 0  # not one expert
    assert lib.moe_shared_workspace_size(ctypes.byref(moe.Dims(2688, 3700, 1, 1)), 0, 64) == 0
    ex = moe.Experts(0, FAKE.value, FAKE.value, None, None, None, None)

    def call(dims=sd, T=64, x=FAKE, e=ex, y=FAKE, yd=1, acc=0, ws=FAKE, wsb=need):
        return lib.moe_shared_forward(ctypes.byref(dims), T, x, e if e is None else ctypes.byref(e),
                                      y, yd, acc, ws, wsb, None)

    assert call(dims=_dims()) == moe.EINVAL
    assert call(dims=moe.Dims(2688, 3712, 1, 2)) == moe.EINVAL
    assert call(dims=moe.Dims(2688, 3700, 1, 1)) == moe.EUNSUPPORTED
    assert call(e=None) == moe.EINVAL
    assert call(x=None) == moe.EINVAL
    assert call(y=None) == moe.EINVAL
    assert call(acc=2) == moe.EINVAL
    assert call(acc=1, yd=0) == moe.EINVAL  # accumulating needs fp32 y
    assert call(x=ctypes.c_void_p(FAKE.value + 8)) == moe.EINVAL
    assert call(wsb=need - 1) == moe.EWORKSPACE
    assert call(T=0, x=None, ws=None, wsb=0) == moe.OK
    # a one-expert bank can be packed (top_k is not used there)
    assert lib.moe_quantize_experts(ctypes.byref(sd), 1, None, FAKE, FAKE, FAKE, None, None, FAKE,
                                    FAKE, None) == moe.EINVAL


def test_noalloc_validation(lib):
    d = _dims()
    ex = moe.Experts(0, FAKE.value, FAKE.value, None, None, None, None)

    def call(T=4, e=ex, x=FAKE):
        return lib.moe_forward_noalloc(ctypes.byref(d), T, x, FAKE, FAKE,
                                       e if e is None else ctypes.byref(e), FAKE, 1, None)

    assert call(e=None) == moe.EINVAL
    assert call(T=-1) == moe.EINVAL
    assert call(e=moe.Experts(7, FAKE.value, FAKE.value, None, None, None, None)) == moe.EINVAL
    # a batch whose workspace exceeds the fixed scratch is refused before any HIP call
    assert lib.moe_workspace_size(ctypes.byref(d), 0, 4096) > moe.NOALLOC_SCRATCH_BYTES
    assert call(T=4096) == moe.EWORKSPACE
    assert call(T=0, x=None) == moe.OK


def test_cache_validation(lib):
    d = _dims()
    assert lib.moe_cache_state_size(ctypes.byref(d), 5) == 0    # fewer slots than top_k
    assert lib.moe_cache_state_size(ctypes.byref(d), 129) == 0  # more slots than experts
    assert lib.moe_cache_state_size(None, 32) == 0
    n = lib.moe_cache_state_size(ctypes.byref(d), 32)
    assert n > 0
    state = (ctypes.c_uint64 * (n // 8 + 1))()
    host = moe.Experts(0, FAKE.value, FAKE.value, None, None, None, None)

    def cache(n_slots=32, h=host, up_s=None, slot_up=FAKE.value, slot_bs=None, slot_of=FAKE.value):
        return moe.Cache(n_slots, h, up_s, up_s, slot_up, FAKE.value, slot_bs, slot_bs, slot_of)

    def init(c, st=state, nb=n):
        return lib.moe_cache_init(ctypes.byref(d), ctypes.byref(c), st, nb, None)

    assert init(cache(n_slots=4)) == moe.EINVAL
    assert init(cache(n_slots=200)) == moe.EINVAL
    assert init(cache(slot_up=None)) == moe.EINVAL
    assert init(cache(slot_of=None)) == moe.EINVAL
    # quantised banks need their resident scales, NVFP4 also block scales
    assert init(cache(h=moe.Experts(1, FAKE.value, FAKE.value, None, None, None, None))) == moe.EINVAL
    nv = moe.Experts(2, FAKE.value, FAKE.value, None, None, None, None)
    assert init(cache(h=nv, up_s=FAKE.value, slot_bs=FAKE.value)) == moe.EINVAL
    assert init(cache(), st=None) == moe.EINVAL
    assert init(cache(), nb=n - 1) == moe.EINVAL
    assert init(cache(), st=ctypes.c_void_p(ctypes.addressof(state) + 4)) == moe.EINVAL
    # a state moe_cache_init has not set up is refused before any launch
    c = cache()
    need = lib.moe_workspace_size(ctypes.byref(d), 0, 4)
    assert lib.moe_forward_cached(ctypes.byref(d), 4, FAKE, FAKE, FAKE, ctypes.byref(c), state,
                                  FAKE, 1, FAKE, need, None, None) == moe.EINVAL
    assert lib.moe_forward_cached(ctypes.byref(d), 4, FAKE, FAKE, FAKE, None, state, FAKE, 1,
                                  FAKE, need, None, None) == moe.EINVAL


def test_quantize_validation(lib):
    d = _dims()
    q = lib.moe_quantize_experts
    assert q(ctypes.byref(d), 0, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None) == moe.EINVAL
    assert q(ctypes.byref(d), 2, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None) == moe.EINVAL
    assert q(ctypes.byref(d), 1, None, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None) == moe.EINVAL
    assert q(ctypes.byref(d), 1, ctypes.c_void_p(FAKE.value + 2), FAKE, FAKE, FAKE, None, None,
             FAKE, FAKE, None) == moe.EINVAL
    a = lib.moe_quantize_activation
    assert a(1, 4, 64, ctypes.c_void_p(FAKE.value + 2), FAKE, None, FAKE, FAKE, 256, None) == moe.EINVAL
    assert a(1, 4, 64, FAKE, ctypes.c_void_p(FAKE.value + 4), None, FAKE, FAKE, 256, None) == moe.EINVAL
    assert a(0, 4, 64, FAKE, FAKE, None, FAKE, FAKE, 256, None) == moe.EINVAL
    assert a(1, 4, 60, FAKE, FAKE, None, FAKE, FAKE, 256, None) == moe.EINVAL
    assert a(2, 4, 64, FAKE, FAKE, None, FAKE, FAKE, 256, None) == moe.EINVAL
    assert a(1, 4, 64, FAKE, FAKE, None, FAKE, FAKE, 16, None) == moe.EWORKSPACE
    assert a(1, 0, 64, FAKE, FAKE, None, FAKE, FAKE, 256, None) == moe.OK
    assert lib.moe_prenorm(4, 63, FAKE, FAKE, None) == moe.EINVAL
    assert lib.moe_prenorm(0, 64, FAKE, FAKE, None) == moe.OK
    assert lib.moe_residual_add(4, 64, None, FAKE, None) == moe.EINVAL
    rp = lib.moe_residual_prenorm
    assert rp(4, 64, None, FAKE, FAKE, None) == moe.EINVAL
    assert rp(4, 64, FAKE, None, FAKE, None) == moe.EINVAL
    assert rp(4, 64, FAKE, FAKE, None, None) == moe.EINVAL
    assert rp(4, 64, FAKE, FAKE, FAKE, None) == moe.EINVAL  # out aliases x
    assert rp(4, 60, FAKE, FAKE, ctypes.c_void_p(FAKE.value + 4096), None) == moe.EINVAL
    assert rp(0, 64, FAKE, FAKE, ctypes.c_void_p(FAKE.value + 4096), None) == moe.OK
    # rows move in 16-byte chunks: misaligned pointers are rejected
    odd = ctypes.c_void_p(FAKE.value + 8)
    assert lib.moe_prenorm(4, 64, odd, FAKE, None) == moe.EINVAL
    assert lib.moe_prenorm(4, 64, FAKE, odd, None) == moe.EINVAL
    assert rp(4, 64, odd, FAKE, ctypes.c_void_p(FAKE.value + 4096), None) == moe.EINVAL
    assert rp(4, 64, FAKE, odd, ctypes.c_void_p(FAKE.value + 4096), None) == moe.EINVAL
    assert rp(4, 64, FAKE, FAKE, ctypes.c_void_p(FAKE.value + 4104), None) == moe.EINVAL


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", os.path.join(ROOT, "no_such_libmoe.so"))
    with pytest.raises(ImportError):
        moe.lib()


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "sparse_moe_routed_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), f
                assert "oracle." not in text.replace("the oracle.", ""), f
