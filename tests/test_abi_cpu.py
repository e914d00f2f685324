"""CPU checks of the C ABI: the shared library loads, exports every function the header declares,
and rejects invalid arguments on the host before touching the GPU (no compute calls here)."""

import ctypes
import math
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "diffattn.h")


# tests/test_abi_sanitized.py re-runs this file against an AddressSanitizer + UBSan build of the
# host layer, named by this variable; otherwise the in-tree library is checked
SANITIZED_LIB = os.environ.get("DIFFATTN_SANITIZED_LIB")


@pytest.fixture(scope="module")
def da():
    import differential_softmax_attention_diff_amd as mod

    if SANITIZED_LIB:
        mod._LIB = mod.load_library(SANITIZED_LIB)
        mod.LIB_PATH = SANITIZED_LIB
        return mod
    if not os.path.exists(mod.LIB_PATH):
        pytest.fail("libdiffattn.so is not built (run __graft_entry__.build())")
    mod.load_library()
    return mod


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(diffattn_\w+)\s*\(", text)))


def test_header_symbols_exported(da):
    names = _declared_functions()
    assert len(names) == 18, names
    lib = ctypes.CDLL(da.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_lambda_init_helper_matches_oracle(da):
    for l in range(1, 41):
        assert da.diffattn_lambda_init(l) == pytest.approx(oracle.lambda_init(l), abs=1e-15)
    assert math.isnan(da.diffattn_lambda_init(0))


def test_status_strings(da):
    for s in range(6):
        assert da.diffattn_status_string(s).startswith(da.STATUS_NAMES[s])
    assert "gfx950" in da.diffattn_version()


def _t(ptr=0x10000, sb=0, sh=0, sn=64):
    return da_mod().DaTensor(ptr, sb, sh, sn)


def da_mod():
    import differential_softmax_attention_diff_amd as mod
    return mod


def _lam(layer=1, dl=64, ptr=0x20000):
    m = da_mod()
    return m.DaLambda(ptr, ptr, ptr, ptr, dl, layer, None, None)


def _v1(lib, ts, B=1, H=1, N=8, d=64, dt=1, lam=None, causal=1, eps=1e-5, flags=0):
    lam = lam if lam is not None else _lam()
    return lib.diffattn_fwd_v1(*ts, B, H, N, d, dt, ctypes.byref(lam), causal, eps, flags, None)


def test_v1_host_validation(da):
    lib = da.load_library()
    good = [_t() for _ in range(6)]
    assert _v1(lib, good, B=0) == 0                         # empty: OK, nothing enqueued
    assert _v1(lib, good, N=0) == 0
    assert _v1(lib, good, B=-1) == 2
    assert _v1(lib, good, d=32) == 3                         # unsupported width
    assert _v1(lib, good, d=0) == 2
    assert _v1(lib, good, dt=7) == 3
    assert _v1(lib, good, eps=-1.0) == 2
    assert _v1(lib, good, eps=float("nan")) == 2
    assert _v1(lib, good, flags=8) == 3
    assert _v1(lib, good, lam=_lam(layer=0)) == 2
    assert _v1(lib, good, lam=_lam(dl=0)) == 2
    assert _v1(lib, good, lam=_lam(ptr=0)) == 1
    bad = list(good)
    bad[2] = _t(ptr=0)
    assert _v1(lib, bad) == 1                                # NULL k1
    bad[2] = _t(ptr=0x10008)
    assert _v1(lib, bad) == 1                                # misaligned
    bad[2] = _t(sn=63)
    assert _v1(lib, bad) == 2                                # row stride breaks alignment
    bad[2] = _t(sn=-64)
    assert _v1(lib, bad) == 2
    assert lib.diffattn_fwd_v1(*good, 1, 1, 8, 64, 1, None, 1, 1e-5, 0, None) == 1  # no lambda


def test_v2_and_decode_host_validation(da):
    lib = da.load_library()
    t5 = [_t() for _ in range(5)]
    lam = _lam(dl=128)
    v2ws = da.diffattn_fwd_v2_workspace_bytes(1, 2, 8, 128)
    v2 = lambda B, P, Hkv, N, D, dt, ws=0x40000, nbytes=v2ws: lib.diffattn_fwd_v2(
        *t5, B, P, Hkv, N, D, dt, ctypes.byref(lam), 1, ws, nbytes, None)
    assert v2(1, 3, 2, 8, 128, 1) == 2  # P % Hkv
    assert v2(1, 4, 2, 8, 64, 1) == 3   # D
    assert v2(1, 4, 2, 8, 128, 0) == 3  # fp32
    assert v2(1, 4, 0, 8, 128, 1) == 2
    assert v2(0, 4, 2, 8, 128, 1) == 0
    assert v2(1, 1 << 16, 2, 1 << 22, 128, 1) == 3  # grid
    assert v2(1, 4, 2, 8, 128, 1, ws=None) == 4     # no workspace
    assert v2(1, 4, 2, 8, 128, 1, nbytes=v2ws - 1) == 4
    assert v2(1, 4, 2, 8, 128, 1, ws=0x40008) == 4  # misaligned workspace
    assert v2(1 << 9, 256, 128, 8, 128, 1) == 3  # B * Hkv beyond the conversion pass's grid
    need = da.diffattn_decode_workspace_bytes(2, 4, 2, 1000, 128)
    assert need > 0
    assert da.diffattn_decode_workspace_bytes(2, 3, 2, 1000, 128) == 0
    dec = lambda ws, nbytes, P=4, Hkv=2, L=1000: lib.diffattn_decode(
        *t5, 2, P, Hkv, L, 128, 1, ctypes.byref(lam), 0, ws, nbytes, None)
    assert dec(None, need) == 4
    assert dec(0x30000, need - 1) == 4
    assert dec(0x30008, need) == 4                           # misaligned workspace
    assert dec(0x30000, need, P=3) == 2
    assert dec(0x30000, need, P=16, Hkv=1) == 3              # 32 query heads on one KV head
    assert dec(0x30000, need, L=0) == 2


def test_decode_noalloc_host_validation(da):
    """The allocation-free decode checks its arguments like diffattn_decode and refuses sizes
    beyond its fixed scratch on the host, before any HIP call (so this runs without a GPU)."""
    lib = da.load_library()
    t5 = [_t() for _ in range(5)]
    lam = _lam(dl=128)
    call = lambda B=2, P=4, Hkv=2, L=1000, D=128, dt=1, splits=0, lamp=ctypes.byref(lam): \
        lib.diffattn_decode_noalloc(*t5, B, P, Hkv, L, D, dt, lamp, splits, None)
    assert call(B=0) == 0
    assert call(P=3) == 2
    assert call(D=64) == 3
    assert call(dt=0) == 3
    assert call(L=0) == 2
    assert call(P=16, Hkv=1) == 3
    assert call(lamp=None) == 1
    bad = list(t5)
    bad[4] = _t(ptr=0x10008)
    assert lib.diffattn_decode_noalloc(*bad, 2, 4, 2, 1000, 128, 1, ctypes.byref(lam), 0, None) == 1
    # 64 x 32 query heads x 16 splits x 130 floats is 17 MB, beyond the 16 MiB scratch
    assert da.diffattn_decode_workspace_bytes(64, 16, 8, 8192, 128, 16) > da.DIFFATTN_DECODE_NOALLOC_MAX_BYTES
    assert call(B=64, P=16, Hkv=8, L=8192, splits=16) == 4
    # the decode workload's own partials fit
    assert da.diffattn_decode_workspace_bytes(64, 16, 8, 32768, 128, 0) <= da.DIFFATTN_DECODE_NOALLOC_MAX_BYTES


def test_v2_workspace_size_formula(da):
    # 16-bit V copy rounded up to 256 bytes, then 4 flag bytes per 32-key tile of each KV head
    assert da.diffattn_fwd_v2_workspace_bytes(1, 1, 1, 128) == 256 + 4
    assert da.diffattn_fwd_v2_workspace_bytes(2, 8, 8192, 128) == 2 * 8 * 8192 * 256 + 2 * 8 * 256 * 4
    assert da.diffattn_fwd_v2_workspace_bytes(1, 2, 33, 128) == 2 * 33 * 256 + 2 * 2 * 4
    assert da.diffattn_fwd_v2_workspace_bytes(1, 2, 33, 64) == 0
    assert da.diffattn_fwd_v2_workspace_bytes(0, 2, 33, 128) == 0


def test_decode_workspace_size_formula(da):
    # B * 2P * splits * (D + 2) floats; the split count never exceeds one per 256 keys
    assert da.diffattn_decode_workspace_bytes(1, 1, 1, 100, 128, 0) == 1 * 2 * 1 * 130 * 4
    # 3 requested splits -> chunks of ceil(1000 / 3) rounded up to 512 keys -> 2 splits
    assert da.diffattn_decode_workspace_bytes(1, 1, 1, 1000, 128, 3) == 2 * 2 * 130 * 4
    assert da.diffattn_decode_workspace_bytes(1, 1, 1, 1000, 128, 50) == 2 * 4 * 130 * 4
    b = da.diffattn_decode_workspace_bytes(64, 16, 8, 32768, 128, 0)
    assert b == 64 * 32 * 8 * 130 * 4


def test_decode_v1_host_validation(da):
    lib = da.load_library()
    t6 = [_t() for _ in range(6)]
    lam = _lam(dl=64)
    need = da.diffattn_decode_v1_workspace_bytes(2, 4, 1000, 64)
    assert need > 0
    assert da.diffattn_decode_v1_workspace_bytes(2, 4, 1000, 128) == 0   # d != 64
    dec = lambda ws, nbytes, B=2, H=4, L=1000, d=64, dt=1, eps=1e-5, flags=0, lam=lam: \
        lib.diffattn_decode_v1(*t6, B, H, L, d, dt, ctypes.byref(lam), eps, flags, 0, ws, nbytes, None)
    assert dec(None, need) == 4                              # no workspace
    assert dec(0x30000, need - 1) == 4                       # too small
    assert dec(0x30008, need) == 4                           # misaligned workspace
    assert dec(0x30000, need, d=128) == 3
    assert dec(0x30000, need, d=0) == 2
    assert dec(0x30000, need, dt=0) == 3                     # fp32
    assert dec(0x30000, need, L=0) == 2
    assert dec(0x30000, need, B=-1) == 2
    assert dec(0x30000, need, B=0) == 0
    assert dec(0x30000, need, eps=float("nan")) == 2
    assert dec(0x30000, need, flags=2) == 3
    assert dec(0x30000, need, lam=_lam(layer=0)) == 2
    bad = [_t() for _ in range(6)]
    bad[2] = _t(ptr=0x10008)                                 # misaligned K1 cache
    assert lib.diffattn_decode_v1(*bad, 2, 4, 1000, 64, 1, ctypes.byref(lam), 1e-5, 0, 0, 0x30000,
                                  need, None) == 1


def test_decode_v1_workspace_size_formula(da):
    # B * H * 2 branches * splits * (2d + 2) floats; at most one split per 256 keys
    assert da.diffattn_decode_v1_workspace_bytes(1, 1, 100, 64, 0) == 1 * 2 * 1 * 130 * 4
    assert da.diffattn_decode_v1_workspace_bytes(1, 1, 1000, 64, 3) == 2 * 2 * 130 * 4
    assert da.diffattn_decode_v1_workspace_bytes(32, 16, 32768, 64, 0) == 32 * 16 * 2 * 8 * 130 * 4


def test_window_host_validation(da):
    lib = da.load_library()
    t6 = [_t() for _ in range(6)]
    lam = _lam()
    w1 = lambda window, B=1, H=1, N=8: lib.diffattn_fwd_v1_window(
        *t6, B, H, N, 64, 1, ctypes.byref(lam), window, 1e-5, 0, None)
    assert w1(0) == 2                      # the window needs at least one key
    assert w1(-3) == 2
    assert w1(4, B=0) == 0
    t5 = [_t() for _ in range(5)]
    lam2 = _lam(dl=128)
    w2 = lambda window, P=4, Hkv=2: lib.diffattn_fwd_v2_window(
        *t5, 1, P, Hkv, 8, 128, 1, ctypes.byref(lam2), window, 0x40000, 1 << 20, None)
    assert w2(0) == 2
    assert w2(5, P=3) == 2                 # P % Hkv
    # the causal entry points reject nothing new
    assert _v1(lib, t6, N=0) == 0


def test_binding_window_requires_causal(da):
    import torch

    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    v = torch.zeros(1, 1, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        da.diffattn_fwd_v1(x, x, x, x, v, layer=1, out=v, causal=False, window=4)


def test_paged_decode_host_validation(da):
    lib = da.load_library()
    t3 = [_t() for _ in range(3)]
    lam = _lam(dl=128)
    need = da.diffattn_decode_workspace_bytes(2, 4, 2, 1000, 128)
    call = lambda page=16, pages=100, mb=64, ml=1000, P=4, Hkv=2, D=128, ws=0x30000, nbytes=need, \
        kp=0x40000, bt=0x50000: lib.diffattn_decode_paged(
            t3[0], t3[1], kp, 0x40000, bt, 0x60000, t3[2], 2, P, Hkv, D, page, pages, mb, ml, 1,
            ctypes.byref(lam), 0, ws, nbytes, None)
    assert call(page=12) == 2            # not a power of two
    assert call(page=0) == 2
    assert call(ml=0) == 2
    assert call(mb=10) == 2              # 10 pages of 16 keys cannot hold 1000
    assert call(pages=0) == 2
    assert call(D=64) == 3
    assert call(P=3) == 2
    assert call(P=16, Hkv=1) == 3        # 32 query heads on one KV head
    assert call(kp=0x40008) == 1         # misaligned page pool
    assert call(kp=0) == 1
    assert call(bt=0x50002) == 1         # misaligned block table
    assert call(ws=None) == 4
    assert call(nbytes=need - 1) == 4


def test_binding_refuses_cpu_tensors(da):
    import torch

    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    v = torch.zeros(1, 1, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        da.diffattn_fwd_v1(x, x, x, x, v, layer=1, out=v, lambda_override=None)


def test_train_and_bwd_sizes(da):
    # stash: O_1, O_2 [2, B, H, N, 2d] fp32, then LSE_1, LSE_2, D_1, D_2 [4, B, H, N] fp32
    bhn = 2 * 3 * 100
    assert da.diffattn_v1_train_stash_bytes(2, 3, 100, 64) == (2 * bhn * 128 + 4 * bhn) * 4
    # workspace: dO bf16 [B, H, N, 2d], then the rows' dlambda shares fp32 [B, H, N]
    assert da.diffattn_bwd_v1_workspace_bytes(2, 3, 100, 64) == bhn * 128 * 2 + bhn * 4
    assert da.diffattn_v1_train_stash_bytes(1, 1, 8, 32) == 0
    assert da.diffattn_bwd_v1_workspace_bytes(0, 1, 8, 64) == 0


def test_train_and_bwd_host_validation(da):
    lib = da.load_library()
    t6 = [_t() for _ in range(6)]
    lam = _lam(dl=64)
    B, H, N = 1, 2, 40
    stash = da.diffattn_v1_train_stash_bytes(B, H, N, 64)
    ws = da.diffattn_bwd_v1_workspace_bytes(B, H, N, 64)

    def train(st=0x40000, nbytes=stash, d=64, dt=1, n=N, eps=1e-5, causal=1, window=0):
        return lib.diffattn_fwd_v1_train(*t6, B, H, n, d, dt, ctypes.byref(lam), causal, window, eps,
                                         st, nbytes, None)

    assert train(n=0) == 0                                   # empty: nothing enqueued
    assert train(n=-1) == 2
    assert train(dt=0) == 3                                  # the training path is bf16 only
    assert train(d=128) == 3
    assert train(st=None) == 4
    assert train(nbytes=stash - 1) == 4
    assert train(st=0x40008) == 4                            # misaligned stash
    assert train(window=-1) == 2
    assert train(window=16, causal=0) == 2                   # the window is a causal one

    g = da_mod().DaLambdaGrad(0x50000, 0x50000, 0x50000, 0x50000)
    grads = [0x60000] * 5

    def bwd(gr=grads, lg=g, st=0x40000, sb=stash, w=0x70000, wb=ws, d=64, dt=1, n=N, eps=1e-5,
            lm=lam, causal=1, window=0):
        return lib.diffattn_bwd_v1(*t6, *gr, B, H, n, d, dt, ctypes.byref(lm),
                                   ctypes.byref(lg) if lg is not None else None, causal, window,
                                   eps, st, sb, w, wb, None)

    assert bwd(n=0) == 0
    assert bwd(n=-3) == 2
    assert bwd(dt=0) == 3
    assert bwd(d=32) == 3
    assert bwd(eps=float("nan")) == 2
    assert bwd(gr=[0x60000, 0, 0x60000, 0x60000, 0x60000]) == 1     # missing dq2
    assert bwd(gr=[0x60008] + [0x60000] * 4) == 1                    # misaligned dq1
    assert bwd(lg=None) == 1                          # lambda vectors need their gradients
    assert bwd(lg=da_mod().DaLambdaGrad(0x50000, None, 0x50000, 0x50000)) == 1
    assert bwd(st=None) == 4
    assert bwd(sb=stash - 16) == 4
    assert bwd(w=None) == 4
    assert bwd(wb=ws - 1) == 4
    assert bwd(w=0x70008) == 4
    assert bwd(lm=_lam(layer=0)) == 2
    assert bwd(window=-2) == 2
    assert bwd(window=8, causal=0) == 2
    bad = list(t6)
    bad[5] = _t(ptr=0)
    assert lib.diffattn_bwd_v1(*bad, *grads, B, H, N, 64, 1, ctypes.byref(lam), ctypes.byref(g), 1,
                               0, 1e-5, 0x40000, stash, 0x70000, ws, None) == 1   # NULL dy
