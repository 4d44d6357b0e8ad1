"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, the host helpers compute what they document, and invalid arguments
are rejected with the documented status before any device work.  The device
pointers passed here are never dereferenced: every call returns in validation."""

import ctypes

import numpy as np
import pytest

import oracle as O
from orthogonal_reparameterized_cnp_amd import binding as B


@pytest.fixture(scope="module")
def L():
    return B.lib()


def test_exports_every_declared_symbol(L):
    names = B.header_symbols()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n


def test_host_helpers(L):
    assert B.poetx_version().startswith("libpoetx")
    assert B.poetx_packed_len(512) == 130816 and B.poetx_packed_len(1) == 0
    # G buffer: [2][nb][b][b]
    assert B.poetx_g_bytes(1376, 256, B.POETX_BF16) == 2 * 6 * 256 * 256 * 2
    assert B.poetx_g_bytes(256, 32, B.POETX_F32) == 2 * 8 * 32 * 32 * 4
    assert B.poetx_g_bytes(256, 32, B.POETX_I8) == 0
    d = B.desc(1024, 5461, 256, "bf16", "i8")
    ldw = 5504
    assert B.poetx_weight_bytes(d) == (1024 * ldw + 255) // 256 * 256 + 4 * ldw
    # bf16: values, then at a 256-byte boundary the transposed copy [n][lead(m)]
    assert B.poetx_weight_bytes(B.desc(1000, 5461, 256, "bf16", "bf16")) == (1000 * ldw * 2 + 255) // 256 * 256 + 5461 * 1024 * 2
    assert B.poetx_weight_bytes(B.desc(1000, 100, 32, "f32", "f32")) == 1000 * 128 * 4
    # saved state: H [T][lead(n)], then at a 256-byte boundary Xt [T][lead(m)]
    assert B.poetx_saved_bytes(d, 10) == (10 * ldw * 2 + 255) // 256 * 256 + 10 * 1024 * 2
    for op in (B.POETX_OP_FWD, B.POETX_OP_BWD, B.POETX_OP_MERGE):
        assert B.poetx_workspace_size(d, 100, op) > 0
    assert B.poetx_workspace_size(B.desc(1024, 5461, 1, "bf16", "bf16"), 100, B.POETX_OP_FWD) == 0
    # Xmem: the saved state is Xt alone; the forward keeps H in its workspace instead
    dm = B.desc(1024, 5461, 256, "bf16", "i8", "xmem")
    assert B.poetx_saved_bytes(dm, 10) == 10 * 1024 * 2
    assert B.poetx_workspace_size(dm, 10, B.POETX_OP_FWD) == B.poetx_workspace_size(d, 10, B.POETX_OP_FWD) + (
        (10 * ldw * 2 + 255) // 256 * 256)
    assert B.poetx_workspace_size(dm, 10, B.POETX_OP_BWD) == B.poetx_workspace_size(d, 10, B.POETX_OP_BWD)
    # Xout: Xt alone as for Xmem; the backward adds one [T][lead(n)] buffer for H taken back from Y
    do = B.desc(1024, 5461, 256, "bf16", "i8", "xout")
    assert B.poetx_saved_bytes(do, 10) == B.poetx_saved_bytes(dm, 10)
    assert B.poetx_workspace_size(do, 10, B.POETX_OP_FWD) == B.poetx_workspace_size(dm, 10, B.POETX_OP_FWD)
    assert B.poetx_workspace_size(do, 10, B.POETX_OP_BWD) == B.poetx_workspace_size(d, 10, B.POETX_OP_BWD) + (
        (10 * ldw * 2 + 255) // 256 * 256)
    bad = B.desc(1024, 5461, 256, "bf16", "i8")
    bad.mode = 3
    assert B.poetx_saved_bytes(bad, 10) == 0 and B.poetx_workspace_size(bad, 10, B.POETX_OP_FWD) == 0


@pytest.mark.parametrize("seed,d", [(0, 1), (1, 2), (123, 1376), (2**64 - 1, 5461), (42, 14336)])
def test_perm_from_seed_matches_oracle(seed, d):
    np.testing.assert_array_equal(B.poetx_perm_from_seed(seed, d), O.perm_from_seed(seed, d))


FAKE = 1 << 20  # an aligned non-null address that validation never dereferences


def _fwd(L, dsc, T=4, X=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return L.poetx_linear_fwd(ctypes.byref(dsc), T, X, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, ws_bytes, None)


def test_validation_statuses(L):
    good = B.desc(256, 256, 32, "f32", "f32")
    assert _fwd(L, B.desc(256, 256, 1, "f32", "f32")) == B.POETX_E_SHAPE
    assert _fwd(L, B.desc(0, 256, 32, "f32", "f32")) == B.POETX_E_SHAPE
    assert _fwd(L, B.desc(256, 256, 32, "f32", "bf16")) == B.POETX_E_DTYPE
    assert _fwd(L, B.desc(256, 256, 32, "bf16", "f32")) == B.POETX_E_DTYPE
    assert _fwd(L, good, T=-1) == B.POETX_E_SHAPE
    assert _fwd(L, good, X=None) == B.POETX_E_NULL
    assert "NULL" in B.poetx_last_error()
    assert _fwd(L, good, ws_bytes=16) == B.POETX_E_WORKSPACE
    assert _fwd(L, good, ws=FAKE + 8) == B.POETX_E_WORKSPACE
    assert _fwd(L, good, T=0) == B.POETX_OK  # empty batch: nothing to do
    assert L.poetx_linear_fwd(None, 4, *([FAKE] * 9), 1 << 40, None) == B.POETX_E_NULL
    # backward / merge / build / premerge
    args = [FAKE] * 13
    assert L.poetx_linear_bwd(ctypes.byref(good), 4, *args[:4], None, *args[5:13], FAKE, 16, None) == B.POETX_E_NULL
    assert L.poetx_linear_bwd(ctypes.byref(good), 4, *args, FAKE, 16, None) == B.POETX_E_WORKSPACE
    # the first tensor slot (the forward's output Y) is read only in the xout mode
    assert L.poetx_linear_bwd(ctypes.byref(good), 4, None, *args[1:], FAKE, 16, None) == B.POETX_E_WORKSPACE
    xout = B.desc(256, 256, 32, "f32", "f32", "xout")
    assert L.poetx_linear_bwd(ctypes.byref(xout), 4, None, *args[1:], FAKE, 1 << 40, None) == B.POETX_E_NULL
    assert "Y is NULL" in B.poetx_last_error()
    assert L.poetx_merge_reinit(ctypes.byref(good), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 2, FAKE, 1 << 40, None) == B.POETX_E_NULL
    assert L.poetx_cnp_build(FAKE, 256, 32, B.POETX_I8, FAKE, FAKE, 1 << 30, None) == B.POETX_E_DTYPE
    assert L.poetx_cnp_build(FAKE, 256, 1, B.POETX_F32, FAKE, FAKE, 1 << 30, None) == B.POETX_E_SHAPE
    assert L.poetx_cnp_build(FAKE, 256, 32, B.POETX_F32, FAKE, FAKE, 8, None) == B.POETX_E_WORKSPACE
    i8 = B.desc(256, 256, 32, "bf16", "i8")
    assert L.poetx_premerge(ctypes.byref(i8), FAKE, 256, None, FAKE, FAKE, FAKE, None) == B.POETX_E_NULL
    assert L.poetx_premerge(ctypes.byref(good), FAKE, 100, None, FAKE, FAKE, FAKE, None) == B.POETX_E_SHAPE
    out = (ctypes.c_int32 * 4)()
    assert L.poetx_perm_from_seed(1, 0, out) == B.POETX_E_SHAPE
    assert L.poetx_perm_from_seed(1, 4, None) == B.POETX_E_NULL


def _pp(*ptrs):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def _ii(*xs):
    return (ctypes.c_int32 * len(xs))(*xs)


def test_batched_cnp_helpers(L):
    f32, bf = B.POETX_F32, B.POETX_BF16
    # one side in a batch needs what the single build needs
    for d, b, dt in ((1376, 256, bf), (256, 32, f32), (5461, 256, bf)):
        single = B.poetx_workspace_size(B.desc(d, 1, b, "bf16" if dt == bf else "f32", "bf16" if dt == bf else "f32"),
                                        0, B.POETX_OP_CNP)
        assert B.poetx_cnp_batch_workspace_size([d], b, dt) == single > 0
    assert B.poetx_cnp_batch_workspace_size([4096, 14336], 512, bf) > B.poetx_cnp_batch_workspace_size([4096], 512, bf)
    assert L.poetx_cnp_batch_workspace_size(0, _ii(256), 32, f32) == 0
    assert B.poetx_cnp_batch_workspace_size([256], 32, B.POETX_I8) == 0
    assert B.poetx_cnp_grad_bytes(10, 512, bf) > B.poetx_cnp_grad_bytes(5, 512, bf) > 0
    assert B.poetx_cnp_grad_bytes(0, 512, bf) == 0
    assert B.poetx_cnp_grad_bytes(10, 1, bf) == 0
    assert B.poetx_cnp_grad_bytes(10, 512, B.POETX_I8) == 0


def test_batched_cnp_validation(L):
    f32 = B.POETX_F32
    big = 1 << 40
    ok3 = (_pp(FAKE, FAKE, FAKE), _ii(256, 96, 300), 32, f32, _pp(FAKE, FAKE, FAKE))
    assert L.poetx_cnp_build_batch(0, *ok3, FAKE, big, None) == B.POETX_E_SHAPE
    assert L.poetx_cnp_build_batch(65, _pp(*[FAKE] * 65), _ii(*[256] * 65), 32, f32, _pp(*[FAKE] * 65), FAKE, big,
                                   None) == B.POETX_E_SHAPE
    assert L.poetx_cnp_build_batch(3, _pp(FAKE, None, FAKE), _ii(256, 96, 300), 32, f32, _pp(FAKE, FAKE, FAKE),
                                   FAKE, big, None) == B.POETX_E_NULL
    assert L.poetx_cnp_build_batch(3, *ok3[:3], B.POETX_I8, ok3[4], FAKE, big, None) == B.POETX_E_DTYPE
    assert L.poetx_cnp_build_batch(3, *ok3, FAKE, 64, None) == B.POETX_E_WORKSPACE
    assert L.poetx_cnp_build_batch(3, ok3[0], _ii(256, 0, 300), 32, f32, ok3[4], FAKE, big, None) == B.POETX_E_SHAPE
    # more than 65535 blocks in one batch
    assert L.poetx_cnp_build_batch(2, _pp(FAKE, FAKE), _ii(1 << 20, 1 << 20), 2, f32, _pp(FAKE, FAKE), FAKE, big,
                                   None) == B.POETX_E_SHAPE
    # backward_dx: gradient state checks come after the bwd checks
    good = B.desc(256, 96, 32, "f32", "f32")  # 8 + 3 blocks
    a = [FAKE] * 11
    bwd_dx = lambda dg, first, total: L.poetx_linear_bwd_dx(ctypes.byref(good), 4, *a, dg, first, total, FAKE, big,
                                                            None)
    assert bwd_dx(None, 0, 11) == B.POETX_E_NULL
    assert bwd_dx(FAKE + 16, 0, 11) == B.POETX_E_WORKSPACE
    assert bwd_dx(FAKE, 1, 11) == B.POETX_E_SHAPE
    assert bwd_dx(FAKE, -1, 20) == B.POETX_E_SHAPE
    assert L.poetx_linear_bwd_dx(ctypes.byref(good), 4, *a, FAKE, 0, 11, FAKE, 16, None) == B.POETX_E_WORKSPACE
    # backward_batch
    need = B.poetx_cnp_grad_bytes(11, 32, f32)
    bb = lambda dq, dg_bytes: L.poetx_cnp_backward_batch(2, _pp(FAKE, FAKE), _ii(256, 96), 32, f32, FAKE, dg_bytes,
                                                         dq, None)
    assert bb(_pp(FAKE, None), need) == B.POETX_E_NULL
    assert bb(_pp(FAKE, FAKE), need - 1) == B.POETX_E_WORKSPACE
    assert L.poetx_cnp_backward_batch(2, _pp(FAKE, FAKE), _ii(256, 96), 32, f32, None, need, _pp(FAKE, FAKE),
                                      None) == B.POETX_E_NULL


def test_adam_validation(L):
    """Every rejected call returns before any launch (no GPU needed)."""
    ll = lambda *xs: (ctypes.c_int64 * len(xs))(*xs)
    hp = lambda **kw: B.AdamParams(**{**dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, t=1), **kw})
    four = [_pp(FAKE, FAKE) for _ in range(4)]
    call = lambda n, lens, arrs, h: L.poetx_adam_step_batch(n, lens, *arrs, ctypes.byref(h) if h else None, None)
    assert call(0, ll(10, 10), four, hp()) == B.POETX_E_SHAPE
    assert L.poetx_adam_step_batch(65, ll(*[1] * 65), *[_pp(*[FAKE] * 65)] * 4, ctypes.byref(hp()), None) == \
        B.POETX_E_SHAPE
    assert call(2, ll(10, 10), four, None) == B.POETX_E_NULL
    assert call(2, None, four, hp()) == B.POETX_E_NULL
    assert call(2, ll(10, 10), [four[0], None, four[2], four[3]], hp()) == B.POETX_E_NULL
    assert call(2, ll(10, 10), [four[0], _pp(FAKE, None), four[2], four[3]], hp()) == B.POETX_E_NULL
    assert call(2, ll(10, -1), four, hp()) == B.POETX_E_SHAPE
    assert call(2, ll(10, (1 << 36) + 1), four, hp()) == B.POETX_E_SHAPE
    for bad in (dict(t=0), dict(beta1=1.0), dict(beta2=-0.1), dict(eps=0.0), dict(lr=-1.0), dict(lr=float("nan")),
                dict(weight_decay=float("inf")), dict(beta1=float("nan"))):
        assert call(2, ll(10, 10), four, hp(**bad)) == B.POETX_E_SHAPE, bad
    assert call(2, ll(10, 10), four, hp(t=0)) == B.POETX_E_SHAPE and "t must be" in B.poetx_last_error()
    assert B.POETX_KC_OPTIM == 6 and L.poetx_timer_enable(B.POETX_KC_OPTIM) == B.POETX_OK
    assert L.poetx_timer_enable(7) == B.POETX_E_SHAPE
    assert L.poetx_timer_enable(0) == B.POETX_OK


def test_spo_helpers_and_validation(L):
    """Sizes of the SPO factor calls, and every rejection before any launch."""
    blk = B.spo_desc(300, 64, "block", "bf16")
    full = B.spo_desc(1000, 256, "full", "f32")
    assert B.poetx_spo_saved_bytes(blk, 96) == 96 * 320 * 2
    assert B.poetx_spo_saved_bytes(full, 10) == 10 * 256 * 4
    assert B.poetx_spo_workspace_size(blk, 96, B.POETX_OP_BWD) > B.poetx_spo_workspace_size(blk, 96, B.POETX_OP_FWD) > 0
    assert B.poetx_spo_workspace_size(blk, 96, B.POETX_OP_MERGE) == 0
    for bad in (B.spo_desc(100, 128, "full", "bf16"), B.spo_desc(0, 64, "block", "bf16"),
                B.spo_desc(64, 1, "block", "bf16"), B.SpoDesc(64, 32, 2, B.POETX_BF16),
                B.SpoDesc(64, 32, 0, B.POETX_I8)):
        assert B.poetx_spo_saved_bytes(bad, 4) == 0
        assert B.poetx_spo_workspace_size(bad, 4, B.POETX_OP_FWD) == 0
    big = 1 << 40
    fwd = lambda dsc, T, X=FAKE, ws=FAKE, wsb=big: L.poetx_spo_fwd(ctypes.byref(dsc), T, X, FAKE, FAKE, FAKE, FAKE,
                                                                    ws, wsb, None)
    assert fwd(B.spo_desc(100, 128, "full", "bf16"), 4) == B.POETX_E_SHAPE
    assert fwd(B.SpoDesc(64, 32, 0, B.POETX_I8), 4) == B.POETX_E_DTYPE
    assert fwd(blk, -1) == B.POETX_E_SHAPE
    assert fwd(blk, 4, X=None) == B.POETX_E_NULL
    assert fwd(blk, 4, wsb=16) == B.POETX_E_WORKSPACE
    assert fwd(blk, 4, ws=FAKE + 8) == B.POETX_E_WORKSPACE
    assert fwd(blk, 0, X=None) == B.POETX_OK  # nothing to do
    bwd = lambda T, q=FAKE, dY=FAKE: L.poetx_spo_bwd(ctypes.byref(blk), T, dY, FAKE, FAKE, q, FAKE, FAKE, FAKE, FAKE,
                                                     big, None)
    assert bwd(4, q=None) == B.POETX_E_NULL
    assert bwd(4, dY=None) == B.POETX_E_NULL
    assert L.poetx_spo_bwd(ctypes.byref(blk), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == \
        B.POETX_E_WORKSPACE


def test_cnp_build_noalloc_limits(L):
    """The no-allocation CNP build rejects, before any device call, a side whose workspace
    exceeds the fixed scratch array (60 MiB): 40 blocks of 512 fit in bf16, 41 do not."""
    lim = 60 << 20
    cnp_ws = lambda d, act: B.poetx_workspace_size(B.desc(d, 1, 512, act, act), 0, B.POETX_OP_CNP)
    assert cnp_ws(40 * 512, "bf16") <= lim < cnp_ws(41 * 512, "bf16")
    assert cnp_ws(20 * 512, "f32") <= lim < cnp_ws(21 * 512, "f32")
    assert L.poetx_cnp_build_noalloc(FAKE, 41 * 512, 512, B.POETX_BF16, FAKE, None) == B.POETX_E_WORKSPACE
    assert L.poetx_cnp_build_noalloc(FAKE, 21 * 512, 512, B.POETX_F32, FAKE, None) == B.POETX_E_WORKSPACE
    assert L.poetx_cnp_build_noalloc(None, 512, 512, B.POETX_BF16, FAKE, None) == B.POETX_E_NULL
    assert L.poetx_cnp_build_noalloc(FAKE, 512, 1, B.POETX_BF16, FAKE, None) == B.POETX_E_SHAPE
    assert L.poetx_cnp_build_noalloc(FAKE, 512, 512, B.POETX_I8, FAKE, None) == B.POETX_E_DTYPE


def test_weight_centric_sizes_and_statuses(L):
    d = B.desc(1000, 300, 256, "bf16", "bf16")
    T = 70
    # state: M and U [m][lead(n)], V^T [n][lead(m)], Xt [T][lead(m)], each at a 256-byte boundary
    al = lambda x: (x + 255) // 256 * 256
    assert B.poetx_wc_state_bytes(d, T) == 2 * al(1000 * 320 * 2) + al(300 * 1024 * 2) + al(T * 1024 * 2)
    assert B.poetx_wc_workspace_size(d, T, B.POETX_OP_FWD) > 0
    assert B.poetx_wc_workspace_size(d, T, B.POETX_OP_BWD) > 0
    assert B.poetx_wc_workspace_size(d, T, B.POETX_OP_MERGE) == 0
    i8 = B.desc(1000, 300, 256, "bf16", "i8")
    assert B.poetx_wc_state_bytes(i8, T) == 0
    args = [FAKE] * 9
    assert L.poetx_wc_fwd(ctypes.byref(i8), T, *args, 1 << 40, None) == B.POETX_E_UNSUPPORTED
    assert L.poetx_wc_fwd(ctypes.byref(d), -1, *args, 1 << 40, None) == B.POETX_E_SHAPE
    assert L.poetx_wc_fwd(ctypes.byref(d), T, *([FAKE] * 8 + [None]), 1 << 40, None) == B.POETX_E_NULL
    assert L.poetx_wc_fwd(ctypes.byref(d), T, *args, 16, None) == B.POETX_E_WORKSPACE
    bargs = [FAKE] * 12  # dZ, perm_R, perm_P, g_R, g_P, q_R, q_P, state, dX, dq_R, dq_P, ws
    assert L.poetx_wc_bwd(ctypes.byref(i8), T, *bargs, 1 << 40, None) == B.POETX_E_UNSUPPORTED
    assert L.poetx_wc_bwd(ctypes.byref(d), T, *([FAKE] * 10 + [None, FAKE]), 1 << 40, None) == B.POETX_E_NULL
    assert L.poetx_wc_bwd(ctypes.byref(d), T, *([FAKE] * 11 + [None]), 1 << 40, None) == B.POETX_E_NULL
    assert L.poetx_wc_bwd(ctypes.byref(d), T, *bargs, 16, None) == B.POETX_E_WORKSPACE


def test_binding_signatures_match_header():
    """Every C entry point the binding types has the header's number of parameters: a missing one
    would make ctypes pass the trailing arguments (the stream handle) with default conversions."""
    import re

    text = open(B.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    decls = {}
    for m in re.finditer(r"\b(poetx_\w+)\s*\(([^;{]*?)\)\s*;", text, re.S):
        params = m.group(2).strip()
        decls[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    assert set(B._SIG) <= set(decls), sorted(set(B._SIG) - set(decls))
    for name, (_, args) in B._SIG.items():
        assert len(args) == decls[name], f"{name}: binding types {len(args)} arguments, header declares {decls[name]}"


def test_fold_and_store_statuses(L):
    d = B.desc(320, 200, 64, "bf16", "bf16")
    fP = B.spo_desc(200, 64, "block", "bf16")
    fR = B.spo_desc(320, 64, "full", "bf16")
    assert B.poetx_fold_workspace_size(d, 1, fP) > 0 and B.poetx_fold_workspace_size(d, 0, fR) > 0
    assert B.poetx_fold_workspace_size(d, 0, fP) == 0  # a P-side factor has d = n, not m
    assert B.poetx_fold_workspace_size(d, 2, fP) == 0
    assert B.poetx_store_workspace_size(d) == 256 * ((200 * 4 + 255) // 256)
    fold = lambda side, f, W=FAKE, ldw=256, ws_bytes=1 << 40: L.poetx_fold_factor(
        ctypes.byref(d), side, ctypes.byref(f), FAKE, FAKE, FAKE, W, ldw, FAKE, ws_bytes, None)
    assert fold(0, fP) == B.POETX_E_SHAPE
    assert fold(1, fP, W=None) == B.POETX_E_NULL
    assert fold(1, fP, ldw=199) == B.POETX_E_SHAPE
    assert fold(1, fP, ws_bytes=16) == B.POETX_E_WORKSPACE
    assert L.poetx_store_weight(ctypes.byref(d), FAKE, 199, FAKE, FAKE, 1 << 40, None) == B.POETX_E_SHAPE
    assert L.poetx_store_weight(ctypes.byref(d), FAKE, 256, None, FAKE, 1 << 40, None) == B.POETX_E_NULL
    assert L.poetx_store_weight(ctypes.byref(d), FAKE, 256, FAKE, FAKE, 16, None) == B.POETX_E_WORKSPACE


def test_block_grads_batch_statuses(L):
    """Argument checks of the batched block gradients (each returns before any launch)."""
    d = [4096, 4096, 4096, 1024, 14336, 4096]
    b, bf = 512, B.DTYPES["bf16"]
    blocks = sum((x + b - 1) // b for x in d)
    # the token range is split for the whole batch; fp32 partials of S splits of every block
    need = B.poetx_block_grads_workspace_size(d, 8192, b, bf)
    assert need > 0 and need % (blocks * b * b * 4) == 0
    assert B.poetx_block_grads_workspace_size(d, 8192, b, B.DTYPES["f32"]) == 0  # fp32: no token splits
    assert B.poetx_block_grads_workspace_size(d, -1, b, bf) == 0
    assert B.poetx_block_grads_workspace_size([], 8192, b, bf) == 0
    dg_bytes = B.poetx_cnp_grad_bytes(blocks, b, bf)
    sides = [B.GradSide(FAKE, x, FAKE, x, x) for x in d]

    def call(sides=sides, rows=8192, dtype=bf, dg=FAKE, dg_bytes=dg_bytes, ws=FAKE, ws_bytes=need, count=None):
        arr = (B.GradSide * len(sides))(*sides) if sides else None
        n = len(sides) if count is None else count
        return L.poetx_block_grads_batch(n, arr, rows, b, dtype, dg, dg_bytes, ws, ws_bytes, None)

    assert call(sides=[]) == B.POETX_E_NULL
    assert call(count=0) == B.POETX_E_SHAPE
    assert call(count=B.POETX_MAX_SIDES + 1) == B.POETX_E_SHAPE
    assert call(rows=-1) == B.POETX_E_SHAPE
    assert call(dtype=B.DTYPES["i8"]) == B.POETX_E_DTYPE
    assert call(dg=None) == B.POETX_E_NULL
    assert call(dg_bytes=dg_bytes - 1) == B.POETX_E_WORKSPACE
    assert call(dg=FAKE + 16) == B.POETX_E_WORKSPACE  # not 256-byte aligned
    assert call(ws_bytes=need - 1) == B.POETX_E_WORKSPACE
    assert call(ws=None) == B.POETX_E_WORKSPACE
    bad = list(sides)
    bad[2] = B.GradSide(FAKE, 4095, FAKE, 4096, 4096)  # lda < d
    assert call(sides=bad) == B.POETX_E_SHAPE
    bad[2] = B.GradSide(None, 4096, FAKE, 4096, 4096)
    assert call(sides=bad) == B.POETX_E_NULL
    bad[2] = B.GradSide(FAKE, 4096, FAKE, 4096, 0)  # d < 1
    assert call(sides=bad) == B.POETX_E_SHAPE


def test_bwd_dx_sides_statuses(L):
    d = B.desc(320, 200, 64, "bf16", "bf16")
    T = 64
    ws = B.poetx_workspace_size(d, T, B.POETX_OP_BWD)
    sides = (B.GradSide * 2)()

    def call(sides=sides, ws_bytes=ws, H=FAKE, perm=FAKE):
        return L.poetx_linear_bwd_dx_sides(ctypes.byref(d), T, None, FAKE, perm, FAKE, FAKE, FAKE, FAKE, H, FAKE,
                                           sides, FAKE, ws_bytes, None)

    assert call(sides=None) == B.POETX_E_NULL
    assert call(ws_bytes=ws - 1) == B.POETX_E_WORKSPACE
    assert call(H=None) == B.POETX_E_NULL
    assert call(perm=None) == B.POETX_E_NULL


def test_group_call_statuses(L):
    d = B.desc(320, 200, 64, "bf16", "bf16")
    d32 = B.desc(320, 200, 32, "bf16", "bf16")
    T = 64
    wf = B.poetx_workspace_size(d, T, B.POETX_OP_FWD)
    wb = B.poetx_workspace_size(d, T, B.POETX_OP_BWD)

    def fwd(desc=d, X=FAKE, ws_bytes=wf):
        return B.FwdCall(ctypes.pointer(desc), X, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes)

    def bwd(desc=d, dZ=FAKE, ws_bytes=wb):
        return B.BwdCall(ctypes.pointer(desc), None, dZ, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes)

    def run_f(*calls, count=None):
        arr = (B.FwdCall * max(len(calls), 1))(*calls)
        return L.poetx_linear_fwd_group(len(calls) if count is None else count, arr, T, None)

    def run_b(*calls, sides=True):
        arr = (B.BwdCall * len(calls))(*calls)
        sd = (B.GradSide * (2 * len(calls)))() if sides else None
        return L.poetx_linear_bwd_dx_group(len(calls), arr, T, sd, None)

    assert L.poetx_linear_fwd_group(1, None, T, None) == B.POETX_E_NULL
    assert run_f(fwd(), count=0) == B.POETX_E_SHAPE
    assert run_f(*[fwd()] * (B.POETX_MAX_GROUP + 1)) == B.POETX_E_SHAPE
    assert run_f(fwd(), fwd(ws_bytes=wf - 1)) == B.POETX_E_WORKSPACE
    assert run_f(fwd(), fwd(X=None)) == B.POETX_E_NULL
    assert run_f(fwd(), fwd(desc=d32, ws_bytes=B.poetx_workspace_size(d32, T, B.POETX_OP_FWD))) == B.POETX_E_SHAPE
    assert run_b(bwd(), sides=False) == B.POETX_E_NULL
    assert run_b(bwd(), bwd(ws_bytes=wb - 1)) == B.POETX_E_WORKSPACE
    assert run_b(bwd(), bwd(dZ=None)) == B.POETX_E_NULL
    assert run_b(bwd(), bwd(desc=d32, ws_bytes=B.poetx_workspace_size(d32, T, B.POETX_OP_BWD))) == B.POETX_E_SHAPE


def test_cnp_backward_reuse_statuses(L):
    d, b, bf = [320, 200], 64, B.DTYPES["bf16"]
    blocks = sum((x + b - 1) // b for x in d)
    dg_bytes = B.poetx_cnp_grad_bytes(blocks, b, bf)
    ws_bytes = B.poetx_cnp_batch_workspace_size(d, b, bf)
    q = (ctypes.c_void_p * 2)(FAKE, FAKE)
    dq = (ctypes.c_void_p * 2)(FAKE, FAKE)
    dd = (ctypes.c_int32 * 2)(*d)

    def call(build=FAKE, build_bytes=ws_bytes, dg=FAKE, dgb=dg_bytes):
        return L.poetx_cnp_backward_batch_reuse(2, q, dd, b, bf, build, build_bytes, dg, dgb, dq, None)

    assert call(build=None) == B.POETX_E_NULL
    assert call(build_bytes=ws_bytes - 1) == B.POETX_E_WORKSPACE
    assert call(build=FAKE + 16) == B.POETX_E_WORKSPACE
    assert call(dgb=dg_bytes - 1) == B.POETX_E_WORKSPACE
    assert L.poetx_cnp_backward_batch_reuse(0, q, dd, b, bf, FAKE, ws_bytes, FAKE, dg_bytes, dq, None) == \
        B.POETX_E_SHAPE
