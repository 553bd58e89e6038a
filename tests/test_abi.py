"""C ABI checks that need no GPU: the library loads, exports every entry
point include/whtq.h declares, and rejects bad arguments with the documented
status before touching the device."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "whtq.h")

OK, EINVAL, EUNSUP, EALIGN, EHIP = 0, 1, 2, 3, 4
P = ctypes.c_void_p(0x10000)       # 16-byte aligned stand-in, never dereferenced
P_MIS = ctypes.c_void_p(0x10004)   # misaligned stand-in
NULL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    from wht_adapters_amd import whtq
    return whtq.raw()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:whtq_status|const char\*|int|int64_t)\s+(\w+)\s*\(", text, flags=re.M)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"wht_batched", "rht_quantize_rtn", "rht_dequantize_inverse",
                          "qwha_adapter_forward", "harp_rotate", "whtq_status_string",
                          "whtq_last_hip_error", "whtq_abi_version", "qwha_csr_transpose",
                          "qwha_permute_values", "qwha_adapter_backward_input",
                          "qwha_grad_values_workspace_bytes", "qwha_adapter_grad_values",
                          "harp_build_blocks", "rht_lowbit_gemv", "qwha_init_error_coeffs",
                          "qwha_init_gram", "qwha_init_channel_errors", "qwha_init_allocate",
                          "qwha_init_select", "qwha_init_refine", "qwha_adapter_grad_values_noalloc",
                          "whtq_stream_probe", "qwha_forward_plan_bytes", "qwha_forward_plan",
                          "qwha_adapter_forward_planned"}
    for nm in names:
        assert hasattr(lib, nm), nm


def test_version_and_strings(lib):
    assert lib.whtq_abi_version() == 4
    for s in range(6):
        assert lib.whtq_status_string(s)
    assert b"unknown" in lib.whtq_status_string(99)


def wht(lib, x=P, xd=0, y=P, yd=0, rows=4, n=64, ldx=64, ldy=64, sb=NULL, mode=0, norm=1):
    return lib.wht_batched(x, xd, y, yd, rows, n, ldx, ldy, sb, mode, norm, NULL)


def test_wht_validation(lib):
    assert wht(lib, n=12, ldx=12, ldy=12) == EUNSUP           # not a power of two
    assert wht(lib, n=16384, ldx=16384, ldy=16384) == EUNSUP   # beyond 8192
    assert wht(lib, ldx=32) == EINVAL                          # ld < n
    assert wht(lib, rows=-1) == EINVAL
    assert wht(lib, xd=7) == EINVAL                            # bad dtype
    assert wht(lib, xd=0, yd=1) == EUNSUP                      # f32 -> bf16 not offered
    assert wht(lib, mode=1) == EINVAL                          # signs required
    assert wht(lib, mode=3, sb=P) == EINVAL
    assert wht(lib, norm=2) == EINVAL
    assert wht(lib, x=NULL) == EINVAL
    assert wht(lib, x=P_MIS) == EALIGN
    assert wht(lib, ldx=65, ldy=64, y=ctypes.c_void_p(0x20000)) == EALIGN  # 65*4 B rows
    assert wht(lib, ldx=64, ldy=72) == EINVAL                  # exact alias needs equal ld
    assert wht(lib, xd=1, yd=0, x=P, y=P) == EINVAL            # alias with different dtypes
    assert wht(lib, rows=0) == OK                              # empty batch: nothing to do


def q(lib, w=P, wd=1, rows=4, n=256, ldw=256, sb=NULL, bits=4, g=64, c=P, s=P):
    return lib.rht_quantize_rtn(w, wd, rows, n, ldw, sb, bits, g, c, s, NULL)


def dq(lib, c=P, s=P, rows=4, n=256, sb=NULL, bits=4, g=64, o=P, od=1, ldo=256):
    return lib.rht_dequantize_inverse(c, s, rows, n, sb, bits, g, o, od, ldo, NULL)


def test_quant_validation(lib):
    for f in (q, dq):
        assert f(lib, bits=5) == EINVAL
        assert f(lib, bits=1) == EINVAL
        assert f(lib, g=48) == EINVAL          # does not divide 256
        assert f(lib, g=4) == EINVAL           # below 8
        assert f(lib, g=512, n=1024) == EUNSUP if f is q else True
        assert f(lib, n=32, g=8) == EUNSUP     # n < 64
        assert f(lib, n=384, g=128) == EUNSUP  # not a power of two
        assert f(lib, rows=-2) == EINVAL
        assert f(lib, rows=0) == OK
    assert q(lib, ldw=128) == EINVAL
    assert q(lib, w=P_MIS) == EALIGN
    assert q(lib, c=P_MIS) == EALIGN
    assert q(lib, sb=ctypes.c_void_p(0x10002)) == EALIGN
    assert q(lib, c=NULL) == EINVAL
    assert dq(lib, o=NULL) == EINVAL
    assert dq(lib, ldo=100) == EINVAL


def lbg(lib, x=P, tokens=1, ldx=8192, c=P, s=P, rows=64, n=8192, sb=NULL, bits=2, g=64, y=P, ldy=64):
    return lib.rht_lowbit_gemv(x, tokens, ldx, c, s, rows, n, sb, bits, g, y, ldy, NULL)


def test_lowbit_gemv_validation(lib):
    assert lbg(lib, bits=3) == EUNSUP                 # 3-bit codes are not offered
    assert lbg(lib, bits=5) == EINVAL
    assert lbg(lib, n=2048, ldx=2048) == EUNSUP       # n is 4096 or 8192
    assert lbg(lib, n=6144, ldx=6144) == EUNSUP
    assert lbg(lib, g=8) == EUNSUP                    # 2-bit codes need g >= 16
    assert lbg(lib, g=48) == EINVAL
    assert lbg(lib, g=512) == EUNSUP
    assert lbg(lib, ldx=4096) == EINVAL               # ldx < n
    assert lbg(lib, ldy=63) == EINVAL                 # ldy < rows
    assert lbg(lib, tokens=-1) == EINVAL
    assert lbg(lib, rows=-1) == EINVAL
    for kw in ("x", "c", "s", "y"):
        assert lbg(lib, **{kw: NULL}) == EINVAL
    assert lbg(lib, x=P_MIS) == EALIGN
    assert lbg(lib, ldx=8196) == EALIGN               # 8196 * 2 B rows are not 16-byte multiples
    assert lbg(lib, c=P_MIS) == EALIGN
    assert lbg(lib, s=P_MIS) == EALIGN
    assert lbg(lib, y=ctypes.c_void_p(0x10001)) == EALIGN
    assert lbg(lib, sb=ctypes.c_void_p(0x10002)) == EALIGN
    assert lbg(lib, tokens=0) == OK                   # nothing to do
    assert lbg(lib, rows=0, ldy=0) == OK


def qw(lib, x=P, xd=1, tokens=8, d_in=4096, ldx=4096, rp=P, ci=P, v=P, vd=1, d_out=4096, nnz=100,
       y=P, yd=1, ldy=4096):
    return lib.qwha_adapter_forward(x, xd, tokens, d_in, ldx, rp, ci, v, vd, d_out, nnz, y, yd, ldy, NULL)


def test_qwha_validation(lib):
    assert qw(lib, ldx=100) == EINVAL
    assert qw(lib, rp=NULL) == EINVAL
    assert qw(lib, nnz=4096 * 4096 + 1) == EINVAL
    assert qw(lib, d_in=3000, ldx=3000) == EUNSUP
    assert qw(lib, d_in=32, ldx=32) == EUNSUP          # d_in a power of two in [64, 8192]
    assert qw(lib, d_in=16384, ldx=16384) == EUNSUP
    assert qw(lib, d_in=8192, ldx=4096) == EINVAL       # ldx < d_in
    assert qw(lib, d_in=2048, ldx=2048, tokens=0) == OK
    assert qw(lib, d_in=8192, ldx=8192, tokens=0) == OK
    assert qw(lib, xd=0) == EUNSUP
    assert qw(lib, vd=2) == EUNSUP
    assert qw(lib, x=P_MIS) == EALIGN
    assert qw(lib, tokens=0) == OK


def hp(lib, x=P, y=ctypes.c_void_p(0x20000), dt=1, tokens=8, d=4096, ldx=4096, ldy=4096, sb=NULL,
       pre=1, rad=(16, 16, 16), blocks=P, bd=0):
    arr = (ctypes.c_int32 * len(rad))(*rad)
    return lib.harp_rotate(x, y, dt, tokens, d, ldx, ldy, sb, pre, arr, len(rad), blocks, bd, NULL)


def test_harp_validation(lib):
    assert hp(lib, rad=(16, 16, 8)) == EINVAL              # product != d
    assert hp(lib, rad=(16, 16, 16, 1)) == EINVAL          # radix < 2
    # the Sylvester preconditioning needs a power-of-two d
    assert hp(lib, d=5120, ldx=5120, ldy=5120, rad=(8, 8, 8, 5, 2)) == EINVAL
    assert hp(lib, rad=(64, 64)) == EUNSUP                 # radix above 16
    assert hp(lib, d=17 * 4, ldx=72, ldy=72, rad=(17, 4), pre=0) == EUNSUP
    assert hp(lib, d=16384, ldx=16384, ldy=16384, rad=(16, 16, 64)) == EUNSUP  # d above 8192
    assert hp(lib, d=5120, ldx=5120, ldy=5120, rad=(8, 8, 8, 5, 2), pre=0, tokens=0) == OK
    assert hp(lib, y=P) == EINVAL                          # in place not allowed
    assert hp(lib, pre=3) == EINVAL
    assert hp(lib, blocks=NULL) == EINVAL
    assert hp(lib, dt=2) == EUNSUP                         # fp16 rows
    assert hp(lib, dt=0, tokens=0) == OK                   # fp32 rows accepted (any schedule)
    assert hp(lib, dt=0, x=ctypes.c_void_p(0x10008)) == EALIGN
    assert hp(lib, bd=7) == EINVAL                         # not a dtype
    assert hp(lib, bd=1) == EUNSUP                         # bf16 blocks: no kernel
    assert hp(lib, bd=2, tokens=0) == OK                   # fp16 blocks accepted
    assert hp(lib, x=P_MIS) == EALIGN
    assert hp(lib, tokens=0) == OK


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="needs a host without a GPU")
def qwp(lib, x=P, tokens=8, d_in=4096, ldx=4096, rp=P, d_out=4096, nnz=100, plan=P, plan_bytes=1 << 20):
    return lib.qwha_adapter_forward_planned(x, 1, tokens, d_in, ldx, rp, P, P, 1, d_out, nnz, plan, plan_bytes,
                                            P, 1, 4096, NULL)


def plan(lib, tokens=8, d_in=4096, rp=P, d_out=4096, nnz=100, out=P, nbytes=1 << 20):
    return lib.qwha_forward_plan(tokens, d_in, rp, d_out, nnz, out, nbytes, NULL)


def test_qwha_forward_plan_validation(lib):
    """Forward plans: sizes, pointers and alignment are checked before the
    device; d_in = 8192 needs no plan (size 0, building is a no-op)."""
    nb = lib.qwha_forward_plan_bytes
    assert nb(0, 4096, 4096, 100) == -1           # tokens >= 1
    assert nb(8, 3000, 4096, 100) == -1           # d_in a power of two
    assert nb(8, 4096, 5000, 100) == -1           # d_out <= 4096
    assert nb(8, 64, 4, 257) == -1                # nnz > d_in d_out
    assert nb(8, 8192, 4096, 100) == 0
    assert plan(lib, tokens=0) == EINVAL
    assert plan(lib, rp=NULL) == EINVAL
    assert plan(lib, rp=ctypes.c_void_p(0x10002)) == EALIGN
    assert plan(lib, d_in=3000) == EUNSUP
    assert plan(lib, d_out=5000) == EUNSUP
    assert plan(lib, nbytes=-1) == EINVAL
    assert plan(lib, d_in=8192) == OK             # nothing to plan
    assert plan(lib, out=NULL) == EINVAL
    assert plan(lib, out=P_MIS) == EALIGN
    # the planned forward: the forward's rules, then the plan's
    assert qwp(lib, ldx=100) == EINVAL
    assert qwp(lib, d_in=3000, ldx=3000) == EUNSUP
    assert qwp(lib, x=P_MIS) == EALIGN
    assert qwp(lib, plan_bytes=100) == EINVAL     # a plan holds at least its 256-byte header
    assert qwp(lib, plan_bytes=-1) == EINVAL
    assert qwp(lib, plan=P_MIS) == EALIGN
    assert qwp(lib, tokens=0) == OK
    assert qwp(lib, tokens=0, plan=NULL, plan_bytes=0) == OK


def test_valid_call_without_device_is_ehip(lib):
    assert wht(lib) == EHIP
    assert lib.whtq_last_hip_error() != 0
    assert q(lib) == EHIP and dq(lib) == EHIP
    assert qw(lib) == EHIP and hp(lib) == EHIP
    assert qwp(lib) == EHIP and plan(lib) == EHIP
    assert lib.qwha_forward_plan_bytes(8, 4096, 4096, 100) == -1  # the split follows the device's CUs


# ---- QWHA backward entry points

def test_csr_transpose_matches_oracle():
    """The host helper is integer work: bit-exact against the oracle's transpose
    (empty rows and columns, a dense row, repeated columns across rows)."""
    import numpy as np
    from oracle import qwha
    from wht_adapters_amd import whtq
    rng = np.random.default_rng(5)
    for d_out, d_in, per_row in ((7, 16, (0, 5)), (300, 4096, (0, 40)), (64, 64, (64, 65))):
        lens = rng.integers(per_row[0], per_row[1], d_out)
        lens[0] = 0
        cols = np.concatenate([np.sort(rng.choice(d_in, int(l), replace=False)) for l in lens]).astype(np.int32)
        rp = np.r_[0, np.cumsum(lens)].astype(np.int32)
        t_rp, t_ci, t_pm = whtq.qwha_csr_transpose(rp, cols, d_in)
        w_rp, w_ci, _, w_pm = qwha.csr_transpose(rp, cols, np.zeros(cols.size), d_in)
        assert np.array_equal(t_rp, w_rp) and np.array_equal(t_ci, w_ci) and np.array_equal(t_pm, w_pm)


def test_csr_transpose_rejects_malformed(lib):
    import numpy as np
    def run(rp, ci, d_out, d_in, nnz):
        rp = np.asarray(rp, np.int32)
        ci = np.asarray(ci, np.int32)
        t_rp = np.empty(d_in + 1, np.int32)
        t_ci = np.empty(max(nnz, 1), np.int32)
        t_pm = np.empty(max(nnz, 1), np.int32)
        vp = ctypes.c_void_p
        return lib.qwha_csr_transpose(rp.ctypes.data_as(vp), ci.ctypes.data_as(vp), d_out, d_in, nnz,
                                      t_rp.ctypes.data_as(vp), t_ci.ctypes.data_as(vp), t_pm.ctypes.data_as(vp))
    assert run([0, 1, 2], [0, 3], 2, 4, 2) == OK
    assert run([0, 1, 2], [0, 4], 2, 4, 2) == EINVAL     # column out of range
    assert run([0, 2, 1], [0, 1], 2, 4, 2) == EINVAL     # decreasing row_ptr
    assert run([1, 1, 2], [0, 1], 2, 4, 2) == EINVAL     # row_ptr[0] != 0
    assert run([0, 1, 1], [0, 1], 2, 4, 2) == EINVAL     # row_ptr[d_out] != nnz
    assert run([0, 0, 0], [0], 2, 4, 0) == OK            # empty F


def bw(lib, dy=P, dyd=1, tokens=8, d_out=4096, lddy=4096, rp=P, ci=P, v=P, vd=1, d_in=4096, nnz=100,
       dx=P, dxd=1, lddx=4096):
    return lib.qwha_adapter_backward_input(dy, dyd, tokens, d_out, lddy, rp, ci, v, vd, d_in, nnz, dx, dxd,
                                           lddx, NULL)


def gv(lib, x=P, dy=P, dt=1, tokens=8, d_in=4096, d_out=4096, ldx=4096, lddy=4096, rp=P, ci=P, nnz=100,
       dc=P, ws=P, wsb=1 << 40):
    return lib.qwha_adapter_grad_values(x, dy, dt, tokens, d_in, d_out, ldx, lddy, rp, ci, nnz, dc, ws, wsb, NULL)


def _gv_args(x=P, dy=P, dt=1, tokens=8, d_in=4096, d_out=4096, ldx=4096, lddy=4096, rp=P, ci=P, nnz=100,
             dc=P):
    return (x, dy, dt, tokens, d_in, d_out, ldx, lddy, rp, ci, nnz, dc, NULL)


def test_qwha_backward_validation(lib):
    assert bw(lib, lddy=100) == EINVAL
    assert bw(lib, lddx=100) == EINVAL
    assert bw(lib, rp=NULL) == EINVAL
    assert bw(lib, v=NULL) == EINVAL
    assert bw(lib, d_in=32, lddx=32) == EUNSUP
    assert bw(lib, d_in=16384, lddx=16384) == EUNSUP
    assert bw(lib, d_in=8192, lddx=4096) == EINVAL
    assert bw(lib, d_in=64, lddx=64, tokens=0) == OK
    assert bw(lib, d_out=5000, lddy=5000) == EUNSUP
    assert bw(lib, dyd=0) == EUNSUP
    assert bw(lib, vd=2) == EUNSUP
    assert bw(lib, dx=P_MIS) == EALIGN
    assert bw(lib, dy=ctypes.c_void_p(0x10001)) == EALIGN
    assert bw(lib, ci=P_MIS) == EALIGN
    assert bw(lib, tokens=0) == OK
    assert gv(lib, ldx=100) == EINVAL
    assert gv(lib, dc=NULL) == EINVAL
    assert gv(lib, ws=NULL) == EINVAL
    assert gv(lib, wsb=16) == EINVAL                        # workspace too small
    assert gv(lib, d_in=32, ldx=32) == EUNSUP
    assert gv(lib, d_in=3000, ldx=3000) == EUNSUP
    assert gv(lib, d_in=8192, ldx=4096) == EINVAL
    assert gv(lib, dt=0) == EUNSUP
    assert gv(lib, x=P_MIS) == EALIGN
    assert gv(lib, ws=ctypes.c_void_p(0x10008)) == EALIGN
    assert gv(lib, nnz=0, dc=NULL, ws=NULL, wsb=0) == OK     # empty support: nothing to do
    # the allocation-free variant: the same checks, then its fixed capacity
    na = lambda **kw: lib.qwha_adapter_grad_values_noalloc(*_gv_args(**kw))
    assert na(ldx=100) == EINVAL
    assert na(dc=NULL) == EINVAL
    assert na(d_in=16384, ldx=16384) == EUNSUP
    assert na(x=P_MIS) == EALIGN
    assert na(nnz=0, dc=NULL) == OK
    assert na(tokens=5000) == 5                              # 5000 x 16 KiB of Hn x > 64 MiB
    assert lib.qwha_grad_values_workspace_bytes(2048, 4096, 262144) <= 64 << 20
    assert lib.qwha_grad_values_workspace_bytes(8, 32, 100) == -1
    assert lib.qwha_grad_values_workspace_bytes(8, 3000, 100) == -1
    assert lib.qwha_grad_values_workspace_bytes(8, 16384, 100) == -1
    # d_in below 4096 keeps the 4096-column Z layout; 8192 doubles it
    assert lib.qwha_grad_values_workspace_bytes(64, 2048, 1000) == lib.qwha_grad_values_workspace_bytes(64, 4096, 1000)
    assert lib.qwha_grad_values_workspace_bytes(64, 8192, 1000) >= 64 * 8192 * 4
    assert na(d_in=8192, ldx=8192, tokens=2500) == 5          # 2500 x 32 KiB of Hn x > 64 MiB
    assert lib.qwha_grad_values_workspace_bytes(0, 4096, 100) == 0
    # Hn x in fp32 (rounded up to 256 B) plus per-token-slab partial sums
    need = lib.qwha_grad_values_workspace_bytes(2048, 4096, 262144)
    assert need >= 2048 * 4096 * 4 and need % 4 == 0
    vp = ctypes.c_void_p
    assert lib.qwha_permute_values(P, 1, NULL, 10, P, NULL) == EINVAL
    assert lib.qwha_permute_values(P, 1, P, 10, P, NULL) == EINVAL    # out aliases vals
    assert lib.qwha_permute_values(P, 2, P, 10, vp(0x20000), NULL) == EUNSUP
    assert lib.qwha_permute_values(P, 1, P, 0, vp(0x20000), NULL) == OK


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="needs a host without a GPU")
def test_backward_valid_call_without_device_is_ehip(lib):
    assert bw(lib) == EHIP and gv(lib) == EHIP


def hb(lib, p=P, pdt=0, sc=NULL, d=64, rad=(4, 16), mix=NULL, out=P, bdt=0):
    arr = (ctypes.c_int32 * len(rad))(*rad)
    return lib.harp_build_blocks(p, pdt, sc, d, arr, len(rad), mix, out, bdt, NULL)


def test_harp_build_validation(lib):
    assert hb(lib, rad=(4, 8)) == EINVAL                   # product != d
    assert hb(lib, pdt=1) == EINVAL                        # bf16 parameters: not offered
    assert hb(lib, pdt=3) == EINVAL                        # int8 needs scales
    assert hb(lib, bdt=1) == EINVAL                        # bf16 blocks: not offered
    assert hb(lib, d=60, rad=(4, 15)) == EINVAL            # no Sylvester mixer for 15
    assert hb(lib, d=68, rad=(4, 17), mix=P) == EUNSUP     # radix above 16
    assert hb(lib, p=NULL) == EINVAL
    assert hb(lib, p=ctypes.c_void_p(0x10002)) == EALIGN   # fp32 parameters, 2-byte aligned
    assert hb(lib, out=ctypes.c_void_p(0x10001), bdt=2) == EALIGN


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="needs a host without a GPU")
def test_harp_build_valid_call_without_device_is_ehip(lib):
    assert hb(lib) == EHIP


def qie(lib, w=P, wd=1, rows=8, n=4096, ldw=4096, c=P, s=P, sb=NULL, bits=4, g=128, f=P, ldf=4096):
    return lib.qwha_init_error_coeffs(w, wd, rows, n, ldw, c, s, sb, bits, g, f, ldf, NULL)


def test_qwha_init_error_coeffs_validation(lib):
    assert qie(lib, bits=5) == EINVAL
    assert qie(lib, g=96) == EINVAL
    assert qie(lib, n=16384, ldw=16384, ldf=16384) == EUNSUP
    assert qie(lib, wd=7) == EINVAL
    assert qie(lib, ldw=4095) == EINVAL
    assert qie(lib, ldf=100) == EINVAL
    for kw in ("w", "c", "s", "f"):
        assert qie(lib, **{kw: NULL}) == EINVAL
    assert qie(lib, f=P, w=P) == EINVAL                  # w aliases f
    assert qie(lib, w=ctypes.c_void_p(0x20001)) == EALIGN
    assert qie(lib, w=ctypes.c_void_p(0x20000), f=P_MIS) == EALIGN
    assert qie(lib, w=ctypes.c_void_p(0x20000), ldf=4097) == EALIGN
    assert qie(lib, w=ctypes.c_void_p(0x20000), c=P_MIS) == EALIGN
    assert qie(lib, w=ctypes.c_void_p(0x20000), sb=ctypes.c_void_p(0x10002)) == EALIGN
    assert qie(lib, rows=0) == OK


def qig(lib, x=P, xd=1, tokens=16, n=4096, ldx=4096, z=ctypes.c_void_p(0x20000), g=ctypes.c_void_p(0x30000),
        acc=0):
    return lib.qwha_init_gram(x, xd, tokens, n, ldx, z, g, acc, NULL)


def test_qwha_init_gram_validation(lib):
    assert qig(lib, n=128, ldx=128) == EUNSUP            # n in [256, 8192]
    assert qig(lib, n=16384, ldx=16384) == EUNSUP
    assert qig(lib, n=3000, ldx=3000) == EINVAL
    assert qig(lib, xd=9) == EINVAL
    assert qig(lib, tokens=-1) == EINVAL
    assert qig(lib, ldx=100) == EINVAL
    assert qig(lib, acc=2) == EINVAL
    for kw in ("x", "z", "g"):
        assert qig(lib, **{kw: NULL}) == EINVAL
    assert qig(lib, g=NULL, tokens=0) == EINVAL          # g is always written or read
    assert qig(lib, x=P_MIS) == EALIGN
    assert qig(lib, z=P_MIS) == EALIGN
    assert qig(lib, g=P_MIS) == EALIGN
    assert qig(lib, tokens=0, acc=1, x=NULL, z=NULL) == OK
    assert qig(lib, z=P, g=P) == EINVAL                  # z overlays g


def qic(lib, f=P, rows=8, n=4096, ldf=4096, g=ctypes.c_void_p(0x20000), p=ctypes.c_void_p(0x30000),
        e=ctypes.c_void_p(0x40000)):
    return lib.qwha_init_channel_errors(f, rows, n, ldf, g, p, e, NULL)


def qis(lib, f=P, rows=8, n=4096, ldf=4096, rp=P, ci=P):
    return lib.qwha_init_select(f, rows, n, ldf, rp, ci, NULL)


def qir(lib, g=P, n=4096, p=P, rows=8, rp=P, ci=P, v=P):
    return lib.qwha_init_refine(g, n, p, rows, rp, ci, v, NULL)


def test_qwha_init_device_calls_validation(lib):
    assert qic(lib, n=64, ldf=64) == EUNSUP
    assert qic(lib, ldf=100) == EINVAL
    assert qic(lib, rows=-1) == EINVAL
    for kw in ("f", "g", "p", "e"):
        assert qic(lib, **{kw: NULL}) == EINVAL
    assert qic(lib, f=P_MIS) == EALIGN
    assert qic(lib, ldf=4098) == EALIGN
    assert qic(lib, p=P_MIS) == EALIGN
    assert qic(lib, e=ctypes.c_void_p(0x10002)) == EALIGN
    assert qic(lib, rows=0) == OK
    Q = ctypes.c_void_p(0x30000)
    assert qic(lib, f=P, g=Q, p=P) == EINVAL             # p overlays f
    assert qic(lib, f=Q, g=P, p=P) == EINVAL             # p overlays g
    assert qic(lib, f=Q, g=ctypes.c_void_p(0x40000), p=P, e=P) == EINVAL   # err overlays p
    assert qis(lib, n=8192 * 2, ldf=8192 * 2) == EUNSUP
    assert qis(lib, ldf=10) == EINVAL
    for kw in ("f", "rp", "ci"):
        assert qis(lib, **{kw: NULL}) == EINVAL
    assert qis(lib, f=P_MIS) == EALIGN
    assert qis(lib, ci=ctypes.c_void_p(0x10002)) == EALIGN
    assert qis(lib, rows=0) == OK
    assert qir(lib, n=100) == EINVAL
    assert qir(lib, rows=-2) == EINVAL
    for kw in ("g", "p", "rp", "ci", "v"):
        assert qir(lib, **{kw: NULL}) == EINVAL
    assert qir(lib, v=ctypes.c_void_p(0x10001)) == EALIGN
    assert qir(lib, rows=0) == OK

