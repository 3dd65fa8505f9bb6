"""The C ABI library on the CPU: it loads, exports every symbol include/rettn.h
declares, builds masks bit-identical to the oracle's independent generators,
and rejects bad arguments before launching anything (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import sparse_attention_diffusion_block_amd as rt
from sparse_attention_diffusion_block_amd import rettn as b
from oracle import masks as om
from workloads import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EINVAL = 1


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "rettn.h")).read()
    return sorted(set(re.findall(r"\b(rettn_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_symbols()
    assert set(names) == set(rt.EXPORTED)
    lib = rt.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = rt.lib()
    for s in range(5):
        assert lib.rettn_status_str(s).decode().startswith("RETTN_")


@pytest.mark.parametrize("n", sorted(CONFIGS))
def test_mask_build_matches_oracle_for_workloads(n):
    for spec in CONFIGS[n].masks:
        got = rt.mask_build(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift)
        ref = om.build_mask(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift)
        assert np.array_equal(got, ref)


def test_mask_build_random_params():
    rng = np.random.Generator(np.random.PCG64(5))
    for _ in range(200):
        kind = int(rng.integers(0, 4))
        nb = int(rng.integers(1, 60))
        w = int(rng.integers(1, nb + 1))
        text = int(rng.integers(0, nb + 1))
        tshift = int(rng.integers(1, nb + 2))
        got = rt.mask_build(kind, nb, w, text, tshift)
        ref = om.build_mask(kind, nb, w, text, tshift)
        assert np.array_equal(got, ref), (kind, nb, w, text, tshift)


@pytest.mark.parametrize("spec", [(7, 4, 1, 0, 0), (b.MASK_BAND, 4, 0, 0, 0), (b.MASK_BAND, 4, 5, 0, 0),
                                  (b.MASK_COGVIDEO3D, 4, 0, 5, 1), (b.MASK_COGVIDEO3D, 4, 0, 1, 0),
                                  (b.MASK_DIAG, 0, 0, 0, 0)])
def test_mask_build_rejects_bad_specs(spec):
    kind, nb, w, text, tshift = spec
    out = np.zeros((max(nb, 1), max(nb, 1)), dtype=np.uint8)
    s = b.MaskSpec(kind, nb, w, text, tshift)
    assert rt.lib().rettn_mask_build(ctypes.byref(s), out.ctypes.data_as(ctypes.c_void_p)) == EINVAL


# ------------------------------------------------------------------ validation (no launch)
FAKE = 1 << 20   # a 16-byte aligned non-null address; never dereferenced because validation fails first


def _good_desc():
    return b.Desc(2, 3, 200, 64, 64, b.RETTN_BF16, 3 * 200 * 64, 200 * 64, 64)


def _idx(nb=4):
    return b.Index(nb, nb, nb, FAKE, FAKE, FAKE)


BAD_DESCS = {
    "B0": dict(B=0), "L0": dict(L=0), "d0": dict(d=0), "d_big": dict(d=136), "d_not_mult8": dict(d=60),
    "block48": dict(block=48), "dtype": dict(dtype=7), "stride_l_small": dict(stride_l=32),
    "stride_misaligned": dict(stride_l=68), "stride_h0": dict(stride_h=0),
}


@pytest.mark.parametrize("name", sorted(BAD_DESCS))
def test_calibrate_and_sparse_reject_bad_descriptors(name):
    d = _good_desc()
    for k, v in BAD_DESCS[name].items():
        setattr(d, k, v)
    lib = rt.lib()
    idx = _idx()
    assert lib.rettn_calibrate(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(idx), FAKE, FAKE, FAKE, None) == EINVAL
    assert lib.rettn_sparse(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(idx), FAKE, FAKE, 0.04, 1, FAKE,
                            None) == EINVAL


def test_reject_index_of_wrong_size_and_bad_pointers():
    lib = rt.lib()
    d = _good_desc()
    bad = _idx(3)   # ceil(200 / 64) = 4 blocks
    assert lib.rettn_calibrate(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(bad), FAKE, FAKE, FAKE, None) == EINVAL
    idx = _idx()
    assert lib.rettn_calibrate(ctypes.byref(d), None, FAKE, FAKE, ctypes.byref(idx), FAKE, FAKE, FAKE, None) == EINVAL
    assert lib.rettn_calibrate(ctypes.byref(d), FAKE + 8, FAKE, FAKE, ctypes.byref(idx), FAKE, FAKE, FAKE,
                               None) == EINVAL
    nomask = b.Index(4, 4, 4, FAKE, FAKE, None)
    assert lib.rettn_calibrate(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(nomask), FAKE, FAKE, FAKE,
                               None) == EINVAL
    assert lib.rettn_calibrate(None, FAKE, FAKE, FAKE, ctypes.byref(idx), FAKE, FAKE, FAKE, None) == EINVAL


@pytest.mark.parametrize("lam,step", [(-0.1, 1), (float("nan"), 1), (float("inf"), 1), (0.04, -1)])
def test_sparse_rejects_bad_ramp(lam, step):
    lib = rt.lib()
    d = _good_desc()
    idx = _idx()
    assert lib.rettn_sparse(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(idx), FAKE, FAKE, lam, step, FAKE,
                            None) == EINVAL


def test_index_build_rejects_bad_arguments():
    lib = rt.lib()
    nnz = ctypes.c_int32(-1)
    assert lib.rettn_index_build(None, 4, 4, FAKE, FAKE, ctypes.byref(nnz), None) == EINVAL
    assert lib.rettn_index_build(FAKE, 0, 4, FAKE, FAKE, ctypes.byref(nnz), None) == EINVAL
    assert lib.rettn_index_build(FAKE, 4, 4, FAKE, FAKE, None, None) == EINVAL
    assert nnz.value == -1


@pytest.mark.parametrize("kind", [-1, 2, 99])
def test_calibrate_residual_rejects_unknown_kind(kind):
    lib = rt.lib()
    d = _good_desc()
    idx = _idx()
    assert lib.rettn_calibrate_residual(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(idx), FAKE, FAKE, FAKE,
                                        kind, None) == EINVAL
    # a bad descriptor is rejected for either valid kind too
    d.d = 0
    for good in (b.RESIDUAL_MASKED, b.RESIDUAL_DIFFERENCE):
        assert lib.rettn_calibrate_residual(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(idx), FAKE, FAKE, FAKE,
                                            good, None) == EINVAL


@pytest.mark.parametrize("slices,col_stride,nnz", [(5, 16, 4), (-1, 16, 4), (6, 3, 4), (3, -1, 0)])
def test_reject_bad_slice_layouts(slices, col_stride, nnz):
    """An index whose slice count is neither 1, H nor B*H, or whose column stride cannot hold nnz."""
    lib = rt.lib()
    d = _good_desc()                     # B = 2, H = 3
    idx = b.Index(4, 4, nnz, FAKE, FAKE, FAKE, slices, col_stride)
    assert lib.rettn_calibrate(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(idx), FAKE, FAKE, FAKE, None) == EINVAL
    assert lib.rettn_sparse(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(idx), FAKE, FAKE, 0.04, 1, FAKE,
                            None) == EINVAL


def test_index_build_sliced_rejects_bad_arguments():
    lib = rt.lib()
    nnz = ctypes.c_int32(-1)
    assert lib.rettn_index_build_sliced(None, 2, 4, 4, FAKE, FAKE, ctypes.byref(nnz), None) == EINVAL
    assert lib.rettn_index_build_sliced(FAKE, 0, 4, 4, FAKE, FAKE, ctypes.byref(nnz), None) == EINVAL
    assert lib.rettn_index_build_sliced(FAKE, 70000, 4, 4, FAKE, FAKE, ctypes.byref(nnz), None) == EINVAL
    assert lib.rettn_index_build_sliced(FAKE, 2, 4, 0, FAKE, FAKE, ctypes.byref(nnz), None) == EINVAL
    assert nnz.value == -1


def test_dynamic_workspace_size():
    lib = rt.lib()
    d = _good_desc()                     # B 2, H 3, L 200, d 64, block 64: 4 blocks
    n = ctypes.c_size_t(0)
    assert lib.rettn_dynamic_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value == 2 * 4 * 2 * 3 * 4 * 64
    assert lib.rettn_dynamic_workspace_bytes(ctypes.byref(d), None) == EINVAL
    d.block = 48
    assert lib.rettn_dynamic_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == EINVAL


def _calib_ws_bytes(d):
    n = ctypes.c_size_t(12345)
    st = rt.lib().rettn_calibrate_workspace_bytes(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def test_calibrate_workspace_size():
    """V's extent in float16 when the 64/128-token-block kernel takes the call, else 0."""
    d = _good_desc()                     # B 2, H 3, L 200, d 64, contiguous
    assert _calib_ws_bytes(d) == (0, 2 * 3 * 200 * 64 * 2)
    d.block = 128
    assert _calib_ws_bytes(d) == (0, 2 * 3 * 200 * 64 * 2)
    d.block = 32                         # the general kernels: no conversion pass
    assert _calib_ws_bytes(d) == (0, 0)
    d = _good_desc()
    d.dtype = b.RETTN_F32
    assert _calib_ws_bytes(d) == (0, 0)
    # strided layouts: the extent up to the last row's d elements, in V's own layout
    d = b.Desc(2, 3, 200, 64, 64, b.RETTN_BF16, 5 * 256 * 96, 256 * 96, 96)      # padded rows and slices
    assert _calib_ws_bytes(d) == (0, (1 * 5 * 256 * 96 + 2 * 256 * 96 + 199 * 96 + 64) * 2)
    d = b.Desc(2, 3, 200, 64, 64, b.RETTN_BF16, 200 * 3 * 64, 64, 3 * 64)         # [B, L, H, d] order
    assert _calib_ws_bytes(d) == (0, (200 * 3 * 64 + 2 * 64 + 199 * 3 * 64 + 64) * 2)
    # a slice past 32-bit offsets takes the general kernel: no workspace
    d = b.Desc(1, 1, 1 << 17, 64, 64, b.RETTN_BF16, (1 << 17) * 8192, (1 << 17) * 8192, 8192)
    assert _calib_ws_bytes(d) == (0, 0)
    # an extent beyond 2^50 elements, a bad descriptor, a null output
    d = b.Desc(2, 1, 200, 64, 64, b.RETTN_BF16, 1 << 60, 200 * 64, 64)
    assert _calib_ws_bytes(d)[0] == 2                 # RETTN_EUNSUPPORTED
    d = _good_desc()
    d.d = 0
    assert _calib_ws_bytes(d)[0] == EINVAL
    assert rt.lib().rettn_calibrate_workspace_bytes(ctypes.byref(_good_desc()), None) == EINVAL


def test_calibrate_ws_rejects_bad_workspaces():
    """Nothing is launched for a workspace that is null, misaligned, too small or overlaps a tensor."""
    lib = rt.lib()
    d = _good_desc()
    need = 2 * 3 * 200 * 64 * 2
    idx = _idx()
    base = 1 << 40                       # tensors far apart, 16-byte aligned; never dereferenced
    q, k, v, o, r, rho = (base + i * (1 << 30) for i in range(6))
    ws_ok = base + 8 * (1 << 30)

    def call(ws=ws_ok, ws_bytes=need, kind=b.RESIDUAL_MASKED, desc=d, **tensors):
        t = dict(q=q, k=k, v=v, o=o, r=r)
        t.update(tensors)
        return lib.rettn_calibrate_ws(ctypes.byref(desc), t["q"], t["k"], t["v"], ctypes.byref(idx), ws, ws_bytes,
                                      t["o"], rho, t["r"], kind, None)
    assert call(ws=None) == EINVAL
    assert call(ws=ws_ok + 8) == EINVAL
    assert call(ws_bytes=need - 1) == EINVAL
    assert call(ws=v) == EINVAL                       # the workspace is V itself
    assert call(ws=o + need - 16) == EINVAL           # its first bytes overlap O's last ones
    assert call(ws=q - need + 16) == EINVAL           # its last bytes overlap Q's first ones
    assert call(ws=rho + 2 * 3 * 200 * 4 - 16) == EINVAL   # overlaps the last floats of rho
    assert call(ws=rho - need + 16) == EINVAL         # its last bytes overlap rho's first ones
    assert call(kind=7) == EINVAL
    bad = _good_desc()
    bad.d = 0
    assert call(desc=bad) == EINVAL
    assert call(q=FAKE + 8) == EINVAL


def test_sparse_workspace_size():
    """V's extent in float16 only for 128-token blocks whose key blocks are each kept by 24 query blocks
    on average (nnz >= 24 nkb); 0 otherwise."""
    lib = rt.lib()

    def size(d, nnz):
        n = ctypes.c_size_t(7)
        nb = -(-d.L // d.block)
        idx = b.Index(nb, nb, nnz, FAKE, FAKE, FAKE)
        return lib.rettn_sparse_workspace_bytes(ctypes.byref(d), ctypes.byref(idx), ctypes.byref(n)), n.value
    d = b.Desc(1, 2, 128 * 60, 128, 128, b.RETTN_BF16, 2 * 128 * 60 * 128, 128 * 60 * 128, 128)
    assert size(d, 24 * 60) == (0, 2 * 128 * 60 * 128 * 2)
    assert size(d, 24 * 60 - 1) == (0, 0)
    d64 = b.Desc(1, 2, 128 * 60, 128, 64, b.RETTN_BF16, 2 * 128 * 60 * 128, 128 * 60 * 128, 128)
    assert size(d64, 120 * 120) == (0, 0)              # 64-token blocks never take the pass
    f32 = b.Desc(1, 2, 128 * 60, 128, 128, b.RETTN_F32, 2 * 128 * 60 * 128, 128 * 60 * 128, 128)
    assert size(f32, 60 * 60) == (0, 0)
    bad = b.Desc(1, 2, 128 * 60, 0, 128, b.RETTN_BF16, 2 * 128 * 60 * 128, 128 * 60 * 128, 128)
    assert size(bad, 60 * 60)[0] == EINVAL
    assert lib.rettn_sparse_workspace_bytes(ctypes.byref(d), None, ctypes.byref(ctypes.c_size_t())) == EINVAL


def test_sparse_ws_rejects_bad_workspaces():
    lib = rt.lib()
    L, nb = 128 * 60, 60
    d = b.Desc(1, 2, L, 128, 128, b.RETTN_BF16, 2 * L * 128, L * 128, 128)
    need = 2 * L * 128 * 2
    idx = b.Index(nb, nb, nb * nb, FAKE, FAKE, FAKE)
    base = 1 << 40
    q, k, v, o, r, rho = (base + i * (1 << 30) for i in range(6))

    def call(ws, ws_bytes, lam=0.04):
        return lib.rettn_sparse_ws(ctypes.byref(d), q, k, v, ctypes.byref(idx), rho, r, lam, 1, ws, ws_bytes, o, None)
    ws_ok = base + 8 * (1 << 30)
    assert call(None, need) == EINVAL
    assert call(ws_ok + 8, need) == EINVAL
    assert call(ws_ok, need - 1) == EINVAL
    assert call(k + 16, need) == EINVAL                 # overlaps K
    assert call(rho + 16, need) == EINVAL               # overlaps rho (read after the conversion pass)
    assert call(ws_ok, need, lam=-1.0) == EINVAL


def test_dynamic_index_rejects_bad_arguments():
    lib = rt.lib()
    d = _good_desc()
    need = 2 * 4 * 2 * 3 * 4 * 64
    ok = dict(q=FAKE, k=FAKE, keep=2, ws=FAKE, ws_bytes=need, mask=FAKE, rp=FAKE, ci=FAKE)

    def call(desc=d, **kw):
        a = {**ok, **kw}
        return lib.rettn_dynamic_index(ctypes.byref(desc), a["q"], a["k"], a["keep"], a["ws"], a["ws_bytes"],
                                       a["mask"], a["rp"], a["ci"], None)
    assert call(keep=0) == EINVAL
    assert call(ws_bytes=need - 1) == EINVAL
    assert call(ws=None) == EINVAL
    assert call(ws=FAKE + 4) == EINVAL
    assert call(q=FAKE + 8) == EINVAL
    assert call(mask=None) == EINVAL
    assert call(ci=FAKE + 2) == EINVAL
    bad = _good_desc()
    bad.d = 60
    assert call(desc=bad) == EINVAL
    big = b.Desc(1, 1, 2049 * 32, 64, 32, b.RETTN_BF16, 2049 * 32 * 64, 2049 * 32 * 64, 64)
    assert call(desc=big, ws_bytes=1 << 40) == 2   # RETTN_EUNSUPPORTED: more than 2048 blocks per side
