"""The no-allocation dynamic index (rettn_dynamic_index_noalloc) against the
entry point that takes a workspace (rettn_dynamic_index), through the C ABI.

The no-allocation entry point keeps the block means in a static per-GPU array
inside the library, so it is checked on consecutive calls of different sizes
(the array keeps the previous call's contents) and must agree bit for bit
with the workspace version on the mask, row pointers and column ids.
"""
import ctypes

import numpy as np
import pytest

import sparse_attention_diffusion_block_amd as rt
from sparse_attention_diffusion_block_amd import rettn as b
from tests.gpu_util import dev, log
from workloads import make_qkv


def _desc(B, H, L, d, block, dtype=b.RETTN_BF16):
    return b.Desc(B, H, L, d, block, dtype, H * L * d, L * d, d)


def test_noalloc_rejects_requests_beyond_its_scratch():
    """Validated on the host before any HIP call: a request whose block means exceed the static
    scratch gets RETTN_ESCRATCH, bad arguments RETTN_EINVAL, and nothing is launched."""
    lib = rt.lib()
    assert lib.rettn_status_str(b.STATUS_ESCRATCH).decode().startswith("RETTN_ESCRATCH")
    buf = ctypes.create_string_buffer(4096 + 256)
    p = (ctypes.addressof(buf) + 255) // 256 * 256          # 256-byte aligned host address: never dereferenced
    # 2 * B*H * nb * d * 4 bytes: B=1, H=64, L=131072, d=128, block 128 -> 2 * 64 * 1024 * 128 * 4 = 64 MiB
    big = _desc(1, 64, 131072, 128, 128)
    need = ctypes.c_size_t(0)
    assert lib.rettn_dynamic_workspace_bytes(ctypes.byref(big), ctypes.byref(need)) == 0
    assert need.value > b.NOALLOC_SCRATCH_BYTES
    assert lib.rettn_dynamic_index_noalloc(ctypes.byref(big), p, p, 9, p, p, p, None) == b.STATUS_ESCRATCH
    small = _desc(1, 2, 300, 64, 64)
    assert lib.rettn_dynamic_index_noalloc(ctypes.byref(small), p, p, 0, p, p, p, None) == 1          # keep < 1
    assert lib.rettn_dynamic_index_noalloc(ctypes.byref(small), None, p, 3, p, p, p, None) == 1       # null Q
    assert lib.rettn_dynamic_index_noalloc(ctypes.byref(small), p + 8, p, 3, p, p, p, None) == 1      # misaligned
    assert lib.rettn_dynamic_index_noalloc(None, p, p, 3, p, p, p, None) == 1


CASES = [
    # B, H, L, d, block, keep, dtype: the second call is smaller than the first, the third smaller again
    (2, 30, 17776, 64, 64, 9, "bf16"),
    (2, 4, 3000, 72, 64, 5, "bf16"),
    (1, 2, 700, 32, 128, 3, "f32"),
]


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rt.lib()
    for call, (B, H, L, d, block, keep, dtype) in enumerate(CASES):
        log(f"no-alloc dynamic index call {call}: B={B} H={H} L={L} d={d} block={block} keep={keep} {dtype}")
        q, k, _ = make_qkv(B, H, L, d, 80 + call, dtype=dtype)
        tq, tk = dev(q, dtype), dev(k, dtype)
        # the workspace version on a workspace full of NaN (nothing may depend on its contents)
        need = rt.dynamic_workspace_bytes(tq, block)
        ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
        ref = rt.dynamic_index(tq, tk, keep, block, workspace=ws)
        got = rt.dynamic_index(tq, tk, keep, block)          # output buffers of the same shape
        for t in (got.mask, got.row_ptr, got.col_idx):
            t.fill_(0x5A)
        rt.dynamic_index_noalloc(tq, tk, keep, block, out=got)
        torch.cuda.synchronize()
        for name, a, r in (("mask", got.mask, ref.mask), ("row_ptr", got.row_ptr, ref.row_ptr),
                           ("col_idx", got.col_idx, ref.col_idx)):
            assert torch.equal(a, r), f"call {call}: {name} differs from the workspace entry point"
        nb = -(-L // block)
        kk = min(keep, nb)
        assert np.array_equal(got.row_ptr.cpu().numpy(), np.tile(np.arange(nb + 1) * kk, (B * H, 1)))
        del ws, ref, got
