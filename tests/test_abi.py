"""C-ABI library: it loads, exports every function include/moe.h declares,
and rejects bad arguments on the host before touching the GPU (CPU only)."""

import ctypes
import os
import re
import subprocess

import pytest
import torch

from sparse_mixture_experts_kept_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _lib():
    if not os.path.exists(moe.LIB_PATH):
        from sparse_mixture_experts_kept_amd import build

        build.build()
    return moe.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for required in ("moe_router_topk", "moe_permute", "moe_grouped_swiglu", "moe_combine", "moe_ffn_forward"):
        assert required in names
    assert set(names) == set(moe.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (moe_[a-z_]+)\b", out))
    assert set(_declared_functions()) <= exported
    assert moe.status_string(moe.MOE_ERR_UNSUPPORTED) == "MOE_ERR_UNSUPPORTED"
    assert lib.moe_version().decode().count(".") == 2


needs_no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                                  reason="host-validation checks with fake pointers run only where no GPU exists")

FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below must fail validation
MISALIGNED = ctypes.c_void_p(0x100002)


def _dims(**kw):
    base = dict(T=16, d=256, f=512, dtype=moe.MOE_BF16, variant=0)
    base.update(kw)
    return moe.make_dims(**base)


@needs_no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), moe.MOE_ERR_INVALID_ARGUMENT),
    (dict(d=200), moe.MOE_ERR_UNSUPPORTED),
    (dict(f=100), moe.MOE_ERR_UNSUPPORTED),
    (dict(d=0), moe.MOE_ERR_UNSUPPORTED),
    (dict(dtype=7), moe.MOE_ERR_UNSUPPORTED),
    (dict(variant=3), moe.MOE_ERR_UNSUPPORTED),
    (dict(gating=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(gating=-1), moe.MOE_ERR_UNSUPPORTED),
    (dict(capacity=-1), moe.MOE_ERR_INVALID_ARGUMENT),
    (dict(T=1 << 31), moe.MOE_ERR_UNSUPPORTED),
])
def test_bad_dims_are_rejected(kw, status):
    lib = _lib()
    dims = _dims(**kw)
    n = ctypes.c_size_t(0)
    assert lib.moe_router_topk(ctypes.byref(dims), FAKE, FAKE, None, FAKE, FAKE, None, None) == status
    assert lib.moe_permute(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(n), None) == status
    assert lib.moe_grouped_swiglu(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == status
    assert lib.moe_combine(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, None) == status
    assert lib.moe_ffn_forward(ctypes.byref(dims), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None, None,
                               None, ctypes.byref(n), None) == status
    assert lib.moe_load_balance_loss(ctypes.byref(dims), FAKE, FAKE, FAKE, None) == status
    assert lib.moe_ffn_forward_routed(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                      ctypes.byref(n), None) == status
    assert lib.moe_rmsnorm_residual_route(ctypes.byref(dims), FAKE, None, FAKE, 1e-5, FAKE, None, FAKE, FAKE,
                                          None) == status


@needs_no_gpu
def test_wrong_expert_count_or_k():
    lib = _lib()
    for E, k in ((4, 2), (8, 1), (16, 2), (8, 3)):
        dims = moe.make_dims(16, 256, 512, moe.MOE_BF16, E=E, k=k)
        assert lib.moe_router_topk(ctypes.byref(dims), FAKE, FAKE, None, FAKE, FAKE, None, None) == \
            moe.MOE_ERR_UNSUPPORTED


@needs_no_gpu
def test_null_and_misaligned_pointers():
    lib = _lib()
    dims = _dims()
    INV = moe.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_router_topk(None, FAKE, FAKE, None, FAKE, FAKE, None, None) == INV
    assert lib.moe_router_topk(ctypes.byref(dims), None, FAKE, None, FAKE, FAKE, None, None) == INV
    assert lib.moe_router_topk(ctypes.byref(dims), MISALIGNED, FAKE, None, FAKE, FAKE, None, None) == INV
    big = ctypes.c_size_t(1 << 20)
    assert lib.moe_permute(ctypes.byref(dims), FAKE, None, FAKE, FAKE, FAKE, ctypes.byref(big), None) == INV
    assert lib.moe_permute(ctypes.byref(dims), FAKE, FAKE, MISALIGNED, FAKE, FAKE, ctypes.byref(big), None) == INV
    assert lib.moe_permute(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, MISALIGNED, ctypes.byref(big), None) == INV
    assert lib.moe_permute(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == INV
    assert lib.moe_grouped_swiglu(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == INV
    assert lib.moe_grouped_swiglu(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, MISALIGNED, FAKE,
                                  None) == INV
    assert lib.moe_combine(ctypes.byref(dims), FAKE, FAKE, FAKE, None, None) == INV
    assert lib.moe_combine(ctypes.byref(dims), MISALIGNED, FAKE, FAKE, FAKE, None) == INV
    assert lib.moe_load_balance_loss(ctypes.byref(dims), None, FAKE, FAKE, None) == INV
    assert lib.moe_load_balance_loss(ctypes.byref(dims), FAKE, FAKE, None, None) == INV
    assert lib.moe_load_balance_loss(ctypes.byref(dims), MISALIGNED, FAKE, FAKE, None) == INV
    assert lib.moe_rmsnorm_residual(4, 256, None, None, FAKE, 1e-5, 1, None) == INV
    assert lib.moe_rmsnorm_residual(-1, 256, FAKE, None, FAKE, 1e-5, 1, None) == INV
    assert lib.moe_rmsnorm_residual(4, 250, FAKE, None, FAKE, 1e-5, 1, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_rmsnorm_residual(4, 256, FAKE, None, FAKE, 1e-5, 5, None) == moe.MOE_ERR_UNSUPPORTED


@needs_no_gpu
def test_router_lds_limit():
    lib = _lib()
    dims = moe.make_dims(16, 8192 + 128, 512, moe.MOE_BF16)
    assert lib.moe_router_topk(ctypes.byref(dims), FAKE, FAKE, None, FAKE, FAKE, None, None) == \
        moe.MOE_ERR_UNSUPPORTED
    dims = moe.make_dims(16, 4096 + 128, 512, moe.MOE_F32)
    assert lib.moe_router_topk(ctypes.byref(dims), FAKE, FAKE, None, FAKE, FAKE, None, None) == \
        moe.MOE_ERR_UNSUPPORTED


@needs_no_gpu
def test_workspace_query_and_too_small():
    lib = _lib()
    T, d, f = 4096, 4096, 14336
    dims = moe.make_dims(T, d, f, moe.MOE_BF16)
    n = ctypes.c_size_t(0)
    assert lib.moe_ffn_forward(ctypes.byref(dims), None, None, None, None, None, None, None, None, None, None,
                               None, ctypes.byref(n), None) == moe.MOE_OK
    slots = T * 2
    # h (bf16) and two y_rows partial buffers (fp32) dominate; routing arrays are small
    assert n.value >= slots * f * 2 + 2 * slots * d * 4
    assert n.value < slots * f * 2 + 2 * slots * d * 4 + (1 << 20)
    small = ctypes.c_size_t(n.value - 1)
    ws = ctypes.c_void_p(0x200000)
    assert lib.moe_ffn_forward(ctypes.byref(dims), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None, None, ws,
                               ctypes.byref(small), None) == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    assert lib.moe_ffn_forward(ctypes.byref(dims), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None, None, ws,
                               None, None) == moe.MOE_ERR_INVALID_ARGUMENT
    big = ctypes.c_size_t(n.value)
    assert lib.moe_ffn_forward(ctypes.byref(dims), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None, None,
                               ctypes.c_void_p(0x200010), ctypes.byref(big), None) == moe.MOE_ERR_INVALID_ARGUMENT


@needs_no_gpu
def test_zero_tokens_is_a_no_op():
    lib = _lib()
    dims = _dims(T=0)
    n = ctypes.c_size_t(0)
    assert lib.moe_router_topk(ctypes.byref(dims), None, None, None, None, None, None, None) == moe.MOE_OK
    assert lib.moe_permute(ctypes.byref(dims), None, None, None, None, None, ctypes.byref(n), None) == moe.MOE_OK
    assert lib.moe_permute(ctypes.byref(dims), None, None, None, None, FAKE, ctypes.byref(n), None) == moe.MOE_OK
    assert lib.moe_grouped_swiglu(ctypes.byref(dims), None, None, None, None, None, None, None, None, None) == \
        moe.MOE_OK
    assert lib.moe_combine(ctypes.byref(dims), None, None, None, None, None) == moe.MOE_OK
    assert lib.moe_ffn_forward(ctypes.byref(dims), None, None, None, None, None, None, None, None, None, None,
                               None, ctypes.byref(n), None) == moe.MOE_OK
    assert lib.moe_rmsnorm_residual(0, 256, None, None, None, 1e-5, 1, None) == moe.MOE_OK
    assert lib.moe_load_balance_loss(ctypes.byref(dims), None, None, None, None) == moe.MOE_OK
    assert lib.moe_ffn_forward_routed(ctypes.byref(dims), None, None, None, None, None, None, None, None, None,
                                      ctypes.byref(n), None) == moe.MOE_OK
    assert lib.moe_rmsnorm_residual_route(ctypes.byref(dims), None, None, None, 1e-5, None, None, None, None,
                                          None) == moe.MOE_OK


@needs_no_gpu
def test_routed_and_fused_glue_validation():
    lib = _lib()
    dims = _dims()
    INV = moe.MOE_ERR_INVALID_ARGUMENT
    n = ctypes.c_size_t(1 << 40)
    # routed layer: no routing (NULL ids or gates), misaligned ids
    assert lib.moe_ffn_forward_routed(ctypes.byref(dims), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                      ctypes.byref(n), None) == INV
    assert lib.moe_ffn_forward_routed(ctypes.byref(dims), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                      ctypes.byref(n), None) == INV
    assert lib.moe_ffn_forward_routed(ctypes.byref(dims), FAKE, MISALIGNED, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                      FAKE, ctypes.byref(n), None) == INV
    # the size query needs no routing and matches moe_ffn_forward's
    q1, q2 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.moe_ffn_forward_routed(ctypes.byref(dims), None, None, None, None, None, None, None, None, None,
                                      ctypes.byref(q1), None) == moe.MOE_OK
    assert lib.moe_ffn_forward(ctypes.byref(dims), None, None, None, None, None, None, None, None, None, None,
                               None, ctypes.byref(q2), None) == moe.MOE_OK
    assert q1.value == q2.value > 0
    # fused glue: required pointers, alignment, and the d limit of the register-resident row
    assert lib.moe_rmsnorm_residual_route(ctypes.byref(dims), None, None, FAKE, 1e-5, FAKE, None, FAKE, FAKE,
                                          None) == INV
    assert lib.moe_rmsnorm_residual_route(ctypes.byref(dims), FAKE, None, FAKE, 1e-5, None, None, FAKE, FAKE,
                                          None) == INV
    assert lib.moe_rmsnorm_residual_route(ctypes.byref(dims), FAKE, MISALIGNED, FAKE, 1e-5, FAKE, None, FAKE, FAKE,
                                          None) == INV
    wide = _dims(d=8192 + 128)
    assert lib.moe_rmsnorm_residual_route(ctypes.byref(wide), FAKE, None, FAKE, 1e-5, FAKE, None, FAKE, FAKE,
                                          None) == moe.MOE_ERR_UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    with pytest.raises(ValueError):
        moe.ptr(torch.zeros(4))


@needs_no_gpu
def test_permute_workspace_query():
    # per-group counts (ceil(T/16) x 8 int32) between 512 and 65536 tokens, a minimal 256 bytes otherwise
    lib = _lib()
    for T, need in ((16, 256), (512, 256), (513, 33 * 8 * 4 + (256 - 33 * 8 * 4 % 256) % 256), (4096, 8192),
                    (65536, 131072), (65537, 256)):
        dims = _dims(T=T)
        n = ctypes.c_size_t(0)
        assert lib.moe_permute(ctypes.byref(dims), None, None, None, None, None, ctypes.byref(n), None) == moe.MOE_OK
        assert n.value == need, (T, n.value)
    dims = _dims(T=4096)
    small = ctypes.c_size_t(8191)
    assert lib.moe_permute(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(small), None) == \
        moe.MOE_ERR_WORKSPACE_TOO_SMALL


@needs_no_gpu
def test_timed_and_residual_entry_points_validate():
    lib = _lib()
    dims = _dims()
    n = ctypes.c_size_t(1 << 30)
    INV = moe.MOE_ERR_INVALID_ARGUMENT
    ws = ctypes.c_void_p(0x200000)
    events = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    holes = (ctypes.c_void_p * 8)(*([FAKE] * 7 + [None]))
    args = (FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None, None, ws, ctypes.byref(n), None)
    assert lib.moe_ffn_forward_timed(ctypes.byref(dims), *args, None, None) == INV  # no events
    assert lib.moe_ffn_forward_timed(ctypes.byref(dims), *args, holes, None) == INV  # a NULL event
    assert lib.moe_ffn_forward_timed(ctypes.byref(dims), *args, events, MISALIGNED) == INV
    # the fused glue: resid, u_out and (with a next router) its outputs are required
    r = (FAKE, FAKE, FAKE, FAKE, FAKE)  # x, idx, w, w1, w3
    assert lib.moe_ffn_forward_routed_residual(ctypes.byref(dims), *r, FAKE, None, FAKE, 1e-5, None, None, None,
                                               None, None, ws, ctypes.byref(n), None) == INV
    assert lib.moe_ffn_forward_routed_residual(ctypes.byref(dims), *r, FAKE, FAKE, FAKE, 1e-5, FAKE, None, None,
                                               FAKE, None, ws, ctypes.byref(n), None) == INV
    assert lib.moe_ffn_forward_routed_residual(ctypes.byref(dims), *r, FAKE, FAKE, MISALIGNED, 1e-5, None, None,
                                               None, None, None, ws, ctypes.byref(n), None) == INV
    big_d = _dims(d=8192 + 128)
    assert lib.moe_ffn_forward_routed_residual(ctypes.byref(big_d), *r, FAKE, FAKE, FAKE, 1e-5, None, None, None,
                                               None, None, ws, ctypes.byref(n), None) == moe.MOE_ERR_UNSUPPORTED
    # size query, as moe_ffn_forward
    q = ctypes.c_size_t(0)
    q2 = ctypes.c_size_t(0)
    assert lib.moe_ffn_forward_routed_residual(ctypes.byref(dims), None, None, None, None, None, None, None, None,
                                               1e-5, None, None, None, None, None, None, ctypes.byref(q), None) == 0
    assert lib.moe_ffn_forward(ctypes.byref(dims), None, None, None, None, None, None, None, None, None, None,
                               None, ctypes.byref(q2), None) == 0
    assert q.value == q2.value > 0


@needs_no_gpu
def test_noalloc_rejects_a_layer_beyond_its_array():
    # the workspace of 400 Mixtral-sized tokens on the prefill kernels exceeds the 32 MiB array:
    # rejected on the host before anything else happens (no device is needed to see it)
    lib = _lib()
    dims = moe.make_dims(400, 4096, 14336, moe.MOE_BF16)
    assert lib.moe_ffn_forward_noalloc(ctypes.byref(dims), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None,
                                       None, None) == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    bad = moe.make_dims(16, 4096, 14336, moe.MOE_BF16, E=4)
    assert lib.moe_ffn_forward_noalloc(ctypes.byref(bad), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None,
                                       None, None) == moe.MOE_ERR_UNSUPPORTED


@needs_no_gpu
def test_mfma_ceiling_validates():
    lib = _lib()
    INV = moe.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_mfma_ceiling(None, FAKE, FAKE, 10, None) == INV
    assert lib.moe_mfma_ceiling(FAKE, None, FAKE, 10, None) == INV
    assert lib.moe_mfma_ceiling(FAKE, FAKE, FAKE, 0, None) == INV
    assert lib.moe_mfma_ceiling(MISALIGNED, FAKE, FAKE, 10, None) == INV


def _expected_workspace(T, d, f, elem, prefill):
    a = lambda n: (n + 255) // 256 * 256  # noqa: E731
    slots = 2 * T
    total = a(slots * 4) * 4 + a(9 * 4) + a((T + 15) // 16 * 8 * 4) + a(slots * f * elem) + a(slots * d * 4)
    if elem == 2 and T <= 64:  # the bf16 small-batch router's partial scores: 16 slices x 64 lanes x 16 B per group
        total += a(16 * ((T + 15) // 16) * 64 * 16)
    return total + (a(slots * d * 4) if prefill else 0)


@needs_no_gpu
@pytest.mark.parametrize("T,d,f,dtype,variant,prefill", [
    (1, 4096, 14336, "bf16", moe.VARIANT_AUTO, False), (32, 4096, 14336, "bf16", moe.VARIANT_AUTO, False),
    (128, 4096, 14336, "bf16", moe.VARIANT_AUTO, False), (129, 4096, 14336, "bf16", moe.VARIANT_AUTO, True),
    (4096, 4096, 14336, "bf16", moe.VARIANT_AUTO, True), (4096, 4096, 14336, "bf16", moe.VARIANT_DECODE, False),
    (16, 512, 1024, "bf16", moe.VARIANT_PREFILL, True), (300, 128, 256, "bf16", moe.VARIANT_AUTO, False),
    (300, 256, 128, "bf16", moe.VARIANT_PREFILL, False), (700, 256, 512, "f32", moe.VARIANT_AUTO, False),
    (600000, 4096, 256, "bf16", moe.VARIANT_AUTO, False)])
def test_workspace_layout(T, d, f, dtype, variant, prefill):
    # The workspace is the routing, the permutation, the router's group
    # counts, the bf16 small-batch router's partial scores (T <= 64), h and
    # y_rows, each 256-byte aligned, plus the second fp32
    # partial region only when the layer runs the bf16 prefill kernels: AUTO
    # streams up to 128 tokens, the prefill kernels need d, f >= 256 and x
    # below 4 GiB (600000 x 4096 bf16 is not), fp32 has its own kernels.
    elem = 2 if dtype == "bf16" else 4
    got = moe.workspace_size(T, d, f, torch.bfloat16 if dtype == "bf16" else torch.float32, variant)
    assert got == _expected_workspace(T, d, f, elem, prefill)


@needs_no_gpu
def test_noalloc_token_limits():
    # the fixed 32 MiB array holds the layer's workspace up to 272 Mixtral-
    # sized tokens with the kernels AUTO picks and 372 with the streaming
    # kernels forced
    lim = 32 << 20
    for variant, top in ((moe.VARIANT_AUTO, 272), (moe.VARIANT_DECODE, 372)):
        assert moe.workspace_size(top, 4096, 14336, torch.bfloat16, variant) <= lim
        assert moe.workspace_size(top + 1, 4096, 14336, torch.bfloat16, variant) > lim
