"""The C-ABI library loads and exports every entry point include/moe.h declares.

Also the host-side argument checks, which return before any HIP call (no
device needed): shape errors, the T = 0 no-op, NULL pointers, misalignment,
workspace sizing.  No compute runs here.
"""

import ctypes
import os
import re

import pytest

import sparse_moe_expert_amd as sme
import sparse_moe_expert_amd.build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sme.LIB_PATH):
        sme.build.build_library()
    return sme.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert names == sorted(sme.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(8):
        assert sme.moe_status_string(s)
    assert sme.moe_status_string(99) == "unknown status"


P = ctypes.c_void_p
A = P(256)           # a fake, 16-byte aligned, never dereferenced address


def test_route_topk_host_checks(lib):
    f = lib.moe_route_topk
    assert f(A, None, 4, 8, 9, A, A, None) == 2     # k > E
    assert f(A, None, 4, 8, 0, A, A, None) == 2     # k < 1
    assert f(A, None, -1, 8, 2, A, A, None) == 2    # T < 0
    assert f(A, None, 4, 2048, 2, A, A, None) == 3  # E beyond envelope
    assert f(A, None, 4, 64, 33, A, A, None) == 3   # k beyond envelope
    assert f(A, None, 0, 8, 2, A, A, None) == 0     # T = 0: nothing launched
    assert f(None, None, 4, 8, 2, A, A, None) == 1
    assert f(P(258), None, 4, 8, 2, A, A, None) == 4


def test_router_logits_host_checks(lib):
    f = lib.moe_router_logits
    assert f(A, A, -1, 64, 8, A, None) == 2         # T < 0
    assert f(A, A, 4, 60, 8, A, None) == 2          # H not a multiple of 8
    assert f(A, A, 4, 0, 8, A, None) == 2           # H < 8
    assert f(A, A, 4, 64, 0, A, None) == 2          # E < 1
    assert f(A, A, 4, 8192, 8, A, None) == 3        # H beyond envelope
    assert f(A, A, 4, 64, 2048, A, None) == 3       # E beyond envelope
    assert f(A, A, 0, 64, 8, A, None) == 0          # T = 0: nothing launched
    assert f(None, A, 4, 64, 8, A, None) == 1
    assert f(A, A, 4, 64, 8, None, None) == 1
    assert f(A, P(258), 4, 64, 8, A, None) == 4


def test_bucket_routes_host_checks(lib):
    f = lib.moe_bucket_routes
    assert f(A, 4, 8, 9, A, A, A, A, A, A, None) == 2
    assert f(A, 0, 8, 2, A, A, A, A, A, A, None) == 0
    assert f(A, 4, 8, 2, A, A, None, A, A, A, None) == 1
    assert f(A, 4, 8, 2, A, A, A, A, P(260), A, None) == 4
    assert f(A, 1 << 22, 8, 8, A, A, A, A, A, A, None) == 3   # R > 2^24


def _ffn(lib, T=4, H=256, I=128, E=8, k=2, ws=1 << 20, null_at=None, bad_at=None):
    ptrs = [A] * 15
    if null_at is not None:
        ptrs[null_at] = None
    if bad_at is not None:
        ptrs[bad_at] = P(264)
    return lib.moe_expert_ffn(*ptrs, T, H, I, E, k, A, ctypes.c_size_t(ws), A, None)


def test_expert_ffn_host_checks(lib):
    assert _ffn(lib, H=48) == 2          # H not a multiple of 32
    assert _ffn(lib, I=100) == 2
    assert _ffn(lib, k=9) == 2
    # H/32 = 3 and I/32 = 20 (not powers of two) pass the envelope and fail
    # on the small workspace (nothing launched); H = 8192 is outside it
    assert _ffn(lib, H=96, ws=16) == 5
    assert _ffn(lib, H=2560, I=640, E=512, k=10, ws=16) == 5
    assert _ffn(lib, H=8192) == 3
    assert _ffn(lib, T=0) == 0
    assert _ffn(lib, null_at=3) == 1
    assert _ffn(lib, bad_at=0) == 4
    need = lib.moe_expert_ffn_workspace_size(4, 256, 128, 8, 2)
    assert need > 0 and need % 256 == 0
    assert _ffn(lib, ws=need - 1) == 5
    assert lib.moe_expert_ffn_workspace_size(0, 256, 128, 8, 2) == 0
    # grows with T*k: h (bf16 [R,I]) and o (fp16 [R,H])
    assert lib.moe_expert_ffn_workspace_size(8, 256, 128, 8, 2) > need


def test_activation_bytes_limit(lib):
    """The activations are read through 32-bit buffer offsets: T*H*2 must stay
    below 2^31 (else MOE_ERR_UNSUPPORTED, nothing launched); one token fewer
    passes the envelope and fails later on the small workspace."""
    T = (1 << 31) // (2 * 2048)
    assert _ffn(lib, T=T, H=2048, I=512, E=512, k=10, ws=16) == 3
    assert _ffn(lib, T=T - 1, H=2048, I=512, E=512, k=10, ws=16) == 5
    assert _step(lib, T=T, H=2048, I=512, E=512, k=10, ws=16) == 3
    assert _step(lib, T=T - 1, H=2048, I=512, E=512, k=10, ws=16) == 5


def test_route_bucket_host_checks(lib):
    f = lib.moe_route_bucket
    assert f(A, None, 4, 8, 9, A, A, A, A, A, A, A, A, None) == 2
    assert f(A, None, 0, 8, 2, A, A, A, A, A, A, A, A, None) == 0
    assert f(A, None, 4, 8, 2, A, A, None, A, A, A, A, A, None) == 1
    assert f(A, None, 4, 2048, 2, A, A, A, A, A, A, A, A, None) == 3


def test_ffn_stage_host_checks(lib):
    ptrs = [A] * 15
    f = lib.moe_expert_ffn_stage
    for bad in (0, 4, -1):
        assert f(bad, *ptrs, 4, 256, 128, 8, 2, A, ctypes.c_size_t(1 << 20), A, None) == 2
    assert f(1, *ptrs, 0, 256, 128, 8, 2, A, ctypes.c_size_t(1 << 20), A, None) == 0


def _step(lib, T=4, H=256, I=128, E=8, k=2, ws=1 << 24, null_at=None, bad_at=None, bias=None):
    ins = [A] * 10          # x, logits, bias, 6 weight arrays, g_scale
    ins[2] = bias
    outs = [A] * 8          # topk_idx, topk_w, 6 bucket arrays
    if null_at is not None:
        (ins if null_at < 10 else outs)[null_at if null_at < 10 else null_at - 10] = None
    if bad_at is not None:
        (ins if bad_at < 10 else outs)[bad_at if bad_at < 10 else bad_at - 10] = P(264)
    return lib.moe_step(*ins, T, H, I, E, k, *outs, A, ctypes.c_size_t(ws), A, None)


def test_step_host_checks(lib):
    assert _step(lib, k=9) == 2
    assert _step(lib, H=48) == 2
    assert _step(lib, H=96, ws=16) == 5
    assert _step(lib, H=2560, I=640, E=512, k=10, ws=16) == 5
    assert _step(lib, H=8192) == 3
    assert _step(lib, E=2048) == 3
    assert _step(lib, T=0) == 0
    assert _step(lib, null_at=1) == 1           # logits
    assert _step(lib, null_at=14) == 1          # an output
    assert _step(lib, bad_at=0) == 4
    assert _step(lib, bias=P(8)) == 4           # a misaligned bias
    need = lib.moe_step_workspace_size(4, 256, 128, 8, 2)
    assert _step(lib, ws=need - 1) == 5


def _workspace_formula(T, H, I, E, k):
    """moe_expert_ffn_workspace_size as the header states it: h (2*I bytes
    per route), o (2*H bytes per route), two work lists (gate/up, down) of
    16 bytes per item for min(E, T*k) + T*k // 128 items rounded up to 8,
    plus 16, an expert
    list of 4 bytes per slot, min(E, T*k) of them, plus 4, and 9 unit
    counters 128 bytes apart; each region rounded up to 256 bytes."""
    up = lambda v: (v + 255) // 256 * 256
    R = T * k
    items = min(E, R) + R // 128
    items = (items + 7) // 8 * 8
    return up(R * I * 2) + up(R * H * 2) + 2 * up(16 + 16 * items) + up(4 + 4 * min(E, R)) + up(9 * 128)


def test_workspace_size_formula(lib):
    for shape in [(4, 256, 128, 8, 2), (4, 2048, 512, 512, 10), (32, 2048, 512, 512, 10),
                  (256, 2048, 512, 512, 10), (4096, 2048, 512, 512, 10), (1, 32, 32, 1, 1)]:
        assert lib.moe_expert_ffn_workspace_size(*shape) == _workspace_formula(*shape), shape
    assert lib.moe_expert_ffn_workspace_size(4, 256, 128, 0, 2) == 0


def test_step_workspace_size(lib):
    for shape in [(4, 2048, 512, 512, 10), (4, 256, 128, 8, 2), (33, 2048, 512, 512, 10), (1, 32, 32, 2, 1)]:
        assert lib.moe_step_workspace_size(*shape) == lib.moe_expert_ffn_workspace_size(*shape)
    assert lib.moe_step_workspace_size(0, 2048, 512, 512, 10) == 0


def test_shared_expert_host_checks(lib):
    """Shape, envelope, pointer and workspace checks of moe_shared_expert
    before any launch (no device work: every case fails on the host)."""
    import ctypes
    buf = (ctypes.c_uint8 * 64)()
    p = ctypes.cast(buf, ctypes.c_void_p)
    al = ctypes.c_void_p((ctypes.addressof(buf) + 15) & ~15)
    f = lib.moe_shared_expert
    assert f(al, al, al, al, -1, 512, 512, al, 1 << 20, al, None) == 2          # T < 0
    assert f(al, al, al, al, 4, 48, 512, al, 1 << 20, al, None) == 2           # H not a multiple of 32
    assert f(al, al, al, al, 4, 256, 512, al, 1 << 20, al, None) == 3          # H not a multiple of 512
    assert f(al, al, al, al, 4, 8192, 512, al, 1 << 20, al, None) == 3         # H > 4096
    assert f(al, al, al, al, 0, 512, 512, None, 0, None, None) == 0            # T = 0: nothing to do
    assert f(None, al, al, al, 4, 512, 512, al, 1 << 20, al, None) == 1        # null x
    assert f(al, al, al, al, 4, 512, 512, al, 16, al, None) == 5               # workspace too small
    mis = ctypes.c_void_p(al.value + 4)
    assert f(mis, al, al, al, 4, 512, 512, al, 1 << 20, al, None) == 4        # misaligned x
    assert lib.moe_shared_expert_workspace_size(4, 2048, 512) == 4096


def test_step_shared_host_checks(lib):
    """moe_step_shared checks the shared expert's arguments, then the step's,
    before any launch (every case fails on the host)."""
    import ctypes
    buf = (ctypes.c_uint8 * 64)()
    al = ctypes.c_void_p((ctypes.addressof(buf) + 15) & ~15)
    f = lib.moe_step_shared

    def call(T=4, H=512, I=256, E=64, k=4, Is=512, se=al, se_bytes=1 << 20, x=al):
        return f(x, al, None, *([al] * 7), None, T, H, I, E, k, *([al] * 8), al, 1 << 30, al,
                 se, al, al, Is, al, se_bytes, al, None)
    assert call(Is=100) == 2                      # Is not a multiple of 32
    assert call(Is=8192) == 3                     # Is above the envelope
    assert call(se=None) == 1                     # null shared-expert weight
    assert call(se_bytes=16) == 5                 # shared workspace too small
    assert call(E=0) == 2                         # the step's own shape check
    assert call(k=65, E=128) == 3                 # the step's envelope (k > 32)
    assert call(T=0, x=None) == 0                 # T = 0: nothing to do
    assert lib.moe_shared_expert_workspace_size(0, 2048, 512) == 0


def _noalloc(lib, T=4, H=256, I=128, E=8, k=2, null_at=None, packed=None):
    ins = [A] * 10          # x, logits, bias, 6 weight arrays, g_scale
    ins[2] = None
    outs = [A] * 8          # topk_idx, topk_w, 6 bucket arrays
    if null_at is not None:
        (ins if null_at < 10 else outs)[null_at if null_at < 10 else null_at - 10] = None
    return lib.moe_step_noalloc(*ins, packed, T, H, I, E, k, *outs, A, None)


def test_step_noalloc_host_checks(lib):
    """moe_step_noalloc checks every argument and the static scratch's size
    (MOE_NOALLOC_SCRATCH_BYTES, 8 MiB) before any HIP call."""
    assert sme.NOALLOC_SCRATCH_BYTES == 8 << 20
    assert _noalloc(lib, k=9) == 2
    assert _noalloc(lib, H=48) == 2
    assert _noalloc(lib, E=2048) == 3
    assert _noalloc(lib, T=0) == 0
    assert _noalloc(lib, null_at=1) == 1
    assert _noalloc(lib, null_at=17) == 1
    assert _noalloc(lib, H=96, I=64, packed=A) == 2      # packed weights need multiples of 64
    assert _noalloc(lib, H=8192) == 3                    # outside the envelope
    # the workspace of 163 tokens at H = 2048, I = 512 fits the scratch, 164 do not
    assert lib.moe_step_workspace_size(163, 2048, 512, 512, 10) <= sme.NOALLOC_SCRATCH_BYTES
    assert lib.moe_step_workspace_size(164, 2048, 512, 512, 10) > sme.NOALLOC_SCRATCH_BYTES
    assert _noalloc(lib, T=164, H=2048, I=512, E=512, k=10) == 7
    assert _noalloc(lib, T=4096, H=2048, I=512, E=512, k=10) == 7


def test_per_route_host_checks(lib):
    """moe_expert_ffn_per_route: shape, envelope, pointer and workspace checks
    before any launch."""
    f = lib.moe_expert_ffn_per_route

    def call(T=4, H=256, I=128, E=8, k=2, ws=1 << 20, null_at=None):
        ptrs = [A] * 10
        if null_at is not None:
            ptrs[null_at] = None
        return f(*ptrs, T, H, I, E, k, A, ctypes.c_size_t(ws), A, None)
    assert call(k=9) == 2
    assert call(H=48) == 2
    assert call(H=8192) == 3
    assert call(T=0) == 0
    assert call(null_at=8) == 1                      # topk_idx
    need = lib.moe_expert_ffn_workspace_size(4, 256, 128, 8, 2)
    assert call(ws=need - 1) == 5


def test_router_route_bucket_host_checks(lib):
    """moe_router_route_bucket: every check before any launch."""
    f = lib.moe_router_route_bucket

    def call(T=4, H=64, E=8, k=2, counter=A, bias=None, x=A):
        return f(x, A, bias, T, H, E, k, A, A, A, *([A] * 6), counter, None)
    assert call(H=60) == 2              # H not a multiple of 8
    assert call(k=9) == 2               # k > E
    assert call(E=2048) == 3            # E beyond the envelope
    assert call(H=8192) == 3            # H beyond the envelope
    assert call(T=0, x=None) == 0       # T = 0: nothing launched
    assert call(counter=None) == 1
    assert call(x=None) == 1
    assert call(counter=P(260)) == 4
    assert call(bias=P(8)) == 4
