"""The C ABI library on the CPU: it loads, exports every symbol the header
declares, and rejects bad arguments on the host before any HIP call (no
compute call is made here: there is no GPU in this container)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vimscan.h")


@pytest.fixture(scope="module")
def nat():
    from vision_mamba_selective_amd import _native
    return _native


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_header_declares_the_entry_points():
    names = header_functions()
    for required in ("vim_scan_bidir", "vim_scan_bidir_conv", "vim_scan_bidir_grad",
                     "vmamba_cross_scan4",
                     "s6_scan_1d", "vs_strerror",
                     "vs_last_error", "vs_abi_version", "vs_workspace_bytes"):
        assert required in names


def test_library_exports_every_declared_symbol(nat):
    raw = ctypes.CDLL(nat.LIB_PATH)
    for name in header_functions():
        assert hasattr(raw, name), name
    assert set(nat.SIGNATURES) == set(header_functions())


def test_version_and_strerror(nat):
    assert nat.lib.vs_abi_version() == 1
    assert nat.lib.vs_strerror(0) == b"VS_OK"
    for code, name in [(-1, b"VS_ERR_NULL"), (-2, b"VS_ERR_SHAPE"), (-3, b"VS_ERR_DTYPE"),
                       (-4, b"VS_ERR_ALIGN"), (-5, b"VS_ERR_ALIAS"), (-6, b"VS_ERR_UNSUPPORTED"),
                       (-7, b"VS_ERR_HIP"), (-8, b"VS_ERR_WORKSPACE"), (-99, b"VS_ERR_UNKNOWN")]:
        assert nat.lib.vs_strerror(code) == name


def test_workspace_bytes(nat):
    f = nat.lib.vs_workspace_bytes
    assert f(0, 8, 768, 4097, nat.VS_BF16) == 8 * 768 * 4097 * 4
    e = 8 * 384 * 4096
    assert f(1, 8, 384, 4096, nat.VS_BF16) == 2 * e * 4 + 2 * e * 2   # 2 merge buffers, u^T, delta^T
    assert f(1, 8, 384, 4096, nat.VS_F32) == e * 4 + 2 * e * 4        # y is the first buffer
    assert f(0, 8, 768, 4097, nat.VS_F32) == 0          # fp32 y holds the partial sums
    assert f(2, 8, 768, 4097, nat.VS_F32) == 0
    assert f(0, 8, 768, 4097, 5) == 0
    assert f(2, 8, 768, 4097, nat.VS_BF16) == 0
    assert f(0, 0, 768, 4097, nat.VS_BF16) == 0


# Fake, well-aligned, non-overlapping device addresses: validation must reject
# the call before it dereferences anything or touches the HIP runtime.
MB = 1 << 20
BASE = 1 << 40


def fake(i):
    return BASE + i * 256 * MB


def far(i):
    return BASE + i * (8 << 30)    # 8 GiB apart: no overlap at the largest sizes


def vim_call(nat, **kw):
    a = dict(batch=2, dim=8, dstate=16, L=33, dtype=nat.VS_BF16, u=fake(0), delta=fake(1),
             z=fake(2), B=fake(3), C=fake(4), A=fake(5), D=fake(6), bias=fake(7), sp=1,
             y=fake(8), ws=fake(9), ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return nat.lib.vim_scan_bidir(a["batch"], a["dim"], a["dstate"], a["L"], a["dtype"], a["u"],
                                  a["delta"], a["z"], a["B"], a["C"], a["A"], a["D"], a["bias"],
                                  a["sp"], a["y"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), -3),
    (dict(batch=0), -2),
    (dict(dim=-1), -2),
    (dict(L=0), -2),
    (dict(dstate=0), -2),
    (dict(dstate=17), -6),
    (dict(u=None), -1),
    (dict(B=None), -1),
    (dict(A=None), -1),
    (dict(y=None), -1),
    (dict(u=fake(0) + 1), -4),
    (dict(dtype=0, u=fake(0) + 2), -4),
    (dict(A=fake(5) + 2), -4),
    (dict(y=fake(0) + 64), -5),           # y inside u
    (dict(y=fake(3) - 64), -5),           # y runs into B
    (dict(ws=None), -8),
    (dict(ws_bytes=100), -8),
    (dict(ws=fake(8) + 128), -5),         # workspace overlaps y
    (dict(ws=fake(1)), -5),               # workspace overlaps delta
])
def test_vim_validation(nat, kw, code):
    assert vim_call(nat, **kw) == code
    assert nat.lib.vs_last_error() != b""


def test_dirs_validation(nat):
    """vim_scan_bidir_dirs: u and delta hold two copies, B and C two
    direction blocks, so both the size limit and the overlap checks see
    twice the bytes of vim_scan_bidir."""
    f = nat.lib.vim_scan_bidir_dirs

    def call(batch=2, dim=8, L=33, u=fake(0), delta=fake(1), B=fake(3), y=fake(8), ptr=fake):
        return f(batch, dim, 16, L, nat.VS_BF16, u, delta, None, B, ptr(4), ptr(5), None, None, 1,
                 y, ptr(9), 1 << 20, None)
    act = 2 * 8 * 33 * 2                            # bytes of one bf16 copy
    # (every call here fails validation, so no kernel is ever launched)
    assert call(y=fake(0) + act + 64) == -5         # y inside u's second copy
    # the same y is outside vim_scan_bidir's u: that call gets as far as the
    # workspace check
    assert vim_call(nat, y=fake(0) + act + 64, ws=None) == -8
    bc = 2 * 16 * 33 * 2                            # bytes of one direction's B block
    assert call(y=fake(3) + bc + 64) == -5          # y inside B's backward block
    L = 1 << 29                                     # 2 * batch * dim * L reaches 2^30
    assert call(batch=1, dim=1, L=L, u=far(0), delta=far(1), B=far(3), y=far(8), ptr=far) == -6


def test_flag_validation(nat):
    """Bits other than VS_FLAG_SOFTPLUS | VS_FLAG_ZOH are refused, and the
    gradient takes VS_FLAG_SOFTPLUS only (both before any launch)."""
    assert vim_call(nat, sp=4) == -6
    assert vim_call(nat, sp=3, ws=None) == -8          # both known flags get past the check
    f = nat.lib.vim_scan_bidir_grad
    need = nat.lib.vs_workspace_bytes(3, 2, 8, 33, nat.VS_BF16)
    assert f(2, 8, 16, 33, nat.VS_BF16, fake(0), fake(1), fake(2), fake(3), fake(4), fake(5),
             None, None, 3, fake(6), fake(7), fake(8), fake(9), fake(10), fake(11), fake(12),
             fake(13), fake(14), fake(15), need, None) == -6


def test_projection_validation(nat):
    """Every call below fails validation, so no kernel is launched."""
    x, o = nat.lib.vim_x_proj, nat.lib.vim_out_proj
    xp = lambda **k: x(k.get("batch", 2), k.get("dim", 64), k.get("N", 16), k.get("L", 37),
                       k.get("dtype", nat.VS_BF16), k.get("u", fake(0)), k.get("W", fake(1)),
                       k.get("B", fake(2)), k.get("C", fake(3)), k.get("dt", fake(4)), None)
    assert xp(dtype=nat.VS_F32) == -6           # bf16 only
    assert xp(dtype=5) == -3
    assert xp(N=17) == -6
    assert xp(N=0) == -2
    assert xp(u=None) == -1
    assert xp(dt=fake(4) + 2) == -4             # fp32 dt misaligned
    assert xp(B=fake(0) + 64) == -5             # B inside u
    assert xp(C=fake(2) + 64) == -5             # C overlaps B
    op = lambda **k: o(k.get("batch", 2), 64, 48, 37, k.get("dtype", nat.VS_BF16),
                       k.get("y", fake(0)), k.get("W", fake(1)), k.get("bias", None),
                       k.get("res", None), k.get("out", fake(3)), None)
    assert op(dtype=nat.VS_F32) == -6
    assert op(W=None) == -1
    assert op(out=fake(0) + 2) == -5            # out inside y
    assert op(res=fake(3) + 2) == -5            # partial overlap with the residual
    assert op(batch=0) == -2
    d = nat.lib.vim_dt_proj
    assert d(2, 8, 37, nat.VS_F32, fake(0), fake(1), fake(2), None) == -6
    assert d(2, 70000, 37, nat.VS_BF16, fake(0), fake(1), fake(2), None) == -6
    assert d(2, 8, 37, nat.VS_BF16, fake(0), fake(1), fake(0) + 8, None) == -5


def test_cross4_validation(nat):
    f = nat.lib.vmamba_cross_scan4
    args = [fake(0), fake(1), None, fake(3), fake(4), fake(5), None, None, 1, fake(8), fake(9),
            1 << 30, None]
    assert f(1, 4, 16, 0, 5, nat.VS_F32, *args) == -2
    assert f(1, 4, 16, 5, -1, nat.VS_F32, *args) == -2
    assert f(1, 4, 32, 5, 7, nat.VS_F32, *args) == -6
    assert f(1, 4, 16, 5, 7, 9, *args) == -3
    # the cross-scan needs a workspace even for fp32 (its second merge buffer)
    no_ws = args[:10] + [None, 0, None]
    assert f(1, 4, 16, 5, 7, nat.VS_F32, *no_ws) == -8
    assert f(1, 4, 16, 1 << 21, 7, nat.VS_F32, *args) == -2


def test_element_limit(nat):
    """Activation tensors of 2^30 elements or more are refused (the kernels
    address them with 32-bit byte offsets); one element fewer is accepted
    by validation (checked here up to the workspace test only)."""
    big = dict(u=far(0), delta=far(1), z=far(2), B=far(3), C=far(4), A=far(5), D=far(6),
               bias=far(7), y=far(8), ws=far(9), ws_bytes=1 << 33)
    assert vim_call(nat, batch=1, dim=16384, L=65536, **big) == -6
    big["ws"] = None
    assert vim_call(nat, batch=1, dim=16384, L=65535, **big) == -8


def test_conv_validation(nat):
    f = nat.lib.vim_scan_bidir_conv
    def call(**kw):
        a = dict(x=fake(0), w=fake(10), b=None, y=fake(8), ws=fake(9))
        a.update(kw)
        return f(2, 8, 16, 33, nat.VS_BF16, a["x"], a["w"], a["b"], fake(1), fake(2), fake(3),
                 fake(4), fake(5), fake(6), fake(7), 1, a["y"], a["ws"], 1 << 20, None)
    assert call(w=None) == -1
    assert call(w=fake(10) + 2) == -4
    assert call(b=fake(11) + 1) == -4
    assert call(y=fake(10) - 64) == -5          # y runs into conv_w
    assert call(x=None) == -1


def test_grad_validation(nat):
    f = nat.lib.vim_scan_bidir_grad
    need = nat.lib.vs_workspace_bytes(3, 2, 8, 33, nat.VS_BF16)
    assert need > 0

    def call(**kw):
        a = dict(u=fake(0), dl=fake(1), z=fake(2), B=fake(3), C=fake(4), A=fake(5), D=None,
                 bias=None, dy=fake(6), du=fake(7), dd=fake(8), dz=fake(9), dB=fake(10),
                 dC=fake(11), dA=fake(12), dD=fake(13), db=fake(14), ws=fake(15), wsb=need)
        a.update(kw)
        return f(2, 8, 16, 33, nat.VS_BF16, a["u"], a["dl"], a["z"], a["B"], a["C"], a["A"],
                 a["D"], a["bias"], 1, a["dy"], a["du"], a["dd"], a["dz"], a["dB"], a["dC"],
                 a["dA"], a["dD"], a["db"], a["ws"], a["wsb"], None)
    assert call(dy=None) == -1
    assert call(dB=None) == -1
    assert call(dz=None) == -1                   # z given: dz required
    assert call(wsb=need - 1) == -8
    assert call(du=fake(0) + 64) == -5           # du inside u
    assert call(dC=fake(10) + 128) == -5         # dC overlaps dB
    assert call(dA=fake(12) + 2) == -4
    # the gradient caps the sequence at 2^26 tokens (one batch row, one channel)
    L = (1 << 26) + 1
    big = nat.lib.vs_workspace_bytes(3, 1, 1, L, nat.VS_F32)
    assert f(1, 1, 16, L, nat.VS_F32, far(0), far(1), None, far(2), far(3), far(4), None, None,
             1, far(5), far(6), far(7), None, far(8), far(9), far(10), far(11), far(12), far(13),
             big, None) == -6


def test_1d_validation(nat):
    f = nat.lib.s6_scan_1d
    assert f(1, 4, 16, 10, nat.VS_F32, 0, None, fake(1), None, fake(3), fake(4), fake(5),
             None, None, 1, fake(8), None) == -1
    assert f(1, 4, 20, 10, nat.VS_F32, 0, fake(0), fake(1), None, fake(3), fake(4), fake(5),
             None, None, 1, fake(8), None) == -6


def test_python_binding_checks_shapes_before_calling():
    import torch
    from vision_mamba_selective_amd import scan
    u = torch.zeros(1, 4, 10)
    with pytest.raises(ValueError):
        scan.vim_scan_bidir(u, u, None, torch.zeros(1, 16, 9), torch.zeros(1, 16, 10),
                            torch.zeros(2, 4, 16))
    with pytest.raises(TypeError):
        scan.vim_scan_bidir(u.double(), u, None, torch.zeros(1, 16, 10), torch.zeros(1, 16, 10),
                            torch.zeros(2, 4, 16))


def test_last_error_is_per_thread(nat):
    """The detailed error text is kept per calling thread: a validation
    failure in one thread leaves another thread's text empty."""
    import threading
    seen = {}

    def bad():
        seen["bad"] = (vim_call(nat, batch=0), nat.lib.vs_last_error())

    def fresh():
        seen["fresh"] = nat.lib.vs_last_error()

    for fn in (bad, fresh):
        t = threading.Thread(target=fn)
        t.start()
        t.join()
    assert seen["bad"][0] == -2 and seen["bad"][1] != b""
    assert seen["fresh"] == b""


def test_noalloc_refuses_sizes_beyond_its_buffer(nat):
    """vim_scan_bidir_noalloc checks the size against its static buffer
    before any HIP call: bf16 with batch*dim*L above VS_NOALLOC_MAX_ELEMS is
    VS_ERR_UNSUPPORTED with a message naming the limit."""
    f = nat.lib.vim_scan_bidir_noalloc
    big = (8, 1024, 4097)                 # 33.6 M elements > 2^25
    assert big[0] * big[1] * big[2] > nat.VS_NOALLOC_MAX_ELEMS
    rc = f(*big[:2], 16, big[2], nat.VS_BF16, far(0), far(1), far(2), far(3), far(4), far(5),
           far(6), far(7), 1, far(8), None)
    assert rc == -6
    assert b"no-allocation maximum" in nat.lib.vs_last_error()
    rc = f(2, 8, 16, 33, nat.VS_BF16, None, far(1), far(2), far(3), far(4), far(5), far(6),
           far(7), 1, far(8), None)
    assert rc == -1


def test_chunked_refuses_what_it_does_not_chunk(nat):
    """vim_scan_bidir_chunked: a negative chunk count is a shape error, and
    chunks with the exact hold are not supported; both before any HIP
    call."""
    f = nat.lib.vim_scan_bidir_chunked
    args = [2, 8, 16, 333, nat.VS_BF16, far(0), far(1), far(2), far(3), far(4), far(5), far(6),
            far(7)]
    rc = f(*args, 1, -1, far(8), far(9), 1 << 40, None)
    assert rc == -2
    rc = f(*args, 3, 2, far(8), far(9), 1 << 40, None)           # VS_FLAG_SOFTPLUS | VS_FLAG_ZOH
    assert rc == -6
    assert b"chunks" in nat.lib.vs_last_error()
    rc = f(*args, 1, 2, far(8), None, 0, None)                   # bf16 needs the workspace
    assert rc == -8


def test_saved_pair_sizes_and_refusals(nat):
    """The saved-state buffer and the saved gradient's workspace split the
    gradient's workspace exactly; bad arguments are refused before any HIP
    call: a short or missing saved buffer, the exact hold, a saved buffer
    that overlaps an output, over-long sequences."""
    ws = nat.lib.vs_workspace_bytes
    for dims in ((2, 8, 33), (8, 768, 4097), (1, 1, 1)):
        full = ws(nat.VS_OP_VIM_GRAD, *dims, nat.VS_BF16)
        sv = ws(nat.VS_OP_VIM_SAVED, *dims, nat.VS_BF16)
        rest = ws(nat.VS_OP_VIM_GRAD_SAVED, *dims, nat.VS_BF16)
        assert sv > 0 and rest > 0 and sv + rest == full
        e = dims[0] * dims[1] * dims[2]
        assert sv >= 4 * e                          # at least the fp32 ungated output
    assert ws(6, 2, 8, 33, nat.VS_BF16) == 0          # unknown operation
    sv = ws(nat.VS_OP_VIM_SAVED, 2, 8, 33, nat.VS_BF16)
    rest = ws(nat.VS_OP_VIM_GRAD_SAVED, 2, 8, 33, nat.VS_BF16)

    fwd = nat.lib.vim_scan_bidir_fwd_saved
    fargs = [2, 8, 16, 33, nat.VS_BF16, fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), None, None]
    assert fwd(*fargs, 1, fake(6), fake(7), sv - 1, None) == -8
    assert b"VS_OP_VIM_SAVED" in nat.lib.vs_last_error()
    assert fwd(*fargs, 1, fake(6), None, sv, None) == -8
    assert fwd(*fargs, 3, fake(6), fake(7), sv, None) == -6         # VS_FLAG_ZOH
    assert fwd(*fargs, 1, fake(6), fake(0) + 64, sv, None) == -5    # saved inside u

    g = nat.lib.vim_scan_bidir_grad_saved

    def call(**kw):
        a = dict(sv=fake(16), svb=sv, dy=fake(6), du=fake(7), dd=fake(8), dz=fake(9), dB=fake(10),
                 dC=fake(11), dA=fake(12), dD=fake(13), db=fake(14), ws=fake(15), wsb=rest, sp=1)
        a.update(kw)
        return g(2, 8, 16, 33, nat.VS_BF16, fake(0), fake(1), fake(2), fake(3), fake(4), fake(5),
                 None, None, a["sp"], a["sv"], a["svb"], a["dy"], a["du"], a["dd"], a["dz"], a["dB"],
                 a["dC"], a["dA"], a["dD"], a["db"], a["ws"], a["wsb"], None)
    assert call(sv=None) == -1
    assert call(svb=sv - 1) == -8
    assert call(wsb=rest - 1) == -8
    assert call(sp=3) == -6
    assert call(du=fake(16) + 64) == -5              # an output inside the saved buffer
    assert call(ws=fake(16)) == -5                   # the workspace on the saved buffer
    # both cap the sequence at 2^26 tokens (one batch row, one channel)
    L = (1 << 26) + 1
    big = ws(nat.VS_OP_VIM_SAVED, 1, 1, L, nat.VS_F32)
    assert fwd(1, 1, 16, L, nat.VS_F32, far(0), far(1), None, far(2), far(3), far(4), None, None,
               1, far(5), far(6), big, None) == -6
