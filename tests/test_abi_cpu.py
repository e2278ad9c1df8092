"""The C-ABI library on the host: it loads, exports every symbol the header
declares, and rejects bad arguments before anything reaches the GPU.

None of these calls launches a kernel: each one fails validation (or only
computes a size), which happens before any HIP call.
"""
import ctypes
import os
import re

import pytest

from cross_token_gated_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tango.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from cross_token_gated_amd import build
        build.build(verbose=False)
    return _lib.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, re.M)))


def test_header_and_binding_agree():
    assert header_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    version = int(re.search(r"#define TANGO_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.tango_version() == version
    for code in range(-8, 1):
        assert lib.tango_status_string(code).decode().startswith(_lib.STATUS[code])


def shape(**kw):
    base = dict(batch=1, seq_len=256, d_model=512, d_gate=2048, n_heads=1, head_dim=128, dtype=1,
                io_dtype=1, rope_base=10000.0, rms_eps=1e-6)
    base.update(kw)
    return _lib.Shape(**base)


FAKE = 0x7F0000000000   # never dereferenced: every call below fails validation first


def weights(**kw):
    base = dict(w_g=FAKE + 0x10000000, w_v=FAKE + 0x20000000, w_q=FAKE + 0x30000000,
                w_k=FAKE + 0x31000000, w_o=FAKE + 0x40000000, rms_gain=None,
                theta=FAKE + 0x50000000, null_bias=None)
    base.update(kw)
    return _lib.Weights(**base)


def call_tango(lib, s, w=None, x=FAKE, out=FAKE + 0x60000000, ws=FAKE + 0x80000000, nbytes=None):
    w = weights() if w is None else w
    if nbytes is None:
        nbytes = lib.tango_workspace_size(ctypes.byref(s))
    return lib.tango_block_fwd(ctypes.byref(s), ctypes.byref(w), x, out, ws, nbytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), "TANGO_ERR_DTYPE"),
    (dict(io_dtype=-1), "TANGO_ERR_DTYPE"),
    (dict(batch=0), "TANGO_ERR_SHAPE"),
    (dict(seq_len=0), "TANGO_ERR_SHAPE"),
    (dict(d_gate=2048, n_heads=3), "TANGO_ERR_SHAPE"),
    (dict(rms_eps=0.0), "TANGO_ERR_SHAPE"),
    (dict(rope_base=-1.0), "TANGO_ERR_SHAPE"),
    (dict(operand_parts=3), "TANGO_ERR_SHAPE"),
    (dict(operand_parts=-1), "TANGO_ERR_SHAPE"),
    (dict(operand_parts=2, dtype=0, io_dtype=0), "TANGO_ERR_SHAPE"),
    (dict(d_model=448), "TANGO_ERR_UNSUPPORTED"),
    (dict(head_dim=96), "TANGO_ERR_UNSUPPORTED"),
    (dict(d_gate=2080), "TANGO_ERR_UNSUPPORTED"),
    (dict(d_gate=1024 + 64, n_heads=17), "TANGO_ERR_UNSUPPORTED"),
    (dict(batch=1 << 20, seq_len=1 << 10), "TANGO_ERR_UNSUPPORTED"),
])
def test_shape_errors(lib, kw, code):
    s = shape(**kw)
    assert call_tango(lib, s, nbytes=1 << 40) == _lib.STATUS_CODE[code]
    assert lib.tango_last_error().decode()
    assert lib.tango_workspace_size(ctypes.byref(s)) == 0


def test_null_pointers(lib):
    s = shape()
    assert lib.tango_block_fwd(None, None, None, None, None, 0, None) == -1
    assert call_tango(lib, s, x=None) == -1
    assert call_tango(lib, s, ws=None) == -1
    assert call_tango(lib, s, w=weights(w_o=None)) == -1
    assert call_tango(lib, s, w=weights(theta=None)) == -1


def test_workspace_too_small(lib):
    s = shape()
    n = lib.tango_workspace_size(ctypes.byref(s))
    assert n > 0
    assert call_tango(lib, s, nbytes=n - 1) == _lib.STATUS_CODE["TANGO_ERR_WORKSPACE"]


def test_alignment_and_aliasing(lib):
    s = shape()
    assert call_tango(lib, s, x=FAKE + 8) == _lib.STATUS_CODE["TANGO_ERR_ALIGN"]
    assert call_tango(lib, s, out=FAKE + 0x10000000 + 256) == _lib.STATUS_CODE["TANGO_ERR_ALIAS"]  # out over w_g
    n = lib.tango_workspace_size(ctypes.byref(s))
    assert call_tango(lib, s, ws=FAKE + 4096, nbytes=n) == _lib.STATUS_CODE["TANGO_ERR_ALIAS"]    # ws over x
    assert call_tango(lib, s, out=FAKE + 1024) == _lib.STATUS_CODE["TANGO_ERR_ALIAS"]   # partial overlap with x


@pytest.mark.parametrize("args,code", [
    ((0, 128, 128), "TANGO_ERR_SHAPE"),         # window < 1
    ((256, 64, 128), "TANGO_ERR_SHAPE"),        # phi_dim != head_dim
    ((256, 128, 32), "TANGO_ERR_UNSUPPORTED"),  # chunk
    ((192, 128, 128), "TANGO_ERR_UNSUPPORTED"), # window % chunk
])
def test_wango_argument_errors(lib, args, code):
    s = shape()
    w = weights()
    window, phi, chunk = args
    assert lib.wango_workspace_size(ctypes.byref(s), window, phi, chunk) == 0
    rc = lib.wango_block_fwd(ctypes.byref(s), ctypes.byref(w), window, phi, chunk, FAKE,
                             FAKE + 0x60000000, FAKE + 0x80000000, 1 << 40, None)
    assert rc == _lib.STATUS_CODE[code]


def test_workspace_sizes_cover_the_layout(lib):
    # TANGO at T=8192: gates, features, gbar (3 x 32 MiB), q/k (2 x 2 MiB),
    # and the float32 split partials
    n = lib.tango_workspace_size(ctypes.byref(shape(seq_len=8192)))
    assert n >= 3 * 8192 * 2048 * 2 + 2 * 8192 * 128 * 2
    # gates, gbar and features in bf16; v in bf16 with one operand part, float32 with two
    n5 = lib.wango_workspace_size(ctypes.byref(shape(batch=2, seq_len=65536)), 512, 128, 128)
    assert n5 >= 2 * 65536 * 2048 * (3 * 2 + 2)
    n5_two = lib.wango_workspace_size(ctypes.byref(shape(batch=2, seq_len=65536, operand_parts=2)), 512, 128, 128)
    assert n5_two >= 2 * 65536 * 2048 * (3 * 2 + 4) and n5_two - n5 >= 2 * 65536 * 2048 * 2


def test_stage_entry_points_validate(lib):
    s = shape()
    w = weights()
    assert lib.tango_stage_proj(ctypes.byref(s), ctypes.byref(w), None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                1 << 40, None) == -1
    n = lib.tango_proj_workspace_size(ctypes.byref(s))
    assert n > 0
    assert lib.tango_stage_proj(ctypes.byref(s), ctypes.byref(w), FAKE, FAKE + 0x1000000,
                                FAKE + 0x2000000, FAKE + 0x3000000, FAKE + 0x4000000,
                                FAKE + 0x5000000, n - 1, None) == -6
    assert lib.tango_stage_aggregate(ctypes.byref(s), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == -6
    assert lib.tango_stage_out(ctypes.byref(shape(dtype=3)), FAKE, FAKE, FAKE, FAKE, FAKE, None) == -3
    assert lib.wango_stage_proj(ctypes.byref(s), ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                FAKE, 1 << 40, None) == -1
    assert lib.wango_stage_scan(ctypes.byref(s), 0, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == -2
    assert lib.wango_stage_scan(ctypes.byref(s), 256, 96, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == -5
    assert lib.wango_stage_band(ctypes.byref(s), FAKE, None, 0, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -2


def test_decode_entry_points_validate(lib):
    s = shape(batch=16, seq_len=8448)
    w = weights()
    ns, nw = lib.tango_decode_state_size(ctypes.byref(s)), lib.tango_decode_workspace_size(ctypes.byref(s))
    # state: keys and gates of every position of every sequence
    assert ns >= 16 * 8448 * (128 + 2048) * 2 and nw > 0
    pos = FAKE + 0x90000000
    args = lambda **kw: dict(dict(pos=pos, x=FAKE, out=FAKE + 0x60000000, st=FAKE + 0x100000000, ns=ns,  # noqa: E731
                                  ws=FAKE + 0x200000000, nw=nw), **kw)

    def call(**kw):
        a = args(**kw)
        return lib.tango_decode_step(ctypes.byref(s), ctypes.byref(w), a["pos"], a["x"], a["out"], a["st"],
                                     a["ns"], a["ws"], a["nw"], None)
    assert call(pos=None) == -1
    assert call(st=None) == -1
    assert call(ns=ns - 1) == -6
    assert call(nw=nw - 1) == -6
    assert call(pos=pos + 2) == -4                    # pos needs 4-byte alignment only
    assert call(out=FAKE + 0x100000000 + 4096) == -7  # out inside the state
    assert call(st=FAKE + 0x10000000) == -7           # state over w_g
    # WANGO: window + 1 ring rows, S and z
    nsw = lib.wango_decode_state_size(ctypes.byref(shape(batch=64)), 256, 128)
    assert nsw >= 64 * 257 * (128 + 2048) * 2 + 64 * 128 * 2048 * 4
    assert lib.wango_decode_state_size(ctypes.byref(shape()), 0, 128) == 0
    assert lib.wango_decode_state_size(ctypes.byref(shape()), 256, 64) == 0
    assert lib.wango_decode_state_size(ctypes.byref(shape()), 4096, 128) == 0
    rc = lib.wango_decode_step(ctypes.byref(shape()), ctypes.byref(w), 4096, 128, pos, FAKE, FAKE + 0x60000000,
                               FAKE + 0x100000000, 1 << 40, FAKE + 0x200000000, 1 << 40, None)
    assert rc == _lib.STATUS_CODE["TANGO_ERR_UNSUPPORTED"]
    assert lib.tango_decode_state_size(ctypes.byref(shape(d_gate=64 * 33, n_heads=33, head_dim=32))) == 0


def test_stack_entry_point_validates(lib):
    """tango_stack_fwd checks every set and application before the first launch
    (the fake pointers would fault if anything ran)."""
    S3 = _lib.Shape * 3
    W3 = _lib.Weights * 3
    shapes = S3(shape(d_gate=704), shape(d_gate=640), shape(d_gate=704))
    need = lib.tango_stack_workspace_size(shapes, 3)
    assert need == max(lib.tango_workspace_size(ctypes.byref(shapes[k])) for k in range(3)) > 0
    assert lib.tango_stack_workspace_size(shapes, 0) == 0
    assert lib.tango_stack_workspace_size(S3(shape(), shape(d_gate=100), shape()), 3) == 0
    sets = W3(weights(), weights(w_g=FAKE + 0x11000000, w_v=FAKE + 0x21000000, w_o=FAKE + 0x41000000),
              weights(w_g=FAKE + 0x12000000, w_v=FAKE + 0x22000000, w_o=FAKE + 0x42000000))
    sched = (ctypes.c_int32 * 4)(0, 1, 1, 2)
    ws = FAKE + 0x80000000

    def run(sh=shapes, st=sets, n_sets=3, sc=sched, n_apps=4, x=FAKE, out=FAKE + 0x60000000, nbytes=need):
        return lib.tango_stack_fwd(sh, st, n_sets, sc, n_apps, x, out, ws, nbytes, None)

    code = _lib.STATUS_CODE
    assert run(sc=(ctypes.c_int32 * 4)(0, 1, 3, 2)) == code["TANGO_ERR_SHAPE"]     # set index out of range
    assert run(sc=(ctypes.c_int32 * 4)(0, -1, 1, 2)) == code["TANGO_ERR_SHAPE"]
    assert run(n_apps=0) == code["TANGO_ERR_SHAPE"]
    assert run(n_sets=0) == code["TANGO_ERR_SHAPE"]
    assert lib.tango_stack_fwd(shapes, sets, 3, None, 4, FAKE, FAKE + 0x60000000, ws, need, None) == -1
    assert run(sh=S3(shape(d_gate=704), shape(d_gate=640, seq_len=128), shape(d_gate=704))) == \
        code["TANGO_ERR_SHAPE"]                                                    # stream shapes differ
    assert run(sh=S3(shape(d_gate=704), shape(d_gate=640, io_dtype=0), shape(d_gate=704))) == \
        code["TANGO_ERR_SHAPE"]
    assert run(nbytes=need - 1) == code["TANGO_ERR_WORKSPACE"]
    assert run(x=None) == -1
    # set 2's W_o overlaps the output: caught before application 0 runs
    bad = W3(sets[0], sets[1], weights(w_g=FAKE + 0x12000000, w_v=FAKE + 0x22000000, w_o=FAKE + 0x60000000))
    assert run(st=bad) == code["TANGO_ERR_ALIAS"]
    assert run(st=W3(sets[0], weights(theta=None), sets[2])) == -1


def test_binding_argument_counts_match_the_header(lib):
    """Every ctypes signature takes as many arguments as the header's
    declaration (a missing one would shift the stream into another slot)."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name in header_functions():
        m = re.search(r"\b" + name + r"\s*\(([^)]*)\)", text)
        params = m.group(1).strip()
        n = 0 if params in ("", "void") else params.count(",") + 1
        assert len(getattr(lib, name).argtypes) == n, name


def test_noalloc_decode_validates_before_touching_the_device(lib):
    """wango_decode_step_noalloc checks every argument, and that the step fits
    the library's scratch array, before it takes the array (the fake pointers
    would fault if anything ran, and there is no device here to take it from)."""
    code = _lib.STATUS_CODE
    w = weights()
    s = shape(batch=64, d_gate=2048, n_heads=2, head_dim=64)
    ns = lib.wango_decode_state_size(ctypes.byref(s), 256, 64)
    need = lib.wango_decode_workspace_size(ctypes.byref(s), 256, 64)
    assert 0 < need <= _lib.NOALLOC_SCRATCH_BYTES
    pos = FAKE + 0x90000000

    def call(sh=s, window=256, phi=64, p=pos, x=FAKE, out=FAKE + 0x60000000, st=FAKE + 0x100000000, n=ns):
        return lib.wango_decode_step_noalloc(ctypes.byref(sh), ctypes.byref(w), window, phi, p, x, out, st, n, None)
    assert call(p=None) == code["TANGO_ERR_NULL"]
    assert call(st=None) == code["TANGO_ERR_NULL"]
    assert call(n=ns - 1) == code["TANGO_ERR_WORKSPACE"]
    assert call(phi=32) == code["TANGO_ERR_SHAPE"]
    assert call(window=0) == code["TANGO_ERR_SHAPE"]
    assert call(out=FAKE + 0x100000000 + 4096) == code["TANGO_ERR_ALIAS"]
    # a batch whose scratch exceeds the array is refused, with the sizes named
    big = shape(batch=4096, d_gate=2048, n_heads=2, head_dim=64)
    assert lib.wango_decode_workspace_size(ctypes.byref(big), 256, 64) > _lib.NOALLOC_SCRATCH_BYTES
    nsb = lib.wango_decode_state_size(ctypes.byref(big), 256, 64)
    assert call(sh=big, n=nsb) == code["TANGO_ERR_WORKSPACE"]
    assert b"TANGO_NOALLOC_SCRATCH_BYTES" in lib.tango_last_error()
    m = re.search(r"#define TANGO_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES


def test_operand_parts_size_the_projection_scratch(lib):
    # two bf16 parts of h * gain need one more [rows, d] bf16 array than one part;
    # 0 reads as one part
    one = lib.tango_proj_workspace_size(ctypes.byref(shape(operand_parts=1)))
    two = lib.tango_proj_workspace_size(ctypes.byref(shape(operand_parts=2)))
    assert lib.tango_proj_workspace_size(ctypes.byref(shape(operand_parts=0))) == one
    assert two - one >= 256 * 512 * 2
    assert lib.tango_workspace_size(ctypes.byref(shape(operand_parts=2))) > \
        lib.tango_workspace_size(ctypes.byref(shape(operand_parts=1)))
