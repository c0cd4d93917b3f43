"""C-ABI checks that need no GPU: exported symbols, host validation, error
codes and the argument checks every entry point performs before it enqueues
anything.  No compute call is made here."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from oracle import ref

paro = pytest.importorskip("rotation_int4_weight_amd")
from rotation_int4_weight_amd import _lib  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared(header):
    """Function names declared in a C header (return type, name, '(')."""
    with open(os.path.join(ROOT, "include", header)) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b((?:paro)_\w+)\s*\(", text, flags=re.M)))


def test_libparo_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared("paro.h")
    assert "paro_w4a16_linear" in names and "paro_scale_rotate" in names
    assert set(_lib.EXPORTS) == set(names)
    for n in names:
        assert getattr(lib, n) is not None
    assert lib.paro_abi_version() == 5


def test_oracle_exports_every_declared_symbol():
    lib = ref.load()
    names = declared("paro_ref.h")
    assert "paro_linear_ref_check" in names
    for n in names:
        assert getattr(lib, n) is not None


def test_oracle_and_gpu_library_share_no_code():
    """The checker and the product are separate libraries with no shared symbol."""
    lib_names = set(declared("paro.h"))
    ref_names = set(declared("paro_ref.h"))
    assert not (lib_names & ref_names)
    with open(os.path.join(ROOT, "oracle", "paro_ref.c")) as f:
        src = f.read()
    assert "paro.h" not in src.replace("paro_ref.h", "")
    for fn in os.listdir(os.path.join(ROOT, "rotation_int4_weight_amd", "csrc")):
        with open(os.path.join(ROOT, "rotation_int4_weight_amd", "csrc", fn)) as f:
            s = f.read()
        assert "paro_ref" not in s and "oracle" not in s.lower()


def test_validate_layer_codes():
    L = synth.make_layer(400, 0, 256, 64)
    _lib.paro_validate_layer(L)
    bad = synth.make_layer(400, 0, 256, 64)
    bad.pairs[3, 200] = 300
    with pytest.raises(_lib.ParoError) as e:
        _lib.paro_validate_layer(bad)
    assert e.value.status == 6
    odd = synth.make_layer(400, 0, 256, 64)
    odd.group_size = 100
    with pytest.raises(_lib.ParoError) as e:
        _lib.paro_validate_layer(odd)
    assert e.value.status == 2


# -- argument checks of the GPU entry points (host side, nothing enqueued) --
#
# The descriptors below point at addresses no kernel ever sees: each case
# fails validation before any launch.  Guard: only run where no GPU exists.

def _no_gpu():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


needs_no_gpu = pytest.mark.skipif(not _no_gpu(), reason="host-only checks; run on a machine without a GPU")

FAKE = 0x100000  # 16-byte aligned, never dereferenced on the host


def fake_layer(I=256, O=64, G=128, krot=8, **over):
    f = dict(pairs=FAKE, theta=FAKE, channel_scales=FAKE, qweight=FAKE, qzeros=FAKE, scales=FAKE,
             bias=FAKE)
    f.update(over)
    return _lib.ParoLayerC(I, O, G, krot, f["pairs"], f["theta"], f["channel_scales"], f["qweight"],
                           f["qzeros"], f["scales"], f["bias"])


def lin(L, x=FAKE, xdt=0, tokens=4, y=FAKE * 2, ydt=0, ws=FAKE * 4, wsb=1 << 30, path=0):
    return _lib.load().paro_w4a16_linear_path(ctypes.byref(L), x, xdt, tokens, y, ydt, ws, wsb, None, path)


@needs_no_gpu
@pytest.mark.parametrize("case,code", [
    (dict(L=dict(G=16)), 5),             # G in {32, 64, 128} on the GPU
    (dict(L=dict(G=256, I=512)), 5),
    (dict(L=dict(G=64, I=320)), 5),      # 128-channel rotation blocks: I % 128 == 0
    (dict(L=dict(G=-1, I=256), path=1), 5),      # one group over the row: no fused decode
    (dict(L=dict(G=-1, I=16384 + 128)), 5),      # one group over the row: I <= 16384 (LDS)
    (dict(L=dict(G=256, I=256), path=1), 5),     # G == I is the same layer as G = -1
    (dict(L=dict(O=60)), 2),             # O % 8
    (dict(L=dict(G=100)), 2),            # G does not divide I
    (dict(L=dict(krot=0)), 2),
    (dict(L=dict(krot=65)), 5),
    (dict(L=dict(I=(1 << 22) + 128)), 5),  # 32-bit tile offsets of the prefill GEMM
    (dict(L=dict(pairs=0)), 1),
    (dict(L=dict(qweight=0)), 1),
    (dict(L=dict(qweight=FAKE + 4)), 4),
    (dict(L=dict(bias=FAKE + 4)), 4),    # bias is read 8 bytes at a time
    (dict(x=0), 1),
    (dict(x=FAKE + 2), 4),
    (dict(xdt=2), 3),                    # fp32 activations not accepted
    (dict(ydt=1), 3),                    # y must be x dtype or fp32
    (dict(tokens=-1), 2),
    (dict(tokens=17, path=1), 5),        # decode paths take <= 16 tokens
    (dict(tokens=17, path=2), 5),
    (dict(ws=0, path=3), 7),
    (dict(wsb=16, path=3), 7),
    (dict(ws=FAKE + 8, path=3), 4),
    (dict(y=FAKE + 64), 2),              # y overlaps x
    (dict(path=9), 2),
])
def test_linear_argument_checks(case, code):
    L = fake_layer(**{k: v for k, v in case.get("L", {}).items() if k in ("I", "O", "G", "krot")},
                   **{k: v for k, v in case.get("L", {}).items() if k not in ("I", "O", "G", "krot")})
    kw = {k: v for k, v in case.items() if k != "L"}
    rc = lin(L, **kw)
    assert rc == code, _lib.paro_last_error()
    assert _lib.paro_last_error()


@needs_no_gpu
def test_zero_tokens_returns_ok_without_touching_memory():
    assert lin(fake_layer(), tokens=0, x=0, y=0, ws=0, wsb=0) == 0
    lib = _lib.load()
    assert lib.paro_scale_rotate(ctypes.byref(fake_layer()), None, 0, 0, None, 0, None) == 0


@needs_no_gpu
def test_scale_rotate_and_dequant_argument_checks():
    lib = _lib.load()
    L = fake_layer()
    assert lib.paro_scale_rotate(ctypes.byref(L), FAKE, 0, 4, FAKE * 2, 7, None) == 3
    assert lib.paro_scale_rotate(ctypes.byref(L), FAKE, 0, 4, FAKE + 32, 0, None) == 2  # partial overlap
    assert lib.paro_scale_rotate(ctypes.byref(L), None, 0, 4, FAKE, 0, None) == 1
    assert lib.paro_w4_unpack_dequant(ctypes.byref(L), None, None, None, 0, None) == 0  # nothing requested
    assert lib.paro_w4_unpack_dequant(ctypes.byref(L), FAKE + 4, None, None, 0, None) == 4
    assert lib.paro_w4_unpack_dequant(ctypes.byref(fake_layer(scales=0)), FAKE, None, None, 0, None) == 1
    assert lib.paro_w4_unpack_dequant(ctypes.byref(L), None, None, FAKE, 9, None) == 3


def test_workspace_sizes_and_path_choice():
    lib = _lib.load()
    L = fake_layer(I=4096, O=4096)
    pick = lambda m: lib.paro_w4a16_linear_choose_path(ctypes.byref(L), m)
    assert pick(1) == 1 and pick(4) == 1 and pick(5) == 2 and pick(16) == 2 and pick(17) == 3
    wsb = lambda m, p: _lib.load().paro_w4a16_linear_workspace_bytes(ctypes.byref(L), m, 0, p)
    # prefill holds X_r (tokens * I * 2 bytes) after the fixed counter area
    assert wsb(2048, 3) - wsb(1024, 3) == 1024 * 4096 * 2
    assert wsb(1, 1) > 0 and wsb(4, 2) > wsb(4, 1)
    assert wsb(0, 1) == 0


@needs_no_gpu
def test_prerotated_argument_checks():
    lib = _lib.load()
    L = fake_layer(pairs=0, theta=0, channel_scales=0)  # rotation tensors are not needed
    call = lambda path, tokens=4, ws=FAKE * 4: lib.paro_w4a16_linear_prerotated(
        ctypes.byref(L), FAKE, 0, tokens, FAKE * 2, 0, ws, 1 << 30, None, path)
    assert call(1) == 2                        # fused path rotates itself
    assert call(2, tokens=17) == 5
    assert call(3, ws=0) == 7
    assert call(0, tokens=0) == 0


@needs_no_gpu
def test_tiled_entry_point_argument_checks():
    lib = _lib.load()
    L = fake_layer(I=256, O=64)
    assert lib.paro_tiled_bytes(ctypes.byref(L), 1) == 16 * 256 * 2
    assert lib.paro_tiled_bytes(ctypes.byref(L), 33) == 48 * 256 * 2
    assert lib.paro_tiled_bytes(ctypes.byref(L), 0) == 0
    assert lib.paro_rotation_matrix_bytes(ctypes.byref(L)) == 256 * 512
    mat = lambda dt=0, hl=FAKE * 8, L=L: lib.paro_rotation_matrix(ctypes.byref(L), dt, hl, None)
    assert mat(dt=2) == 3
    assert mat(hl=0) == 1
    assert mat(hl=FAKE * 8 + 4) == 4
    assert mat(L=fake_layer(pairs=0)) == 1
    assert mat(L=fake_layer(theta=0)) == 1
    assert mat(L=fake_layer(G=16)) == 5
    assert mat(L=fake_layer(G=-1)) == 5      # no dense form of one group over the whole row
    rot = lambda x=FAKE, dt=0, tokens=4, xt=FAKE * 2, hl=FAKE * 8, L=L: lib.paro_scale_rotate_tiled(
        ctypes.byref(L), hl, x, dt, tokens, xt, None)
    assert rot(dt=2) == 3                      # fp32 activations not accepted
    assert rot(x=0) == 1
    assert rot(hl=0) == 1
    assert rot(xt=FAKE * 2 + 8) == 4
    assert rot(hl=FAKE * 8 + 8) == 4
    assert rot(xt=FAKE + 64) == 2              # overlaps x
    assert rot(hl=FAKE * 2 + 4096) == 2        # x_t overlaps hl
    assert rot(tokens=0, x=0, xt=0, hl=0) == 0
    assert rot(tokens=-1) == 2
    assert rot(L=fake_layer(G=16)) == 5
    lin = lambda xt=FAKE, dt=0, tokens=4, y=FAKE * 4, ydt=0, L=L: lib.paro_w4a16_linear_tiled(
        ctypes.byref(L), xt, dt, tokens, y, ydt, None)
    assert lin(ydt=1) == 3                     # y must be x dtype or fp32
    assert lin(y=0) == 1
    assert lin(y=FAKE + 64) == 2               # overlaps the tiled x
    assert lin(L=fake_layer(qweight=0)) == 1
    assert lin(L=fake_layer(G=16)) == 5
    assert lin(tokens=0, xt=0, y=0) == 0
    assert lin(L=fake_layer(pairs=0, theta=0, channel_scales=0)) != 1  # rotation tensors unused


@needs_no_gpu
def test_quantize_pack_argument_checks():
    lib = _lib.load()
    L = fake_layer(I=256, O=64)
    qz_off = 256 * 64 // 2            # qweight bytes
    sc_off = qz_off + 2 * 64 // 2     # + qzeros bytes
    call = lambda w=FAKE * 8, dt=0, qw=FAKE, qz=FAKE + qz_off, sc=FAKE + sc_off, L=L: lib.paro_w4_quantize_pack(
        ctypes.byref(L), w, dt, 1, qw, qz, sc, None)
    assert call(dt=3) == 3                        # no such dtype
    assert call(w=0) == 1
    assert call(qz=0) == 1
    assert call(w=FAKE * 8 + 2) == 4              # 16-bit weights: 4-byte aligned
    assert call(w=FAKE * 8 + 4, dt=2) == 4        # fp32 weights: 8-byte aligned
    assert call(qw=FAKE + 2) == 4
    assert call(sc=FAKE + sc_off + 1) == 4
    assert call(w=FAKE) == 2                      # w overlaps qweight
    assert call(qz=FAKE + 64) == 2                # qzeros inside qweight
    assert call(L=fake_layer(I=256, O=64, G=16)) == 5
    assert call(L=fake_layer(I=256, O=64, G=-1)) == 5
    assert call(L=fake_layer(I=256, O=64, pairs=0)) == 1
    # G = 32: qzeros [I/32][O/8] int32 = 8 * 8 * 4 = 256 bytes, so scales
    # starting 128 bytes into them overlap (with I/128 groups, 64 bytes, they
    # would not); and scales [I/32][O] fp16 = 1 KB reach a buffer 512 bytes on
    g32 = fake_layer(I=256, O=64, G=32)
    assert call(L=g32, sc=FAKE + qz_off + 128) == 2, _lib.paro_last_error()
    assert call(L=g32, sc=FAKE * 8 - 512, w=FAKE * 8) == 2, _lib.paro_last_error()


@needs_no_gpu
def test_scale_rotate_backward_argument_checks():
    lib = _lib.load()
    L = fake_layer(I=256, O=64, krot=8)
    need = lib.paro_scale_rotate_backward_workspace_bytes(ctypes.byref(L), 4)
    # dense R' (H and L, 2 groups), one Gram split of 2 x 128 x 128 fp32, 16 x krot x I/2 fp32 partials
    assert need == 2 * 2 * 128 * 128 * 2 + 2 * 128 * 128 * 4 + 16 * 8 * 128 * 4
    assert lib.paro_scale_rotate_backward_workspace_bytes(ctypes.byref(L), 65) == need + 2 * 128 * 128 * 4
    assert lib.paro_scale_rotate_backward_workspace_bytes(ctypes.byref(L), 0) == need   # the walk still runs
    assert lib.paro_scale_rotate_backward_workspace_bytes(ctypes.byref(fake_layer(G=16)), 4) == 0
    assert lib.paro_scale_rotate_backward_workspace_bytes(ctypes.byref(fake_layer(G=-1)), 4) == 0
    assert lib.paro_scale_rotate_backward_workspace_bytes(ctypes.byref(fake_layer(G=64)), 4) == need

    def call(x=FAKE * 8, xdt=0, g=FAKE * 9, gdt=2, tokens=4, gx=FAKE * 10, gxdt=2, gth=FAKE * 11,
             gcs=FAKE * 12, ws=FAKE * 13, wsb=need, L=L):
        return lib.paro_scale_rotate_backward(ctypes.byref(L), x, xdt, g, gdt, tokens, gx, gxdt, gth, gcs, ws,
                                              wsb, None)
    assert call(xdt=2) == 3                           # x must be 16-bit
    assert call(gdt=1) == 3                           # g: F32 or x's dtype
    assert call(gxdt=1) == 3
    assert call(gth=0) == 1
    assert call(gcs=0, tokens=0) == 1                 # the sums are written even with no tokens
    assert call(x=0) == 1
    assert call(gx=0) == 1
    assert call(ws=0) == 7
    assert call(wsb=need - 1) == 7
    assert call(x=FAKE * 8 + 4) == 4                  # 16-byte aligned
    assert call(gx=FAKE * 10 + 8) == 4
    assert call(ws=FAKE * 13 + 8) == 4                # 16-byte aligned
    assert call(gcs=FAKE * 12 + 2) == 4
    assert call(gx=FAKE * 8 + 1024) == 2              # gx overlaps x
    assert call(gx=FAKE * 9 + 16) == 2                # gx overlaps g
    assert call(ws=FAKE * 10 + 16) == 2               # workspace overlaps gx
    assert call(gcs=FAKE * 11 + 16) == 2              # gcs overlaps gtheta
    assert call(tokens=-1) == 2
    assert call(L=fake_layer(G=16)) == 5
    assert call(L=fake_layer(pairs=0)) == 1


@needs_no_gpu
def test_moe_linear_argument_checks():
    lib = _lib.load()
    L = fake_layer(I=256, O=64)
    ws = lib.paro_w4a16_moe_linear_workspace_bytes(ctypes.byref(L), 40, 1)
    assert ws == lib.paro_w4a16_linear_workspace_bytes(ctypes.byref(L), 40, 1, 3)   # the prefill path's

    def call(E=4, offs=FAKE * 16, x=FAKE, xdt=1, tokens=40, y=FAKE * 2, ydt=1, wsp=FAKE * 4, wsb=ws, L=L):
        return lib.paro_w4a16_moe_linear(ctypes.byref(L), E, offs, x, xdt, tokens, y, ydt, wsp, wsb, None)
    assert call(E=0) == 2
    assert call(E=-1) == 2
    assert call(E=1025) == 2
    assert call(offs=0) == 1
    assert call(offs=FAKE * 16 + 4) == 4
    assert call(x=0) == 1
    assert call(xdt=2) == 3
    assert call(wsb=ws - 1) == 7
    assert call(y=FAKE + 64) == 2                    # y overlaps x
    assert call(L=fake_layer(G=16)) == 5
    assert call(tokens=0, x=0, y=0) == 0             # nothing to do


@needs_no_gpu
def test_mxfp4_argument_checks():
    lib = _lib.load()
    L = fake_layer(I=256, O=64)
    qw = lambda w=FAKE * 8, dt=1, c=FAKE * 9, s=FAKE * 10, L=L: lib.paro_mxfp4_quantize_weight(
        ctypes.byref(L), w, dt, c, s, None)
    assert qw(dt=5) == 3
    assert qw(w=0) == 1
    assert qw(c=FAKE * 9 + 4) == 4                  # codes 16-byte aligned
    assert qw(s=FAKE * 10 + 2) == 4
    assert qw(c=FAKE * 8 + 64) == 2                 # codes overlap w
    assert qw(L=fake_layer(G=16)) == 5
    aws = lib.paro_mxfp4_activation_workspace_bytes(ctypes.byref(L))
    assert aws == 2 * 2 * 128 * 128 * 2             # the dense R' (H and L) of two groups
    qa = lambda x=FAKE * 8, dt=0, t=4, c=FAKE * 9, s=FAKE * 10, ws=FAKE * 11, wsb=aws: \
        lib.paro_mxfp4_quantize_activations(ctypes.byref(L), x, dt, t, c, s, ws, wsb, None)
    assert qa(dt=2) == 3                            # activations are 16-bit
    assert qa(t=-1) == 2
    assert qa(t=0, x=0, c=0, s=0) == 0
    assert qa(wsb=aws - 1) == 7
    assert qa(x=FAKE * 8 + 4) == 4
    assert qa(ws=FAKE * 8 + 64) == 2                # workspace overlaps x
    gm = lambda ac=FAKE, as_=FAKE * 2, t=4, wc=FAKE * 3, ws=FAKE * 4, O=64, I=256, b=0, y=FAKE * 5, ydt=2: \
        lib.paro_mxfp4_gemm(ac, as_, t, wc, ws, O, I, b, y, ydt, None)
    assert gm(I=200) == 2
    assert gm(O=60) == 2
    assert gm(ydt=7) == 3
    assert gm(wc=0) == 1
    assert gm(ac=FAKE + 8) == 4
    assert gm(y=FAKE * 3 + 16) == 2                 # y overlaps the weight codes
    assert gm(t=1 << 24, I=1 << 12) == 5            # beyond 32-bit buffer offsets
    need = lib.paro_mxfp4_linear_workspace_bytes(ctypes.byref(L), 4)
    assert need == 512 + 256 + aws                  # 4 x 128 code bytes, 4 x 8 scale bytes, R' (each 256-aligned)
    ln = lambda wsb=need, ws=FAKE * 6, xdt=0: lib.paro_mxfp4_linear(
        ctypes.byref(L), FAKE * 3, FAKE * 4, FAKE, xdt, 4, FAKE * 5, 0, ws, wsb, None)
    assert ln(wsb=need - 1) == 7
    assert ln(ws=0) == 7
    assert ln(xdt=2) == 3
    pneed = lib.paro_mxfp4_linear_prepared_workspace_bytes(ctypes.byref(L), 4)
    assert pneed == 512 + 256                       # no room for R': the caller built it
    lp = lambda hl=FAKE * 7, wsb=pneed, ws=FAKE * 6: lib.paro_mxfp4_linear_prepared(
        ctypes.byref(L), hl, FAKE * 3, FAKE * 4, FAKE, 0, 4, FAKE * 5, 0, ws, wsb, None)
    assert lp(hl=0) == 1
    assert lp(wsb=pneed - 1) == 7
    assert lp(hl=FAKE * 7 + 8) == 4                 # hl 16-byte aligned
    assert lp(hl=FAKE * 6 + 256) == 2               # hl overlaps the workspace
    assert lp(hl=FAKE * 5) == 2                     # hl overlaps y


@needs_no_gpu
def test_whole_row_group_workspace_and_path():
    """group_size -1 (one group over all I channels): decode takes the split
    path, and the prefill workspace holds no dense rotation matrix."""
    lib = _lib.load()
    L = fake_layer(I=4096, O=1024, G=-1)
    assert lib.paro_w4a16_linear_choose_path(ctypes.byref(L), 1) == 2
    assert lib.paro_w4a16_linear_choose_path(ctypes.byref(L), 16) == 2
    assert lib.paro_w4a16_linear_choose_path(ctypes.byref(L), 17) == 3
    L128 = fake_layer(I=4096, O=1024, G=128)
    counters = (1 << 21) // 128 * 128
    assert lib.paro_w4a16_linear_workspace_bytes(ctypes.byref(L), 32, 1, 3) == counters + 32 * 4096 * 2
    assert lib.paro_w4a16_linear_workspace_bytes(ctypes.byref(L128), 32, 1, 3) == counters + 32 * 4096 * 2 + 4096 * 512
    assert lib.paro_w4a16_linear_prepared_workspace_bytes(ctypes.byref(L), 32) == 0   # no prebuilt form


def multi(layers, n=None, hl=(FAKE * 8, FAKE * 9), x=FAKE, xdt=0, tokens=32, y=(FAKE * 2, FAKE * 3), ydt=0,
          ws=FAKE * 16, wsb=1 << 30):
    """paro_w4a16_linear_prepared_multi on fake descriptors (validation only)."""
    arr = (_lib.ParoLayerC * len(layers))(*layers) if layers is not None else None
    hla = (ctypes.c_void_p * len(hl))(*hl) if hl is not None else None
    ya = (ctypes.c_void_p * len(y))(*y) if y is not None else None
    if n is None:
        n = len(layers) if layers is not None else 2
    return _lib.load().paro_w4a16_linear_prepared_multi(arr, n, hla, x, xdt, tokens, ya, ydt, ws, wsb, None)


@needs_no_gpu
@pytest.mark.parametrize("case,code", [
    (dict(n=0), 2),                                    # 1..4 layers
    (dict(n=5), 2),
    (dict(layers=None), 1),
    (dict(hl=None), 1),
    (dict(y=None), 1),
    (dict(hl=(FAKE * 8, 0)), 1),                       # every layer needs its rotation matrix
    (dict(y=(FAKE * 2, 0)), 1),
    (dict(L1=dict(I=384)), 2),                         # the layers share in_features, group size, krot
    (dict(L1=dict(G=64)), 2),
    (dict(L1=dict(krot=4)), 2),
    (dict(L1=dict(G=16)), 5),
    (dict(xdt=2), 3),
    (dict(ydt=1), 3),
    (dict(x=FAKE + 2), 4),
    (dict(hl=(FAKE * 8, FAKE * 9 + 4)), 4),
    (dict(y=(FAKE * 2, FAKE * 2 + 64)), 2),            # the two outputs overlap
    (dict(y=(FAKE * 2, FAKE + 32)), 2),                # an output overlaps x
    (dict(wsb=64), 7),
    (dict(ws=0), 7),
    (dict(L1=dict(qweight=0)), 1),
])
def test_multi_linear_argument_checks(case, code):
    L0 = fake_layer(I=256, O=64)
    L1 = fake_layer(**{"I": 256, "O": 64, **case.get("L1", {})})
    kw = {k: v for k, v in case.items() if k not in ("L1",)}
    layers = kw.pop("layers", [L0, L1])
    rc = multi(layers, **kw)
    assert rc == code, _lib.paro_last_error()
    assert _lib.paro_last_error()


@needs_no_gpu
def test_multi_linear_zero_tokens_is_a_noop():
    assert multi([fake_layer(), fake_layer()], tokens=0, x=0, ws=0, wsb=0) == 0


def test_multi_linear_workspace_sizes():
    lib = _lib.load()
    L = fake_layer(I=4096, O=1024)
    arr = lambda n: (_lib.ParoLayerC * n)(*([L] * n))
    mw = lambda n, m: lib.paro_w4a16_linear_prepared_multi_workspace_bytes(arr(n), n, m)
    one = lambda m: lib.paro_w4a16_linear_prepared_workspace_bytes(ctypes.byref(L), m)
    # prefill: one tiled X_r per layer after the counters; decode: one layer's workspace
    assert mw(2, 4096) - mw(1, 4096) == 4096 * 4096 * 2
    assert mw(1, 4096) == one(4096)
    assert mw(3, 16) == one(16) and mw(2, 1) == one(1)
    assert mw(0, 4096) == 0 and mw(5, 4096) == 0 and mw(2, 0) == 0
    # out_features may differ: prefill still one tiled X_r per layer (it
    # depends on in_features alone); decode the largest single-layer need
    Lw = fake_layer(I=4096, O=14336)
    mixed = (_lib.ParoLayerC * 2)(L, Lw)
    mwx = lambda m: lib.paro_w4a16_linear_prepared_multi_workspace_bytes(mixed, 2, m)
    assert mwx(4096) == mw(2, 4096)
    assert mwx(16) == max(one(16), lib.paro_w4a16_linear_prepared_workspace_bytes(ctypes.byref(Lw), 16))
    assert mwx(16) > one(16)


@needs_no_gpu
def test_tiled_multi_argument_checks():
    lib = _lib.load()
    arr = lambda ls: (_lib.ParoLayerC * len(ls))(*ls)
    ptrs = lambda *v: (ctypes.c_void_p * len(v))(*v)
    L0, L1 = fake_layer(I=256, O=64), fake_layer(I=256, O=64)
    call = lambda ls, n, xt, y, tokens=32: lib.paro_w4a16_linear_tiled_multi(arr(ls), n, xt, 0, tokens, y, 0, None)
    ok_xt, ok_y = ptrs(FAKE * 4, FAKE * 5), ptrs(FAKE * 6, FAKE * 7)
    assert call([L0, L1], 0, ok_xt, ok_y) == 2
    assert call([L0, L1], 5, ok_xt, ok_y) == 2
    assert call([L0, fake_layer(I=384, O=64)], 2, ok_xt, ok_y) == 2          # one in_features
    assert call([L0, fake_layer(I=256, O=64, G=64)], 2, ok_xt, ok_y) == 2    # one group size
    # outputs sized by each layer's out_features: a 128-wide layer's output
    # at 32 tokens (8 KB as fp16) reaches the next one 4 KB on
    assert call([fake_layer(I=256, O=128), L1], 2, ok_xt, ptrs(FAKE * 6, FAKE * 6 + 4096)) == 2
    assert call([L0, L1], 2, ptrs(FAKE * 4, 0), ok_y) == 1
    assert call([L0, L1], 2, ok_xt, ptrs(FAKE * 6, FAKE * 6 + 64)) == 2      # outputs overlap
    assert call([L0, L1], 2, ok_xt, ptrs(FAKE * 6, FAKE * 5 + 32)) == 2      # an output overlaps an x_t
    assert call([L0, L1], 2, ptrs(FAKE * 4 + 4, FAKE * 5), ok_y) == 4
    assert call([L0, L1], 2, None, None, tokens=0) == 1                      # arrays are required
