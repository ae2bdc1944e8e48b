"""The C ABI library loads, exports every function include/moe.h declares, and rejects bad
arguments on the host before launching anything (no GPU needed for these)."""
import ctypes
import os
import re
import subprocess

import pytest

from expert_ffn_layer_amd import native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "moe.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", txt)))


def test_header_and_binding_agree():
    assert _declared() == sorted(N.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = N.load()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", N.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (moe_\w+)", out))
    assert exported == set(_declared())  # nothing undeclared leaks out


def test_status_strings():
    lib = N.load()
    for code, name in N.STATUS.items():
        assert lib.moe_status_string(code).decode() == name


def _shape(**kw):
    base = dict(T=4, H=256, E=8, k=2, I=128, I_shared=0, act="bf16", w_routed="bf16", w_shared="bf16")
    base.update(kw)
    return N.make_shape(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), 1), (dict(H=100), 1), (dict(I=64), 1), (dict(E=0), 1), (dict(E=2000), 1),
    (dict(k=0), 1), (dict(k=9), 1), (dict(E=32, k=17), 1), (dict(I_shared=256), 2),
    (dict(act="fp8"), 1), (dict(act="f32"), 2), (dict(w_routed="f32"), 2),
    # W4A8: routed experts only (bf16 activations, I % 256, H % 512)
    (dict(H=512, I=256, I_shared=256, w_routed="mxfp4a8", w_shared="mxfp4a8"), 2),
    (dict(H=512, I=128, w_routed="mxfp4a8"), 2), (dict(H=256, I=256, w_routed="mxfp4a8"), 2),
    # W8A8 MXFP8: the shared expert only, beside W4A8 routed experts
    (dict(H=512, I=256, w_routed="mxfp8a8"), 2),
    (dict(H=512, I=256, I_shared=256, w_routed="bf16", w_shared="mxfp8a8"), 2),
    (dict(H=512, I=256, I_shared=256, w_routed="mxfp4", w_shared="mxfp8a8"), 2),
    (dict(act="f32", w_routed="f32", I_shared=128, w_shared="mxfp8a8"), 2),
    # Int8 W8A8: routed and shared both INT8 (or no shared expert)
    (dict(H=512, I=256, I_shared=256, w_routed="int8", w_shared="bf16"), 2),
    (dict(H=512, I=256, I_shared=256, w_routed="bf16", w_shared="int8"), 2),
    (dict(H=256, I=256, w_routed="int8"), 2),
    # a group of more than 65535 64-row blocks (the plan's block index): T*k above 4194240
    (dict(T=524281, k=8), 2),
])
def test_shape_validation(kw, status):
    with pytest.raises(N.MoeError) as e:
        N.moe_workspace_size(_shape(**kw))
    assert e.value.status == status


def test_w4a8_shape_is_accepted_and_adds_quantised_activations():
    base = N.moe_workspace_size(_shape(H=512, I=256, w_routed="mxfp4"))
    a8 = N.moe_workspace_size(_shape(H=512, I=256, w_routed="mxfp4a8"))
    assert a8 > base
    assert N.moe_workspace_size(_shape(H=512, I=256, I_shared=256, w_routed="mxfp4a8", w_shared="bf16")) > a8


def test_w4a8_accepts_both_paths():
    for path in ("decode", "prefill", "auto"):
        assert N.moe_workspace_size(_shape(H=512, I=256, I_shared=256, w_routed="mxfp4a8", w_shared="bf16",
                                           path=path)) > 0
        assert N.moe_workspace_size(_shape(H=512, I=256, I_shared=256, w_routed="mxfp4a8", w_shared="mxfp8a8",
                                           path=path)) > 0


def test_hybrid_shape_is_accepted_and_quantises_the_shared_rows_of_h():
    bf = N.moe_workspace_size(_shape(H=512, I=256, I_shared=256, w_routed="mxfp4a8", w_shared="bf16"))
    mx = N.moe_workspace_size(_shape(H=512, I=256, I_shared=256, w_routed="mxfp4a8", w_shared="mxfp8a8"))
    # T more rows of h as MXFP8 codes (I bytes each) and exponents (I / 32 bytes each; regions are
    # 256-byte aligned, so 4 rows of exponents may fit the padding already there)
    assert mx - bf >= 4 * 256


def test_int8_shape_is_accepted_with_and_without_a_shared_expert():
    assert N.moe_workspace_size(_shape(H=512, I=256, w_routed="int8")) > 0
    assert N.moe_workspace_size(_shape(H=512, I=256, I_shared=256, w_routed="int8", w_shared="int8")) > \
        N.moe_workspace_size(_shape(H=512, I=256, w_routed="int8"))


def test_largest_plannable_routing_is_accepted():
    # T*k = 65535 * 64 exactly: every group's blocks fit the plan's 16-bit index
    assert N.moe_workspace_size(_shape(T=65535 * 8, k=8)) > 0


def test_workspace_grows_with_tokens_and_shared_expert():
    a = N.moe_workspace_size(_shape(T=4))
    b = N.moe_workspace_size(_shape(T=64))
    c = N.moe_workspace_size(_shape(T=64, I_shared=128))
    assert 0 < a < b < c
    assert N.moe_workspace_size(_shape(T=0)) > 0


def test_pack_sizes():
    assert N.moe_pack_size("bf16", 3, 4096, 1536) == (3 * 4096 * 1536 * 2, 0)
    assert N.moe_pack_size("f32", 1, 256, 128) == (256 * 256 * 4, 0)  # 128 features pad to 256
    assert N.moe_pack_size("fp8", 2, 7168, 2048) == (2 * 7168 * 2048, 2 * 56 * 16 * 4)
    assert N.moe_pack_size("mxfp4", 1, 7168, 3072) == (7168 * 3072 // 2, 7168 * 3072 // 32)
    # W4A8 weights are stored and packed exactly as MXFP4
    assert N.moe_pack_size("mxfp4a8", 2, 7168, 3072) == N.moe_pack_size("mxfp4", 2, 7168, 3072)
    # MXFP8: fp8-sized packets (features padded to 512), one exponent byte per lane per pair of
    # packets: 32 feature tiles x 2 pairs x 64
    assert N.moe_pack_size("mxfp8a8", 1, 256, 384) == (32 * 4 * 1024, 32 * 2 * 64)
    assert N.moe_pack_size("mxfp8a8", 2, 7168, 3072) == (2 * 7168 * 3072, 2 * 7168 * 3072 // 32)
    # INT8: fp8-sized packets, one fp32 scale per padded feature
    assert N.moe_pack_size("int8", 3, 256, 384) == (3 * 32 * 4 * 1024, 3 * 512 * 4)
    # the router's E is padded to 256 features (the width of one MFMA item)
    assert N.moe_pack_size("bf16", 1, 256, 8) == (256 * 256 * 2, 0)
    assert N.moe_pack_size("bf16", 1, 7168, 384) == (7168 * 512 * 2, 0)
    for fmt, K, Nn in (("fp8", 7168, 100), ("fp8", 100, 128), ("bf16", 48, 64), ("mxfp4", 128, 3),
                       ("mxfp8a8", 64, 256), ("int8", 64, 256)):
        with pytest.raises(N.MoeError):
            N.moe_pack_size(fmt, 1, K, Nn)


def test_logical_workspace_adds_the_packed_matrices():
    """moe_layer_forward_logical's workspace: the layer's, then the packed router and experts, each
    rounded up to the 256-byte alignment."""
    def up(n):
        return (n + 255) // 256 * 256
    for kw in (dict(), dict(I_shared=128), dict(w_routed="fp8", w_shared="fp8", I_shared=128, H=256, I=128)):
        s = _shape(**kw)
        fmt = kw.get("w_routed", "bf16")
        H, I, E = s.H, s.I, s.E
        extra = up(N.moe_pack_size("bf16", 1, H, E)[0])
        mats = [(fmt, E)] + ([(kw.get("w_shared", "bf16"), 1)] if s.I_shared else [])
        for f, count in mats:
            g, gs = N.moe_pack_size(f, count, H, I)
            d, ds = N.moe_pack_size(f, count, I, H)
            extra += 2 * (up(g) + up(max(gs, 1))) + up(d) + up(max(ds, 1))
        assert N.moe_logical_workspace_size(s) == N.moe_workspace_size(s) + extra


def test_entry_points_reject_null_and_small_workspace_before_launch():
    lib = N.load()
    s = _shape()
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: validation fails first
    assert lib.moe_route(ctypes.byref(s), None, fake, None, fake, fake, fake, 1 << 30, None) == 1
    # workspace too small
    assert lib.moe_route(ctypes.byref(s), fake, fake, None, fake, fake, fake, 16, None) == 3
    w = N.MoeWeights(0x1000, 0x1000, None, None, None, None)
    assert lib.moe_grouped_ffn(ctypes.byref(s), fake, fake, fake, ctypes.byref(w), None, fake, None, fake,
                               1 << 30, None) == 1
    s8 = _shape(w_routed="fp8")
    w8 = N.MoeWeights(0x1000, 0x1000, 0x1000, None, None, None)  # fp8 needs scales
    assert lib.moe_layer_forward(ctypes.byref(s8), fake, fake, None, ctypes.byref(w8), None, fake, None, None,
                                 fake, 1 << 30, None) == 1
    assert "scales" in lib.moe_last_error().decode()
    sh = _shape(I_shared=128)
    wf = N.MoeWeights(0x1000, 0x1000, 0x1000, None, None, None)
    assert lib.moe_layer_forward(ctypes.byref(sh), fake, fake, None, ctypes.byref(wf), None, fake, None, None,
                                 fake, 1 << 30, None) == 1  # shared weights missing
    # hash routing: missing ids or table, vocab < 1
    assert lib.moe_route_hash(ctypes.byref(s), fake, fake, None, None, fake, 10, fake, fake, fake, 1 << 30, None) == 1
    assert lib.moe_route_hash(ctypes.byref(s), fake, fake, None, fake, fake, 0, fake, fake, fake, 1 << 30, None) == 1
    assert lib.moe_layer_forward_hash(ctypes.byref(s), fake, fake, None, fake, None, 10, ctypes.byref(wf), None, fake,
                                      None, None, fake, 1 << 30, None) == 1
    # misaligned workspace
    assert lib.moe_permute(ctypes.byref(s), fake, fake, fake, fake, P(0x1001), 1 << 30, None) == 1
    # logical weights: NULL router, the packed copies not fitting the workspace
    assert lib.moe_layer_forward_logical(ctypes.byref(sh), fake, None, None, ctypes.byref(wf), ctypes.byref(wf), fake,
                                         None, None, fake, 1 << 40, None) == 1
    need = N.moe_logical_workspace_size(sh)
    assert lib.moe_layer_forward_logical(ctypes.byref(sh), fake, fake, None, ctypes.byref(wf), ctypes.byref(wf), fake,
                                         None, None, fake, need - 1, None) == 3


def test_quantisers_validate_before_launch():
    lib = N.load()
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: validation fails first (or rows == 0 returns)
    for fn, k_ok in ((lib.moe_quantize_mxfp8, 64), (lib.moe_quantize_int8, 64)):
        assert fn(fake, 0, k_ok, fake, fake, None) == 0        # no rows: nothing to do
        assert fn(fake, -1, k_ok, fake, fake, None) == 1       # negative rows
        assert fn(None, 4, k_ok, fake, fake, None) == 1        # NULL input
        assert fn(fake, 4, k_ok, None, fake, None) == 1        # NULL codes
        assert fn(fake, 4, k_ok, fake, None, None) == 1        # NULL scales
        assert fn(P(0x1008), 4, k_ok, fake, fake, None) == 1   # x not 16-byte aligned
        assert fn(fake, 4, k_ok, P(0x1004), fake, None) == 1   # codes not 8-byte aligned
    assert lib.moe_quantize_mxfp8(fake, 4, 48, fake, fake, None) == 1    # K not a multiple of 32
    assert lib.moe_quantize_mxfp8(fake, 4, 0, fake, fake, None) == 1
    assert lib.moe_quantize_mxfp8(fake, 1 << 30, 1 << 12, fake, fake, None) == 1  # rows * K > 2^40
    assert lib.moe_quantize_int8(fake, 4, 12, fake, fake, None) == 1     # K not a multiple of 8
    assert lib.moe_quantize_int8(fake, 4, 8200, fake, fake, None) == 1   # K above 8192
    assert lib.moe_quantize_int8(fake, 4, 64, fake, P(0x1002), None) == 1  # scales not 4-byte aligned
    assert "aligned" in lib.moe_last_error().decode()


def test_misaligned_pointers_are_refused_before_launch():
    """Activations, outputs and packed matrices need 16-byte alignment (vector loads, DMA to LDS),
    scales, index and routing-weight arrays 4-byte alignment."""
    lib = N.load()
    s = _shape()
    P = ctypes.c_void_p
    a, m8, m2 = P(0x10000), P(0x10008), P(0x10002)  # aligned, 8 off a 16-byte boundary, 2 off
    ws = 1 << 30
    w = N.MoeWeights(0x10000, 0x10000, 0x10000, None, None, None)
    wm = N.MoeWeights(0x10000, 0x10008, 0x10000, None, None, None)
    assert lib.moe_route(ctypes.byref(s), m8, a, None, a, a, a, ws, None) == 1          # x
    assert lib.moe_route(ctypes.byref(s), a, a, m2, a, a, a, ws, None) == 1             # bias
    assert lib.moe_permute(ctypes.byref(s), a, a, m2, a, a, ws, None) == 1              # slot_token
    assert lib.moe_grouped_ffn(ctypes.byref(s), a, a, a, ctypes.byref(wm), None, a, None, a, ws, None) == 1
    assert "packed weights" in lib.moe_last_error().decode()
    assert lib.moe_grouped_ffn(ctypes.byref(s), a, a, a, ctypes.byref(w), None, m8, None, a, ws, None) == 1
    assert lib.moe_combine(ctypes.byref(s), a, a, a, None, m8, None) == 1               # y
    assert lib.moe_combine(ctypes.byref(s), a, m2, a, None, a, None) == 1               # pair_slot
    assert lib.moe_layer_forward(ctypes.byref(s), a, a, None, ctypes.byref(w), None, m8, None, None,
                                 a, ws, None) == 1                                      # y
    assert lib.moe_layer_forward(ctypes.byref(s), a, m8, None, ctypes.byref(w), None, a, None, None,
                                 a, ws, None) == 1                                      # Wr_packed
    s8 = _shape(w_routed="fp8")
    w8 = N.MoeWeights(0x10000, 0x10000, 0x10000, 0x10000, 0x10002, 0x10000)
    assert lib.moe_layer_forward(ctypes.byref(s8), a, a, None, ctypes.byref(w8), None, a, None, None,
                                 a, ws, None) == 1
    assert "packed scales" in lib.moe_last_error().decode()
    assert lib.moe_pack(N.DTYPE["bf16"], 1, 256, 128, a, None, m8, None, None) == 1     # packed
    assert lib.moe_pack(N.DTYPE["f32"], 1, 256, 128, m2, None, a, None, None) == 1      # f32 source
    assert lib.moe_pack(N.DTYPE["fp8"], 1, 256, 256, a, m2, a, a, None) == 1            # fp32 scales


C_PROGRAM = r"""
#include "moe.h"
#include <stdio.h>
#include <string.h>

int main(void) {
  moe_shape s;
  size_t bytes = 0, logical = 0, pb = 0, ps = 0;
  moe_status st;
  memset(&s, 0, sizeof s);
  s.T = 64; s.H = 4096; s.E = 128; s.k = 8; s.I = 1536; s.I_shared = 0;
  s.act = MOE_BF16; s.w_routed = MOE_BF16; s.w_shared = MOE_BF16; s.path = MOE_PATH_AUTO;
  st = moe_workspace_size(&s, &bytes);
  printf("workspace %d %lu\n", (int)st, (unsigned long)bytes);
  st = moe_logical_workspace_size(&s, &logical);
  printf("logical %d %lu\n", (int)st, (unsigned long)logical);
  st = moe_pack_size(MOE_FP8_E4M3_B128, 2, 7168, 2048, &pb, &ps);
  printf("pack %d %lu %lu\n", (int)st, (unsigned long)pb, (unsigned long)ps);
  s.k = 0;
  st = moe_workspace_size(&s, &bytes);
  printf("bad %d %s\n", (int)st, moe_status_string(st));
  return 0;
}
"""


def test_header_is_c99_and_the_library_links_from_c(tmp_path):
    """include/moe.h compiles as strict C99 (no C++ in the ABI) and a C program linked against
    libmoe.so gets the same host-side answers as the binding."""
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(N.LIB_PATH)
    cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                         "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                         N.LIB_PATH, "-Wl,-rpath," + libdir], capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    out = dict((l.split()[0], l.split()[1:]) for l in run.stdout.splitlines())
    shape = N.make_shape(64, 4096, 128, 8, 1536)
    assert out["workspace"] == ["0", str(N.moe_workspace_size(shape))]
    assert out["logical"] == ["0", str(N.moe_logical_workspace_size(shape))]
    assert out["pack"] == ["0"] + [str(v) for v in N.moe_pack_size("fp8", 2, 7168, 2048)]
    assert out["bad"] == ["1", N.STATUS[1]]
