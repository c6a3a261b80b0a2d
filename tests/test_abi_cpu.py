"""Host-side checks of the C ABI: the library loads, exports every function
include/flce.h declares, and rejects bad arguments before touching the GPU.
No kernel is launched here."""

import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_PATH = os.path.join(ROOT, "linear_cross_entropy_03_amd", "liblce03.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB_PATH),
                                reason="liblce03.so not built (run __graft_entry__.build())")


@pytest.fixture(scope="module")
def B():
    from linear_cross_entropy_03_amd import binding
    binding.lib()
    return binding


def test_exports_every_declared_function(B):
    names = B.header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(B.lib(), n), n
        assert n in B._SIGNATURES, f"binding lacks {n}"


@pytest.mark.parametrize("lang,std", [("c", "-std=c99"), ("c++", "-std=c++17")])
def test_header_compiles_standalone(tmp_path, lang, std):
    """include/flce.h needs nothing but the standard headers it includes."""
    import shutil
    import subprocess
    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None:
        pytest.skip("no host compiler")
    src = tmp_path / ("use.c" if lang == "c" else "use.cpp")
    src.write_text('#include "flce.h"\nint use(void) { return FLCE_OK; }\n')
    r = subprocess.run([cc, std, "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), str(src)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr


def test_status_strings(B):
    for code in range(6):
        assert B.status_text(code)
    assert B.status_text(99) == "unknown status"


def test_workspace_queries_and_plan(B):
    assert B.flce_workspace_bytes(0, 64, 1024, B.F32) > 0
    assert B.flce_workspace_bytes(10, 0, 1024, B.F32) == 0
    assert B.flce_workspace_bytes(10, 64, 1024, 7) == 0
    small = B.flce_workspace_bytes(32768, 4096, 128256, B.BF16, 1024)
    big = B.flce_workspace_bytes(32768, 4096, 128256, B.BF16, 4096)
    assert big > small >= 1024 * 128256 * 2
    # The automatic chunk never holds all rows of a multi-chunk batch.
    for N, H, V in ((8192, 2048, 128256), (32768, 4096, 128256), (32768, 4096, 256000)):
        c, s = B.flce_plan(N, H, V, B.BF16)
        assert c % 256 == 0 and c < N
        # one chunk of logits stays within the 2.4 GB budget, or within twice
        # it when that reaches 8192 rows (the grad_W product's K)
        assert c * ((V + 7) // 8 * 8) * 2 <= (2.5e9 if c < 8192 else 4.8e9)
        assert s in (1, 2, 4, 8)
    assert B.flce_plan(256, 64, 1024, B.F32) == (256, 1)
    assert B.flce_plan(300, 64, 1000, B.F32, 64)[0] == 64
    assert B.ce_workspace_bytes(1024, 32768) >= 1024 * 4
    assert B.ce_workspace_bytes(-1, 5) == 0


def test_row_packing_switch_and_workspace(B):
    """The packing switch returns the previous setting and does not change the
    workspace size; 16-bit plans hold the packing lists (row map and packed
    targets, 4 bytes per row each, plus block counts) and at least one split-K
    partial of chunk x H float32, whose first half also takes the chunk's
    gathered 16-bit rows; float32 plans hold neither."""
    was = B.flce_set_row_packing(False)
    try:
        assert B.flce_set_row_packing(True) is False
        assert B.flce_set_row_packing(True) is True
        N, H, V = 4096, 512, 3000
        ldz = (V + 7) // 8 * 8
        for C in (1024, 256):
            on = B.flce_workspace_bytes(N, H, V, B.BF16, C)
            B.flce_set_row_packing(False)
            assert B.flce_workspace_bytes(N, H, V, B.BF16, C) == on
            B.flce_set_row_packing(True)
            f32 = B.flce_workspace_bytes(N, H, V, B.F32, C)
            assert 256 + N * 4 + C * ldz * 4 <= f32 < 256 + N * 4 + C * ldz * 4 + 4 * 256
            base16 = 256 + N * 4 + C * ldz * 2 + C * H * 4 + 2 * N * 4
            assert base16 <= on < base16 + 16 * 256
            parts = B.flce_workspace_parts(N, H, V, B.BF16, C)
            assert sum(parts.values()) == on
            assert parts["split_partials"] >= C * H * 4 >= 2 * C * H * 2
    finally:
        B.flce_set_row_packing(was)


def _fb(B, **kw):
    args = dict(X=16, W=16, bias=None, targets=16, N=4, H=8, V=10, dtype=B.BF16, ign=-100, red=2,
                loss=16, gX=16, gW=16, gb=None, ws=16, wsb=1 << 30, chunk=0, stream=None)
    args.update(kw)
    return B.lib().flce_forward_backward(
        args["X"], args["W"], args["bias"], args["targets"], args["N"], args["H"], args["V"],
        args["dtype"], args["ign"], args["red"], args["loss"], args["gX"], args["gW"], args["gb"],
        args["ws"], args["wsb"], args["chunk"], args["stream"])


def test_flce_argument_errors(B):
    # Pointers here are fake (aligned integers): every call must fail in
    # validation, before anything is enqueued.
    assert _fb(B, W=None) == B.E_INVALID_ARG
    assert _fb(B, loss=None) == B.E_INVALID_ARG
    assert _fb(B, X=None) == B.E_INVALID_ARG
    assert _fb(B, targets=None) == B.E_INVALID_ARG
    assert _fb(B, N=-1) == B.E_INVALID_ARG
    assert _fb(B, H=0) == B.E_INVALID_ARG
    assert _fb(B, V=0) == B.E_INVALID_ARG
    assert _fb(B, dtype=5) == B.E_INVALID_ARG
    assert _fb(B, red=3) == B.E_INVALID_ARG
    assert _fb(B, gb=16) == B.E_INVALID_ARG          # grad_bias without bias
    assert _fb(B, chunk=-2) == B.E_INVALID_ARG
    assert _fb(B, X=24) == B.E_UNSUPPORTED           # misaligned
    assert _fb(B, H=12) == B.E_UNSUPPORTED           # bf16 needs H % 8 == 0
    assert _fb(B, ws=None) == B.E_WORKSPACE
    assert _fb(B, wsb=64) == B.E_WORKSPACE


def test_flce_ex_gradient_type_errors(B):
    """The 16-bit-gradient entry point accepts FLCE_F32 or the input's own
    16-bit type only; everything here fails before any launch."""
    L = B.lib()

    def ex(dtype, gdt, wsb=1 << 30):
        return L.flce_forward_backward_ex(16, 16, None, 16, 4, 8, 10, dtype, -100, 2, gdt, 16, 16, 16,
                                          None, 16, wsb, 0, None)
    assert ex(B.BF16, 7) == B.E_INVALID_ARG
    assert ex(B.BF16, B.F16) == B.E_INVALID_ARG
    assert ex(B.F16, B.BF16) == B.E_INVALID_ARG
    assert ex(B.F32, B.BF16) == B.E_INVALID_ARG
    assert ex(B.BF16, B.BF16, wsb=64) == B.E_WORKSPACE
    assert ex(B.F16, B.F32, wsb=64) == B.E_WORKSPACE


def test_ce_and_shard_argument_errors(B):
    L = B.lib()
    assert L.ce_forward_backward(16, 16, 16, 4, 10, B.BF16, -100, 9, 16, 16, 1 << 20, None) == B.E_INVALID_ARG
    assert L.ce_forward_backward(16, 16, 16, 4, 0, B.BF16, -100, 1, 16, 16, 1 << 20, None) == B.E_INVALID_ARG
    assert L.ce_forward_backward(16, 16, 16, 4, 10, B.BF16, -100, 1, 16, 16, 8, None) == B.E_WORKSPACE
    assert L.ce_forward_backward(16, 40, 16, 4, 10, B.BF16, -100, 1, 16, 16, 1 << 20, None) == B.E_UNSUPPORTED
    # shard must fit inside the global vocabulary
    assert L.ce_shard_stats(16, 16, 4, 10, 5, 12, B.BF16, -100, 16, 16, 16, 16, 1 << 20, None) == B.E_INVALID_ARG
    assert L.flce_shard_stats(16, 16, None, 16, 4, 8, 10, 0, 10, B.BF16, -100, 16, 16, 16, 16, 8, 0,
                              None) == B.E_WORKSPACE
    assert L.flce_check_device_error(None, None) == B.E_INVALID_ARG


def test_row_launch_limit(B):
    """Standalone CE and shard statistics cover all N rows in one launch of
    one workgroup (up to 1024 lanes) per row, so N is limited to 2^22 - 1
    rows: one more is refused before anything runs (no device needed)."""
    L = B.lib()
    big = 1 << 22
    assert L.ce_forward_backward(16, 16, 16, big, 32768, B.BF16, -100, 2, 16, 16, 1 << 40,
                                 None) == B.E_UNSUPPORTED
    assert L.ce_shard_stats(16, 16, big, 16, 0, 32, B.BF16, -100, 16, 16, 16, 16, 1 << 40,
                            None) == B.E_UNSUPPORTED
    assert L.ce_forward_backward_noalloc(16, 16, 16, big, 32768, B.BF16, -100, 2, 16,
                                         None) == B.E_UNSUPPORTED
    # FLCE chunks are clamped to the same count
    assert B.flce_plan(1 << 23, 64, 1000, B.BF16, 1 << 23)[0] == big - 1


def test_noalloc_ce_argument_errors(B):
    """The entry point without a workspace rejects sizes beyond its static
    scratch (and other bad arguments) before touching the device."""
    L = B.lib()
    assert L.ce_forward_backward_noalloc(16, 16, 16, 1 << 22, 10, B.BF16, -100, 2, 16,
                                         None) == B.E_UNSUPPORTED
    assert L.ce_forward_backward_noalloc(16, 16, 16, 4, 10, B.BF16, -100, 9, 16, None) == B.E_INVALID_ARG
    assert L.ce_forward_backward_noalloc(16, 16, 16, 4, 0, B.BF16, -100, 2, 16, None) == B.E_INVALID_ARG
    assert L.ce_forward_backward_noalloc(16, 16, 16, 4, 10, B.BF16, -100, 2, None, None) == B.E_INVALID_ARG
    assert L.ce_forward_backward_noalloc(None, 16, 16, 4, 10, B.BF16, -100, 2, 16, None) == B.E_INVALID_ARG


def test_vocab_parallel_argument_errors(B):
    L = B.lib()
    # ce_combine_shard_stats(max, sumexp, target, P, N, targets, V_global, ign, red, lse, loss, ws, wsb, stream)
    ok = dict(m=16, s=16, t=16, P=2, N=4, y=16, Vg=10, ign=-100, red=2, lse=16, loss=16, ws=16, wsb=1 << 20)

    def comb(**kw):
        a = dict(ok, **kw)
        return L.ce_combine_shard_stats(a["m"], a["s"], a["t"], a["P"], a["N"], a["y"], a["Vg"], a["ign"],
                                        a["red"], a["lse"], a["loss"], a["ws"], a["wsb"], None)
    assert comb(P=0) == B.E_INVALID_ARG
    assert comb(red=7) == B.E_INVALID_ARG
    assert comb(loss=None) == B.E_INVALID_ARG
    assert comb(m=None) == B.E_INVALID_ARG
    assert comb(lse=40) == B.E_UNSUPPORTED           # misaligned
    assert comb(wsb=8) == B.E_WORKSPACE

    # flce_shard_backward(X, Ws, bs, y, N, H, Vl, v0, Vg, dtype, ign, red, lse, gX, gW, gb, ws, wsb, chunk, stream)
    okb = dict(X=16, Ws=16, bs=None, y=16, N=4, H=8, Vl=10, v0=0, Vg=10, dt=B.BF16, ign=-100, red=2,
               lse=16, gX=16, gW=16, gb=None, ws=16, wsb=1 << 30, chunk=0)

    def bwd(**kw):
        a = dict(okb, **kw)
        return L.flce_shard_backward(a["X"], a["Ws"], a["bs"], a["y"], a["N"], a["H"], a["Vl"], a["v0"],
                                     a["Vg"], a["dt"], a["ign"], a["red"], a["lse"], a["gX"], a["gW"],
                                     a["gb"], a["ws"], a["wsb"], a["chunk"], None)
    assert bwd(v0=5) == B.E_INVALID_ARG              # shard past the global vocabulary
    assert bwd(lse=None) == B.E_INVALID_ARG
    assert bwd(gb=16) == B.E_INVALID_ARG             # grad_bias without bias
    assert bwd(Ws=None) == B.E_INVALID_ARG
    assert bwd(H=12) == B.E_UNSUPPORTED
    assert bwd(ws=None) == B.E_WORKSPACE


def test_shift_labels_argument_errors(B):
    L = B.lib()
    assert L.flce_shift_labels(None, 2, 3, -100, 16, None) == B.E_INVALID_ARG
    assert L.flce_shift_labels(16, 2, 0, -100, 32, None) == B.E_INVALID_ARG
    assert L.flce_shift_labels(16, 2, 3, -100, 16, None) == B.E_INVALID_ARG   # in place
    assert L.flce_shift_labels(None, 0, 3, -100, None, None) == B.OK          # nothing to do


def test_multihead_argument_errors(B):
    L = B.lib()
    assert B.flce_multihead_workspace_bytes(64, 8, 100, 0) == 0
    one = B.flce_multihead_workspace_bytes(64, 8, 100, 1)
    assert B.flce_multihead_workspace_bytes(64, 8, 100, 3) > one > B.flce_workspace_bytes(64, 8, 100)

    def mh(K=2, wsb=1 << 30, **kw):
        a = dict(X=16, W=16, bias=None, y=16, N=4, H=8, V=10, dt=B.BF16, red=2, loss=16, gX=16,
                 gW=16, gb=None, ws=16)
        a.update(kw)
        return L.flce_multihead_forward_backward(a["X"], a["W"], a["bias"], a["y"], a["N"], a["H"],
                                                 a["V"], K, a["dt"], -100, a["red"], a["loss"],
                                                 a["gX"], a["gW"], a["gb"], a["ws"], wsb, 0, None)
    assert mh(K=0) == B.E_INVALID_ARG
    assert mh(W=None) == B.E_INVALID_ARG
    assert mh(gb=16) == B.E_INVALID_ARG
    assert mh(H=12) == B.E_UNSUPPORTED
    assert mh(wsb=B.flce_workspace_bytes(4, 8, 10)) == B.E_WORKSPACE


def test_16bit_stride_limit(B):
    """16-bit GEMM tiles use 32-bit byte offsets: H and round_up(V, 8) below 2^22."""
    big = 1 << 22
    assert _fb(B, H=big) == B.E_UNSUPPORTED
    assert _fb(B, V=big - 3) == B.E_UNSUPPORTED          # rounds up to 2^22
    assert _fb(B, dtype=B.F16, V=big + 8) == B.E_UNSUPPORTED
    assert _fb(B, dtype=B.F32, H=big, wsb=64) == B.E_WORKSPACE   # fp32 path has no such limit


def test_jsd_argument_errors(B):
    L = B.lib()

    def jsd(**kw):
        a = dict(Xs=16, Ws=16, Xt=16, Wt=16, y=16, N=4, Hs=8, Ht=8, V=10, dt=B.BF16, red=2, T=1.0,
                 loss=16, gX=16, gW=16, ws=16, wsb=1 << 30)
        a.update(kw)
        return L.flce_jsd_forward_backward(a["Xs"], a["Ws"], a["Xt"], a["Wt"], a["y"], a["N"], a["Hs"],
                                           a["Ht"], a["V"], a["dt"], -100, a["red"], a["T"], a["loss"],
                                           a["gX"], a["gW"], a["ws"], a["wsb"], 0, None)
    assert jsd(T=0.0) == B.E_INVALID_ARG
    assert jsd(T=-1.0) == B.E_INVALID_ARG
    assert jsd(Wt=None) == B.E_INVALID_ARG
    assert jsd(Xt=None) == B.E_INVALID_ARG
    assert jsd(Ht=12) == B.E_UNSUPPORTED
    assert jsd(Xt=24) == B.E_UNSUPPORTED
    assert jsd(wsb=B.flce_workspace_bytes(4, 8, 10)) == B.E_WORKSPACE
    assert B.flce_jsd_workspace_bytes(4, 8, 10) > B.flce_workspace_bytes(4, 8, 10)


def test_dpo_argument_errors(B):
    L = B.lib()

    def dpo(**kw):
        a = dict(X=16, W=16, y=16, P=2, S=3, H=8, V=10, dt=B.BF16, ref=16, beta=0.1, loss=16, pl=None,
                 gX=16, gW=16, ws=16, wsb=1 << 30)
        a.update(kw)
        return L.flce_dpo_forward_backward(a["X"], a["W"], a["y"], a["P"], a["S"], a["H"], a["V"],
                                           a["dt"], -100, a["ref"], a["beta"], a["loss"], a["pl"],
                                           a["gX"], a["gW"], a["ws"], a["wsb"], 0, None)
    assert dpo(beta=0.0) == B.E_INVALID_ARG
    assert dpo(S=0) == B.E_INVALID_ARG
    assert dpo(ref=None) == B.E_INVALID_ARG
    assert dpo(pl=24) == B.E_UNSUPPORTED
    assert dpo(wsb=B.flce_workspace_bytes(12, 8, 10)) == B.E_WORKSPACE


def _device_code_objects(lib_path, tmp_path):
    """The gfx950 code objects inside the library's offload bundles (one per
    compiled HIP source), from its .hip_fatbin section."""
    import shutil
    import struct
    import subprocess
    objcopy = shutil.which("llvm-objcopy", path="/opt/rocm/llvm/bin")
    if objcopy is None:
        pytest.skip("llvm-objcopy not available")
    fat = tmp_path / "fatbin.bin"
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fat}", lib_path, str(tmp_path / "lib.tmp")],
                   check=True, capture_output=True)
    data = fat.read_bytes()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    out, pos = [], 0
    while (i := data.find(magic, pos)) >= 0:
        (n,) = struct.unpack_from("<Q", data, i + len(magic))
        off = i + len(magic) + 8
        for _ in range(n):
            e_off, e_size, t_size = struct.unpack_from("<QQQ", data, off)
            off += 24
            triple = data[off:off + t_size].decode()
            off += t_size
            if triple.endswith("gfx950"):
                out.append(data[i + e_off:i + e_off + e_size])
        pos = i + 1
    return out


def test_no_kernel_uses_scratch(tmp_path):
    """Every kernel of the library keeps its state in registers and LDS: a
    private segment would mean register spills to scratch memory, which the
    row kernels would run through on every element (the ring GEMM's launcher
    refuses such a build at run time as well). Reads the AMDGPU kernel
    metadata of the library's own device code."""
    import shutil
    import subprocess
    readelf = shutil.which("llvm-readelf", path="/opt/rocm/llvm/bin")
    if readelf is None:
        pytest.skip("llvm-readelf not available")
    kernels, spilled = 0, []
    for k, co in enumerate(_device_code_objects(LIB_PATH, tmp_path)):
        path = tmp_path / f"co{k}.o"
        path.write_bytes(co)
        notes = subprocess.run([readelf, "--notes", str(path)], check=True, capture_output=True,
                               text=True).stdout
        priv = [int(l.split(":", 1)[1]) for l in notes.splitlines()
                if l.strip().startswith(".private_segment_fixed_size:")]
        syms = [l.split(":", 1)[1].strip() for l in notes.splitlines() if l.strip().startswith(".symbol:")]
        assert len(priv) == len(syms)
        kernels += len(syms)
        spilled += [s for s, p in zip(syms, priv) if p != 0]
    assert kernels >= 100, kernels
    assert not spilled, spilled
