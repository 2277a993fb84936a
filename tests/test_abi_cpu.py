"""CPU-only checks of the C-ABI library: it loads, exports every function the header
declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import subprocess

import pytest
import torch

import moe_groupgemm_amd as mk

LIB = mk.LIB_PATH


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        pytest.fail("libmoe_mk.so is not built (run __graft_entry__.build())")
    return mk.lib()


def test_header_declares_the_boundary():
    names = mk.header_functions()
    for n in ("moe_mk_plan", "moe_mk_forward", "moe_mk_workspace_bytes", "moe_mk_workspace_init",
              "moe_mk_routing_view", "moe_mk_plan_destroy", "moe_mk_status_str"):
        assert n in names


def test_library_exports_every_header_function(L):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in mk.header_functions():
        assert name in exported, name
        assert hasattr(L, name)


def test_library_is_built_for_gfx950_only(tmp_path):
    fb = tmp_path / "fatbin.bin"
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", LIB, str(fb)], check=True)
    out = subprocess.run(["/opt/rocm/llvm/bin/clang-offload-bundler", "--list", "--type=o", f"--input={fb}"],
                         capture_output=True, text=True, check=True)
    targets = [t for t in out.stdout.split() if "amdgcn" in t]
    assert targets and all(t.endswith("gfx950") for t in targets)


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5):
        assert mk.moe_mk_status_str(code)
    assert mk.moe_mk_status_str(0) == "ok"


def test_null_and_bad_arguments_are_rejected(L):
    assert L.moe_mk_workspace_bytes(None, 4) == 0
    assert L.moe_mk_forward(None, None, None, None, None, None, None, None, 4, None, 0, None) == -1
    assert L.moe_mk_plan(None, 8, 2, 256, 512, 0) == -1
    p = ctypes.c_void_p()
    assert L.moe_mk_plan(ctypes.byref(p), 8, 2, 256, 512, 7) == -1           # bad schedule
    assert L.moe_mk_plan(ctypes.byref(p), 0, 1, 256, 512, 0) == -2           # E = 0
    assert L.moe_mk_plan(ctypes.byref(p), 300, 2, 256, 512, 0) == -2         # E > 256
    assert L.moe_mk_plan(ctypes.byref(p), 8, 9, 256, 512, 0) == -2           # k > E
    assert L.moe_mk_plan(ctypes.byref(p), 32, 17, 256, 512, 0) == -2         # k > 16
    assert L.moe_mk_plan(ctypes.byref(p), 8, 2, 200, 512, 0) == -2           # d not a multiple of 128
    assert L.moe_mk_plan(ctypes.byref(p), 8, 2, 256, 100, 0) == -2           # f not a multiple of 128
    assert L.moe_mk_plan_info(None, b"E") == -1
    assert L.moe_mk_plan_set_debug(None, 0, 0) == -1
    L.moe_mk_plan_destroy(None)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_plan_without_a_gpu_fails_cleanly(L):
    p = ctypes.c_void_p()
    rc = L.moe_mk_plan(ctypes.byref(p), 8, 2, 256, 512, 0)
    assert rc in (-2, -4) and not p.value


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(mk, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(mk, "_lib", None)
    with pytest.raises(RuntimeError):
        mk.lib()


def test_every_kernel_launched_by_the_host_exists_in_the_device_code(tmp_path):
    # A kernel whose host-side and device-side signatures mangle differently would be
    # launched under a name the code object does not contain.
    fb, co = tmp_path / "fatbin.bin", tmp_path / "dev.co"
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", LIB, str(fb)], check=True)
    subprocess.run(["/opt/rocm/llvm/bin/clang-offload-bundler", "--unbundle", "--type=o", f"--input={fb}",
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"], check=True)
    syms = subprocess.run(["/opt/rocm/llvm/bin/llvm-readelf", "--syms", str(co)], capture_output=True, text=True,
                          check=True).stdout
    device = {line.split()[-1] for line in syms.splitlines() if " FUNC " in line}
    host = subprocess.run(["nm", LIB], capture_output=True, text=True, check=True).stdout
    stubs = [line.split()[-1] for line in host.splitlines() if "__device_stub__" in line]
    assert stubs
    for stub in stubs:
        # _ZN2mk<len>__device_stub__<name>... -> _ZN2mk<len'><name>...
        import re
        m = re.match(r"(_ZN\d+\w+?)(\d+)__device_stub__(\w+)", stub)
        assert m, stub
        prefix, n, rest = m.group(1), int(m.group(2)), m.group(3)
        name_len = n - len("__device_stub__")
        kernel = f"{prefix}{name_len}{rest}"
        assert kernel in device, f"{kernel} (host stub {stub}) missing from the device code object"


def test_binding_rejects_mis_shaped_tensors():
    # the C ABI sees only pointers, so the binding checks every shape against the plan's
    # (E, k, d, f) and B before anything reaches the library (CPU tensors: the check comes
    # before any device pointer is taken)
    E, k, d, f, B = 4, 2, 128, 256, 5
    fake_plan = 0x7E57
    mk._SHAPES[fake_plan] = (E, k, d, f)
    try:
        t = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt)
        good = dict(x=t(B, d), Wr=t(d, E, dt=torch.float32), router_bias=None, W1=t(E, d, f), W3=t(E, d, f),
                    W2=t(E, f, d), out=t(B, d), B=B, ws=t(64, dt=torch.uint8))
        mk._check_forward_args(fake_plan, **good)
        bad = [("x", t(B, d + 128)), ("x", t(B - 1, d)), ("out", t(B - 1, d)), ("out", t(B, d, 1)),
               ("Wr", t(E, d, dt=torch.float32)), ("router_bias", t(E + 1, dt=torch.float32)),
               ("W1", t(E, f, d)), ("W3", t(E - 1, d, f)), ("W2", t(E, d, f)), ("B", -1)]
        for name, val in bad:
            args = dict(good, **{name: val})
            with pytest.raises(ValueError):
                mk.moe_mk_forward(fake_plan, **args)
    finally:
        mk._SHAPES.pop(fake_plan, None)


def test_every_declaration_states_its_source():
    # each function and type of the C ABI carries, in the comment block right above it, a
    # "Source:" line citing the page and section that defines the operation (or saying that
    # it is library bookkeeping with no counterpart on the pages)
    import re
    text = open(mk.HEADER).read()
    body = text[text.index('extern "C" {'):]
    decls = [m for m in re.finditer(r"^(?:typedef [^;{]*\{|typedef struct \w+ \*\w+;|[a-z_][\w ]*\*?\s*(moe_mk_\w+)\s*\()",
                                     body, re.M)]
    covered = {m.group(1) for m in decls if m.group(1)}
    assert covered == set(mk.header_functions())  # every function declaration is checked
    assert len(decls) - len(covered) == 4          # and the four types
    for m in decls:
        before = body[:m.start()]
        block = before[before.rfind("\n/*") + 1:]  # the last comment block that starts a line
        assert "*/" in block, m.group(0)
        # the comment block may be followed by #define lines, but by no other declaration
        between = block[block.index("*/") + 2:]
        assert all(ln.startswith("#define") or ln.startswith(" ") or not ln.strip() for ln in between.splitlines()), \
            (m.group(0), between)
        assert "Source:" in block, f"no Source: line above {m.group(0)!r}"
