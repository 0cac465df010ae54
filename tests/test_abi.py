"""Host-side checks of the C ABI: the library loads, exports every function
include/moe.h declares, sizes workspaces, and rejects bad arguments before
touching the GPU.  No kernel is launched here."""
import ctypes
import os
import re
import subprocess

import pytest

import routing_expert_ffn_amd as moe
from workloads import CONFIGS, TEST_SHAPES

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward", "moe_workspace_size",
              "moe_last_error", "moe_version"):
        assert n in names


def test_library_exports_every_declared_function():
    L = moe.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (moe_\w+)", out))
    assert set(declared_functions()) <= exported
    assert set(moe.EXPORTS) <= exported


def test_config_struct_layout_matches_the_header(tmp_path):
    """The binding's moe_config has the size and field offsets the C compiler
    gives the header's struct (capacity_factor is a double: 8-byte aligned)."""
    fields = [f[0] for f in moe.moe_config._fields_]
    prog = tmp_path / "layout.c"
    prog.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "moe.h"\nint main(void){\n'
                    '  printf("size %zu\\n", sizeof(moe_config));\n' +
                    "".join('  printf("%s %%zu\\n", offsetof(moe_config, %s));\n' % (f, f) for f in fields) +
                    "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)])
    got = dict(line.split() for line in subprocess.check_output([str(exe)], text=True).splitlines())
    assert int(got["size"]) == ctypes.sizeof(moe.moe_config)
    for f in fields:
        assert int(got[f]) == getattr(moe.moe_config, f).offset, f
    assert moe.moe_config.capacity_factor.size == 8


def test_noalloc_checks_its_scratch_limit_before_any_launch():
    """moe_forward_noalloc runs on a 64 MiB static scratch: a layer and batch
    whose workspace is larger is rejected with MOE_ERR_WORKSPACE (and FP8
    layers with MOE_ERR_INVALID_ARG) before any HIP call; T == 0 is a no-op."""
    L = moe.lib()
    nulls = [None] * 12
    cfg = moe.make_config(CONFIGS["deepseek_v3_prefill"])
    assert moe.workspace_size(cfg, 16384) > 64 << 20
    assert L.moe_forward_noalloc(ctypes.byref(cfg), 16384, *nulls, None) == -3
    assert "static scratch" in L.moe_last_error().decode()
    assert moe.workspace_size(cfg, 128) <= 64 << 20
    assert L.moe_forward_noalloc(ctypes.byref(cfg), 0, *nulls, None) == 0
    cfg8 = moe.make_config(CONFIGS["deepseek_v3_decode_fp8"])
    assert L.moe_forward_noalloc(ctypes.byref(cfg8), 128, *nulls, None) == -1


def test_version_and_clean_error_state():
    assert "gfx950" in moe.version()


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_workspace_sizes(name):
    s = CONFIGS[name]
    cfg = moe.make_config(s)
    n = moe.workspace_size(cfg, s.T)
    hsz = {"fp8": 1, "bf16": 2, "f32": 4}[s.dtype]
    rows = s.T * s.k + s.S * s.T
    # at least the SwiGLU activations (E4M3, bf16 or fp32) and the fp32 expert rows
    assert n >= rows * (s.I * hsz + s.H * 4)
    if s.dtype == "fp8":  # and x's E4M3 codes
        assert n >= rows * (s.I + s.H * 4) + s.T * s.H
    assert n % 256 == 0
    assert moe.workspace_size(cfg, 0) < n


def bad(**kw):
    c = moe.make_config(TEST_SHAPES["v3_small"])
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,status", [
    ("n_group", 3, -1),             # does not divide 256
    ("topk_group", 9, -1),          # more groups kept than exist
    ("top_k", 0, -1),
    ("top_k", 40, -2),              # > 32 unsupported
    ("n_routed_experts", 1024, -2),  # > 512 unsupported
    ("hidden_size", 500, -2),       # bf16 needs H % 256
    ("moe_intermediate_size", 100, -2),
    ("scoring", 7, -1),
    ("dtype", 5, -1),
    ("n_shared_experts", -1, -1),
])
def test_invalid_configs_are_rejected(field, value, status):
    c = bad(**{field: value})
    n = ctypes.c_size_t(0)
    st = moe.lib().moe_workspace_size(ctypes.byref(c), 16, ctypes.byref(n))
    assert st == status
    assert moe.lib().moe_last_error().decode()


def test_null_and_short_workspace_rejected_before_launch():
    L = moe.lib()
    c = moe.make_config(TEST_SHAPES["v3_small"])
    # forward with NULL tensors
    st = L.moe_forward(ctypes.byref(c), 16, None, None, None, None, None, None, None, None, None, None, None, None,
                       None, 0, None)
    assert st == -1
    # permute with a too-small workspace (fake, never dereferenced: validation fails first)
    fake = ctypes.c_void_p(256 * 1024)
    st = L.moe_permute(ctypes.byref(c), 16, fake, fake, fake, fake, fake, fake, 256, None)
    assert st == -3
    assert "workspace" in L.moe_last_error().decode()
    # misaligned workspace
    st = L.moe_permute(ctypes.byref(c), 16, fake, fake, fake, fake, fake, ctypes.c_void_p(256 * 1024 + 8),
                       1 << 40, None)
    assert st == -3
    # T < 0
    assert L.moe_combine(ctypes.byref(c), -1, fake, fake, fake, fake, None) == -1


def test_expert_ffn_rejects_x_past_2gib_before_launch():
    """bf16/FP8 expert FFNs address x through a 32-bit buffer resource: a
    batch with 2^31 bytes of x or more is rejected with MOE_ERR_UNSUPPORTED
    before any launch (fake pointers, never dereferenced), one byte less is
    not rejected for its size."""
    L = moe.lib()
    fake = ctypes.c_void_p(256 * 1024)
    for dtype, esz in (("bf16", 2), ("fp8", 1)):
        shape = TEST_SHAPES["v3_small"].with_(dtype=dtype)
        c = moe.make_config(shape)
        T_big = (1 << 31) // (shape.H * esz)          # T * H * esz == 2^31
        if dtype == "bf16":
            st = L.moe_expert_ffn(ctypes.byref(c), T_big, fake, fake, fake, fake, fake, fake, fake, fake, 256, None)
        else:
            st = L.moe_expert_ffn_fp8(ctypes.byref(c), T_big, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                      fake, fake, 256, None)
        assert st == -2 and "2 GiB" in L.moe_last_error().decode(), dtype
        st = L.moe_forward(ctypes.byref(c), T_big, fake, fake, None, None, fake, fake, fake, fake, None, None, None,
                           None, fake, 256, None) if dtype == "bf16" else None
        if st is not None:
            assert st == -2
        # just below the limit the size check passes and the short workspace is what fails
        if dtype == "bf16":
            st = L.moe_expert_ffn(ctypes.byref(c), T_big - 1, fake, fake, fake, fake, fake, fake, fake, fake, 256,
                                  None)
            assert st == -3 and "workspace" in L.moe_last_error().decode()


def test_route_needs_workspace_when_it_computes_bf16_logits():
    """bf16 routing from x writes logits (and K-slice partials) into the
    workspace: a NULL or short workspace is an error before any launch, while
    routing given logits without a capacity limit needs none."""
    L = moe.lib()
    c = moe.make_config(TEST_SHAPES["v3_small"])  # bf16, no capacity limit
    fake = ctypes.c_void_p(256 * 1024)
    st = L.moe_route(ctypes.byref(c), 16, fake, fake, None, None, None, None, fake, fake, None, None, 0, None)
    assert st == -3 and "workspace" in L.moe_last_error().decode()
    st = L.moe_route(ctypes.byref(c), 16, fake, fake, None, None, None, None, fake, fake, None, fake, 256, None)
    assert st == -3


def test_variant_entry_points_validate_before_launch():
    """Hash routing, FP8 and quantisation calls reject bad arguments on the
    host (fake pointers are never dereferenced: validation fails first)."""
    L = moe.lib()
    fake = ctypes.c_void_p(256 * 1024)
    base = TEST_SHAPES["v3_small"]
    # hash routing with a re-route capacity: no next-best expert exists
    c = moe.make_config(base.with_(capacity_factor=1.0, drop_tokens=False))
    st = L.moe_route_hash(ctypes.byref(c), 16, fake, fake, None, fake, None, fake, fake, 10, fake, fake, None, fake,
                          1 << 40, None)
    assert st == -1 and "drop_tokens" in L.moe_last_error().decode()
    # negative vocabulary, missing token ids
    c = moe.make_config(base)
    assert L.moe_route_hash(ctypes.byref(c), 16, fake, fake, None, fake, None, fake, fake, -1, fake, fake, None,
                            None, 0, None) == -1
    assert L.moe_route_hash(ctypes.byref(c), 16, fake, fake, None, fake, None, None, fake, 10, fake, fake, None,
                            None, 0, None) == -1
    # FP8 entry points need dtype MOE_FP8, and MOE_FP8 layers need them
    c = moe.make_config(base)
    st = L.moe_forward_fp8(ctypes.byref(c), 16, fake, fake, None, None, fake, fake, fake, fake, fake, fake, fake,
                           None, None, None, None, fake, 1 << 40, None)
    assert st == -1 and "MOE_FP8" in L.moe_last_error().decode()
    c8 = moe.make_config(base.with_(dtype="fp8"))
    st = L.moe_forward(ctypes.byref(c8), 16, fake, fake, None, None, fake, fake, fake, fake, None, None, None, None,
                       fake, 1 << 40, None)
    assert st == -1 and "moe_forward_fp8" in L.moe_last_error().decode()
    st = L.moe_expert_ffn(ctypes.byref(c8), 16, fake, fake, fake, fake, fake, fake, fake, fake, 1 << 40, None)
    assert st == -1
    st = L.moe_forward_fp8(ctypes.byref(c8), 16, fake, fake, None, None, fake, None, fake, fake, fake, fake, fake,
                           None, None, None, None, fake, 1 << 40, None)
    assert st == -1 and "scale" in L.moe_last_error().decode()
    # quantisation: K must be a multiple of 128, the scale stride cover K/128
    assert L.moe_quantize_fp8(4, 100, fake, fake, fake, 1, None) == -1
    assert L.moe_quantize_fp8(4, 256, fake, fake, fake, 1, None) == -1
    assert L.moe_quantize_fp8(-1, 256, fake, fake, fake, 2, None) == -1
    assert L.moe_quantize_fp8(0, 256, None, None, None, 2, None) == 0


def test_empty_batch_is_a_noop():
    L = moe.lib()
    c = moe.make_config(TEST_SHAPES["v3_small"])
    assert L.moe_forward(ctypes.byref(c), 0, None, None, None, None, None, None, None, None, None, None, None, None,
                         None, 0, None) == 0
    assert L.moe_combine(ctypes.byref(c), 0, None, None, None, None, None) == 0


def test_product_and_oracle_are_separate():
    """The GPU package never reaches the oracle, and the oracle never includes
    or imports the GPU library."""
    pkg = os.path.join(ROOT, "routing_expert_ffn_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text, f
    osrc = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert "#include \"" not in osrc and "moe.h" not in osrc
    opy = open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    assert "routing_expert_ffn_amd" not in opy


def test_every_kernel_launch_stub_is_defined():
    """A kernel whose host-side stub was dropped by the compiler leaves an
    undefined __device_stub__ symbol and the library fails to load on a GPU
    host; catch it at build time."""
    out = subprocess.run(["nm", "-u", moe.LIB_PATH], capture_output=True, text=True).stdout
    assert "__device_stub__" not in out
