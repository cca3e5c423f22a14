"""The C ABI without a GPU: the library loads and exports every function
include/ar.h declares, the host-only calls agree with the oracle's chunk
plan, and every argument error is reported before anything touches a device.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle.ring import chunk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from ring_allreduce_reduction_virtual_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return _lib.lib()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "ar.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ar_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported(lib):
    from ring_allreduce_reduction_virtual_amd import _lib

    declared = _declared_functions()
    assert len(declared) >= 11
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(_lib.EXPORTS) == declared


def test_chunk_range_matches_the_oracle(lib):
    import ring_allreduce_reduction_virtual_amd as ar

    for n in (1, 2, 3, 5, 8, 16, 64, 128):
        for count in (0, 1, n - 1, n, n + 1, 1003, (1 << 26) + 7, (1 << 40) + 3):
            for c in sorted({0, 1 % n, n // 2, n - 1}):
                assert ar.ar_chunk_range(c, count, n) == chunk(c, n, count)


def test_error_strings(lib):
    for code, text in ((0, b"success"), (1, b"invalid argument"), (3, b"HIP runtime error")):
        assert lib.ar_get_error_string(code) == text
    assert [lib.ar_dtype_size(d) for d in range(5)] == [4, 2, 4, 2, 2]
    assert lib.ar_dtype_size(7) == 0


def test_workspace_sizes(lib):
    import ring_allreduce_reduction_virtual_amd as ar

    assert ar.ar_workspace_bytes("allreduce", "ring", 1000, "f32", 8) == 0
    assert ar.ar_workspace_bytes("reduce_scatter", "fused", 1000, "f32", 8) == 0
    assert ar.ar_workspace_bytes("reduce_scatter", "ring", 1000, "f32", 2) == 0
    assert ar.ar_workspace_bytes("reduce_scatter", "ring", 1000, "bf16", 8) >= 2000
    with pytest.raises(ValueError):
        ar.ar_workspace_bytes("reduce_scatter", "ring", 1000, "f32", 0)


def _ptrs(vals):
    arr = (ctypes.c_void_p * len(vals))()
    for i, v in enumerate(vals):
        arr[i] = v
    return arr


# fake device addresses: validation only compares them, never dereferences
BASE = 0x7F0000000000


def _call_ar(lib, sends, recvs, count, dtype=0, op=0, n=None):
    n = len(sends) if n is None else n
    return lib.ar_allreduce(_ptrs(sends), _ptrs(recvs), count, dtype, op, n, None)


def test_argument_errors_are_caught_on_the_host(lib):
    S = 1 << 20
    sends = [BASE + r * S for r in range(4)]
    recvs = [BASE + (8 + r) * S for r in range(4)]
    assert lib.ar_allreduce(None, _ptrs(recvs), 10, 0, 0, 4, None) == 1
    assert _call_ar(lib, sends, recvs, 10, n=0) == 1
    assert _call_ar(lib, sends * 33, recvs * 33, 10, n=129) == 1
    assert _call_ar(lib, sends, recvs, 10, dtype=5) == 1
    assert _call_ar(lib, sends, recvs, 10, dtype=-1) == 1
    assert _call_ar(lib, sends, recvs, 10, op=5) == 1
    assert b"op" in lib.ar_get_last_error_detail()
    assert _call_ar(lib, [0] + sends[1:], recvs, 10) == 1               # null buffer
    assert _call_ar(lib, [sends[0] + 2] + sends[1:], recvs, 10) == 1    # not 4-byte aligned
    assert _call_ar(lib, sends, [recvs[0], recvs[0] + 8] + recvs[2:], 10) == 1   # receive buffers overlap
    assert _call_ar(lib, sends, [sends[1]] + recvs[1:], 10) == 1         # recv[0] is rank 1's send
    assert _call_ar(lib, sends, recvs, (1 << 64) // 100) == 1            # count too large
    # empty work is a success without touching a device
    assert _call_ar(lib, sends, recvs, 0) == 0
    assert _call_ar(lib, [0] * 4, [0] * 4, 0) == 0
    assert lib.ar_get_last_error_detail() == b""


def test_noalloc_refuses_an_oversized_workspace_on_the_host(lib):
    """ar_reduce_scatter_noalloc checks the workspace a call needs against its fixed
    array before anything else: too large is an argument error, with no GPU touched."""
    from ring_allreduce_reduction_virtual_amd import _lib

    text = open(os.path.join(ROOT, "include", "ar.h")).read()
    m = re.search(r"#define\s+AR_NOALLOC_SCRATCH_BYTES\s+\((\d+)ull\s*<<\s*(\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES
    n = 3
    count = (_lib.NOALLOC_SCRATCH_BYTES - 1024) // 4 + 1           # float32 ring: one element too many
    sends = [BASE + r * (1 << 30) for r in range(n)]
    recvs = [BASE + (8 + r) * (1 << 30) for r in range(n)]
    for algo in ("ring", "ring_pipelined"):
        rc = lib.ar_reduce_scatter_noalloc(_ptrs(sends), _ptrs(recvs), count, 0, 0, n, _lib.ALGOS[algo], None)
        assert rc == 1 and b"scratch" in lib.ar_get_last_error_detail()
    # arguments the ordinary validation rejects are reported as it reports them
    assert lib.ar_reduce_scatter_noalloc(_ptrs(sends), _ptrs(recvs), 10, 0, 9, n, _lib.ALGOS["ring"], None) == 1
    assert b"op" in lib.ar_get_last_error_detail()
    assert lib.ar_reduce_scatter_noalloc(_ptrs(sends), _ptrs(recvs), 10, 0, 0, n, _lib.ALGOS["tree"], None) == 2
    # empty work succeeds without a device
    assert lib.ar_reduce_scatter_noalloc(_ptrs(sends), _ptrs(recvs), 0, 0, 0, n, _lib.ALGOS["ring"], None) == 0


def test_in_place_layouts_are_accepted_others_rejected(lib):
    """Validation of the aliasing rules, stopped before any launch by count checks."""
    n, count = 4, 1000
    S = 1 << 20
    sends = [BASE + r * S for r in range(n)]
    starts = [chunk(r, n, count)[0] for r in range(n)]
    # reduce-scatter: recv[r] == send[r] + start(r) is in place; recv[r] == send[r] + start(r) + 1 is not
    shards_ok = [sends[r] + 4 * starts[r] for r in range(n)]
    shards_bad = [sends[r] + 4 * starts[r] + 4 for r in range(n)]
    rs = lib.ar_reduce_scatter_ex
    # with algo = 99 (unknown) the call stops after the aliasing checks would have passed
    assert rs(_ptrs(sends), _ptrs(shards_ok), count, 0, 0, n, 99, None, 0, None) == 1
    assert b"algo" in lib.ar_get_last_error_detail()
    assert rs(_ptrs(sends), _ptrs(shards_bad), count, 0, 0, n, 0, None, 0, None) == 1
    assert b"overlaps" in lib.ar_get_last_error_detail()
    # all-gather: send[r] == recv[r] + start(r)
    recvs = [BASE + (8 + r) * S for r in range(n)]
    ag = lib.ar_all_gather_ex
    assert ag(_ptrs([recvs[r] + 4 * starts[r] + 4 for r in range(n)]), _ptrs(recvs), count, 0, n, 0, None, 0, None) == 1
    assert b"overlaps" in lib.ar_get_last_error_detail()


def test_missing_library_fails_loudly(monkeypatch):
    from ring_allreduce_reduction_virtual_amd import _lib

    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libar.so")
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.lib()


def test_product_and_oracle_do_not_import_each_other():
    pkg = os.path.join(ROOT, "ring_allreduce_reduction_virtual_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", src, flags=re.M), f
                assert "oracle/" not in src, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            src = open(os.path.join(ROOT, "oracle", f)).read()
            assert "ring_allreduce_reduction_virtual_amd" not in src, f
            assert not re.search(r"^\s*(from|import)\s+inputs\b", src, flags=re.M), f


def test_binding_has_every_c_name():
    """The Python binding offers a function of the same name for every entry point ar.h declares."""
    import ring_allreduce_reduction_virtual_amd as ar
    from ring_allreduce_reduction_virtual_amd import _lib

    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "ar.h")).read(), flags=re.S)
    declared = set(re.findall(r"\b(ar_[a-z_]+)\s*\(", text))
    assert declared == set(_lib.EXPORTS)
    assert all(callable(getattr(ar, name, None)) for name in declared), sorted(
        n for n in declared if not callable(getattr(ar, n, None)))


def test_bench_uses_the_oracle_only_for_its_cpu_baseline():
    """bench.py imports the oracle only inside its cpu_baseline_* functions, which
    time it; results are checked by the GPU tests, never by the benchmark."""
    import ast

    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    allowed = set()
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef) and fn.name.startswith("cpu_baseline_"):
            allowed.update(id(n) for n in ast.walk(fn))
    for node in ast.walk(tree):
        names = ([a.name for a in node.names] if isinstance(node, ast.Import)
                 else [node.module or ""] if isinstance(node, ast.ImportFrom) else [])
        if any(n == "oracle" or n.startswith("oracle.") for n in names):
            assert id(node) in allowed, f"bench.py imports the oracle at line {node.lineno}"


def test_input_generators_are_seeded_and_prefix_stable():
    from inputs import WORKLOADS, make_inputs, make_rank

    w = WORKLOADS["c5"]
    a = make_rank(w, 3, count=5000)
    b = make_rank(w, 3, count=5000)
    assert np.array_equal(a, b)
    assert np.array_equal(make_rank(w, 3, count=2000), a[:2000])
    xs = make_inputs(WORKLOADS["c1"])
    assert len(xs) == 4 and all(x.dtype == np.float32 and x.min() >= -8 and x.max() <= 8 for x in xs)
    assert all(np.all(x == np.round(x)) for x in xs)
    c3 = make_rank(WORKLOADS["c3"], 0, count=100000)
    assert c3.dtype == np.uint16
    c4 = make_rank(WORKLOADS["c4"], 0, count=100000)
    assert c4.dtype == np.int32 and c4.min() < -(2**30) and c4.max() > 2**30
    frac = np.mean(np.abs(make_rank(w, 0, count=200000)) > 100)
    assert 0.005 < frac < 0.015          # about 1% outliers scaled by 1e4


def test_persistent_plan_host_side(lib):
    """Plan creation validates like the one-shot calls; empty work plans no launch."""
    S = 1 << 20
    sends = [BASE + r * S for r in range(4)]
    recvs = [BASE + (8 + r) * S for r in range(4)]
    plan = ctypes.c_void_p(12345)
    # invalid op: error, and the plan handle is cleared
    rc = lib.ar_allreduce_init(_ptrs(sends), _ptrs(recvs), 10, 0, 9, 4, 0, None, 0, ctypes.byref(plan))
    assert rc == 1 and plan.value is None
    # overlapping receive buffers
    rc = lib.ar_allreduce_init(_ptrs(sends), _ptrs([recvs[0]] * 4), 10, 0, 0, 4, 0, None, 0, ctypes.byref(plan))
    assert rc == 1 and b"overlaps" in lib.ar_get_last_error_detail()
    # ring reduce-scatter without its workspace
    rc = lib.ar_reduce_scatter_init(_ptrs(sends), _ptrs(recvs), 1000, 0, 0, 4, 1, None, 0, ctypes.byref(plan))
    assert rc == 1 and b"workspace" in lib.ar_get_last_error_detail()
    # count == 0: a valid plan that launches nothing and starts without a device
    rc = lib.ar_allreduce_init(_ptrs(sends), _ptrs(recvs), 0, 0, 0, 4, 1, None, 0, ctypes.byref(plan))
    assert rc == 0 and plan.value
    assert lib.ar_plan_num_launches(plan) == 0
    assert lib.ar_plan_start(plan, None) == 0
    assert lib.ar_plan_free(plan) == 0
    assert lib.ar_plan_num_launches(None) == -1
    assert lib.ar_plan_start(None, None) == 1
    assert lib.ar_plan_limit_blocks(None, 4) == 1
    assert lib.ar_plan_free(None) == 0
    assert lib.ar_allreduce_init(_ptrs(sends), _ptrs(recvs), 0, 0, 0, 4, 0, None, 0, None) == 1


def test_workspace_sizes_for_float32_partials(lib):
    import ring_allreduce_reduction_virtual_amd as ar

    assert ar.ar_workspace_bytes("allreduce", "ring", 1000, "bf16acc32", 8) == 1000 * 4 + 1024
    assert ar.ar_workspace_bytes("allreduce", "ring", 1000, "bf16acc32", 2) == 0
    assert ar.ar_workspace_bytes("allreduce", "fused", 1000, "bf16acc32", 8) == 0
    assert ar.ar_workspace_bytes("allreduce", "ring", 1000, "f16", 8) == 0
    assert ar.ar_workspace_bytes("reduce_scatter", "ring", 1000, "bf16acc32", 8) == 1000 * 4 + 1024
    assert ar.ar_workspace_bytes("reduce_scatter", "ring", 1000, "f16", 8) == 1000 * 2 + 1024
    assert ar.ar_workspace_bytes("all_gather", "ring", 1000, "bf16acc32", 8) == 0


def test_plain_c_consumer_of_the_header(tmp_path, lib):
    """include/ar.h compiles as C and its host-side calls behave from a C program."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    from ring_allreduce_reduction_virtual_amd import _lib

    exe = tmp_path / "abi_host_check"
    libdir = os.path.dirname(_lib.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c_abi", "abi_host_check.c"),
           "-L", libdir, "-l:libar.so", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stderr
    assert "passed" in res.stdout


def test_tree_algorithm_host_rules(lib):
    """Tree-order algorithms: AllReduce only, power-of-two N where the schedule needs it,
    and float32 partial slabs for the staged forms of bf16acc32."""
    import ring_allreduce_reduction_virtual_amd as ar
    from ring_allreduce_reduction_virtual_amd import _lib

    slab = ((1000 * 4 + 255) // 256) * 256
    for algo in ("tree_steps", "recursive_doubling", "halving_doubling_steps", "double_binary_tree_steps"):
        assert ar.ar_workspace_bytes("allreduce", algo, 1000, "bf16acc32", 8) == 8 * slab + 1024
        assert ar.ar_workspace_bytes("allreduce", algo, 1000, "bf16acc32", 1) == 0
        assert ar.ar_workspace_bytes("allreduce", algo, 1000, "bf16", 8) == 0
        assert ar.ar_workspace_bytes("allreduce", algo, 0, "bf16acc32", 8) == 0
    for algo in ("tree", "halving_doubling", "double_binary_tree"):
        assert ar.ar_workspace_bytes("allreduce", algo, 1000, "bf16acc32", 8) == 0
    S = 1 << 20
    sends = [BASE + r * S for r in range(8)]
    recvs = [BASE + (16 + r) * S for r in range(8)]
    for name in _lib.TREE_ALGOS:
        algo = _lib.ALGOS[name]
        # reduce-scatter and all-gather have no tree form
        assert lib.ar_reduce_scatter_ex(_ptrs(sends), _ptrs(recvs), 100, 0, 0, 8, algo, None, 0, None) == 2
        assert b"AllReduce only" in lib.ar_get_last_error_detail()
        assert lib.ar_all_gather_ex(_ptrs(sends), _ptrs(recvs), 100, 0, 8, algo, None, 0, None) == 2
        # six ranks: the binomial tree and the double binary tree are defined, the rest need a power of two
        rc = lib.ar_allreduce_ex(_ptrs(sends[:6]), _ptrs(recvs[:6]), 100, 0, 0, 6, algo, None, 0, None)
        if name in ("tree", "tree_steps", "double_binary_tree", "double_binary_tree_steps"):
            assert rc in (0, 3)   # valid: reaches the device (none here) or succeeds
        else:
            assert rc == 2 and b"power-of-two" in lib.ar_get_last_error_detail()
        # empty work plans no launch
        plan = ctypes.c_void_p()
        assert lib.ar_allreduce_init(_ptrs(sends), _ptrs(recvs), 0, 0, 0, 8, algo, None, 0, ctypes.byref(plan)) == 0
        assert lib.ar_plan_num_launches(plan) == 0
        assert lib.ar_plan_free(plan) == 0
    # the staged forms of bf16acc32 need their workspace
    for name in ("tree_steps", "double_binary_tree_steps"):
        rc = lib.ar_allreduce_ex(_ptrs(sends), _ptrs(recvs), 100, 4, 0, 8, _lib.ALGOS[name], None, 0, None)
        assert rc == 1 and b"workspace" in lib.ar_get_last_error_detail()


def test_pipelined_ring_host_rules(lib):
    """The pipelined ring takes every collective and needs the ring's workspace
    where the ring's launches do (reduce-scatter; AllReduce of float32 partials),
    none elsewhere; a missing workspace is refused before anything launches."""
    import ring_allreduce_reduction_virtual_amd as ar
    from ring_allreduce_reduction_virtual_amd import _lib

    for coll, dt in (("allreduce", "f32"), ("allreduce", "bf16"), ("allreduce", "bf16acc32"),
                     ("reduce_scatter", "f32"), ("reduce_scatter", "bf16acc32"), ("all_gather", "bf16")):
        for n in (2, 3, 8, 64):
            assert (ar.ar_workspace_bytes(coll, "ring_pipelined", 1000, dt, n)
                    == ar.ar_workspace_bytes(coll, "ring", 1000, dt, n)), (coll, dt, n)
    algo = _lib.ALGOS["ring_pipelined"]
    S = 1 << 20
    sends = [BASE + r * S for r in range(8)]
    recvs = [BASE + (16 + r) * S for r in range(8)]
    rc = lib.ar_reduce_scatter_ex(_ptrs(sends), _ptrs(recvs), 100, 0, 0, 8, algo, None, 0, None)
    assert rc == 1 and b"workspace" in lib.ar_get_last_error_detail()
    rc = lib.ar_allreduce_ex(_ptrs(sends), _ptrs(recvs), 100, 4, 0, 8, algo, None, 0, None)
    assert rc == 1 and b"workspace" in lib.ar_get_last_error_detail()
    for init in ("ar_allreduce_init", "ar_reduce_scatter_init"):
        plan = ctypes.c_void_p()
        assert getattr(lib, init)(_ptrs(sends), _ptrs(recvs), 0, 0, 0, 8, algo, None, 0, ctypes.byref(plan)) == 0
        assert lib.ar_plan_num_launches(plan) == 0
        assert lib.ar_plan_free(plan) == 0
    plan = ctypes.c_void_p()
    assert lib.ar_all_gather_init(_ptrs(sends), _ptrs(recvs), 0, 0, 8, algo, None, 0, ctypes.byref(plan)) == 0
    assert lib.ar_plan_num_launches(plan) == 0
    assert lib.ar_plan_free(plan) == 0


@pytest.mark.parametrize("name", ["ring_persistent"])
def test_one_launch_ring_host_rules(lib, name):
    """The persistent ring: AllReduce only, no float32-partials form, no workspace."""
    import ring_allreduce_reduction_virtual_amd as ar
    from ring_allreduce_reduction_virtual_amd import _lib

    algo = _lib.ALGOS[name]
    assert ar.ar_workspace_bytes("allreduce", name, 1000, "bf16", 8) == 0
    S = 1 << 20
    sends = [BASE + r * S for r in range(8)]
    recvs = [BASE + (16 + r) * S for r in range(8)]
    assert lib.ar_reduce_scatter_ex(_ptrs(sends), _ptrs(recvs), 100, 0, 0, 8, algo, None, 0, None) == 2
    assert lib.ar_all_gather_ex(_ptrs(sends), _ptrs(recvs), 100, 0, 8, algo, None, 0, None) == 2
    rc = lib.ar_allreduce_ex(_ptrs(sends), _ptrs(recvs), 100, 4, 0, 8, algo, None, 0, None)
    assert rc == 2 and b"float32 partials" in lib.ar_get_last_error_detail()
    plan = ctypes.c_void_p()
    assert lib.ar_allreduce_init(_ptrs(sends), _ptrs(recvs), 0, 0, 0, 8, algo, None, 0, ctypes.byref(plan)) == 0
    assert lib.ar_plan_num_launches(plan) == 0
    assert lib.ar_plan_free(plan) == 0


def test_binding_tables_match_the_header_enums():
    """Every name the Python binding maps to an enum value carries the value ar.h gives it."""
    from ring_allreduce_reduction_virtual_amd import _lib

    text = open(os.path.join(ROOT, "include", "ar.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    values = {m.group(1): int(m.group(2)) for m in re.finditer(r"\b(AR_[A-Z0-9_]+)\s*=\s*(\d+)", text)}
    dtypes = {"f32": "AR_FLOAT32", "bf16": "AR_BFLOAT16", "i32": "AR_INT32", "f16": "AR_FLOAT16",
              "bf16acc32": "AR_BFLOAT16_ACC_F32"}
    assert {k: values[v] for k, v in dtypes.items()} == _lib.DTYPES
    assert {k: values["AR_" + k.upper()] for k in _lib.OPS} == _lib.OPS
    assert {k: values["AR_ALGO_" + k.upper()] for k in _lib.ALGOS} == _lib.ALGOS
    assert {k: values["AR_COLL_" + k.upper()] for k in _lib.COLLS} == _lib.COLLS
    assert {values[v]: v for v in _lib.RESULT_NAMES.values()} == _lib.RESULT_NAMES
    # every algorithm the header declares is reachable from Python
    assert sorted(v for k, v in values.items() if k.startswith("AR_ALGO_")) == sorted(_lib.ALGOS.values())
    defines = dict(re.findall(r"#define\s+(AR_[A-Z_]+)\s+(\d+)", text))
    assert int(defines["AR_MAX_RANKS"]) == _lib.MAX_RANKS
