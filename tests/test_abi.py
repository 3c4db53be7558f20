"""The C-ABI library loads, exports every symbol include/lbt.h declares, and
its host-side checks and size queries behave (no GPU work is launched)."""
import ctypes
import os
import re

import pytest

import oracle
import load_balanced_token_amd as lbt
from load_balanced_token_amd import binding
from workloads import WORKLOADS

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "lbt.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(lbt_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    L = lbt.lib()
    names = declared_functions()
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    assert L.lbt_version() == 4


def test_sizes_match_oracle_capacity_for_every_workload():
    for name, w in WORKLOADS.items():
        z = lbt.query_sizes(lbt.Shape(w.E, w.K, w.R, w.S, w.H, w.B, w.blk))
        assert z["C"] == oracle.capacity(w.E, w.K, w.S, w.blk), name
        assert z["P"] == w.P and z["N"] == w.N and z["SK"] == w.SK
        assert z["n_blocks"] * w.blk == z["C"]
        nh = w.E // w.R
        assert z["max_seg"] == nh + min(w.E - nh, w.SK)
        assert z["n_tiles"] == w.R * -(-w.S // z["tile_tokens"])
        # per-expert counts of every 32-token sub-tile, then a prefix per tile
        assert z["work_words"] == w.E * (w.R * -(-w.S // 32) + z["n_tiles"])
        # offsets are increasing and the blob ends at plan_words
        offs = [z[k] for k in binding._SIZE_FIELDS if k.startswith("off_")]
        assert offs == sorted(offs) and offs[-1] < z["plan_words"]


@pytest.mark.parametrize("name,x", [("dsv3", 2), ("wideep", 3), ("decode128", 2), ("tiny", 4)])
def test_sizes_with_a_larger_threshold_bound(name, x):
    """tau_max sizes the static capacity like the oracle's capacity()."""
    w = WORKLOADS[name]
    z = lbt.query_sizes(lbt.Shape(w.E, w.K, w.R, w.S, w.H, w.B, w.blk, tau_max=x * w.SK))
    assert z["C"] == oracle.capacity(w.E, w.K, w.S, w.blk, 0, x * w.SK)
    nh = w.E // w.R
    assert z["max_seg"] == nh + min(w.E - nh, x * w.SK)


@pytest.mark.parametrize("kw,code", [
    (dict(E=10, R=4), -1), (dict(K=9), -1), (dict(H=60), -1), (dict(H=0), -1),
    (dict(blk=0), -1), (dict(S=-1), -1), (dict(score_fn=5), -1), (dict(cap=17), -1),
    (dict(E=1024, R=8), -3), (dict(K=65, E=128, R=8), -3), (dict(blk=2048), -3),
    (dict(tau_max=15), -1), (dict(tau_max=1 << 30), -1), (dict(tau_max=-2), -1),
])
def test_invalid_shapes_are_rejected(kw, code):
    base = dict(E=8, K=2, R=4, S=8, H=64, B=1, blk=16, score_fn=1, renorm=0, cap=0, tau_max=0)
    base.update(kw)
    sh = binding.LbtShape(*[base[f] for f in ("E", "K", "R", "S", "H", "B", "blk",
                                              "score_fn", "renorm", "cap", "tau_max")])
    z = binding.LbtSizes()
    assert lbt.lib().lbt_query_sizes(ctypes.byref(sh), ctypes.byref(z)) == code
    assert lbt.lib().lbt_strerror(code)


def test_host_checks_reject_bad_pointers_before_any_launch():
    """Null or misaligned pointers are refused on the host (nothing runs)."""
    L = lbt.lib()
    sh = lbt.Shape(E=8, K=2, R=4, S=8, H=64, B=1, blk=16).c()
    P = ctypes.c_void_p
    assert L.lbt_dispatch(ctypes.byref(sh), P(0x1002), P(0x2000), P(0x3000), None) == -1
    assert L.lbt_dispatch(ctypes.byref(sh), None, P(0x2000), P(0x3000), None) == -1
    assert L.lbt_combine(ctypes.byref(sh), P(0x1000), P(0x2000), P(0x3000), 0, P(0x4008), None) == -1
    assert L.lbt_combine(ctypes.byref(sh), P(0x1000), P(0x2000), P(0x3000), 7, P(0x4000), None) == -1
    assert L.lbt_plan_balance(ctypes.byref(sh), None, P(0x1000), None, None) == -1
    assert L.lbt_plan_quota(ctypes.byref(sh), None, P(0x1000), None, None) == -1
    assert L.lbt_plan_quota(ctypes.byref(sh), P(0x1000), None, None, None) == -1
    assert L.lbt_route_topk(ctypes.byref(sh), None, None, P(1), P(2), P(3), P(4), None) == -1
    assert L.lbt_route_plan(ctypes.byref(sh), P(1), None, P(1), P(2), P(3), P(4), None, None,
                            None) == -1
    assert L.lbt_route_plan(ctypes.byref(sh), None, None, P(1), P(2), P(3), P(4), P(5), None,
                            None) == -1
    assert L.lbt_front(ctypes.byref(sh), P(1), None, P(1), P(2), P(3), P(4), P(5), None, P(6),
                       P(7), P(8), None, None) == -1
    assert L.lbt_align_sort(ctypes.byref(sh), P(1), P(2), None, P(3), P(4), P(5), P(6), None, None) == -1
    assert L.lbt_histogram(None, P(1), P(2), P(3), None, None) == -1
    # align + dispatch: null and misaligned rows, missing outputs
    ad = lambda *a: L.lbt_align_dispatch(ctypes.byref(sh), *a, None)   # noqa: E731
    assert ad(P(1), P(2), P(3), P(0x1008), P(4), P(5), P(6), P(7), P(0x2000), None) == -1
    assert ad(P(1), P(2), P(3), P(0x1000), P(4), P(5), P(6), P(7), P(0x2004), None) == -1
    assert ad(P(1), P(2), P(3), None, P(4), P(5), P(6), P(7), P(0x2000), None) == -1
    assert ad(P(1), P(2), P(3), P(0x1000), P(4), P(5), P(6), P(7), None, None) == -1
    assert ad(P(1), P(2), None, P(0x1000), P(4), P(5), P(6), P(7), P(0x2000), None) == -1
    # front + dispatch: the same, and the front's own arguments
    fd = lambda *a: L.lbt_front_dispatch(ctypes.byref(sh), *a, None)   # noqa: E731
    assert fd(P(1), None, P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), P(9), P(0x1008),
              P(0x2000), None) == -1
    assert fd(P(1), None, P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), P(9), P(0x1000),
              None, None) == -1
    assert fd(None, None, P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), P(9), P(0x1000),
              P(0x2000), None) == -1
    assert fd(P(1), None, P(1), P(2), None, P(4), P(5), P(6), P(7), P(8), P(9), P(0x1000),
              P(0x2000), None) == -1
    # training side: row sizes, null and misaligned pointers
    assert L.lbt_prefetch_weights(ctypes.byref(sh), P(0x1000), P(0x2000), P(0x3000), 24, None) == -1
    assert L.lbt_prefetch_weights(ctypes.byref(sh), P(0x1000), P(0x2008), P(0x3000), 32, None) == -1
    assert L.lbt_prefetch_weights(ctypes.byref(sh), None, P(0x2000), P(0x3000), 32, None) == -1
    assert L.lbt_prefetch_weights(ctypes.byref(sh), P(0x1000), P(0x2000), P(0x3000), 0, None) == -1
    assert L.lbt_reduce_grad(ctypes.byref(sh), P(0x1000), P(0x2000), P(0x3000), 6, None) == -1
    assert L.lbt_reduce_grad(ctypes.byref(sh), P(0x1000), None, P(0x3000), 8, None) == -1
    assert L.lbt_combine_bwd(ctypes.byref(sh), P(0x1000), P(0x2000), P(0x3000), 0, P(0x4000),
                             P(0x5008), P(0x6000), None) == -1
    assert L.lbt_combine_bwd(ctypes.byref(sh), P(0x1000), P(0x2000), P(0x3000), 3, P(0x4000),
                             P(0x5000), P(0x6000), None) == -1
    assert L.lbt_combine_bwd(ctypes.byref(sh), P(0x1000), P(0x2000), P(0x3000), 0, P(0x4000),
                             P(0x5000), None, None) == -1
    assert L.lbt_dispatch_bwd(ctypes.byref(sh), P(0x1000), P(0x2000), 0, P(0x3004), None) == -1
    assert L.lbt_dispatch_bwd(ctypes.byref(sh), P(0x1000), P(0x2000), 9, P(0x3000), None) == -1


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 exits with a message (no GPU
    needed to check it)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_binding_structs_follow_the_header():
    """The binding's ABI version, lbt_sizes field order and header word
    indices are those include/lbt.h declares (the ctypes structs would
    misread the library otherwise)."""
    from load_balanced_token_amd import binding as b
    h = open(HEADER).read()
    assert int(re.search(r"#define LBT_VERSION (\d+)", h).group(1)) == b.ABI_VERSION
    body = h[h.index("typedef struct lbt_sizes {"):h.index("} lbt_sizes;")]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = []
    for decl in re.findall(r"int64_t\s+([^;]+);", body):
        fields += [f.strip() for f in decl.split(",")]
    assert tuple(fields) == b._SIZE_FIELDS
    for name, val in re.findall(r"#define LBT_HDR_(\w+) (\d+)", h):
        if name != "WORDS":
            assert getattr(b, "HDR_" + name) == int(val), name
    codes = dict(re.findall(r"#define LBT_(OK|E[A-Z]+) \(?(-?\d+)\)?", h))
    assert codes and {k: int(v) for k, v in codes.items()} == \
        {k: getattr(b, k) for k in codes}


def test_last_hip_error_starts_clean():
    """Before any failed launch the calling thread's HIP error is hipSuccess
    (a string lookup: no device needed)."""
    import threading
    seen = []
    t = threading.Thread(target=lambda: seen.append(lbt.lib().lbt_last_hip_error().decode()))
    t.start()
    t.join()
    assert seen == ["hipSuccess"]


def test_one_hip_runtime_when_the_library_loads_before_torch():
    """Loading the library first (a size query before any torch call) must
    still leave a single HIP runtime in the process: torch's, which the
    library then shares (two copies would make every launch on a torch
    stream fail)."""
    import subprocess
    import sys
    code = (
        "import load_balanced_token_amd as lbt\n"
        "lbt.query_sizes(lbt.Shape(E=8, K=2, R=4, S=8, H=64, B=1, blk=16))\n"
        "import torch\n"
        "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
        "print(len(paths), sorted(paths))\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stderr
    n = int(r.stdout.split()[0])
    assert n == 1, r.stdout
