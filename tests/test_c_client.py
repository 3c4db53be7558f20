"""The C ABI used from plain C: tests/c_client/lbt_step.c is built with gcc
(C99, warnings as errors) against include/lbt.h, liblbt.so and the HIP
runtime.  On the GPU it runs one pass of the path (route, plan, align,
dispatch, combine of the identity expert) on buffers it allocates itself;
its outputs must equal the oracle's: ids, counts, plan, slots, sorted ids and
block tables bit for bit, every dispatched row bitwise, gates and combine
within their tolerances."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import load_balanced_token_amd as lbt
from workloads import WORKLOADS, router_logits, activations
from tests import gpu_util as gu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_client", "lbt_step.c")
LIBDIR = os.path.join(ROOT, "load_balanced_token_amd")
ROCM = "/opt/rocm"


def build_client(out_dir) -> str:
    if not os.path.exists(os.path.join(LIBDIR, "liblbt.so")):
        pytest.skip("liblbt.so is not built")
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    exe = os.path.join(str(out_dir), "lbt_step")
    cmd = [gcc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", LIBDIR, "-llbt", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def test_c_client_builds(tmp_path):
    build_client(tmp_path)


def _write_input(path, w, logits, x_bits):
    score = lbt.SOFTMAX if w.score == "softmax" else lbt.SIGMOID
    hdr = np.array([w.E, w.K, w.R, w.S, w.H, w.B, w.blk, score], np.int32)
    with open(path, "wb") as f:
        f.write(hdr.tobytes())
        f.write(np.ascontiguousarray(logits, np.float32).tobytes())
        f.write(np.ascontiguousarray(x_bits, np.uint16).tobytes())


def _read_output(path, w, plan_words_expected):
    raw = open(path, "rb").read()
    N, P, C, nb, pw = np.frombuffer(raw[:40], np.int64).tolist()
    assert (N, P, pw) == (w.N, w.P, plan_words_expected)
    out, at = {}, 40
    for key, dtype, count in (("ids", np.int32, N * w.K), ("gates", np.float32, N * w.K),
                              ("counts", np.int32, w.R * w.E), ("plan", np.int32, pw),
                              ("slot", np.int32, P), ("sorted_ids", np.int32, w.R * C),
                              ("block_wrow", np.int32, w.R * nb),
                              ("block_expert", np.int32, w.R * nb), ("status", np.int32, 1),
                              ("y", np.float32, N * w.H), ("recv", np.uint16, w.R * C * w.H)):
        n = count * np.dtype(dtype).itemsize
        out[key] = np.frombuffer(raw[at:at + n], dtype).copy()
        at += n
    assert at == len(raw)
    out["ids"] = out["ids"].reshape(N, w.K)
    out["gates"] = out["gates"].reshape(N, w.K)
    out["counts"] = out["counts"].reshape(w.R, w.E)
    out["block_wrow"] = out["block_wrow"].reshape(w.R, nb)
    out["block_expert"] = out["block_expert"].reshape(w.R, nb)
    out["y"] = out["y"].reshape(N, w.H)
    out["recv"] = out["recv"].reshape(w.R * C, w.H)
    return out, C


@pytest.mark.gpu
@pytest.mark.parametrize("name,S,H", [("tiny", None, None), ("dsv3", 64, 64), ("decode1", None, 512)])
def test_c_client_step_matches_oracle(tmp_path, name, S, H):
    w = WORKLOADS[name]
    if S is not None:
        w = w.with_(S=S)
    if H is not None:
        w = w.with_(H=H)
    exe = build_client(tmp_path)
    logits = router_logits(w, 0)
    x_bits = activations(w, 0)
    fin, fout = os.path.join(str(tmp_path), "in.bin"), os.path.join(str(tmp_path), "out.bin")
    _write_input(fin, w, logits, x_bits)
    print(f"[c-client] {name} N={w.N} H={w.H}", flush=True)
    r = subprocess.run([exe, fin, fout], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    sizes = lbt.query_sizes(gu.shape_of(w))
    got, C = _read_output(fout, w, sizes["plan_words"])
    ref = gu.run_oracle(w, logits)
    gu.check_route(got, ref)
    got["plan_fields"] = lbt.plan_fields(got["plan"], sizes, w.R, w.E)
    gu.check_plan(got["plan_fields"], ref["plan"], w.P)
    gu.check_align(got, ref, w.R, C)
    slot = ref["align"]["slot"]
    want = oracle.dispatch(x_bits, slot, w.K, w.R, C)
    used = np.zeros(w.R * C, bool)
    used[slot] = True
    assert np.array_equal(got["recv"][used], want[used]), "dispatched rows differ"
    gates32 = ref["gates"].astype(np.float32)
    yref, mag = oracle.combine(lambda rows: want[rows], slot, gates32, w.K)
    err = np.abs(got["y"].astype(np.float64) - yref)
    assert (err <= gu.COMBINE_RTOL * mag + 1e-30).all()
