"""The C ABI from a C99 program (tests/c_abi_path.c).

CPU: the program compiles with gcc against include/dsa.h (the header is plain C) and links
against libdsa.so.  GPU: it runs one decode step of a GLM-shaped batch on inputs written
here, with its own device buffers and workspaces.  Its outputs must equal the Python
binding's bit for bit (same library, deterministic kernels) and meet the oracle's bar; it
also checks that a refused call writes nothing.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import dsa_testlib as tl
from deepseek_sparse_mla_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "deepseek_sparse_mla_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _compile(tmp_path):
    exe = str(tmp_path / "c_abi_path")
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_path.c"), "-o", exe,
           "-L" + LIBDIR, "-ldsa", "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + LIBDIR + ":" + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_program_compiles_and_links(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libdsa.so")):
        pytest.skip("libdsa.so not built")
    assert os.path.exists(_compile(tmp_path))


def _raw(t):
    return t.detach().contiguous().cpu().view(torch.uint8).numpy().tobytes()


@pytest.mark.gpu
def test_c_program_decode_step(tmp_path):
    case = synth.make_case("c_abi", 2, ctx=[300, 2600, 9000], kv_dt="fp8", sm_scale=1.0 / 16, device="cuda")
    L = case.layers[0]
    hdr = np.array([case.B, case.T, case.H_I, case.D_I, case.H, case.Dc, case.Dr, case.topk], np.int32)
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(fin, "wb") as f:
        f.write(hdr.tobytes() + np.int64(case.max_ctx).tobytes() + np.float32(case.sm_scale).tobytes()
                + np.float32(L.kv_scale).tobytes())
        for t in (case.kv_indptr, case.iq, case.iw, case.ik, case.ik_scale, L.q, L.kv):
            f.write(_raw(t))
    exe = _compile(tmp_path)
    r = subprocess.run([exe, str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "refused call" in r.stdout and "decode step" in r.stdout

    T, H, k, ld = case.T, case.H, case.topk, case.max_ctx
    raw = np.fromfile(fout, np.uint8)
    sizes = [T * ld * 4, T * k * 4, T * H * case.Dc * 2, T * H * 4]
    assert raw.size == sum(sizes)
    parts = np.split(raw, np.cumsum(sizes)[:-1])
    c_scores = parts[0].view(np.float32).reshape(T, ld)
    c_idx = parts[1].view(np.int32).reshape(T, k)
    c_out = torch.from_numpy(parts[2].view(np.int16).reshape(T, H, case.Dc).copy()).view(torch.bfloat16)
    c_lse = parts[3].view(np.float32).reshape(T, H)

    # the binding's run of the same step: identical bits
    scores, idx, outs, lses = tl.gpu_path(case)
    n = tl.visible(case)
    s_py = scores.cpu().numpy()
    for i in range(T):
        assert np.array_equal(c_scores[i, :n[i]], s_py[i, :n[i]]), "scores row %d" % i
    assert np.array_equal(c_idx, idx.cpu().numpy())
    assert torch.equal(c_out, outs[0].cpu())
    assert np.array_equal(c_lse, lses[0].cpu().numpy())

    # and the oracle's bar
    o_scores = tl.oracle_scores_rows(case, range(T))
    o_mla, _ = tl.oracle_mla_rows(case, range(T), c_idx)
    g = tl.to_f64(c_out)
    for i in range(T):
        tl.check_scores(c_scores[i, :n[i]], o_scores[i], "C row %d" % i)
        tl.check_topk_same_array(c_idx[i], c_scores[i, :n[i]], k, "C row %d" % i)
        tl.check_attention(g[i], o_mla[i], tl.ATTN_ATOL_LOWP, "C row %d" % i)
