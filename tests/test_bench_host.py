"""Host logic of bench.py (CPU only): the one-GPU contract, the counter arithmetic behind
roofline.traffic, and the algorithmic byte and flop model against closed forms of the
workloads (the model is what roofline.achieved divides by the measured time)."""
import csv
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_batch_sweep_is_decode_only():
    r = _run("--workload", "ragged", "--batch", "16")
    assert r.returncode == 2 and "decode" in r.stderr


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value", "Grid_Size"])
        w.writeheader()
        for name, counter, value, grid in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value, "Grid_Size": grid})


def test_traffic_from_scales_each_counter_by_the_copy(tmp_path):
    """FETCH_SIZE reads half the bytes a copy moves and WRITE_SIZE all of them: per stage call,
    bytes = sum over the stage's kernels of fetch KiB * 1024 / 0.5 + write KiB * 1024 / 1.0."""
    copy_mib = 64
    kib = copy_mib * 1024
    f, w, cf, cw = (tmp_path / n for n in ("f.csv", "w.csv", "cf.csv", "cw.csv"))
    rows_f, rows_w = [], []
    for _ in range(3):  # three calls of each stage
        rows_f += [("void dsa::idx_decode_kernel<false>(dsa::LayoutDev, ...)", "FETCH_SIZE", 1000, 65536),
                   ("dsa::mla_hh_kernel<false>(...)", "FETCH_SIZE", 2000, 65536),
                   ("dsa::mla_combine_kernel<false>(...)", "FETCH_SIZE", 500, 65536)]
        rows_w += [("void dsa::idx_decode_kernel<false>(dsa::LayoutDev, ...)", "WRITE_SIZE", 10, 65536),
                   ("dsa::mla_hh_kernel<false>(...)", "WRITE_SIZE", 300, 65536),
                   ("dsa::mla_combine_kernel<false>(...)", "WRITE_SIZE", 40, 65536)]
    _counter_csv(f, rows_f)
    _counter_csv(w, rows_w)
    _counter_csv(cf, [("__amd_rocclr_copyBuffer", "FETCH_SIZE", kib // 2, 1 << 20)] * 2)
    _counter_csv(cw, [("__amd_rocclr_copyBuffer", "WRITE_SIZE", kib, 1 << 20)] * 2)
    r = _run("--traffic-from", str(f), str(w), str(cf), str(cw), "--workload", "decode", "--copy-mib", str(copy_mib))
    assert r.returncode == 0, r.stderr
    out = json.loads(r.stdout)
    assert out["fetch_factor"] == 0.5 and out["write_factor"] == 1.0
    mla = out["stages"]["mla"]
    assert mla["kernels"] == ["mla_combine_kernel", "mla_hh_kernel"] and mla["calls"] == 3
    assert mla["hbm_bytes_per_call"] == (2000 + 500) * 1024 * 2 + (300 + 40) * 1024
    assert out["stages"]["indexer"]["hbm_bytes_per_call"] == 1000 * 1024 * 2 + 10 * 1024
    assert "topk" not in out["stages"]


def _case(ctx, q_len, iq_dt, kv_dt, topk=2048):
    return SimpleNamespace(ctx=ctx, q_len=q_len, B=len(ctx), T=sum(q_len), H_I=32, D_I=128, iq_dt=iq_dt,
                           ik_dt="fp8", ik_scale=object(), iq_scale=object() if iq_dt == "fp8" else None,
                           topk=topk, Dc=512, Dr=64, H=64, out_dt="bf16",
                           layers=[SimpleNamespace(kv_dt=kv_dt, q=SimpleNamespace(dtype=torch.bfloat16))])


def test_decode_model_closed_forms():
    """8 x 8192 decode: the indexer reads 132 B and writes a 4-B score per visible token, plus
    q and w; the MLA stage gathers 2048 rows of 1152 B per row and reads q [64, 576] bf16,
    writes [64, 512] bf16, reads 2048 indices; the path total leaves out the score array's
    write and read."""
    m = bench.algorithmic_model(_case([8192] * 8, [1] * 8, "bf16", "bf16"))
    idx_in = 8 * 8192 * 132 + 8 * 32 * (128 * 2 + 4)
    assert m["indexer"]["bytes"] == idx_in + 8 * 8192 * 4
    assert m["mla"]["bytes"] == 8 * 2048 * 1152 + 8 * 64 * (576 * 2 + 512 * 2) + 8 * 2048 * 4 == 20054016
    assert m["topk"]["bytes"] == 8 * 8192 * 4 + 8 * 2048 * 4
    assert m["path_bytes"] == idx_in + 8 * 2048 * 4 + m["mla"]["bytes"]


def test_prefill_model_closed_forms():
    """4096 causal queries after 28672 tokens: row j sees 28673 + j tokens, so the indexer
    does 2 * 32 * 128 flops on sum_j (28673 + j) pairs; every row selects 2048 keys, each
    2 * 64 * (576 + 512) flops."""
    m = bench.algorithmic_model(_case([32768], [4096], "fp8", "bf16"))
    pairs = 4096 * 28673 + 4096 * 4095 // 2
    assert m["indexer"]["flops"] == 2.0 * 32 * 128 * pairs
    assert abs(m["indexer"]["flops"] - 1.0308e12) < 1e8
    assert m["mla"]["flops"] == 2.0 * 64 * 2048 * 4096 * (576 + 512)


def test_short_rows_select_fewer_than_k():
    """A row that sees fewer than k tokens gathers only those."""
    m = bench.algorithmic_model(_case([100, 5000], [1, 1], "bf16", "fp8"))
    sel = 100 + 2048
    assert m["mla"]["flops"] == 2.0 * 64 * sel * (576 + 512)
    assert m["mla"]["bytes"] == sel * 576 + 2 * 64 * (576 * 2 + 512 * 2) + 2 * 2048 * 4
