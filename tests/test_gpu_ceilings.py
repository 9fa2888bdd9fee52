"""The two measurement aids on the GPU: the indexer's load stream (dsa_read_ceiling) reads every
key row and scale of the index cache exactly once, for each load pattern, on key planes and on
132-byte entries; bench.py --read-ceiling prints its line."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import deepseek_sparse_mla_amd as dsa

pytestmark = pytest.mark.gpu

DEV = "cuda"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _xor(words: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(words.astype(np.uint32).ravel(), initial=np.uint32(0)))


@pytest.mark.parametrize("n,blocks", [(1, 512), (70001, 512), (70001, 7), (4096, 3)])
@pytest.mark.parametrize("pattern", [0, 1, 2])
def test_read_ceiling_reads_every_row_once(n, blocks, pattern):
    g = torch.Generator(device=DEV).manual_seed(n + blocks)
    keys = torch.randint(0, 256, (n + 40, 128), generator=g, device=DEV, dtype=torch.uint8)
    scales = torch.rand(n + 40, generator=g, device=DEV) + 0.5
    sink = torch.zeros(blocks, dtype=torch.int32, device=DEV)
    dsa.dsa_read_ceiling(keys, scales, sink, n, pattern=pattern, blocks=blocks)
    torch.cuda.synchronize()
    want = _xor(keys[:n].cpu().numpy().view(np.uint32)) ^ _xor(scales[:n].cpu().numpy().view(np.uint32))
    assert _xor(sink.cpu().numpy().view(np.uint32)) == want


def test_read_ceiling_on_132_byte_entries():
    n = 9000
    g = torch.Generator(device=DEV).manual_seed(5)
    ent = torch.randint(0, 256, (n, 132), generator=g, device=DEV, dtype=torch.uint8)
    sink = torch.zeros(64, dtype=torch.int32, device=DEV)
    dsa.dsa_read_ceiling(ent, ent.view(torch.float32).view(-1)[32:], sink, n, pattern=0, blocks=64,
                         k_row_stride=132, k_scale_stride=33)
    torch.cuda.synchronize()
    host = ent.cpu().numpy()
    want = _xor(np.ascontiguousarray(host[:, :128]).view(np.uint32)) ^ _xor(
        np.ascontiguousarray(host[:, 128:]).view(np.uint32))
    assert _xor(sink.cpu().numpy().view(np.uint32)) == want


def test_bench_read_ceiling_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--read-ceiling", "--workload", "decode",
                        "--steps", "3", "--warmup", "1"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads([l for l in r.stdout.splitlines() if l.startswith("{")][-1])
    assert d["tokens"] == 8 * 8192 and d["bytes_read"] == 8 * 8192 * 132
    for key in ("pattern0_GBps", "pattern1_GBps", "pattern2_GBps", "indexer_GBps_read"):
        assert d[key] > 0
