"""Seeded synthetic inputs for the DSA path.

This module draws random inputs and encodes them into the storage formats the
path reads (fp32, bf16, OCP E4M3FN codes with fp32 scales).  It holds none of
the path's arithmetic (no scores, no selection, no attention), so both the HIP
library's tests and the fp64 oracle can consume its bytes.

Workloads (sizes from the GLM-5.2 anatomy page: 32 index heads x 128 dims,
132-byte index-cache entries, top-2048, 64 MLA heads over 576-wide latent
rows of which 512 form the output):

  1 tiny     1 query, context 64; indexer 4x32 fp32; top-16; MLA 4 heads,
             48-wide rows (32 latent + 16 rope), fp32 everywhere.
  2 decode   batch 8, context 8192 each; q bf16; index keys fp8 + per-token
             power-of-two scale; latent KV bf16.
  3 ragged   batch 64, contexts uniform in [4096, 65536]; latent KV fp8 with a
             per-tensor fp32 scale.
  4 prefill  4096 new queries after a 28672-token prefix (32768 total), causal;
             indexer q fp8 with a power-of-two scale per (row, head).
  5 share    batch 32, context 131072; one index cache, 4 MLA layers each with
             its own fp8 latent KV and bf16 q.

Random streams: tensor t of workload c under seed s is drawn from a
``torch.Generator`` seeded with ``(s * 1_000_003 + c) * 1_000_003 + t`` on the
device the tensor lives on (Philox on GPUs, Mersenne twister on the CPU), so a
case is reproducible per device type.  Values are N(0, 1) before rounding;
indexer weights are N(0, 1/H_I) (variance).  Ragged contexts are always drawn
on the CPU so every device sees the same lengths.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

FP8_MAX = 448.0

# tensor ids of the random streams
_T_CTX, _T_IQ, _T_IW, _T_IK, _T_MQ0, _T_KV0 = 0, 1, 2, 3, 4, 5


def _gen(seed: int, cfg: int, tensor: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 1_000_003 + cfg) * 1_000_003 + tensor) & ((1 << 63) - 1))
    return g


def _randn(shape, seed, cfg, tensor, device, chunk_rows=1 << 20):
    """N(0,1) fp32, drawn in fixed row chunks so peak memory stays bounded."""
    g = _gen(seed, cfg, tensor, device)
    out = torch.empty(shape, dtype=torch.float32, device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device)
    return out


def fp8_codes(x: torch.Tensor) -> torch.Tensor:
    """Round to OCP E4M3FN (nearest, ties to even), saturating at +-448; raw uint8 codes."""
    return x.clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


def pow2_scale(amax: torch.Tensor) -> torch.Tensor:
    """Smallest power of two s with amax / s <= 448 (1 for an all-zero group)."""
    ratio = amax.float() / FP8_MAX
    mant, ex = torch.frexp(ratio)  # ratio = mant * 2**ex, mant in [0.5, 1)
    ex = ex - (mant == 0.5).to(ex.dtype)
    s = torch.ldexp(torch.ones_like(ratio), ex)
    return torch.where(amax > 0, s, torch.ones_like(s))


def quant_rows_pow2(x: torch.Tensor):
    """Per-row (last axis) fp8 codes with a power-of-two fp32 scale."""
    amax = x.abs().amax(dim=-1)
    s = pow2_scale(amax)
    return fp8_codes(x / s.unsqueeze(-1)), s.float()


def quant_tensor(x: torch.Tensor):
    """Whole-tensor fp8 codes with one plain fp32 scale amax / 448."""
    amax = float(x.abs().max())
    s = amax / FP8_MAX if amax > 0 else 1.0
    s = float(torch.tensor(s, dtype=torch.float32))
    return fp8_codes(x / s), s


@dataclass
class MlaLayer:
    q: torch.Tensor          # [T, H, Dc+Dr]  fp32 or bf16
    kv: torch.Tensor         # [N, Dc+Dr]     fp32, bf16 or uint8 fp8 codes
    kv_dt: str               # "f32" | "bf16" | "fp8"
    kv_scale: float = 1.0


@dataclass
class Case:
    name: str
    cfg: int
    B: int
    T: int
    ctx: List[int]
    kv_indptr: torch.Tensor               # int64 [B+1] on device
    q_indptr: Optional[torch.Tensor]      # int32 [B+1] on device, None for one query per sequence
    q_len: List[int]
    # indexer
    H_I: int
    D_I: int
    iq: torch.Tensor                      # [T, H_I, D_I] fp32 / bf16 / uint8 codes
    iq_dt: str
    iq_scale: Optional[torch.Tensor]      # [T, H_I] fp32 (fp8 q only)
    iw: torch.Tensor                      # [T, H_I] fp32
    ik: torch.Tensor                      # [N, D_I] fp32 or uint8 codes
    ik_dt: str
    ik_scale: Optional[torch.Tensor]      # [N] fp32 (fp8 keys only)
    # selection
    topk: int
    # sparse MLA
    H: int
    Dc: int
    Dr: int
    sm_scale: float
    out_dt: str
    layers: List[MlaLayer] = field(default_factory=list)

    @property
    def max_ctx(self) -> int:
        return max(self.ctx)

    @property
    def N(self) -> int:
        return sum(self.ctx)


def make_case(name="custom", cfg=0, ctx=(64,), q_len=None, H_I=32, D_I=128, iq_dt="bf16",
              ik_dt="fp8", topk=2048, H=64, Dc=512, Dr=64, sm_scale=None, mla_q_dt="bf16",
              kv_dt="bf16", out_dt="bf16", n_layers=1, seed=0, device="cpu") -> Case:
    """Build one seeded case.  q_len=None means one query per sequence."""
    ctx = [int(c) for c in ctx]
    B = len(ctx)
    kv_indptr_l = [0]
    for c in ctx:
        kv_indptr_l.append(kv_indptr_l[-1] + c)
    N = kv_indptr_l[-1]
    if q_len is None:
        qlens = [1] * B
        q_indptr = None
    else:
        qlens = [int(x) for x in q_len]
        assert len(qlens) == B and all(1 <= ql <= c for ql, c in zip(qlens, ctx))
        qi = [0]
        for ql in qlens:
            qi.append(qi[-1] + ql)
        q_indptr = torch.tensor(qi, dtype=torch.int32, device=device)
    T = sum(qlens)
    kv_indptr = torch.tensor(kv_indptr_l, dtype=torch.int64, device=device)

    # indexer inputs
    xq = _randn((T, H_I, D_I), seed, cfg, _T_IQ, device)
    iq_scale = None
    if iq_dt == "f32":
        iq = xq
    elif iq_dt == "bf16":
        iq = xq.to(torch.bfloat16)
    elif iq_dt == "fp8":
        iq, iq_scale = quant_rows_pow2(xq)
    else:
        raise ValueError(iq_dt)
    del xq
    iw = _randn((T, H_I), seed, cfg, _T_IW, device) * (1.0 / math.sqrt(H_I))
    xk = _randn((N, D_I), seed, cfg, _T_IK, device)
    ik_scale = None
    if ik_dt == "f32":
        ik = xk
    elif ik_dt == "bf16":
        ik = xk.to(torch.bfloat16)
    elif ik_dt == "fp8":
        ik, ik_scale = quant_rows_pow2(xk)
    else:
        raise ValueError(ik_dt)
    del xk

    Dqk = Dc + Dr
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(Dqk)
    layers = []
    for l in range(n_layers):
        xq = _randn((T, H, Dqk), seed, cfg, _T_MQ0 + 2 * l, device)
        q = xq if mla_q_dt == "f32" else xq.to(torch.bfloat16)
        del xq
        xkv = _randn((N, Dqk), seed, cfg, _T_KV0 + 2 * l, device)
        if kv_dt == "f32":
            layers.append(MlaLayer(q, xkv, "f32", 1.0))
        elif kv_dt == "bf16":
            layers.append(MlaLayer(q, xkv.to(torch.bfloat16), "bf16", 1.0))
            del xkv
        elif kv_dt == "fp8":
            codes, s = quant_tensor(xkv)
            del xkv
            layers.append(MlaLayer(q, codes, "fp8", s))
        else:
            raise ValueError(kv_dt)

    return Case(name=name, cfg=cfg, B=B, T=T, ctx=ctx, kv_indptr=kv_indptr, q_indptr=q_indptr,
                q_len=qlens, H_I=H_I, D_I=D_I, iq=iq, iq_dt=iq_dt, iq_scale=iq_scale, iw=iw, ik=ik,
                ik_dt=ik_dt, ik_scale=ik_scale, topk=topk, H=H, Dc=Dc, Dr=Dr,
                sm_scale=float(sm_scale), out_dt=out_dt, layers=layers)


def ragged_contexts(B=64, lo=4096, hi=65536, seed=0, cfg=3) -> List[int]:
    g = _gen(seed, cfg, _T_CTX, "cpu")
    return [int(x) for x in torch.randint(lo, hi + 1, (B,), generator=g)]


def config(cfg: int, device="cpu", seed=0) -> Case:
    """The five named workloads at their full sizes."""
    if cfg == 1:
        return make_case("tiny", 1, ctx=[64], H_I=4, D_I=32, iq_dt="f32", ik_dt="f32", topk=16,
                         H=4, Dc=32, Dr=16, sm_scale=1.0 / math.sqrt(48), mla_q_dt="f32",
                         kv_dt="f32", out_dt="f32", seed=seed, device=device)
    if cfg == 2:
        return make_case("glm52_decode_b8_ctx8192", 2, ctx=[8192] * 8, sm_scale=1.0 / 16,
                         kv_dt="bf16", seed=seed, device=device)
    if cfg == 3:
        return make_case("ragged_decode_b64_ctx4k_64k", 3, ctx=ragged_contexts(seed=seed),
                         sm_scale=1.0 / 16, kv_dt="fp8", seed=seed, device=device)
    if cfg == 4:
        return make_case("prefill_4096_on_28672", 4, ctx=[32768], q_len=[4096], iq_dt="fp8",
                         sm_scale=1.0 / 16, kv_dt="bf16", seed=seed, device=device)
    if cfg == 5:
        return make_case("indexshare_b32_ctx131072_l4", 5, ctx=[131072] * 32, sm_scale=1.0 / 16,
                         kv_dt="fp8", n_layers=4, seed=seed, device=device)
    raise ValueError("unknown workload %r" % cfg)


@dataclass
class WriterCase:
    """Inputs of the index-cache writer for one prefill chunk: the chunk's index queries
    [T, H_I, 128] and new index keys [T, 128] (bf16, N(0, 1)), their positions (prefix ..
    prefix + T - 1) and the cache rows the keys go to (the same positions: one sequence)."""
    name: str
    q: torch.Tensor
    k: torch.Tensor
    positions: torch.Tensor
    slots: torch.Tensor
    cache_rows: int


_T_WQ, _T_WK = 20, 21


def writer_case(seed=0, device="cpu", T=4096, H_I=32, prefix=28672) -> WriterCase:
    """The prefill chunk's writer inputs: 4096 new rows after a 28672-token prefix."""
    q = _randn((T, H_I, 128), seed, 4, _T_WQ, device).to(torch.bfloat16)
    k = _randn((T, 128), seed, 4, _T_WK, device).to(torch.bfloat16)
    pos = torch.arange(prefix, prefix + T, dtype=torch.int64, device=device)
    return WriterCase("prefill_writer_%d_on_%d" % (T, prefix), q, k, pos, pos.clone(), prefix + T)


# ----------------------------------------------------------------------------------------------
# host views for the oracle (raw storage as numpy: float32, uint16 bf16 bits, uint8 fp8 codes)

def rope_table(max_pos: int, rope_dim: int = 64, theta: float = 8e6, device="cpu") -> torch.Tensor:
    """Rope table fp32 [max_pos, rope_dim], the writer's caller-supplied input: cos of the
    rope_dim/2 frequencies theta^(-2i/rope_dim) at each position, then their sin.  Angles and
    their cos/sin are taken in fp64 and rounded once to fp32.  theta 8e6 is GLM-5.2's rope base
    ("GLM-5.2 架构解剖", configuration table), given there without YaRN scaling."""
    import numpy as np
    inv = theta ** (-np.arange(0, rope_dim, 2, dtype=np.float64) / rope_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    tab = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    return torch.from_numpy(tab).to(device)


def host(t: Optional[torch.Tensor]):
    """Copy a tensor to host numpy, keeping raw bits of bf16 tensors."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
