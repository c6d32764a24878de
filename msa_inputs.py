"""Seeded synthetic inputs for MiniMax Sparse Attention workloads.

Shared by the tests, the smoke check and the benchmark; holds none of the
method's arithmetic (no scores, pooling, selection or softmax), only the
shapes, distributions and seeds of the workloads.  Both the oracle and the
library are fed the exact tensors built here; the oracle reads them back
bit-for-bit, so host/device generator parity is never needed.

Workloads (all causal, block 128 unless stated):
  fwd-f32-n1k        B=1 N=1024   H_q=4  H_kv=1 d=64  d_idx=32 topk=4  fp32, forward
  fwd-bf16-n8k       B=1 N=8192   H_q=32 H_kv=8 d=128 d_idx=64 topk=16 bf16, forward
  fwdbwd-bf16-b4-n8k B=4 N=8192   H_q=32 H_kv=8 d=128 d_idx=64 topk=16 bf16, fwd+bwd
  fwd-bf16-n128k     B=1 N=131072 H_q=64 H_kv=8 d=128 d_idx=64 topk=16 bf16, forward
  fwdbwd-bf16-n128k  same shapes as fwd-bf16-n128k, forward + backward
  fwdbwd-bf16-n1m    B=1 N=1048576 H_q=32 H_kv=8 d=128 d_idx=64 topk=16 bf16, fwd+bwd

Variants:
  normal   every tensor i.i.d. N(0,1) drawn in fp32, then rounded to the dtype
  int      every tensor i.i.d. uniform over {-2,-1,0,1,2} (exact index scores,
           many exact ties)
  planted  as normal, then a seeded unit vector c in R^{d_idx} is planted with
           beta = 10: each index-query row q gets q - (q.c) c + beta c, and the
           index keys of every 64th block (j % 64 == 0) get + beta c; the
           main-branch q/k/v stay N(0,1)
"""

from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int
    H_q: int
    H_kv: int
    d: int
    d_idx: int
    topk: int
    block_size: int = 128
    causal: bool = True
    dtype: str = "bf16"          # "bf16" or "f32"
    backward: bool = False
    seed: int = 0

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def nblk(self) -> int:
        return (self.N + self.block_size - 1) // self.block_size

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("fwd-f32-n1k", B=1, N=1024, H_q=4, H_kv=1, d=64, d_idx=32, topk=4,
                 dtype="f32", seed=1),
        Workload("fwd-bf16-n8k", B=1, N=8192, H_q=32, H_kv=8, d=128, d_idx=64, topk=16, seed=2),
        Workload("fwdbwd-bf16-b4-n8k", B=4, N=8192, H_q=32, H_kv=8, d=128, d_idx=64, topk=16,
                 backward=True, seed=3),
        Workload("fwd-bf16-n128k", B=1, N=131072, H_q=64, H_kv=8, d=128, d_idx=64, topk=16,
                 seed=4),
        Workload("fwdbwd-bf16-n128k", B=1, N=131072, H_q=64, H_kv=8, d=128, d_idx=64, topk=16,
                 backward=True, seed=4),
        Workload("fwdbwd-bf16-n1m", B=1, N=1048576, H_q=32, H_kv=8, d=128, d_idx=64, topk=16,
                 backward=True, seed=5),
    ]
}

VARIANT_SEED_OFFSET = {"normal": 0, "int": 100, "planted": 100}
PLANT_BETA = 10.0
PLANT_EVERY = 64


def _draw(shape, gen, device, variant):
    if variant == "int":
        return torch.randint(-2, 3, shape, generator=gen, device=device).to(torch.float32)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def make_inputs(w: Workload, variant: str = "normal", seed: int | None = None,
                device="cpu", with_grad_out: bool | None = None, index_fp8: bool = False) -> dict:
    """Build the workload's tensors on `device` from a fixed seed.

    Returns q [B,N,H_q,d], k, v [B,N,H_kv,d], q_idx [B,N,H_kv,d_idx],
    k_idx [B,N,d_idx] in the workload dtype, plus dO [B,N,H_q,d] when the
    workload has a backward (or when asked).  index_fp8: q_idx and k_idx are
    instead rounded from the same fp32 draws to float8_e4m3fn (torch's cast,
    round to nearest even)."""
    if variant not in VARIANT_SEED_OFFSET:
        raise ValueError(f"unknown variant {variant!r}")
    seed = (w.seed + VARIANT_SEED_OFFSET[variant]) if seed is None else seed
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = w.torch_dtype
    out = {}
    # Draw order is fixed: q, k, v, q_idx, k_idx, dO, then the planted vector.
    out["q"] = _draw((w.B, w.N, w.H_q, w.d), gen, device, variant).to(dt)
    out["k"] = _draw((w.B, w.N, w.H_kv, w.d), gen, device, variant).to(dt)
    out["v"] = _draw((w.B, w.N, w.H_kv, w.d), gen, device, variant).to(dt)
    qi = _draw((w.B, w.N, w.H_kv, w.d_idx), gen, device, variant)
    ki = _draw((w.B, w.N, w.d_idx), gen, device, variant)
    want_do = w.backward if with_grad_out is None else with_grad_out
    if want_do:
        out["dO"] = _draw((w.B, w.N, w.H_q, w.d), gen, device, variant).to(dt)
    if variant == "planted":
        c = torch.randn((w.d_idx,), generator=gen, device=device, dtype=torch.float32)
        c = c / c.norm()
        qi = qi - (qi @ c)[..., None] * c + PLANT_BETA * c
        blk = torch.arange(w.N, device=device) // w.block_size
        planted = (blk % PLANT_EVERY == 0).to(torch.float32)
        ki = ki + PLANT_BETA * planted[None, :, None] * c
    idt = torch.float8_e4m3fn if index_fp8 else dt
    out["q_idx"] = qi.to(idt)
    out["k_idx"] = ki.to(idt)
    return out


def planted_blocks(w: Workload) -> list[int]:
    """KV blocks whose index keys carry the planted direction."""
    return [j for j in range(w.nblk) if j % PLANT_EVERY == 0]


def to_numpy64(x: torch.Tensor):
    """Exact upcast of a tensor's bits to float64 on the host."""
    return x.detach().to("cpu", torch.float64).numpy()
