"""Seeded synthetic inputs for the HyperAttention forward.

Only random inputs live here -- none of the method's arithmetic -- so the
same tensors can be handed to the HIP library and to the CPU oracle.

Named workloads (shapes and value structure of the single-layer tests on
the HyperAttention pages: a long-context layer at n ~ 131k, a ChatGLM2-like
32k layer with grouped KV heads, and a 512k stress case):

  small      1 x 1 head,  n=1024,   d=64,  fp32, iid,       b=64,  m=64,  r=7, non-causal
  c32k       1 x 32/32,   n=32768,  d=128, bf16, iid,       b=256, m=256, r=7, non-causal
  glm32k     1 x 32/2,    n=32768,  d=128, bf16, sink keys, b=256, m=256, r=7, causal s=4096
  long131k   1 x 32/32,   n=131072, d=64,  bf16, planted,   b=256, m=256, r=7, (non-)causal s=4096
  stress512k 1 x 8/8,     n=524288, d=128, bf16, clusters,  b=512, m=512, r=8, causal s=8192

Value recipes (all scaled by d^-1/4 after drawing, then rounded to the
dtype, ties to even):
  iid       Q, K, V ~ N(0, 1)
  sink      iid, then the first 32 key rows of every KV head x 4
  planted   iid, then per head 1% of the key rows (chosen without
            replacement) become q_u + 0.1 N(0, 1) for a uniform query row u
  clusters  per head 64 means ~ N(0, I); every row of Q, K, V picks a
            mean uniformly and adds 0.3 N(0, I)
The generator is torch's, seeded with ``data_seed`` on the device the
tensors are made on.
"""

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    kv_heads: int
    n: int
    d: int
    dtype: torch.dtype
    block: int
    samples: int
    proj_bits: int
    causal: bool
    min_seq_len: int
    kind: str = "iid"
    seed: int = 0          # method seed (projections and samples)
    data_seed: int = 1

    def method_args(self):
        return dict(block=self.block, samples=self.samples, proj_bits=self.proj_bits,
                    causal=self.causal, min_seq_len=self.min_seq_len, seed=self.seed)

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "small": Workload("small", 1, 1, 1, 1024, 64, torch.float32, 64, 64, 7, False, 0, "iid", 0, 1),
    "c32k": Workload("c32k", 1, 32, 32, 32768, 128, torch.bfloat16, 256, 256, 7, False, 0, "iid", 0, 2),
    "glm32k": Workload("glm32k", 1, 32, 2, 32768, 128, torch.bfloat16, 256, 256, 7, True, 4096, "sink", 0, 3),
    "long131k": Workload("long131k", 1, 32, 32, 131072, 64, torch.bfloat16, 256, 256, 7, False, 4096, "planted", 0, 4),
    "long131k_causal": Workload("long131k_causal", 1, 32, 32, 131072, 64, torch.bfloat16, 256, 256, 7, True, 4096, "planted", 0, 4),
    "stress512k": Workload("stress512k", 1, 8, 8, 524288, 128, torch.bfloat16, 512, 512, 8, True, 8192, "clusters", 0, 5),
}


def make_inputs(w: Workload, device="cpu"):
    """(q, k, v) for workload ``w`` on ``device``: q [B, H, n, d],
    k, v [B, Hkv, n, d] in w.dtype."""
    g = torch.Generator(device=device)
    g.manual_seed(w.data_seed)
    B, H, Hkv, n, d = w.batch, w.heads, w.kv_heads, w.n, w.d
    scale = d ** -0.25

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)

    if w.kind == "clusters":
        def mixture(heads):
            mu = randn(B, heads, 64, d)
            c = torch.randint(0, 64, (B, heads, n), generator=g, device=device)
            x = torch.gather(mu, 2, c[..., None].expand(B, heads, n, d))
            return (x + 0.3 * randn(B, heads, n, d)) * scale
        q = mixture(H)
        k = mixture(Hkv)
        v = mixture(Hkv)
    else:
        q = randn(B, H, n, d) * scale
        k = randn(B, Hkv, n, d) * scale
        v = randn(B, Hkv, n, d) * scale
        if w.kind == "sink":
            k[:, :, :32, :] *= 4.0
        elif w.kind == "planted":
            nrep = max(1, round(0.01 * n))
            G = H // Hkv
            for b in range(B):
                for hk in range(Hkv):
                    rows = torch.randperm(n, generator=g, device=device)[:nrep]
                    src = torch.randint(0, n, (nrep,), generator=g, device=device)
                    k[b, hk, rows] = q[b, hk * G, src] + 0.1 * randn(nrep, d) * scale
        elif w.kind != "iid":
            raise ValueError(f"unknown input kind {w.kind}")
    return (q.to(w.dtype).contiguous(), k.to(w.dtype).contiguous(), v.to(w.dtype).contiguous())
