"""Seeded synthetic inputs shaped like the workloads of the NVFP4 pretraining pages.

This module holds random-number recipes only -- none of the quantization
arithmetic -- so that the GPU path and the CPU oracle can be fed the very same
host arrays.  Every tensor is drawn on the CPU from ``torch.Generator`` with an
explicit seed, in binary32, and rounded to bfloat16 (nearest-even) where the
workload is bfloat16.

Workloads (a 3B decoder: hidden 3072, FFN 9216, 24 query heads and 12 KV heads
of dimension 128, 4 sequences of 2048 tokens; Full-Stack FP4 sec. 4 and the
sotapapers summary's model description):
  tiny     X, W fp32 128x256, N(0,1) with 1% of entries scaled by 50
  qkv      X bf16 8192x3072 N(0,1) with 8 outlier channels x30; W bf16 6144x3072 N(0,0.02^2)
  ffn      X as qkv; W_up 9216x3072, W_down 3072x9216 N(0,0.02^2);
           H bf16 8192x9216 N(0,1) with 8 outlier channels x30
  wgrad    dY bf16 8192x9216, Student-t (nu = 3) rescaled to std 1e-3; X as qkv
  qadamw   v fp32 9216x3072 log-normal exp(-18 + 3 N(0,1))
  lora     rank-64 factors of the FFN-up LoRA-SVD branch: L1 bf16 64x3072 N(0, 1/3072),
           L2 bf16 9216x64 N(0,0.02^2), beta 0.5 (rank and beta are not on the pages)
Real activations, weights, gradients and optimizer states of the pages' trained
model are not available; these distributions stand in for them.
"""
import torch

DATA_SEEDS = {"tiny": 1, "qkv": 2, "ffn": 3, "wgrad": 4, "qadamw": 5, "lora": 6}
RHT_SEED_WGRAD = 0x5EED4
RHT_SEED_QADAMW = 0x5EED5


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def normal(shape, seed, std=1.0):
    """N(0, std^2) binary32."""
    return torch.randn(*shape, generator=_gen(seed), dtype=torch.float32) * std


def spiky(shape, seed, frac=0.01, factor=50.0):
    """N(0,1) with an independent Bernoulli(frac) mask of entries multiplied by factor."""
    g = _gen(seed)
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    mask = torch.rand(*shape, generator=g, dtype=torch.float32) < frac
    return torch.where(mask, x * factor, x)


def outlier_channels(shape, seed, n_outliers=8, factor=30.0):
    """N(0,1) activations [tokens][channels] with n_outliers whole channels scaled."""
    g = _gen(seed)
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    cols = torch.randperm(shape[1], generator=g)[:n_outliers]
    x[:, cols] *= factor
    return x


def student_t3(shape, seed, std=1e-3):
    """Heavy-tailed gradient: z / sqrt(chi2_3 / 3), rescaled from std sqrt(3) to std."""
    g = _gen(seed)
    z = torch.randn(*shape, generator=g, dtype=torch.float32)
    chi2 = torch.zeros(*shape, dtype=torch.float32)
    for _ in range(3):
        e = torch.randn(*shape, generator=g, dtype=torch.float32)
        chi2 += e * e
    t = z / torch.sqrt(chi2 / 3.0)
    return t * (std / 3.0 ** 0.5)


def lognormal(shape, seed, mu=-18.0, sigma=3.0):
    """Non-negative second-moment state exp(mu + sigma N(0,1))."""
    return torch.exp(mu + sigma * torch.randn(*shape, generator=_gen(seed), dtype=torch.float32))


def bf16(x):
    return x.to(torch.bfloat16)


# ---------------------------------------------------------------- named workloads
def tiny(rows=128, cols=256, seed=DATA_SEEDS["tiny"]):
    return {"X": spiky((rows, cols), seed), "W": spiky((rows, cols), seed + 1000)}


def qkv(tokens=8192, hidden=3072, out=6144, seed=DATA_SEEDS["qkv"]):
    return {"X": bf16(outlier_channels((tokens, hidden), seed)),
            "W": bf16(normal((out, hidden), seed + 1000, 0.02))}


def ffn(tokens=8192, hidden=3072, ffn_dim=9216, seed=DATA_SEEDS["ffn"]):
    return {"X": bf16(outlier_channels((tokens, hidden), seed)),
            "W_up": bf16(normal((ffn_dim, hidden), seed + 1000, 0.02)),
            "W_down": bf16(normal((hidden, ffn_dim), seed + 2000, 0.02)),
            "H": bf16(outlier_channels((tokens, ffn_dim), seed + 3000))}


def wgrad(tokens=8192, hidden=3072, ffn_dim=9216, seed=DATA_SEEDS["wgrad"]):
    return {"dY": bf16(student_t3((tokens, ffn_dim), seed)),
            "X": bf16(outlier_channels((tokens, hidden), seed + 1000))}


def qadamw(rows=9216, cols=3072, seed=DATA_SEEDS["qadamw"]):
    return {"v": lognormal((rows, cols), seed)}


def lora(rank=64, hidden=3072, ffn_dim=9216, seed=DATA_SEEDS["lora"]):
    return {"L1": bf16(normal((rank, hidden), seed, hidden ** -0.5)),
            "L2": bf16(normal((ffn_dim, rank), seed + 1000, 0.02)),
            "beta": 0.5}


def random_nvfp4_parts(n, k, seed, device="cpu", max_scale_code=0x7E):
    """Codes and scale bytes of an n x k NVFP4 copy drawn uniformly with a seeded torch
    generator on `device`: every byte is two valid E2M1 codes, and E4M3 scale codes run up to
    max_scale_code (0x7F is the format's NaN).  An operand with no quantization pass behind
    it, for shapes too large to quantize on the host."""
    g = torch.Generator(device=device).manual_seed(seed)
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=device).random_(0, 256, generator=g)
    scales = torch.empty((n, k // 16), dtype=torch.uint8, device=device).random_(
        0, max_scale_code + 1, generator=g)
    return codes, scales


def uniform_bf16(shape, seed, device="cpu"):
    """Uniform [-1, 1) values rounded to bfloat16, drawn with a seeded torch generator on
    `device` (for inputs too large to build on the host)."""
    g = torch.Generator(device=device).manual_seed(seed)
    x = torch.empty(shape, dtype=torch.float32, device=device).uniform_(-1.0, 1.0, generator=g)
    return x.to(torch.bfloat16)

