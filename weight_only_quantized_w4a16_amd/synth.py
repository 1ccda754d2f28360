"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds none of the method's arithmetic: it draws normal numbers,
rounds them to bf16 with torch's own CPU cast, and lists the Llama-3 layer
shapes.  Both the oracle side and the HIP side receive what it returns.

Recipe (stands in for the Meta-Llama-3 checkpoints, which are not used):
  activations  bf16 ~ N(0, 1)
  weights      bf16 ~ N(0, 0.02^2)   (standard deviation 0.02)
  generator    numpy PCG64 (np.random.default_rng(seed)), float32 draws,
               scaled in float32, rounded to bf16 by torch's CPU cast.
Weights are [K, N] with K the input dimension; activations are [M, K].
"""
import numpy as np

WEIGHT_STD = 0.02

# Llama-3-8B decode linears: (name, K, N), 32 layers, plus the LM head.
LLAMA3_8B_LAYER = (("qkv", 4096, 6144), ("o", 4096, 4096),
                   ("gate_up", 4096, 28672), ("down", 14336, 4096))
LLAMA3_8B_HEAD = ("lm_head", 4096, 128256)
LLAMA3_8B_LAYERS = 32

# Llama-3-70B decode linears, 80 layers, plus the LM head.
LLAMA3_70B_LAYER = (("qkv", 8192, 10240), ("o", 8192, 8192),
                    ("gate_up", 8192, 57344), ("down", 28672, 8192))
LLAMA3_70B_HEAD = ("lm_head", 8192, 128256)
LLAMA3_70B_LAYERS = 80


# Qwen3-30B-A3B routed experts: 48 layers of 128 experts, top-8 routing;
# each expert holds gate_up 2048 -> 2 x 768 and down 768 -> 2048.
QWEN3_MOE_LAYERS = 48
QWEN3_MOE_EXPERTS = 128
QWEN3_MOE_TOPK = 8
QWEN3_MOE_SHAPES = (("gate_up", 2048, 1536), ("down", 768, 2048))


def moe_routing(B, E, k, seed):
    """Uniform top-k routing of B tokens to E experts, k distinct experts per token
    (seeded).  Returns (token_of_row [B*k], offsets [E+1]): the routed rows grouped
    by expert (ascending), tokens ascending inside an expert; expert e owns rows
    offsets[e] .. offsets[e+1]-1."""
    rng = np.random.default_rng(seed)
    choice = np.argsort(rng.random((B, E)), axis=1)[:, :k]          # k distinct experts per token
    expert = choice.reshape(-1)
    token = np.repeat(np.arange(B), k)
    order = np.lexsort((token, expert))
    counts = np.bincount(expert, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return token[order].astype(np.int32), offsets


def stack_shapes(model="8b", with_head=True):
    """Every GEMM of one decode step, in execution order: list of (name, K, N)."""
    if model == "8b":
        layer, head, n = LLAMA3_8B_LAYER, LLAMA3_8B_HEAD, LLAMA3_8B_LAYERS
    elif model == "70b":
        layer, head, n = LLAMA3_70B_LAYER, LLAMA3_70B_HEAD, LLAMA3_70B_LAYERS
    else:
        raise ValueError(model)
    out = [(f"L{i}.{name}", K, N) for i in range(n) for (name, K, N) in layer]
    if with_head:
        out.append(head)
    return out


def stack_params(model="8b", with_head=True):
    return sum(K * N for _, K, N in stack_shapes(model, with_head))


def weight_seed(layer, j):
    """Seed of weight j (0 qkv, 1 o, 2 gate_up, 3 down) of a layer; the head uses layer 32."""
    return 1000 + 4 * layer + j


def activation_seed(layer, j):
    return 2000 + 4 * layer + j


def _to_bf16_bits(x32):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(shape, seed, std=1.0):
    """bf16 bit patterns (uint16) of N(0, std^2) draws."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return _to_bf16_bits(x)


def activations(M, K, seed):
    return normal_bf16((M, K), seed, 1.0)


def weights(K, N, seed, std=WEIGHT_STD):
    return normal_bf16((K, N), seed, std)


def normal_bf16_device(shape, seed, std, device):
    """Large draws made on the device itself (timing inputs only; values do not
    affect timing).  Returns a torch bf16 tensor."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)
