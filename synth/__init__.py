"""Seeded synthetic inputs for the Q4 verify GEMM.

This module is the only code that both the HIP path's tests/benchmarks and the
CPU oracle's checks draw on.  It holds none of the method's arithmetic: it
draws random codes, scales, biases and activations and lays the three weight
planes side by side in one byte buffer.  It never dequantises or multiplies.

Value distributions (the synthetic workload that stands in for real model
weights and activations):

* 4-bit codes uniform on 0..15 (every byte uniform on 0..255);
* scale = bf16(|N(0, 0.02)| + 1e-3), one per output row and group of 64;
* bias  = bf16(-8 * scale + N(0, 0.002)) using the already rounded scale, so
  the affine weights centre near zero as in a symmetric 4-bit code;
* activations x = bf16(N(0, 1)).

Buffer layout (planar, the library's layout 0): ``[codes N*K/2 bytes]
[scales N*K/64 bf16][biases N*K/64 bf16]``, each plane row-major by output
row; two codes per byte, the even input in the low nibble.

Random numbers come from torch's generator on the target device, seeded by a
SplitMix64 hash of ``(seed, stream id)``, so GB-sized weights are drawn on the
GPU in milliseconds.  Values drawn on the CPU and on a GPU differ; every check
therefore hands the oracle the very bytes the GPU consumed.
"""
from __future__ import annotations

import torch

GROUP = 64
_MASK64 = (1 << 64) - 1


def _splitmix64(z: int) -> int:
    """One SplitMix64 output step (Steele, Lea and Flood, 2014)."""
    z = (z + 0x9E3779B97F4A7C15) & _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def stream_seed(seed: int, *ids: int) -> int:
    """63-bit generator seed for tensor stream ``ids`` under ``seed``."""
    z = _splitmix64(int(seed) & _MASK64)
    for i in ids:
        z = _splitmix64(z ^ (int(i) & _MASK64))
    return z >> 1


def _gen(device, seed: int, *ids: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, *ids))
    return g


def packed_size(N: int, K: int) -> int:
    """Byte count of the planar buffer (plane sizes added up)."""
    return N * K // 2 + 2 * (2 * (N * K // GROUP))


def planes(packed: torch.Tensor, N: int, K: int):
    """Views ``(codes [N, K/2] u8, scales [N, K/64] bf16, biases [N, K/64]
    bf16)`` into a planar buffer."""
    G = K // GROUP
    a = N * K // 2
    b = a + 2 * N * G
    c = b + 2 * N * G
    codes = packed[:a].view(N, K // 2)
    scales = packed[a:b].view(torch.bfloat16).view(N, G)
    biases = packed[b:c].view(torch.bfloat16).view(N, G)
    return codes, scales, biases


def q4_weights(N: int, K: int, seed: int = 0, stream: int = 0,
               device="cpu") -> torch.Tensor:
    """Seeded packed Q4 weights [N, K] as a flat uint8 tensor on ``device``."""
    if K % GROUP or N < 1 or K < GROUP:
        raise ValueError(f"need N >= 1 and K a positive multiple of {GROUP}")
    dev = torch.device(device)
    packed = torch.empty(packed_size(N, K), dtype=torch.uint8, device=dev)
    codes, scales, biases = planes(packed, N, K)
    G = K // GROUP
    codes.copy_(torch.randint(0, 256, (N, K // 2), dtype=torch.uint8,
                              device=dev, generator=_gen(dev, seed, stream, 1)))
    s32 = torch.randn((N, G), dtype=torch.float32, device=dev,
                      generator=_gen(dev, seed, stream, 2)).mul_(0.02).abs_()
    s16 = s32.add_(1e-3).to(torch.bfloat16)
    scales.copy_(s16)
    noise = torch.randn((N, G), dtype=torch.float32, device=dev,
                        generator=_gen(dev, seed, stream, 3)).mul_(0.002)
    biases.copy_((s16.float() * -8.0 + noise).to(torch.bfloat16))
    return packed


def activations(M: int, K: int, seed: int = 0, stream: int = 0,
                device="cpu") -> torch.Tensor:
    """Seeded bf16 activations x [M, K] ~ N(0, 1)."""
    dev = torch.device(device)
    x = torch.randn((M, K), dtype=torch.float32, device=dev,
                    generator=_gen(dev, seed, stream, 4))
    return x.to(torch.bfloat16)


def bf16_bits(t: torch.Tensor):
    """Raw bf16 bit patterns of a tensor as a numpy uint16 array (CPU)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(
        "uint16")


def from_bf16_bits(bits, device="cpu") -> torch.Tensor:
    """bf16 tensor from raw uint16 bit patterns."""
    import numpy as np
    arr = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(arr.copy()).view(torch.bfloat16).to(device)


def sample_inputs(M: int, V: int, draft_k: int, seed: int = 0,
                  stream: int = 0, device="cpu") -> dict:
    """Inputs of the verify sampling epilogue beside the logits, seeded:
    per row draft_k distinct draft candidate tokens (uniform over the
    vocabulary), their probabilities q (Dirichlet(1), float32), the drafted
    token drawn from q, and the uniforms u, v in [0, 1) (float32)."""
    import numpy as np
    rng = np.random.default_rng(stream_seed(seed, 7, stream))
    out = {}
    if draft_k:
        idx = np.stack([rng.choice(V, size=draft_k, replace=False)
                        for _ in range(M)]).astype(np.int32)
        q = rng.dirichlet(np.ones(draft_k), size=M).astype(np.float32)
        pick = np.array([rng.choice(draft_k, p=q[m] / q[m].sum())
                         for m in range(M)])
        tok = idx[np.arange(M), pick]
    else:
        idx = np.zeros((M, 0), dtype=np.int32)
        q = np.zeros((M, 0), dtype=np.float32)
        tok = rng.integers(0, V, size=M).astype(np.int32)
    out["draft_idx"] = torch.from_numpy(idx).to(device)
    out["draft_q"] = torch.from_numpy(q).to(device)
    out["draft_tok"] = torch.from_numpy(tok.astype(np.int32)).to(device)
    out["u"] = torch.from_numpy(rng.random(M).astype(np.float32)).to(device)
    out["v"] = torch.from_numpy(rng.random(M).astype(np.float32)).to(device)
    return out


def gdn_inputs(L: int, H: int, Hk: int, M: int, dv: int = 128,
               dk: int = 128, seed: int = 0, stream: int = 0,
               device="cpu") -> dict:
    """Seeded inputs of the Gated DeltaNet state step, float32:

    * state S [L, H, dv, dk] ~ N(0, 1);
    * per layer and tree node: queries and keys [L, M, Hk, dk] drawn N(0, 1)
      and scaled to unit length (the layer normalises them before the state
      sees them), values [L, M, H, dv] ~ N(0, 1), gates alpha = exp(-U(0, 2))
      in (0.135, 1] and strengths beta = sigmoid(N(0, 1)) [L, M, H];
    * a draft tree of M nodes: parent[0] = -1, parent[i] uniform on
      -1 .. i-1 with a bias towards i - 1 (long chains, as in a draft tree).
    """
    g = _gen(device, seed, 11, stream)
    f32 = torch.float32
    S = torch.randn((L, H, dv, dk), generator=g, device=device, dtype=f32)
    q = torch.randn((L, M, Hk, dk), generator=g, device=device, dtype=f32)
    k = torch.randn((L, M, Hk, dk), generator=g, device=device, dtype=f32)
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn((L, M, H, dv), generator=g, device=device, dtype=f32)
    alpha = torch.exp(-2.0 * torch.rand((L, M, H), generator=g,
                                        device=device, dtype=f32))
    beta = torch.sigmoid(torch.randn((L, M, H), generator=g, device=device,
                                     dtype=f32))
    import numpy as np
    rng = np.random.default_rng(stream_seed(seed, 12, stream))
    parent = np.full(M, -1, dtype=np.int32)
    for i in range(1, M):
        parent[i] = i - 1 if rng.random() < 0.5 else rng.integers(-1, i)
    return {"S": S, "q": q, "k": k, "v": v, "alpha": alpha, "beta": beta,
            "parent": parent}


def tree_path(parent, node: int):
    """Node indices from the tree's root down to ``node`` (inclusive)."""
    path = []
    while node >= 0:
        path.append(int(node))
        node = int(parent[node])
    return path[::-1]


def ancestor_sets(parent):
    """int32 [M] holding uint32 bit sets: bit j of entry i set iff node j is
    node i or one of its ancestors (tree bookkeeping for the attention mask;
    parent[i] < i, -1 for a child of the context)."""
    import numpy as np
    out = np.zeros(len(parent), dtype=np.uint32)
    for i in range(len(parent)):
        n = i
        while n >= 0:
            out[i] |= np.uint32(1) << np.uint32(n)
            n = int(parent[n])
    return out.view(np.int32)


def attn_inputs(M: int, Hq: int, Hkv: int, ctx_len: int, D: int = 256,
                seed: int = 0, stream: int = 0, spare_pages: int = 3,
                device="cpu") -> dict:
    """Seeded inputs of one tree-verify attention layer:

    * queries q [M, Hq, D] = bf16(N(0, 1));
    * a paged int8 cache holding ctx_len + M positions (the tree's keys and
      values after the context): codes round(N(0, 40)) clamped to -127..127,
      per token and head scales U(0.005, 0.02) for keys and for values; keys
      [pool, Hkv, 32, D], values stored transposed [pool, Hkv, D, 32];
    * the pool has spare_pages more pages than needed, filled with codes too,
      and the page table is a random permutation of the pool;
    * a draft tree (as gdn_inputs draws it) and its ancestor-or-self sets.
    """
    import numpy as np
    rng = np.random.default_rng(stream_seed(seed, 13, stream))
    pages = (ctx_len + M + 31) // 32
    pool = pages + spare_pages
    kp = np.clip(np.rint(rng.normal(0, 40, size=(pool, Hkv, 32, D))), -127,
                 127).astype(np.int8)
    vp = np.clip(np.rint(rng.normal(0, 40, size=(pool, Hkv, D, 32))), -127,
                 127).astype(np.int8)
    ks = rng.uniform(0.005, 0.02, size=(pool, Hkv, 32)).astype(np.float32)
    vs = rng.uniform(0.005, 0.02, size=(pool, Hkv, 32)).astype(np.float32)
    table = rng.permutation(pool)[:pages].astype(np.int32)
    parent = np.full(M, -1, dtype=np.int32)
    for i in range(1, M):
        parent[i] = i - 1 if rng.random() < 0.5 else rng.integers(-1, i)
    g = _gen(device, seed, 14, stream)
    q = torch.randn((M, Hq, D), generator=g, device=device,
                    dtype=torch.float32).to(torch.bfloat16)
    t = lambda a: torch.from_numpy(a).to(device)
    return {"q": q, "k_pages": t(kp), "v_pages": t(vp), "k_scale": t(ks),
            "v_scale": t(vs), "page_table": t(table), "parent": parent,
            "anc": t(ancestor_sets(parent)), "ctx_len": ctx_len}
