"""Seeded synthetic inputs shaped like the KV-cache workloads.

This module holds no arithmetic of the conversions themselves: it only draws
random caches, paging tables, sequence lengths and token ids.  Both the HIP
path (tests, benchmark) and the CPU oracle consume what it draws.

Workloads (the ExLlamaV2 cache page gives the layouts: contiguous
[batch, seq, heads, head_dim] windows, and paged caches addressed through
block_table / cache_seqlens with page_size 256 in its example):

  fp8_contig    K,V [1,256,8,128] ~N(0,1); offset 0, width 256
  q4_contig     K,V [4,2048,8,128] ~N(0,1), 1% of elements x20 (outliers);
                offset 1024, width 512
  q6_contig     K,V [8,4096,8,128] ~N(0,0.5), 33 all-zero tokens (0.1%);
                offset 0, width 4096
  q4_paged      K,V [4096 pages,256,8,128] ~N(0,1); batch 32, block_table
                [32,32] = first 1024 entries of a permutation of the pages,
                cache_seqlens uniform in [0,7936]; width 256
  mix_paged     K,V [16384 pages,256,8,128]; batch 64, block_table [64,256] =
                a permutation of all pages, cache_seqlens uniform in
                [0,65280]; width 256; K at 4 bits, V at 6 bits; token ids
                int32 uniform in [0,2^17) of length 65536 with a planted first
                mismatch

(The "ExLlamaV2 cache page" in this file is the page "Implementation: Turboderp org
Exllamav2 Ext Cache".)
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

HEADS = 8
HEAD_DIM = 128

SEEDS = {"fp8_contig": 1001, "q4_contig": 1002, "q6_contig": 1003,
         "q4_paged": 1004, "mix_paged": 1005}


def normal_f16(rng, shape, std=1.0):
    """iid N(0, std^2) drawn in float32, cast to fp16 (round-to-nearest)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x.astype(np.float16)


def with_outliers(rng, x_f32, frac=0.01, factor=20.0):
    """Multiply an iid Bernoulli(frac) subset of elements by `factor`."""
    mask = rng.random(size=x_f32.shape, dtype=np.float32) < frac
    x_f32[mask] *= np.float32(factor)
    return x_f32


def paging(rng, batch, cols, num_pages, seqlen_hi, page_size=256, width=256):
    """block_table [batch, cols] = the first batch*cols entries of a seeded
    permutation of the physical pages (injective: no page is shared);
    cache_seqlens uniform integers in [0, seqlen_hi]."""
    perm = rng.permutation(num_pages).astype(np.int32)
    block_table = perm[: batch * cols].reshape(batch, cols).copy()
    cache_seqlens = rng.integers(0, seqlen_hi + 1, size=batch, dtype=np.int64).astype(np.int32)
    assert seqlen_hi + width <= cols * page_size
    return cache_seqlens, block_table


@dataclass
class Workload:
    name: str
    shape: tuple                 # physical cache shape [dim0, dim1, heads, head_dim]
    batch_size: int
    offset: int
    width: int
    page_size: int
    wbits_k: int                 # 0 = 8-bit (fp16 high byte) path
    wbits_v: int
    std: float = 1.0
    k: Optional[np.ndarray] = None          # host fp16 caches (small workloads)
    v: Optional[np.ndarray] = None
    cache_seqlens: Optional[np.ndarray] = None
    block_table: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)


def fp8_contig(seed=SEEDS["fp8_contig"]):
    rng = np.random.default_rng(seed)
    shape = (1, 256, HEADS, HEAD_DIM)
    return Workload("fp8_contig", shape, 1, 0, 256, 0, 0, 0,
                    k=normal_f16(rng, shape), v=normal_f16(rng, shape))


def q4_contig(seed=SEEDS["q4_contig"]):
    rng = np.random.default_rng(seed)
    shape = (4, 2048, HEADS, HEAD_DIM)
    ks = []
    for _ in range(2):
        x = rng.standard_normal(size=shape, dtype=np.float32)
        ks.append(with_outliers(rng, x).astype(np.float16))
    return Workload("q4_contig", shape, 4, 1024, 512, 0, 4, 4, k=ks[0], v=ks[1])


def q6_contig(seed=SEEDS["q6_contig"]):
    rng = np.random.default_rng(seed)
    shape = (8, 4096, HEADS, HEAD_DIM)
    k = normal_f16(rng, shape, 0.5)
    v = normal_f16(rng, shape, 0.5)
    ntok = shape[0] * shape[1]
    nzero = int(round(0.001 * ntok))                       # 33 tokens
    zt = rng.choice(ntok, size=nzero, replace=False)
    k.reshape(ntok, -1)[zt] = 0
    v.reshape(ntok, -1)[zt] = 0
    w = Workload("q6_contig", shape, 8, 0, 4096, 0, 6, 6, std=0.5, k=k, v=v)
    w.extra["zero_tokens"] = np.sort(zt)
    return w


def q4_paged(seed=SEEDS["q4_paged"], draws=1):
    """Paged Q4 workload.  The physical caches (2 GiB each) are filled on the
    device by `device_normal_f16`; `draws` independent (cache_seqlens,
    block_table) pairs are drawn for cold-data rotation."""
    rng = np.random.default_rng(seed)
    shape = (4096, 256, HEADS, HEAD_DIM)
    tables = [paging(rng, 32, 32, 4096, 7936) for _ in range(draws)]
    w = Workload("q4_paged", shape, 32, 0, 256, 256, 4, 4,
                 cache_seqlens=tables[0][0], block_table=tables[0][1])
    w.extra["tables"] = tables
    w.extra["device_seed"] = seed
    return w


def mix_paged(seed=SEEDS["mix_paged"], draws=1):
    """Large paged K-Q4 / V-Q6 workload; `draws` independent (cache_seqlens,
    block_table) pairs (the first is the workload's own) for cold rotation."""
    rng = np.random.default_rng(seed)
    shape = (16384, 256, HEADS, HEAD_DIM)
    sl, bt = paging(rng, 64, 256, 16384, 65280)
    w = Workload("mix_paged", shape, 64, 0, 256, 256, 4, 6, cache_seqlens=sl, block_table=bt)
    w.extra["device_seed"] = seed
    ids_a, ids_b, m = token_ids(rng, 65536)
    w.extra["ids_a"], w.extra["ids_b"], w.extra["match"] = ids_a, ids_b, m
    w.extra["tables"] = [(sl, bt)] + [paging(rng, 64, 256, 16384, 65280) for _ in range(draws - 1)]
    return w


def token_ids(rng, n, vocab=1 << 17):
    """Two int32 id arrays of length n equal up to a seeded first mismatch m
    in [0, n] (m == n: identical)."""
    a = rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)
    b = a.copy()
    m = int(rng.integers(0, n + 1))
    if m < n:
        b[m] = (a[m] + 1 + int(rng.integers(0, vocab - 1))) % vocab
    return a, b, m


def device_normal_f16(torch, shape, seed, std=1.0, device="cuda", slab_rows=65536):
    """Fill a device fp16 tensor of `shape` with iid N(0, std^2) values from a
    seeded torch generator on that device, one slab of leading rows at a time
    (keeps the fp32 temporary small for multi-GiB caches)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.float16, device=device)
    flat = out.view(shape[0] * shape[1], -1)
    for r0 in range(0, flat.shape[0], slab_rows):
        r1 = min(r0 + slab_rows, flat.shape[0])
        t = torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        flat[r0:r1].copy_(t)
    return out


WORKLOADS = {"fp8_contig": fp8_contig, "q4_contig": q4_contig, "q6_contig": q6_contig,
             "q4_paged": q4_paged, "mix_paged": mix_paged}
