"""Seeded synthetic step workloads.

This module only draws random inputs: request lengths, token histories,
physical block lists, sampling parameters and K/V / hidden payloads.  It holds
none of the arithmetic of the method (no prefix sums, no position or slot
computation, no padding lookup), so both the CPU oracle tests and the GPU path
can take their inputs from here without sharing any of the computation.

Five configurations are provided, named by what they are:

* ``worked_example``   3 requests (full prefill 7, decode 5+1, chunk 10..21)
* ``decode_heavy``     256 single-token decodes, contexts U[128,4096], 32 layers
* ``mixed``            2 prefills, 2 chunk middles, 120 decodes
* ``churn``            1024-row persistent batch, 10% finish, condense, refill
* ``long_context``     4 x 8192-token chunks of 131072-token prompts, block 64

Every draw comes from ``numpy.random.default_rng(SEED_BASE + index)`` (PCG64),
so each configuration is reproducible bit for bit.  Block ids are drawn without
replacement from ``[1, num_kv_blocks)``; block 0 is the reserved null block.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

SEED_BASE = 0x5EED0000

# Capture sizes used for the padded token count: 1, 2, 4, 8, then every
# multiple of 16 up to 512 (the nano-vllm capture list).  Above the largest
# size the step runs unpadded.
CAPTURE_SIZES = [1, 2, 4, 8] + list(range(16, 513, 16))

CONFIG_NAMES = ["worked_example", "decode_heavy", "mixed", "churn", "long_context"]


@dataclass
class Req:
    """One request as the scheduler hands it to the runner.

    ``tokens`` is the full token history ``[0, num_tokens)``; ``blocks`` the
    physical block ids in logical order; ``num_computed``/``num_scheduled`` are
    this step's (cached, new) lengths.
    """
    req_id: int
    tokens: np.ndarray
    num_prompt: int
    num_computed: int
    num_scheduled: int
    blocks: np.ndarray
    temperature: float = 1.0
    top_p: float = 1.0
    top_k: int = 0
    rep_penalty: float = 1.0

    @property
    def num_tokens(self) -> int:
        return int(self.tokens.shape[0])


@dataclass
class Workload:
    name: str
    block_size: int
    max_num_reqs: int
    max_model_len: int
    max_blocks_per_req: int
    max_num_batched_tokens: int
    num_kv_blocks: int
    kv_heads: int
    head_dim: int
    kv_dtype: str            # "f16" or "bf16"
    num_layers: int
    hidden_size: int
    gather: str              # "all": one row per request; "compacted": rows that may sample
    initial: List[Req]       # added, in order, to an empty batch
    finished: List[int] = field(default_factory=list)   # removed before condense
    refill: List[Req] = field(default_factory=list)     # added after condense
    capture_sizes: List[int] = field(default_factory=lambda: list(CAPTURE_SIZES))
    seed: int = 0
    null_block: int = 0

    @property
    def row_bytes(self) -> int:
        """Bytes of one token's K (or V) row: kv_heads * head_dim * 2."""
        return self.kv_heads * self.head_dim * 2

    def live_requests(self) -> List[Req]:
        """Requests alive after the history (initial - finished + refill), in id order."""
        gone = set(self.finished)
        return [r for r in self.initial if r.req_id not in gone] + list(self.refill)

    def by_id(self) -> dict:
        return {r.req_id: r for r in self.initial + self.refill}


def _rng(index: int, variant: int = 0) -> np.random.Generator:
    return np.random.default_rng(SEED_BASE + index + (variant << 8))


def _sampling(rng: np.random.Generator):
    return dict(temperature=float(np.float32(rng.uniform(0.0, 2.0))),
                top_p=float(np.float32(rng.uniform(0.05, 1.0))),
                top_k=int(rng.integers(0, 101)),
                rep_penalty=float(np.float32(rng.uniform(1.0, 2.0))))


class _BlockPool:
    """Hands out a seeded permutation of [1, num_blocks) without replacement."""

    def __init__(self, rng: np.random.Generator, num_blocks: int):
        self.ids = (rng.permutation(num_blocks - 1) + 1).astype(np.int32)
        self.next = 0

    def take(self, n: int) -> np.ndarray:
        if self.next + n > self.ids.shape[0]:
            raise ValueError("block pool exhausted")
        out = self.ids[self.next:self.next + n].copy()
        self.next += n
        return out


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _mk(rng, pool, req_id, vocab, block_size, c, q, P, T) -> Req:
    assert 0 <= c and q >= 1 and c + q <= T and P <= T
    tokens = rng.integers(0, vocab, size=T, dtype=np.int32)
    blocks = pool.take(_ceil_div(c + q, block_size))
    return Req(req_id, tokens, P, c, q, blocks, **_sampling(rng))


def worked_example(variant: int = 0) -> Workload:
    """Rows A (prefill 7), B (decode, 5 cached + 1 new), C (chunk computing 10..21)."""
    rng = _rng(0, variant)
    pool = _BlockPool(rng, 32)
    B = 16
    a = _mk(rng, pool, 0, 32000, B, c=0, q=7, P=7, T=7)
    b = _mk(rng, pool, 1, 32000, B, c=5, q=1, P=5, T=6)
    c = _mk(rng, pool, 2, 32000, B, c=10, q=12, P=22, T=22)
    return Workload("worked_example", block_size=B, max_num_reqs=4, max_model_len=64,
                    max_blocks_per_req=4, max_num_batched_tokens=32, num_kv_blocks=32,
                    kv_heads=2, head_dim=64, kv_dtype="f16", num_layers=1, hidden_size=128,
                    gather="all", initial=[a, b, c], seed=SEED_BASE + 0 + (variant << 8))


def decode_heavy(variant: int = 0) -> Workload:
    """256 decodes, cached context U[128,4096], prompt U[1,c]; 32 layers of K/V."""
    rng = _rng(1, variant)
    pool = _BlockPool(rng, 131072)
    B = 16
    reqs = []
    for i in range(256):
        c = int(rng.integers(128, 4097))
        P = int(rng.integers(1, c + 1))
        reqs.append(_mk(rng, pool, i, 128256, B, c=c, q=1, P=P, T=c + 1))
    return Workload("decode_heavy", block_size=B, max_num_reqs=512, max_model_len=8192,
                    max_blocks_per_req=512, max_num_batched_tokens=256, num_kv_blocks=131072,
                    kv_heads=8, head_dim=128, kv_dtype="bf16", num_layers=32, hidden_size=4096,
                    gather="all", initial=reqs, seed=SEED_BASE + 1 + (variant << 8))


def mixed(variant: int = 0) -> Workload:
    """Prefills of 2000 and 512, two 2048-token chunk middles over 2048 cached
    tokens of 8192-token prompts, and 120 decodes with contexts U[256,8192];
    rows in a seeded order."""
    rng = _rng(2, variant)
    pool = _BlockPool(rng, 65536)
    B = 16
    shapes = [(0, 2000, 2000, 2000), (0, 512, 512, 512),
              (2048, 2048, 8192, 8192), (2048, 2048, 8192, 8192)]
    for _ in range(120):
        c = int(rng.integers(256, 8193))
        shapes.append((c, 1, int(rng.integers(1, c + 1)), c + 1))
    order = rng.permutation(len(shapes))
    reqs = [_mk(rng, pool, i, 128256, B, *shapes[k]) for i, k in enumerate(order)]
    return Workload("mixed", block_size=B, max_num_reqs=128, max_model_len=16384,
                    max_blocks_per_req=1024, max_num_batched_tokens=8704, num_kv_blocks=65536,
                    kv_heads=8, head_dim=128, kv_dtype="bf16", num_layers=1, hidden_size=4096,
                    gather="all", initial=reqs, seed=SEED_BASE + 2 + (variant << 8))


def churn(variant: int = 0) -> Workload:
    """1024 live rows; a seeded 102 finish; the batch is condensed and 102 new
    requests fill the tail.  The 1024 rows then alive get seeded roles: 960
    decodes and 64 prefill chunks whose sizes are a seeded composition of 15424
    (token budget 16384)."""
    rng = _rng(3, variant)
    pool = _BlockPool(rng, 1 << 20)
    B, M = 16, 32768
    n_init, n_fin = 1024, 102
    finished = sorted(int(x) for x in rng.choice(n_init, n_fin, replace=False))
    alive_ids = [i for i in range(n_init) if i not in set(finished)] + \
        list(range(n_init, n_init + n_fin))
    prefill_ids = set(int(x) for x in rng.choice(alive_ids, 64, replace=False))
    cuts = np.sort(rng.choice(np.arange(1, 15424), 63, replace=False))
    sizes = np.diff(np.concatenate([[0], cuts, [15424]])).astype(int)
    size_of = dict(zip(sorted(prefill_ids), sizes.tolist()))

    def shape_for(req_id):
        if req_id in prefill_ids:
            q = size_of[req_id]
            c = int(rng.integers(0, 16385))
            P = c + q if rng.random() < 0.5 else c + q + int(rng.integers(1, 4097))
            return c, q, P, P
        c = int(rng.integers(128, 16385))
        return c, 1, int(rng.integers(1, c + 1)), c + 1

    initial = [_mk(rng, pool, i, 128256, B, *shape_for(i)) for i in range(n_init)]
    refill = [_mk(rng, pool, i, 128256, B, *shape_for(i)) for i in range(n_init, n_init + n_fin)]
    return Workload("churn", block_size=B, max_num_reqs=1024, max_model_len=M,
                    max_blocks_per_req=M // B, max_num_batched_tokens=16384,
                    num_kv_blocks=1 << 20, kv_heads=8, head_dim=128, kv_dtype="bf16",
                    num_layers=1, hidden_size=4096, gather="all", initial=initial,
                    finished=finished, refill=refill, seed=SEED_BASE + 3 + (variant << 8))


def long_context(force_complete: bool = False, variant: int = 0) -> Workload:
    """4 requests with 131072-token prompts, each computing an 8192-token chunk
    on a seeded cached prefix U[0,122880]; block size 64.  With
    ``force_complete`` request 0 sits at the last chunk (cached 122880), so the
    compacted hidden-state gather has at least one row."""
    rng = _rng(4, variant)
    pool = _BlockPool(rng, 16384)
    B, M = 64, 131072
    reqs = []
    for i in range(4):
        c = int(rng.integers(0, 122881))
        if force_complete and i == 0:
            c = 122880
        reqs.append(_mk(rng, pool, i, 152064, B, c=c, q=8192, P=M, T=M))
    return Workload("long_context" + ("_forced" if force_complete else ""), block_size=B,
                    max_num_reqs=4, max_model_len=M, max_blocks_per_req=M // B,
                    max_num_batched_tokens=32768, num_kv_blocks=16384, kv_heads=8,
                    head_dim=128, kv_dtype="bf16", num_layers=1, hidden_size=8192,
                    gather="compacted", initial=reqs, seed=SEED_BASE + 4 + (variant << 8))


def long_context_tp8(variant: int = 0) -> Workload:
    """long_context as one rank of an 8-way tensor-parallel split sees it: the
    same requests, schedule and block tables, one K/V head of 128 (256-byte
    rows) instead of eight."""
    w = long_context(False, variant)
    return dataclasses.replace(w, name="long_context_tp8", kv_heads=1)


_BUILDERS = {"worked_example": worked_example, "decode_heavy": decode_heavy,
             "mixed": mixed, "churn": churn, "long_context": long_context,
             "long_context_forced": lambda variant=0: long_context(True, variant),
             "long_context_tp8": long_context_tp8}


def get(name: str, variant: int = 0) -> Workload:
    """The named configuration; ``variant`` > 0 draws an independent instance
    of the same configuration (same shapes and distributions, other seed)."""
    return _BUILDERS[name](variant=variant)


def random_batch(rng: np.random.Generator, *, num_reqs: int, block_size: int,
                 max_model_len: int, num_kv_blocks: int, max_q: int, max_c: int,
                 vocab: int = 1000, prompt_mode: Optional[str] = None) -> List[Req]:
    """Small random batch for brute-force style tests.  ``prompt_mode`` picks
    the prompt length relative to c+q: "short" (c+q-1), "exact" (c+q), "long"
    (c+q+1) or None (random among the three)."""
    pool = _BlockPool(rng, num_kv_blocks)
    reqs = []
    for i in range(num_reqs):
        q = int(rng.integers(1, max_q + 1))
        c = int(rng.integers(0, max_c + 1))
        mode = prompt_mode or ["short", "exact", "long"][int(rng.integers(0, 3))]
        P = {"short": max(1, c + q - 1), "exact": c + q, "long": c + q + 1}[mode]
        T = max(P, c + q)
        if T > max_model_len:
            raise ValueError("random_batch: token history exceeds max_model_len")
        reqs.append(_mk(rng, pool, i, vocab, block_size, c=c, q=q, P=P, T=T))
    return reqs


def payload_numpy(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) values rounded to f16 or bf16, returned as their uint16 bit patterns.
    bf16 uses round-to-nearest-even of the float32 value."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        bits = x.view(np.uint32)
        bits = bits + (((bits >> 16) & 1) + 0x7FFF).astype(np.uint32)
        return (bits >> 16).astype(np.uint16)
    raise ValueError(dtype)


def payload_torch(shape, dtype: str, seed: int, device):
    """Same distribution drawn on a device with a seeded torch generator (for
    payloads too large to draw on the host in reasonable time)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(tdt)
