"""Seeded synthetic inputs for the five workloads.

This module only draws random numbers and lays out page tables.  It holds
none of the NVFP4 arithmetic (no scales, no quantization, no attention), so
both the CPU oracle side and the GPU side can take their inputs from it.

Every workload k draws from ``numpy.random.SeedSequence(100 + k)`` spawned
into named sub-streams::

    0 = Q, 1 = K, 2 = V, 3 = outlier channels, 4 = drift,
    5 = sequence lengths, 6 = page permutation, 7 = appended K/V

K and V of sequence b come from the b-th child of streams 1 and 2, so one
sequence can be regenerated on its own (the full-size checks sample
sequences).  Values are N(0, 1) in FP32, rounded to bfloat16 (nearest-even
on the FP32 bit pattern) when the workload's dtype is bf16; the returned
arrays are FP32 holding those bf16-exact values.

The workloads (shapes from the task's configuration list; the source pages
measure only on model benchmarks that are not available here, so these
seeded inputs stand in for them at the same shapes):

1 tiny       B=1, Hq=Hkv=1, L=1024, FP32 K/V/Q, identity pages.
2 gqa        B=8, Hq=32, Hkv=8, L=4096 then 16 decode steps of one new token
             per sequence; bf16; 4 seeded channels per KV head scaled x20 in
             K and V.
3 long       B=1, Hq=64, Hkv=8, L=65536; bf16 K/V times a per-token
             log-normal factor exp(0.5 z), z ~ N(0,1) iid per token,
             independent for K and V, shared over heads and dims.
4 paged      B=128, Hq=32, Hkv=8, L_b ~ U{1024..8192}; 16-token pages placed
             by a seeded permutation of all pages; bf16.
5 prefill    prefix 32768 + chunk 2048 (causal in the chunk), Hq=64, Hkv=8,
             bf16 Q/K/V; contiguous pages.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D = 128
PAGE = 16

S_Q, S_K, S_V, S_OUTLIER, S_DRIFT, S_LENS, S_PERM, S_APPEND = range(8)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """FP32 -> nearest bfloat16 (ties to even), returned as FP32."""
    x = np.ascontiguousarray(x, np.float32)
    u = x.view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def _streams(k: int):
    return np.random.SeedSequence(100 + k).spawn(8)


def _normal(ss: np.random.SeedSequence, shape) -> np.ndarray:
    return np.random.default_rng(ss).standard_normal(shape, dtype=np.float32)


@dataclass
class DecodeWorkload:
    """Inputs of a decode workload (configurations 1-4)."""
    cfg: int
    name: str
    B: int
    Hq: int
    Hkv: int
    lens: np.ndarray            # [B] int32: cached tokens per sequence
    dtype: str                  # "f32" or "bf16"
    page_table: np.ndarray      # [B][max_pages] int32
    num_pages: int
    steps: int = 0              # appended decode steps (configuration 2)
    outlier_channels: np.ndarray | None = None   # [Hkv][4]
    drift: bool = False
    _child_k: list = field(default_factory=list, repr=False)
    _child_v: list = field(default_factory=list, repr=False)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_pages(self) -> int:
        return self.page_table.shape[1]

    def _round(self, x):
        return round_bf16(x) if self.dtype == "bf16" else np.ascontiguousarray(x, np.float32)

    def _shape_kv(self, x, b, which):
        if self.outlier_channels is not None:
            for h in range(self.Hkv):
                x[:, h, self.outlier_channels[h]] *= np.float32(20.0)
        if self.drift:
            ss = _streams(self.cfg)[S_DRIFT].spawn(2)[0 if which == "k" else 1]
            z = np.random.default_rng(ss.spawn(self.B)[b]).standard_normal(
                x.shape[0], dtype=np.float32)
            x *= np.exp(np.float32(0.5) * z).astype(np.float32)[:, None, None]
        return self._round(x)

    def kv(self, b: int):
        """(K, V) of sequence b's first lens[b] tokens: [L_b][Hkv][128] FP32."""
        L = int(self.lens[b])
        k = _normal(self._child_k[b], (L, self.Hkv, D))
        v = _normal(self._child_v[b], (L, self.Hkv, D))
        return self._shape_kv(k, b, "k"), self._shape_kv(v, b, "v")

    def q(self, step: int = 0) -> np.ndarray:
        """Queries [B][Hq][128] FP32 for decode step `step`."""
        ss = _streams(self.cfg)[S_Q].spawn(max(self.steps, 1))[step]
        return self._round(_normal(ss, (self.B, self.Hq, D)))

    def append_kv(self, step: int):
        """(K, V) of the token appended at step `step`: [B][Hkv][128] each."""
        ss = _streams(self.cfg)[S_APPEND].spawn(max(self.steps, 1))[step].spawn(2)
        k = _normal(ss[0], (self.B, self.Hkv, D))
        v = _normal(ss[1], (self.B, self.Hkv, D))
        if self.outlier_channels is not None:
            for h in range(self.Hkv):
                k[:, h, self.outlier_channels[h]] *= np.float32(20.0)
                v[:, h, self.outlier_channels[h]] *= np.float32(20.0)
        return self._round(k), self._round(v)


def _contiguous_pages(B, pages_per_seq):
    pt = np.zeros((B, max(pages_per_seq)), np.int32)
    nxt = 0
    for b in range(B):
        pt[b, :pages_per_seq[b]] = np.arange(nxt, nxt + pages_per_seq[b], dtype=np.int32)
        nxt += pages_per_seq[b]
    return pt, nxt


def decode_workload(cfg: int, reserve_tokens: int = 16) -> DecodeWorkload:
    """Configuration 1-4.  Each sequence owns ceil((L_b + reserve)/16) pages so
    that decode steps can append `reserve_tokens` tokens."""
    st = _streams(cfg)
    outliers = None
    drift = False
    steps = 0
    if cfg == 1:
        B, Hq, Hkv, dtype = 1, 1, 1, "f32"
        lens = np.array([1024], np.int32)
    elif cfg == 2:
        B, Hq, Hkv, dtype = 8, 32, 8, "bf16"
        lens = np.full(B, 4096, np.int32)
        steps = 16
        rng = np.random.default_rng(st[S_OUTLIER])
        outliers = np.stack([rng.choice(D, 4, replace=False) for _ in range(Hkv)]).astype(np.int64)
    elif cfg == 3:
        B, Hq, Hkv, dtype = 1, 64, 8, "bf16"
        lens = np.array([65536], np.int32)
        drift = True
    elif cfg == 4:
        B, Hq, Hkv, dtype = 128, 32, 8, "bf16"
        lens = np.random.default_rng(st[S_LENS]).integers(1024, 8192, size=B,
                                                            endpoint=True).astype(np.int32)
    else:
        raise ValueError(f"no decode workload {cfg}")
    pages_per_seq = [-(-(int(L) + reserve_tokens) // PAGE) for L in lens]
    if cfg == 4:
        total = int(sum(pages_per_seq))
        perm = np.random.default_rng(st[S_PERM]).permutation(total).astype(np.int32)
        pt = np.zeros((B, max(pages_per_seq)), np.int32)
        nxt = 0
        for b in range(B):
            pt[b, :pages_per_seq[b]] = perm[nxt:nxt + pages_per_seq[b]]
            nxt += pages_per_seq[b]
        num_pages = total
    else:
        pt, num_pages = _contiguous_pages(B, pages_per_seq)
    names = {1: "tiny", 2: "gqa", 3: "long", 4: "paged"}
    return DecodeWorkload(cfg=cfg, name=names[cfg], B=B, Hq=Hq, Hkv=Hkv, lens=lens, dtype=dtype,
                          page_table=pt, num_pages=num_pages, steps=steps,
                          outlier_channels=outliers, drift=drift,
                          _child_k=st[S_K].spawn(B), _child_v=st[S_V].spawn(B))


def custom_decode(seed: int, B: int, Hq: int, Hkv: int, lens, dtype: str = "bf16",
                  permute: bool = True, reserve_tokens: int = 16, steps: int = 0,
                  outliers: bool = False) -> DecodeWorkload:
    """A reduced decode workload for parity tests (seed streams 5000 + seed):
    given sequence lengths, pages handed out from a seeded permutation (or
    contiguously), optional x20 outlier channels."""
    st = np.random.SeedSequence(5000 + seed).spawn(8)
    lens = np.asarray(lens, np.int32)
    pages_per_seq = [max(1, -(-(int(L) + reserve_tokens) // PAGE)) for L in lens]
    total = int(sum(pages_per_seq))
    order = (np.random.default_rng(st[S_PERM]).permutation(total) if permute
             else np.arange(total)).astype(np.int32)
    pt = np.zeros((B, max(pages_per_seq)), np.int32)
    nxt = 0
    for b in range(B):
        pt[b, :pages_per_seq[b]] = order[nxt:nxt + pages_per_seq[b]]
        nxt += pages_per_seq[b]
    oc = None
    if outliers:
        rng = np.random.default_rng(st[S_OUTLIER])
        oc = np.stack([rng.choice(D, 4, replace=False) for _ in range(Hkv)]).astype(np.int64)
    w = DecodeWorkload(cfg=5000 + seed, name=f"custom{seed}", B=B, Hq=Hq, Hkv=Hkv, lens=lens, dtype=dtype,
                       page_table=pt, num_pages=total, steps=steps, outlier_channels=oc,
                       _child_k=st[S_K].spawn(B), _child_v=st[S_V].spawn(B))
    return w


@dataclass
class PrefillWorkload:
    """Configuration 5: a causal chunk of T queries after a cached prefix."""
    prefix: int = 32768
    T: int = 2048
    Hq: int = 64
    Hkv: int = 8
    cfg: int = 5
    name: str = "prefill"

    @property
    def total(self) -> int:
        return self.prefix + self.T

    @property
    def num_pages(self) -> int:
        return -(-self.total // PAGE)

    def page_table(self) -> np.ndarray:
        return np.arange(self.num_pages, dtype=np.int32)[None, :]

    def prefix_kv(self):
        st = _streams(self.cfg)
        k = round_bf16(_normal(st[S_K], (self.prefix, self.Hkv, D)))
        v = round_bf16(_normal(st[S_V], (self.prefix, self.Hkv, D)))
        return k, v

    def chunk_kv(self):
        ss = _streams(self.cfg)[S_APPEND].spawn(2)
        k = round_bf16(_normal(ss[0], (self.T, self.Hkv, D)))
        v = round_bf16(_normal(ss[1], (self.T, self.Hkv, D)))
        return k, v

    def q(self) -> np.ndarray:
        return round_bf16(_normal(_streams(self.cfg)[S_Q], (self.T, self.Hq, D)))


def small_prefill(prefix: int, T: int, Hq: int = 8, Hkv: int = 2, seed_cfg: int = 5) -> PrefillWorkload:
    """A reduced prefill (for parity tests the oracle finishes quickly)."""
    return PrefillWorkload(prefix=prefix, T=T, Hq=Hq, Hkv=Hkv, cfg=seed_cfg, name="prefill-small")


def random_rows(seed: int, n: int, dist: str = "normal", dtype: str = "bf16") -> np.ndarray:
    """[n][128] rows for codec tests.  dist: normal | outlier | tiny | mixed."""
    rng = np.random.default_rng(np.random.SeedSequence(9000 + seed))
    x = rng.standard_normal((n, D), dtype=np.float32)
    if dist == "outlier":
        x[:, rng.choice(D, 4, replace=False)] *= np.float32(20.0)
    elif dist == "tiny":
        x *= np.float32(1e-30)
    elif dist == "mixed":
        scale = np.exp(rng.standard_normal((n, 1)).astype(np.float32) * np.float32(3.0))
        x *= scale.astype(np.float32)
        x[rng.random((n, D)) < 0.05] = np.float32(0.0)
        x[rng.random((n, D)) < 0.02] = np.float32(-0.0)
    return round_bf16(x) if dtype == "bf16" else x
