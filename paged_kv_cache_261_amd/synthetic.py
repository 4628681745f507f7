"""Seeded synthetic decode workloads for paged KV-cache attention.

This module builds inputs only: context lengths, which sequences share a
prefix, the physical block each logical block lands in, the slot of every
token to be written, and the q/K/V values.  It holds none of the attention
arithmetic, and it is the one module that both the GPU path and the CPU
checker read their inputs from.

Recipe (per workload ``k``, one ``numpy.random.default_rng(seed)``; draws in
this fixed order):

1. context lengths (the length the measured step's query sees, including the
   token that step appends);
2. which sequences share a prefix (where the workload has sharing);
3. q for step 0.

The initial free stack (bottom first; blocks are taken from the top, like a
LIFO free list) is a permutation of the physical block ids drawn from its own
stream, ``default_rng([seed, 3])``, so a variant with a different pool size
keeps every other draw.

K/V values come from counter-keyed streams so they can be drawn in parallel
and still not depend on the thread count: prefill chunk ``c`` (2048 tokens,
K then V) uses ``default_rng([seed, 5, c])``; the tokens appended at step
``s`` use ``default_rng([seed, 6, s, c])``; q for step ``s >= 1`` uses
``default_rng([seed, 7, s])``.  Values are N(0, 1) drawn in float32; bf16
workloads round them to bfloat16 (round to nearest, ties to even) and store
the 16-bit patterns as ``uint16``.

Block assignment: every sequence's prefill (positions ``0 .. ctx-2``) takes
its blocks in sequence order, then each step's appended token takes a new
block only when its position starts a block.  A shared prefix is written once,
by the first member of its group, whose blocks then also head the other
members' tables.
"""
from __future__ import annotations

import concurrent.futures as cf
import math
import os
from dataclasses import dataclass, field

import numpy as np

CHUNK_TOKENS = 2048


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    dtype: str                      # "f32" or "bf16"
    scale: float
    description: str
    # split mode the benchmark launches: -1 the library chooses, -3 reads
    # blocks shared inside a pack of sequences once, > 0 fixed partitions
    partition_size: int = -1
    # context lengths: ("fixed", [..]) | ("uniform", lo, hi) | ("const", n)
    ctx_rule: tuple = ()
    # prefix sharing: None | ("random_group", n_members, n_shared_blocks, min_ctx)
    #                       | ("fork", n_prompts, samples_per_prompt, prompt_len)
    sharing: tuple | None = None


CONFIGS = {
    "tiny_f32": Config(
        name="tiny_f32", seed=1, num_seqs=4, num_q_heads=4, num_kv_heads=4, head_dim=16,
        block_size=4, num_blocks=64, max_blocks_per_seq=16, dtype="f32", scale=1 / 4,
        ctx_rule=("fixed", [5, 17, 33, 64]),
        description="fp32 tiny decode: 4 sequences (ctx 5/17/33/64), 4 MHA heads, head_dim 16, "
                    "block 4, 64 physical blocks"),
    "mha_f32": Config(
        name="mha_f32", seed=2, num_seqs=32, num_q_heads=8, num_kv_heads=8, head_dim=64,
        block_size=16, num_blocks=8192, max_blocks_per_seq=129, dtype="f32", scale=1 / 8,
        ctx_rule=("uniform", 1, 2048), sharing=("random_group", 8, 4, 65),
        description="fp32 MHA decode: 32 sequences, ctx U[1,2048], 8 heads, head_dim 64, block 16, "
                    "8192 blocks, 8 sequences share their first 4 blocks"),
    "gqa_bf16": Config(
        name="gqa_bf16", seed=3, num_seqs=256, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=16, num_blocks=65536, max_blocks_per_seq=256, dtype="bf16",
        scale=1 / math.sqrt(128), ctx_rule=("uniform", 512, 4096),
        description="bf16 GQA decode (Llama-3-8B layer shape): 256 sequences, ctx U[512,4096], "
                    "32 q / 8 kv heads, head_dim 128, block 16"),
    "shared_prefix_bf16": Config(
        name="shared_prefix_bf16", seed=4, num_seqs=256, num_q_heads=32, num_kv_heads=8,
        head_dim=128, block_size=16, num_blocks=16384, max_blocks_per_seq=160, dtype="bf16",
        scale=1 / math.sqrt(128), ctx_rule=("const", 2560), sharing=("fork", 32, 8, 2048),
        partition_size=-3,
        description="bf16 shared-prefix parallel sampling: 32 prompts of 2048 tokens x 8 samples, "
                    "512 private tokens each (ctx 2560), 32 q / 8 kv heads, head_dim 128, block 16"),
    "long_split_bf16": Config(
        name="long_split_bf16", seed=5, num_seqs=16, num_q_heads=64, num_kv_heads=8,
        head_dim=128, block_size=16, num_blocks=32768, max_blocks_per_seq=2048, dtype="bf16",
        scale=1 / math.sqrt(128), ctx_rule=("const", 32768), partition_size=512,
        description="bf16 long-context split decode: 16 sequences x ctx 32768, 64 q / 8 kv heads, "
                    "head_dim 128, block 16, 512-token partitions"),
}
CONFIG_ORDER = ["tiny_f32", "mha_f32", "gqa_bf16", "shared_prefix_bf16", "long_split_bf16"]


# --------------------------------------------------------------------------
# Value helpers
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def storage_dtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.float32


def _workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


# --------------------------------------------------------------------------
# Workload
# --------------------------------------------------------------------------
@dataclass
class Workload:
    cfg: Config
    num_steps: int
    context_lens: np.ndarray            # int32 [B], at step 0 (includes step 0's token)
    tables: np.ndarray                  # int32 [B, max_blocks], every block the run uses
    n_blocks_at: list                   # per step: int array [B] of table entries in use
    prefill_slots: np.ndarray           # int64 [T]
    prefill_k: np.ndarray               # [T, Hkv, d]
    prefill_v: np.ndarray
    step_slots: list                    # per step: int64 [B]
    step_k: list                        # per step: [B, Hkv, d]
    step_v: list
    q: list                             # per step: [B, Hq, d]
    groups: list = field(default_factory=list)   # shared groups: (members, n_shared_blocks)
    free_order: np.ndarray | None = None         # initial free stack, bottom first

    def ctx_at(self, step: int) -> np.ndarray:
        return (self.context_lens + step).astype(np.int32)

    def tables_at(self, step: int) -> np.ndarray:
        """Block tables as the given step sees them: -1 past the blocks in use."""
        t = np.full_like(self.tables, -1)
        n = self.n_blocks_at[step]
        for b in range(self.cfg.num_seqs):
            t[b, :n[b]] = self.tables[b, :n[b]]
        return t

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) + self.num_steps - 1

    def kv_logical_bytes(self, step: int = 0) -> int:
        c = self.cfg
        es = 2 if c.dtype == "bf16" else 4
        return int(self.ctx_at(step).astype(np.int64).sum()) * c.num_kv_heads * c.head_dim * 2 * es

    def kv_unique_bytes(self, step: int = 0) -> int:
        """K and V bytes of the distinct token rows the decode step can see:
        a physical block referenced by several sequences counts once, with
        the most rows any of them sees (rows past a context are not read)."""
        c = self.cfg
        es = 2 if c.dtype == "bf16" else 4
        t = self.tables_at(step)
        ctx = self.ctx_at(step).astype(np.int64)
        j = np.arange(t.shape[1], dtype=np.int64)[None, :]
        vis = np.clip(ctx[:, None] - j * c.block_size, 0, c.block_size)
        use = vis > 0
        best = np.zeros(c.num_blocks, dtype=np.int64)
        np.maximum.at(best, t[use], vis[use])
        return int(best.sum()) * c.num_kv_heads * c.head_dim * 2 * es


def _context_lengths(cfg: Config, rng) -> np.ndarray:
    rule = cfg.ctx_rule
    if rule[0] == "fixed":
        return np.asarray(rule[1], dtype=np.int32)
    if rule[0] == "uniform":
        return rng.integers(rule[1], rule[2] + 1, size=cfg.num_seqs).astype(np.int32)
    if rule[0] == "const":
        return np.full(cfg.num_seqs, rule[1], dtype=np.int32)
    raise ValueError(rule)




def _draw_tokens(key, n_tokens, hkv, d, dtype, chunk=CHUNK_TOKENS):
    """K and V for n_tokens tokens; chunk c comes from default_rng(key + [c])
    (K first, then V), drawn in parallel, independent of the thread count."""
    sd = storage_dtype(dtype)
    k = np.empty((n_tokens, hkv, d), dtype=sd)
    v = np.empty((n_tokens, hkv, d), dtype=sd)
    n_chunks = (n_tokens + chunk - 1) // chunk

    def one(c):
        lo, hi = c * chunk, min(n_tokens, (c + 1) * chunk)
        rng = np.random.default_rng(list(key) + [c])
        k[lo:hi] = _normal(rng, (hi - lo, hkv, d), dtype)
        v[lo:hi] = _normal(rng, (hi - lo, hkv, d), dtype)

    if n_chunks <= 1:
        for c in range(n_chunks):
            one(c)
    else:
        with cf.ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(one, range(n_chunks)))
    return k, v


class _FreeStack:
    def __init__(self, order):
        self.stack = [int(x) for x in order]

    def pop(self):
        if not self.stack:
            raise RuntimeError("workload needs more physical blocks than the pool holds")
        return self.stack.pop()


def make_workload(name_or_cfg, num_steps: int = 1, share: bool = True,
                  num_blocks: int | None = None, with_values: bool = True) -> Workload:
    """Build a workload of ``num_steps`` consecutive decode steps.

    ``share=False`` keeps the same logical content (the same q/K/V values at
    every position) but gives every sequence private blocks for what would
    have been shared: the "each sequence its own KV" layout.  It may need a
    larger ``num_blocks``.  ``with_values=False`` builds the layout only.
    """
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    if num_blocks is not None:
        cfg = Config(**{**cfg.__dict__, "num_blocks": int(num_blocks)})
    B, bs, hkv, d = cfg.num_seqs, cfg.block_size, cfg.num_kv_heads, cfg.head_dim
    rng = np.random.default_rng(cfg.seed)

    # (1) context lengths
    ctx = _context_lengths(cfg, rng)
    if ctx.min() < 1:
        raise ValueError("every sequence needs at least the token of step 0")
    # (2) sharing structure: leader[b] holds the values of b's shared prefix
    leader = np.arange(B)
    n_shared = np.zeros(B, dtype=np.int64)          # shared prefix, in blocks
    groups = []
    if cfg.sharing and cfg.sharing[0] == "random_group":
        _, n_members, n_sh, min_ctx = cfg.sharing
        eligible = np.flatnonzero(ctx >= min_ctx)
        members = np.sort(rng.choice(eligible, size=n_members, replace=False))
        leader[members] = members[0]
        n_shared[members] = n_sh
        groups.append((members.tolist(), int(n_sh)))
    elif cfg.sharing and cfg.sharing[0] == "fork":
        _, n_prompts, n_samples, prompt_len = cfg.sharing
        assert n_prompts * n_samples == B and prompt_len % bs == 0
        for p in range(n_prompts):
            members = np.arange(p * n_samples, (p + 1) * n_samples)
            leader[members] = members[0]
            n_shared[members] = prompt_len // bs
            groups.append((members.tolist(), prompt_len // bs))
    # (3) q for step 0
    q0 = _normal(rng, (B, cfg.num_q_heads, d), cfg.dtype)
    # free stack, from its own stream
    free_order = np.random.default_rng([cfg.seed, 3]).permutation(cfg.num_blocks).astype(np.int32)
    free = _FreeStack(free_order)

    max_ctx = int(ctx.max()) + num_steps - 1
    if (max_ctx + bs - 1) // bs > cfg.max_blocks_per_seq:
        raise ValueError("max_blocks_per_seq too small for the run")
    tables = np.full((B, cfg.max_blocks_per_seq), -1, dtype=np.int32)
    n_tab = np.zeros(B, dtype=np.int64)

    # Prefill, sequence by sequence: positions 0 .. ctx-2.
    # value_seq/value_pos: the tokens whose K/V values are drawn (a shared
    # prefix once, under its leader); write_*: the tokens written to the pool.
    value_seq, value_pos, first_value = [], [], np.zeros(B, dtype=np.int64)
    write_seq, write_pos, write_src = [], [], []
    n_values = 0
    for b in range(B):
        n_prefill = int(ctx[b]) - 1
        need = (n_prefill + bs - 1) // bs
        follower = leader[b] != b
        first_own = int(n_shared[b]) * bs if follower else 0
        if follower and share:
            tables[b, :n_shared[b]] = tables[leader[b], :n_shared[b]]
            n_tab[b] = n_shared[b]
        for i in range(int(n_tab[b]), need):
            tables[b, i] = free.pop()
        n_tab[b] = max(n_tab[b], need)
        own = np.arange(first_own, n_prefill, dtype=np.int64)
        first_value[b] = n_values - first_own
        value_seq.append(np.full(own.size, b, dtype=np.int64))
        value_pos.append(own)
        if follower and not share:
            pre = np.arange(0, first_own, dtype=np.int64)
            write_seq.append(np.full(pre.size, b, dtype=np.int64))
            write_pos.append(pre)
            write_src.append(first_value[leader[b]] + pre)
        write_seq.append(np.full(own.size, b, dtype=np.int64))
        write_pos.append(own)
        write_src.append(n_values + np.arange(own.size, dtype=np.int64))
        n_values += own.size
    write_seq = np.concatenate(write_seq)
    write_pos = np.concatenate(write_pos)
    write_src = np.concatenate(write_src)

    # Decode steps: the appended token takes a new block only at a block start.
    n_blocks_at, step_pos = [], []
    for s in range(num_steps):
        pos = ctx.astype(np.int64) - 1 + s
        for b in range(B):
            if pos[b] // bs >= n_tab[b]:
                tables[b, n_tab[b]] = free.pop()
                n_tab[b] += 1
        n_blocks_at.append(n_tab.copy())
        step_pos.append(pos)

    def slots_of(seqs, poss):
        return tables[seqs, poss // bs].astype(np.int64) * bs + poss % bs

    prefill_slots = slots_of(write_seq, write_pos)
    step_slots = [slots_of(np.arange(B), p) for p in step_pos]

    sd = storage_dtype(cfg.dtype)
    if with_values:
        vk, vv = _draw_tokens([cfg.seed, 5], n_values, hkv, d, cfg.dtype)
        if np.array_equal(write_src, np.arange(n_values)):
            pk, pv = vk, vv
        else:
            pk, pv = vk[write_src], vv[write_src]
        sk, sv, qs = [], [], [q0]
        for s in range(num_steps):
            k, v = _draw_tokens([cfg.seed, 6, s], B, hkv, d, cfg.dtype)
            sk.append(k)
            sv.append(v)
            if s >= 1:
                qs.append(_normal(np.random.default_rng([cfg.seed, 7, s]),
                                  (B, cfg.num_q_heads, d), cfg.dtype))
    else:
        pk = pv = np.zeros((0, hkv, d), dtype=sd)
        sk, sv, qs = [], [], [q0]

    return Workload(cfg=cfg, num_steps=num_steps, context_lens=ctx, tables=tables,
                    n_blocks_at=n_blocks_at, prefill_slots=prefill_slots, prefill_k=pk,
                    prefill_v=pv, step_slots=step_slots, step_k=sk, step_v=sv, q=qs,
                    groups=groups if share else [], free_order=free_order)


# --------------------------------------------------------------------------
# Beam-search workload: per-step fork/free churn over shared blocks
# --------------------------------------------------------------------------
# Shaped like the beam-search demo of "CS349E 第 7 讲 01_paged_attention.py"
# (demo 4: a prompt, k candidates that share it and the path they walked
# together, copy-on-write only when a candidate writes into a shared last
# block).  The candidates' choices come from a seeded stream, not a model:
# at step s, new beam j of request r continues old beam parents[s][r][j]
# (sorted, as a top-k over candidates grouped by parent would order them).
#
# Per step, in this order: every new beam forks its parent (reference counts
# up), every old beam is freed (counts down; a block reaching zero goes back
# on the free stack, table order), then every new beam appends one token: a
# fresh block when the position starts a block, else a copy of the last block
# first when that block is shared.  The block manager below keeps only the
# bookkeeping the schedule needs (which block ids the tables hold); it moves
# no data.  Random streams: parents from default_rng(seed); the free stack
# from default_rng([seed, 3]); prompt K/V of request r from
# default_rng([seed, 5, r]); step s tokens from default_rng([seed, 6, s]);
# q of step s from default_rng([seed, 7, s]).

@dataclass(frozen=True)
class BeamConfig:
    name: str
    seed: int
    num_requests: int
    beam_width: int
    prompt_len: int
    steps: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    dtype: str
    scale: float
    description: str
    partition_size: int = -3

    @property
    def num_seqs(self) -> int:
        return self.num_requests * self.beam_width

    @property
    def max_blocks_per_seq(self) -> int:
        return (self.prompt_len + self.steps + self.block_size - 1) // self.block_size


BEAM_CONFIGS = {
    "beam_tiny_bf16": BeamConfig(
        name="beam_tiny_bf16", seed=11, num_requests=2, beam_width=4, prompt_len=64, steps=32,
        num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16, num_blocks=256,
        dtype="bf16", scale=1 / math.sqrt(128),
        description="bf16 beam search, demo size: 2 requests x 4 beams, 64-token prompts, "
                    "32 steps, block 16, 8 q / 2 kv heads, head_dim 128"),
    "beam_bf16": BeamConfig(
        name="beam_bf16", seed=12, num_requests=64, beam_width=4, prompt_len=1024, steps=64,
        num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, num_blocks=16384,
        dtype="bf16", scale=1 / math.sqrt(128),
        description="bf16 beam search: 64 requests x 4 beams, 1024-token prompts, 64 steps, "
                    "block 16, 32 q / 8 kv heads, head_dim 128"),
}


class _RefPool:
    """Reference-counted block ids with a LIFO free stack (bookkeeping only)."""

    def __init__(self, free_order, block_size):
        self.free = [int(x) for x in free_order]
        self.ref = np.zeros(len(free_order), dtype=np.int64)
        self.bs = block_size
        self.tables, self.lens = {}, {}
        self.next_id = 0
        self.copies = 0

    def _alloc(self):
        if not self.free:
            raise RuntimeError("workload needs more physical blocks than the pool holds")
        b = self.free.pop()
        self.ref[b] = 1
        return b

    def new_seq(self):
        s = self.next_id
        self.next_id += 1
        self.tables[s], self.lens[s] = [], 0
        return s

    def fork(self, s):
        t = self.new_seq()
        self.tables[t] = list(self.tables[s])
        self.lens[t] = self.lens[s]
        for b in self.tables[t]:
            self.ref[b] += 1
        return t

    def free_seq(self, s):
        for b in self.tables.pop(s):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.lens[s]

    def append(self, s):
        """Slot of the token at position len(s); (src, dst) when it copied."""
        pos, tab, cow = self.lens[s], self.tables[s], None
        if pos % self.bs == 0:
            tab.append(self._alloc())
        else:
            b = tab[pos // self.bs]
            if self.ref[b] > 1:
                nb = self._alloc()
                self.ref[b] -= 1
                tab[pos // self.bs] = nb
                self.copies += 1
                cow = (b, nb)
        self.lens[s] = pos + 1
        return tab[pos // self.bs] * self.bs + pos % self.bs, cow


@dataclass
class BeamStep:
    parents: np.ndarray      # int [R, k]: old beam each new beam continues
    tables: np.ndarray       # int32 [R*k, max_blocks] after the step's append (-1 padded)
    ctx: np.ndarray          # int32 [R*k], including the step's token
    slots: np.ndarray        # int64 [R*k], slot of the step's token
    cow: np.ndarray          # int32 [n, 2] (src, dst) copies made before the step's writes
    k: np.ndarray            # [R*k, Hkv, d]
    v: np.ndarray
    q: np.ndarray            # [R*k, Hq, d]
    used_blocks: int         # blocks held after the step
    unshared_blocks: int     # blocks the beams would hold without sharing


@dataclass
class BeamWorkload:
    cfg: BeamConfig
    free_order: np.ndarray
    prefill_slots: np.ndarray
    prefill_k: np.ndarray
    prefill_v: np.ndarray
    steps: list
    n_copies: int

    def kv_logical_bytes(self, s: int) -> int:
        c = self.cfg
        es = 2 if c.dtype == "bf16" else 4
        return int(self.steps[s].ctx.astype(np.int64).sum()) * c.num_kv_heads * c.head_dim * 2 * es

    def kv_unique_bytes(self, s: int) -> int:
        c = self.cfg
        es = 2 if c.dtype == "bf16" else 4
        st = self.steps[s]
        j = np.arange(st.tables.shape[1], dtype=np.int64)[None, :]
        vis = np.clip(st.ctx.astype(np.int64)[:, None] - j * c.block_size, 0, c.block_size)
        use = vis > 0
        best = np.zeros(c.num_blocks, dtype=np.int64)
        np.maximum.at(best, st.tables[use], vis[use])
        return int(best.sum()) * c.num_kv_heads * c.head_dim * 2 * es


def make_beam_workload(name_or_cfg, with_values: bool = True) -> BeamWorkload:
    cfg = BEAM_CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    R, k, bs, hkv, d = cfg.num_requests, cfg.beam_width, cfg.block_size, cfg.num_kv_heads, \
        cfg.head_dim
    rng = np.random.default_rng(cfg.seed)
    free_order = np.random.default_rng([cfg.seed, 3]).permutation(cfg.num_blocks).astype(np.int32)
    pool = _RefPool(free_order, bs)
    sd = storage_dtype(cfg.dtype)

    # prompts: one sequence per request, then k - 1 forks of it
    beams, pre_slots = [], []
    for r in range(R):
        lead = pool.new_seq()
        pre_slots.extend(pool.append(lead)[0] for _ in range(cfg.prompt_len))
        beams.append([lead] + [pool.fork(lead) for _ in range(k - 1)])
    if with_values:
        pk = np.empty((R * cfg.prompt_len, hkv, d), dtype=sd)
        pv = np.empty_like(pk)
        for r in range(R):
            kr, vr = _draw_tokens([cfg.seed, 5, r], cfg.prompt_len, hkv, d, cfg.dtype)
            pk[r * cfg.prompt_len:(r + 1) * cfg.prompt_len] = kr
            pv[r * cfg.prompt_len:(r + 1) * cfg.prompt_len] = vr
    else:
        pk = pv = np.zeros((0, hkv, d), dtype=sd)

    steps = []
    mb = cfg.max_blocks_per_seq
    for s in range(cfg.steps):
        parents = np.sort(rng.integers(0, k, size=(R, k)), axis=1)
        new = [[pool.fork(beams[r][parents[r, j]]) for j in range(k)] for r in range(R)]
        for r in range(R):
            for old in beams[r]:
                pool.free_seq(old)
        beams = new
        order = [x for r in range(R) for x in beams[r]]
        slots, cow = [], []
        for x in order:
            slot, c = pool.append(x)
            slots.append(slot)
            if c is not None:
                cow.append(c)
        tables = np.full((R * k, mb), -1, dtype=np.int32)
        for i, x in enumerate(order):
            tables[i, :len(pool.tables[x])] = pool.tables[x]
        ctx = np.array([pool.lens[x] for x in order], dtype=np.int32)
        if with_values:
            kk, vv = _draw_tokens([cfg.seed, 6, s], R * k, hkv, d, cfg.dtype)
            q = _normal(np.random.default_rng([cfg.seed, 7, s]), (R * k, cfg.num_q_heads, d),
                        cfg.dtype)
        else:
            kk = vv = np.zeros((0, hkv, d), dtype=sd)
            q = np.zeros((0, cfg.num_q_heads, d), dtype=sd)
        steps.append(BeamStep(
            parents=parents, tables=tables, ctx=ctx, slots=np.array(slots, dtype=np.int64),
            cow=np.array(cow, dtype=np.int32).reshape(-1, 2), k=kk, v=vv, q=q,
            used_blocks=int((pool.ref > 0).sum()),
            unshared_blocks=int(sum((pool.lens[x] + bs - 1) // bs for x in order))))
    return BeamWorkload(cfg=cfg, free_order=free_order,
                        prefill_slots=np.array(pre_slots, dtype=np.int64), prefill_k=pk,
                        prefill_v=pv, steps=steps, n_copies=pool.copies)


# --------------------------------------------------------------------------
# Prefill workload: a chunk of new tokens per sequence over a cached prefix
# --------------------------------------------------------------------------
# Each sequence has a cached prefix (its K/V written before the measured
# step) and a chunk of new tokens: the measured step writes the chunk's K/V
# through slot_mapping and runs causal prefill for the chunk's queries.
# Draw order from default_rng(seed): prefix lengths, chunk lengths, q.  Free
# stack from default_rng([seed, 3]); blocks are taken sequence by sequence in
# position order.  Prefix K/V of sequence b from default_rng([seed, 5, b]),
# chunk K/V from default_rng([seed, 6, b]).

@dataclass(frozen=True)
class PrefillConfig:
    name: str
    seed: int
    num_seqs: int
    prefix_rule: tuple          # ("uniform", lo, hi) | ("fixed", [..])
    chunk_rule: tuple           # ("const", n) | ("fixed", [..])
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    dtype: str
    scale: float
    description: str


PREFILL_CONFIGS = {
    "prefill_bf16": PrefillConfig(
        name="prefill_bf16", seed=21, num_seqs=16, prefix_rule=("uniform", 0, 1536),
        chunk_rule=("const", 512), num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
        num_blocks=4096, max_blocks_per_seq=128, dtype="bf16", scale=1 / math.sqrt(128),
        description="bf16 chunked prefill: 16 sequences, 512-token chunks over cached prefixes "
                    "U[0,1536], 32 q / 8 kv heads, head_dim 128, block 16"),
}


@dataclass
class PrefillWorkload:
    cfg: PrefillConfig
    prefix_lens: np.ndarray
    chunk_lens: np.ndarray
    ctx: np.ndarray             # prefix + chunk
    cu_seqlens_q: np.ndarray    # [B + 1]
    tables: np.ndarray
    prefix_slots: np.ndarray
    prefix_k: np.ndarray
    prefix_v: np.ndarray
    chunk_slots: np.ndarray
    chunk_k: np.ndarray
    chunk_v: np.ndarray
    q: np.ndarray               # [total_q, Hq, d]

    def flops(self) -> int:
        """Multiply-adds x 2 of the causal prefill: 4 d Hq per (query row, key)."""
        c = self.cfg
        keys = 0
        for p, n in zip(self.prefix_lens, self.chunk_lens):
            keys += int(n) * int(p) + int(n) * (int(n) + 1) // 2
        return 4 * c.head_dim * c.num_q_heads * keys

    def kv_bytes(self) -> int:
        c = self.cfg
        es = 2 if c.dtype == "bf16" else 4
        return int(self.ctx.astype(np.int64).sum()) * c.num_kv_heads * c.head_dim * 2 * es


def _lengths(rule, rng, n):
    if rule[0] == "fixed":
        return np.asarray(rule[1], dtype=np.int32)
    if rule[0] == "const":
        return np.full(n, rule[1], dtype=np.int32)
    if rule[0] == "uniform":
        return rng.integers(rule[1], rule[2] + 1, size=n).astype(np.int32)
    raise ValueError(rule)


def make_prefill_workload(name_or_cfg) -> PrefillWorkload:
    cfg = PREFILL_CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    B, bs, hkv, d = cfg.num_seqs, cfg.block_size, cfg.num_kv_heads, cfg.head_dim
    rng = np.random.default_rng(cfg.seed)
    prefix = _lengths(cfg.prefix_rule, rng, B)
    chunk = _lengths(cfg.chunk_rule, rng, B)
    ctx = (prefix + chunk).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q = _normal(rng, (int(cu[-1]), cfg.num_q_heads, d), cfg.dtype)
    free = _FreeStack(np.random.default_rng([cfg.seed, 3]).permutation(cfg.num_blocks))
    if int(((ctx + bs - 1) // bs).max()) > cfg.max_blocks_per_seq:
        raise ValueError("max_blocks_per_seq too small")
    tables = np.full((B, cfg.max_blocks_per_seq), -1, dtype=np.int32)
    for b in range(B):
        for i in range((int(ctx[b]) + bs - 1) // bs):
            tables[b, i] = free.pop()

    def slots(b, lo, hi):
        pos = np.arange(lo, hi, dtype=np.int64)
        return tables[b, pos // bs].astype(np.int64) * bs + pos % bs

    sd = storage_dtype(cfg.dtype)
    pk, pv, ck, cv, ps, cs = [], [], [], [], [], []
    for b in range(B):
        k, v = _draw_tokens([cfg.seed, 5, b], int(prefix[b]), hkv, d, cfg.dtype)
        pk.append(k)
        pv.append(v)
        ps.append(slots(b, 0, int(prefix[b])))
        k, v = _draw_tokens([cfg.seed, 6, b], int(chunk[b]), hkv, d, cfg.dtype)
        ck.append(k)
        cv.append(v)
        cs.append(slots(b, int(prefix[b]), int(ctx[b])))
    cat = lambda xs, shape: np.concatenate(xs) if xs else np.zeros(shape, dtype=sd)  # noqa: E731
    return PrefillWorkload(cfg=cfg, prefix_lens=prefix, chunk_lens=chunk, ctx=ctx,
                           cu_seqlens_q=cu, tables=tables, prefix_slots=np.concatenate(ps),
                           prefix_k=cat(pk, (0, hkv, d)), prefix_v=cat(pv, (0, hkv, d)),
                           chunk_slots=np.concatenate(cs), chunk_k=cat(ck, (0, hkv, d)),
                           chunk_v=cat(cv, (0, hkv, d)), q=q)
