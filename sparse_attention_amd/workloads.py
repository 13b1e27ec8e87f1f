"""Seeded synthetic inputs shaped like the DSA workloads the GLM-5 pages describe.

This module draws random numbers and packs them; it holds none of the
method's arithmetic.  Both the HIP path and the CPU oracle consume exactly the
arrays made here (bf16 inputs as uint16 bit patterns).

Recipe (every tensor from its own stream):
    Generator(PCG64(SeedSequence(seed, spawn_key=(tensor_id, seq_id))))
    tensor_id: 0 q_idx, 1 w, 2 k_idx, 3 q_abs, 4 kv_latent, 5 lengths,
               6 tie prototypes, 7 tie assignment
    seq_id:    the query row for per-row tensors (0, 1, 3), the sequence for
               per-sequence caches (2, 4, 6, 7), 0 for the length draw (5)
  - entries: standard_normal(float32) rounded to bf16 (round-to-nearest-even)
  - w = fp32(bf16(N(0,1))) * fp32(32**-0.5): the indexer's weight projection
    output scaled by index_n_heads**-1/2 ("GLM-5.1 架构深度拆解" §3.6 step 4)
  - index_scale = 1, softmax_scale = fp32(1/sqrt(256)) (the 192 + 64 = 256
    original QK head, "GLM-5.2 架构 QA" Q1.1)
  - caches are packed: sequence s occupies rows [base_s, base_s + T_s)

Workloads (seed in brackets):
  c1 decode, 1 row, T = 4096 [0]
  c2 causal prefill of one sequence, T = 8192, row i sees i + 1 positions [1];
     tie variant: every index-key row is one of 8 seeded bf16 prototype rows
  c3 batched decode, 64 sequences x T = 32,768, one row each [2]
  c4 long-context decode, 16 sequences x T = 202,752, one row each [3]
  c5 ragged: 128 decode rows with T = floor(exp(U(ln 512, ln 131072))), plus a
     16,384-row causal chunk appended to a 49,152-position history (T = 65,536)
     whose rows see 49,153 .. 65,536 positions [4]
"""
import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np

INDEX_HEADS, INDEX_DIM, HEADS, ROW_DIM = 32, 128, 64, 576
TOPK = 2048
SOFTMAX_SCALE = float(np.float32(1.0 / math.sqrt(256.0)))
INDEX_SCALE = 1.0
W_SCALE = np.float32(32.0 ** -0.5)

(T_Q_IDX, T_W, T_K_IDX, T_Q_ABS, T_KV, T_LEN, T_TIE_PROTO, T_TIE_ASSIGN, T_Q_NOPE, T_Q_PE, T_KVB, T_O, T_LAYER,
 T_HIDDEN, T_WK, T_KVA, T_NORM, T_POS) = range(18)
HIDDEN = 6144
KVB_SCALE = np.float32(512.0 ** -0.5)   # kv_b_proj rows ~ N(0, 1/512): unit-variance outputs


def rng(seed, tensor_id, seq_id):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor_id, seq_id))))


def f32_to_bf16_bits(x):
    """Round fp32 to bf16 with round-to-nearest-even; returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(seed, tensor_id, seq_id, shape):
    return f32_to_bf16_bits(rng(seed, tensor_id, seq_id).standard_normal(shape, dtype=np.float32))


def _threads():
    n = os.cpu_count() or 1
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    return max(1, min(16, n))


@dataclass
class Workload:
    name: str
    seed: int
    visible_len: np.ndarray      # [R] int32
    row_cache_base: np.ndarray   # [R] int64
    seq_len: np.ndarray          # [S] int64, length of each packed sequence
    seq_base: np.ndarray         # [S] int64
    row_seq: np.ndarray          # [R] int64, sequence of each row
    tie_keys: bool = False
    k: int = TOPK
    description: str = ""
    arrays: dict = field(default_factory=dict)

    @property
    def num_rows(self):
        return int(self.visible_len.shape[0])

    @property
    def max_visible(self):
        return int(self.visible_len.max())

    @property
    def cache_rows(self):
        return int(self.seq_len.sum())

    def generate(self, rows=None, with_caches=True):
        """Draws the inputs.  `rows` restricts the per-row tensors to a subset
        (the caches are always whole).  Returns a dict of numpy arrays."""
        rows = np.arange(self.num_rows) if rows is None else np.asarray(rows)
        out = {}
        ex = ThreadPoolExecutor(_threads())
        q = np.empty((len(rows), INDEX_HEADS, INDEX_DIM), np.uint16)
        w = np.empty((len(rows), INDEX_HEADS), np.float32)
        qa = np.empty((len(rows), HEADS, ROW_DIM), np.uint16)

        def per_row(i):
            r = int(rows[i])
            q[i] = normal_bf16(self.seed, T_Q_IDX, r, (INDEX_HEADS, INDEX_DIM))
            w[i] = bf16_bits_to_f32(normal_bf16(self.seed, T_W, r, (INDEX_HEADS,))) * W_SCALE
            qa[i] = normal_bf16(self.seed, T_Q_ABS, r, (HEADS, ROW_DIM))

        list(ex.map(per_row, range(len(rows))))
        out.update(q_idx=q, w=w, q_abs=qa)
        if with_caches:
            kc = np.empty((self.cache_rows, INDEX_DIM), np.uint16)
            kv = np.empty((self.cache_rows, ROW_DIM), np.uint16)

            def per_seq(s):
                b, T = int(self.seq_base[s]), int(self.seq_len[s])
                if self.tie_keys:
                    proto = normal_bf16(self.seed, T_TIE_PROTO, s, (8, INDEX_DIM))
                    pick = rng(self.seed, T_TIE_ASSIGN, s).integers(0, 8, size=T)
                    kc[b:b + T] = proto[pick]
                else:
                    kc[b:b + T] = normal_bf16(self.seed, T_K_IDX, s, (T, INDEX_DIM))
                kv[b:b + T] = normal_bf16(self.seed, T_KV, s, (T, ROW_DIM))

            list(ex.map(per_seq, range(len(self.seq_len))))
            out.update(k_idx=kc, kv_latent=kv)
        ex.shutdown()
        out.update(visible_len=self.visible_len[rows].astype(np.int32),
                   row_cache_base=self.row_cache_base[rows].astype(np.int64))
        return out


def _decode(name, seed, lengths, description):
    lengths = np.asarray(lengths, dtype=np.int64)
    base = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    return Workload(name=name, seed=seed, visible_len=lengths.astype(np.int32), row_cache_base=base,
                    seq_len=lengths, seq_base=base, row_seq=np.arange(len(lengths), dtype=np.int64),
                    description=description)


def decode(num_seqs, T, seed=0, name="decode"):
    """num_seqs sequences of T positions, one decode row each (sees all T)."""
    return _decode(name, seed, [T] * num_seqs, f"decode {num_seqs} x {T}")


def prefill(T, seed=1, tie_keys=False, name="prefill"):
    """One causal prefill of T positions: row i sees i + 1 positions."""
    vis = np.arange(1, T + 1, dtype=np.int32)
    return Workload(name=name, seed=seed, visible_len=vis, row_cache_base=np.zeros(T, np.int64),
                    seq_len=np.array([T], np.int64), seq_base=np.array([0], np.int64),
                    row_seq=np.zeros(T, np.int64), tie_keys=tie_keys,
                    description=f"causal prefill T={T}" + (" (8-prototype index keys)" if tie_keys else ""))


def ragged(seed=4, num_decode=128, lo=512, hi=131072, history=49152, chunk=16384, name="ragged"):
    """Decode rows with log-uniform lengths plus one causal prefill chunk."""
    u = rng(seed, T_LEN, 0).uniform(math.log(lo), math.log(hi), size=num_decode)
    dec = np.floor(np.exp(u)).astype(np.int64)
    T_chunk = history + chunk
    seq_len = np.concatenate([dec, [T_chunk]]).astype(np.int64)
    seq_base = np.concatenate([[0], np.cumsum(seq_len)[:-1]]).astype(np.int64)
    vis = np.concatenate([dec, np.arange(history + 1, T_chunk + 1)]).astype(np.int32)
    row_seq = np.concatenate([np.arange(num_decode), np.full(chunk, num_decode)]).astype(np.int64)
    base = seq_base[row_seq]
    return Workload(name=name, seed=seed, visible_len=vis, row_cache_base=base, seq_len=seq_len,
                    seq_base=seq_base, row_seq=row_seq,
                    description=f"ragged: {num_decode} decode rows log-uniform [{lo}, {hi}] + "
                                f"{chunk}-row chunk on {history} history")


def config(name):
    """The five workloads by short name c1..c5 (c2t = c2 with tied index keys)."""
    if name == "c1":
        return decode(1, 4096, seed=0, name="c1")
    if name == "c2":
        return prefill(8192, seed=1, name="c2")
    if name == "c2t":
        return prefill(8192, seed=1, tie_keys=True, name="c2t")
    if name == "c3":
        return decode(64, 32768, seed=2, name="c3")
    if name == "c4":
        return decode(16, 202752, seed=3, name="c4")
    if name == "c5":
        return ragged(seed=4, name="c5")
    raise KeyError(name)


def layer_stack(lengths, num_layers, seed=6):
    """Inputs of `num_layers` consecutive layers over the same decode batch
    (one row per sequence of the given lengths): layer l is a decode workload
    whose seed is drawn from SeedSequence(seed, spawn_key=(T_LAYER, l)), so
    every layer has its own queries, index keys and latent cache."""
    out = []
    for l in range(num_layers):
        s_l = int(np.random.SeedSequence(seed, spawn_key=(T_LAYER, l)).generate_state(1)[0])
        out.append(_decode(f"layer{l}", s_l, lengths, f"layer {l}").generate())
    return out


def cache_write_inputs(N, seed=7, max_position=1 << 20, cache_rows=None):
    """Synthetic inputs of the cache writers for N new tokens: hidden [N,6144]
    bf16 N(0,1); wk [128,6144] and kv_a [576,6144] bf16 N(0,1/6144) (unit
    variance outputs); LayerNorm weight 1 + 0.1 N(0,1) and bias 0.1 N(0,1)
    [128], RMSNorm weight 1 + 0.1 N(0,1) [512] (fp32); positions uniform in
    [0, max_position) with 0 and max_position - 1 included; slots a random
    injection into [0, cache_rows) (default 2N + 7), every 7th token -1
    (skipped)."""
    g = lambda tid: rng(seed, tid, 0)
    s = np.float32(HIDDEN ** -0.5)
    x = np.stack([normal_bf16(seed, T_HIDDEN, t, (HIDDEN,)) for t in range(N)])
    wk = f32_to_bf16_bits(g(T_WK).standard_normal((128, HIDDEN), dtype=np.float32) * s)
    kva = f32_to_bf16_bits(g(T_KVA).standard_normal((576, HIDDEN), dtype=np.float32) * s)
    gn = g(T_NORM)
    kg = (1 + 0.1 * gn.standard_normal(128)).astype(np.float32)
    kb = (0.1 * gn.standard_normal(128)).astype(np.float32)
    kvg = (1 + 0.1 * gn.standard_normal(512)).astype(np.float32)
    gp = g(T_POS)
    pos = gp.integers(0, max_position, size=N).astype(np.int32)
    pos[0] = 0
    if N > 1:
        pos[-1] = max_position - 1
    rows = 2 * N + 7 if cache_rows is None else cache_rows
    slots = gp.permutation(rows)[:N].astype(np.int64)
    slots[3::7] = -1
    return dict(hidden=x, wk=wk, k_norm_weight=kg, k_norm_bias=kb, kv_a=kva, kv_norm_weight=kvg, positions=pos,
                slots=slots, cache_rows=rows)


def projection_inputs(R, seed=5):
    """Synthetic inputs of the two projections around the path, shaped like the
    model's: q_nope [R,64,192] and q_pe [R,64,64] bf16 N(0,1); the kv_b_proj
    weight [64,448,512] bf16 N(0,1/512) (rows 0..191 of a head: W_UK, rows
    192..447: W_UV); an attention latent output o [R,64,512] fp32 N(0,1/4)."""
    kvb = f32_to_bf16_bits(rng(seed, T_KVB, 0).standard_normal((HEADS, 448, 512), dtype=np.float32) * KVB_SCALE)
    q_nope = np.stack([normal_bf16(seed, T_Q_NOPE, r, (HEADS, 192)) for r in range(R)])
    q_pe = np.stack([normal_bf16(seed, T_Q_PE, r, (HEADS, 64)) for r in range(R)])
    o = np.stack([rng(seed, T_O, r).standard_normal((HEADS, 512), dtype=np.float32) * np.float32(0.5)
                  for r in range(R)])
    return dict(q_nope=q_nope, q_pe=q_pe, kv_b=kvb, o=o)


def random_scores(seed, R, n, ld=None, kind="normal"):
    """Synthetic fp32 score rows for exercising the top-k alone.
    kind: normal | ties (8 distinct values) | zeros | signed_zeros | coarse | tiny"""
    ld = n if ld is None else ld
    g = rng(seed, 100, 0)
    if kind == "normal":
        s = g.standard_normal((R, ld), dtype=np.float32) * np.float32(8)
    elif kind == "ties":
        s = g.integers(0, 8, size=(R, ld)).astype(np.float32)
    elif kind == "zeros":
        s = np.zeros((R, ld), np.float32)
    elif kind == "signed_zeros":
        s = np.where(g.integers(0, 2, size=(R, ld)) == 0, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        s[:, ::7] = np.float32(1.0)
    elif kind == "coarse":
        s = np.round(g.standard_normal((R, ld), dtype=np.float32) * 4).astype(np.float32)
    elif kind == "tiny":
        # fp32 denormals (multiples of 2^-149, both signs) and signed zeros
        v = g.integers(-40, 41, size=(R, ld))
        s = (v.astype(np.float32) * np.float32(2.0 ** -149)).astype(np.float32)
        s[(v == 0) & (g.integers(0, 2, size=(R, ld)) == 0)] = np.float32(-0.0)
    else:
        raise KeyError(kind)
    return np.ascontiguousarray(s)
