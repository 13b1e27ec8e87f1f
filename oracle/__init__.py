"""CPU oracle for the DSA hot path -- TEST INFRASTRUCTURE ONLY.

Plain fp64 C loops (dsa_oracle.c) behind ctypes.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import this package; the product
library never does, and this package imports nothing from it.  See
dsa_oracle.c for what each function computes and which page passage it
follows.

Parity status: every function here is pinned by tests/test_oracle_pins.py
(closed forms, special cases reducing to library routines, brute force on tiny
inputs, and the pages' printed counts).
"""
import ctypes
import os

import numpy as np

from .build import build_oracle, ORACLE_LIB

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(ORACLE_LIB):
            build_oracle()
        lib = ctypes.CDLL(ORACLE_LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.oracle_set_threads.argtypes = [i32]
        lib.oracle_indexer_scores.argtypes = [i32, P, P, P, P, P, f64, P, i64]
        lib.oracle_round_to_f32.argtypes = [i64, P, P]
        lib.oracle_topk.argtypes = [i32, P, P, i64, i32, P]
        lib.oracle_sparse_mla.argtypes = [i32, P, P, P, P, i32, f64, P, P]
        lib.oracle_absorb_queries.argtypes = [i32, P, P, P, P]
        lib.oracle_v_up_proj.argtypes = [i32, P, P, P]
        lib.oracle_cache_rows.argtypes = [i32, P, P, P, P, f64, P, P, f64, P, f64, P, P]
        lib.oracle_version.restype = ctypes.c_char_p
        _LIB = lib
    return _LIB


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def set_threads(n):
    """Thread count of later calls: sets OMP_NUM_THREADS (read when the OpenMP
    runtime starts) and the running library's own count."""
    os.environ["OMP_NUM_THREADS"] = str(int(n))
    _lib().oracle_set_threads(int(n))


def indexer_scores(visible_len, row_cache_base, q_idx, w, k_idx, index_scale=1.0, ld=None):
    """fp64 scores [R, ld]; entries t >= visible_len[r] are NaN."""
    vis = _c(visible_len, np.int32)
    base = _c(row_cache_base, np.int64)
    R = vis.shape[0]
    ld = int(vis.max()) if ld is None else int(ld)
    q = _c(q_idx, np.uint16).reshape(R, 32, 128)
    ww = _c(w, np.float32).reshape(R, 32)
    kc = _c(k_idx, np.uint16)
    out = np.full((R, ld), np.nan, np.float64)
    _lib().oracle_indexer_scores(R, _p(vis), _p(base), _p(q), _p(ww), _p(kc), float(index_scale), _p(out), ld)
    return out


def round_to_f32(x):
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.float32)
    _lib().oracle_round_to_f32(x.size, _p(x), _p(out))
    return out


def topk(visible_len, scores_f32, k):
    """int32 [R, k]: the k_r best positions ascending, then -1."""
    vis = _c(visible_len, np.int32)
    s = _c(scores_f32, np.float32)
    R, ld = s.shape
    out = np.empty((R, k), np.int32)
    _lib().oracle_topk(R, _p(vis), _p(s), ld, int(k), _p(out))
    return out


def sparse_mla(row_cache_base, q_abs, kv_latent, indices, softmax_scale):
    """(out [R,64,512] fp64, lse [R,64] fp64) over entries indices >= 0."""
    base = _c(row_cache_base, np.int64)
    R = base.shape[0]
    qa = _c(q_abs, np.uint16).reshape(R, 64, 576)
    kv = _c(kv_latent, np.uint16)
    idx = _c(indices, np.int32)
    k = idx.shape[1]
    out = np.empty((R, 64, 512), np.float64)
    lse = np.empty((R, 64), np.float64)
    _lib().oracle_sparse_mla(R, _p(base), _p(qa), _p(kv), _p(idx), k, float(softmax_scale), _p(out), _p(lse))
    return out, lse


def absorb_queries(q_nope, q_pe, kv_b):
    """q_abs [R,64,576] fp64 = [W_UK^T q_nope || q_pe] per head (bf16-bit inputs;
    kv_b is the kv_b_proj weight [64,448,512])."""
    qn = _c(q_nope, np.uint16).reshape(-1, 64, 192)
    R = qn.shape[0]
    qp = _c(q_pe, np.uint16).reshape(R, 64, 64)
    w = _c(kv_b, np.uint16).reshape(64, 448, 512)
    out = np.empty((R, 64, 576), np.float64)
    _lib().oracle_absorb_queries(R, _p(qn), _p(qp), _p(w), _p(out))
    return out


def v_up_proj(o, kv_b):
    """out [R,64,256] fp64 = W_UV o per head (o taken as given, in fp64)."""
    oo = _c(o, np.float64).reshape(-1, 64, 512)
    R = oo.shape[0]
    w = _c(kv_b, np.uint16).reshape(64, 448, 512)
    out = np.empty((R, 64, 256), np.float64)
    _lib().oracle_v_up_proj(R, _p(oo), _p(w), _p(out))
    return out


def decode_step(visible_len, row_cache_base, q_idx, w, k_idx, q_abs, kv_latent, k, index_scale, softmax_scale):
    """The whole path: fp64 scores, rounded to fp32 for the top-k, then attention."""
    s64 = indexer_scores(visible_len, row_cache_base, q_idx, w, k_idx, index_scale)
    s32 = round_to_f32(np.nan_to_num(s64, nan=0.0))
    idx = topk(visible_len, s32, k)
    out, lse = sparse_mla(row_cache_base, q_abs, kv_latent, idx, softmax_scale)
    return s64, s32, idx, out, lse


def cache_rows(hidden, wk, k_norm_weight, k_norm_bias, k_norm_eps, kv_a, kv_norm_weight, kv_norm_eps, positions,
               rope_theta):
    """(key [N,128], latent [N,576]) in fp64: the indexer-cache and latent-cache
    rows of N new tokens (bf16-bit hidden and weights, fp32 norm parameters)."""
    x = _c(hidden, np.uint16).reshape(-1, 6144)
    N = x.shape[0]
    wk_ = _c(wk, np.uint16).reshape(128, 6144)
    kva = _c(kv_a, np.uint16).reshape(576, 6144)
    kg, kb = _c(k_norm_weight, np.float32), _c(k_norm_bias, np.float32)
    kvg = _c(kv_norm_weight, np.float32)
    pos = _c(positions, np.int64)
    assert kg.shape == (128,) and kb.shape == (128,) and kvg.shape == (512,) and pos.shape == (N,)
    key = np.empty((N, 128), np.float64)
    lat = np.empty((N, 576), np.float64)
    _lib().oracle_cache_rows(N, _p(x), _p(wk_), _p(kg), _p(kb), ctypes.c_double(k_norm_eps), _p(kva), _p(kvg),
                             ctypes.c_double(kv_norm_eps), _p(pos), ctypes.c_double(rope_theta), _p(key), _p(lat))
    return key, lat


def depage(pool, block_table_row, length, block_size):
    """The logical cache rows [length, D] of one sequence held in a paged
    pool: position p is pool row block_table_row[p // block_size] *
    block_size + p % block_size (the block-table addressing of a paged KV
    cache, vLLM's PagedAttention, which "GLM-5.2 架构 QA" CH2 Q2.6 names)."""
    rows = [int(block_table_row[p // block_size]) * block_size + p % block_size for p in range(int(length))]
    return np.asarray(pool)[np.asarray(rows, dtype=np.int64)]


# The 78-entry indexer_types array of GLM-5.2 as "GLM-5.2 架构 QA" CH1 Q1.2
# spells it out: a cold-start block of 3 full then 3 shared layers, then 18
# periods of one full layer followed by 3 shared ones.
GLM52_INDEXER_TYPES = ["full"] * 3 + ["shared"] * 3 + (["full"] + ["shared"] * 3) * 18


def index_share_layers(types, layers, visible_len, row_cache_base, k, index_scale, softmax_scale):
    """IndexShare over consecutive layers ("GLM-5.2 架构 QA" CH2 Q2.1, Q2.2):
    a "full" layer runs the whole path on its own indexer inputs and its list
    becomes the shared one; a "shared" layer runs attention alone over the
    latest full layer's list.  `layers[i]` holds layer i's q_abs and kv_latent
    (and q_idx, w, k_idx for a full layer).  Returns, per layer, (idx, out,
    lse) with idx the list the layer attended over."""
    shared_idx = None
    res = []
    for kind, x in zip(types, layers):
        if kind == "full":
            _, _, shared_idx, out, lse = decode_step(visible_len, row_cache_base, x["q_idx"], x["w"], x["k_idx"],
                                                     x["q_abs"], x["kv_latent"], k, index_scale, softmax_scale)
        elif kind == "shared":
            if shared_idx is None:
                raise ValueError("a shared layer needs a full layer before it")
            out, lse = sparse_mla(row_cache_base, x["q_abs"], x["kv_latent"], shared_idx, softmax_scale)
        else:
            raise ValueError(kind)
        res.append((shared_idx, out, lse))
    return res


def version():
    return _lib().oracle_version().decode()
