"""Python binding of libdsa (the DSA hot path on MI355X / gfx950).

Argument marshalling only: every function below checks tensor placement and
dtype, turns tensors into device pointers and calls the C ABI entry point of
the same name declared in include/dsa.h.  All arithmetic runs in the HIP
kernels of libdsa.so.  There is no fallback: if the library is missing or the
device is not a gfx950, calls raise.

PyTorch supplies device memory and streams only.  bf16 inputs are
torch.bfloat16 tensors (or int16/uint16 views of the same bits).
"""
import ctypes
import os

import torch

__all__ = [
    "DsaError", "Rows", "library_path", "load_library", "dsa_version", "exported_symbols",
    "dsa_indexer_scores", "dsa_topk_workspace_size", "dsa_topk_select",
    "dsa_sparse_mla_workspace_size", "dsa_sparse_mla_attn",
    "dsa_decode_step_workspace_size", "dsa_decode_step", "workspace", "dsa_absorb_queries", "dsa_v_up_proj",
    "dsa_index_share_source", "dsa_cache_write_workspace_size", "dsa_cache_write", "Paged",
    "dsa_indexer_scores_paged", "dsa_sparse_mla_paged_workspace_size", "dsa_sparse_mla_attn_paged",
    "dsa_decode_step_paged_workspace_size", "dsa_decode_step_paged", "HIDDEN",
    "INDEX_HEADS", "INDEX_DIM", "HEADS", "LATENT_DIM", "ROPE_DIM", "ROW_DIM", "TOPK_MAX",
    "ROWS_DISTINCT_SEQUENCES", "dsa_decode_step_noalloc", "NOALLOC_SCRATCH_BYTES",
]

INDEX_HEADS = 32
INDEX_DIM = 128
HEADS = 64
LATENT_DIM = 512
ROPE_DIM = 64
ROW_DIM = 576
TOPK_MAX = 2048
HIDDEN = 6144
NOALLOC_SCRATCH_BYTES = 128 << 20

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB = None

STATUS_NAMES = {
    0: "DSA_OK", 1: "DSA_ERR_INVALID_ARGUMENT", 2: "DSA_ERR_MISALIGNED",
    3: "DSA_ERR_WORKSPACE_TOO_SMALL", 4: "DSA_ERR_NO_DEVICE", 5: "DSA_ERR_HIP",
}


class DsaError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        self.detail = detail
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")


class _CRows(ctypes.Structure):
    _fields_ = [
        ("num_rows", ctypes.c_int32),
        ("max_visible", ctypes.c_int32),
        ("visible_len", ctypes.c_void_p),
        ("row_cache_base", ctypes.c_void_p),
        ("flags", ctypes.c_uint32),
    ]


def library_path():
    return os.path.join(_PKG_DIR, "libdsa.so")


def load_library():
    """Load libdsa.so (built by __graft_entry__.build()); raises if absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    rows_p = ctypes.POINTER(_CRows)
    paged_p = ctypes.POINTER(_CPaged)
    sigs = {
        "dsa_version": ([], ctypes.c_char_p),
        "dsa_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "dsa_last_error_detail": ([], ctypes.c_char_p),
        "dsa_indexer_scores": ([rows_p, P, P, P, f32, P, i64, P], ctypes.c_int),
        "dsa_topk_workspace_size": ([i32, i32, i32], sz),
        "dsa_topk_select": ([rows_p, P, i64, i32, P, P, sz, P], ctypes.c_int),
        "dsa_sparse_mla_workspace_size": ([i32, i32], sz),
        "dsa_sparse_mla_attn": ([rows_p, P, P, P, i32, f32, P, P, P, sz, P], ctypes.c_int),
        "dsa_decode_step_workspace_size": ([i32, i32, i32], sz),
        "dsa_decode_step": ([rows_p, P, P, P, f32, P, P, f32, i32, P, P, P, P, sz, P], ctypes.c_int),
        "dsa_absorb_queries": ([i32, P, P, P, P, P], ctypes.c_int),
        "dsa_v_up_proj": ([i32, P, P, P, P], ctypes.c_int),
        "dsa_index_share_source": ([i32, i32, i32, i32], i32),
        "dsa_cache_write_workspace_size": ([i32], sz),
        "dsa_indexer_scores_paged": ([rows_p, paged_p, P, P, P, f32, P, i64, P], ctypes.c_int),
        "dsa_sparse_mla_paged_workspace_size": ([i32, i32], sz),
        "dsa_sparse_mla_attn_paged": ([rows_p, paged_p, P, P, P, i32, f32, P, P, P, sz, P], ctypes.c_int),
        "dsa_decode_step_paged_workspace_size": ([i32, i32, i32], sz),
        "dsa_decode_step_paged": ([rows_p, paged_p, P, P, P, f32, P, P, f32, i32, P, P, P, P, sz, P], ctypes.c_int),
        "dsa_cache_write": ([i32, P, P, P, P, f32, P, P, f32, P, P, ctypes.c_double, P, P, P, sz, P], ctypes.c_int),
        "dsa_decode_step_noalloc": ([rows_p, P, P, P, f32, P, P, f32, i32, P, P, P, P], ctypes.c_int),
    }
    for name, (argtypes, restype) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = restype
    _LIB = lib
    return lib


def exported_symbols():
    """Names of the C ABI entry points the binding expects."""
    return [
        "dsa_version", "dsa_status_string", "dsa_last_error_detail", "dsa_indexer_scores",
        "dsa_topk_workspace_size", "dsa_topk_select", "dsa_sparse_mla_workspace_size",
        "dsa_sparse_mla_attn", "dsa_decode_step_workspace_size", "dsa_decode_step", "dsa_absorb_queries",
        "dsa_v_up_proj", "dsa_index_share_source", "dsa_cache_write_workspace_size", "dsa_cache_write",
        "dsa_indexer_scores_paged", "dsa_sparse_mla_paged_workspace_size", "dsa_sparse_mla_attn_paged",
        "dsa_decode_step_paged_workspace_size", "dsa_decode_step_paged", "dsa_decode_step_noalloc",
    ]


def dsa_version():
    return load_library().dsa_version().decode()


def _check(status):
    if status != 0:
        lib = load_library()
        raise DsaError(status, lib.dsa_last_error_detail().decode())


def _ptr(t, name, dtypes=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t.data_ptr()


def _need(t, count, name):
    """Raises DsaError (invalid argument) unless tensor t holds at least
    `count` elements.  The C ABI sees only pointers, so the binding checks
    every buffer against the call's dimensions before any kernel could read
    or write past it."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.numel() < count:
        raise DsaError(1, f"{name} holds {t.numel()} elements, the call needs at least {count}")


def _scores_ld(rows, scores, ld):
    """Row stride of a scores buffer: its last dimension unless given; the
    buffer must hold num_rows rows of that stride, each >= max_visible."""
    if scores is None:
        return 0 if ld is None else int(ld)
    ld = int(scores.shape[-1]) if ld is None else int(ld)
    if ld < rows.max_visible:
        raise DsaError(1, f"scores row stride {ld} < max_visible {rows.max_visible}")
    _need(scores, rows.num_rows * ld, "scores")
    return ld


def _need_rows(rows, q_idx=None, w=None, q_abs=None, indices=None, k=None, out_latent=None, out_lse=None):
    R = rows.num_rows
    _need(q_idx, R * INDEX_HEADS * INDEX_DIM, "q_idx")
    _need(w, R * INDEX_HEADS, "w")
    _need(q_abs, R * HEADS * ROW_DIM, "q_abs")
    if indices is not None and k is not None:
        _need(indices, R * int(k), "indices")
    _need(out_latent, R * HEADS * LATENT_DIM, "out_latent")
    _need(out_lse, R * HEADS, "out_lse")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _stream(stream, ref):
    if stream is None:
        return torch.cuda.current_stream(ref.device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


ROWS_DISTINCT_SEQUENCES = 1


class _CPaged(ctypes.Structure):
    _fields_ = [
        ("block_table", ctypes.c_void_p),
        ("max_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
    ]


class Rows:
    """Query-row description (dsa_rows_t): device visible_len [R] int32,
    device row_cache_base [R] int64, the host bound max_visible and the
    DSA_ROWS_* hint flags (performance only; results never depend on them)."""

    def __init__(self, visible_len, row_cache_base, max_visible, flags=0):
        if visible_len.dtype != torch.int32 or row_cache_base.dtype != torch.int64:
            raise TypeError("visible_len must be int32 and row_cache_base int64")
        if visible_len.numel() != row_cache_base.numel():
            raise ValueError("visible_len and row_cache_base differ in length")
        self.visible_len = visible_len
        self.row_cache_base = row_cache_base
        self.num_rows = int(visible_len.numel())
        self.max_visible = int(max_visible)
        self.flags = int(flags)
        self._c = _CRows(self.num_rows, self.max_visible, _ptr(visible_len, "visible_len", (torch.int32,)),
                         _ptr(row_cache_base, "row_cache_base", (torch.int64,)), self.flags)

    @property
    def c(self):
        return ctypes.byref(self._c)


class Paged:
    """Paged-cache description (dsa_paged_t): device block_table [S, max_blocks]
    int32 of pool block numbers and the block size (a power of two >= 16).
    In paged calls a Rows object's row_cache_base holds each row's block-table
    row."""

    def __init__(self, block_table, block_size):
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
            raise TypeError("block_table must be a contiguous 2-D int32 tensor")
        self.block_table = block_table
        self.max_blocks = int(block_table.shape[1])
        self.block_size = int(block_size)
        self._c = _CPaged(_ptr(block_table, "block_table", (torch.int32,)), self.max_blocks, self.block_size)

    @property
    def c(self):
        return ctypes.byref(self._c)


def workspace(nbytes, device):
    """A device byte buffer of at least nbytes (torch allocations are 256-B aligned)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def dsa_indexer_scores(rows, q_idx, w, k_idx, index_scale, scores, ld=None, stream=None):
    lib = load_library()
    _need_rows(rows, q_idx=q_idx, w=w)
    ld = _scores_ld(rows, scores, ld)
    _check(lib.dsa_indexer_scores(rows.c, _ptr(q_idx, "q_idx", _BF16), _ptr(w, "w", (torch.float32,)),
                                  _ptr(k_idx, "k_idx", _BF16), float(index_scale),
                                  _ptr(scores, "scores", (torch.float32,)), int(ld), _stream(stream, scores)))


def dsa_topk_workspace_size(num_rows, max_visible, k):
    return int(load_library().dsa_topk_workspace_size(int(num_rows), int(max_visible), int(k)))


def dsa_topk_select(rows, scores, k, indices, ws, ld=None, stream=None):
    lib = load_library()
    _need_rows(rows, indices=indices, k=k)
    ld = _scores_ld(rows, scores, ld)
    _check(lib.dsa_topk_select(rows.c, _ptr(scores, "scores", (torch.float32,)), int(ld), int(k),
                               _ptr(indices, "indices", (torch.int32,)), _ptr(ws, "ws"),
                               ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream, scores)))


def dsa_sparse_mla_workspace_size(num_rows, k):
    return int(load_library().dsa_sparse_mla_workspace_size(int(num_rows), int(k)))


def dsa_sparse_mla_attn(rows, q_abs, kv_latent, indices, k, softmax_scale, out_latent, out_lse=None, ws=None,
                        stream=None):
    lib = load_library()
    _need_rows(rows, q_abs=q_abs, indices=indices, k=k, out_latent=out_latent, out_lse=out_lse)
    _check(lib.dsa_sparse_mla_attn(rows.c, _ptr(q_abs, "q_abs", _BF16), _ptr(kv_latent, "kv_latent", _BF16),
                                   _ptr(indices, "indices", (torch.int32,)), int(k), float(softmax_scale),
                                   _ptr(out_latent, "out_latent", (torch.float32,)),
                                   _ptr(out_lse, "out_lse", (torch.float32,)), _ptr(ws, "ws"),
                                   ws.numel() * ws.element_size() if ws is not None else 0,
                                   _stream(stream, out_latent)))


def dsa_decode_step_workspace_size(num_rows, max_visible, k):
    return int(load_library().dsa_decode_step_workspace_size(int(num_rows), int(max_visible), int(k)))


def dsa_decode_step(rows, q_idx, w, k_idx, index_scale, q_abs, kv_latent, softmax_scale, k, indices, out_latent,
                    out_lse=None, ws=None, stream=None):
    lib = load_library()
    _need_rows(rows, q_idx=q_idx, w=w, q_abs=q_abs, indices=indices, k=k, out_latent=out_latent, out_lse=out_lse)
    _check(lib.dsa_decode_step(rows.c, _ptr(q_idx, "q_idx", _BF16), _ptr(w, "w", (torch.float32,)),
                               _ptr(k_idx, "k_idx", _BF16), float(index_scale), _ptr(q_abs, "q_abs", _BF16),
                               _ptr(kv_latent, "kv_latent", _BF16), float(softmax_scale), int(k),
                               _ptr(indices, "indices", (torch.int32,)),
                               _ptr(out_latent, "out_latent", (torch.float32,)),
                               _ptr(out_lse, "out_lse", (torch.float32,)), _ptr(ws, "ws"),
                               ws.numel() * ws.element_size() if ws is not None else 0,
                               _stream(stream, out_latent)))


def dsa_absorb_queries(q_nope, q_pe, kv_b_weight, q_abs, stream=None):
    """q_abs [R,64,576] bf16 = [W_UK^T q_nope || q_pe] per head."""
    lib = load_library()
    R = int(q_nope.shape[0])
    _need(q_nope, R * HEADS * 192, "q_nope")
    _need(q_pe, R * HEADS * ROPE_DIM, "q_pe")
    _need(kv_b_weight, HEADS * 448 * LATENT_DIM, "kv_b_weight")
    _need(q_abs, R * HEADS * ROW_DIM, "q_abs")
    _check(lib.dsa_absorb_queries(R, _ptr(q_nope, "q_nope", _BF16), _ptr(q_pe, "q_pe", _BF16),
                                  _ptr(kv_b_weight, "kv_b_weight", _BF16), _ptr(q_abs, "q_abs", _BF16),
                                  _stream(stream, q_abs)))


def dsa_v_up_proj(o_latent, kv_b_weight, out, stream=None):
    """out [R,64,256] fp32 = W_UV bf16(o_latent) per head."""
    lib = load_library()
    R = int(o_latent.shape[0])
    _need(o_latent, R * HEADS * LATENT_DIM, "o_latent")
    _need(kv_b_weight, HEADS * 448 * LATENT_DIM, "kv_b_weight")
    _need(out, R * HEADS * 256, "out")
    _check(lib.dsa_v_up_proj(R, _ptr(o_latent, "o_latent", (torch.float32,)),
                             _ptr(kv_b_weight, "kv_b_weight", _BF16), _ptr(out, "out", (torch.float32,)),
                             _stream(stream, out)))


def dsa_index_share_source(layer, num_layers=78, leading_full=3, freq=4):
    """The layer whose top-k selection `layer` attends over (itself for a full
    layer); raises on arguments the C call rejects."""
    src = load_library().dsa_index_share_source(int(layer), int(num_layers), int(leading_full), int(freq))
    if src < 0:
        raise DsaError(1, f"dsa_index_share_source({layer}, {num_layers}, {leading_full}, {freq}): bad arguments")
    return int(src)


def dsa_cache_write_workspace_size(num_tokens):
    return int(load_library().dsa_cache_write_workspace_size(int(num_tokens)))


def dsa_cache_write(hidden, wk_weight, k_norm_weight, k_norm_bias, k_norm_eps, kv_a_weight, kv_norm_weight,
                    kv_norm_eps, positions, slots, rope_theta, k_idx_cache, kv_latent_cache, ws, stream=None):
    """Writes the indexer-key and latent rows of len(hidden) new tokens at
    rows `slots` of the two caches (negative slot: token skipped)."""
    lib = load_library()
    N = int(hidden.shape[0])
    _need(hidden, N * HIDDEN, "hidden")
    _need(wk_weight, INDEX_DIM * HIDDEN, "wk_weight")
    _need(k_norm_weight, INDEX_DIM, "k_norm_weight")
    _need(k_norm_bias, INDEX_DIM, "k_norm_bias")
    _need(kv_a_weight, ROW_DIM * HIDDEN, "kv_a_weight")
    _need(kv_norm_weight, LATENT_DIM, "kv_norm_weight")
    _need(positions, N, "positions")
    _need(slots, N, "slots")
    _check(lib.dsa_cache_write(N, _ptr(hidden, "hidden", _BF16), _ptr(wk_weight, "wk_weight", _BF16),
                               _ptr(k_norm_weight, "k_norm_weight", (torch.float32,)),
                               _ptr(k_norm_bias, "k_norm_bias", (torch.float32,)), float(k_norm_eps),
                               _ptr(kv_a_weight, "kv_a_weight", _BF16),
                               _ptr(kv_norm_weight, "kv_norm_weight", (torch.float32,)), float(kv_norm_eps),
                               _ptr(positions, "positions", (torch.int32,)), _ptr(slots, "slots", (torch.int64,)),
                               float(rope_theta), _ptr(k_idx_cache, "k_idx_cache", _BF16),
                               _ptr(kv_latent_cache, "kv_latent_cache", _BF16), _ptr(ws, "ws"),
                               ws.numel() * ws.element_size() if ws is not None else 0,
                               _stream(stream, hidden)))


def dsa_indexer_scores_paged(rows, paged, q_idx, w, k_pool, index_scale, scores, ld=None, stream=None):
    lib = load_library()
    _need_rows(rows, q_idx=q_idx, w=w)
    ld = _scores_ld(rows, scores, ld)
    _check(lib.dsa_indexer_scores_paged(rows.c, paged.c, _ptr(q_idx, "q_idx", _BF16), _ptr(w, "w", (torch.float32,)),
                                        _ptr(k_pool, "k_pool", _BF16), float(index_scale),
                                        _ptr(scores, "scores", (torch.float32,)), int(ld), _stream(stream, scores)))


def dsa_sparse_mla_paged_workspace_size(num_rows, k):
    return int(load_library().dsa_sparse_mla_paged_workspace_size(int(num_rows), int(k)))


def dsa_sparse_mla_attn_paged(rows, paged, q_abs, kv_pool, indices, k, softmax_scale, out_latent, out_lse=None,
                              ws=None, stream=None):
    lib = load_library()
    _need_rows(rows, q_abs=q_abs, indices=indices, k=k, out_latent=out_latent, out_lse=out_lse)
    _check(lib.dsa_sparse_mla_attn_paged(rows.c, paged.c, _ptr(q_abs, "q_abs", _BF16), _ptr(kv_pool, "kv_pool", _BF16),
                                         _ptr(indices, "indices", (torch.int32,)), int(k), float(softmax_scale),
                                         _ptr(out_latent, "out_latent", (torch.float32,)),
                                         _ptr(out_lse, "out_lse", (torch.float32,)), _ptr(ws, "ws"),
                                         ws.numel() * ws.element_size() if ws is not None else 0,
                                         _stream(stream, out_latent)))


def dsa_decode_step_paged_workspace_size(num_rows, max_visible, k):
    return int(load_library().dsa_decode_step_paged_workspace_size(int(num_rows), int(max_visible), int(k)))


def dsa_decode_step_paged(rows, paged, q_idx, w, k_pool, index_scale, q_abs, kv_pool, softmax_scale, k, indices,
                          out_latent, out_lse=None, ws=None, stream=None):
    lib = load_library()
    _need_rows(rows, q_idx=q_idx, w=w, q_abs=q_abs, indices=indices, k=k, out_latent=out_latent, out_lse=out_lse)
    _check(lib.dsa_decode_step_paged(rows.c, paged.c, _ptr(q_idx, "q_idx", _BF16), _ptr(w, "w", (torch.float32,)),
                                     _ptr(k_pool, "k_pool", _BF16), float(index_scale), _ptr(q_abs, "q_abs", _BF16),
                                     _ptr(kv_pool, "kv_pool", _BF16), float(softmax_scale), int(k),
                                     _ptr(indices, "indices", (torch.int32,)),
                                     _ptr(out_latent, "out_latent", (torch.float32,)),
                                     _ptr(out_lse, "out_lse", (torch.float32,)), _ptr(ws, "ws"),
                                     ws.numel() * ws.element_size() if ws is not None else 0,
                                     _stream(stream, out_latent)))


def dsa_decode_step_noalloc(rows, q_idx, w, k_idx, index_scale, q_abs, kv_latent, softmax_scale, k, indices,
                            out_latent, out_lse=None, stream=None):
    """dsa_decode_step without a workspace argument: the library's per-device
    scratch array serves as the workspace (nothing is allocated; calls that
    overlap on one device race)."""
    lib = load_library()
    _need_rows(rows, q_idx=q_idx, w=w, q_abs=q_abs, indices=indices, k=k, out_latent=out_latent, out_lse=out_lse)
    _check(lib.dsa_decode_step_noalloc(rows.c, _ptr(q_idx, "q_idx", _BF16), _ptr(w, "w", (torch.float32,)),
                                       _ptr(k_idx, "k_idx", _BF16), float(index_scale), _ptr(q_abs, "q_abs", _BF16),
                                       _ptr(kv_latent, "kv_latent", _BF16), float(softmax_scale), int(k),
                                       _ptr(indices, "indices", (torch.int32,)),
                                       _ptr(out_latent, "out_latent", (torch.float32,)),
                                       _ptr(out_lse, "out_lse", (torch.float32,)), _stream(stream, out_latent)))
