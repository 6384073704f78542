"""Python binding of libpagedkv (paged decode attention for MI355X / gfx950).

Thin ctypes marshalling over the C ABI in include/pagedkv.h; the functions
carry the C names. Tensors are PyTorch device tensors (PyTorch supplies
device memory and the stream); every step of the computation runs in the
HIP kernels of libpagedkv.so. The library is loaded on first use and a
missing build is an error: there is no fallback path.

    pa_decode(q, k_pool, v_pool, block_tables, seq_lens, scale, out, ...)
    pa_decode_append(q, k_new, v_new, slot_mapping, k_pool, v_pool,
                     block_tables, seq_lens, scale, out, ...)
    pa_prefill(q, k_pool, v_pool, block_tables, seq_lens, query_start, scale, out)
    pa_write_kv(k_new, v_new, slot_mapping, k_pool, v_pool)
    pa_copy_blocks(k_pool, v_pool, block_mapping)
    pa_decode_workspace_bytes(dims)
    pa_latent_decode(q, kv_pool, block_tables, seq_lens, scale, out, ...)
    pa_latent_write(kv_new, slot_mapping, kv_pool)
    pa_latent_workspace_bytes(dims)

Layouts: q/out [B, Hq, D]; k_pool [NB, Hkv, BS, D]; v_pool [NB, Hkv, D, BS]
(BS = 16 tokens per block; 8 .. 256 with the balanced split, V as
[NB, Hkv, BS // 16, D, 16] beyond 16);
block_tables int32 [B, MB]; seq_lens int32 [B]; k_new/v_new [T, Hkv, D];
slot_mapping int32 [T]; block_mapping int32 [n, 2].
Latent decode: q [B, 128, 576], kv_pool [NB, 64, 576], out [B, 128, 512],
kv_new [T, 576].
"""

from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

__all__ = [
    "PA_OK", "PA_ERR_INVALID_ARG", "PA_ERR_UNSUPPORTED", "PA_ERR_LAUNCH",
    "PaDims", "PagedKVError", "SYMBOLS", "load_library", "make_dims",
    "PARTITION_AUTO", "pa_decode", "pa_decode_append", "pa_decode_noalloc", "pa_decode_contiguous",
    "pa_decode_workspace_bytes",
    "pa_prefill", "pa_write_kv", "NOALLOC_SCRATCH_BYTES",
    "pa_copy_blocks", "PaLatentDims", "make_latent_dims", "pa_latent_decode",
    "pa_latent_write", "pa_latent_workspace_bytes",
    "pa_status_string", "pa_version", "validate",
]

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_LAUNCH = 0, 1, 2, 3
PA_F32, PA_BF16 = 0, 1
PARTITION_AUTO = -1  # PA_PARTITION_AUTO: the library's split, chosen from the dims
KERNELS = {"auto": 0, "valu": 1, "mfma": 2}
BLOCK_SIZE = 16

SYMBOLS = ("pa_decode_workspace_bytes", "pa_decode", "pa_decode_noalloc", "pa_decode_contiguous",
           "pa_decode_append",
           "pa_prefill",
           "pa_write_kv", "pa_copy_blocks", "pa_latent_workspace_bytes", "pa_latent_decode",
           "pa_latent_write", "pa_status_string", "pa_version")
LATENT_HEADS, LATENT_DIM, LATENT_VALUE_DIM, LATENT_BLOCK = 128, 576, 512, 64
NOALLOC_SCRATCH_BYTES = 32 << 20  # PA_NOALLOC_SCRATCH_BYTES


class PaDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "block_size",
        "max_blocks_per_seq", "num_blocks", "partition_tokens", "dtype",
        "kernel")]


class PaLatentDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_heads", "latent_dim", "value_dim", "block_size",
        "max_blocks_per_seq", "num_blocks", "dtype")]


class PagedKVError(RuntimeError):
    def __init__(self, call, status):
        super().__init__(f"{call}: {pa_status_string(status)} (status {status})")
        self.status = status


_LIB = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpagedkv.so once; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m paged_kv_cache_55_amd.build` "
            "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P, I32, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    D = ctypes.POINTER(PaDims)
    lib.pa_decode_workspace_bytes.argtypes = [D]
    lib.pa_decode_workspace_bytes.restype = SZ
    lib.pa_decode.argtypes = [P, P, P, P, P, F32, P, D, P, SZ, P]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_contiguous.argtypes = [P, P, P, P, F32, P, D, P, SZ, P]
    lib.pa_decode_contiguous.restype = ctypes.c_int
    lib.pa_decode_noalloc.argtypes = [P, P, P, P, P, F32, P, D, P]
    lib.pa_decode_noalloc.restype = ctypes.c_int
    lib.pa_decode_append.argtypes = [P, P, P, P, P, P, P, P, F32, P, D, P, SZ, P]
    lib.pa_decode_append.restype = ctypes.c_int
    lib.pa_prefill.argtypes = [P, P, P, P, P, P, I32, F32, P, D, P]
    lib.pa_prefill.restype = ctypes.c_int
    lib.pa_write_kv.argtypes = [P, P, P, I32, P, P, D, P]
    lib.pa_write_kv.restype = ctypes.c_int
    lib.pa_copy_blocks.argtypes = [P, P, P, I32, D, P]
    lib.pa_copy_blocks.restype = ctypes.c_int
    LD = ctypes.POINTER(PaLatentDims)
    lib.pa_latent_workspace_bytes.argtypes = [LD]
    lib.pa_latent_workspace_bytes.restype = SZ
    lib.pa_latent_decode.argtypes = [P, P, P, P, F32, P, LD, P, SZ, P]
    lib.pa_latent_decode.restype = ctypes.c_int
    lib.pa_latent_write.argtypes = [P, P, I32, P, LD, P]
    lib.pa_latent_write.restype = ctypes.c_int
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_version.argtypes = []
    lib.pa_version.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def pa_status_string(status: int) -> str:
    return load_library().pa_status_string(int(status)).decode()


def pa_version() -> str:
    return load_library().pa_version().decode()


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def make_dims(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
              num_blocks, dtype, partition_tokens=512, kernel="auto",
              block_size=BLOCK_SIZE) -> PaDims:
    return PaDims(int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_dim),
                  int(block_size), int(max_blocks_per_seq), int(num_blocks),
                  int(partition_tokens), int(dtype), KERNELS[kernel])


def _pool_dims(k_pool, v_pool):
    """(NB, Hkv, D, block size) of a K/V pool pair; the library checks that
    the block size is supported. V is [NB, Hkv, D, BS] for blocks of up to
    16 tokens and [NB, Hkv, BS // 16, D, 16] (a dim-major tile per 16
    tokens) for longer ones."""
    _need(k_pool.dim() == 4, "k_pool must be [NB, Hkv, BS, D]")
    NB, Hkv, BS, D = k_pool.shape
    if BS <= BLOCK_SIZE:
        _need(tuple(v_pool.shape) == (NB, Hkv, D, BS), "v_pool must be [NB, Hkv, D, BS]")
    else:
        _need(tuple(v_pool.shape) == (NB, Hkv, BS // BLOCK_SIZE, D, BLOCK_SIZE)
              and BS % BLOCK_SIZE == 0, "v_pool must be [NB, Hkv, BS // 16, D, 16]")
    _need(k_pool.dtype == v_pool.dtype, "k_pool and v_pool dtypes differ")
    _need(k_pool.is_contiguous() and v_pool.is_contiguous(), "pools must be contiguous")
    _need(k_pool.is_cuda and v_pool.is_cuda, "pools must be device tensors")
    return NB, Hkv, D, BS


def pa_decode_workspace_bytes(dims: PaDims) -> int:
    return int(load_library().pa_decode_workspace_bytes(ctypes.byref(dims)))


def _decode_dims(q, k_pool, v_pool, block_tables, seq_lens, out, partition_tokens, kernel):
    torch = _torch()
    NB, Hkv, D, BS = _pool_dims(k_pool, v_pool)
    _need(q.dim() == 3 and q.shape[2] == D, "q must be [B, Hq, D]")
    B, Hq, _ = q.shape
    _need(q.dtype == k_pool.dtype, "q and pools must share a dtype")
    _need(q.is_contiguous() and q.is_cuda, "q must be a contiguous device tensor")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == B and block_tables.is_contiguous()
          and block_tables.is_cuda, "block_tables must be int32 [B, MB] on the device")
    _need(seq_lens.dtype == torch.int32 and tuple(seq_lens.shape) == (B,)
          and seq_lens.is_contiguous() and seq_lens.is_cuda,
          "seq_lens must be int32 [B] on the device")
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous()
          and out.is_cuda, "out must match q")
    dims = make_dims(B, Hq, Hkv, D, block_tables.shape[1], NB, _dtype_code(q),
                     partition_tokens, kernel, BS)
    return dims, out


def _workspace(dims, workspace, device):
    need = pa_decode_workspace_bytes(dims)
    if need and workspace is None:
        # zero-filled once; pa_decode leaves it reusable
        workspace = _torch().zeros(need, dtype=_torch().uint8, device=device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, ws_bytes


def pa_decode(q, k_pool, v_pool, block_tables, seq_lens, scale, out=None, *,
              partition_tokens=PARTITION_AUTO, kernel="auto", workspace=None, stream=None):
    """out[b, h] = softmax(scale * q[b, h] K_b^T) V_b over the paged K/V.

    ``partition_tokens`` > 0 splits each sequence into partitions of that
    many tokens; 0 asks for the balanced split (matrix-core kernel) or one
    partition per sequence (vector-ALU kernel); PARTITION_AUTO (the
    default) lets the library choose from the dims. A caller-provided
    ``workspace`` (uint8 device tensor of at least
    pa_decode_workspace_bytes bytes) must be zero-filled before its first
    use; calls with the same dims leave it reusable (zero-fill it again
    before a call with other dims or another split). One workspace must not
    serve two calls that can run at the same time.
    """
    dims, out = _decode_dims(q, k_pool, v_pool, block_tables, seq_lens, out,
                             partition_tokens, kernel)
    workspace, ws_bytes = _workspace(dims, workspace, q.device)
    st = load_library().pa_decode(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                  _ptr(seq_lens), ctypes.c_float(scale), _ptr(out),
                                  ctypes.byref(dims), _ptr(workspace), ctypes.c_size_t(ws_bytes),
                                  _stream(stream))
    if st != PA_OK:
        raise PagedKVError("pa_decode", st)
    return out


def pa_decode_contiguous(q, k_cache, v_cache, seq_lens, scale, out=None, *, workspace=None,
                         stream=None):
    """Decode attention over an unpaged cache: k_cache [B, Hkv, Lmax, D],
    v_cache [B, Hkv, Lmax // 16, D, 16]; token t of row b at slot t, no
    table. The balanced split of the matrix-core kernel (bf16)."""
    torch = _torch()
    _need(k_cache.dim() == 4 and v_cache.dim() == 5, "k_cache [B, Hkv, Lmax, D], "
          "v_cache [B, Hkv, Lmax // 16, D, 16]")
    B, Hkv, lmax, D = k_cache.shape
    _need(lmax % BLOCK_SIZE == 0 and tuple(v_cache.shape) == (B, Hkv, lmax // BLOCK_SIZE, D,
                                                              BLOCK_SIZE),
          "v_cache must be [B, Hkv, Lmax // 16, D, 16] with Lmax a multiple of 16")
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (q, "q")):
        _need(t.is_contiguous() and t.is_cuda and t.dtype == k_cache.dtype,
              f"{n} must be a contiguous device tensor of the caches' dtype")
    _need(q.dim() == 3 and q.shape[0] == B and q.shape[2] == D, "q must be [B, Hq, D]")
    _need(seq_lens.dtype == torch.int32 and tuple(seq_lens.shape) == (B,)
          and seq_lens.is_contiguous() and seq_lens.is_cuda,
          "seq_lens must be int32 [B] on the device")
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous()
          and out.is_cuda, "out must match q")
    dims = make_dims(B, q.shape[1], Hkv, D, lmax // BLOCK_SIZE, B, _dtype_code(q), 0, "mfma")
    workspace, ws_bytes = _workspace(dims, workspace, q.device)
    st = load_library().pa_decode_contiguous(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                             _ptr(seq_lens), ctypes.c_float(scale), _ptr(out),
                                             ctypes.byref(dims), _ptr(workspace),
                                             ctypes.c_size_t(ws_bytes), _stream(stream))
    if st != PA_OK:
        raise PagedKVError("pa_decode_contiguous", st)
    return out


def pa_decode_noalloc(q, k_pool, v_pool, block_tables, seq_lens, scale, out=None, *,
                      partition_tokens=PARTITION_AUTO, kernel="auto", stream=None):
    """pa_decode with the library's own per-GPU scratch array as workspace:
    the library call allocates nothing (pass ``out`` to allocate nothing
    here either). Calls that may overlap in time on one GPU race."""
    dims, out = _decode_dims(q, k_pool, v_pool, block_tables, seq_lens, out,
                             partition_tokens, kernel)
    st = load_library().pa_decode_noalloc(_ptr(q), _ptr(k_pool), _ptr(v_pool),
                                          _ptr(block_tables), _ptr(seq_lens),
                                          ctypes.c_float(scale), _ptr(out), ctypes.byref(dims),
                                          _stream(stream))
    if st != PA_OK:
        raise PagedKVError("pa_decode_noalloc", st)
    return out


def pa_decode_append(q, k_new, v_new, slot_mapping, k_pool, v_pool, block_tables, seq_lens,
                     scale, out=None, *, partition_tokens=PARTITION_AUTO, kernel="auto",
                     workspace=None,
                     stream=None):
    """One decode step: row b's new token (k_new/v_new[b], [B, Hkv, D]) is
    stored at slot_mapping[b] (negative = none), which must be the slot of
    position seq_lens[b] - 1 of row b, then out = pa_decode(...) over the
    updated pools. With the balanced split this is a single kernel."""
    torch = _torch()
    dims, out = _decode_dims(q, k_pool, v_pool, block_tables, seq_lens, out,
                             partition_tokens, kernel)
    B, Hkv, D = dims.num_seqs, dims.num_kv_heads, dims.head_dim
    _need(slot_mapping.dtype == torch.int32 and tuple(slot_mapping.shape) == (B,)
          and slot_mapping.is_contiguous() and slot_mapping.is_cuda,
          "slot_mapping must be int32 [B] on the device")
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(tuple(t.shape) == (B, Hkv, D) and t.dtype == k_pool.dtype
              and t.is_contiguous() and t.is_cuda, f"{n} must be [B, Hkv, D] like the pools")
    workspace, ws_bytes = _workspace(dims, workspace, q.device)
    st = load_library().pa_decode_append(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_pool), _ptr(v_pool),
        _ptr(block_tables), _ptr(seq_lens), ctypes.c_float(scale), _ptr(out),
        ctypes.byref(dims), _ptr(workspace), ctypes.c_size_t(ws_bytes), _stream(stream))
    if st != PA_OK:
        raise PagedKVError("pa_decode_append", st)
    return out


def pa_prefill(q, k_pool, v_pool, block_tables, seq_lens, query_start, scale, out=None, *,
               stream=None):
    """Chunked-prefill attention: sequence s owns q rows query_start[s] ..
    query_start[s + 1] - 1 (its newest tokens, already in the pools), each
    attending causally to the sequence's tokens up to its own position."""
    torch = _torch()
    NB, Hkv, D, BS = _pool_dims(k_pool, v_pool)
    _need(q.dim() == 3 and q.shape[2] == D and q.dtype == k_pool.dtype
          and q.is_contiguous() and q.is_cuda, "q must be [T, Hq, D] like the pools")
    T, Hq, _ = q.shape
    S = seq_lens.shape[0]
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == S and block_tables.is_contiguous()
          and block_tables.is_cuda, "block_tables must be int32 [S, MB] on the device")
    _need(seq_lens.dtype == torch.int32 and seq_lens.dim() == 1 and seq_lens.is_contiguous()
          and seq_lens.is_cuda, "seq_lens must be int32 [S] on the device")
    _need(query_start.dtype == torch.int32 and tuple(query_start.shape) == (S + 1,)
          and query_start.is_contiguous() and query_start.is_cuda,
          "query_start must be int32 [S + 1] on the device")
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous()
          and out.is_cuda, "out must match q")
    dims = make_dims(S, Hq, Hkv, D, block_tables.shape[1], NB, _dtype_code(q), 0, "mfma", BS)
    st = load_library().pa_prefill(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                   _ptr(seq_lens), _ptr(query_start), T, ctypes.c_float(scale),
                                   _ptr(out), ctypes.byref(dims), _stream(stream))
    if st != PA_OK:
        raise PagedKVError("pa_prefill", st)
    return out


def pa_write_kv(k_new, v_new, slot_mapping, k_pool, v_pool, *, stream=None):
    """k_pool/v_pool[slot] = k_new/v_new[t] for every t with slot >= 0."""
    torch = _torch()
    NB, Hkv, D, BS = _pool_dims(k_pool, v_pool)
    T = slot_mapping.shape[0]
    _need(slot_mapping.dtype == torch.int32 and slot_mapping.dim() == 1
          and slot_mapping.is_contiguous() and slot_mapping.is_cuda,
          "slot_mapping must be int32 [T] on the device")
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(tuple(t.shape) == (T, Hkv, D) and t.dtype == k_pool.dtype
              and t.is_contiguous() and t.is_cuda, f"{n} must be [T, Hkv, D] like the pools")
    dims = make_dims(1, Hkv, Hkv, D, 1, NB, _dtype_code(k_pool), block_size=BS)
    st = load_library().pa_write_kv(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), T,
                                    _ptr(k_pool), _ptr(v_pool), ctypes.byref(dims),
                                    _stream(stream))
    if st != PA_OK:
        raise PagedKVError("pa_write_kv", st)


def pa_copy_blocks(k_pool, v_pool, block_mapping, *, stream=None):
    """Whole-block copy dst <- src for every (src, dst) row of block_mapping."""
    torch = _torch()
    NB, Hkv, D, BS = _pool_dims(k_pool, v_pool)
    _need(block_mapping.dtype == torch.int32 and block_mapping.dim() == 2
          and block_mapping.shape[1] == 2 and block_mapping.is_contiguous()
          and block_mapping.is_cuda, "block_mapping must be int32 [n, 2] on the device")
    dims = make_dims(1, Hkv, Hkv, D, 1, NB, _dtype_code(k_pool), block_size=BS)
    st = load_library().pa_copy_blocks(_ptr(k_pool), _ptr(v_pool), _ptr(block_mapping),
                                       block_mapping.shape[0], ctypes.byref(dims),
                                       _stream(stream))
    if st != PA_OK:
        raise PagedKVError("pa_copy_blocks", st)


# --------------------------------------------------------------------------
# latent (MLA-style) decode
# --------------------------------------------------------------------------

def make_latent_dims(num_seqs, max_blocks_per_seq, num_blocks, dtype=PA_BF16,
                     num_heads=LATENT_HEADS, latent_dim=LATENT_DIM,
                     value_dim=LATENT_VALUE_DIM, block_size=LATENT_BLOCK) -> PaLatentDims:
    return PaLatentDims(int(num_seqs), int(num_heads), int(latent_dim), int(value_dim),
                        int(block_size), int(max_blocks_per_seq), int(num_blocks), int(dtype))


def pa_latent_workspace_bytes(dims: PaLatentDims) -> int:
    return int(load_library().pa_latent_workspace_bytes(ctypes.byref(dims)))


def _latent_pool(kv_pool):
    _need(kv_pool.dim() == 3 and kv_pool.is_contiguous() and kv_pool.is_cuda,
          "kv_pool must be a contiguous device tensor [NB, BS, C]")
    return kv_pool.shape


def pa_latent_decode(q, kv_pool, block_tables, seq_lens, scale, out=None, *, workspace=None,
                     stream=None):
    """out[b, h] = softmax(scale * q[b, h] . c_t) weighted sum of c_t[:512]
    over row b's latents c_t (MLA decode with absorbed queries). A
    caller-provided ``workspace`` (uint8 device tensor of at least
    pa_latent_workspace_bytes bytes) must be zero-filled before its first
    use; calls leave it reusable, and two calls that can run at the same
    time need two workspaces."""
    torch = _torch()
    NB, BS, C = _latent_pool(kv_pool)
    _need(q.dim() == 3 and q.shape[2] == C and q.dtype == kv_pool.dtype and q.is_contiguous()
          and q.is_cuda, "q must be [B, H, C] like the pool")
    B, H, _ = q.shape
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == B and block_tables.is_contiguous()
          and block_tables.is_cuda, "block_tables must be int32 [B, MB] on the device")
    _need(seq_lens.dtype == torch.int32 and tuple(seq_lens.shape) == (B,)
          and seq_lens.is_contiguous() and seq_lens.is_cuda,
          "seq_lens must be int32 [B] on the device")
    dims = make_latent_dims(B, block_tables.shape[1], NB, _dtype_code(q), num_heads=H,
                            latent_dim=C, block_size=BS)
    if out is None:
        out = torch.empty((B, H, dims.value_dim), dtype=q.dtype, device=q.device)
    _need(tuple(out.shape) == (B, H, dims.value_dim) and out.dtype == q.dtype
          and out.is_contiguous() and out.is_cuda, "out must be [B, H, 512] like q")
    need = pa_latent_workspace_bytes(dims)
    if workspace is None and need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().pa_latent_decode(_ptr(q), _ptr(kv_pool), _ptr(block_tables),
                                         _ptr(seq_lens), ctypes.c_float(scale), _ptr(out),
                                         ctypes.byref(dims), _ptr(workspace),
                                         ctypes.c_size_t(ws_bytes), _stream(stream))
    if st != PA_OK:
        raise PagedKVError("pa_latent_decode", st)
    return out


def pa_latent_write(kv_new, slot_mapping, kv_pool, *, stream=None):
    """kv_pool row slot = kv_new[t] for every t with slot_mapping[t] >= 0."""
    torch = _torch()
    NB, BS, C = _latent_pool(kv_pool)
    T = slot_mapping.shape[0]
    _need(slot_mapping.dtype == torch.int32 and slot_mapping.dim() == 1
          and slot_mapping.is_contiguous() and slot_mapping.is_cuda,
          "slot_mapping must be int32 [T] on the device")
    _need(tuple(kv_new.shape) == (T, C) and kv_new.dtype == kv_pool.dtype
          and kv_new.is_contiguous() and kv_new.is_cuda, "kv_new must be [T, C] like the pool")
    dims = make_latent_dims(1, 1, NB, _dtype_code(kv_pool), latent_dim=C, block_size=BS)
    st = load_library().pa_latent_write(_ptr(kv_new), _ptr(slot_mapping), T, _ptr(kv_pool),
                                        ctypes.byref(dims), _stream(stream))
    if st != PA_OK:
        raise PagedKVError("pa_latent_write", st)


from .validate import validate  # noqa: E402
