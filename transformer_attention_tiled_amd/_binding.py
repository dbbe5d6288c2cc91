"""ctypes binding of libattn.so (the C ABI declared in include/attn.h).

Argument marshalling only: tensors become raw device pointers, the current
HIP stream is passed through, and a non-zero status becomes ``AttnError``.
No computation happens here, and there is no fallback of any kind: if the
library cannot be loaded, every entry point raises.
"""

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libattn.so"
_lib = None

ATTN_F32 = 0
ATTN_BF16 = 1

_STATUS_NAMES = {
    0: "ATTN_OK",
    -1: "ATTN_ERR_NULL",
    -2: "ATTN_ERR_SHAPE",
    -3: "ATTN_ERR_UNSUPPORTED",
    -4: "ATTN_ERR_ALIGN",
    -5: "ATTN_ERR_WORKSPACE",
    -6: "ATTN_ERR_LAUNCH",
    -7: "ATTN_ERR_SCRATCH",
}

# bytes of the fixed device array behind decode_paged_noalloc (include/attn.h)
DECODE_NOALLOC_SCRATCH_BYTES = 64 << 20


class AttnError(RuntimeError):
    """A libattn call returned a negative status."""

    def __init__(self, status, where):
        self.status = status
        self.name = _STATUS_NAMES.get(status, str(status))
        try:
            text = status_string(status)
        except Exception:  # library not loadable: keep the code only
            text = ""
        super().__init__(f"{where}: {self.name} ({status}) {text}")


def library_path():
    return os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load libattn.so (once). Raises if it is missing or broken."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    c_int, c_float, c_size_t, c_void_p = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
    lib.attn_prefill.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_int, c_int, c_int, c_int, c_int, c_float, c_int,
                                 c_int, c_void_p, c_void_p]
    lib.attn_prefill.restype = c_int
    lib.attn_decode_paged_partition_size.argtypes = [c_int, c_int, c_int]
    lib.attn_decode_paged_partition_size.restype = c_int
    lib.attn_decode_paged_workspace_size.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int]
    lib.attn_decode_paged_workspace_size.restype = c_size_t
    lib.attn_paged_workspace_size.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                              c_int]
    lib.attn_paged_workspace_size.restype = c_size_t
    lib.attn_decode_paged.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p,
                                      c_int, c_int, c_int, c_int, c_int,
                                      c_int, c_int, c_int, c_int, ctypes.c_int64, c_float,
                                      c_int, c_int, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.attn_decode_paged.restype = c_int
    lib.attn_decode_paged_noalloc.argtypes = lib.attn_decode_paged.argtypes[:-3] + [c_void_p]
    lib.attn_decode_paged_noalloc.restype = c_int
    lib.attn_kv_append.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                   ctypes.c_int64, c_int, c_void_p]
    lib.attn_kv_append.restype = c_int
    lib.attn_add_rmsnorm.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                     c_int, c_float, c_int, c_void_p]
    lib.attn_add_rmsnorm.restype = c_int
    lib.attn_status_string.argtypes = [c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status):
    return load_library().attn_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return ATTN_BF16
    if dt == torch.float32:
        return ATTN_F32
    return -1  # the library rejects it with ATTN_ERR_UNSUPPORTED


def _check(status, where):
    if status != 0:
        raise AttnError(status, where)


class _Args:
    """Checks of the tensors handed to one entry point, made before any
    library or device call: the C ABI sees raw pointers only, so a tensor on
    the wrong device, of the wrong element type, not contiguous, or of a
    shape the other arguments contradict would reach the kernels unnoticed
    (an index tensor of the wrong width would even be read silently). Every
    failure raises ValueError and nothing is launched."""

    def __init__(self, where):
        self.where = where
        self.device = None
        self.pending = []  # tensors whose device is checked last

    def fail(self, msg):
        raise ValueError(f"{self.where}: {msg}")

    def tensor(self, name, t, *, dtype=None, shape=None, ndim=None, optional=False):
        if t is None:
            if not optional:
                self.fail(f"{name} is required")
            return None
        if not torch.is_tensor(t):
            self.fail(f"{name} must be a torch.Tensor")
        if ndim is not None and t.dim() != ndim:
            self.fail(f"{name} must have {ndim} dimensions, has shape {tuple(t.shape)}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            self.fail(f"{name} must have shape {tuple(shape)}, has {tuple(t.shape)}")
        if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
            self.fail(f"{name} must be {dtype}, is {t.dtype}")
        if not t.is_contiguous():
            self.fail(f"{name} must be contiguous")
        self.pending.append((name, t))
        return t

    def devices(self):
        """All tensors on one GPU (the first one's); call after the shape checks."""
        for name, t in self.pending:
            if t.device.type != "cuda":
                self.fail(f"{name} must be on a GPU, is on {t.device}")
            if self.device is None:
                self.device = t.device
            elif t.device != self.device:
                self.fail(f"{name} is on {t.device}, the others on {self.device}")
        return self.device


def prefill(q, k, v, o=None, *, scale=None, causal=True, lse=None):
    """attn_prefill on contiguous tensors q [B,Hq,T,d], k/v [B,Hkv,T,d].

    Returns o (allocated like q when not given). ``lse`` (fp32 [B,Hq,T]) is
    filled when given.
    """
    A = _Args("prefill")
    A.tensor("q", q, ndim=4)
    B, Hq, T, d = q.shape
    A.tensor("k", k, ndim=4, dtype=q.dtype)
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, T, d):
        A.fail(f"k must have shape [B={B}, Hkv, T={T}, d={d}], has {tuple(k.shape)}")
    A.tensor("v", v, dtype=q.dtype, shape=k.shape)
    A.tensor("o", o, dtype=q.dtype, shape=q.shape, optional=True)
    A.tensor("lse", lse, dtype=torch.float32, shape=(B, Hq, T), optional=True)
    dev = A.devices()
    lib = load_library()
    if o is None:
        o = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    status = lib.attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, Hq, Hkv, T, d,
                              float(scale), int(bool(causal)), _dtype_code(q.dtype), _ptr(lse),
                              _stream(dev))
    _check(status, "attn_prefill")
    return o


def decode_paged_partition_size(num_seqs, Hkv, max_seq_len):
    return int(load_library().attn_decode_paged_partition_size(num_seqs, Hkv, max_seq_len))


def decode_paged_workspace_size(num_seqs, Hq, Hkv, d, max_seq_len, partition_size=0):
    return int(load_library().attn_decode_paged_workspace_size(num_seqs, Hq, Hkv, d, max_seq_len,
                                                               partition_size))


def paged_workspace_size(num_seqs, num_tokens, Hq, Hkv, d, max_seq_len, max_query_len=1,
                         partition_size=0):
    """attn_paged_workspace_size: workspace bytes for a batch that may hold
    chunk rows (several query tokens per sequence)."""
    return int(load_library().attn_paged_workspace_size(num_seqs, num_tokens, Hq, Hkv, d,
                                                        max_seq_len, max_query_len,
                                                        partition_size))


def _paged_common(A, q, k_cache, v_cache, block_table, seq_lens, query_start_loc):
    A.tensor("q", q, ndim=3)
    num_tokens, Hq, d = q.shape
    A.tensor("k_cache", k_cache, ndim=4, dtype=q.dtype)
    num_blocks, Hkv, block_size, dk = k_cache.shape
    if dk != d:
        A.fail(f"k_cache head size {dk} differs from q's {d}")
    A.tensor("v_cache", v_cache, dtype=q.dtype, shape=k_cache.shape)
    A.tensor("seq_lens", seq_lens, ndim=1, dtype=torch.int32)
    num_seqs = seq_lens.shape[0]
    A.tensor("block_table", block_table, ndim=2, dtype=torch.int32)
    if block_table.shape[0] != num_seqs:
        A.fail(f"block_table has {block_table.shape[0]} rows for {num_seqs} sequences")
    A.tensor("query_start_loc", query_start_loc, dtype=torch.int32, shape=(num_seqs + 1,),
             optional=True)
    return num_tokens, Hq, d, num_blocks, Hkv, block_size, num_seqs


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, *, max_seq_len, max_query_len=1,
                 query_start_loc=None, o=None, scale=None, partition_size=0, lse=None,
                 workspace=None):
    """attn_decode_paged. q [num_tokens,Hq,d]; caches [num_blocks,Hkv,16,d];
    block_table int32 [num_seqs, max_blocks_per_seq]; seq_lens int32
    [num_seqs]; query_start_loc int32 [num_seqs+1] or None.

    ``max_seq_len`` / ``max_query_len`` are host-side bounds the caller knows
    (nothing is read back from the device). A workspace is allocated when not
    given. Returns o.
    """
    A = _Args("decode_paged")
    num_tokens, Hq, d, num_blocks, Hkv, block_size, num_seqs = _paged_common(
        A, q, k_cache, v_cache, block_table, seq_lens, query_start_loc)
    A.tensor("o", o, dtype=q.dtype, shape=q.shape, optional=True)
    A.tensor("lse", lse, dtype=torch.float32, shape=(num_tokens, Hq), optional=True)
    A.tensor("workspace", workspace, optional=True)
    dev = A.devices()
    lib = load_library()
    if o is None:
        o = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_bytes = paged_workspace_size(num_seqs, num_tokens, Hq, Hkv, d, max_seq_len,
                                    max_query_len, partition_size)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    status = lib.attn_decode_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
        _ptr(query_start_loc), _ptr(o), num_seqs, num_tokens, Hq, Hkv, d, block_size,
        block_table.shape[1], int(max_seq_len), int(max_query_len), num_blocks, float(scale),
        _dtype_code(q.dtype), int(partition_size), _ptr(lse), _ptr(workspace), ws_have,
        _stream(dev))
    _check(status, "attn_decode_paged")
    return o


def decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens, o, *, max_seq_len,
                         max_query_len=1, query_start_loc=None, scale=None, partition_size=0,
                         lse=None):
    """attn_decode_paged_noalloc: decode_paged with no allocation at all, for
    callers that cannot allocate (graph capture, tight serving loops). The
    caller passes the output ``o``; the split-KV partials go to the library's
    fixed per-GPU array of DECODE_NOALLOC_SCRATCH_BYTES. Calls that overlap in
    time on one GPU race (they share that array). Returns o."""
    A = _Args("decode_paged_noalloc")
    num_tokens, Hq, d, num_blocks, Hkv, block_size, num_seqs = _paged_common(
        A, q, k_cache, v_cache, block_table, seq_lens, query_start_loc)
    A.tensor("o", o, dtype=q.dtype, shape=q.shape)
    A.tensor("lse", lse, dtype=torch.float32, shape=(num_tokens, Hq), optional=True)
    dev = A.devices()
    lib = load_library()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    status = lib.attn_decode_paged_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
        _ptr(query_start_loc), _ptr(o), num_seqs, num_tokens, Hq, Hkv, d, block_size,
        block_table.shape[1], int(max_seq_len), int(max_query_len), num_blocks, float(scale),
        _dtype_code(q.dtype), int(partition_size), _ptr(lse), _stream(dev))
    _check(status, "attn_decode_paged_noalloc")
    return o


def kv_append(k_new, v_new, k_cache, v_cache, block_table, seq_lens, *, max_query_len=1,
              query_start_loc=None):
    """attn_kv_append: write k_new / v_new [num_tokens,Hkv,d] into the paged
    caches [num_blocks,Hkv,16,d] in place, at the positions block_table /
    seq_lens / query_start_loc give (the convention of decode_paged).
    ``max_query_len`` is a host-side bound on the new rows per sequence."""
    A = _Args("kv_append")
    A.tensor("k_new", k_new, ndim=3)
    num_tokens, Hkv, d = k_new.shape
    A.tensor("v_new", v_new, dtype=k_new.dtype, shape=k_new.shape)
    A.tensor("k_cache", k_cache, ndim=4, dtype=k_new.dtype)
    num_blocks, hc, block_size, dc = k_cache.shape
    if (hc, dc) != (Hkv, d):
        A.fail(f"k_cache has Hkv={hc}, d={dc}; the new rows Hkv={Hkv}, d={d}")
    A.tensor("v_cache", v_cache, dtype=k_new.dtype, shape=k_cache.shape)
    A.tensor("seq_lens", seq_lens, ndim=1, dtype=torch.int32)
    num_seqs = seq_lens.shape[0]
    A.tensor("block_table", block_table, ndim=2, dtype=torch.int32)
    if block_table.shape[0] != num_seqs:
        A.fail(f"block_table has {block_table.shape[0]} rows for {num_seqs} sequences")
    A.tensor("query_start_loc", query_start_loc, dtype=torch.int32, shape=(num_seqs + 1,),
             optional=True)
    dev = A.devices()
    lib = load_library()
    status = lib.attn_kv_append(
        _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(seq_lens), _ptr(query_start_loc), num_seqs, num_tokens, Hkv, d, block_size,
        block_table.shape[1], int(max_query_len), num_blocks, _dtype_code(k_new.dtype),
        _stream(dev))
    _check(status, "attn_kv_append")


def add_rmsnorm(x, residual, weight, eps, *, out=None, residual_out=None):
    """attn_add_rmsnorm on [rows, hidden] tensors: returns (out, residual_out),
    out = RMSNorm(x + residual) * weight and residual_out = x + residual.
    Pass residual_out=residual to update the residual stream in place."""
    A = _Args("add_rmsnorm")
    A.tensor("x", x)
    if x.dim() < 1:
        A.fail("x must have at least one dimension")
    hidden = x.shape[-1]
    rows = x.numel() // hidden if hidden else 0
    A.tensor("residual", residual, dtype=x.dtype, shape=x.shape)
    A.tensor("weight", weight, dtype=x.dtype, shape=(hidden,))
    A.tensor("out", out, dtype=x.dtype, shape=x.shape, optional=True)
    A.tensor("residual_out", residual_out, dtype=x.dtype, shape=x.shape, optional=True)
    dev = A.devices()
    lib = load_library()
    if out is None:
        out = torch.empty_like(x)
    if residual_out is None:
        residual_out = torch.empty_like(x)
    status = lib.attn_add_rmsnorm(_ptr(x), _ptr(residual), _ptr(weight), _ptr(out),
                                  _ptr(residual_out), rows, hidden, float(eps),
                                  _dtype_code(x.dtype), _stream(dev))
    _check(status, "attn_add_rmsnorm")
    return out, residual_out
