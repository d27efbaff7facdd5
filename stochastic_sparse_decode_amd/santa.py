"""ctypes binding of libsanta (argument marshalling only).

Every function here has the name of a C entry point in include/santa.h and
does nothing but check tensor dtypes/shapes/devices, pass ``data_ptr()``
values, sizes and the current HIP stream, and turn a non-zero status into an
exception.  All computation runs in the library's HIP kernels; there is no
fallback path.  PyTorch is used for device memory and streams only.
"""

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsanta.so")

IID, STRATIFIED, SYSTEMATIC, GUMBEL = 0, 1, 2, 3
MODES = {"iid": IID, "stratified": STRATIFIED, "systematic": SYSTEMATIC, "gumbel": GUMBEL}
MAX_S = 1024
DETERMINISTIC = 1  # santa_problem.flags: bit-reproducible out (exact sum, one rounding)
ERR_SPIN_TIMEOUT = 1


class SantaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s" % (where, status_string(status)))


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_n_k", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
    ]


_lib = None


def library():
    """Load libsanta.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libsanta.so is not built; run `python -m stochastic_sparse_decode_amd.build` "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(Problem)
    vp, i32, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
    lib.santa_workspace_bytes.argtypes = [P, i32]
    lib.santa_workspace_bytes.restype = sz
    lib.santa_decode.argtypes = [P, vp, vp, vp, vp, i32, i32, u64, vp, vp, vp, vp, sz, vp]
    lib.santa_decode.restype = ctypes.c_int
    lib.santa_decode_fp8k.argtypes = [P, vp, vp, vp, vp, vp, i32, i32, u64, vp, vp, vp, vp, sz, vp]
    lib.santa_decode_fp8k.restype = ctypes.c_int
    lib.santa_decode_paged.argtypes = [P, vp, vp, vp, vp, i32, i32, vp, i32, i32, u64, vp, vp, vp, vp, sz, vp]
    lib.santa_decode_paged.restype = ctypes.c_int
    lib.santa_dense_decode.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.santa_dense_decode.restype = ctypes.c_int
    lib.santa_bernoulli_qk.argtypes = [P, vp, vp, vp, vp, i32, i32, u64, vp, vp, vp, vp, vp, sz, vp]
    lib.santa_bernoulli_qk.restype = ctypes.c_int
    lib.santa_bernoulli_qk_budget.argtypes = [P, vp, vp, vp, vp, i32, i32, u64, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.santa_bernoulli_qk_budget.restype = ctypes.c_int
    lib.santa_pack_k_feature_major.argtypes = [P, vp, vp, vp]
    lib.santa_pack_k_feature_major.restype = ctypes.c_int
    lib.santa_decode_noalloc.argtypes = [P, vp, vp, vp, vp, i32, i32, u64, vp, vp, vp, vp, vp]
    lib.santa_decode_noalloc.restype = ctypes.c_int
    lib.santa_stream_read.argtypes = [vp, sz, i32, vp, vp]
    lib.santa_stream_read.restype = ctypes.c_int
    lib.santa_workspace_error.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32), vp]
    lib.santa_workspace_error.restype = ctypes.c_int
    lib.santa_status_string.argtypes = [ctypes.c_int]
    lib.santa_status_string.restype = ctypes.c_char_p
    lib.santa_abi_version.argtypes = []
    lib.santa_abi_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def status_string(status):
    return library().santa_status_string(int(status)).decode()


def _check(status, where):
    if status != 0:
        raise SantaError(status, where)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def problem(q, K, scale, deterministic=False):
    """santa_problem for q (B, H_q, d) and K (B, H_kv, max_n_k, d)."""
    B, Hq, d = q.shape
    return Problem(B, Hq, K.shape[1], d, K.shape[2], float(scale), DETERMINISTIC if deterministic else 0)


def problem_fm(q, K_fm, scale, deterministic=False):
    """santa_problem for q and a feature-major K (B, H_kv, max_n_k/64, d, 64)."""
    B, Hq, d = q.shape
    return Problem(B, Hq, K_fm.shape[1], d, K_fm.shape[2] * K_fm.shape[4], float(scale),
                   DETERMINISTIC if deterministic else 0)


def workspace_bytes(prob, S=MAX_S):
    """santa_workspace_bytes for calls with sample counts up to S."""
    return int(library().santa_workspace_bytes(ctypes.byref(prob), int(S)))


def new_workspace(prob, device, S=MAX_S):
    """Zero-filled workspace tensor of santa_workspace_bytes(prob, S) bytes."""
    n = workspace_bytes(prob, S)
    if n == 0:
        raise SantaError(2, "santa_workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _expect(t, name, dtype, device, ndim=None):
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))


def _shape(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _check_q(q):
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a (B, H_q, d) tensor, got %s" % (tuple(q.shape) if hasattr(q, "shape") else q,))


def _on_gpu(q):
    if q.device.type != "cuda":
        raise ValueError("the decode step runs on a GPU: q is on %s" % q.device)


def _check_step(q, kv, kv_names, n_k, out, indices, scores, S, max_n_k, extra=()):
    """Dtype, shape, contiguity and device of every tensor of a decode step,
    against the problem that q (B, H_q, d) and the key cache define; raises
    before the library is called (the library cannot check device buffer
    sizes).  kv: the key and value caches, already shape-checked by the
    caller; extra: further (tensor, name, dtype, shape) entries."""
    if q.dim() != 3:
        raise ValueError("q must be (B, H_q, d), got shape %s" % (tuple(q.shape),))
    B, Hq, d = q.shape
    dev = q.device
    _expect(q, "q", torch.float16, dev)
    for t, nm in zip(kv, kv_names):
        _expect(t, nm, t.dtype, dev)
    _expect(n_k, "n_k", torch.int32, dev, 1)
    _shape(n_k, "n_k", (B,))
    if out is not None:
        _expect(out, "out", torch.float32, dev)
        _shape(out, "out", (B, Hq, d))
    if indices is not None:
        _expect(indices, "indices", torch.int32, dev)
        _shape(indices, "indices", (B, Hq, int(S)))
    if scores is not None:
        _expect(scores, "scores", torch.float32, dev)
        _shape(scores, "scores", (B, Hq, max_n_k))
    for t, nm, dt, shp in extra:
        _expect(t, nm, dt, dev)
        _shape(t, nm, shp)
    _on_gpu(q)


def _check_workspace(workspace, prob, dev, S=1):
    need = workspace_bytes(prob, S)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 vector (see new_workspace)")
    if workspace.device != dev:
        raise ValueError("workspace must be on %s" % dev)
    if workspace.numel() < need:
        raise ValueError("workspace holds %d bytes, the problem needs %d" % (workspace.numel(), need))


def _kv_pair(q, K, V, dtype_k=torch.float16, name_k="K"):
    """K (B, H_kv, max_n_k, d) and V of the same shape, H_q a multiple of H_kv."""
    B, Hq, d = q.shape
    if K.dim() != 4 or K.shape[0] != B or K.shape[3] != d or Hq % max(K.shape[1], 1) != 0:
        raise ValueError("%s must be (B=%d, H_kv, max_n_k, d=%d) with H_q=%d a multiple of H_kv, got %s"
                         % (name_k, B, d, Hq, tuple(K.shape)))
    if K.dtype != dtype_k:
        raise TypeError("%s must be %s, got %s" % (name_k, dtype_k, K.dtype))
    _expect(V, "V", torch.float16, q.device, 4)
    _shape(V, "V", K.shape)


def santa_decode(q, K, V, n_k, S, mode, seed, scale, out=None, indices=None, scores=None,
                 workspace=None, stream=None, deterministic=False):
    """SANTA decode step; returns ``out`` (B, H_q, d) fp32.

    q (B, H_q, d), K and V (B, H_kv, max_n_k, d): contiguous fp16 on one GPU;
    n_k (B,) int32 on the same GPU.  ``indices`` (B, H_q, S) int32 and
    ``scores`` (B, H_q, max_n_k) fp32, if given, receive the sampled indices
    and the scores.  ``workspace``: from ``new_workspace`` (allocated here if
    None).  ``deterministic``: the SANTA_DETERMINISTIC flag (bit-reproducible
    ``out``).
    """
    _check_q(q)
    _kv_pair(q, K, V)
    _check_step(q, (K, V), ("K", "V"), n_k, out, indices, scores, S, K.shape[2])
    dev = q.device
    prob = problem(q, K, scale, deterministic)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = new_workspace(prob, dev, S)
    _check_workspace(workspace, prob, dev, S)
    mode = MODES.get(mode, mode)
    st = library().santa_decode(ctypes.byref(prob), _ptr(q), _ptr(K), _ptr(V), _ptr(n_k), int(S), int(mode),
                                int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(out), _ptr(indices), _ptr(scores),
                                _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "santa_decode")
    return out


def santa_decode_noalloc(q, K, V, n_k, S, mode, seed, scale, out=None, indices=None, scores=None,
                         error_flags=None, stream=None, deterministic=False):
    """santa_decode with the library's own workspace (no allocation by the
    library; ``out`` is allocated here only if not given).  ``error_flags``:
    an optional int32 tensor of one element on the GPU that receives the
    device error bits (OR-ed in)."""
    _check_q(q)
    _kv_pair(q, K, V)
    extra = ((error_flags, "error_flags", torch.int32, (1,)),) if error_flags is not None else ()
    _check_step(q, (K, V), ("K", "V"), n_k, out, indices, scores, S, K.shape[2], extra=extra)
    prob = problem(q, K, scale, deterministic)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    mode = MODES.get(mode, mode)
    st = library().santa_decode_noalloc(ctypes.byref(prob), _ptr(q), _ptr(K), _ptr(V), _ptr(n_k), int(S), int(mode),
                                        int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(out), _ptr(indices), _ptr(scores),
                                        _ptr(error_flags), _stream(stream))
    _check(st, "santa_decode_noalloc")
    return out


def santa_decode_fp8k(q, K8, k_scale, V, n_k, S, mode, seed, scale, out=None, indices=None, scores=None,
                      workspace=None, stream=None, deterministic=False):
    """SANTA decode step on an fp8 key cache; returns ``out`` (B, H_q, d) fp32.

    K8 (B, H_kv, max_n_k, d) uint8 holds OCP E4M3 bytes and k_scale (B, H_kv)
    fp32 their scales (K = k_scale * decoded K8); q, V, n_k and the optional
    outputs are as for ``santa_decode``.
    """
    _check_q(q)
    _kv_pair(q, K8, V, torch.uint8, "K8")
    B, Hq, d = q.shape
    _check_step(q, (K8, V), ("K8", "V"), n_k, out, indices, scores, S, K8.shape[2],
                extra=((k_scale, "k_scale", torch.float32, K8.shape[:2]),))
    dev = q.device
    prob = problem(q, K8, scale, deterministic)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = new_workspace(prob, dev, S)
    _check_workspace(workspace, prob, dev, S)
    mode = MODES.get(mode, mode)
    st = library().santa_decode_fp8k(ctypes.byref(prob), _ptr(q), _ptr(K8), _ptr(k_scale), _ptr(V), _ptr(n_k),
                                     int(S), int(mode), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(out), _ptr(indices),
                                     _ptr(scores), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "santa_decode_fp8k")
    return out


def problem_paged(q, K_cache, block_table, scale, deterministic=False):
    """santa_problem for q and a paged cache (num_blocks, H_kv, P, d) with a
    block table (B, max_blocks): max_n_k = max_blocks * P."""
    B, Hq, d = q.shape
    return Problem(B, Hq, K_cache.shape[1], d, block_table.shape[1] * K_cache.shape[2], float(scale),
                   DETERMINISTIC if deterministic else 0)


def santa_decode_paged(q, K_cache, V_cache, block_table, n_k, S, mode, seed, scale, out=None, indices=None,
                       scores=None, workspace=None, stream=None, deterministic=False):
    """SANTA decode step on a paged KV cache; returns ``out`` (B, H_q, d) fp32.

    K_cache, V_cache (num_blocks, H_kv, block_size, d) fp16; block_table
    (B, max_blocks) int32: key j of sequence b is row j % block_size of block
    block_table[b, j // block_size].  The rest is as for ``santa_decode``.
    """
    _check_q(q)
    B, Hq, d = q.shape
    if K_cache.dim() != 4 or K_cache.shape[3] != d or Hq % max(K_cache.shape[1], 1) != 0:
        raise ValueError("K_cache must be (num_blocks, H_kv, block_size, d=%d), got %s" % (d, tuple(K_cache.shape)))
    if K_cache.dtype != torch.float16:
        raise TypeError("K_cache must be torch.float16, got %s" % K_cache.dtype)
    _expect(V_cache, "V_cache", torch.float16, q.device, 4)
    _shape(V_cache, "V_cache", K_cache.shape)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be (B=%d, max_blocks), got %s" % (B, tuple(block_table.shape)))
    _check_step(q, (K_cache, V_cache), ("K_cache", "V_cache"), n_k, out, indices, scores, S,
                block_table.shape[1] * K_cache.shape[2],
                extra=((block_table, "block_table", torch.int32, block_table.shape),))
    dev = q.device
    prob = problem_paged(q, K_cache, block_table, scale, deterministic)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = new_workspace(prob, dev, S)
    _check_workspace(workspace, prob, dev, S)
    mode = MODES.get(mode, mode)
    st = library().santa_decode_paged(ctypes.byref(prob), _ptr(q), _ptr(K_cache), _ptr(V_cache), _ptr(block_table),
                                      int(K_cache.shape[2]), int(K_cache.shape[0]), _ptr(n_k), int(S), int(mode),
                                      int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(out), _ptr(indices), _ptr(scores),
                                      _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "santa_decode_paged")
    return out


def santa_dense_decode(q, K, V, n_k, scale, out=None, workspace=None, stream=None):
    """Exact split-K decode attention; returns ``out`` (B, H_q, d) fp32."""
    _check_q(q)
    _kv_pair(q, K, V)
    _check_step(q, (K, V), ("K", "V"), n_k, out, None, None, 1, K.shape[2])
    dev = q.device
    prob = problem(q, K, scale)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = new_workspace(prob, dev)
    _check_workspace(workspace, prob, dev)
    st = library().santa_dense_decode(ctypes.byref(prob), _ptr(q), _ptr(K), _ptr(V), _ptr(n_k), _ptr(out),
                                      _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "santa_dense_decode")
    return out


def santa_pack_k_feature_major(K, K_fm=None, stream=None):
    """Feature-major copy of K: (B, H_kv, max_n_k/64, d, 64) fp16."""
    _expect(K, "K", torch.float16, K.device, 4)
    B, Hkv, n, d = K.shape
    if K.device.type != "cuda":
        raise ValueError("K must be on a GPU, got %s" % K.device)
    if n % 64 != 0:
        raise ValueError("max_n_k (%d) must be a multiple of 64 for the feature-major layout" % n)
    if K_fm is None:
        K_fm = torch.empty((B, Hkv, n // 64, d, 64), dtype=torch.float16, device=K.device)
    _expect(K_fm, "K_fm", torch.float16, K.device)
    _shape(K_fm, "K_fm", (B, Hkv, n // 64, d, 64))
    prob = Problem(B, Hkv, Hkv, d, n, 1.0, 0)
    st = library().santa_pack_k_feature_major(ctypes.byref(prob), _ptr(K), _ptr(K_fm), _stream(stream))
    _check(st, "santa_pack_k_feature_major")
    return K_fm


def santa_bernoulli_qk(q, K_fm, V, n_k, S, mode, seed, scale, out=None, indices=None, scores=None,
                       kept=None, workspace=None, stream=None, budget=0, deterministic=False):
    """Bernoulli qK^T step + SANTA value stage; returns ``out`` (B, H_q, d) fp32.

    budget = 0: ternary queries (keep probability |q_i| / max|q|); budget = m
    in [1, d]: the budget variant (keep probability min(1, m |q_i| / ||q||_1)).
    """
    _check_q(q)
    B, Hq, d = q.shape
    if (K_fm.dim() != 5 or K_fm.shape[0] != B or K_fm.shape[3] != d or K_fm.shape[4] != 64
            or Hq % max(K_fm.shape[1], 1) != 0):
        raise ValueError("K_fm must be (B=%d, H_kv, max_n_k/64, d=%d, 64), got %s" % (B, d, tuple(K_fm.shape)))
    if K_fm.dtype != torch.float16:
        raise TypeError("K_fm must be torch.float16, got %s" % K_fm.dtype)
    max_n_k = K_fm.shape[2] * 64
    _expect(V, "V", torch.float16, q.device, 4)
    _shape(V, "V", (B, K_fm.shape[1], max_n_k, d))
    extra = ((kept, "kept", torch.uint8, (B, Hq, d)),) if kept is not None else ()
    _check_step(q, (K_fm, V), ("K_fm", "V"), n_k, out, indices, scores, S, max_n_k, extra=extra)
    dev = q.device
    prob = problem_fm(q, K_fm, scale, deterministic)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = new_workspace(prob, dev, S)
    _check_workspace(workspace, prob, dev, S)
    mode = MODES.get(mode, mode)
    if budget:
        st = library().santa_bernoulli_qk_budget(ctypes.byref(prob), _ptr(q), _ptr(K_fm), _ptr(V), _ptr(n_k),
                                                 int(S), int(mode), int(seed) & 0xFFFFFFFFFFFFFFFF, int(budget),
                                                 _ptr(out), _ptr(indices), _ptr(scores), _ptr(kept),
                                                 _ptr(workspace), workspace.numel(), _stream(stream))
        _check(st, "santa_bernoulli_qk_budget")
    else:
        st = library().santa_bernoulli_qk(ctypes.byref(prob), _ptr(q), _ptr(K_fm), _ptr(V), _ptr(n_k), int(S),
                                          int(mode), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(out), _ptr(indices),
                                          _ptr(scores), _ptr(kept), _ptr(workspace), workspace.numel(),
                                          _stream(stream))
        _check(st, "santa_bernoulli_qk")
    return out


def santa_stream_read(buf, workgroups_per_cu=2, sink=None, stream=None):
    """Read every byte of the contiguous device tensor ``buf`` once (the
    bare-read bandwidth ceiling; writes nothing but, practically never, sink)."""
    if not buf.is_contiguous() or buf.device.type != "cuda":
        raise ValueError("buf must be a contiguous GPU tensor")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check(library().santa_stream_read(_ptr(buf), nbytes, int(workgroups_per_cu), _ptr(sink), _stream(stream)),
           "santa_stream_read")
    return sink


def santa_workspace_error(workspace, stream=None):
    """Device error bits of a workspace (synchronises the stream)."""
    flags = ctypes.c_uint32(0)
    _check(library().santa_workspace_error(_ptr(workspace), ctypes.byref(flags), _stream(stream)),
           "santa_workspace_error")
    return flags.value


def santa_abi_version():
    return int(library().santa_abi_version())
