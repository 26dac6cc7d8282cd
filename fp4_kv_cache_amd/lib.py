"""ctypes binding of libfp4kv.so (include/fp4kv.h): argument marshalling only.

The functions below carry the C names and take the same arguments (device
pointers as Python ints, ``stream`` as the integer hipStream_t); they return
the C status code.  ``PagedFP4Cache`` is a convenience holder that allocates
the cache buffers as torch device tensors (torch is used for device memory
and streams only) and raises on a non-zero status.  Every computation runs in
the HIP library; there is no fallback: if the library is missing, loading
fails with an error.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp4kv.so")
# the ablation-study build (same sources with -DFP4KV_ABLATION): the product entry points plus
# fp4kv_ablation_set, whose switches turn techniques of the method off (study only)
LIB_ABLATION_PATH = os.path.join(HERE, "libfp4kv_ablate.so")
ABL_SINGLE_Q, ABL_NO_ROTATION, ABL_NO_SEARCH, ABL_NORMALIZED_P = 1, 2, 4, 8

NVFP4, MXFP4 = 0, 1
F32, BF16 = 0, 1
GQA, MLA = 0, 1
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4

_c_int = ctypes.c_int
_c_size = ctypes.c_size_t
_vp = ctypes.c_void_p


class BF16KVCache(ctypes.Structure):
    """Mirror of ``struct fp4kv_bf16_cache`` (the BF16 comparison cache)."""
    _fields_ = [("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("k", _vp), ("v", _vp)]


class FP4KVCache(ctypes.Structure):
    """Mirror of ``struct fp4kv_cache``."""
    _fields_ = [
        ("format", ctypes.c_int32), ("attn", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32), ("max_seqs", ctypes.c_int32),
        ("k_codes", _vp), ("k_scales", _vp), ("v_codes", _vp), ("v_scales", _vp), ("stage", _vp),
        ("k_rope", _vp), ("k_tensor_scale", _vp), ("v_tensor_scale", _vp), ("k_smooth_inv", _vp),
        ("q_smooth", _vp),
    ]


_SIGS = {
    "fp4kv_cache_layout": (_c_int, [ctypes.POINTER(FP4KVCache), ctypes.POINTER(_c_size)]),
    "kv_quant_append": (_c_int, [ctypes.POINTER(FP4KVCache), _vp, _vp, _c_int, _c_int, _vp, _vp, _vp,
                                 _vp, _vp]),
    "fp4_decode_workspace_bytes": (_c_size, [ctypes.POINTER(FP4KVCache), _c_int, _c_int, _c_int]),
    "fp4_decode_attention": (_c_int, [ctypes.POINTER(FP4KVCache), _vp, _c_int, _c_int, _c_int, _vp,
                                      _c_int, _vp, ctypes.c_float, _vp, _vp, _c_size, _vp, _vp]),
    "fp4_decode_partials": (_c_int, [ctypes.POINTER(FP4KVCache), _vp, _c_int, _c_int, _c_int, _vp,
                                     _c_int, _vp, ctypes.c_float, _vp, _c_size, _vp, _vp]),
    "fp4_decode_merge": (_c_int, [ctypes.POINTER(FP4KVCache), _c_int, _c_int, _c_int, _vp, _vp, _vp,
                                  _c_size, _vp]),
    "fp4kv_cache_read": (_c_int, [ctypes.POINTER(FP4KVCache), _c_int, _c_int, _vp, _c_int, _vp, _vp, _c_size,
                                  _vp]),
    "fp4kv_cache_read_sink_words": (_c_size, [ctypes.POINTER(FP4KVCache), _c_int, _c_int, _c_int]),
    "fp4_decode_attention_noalloc": (_c_int, [ctypes.POINTER(FP4KVCache), _vp, _c_int, _c_int, _c_int, _vp, _c_int,
                                              _vp, ctypes.c_float, _vp, _vp, _vp]),
    "bf16kv_cache_layout": (_c_int, [ctypes.POINTER(BF16KVCache), ctypes.POINTER(_c_size)]),
    "bf16kv_append": (_c_int, [ctypes.POINTER(BF16KVCache), _vp, _vp, _c_int, _c_int, _vp, _vp]),
    "bf16_decode_workspace_bytes": (_c_size, [ctypes.POINTER(BF16KVCache), _c_int, _c_int, _c_int]),
    "bf16_decode_attention": (_c_int, [ctypes.POINTER(BF16KVCache), _vp, _c_int, _c_int, _c_int, _vp, _c_int,
                                       _vp, ctypes.c_float, _vp, _vp, _c_size, _vp]),
    "fp4kv_pack_e2m1": (_c_int, [_vp, _c_size, _c_int, _vp, _vp]),
    "fp4_decode_multi_workspace_bytes": (_c_size, [ctypes.POINTER(FP4KVCache), _c_int, _c_int, _c_int, _c_int]),
    "fp4_decode_attention_multi": (_c_int, [ctypes.POINTER(FP4KVCache), _vp, _c_int, _c_int, _c_int, _c_int, _vp,
                                            _c_int, _vp, ctypes.c_float, _vp, _vp, _c_size, _vp, _vp]),
    "fp4kv_stream_read": (_c_int, [_vp, _c_size, _vp, _vp]),
    "fp4kv_stream_copy": (_c_int, [_vp, _vp, _c_size, _vp]),
    "fp4kv_status_string": (ctypes.c_char_p, [_c_int]),
}

_lib = None


def _open(path):
    if not os.path.exists(path):
        raise RuntimeError("%s not found: build it with `python -m fp4_kv_cache_amd.build`" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def load():
    """Load libfp4kv.so from the package directory (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


_abl = None


def load_ablation():
    """Load the ablation-study build libfp4kv_ablate.so (raises if it has not been built)."""
    global _abl
    if _abl is None:
        lib = _open(LIB_ABLATION_PATH)
        lib.fp4kv_ablation_set.restype = _c_int
        lib.fp4kv_ablation_set.argtypes = [_c_int]
        _abl = lib
    return _abl


class ablation:
    """Context manager: inside the block every entry point of this module runs on the
    ablation-study build with the given technique switches (ABL_* bits, GQA only)."""

    def __init__(self, flags):
        self.flags = flags

    def __enter__(self):
        global _lib
        load()
        self.saved = _lib
        lib = load_ablation()
        check(lib.fp4kv_ablation_set(self.flags), "fp4kv_ablation_set")
        _lib = lib
        return self

    def __exit__(self, *exc):
        global _lib
        _abl.fp4kv_ablation_set(0)
        _lib = self.saved
        return False


def _ref(cache):
    return ctypes.byref(cache) if cache is not None else None


def fp4kv_cache_layout(cache):
    out = (_c_size * 6)()
    st = load().fp4kv_cache_layout(_ref(cache), out)
    return st, list(out)


def kv_quant_append(cache, k_new, v_new, dtype, num_tokens, slot_mapping, seq_ids, positions,
                    k_rope_new, stream):
    return load().kv_quant_append(_ref(cache), k_new, v_new, dtype, num_tokens, slot_mapping, seq_ids,
                                  positions, k_rope_new, stream)


def fp4_decode_workspace_bytes(cache, batch, num_q_heads, max_seq_len):
    return load().fp4_decode_workspace_bytes(_ref(cache), batch, num_q_heads, max_seq_len)


def fp4_decode_attention(cache, q, q_dtype, batch, num_q_heads, block_table, max_pages_per_seq,
                         seq_lens, softmax_scale, out, workspace, workspace_bytes, zero_block_count,
                         stream):
    return load().fp4_decode_attention(_ref(cache), q, q_dtype, batch, num_q_heads, block_table,
                                       max_pages_per_seq, seq_lens, softmax_scale, out, workspace,
                                       workspace_bytes, zero_block_count, stream)


def fp4_decode_partials(cache, q, q_dtype, batch, num_q_heads, block_table, max_pages_per_seq,
                        seq_lens, softmax_scale, workspace, workspace_bytes, zero_block_count, stream):
    return load().fp4_decode_partials(_ref(cache), q, q_dtype, batch, num_q_heads, block_table,
                                      max_pages_per_seq, seq_lens, softmax_scale, workspace,
                                      workspace_bytes, zero_block_count, stream)


def fp4_decode_merge(cache, batch, num_q_heads, max_pages_per_seq, seq_lens, out, workspace,
                     workspace_bytes, stream):
    return load().fp4_decode_merge(_ref(cache), batch, num_q_heads, max_pages_per_seq, seq_lens, out,
                                   workspace, workspace_bytes, stream)


def fp4_decode_attention_noalloc(cache, q, q_dtype, batch, num_q_heads, block_table, max_pages_per_seq,
                                 seq_lens, softmax_scale, out, zero_block_count, stream):
    return load().fp4_decode_attention_noalloc(_ref(cache), q, q_dtype, batch, num_q_heads, block_table,
                                               max_pages_per_seq, seq_lens, softmax_scale, out,
                                               zero_block_count, stream)


def bf16kv_cache_layout(cache):
    out = (_c_size * 2)()
    st = load().bf16kv_cache_layout(_ref(cache), out)
    return st, list(out)


def bf16kv_append(cache, k_new, v_new, dtype, num_tokens, slot_mapping, stream):
    return load().bf16kv_append(_ref(cache), k_new, v_new, dtype, num_tokens, slot_mapping, stream)


def bf16_decode_workspace_bytes(cache, batch, num_q_heads, max_seq_len):
    return load().bf16_decode_workspace_bytes(_ref(cache), batch, num_q_heads, max_seq_len)


def bf16_decode_attention(cache, q, q_dtype, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                          softmax_scale, out, workspace, workspace_bytes, stream):
    return load().bf16_decode_attention(_ref(cache), q, q_dtype, batch, num_q_heads, block_table,
                                        max_pages_per_seq, seq_lens, softmax_scale, out, workspace,
                                        workspace_bytes, stream)


def fp4kv_pack_e2m1(x, n, scale_exp, out, stream):
    return load().fp4kv_pack_e2m1(x, n, scale_exp, out, stream)


def fp4_decode_multi_workspace_bytes(cache, batch, q_len, num_q_heads, max_seq_len):
    return load().fp4_decode_multi_workspace_bytes(_ref(cache), batch, q_len, num_q_heads, max_seq_len)


def fp4_decode_attention_multi(cache, q, q_dtype, batch, q_len, num_q_heads, block_table, max_pages_per_seq,
                               seq_lens, softmax_scale, out, workspace, workspace_bytes, zero_block_count, stream):
    return load().fp4_decode_attention_multi(_ref(cache), q, q_dtype, batch, q_len, num_q_heads, block_table,
                                             max_pages_per_seq, seq_lens, softmax_scale, out, workspace,
                                             workspace_bytes, zero_block_count, stream)


def fp4kv_cache_read(cache, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens, sink, sink_words,
                     stream):
    return load().fp4kv_cache_read(_ref(cache), batch, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                                   sink, sink_words, stream)


def fp4kv_cache_read_sink_words(cache, batch, num_q_heads, max_seq_len):
    return load().fp4kv_cache_read_sink_words(_ref(cache), batch, num_q_heads, max_seq_len)


def fp4kv_stream_read(src, nbytes, sink, stream):
    return load().fp4kv_stream_read(src, nbytes, sink, stream)


def fp4kv_stream_copy(src, dst, nbytes, stream):
    return load().fp4kv_stream_copy(src, dst, nbytes, stream)


def fp4kv_status_string(status):
    return load().fp4kv_status_string(status).decode()


class Fp4KVError(RuntimeError):
    pass


def check(status, what=""):
    if status != OK:
        raise Fp4KVError("%s failed: %s (%d)" % (what, fp4kv_status_string(status), status))


# ----------------------------------------------------------------------------- torch holder

class PagedFP4Cache:
    """Cache buffers allocated as torch device tensors plus the C descriptor.

    Calibration inputs (per KV head): ``k_smooth_inv``/``q_smooth`` [Hkv, d] and the
    NVFP4 tensor scales ``g_k``/``g_v`` [Hkv] (numpy or torch, copied to the device).
    """

    def __init__(self, fmt, attn, num_pages, page_size, num_kv_heads, head_dim, max_seqs,
                 k_smooth_inv, q_smooth, g_k=None, g_v=None, rope_dim=0, device="cuda"):
        import torch
        self.torch = torch
        c = FP4KVCache(fmt, attn, num_pages, page_size, num_kv_heads, head_dim, rope_dim, max_seqs)
        st, sizes = fp4kv_cache_layout(c)
        check(st, "fp4kv_cache_layout")
        self.sizes = sizes
        dev = torch.device(device)
        u8 = lambda n: torch.zeros(max(n, 1), dtype=torch.uint8, device=dev)
        self.k_codes = u8(sizes[0])
        self.k_scales = u8(sizes[1])
        self.v_codes = u8(sizes[2]) if sizes[2] else None
        self.v_scales = u8(sizes[3]) if sizes[3] else None
        self.stage = torch.zeros(max(sizes[4] // 4, 1), dtype=torch.float32, device=dev)
        self.k_rope = torch.zeros(max(sizes[5] // 2, 1), dtype=torch.int16, device=dev) if sizes[5] else None
        f32 = lambda x: torch.as_tensor(x, dtype=torch.float32).reshape(-1).to(dev).contiguous()
        self.k_smooth_inv = f32(k_smooth_inv)
        self.q_smooth = f32(q_smooth)
        self.g_k = f32(g_k) if g_k is not None else None
        self.g_v = f32(g_v) if g_v is not None else None
        p = lambda t: t.data_ptr() if t is not None else None
        c.k_codes, c.k_scales, c.v_codes, c.v_scales = p(self.k_codes), p(self.k_scales), p(self.v_codes), p(self.v_scales)
        c.stage, c.k_rope = p(self.stage), p(self.k_rope)
        c.k_tensor_scale, c.v_tensor_scale = p(self.g_k), p(self.g_v)
        c.k_smooth_inv, c.q_smooth = p(self.k_smooth_inv), p(self.q_smooth)
        self.desc = c
        self.fmt, self.attn, self.page_size = fmt, attn, page_size
        self.num_kv_heads, self.head_dim, self.rope_dim = num_kv_heads, head_dim, rope_dim

    def _stream(self):
        return self.torch.cuda.current_stream().cuda_stream

    def append(self, k_new, v_new, slot_mapping, seq_ids, positions, k_rope_new=None):
        torch = self.torch
        dt = BF16 if k_new.dtype == torch.bfloat16 else F32
        for t in (k_new, v_new, k_rope_new):
            assert t is None or t.is_contiguous()
        n = int(slot_mapping.numel())
        st = kv_quant_append(self.desc, k_new.data_ptr(), v_new.data_ptr() if v_new is not None else None,
                             dt, n, slot_mapping.data_ptr(), seq_ids.data_ptr(), positions.data_ptr(),
                             k_rope_new.data_ptr() if k_rope_new is not None else None, self._stream())
        check(st, "kv_quant_append")

    def workspace_bytes(self, batch, num_q_heads, max_seq_len):
        return fp4_decode_workspace_bytes(self.desc, batch, num_q_heads, max_seq_len)

    def decode(self, q, block_table, seq_lens, softmax_scale, out=None, workspace=None,
               zero_block_count=None):
        torch = self.torch
        batch, hq = q.shape[0], q.shape[1]
        maxp = block_table.shape[1]
        if out is None:
            out = torch.empty((batch, hq, self.head_dim), dtype=torch.float32, device=q.device)
        if workspace is None:
            nb = self.workspace_bytes(batch, hq, maxp * self.page_size)
            workspace = torch.empty(max(nb, 4), dtype=torch.uint8, device=q.device)
        dt = BF16 if q.dtype == torch.bfloat16 else F32
        st = fp4_decode_attention(self.desc, q.data_ptr(), dt, batch, hq, block_table.data_ptr(), maxp,
                                  seq_lens.data_ptr(), float(softmax_scale), out.data_ptr(),
                                  workspace.data_ptr(), workspace.numel(),
                                  zero_block_count.data_ptr() if zero_block_count is not None else None,
                                  self._stream())
        check(st, "fp4_decode_attention")
        return out

    def decode_multi(self, q, block_table, seq_lens, softmax_scale, out=None, workspace=None,
                     zero_block_count=None):
        """q [batch, q_len, hq, d]: the q_len newest tokens of every sequence (already in the
        cache), causal; returns [batch, q_len, hq, d] float32."""
        torch = self.torch
        batch, q_len, hq = q.shape[0], q.shape[1], q.shape[2]
        maxp = block_table.shape[1]
        if out is None:
            out = torch.empty((batch, q_len, hq, self.head_dim), dtype=torch.float32, device=q.device)
        if workspace is None:
            nb = fp4_decode_multi_workspace_bytes(self.desc, batch, q_len, hq, maxp * self.page_size)
            workspace = torch.empty(max(nb, 4), dtype=torch.uint8, device=q.device)
        dt = BF16 if q.dtype == torch.bfloat16 else F32
        st = fp4_decode_attention_multi(self.desc, q.data_ptr(), dt, batch, q_len, hq, block_table.data_ptr(),
                                        maxp, seq_lens.data_ptr(), float(softmax_scale), out.data_ptr(),
                                        workspace.data_ptr(), workspace.numel(),
                                        zero_block_count.data_ptr() if zero_block_count is not None else None,
                                        self._stream())
        check(st, "fp4_decode_attention_multi")
        return out

    def views(self):
        """Cache buffers reshaped to the documented layout (device tensors)."""
        P, h, d = self.page_size, self.num_kv_heads, self.head_dim
        B = 16 if self.fmt == NVFP4 else 32
        np_ = self.desc.num_pages
        v = {"k_codes": self.k_codes.view(np_, h, P, d // 2)}
        if self.attn == GQA:
            v["k_scales"] = self.k_scales.view(np_, h, P * d // B)
            v["v_codes"] = self.v_codes.view(np_, h, d, P // 2)
            v["v_scales"] = self.v_scales.view(np_, h, d * P // B)
        else:
            v["k_scales"] = self.k_scales.view(np_, 1, P // B, d // B)
            v["k_rope"] = self.k_rope.view(np_, 1, P, self.rope_dim)
        return v


class PagedBF16Cache:
    """The BF16 comparison cache: k and v as torch uint16 device tensors in the library's layout."""

    def __init__(self, num_pages, page_size, num_kv_heads, device="cuda"):
        import torch
        self.torch = torch
        c = BF16KVCache(num_pages, page_size, num_kv_heads, 128)
        st, sizes = bf16kv_cache_layout(c)
        check(st, "bf16kv_cache_layout")
        dev = torch.device(device)
        self.k = torch.zeros(sizes[0] // 2, dtype=torch.int16, device=dev)
        self.v = torch.zeros(sizes[1] // 2, dtype=torch.int16, device=dev)
        c.k, c.v = self.k.data_ptr(), self.v.data_ptr()
        self.desc = c
        self.page_size, self.num_kv_heads, self.head_dim = page_size, num_kv_heads, 128

    def append(self, k_new, v_new, slot_mapping):
        torch = self.torch
        dt = BF16 if k_new.dtype == torch.bfloat16 else F32
        assert k_new.is_contiguous() and v_new.is_contiguous()
        st = bf16kv_append(self.desc, k_new.data_ptr(), v_new.data_ptr(), dt, int(slot_mapping.numel()),
                           slot_mapping.data_ptr(), torch.cuda.current_stream().cuda_stream)
        check(st, "bf16kv_append")

    def decode(self, q, block_table, seq_lens, softmax_scale, out=None, workspace=None):
        torch = self.torch
        batch, hq = q.shape[0], q.shape[1]
        maxp = block_table.shape[1]
        if out is None:
            out = torch.empty((batch, hq, 128), dtype=torch.float32, device=q.device)
        if workspace is None:
            nb = bf16_decode_workspace_bytes(self.desc, batch, hq, maxp * self.page_size)
            workspace = torch.empty(max(nb, 4), dtype=torch.uint8, device=q.device)
        dt = BF16 if q.dtype == torch.bfloat16 else F32
        st = bf16_decode_attention(self.desc, q.data_ptr(), dt, batch, hq, block_table.data_ptr(), maxp,
                                   seq_lens.data_ptr(), float(softmax_scale), out.data_ptr(), workspace.data_ptr(),
                                   workspace.numel(), torch.cuda.current_stream().cuda_stream)
        check(st, "bf16_decode_attention")
        return out

    def views(self):
        """k [pages][Hkv][P][128] and v [pages][Hkv][128][P] as uint16 device tensors."""
        P, h = self.page_size, self.num_kv_heads
        np_ = self.desc.num_pages
        return {"k": self.k.view(np_, h, P, 128), "v": self.v.view(np_, h, 128, P)}
