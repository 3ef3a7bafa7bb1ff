"""ctypes binding of the C ABI in include/tq.h (argument marshalling only).

Every entry point keeps the C name.  Arguments that are device buffers accept
either a torch tensor (its ``data_ptr()`` is passed) or a plain integer
address; ``stream`` accepts a torch stream, an integer hipStream_t, or None
(torch's current stream on the current device).  A negative tq_status raises
``TQError``.  The shared library is loaded from this directory and nowhere
else; if it is missing, loading fails loudly -- there is no fallback.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtq_mi355x.so")

TQ_OK = 0
STATUS = {0: "TQ_OK", -1: "TQ_ERR_INVALID_ARG", -2: "TQ_ERR_UNSUPPORTED", -3: "TQ_ERR_ALIGNMENT",
          -4: "TQ_ERR_WORKSPACE", -5: "TQ_ERR_HIP", -6: "TQ_ERR_NO_DEVICE"}
PRESETS = {"turboquant_k8v4": 0, "turboquant_4bit_nc": 1, "turboquant_k3v4_nc": 2, "turboquant_3bit_nc": 3}
CODEBOOK_MODES = {"exact": 0, "page_trapz": 1, "beta": 2}
LAYOUTS = {"aos": 0, "soa": 1}
DECODE_KERNELS = {"": 0, "auto": 0, "ring": 1, "page": 2, "staged": 3, "direct": 4, "general": 5}


class DecodeOptions(ctypes.Structure):
    """tq_decode_options of include/tq.h."""
    _fields_ = [("kernel", ctypes.c_int), ("dynamic_claims", ctypes.c_int),
                ("ring_waves", ctypes.c_int), ("page_heads", ctypes.c_int)]

# every symbol include/tq.h declares
EXPORTS = ("tq_codebook_init", "tq_codebook_init_layout", "tq_layout_of", "tq_destroy", "tq_slot_bytes", "tq_cache_bytes", "tq_get_tables",
           "tq_store", "tq_decode_workspace_bytes", "tq_decode", "tq_dequant",
           "tq_continuation_workspace_bytes", "tq_decode_continuation", "tq_get_device_error",
           "tq_set_decode_options", "tq_get_decode_options", "tq_decode_noalloc",
           "tq_decode_noalloc_max_bytes",
           "tq_host_codebook", "tq_host_rotation_signs", "tq_host_haar_matrix", "tq_host_slot_bytes",
           "tq_status_str")
# every symbol include/tq_probe.h declares (measurement helpers)
PROBE_EXPORTS = ("tq_probe_sink_words", "tq_probe_read")
PROBE_MODES = {"regs": 0, "regs_nt": 1, "lds": 2, "lds_nt": 3}


class TQError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")


_lib = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_int = ctypes.c_int


def load(path=None):
    """Load the in-tree HIP library (raises OSError if it is not built).
    ``path`` loads another build of it instead (the host-sanitizer build of
    build_lib.build_host_asan); that one becomes the module's library."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise OSError(f"HIP library not built: {path} (run python -m "
                      f"packed_cache_decode_amd.build_lib)")
    lib = ctypes.CDLL(path)
    sig = {
        "tq_codebook_init": (_int, [ctypes.POINTER(_vp), _int, _int, _int, _int, ctypes.c_uint64,
                                    _int, _int, _vp]),
        "tq_codebook_init_layout": (_int, [ctypes.POINTER(_vp), _int, _int, _int, _int,
                                           ctypes.c_uint64, _int, _int, _int, _vp]),
        "tq_layout_of": (_int, [_vp]),
        "tq_destroy": (_int, [_vp]),
        "tq_slot_bytes": (_i64, [_vp]),
        "tq_cache_bytes": (_i64, [_vp, _i64]),
        "tq_get_tables": (_int, [_vp, _vp, _vp, _vp]),
        "tq_store": (_int, [_vp, _vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
        "tq_decode_workspace_bytes": (ctypes.c_size_t, [_vp, _int, _int, _int]),
        "tq_decode": (_int, [_vp, _vp, _vp, _i64, _vp, _int, _vp, _int, _int, _int, ctypes.c_float,
                             _vp, _int, _vp, ctypes.c_size_t, _vp]),
        "tq_decode_noalloc": (_int, [_vp, _vp, _vp, _i64, _vp, _int, _vp, _int, _int, _int,
                                     ctypes.c_float, _vp, _int, _vp]),
        "tq_decode_noalloc_max_bytes": (ctypes.c_size_t, []),
        "tq_dequant": (_int, [_vp, _vp, _i64, _vp, _int, _int, _vp, _vp, _int, _vp]),
        "tq_continuation_workspace_bytes": (ctypes.c_size_t, [_vp, _int, _int, _int, _int]),
        "tq_decode_continuation": (_int, [_vp, _vp, _vp, _i64, _vp, _int, _int, _int, _int, ctypes.c_float,
                                          _vp, _int, _vp, ctypes.c_size_t, _vp]),
        "tq_get_device_error": (_int, [_vp, ctypes.POINTER(_i32), _int, _vp]),
        "tq_set_decode_options": (_int, [_vp, ctypes.POINTER(DecodeOptions)]),
        "tq_get_decode_options": (_int, [_vp, ctypes.POINTER(DecodeOptions)]),
        "tq_host_codebook": (_int, [_int, _int, _int, _vp, _vp]),
        "tq_host_rotation_signs": (_int, [ctypes.c_uint64, _int, _int, _vp]),
        "tq_host_haar_matrix": (_int, [ctypes.c_uint64, _int, _vp]),
        "tq_host_slot_bytes": (_i64, [_int, _int]),
        "tq_status_str": (ctypes.c_char_p, [_int]),
        "tq_probe_sink_words": (_i64, [_i64]),
        "tq_probe_read": (_int, [_int, _vp, _i64, _vp, _vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):            # numpy host array
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(fn, st):
    if st != TQ_OK:
        raise TQError(fn, st)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

ROTATIONS = {"hadamard": 0, "signed_hadamard": 1, "haar": 2}


def _rotation(sign_flip):
    """sign_flip as the C ABI's tq_rotation: True/False, 0/1/2 or a name."""
    if isinstance(sign_flip, str):
        return ROTATIONS[sign_flip]
    return int(sign_flip)


def tq_codebook_init(preset, head_dim, num_kv_heads, block_size, rot_seed, sign_flip=1,
                     codebook_mode=0, stream=None):
    lib = load()
    if isinstance(preset, str):
        preset = PRESETS[preset]
    if isinstance(codebook_mode, str):
        codebook_mode = CODEBOOK_MODES[codebook_mode]
    h = _vp()
    _check("tq_codebook_init", lib.tq_codebook_init(ctypes.byref(h), preset, head_dim, num_kv_heads,
                                                    block_size, rot_seed, _rotation(sign_flip),
                                                    codebook_mode, _stream(stream)))
    return h.value


def tq_codebook_init_layout(preset, head_dim, num_kv_heads, block_size, rot_seed, sign_flip=1,
                            codebook_mode=0, layout=0, stream=None):
    lib = load()
    if isinstance(preset, str):
        preset = PRESETS[preset]
    if isinstance(codebook_mode, str):
        codebook_mode = CODEBOOK_MODES[codebook_mode]
    if isinstance(layout, str):
        layout = LAYOUTS[layout]
    h = _vp()
    _check("tq_codebook_init_layout",
           lib.tq_codebook_init_layout(ctypes.byref(h), preset, head_dim, num_kv_heads, block_size,
                                       rot_seed, _rotation(sign_flip), codebook_mode, layout,
                                       _stream(stream)))
    return h.value


def tq_layout_of(ctx):
    return load().tq_layout_of(ctx)


def tq_destroy(ctx):
    _check("tq_destroy", load().tq_destroy(ctx))


def tq_slot_bytes(ctx):
    return load().tq_slot_bytes(ctx)


def tq_cache_bytes(ctx, num_blocks):
    return load().tq_cache_bytes(ctx, num_blocks)


def tq_get_tables(ctx, centroids=None, midpoints=None, signs=None):
    _check("tq_get_tables", load().tq_get_tables(ctx, _ptr(centroids), _ptr(midpoints), _ptr(signs)))


def tq_store(ctx, k, v, kv_token_stride, slot_mapping, num_tokens, cache, num_blocks, stream=None):
    _check("tq_store", load().tq_store(ctx, _ptr(k), _ptr(v), kv_token_stride, _ptr(slot_mapping),
                                       num_tokens, _ptr(cache), num_blocks, _stream(stream)))


def tq_decode_workspace_bytes(ctx, batch, num_q_heads, max_seq_len):
    return load().tq_decode_workspace_bytes(ctx, batch, num_q_heads, max_seq_len)


def tq_decode(ctx, q, cache, num_blocks, block_table, max_blocks_per_seq, seq_lens, batch,
              num_q_heads, max_seq_len, sm_scale, out, out_is_fp32, workspace, workspace_bytes,
              stream=None):
    _check("tq_decode", load().tq_decode(ctx, _ptr(q), _ptr(cache), num_blocks, _ptr(block_table),
                                         max_blocks_per_seq, _ptr(seq_lens), batch, num_q_heads,
                                         max_seq_len, float(sm_scale), _ptr(out), int(out_is_fp32),
                                         _ptr(workspace), workspace_bytes, _stream(stream)))


def tq_decode_noalloc(ctx, q, cache, num_blocks, block_table, max_blocks_per_seq, seq_lens, batch,
                      num_q_heads, max_seq_len, sm_scale, out, out_is_fp32, stream=None):
    _check("tq_decode_noalloc",
           load().tq_decode_noalloc(ctx, _ptr(q), _ptr(cache), num_blocks, _ptr(block_table),
                                    max_blocks_per_seq, _ptr(seq_lens), batch, num_q_heads,
                                    max_seq_len, float(sm_scale), _ptr(out), int(out_is_fp32),
                                    _stream(stream)))


def tq_decode_noalloc_max_bytes():
    return load().tq_decode_noalloc_max_bytes()


def tq_dequant(ctx, cache, num_blocks, block_table_row, max_blocks, seq_len, k_out, v_out, out_is_fp32,
               stream=None):
    _check("tq_dequant", load().tq_dequant(ctx, _ptr(cache), num_blocks, _ptr(block_table_row), max_blocks,
                                           seq_len, _ptr(k_out), _ptr(v_out), int(out_is_fp32),
                                           _stream(stream)))


def tq_continuation_workspace_bytes(ctx, q_len, num_q_heads, seq_len, max_blocks):
    return load().tq_continuation_workspace_bytes(ctx, q_len, num_q_heads, seq_len, max_blocks)


def tq_decode_continuation(ctx, q, cache, num_blocks, block_table_row, max_blocks, seq_len, q_len,
                           num_q_heads, sm_scale, out, out_is_fp32, workspace, workspace_bytes,
                           stream=None):
    _check("tq_decode_continuation",
           load().tq_decode_continuation(ctx, _ptr(q), _ptr(cache), num_blocks, _ptr(block_table_row),
                                         max_blocks, seq_len, q_len, num_q_heads, float(sm_scale),
                                         _ptr(out), int(out_is_fp32), _ptr(workspace), workspace_bytes,
                                         _stream(stream)))


def tq_get_device_error(ctx, clear=True, stream=None):
    code = _i32(0)
    _check("tq_get_device_error", load().tq_get_device_error(ctx, ctypes.byref(code), int(clear),
                                                             _stream(stream)))
    return code.value


def tq_set_decode_options(ctx, kernel=0, dynamic_claims=0, ring_waves=0, page_heads=0):
    """kernel: a tq_decode_kernel value or one of DECODE_KERNELS' names."""
    if isinstance(kernel, str):
        kernel = DECODE_KERNELS[kernel]
    o = DecodeOptions(int(kernel), int(dynamic_claims), int(ring_waves), int(page_heads))
    _check("tq_set_decode_options", load().tq_set_decode_options(ctx, ctypes.byref(o)))


def tq_get_decode_options(ctx):
    o = DecodeOptions()
    _check("tq_get_decode_options", load().tq_get_decode_options(ctx, ctypes.byref(o)))
    return dict(kernel=o.kernel, dynamic_claims=o.dynamic_claims, ring_waves=o.ring_waves,
                page_heads=o.page_heads)


def tq_host_codebook(head_dim, bits, codebook_mode=0):
    import numpy as np
    if isinstance(codebook_mode, str):
        codebook_mode = CODEBOOK_MODES[codebook_mode]
    c = np.zeros(1 << bits, np.float32)
    m = np.zeros((1 << bits) - 1, np.float32)
    _check("tq_host_codebook", load().tq_host_codebook(head_dim, bits, codebook_mode, c.ctypes.data,
                                                        m.ctypes.data))
    return c, m


def tq_host_rotation_signs(rot_seed, head_dim, sign_flip=1):
    import numpy as np
    s = np.zeros(head_dim, np.int8)
    _check("tq_host_rotation_signs", load().tq_host_rotation_signs(rot_seed, head_dim, int(sign_flip),
                                                                    s.ctypes.data))
    return s


def tq_host_haar_matrix(rot_seed, head_dim):
    import numpy as np
    q = np.zeros((head_dim, head_dim), np.float32)
    _check("tq_host_haar_matrix", load().tq_host_haar_matrix(rot_seed, head_dim, q.ctypes.data))
    return q


def tq_host_slot_bytes(preset, head_dim):
    if isinstance(preset, str):
        preset = PRESETS[preset]
    return load().tq_host_slot_bytes(preset, head_dim)


def tq_status_str(status):
    return load().tq_status_str(status).decode()


def tq_probe_sink_words(nbytes):
    return load().tq_probe_sink_words(nbytes)


def tq_probe_read(mode, src, nbytes, sink, stream=None):
    """One streaming read of ``src`` with a load form of PROBE_MODES."""
    if isinstance(mode, str):
        mode = PROBE_MODES[mode]
    _check("tq_probe_read", load().tq_probe_read(mode, _ptr(src), nbytes, _ptr(sink), _stream(stream)))
