"""ctypes declarations of the C ABI in include/pkv.h (argument marshalling only)."""
import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIB_PATH selects another build of the same library (the host-sanitizer
# build that tests/test_host_sanitizers.py makes); the default is the in-tree one.
LIB_PATH = os.environ.get("PKV_LIB_PATH") or os.path.join(HERE, "libpkv.so")

c_status = C.c_int
vp = C.c_void_p
i32p = C.c_void_p  # device int32 pointers are passed as plain addresses
size_t = C.c_size_t


class CacheDesc(C.Structure):
    _fields_ = [("num_layers", C.c_int32), ("num_blocks", C.c_int32), ("block_size", C.c_int32),
                ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("dtype", C.c_int32)]


class ModelDesc(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("ffn", C.c_int32), ("vocab", C.c_int32),
                ("num_layers", C.c_int32), ("max_positions", C.c_int32),
                ("rms_eps", C.c_float), ("rope_theta", C.c_float)]


class LayerWeights(C.Structure):
    _fields_ = [("w_in", vp), ("w_qkv", vp), ("b_qkv", vp), ("w_o", vp), ("w_post", vp),
                ("w_gate_up", vp), ("w_down", vp)]


# name -> (restype, argtypes); the symbol list mirrors include/pkv.h
SIGNATURES = {
    "pkv_last_error": (C.c_char_p, []),
    "pkv_cache_bytes": (c_status, [C.POINTER(CacheDesc), C.POINTER(size_t)]),
    "pkv_kv_cache_create": (c_status, [C.POINTER(CacheDesc), vp, size_t, C.POINTER(C.c_float),
                                       C.POINTER(C.c_float), C.POINTER(vp)]),
    "pkv_kv_cache_destroy": (None, [vp]),
    "pkv_kv_cache_layer": (c_status, [vp, C.c_int, C.POINTER(vp), C.POINTER(vp)]),
    "pkv_kv_append": (c_status, [vp, C.c_int, vp, vp, i32p, C.c_int, i32p, C.c_int, vp]),
    "pkv_attn_workspace_bytes": (c_status, [vp, C.c_int, C.c_int, C.c_int, C.POINTER(size_t)]),
    "pkv_paged_attn_decode": (c_status, [vp, C.c_int, vp, vp, vp, i32p, C.c_int, i32p, C.c_int,
                                         C.c_int, C.c_int, C.c_float, vp, size_t, vp]),
    "pkv_paged_attn_decode_noalloc": (c_status, [vp, C.c_int, vp, vp, vp, i32p, C.c_int, i32p, C.c_int,
                                                 C.c_int, C.c_int, C.c_float, vp]),
    "pkv_model_create": (c_status, [C.POINTER(ModelDesc), vp, C.POINTER(LayerWeights), vp, vp,
                                    C.POINTER(vp)]),
    "pkv_model_destroy": (None, [vp]),
    "pkv_model_set_option": (c_status, [vp, C.c_int, C.c_int]),
    "pkv_debug_attn_merge_wait": (c_status, [C.c_ulonglong]),
    "pkv_debug_attn_worklist": (c_status, [C.c_int]),
    "pkv_step_workspace_bytes": (c_status, [vp, vp, C.c_int, C.c_int, C.POINTER(size_t)]),
    "pkv_decode_layer": (c_status, [vp, vp, C.c_int, vp, i32p, C.c_int, i32p, C.c_int, C.c_int,
                                    vp, size_t, vp]),
    "pkv_decode_layer_xr": (c_status, [vp, vp, C.c_int, vp, vp, i32p, C.c_int, i32p, C.c_int, C.c_int,
                                       vp, size_t, vp]),
    "pkv_layer_op": (c_status, [vp, vp, C.c_int, C.c_int, vp, i32p, C.c_int, i32p, C.c_int, C.c_int,
                                vp, size_t, vp]),
    "pkv_decode_step": (c_status, [vp, vp, i32p, i32p, C.c_int, i32p, C.c_int, C.c_int, vp, vp,
                                   vp, size_t, vp]),
    "pkv_argmax": (c_status, [vp, C.c_int, C.c_int, i32p, i32p, vp]),
    "pkv_stream_read": (c_status, [vp, size_t, i32p, vp]),
    "pkv_prefill_workspace_bytes": (c_status, [vp, vp, C.c_int, C.c_int, C.c_int, C.POINTER(C.c_size_t)]),
    "pkv_prefill": (c_status, [vp, vp, i32p, i32p, i32p, C.c_int, C.c_int, i32p, C.c_int, C.c_int, vp, vp,
                               C.c_size_t, vp]),
    "pkv_sample": (c_status, [vp, C.c_int, C.c_int, vp, i32p, vp, vp, i32p, i32p, vp]),
    "pkv_sample_penalized": (c_status, [vp, C.c_int, C.c_int, vp, i32p, vp, vp, vp, vp, vp, i32p, i32p, i32p,
                                        vp]),
    "pkv_graph_capture": (c_status, [vp, vp, i32p, i32p, C.c_int, i32p, C.c_int, C.c_int, vp, vp,
                                     vp, size_t, vp, C.POINTER(vp)]),
    "pkv_graph_replay": (c_status, [vp, vp]),
    "pkv_graph_destroy": (None, [vp]),
    "pkv_graph_set_capture": (c_status, [vp, vp, i32p, C.c_int, i32p, i32p, C.c_int, i32p, C.c_int, vp, vp,
                                         vp, size_t, vp, C.POINTER(vp)]),
    "pkv_graph_set_replay": (c_status, [vp, C.c_int, vp, C.POINTER(C.c_int)]),
    "pkv_graph_set_destroy": (None, [vp]),
    "pkv_alloc_create": (c_status, [C.c_int, C.c_uint64, C.POINTER(vp)]),
    "pkv_alloc_grow": (c_status, [vp, C.POINTER(C.c_int32), C.c_int, C.c_int, C.c_int]),
    "pkv_alloc_release": (c_status, [vp, C.POINTER(C.c_int32), C.c_int]),
    "pkv_alloc_free_blocks": (C.c_int, [vp]),
    "pkv_alloc_destroy": (None, [vp]),
    "pkv_validate_metadata": (c_status, [C.POINTER(C.c_int32), C.c_int, C.POINTER(C.c_int32),
                                         C.c_int, C.c_int, C.c_int]),
}

STATUS = {0: "PKV_OK", 1: "PKV_E_ARG", 2: "PKV_E_UNSUPPORTED", 3: "PKV_E_NOMEM",
          4: "PKV_E_CAPACITY", 5: "PKV_E_HIP", 6: "PKV_E_STATE"}


class PkvError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python paged_kv_gqa_05_amd/build.py`")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)  # AttributeError if the library lacks a symbol
        fn.restype = res
        fn.argtypes = args
    return lib
