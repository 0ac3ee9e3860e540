"""ctypes view of the C ABI in include/bdlm_attn.h (argument marshalling only).

Loading fails loudly when libbdlm_attn.so has not been built: there is no
fallback implementation anywhere in this package.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbdlm_attn.so")

BDLM_OK = 0
BDLM_ERR_INVALID_ARG = 1
BDLM_ERR_UNSUPPORTED = 2
BDLM_ERR_WORKSPACE = 3
BDLM_ERR_HIP = 4
BDLM_F32 = 0
BDLM_BF16 = 1
BDLM_MAX_LOCAL_BLOCKS = 256
BDLM_MAX_MERGE_PARTS = 64

EXPORTED = (
    "bdlm_attn_workspace_bytes", "bdlm_attn_check_desc", "bdlm_attn_fwd", "bdlm_attn_bwd",
    "bdlm_attn_merge_partials", "bdlm_attn_schedule_walk", "bdlm_status_str",
    "bdlm_attn_version", "bdlm_attn_profile_begin", "bdlm_attn_profile_end",
    "bdlm_attn_bwd_noalloc", "bdlm_attn_noalloc_scratch_bytes", "bdlm_calib_mfma",
)


class BdlmDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("block", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("num_local_blocks", ctypes.c_int32), ("block_ids", ctypes.POINTER(ctypes.c_int32)),
        ("kv_begin", ctypes.c_int32), ("kv_end", ctypes.c_int32), ("own_block", ctypes.c_int32),
        ("clean_queries", ctypes.c_int32), ("accumulate", ctypes.c_int32),
        ("kv_staged", ctypes.c_int32),
    ]


class BdlmKernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


class BdlmError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libbdlm_attn.so (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m masked_attention_bdlm_amd.build` "
                           "(hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    dp = ctypes.POINTER(BdlmDesc)
    lib.bdlm_attn_workspace_bytes.argtypes = [dp, ctypes.c_int]
    lib.bdlm_attn_workspace_bytes.restype = sz
    lib.bdlm_attn_check_desc.argtypes = [dp]
    lib.bdlm_attn_check_desc.restype = ctypes.c_int
    lib.bdlm_attn_fwd.argtypes = [dp] + [vp] * 10 + [vp, sz, vp]
    lib.bdlm_attn_fwd.restype = ctypes.c_int
    lib.bdlm_attn_bwd.argtypes = [dp] + [vp] * 18 + [vp, sz, vp]
    lib.bdlm_attn_bwd.restype = ctypes.c_int
    lib.bdlm_attn_bwd_noalloc.argtypes = [dp] + [vp] * 18 + [vp]
    lib.bdlm_attn_bwd_noalloc.restype = ctypes.c_int
    lib.bdlm_attn_noalloc_scratch_bytes.argtypes = []
    lib.bdlm_attn_noalloc_scratch_bytes.restype = sz
    lib.bdlm_attn_merge_partials.argtypes = [i32, i32, i64, i32, i32, ctypes.POINTER(vp),
                                             ctypes.POINTER(vp), vp, i32, vp, vp]
    lib.bdlm_attn_merge_partials.restype = ctypes.c_int
    lib.bdlm_attn_schedule_walk.argtypes = [dp, ctypes.c_int, vp, i64, ctypes.POINTER(i64)]
    lib.bdlm_attn_schedule_walk.restype = ctypes.c_int
    lib.bdlm_status_str.argtypes = [ctypes.c_int]
    lib.bdlm_status_str.restype = ctypes.c_char_p
    lib.bdlm_attn_version.argtypes = []
    lib.bdlm_attn_version.restype = ctypes.c_int
    lib.bdlm_attn_profile_begin.argtypes = [i32]
    lib.bdlm_attn_profile_begin.restype = ctypes.c_int
    lib.bdlm_attn_profile_end.argtypes = [ctypes.POINTER(BdlmKernelTime), i32, ctypes.POINTER(i32)]
    lib.bdlm_attn_profile_end.restype = ctypes.c_int
    lib.bdlm_calib_mfma.argtypes = [i32, i32, i32, vp, vp, vp]
    lib.bdlm_calib_mfma.restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().bdlm_status_str(status).decode()


def check(fn: str, status: int) -> None:
    if status != BDLM_OK:
        raise BdlmError(fn, status, status_str(status))


def make_desc(batch, seqlen, block, hq, hkv, head_dim, dtype, scale, block_ids=None,
              kv_begin=0, kv_end=0, own_block=0, clean_queries=0, accumulate=0, kv_staged=0):
    """Build a descriptor; keeps the host block-id array alive on the object."""
    d = BdlmDesc()
    d.batch, d.seqlen, d.block = int(batch), int(seqlen), int(block)
    d.num_q_heads, d.num_kv_heads, d.head_dim = int(hq), int(hkv), int(head_dim)
    d.dtype = int(dtype)
    d.softmax_scale = float(scale)
    if block_ids is not None and len(block_ids) > 0:
        arr = (ctypes.c_int32 * len(block_ids))(*[int(x) for x in block_ids])
        d._ids = arr
        d.num_local_blocks = len(block_ids)
        d.block_ids = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
        d.kv_begin, d.kv_end, d.own_block = int(kv_begin), int(kv_end), int(own_block)
        d.clean_queries = int(clean_queries)
        d.accumulate = int(accumulate)
        d.kv_staged = int(kv_staged)
    else:
        d.num_local_blocks = 0
        d.block_ids = None
        d.clean_queries = int(clean_queries)
        d.accumulate = int(accumulate)
        d.kv_staged = int(kv_staged)
    return d
