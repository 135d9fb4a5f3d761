"""ctypes declarations of libsparsesam.so (include/sparsesam.h)."""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparsesam.so")

SPARSESAM_F32 = 0
SPARSESAM_BF16 = 1

STATUS = {
    0: "SPARSESAM_OK",
    1: "SPARSESAM_ERR_INVALID_ARGUMENT",
    2: "SPARSESAM_ERR_UNSUPPORTED",
    3: "SPARSESAM_ERR_WORKSPACE",
    4: "SPARSESAM_ERR_OUT_OF_MEMORY",
    5: "SPARSESAM_ERR_HIP",
    6: "SPARSESAM_ERR_NO_DEVICE",
}

# Every symbol the header declares.
EXPORTS = [
    "sparsesam_plan_create",
    "sparsesam_plan_get_info",
    "sparsesam_plan_tile_list",
    "sparsesam_plan_info_get",
    "sparsesam_plan_block_list",
    "sparsesam_plan_destroy",
    "sparsesam_status_string",
    "sparsesam_last_error",
    "sparsesam_importance",
    "sparsesam_permute",
    "sparsesam_attn",
    "sparsesam_attn_relpos",
    "sparsesam_mlp",
    "sparsesam_block",
    "sparsesam_forward",
    "sparsesam_encoder",
    "sparsesam_noalloc_scratch_bytes",
    "sparsesam_block_noalloc",
    "sparsesam_route_topk",
    "sparsesam_block_dynamic",
    "sparsesam_encoder_permuted_workspace",
    "sparsesam_encoder_permuted",
]


class PlanDesc(ctypes.Structure):
    _fields_ = [
        ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32), ("window", ctypes.c_int32),
        ("stripes", ctypes.c_int32), ("block", ctypes.c_int32), ("global_tokens", ctypes.c_int32),
        ("band_radius", ctypes.c_int32), ("attn_density", ctypes.c_float), ("mlp_density", ctypes.c_float),
        ("channels", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("mlp_hidden", ctypes.c_int32), ("max_batch", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("ordering", ctypes.c_int32), ("order_seed", ctypes.c_uint32), ("rel_pos", ctypes.c_int32),
        ("routing", ctypes.c_int32), ("mlp_merge", ctypes.c_int32),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("seq_len", ctypes.c_int32), ("segments_per_image", ctypes.c_int32), ("band_radius", ctypes.c_int32),
        ("tiles_per_stripe", ctypes.c_int32), ("tiles", ctypes.c_int32), ("tiles_kept", ctypes.c_int32),
        ("pairs_kept", ctypes.c_int64), ("realised_density", ctypes.c_double),
        ("routed_per_image", ctypes.c_int32), ("reserved0", ctypes.c_int32),
        ("block_workspace_bytes", ctypes.c_size_t), ("mlp_workspace_bytes", ctypes.c_size_t),
        ("attn_workspace_bytes", ctypes.c_size_t),
        ("has_device_copy", ctypes.c_int32), ("device", ctypes.c_int32),
        ("relpos_workspace_bytes", ctypes.c_size_t),
    ]


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_proj", "b_proj", "ln2_g", "ln2_b", "w1", "b1", "w2", "b2",
                 "rel_pos_h", "rel_pos_w")]


_lib = None


def load():
    """Load libsparsesam.so from the package directory; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libsparsesam.so is not built (expected at %s); run `python -m structured_sparse_vit_amd.build`"
            % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "sparsesam_plan_create": ([ctypes.POINTER(PlanDesc), ctypes.POINTER(P)], I32),
        "sparsesam_plan_get_info": ([P, ctypes.POINTER(PlanInfo)], I32),
        "sparsesam_plan_tile_list": ([P, P, P], I32),
        "sparsesam_plan_info_get": ([P, ctypes.POINTER(PlanInfo)], I32),
        "sparsesam_plan_block_list": ([P, P, P], I32),
        "sparsesam_plan_destroy": ([P], None),
        "sparsesam_status_string": ([I32], ctypes.c_char_p),
        "sparsesam_last_error": ([], ctypes.c_char_p),
        "sparsesam_importance": ([P, I32, I32, I32, I32, P, P], I32),
        "sparsesam_permute": ([P, P, I32, P, P, P, P], I32),
        "sparsesam_attn": ([P, I32, P, P, P, P, F32, P, SZ, P], I32),
        "sparsesam_attn_relpos": ([P, I32, P, P, P, P, F32, P, P, P, P, SZ, P], I32),
        "sparsesam_mlp": ([P, P, I64, P, I32, P, P, P, P, P, P, P, SZ, P], I32),
        "sparsesam_block": ([P, ctypes.POINTER(BlockWeights), P, I32, P, P, P, SZ, P], I32),
        "sparsesam_forward": ([P, ctypes.POINTER(BlockWeights), P, I32, I32, I32, I32, P, P, P, P, P, P, SZ, P], I32),
        "sparsesam_encoder": ([P, P, ctypes.POINTER(BlockWeights), P, I32, P, I32, P, P, P, P, P, SZ, P], I32),
        "sparsesam_noalloc_scratch_bytes": ([], SZ),
        "sparsesam_block_noalloc": ([P, ctypes.POINTER(BlockWeights), P, I32, P, P, P], I32),
        "sparsesam_route_topk": ([P, P, I32, P, P], I32),
        "sparsesam_block_dynamic": ([P, ctypes.POINTER(BlockWeights), P, I32, P, P, P, P, SZ, P], I32),
        "sparsesam_encoder_permuted_workspace": ([P, P, I32, ctypes.POINTER(SZ)], I32),
        "sparsesam_encoder_permuted": ([P, P, ctypes.POINTER(BlockWeights), P, I32, P, I32, P, P, P, P, P, SZ, P],
                                       I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


class SparseSAMError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.sparsesam_last_error().decode(errors="replace")
        super().__init__("%s failed: %s (%s)" % (where, STATUS.get(status, status), msg))
        self.status = status


def check(status: int, where: str):
    if status != 0:
        raise SparseSAMError(status, where)
