"""ctypes view of libdfx.so (include/dfx.h). Marshalling only: no arithmetic here."""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdfx.so")

DFX_OK, DFX_EINVAL, DFX_EUNSUPPORTED, DFX_EWORKSPACE, DFX_EHIP = range(5)
DFX_F32, DFX_BF16 = 0, 1
DFX_W_ROW_MAJOR, DFX_W_PACKED = 0, 1
STATUS_NAMES = {0: "DFX_OK", 1: "DFX_EINVAL", 2: "DFX_EUNSUPPORTED", 3: "DFX_EWORKSPACE", 4: "DFX_EHIP"}

# every function the header declares, with (restype, argtypes)
P, I32, I64, SZ, F32, U32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                             ctypes.c_float, ctypes.c_uint32)


class DfxError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class KVCacheStruct(ctypes.Structure):
    _fields_ = [("dtype", I32), ("num_kv_heads", I32), ("head_dim", I32), ("block_size", I32),
                ("num_blocks", I64), ("k", P), ("v", P), ("block_table", P),
                ("max_blocks_per_seq", I32), ("reserved", I32)]


class LayerWeightsStruct(ctypes.Structure):
    _fields_ = [("hidden", I32), ("num_q_heads", I32), ("num_kv_heads", I32), ("head_dim", I32),
                ("intermediate", I32), ("rms_eps", F32), ("attn_norm_gain", P), ("w_qkv", P),
                ("w_o", P), ("mlp_norm_gain", P), ("w_gate_up", P), ("w_down", P),
                ("couple_a", P), ("couple_b", P), ("couple_c", P)]


class LayerTapsStruct(ctypes.Structure):
    _fields_ = [("h1", ctypes.c_size_t), ("q", ctypes.c_size_t), ("o", ctypes.c_size_t),
                ("h2", ctypes.c_size_t), ("inter", ctypes.c_size_t)]


class MoeWeightsStruct(ctypes.Structure):
    _fields_ = [("hidden", I32), ("num_experts", I32), ("intermediate", I32), ("top_k_primary", I32),
                ("top_k_aux", I32), ("rms_eps", F32), ("norm_gain", P), ("w_router", P), ("w_gate_up", P),
                ("w_down", P), ("couple_b", P), ("couple_c", P)]


class MoeTapsStruct(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("h", "logits", "ids", "weights", "counts", "seqs", "inter",
                                               "inter_stride")]


KVP = ctypes.POINTER(KVCacheStruct)
MWP = ctypes.POINTER(MoeWeightsStruct)
LWP = ctypes.POINTER(LayerWeightsStruct)
PSZ = ctypes.POINTER(ctypes.c_size_t)
PI32 = ctypes.POINTER(ctypes.c_int32)

SIGNATURES = {
    "dfx_version": (ctypes.c_int, []),
    "dfx_last_error": (ctypes.c_char_p, []),
    "dfx_decode_attn_plan": (I32, [KVP, I32, I32, I32, I32, I32, PI32, PSZ]),
    "dfx_decode_attn_workspace_size": (I32, [I32, I32, I32, KVP, I32, I32, PSZ]),
    "dfx_decode_attn": (I32, [KVP, P, I32, I32, I32, I32, P, P, I64, P, I32, F32, P, P, P, I32, P, SZ, P]),
    "dfx_decode_attn_noalloc": (I32, [KVP, P, I32, I32, I32, I32, P, P, I64, P, I32, F32, P, P, P, I32, P]),
    "dfx_kv_append_primary": (I32, [KVP, I32, P, I32, P, P, I64, P]),
    "dfx_grouped_linear_workspace_size": (I32, [I32, I32, I32, I32, PSZ]),
    "dfx_grouped_linear": (I32, [I32, I32, I32, I32, I32, P, P, I32, I32, P, P, P, P, SZ, P]),
    "dfx_pack_weight": (I32, [I32, I32, P, P, P]),
    "dfx_rmsnorm": (I32, [I32, I32, P, P, F32, P, P]),
    "dfx_swiglu_couple": (I32, [I32, I32, I32, P, P, P, P]),
    "dfx_dual_flow_decode_layer_workspace_size": (I32, [LWP, KVP, I32, I32, I32, PSZ]),
    "dfx_dual_flow_decode_layer": (I32, [LWP, KVP, P, I32, I32, I32, P, P, SZ, P]),
    "dfx_dual_flow_decode_layer_taps": (I32, [LWP, KVP, I32, I32, I32, ctypes.POINTER(LayerTapsStruct)]),
    "dfx_dual_flow_decode_step_workspace_size": (I32, [LWP, KVP, I32, I32, I32, I32, PSZ]),
    "dfx_dual_flow_decode_step": (I32, [LWP, KVP, I32, P, I32, P, P, P, I32, I32, I32, P, P, SZ, P]),
    "dfx_dual_flow_output_head_workspace_size": (I32, [I32, I32, I32, I32, PSZ]),
    "dfx_dual_flow_output_head_taps": (I32, [I32, I32, I32, I32, PSZ, PSZ]),
    "dfx_dual_flow_output_head": (I32, [I32, I32, I32, I32, P, P, F32, P, P, P, P, P, P, SZ, P]),
    "dfx_dual_flow_moe_mlp_workspace_size": (I32, [MWP, I32, I32, PSZ]),
    "dfx_dual_flow_moe_mlp_taps": (I32, [MWP, I32, I32, ctypes.POINTER(MoeTapsStruct)]),
    "dfx_dual_flow_moe_mlp": (I32, [MWP, I32, I32, P, P, SZ, P]),
    "dfx_prefill_attn": (I32, [KVP, P, I32, I32, I32, I32, P, I64, P, P, P]),
    "dfx_prefill_dual_attn": (I32, [KVP, P, I32, I32, I32, I32, P, P, P, I32, I64, P, P, P, P]),
    "dfx_prefill_layer_workspace_size": (I32, [LWP, KVP, I32, I32, I32, PSZ]),
    "dfx_prefill_layer_taps": (I32, [LWP, KVP, I32, I32, I32, ctypes.POINTER(LayerTapsStruct)]),
    "dfx_prefill_layer": (I32, [LWP, KVP, P, I32, I32, I32, P, P, SZ, P]),
    "dfx_prefill_step_workspace_size": (I32, [LWP, KVP, I32, I32, I32, I32, PSZ]),
    "dfx_prefill_step": (I32, [LWP, KVP, I32, P, I32, P, P, I32, I32, I32, P, P, SZ, P]),
    "dfx_copy_bytes": (I32, [P, P, SZ, P]),
    "dfx_read_bytes": (I32, [P, SZ, P, P]),
    "dfx_fill_bytes": (I32, [P, SZ, U32, P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libdfx.so from the package directory. There is no fallback: without the
    built library every call fails here."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m dual_flow_shared_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def check(status: int) -> None:
    if status != DFX_OK:
        raise DfxError(status, lib().dfx_last_error().decode())
