"""Python binding of libqmoe (the MoE step with group-affine quantized experts on
MI355X). Argument marshalling only: every step runs in the HIP kernels behind
the C ABI declared in include/qmoe.h. PyTorch supplies device memory and the
current stream.

The binding raises if ``libqmoe.so`` is missing; there is no fallback path.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqmoe.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_SHAPE, MOE_ERR_ALIGN = 0, -1, -2, -3
MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_DEVICE = -4, -5, -6, -7
MOE_F_RMSNORM, MOE_F_RESIDUAL, MOE_F_SELECT_BY_BIAS = 1, 2, 4
MOE_F_PREFILL_BF16, MOE_F_PHASED = 8, 16

EXPORTS = ["moe_packed_expert_bytes", "moe_workspace_bytes", "moe_pack_weights", "moe_route",
           "moe_expert_forward", "moe_layer_forward", "moe_stack_decode", "moe_stack_decode_streamed",
           "moe_stack_decode_noalloc",
           "moe_qkv_packed_bytes", "moe_qkv_pack", "moe_qkv_forward", "moe_last_error", "moe_device_status"]


class MoeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"status {status}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group", ctypes.c_int32), ("flags", ctypes.c_int32), ("eps", ctypes.c_float)]

    @classmethod
    def make(cls, hidden, inter, n_experts, top_k=4, n_shared=1, bits=4, flags=0, eps=1e-6, group=64):
        return cls(hidden, inter, n_experts, top_k, n_shared, bits, group, flags, eps)

    def with_flags(self, flags):
        return Config(self.hidden, self.inter, self.n_experts, self.top_k, self.n_shared, self.bits,
                      self.group, flags, self.eps)


class QkvConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("q_rows", ctypes.c_int32), ("k_rows", ctypes.c_int32),
                ("v_rows", ctypes.c_int32), ("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("eps", ctypes.c_float)]

    @classmethod
    def make(cls, hidden, q_rows, k_rows, v_rows, bits=4, flags=0, eps=1e-6, group=64):
        return cls(hidden, q_rows, k_rows, v_rows, bits, group, flags, eps)


class LayerWeights(ctypes.Structure):
    _fields_ = [("experts", ctypes.c_void_p), ("shared", ctypes.c_void_p),
                ("router_w", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("shared_gate", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, C = ctypes.c_void_p, ctypes.POINTER(Config)
        sz, i32, st = ctypes.c_size_t, ctypes.c_int32, ctypes.c_int
        L.moe_packed_expert_bytes.restype = sz
        L.moe_packed_expert_bytes.argtypes = [C]
        L.moe_workspace_bytes.restype = sz
        L.moe_workspace_bytes.argtypes = [C, i32, i32]
        L.moe_pack_weights.restype = st
        L.moe_pack_weights.argtypes = [C, i32, P, P, P, P, sz, P, sz, P]
        L.moe_route.restype = st
        L.moe_route.argtypes = [C, i32, P, P, P, P, P, P, P, P, P, sz, P]
        L.moe_expert_forward.restype = st
        L.moe_expert_forward.argtypes = [C, P, i32, P, P, P, sz, P]
        L.moe_layer_forward.restype = st
        L.moe_layer_forward.argtypes = [C, ctypes.POINTER(LayerWeights), i32, P, P, P, P, P, P, P, sz, P]
        L.moe_stack_decode.restype = st
        L.moe_stack_decode.argtypes = [C, i32, ctypes.POINTER(LayerWeights), i32, P, P, P, P, P, P, sz, P]
        L.moe_stack_decode_noalloc.restype = st
        L.moe_stack_decode_noalloc.argtypes = [C, i32, ctypes.POINTER(LayerWeights), i32, P, P, P, P, P, P, P]
        L.moe_stack_decode_streamed.restype = st
        L.moe_stack_decode_streamed.argtypes = [C, i32, ctypes.POINTER(LayerWeights), i32, P, P, P, P, P, P,
                                                P, sz, i32, P, sz, P]
        Q = ctypes.POINTER(QkvConfig)
        L.moe_qkv_packed_bytes.restype = sz
        L.moe_qkv_packed_bytes.argtypes = [Q]
        L.moe_qkv_pack.restype = st
        L.moe_qkv_pack.argtypes = [Q, P, P, P, P, sz, P, sz, P]
        L.moe_qkv_forward.restype = st
        L.moe_qkv_forward.argtypes = [Q, P, P, i32, P, P, P, P, P]
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_device_status.restype = st
        L.moe_device_status.argtypes = [P, sz, P]
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(status):
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())
    return status


def moe_packed_expert_bytes(cfg):
    return lib().moe_packed_expert_bytes(ctypes.byref(cfg))


def moe_workspace_bytes(cfg, n_tokens, n_layers=1):
    return lib().moe_workspace_bytes(ctypes.byref(cfg), n_tokens, n_layers)


def moe_last_error():
    return lib().moe_last_error().decode()


def moe_pack_weights(cfg, n, codes, scales, biases, packed, ws, stream=None):
    return _check(lib().moe_pack_weights(ctypes.byref(cfg), n, _ptr(codes), _ptr(scales), _ptr(biases),
                                         _ptr(packed), packed.numel() * packed.element_size(), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(stream)))


def moe_route(cfg, T, x, router_w, idx_out, w_out, ws, gamma=None, sel_bias=None, boosted=None,
              logits_out=None, stream=None):
    return _check(lib().moe_route(ctypes.byref(cfg), T, _ptr(x), _ptr(router_w), _ptr(gamma),
                                  _ptr(sel_bias), _ptr(boosted), _ptr(idx_out), _ptr(w_out),
                                  _ptr(logits_out), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)))


def moe_expert_forward(cfg, packed_expert, T, x, y, ws, stream=None):
    return _check(lib().moe_expert_forward(ctypes.byref(cfg), _ptr(packed_expert), T, _ptr(x), _ptr(y),
                                           _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def layer_weights(experts, shared, router_w, gamma=None, shared_gate=None):
    return LayerWeights(experts.data_ptr(), shared.data_ptr() if shared is not None else None,
                        router_w.data_ptr(), gamma.data_ptr() if gamma is not None else None,
                        shared_gate.data_ptr() if shared_gate is not None else None)


def moe_layer_forward(cfg, layer, T, x, y, ws, sel_bias=None, boosted=None, idx_out=None, w_out=None,
                      stream=None):
    return _check(lib().moe_layer_forward(ctypes.byref(cfg), ctypes.byref(layer), T, _ptr(x), _ptr(y),
                                          _ptr(sel_bias), _ptr(boosted), _ptr(idx_out), _ptr(w_out),
                                          _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_stack_decode(cfg, layers, T, x0, y, ws, boost_mask=None, idx_trace=None, w_trace=None,
                     stream=None):
    arr = (LayerWeights * len(layers))(*layers)
    return _check(lib().moe_stack_decode(ctypes.byref(cfg), len(layers), arr, T, _ptr(x0), _ptr(boost_mask),
                                         _ptr(y), _ptr(idx_trace), _ptr(w_trace), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(stream)))


def moe_stack_decode_noalloc(cfg, layers, T, x0, y, boost_mask=None, idx_trace=None, w_trace=None,
                             dev_err=None, stream=None):
    """moe_stack_decode on the library's fixed scratch array (no workspace)."""
    arr = (LayerWeights * len(layers))(*layers)
    return _check(lib().moe_stack_decode_noalloc(ctypes.byref(cfg), len(layers), arr, T, _ptr(x0),
                                                 _ptr(boost_mask), _ptr(y), _ptr(idx_trace), _ptr(w_trace),
                                                 _ptr(dev_err), _stream(stream)))


def moe_stack_decode_streamed(cfg, layers, T, x0, y, ws, cache, cache_slots, boost_mask=None, idx_trace=None,
                              w_trace=None, hit_trace=None, stream=None):
    """layers[l].experts must point to pinned host memory (e.g. a torch CPU tensor
    made with pin_memory=True); cache is a device byte tensor."""
    arr = (LayerWeights * len(layers))(*layers)
    return _check(lib().moe_stack_decode_streamed(
        ctypes.byref(cfg), len(layers), arr, T, _ptr(x0), _ptr(boost_mask), _ptr(y), _ptr(idx_trace),
        _ptr(w_trace), _ptr(hit_trace), _ptr(cache), cache.numel() * cache.element_size(), cache_slots,
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_qkv_packed_bytes(cfg):
    return lib().moe_qkv_packed_bytes(ctypes.byref(cfg))


def moe_qkv_pack(cfg, codes, scales, biases, packed, ws, stream=None):
    return _check(lib().moe_qkv_pack(ctypes.byref(cfg), _ptr(codes), _ptr(scales), _ptr(biases), _ptr(packed),
                                     packed.numel() * packed.element_size(), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)))


def moe_qkv_forward(cfg, packed, T, x, q_out, k_out, v_out, gamma=None, stream=None):
    return _check(lib().moe_qkv_forward(ctypes.byref(cfg), _ptr(packed), _ptr(gamma), T, _ptr(x), _ptr(q_out),
                                        _ptr(k_out), _ptr(v_out), _stream(stream)))


def moe_device_status(ws, stream=None):
    return _check(lib().moe_device_status(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
