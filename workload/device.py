"""Device-side fill of the synthetic workload (same bits as ``workload.gen``).

Used by the GPU tests and the benchmark to materialise large weight sets in
HBM directly, and the read-only HBM stream probe of the benchmark. Generation and
measurement only; no MoE arithmetic.
"""
import ctypes
import os
import subprocess

import numpy as np

from . import gen

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen_device.hip")
_LIB = os.path.join(_HERE, "libqmoe_gen.so")
_lib = None


def build(verbose=False):
    tmp = _LIB + ".tmp"
    cmd = [os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), "--offload-arch=gfx950", "-O3", "-fPIC",
           "-shared", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", tmp, _SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB)
        L.qgen_codes.restype = ctypes.c_int
        L.qgen_codes.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p]
        L.qgen_normal.restype = ctypes.c_int
        L.qgen_normal.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_double,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        L.qgen_zero_mean_bias.restype = ctypes.c_int
        L.qgen_zero_mean_bias.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong,
                                          ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p]
        L.qgen_read_probe.restype = ctypes.c_int
        L.qgen_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def _keys_tensor(keys, device):
    import torch
    a = np.array([k & ((1 << 64) - 1) for k in keys], dtype=np.uint64).view(np.int64)
    return torch.from_numpy(a).to(device)


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def fill_codes(keys, n, bits, out):
    """out: uint8 CUDA tensor with len(keys) * n elements."""
    kt = _keys_tensor(keys, out.device)
    rc = lib().qgen_codes(kt.data_ptr(), len(keys), n, bits, out.data_ptr(), _stream())
    if rc != 0:
        raise RuntimeError(f"qgen_codes failed: hipError {rc}")
    return kt  # keep alive until the stream passes


def fill_normal(keys, n, sigma, out, absolute=False):
    """out: float32 or bf16-bits (int16/uint16) CUDA tensor with len(keys) * n elements."""
    import torch
    as_bf16 = out.dtype in (torch.int16, torch.uint16, torch.bfloat16)
    kt = _keys_tensor(keys, out.device)
    rc = lib().qgen_normal(kt.data_ptr(), len(keys), n, float(sigma), int(absolute), int(as_bf16),
                           out.data_ptr(), _stream())
    if rc != 0:
        raise RuntimeError(f"qgen_normal failed: hipError {rc}")
    return kt


def fill_zero_mean_bias(skeys, bkeys, n, sigma_scale, sigma_bias, bits, out):
    """out: bf16-bits CUDA tensor with len(bkeys) * n elements (the zero-mean bias of gen.py)."""
    st = _keys_tensor(skeys, out.device)
    bt = _keys_tensor(bkeys, out.device)
    rc = lib().qgen_zero_mean_bias(st.data_ptr(), bt.data_ptr(), len(bkeys), n, float(sigma_scale),
                                   float(sigma_bias), int(bits), out.data_ptr(), _stream())
    if rc != 0:
        raise RuntimeError(f"qgen_zero_mean_bias failed: hipError {rc}")
    return (st, bt)


def read_probe(buf, sink):
    """Launch the read-only stream probe over the device tensor buf (its bytes a
    multiple of 16) on torch's current stream; sink is a device int32 tensor."""
    rc = lib().qgen_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), _stream())
    if rc != 0:
        raise RuntimeError(f"qgen_read_probe failed: hipError {rc}")


def experts_canonical(spec, seed, layer, experts, codes, scales, biases):
    """Fill canonical tensors for the listed experts: codes uint8 [n][3][H*I],
    scales/biases int16 [n][3][H*I/64] (bf16 bits)."""
    n_el = spec.hidden * spec.inter
    ck = [gen.stream_key(seed, gen.KIND_CODES, layer, e, m) for e in experts for m in range(3)]
    sk = [gen.stream_key(seed, gen.KIND_SCALE, layer, e, m) for e in experts for m in range(3)]
    bk = [gen.stream_key(seed, gen.KIND_BIAS, layer, e, m) for e in experts for m in range(3)]
    keep = [fill_codes(ck, n_el, spec.bits, codes),
            fill_normal(sk, n_el // 64, spec.sigma_scale, scales, absolute=True)]
    if getattr(spec, "zero_mean", False):
        keep.append(fill_zero_mean_bias(sk, bk, n_el // 64, spec.sigma_scale, spec.sigma_bias, spec.bits, biases))
    else:
        keep.append(fill_normal(bk, n_el // 64, spec.sigma_bias, biases))
    return keep


def router(seed, layer, n_experts, hidden, out, sigma=0.02):
    return fill_normal([gen.stream_key(seed, gen.KIND_ROUTER, layer, 0, 0)], n_experts * hidden, sigma, out)


def tokens_x(seed, n_tokens, hidden, out, first_token=0):
    keys = [gen.stream_key(seed, gen.KIND_X, 0, first_token + t, 0) for t in range(n_tokens)]
    return fill_normal(keys, hidden, 1.0, out)
