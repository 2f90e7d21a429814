"""CPU-side checks of the C ABI: the library loads, exports every entry point the
header declares, computes the closed-form sizes, and rejects bad arguments
before touching the GPU."""
import ctypes
import os
import re

import pytest

import quantized_expert_mat_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared():
    src = open(os.path.join(ROOT, "include", "qmoe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared()
    assert set(names) == set(q.EXPORTS)
    L = ctypes.CDLL(q.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_packed_expert_bytes_closed_form():
    # 3 matrices of H*I codes at bits/8 bytes + one bf16 (scale, bias) pair per 64 codes
    for H, I, bits in [(4096, 1024, 4), (4096, 1024, 3), (4096, 1024, 2), (1024, 256, 4), (64, 64, 2),
                       (64, 64, 3), (4096, 4096, 4)]:
        cfg = q.Config.make(H, I, 8, 4, 1, bits)
        assert q.moe_packed_expert_bytes(cfg) == 3 * H * I * bits // 8 + 3 * H * I // 64 * 4
    assert q.moe_packed_expert_bytes(q.Config.make(4096, 1024, 512)) == 7_077_888  # 6.75 MiB
    assert q.moe_packed_expert_bytes(q.Config.make(4096, 1024, 512, bits=2)) == 3_932_160
    assert q.moe_packed_expert_bytes(q.Config.make(4096, 1024, 512, bits=3)) == 5_505_024


def test_workspace_bytes_positive_and_monotone():
    cfg = q.Config.make(4096, 1024, 512)
    a = q.moe_workspace_bytes(cfg, 1, 1)
    b = q.moe_workspace_bytes(cfg, 256, 60)
    assert 0 < a <= b
    assert q.moe_workspace_bytes(cfg, -1, 1) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(bits=5), q.MOE_ERR_UNSUPPORTED), (dict(bits=1), q.MOE_ERR_UNSUPPORTED),
    (dict(hidden=1000), q.MOE_ERR_UNSUPPORTED),
    (dict(hidden=8192), q.MOE_ERR_UNSUPPORTED), (dict(top_k=17), q.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=2, top_k=4), q.MOE_ERR_SHAPE), (dict(n_experts=2000), q.MOE_ERR_SHAPE),
    (dict(n_shared=3), q.MOE_ERR_UNSUPPORTED), (dict(group=32), q.MOE_ERR_UNSUPPORTED),
    (dict(flags=1 << 10), q.MOE_ERR_ARG), (dict(flags=q.MOE_F_RMSNORM, eps=0.0), q.MOE_ERR_ARG),
])
def test_bad_config_rejected(kw, status):
    base = dict(hidden=1024, inter=256, n_experts=64)
    base.update(kw)
    cfg = q.Config.make(**base)
    assert q.moe_packed_expert_bytes(cfg) == 0
    L = q.lib()
    fake = ctypes.c_void_p(1 << 20)
    rc = L.moe_expert_forward(ctypes.byref(cfg), fake, 1, fake, fake, fake, 1 << 20, None)
    assert rc == status
    assert L.moe_last_error()


def test_null_misaligned_and_small_workspace_rejected():
    L = q.lib()
    cfg = q.Config.make(1024, 256, 64)
    p = ctypes.c_void_p(1 << 20)
    big = q.moe_workspace_bytes(cfg, 4, 1)
    assert L.moe_expert_forward(ctypes.byref(cfg), None, 1, p, p, p, big, None) == q.MOE_ERR_ARG
    assert L.moe_expert_forward(ctypes.byref(cfg), ctypes.c_void_p((1 << 20) + 8), 1, p, p, p, big,
                                None) == q.MOE_ERR_ALIGN
    assert L.moe_expert_forward(ctypes.byref(cfg), p, 4, p, p, p, 10, None) == q.MOE_ERR_WORKSPACE
    assert L.moe_expert_forward(ctypes.byref(cfg), p, -1, p, p, p, big, None) == q.MOE_ERR_ARG
    # T == 0 is a no-op that touches nothing
    assert L.moe_expert_forward(ctypes.byref(cfg), None, 0, None, None, None, 0, None) == q.MOE_OK
    assert L.moe_pack_weights(ctypes.byref(cfg), 1, p, p, p, p, 10, p, big, None) == q.MOE_ERR_SHAPE
    lw = q.LayerWeights(1 << 20, 1 << 20, 1 << 20, None)
    cfg_sel = cfg.with_flags(q.MOE_F_SELECT_BY_BIAS)
    assert L.moe_layer_forward(ctypes.byref(cfg_sel), ctypes.byref(lw), 1, p, p, None, None, None, None, p,
                               big, None) == q.MOE_ERR_ARG
    # a shared-expert gate must be 16-byte aligned
    lw_gate = q.LayerWeights(1 << 20, 1 << 20, 1 << 20, None, (1 << 20) + 4)
    assert L.moe_layer_forward(ctypes.byref(cfg), ctypes.byref(lw_gate), 1, p, p, None, None, None, None,
                               p, big, None) == q.MOE_ERR_ALIGN
    arr = (q.LayerWeights * 1)(lw)
    assert L.moe_stack_decode(ctypes.byref(cfg_sel), 1, arr, 1, p, None, p, None, None, p, big,
                              None) == q.MOE_ERR_ARG
    assert L.moe_device_status(None, 0, None) == q.MOE_ERR_ARG


def test_stack_validates_every_layer_before_any_device_call():
    """moe_stack_decode checks all L layers before it enqueues anything: a bad layer
    70 of 100 is an argument error naming that layer. On a host without a GPU any
    enqueue would fail with MOE_ERR_HIP first, so an argument error here shows
    that nothing was enqueued; with every layer valid the call gets as far as the
    device (and fails there only because there is none)."""
    L = q.lib()
    cfg = q.Config.make(1024, 256, 64, flags=q.MOE_F_RMSNORM | q.MOE_F_RESIDUAL)
    p = ctypes.c_void_p(1 << 20)
    n = 100
    big = q.moe_workspace_bytes(cfg, 2, n)
    good = [q.LayerWeights(1 << 20, 1 << 21, 1 << 22, None) for _ in range(n)]
    bad = list(good)
    bad[70] = q.LayerWeights(None, 1 << 21, 1 << 22, None)
    arr = (q.LayerWeights * n)(*bad)
    assert L.moe_stack_decode(ctypes.byref(cfg), n, arr, 2, p, None, p, None, None, p, big, None) == q.MOE_ERR_ARG
    assert b"layer 70" in L.moe_last_error()
    misaligned = list(good)
    misaligned[99] = q.LayerWeights(1 << 20, 1 << 21, (1 << 22) + 64, None)
    arr = (q.LayerWeights * n)(*misaligned)
    assert L.moe_stack_decode(ctypes.byref(cfg), n, arr, 2, p, None, p, None, None, p, big, None) == q.MOE_ERR_ALIGN
    assert b"layer 99" in L.moe_last_error()
    arr = (q.LayerWeights * n)(*good)
    import torch
    if not torch.cuda.is_available():
        assert L.moe_stack_decode(ctypes.byref(cfg), n, arr, 2, p, None, p, None, None, p, big,
                                  None) == q.MOE_ERR_HIP


def test_binding_raises_with_message():
    cfg = q.Config.make(1024, 256, 64, bits=5)
    with pytest.raises(q.MoeError) as ei:
        q._check(q.lib().moe_expert_forward(ctypes.byref(cfg), None, 1, None, None, None, 0, None))
    assert "bits=5" in str(ei.value)


def test_streamed_stack_validation():
    """The streamed stack rejects bad cache arguments before any device call."""
    L = q.lib()
    cfg = q.Config.make(1024, 256, 64)
    p = ctypes.c_void_p(1 << 20)
    big = q.moe_workspace_bytes(cfg, 2, 2)
    cache_need = 2 * 8 * q.moe_packed_expert_bytes(cfg)
    arr = (q.LayerWeights * 2)(q.LayerWeights(1 << 20, 1 << 20, 1 << 20, None),
                               q.LayerWeights(1 << 20, 1 << 20, 1 << 20, None))

    def call(c=cfg, slots=8, cache=p, cache_bytes=cache_need, ws_bytes=big):
        return L.moe_stack_decode_streamed(ctypes.byref(c), 2, arr, 2, p, None, p, None, None, None, cache,
                                           cache_bytes, slots, p, ws_bytes, None)

    assert call(slots=3) == q.MOE_ERR_ARG          # fewer slots than top_k
    assert call(slots=65) == q.MOE_ERR_ARG         # more than 64
    assert call(cache_bytes=cache_need - 1) == q.MOE_ERR_ARG
    assert call(cache=ctypes.c_void_p((1 << 20) + 64)) == q.MOE_ERR_ALIGN
    assert call(cache=None) == q.MOE_ERR_ARG
    assert call(c=cfg.with_flags(q.MOE_F_PHASED)) == q.MOE_ERR_ARG
    assert call(ws_bytes=10) == q.MOE_ERR_WORKSPACE
    assert L.moe_stack_decode_streamed(ctypes.byref(cfg), 2, arr, 0, None, None, None, None, None, None, None, 0,
                                       0, None, 0, None) == q.MOE_OK  # T == 0: no-op


def test_qkv_sizes_and_validation():
    # Rq + Rk + Rv rows of H codes at bits/8 bytes + one (scale, bias) pair per 64 codes
    for H, rows, bits in [(4096, (4096, 512, 512), 4), (4096, (4096, 512, 512), 3), (512, (200, 40, 44), 4),
                          (64, (5, 3, 2), 2)]:
        cfg = q.QkvConfig.make(H, *rows, bits=bits)
        P = 64 // (H // 64)  # rows per block
        nblk = -(-sum(rows) // P)
        assert q.moe_qkv_packed_bytes(cfg) == nblk * P * H * bits // 8 + nblk * P * (H // 64) * 4
    assert q.moe_qkv_packed_bytes(q.QkvConfig.make(4096, 4096, 512, 512)) == 11_796_480
    for bad in [q.QkvConfig.make(1000, 8, 8, 8), q.QkvConfig.make(512, 0, 8, 8), q.QkvConfig.make(512, 8, 8, 8, bits=5),
                q.QkvConfig.make(512, 8, 8, 8, flags=q.MOE_F_RESIDUAL), q.QkvConfig.make(512, 65536, 1, 1)]:
        assert q.moe_qkv_packed_bytes(bad) == 0
    L = q.lib()
    cfg = q.QkvConfig.make(512, 8, 8, 8)
    p = ctypes.c_void_p(1 << 20)
    assert L.moe_qkv_forward(ctypes.byref(cfg), p, None, 1, p, p, p, None, None) == q.MOE_ERR_ARG
    assert L.moe_qkv_forward(ctypes.byref(cfg), ctypes.c_void_p((1 << 20) + 16), None, 1, p, p, p, p,
                             None) == q.MOE_ERR_ALIGN
    assert L.moe_qkv_forward(ctypes.byref(cfg), None, None, 0, None, None, None, None, None) == q.MOE_OK
    assert L.moe_qkv_pack(ctypes.byref(cfg), p, p, p, p, 10, p, 1024, None) == q.MOE_ERR_SHAPE
    assert L.moe_qkv_pack(ctypes.byref(cfg), p, p, p, p, 1 << 20, p, 100, None) == q.MOE_ERR_WORKSPACE



def test_c_program_links_and_calls_the_abi(tmp_path):
    """The header is plain C99 and a C program links against the library: it calls
    the size functions (no device needed) and gets the closed forms."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(r"""
#include <stdio.h>
#include "qmoe.h"
int main(void) {
  moe_config c = {4096, 1024, 512, 4, 1, 4, 64, 0, 1e-6f};
  moe_qkv_config k = {4096, 4096, 512, 512, 4, 64, 0, 1e-6f};
  moe_config bad = c;
  bad.bits = 5;
  printf("%zu %zu %zu\n", moe_packed_expert_bytes(&c), moe_qkv_packed_bytes(&k), moe_packed_expert_bytes(&bad));
  return 0;
}
""")
    lib_dir = os.path.dirname(q.LIB_PATH)
    exe = tmp_path / "abi"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    "-L", lib_dir, "-lqmoe", f"-Wl,-rpath,{lib_dir}"], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    assert out == ["7077888", "11796480", "0"]


def test_noalloc_stack_limits_checked_before_any_device_call():
    """moe_stack_decode_noalloc rejects what its fixed 4 MiB scratch array cannot
    hold (more than 128 layers; a shape whose workspace exceeds it) and bad layers,
    all before any HIP call; the pages' shape (hidden 4096, inter 1024, 512 experts)
    fits."""
    L = q.lib()
    p = ctypes.c_void_p(1 << 20)
    lw = q.LayerWeights(1 << 20, 1 << 21, 1 << 22, None)
    arr = (q.LayerWeights * 129)(*([lw] * 129))
    cfg = q.Config.make(4096, 1024, 512, flags=q.MOE_F_RMSNORM | q.MOE_F_RESIDUAL)
    assert L.moe_stack_decode_noalloc(ctypes.byref(cfg), 129, arr, 2, p, None, p, None, None, None,
                                      None) == q.MOE_ERR_UNSUPPORTED
    wide = q.Config.make(4096, 4096, 512, flags=q.MOE_F_RMSNORM | q.MOE_F_RESIDUAL)
    assert L.moe_stack_decode_noalloc(ctypes.byref(wide), 60, arr, 2, p, None, p, None, None, None,
                                      None) == q.MOE_ERR_WORKSPACE
    assert b"scratch" in L.moe_last_error()
    bad = (q.LayerWeights * 60)(*([lw] * 59 + [q.LayerWeights(None, 1 << 21, 1 << 22, None)]))
    assert L.moe_stack_decode_noalloc(ctypes.byref(cfg), 60, bad, 256, p, None, p, None, None, None,
                                      None) == q.MOE_ERR_ARG
    assert b"layer 59" in L.moe_last_error()
    assert L.moe_stack_decode_noalloc(ctypes.byref(cfg), 60, arr, 256, p, None, p, None, None,
                                      ctypes.c_void_p((1 << 20) + 2), None) == q.MOE_ERR_ALIGN
    assert L.moe_stack_decode_noalloc(ctypes.byref(cfg), 60, arr, 0, p, None, p, None, None, None,
                                      None) == q.MOE_OK
    import torch
    if not torch.cuda.is_available():
        assert L.moe_stack_decode_noalloc(ctypes.byref(cfg), 60, arr, 256, p, None, p, None, None, None,
                                          None) == q.MOE_ERR_HIP
