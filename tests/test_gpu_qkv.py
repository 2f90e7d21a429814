"""GPU parity of the fused Q/K/V projection (moe_qkv_pack + moe_qkv_forward)
against the oracle's three dequant mat-vecs, through the C ABI."""
import numpy as np
import pytest

import quantized_expert_mat_amd as q
import workload as wl
from oracle import ref
from tests.helpers import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BF16_ONE = 0x3F80


def canon(rng, H, rows, bits, s_sigma):
    R = sum(rows)
    codes = rng.integers(0, 1 << bits, size=(R, H), dtype=np.uint8)
    sc = wl.bf16_bits_from_f32(np.abs(rng.normal(0, s_sigma, (R, H // 64))).astype(np.float32))
    bi = wl.bf16_bits_from_f32(rng.normal(0, 0.01, (R, H // 64)).astype(np.float32))
    return codes, sc, bi


def split(codes, sc, bi, rows):
    out, r0 = [], 0
    for r in rows:
        out.append((codes[r0:r0 + r], sc[r0:r0 + r], bi[r0:r0 + r]))
        r0 += r
    return out


def pack(cfg, codes, sc, bi):
    packed = torch.empty(q.moe_qkv_packed_bytes(cfg), dtype=torch.uint8, device="cuda")
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    q.moe_qkv_pack(cfg, torch.from_numpy(codes).cuda(), torch.from_numpy(sc.view(np.int16)).cuda(),
                   torch.from_numpy(bi.view(np.int16)).cuda(), packed, ws)
    q.moe_device_status(ws)
    return packed


def run(cfg, packed, x, gamma=None):
    T = x.shape[0]
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    outs = [torch.empty((T, r), dtype=torch.float32, device="cuda") for r in (cfg.q_rows, cfg.k_rows, cfg.v_rows)]
    g = torch.from_numpy(gamma).cuda() if gamma is not None else None
    q.moe_qkv_forward(cfg, packed, T, xd, *outs, gamma=g)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


@pytest.mark.parametrize("bits,H,rows,T,norm,with_gamma", [
    (4, 512, (200, 40, 44), 3, False, False),   # ragged: the last block is partly used
    (4, 512, (200, 40, 44), 2, True, True),
    (3, 1024, (256, 64, 64), 2, True, False),
    (2, 256, (64, 32, 33), 3, False, True),
    (4, 64, (5, 3, 2), 2, True, True),           # one group per row: 64 rows per block
    (4, 4096, (4096, 512, 512), 2, True, True),  # an attention-sized projection of hidden 4096
    (3, 4096, (4096, 512, 512), 1, True, True),
])
def test_qkv_parity(bits, H, rows, T, norm, with_gamma):
    rng = np.random.default_rng(hash((bits, H, rows, T, norm)) % 2**32)
    cfg = q.QkvConfig.make(H, *rows, bits=bits, flags=q.MOE_F_RMSNORM if norm else 0)
    codes, sc, bi = canon(rng, H, rows, bits, {4: 0.02, 3: 0.04, 2: 0.06}[bits])
    packed = pack(cfg, codes, sc, bi)
    x = wl.tokens_x(int(rng.integers(1 << 30)), T, H)
    gamma = (1.0 + 0.1 * rng.normal(size=H)).astype(np.float32) if with_gamma else None
    outs = run(cfg, packed, x, gamma)
    mats = split(codes, sc, bi, rows)
    for t in range(T):
        want = ref.qkv(mats, x[t], gamma=gamma, norm=norm)
        for name, got, ref_y in zip("qkv", outs, want):
            parity(got[t], ref_y, f"{name} token {t}")


def test_qkv_integer_sums():
    """scale 1, bias 0, integer x, no norm: every output is an integer sum (met to
    float32 rounding of the encoded input), so a wrong row, a swapped output or a
    misread code shows as an O(1) error."""
    rng = np.random.default_rng(5)
    H, rows, T = 1024, (96, 16, 24), 2
    cfg = q.QkvConfig.make(H, *rows, bits=4)
    R = sum(rows)
    codes = rng.integers(0, 16, size=(R, H), dtype=np.uint8)
    sc = np.full((R, H // 64), BF16_ONE, np.uint16)
    bi = np.zeros((R, H // 64), np.uint16)
    packed = pack(cfg, codes, sc, bi)
    x = rng.integers(-8, 9, size=(T, H)).astype(np.float32)
    outs = run(cfg, packed, x)
    mats = split(codes, sc, bi, rows)
    for t in range(T):
        for got, (c, _, _) in zip(outs, mats):
            want = (c.astype(np.int64) @ x[t].astype(np.int64)).astype(np.float64)
            np.testing.assert_allclose(got[t], want, rtol=2e-6, atol=1e-6 * np.abs(want).max())


def test_qkv_zero_tokens_and_bad_config():
    cfg = q.QkvConfig.make(512, 8, 8, 8)
    packed = torch.empty(q.moe_qkv_packed_bytes(cfg), dtype=torch.uint8, device="cuda")
    x = torch.zeros((1, 512), device="cuda")
    o = torch.full((1, 8), 7.0, device="cuda")
    q.moe_qkv_forward(cfg, packed, 0, x, o, o, o)
    torch.cuda.synchronize()
    assert float(o.max()) == 7.0
    with pytest.raises(q.MoeError):
        q.moe_qkv_forward(q.QkvConfig.make(512, 0, 8, 8), packed, 1, x, o, o, o)


@pytest.mark.parametrize("bits,H,rows,T,norm", [
    (4, 4096, (4096, 512, 512), 9, True),   # two full passes of four tokens and one token
    (3, 512, (200, 40, 44), 4, True),       # exactly one pass, ragged last block
    (2, 256, (64, 32, 33), 6, False),       # a full pass and a half pass
])
def test_qkv_batched_tokens(bits, H, rows, T, norm):
    """Several tokens per call (the batched kernel: four tokens per pass, a partial
    last pass) against the oracle, and every token bit-identical to a call with that
    token alone (the single-token kernel: the same encoding and reduction order)."""
    rng = np.random.default_rng(hash((bits, H, rows, T, 7)) % 2**32)
    cfg = q.QkvConfig.make(H, *rows, bits=bits, flags=q.MOE_F_RMSNORM if norm else 0)
    codes, sc, bi = canon(rng, H, rows, bits, {4: 0.02, 3: 0.04, 2: 0.06}[bits])
    packed = pack(cfg, codes, sc, bi)
    x = wl.tokens_x(int(rng.integers(1 << 30)), T, H)
    gamma = (1.0 + 0.1 * rng.normal(size=H)).astype(np.float32)
    outs = run(cfg, packed, x, gamma)
    mats = split(codes, sc, bi, rows)
    for t in range(T):
        want = ref.qkv(mats, x[t], gamma=gamma, norm=norm)
        for name, got, ref_y in zip("qkv", outs, want):
            parity(got[t], ref_y, f"{name} token {t}")
        one = run(cfg, packed, x[t:t + 1], gamma)
        for name, got, got1 in zip("qkv", outs, one):
            np.testing.assert_array_equal(got[t], got1[0], err_msg=f"{name} token {t}: batched vs one token")
