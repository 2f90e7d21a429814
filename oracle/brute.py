"""Independent pure-Python MoE decode layer for tiny shapes (a pin for the oracle).

TEST INFRASTRUCTURE ONLY. Lists and loops, no numpy and no shared code with
``oracle/ref.py`` or ``qmoe_oracle.c``. Written from the same definitions
(flash-moe page, vi.news.hada.io: "Kiến trúc mô hình", "Kernel dequant tối ưu
FMA", "Metal Compute Shaders"): w = q*scale + bias per 64-group, SwiGLU expert,
softmax top-K renormalised, weighted combine plus shared expert plus residual.
Exact rationals are not needed: float64 arithmetic in a different summation
structure (full sort instead of K argmax passes, dequantised matrices built
first) is the independent check.
"""
import math
import struct


def _bf16(bits):
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _f32(v):
    return struct.unpack("<f", struct.pack("<f", v))[0]


def dequant(codes, scales, biases):
    """codes: list of rows; scales/biases: list of rows of bf16 bit patterns."""
    out = []
    for r, row in enumerate(codes):
        out.append([_f32(_f32(float(q) * _bf16(scales[r][c // 64])) + _bf16(biases[r][c // 64]))
                    for c, q in enumerate(row)])
    return out


def _mv(W, x):
    return [math.fsum(w * v for w, v in zip(row, x)) for row in W]


def layer(x, router_rows, experts, shared, K, rmsnorm=True, residual=True, eps=1e-6, shared_gate=None):
    """experts/shared: lists of (codes[3], scales[3], biases[3]) as nested lists.
    shared_gate: one row per shared expert (its output scaled by 1/(1+e^-(row.x_n))) or None."""
    H = len(x)
    if rmsnorm:
        r = math.sqrt(math.fsum(v * v for v in x) / H + eps)
        xn = [v / r for v in x]
    else:
        xn = list(x)
    logits = [math.fsum(w * v for w, v in zip(row, xn)) for row in router_rows]
    order = sorted(range(len(logits)), key=lambda e: (-logits[e], e))
    idx = order[:K]
    m = max(logits)
    ex = [math.exp(l - m) for l in logits]
    z = math.fsum(ex)
    p = [v / z for v in ex]
    ps = math.fsum(p[i] for i in idx)
    w = [p[i] / ps for i in idx]

    def run(ex_):
        cs, ss, bs = ex_
        G, U, D = (dequant(cs[m], ss[m], bs[m]) for m in range(3))
        g, u = _mv(G, xn), _mv(U, xn)
        h = [gj / (1.0 + math.exp(-gj)) * uj for gj, uj in zip(g, u)]
        return _mv(D, h)

    outs = [run(experts[i]) for i in idx]
    sh = [run(s) for s in shared]
    if shared_gate is not None:
        for j, row in enumerate(shared_gate):
            c = 1.0 / (1.0 + math.exp(-math.fsum(g * v for g, v in zip(row, xn))))
            sh[j] = [c * v for v in sh[j]]
    y = []
    for i in range(H):
        terms = ([x[i]] if residual else []) + [w[k] * outs[k][i] for k in range(K)] + [o[i] for o in sh]
        y.append(math.fsum(terms))
    return y, idx, w
