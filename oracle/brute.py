"""Independent pure-Python MoE decode layer, stack and prefill token for tiny shapes
(a pin for the oracle).

TEST INFRASTRUCTURE ONLY. Lists and loops, no numpy and no shared code with
``oracle/ref.py`` or ``qmoe_oracle.c``. Written from the same definitions
(flash-moe page, vi.news.hada.io: "Kiến trúc mô hình", "Kernel dequant tối ưu
FMA", "Metal Compute Shaders", "Deferred GPU Expert Compute"): w = q*scale + bias
per 64-group, SwiGLU expert, softmax top-K renormalised, weighted combine plus
shared expert plus residual, and the layer output feeding the next layer.
Exact rationals are not needed: float64 arithmetic in a different summation
structure (full sort instead of K argmax passes, dequantised matrices built
first, math.fsum instead of running sums) is the independent check.

Beyond one layer it covers:
  * RMSNorm with a per-element weight gamma;
  * the temporal tier: boosted experts are ranked ahead of every other expert,
    then score, then lower index (the 27% repeat of "Autoresearch impulsa a
    Qwen3.5-397B ...", section "Optimizaciones Efectivas", read as a selection
    tier);
  * the L-layer stack: layer l + 1 takes layer l's output, and at token t the
    boosted experts of layer l are the marked slots of token t-1's set there
    (sorted by expert index);
  * the prefill rounding points (the input, the expert input, every dequantised
    weight and the SwiGLU output rounded to bf16; the router sees the unrounded
    normalised input), with its own bf16 rounding on the IEEE double bit pattern.
"""
import math
import struct


def _bf16(bits):
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _f32(v):
    return struct.unpack("<f", struct.pack("<f", v))[0]


def bf16_round(v):
    """Round a float64 to 8 significant bits, ties to even, on its IEEE-754 bit
    pattern: the 45 low mantissa bits are dropped with round-half-even (a carry
    into the exponent is the correct rounding up to the next binade)."""
    if v == 0.0 or v != v or v in (float("inf"), float("-inf")):
        return v
    u = struct.unpack("<Q", struct.pack("<d", v))[0]
    keep = (u >> 45) & 1
    u = ((u + (1 << 44) - 1 + keep) >> 45) << 45
    return struct.unpack("<d", struct.pack("<Q", u))[0]


def dequant(codes, scales, biases, to_bf16=False):
    """codes: list of rows; scales/biases: list of rows of bf16 bit patterns."""
    out = []
    for r, row in enumerate(codes):
        vals = [_f32(_f32(float(q) * _bf16(scales[r][c // 64])) + _bf16(biases[r][c // 64]))
                for c, q in enumerate(row)]
        out.append([bf16_round(v) for v in vals] if to_bf16 else vals)
    return out


def _mv(W, x):
    return [math.fsum(w * v for w, v in zip(row, x)) for row in W]


def _select(logits, K, boosted=(), sel=None, by_sel=False):
    """Full sort by (tier desc, score desc, index asc); weights from the plain logits."""
    E = len(logits)
    tier = [1 if e in set(boosted) else 0 for e in range(E)]
    if sel is None:
        score = list(logits)
    elif by_sel:
        score = list(sel)
    else:
        score = [a + b for a, b in zip(logits, sel)]
    order = sorted(range(E), key=lambda e: (-tier[e], -score[e], e))
    idx = order[:K]
    m = max(logits)
    ex = [math.exp(l - m) for l in logits]
    z = math.fsum(ex)
    p = [v / z for v in ex]
    ps = math.fsum(p[i] for i in idx)
    return idx, [p[i] / ps for i in idx]


def layer(x, router_rows, experts, shared, K, rmsnorm=True, residual=True, eps=1e-6, shared_gate=None,
          gamma=None, boosted=(), sel=None, by_sel=False, bf16_points=False):
    """experts/shared: lists of (codes[3], scales[3], biases[3]) as nested lists.
    shared_gate: one row per shared expert (its output scaled by 1/(1+e^-(row.x_n))) or None.
    gamma: per-element RMSNorm weight (None: all ones).
    bf16_points: the prefill rounding points (see the module docstring): True for all
    of them, or a subset of {"x", "a", "w", "h"} (input, expert input, weights, SwiGLU
    output), which lets a test show that each point changes the result."""
    H = len(x)
    pts = {"x", "a", "w", "h"} if bf16_points is True else set(bf16_points or ())
    x = [float(v) for v in x]
    if "x" in pts:
        x = [bf16_round(_f32(v)) for v in x]
    if rmsnorm:
        r = math.sqrt(math.fsum(v * v for v in x) / H + eps)
        xn = [v / r for v in x]
        if gamma is not None:
            xn = [v * float(g) for v, g in zip(xn, gamma)]
    else:
        xn = list(x)
    logits = [math.fsum(w * v for w, v in zip(row, xn)) for row in router_rows]
    idx, w = _select(logits, K, boosted, sel, by_sel)
    a = [bf16_round(v) for v in xn] if "a" in pts else xn

    def run(ex_):
        cs, ss, bs = ex_
        G, U, D = (dequant(cs[m], ss[m], bs[m], to_bf16="w" in pts) for m in range(3))
        g, u = _mv(G, a), _mv(U, a)
        h = [gj / (1.0 + math.exp(-gj)) * uj for gj, uj in zip(g, u)]
        if "h" in pts:
            h = [bf16_round(v) for v in h]
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


def stack(xs, layers, K, boost=None, rmsnorm=True, residual=True, eps=1e-6):
    """Tokens in order; each token through every layer, layer l's output being layer
    l + 1's input (the rest of the model is the identity).
    layers: list of dicts with keys router, experts, shared and optionally gamma.
    boost[t][l][j]: boost slot j of token t-1's set at layer l (sorted by index).
    Returns (outputs per token, selected sets per token and layer, sorted)."""
    ys, sets = [], []
    prev = None
    for t, x in enumerate(xs):
        cur = list(x)
        tsets = []
        for l, ly in enumerate(layers):
            boosted = ()
            if boost is not None and prev is not None:
                ps = sorted(prev[l])
                boosted = tuple(ps[j] for j in range(K) if boost[t][l][j])
            cur, idx, _ = layer(cur, ly["router"], ly["experts"], ly["shared"], K, rmsnorm=rmsnorm,
                                residual=residual, eps=eps, gamma=ly.get("gamma"), boosted=boosted)
            tsets.append(sorted(idx))
        ys.append(cur)
        sets.append(tsets)
        prev = tsets
    return ys, sets
