"""Pure-Python brute force of the MoE layer for tiny inputs (test helper; pins the oracle).

Written independently of oracle/: Python floats (IEEE binary64), explicit loops, an fp16
rounding routine written from the IEEE 754 binary16 definition, and top-k by enumerating
every k-subset.
"""
import itertools
import math


def fp16_round(v: float) -> float:
    """Round a binary64 value to the nearest binary16 value, ties to even."""
    if v != v:
        return v
    if v == 0.0:
        return v
    sign = -1.0 if v < 0 else 1.0
    a = abs(v)
    if a >= 65520.0:            # halfway between 65504 and 2^16 rounds up to infinity
        return sign * math.inf
    m, ex = math.frexp(a)      # a = m * 2^ex, 0.5 <= m < 1  ->  a = (2m) * 2^(ex-1)
    E = ex - 1
    spacing = 2.0 ** (E - 10) if E >= -14 else 2.0 ** -24
    q = a / spacing            # exact: division by a power of two
    r = round(q)               # Python rounds exact halves to even
    return sign * r * spacing


def _beats(la, ea, lb, eb):
    """Expert a comes before expert b: larger logit, or equal logit and smaller index."""
    return la > lb or (la == lb and ea < eb)


def brute_topk(row, k):
    E = len(row)
    best = None
    for S in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in S]
        if all(_beats(row[a], a, row[b], b) for a in S for b in rest):
            best = S
            break
    # order the chosen set by the same total order (selection sort, no library sort)
    chosen = list(best)
    ordered = []
    while chosen:
        top = chosen[0]
        for e in chosen[1:]:
            if _beats(row[e], e, row[top], top):
                top = e
        ordered.append(top)
        chosen.remove(top)
    return ordered


def brute_gate_weights(row, ids, gate_mode):
    pool = [row[e] for e in ids] if gate_mode == "topk" else list(row)
    m = max(pool)
    denom = 0.0
    for v in pool:
        denom += math.exp(v - m)
    return [math.exp(row[e] - m) / denom for e in ids]


def brute_dequant(codes, scales, group):
    """codes: nested lists [K][N] ints; scales: [G][N] floats (fp16 values) -> [K][N]."""
    K, N = len(codes), len(codes[0])
    return [[fp16_round(codes[m][n] * scales[0 if group == 0 else m // group][n])
             for n in range(N)] for m in range(K)]


def _silu(z):
    return z / (1.0 + math.exp(-z))


def brute_ffn(a, w1, w2, act):
    d, N1 = len(w1), len(w1[0])
    h = [sum(a[i] * w1[i][n] for i in range(d)) for n in range(N1)]
    if act == "relu":
        h = [v if v > 0 else 0.0 for v in h]
    else:
        inter = N1 // 2
        h = [_silu(h[n]) * h[inter + n] for n in range(inter)]
    dout = len(w2[0])
    return [sum(h[i] * w2[i][c] for i in range(len(h))) for c in range(dout)]


def brute_layer(x, logits, codes1, scales1, codes2, scales2, group, k, gate_mode, act,
                shared=(), active=None):
    """All arguments are nested Python lists of Python numbers.  active: list of 0/1 per
    token or None; a finished token (0) takes no routed expert."""
    T = len(x)
    cache = {}
    out = []
    for t in range(T):
        ids = brute_topk(logits[t], k) if active is None or active[t] else []
        w = brute_gate_weights(logits[t], ids, gate_mode) if ids else []
        acc = [0.0] * len(x[t])
        for e, we in zip(ids, w):
            if e not in cache:
                cache[e] = (brute_dequant(codes1[e], scales1[e], group),
                            brute_dequant(codes2[e], scales2[e], group))
            y = brute_ffn(x[t], cache[e][0], cache[e][1], act)
            acc = [acc[c] + we * y[c] for c in range(len(acc))]
        for w1, w2 in shared:
            y = brute_ffn(x[t], w1, w2, "swiglu")
            acc = [acc[c] + y[c] for c in range(len(acc))]
        out.append(acc)
    return out
