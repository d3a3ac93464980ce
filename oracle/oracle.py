"""fp64 NumPy oracle of the quantized MoE expert layer (test infrastructure only).

Sources (page title, section):
  [W]  "Who Says Elephants Can't Run: Bringing Large Scale MoE Models into Cloud Scale
       Production" review -- section 3 "core formulas" (symmetric per-channel expert
       quantization, Algorithm 1) and section 3 "workflow" (token routing by a sort keyed
       on expert index with the row index attached, permute, grouped GEMM, unpermute with
       expert_scale).
  [S]  "Specter" summary -- "Background / MoE" (router scores, top-k experts run),
       "Background / GPTQ INT4" (group size 128, router kept in fp16), "Method steps"
       step 5 (verify groups tokens by expert, computes, scatters back; equivalent).

Readings taken where the pages are silent (each is listed with its reason in the design
notes of the repository):
  * top-k order: logit descending, expert index ascending on ties; +0 == -0.
  * selection is made on the fp32 logits, not on probabilities.
  * gate weights: softmax over the k selected logits ("topk") or over all E ("all").
  * the sort payload is the flat slot f = t*k + j; ties keep ascending f.
  * Algorithm 1's scale S[e, n] is S[e, 0, n] of the (E,1,N) tensor; with 128-groups along
    K it is S[e, m // 128, n].
  * Algorithm 1's product is taken in fp16: the exact product of the integer code and the
    fp16 scale, rounded once to nearest-even fp16.
  * SwiGLU (no bias): h = silu(x Wg) * (x Wu), silu(z) = z / (1 + exp(-z)); the first GEMM's
    columns are [gate | up].
"""
import numpy as np

GATE_TOPK = "topk"
GATE_ALL = "all"


# --------------------------------------------------------------------------------------
# Routing  [S] Background / MoE: the router scores every expert, only the top-k run.
# --------------------------------------------------------------------------------------
def topk_route(logits: np.ndarray, k: int, gate_mode: str):
    """Top-k gating.  Returns ids int32 [T, k] and gate weights float64 [T, k].

    Order: logit descending, then expert index ascending.  Weights are a softmax (in fp64)
    over the k chosen logits (gate_mode "topk") or over all E logits ("all").
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    idx = np.arange(E)
    for t in range(T):
        row = logits[t].astype(np.float64)
        # lexsort sorts by the last key first: primary key -logit, secondary key index.
        order = np.lexsort((idx, -row))
        sel = order[:k]
        ids[t] = sel
        pool = row[sel] if gate_mode == GATE_TOPK else row
        m = pool.max()
        denom = np.exp(pool - m).sum()
        w[t] = np.exp(row[sel] - m) / denom
    return ids, w


# --------------------------------------------------------------------------------------
# Token routing by sort  [W] section 3 workflow: attach the row index to the gating output,
# sort with expert_idx as key, permute the activations.
# --------------------------------------------------------------------------------------
def stable_expert_sort(ids: np.ndarray, E: int):
    """Stable sort of the flat slots f = t*k + j by expert id.

    Returns perm [R] (perm[p] = slot at sorted position p), inv_perm [R]
    (inv_perm[f] = sorted position of slot f) and offsets [E+1] (rows of expert e are
    sorted positions offsets[e] .. offsets[e+1]-1).
    """
    key = np.asarray(ids, dtype=np.int64).ravel()
    R = key.size
    perm = np.argsort(key, kind="stable").astype(np.int32)
    inv_perm = np.empty(R, dtype=np.int32)
    inv_perm[perm] = np.arange(R, dtype=np.int32)
    counts = np.bincount(key, minlength=E)[:E] if R else np.zeros(E, np.int64)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return perm, inv_perm, offsets


def permute_rows(x: np.ndarray, perm: np.ndarray, k: int):
    """Row gather: x_perm[p] = x[perm[p] // k] (bit copy)."""
    return np.asarray(x)[np.asarray(perm, dtype=np.int64) // k]


# --------------------------------------------------------------------------------------
# Algorithm 1  [W] section 3: for every e, m, n: f = IntToFloat(W[e,m,n]); W_dq = f * S[e,n].
# --------------------------------------------------------------------------------------
def dequant_algorithm1(codes: np.ndarray, scales: np.ndarray, group: int):
    """fp16 dequantized weights [E, K, N].

    The code (an integer of at most 8 bits) and the fp16 scale multiply exactly in fp32;
    the cast to fp16 is the single round-to-nearest-even of the fp16 product.
    scales has shape (E, 1, N) (group == 0, per output channel) or (E, K/group, N).
    """
    codes = np.asarray(codes)
    E, K, N = codes.shape
    s = np.asarray(scales, dtype=np.float16).astype(np.float32)
    if group == 0:
        s_full = np.broadcast_to(s[:, 0:1, :], (E, K, N))
    else:
        s_full = np.repeat(s, group, axis=1)
    return (codes.astype(np.float32) * s_full).astype(np.float16)


def dense_weights(w: np.ndarray):
    """fp16 weights used as they are (shared experts); fp64 copy for the FFN."""
    return np.asarray(w, dtype=np.float16).astype(np.float64)


# --------------------------------------------------------------------------------------
# Expert FFN (fp64).
# --------------------------------------------------------------------------------------
def _silu(z):
    return z / (1.0 + np.exp(-z))


def _act(h, act: str, inter: int):
    if act == "relu":
        return np.maximum(h, 0.0)
    if act == "swiglu":
        g, u = h[:, :inter], h[:, inter:]
        return _silu(g) * u
    if act == "none":
        return h
    raise ValueError(act)


def expert_ffn(a: np.ndarray, w1_dq: np.ndarray, w2_dq: np.ndarray, act: str):
    """y = act(a @ W1) @ W2 in fp64 for the rows a [M, d] routed to one expert."""
    a64 = np.asarray(a, dtype=np.float64)
    h = a64 @ np.asarray(w1_dq, dtype=np.float64)
    inter = w2_dq.shape[0]
    h = _act(h, act, inter)
    return h @ np.asarray(w2_dq, dtype=np.float64)


def grouped_gemm(a: np.ndarray, offsets: np.ndarray, w_dq: np.ndarray, act: str,
                 row_scale=None):
    """One grouped GEMM step in fp64: rows offsets[e]..offsets[e+1]-1 of a use expert e.

    out[p] = row_scale[p] * act(a[p] @ w_dq[e]); act in {"none", "relu", "swiglu"} (for
    "swiglu" w_dq has 2I columns [gate | up] and out has I columns).
    """
    a64 = np.asarray(a, dtype=np.float64)
    E, K, N = w_dq.shape
    n_out = N // 2 if act == "swiglu" else N
    out = np.zeros((a64.shape[0], n_out), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            h = a64[lo:hi] @ np.asarray(w_dq[e], dtype=np.float64)
            out[lo:hi] = _act(h, act, n_out)
    if row_scale is not None:
        out *= np.asarray(row_scale, dtype=np.float64)[:, None]
    return out


# --------------------------------------------------------------------------------------
# Unpermute + expert_scale  [W] section 3 workflow: restore the original row order and
# apply the gate weight; the k contributions of a token are summed.
# --------------------------------------------------------------------------------------
def unpermute_combine(y_perm: np.ndarray, inv_perm: np.ndarray, k: int, w=None,
                      addend=None):
    """out[t] = sum_j w[t,j] * y_perm[inv_perm[t*k+j]] (+ addend[t]), fp64, j ascending."""
    y = np.asarray(y_perm, dtype=np.float64)
    R = inv_perm.size
    T = R // k
    d = y.shape[1]
    out = np.zeros((T, d), dtype=np.float64)
    for j in range(k):
        rows = y[np.asarray(inv_perm, dtype=np.int64).reshape(T, k)[:, j]]
        if w is not None:
            rows = rows * np.asarray(w, dtype=np.float64)[:, j:j + 1]
        out += rows
    if addend is not None:
        out += np.asarray(addend, dtype=np.float64)
    return out


def shared_ffn(x: np.ndarray, shared):
    """Sum of the always-on fp16 SwiGLU shared experts, weight 1 each (fp64)."""
    x64 = np.asarray(x, dtype=np.float64)
    out = np.zeros((x64.shape[0], shared[0][1].shape[1]), dtype=np.float64)
    for w1, w2 in shared:
        out += expert_ffn(x64, dense_weights(w1), dense_weights(w2), "swiglu")
    return out


# --------------------------------------------------------------------------------------
# The whole layer, by its plain definition (no sort, no permute):
#   out[t] = sum_j w[t,j] * FFN_{ids[t,j]}(x[t])  (+ shared experts)
# [S] Method steps, step 5: grouping tokens by expert and scattering back is equivalent to
# this per-token definition.
# --------------------------------------------------------------------------------------
def moe_layer_tokens(inp, tokens, gate_mode=None, act=None, active=None):
    """Layer output (fp64) for the token rows `tokens` only.  Each token needs only its own
    x row and logits; experts are dequantized one at a time to bound memory.

    active (bool [T] or None): batch pruning ([W] Fig. 1 caption and the list of
    optimizations: a finished sentence is left out of the computation).  A finished token
    takes no routed expert, so its row is the shared experts' output alone (0 without
    shared experts)."""
    cfg = inp.cfg
    gate_mode = gate_mode or cfg.gate_mode
    act = act or cfg.act
    tokens = np.asarray(tokens, dtype=np.int64)
    ids, w = topk_route(inp.logits[tokens], cfg.k, gate_mode)
    running = np.ones(tokens.size, dtype=bool) if active is None else \
        np.asarray(active, dtype=bool)[tokens]
    x = inp.x[tokens]
    out = np.zeros((tokens.size, cfg.d), dtype=np.float64)
    for e in np.unique(ids[running]):
        if inp.wtype == "fp16":
            # unquantized experts (the FP16 baseline of [W] section 4's quantized-vs-FP16
            # comparison): the weights are used as they are
            w1, w2 = dense_weights(inp.codes1[e]), dense_weights(inp.codes2[e])
        else:
            w1 = dequant_algorithm1(inp.codes1[e:e + 1], inp.scales1[e:e + 1], cfg.group)[0]
            w2 = dequant_algorithm1(inp.codes2[e:e + 1], inp.scales2[e:e + 1], cfg.group)[0]
        rows, slots = np.nonzero((ids == e) & running[:, None])
        y = expert_ffn(x[rows], w1, w2, act)
        out[rows] += w[rows, slots][:, None] * y
    if inp.shared:
        out += shared_ffn(x, inp.shared)
    return out


def moe_layer(inp, gate_mode=None, act=None, active=None):
    """Layer output (fp64) for all T tokens (active: batch pruning, as above)."""
    return moe_layer_tokens(inp, np.arange(inp.T), gate_mode=gate_mode, act=act, active=active)


# ---------------------------------------------------------------- expert lookahead buffer
def elb_accumulate(counts: np.ndarray, step_ids: np.ndarray, E: int) -> np.ndarray:
    """One draft step of the expert lookahead buffer ("Specter" summary, Method steps, step 2:
    ELB_cnt[j, e] = sum over draft steps i of [e in ELB_route[i, j]]).

    counts int [L, E]; step_ids int [L, T, k] = the step's routing in each of L layers (T draft
    tokens, k experts each).  Membership: an expert used by several tokens of the step counts
    once.  Ids outside [0, E) (a finished token's -1) are not routing.  Returns new counts."""
    out = np.array(counts, dtype=np.int64, copy=True)
    ids = np.asarray(step_ids)
    for j in range(ids.shape[0]):
        lay = ids[j].ravel()
        used = np.unique(lay[(lay >= 0) & (lay < E)])
        out[j, used] += 1
    return out


def elb_top_m(counts: np.ndarray, M: int):
    """The planner's snapshot ("Specter" summary, Method steps, step 3): per layer, the M experts
    with the largest counts, ties to the smaller expert index.  Returns (experts [L, M],
    their counts [L, M])."""
    counts = np.asarray(counts)
    L, E = counts.shape
    experts = np.empty((L, M), dtype=np.int64)
    for j in range(L):
        experts[j] = np.lexsort((np.arange(E), -counts[j]))[:M]
    return experts, np.take_along_axis(counts, experts, axis=1)


# ---------------------------------------------------------------- BF16 bit-field recombination
# "ZipMoE" note, key design "BF16 bit-field lossless compression": a BF16 value is split into
# its exponent bits (which are compressed) and its sign and mantissa bits (packed byte-aligned);
# recovery merges the decompressed exponents with the sign-mantissa bytes.  Reading of the
# byte layout: one exponent byte per value (the 8 exponent bits), and one sign-mantissa byte
# per value holding the sign in bit 7 and the 7 mantissa bits in bits 6..0 (the BF16 bit order
# with the exponent field taken out).
def bf16_decompose(bits: np.ndarray):
    """BF16 bit patterns (uint16) -> (exponent bytes, sign-mantissa bytes), both uint8."""
    v = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    exponent = (v >> 7) & 0xFF
    sign_mantissa = ((v >> 8) & 0x80) | (v & 0x7F)
    return exponent.astype(np.uint8), sign_mantissa.astype(np.uint8)


def bf16_recombine(exponent: np.ndarray, sign_mantissa: np.ndarray) -> np.ndarray:
    """(exponent bytes, sign-mantissa bytes) -> BF16 bit patterns (uint16)."""
    e = np.asarray(exponent, dtype=np.uint8).astype(np.uint32)
    sm = np.asarray(sign_mantissa, dtype=np.uint8).astype(np.uint32)
    return (((sm & 0x80) << 8) | (e << 7) | (sm & 0x7F)).astype(np.uint16)
