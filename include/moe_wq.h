/*
 * moe_wq.h -- C ABI of the weight-only-quantized MoE expert layer for AMD MI355X (gfx950).
 *
 * The layer, for T tokens of hidden size d, E routed experts and k experts per token:
 *   1. moe_route_topk        top-k gating over fp32 router logits
 *   2. moe_permute           stable sort of the T*k routed rows by expert + row gather
 *   3. moe_grouped_gemm_wq   grouped GEMM over all active experts, int4/int8 codes
 *                            dequantized in registers, fused activation / gate weight
 *   4. moe_unpermute_combine restore token order, scale by gate weight, sum the k rows
 *   and moe_dequant          the standalone per-expert dequantization (Algorithm 1);
 *   moe_decode_layer         steps 1-4 for the few tokens of a decode / verify step, in three
 *                            launches (moe_decode_layer_shared: with the shared experts in
 *                            the same launches; moe_decode_layer_noalloc: on the library's
 *                            own scratch memory, for callers that cannot allocate)
 *   moe_elb_accumulate / moe_elb_top_m   the expert lookahead buffer of a speculative draft
 *   moe_bf16_recombine       BF16 values from separately stored exponent / sign-mantissa bytes
 *
 * Sources (page, section):
 *   [W] "Who Says Elephants Can't Run: Bringing Large Scale MoE Models into Cloud Scale
 *       Production" review, section 3: symmetric per-channel expert quantization with
 *       scales of shape (E,1,N); Algorithm 1 (dequantization); optimized int-to-float
 *       conversion (exponent of 1024; 8-bit and 4-bit variants); workflow (sort keyed on
 *       expert index with the row index attached, permute, grouped GEMM, unpermute with
 *       expert_scale); section 4: fused GEMM + dequantization.
 *   [S] "Specter" summary: Background / MoE (top-k routing), Background / GPTQ INT4
 *       (symmetric, group size 128), Method steps, step 5 (tokens grouped by expert into
 *       one GEMM per expert, then scattered back).
 *   [Z] "ZipMoE" note: key design, BF16 bit-field lossless compression.
 *
 * Conventions for every call:
 *   - Pointers are device pointers owned by the caller unless marked [host].  fp16 values
 *     travel as uint16_t bit patterns.  Tensors are dense row-major.
 *   - Calls never allocate device memory and never synchronize: work is enqueued on
 *     `stream` (a hipStream_t passed as void*; NULL = the default stream).
 *   - Arguments are validated on the host before anything is enqueued.  On any error
 *     nothing is enqueued and outputs are untouched.
 *   - T == 0 (or R == 0) returns MOE_OK and enqueues nothing.
 *   - Pointers must be 16-byte aligned.
 *   - Apart from the scratch array of moe_decode_layer_noalloc, the library keeps no mutable
 *     global state; the other calls are thread-safe.  Results are deterministic: two
 *     identical calls give identical bits.
 */
#ifndef MOE_WQ_H
#define MOE_WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define MOE_OK               0
#define MOE_ERR_INVALID     -1   /* bad argument: null pointer, bad size, misaligned, ... */
#define MOE_ERR_UNSUPPORTED -2   /* valid but outside what this library implements */
#define MOE_ERR_WORKSPACE   -3   /* workspace missing or too small */
#define MOE_ERR_NO_DEVICE   -4   /* no usable gfx950 device */
#define MOE_ERR_HIP         -5   /* a HIP runtime call failed */

/* ---- enumerations ---- */
enum moe_gate  { MOE_GATE_SOFTMAX_TOPK = 0,   /* softmax over the k chosen logits        */
                 MOE_GATE_SOFTMAX_ALL  = 1 }; /* softmax over all E, then keep the top k */
enum moe_wtype { MOE_W_INT4 = 0, MOE_W_INT8 = 1, MOE_W_FP16 = 2 };
enum moe_act   { MOE_ACT_NONE = 0, MOE_ACT_RELU = 1, MOE_ACT_SWIGLU = 2 };
enum moe_path  { MOE_PATH_AUTO = 0,           /* chosen from R, E, K, N                  */
                 MOE_PATH_STREAM = 1,         /* weight-streaming path, 16-row tiles     */
                 MOE_PATH_TILE = 2 };         /* LDS-staged MFMA tile path, 48/64-row tiles */

/* Optional per-call GEMM settings.  Pass NULL for the defaults (all fields 0). */
enum moe_tile  { MOE_TILE_AUTO = 0,           /* chosen from R, E, K, N                  */
                 MOE_TILE_64x256 = 1,         /* tile path: 64 rows x 256 weight columns */
                 MOE_TILE_64x128 = 2,         /*            64 rows x 128 weight columns */
                 MOE_TILE_128x128 = 3,        /*           128 rows x 128 weight columns */
                 MOE_TILE_48x256 = 4,         /*            48 rows x 256 weight columns */
                 MOE_TILE_48x128 = 5 };       /*            48 rows x 128 weight columns */

typedef struct moe_gemm_opts {
    int32_t path;      /* enum moe_path                                              */
    int32_t split_k;   /* 0 = automatic; 1..MOE_MAX_SPLIT_K forces the number of  */
                       /* waves that split K per stream-path block (the tile path  */
                       /* ignores it)                                              */
    int32_t tile;      /* enum moe_tile: block tile of the tile path (automatic:   */
                       /* 48-row tiles for per-channel scales and for experts with */
                       /* under ~96 rows, 64x256 for group scales beyond that,     */
                       /* 128-column tiles for 8-bit codes)                        */
    int32_t i2f;       /* enum moe_i2f: how codes become fp16 in the tile path      */
    int32_t reserved[4];
} moe_gemm_opts;

/* Int-to-float conversion of the codes inside the GEMM ([W] section 3, optimized I2F).  Both give
 * the same fp16 values, so the same results bit for bit; NATIVE is the baseline the exponent-of-
 * 1024 construction is measured against.  NATIVE is built for the tile path with per-channel
 * scales, ReLU or no activation (the MT encoder's two GEMMs), 4- or 8-bit codes and the 48x256,
 * 48x128, 64x128 and 64x256 tiles; other calls that ask for it get MOE_ERR_UNSUPPORTED. */
enum moe_i2f   { MOE_I2F_TRICK = 0,           /* OR into the mantissa of 1024, subtract    */
                 MOE_I2F_NATIVE = 1 };        /* byte-to-float conversion instructions     */

/* Limits. */
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK      8
#define MOE_MAX_SPLIT_K   8
#define MOE_DECODE_MAX_TOKENS 64    /* moe_decode_layer: T <= 64 ...      */
#define MOE_DECODE_MAX_ROWS  512    /*                   ... and T*k <= 512 */

/*
 * moe_route_topk -- top-k gating.   [S] Background / MoE: the router scores every expert
 * and only the k best-scoring experts run for a token.
 *
 *   logits    fp32 [T, E]   router logits (finite values; NaN gives an unspecified order)
 *   topk_ids  int32 [T, k]  out: chosen experts, ordered by logit descending, ties broken
 *                           by the smaller expert index (+0 and -0 compare equal)
 *   topk_w    fp32 [T, k]   out: gate weights.  MOE_GATE_SOFTMAX_TOPK: softmax over the k
 *                           chosen logits (renormalised).  MOE_GATE_SOFTMAX_ALL: softmax
 *                           over all E logits, then the k chosen entries (no renorm).
 *   Selection is made on the fp32 logits themselves, so indices are exact.
 *   Requires 1 <= E <= 256, 1 <= k <= min(E, 8), T >= 0.
 */
int32_t moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t gate_mode,
                       int32_t* topk_ids, float* topk_w, void* stream);

/*
 * moe_route_topk_active -- moe_route_topk with batch pruning.  [W] Fig. 1 and its list of
 * optimizations: with batch pruning, finished sentences are removed from the computation, so
 * experts that only they would use load no weights.
 *
 *   active    uint8 [T] or NULL (= all active): a token with active[t] == 0 is finished; its k
 *             slots get topk_ids -1 and topk_w 0.  moe_permute drops such slots (no rows, so an
 *             expert with only finished tokens reads no weights), and moe_unpermute_combine
 *             then writes the token's row as fp16(addend[t]) (0 without an addend).
 *   Everything else as moe_route_topk, which is this call with active = NULL.
 */
int32_t moe_route_topk_active(const float* logits, const uint8_t* active, int32_t T, int32_t E,
                              int32_t k, int32_t gate_mode, int32_t* topk_ids, float* topk_w,
                              void* stream);

/*
 * moe_permute -- stable counting sort of routed rows by expert, then row gather.
 *   [W] section 3 workflow: the row index is attached to the gating output, the tuples are
 *   sorted with the expert index as key, and the activation matrix is permuted.
 *
 *   topk_ids        int32 [T, k]  expert of flat slot f = t*k + j (values in [0, E))
 *   topk_w          fp32  [T, k]  gate weights, or NULL (then w_perm must be NULL)
 *   x               fp16  [T, d]  token activations (may be NULL when x_perm is NULL)
 *   perm            int32 [T*k]   out: perm[p] = flat slot at sorted position p; slots of one
 *                                 expert keep ascending f (stable)
 *   inv_perm        int32 [T*k]   out: inv_perm[f] = sorted position of slot f
 *   expert_offsets  int32 [E+1]   out: rows of expert e are positions offsets[e]..offsets[e+1]-1
 *   x_perm          fp16  [T*k, d] out: x_perm[p] = x[perm[p] / k] (bit copy), or NULL to
 *                                 skip the copy (moe_grouped_gemm_wq_rows then reads x
 *                                 through perm itself)
 *   w_perm          fp32  [T*k]   out (optional): w_perm[p] = topk_w.flat[perm[p]]
 *   ws, ws_bytes    workspace of at least moe_permute_workspace_size(T, k, E) bytes: 0 up
 *                   to 8192 slots (NULL allowed), else 4 * E * ceil(T*k / 1024) (per-block
 *                   expert counts of the two-launch sort); MOE_ERR_WORKSPACE if short
 *   Requires 1 <= E <= 256, 1 <= k <= 8, d % 8 == 0.  A slot whose id is outside [0, E)
 *   (-1 from moe_route_topk_active for a finished token) is not routed: it gets no sorted
 *   position (inv_perm -1), and offsets[E] = the number of routed slots < T*k; the positions
 *   from offsets[E] on hold perm -1 (and w_perm 0).
 */
int32_t moe_permute(const int32_t* topk_ids, const float* topk_w, const uint16_t* x,
                    int32_t T, int32_t k, int32_t E, int32_t d,
                    int32_t* perm, int32_t* inv_perm, int32_t* expert_offsets,
                    uint16_t* x_perm, float* w_perm,
                    void* ws, size_t ws_bytes, void* stream);
size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t E);

/*
 * moe_grouped_gemm_wq -- grouped GEMM over all experts with in-register dequantization.
 *   [W] section 3 Fig. 1 / workflow (one sub-matrix per expert, all experts in one grouped
 *   GEMM), section 4 (dequantization fused into the GEMM), section 3 optimized I2F; the
 *   dequantized weight is W_dq[e,m,n] = code * S[e, g(m), n] (Algorithm 1).
 *
 *   a               fp16 [R, K]  rows sorted by expert (x_perm, or the first GEMM's output)
 *   expert_offsets  int32 [E+1]  rows of expert e are a[offsets[e] .. offsets[e+1]-1];
 *                                offsets[0] == 0, non-decreasing, offsets[E] <= R.
 *                                Experts with no rows read no weights.
 *   w_packed        weights packed by moe_pack_wq for (wtype, E, K, N)
 *   scales          fp16 [E, G, N], G = 1 (group_size 0: one scale per output channel,
 *                   shape (E,1,N)) or K/128 (group_size 128: groups along K).  NULL for
 *                   MOE_W_FP16.
 *   act             MOE_ACT_NONE / RELU: out = act(a W_dq) [R, N].
 *                   MOE_ACT_SWIGLU: W columns are [gate | up] (N = 2I); out [R, I] =
 *                   silu(a W_gate) * (a W_up), silu(z) = z / (1 + exp(-z)).
 *   row_scale       fp32 [R] or NULL: each output row is multiplied by row_scale[p]
 *                   (the gate weight, w_perm) after the activation.
 *   out             fp16 [R, N or N/2]; rows at or beyond offsets[E] are not written.
 *   opts            [host] NULL or settings (path, split).
 *   ws, ws_bytes    workspace of at least moe_gemm_workspace_size(...) bytes (currently
 *                   0 for every argument set: NULL / 0 may be passed).
 *   Accumulation is fp32, the result is rounded once to fp16 (nearest even).
 *   Requires K % 128 == 0, N % 16 == 0 (N % 32 for SWIGLU), E <= 256, group_size in
 *   {0, 128} (0 only for FP16 weights).
 */
int32_t moe_grouped_gemm_wq(const uint16_t* a, const int32_t* expert_offsets,
                            int32_t R, int32_t E, int32_t K, int32_t N,
                            const void* w_packed, const uint16_t* scales,
                            int32_t wtype, int32_t group_size, int32_t act,
                            const float* row_scale, uint16_t* out,
                            const moe_gemm_opts* opts, void* ws, size_t ws_bytes,
                            void* stream);
size_t moe_gemm_workspace_size(int32_t R, int32_t E, int32_t K, int32_t N, int32_t wtype,
                               int32_t act, const moe_gemm_opts* opts);

/*
 * moe_grouped_gemm_wq_rows -- moe_grouped_gemm_wq with the permute and the unpermute of
 * [W] section 3's workflow folded into its loads and stores: GEMM row p (sorted position p,
 * the rows of expert e being offsets[e] .. offsets[e+1]-1 as above) reads activation row
 *     a[a_rows[p] / a_row_div]      (a[p] when a_rows is NULL)
 * and writes output row
 *     out[out_rows[p]]              (out[p] when out_rows is NULL).
 * With a = x, a_rows = perm and a_row_div = k this is the first GEMM without x_perm; with
 * k = 1, out = the layer output and out_rows = perm it is the second GEMM plus the
 * unpermute (the gate weight goes in row_scale, indexed by p).  Everything else -- weights,
 * scales, act, row_scale, opts, workspace, numerics -- is as for moe_grouped_gemm_wq.
 *
 *   a_nrows      rows of a when a_rows is given (source rows are clamped into [0, a_nrows);
 *                in-range a_rows are the caller's duty, a clamped row gives a wrong but
 *                harmless result)
 *   a_rows       int32 [R] or NULL;  a_row_div >= 1
 *   out_nrows    rows of out when out_rows is given; a destination outside [0, out_nrows) is
 *                not written.  Destinations must be distinct (rows are written, not added).
 *   out_rows     int32 [R] or NULL
 * Errors: as moe_grouped_gemm_wq, plus MOE_ERR_INVALID for a_row_div < 1, negative row
 * counts or misaligned (non-4-byte) row maps.
 */
int32_t moe_grouped_gemm_wq_rows(const uint16_t* a, int32_t a_nrows, const int32_t* a_rows,
                                 int32_t a_row_div, const int32_t* expert_offsets, int32_t R,
                                 int32_t E, int32_t K, int32_t N, const void* w_packed,
                                 const uint16_t* scales, int32_t wtype, int32_t group_size,
                                 int32_t act, const float* row_scale, uint16_t* out,
                                 int32_t out_nrows, const int32_t* out_rows,
                                 const moe_gemm_opts* opts, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * moe_decode_layer -- the whole routed layer for the few tokens of a decode or verify step:
 * gating, sort, both grouped GEMMs, gate weight, unpermute and combine, in three launches.
 *   [S] Method steps, step 5 and Technical novelty: the draft's expert sub-computations in
 *   one fused launch; the verify step groups tokens by expert into one GEMM per expert and
 *   scatters the results back.  [W] section 3 workflow and Algorithm 1 as for the calls above.
 *
 *   logits    fp32 [T, E]      router logits;  x fp16 [T, d]  token activations
 *   active    uint8 [T] or NULL: batch pruning as for moe_route_topk_active (a finished token
 *             takes no expert, its output row is fp16(addend[t]) or 0)
 *   gate_mode enum moe_gate;   act: MOE_ACT_NONE / RELU (W1 is [d, inter]) or SWIGLU (W1 is
 *             [d, 2*inter], columns [gate | up])
 *   w1, s1    first-GEMM weights packed by moe_pack_wq for (wtype, E, d, inter or 2*inter) and
 *             their scales (NULL for MOE_W_FP16), as for moe_grouped_gemm_wq
 *   w2, s2    second-GEMM weights for (wtype, E, inter, d) and scales
 *   addend    fp16 [T, d] or NULL: added with weight 1 (e.g. shared experts)
 *   addend_ready  hipEvent_t (as void*) or NULL: the call makes `stream` wait for this event
 *             just before its last launch, the first to read addend, so the caller may compute
 *             the addend on another stream while the gating, sort and first GEMM run
 *   topk_ids, topk_w  int32 / fp32 [T, k]  out: exactly what moe_route_topk returns
 *   out       fp16 [T, d]  out: out[t] = fp16( sum_j topk_w[t,j] * FFN_{topk_ids[t,j]}(x[t])
 *             + addend[t] ).  The hidden activations are rounded to fp16 as in
 *             moe_grouped_gemm_wq; the k expert outputs are summed in fp32 without the fp16
 *             rounding of each one, in an order fixed by the routing (deterministic), so out
 *             agrees with the five-call sequence within rounding, not bit for bit.
 *   ws        workspace of at least moe_decode_workspace_size(...) bytes; contents on entry
 *             do not matter, and calls that share one workspace must not overlap in time.
 * Errors: MOE_ERR_UNSUPPORTED for T > MOE_DECODE_MAX_TOKENS, T*k > MOE_DECODE_MAX_ROWS,
 * d % 128 != 0 or inter % 128 != 0, group_size not in {0, 128} (0 for FP16); otherwise as
 * moe_route_topk and moe_grouped_gemm_wq; MOE_ERR_WORKSPACE for a missing or short workspace.
 */
int32_t moe_decode_layer(const float* logits, const uint8_t* active, const uint16_t* x,
                         int32_t T, int32_t E, int32_t k, int32_t gate_mode, int32_t d,
                         int32_t inter, int32_t act,
                         const void* w1, const uint16_t* s1, const void* w2,
                         const uint16_t* s2, int32_t wtype, int32_t group_size,
                         const uint16_t* addend, void* addend_ready, int32_t* topk_ids,
                         float* topk_w, uint16_t* out, void* ws, size_t ws_bytes,
                         void* stream);
/* Workspace bytes of moe_decode_layer (0 for arguments it does not accept). */
size_t moe_decode_workspace_size(int32_t T, int32_t k, int32_t E, int32_t d, int32_t inter,
                                 int32_t wtype);

/*
 * moe_decode_layer_shared -- moe_decode_layer for a layer with shared experts (every token
 * passes through them with weight 1 beside its k routed experts), computed inside the same
 * launches: the shared first GEMM runs as extra blocks of the routed first-GEMM launch (as a
 * launch of its own when T*k > 128), the shared second GEMM as extra blocks of the
 * second-GEMM launch, and the final reduction adds its output.
 *   [S] Core method (the router and the shared experts stay fp16 in the quantized copy) and
 *   Method step 5, as for moe_decode_layer.
 *
 *   shared_w1     fp16 weights packed by moe_pack_wq for (MOE_W_FP16, 1, d, 2*shared_inter),
 *                 columns [gate | up] of all shared experts side by side (SwiGLU)
 *   shared_w2     fp16 weights packed for (MOE_W_FP16, 1, shared_inter, d)
 *   shared_inter  the shared experts' combined intermediate size
 *   out           fp16 [T, d]  out: out[t] = fp16( sum_j topk_w[t,j] * FFN_{topk_ids[t,j]}(x[t])
 *                 + fp16(SwiGLU-FFN_shared(x[t])) ): the shared output is rounded to fp16
 *                 once, as moe_grouped_gemm_wq writes it, then added in fp32.  A finished
 *                 token (active[t] == 0) still receives the shared output.
 *   The other arguments, the numerics of the routed part and the errors are those of
 *   moe_decode_layer (no addend: the shared output takes its place), plus MOE_ERR_INVALID for
 *   shared_inter <= 0 or a NULL shared weight, MOE_ERR_UNSUPPORTED for fp16 routed weights or
 *   shared_inter % 128 != 0.  ws: at least moe_decode_shared_workspace_size(...) bytes.
 */
int32_t moe_decode_layer_shared(const float* logits, const uint8_t* active, const uint16_t* x,
                                int32_t T, int32_t E, int32_t k, int32_t gate_mode, int32_t d,
                                int32_t inter, int32_t act, const void* w1, const uint16_t* s1,
                                const void* w2, const uint16_t* s2, int32_t wtype,
                                int32_t group_size, const void* shared_w1,
                                const void* shared_w2, int32_t shared_inter, int32_t* topk_ids,
                                float* topk_w, uint16_t* out, void* ws, size_t ws_bytes,
                                void* stream);
/* Workspace bytes of moe_decode_layer_shared (0 for arguments it does not accept). */
size_t moe_decode_shared_workspace_size(int32_t T, int32_t k, int32_t E, int32_t d,
                                        int32_t inter, int32_t wtype, int32_t shared_inter);

/*
 * moe_decode_layer_noalloc -- moe_decode_layer without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is the library's own scratch array of
 * MOE_DECODE_SCRATCH_BYTES bytes in device memory: each device the library runs on holds one
 * copy, from the library's load until the process ends.  The call allocates and frees
 * nothing.  Every call on a device uses that device's one array, so calls that overlap in time
 * on one device (different streams or threads) race and give undefined results; serialise
 * them.  Nothing in the array needs to start at any value: every part of the workspace is
 * written before it is read within a call (the previous call's contents are left behind).
 *   Arguments, outputs, numerics and errors are those of moe_decode_layer (without ws and
 *   ws_bytes), plus MOE_ERR_UNSUPPORTED for a step whose workspace,
 *   moe_decode_workspace_size(T, k, E, d, inter, wtype), exceeds MOE_DECODE_SCRATCH_BYTES, and
 *   MOE_ERR_HIP if the array's device address cannot be obtained.
 */
#define MOE_DECODE_SCRATCH_BYTES (8u << 20)
int32_t moe_decode_layer_noalloc(const float* logits, const uint8_t* active, const uint16_t* x,
                                 int32_t T, int32_t E, int32_t k, int32_t gate_mode, int32_t d,
                                 int32_t inter, int32_t act,
                                 const void* w1, const uint16_t* s1, const void* w2,
                                 const uint16_t* s2, int32_t wtype, int32_t group_size,
                                 const uint16_t* addend, void* addend_ready, int32_t* topk_ids,
                                 float* topk_w, uint16_t* out, void* stream);

/*
 * Attainable-peak probes (measurement aids, not part of the layer): what plain code reaches on
 * this device, timed by the caller beside the layer's kernels.
 *
 * moe_probe_read  -- reads `bytes` (a multiple of 16) at src once, grid-stride, four 16-byte
 *                    non-temporal loads in flight per thread, `blocks` blocks of 256 threads;
 *                    sink[b] (uint32 [blocks]) = XOR of the 32-bit words block b read.
 * moe_probe_mfma  -- `blocks` blocks of 4 waves, each wave `iters` x 16 independent
 *                    v_mfma_f32_16x16x32_f16 on all-ones operands (16384 flop each);
 *                    out[thread] (fp32 [blocks * 256]) = 512 * iters exactly.  iters < 32768.
 * Errors: MOE_ERR_INVALID for blocks < 1, a misaligned pointer or an out-of-range size.
 */
int32_t moe_probe_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                       void* stream);
int32_t moe_probe_mfma(int32_t iters, float* out, int32_t blocks, void* stream);

/*
 * moe_unpermute_combine -- [W] section 3 workflow: rows are restored to the original order
 * and scaled by the gate weight (expert_scale); the k rows of a token are summed.
 *
 *   out[t] = fp16( sum_{j=0..k-1} w[t,j] * y_perm[inv_perm[t*k+j]]  + addend[t] )
 *   evaluated in fp32 in ascending j, then the addend, then one rounding to fp16.
 *   y_perm    fp16 [R, d] (R >= T*k rows; only rows inv_perm points at are read)
 *   inv_perm  int32 [T*k] (from moe_permute)
 *   topk_w    fp32 [T, k] or NULL (rows already scaled, e.g. by row_scale in the GEMM)
 *   addend    fp16 [T, d] or NULL (added with weight 1, e.g. shared experts)
 *   out       fp16 [T, d]
 *   Requires 1 <= k <= 8, d % 8 == 0.
 */
int32_t moe_unpermute_combine(const uint16_t* y_perm, const int32_t* inv_perm,
                              const float* topk_w, const uint16_t* addend,
                              int32_t T, int32_t k, int32_t d, uint16_t* out, void* stream);

/*
 * Expert lookahead buffer.  [S] Method steps, step 2: while the draft advances, the analyzer
 * counts per MoE layer j and expert e the draft steps whose routing used e in layer j,
 * ELB_cnt[j, e] = sum over steps i of [e in ELB_route[i, j]]; step 3: at a chunk boundary the
 * planner takes each layer's top-M experts as the prefetch plan.
 *
 * moe_elb_accumulate -- one draft step.
 *   ids     int32 [L, T, k]  the step's routing in each of L layers (T draft tokens, k experts
 *                            each, e.g. moe_route_topk's output per layer); ids outside [0, E)
 *                            route nowhere and are ignored
 *   counts  int32 [L, E]     in/out: counts[j][e] += 1 if e appears among layer j's ids
 *                            (once per step, however many tokens chose it)
 *   Requires 1 <= E <= 256, k >= 1.  L == 0 enqueues nothing; T == 0 adds nothing.
 *
 * moe_elb_top_m -- the planner's snapshot.
 *   counts      int32 [L, E]
 *   experts     int32 [L, M] out: per layer the M experts with the largest counts, in that
 *                            order, ties to the smaller expert index (experts with count 0
 *                            fill the tail when fewer than M were used)
 *   top_counts  int32 [L, M] out (nullable): their counts
 *   Requires 1 <= M <= E <= 256.
 */
int32_t moe_elb_accumulate(const int32_t* ids, int32_t L, int32_t T, int32_t k, int32_t E,
                           int32_t* counts, void* stream);
int32_t moe_elb_top_m(const int32_t* counts, int32_t L, int32_t E, int32_t M, int32_t* experts,
                      int32_t* top_counts, void* stream);

/*
 * moe_bf16_recombine -- [Z] "ZipMoE" note, key design (BF16 bit-field lossless compression):
 * an expert tensor is kept as its exponent bits (compressed, then decompressed before use) and
 * its sign and mantissa bits (byte-aligned); recovery merges them into the original BF16.
 *   exponents      uint8 [n]   the 8 exponent bits of each value
 *   sign_mantissa  uint8 [n]   sign in bit 7, the 7 mantissa bits in bits 6..0
 *   out            uint16 [n]  BF16 bits: (sm & 0x80) << 8 | e << 7 | (sm & 0x7F)
 *   All three pointers 16-byte aligned; any n (a tail of n % 16 values is handled apart).
 *   Exact: recombining the fields of any BF16 value gives its bits back.
 */
int32_t moe_bf16_recombine(const uint8_t* exponents, const uint8_t* sign_mantissa, size_t n,
                           uint16_t* out, void* stream);

/*
 * moe_dequant -- Algorithm 1 of [W] section 3:
 *   for e, m, n:  W_dq[e, m, n] = IntToFloat(W[e, m, n]) * S[e, g(m), n]   (fp16)
 * with IntToFloat done by the exponent-of-1024 construction and one fp16 multiply (round
 * to nearest even), so the result is the correctly rounded fp16 product.
 *   w_packed  packed by moe_pack_wq; scales fp16 [E, G, N] as for the GEMM
 *   w_out     fp16 [E, K, N], logical (unpacked) layout
 *   Requires wtype INT4 or INT8, K % 128 == 0, N % 16 == 0.
 */
int32_t moe_dequant(const void* w_packed, const uint16_t* scales, int32_t wtype,
                    int32_t group_size, int32_t E, int32_t K, int32_t N, uint16_t* w_out,
                    void* stream);

/* ---- host-only helpers (no device needed) ---- */

/* Bytes of the packed weights of (wtype, E, K, N): E*K*N/2 (INT4), E*K*N (INT8),
 * 2*E*K*N (FP16); 0 if the shape is unsupported. */
size_t moe_packed_bytes(int32_t wtype, int32_t E, int32_t K, int32_t N);

/*
 * moe_pack_wq -- pack weights into the library's layout (host memory to host memory).
 *   codes   [host] int8 [E, K, N] codes (INT4: values in [-8, 7]; INT8: [-128, 127]), or
 *           uint16 fp16 bit patterns [E, K, N] for MOE_W_FP16.
 *   packed  [host] moe_packed_bytes(wtype, E, K, N) bytes.
 *   Layout: 16-column blocks, each contiguous along K in 1 KiB units; inside a 32-bit word
 *   8 int4 codes of 8 consecutive K rows of one column, stored offset by +8 in the nibble
 *   order [e0,e2,e4,e6,e1,e3,e5,e7] of [W] section 3 (4-bit variant); int8 codes are stored
 *   offset by +128, 4 consecutive K rows per word in natural byte order (8-bit variant).
 *   Returns MOE_ERR_INVALID for a code outside its range (packed is then undefined).
 */
int32_t moe_pack_wq(const void* codes, int32_t wtype, int32_t E, int32_t K, int32_t N,
                    void* packed);

/* Text of a status code (static storage). */
const char* moe_status_str(int32_t status);

/* Library version, e.g. 100 for 0.1.0. */
int32_t moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_WQ_H */
