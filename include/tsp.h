/*
 * tsp.h - C ABI of the MI355X (gfx950) TSP rank-share layer library (libtsp.so).
 *
 * Tensor + Sequence Parallelism (TSP) folds tensor parallelism (weights
 * sharded) and sequence parallelism (tokens sharded) onto one device-mesh axis
 * of size D: each device holds 1/D of every weight matrix and 1/D of the
 * sequence (zubnet.ai, "Zyphra TSP folds TP+SP onto one GPU axis", para. 1).
 * For attention the weight shards are applied one after another to the local
 * tokens and K/V are gathered over a zigzag partition; for the MLP the weight
 * shard pairs are applied in ring order and the partial products are summed
 * locally, which replaces the all-reduce of tensor parallelism (same page,
 * para. 2).  This library is the computation of ONE device for one decoder
 * layer.  The collectives are not part of it: the gathered K/V and the weight
 * shards are caller-owned device buffers.
 *
 * Conventions for every entry point:
 *   - bf16 tensors are passed as uint16_t bit patterns; all tensors are dense
 *     row-major.  Weights are stored out x in (nn.Linear layout).
 *   - "device" pointers point to memory of the current HIP device, must be
 *     16-byte aligned and must not alias outputs unless stated.
 *   - weight shards are a HOST array of D device pointers (D <= TSP_MAX_D).
 *   - the caller owns every buffer, including the workspace; the library keeps
 *     no global state, allocates nothing and never synchronises.  Calls are
 *     reentrant; calls on different streams that write the same buffers race.
 *   - all arguments are validated before anything is enqueued; a status other
 *     than TSP_OK means nothing was enqueued, except TSP_ERR_HIP (a launch
 *     failed; earlier launches of the same call may have been enqueued).
 *     Faults inside kernels surface at the caller's next synchronisation.
 *   - work is enqueued on `stream` (0 = the null stream) and returns at once.
 *
 * Layer (one rank, local rows in plan order):
 *   q,k,v  = x W_q^T, x W_k^T, x W_v^T       (shard-iterated, tsp_attn_project)
 *   k_full/v_full rows at the rank's own positions <- k, v
 *   a      = causal softmax(q k_full^T / sqrt(hd)) v_full    (tsp_attn_core)
 *   h1     = x + a W_o^T                     (split-K over head shards, tsp_attn_out)
 *   out    = h1 + GELU_tanh(h1 W1^T) W2^T    (ring split-K over FFN shards, tsp_mlp_forward)
 */
#ifndef TSP_H
#define TSP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TSP_MAX_D 16

typedef enum {
  TSP_OK = 0,
  TSP_ERR_INVALID_ARG = 1, /* null pointer, bad enum value, out-of-range rank or start shard */
  TSP_ERR_SHAPE = 2,       /* shapes inconsistent with the method (see each call) */
  TSP_ERR_ALIGNMENT = 3,   /* a device pointer is not 16-byte aligned */
  TSP_ERR_WORKSPACE = 4,   /* workspace null or smaller than tsp_workspace_size() */
  TSP_ERR_UNSUPPORTED = 5, /* valid for the method but not implemented (head_dim, widths) */
  TSP_ERR_HIP = 6,         /* a kernel launch failed */
  TSP_ERR_SCRATCH = 7      /* more scratch than the fixed array of tsp_attn_forward_noalloc */
} tsp_status;

/* Rank's share of the sequence (plain data, host memory). */
typedef struct {
  int64_t seq_len;        /* S, total sequence length */
  int64_t chunk_len;      /* C = S / (2D) */
  int64_t n_local;        /* n = S / D = 2C local tokens */
  int32_t D;              /* TSP axis size */
  int32_t rank;           /* r in [0, D) */
  int32_t chunk_id[2];    /* r and 2D-1-r */
  int64_t chunk_start[2]; /* chunk_id[i] * C */
} tsp_plan;

/* Layer shape. hidden = n_heads * head_dim. */
typedef struct {
  int32_t hidden;
  int32_t n_heads;
  int32_t head_dim;
  int32_t ffn;
} tsp_dims;

/* Workspace kinds for tsp_workspace_size(). */
typedef enum {
  TSP_WS_ATTN = 0,
  TSP_WS_MLP = 1,
  TSP_WS_LAYER = 2,
  TSP_WS_POST = 3,
  TSP_WS_CORE = 4,
  TSP_WS_OUT_SHARD = 5,
  TSP_WS_MLP_SHARD = 6,
  TSP_WS_MLP_BWD = 7,
  TSP_WS_ATTN_BWD = 8,
  TSP_WS_OUT_BWD = 9,
  TSP_WS_PROJ_BWD = 10,
  TSP_WS_RMS_BWD = 11
} tsp_ws_kind;

/*
 * Zigzag plan (zubnet.ai TSP page, para. 2: K/V are gathered over a zigzag
 * partition for load balance).  The sequence is cut into 2D chunks of C = S/(2D)
 * tokens; rank r holds chunks r and 2D-1-r, so every rank has the same causal
 * work.  Local row i < C is global position chunk_start[0] + i, row i >= C is
 * chunk_start[1] + (i - C).  Ring order of weight shards for the MLP:
 * ring_order[k] = (r + k) mod D.
 *   seq_len, D, rank: S > 0, D in [1, TSP_MAX_D], S % (2D) == 0, 0 <= rank < D.
 *   plan            : host out, required.
 *   local_to_global : host out, nullable; int64[n_local].
 *   ring_order      : host out, nullable; int32[D].
 * Errors: TSP_ERR_INVALID_ARG (plan null, rank out of range, D out of range),
 *         TSP_ERR_SHAPE (S <= 0 or S % 2D != 0).  Host only; no device work.
 */
tsp_status tsp_zigzag_plan(int64_t seq_len, int32_t D, int32_t rank, tsp_plan* plan,
                           int64_t* local_to_global, int32_t* ring_order);

/*
 * Bytes of workspace that tsp_attn_forward (TSP_WS_ATTN), tsp_mlp_forward
 * (TSP_WS_MLP), tsp_layer_forward (TSP_WS_LAYER), tsp_layer_post (TSP_WS_POST)
 * or tsp_attn_core (TSP_WS_CORE) need for n_tokens local tokens (the kinds
 * that hold attention state size it for a sequence of D * n_tokens keys), and
 * the shard-streaming calls tsp_attn_out_shard (TSP_WS_OUT_SHARD) and
 * tsp_mlp_shard (TSP_WS_MLP_SHARD), and tsp_mlp_backward (TSP_WS_MLP_BWD).  Returns 0 for invalid dims or kind.
 * Workspace contents are scratch: nothing persists between calls, except the
 * fp32 accumulator (and row exponents) that the D calls of one ring of a
 * shard-streaming entry point pass from step to step.
 */
size_t tsp_workspace_size(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t kind);

/*
 * QKV projection, shard-iterated (para. 2: the attention weight shards are
 * applied one after another to the local tokens).  For d = 0..D-1:
 *   [Q_d | K_d | V_d] = x_local W_qkv_d^T
 * Q_d goes to q_out[:, heads of shard d]; K_d and V_d rows are written into
 * k_full / v_full at the rank's own global positions (the rank's contribution
 * to the K/V all-gather).  Other rows of k_full / v_full are not touched.
 *   plan      : from tsp_zigzag_plan; its D is the shard count.
 *   dims      : n_heads % D == 0, hidden = n_heads * head_dim, head_dim in {64, 128},
 *               hidden % 64 == 0.
 *   x_local   : device, bf16 [n_local x hidden].
 *   wqkv      : host array of D device pointers, each bf16 [3 * H_s * head_dim x hidden],
 *               rows = shard d's Q heads, then its K heads, then its V heads
 *               (H_s = n_heads / D; shard d owns heads d*H_s .. (d+1)*H_s - 1).
 *   k_full, v_full : device, bf16 [seq_len x hidden], in/out.
 *   q_out     : device, bf16 [n_local x hidden], out.
 */
tsp_status tsp_attn_project(const tsp_plan* plan, const tsp_dims* dims, const uint16_t* x_local,
                            const uint16_t* const* wqkv, uint16_t* k_full, uint16_t* v_full,
                            uint16_t* q_out, hipStream_t stream);

/*
 * Causal attention of the local queries (two zigzag chunks) against the whole
 * gathered K/V (para. 2).  Per head a and local row t at global position p:
 *   attn[t, a] = sum_{j <= p} softmax_j(q[t, a] . k_full[j, a] / sqrt(head_dim)) v_full[j, a]
 * (the diagonal is included).  fp32 online softmax, bf16 MFMA products.
 *   dims   : hidden = n_heads * head_dim, head_dim in {64, 128}, hidden % 64 == 0
 *            (the heads need not divide over D: no weight shard is read here).
 *   q      : device, bf16 [n_local x hidden] (as tsp_attn_project writes it).
 *   k_full, v_full : device, bf16 [seq_len x hidden], read only.
 *   attn_out : device, bf16 [n_local x hidden], out; must not alias q.
 *   attn_lo  : device, bf16 [n_local x hidden], out, nullable: the rounding
 *              residual bf16(attn - attn_out), so that attn_out + attn_lo carries
 *              the fp32 result to about 16 significant bits (tsp_attn_out and
 *              tsp_layer_post contract both parts).
 *   workspace: device, >= tsp_workspace_size(n_local, dims, D, TSP_WS_CORE) bytes:
 *              for short sequences (fewer than 512 work items of 256 queries
 *              and one head), where the late chunk's key range is processed in
 *              two halves, the halves' fp32 partial outputs, maxima and sums;
 *              otherwise no bytes, and workspace may be null.
 */
tsp_status tsp_attn_core(const tsp_plan* plan, const tsp_dims* dims, const uint16_t* q,
                         const uint16_t* k_full, const uint16_t* v_full, uint16_t* attn_out,
                         uint16_t* attn_lo, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * tsp_attn_core that also keeps, for the backward, the natural log of each
 * query row's softmax normaliser:
 *   lse[a * n_local + t] = ln sum_{j <= p} exp(q[t, a] . k_full[j, a] / sqrt(head_dim))
 *   lse : device, fp32 [n_heads x n_local], out.
 * Everything else (arguments, workspace TSP_WS_CORE, errors) as tsp_attn_core.
 */
tsp_status tsp_attn_core_lse(const tsp_plan* plan, const tsp_dims* dims, const uint16_t* q,
                             const uint16_t* k_full, const uint16_t* v_full, uint16_t* attn_out,
                             uint16_t* attn_lo, float* lse, void* workspace, size_t ws_bytes,
                             hipStream_t stream);

/*
 * Backward of tsp_attn_core (the TSP page names long-context training as a use
 * of the method, zubnet.ai TSP page, paras. 2 and 4; the gradients are the
 * chain rule of the forward above).  Per head, with P the causal softmax rows, o = P v_full and dO the
 * gradient of o:
 *   dv_full = P^T dO,  dS = P * (dO v_full^T - rowsum(dO * o)),
 *   dq = dS k_full / sqrt(head_dim),  dk_full = dS^T q / sqrt(head_dim).
 * dk_full / dv_full are this rank's contributions for every key row (zero for
 * keys no local query sees); in TSP each key row's owner would sum them over
 * the ranks, the reverse of the K/V all-gather (para. 2).  MHA only.
 *   q, k_full, v_full : as tsp_attn_core (bf16).
 *   attn_out, attn_lo : the forward's output (bf16; attn_lo nullable), read.
 *   lse      : device, fp32 [n_heads x n_local], from tsp_attn_core_lse.
 *   d_attn   : device, bf16 [n_local x hidden], the gradient of attn_out.
 *   dq       : device, fp32 [n_local x hidden], out.
 *   dk_full, dv_full : device, fp32 [seq_len x hidden], out (every row written).
 *   workspace: device, >= tsp_workspace_size(n_local, dims, D, TSP_WS_ATTN_BWD)
 *              bytes (per-row stats; at head_dim 64 also transposed tiles of
 *              k_full, q and d_attn).
 * P is rebuilt from the scores and lse; P and dS enter the products as bf16,
 * accumulation is fp32.  Errors: as tsp_attn_core, plus TSP_ERR_INVALID_ARG
 * when two of dq, dk_full, dv_full are the same buffer.
 */
tsp_status tsp_attn_core_backward(const tsp_plan* plan, const tsp_dims* dims, const uint16_t* q,
                                  const uint16_t* k_full, const uint16_t* v_full, const uint16_t* attn_out,
                                  const uint16_t* attn_lo, const float* lse, const uint16_t* d_attn, float* dq,
                                  float* dk_full, float* dv_full, void* workspace, size_t ws_bytes,
                                  hipStream_t stream);

/*
 * Backward of the O projection (tsp_attn_out's product; the attention
 * projections are iterated over the weight shards, zubnet.ai TSP page, para. 2):
 * with out = [residual +] sum_d attn[:, block d] W_o_d^T and d_out its gradient,
 *   d_attn[:, block d] = d_out W_o_d,    dwo[d] = d_out^T attn[:, block d]
 * (block d: shard d's heads, columns d*H_s*hd ..).  dwo[d] is this rank's
 * contribution to shard d's gradient (in TSP the shard's owner would sum the
 * ranks' contributions); the residual's gradient is d_out itself.  Shards are
 * visited in ring order from start_shard.
 *   attn     : device, bf16 [n_tokens x hidden], the forward's attention output
 *              (its high part: the low part's contribution is below bf16 rounding).
 *   wo       : host array of D device pointers, bf16 [hidden x H_s*hd].
 *   d_out    : device, bf16 [n_tokens x hidden].
 *   d_attn   : device, bf16 [n_tokens x hidden], out; aliases neither attn nor d_out.
 *   dwo      : host array of D device pointers, fp32 [hidden x H_s*hd], out.
 *   workspace: >= tsp_workspace_size(n_tokens, dims, D, TSP_WS_OUT_BWD) bytes.
 * n_tokens = 0 writes zero weight gradients and nothing else; the token
 * buffers and the workspace may then be null.
 * Errors: as tsp_attn_out, plus TSP_ERR_WORKSPACE.
 */
tsp_status tsp_attn_out_backward(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t start_shard,
                                 const uint16_t* attn, const uint16_t* const* wo, const uint16_t* d_out,
                                 uint16_t* d_attn, float* const* dwo, void* workspace, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * Backward of the shard-iterated QKV projection (para. 2): with
 * [q_d | k_d | v_d] = x W_qkv_d^T for every shard d,
 *   dx = [dy +] sum_d (dq[:, block d] Wq_d + dk[:, block d] Wk_d + dv[:, block d] Wv_d)
 *   dwqkv[d] = [dq[:, block d]^T x ; dk[:, block d]^T x ; dv[:, block d]^T x]
 * (Wq_d, Wk_d, Wv_d: the row blocks of wqkv[d]).  dk and dv are the rank's
 * own K/V rows' gradients, i.e. its rows of every rank's dk_full / dv_full
 * contributions summed (the reduce-scatter of tsp_attn_core_backward's output;
 * on one rank, its own rows).  dy is the gradient that reaches x through the
 * layer's residual (nullable).  dx is accumulated in one fp32 accumulator over
 * the 3D (part, shard) blocks, from block start_shard onwards.
 *   x        : device, bf16 [n_tokens x hidden], the forward's input.
 *   wqkv     : as tsp_attn_project.
 *   dq, dk, dv : device, fp32 [n_tokens x hidden] (rounded to bf16 for the products).
 *   dy       : device, bf16 [n_tokens x hidden], nullable.
 *   dx       : device, bf16 [n_tokens x hidden], out; must not alias x.
 *   dwqkv    : host array of D device pointers, fp32 [3*H_s*hd x hidden], out.
 *   workspace: >= tsp_workspace_size(n_tokens, dims, D, TSP_WS_PROJ_BWD) bytes.
 * n_tokens = 0 writes zero weight gradients and nothing else; the token
 * buffers and the workspace may then be null.
 * Errors: as tsp_attn_project, plus TSP_ERR_WORKSPACE.
 */
tsp_status tsp_attn_project_backward(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t start_shard,
                                     const uint16_t* x, const uint16_t* const* wqkv, const float* dq, const float* dk,
                                     const float* dv, const uint16_t* dy, uint16_t* dx, float* const* dwqkv,
                                     void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * O projection as a split-K over the D head shards (the attention projections
 * iterated over the weight shards, para. 2; W_o is taken in row blocks by head
 * shard).  Shards are visited in ring order d_k = (start_shard + k) mod D with
 * one fp32 accumulator across all of them:
 *   out = [residual +] sum_k attn[:, heads of d_k] W_o_{d_k}^T
 *   n_tokens  : rows of attn / out (>= 0; 0 enqueues nothing).
 *   attn      : device, bf16 [n_tokens x hidden].
 *   attn_lo   : device, bf16 [n_tokens x hidden], nullable: low part of the
 *               attention output (tsp_attn_core); when given, the product is
 *               (attn + attn_lo) W_o^T.
 *   wo        : host array of D device pointers, each bf16 [hidden x H_s * head_dim].
 *   residual  : device, bf16 [n_tokens x hidden], nullable (then no residual).
 *   out       : device, bf16 [n_tokens x hidden]; may alias residual, not attn.
 */
tsp_status tsp_attn_out(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t start_shard,
                        const uint16_t* attn, const uint16_t* attn_lo, const uint16_t* const* wo,
                        const uint16_t* residual, uint16_t* out, hipStream_t stream);

/*
 * Attention half of the layer: tsp_attn_project, tsp_attn_core (with the low
 * part of its output), then tsp_attn_out with start_shard = plan->rank.
 *   residual  : nullable; the layer passes x_local.
 *   out       : device, bf16 [n_local x hidden]; must not alias x_local.
 *   workspace : device, >= tsp_workspace_size(n_local, dims, D, TSP_WS_ATTN) bytes.
 */
tsp_status tsp_attn_forward(const tsp_plan* plan, const tsp_dims* dims, const uint16_t* x_local,
                            const uint16_t* const* wqkv, const uint16_t* const* wo,
                            uint16_t* k_full, uint16_t* v_full, const uint16_t* residual,
                            uint16_t* out, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * tsp_attn_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * must not call hipMalloc, harnesses that forbid it).  The scratch that
 * tsp_attn_forward takes from its workspace (Q, the attention output as a bf16
 * pair, the split partials of short sequences: tsp_workspace_size(n_local,
 * dims, D, TSP_WS_ATTN) bytes) lives in a fixed device array of the library of
 * TSP_NOALLOC_SCRATCH_BYTES (96 MiB) per GPU, held until the process ends; a
 * call that needs more returns TSP_ERR_SCRATCH and enqueues nothing (the 7B
 * attention half fits at 2048 local tokens, 84 MB; not at 16384).
 * Every call on one GPU uses that GPU's one array: calls that overlap on one
 * GPU (other streams, other threads) race and must be ordered by the caller.
 * Nothing in the array needs to start at zero: each call writes every byte it
 * reads.  The array's device address is resolved on the first call on each
 * device (hipGetSymbolAddress, with that device current); make that first call
 * before capturing a graph.  Arguments, results and other errors as
 * tsp_attn_forward.
 */
#define TSP_NOALLOC_SCRATCH_BYTES (96u * 1024u * 1024u)
tsp_status tsp_attn_forward_noalloc(const tsp_plan* plan, const tsp_dims* dims, const uint16_t* x_local,
                                    const uint16_t* const* wqkv, const uint16_t* const* wo, uint16_t* k_full,
                                    uint16_t* v_full, const uint16_t* residual, uint16_t* out, hipStream_t stream);

/*
 * MLP with the shard pairs in ring order (para. 2): the shard loop is a split-K
 * over the FFN dimension with one fp32 accumulator, in place of the
 * all-reduce of tensor parallelism:
 *   y = [residual +] sum_{k=0}^{D-1} GELU_tanh(x W1_{d_k}^T) W2_{d_k}^T,  d_k = (start_shard + k) mod D
 * Precision: x W1^T runs on bf16 operands; the GELU output is held in fp16,
 * each token row scaled by a power of two from the RMS of its x row (exact,
 * undone before the residual), and W2 meets it as an fp16 copy of its shards
 * (bf16 weights are exact in fp16 above 2^-14; smaller ones keep an absolute
 * error below 2^-25; magnitudes beyond 65504 saturate).
 *   n_tokens : rows (>= 0).
 *   dims     : ffn % D == 0, ffn / D % 64 == 0, hidden % 64 == 0.
 *   x        : device, bf16 [n_tokens x hidden].
 *   w1       : host array of D device pointers, each bf16 [ffn/D x hidden].
 *   w2       : host array of D device pointers, each bf16 [hidden x ffn/D].
 *   residual : device, nullable.  y: device, bf16 [n_tokens x hidden]; may alias
 *              residual, must not alias x unless residual == x.
 *   workspace: >= tsp_workspace_size(n_tokens, dims, D, TSP_WS_MLP) bytes.
 */
tsp_status tsp_mlp_forward(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t start_shard,
                           const uint16_t* x, const uint16_t* const* w1, const uint16_t* const* w2,
                           const uint16_t* residual, uint16_t* y, void* workspace, size_t ws_bytes,
                           hipStream_t stream);

/*
 * Post-attention half of the layer for n_tokens rows:
 *   h1  = x + attn W_o^T   (split-K over head shards in ring order from start_shard, fp32 result)
 *   out = h1 + sum_k GELU_tanh(h1 W1_{d_k}^T) W2_{d_k}^T   (ring from start_shard)
 * h1 stays in fp32 for the residual; both MLP GEMMs run on fp16 operands (h1
 * and the GELU output scaled per row by a power of two from the RMS of the h1
 * row, W1 and W2 as fp16 copies of the bf16 shards; see tsp_mlp_forward).
 * Weight magnitudes: W1 and W2 elements beyond the fp16 range (|w| > 65504)
 * saturate to +-65504 in their copies, and those below 2^-14 keep an absolute
 * error under 2^-25; no status reports either (N(0, 0.02) weights are far
 * inside both limits).
 *   dims      : as for tsp_layer_forward.
 *   attn      : device, bf16 [n_tokens x hidden] (tsp_attn_core output).
 *   attn_lo   : device, bf16, nullable: its low part (see tsp_attn_core).
 *   x         : device, bf16 [n_tokens x hidden] (the layer input, first residual).
 *   wo, w1, w2: host arrays of D device pointers (layouts as above).
 *   out       : device, bf16 [n_tokens x hidden]; must not alias x, attn or attn_lo.
 *   workspace : >= tsp_workspace_size(n_tokens, dims, D, TSP_WS_POST) bytes.
 */
tsp_status tsp_layer_post(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t start_shard,
                          const uint16_t* attn, const uint16_t* attn_lo, const uint16_t* x,
                          const uint16_t* const* wo, const uint16_t* const* w1, const uint16_t* const* w2,
                          uint16_t* out, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * One decoder layer for the rank's local tokens: tsp_attn_project, then
 * tsp_attn_core, then tsp_layer_post with start_shard = plan->rank, i.e.
 *   h1 = x + Attn(x), out = h1 + MLP(h1).  No norm, no bias.  The MLP's
 * precision and weight-magnitude limits are tsp_layer_post's.
 *   out       : device, bf16 [n_local x hidden]; must not alias x_local.
 *   workspace : >= tsp_workspace_size(n_local, dims, D, TSP_WS_LAYER) bytes.
 */
tsp_status tsp_layer_forward(const tsp_plan* plan, const tsp_dims* dims, const uint16_t* x_local,
                             const uint16_t* const* wqkv, const uint16_t* const* wo,
                             const uint16_t* const* w1, const uint16_t* const* w2,
                             uint16_t* k_full, uint16_t* v_full, uint16_t* out, void* workspace,
                             size_t ws_bytes, hipStream_t stream);

/*
 * ---- Shard streaming (the ring one shard at a time) ----
 * In TSP the weight shards of a layer reach a device one after another (para. 2:
 * the MLP's shard pairs travel a ring, the attention weights are broadcast).
 * The calls below do the work of one shard, so that a caller can start each
 * shard's compute as soon as that shard has arrived: make the stream wait for
 * the shard's arrival (hipStreamWaitEvent on the event recorded after its
 * copy) before the call.  The D calls of one ring go on one stream, in ring
 * order; they run the same kernels as the all-shard calls.
 *
 * tsp_attn_project_shard: the QKV projection of head shard `shard` alone
 * (tsp_attn_project restricted to d = shard): Q columns of the shard's heads,
 * and the shard's K/V columns of the rank's own rows of k_full / v_full.
 * Results are bit-identical to tsp_attn_project's for those columns.
 *   shard : 0 <= shard < plan->D.   wqkv_d: device, bf16 [3 * H_s * head_dim x hidden].
 *   Other arguments and errors as tsp_attn_project.
 */
tsp_status tsp_attn_project_shard(const tsp_plan* plan, const tsp_dims* dims, int32_t shard,
                                  const uint16_t* x_local, const uint16_t* wqkv_d, uint16_t* k_full,
                                  uint16_t* v_full, uint16_t* q_out, hipStream_t stream);

/*
 * Step `pos` of the O projection's ring (tsp_attn_out one shard at a time):
 *   acc  = [residual +] attn[:, heads of shard] W_o_shard^T          (pos == 0)
 *   acc += attn[:, heads of shard] W_o_shard^T                       (0 < pos < D-1)
 *   out  = bf16(acc + attn[:, heads of shard] W_o_shard^T)           (pos == D-1)
 * acc is fp32 [n_tokens x hidden] at the start of the workspace; with D == 1
 * the single step reads the residual and writes out.  The ring order is the
 * order of the calls: for tsp_attn_out's order, call pos = 0..D-1 with
 * shard = (start_shard + pos) mod D.  Each step's partial product is summed in
 * fp32 registers over its K range and added to acc in fp32, so the result
 * differs from tsp_attn_out's only in fp32 rounding order.
 *   pos, shard : 0 <= pos, shard < D.
 *   attn, attn_lo, residual, out : as tsp_attn_out (residual is read at pos 0,
 *                 out written at pos D-1; out may alias residual).
 *   wo_d      : device, bf16 [hidden x H_s * head_dim].
 *   workspace : >= tsp_workspace_size(n_tokens, dims, D, TSP_WS_OUT_SHARD) bytes,
 *               the same buffer for the D steps of one ring.
 * Errors: as tsp_attn_out, plus TSP_ERR_INVALID_ARG for pos or shard out of
 * range, TSP_ERR_WORKSPACE for a missing or short workspace.
 */
tsp_status tsp_attn_out_shard(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t pos, int32_t shard,
                              const uint16_t* attn, const uint16_t* attn_lo, const uint16_t* wo_d,
                              const uint16_t* residual, uint16_t* out, void* workspace, size_t ws_bytes,
                              hipStream_t stream);

/*
 * Step `pos` of the MLP ring (tsp_mlp_forward one shard pair at a time):
 *   H    = GELU_tanh(x W1_d^T)                  (fp16, rows scaled as in tsp_mlp_forward)
 *   acc  = [residual +] H W2_d^T    (pos == 0; also computes the row exponents of x)
 *   acc += H W2_d^T                 (0 < pos < D-1)
 *   y    = bf16(acc + H W2_d^T)     (pos == D-1)
 * with acc fp32 [n_tokens x hidden] and the row exponents in the workspace.
 * The shard index itself is not needed: a shard pair's contribution does not
 * depend on which pair it is; the ring order is the order of the calls.
 * Precision as tsp_mlp_forward; the result differs from it only in fp32
 * rounding order.
 *   pos       : 0 <= pos < D.
 *   x         : device, bf16 [n_tokens x hidden], the same for the D steps.
 *   w1_d      : device, bf16 [ffn/D x hidden];  w2_d: device, bf16 [hidden x ffn/D].
 *   residual  : nullable, read at pos 0.  y: written at pos D-1; may alias
 *               residual, must not alias x.
 *   workspace : >= tsp_workspace_size(n_tokens, dims, D, TSP_WS_MLP_SHARD) bytes,
 *               the same buffer for the D steps of one ring.
 * Errors: as tsp_mlp_forward, plus TSP_ERR_INVALID_ARG for pos out of range.
 */
tsp_status tsp_mlp_shard(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t pos, const uint16_t* x,
                         const uint16_t* w1_d, const uint16_t* w2_d, const uint16_t* residual, uint16_t* y,
                         void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * ---- Calls that wait for their shards inside the kernels ----
 * The all-shard calls below take the same arguments as tsp_attn_project,
 * tsp_attn_out and tsp_mlp_forward, plus an arrival counter: they can be
 * launched before the layer's shards have arrived (para. 2: the shards reach a
 * device one after another, by broadcast or around the ring), and each tile
 * of their GEMMs reads a shard only once the counter shows it.  A shard that
 * has arrived costs a tile one poll; the fp32 accumulator of the K-sharded
 * products stays in registers across the shards, as in the all-shard calls,
 * and the results are bit-identical to theirs.
 *
 * The producer (a copy engine, a peer's transfer, tsp_simulate_arrival)
 * delivers the shards in ring order, position p = 0..D-1 being shard
 * (start_shard + p) mod D; for the MLP, position p is the pair
 * (W1_d, W2_d).  After the bytes of position p are in device memory it raises
 * the counter to base + p + 1 with release semantics (or any larger value).
 *
 *   counter    : device, uint32, 4-byte aligned; read with system-scope loads
 *                by one wave per workgroup, with a sleep between polls.
 *   base       : the counter's value before this call's first shard; the
 *                comparison is modulo 2^32, so a counter may run across calls.
 *   spin_limit : polls of one wait before it gives up (0: TSP_ARRIVAL_SPIN_DEFAULT,
 *                a few seconds); a wait that gives up sets *status = 1 and the
 *                call then reads whatever the shard buffers hold.
 *   status     : device, uint32, 4-byte aligned, required; set to 1 by a wait
 *                that gave up, never cleared by the library.
 * The waiting workgroups occupy their CUs: a producer that needs CUs (a copy
 * kernel) must already be resident, or the grid must leave CUs free.  A
 * producer on the same device must also not be queued behind the call: HIP
 * streams share hardware queues once there are more streams than queues, so
 * enqueue the producer first (it then either runs alongside or completes
 * before the call starts).
 */
typedef struct {
  const uint32_t* counter;
  uint32_t base;
  uint32_t spin_limit;
  uint32_t* status;
} tsp_arrival;
#define TSP_ARRIVAL_SPIN_DEFAULT (1u << 20)

/* tsp_attn_project with arrival; position p is head shard (start_shard + p) mod D
 * (0 <= start_shard < D).  Errors: as tsp_attn_project, plus TSP_ERR_INVALID_ARG
 * for a null arrival, counter or status or start_shard out of range,
 * TSP_ERR_ALIGNMENT for a counter or status not 4-byte aligned. */
tsp_status tsp_attn_project_arrival(const tsp_plan* plan, const tsp_dims* dims, int32_t start_shard,
                                    const uint16_t* x_local, const uint16_t* const* wqkv, uint16_t* k_full,
                                    uint16_t* v_full, uint16_t* q_out, const tsp_arrival* arrival,
                                    hipStream_t stream);

/* tsp_attn_out with arrival.  Errors: as tsp_attn_out, plus those of the arrival. */
tsp_status tsp_attn_out_arrival(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t start_shard,
                                const uint16_t* attn, const uint16_t* attn_lo, const uint16_t* const* wo,
                                const uint16_t* residual, uint16_t* out, const tsp_arrival* arrival,
                                hipStream_t stream);

/* tsp_mlp_forward with arrival (workspace TSP_WS_MLP).  The fp16 copy of W2 is
 * made after the W1 GEMM, which has then seen every pair arrive.  Errors: as
 * tsp_mlp_forward, plus those of the arrival. */
tsp_status tsp_mlp_forward_arrival(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t start_shard,
                                   const uint16_t* x, const uint16_t* const* w1, const uint16_t* const* w2,
                                   const uint16_t* residual, uint16_t* y, void* workspace, size_t ws_bytes,
                                   const tsp_arrival* arrival, hipStream_t stream);

/*
 * Simulated arrival, for tests and measurements on one device: a one-workgroup
 * kernel that, for i = 0..n-1, waits until (i + 1) * delay_us microseconds
 * after it started, copies bytes[i] from src[i] to dst[i], writes the copy back
 * to memory and raises *counter to base + i + 1 (system scope).  It stands in
 * for the shard transfers of the other ranks (para. 2).
 *   n        : 0 <= n <= 64.   src, dst: host arrays of n device pointers,
 *              16-byte aligned; dst[i] must not overlap any src or other dst.
 *   bytes    : host array of n sizes, each a multiple of 16.
 *   counter  : device, uint32, 4-byte aligned.   delay_us: <= 10^6.
 * Errors: TSP_ERR_INVALID_ARG (null pointers, n or delay out of range),
 *         TSP_ERR_ALIGNMENT, TSP_ERR_SHAPE (a size not a multiple of 16).
 */
tsp_status tsp_simulate_arrival(int32_t n, const void* const* src, void* const* dst, const size_t* bytes,
                                uint32_t* counter, uint32_t base, uint32_t delay_us, hipStream_t stream);

/*
 * ---- Layer variants of a real decoder ----
 * Not on the TSP pages (their layer has no norm, no positional encoding, and
 * 32 K/V heads for 32 query heads); these are the published definitions, for
 * decoders that have them.
 *
 * RMSNorm (Zhang & Sennrich 2019) of each row of x [n_tokens x hidden]:
 *   y = x / sqrt(mean_j x_j^2 + eps) * gain            (fp32 inside, bf16 out)
 *   gain : device, bf16 [hidden].  y may alias x.  hidden % 8 == 0; eps >= 0.
 * Errors: TSP_ERR_SHAPE (n < 0, hidden <= 0), TSP_ERR_UNSUPPORTED (hidden % 8),
 *         TSP_ERR_INVALID_ARG (null pointer, eps negative or not finite),
 *         TSP_ERR_ALIGNMENT.
 */
tsp_status tsp_rms_norm(int64_t n_tokens, int32_t hidden, const uint16_t* x, const uint16_t* gain, float eps,
                        uint16_t* y, hipStream_t stream);

/*
 * Rotary position embedding (RoFormer, Su et al. 2021; the interleaved pairs of
 * that paper), in place, at the tokens' global zigzag positions p: in every
 * head the pair (x_{2i}, x_{2i+1}) is rotated by p * theta^(-2i/head_dim).
 *   q      : device, bf16 [n_local x n_heads*head_dim], nullable; local row t
 *            is at the plan's global position of t.
 *   k_full : device, bf16 [seq_len x n_kv_heads*head_dim], nullable; only the
 *            rank's own rows are rotated (the other ranks rotate theirs before
 *            the all-gather).
 *   theta  : > 1 (10000 in RoFormer).  Angles and their sine and cosine are
 *            computed in fp64, the rotation in fp32, the result rounded to bf16.
 * Errors: as tsp_zigzag_plan's plan check; TSP_ERR_SHAPE (non-positive sizes),
 *         TSP_ERR_UNSUPPORTED (head_dim % 8), TSP_ERR_INVALID_ARG (theta).
 */
tsp_status tsp_rope(const tsp_plan* plan, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, double theta,
                    uint16_t* q, uint16_t* k_full, hipStream_t stream);

/*
 * Backward of tsp_rope: the rotation of each pair is orthogonal, so the
 * gradient is the rotation by -angle, applied in place to fp32 gradients:
 *   dq     : device, fp32 [n_local x n_heads*head_dim], nullable; local rows.
 *   dk_own : device, fp32 [n_local x n_kv_heads*head_dim], nullable: the
 *            gradients of the rank's own K rows, in local row order (its rows
 *            of the K gradients after every rank's contributions are summed).
 * Errors: as tsp_rope, plus TSP_ERR_INVALID_ARG when dq and dk_own coincide.
 */
tsp_status tsp_rope_backward(const tsp_plan* plan, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                             double theta, float* dq, float* dk_own, hipStream_t stream);

/*
 * Backward of tsp_rms_norm (Zhang & Sennrich 2019): with r = sqrt(mean x^2 + eps)
 * per row and t = sum_j gain_j dy_j x_j,
 *   dx_j = gain_j dy_j / r - x_j t / (hidden r^3)      (bf16 out)
 *   dgain_j = sum over the rows of dy_j x_j / r        (fp32 out, summed in a
 *                                                       fixed order: deterministic)
 *   x, gain, dy : device, bf16 ([n x hidden], [hidden], [n x hidden]); hidden % 8 == 0, <= 8192.
 *   dx     : device, bf16 [n x hidden], out; aliases neither x nor dy.
 *   dgain  : device, fp32 [hidden], out.
 *   workspace: >= tsp_workspace_size(n_tokens, dims with this hidden, 1, TSP_WS_RMS_BWD)
 *              bytes (fp32 partial sums per 32-row block).
 * n_tokens = 0 writes dgain = 0 and nothing else; x, dy, dx may then be null.
 */
tsp_status tsp_rms_norm_backward(int64_t n_tokens, int32_t hidden, const uint16_t* x, const uint16_t* gain, float eps,
                                 const uint16_t* dy, uint16_t* dx, float* dgain, void* workspace, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * Grouped-query attention (Ainslie et al. 2023): n_kv_heads K/V heads, query
 * head a reads K/V head a / (n_heads / n_kv_heads).
 * tsp_attn_project_gqa: tsp_attn_project with shard d's weights
 *   wqkv[d] bf16 [(H_s + 2 Hkv_s) * head_dim x hidden], columns [Q heads | K
 *   heads | V heads] (H_s = n_heads / D query heads, Hkv_s = n_kv_heads / D K/V
 *   heads), k_full / v_full [seq_len x n_kv_heads * head_dim].
 * tsp_attn_core_gqa: tsp_attn_core with k_full / v_full
 *   [seq_len x n_kv_heads * head_dim]; the workspace of tsp_attn_core
 *   (TSP_WS_CORE) is enough.
 *   n_kv_heads : divides n_heads (and, for the projection, is a multiple of D).
 * Errors: as the MHA calls, plus TSP_ERR_SHAPE for n_kv_heads.
 */
tsp_status tsp_attn_project_gqa(const tsp_plan* plan, const tsp_dims* dims, int32_t n_kv_heads,
                                const uint16_t* x_local, const uint16_t* const* wqkv, uint16_t* k_full,
                                uint16_t* v_full, uint16_t* q_out, hipStream_t stream);
tsp_status tsp_attn_core_gqa(const tsp_plan* plan, const tsp_dims* dims, int32_t n_kv_heads, const uint16_t* q,
                             const uint16_t* k_full, const uint16_t* v_full, uint16_t* attn_out, uint16_t* attn_lo,
                             void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Grouped-query forms of tsp_attn_core_lse and tsp_attn_core_backward: k_full,
 * v_full, dk_full and dv_full are [seq_len x n_kv_heads*head_dim]; the K/V
 * gradients of one K/V head sum over the n_heads / n_kv_heads query heads that
 * read it.  Workspaces: TSP_WS_CORE and TSP_WS_ATTN_BWD (those of MHA) are
 * enough.  Errors: as the MHA calls, plus TSP_ERR_SHAPE for n_kv_heads.
 */
tsp_status tsp_attn_core_gqa_lse(const tsp_plan* plan, const tsp_dims* dims, int32_t n_kv_heads, const uint16_t* q,
                                 const uint16_t* k_full, const uint16_t* v_full, uint16_t* attn_out,
                                 uint16_t* attn_lo, float* lse, void* workspace, size_t ws_bytes,
                                 hipStream_t stream);
tsp_status tsp_attn_core_gqa_backward(const tsp_plan* plan, const tsp_dims* dims, int32_t n_kv_heads,
                                      const uint16_t* q, const uint16_t* k_full, const uint16_t* v_full,
                                      const uint16_t* attn_out, const uint16_t* attn_lo, const float* lse,
                                      const uint16_t* d_attn, float* dq, float* dk_full, float* dv_full,
                                      void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Backward pass of the MLP ring for the rank's own tokens (the pages describe
 * the forward schedule; this is its chain rule).  For the forward
 * y = [x +] sum_d GELU_tanh(x W1_d^T) W2_d^T and dy = dL/dy:
 *   U_d = x W1_d^T,  dU_d = (dy W2_d) * GELU'(U_d)
 *   dx    = [dy +] sum_k dU_{d_k} W1_{d_k},  d_k = (start_shard + k) mod D
 *           (the ring's split-K, fp32 across all shards, like the forward W2)
 *   dW1_d = dU_d^T x        fp32 [ffn/D x hidden]
 *   dW2_d = dy^T GELU(U_d)  fp32 [hidden x ffn/D]
 * The weight gradients are this rank's contributions over its tokens: shard
 * d's full gradient is the sum of the D ranks' contributions (the
 * reduce-scatter to the shard's owner).  Operands are bf16 with fp32
 * accumulation; U is kept in fp32, dU and GELU(U) are rounded to bf16.
 *   residual : nonzero when the forward added x (then dx includes dy).
 *   x, dy    : device, bf16 [n_tokens x hidden].
 *   w1, w2   : host arrays of D device pointers, bf16, as tsp_mlp_forward.
 *   dx       : device, bf16 [n_tokens x hidden]; must not alias x or dy.
 *   dw1, dw2 : host arrays of D device pointers, fp32 [ffn/D x hidden] and
 *              [hidden x ffn/D], overwritten.
 *   workspace: >= tsp_workspace_size(n_tokens, dims, D, TSP_WS_MLP_BWD) bytes.
 * n_tokens = 0 writes zero weight gradients and nothing else; the token
 * buffers and the workspace may then be null.
 * Errors: as tsp_mlp_forward.
 */
tsp_status tsp_mlp_backward(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t start_shard,
                            int32_t residual, const uint16_t* x, const uint16_t* const* w1,
                            const uint16_t* const* w2, const uint16_t* dy, uint16_t* dx, float* const* dw1,
                            float* const* dw2, void* workspace, size_t ws_bytes, hipStream_t stream);

/* Per-rank memory of a decoder stack, in bytes (see tsp_memory_footprint). */
typedef struct {
  uint64_t weights;      /* own 1/D share of every layer's weights, bf16 */
  uint64_t streamed;     /* TSP: the D-1 other weight shards of the layer being computed, bf16 */
  uint64_t kv;           /* TSP: gathered K and V of one layer [S x hidden]; TP: own heads' K, V [S x hidden/D] */
  uint64_t activations;  /* token buffers and workspace of one layer's forward */
  uint64_t train_state;  /* training: bf16 grads, fp32 master weights, Adam m and v of the own share,
                            and every layer's input kept for recomputation */
  uint64_t grads;        /* training: fp32 weight-gradient contributions of one layer */
  uint64_t total;
} tsp_memory;

/* Layouts compared by tsp_memory_footprint. */
typedef enum {
  TSP_MEM_TSP = 0, /* TSP: one axis of size D shards weights and tokens (S/D local tokens) */
  TSP_MEM_TP = 1   /* plain tensor parallelism: heads and FFN sharded, all S tokens on every rank */
} tsp_mem_scheme;

/*
 * Per-rank memory accounting for n_layers decoder layers of `dims` at total
 * sequence seq_len on an axis of D ranks, for comparing TSP with plain tensor
 * parallelism (zubnet.ai TSP page, para. 1: parameter and activation memory
 * both fall by 1/D under TSP; para. 2: 38.8 GB per GPU for TSP against 70.0 GB
 * for plain TP at 128K tokens on 8 GPUs, with what those hold not stated).
 * Counted, per rank (host arithmetic only, nothing allocated):
 *   weights     : n_layers * (4 h^2 + 2 h F) / D parameters, 2 bytes each (both schemes);
 *   streamed    : TSP only, the other D-1 shards of one layer, which this
 *                 library's per-layer calls take resident (0 for TP and D = 1);
 *   kv          : TSP 2 * S * h * 2 bytes (the gathered K/V of one layer);
 *                 TP 2 * S * (h/D) * 2 bytes (the rank's heads, no gather);
 *   activations : one layer's forward with this library's kernels: the input
 *                 and output rows plus tsp_workspace_size(n, ., D, TSP_WS_LAYER)
 *                 for TSP (n = S/D tokens, all heads); for TP the same buffers
 *                 for all S tokens with the rank's H/D heads and F/D FFN
 *                 columns (attention workspace, fp16 weight copies and GELU
 *                 block narrowed, token rows of width h full);
 *   train_state : training != 0 only: 14 bytes per own parameter (bf16 grad,
 *                 fp32 master, Adam m and v) plus n_layers layer inputs,
 *                 [tokens x h] bf16 (full recomputation of each layer);
 *   grads       : training != 0 only: the fp32 weight-gradient contributions
 *                 of one layer that the backward writes before they are
 *                 reduced to the shard owners: every shard under TSP
 *                 ((4 h^2 + 2 h F) * 4 bytes), the own shard under TP;
 *   total       : the sum.
 * The backward calls' own workspaces (tsp_workspace_size, kinds *_BWD) and
 * the embedding and output layers are not counted.  With D = 1 both schemes
 * count the same buffers.
 *   dims  : as tsp_layer_forward (head_dim 64 or 128, H % D == 0, F/D % 64 == 0).
 *   out   : host out, required.
 * Errors: TSP_ERR_INVALID_ARG (out or dims null, D out of range, n_layers < 0,
 *         unknown scheme), TSP_ERR_SHAPE / TSP_ERR_UNSUPPORTED (as
 *         tsp_zigzag_plan and tsp_layer_forward for S, D and dims).
 */
tsp_status tsp_memory_footprint(int64_t seq_len, const tsp_dims* dims, int32_t D, int32_t n_layers,
                                int32_t scheme, int32_t training, tsp_memory* out);

/* Static text for a status code (never null). */
const char* tsp_status_string(tsp_status status);

#ifdef __cplusplus
}
#endif

#endif /* TSP_H */
