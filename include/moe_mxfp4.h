/*
 * moe_mxfp4.h - C ABI of the MI355X (gfx950) routed-expert MXFP4 MoE decode layer.
 *
 * One call computes, for one expert-parallel slice of a mixture-of-experts
 * layer, top-k routing, the fused gate/up projection with its activation, the
 * down projection and the routing-weighted combine, reading every weight
 * straight from packed OCP MXFP4.
 *
 * Sources (page, section):
 *  - "MXFP4 MoE decode kernels", Design, Read the served layout: the tensor
 *    layouts below; The bottleneck: E2M1 values two per byte, one E8M0 scale
 *    per 32 values; Design, Fused epilogues: bias and activation in fp32, bf16
 *    intermediate, routing-weighted bias added once per route, fp32 per-token
 *    sums, bf16 output; Design, Routing inside the kernel: routes are counting
 *    sorted by local expert and routes to other ranks are skipped; Limitations
 *    and pitfalls: unsupported inputs are refused with a reason, and unexpected
 *    dtypes must be rejected.
 *  - "GLM-5.2 and GLM-5.3 (744B) in MXFP4 on Gaudi 2", What was built,
 *    Byte-exact repack: E2M1 low nibble first, E8M0 scales, blocks of 32; Why it
 *    needed a port, items 1, 2 and 4: w13 rows are [gate; up], experts are
 *    sliced by expert-parallel rank, routing ids are int32.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers, row-major and contiguous, owned by
 *    the caller; the library allocates nothing, never synchronises and never
 *    logs.  Work is enqueued on `stream` (a hipStream_t; NULL is the default
 *    stream) and runs asynchronously, like a kernel launch.
 *  - A workspace is in use until the work enqueued with it has completed on
 *    its stream: calls that may overlap (other streams or threads) need
 *    distinct workspaces, and a workspace freed or reused elsewhere before
 *    then gives wrong results or faults (the plan it holds is read by the
 *    later kernels of the call).
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - Every argument check runs on the host before anything is enqueued: on
 *    any status other than MOE_ERR_HIP nothing has been launched and no
 *    output has been written.  MOE_ERR_HIP reports the first launch the HIP
 *    runtime refused (each launch's own status; errors left by other work on
 *    the thread are neither reported nor cleared); the launches of the call
 *    before it stay enqueued, so outputs may be partly written.
 *  - Size limits below (K, I <= 8192; E_local <= 512; top_k <= 64; E_global
 *    <= 1024 in router-logits mode; T * top_k <= 2^24) are this library's,
 *    not the pages': they size its on-chip buffers (per-row scale strips of
 *    K/32 or I/32 bytes in LDS, one 16-lane histogram row per local expert,
 *    one lane per route of a token, 16 logits per lane in the top-k wave)
 *    and its 32-bit buffer offsets.  Calls outside them are refused with
 *    MOE_ERR_SHAPE, never served by another path.
 *  - Status codes are the MOE_* values below; moe_mxfp4_status_string() names
 *    them.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MOE_OK             0
#define MOE_ERR_NULL      (-1)  /* a required pointer is NULL                          */
#define MOE_ERR_SHAPE     (-2)  /* a size is out of range (see moe_mxfp4_desc)        */
#define MOE_ERR_MODE      (-3)  /* both or neither routing input; bad enum value       */
#define MOE_ERR_ALIGN     (-4)  /* a tensor pointer is not 16-byte aligned             */
#define MOE_ERR_WORKSPACE (-5)  /* workspace NULL or smaller than the query says       */
#define MOE_ERR_HIP       (-6)  /* the HIP runtime refused a launch of this call         */

/* ---- enums ------------------------------------------------------------- */
#define MOE_SCORING_SOFTMAX 0   /* softmax over the top_k selected logits             */
#define MOE_SCORING_SIGMOID 1   /* sigmoid(logit) renormalised over the top_k selected */

#define MOE_ACT_SILU_MUL    0   /* a = silu(gate) * up                                 */
#define MOE_ACT_SWIGLU_OAI  1   /* g = min(gate, L), u = clamp(up, -L, L),
                                   a = g * sigmoid(alpha * g) * (u + 1)                */

#define MOE_DTYPE_F32  0
#define MOE_DTYPE_BF16 1

/* Shared-exponent rule of the MXFP4 encoder (moe_mxfp4_encode).             */
#define MOE_ENCODE_OCP     0    /* shared exponent floor(log2(amax)) - 2             */
#define MOE_ENCODE_QUARK   1    /* the same, plus one when amax / 2^X >= 7           */

/* Storage order of the packed weights w13_packed and w2_packed (scales always
 * keep the row layout).  MOE_LAYOUT_TILE16 is this library's own order, made
 * in place from the row layout by moe_mxfp4_tile_weights(): in every group of
 * 16 consecutive rows, the 16-byte blocks (32 values each) are stored
 * block-major, block b of row r at byte 256*b + 16*r of the group.  Each step
 * of the expert kernels then reads one contiguous 1 KB run per wave; the row
 * layout is read in 64-byte pieces of 16 rows.  Same bytes, one copy.       */
#define MOE_LAYOUT_ROWS    0    /* the served layout of "Read the served layout"      */
#define MOE_LAYOUT_TILE16  1

/* Row order of w13_packed, w13_scales and w13_bias ("MXFP4 MoE decode
 * kernels", Beyond gpt-oss: kernels for [gate; up] rows and for interleaved
 * gate/up rows).  GATE_UP: row n < I is gate row n, row I + n is up row n.
 * INTERLEAVED: row 2n is gate row n, row 2n + 1 is up row n.  The activation
 * (desc.activation) is chosen independently of the order.                   */
#define MOE_W13_GATE_UP      0
#define MOE_W13_INTERLEAVED  1

/* Row pairing of the down projection (a performance control; the results
 * are bit-identical either way).  Paired, each wave of the stream kernel, or
 * of the MFMA kernel at many routes per expert, computes two 16-row sets 16
 * rows apart, so every step loads two weight blocks per lane and each
 * activation fragment feeds two MFMAs, as in the gate/up projection; it
 * needs K % 32 == 0.  AUTO pairs when the paired work items still fill every
 * resident workgroup slot of the GPU.                                        */
#define MOE_PAIRING_AUTO   0
#define MOE_PAIRING_ON     1    /* whenever K % 32 == 0                               */
#define MOE_PAIRING_OFF    2

/* Matrix instructions for experts with many routes in one call (the MFMA
 * list path; calls served by the decode-regime stream kernel and experts
 * with one or two routes are not affected).
 *   BF16:       each E2M1 weight block is decoded with its E8M0 scale to bf16
 *               in registers and fed to v_mfma_f32_16x16x32_bf16 with the bf16
 *               activations (exact products, fp32 sums).
 *   SCALED_FP4: the packed E2M1 blocks and E8M0 scales go to
 *               v_mfma_scale_f32_16x16x128_f8f6f4 as stored; the activations
 *               are first split, row by row, into hi + lo E4M3 parts with one
 *               E8M0 scale each (about the precision of bf16), and every
 *               128-value chunk takes two scaled MFMAs.  Needs extra
 *               workspace for the split rows (moe_mxfp4_workspace_bytes
 *               includes it).                                              */
#define MOE_MMA_BF16        0
#define MOE_MMA_SCALED_FP4  1

/* ---- layer descriptor --------------------------------------------------- */
typedef struct moe_mxfp4_desc {
    int32_t T;              /* tokens in the call, >= 0 (T = 0 is a no-op); T * top_k
                               <= 2^24, and x (T * K) and the intermediate
                               (T * top_k * I, bf16) each below 2 GiB                   */
    int32_t K;              /* hidden size, multiple of 32, 32..8192                      */
    int32_t I;              /* intermediate size per expert, multiple of 32, 32..8192     */
    int32_t E_global;       /* experts the router scores, >= 1 (<= 1024 with logits)     */
    int32_t E_local;        /* experts held in w13/w2, 1..512                             */
    int32_t expert_offset;  /* global id of local expert 0; the slice is
                               [expert_offset, expert_offset + E_local) within E_global */
    int32_t top_k;          /* routes per token, 1..min(64, E_global)                    */
    int32_t scoring;        /* MOE_SCORING_*  (used in router-logits mode only)          */
    int32_t activation;     /* MOE_ACT_*                                                  */
    float   swiglu_alpha;   /* 1.702 for gpt-oss  (MOE_ACT_SWIGLU_OAI only)              */
    float   swiglu_limit;   /* 7.0 for gpt-oss    (MOE_ACT_SWIGLU_OAI only)              */
    int32_t weight_layout;  /* MOE_LAYOUT_* of w13_packed and w2_packed                   */
    int32_t down_pairing;   /* MOE_PAIRING_* (0 = automatic)                              */
    int32_t w13_order;      /* MOE_W13_* row order of the w13 tensors                      */
    int32_t mma;            /* MOE_MMA_* for experts with many routes (0 = bf16); with
                               SCALED_FP4 the split rows, T * 256 * ceil(K / 128) and
                               T * top_k * 256 * ceil(I / 128) bytes, each below 2 GiB  */
} moe_mxfp4_desc;

/*
 * Device workspace needed by moe_mxfp4_decode / _gate_up / _down / _bucket for
 * this descriptor (host-only query, nothing is launched).  It holds the routing
 * table, the bucketing plan, the bf16 intermediate and the per-route fp32 down
 * projection, each sized for the worst case T*top_k local routes.
 * Returns MOE_OK and writes *bytes, or MOE_ERR_NULL / MOE_ERR_SHAPE / MOE_ERR_MODE.
 */
int moe_mxfp4_workspace_bytes(const moe_mxfp4_desc* desc, size_t* bytes);

/*
 * The layer call ("MXFP4 MoE decode kernels", Design: gate/up GEMV + bias +
 * activation, then down GEMV + routing-weighted bias + weighted sum per token).
 *
 *  x            bf16 [T, K]
 *  router_logits fp32 [T, E_global], or NULL  (router-logits mode: top_k by
 *               logit descending, ties to the lower id; weights per `scoring`)
 *  topk_ids     int32 [T, top_k] global expert ids, or NULL   (ids mode:
 *  topk_weights fp32 [T, top_k], or NULL       weights are used as given)
 *               Exactly one of router_logits and (topk_ids, topk_weights)
 *               must be given, else MOE_ERR_MODE.  Ids outside the local
 *               slice (including -1 padding) are skipped; a repeated id is a
 *               separate route.
 *  w13_packed   u8 [E_local, 2I, K/2]: rows in desc->w13_order (GATE_UP:
 *               row n < I is gate row n, row I+n is up row n); byte c of a
 *               row holds element 2c in its low nibble and element 2c+1 in
 *               its high nibble (E2M1 codes)
 *  w13_scales   u8 [E_local, 2I, K/32]: E8M0 scale of elements 32b..32b+31
 *  w13_bias     bf16 [E_local, 2I], or NULL (added to the fp32 projection
 *               before the activation)
 *  w2_packed    u8 [E_local, K, I/2]: row k is output feature k
 *  w2_scales    u8 [E_local, K, I/32]
 *  w2_bias      bf16 [E_local, K], or NULL (added once per route, before the
 *               routing weight multiplies)
 *  out          bf16 [T, K], fully overwritten; a token with no local route
 *               gets zeros (the slice's partial sum; an expert-parallel caller
 *               sums the slices)
 *  workspace    device buffer of at least moe_mxfp4_workspace_bytes() bytes,
 *               16-byte aligned; contents on entry are ignored
 *
 * Pointers to x, the packed weights, the scales, the biases (when given), out
 * and workspace must be 16-byte aligned (MOE_ERR_ALIGN); the same holds for
 * every entry point below.  Preconditions not checked: finite x and logits,
 * buffers of the stated sizes.  Results are deterministic: no
 * floating-point atomics; a call repeated on the same inputs is bit-identical.
 */
int moe_mxfp4_decode(const moe_mxfp4_desc* desc,
                     const uint16_t* x,
                     const float* router_logits,
                     const int32_t* topk_ids, const float* topk_weights,
                     const uint8_t* w13_packed, const uint8_t* w13_scales, const uint16_t* w13_bias,
                     const uint8_t* w2_packed, const uint8_t* w2_scales, const uint16_t* w2_bias,
                     uint16_t* out,
                     void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * moe_mxfp4_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a fixed array of
 * MOE_SCRATCH_BYTES in the library's device memory, one per GPU, held until
 * the process ends; nothing is allocated or freed in the call.  Arguments,
 * results and errors are those of moe_mxfp4_decode, plus MOE_ERR_WORKSPACE
 * when moe_mxfp4_workspace_bytes() of the descriptor exceeds
 * MOE_SCRATCH_BYTES (e.g. up to T * top_k = 256 routes at K = 7168,
 * I = 2048), and MOE_ERR_HIP when the array's device address cannot be
 * found.  Every call on one GPU uses that GPU's one array: calls that may
 * overlap on a GPU (other streams or host threads) race and give wrong
 * results; serialise them, or use moe_mxfp4_decode with distinct workspaces.
 */
#define MOE_SCRATCH_BYTES ((size_t)64 << 20)
int moe_mxfp4_decode_noalloc(const moe_mxfp4_desc* desc,
                             const uint16_t* x,
                             const float* router_logits,
                             const int32_t* topk_ids, const float* topk_weights,
                             const uint8_t* w13_packed, const uint8_t* w13_scales, const uint16_t* w13_bias,
                             const uint8_t* w2_packed, const uint8_t* w2_scales, const uint16_t* w2_bias,
                             uint16_t* out, void* stream);

/*
 * The three steps of moe_mxfp4_decode, callable one by one on the same
 * workspace (decode = plan, then gate_up, then down, with identical launches).
 *
 * moe_mxfp4_plan: routing and bucketing.  With router_logits (fp32
 * [T, E_global]) it runs the top-k router; with topk_ids + topk_weights it
 * takes them as given (exactly one mode, else MOE_ERR_MODE).  It then
 * counting-sorts the local routes by local expert into the workspace ("MXFP4
 * MoE decode kernels", Design, Routing inside the kernel) and keeps a copy of
 * the routing weights there, so later steps read nothing else of the caller's
 * routing inputs.
 */
int moe_mxfp4_plan(const moe_mxfp4_desc* desc, const float* router_logits,
                   const int32_t* topk_ids, const float* topk_weights,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_mxfp4_gate_up: for every local route of the plan, the gate/up projection
 * of its token with bias and activation, rounded to bf16 ("MXFP4 MoE decode
 * kernels", Design, Fused epilogues).  Writes the intermediate a
 * [T*top_k, I] bf16 whose row p (p < local routes) belongs to the p-th route
 * of the plan's order (see moe_mxfp4_bucket); rows past the local routes are
 * not written.  a == NULL writes the workspace's own copy (what
 * moe_mxfp4_down reads when its a is NULL).  Needs moe_mxfp4_plan first.
 */
int moe_mxfp4_gate_up(const moe_mxfp4_desc* desc, const uint16_t* x,
                      const uint8_t* w13_packed, const uint8_t* w13_scales, const uint16_t* w13_bias,
                      uint16_t* a, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_mxfp4_down: down projection of every local route's intermediate row
 * (a [>= local routes, I] bf16 in plan order, or NULL for the workspace copy),
 * plus the w2 bias, then out [T, K] bf16 = per token, the sum over its local
 * routes in route order of weight * (W2 a + b2) ("MXFP4 MoE decode kernels",
 * Design, Fused epilogues).  Tokens without a local route get zeros.  Needs
 * moe_mxfp4_plan first.
 */
int moe_mxfp4_down(const moe_mxfp4_desc* desc, const uint16_t* a,
                   const uint8_t* w2_packed, const uint8_t* w2_scales, const uint16_t* w2_bias,
                   uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-route output ("MXFP4 MoE decode kernels", Beyond gpt-oss: a down kernel
 * with one output row per route, for models that apply a per-route operation
 * before the token sum).  Same arguments as moe_mxfp4_decode and
 * moe_mxfp4_down, except the output:
 *  out_routes   fp32 [T * top_k, K], fully overwritten: row r = t*top_k + j
 *               holds W2 a_r + b2 of route r (no routing weight) when the
 *               route's expert is in the local slice, else zeros.  The routing
 *               weights of logits mode are in no output; moe_mxfp4_route
 *               computes the same ones.
 * moe_mxfp4_decode_routes runs plan, gate_up and the per-route down step;
 * moe_mxfp4_down_routes is the last step alone, on a workspace that holds a
 * plan (and, when a is NULL, the gate/up result).
 */
int moe_mxfp4_decode_routes(const moe_mxfp4_desc* desc,
                            const uint16_t* x,
                            const float* router_logits,
                            const int32_t* topk_ids, const float* topk_weights,
                            const uint8_t* w13_packed, const uint8_t* w13_scales, const uint16_t* w13_bias,
                            const uint8_t* w2_packed, const uint8_t* w2_scales, const uint16_t* w2_bias,
                            float* out_routes,
                            void* workspace, size_t workspace_bytes,
                            void* stream);
int moe_mxfp4_down_routes(const moe_mxfp4_desc* desc, const uint16_t* a,
                          const uint8_t* w2_packed, const uint8_t* w2_scales, const uint16_t* w2_bias,
                          float* out_routes, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Prefill path ("MXFP4 MoE decode kernels", Prefill: unpack once, then the
 * stock op): the touched experts' weights are unpacked to bf16 in the
 * workspace in one pass, then grouped MFMA GEMMs read the bf16 weights.  Same
 * arguments and results as moe_mxfp4_decode (the products are the same in
 * the same order: outputs are bit-identical to moe_mxfp4_decode wherever the
 * latter takes its MFMA path), with a larger workspace:
 * moe_mxfp4_prefill_workspace_bytes() = the decode workspace plus
 * E_local * 3 * I * K bf16 values (the unpacked w13 and w2 of every local
 * expert; untouched experts' regions are left unwritten).  This path moves
 * about five times the bytes of the decode path (unpacked bf16 weights are
 * read back after being written) and exists for callers that want the
 * pages' prefill structure; moe_mxfp4_decode serves every token count.
 */
int moe_mxfp4_prefill_workspace_bytes(const moe_mxfp4_desc* desc, size_t* bytes);
int moe_mxfp4_prefill(const moe_mxfp4_desc* desc,
                      const uint16_t* x,
                      const float* router_logits,
                      const int32_t* topk_ids, const float* topk_weights,
                      const uint8_t* w13_packed, const uint8_t* w13_scales, const uint16_t* w13_bias,
                      const uint8_t* w2_packed, const uint8_t* w2_scales, const uint16_t* w2_bias,
                      uint16_t* out,
                      void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * The unpack step alone: for every local expert with a route in the plan held
 * in `workspace` (moe_mxfp4_plan first), w13_out bf16 [E_local, 2I, K] and
 * w2_out bf16 [E_local, K, I] get the exact values of the packed weights
 * (every E2M1 x E8M0 product is a bf16 value), in the stored row order and
 * the row layout whatever desc->weight_layout says; other experts' rows are
 * not written.  Pointers 16-byte aligned.
 */
int moe_mxfp4_unpack(const moe_mxfp4_desc* desc, const uint8_t* w13_packed, const uint8_t* w13_scales,
                     const uint8_t* w2_packed, const uint8_t* w2_scales, uint16_t* w13_out, uint16_t* w2_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Routing step alone (test hook, the router of calls with T > 64; smaller
 * calls route inside moe_mxfp4_plan with the same selection and weights):
 * router logits fp32 [T, E_global] -> ids int32 [T, top_k] (logit
 * descending, ties to the lower id; a NaN logit ranks below every number)
 * and weights fp32 [T, top_k] (softmax over the selected logits, or sigmoid
 * renormalised over the selected, per desc->scoring).  Sources: "MXFP4 MoE
 * decode kernels", At a glance and Parity (gpt-oss's top-4 softmax routing);
 * "GLM-5.3-Flash on Gaudi 2", Why (top-8 sigmoid scoring); "GLM-5.2 and
 * GLM-5.3 (744B) in MXFP4 on Gaudi 2", Why it needed a port, item 4 (int32
 * ids).  E_global <= 1024 (MOE_ERR_SHAPE); all pointers device pointers.
 */
int moe_mxfp4_route(const moe_mxfp4_desc* desc, const float* router_logits,
                    int32_t* topk_ids, float* topk_weights, void* stream);

/*
 * Bucketing step alone (test hook): ids int32 [T, top_k] -> per local expert
 * counts int32 [E_local], exclusive offsets int32 [E_local + 1], and
 * routes int32 [T*top_k] whose first offsets[E_local] entries are the local
 * route indices r = t*top_k + j grouped by local expert, ascending r inside
 * each group (a stable counting sort); the remaining entries are -1.  Ids
 * outside [expert_offset, expert_offset + E_local) (including -1 padding)
 * are not local.  Source: "MXFP4 MoE decode kernels", Design, Routing inside
 * the kernel (routes counting-sorted by local expert, routes to other
 * expert-parallel ranks skipped); "GLM-5.2 and GLM-5.3 (744B) in MXFP4 on
 * Gaudi 2", Why it needed a port, item 2 (experts sliced by rank).  Needs
 * the workspace of moe_mxfp4_workspace_bytes(); its contents afterwards hold
 * no plan a layer step can use.
 */
int moe_mxfp4_bucket(const moe_mxfp4_desc* desc, const int32_t* topk_ids,
                     int32_t* counts, int32_t* offsets, int32_t* routes,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * MXFP4 -> dense dequantisation (test hook): packed u8 [rows, cols/2] (row
 * layout) + scales u8 [rows, cols/32] -> out [rows, cols] as fp32
 * (out_dtype MOE_DTYPE_F32) or bf16 bits (MOE_DTYPE_BF16).  Value =
 * E2M1(code) * 2^(scale - 127) with code of element 2c the low nibble of
 * byte c, scale 255 -> NaN, computed with the same decode the layer kernels
 * use.  Sources: "GLM-5.2 and GLM-5.3 (744B) in MXFP4 on Gaudi 2", What was
 * built, Byte-exact repack (E2M1 low nibble first, E8M0 scales, blocks of
 * 32); "MXFP4 MoE decode kernels", The bottleneck (two values per byte, one
 * scale per 32).  cols % 32 == 0 (MOE_ERR_SHAPE); packed and out 16-byte
 * aligned (MOE_ERR_ALIGN).
 */
int moe_mxfp4_dequant(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t cols,
                      int32_t out_dtype, void* out, void* stream);

/*
 * Copy of the plan a moe_mxfp4_plan (or a layer call) left in `workspace`
 * (test hook: the routing and bucketing the layer kernels actually used):
 * ids int32 [T, top_k] and weights fp32 [T, top_k] (logits mode: the
 * router's choice, made inside the gate/up launch for the small calls
 * that plan there, inside the plan kernel for other calls of T <= 64 with
 * E_global <= 256, and by the one-wave-per-token router for the rest; ids
 * mode: the caller's), counts int32 [E_local], offsets int32 [E_local + 1]
 * and routes int32 [T*top_k] (local route indices grouped by local expert,
 * -1 past the local routes), as moe_mxfp4_route and moe_mxfp4_bucket define
 * them.  Any output may be NULL (not written).  Same descriptor as the call
 * that planned; enqueued on `stream` after it.
 */
int moe_mxfp4_plan_read(const moe_mxfp4_desc* desc, const void* workspace, size_t workspace_bytes,
                        int32_t* topk_ids, float* topk_weights, int32_t* counts, int32_t* offsets,
                        int32_t* routes, void* stream);

/*
 * MXFP4 encoder ("GLM-5.2 and GLM-5.3 (744B) in MXFP4 on Gaudi 2", What was
 * built, MXFP4 encoder): in [rows, cols] fp32 (in_dtype MOE_DTYPE_F32) or
 * bf16 bits (MOE_DTYPE_BF16) -> packed u8 [rows, cols/2] (element 2c in the
 * low nibble of byte c) and scales u8 [rows, cols/32] (E8M0).  Per block of
 * 32: X = floor(log2(amax)) - 2 (MOE_ENCODE_OCP), plus one when
 * amax / 2^X >= 7 (MOE_ENCODE_QUARK); each element v / 2^X rounds to the
 * nearest E2M1 value with ties to the even code, saturating at 6, and keeps
 * the sign bit of v; amax = 0 gives scale byte 0; X is clipped to
 * [-127, 127].  Inputs must be finite.  cols % 32 == 0 (MOE_ERR_SHAPE);
 * in and packed 16-byte aligned (MOE_ERR_ALIGN).  A weight-preparation step
 * (the input of the layer), not part of a layer call.
 */
int moe_mxfp4_encode(const void* in, int32_t in_dtype, int64_t rows, int64_t cols, int32_t rule,
                     uint8_t* packed, uint8_t* scales, void* stream);

/*
 * In-place change of packed weight storage order between MOE_LAYOUT_ROWS and
 * MOE_LAYOUT_TILE16 (inverse = 0: rows -> tiled; 1: tiled -> rows).
 * packed: u8 [rows, cols/2], e.g. w13_packed as [E_local * 2I, K/2] or
 * w2_packed as [E_local * K, I/2]; rows % 16 == 0, cols % 32 == 0 and
 * 32 <= cols <= 8192 (MOE_ERR_SHAPE), packed 16-byte aligned (MOE_ERR_ALIGN).
 * A one-time step at weight load: a call that overlaps a layer call reading
 * the same weights races with it.
 */
int moe_mxfp4_tile_weights(uint8_t* packed, int64_t rows, int64_t cols, int32_t inverse, void* stream);

/* Static string naming a status code. */
const char* moe_mxfp4_status_string(int status);

/* Static version string of the library build. */
const char* moe_mxfp4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
