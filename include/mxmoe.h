/*
 * mxmoe.h -- block-scaled routed-expert MoE layer and dense block-32 FP8
 * projection for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * What is computed (sources are the three web pages on serving DeepSeek V4.1
 * Flash on DGX Spark; the element/scale encodings are those of the OCP
 * Microscaling Formats v1.0 specification, which the pages' "MXFP8"/"MXFP4"
 * names refer to):
 *   - "New Deepseek 4.1 flash recipe" forum thread, post #6, "How it works":
 *     routed experts with FP8 activations x FP4 weights on block-scaled MMAs,
 *     dense MXFP8 projections; post #6, "Why TileLang": MoE top-k gate,
 *     SwiGLU and per-block FP8/FP4 quantization casts, reductions in a fixed
 *     order so a row's result does not depend on its batch.
 *   - same thread, post #2, "What changed": verification rows whose estimated
 *     survival is below 0.2 skip the expert weight reads.
 *   - spark-ds41f README, "Current baseline": block-32 FP8 projections,
 *     FP8 x FP4 routed experts, batch-independent results, decode and prefill.
 *   - DeepSeek-V4.1-Flash-4x-DGX-Spark-TP4 README, settings table, row
 *     "Experts": per-slot buffer and a fixed-order sum instead of atomics.
 *
 * Encodings (all byte arrays are row-major, contiguous):
 *   FP8  = E4M3 (bias 7, max 448, S.1111.111 NaN), one byte per element.
 *   FP4  = E2M1 (values 0, .5, 1, 1.5, 2, 3, 4, 6 and negatives), two per
 *          byte, element 2j in the LOW nibble of byte j.
 *   SC   = E8M0 scale 2^(c-127), one byte per 32 consecutive elements along
 *          the reduction (K) dimension; code 255 (NaN) is not supported.
 *   Value of an element = decode(element) * decode(its block's SC).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers (hipMalloc / torch CUDA memory),
 *     16-byte aligned unless stated; the caller owns every buffer.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls
 *     are asynchronous: they validate on the host, launch kernels on
 *     `stream` and return.  They never allocate, free, synchronize or read
 *     device memory on the host, so they can be captured in a HIP graph.
 *   - Every argument is checked on the host BEFORE any launch; on error
 *     nothing is launched and a negative status is returned.  There is no
 *     fallback path and no printing; mx_status_string() names the error.
 *   - Inputs must be finite; NaN/Inf inputs give unspecified (but
 *     deterministic) results.
 *   - Results are deterministic: the same inputs give the same bits, and
 *     each output row is bitwise independent of the other rows in the batch.
 */
#ifndef MXMOE_H
#define MXMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int mx_status;
#define MX_OK            0
#define MX_EINVAL       -1   /* null pointer, bad shape or range */
#define MX_EUNSUPPORTED -2   /* valid request the kernels do not implement */
#define MX_EWORKSPACE   -3   /* workspace missing or too small */
#define MX_EHIP         -4   /* a HIP launch or runtime call failed */

#define MX_FMT_E4M3 0        /* FP8 elements */
#define MX_FMT_E2M1 1        /* FP4 elements, packed two per byte */

#define MX_IN_F32  0         /* fp32 source values */
#define MX_IN_BF16 1         /* bf16 source values (uint16 bit patterns) */

#define MX_OUT_BF16 0        /* bf16 output, round to nearest even from fp32 */
#define MX_OUT_F32  1        /* fp32 output */

/*
 * Block-32 quantizer (the per-block FP8/FP4 casts of post #6, "Why TileLang").
 * src: [rows][cols] fp32 or bf16 (src_dtype).  cols % 32 == 0.
 * q:   E4M3 [rows][cols] bytes, or E2M1 [rows][cols/2] packed bytes.
 * sc:  E8M0 [rows][cols/32].
 * Scale rule (OCP MX v1.0): X = 2^(floor(log2(amax)) - emax) with emax = 8
 * (E4M3) or 2 (E2M1), clamped to codes 0..254; amax == 0 gives code 0.
 * Elements: round to nearest, ties to even, saturate to +-448 / +-6, sign
 * kept (negative values that round to zero give -0).  The routed-expert FFN
 * uses the same device routine for its FP8 requant of the intermediate.
 * src and q must be 16-byte aligned; sc needs no alignment.
 */
mx_status mx_quantize(const void* src, int src_dtype, int64_t rows, int64_t cols, int fmt,
                      uint8_t* q, uint8_t* sc, void* stream);

/*
 * Router logits, the scores the top-k gate ranks (post #6 "How it works"
 * item 3: the MoE top-k gate; "Kernel by kernel against B12X": the router's
 * time per step).  A linear map without bias:
 *   logits[t][e] = sum_j hidden[t][j] * w_gate[e][j]
 * hidden: bf16 [T][H] (uint16 bit patterns), w_gate: bf16 [E][H], both
 * 16-byte aligned, row-major, read only.  logits: fp32 [T][E] (4-byte
 * aligned), written for every (t, e); caller-owned device memory.
 * Products are accumulated in fp32 on the matrix cores in one fixed order
 * per element (K steps of 32, parts of 256 each chained from zero, parts
 * added left to right), the same for every T, so a row's logits never
 * depend on the rows beside it.
 * Supported: T >= 0, E >= 1, H % 32 == 0, 32 <= H <= 16384, and T*H, E*H,
 * T*E < 2^31.  ws: device scratch of at least
 * moe_router_logits_workspace_bytes(T, H, E) bytes (256-byte aligned;
 * contents on entry ignored; may be NULL when that size is 0): few rows
 * (T < 1024) split K over workgroups and keep the per-part sums there.
 * MX_EINVAL for null pointers, misalignment or a bad shape, MX_EWORKSPACE
 * for a missing or short workspace, MX_EUNSUPPORTED beyond the limits.
 * Asynchronous on stream.
 */
size_t    moe_router_logits_workspace_bytes(int T, int H, int E);
mx_status moe_router_logits(const uint16_t* hidden, int T, int H, const uint16_t* w_gate, int E,
                            float* logits, void* ws, size_t ws_bytes, void* stream);

/*
 * Top-k gate + bucketing (post #6 "How it works" item 3: the MoE top-k gate;
 * post #2 "What changed": dead verification rows; TP4 README "Experts": the
 * route planner and per-slot buffer).
 * logits:   fp32 [T][E].  1 <= k <= min(E, 16), E <= 1024, T >= 0.
 * survival: fp32 [T] or NULL (all rows live).  Row t is dead iff
 *           survival[t] < skip_below (strict).  Dead rows keep their ids and
 *           weights but join no bucket; their MoE output rows are +0.
 * Outputs (all device):
 *   topk_ids       int32 [T][k]: experts ordered by (logit descending,
 *                  expert index ascending); exact ties go to the lower index.
 *   topk_w         fp32 [T][k]: softmax over the k selected logits,
 *                  w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).
 *   expert_offsets int32 [E+1]: first bucket position of each expert;
 *                  expert_offsets[E] = P, the number of live pairs.
 *   perm           int32 [T*k]: perm[p] = t*k + j for p < P (pairs sorted by
 *                  expert, then token ascending), -1 for p >= P.
 *   slot_pos       int32 [T][k]: the bucket position p of pair (t, j), or -1.
 * ws: device scratch of at least moe_route_workspace_bytes(T, E, k) bytes
 *     (256-byte aligned); contents on entry are ignored.
 */
size_t    moe_route_workspace_bytes(int T, int E, int k);

/*
 * Top-k gate with router-live verification rows (TP4 README, settings
 * table, row "Verify length": rows the confidence estimate does not expect
 * to survive reuse the anchor row's experts inside the router, so they read
 * no weights the anchor does not, and still get an output).
 * As moe_route, except:
 *   anchor  int32 [T] (device): the anchor row of each row (itself for an
 *           anchor).  Row t with survival[t] < reuse_below (strict) and
 *           0 <= anchor[t] < T takes row anchor[t]'s own top-k experts, in
 *           that row's slot order (whatever its survival), and weights
 *           w_j = exp(l_j - m) / sum_i exp(l_i - m) over its OWN logits l at
 *           those experts (m = their maximum).  Other rows (anchor out of
 *           range or t itself, or survival NULL) keep their own top-k.
 *   Every row is live: all T*k pairs join the buckets, no slot_pos is -1,
 *   expert_offsets[E] = T*k.
 * anchor must be non-null when T > 0.  ws: moe_route_workspace_bytes(T, E, k).
 */
mx_status moe_route_live(const float* logits, int T, int E, int k,
                         const float* survival, float reuse_below, const int32_t* anchor,
                         int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                         int32_t* perm, int32_t* slot_pos,
                         void* ws, size_t ws_bytes, void* stream);
mx_status moe_route(const float* logits, int T, int E, int k,
                    const float* survival, float skip_below,
                    int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                    int32_t* perm, int32_t* slot_pos,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * Routed-expert FFN + fixed-order combine (post #6 "How it works" item 2:
 * routed experts, FP8 activations x FP4 weights; "Why TileLang": SwiGLU,
 * FP8 quantization, fixed-order reductions; TP4 README "Experts").
 * x      FP8 [T][H],  x_sc  SC [T][H/32]          activations
 * w13    FP4 [E][2I][H/2], w13_sc SC [E][2I][H/32] rows [0, I) gate, [I, 2I) up
 * w2     FP4 [E][H][I/2],  w2_sc  SC [E][H][I/32]  down projection
 *        (x, w13, w2 and y 16-byte aligned; x_sc, w13_sc, w2_sc 4-byte)
 * topk_w, expert_offsets, perm, slot_pos: as written by moe_route (k slots).
 * y      fp32 [T][H]: y_t = sum_{j=0..k-1} w_tj * o_tj, added in slot order,
 *        where o_tj = down(requant_fp8(silu(gate) * up)) of pair (t, j);
 *        rows with no live pair are +0.
 * Every product is accumulated in fp32 on the matrix cores in one fixed
 * order per output element, the same for every batch size and path.
 * Supported: H % 128 == 0, I % 32 == 0, 1 <= k <= 16, T*k < 2^31,
 *            T*H < 2^32 (the activations fit 32-bit byte offsets), and a
 *            layer shape that the kernels of the selected path implement
 *            (mx_set_ffn_path; automatic = either): the decode kernels take
 *            H <= 5120 and I <= 2048, the prefill kernels H % 256 == 0 and
 *            I <= 608.  Any other (H, I) returns MX_EUNSUPPORTED before
 *            anything is launched (e.g. H = 6144 with I = 1024).
 * ws: device scratch of at least moe_expert_ffn_workspace_bytes(T,H,E,I,k)
 *     bytes (256-byte aligned).  Its layout is documented for diagnostics
 *     and filled in by moe_ws_layout(): the FP8 intermediate q [T*k][I] and
 *     its scales SC [T*k][I/32] (row p = bucket position, written by every
 *     path) and the o region: the fp32 per-slot outputs o [T*k][H] when
 *     T > 1; for one row (T = 1) its first k*I floats hold the SwiGLU rows
 *     a [k][I] in slot order, which the down kernel requantizes.
 */
size_t    moe_expert_ffn_workspace_bytes(int T, int H, int E, int I, int k);
mx_status moe_ws_layout(int T, int H, int I, int k, size_t* off_q, size_t* off_q_sc, size_t* off_o);
mx_status moe_expert_ffn(const uint8_t* x, const uint8_t* x_sc, int T, int H,
                         const float* topk_w, const int32_t* expert_offsets,
                         const int32_t* perm, const int32_t* slot_pos, int k,
                         const uint8_t* w13, const uint8_t* w13_sc,
                         const uint8_t* w2, const uint8_t* w2_sc, int E, int I,
                         float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, kernels and results, bit for bit, as moe_expert_ffn,
 * with the workspace replaced by a device array inside the library, one per
 * GPU, of moe_expert_ffn_noalloc_max_bytes() bytes (16 MiB), held from the
 * library's first use on that GPU until the process ends.  The call itself
 * allocates and frees nothing.  A shape whose
 * moe_expert_ffn_workspace_bytes(T, H, E, I, k) exceeds that size returns
 * MX_EWORKSPACE before anything is launched (at H = 4096, I = 576: up to
 * about 980 row pairs T*k, e.g. 48 rows at k = 16).  Every call on one GPU
 * uses that GPU's one array: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialized by the caller.  The array keeps
 * the last call's contents; nothing in it needs to start at zero (the work
 * queue counters are cleared by a kernel of each call).  Other arguments and
 * errors as moe_expert_ffn.
 */
size_t    moe_expert_ffn_noalloc_max_bytes(void);
mx_status moe_expert_ffn_noalloc(const uint8_t* x, const uint8_t* x_sc, int T, int H,
                                 const float* topk_w, const int32_t* expert_offsets,
                                 const int32_t* perm, const int32_t* slot_pos, int k,
                                 const uint8_t* w13, const uint8_t* w13_sc,
                                 const uint8_t* w2, const uint8_t* w2_sc, int E, int I,
                                 float* y, void* stream);

/*
 * The routed-expert layer of ONE row in one launch (or two): moe_route and
 * moe_expert_ffn for T = 1 fused, the top-k gate running inside every
 * workgroup (each ranks the row's E logits itself, so the experts' weight
 * loads start without waiting for a route kernel).  With k <= 8 and
 * I <= 640, gate/up and the down projection + combine run in ONE launch:
 * each gate/up workgroup requantizes one block of 32 intermediate values and
 * hands the block's FP8 and scale codes to the down workgroups through the
 * workspace, every 8-byte word carrying a per-call tag beside its payload,
 * while the down workgroups stream their W2 rows.  Nothing in the workspace
 * needs to be cleared first: an eager call's tag is a per-process count
 * (bit 31 clear), so a stale word could only pass for a fresh one after 2^31
 * calls that all left it unwritten; under graph capture a one-thread kernel
 * recorded before the launch advances a call counter kept in the workspace
 * (the 32-bit word after the status word below), and each replay's tag is
 * that count with bit 31 set.  Every wait in that handoff is bounded
 * (20 ms); one that runs out sets bit 0 of the 32-bit status word at byte
 * offset off_o + k * max(H, I) * 4 rounded up to 256 of ws (off_o from
 * moe_ws_layout(1, H, I, k); never expected, and that call's y is then
 * undefined); callers may clear and check that word.  Otherwise the layer
 * runs as two launches.  Both forms give the same bits, and the same arguments and
 * results as moe_route (T = 1, skip mode) followed by moe_expert_ffn (T = 1):
 * topk_ids, topk_w, expert_offsets, perm, slot_pos are written as moe_route
 * writes them, y as moe_expert_ffn, and the workspace's q, its scales and
 * the SwiGLU rows as moe_expert_ffn at T = 1.  Calls that share a workspace
 * must not overlap.  ws: moe_expert_ffn_workspace_bytes(1, H, E, I, k) bytes.
 * Supported: the moe_expert_ffn decode-path shapes (H % 128 == 0, H <= 5120,
 * I <= 2048).
 * (Forum thread post #6, "How it works": the MoE top-k gate and the routed
 * experts; "Kernel by kernel against B12X": router and routed experts are
 * the decode step's largest groups after the dense projections.)
 */
mx_status moe_layer_decode1(const float* logits, int E, int k, const float* survival, float skip_below,
                            const uint8_t* x, const uint8_t* x_sc, int H,
                            const uint8_t* w13, const uint8_t* w13_sc,
                            const uint8_t* w2, const uint8_t* w2_sc, int I,
                            int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                            int32_t* perm, int32_t* slot_pos, float* y,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * The whole MoE layer of ONE row, routed and shared experts, in the launches
 * of moe_layer_decode1 alone, with the shared expert's work carried by its
 * kernels instead of a separate moe_shared_expert call (forum thread post #6,
 * "Kernel by kernel against B12X": the shared expert runs beside the routed
 * experts on a side stream; TP4 README, settings table, row "Kernels").
 * Where moe_layer_decode1 runs in one launch and Is <= 640, this is ONE
 * launch too: the shared gate/up workgroups (8 intermediate columns each)
 * run beside the routed ones and hand their SwiGLU values, as tagged words
 * in the shared workspace part, to the down workgroups, which run the shared
 * down projection of their 16 columns beside the routed one; every wait is
 * bounded, and one that runs out sets bit 0 of the status word at the offset
 * moe_layer_decode1 documents (in the routed part).  Otherwise two launches
 * (the shared gate/up K parts beside the routed gate/up, the shared down
 * tiles beside the routed down projection and combine).  Results, bit for
 * bit: topk_ids, topk_w, expert_offsets, perm,
 * slot_pos and y as moe_layer_decode1; y_shared [H] fp32 as
 * moe_shared_expert(x, x_sc, T = 1, H, sw13, sw13_sc, sw2, sw2_sc, Is).  The
 * skip mask applies to the routed experts only (a dead row still gets its
 * shared expert).  The caller adds y and y_shared.  sw13 FP8 [2Is][H] + SC
 * [2Is][H/32]; sw2 FP8 [H][Is] + SC [H][Is/32]; sw13, sw2 16-byte aligned,
 * their scales and y_shared 4-byte aligned.  Supported: the
 * moe_layer_decode1 shapes and Is % 32 == 0, Is <= 1024 (else
 * MX_EUNSUPPORTED).  ws: moe_layer_decode1_shared_workspace_bytes(H, E, I,
 * k, Is) bytes, 256-byte aligned: the routed part (the moe_expert_ffn
 * layout, moe_ws_layout(1, H, I, k)) padded to 256 bytes, then the shared
 * part (the moe_shared_expert layout at T = 1).  Other arguments and errors
 * as moe_layer_decode1; the workspace size function returns 0 for invalid
 * shapes.
 */
size_t    moe_layer_decode1_shared_workspace_bytes(int H, int E, int I, int k, int Is);
mx_status moe_layer_decode1_shared(const float* logits, int E, int k, const float* survival, float skip_below,
                                   const uint8_t* x, const uint8_t* x_sc, int H,
                                   const uint8_t* w13, const uint8_t* w13_sc,
                                   const uint8_t* w2, const uint8_t* w2_sc, int I,
                                   const uint8_t* sw13, const uint8_t* sw13_sc,
                                   const uint8_t* sw2, const uint8_t* sw2_sc, int Is,
                                   int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                                   int32_t* perm, int32_t* slot_pos, float* y, float* y_shared,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * Dense block-32 FP8 GEMM (post #2 "Known issues and next steps": dense FP8
 * GEMMs are the largest remaining decode lever; post #6 "How it works":
 * MXFP8 projections, decode rows on small row tiles).
 * a FP8 [M][K] + a_sc SC [M][K/32];  w FP8 [N][K] + w_sc SC [N][K/32].
 * y[m][n] = sum_k a[m][k] * w[n][k] (decoded), fp32 accumulate in one fixed
 * order per element; y is [M][N] bf16 (MX_OUT_BF16, RNE of the fp32 result)
 * or fp32 (MX_OUT_F32).  Supported: K % 32 == 0 (a K that is not a multiple
 * of 128 ends in a partial MFMA step, zero-filled on both operands; scale
 * rows then need no alignment), K <= 16384, N % 16 == 0, M >= 1, M*N < 2^31,
 * and M*K, N*K < 2^32 (operands addressed with 32-bit byte offsets); beyond
 * these MX_EUNSUPPORTED.  a, w 16-byte aligned; a_sc, w_sc, y 4-byte aligned.
 */
mx_status fp8_block_gemm(const uint8_t* a, const uint8_t* a_sc,
                         const uint8_t* w, const uint8_t* w_sc,
                         int M, int N, int K, void* y, int y_dtype, void* stream);

/*
 * Shared expert: a dense SwiGLU MLP on every row with block-32 FP8 operands
 * (post #6 "Kernel by kernel against B12X": the shared expert's two kernels
 * per call; TP4 README, settings table, row "Kernels", and its boot-log
 * lines: the shared expert's down weight (5120, 576), K padded to 640 there;
 * here K = I is used as is).
 * x   FP8 [T][H] + x_sc SC [T][H/32];  w13 FP8 [2I][H] + w13_sc SC [2I][H/32]
 * (rows [0, I) gate, [I, 2I) up);  w2 FP8 [H][I] + w2_sc SC [H][I/32].
 * y   fp32 [T][H] = requant_fp8(silu(x.gate^T) * (x.up^T)) . w2^T, each GEMM
 *     in the dense projection's fixed order (fp8_block_gemm), the requant
 *     the routed experts' (E4M3 block-32 along I).
 * Supported: H % 32 == 0, I % 32 == 0 (no K % 128 restriction), H, I <=
 * 16384, T*H and T*2I < 2^31.  x, w13, w2 16-byte aligned; scales and y
 * 4-byte aligned.  ws: moe_shared_expert_workspace_bytes(T, H, I) bytes
 * (256-byte aligned, contents ignored): the fp32 gate/up values
 * [T][2I], then the FP8 intermediate [T][I] and its scales [T][I/32], each
 * 256-byte aligned.  Asynchronous on stream.
 * One row (T = 1, I <= 1024) has decode forms of its own: with H % 128 == 0,
 * ONE launch, whose gate/up workgroups (8 intermediate columns each, all of
 * K) hand their SwiGLU values to the down workgroups through the workspace
 * as 8-byte words that carry a per-call tag (nothing needs clearing first;
 * under graph capture the tag comes from a call counter in the workspace,
 * the 32-bit word after the status word, advanced by a one-thread kernel
 * recorded before the launch, as moe_layer_decode1 describes); each wait is
 * bounded (20 ms) and one that runs out sets bit 0 of the 32-bit status
 * word in the workspace's last 256 bytes (offset
 * moe_shared_expert_workspace_bytes(1, H, I) - 256; never expected, and that
 * call's y is then undefined; callers may clear and check it).  Otherwise
 * two launches (gate/up K parts, then the down projection with the SwiGLU
 * and requant in its prologue).  Both give the same bits as the T > 1 path's
 * rows.  Calls that share a workspace must not overlap.
 */
size_t    moe_shared_expert_workspace_bytes(int T, int H, int I);
mx_status moe_shared_expert(const uint8_t* x, const uint8_t* x_sc, int T, int H,
                            const uint8_t* w13, const uint8_t* w13_sc,
                            const uint8_t* w2, const uint8_t* w2_sc, int I,
                            float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * Weight prefetch (spark-ds41f README, "Current baseline": the next layer's
 * weights and scale words stream into L2 while latency-bound kernels run;
 * TP4 README, settings table, row "L2 prefetch": a side-stream kernel in
 * the idle phases of a decode step, data untouched).  Reads [p, p + bytes)
 * and discards it, so that a later kernel finds it in cache: workgroup i
 * reads bytes [i*chunk_bytes, (i+1)*chunk_bytes), which land in the L2 of
 * the XCD that runs it and in the memory-side cache (MALL) shared by all
 * XCDs.  A chunk_bytes equal to a consumer kernel's per-workgroup slice
 * (same block count) puts each slice in the L2 of its consumer's XCD.
 * chunk_bytes 0 means 64 KiB.  Whole 16-byte units only (a trailing partial
 * unit is not read).  p 16-byte aligned, chunk_bytes % 16 == 0 (else
 * MX_EINVAL).  Writes nothing; asynchronous on stream (use a side stream
 * to overlap it with latency-bound work).
 */
mx_status mx_prefetch(const void* p, uint64_t bytes, uint64_t chunk_bytes, void* stream);

/* Name of a status code (static string). */
const char* mx_status_string(mx_status s);

/* Kernel variants launched by this thread's last successful call (static,
 * thread-local string), so that a caller can check which path ran. */
const char* mx_last_variant(void);

/*
 * Path selection for moe_expert_ffn: 0 = automatic (by T*k and the layer
 * shape), 1 = decode kernels (16-row matrix-core tiles, weights streamed
 * straight to registers), 2 = prefill kernels (128-row gate/up tiles and
 * 32-row down tiles staged through LDS).  Both paths give bitwise identical
 * results; this exists so tests can prove it.  A shape the selected path
 * does not implement makes moe_expert_ffn return MX_EUNSUPPORTED.
 * Process-wide; returns the previous setting, or MX_EINVAL for other values.
 */
int mx_set_ffn_path(int path);

/*
 * Single-launch forms of moe_layer_decode1, moe_layer_decode1_shared and of
 * moe_shared_expert at T = 1 (see there): 1 = used wherever they apply (the default), 0 = always two
 * launches.  Both give bitwise the same
 * results; this exists so tests can prove it and benchmarks compare them.
 * Process-wide; returns the previous setting, or MX_EINVAL for other values.
 */
int mx_set_layer1_single_launch(int on);

/*
 * Diagnostic gate/up output (for parity tests of the gate/up GEMM: the
 * product path never writes it).  With h set, every later moe_expert_ffn and
 * moe_layer_decode1 call of this thread, on either path, also writes the fp32
 * gate/up values of every live pair to h: row p = bucket position, [2I]
 * floats (gate columns, then up columns), the values the SwiGLU consumed.
 * h: caller-owned device memory, 16-byte aligned; h_bytes its size.  A call
 * whose T*k*2I*4 bytes exceed h_bytes returns MX_EWORKSPACE.  h = NULL stops
 * the writes.  MX_EINVAL for a misaligned h.
 */
mx_status mx_set_ffn_diag(float* h, size_t h_bytes);

/*
 * Diagnostic for the intermediate requant (FP8 E4M3 under the block's E8M0
 * scale, OCP MX v1.0 "Conversion"; post #6 "Why TileLang": FP8
 * quantization): every finite float whose magnitude bit pattern lies in
 * [lo, hi) is encoded with both signs by the hardware conversion the FFN
 * kernels use (clamp to +-448, round to nearest even) and by the integer
 * rounding encoder the quantize kernels use; the number of differing codes is
 * added to *mismatches (device memory, 8-byte aligned, initialised by the
 * caller).  hi <= 0x7F800000 (the finite floats).  Asynchronous on stream.
 * MX_EINVAL for a null or misaligned counter or lo > hi.
 */
mx_status mx_check_requant(uint32_t lo, uint32_t hi, unsigned long long* mismatches, void* stream);

/*
 * Diagnostic timing of moe_expert_ffn's phases (for benchmarks: a call's
 * kernels cannot be bracketed from outside it).  With n = 4 caller-owned
 * hipEvent_t handles set, every later moe_expert_ffn call of this thread
 * records, on the call's stream, events[0] before its first kernel,
 * events[1] after the gate/up kernel, events[2] after the down projection
 * and events[3] after its last kernel (on the single-row path the down kernel
 * also combines, so events[2] and events[3] are recorded together).  n = 0
 * stops the recording.  MX_EINVAL for another n or a null handle.
 */
mx_status mx_set_phase_events(void* const* events, int n);

#ifdef __cplusplus
}
#endif
#endif /* MXMOE_H */
