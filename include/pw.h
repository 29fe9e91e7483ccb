/*
 * pw.h -- C ABI of the MI355X (gfx950) fused mixed-precision MoE expert
 * library: PagedWeight's data-parallel hot path.
 *
 * Source of the method: the PagedWeight pages ("Technical summary:
 * PagedWeight", "Core components" 1 and 3).  Expert weights are handled per
 * linear block (layer, expert, gate_up | down), held in the Any-Precision
 * overlaid bit-plane form with per-row look-up tables; a weight page table
 * records each block's committed width q_i; one fused MoE operation reads the
 * planes and LUTs directly at each block's own q_i; width changes are
 * committed only at safe boundaries, with pages moved asynchronously between
 * host and device memory.
 *
 * Conventions for every function:
 *  - Return a pw_status; nothing is thrown across the ABI.  On any error the
 *    call enqueues no GPU work and changes no library state, and
 *    pw_last_error() describes the failure (thread-local, valid until the next
 *    call on the same thread).
 *  - "dev" pointers are device memory owned by the caller (for example torch
 *    tensors); "host" pointers are ordinary host memory owned by the caller.
 *    Activation arrays (x, y) must be 16-byte aligned, the workspace 256-byte
 *    aligned, every other device array 4-byte aligned.  Nothing the caller passes is
 *    retained after the call returns, except through work enqueued on the
 *    given stream.
 *  - Hot-path calls (pw_route_topk, pw_permute_by_expert, pw_route_permute,
 *    pw_moe_ffn_bitplane, pw_moe_layer)
 *    are asynchronous on `stream`: no host synchronisation, no allocation.
 *    Kernel faults surface at the caller's next synchronisation.
 *  - A context is not thread-safe: drive it from one host thread.
 *
 * Data formats (all little-endian):
 *  - Parent codes are p = 8 bits.  The child code at width q (3..8) is
 *    code8 >> (8 - q), and the weight is LUT_q[row][child code].
 *  - Bit-planes: plane p (0..7) holds bit (7 - p) of every parent code, so a
 *    width-q read uses planes 0..q-1 only.  A block with R rows and K columns
 *    (K a multiple of 32) has K/32 words per row per plane; word w of row r
 *    covers columns 32w..32w+31, and column 32w + 8P + 2i + h
 *    (P, i in 0..3, h in 0..1) sits at bit 8i + 4h + P of that word.  Words
 *    are stored chunk-major: plane p is an array [ceil(K/128)][R][4] of
 *    uint32 (4 consecutive words = 128 columns of one row are contiguous,
 *    rows follow each other inside a 128-column chunk; missing words of a
 *    last partial chunk are zero).
 *  - LUTs: fp16, for each child width k = 3..8 an array [R][2^k], the six
 *    arrays concatenated in k order (R * 504 halves per block).
 *  - gate_up blocks have R = 2*I rows (rows [0, I) gate, [I, 2I) up) and
 *    K = H; down blocks have R = H, K = I.  The FFN of one expert is
 *    h = silu(gate x) * (up x), d = down h; token t's output is
 *    y_t = sum_j w[t][j] * d_(t, idx[t][j]) (+ shared expert d, weight 1).
 */
#ifndef PW_H_
#define PW_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PW_OK = 0,
    PW_ERR_INVALID = 1, /* bad argument: null/misaligned pointer, size or id out of range */
    PW_ERR_OOM = 2,     /* device or pinned host allocation failed                     */
    PW_ERR_HIP = 3,     /* a HIP runtime call failed; pw_last_error() has its message   */
    PW_ERR_STATE = 4    /* the call does not fit the context's state (e.g. a block not
                           registered yet)                                             */
} pw_status;

typedef struct pw_ctx pw_ctx;

/* Opaque HIP stream handle (hipStream_t); NULL is the device's null stream. */
typedef void *pw_stream;

/* Shape of the MoE model whose expert blocks a context manages. */
typedef struct {
    int32_t num_layers;        /* >= 1                                            */
    int32_t num_experts;       /* routed experts per layer, 1..256                 */
    int32_t hidden;            /* H, multiple of 32, 32..32768                     */
    int32_t inter;             /* I of a routed expert, multiple of 32             */
    int32_t inter_shared;      /* I of the shared expert (multiple of 32), 0 = none */
    int32_t top_k;             /* experts per token, 1..min(8, num_experts)        */
    int32_t keep_host_masters; /* 1: keep all 8 planes and all LUTs in pinned host
                                  memory so pw_set_committed_bits can raise widths;
                                  0: keep nothing on the host; every width is then
                                  fixed at its registered value (a change fails
                                  with PW_ERR_STATE)                              */
} pw_model_desc;

#define PW_QMIN 3
#define PW_QMAX 8
#define PW_MAX_TOKENS 65536
#define PW_MODULE_GATE_UP 0
#define PW_MODULE_DOWN 1
#define PW_EXPERT_SHARED (-1)

/* Message of the last failure on this thread ("" if none). */
const char *pw_last_error(void);

/* Create a context on HIP device `hip_device` for the model `desc`.
 * *out receives the context.  Errors: INVALID (desc out of range), HIP, OOM. */
pw_status pw_create(pw_ctx **out, int hip_device, const pw_model_desc *desc);

/* Release every device slab, pinned master and the page table.  The caller
 * must have synchronised all streams that used the context. NULL is a no-op. */
pw_status pw_destroy(pw_ctx *ctx);

/* Host bit-plane packer ("overlaid bit-plane format", Core components 1).
 * codes: host uint8 [R][K] parent codes; planes: host uint32 output of
 * 8 * ceil(K/128) * R * 4 words in the plane layout above (plane p at offset
 * p * ceil(K/128) * R * 4).  K must be a multiple of 32.  Pure host code; needs
 * no device. */
pw_status pw_pack_bitplanes(const uint8_t *codes, int64_t R, int64_t K, uint32_t *planes);

/* Number of uint32 words of one plane of an R x K block (ceil(K/128)*R*4). */
int64_t pw_plane_words(int64_t R, int64_t K);

/* Register one linear block (layer, expert, module) of the weight page table
 * (Core components 1: the page table tracks each block's committed width).
 * expert = 0..E-1 or PW_EXPERT_SHARED; module = PW_MODULE_GATE_UP / _DOWN.
 * host_planes: 8 planes as written by pw_pack_bitplanes; host_luts: LUTs for
 * k = 3..8 as described above.  The library copies planes 0..q_init-1 and
 * LUT_{q_init} to device memory (synchronously) and, if keep_host_masters,
 * keeps a pinned host copy of all planes and LUTs.  Re-registering a block
 * replaces it.  Call only while no work using this layer is in flight.
 * Errors: INVALID (ids, q_init outside 3..8, null pointers), OOM, HIP, STATE
 * (the block has a pw_request_widths request in flight). */
pw_status pw_register_block(pw_ctx *ctx, int layer, int expert, int module,
                            const uint32_t *host_planes, const uint16_t *host_luts, int q_init);

/* Bytes of workspace pw_moe_ffn_bitplane needs for T tokens (0 if T <= 0). */
size_t pw_workspace_size(const pw_ctx *ctx, int T);

/* Tokens per pass the decode contraction uses for a call of T tokens on a
 * layer of E experts, top_k, shared-expert width I_shared (0: none): 8, 16 or
 * 32, the smallest that covers the largest token count a work unit is
 * expected to hold (the shared expert's T; routed experts: T top_k / E plus
 * two standard deviations of a Poisson count).  A unit holding more tokens
 * takes several passes, each decoding its weights again.  Where this is 16
 * and the gate_up launch is expected to hold more than three 128-row units
 * per compute unit (active experts estimated as E (1 - (1 - top_k/E)^T)),
 * gate_up runs 32-token passes over whole 128-row tiles instead; the down
 * launch keeps 16.  0 when T <= 0 or the call takes the prefill GEMM path
 * (T >= 256; there an expert's tail of fewer than 96 tokens past its last
 * 512-token GEMM tile runs on the decode contraction in 32-token passes).
 * Pure function; no GPU. */
int32_t pw_decode_tokens_per_pass(int T, int top_k, int E, int I_shared);

/* Fix the decode contraction's tokens per pass of this context's later calls
 * to 8, 16 or 32 for both launches (0: chosen per call as
 * pw_decode_tokens_per_pass states),
 * for callers that know their batches' spread over the experts better than
 * that estimate.  Results do not depend on it beyond rounding: 8- and
 * 32-token passes give bit-identical y, 16-token passes split K over four
 * waves of 64-row gate_up tiles instead of two.  Errors: INVALID. */
pw_status pw_set_tokens_per_pass(pw_ctx *ctx, int tokens);

/* Top-k routing (Problem statement: each token activates a subset of the
 * experts).  logits: dev fp32 [T][E]; topk_idx: dev int32 [T][k]; topk_w: dev
 * fp32 [T][k].  Per token the k largest logits are chosen in the order
 * (logit descending, expert index ascending); topk_w is the softmax over those
 * k logits only.  Logits must be finite.  T = 0 enqueues nothing. */
pw_status pw_route_topk(pw_ctx *ctx, const float *logits, int T, int32_t *topk_idx,
                        float *topk_w, pw_stream stream);

/* Group the T*k assignments a = t*k + j by expert: a stable counting sort.
 * ("Technical summary: PagedWeight", Problem statement: each token activates
 * only a few experts; Core components 3: the fused operation reads each
 * expert's linear blocks at their own widths.  Grouping the tokens routed to
 * an expert lets its planes and LUT be read once for all of them.)
 * expert_offsets: dev int32 [E+1] (offsets[0] = 0, offsets[E] = T*k);
 * sorted_assign: dev int32 [T*k], the assignments routed to expert e, in
 * ascending a, at [offsets[e], offsets[e+1]).  topk_idx entries must be in
 * 0..E-1. */
pw_status pw_permute_by_expert(pw_ctx *ctx, const int32_t *topk_idx, int T,
                               int32_t *expert_offsets, int32_t *sorted_assign, pw_stream stream);

/* pw_route_topk followed by pw_permute_by_expert in one call, with the same
 * outputs (bit for bit).  For T * k <= 4096 a single workgroup routes the
 * tokens and sorts the assignments without a round trip through memory (one
 * launch instead of two, for decode-sized batches); larger batches run the
 * two kernels.  Arguments and errors as for the two calls. */
pw_status pw_route_permute(pw_ctx *ctx, const float *logits, int T, int32_t *topk_idx, float *topk_w,
                           int32_t *expert_offsets, int32_t *sorted_assign, pw_stream stream);

/* The fused mixed-precision MoE FFN of one layer ("Technical summary:
 * PagedWeight", Core components 3: one operation reads the bit-planes and LUTs
 * directly, each linear block at its own width).  Every block is decoded at the width
 * committed in the device page table when the work runs.
 * x: dev fp16 [T][H]; topk_idx / topk_w: as written by pw_route_topk;
 * expert_offsets / sorted_assign: as written by pw_permute_by_expert;
 * y: dev fp16 [T][H] output (fp32 accumulation, rounded once to fp16);
 * workspace: dev, >= pw_workspace_size(ctx, T) bytes, 256-byte aligned,
 * contents undefined on entry and exit.  Every routed block of `layer` (and
 * the shared expert's, if the model has one) must be registered, else STATE.
 * From T = 256 on (the prefill GEMM path) x and the workspace's fp16 h
 * (T * (k + 1) rows of max(I, I_shared)) must each span at most 4 GiB, else
 * INVALID: split such a batch into several calls. */
pw_status pw_moe_ffn_bitplane(pw_ctx *ctx, int layer, const uint16_t *x, int T,
                              const int32_t *topk_idx, const float *topk_w,
                              const int32_t *expert_offsets, const int32_t *sorted_assign,
                              uint16_t *y, void *workspace, size_t ws_bytes, pw_stream stream);

/* One whole MoE layer step: pw_route_permute followed by pw_moe_ffn_bitplane,
 * with the same outputs (topk_idx, topk_w, expert_offsets, sorted_assign and
 * y, bit for bit).  For decode-sized batches (T * k <= 64, T below the
 * prefill crossover of 256 tokens, and few enough gate_up work units that
 * all of them run at once: at most two per compute unit, counting the
 * shared expert's 64-row tiles and those of the E (1 - (1 - k/E)^T) routed
 * blocks a batch is expected to activate)
 * the routing runs inside the gate_up launch:
 * every workgroup with routed work routes and sorts the batch in LDS (3-5 us
 * of its start-up, while the shared expert's workgroups already stream)
 * instead of waiting for a separate routing launch, and one of them writes
 * the routing outputs for the caller and for the down and combine launches.  Larger batches run the separate
 * launches.  logits: dev fp32 [T][E]; the other arguments, the errors and the
 * workspace rule are those of the two calls.  T = 0 sets expert_offsets to
 * zero and enqueues nothing else. */
pw_status pw_moe_layer(pw_ctx *ctx, int layer, const float *logits, const uint16_t *x, int T,
                       int32_t *topk_idx, float *topk_w, int32_t *expert_offsets,
                       int32_t *sorted_assign, uint16_t *y, void *workspace, size_t ws_bytes,
                       pw_stream stream);

/* Allocation-free form of pw_moe_layer, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same work and outputs, with the workspace taken from a
 * device buffer the library holds for each GPU (PW_STATIC_SCRATCH_BYTES,
 * 16 MiB, kept until the process ends) instead of from the caller.  It
 * enqueues no allocation and no free.  T with pw_workspace_size(ctx, T)
 * above PW_STATIC_SCRATCH_BYTES is refused with INVALID (the decode sizes fit:
 * e.g. 64 tokens of a 4096 x 14336 top-2 layer need 12.1 MB).  Every call on
 * one GPU uses the same buffer, whatever the context or stream: calls that
 * overlap on a GPU race, so the caller serialises them (one stream, or an
 * event between streams).  Errors: as pw_moe_layer. */
#define PW_STATIC_SCRATCH_BYTES (16u << 20)
pw_status pw_moe_layer_noalloc(pw_ctx *ctx, int layer, const float *logits, const uint16_t *x, int T,
                               int32_t *topk_idx, float *topk_w, int32_t *expert_offsets, int32_t *sorted_assign,
                               uint16_t *y, pw_stream stream);

/* Routing-mass accumulator (Core components 2: online routing statistics,
 * the routing mass of an expert = how often and how strongly it is chosen).
 * pw_routing_mass_enable(ctx, 1) allocates a device array mass [L][E] fp64,
 * zeroed (synchronous, the first time only); while enabled, every
 * pw_moe_layer call adds to mass[layer][e], for each expert e, the sum of the
 * gate weights of the assignments routed to e in that call, summed in fp64 in
 * sorted (ascending assignment) order.  Decode-sized calls do it inside the
 * routing gate_up launch, others with one extra one-workgroup launch.
 * enable(ctx, 0) stops accumulating and keeps the values.  _reset zeroes the
 * array (asynchronous on `stream`, a fill kernel, so it may be captured);
 * _read copies it to host_out [L * E] after the work enqueued on `stream` and
 * waits for that copy.  Errors: INVALID, OOM, HIP, STATE (reset / read before
 * the first enable). */
pw_status pw_routing_mass_enable(pw_ctx *ctx, int on);
pw_status pw_routing_mass_reset(pw_ctx *ctx, pw_stream stream);
pw_status pw_routing_mass_read(pw_ctx *ctx, double *host_out, pw_stream stream);

/* Parameters of pw_plan_widths. */
typedef struct {
    int q_min;        /* lowest width of a block (3..8) */
    int q_max;        /* highest width (q_min..8) */
    int hot_floor;    /* lowest width of a hot expert's blocks */
    double hot_share; /* an expert is hot if its share of its layer's routing mass is >= hot_share (0: none) */
    double hot_mult;  /* damage multiplier of a hot expert's blocks */
    double mass_eps;  /* added to every share, so unrouted experts still count */
} pw_plan_params;

/* Quality-aware width planner (Core components 2: greedy lowest damage per
 * byte under a memory target; hot experts protected by a higher width floor
 * and a damage multiplier).  Pure host function, no context or device.
 * Routed blocks b = (layer * E + expert) * 2 + module (gate_up R = 2I x K = H,
 * down R = H x K = I) at width q count their q bit-planes plus LUT_q:
 * R * K * q / 8 + R * 2^q * 2 bytes (the device storage adds only the padding
 * of K to a multiple of 128 columns and of the LUT to whole 64-slot groups,
 * none when 128 divides both R and K).  With share = mass[l][e] / sum over the
 * layer (0 if the layer has none) and hot = share >= hot_share, block b's
 * weight is sensitivity[b] * (share + mass_eps) * (hot ? hot_mult : 1), its
 * floor max(q_min, hot_floor) if hot else q_min, and lowering it from q to
 * q - 1 adds damage weight * 3 * 4^(8 - q) (error power about 4x per dropped
 * bit).  Steps: clamp q_cur into [floor, q_max]; if the total bytes exceed
 * byte_target, repeatedly lower the block with the least damage per byte
 * saved (ties: lower b) until the total fits or every block is at its floor;
 * otherwise repeatedly raise the block with the most damage removed per byte
 * added among those that still fit the target (ties: lower b).  The planner
 * ignores shared experts (their bytes are outside byte_target).
 * q_cur, q_out: uint8 [L][E][2]; mass: [L][E]; sensitivity: [L][E][2], >= 0;
 * bytes_out (may be NULL): total bytes of the routed blocks at q_out.
 * Errors: INVALID. */
pw_status pw_plan_widths(int L, int E, int H, int I, const uint8_t *q_cur, const double *mass,
                         const float *sensitivity, const pw_plan_params *params, int64_t byte_target,
                         uint8_t *q_out, int64_t *bytes_out);

/* Change the committed width of n blocks (Core components 3: asynchronous page
 * movement; widths committed only at safe boundaries).  block_ids: host, each
 * = (layer * (E + 1) + slot) * 2 + module with slot = expert or E for the
 * shared expert (see pw_block_id); q_new: host, 3..8.  Lowering frees planes
 * q_new..q_old-1 once the work already enqueued on `compute` is done.
 * Raising copies planes q_old..q_new-1 and LUT_{q_new} from the pinned host
 * masters with asynchronous copies on `copy`; `compute` waits for those
 * copies before the page-table update (one kernel on `copy` reads the pinned
 * masters directly, the fastest copy when compute waits for it).  The new
 * widths apply to all work
 * enqueued on `compute` after this call returns and never to earlier work.
 * Errors: INVALID (ids, q outside 3..8, duplicate ids), STATE (a change
 * without host masters, or a block with a pw_request_widths request in
 * flight), OOM, HIP.  On error nothing changes. */
pw_status pw_set_committed_bits(pw_ctx *ctx, int n, const int32_t *block_ids,
                                const uint8_t *q_new, pw_stream compute, pw_stream copy);

/* Non-blocking width changes (Core components 1 and 3: the page table tracks
 * a desired width d_i and a committed width q_i; pages move asynchronously
 * and new widths are committed only at safe boundaries).
 * pw_request_widths records d_i = q_desired for n blocks and starts the
 * moves on `copy` right away: new slabs for planes q_i..d_i-1 and LUT_{d_i}
 * from the pinned host masters (lowering copies only the smaller LUT).  The
 * copies go through library-held staging (up to 16 chunks of 32 MB pinned
 * host and 32 MB device memory, kept until pw_destroy): host threads of the
 * library gather the source ranges into a pinned chunk (about 3 ms per 300 MB
 * on eight threads) in a host function on a library-owned stream, so this
 * call returns once the work is enqueued; one DMA per chunk on `copy` waits
 * for its gather, and one short kernel on `copy` scatters it into the new
 * slabs, so the kernels running meanwhile lose little to the copies.  The
 * committed widths do not change.  Errors as pw_set_committed_bits, plus
 * STATE for a block that already has a request in flight (one request per
 * block until it is committed).
 * pw_commit_ready is the safe-boundary call (between layer steps): every
 * requested block whose copies have landed is committed, stream-ordered on
 * `compute` (work enqueued before keeps the old widths); blocks still in
 * transfer stay pending and nothing on `compute` waits for `copy`.
 * *n_committed (may be NULL) receives the number of blocks committed.
 * Slabs a commit drops are recycled after the work enqueued on `compute`
 * before it.
 * pw_block_state reports q_i, d_i and the block's page state. */
enum { PW_PAGE_RESIDENT = 0, PW_PAGE_IN_TRANSFER = 1, PW_PAGE_READY = 2 };
pw_status pw_request_widths(pw_ctx *ctx, int n, const int32_t *block_ids, const uint8_t *q_desired,
                            pw_stream copy);
pw_status pw_commit_ready(pw_ctx *ctx, pw_stream compute, int *n_committed);
pw_status pw_block_state(const pw_ctx *ctx, int32_t block_id, int32_t *q_committed, int32_t *q_desired,
                         int32_t *state);

/* Per-plane page states of one block ("Technical summary: PagedWeight", Core
 * components 1: pages reside on the GPU, on the CPU, or are in transfer).
 * states: host int32 [9]; states[p] for bit-plane p = 0..7, states[8] for
 * the LUT of the desired width d_i.  A plane is PW_PLANE_GPU while a device
 * copy is in use (planes q_i..d_i-1 of a lowering request stay in use until
 * its commit); IN_TRANSFER / READY while a raise request's copy is in flight /
 * has landed and awaits the commit; PW_PLANE_CPU when only the pinned host
 * master holds it; PW_PLANE_ABSENT when no copy is kept (a context without
 * host masters).  Errors: INVALID (null pointer, unregistered block), HIP. */
enum { PW_PLANE_GPU = 0, PW_PLANE_IN_TRANSFER = 1, PW_PLANE_READY = 2, PW_PLANE_CPU = 3, PW_PLANE_ABSENT = 4 };
pw_status pw_plane_states(const pw_ctx *ctx, int32_t block_id, int32_t *states);

/* Committed width of every block, by block id (host uint8 [num_layers *
 * (num_experts + 1) * 2]; 0 for a block not registered). */
pw_status pw_committed_widths(const pw_ctx *ctx, uint8_t *q_out);

/* Copy the routing-mass accumulator [L][E] fp64 to `dst` (device memory or
 * pinned host memory) after the work enqueued on `stream`, without waiting:
 * the caller synchronises on the stream (or an event recorded after this
 * call) before reading.  Errors: INVALID, STATE (never enabled), HIP. */
pw_status pw_routing_mass_copy(pw_ctx *ctx, double *dst, pw_stream stream);

/* One commit event of a fixed-fraction schedule (Core components 2 and 3:
 * the lowest-mass blocks change first, widths change by whole planes).
 * Pure host function.  Among the routed blocks b = (l * E + e) * 2 + m with
 * skip[b] == 0 (skip may be NULL) and not at the bound (q_cur[b] > 3 when
 * `lower`, < 8 otherwise), the n_change blocks with the least mass[l][e]
 * (ties: lower block id) move one bit down (lower) or up.  ids_out receives
 * their library block ids (l * (E + 1) + e) * 2 + m in that order, q_out
 * their new widths, *n_out how many (fewer than n_change if fewer qualify).
 * q_cur, skip: uint8 [L][E][2]; mass: fp64 [L][E].  Errors: INVALID. */
pw_status pw_plan_event(int L, int E, const uint8_t *q_cur, const double *mass, const uint8_t *skip, int lower,
                        int n_change, int32_t *ids_out, uint8_t *q_out, int *n_out);

/* Memory-target trigger (Core components 2: the planner runs when memory
 * pressure, e.g. a growing KV cache, sets a new budget for the weights).
 * Plans the routed blocks' widths with pw_plan_widths against byte_target,
 * starting from each block's desired width d_i, and issues pw_request_widths
 * (on `copy`) for every block whose planned width differs and that has no
 * request in flight; the new widths are committed later by pw_commit_ready
 * at a safe boundary.  mass, sens, params: as pw_plan_widths.
 * *n_requested (may be NULL): blocks requested; *planned_bytes (may be NULL):
 * the plan's routed bytes.  Errors: INVALID, STATE (a routed block not
 * registered, or no host masters), OOM, HIP. */
pw_status pw_retarget(pw_ctx *ctx, int64_t byte_target, const double *mass, const float *sens,
                      const pw_plan_params *params, pw_stream copy, int *n_requested, int64_t *planned_bytes);

/* Return to the device (hipFree) every slab chunk none of whose slabs is
 * used by a block any more (planes dropped by lowered widths, replaced LUTs):
 * dropping plane p of many blocks frees whole plane-p chunks.  Slabs whose
 * last reader may still be running are kept until a later call.  Not for the
 * hot path: hipFree may synchronise the device.  *freed_bytes (may be NULL)
 * receives the bytes returned.  Errors: INVALID, HIP. */
pw_status pw_trim(pw_ctx *ctx, int64_t *freed_bytes);

/* Device-slab accounting.  Plane and LUT slabs are carved from chunks of
 * about 32 MiB, one chunk per class (slab size, plane index or LUT), so that
 * width changes rarely allocate device memory (each hipMalloc stalls the
 * kernels running on the device).  Outputs (any may be NULL): bytes of slabs
 * in use by committed widths (as pw_resident_bytes), bytes of free slabs kept
 * for reuse, bytes of released slabs still waiting for their last reader,
 * bytes of device memory the chunks hold, the number of device allocations
 * made so far, and HIP events created so far (events are recycled once no
 * pending work refers to them). */
pw_status pw_pool_stats(const pw_ctx *ctx, int64_t *resident, int64_t *cached, int64_t *waiting, int64_t *held,
                        int64_t *device_allocs, int64_t *events);

/* Host view of one block's committed width (0 if not registered). */
pw_status pw_get_committed_bits(const pw_ctx *ctx, int32_t block_id, int32_t *q_out);

/* Block id of (layer, expert or PW_EXPERT_SHARED, module); -1 if out of range. */
int32_t pw_block_id(const pw_ctx *ctx, int layer, int expert, int module);

/* Device bytes held for planes and LUTs of committed widths. */
int64_t pw_resident_bytes(const pw_ctx *ctx);

/* Test exports: one block's decode at its committed width, run by the very
 * routines an FFN path uses (the same LUT staging into LDS, lane-to-row
 * mapping, plane loads, code gather and LDS look-up), with the codes and
 * weights written out instead of multiplied.  The decode is defined in
 * "Technical summary: PagedWeight", Core components 1 (overlaid bit-planes
 * read at a block's own width, weights from its LUT): the child code is
 * code8 >> (8 - q) and the weight LUT_q[row][child code].
 * path selects the FFN path whose decode runs:
 *   PW_DECODE_PATH_TILE128: the decode contraction with 128-row tiles (the
 *     decode gate_up's whole tiles: 64 gate rows with their 64 up rows);
 *   PW_DECODE_PATH_TILE64: the decode contraction with 64-row tiles (the
 *     decode down tiles and the gate_up half tiles);
 *   PW_DECODE_PATH_PREFILL: the prefill GEMM's weight-tile decoder;
 *   PW_DECODE_PATH_TILE64_WIDE: 64-row tiles of the 16- and 32-token passes
 *     (single tables at q = 4) that decode batches whose fullest unit is
 *     expected to hold more than 8 tokens use.
 * codes_out: dev uint8 [R][K] child codes; w_out: dev fp16 [R][K] weights
 * (bit patterns); either may be NULL, not both.  Asynchronous on `stream`.
 * Errors: INVALID (null outputs, unregistered block, path out of range), HIP. */
enum { PW_DECODE_PATH_TILE128 = 0, PW_DECODE_PATH_TILE64 = 1, PW_DECODE_PATH_PREFILL = 2, PW_DECODE_PATH_TILE64_WIDE = 3 };
pw_status pw_debug_decode(pw_ctx *ctx, int32_t block_id, int path, uint8_t *codes_out, uint16_t *w_out,
                          pw_stream stream);

/* pw_debug_decode on the decode contraction's tile of the block's module
 * (gate_up: PW_DECODE_PATH_TILE128; down: PW_DECODE_PATH_TILE64), codes only
 * (pw_debug_decode_codes) or weights only (pw_debug_dequant). */
pw_status pw_debug_decode_codes(pw_ctx *ctx, int32_t block_id, uint8_t *out, pw_stream stream);
pw_status pw_debug_dequant(pw_ctx *ctx, int32_t block_id, uint16_t *out, pw_stream stream);

/* Optional per-kernel timing with HIP events on the launch stream.  While
 * enabled, every kernel the context launches is bracketed by events; the
 * totals are read (after the caller synchronised the stream) with
 * pw_profile_read.  Names: "route", "permute", "gate_up", "down", "combine". */
pw_status pw_profile_enable(pw_ctx *ctx, int on);
pw_status pw_profile_read(pw_ctx *ctx, const char *kernel, double *total_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif
#endif /* PW_H_ */
