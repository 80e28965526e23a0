/*
 * strata_window.h - C ABI of the batched verify-window MoE layer for gfx950 (MI355X).
 *
 * What the layer computes (Strata, docs/BATCHING.md "Several requests at once (batch
 * slots)", opening paragraph): a verify window carries one row per active conversation
 * slot (two rows per slot when each slot also verifies one MTP proposal, same page,
 * the --batch-mtp paragraph), at most eight rows (same page, option table and the
 * paragraph after it; PR #1636 "What changed": the hand-off bound is kVerifyMaxT rows).
 * The router, the shared expert, every routed expert used by any row of the window and
 * the output head are fetched a single time per window, whichever rows use them. A row's
 * arithmetic does not depend on which other rows share the window (same page,
 * "Exactness"), so every kernel behind this ABI computes a row the same way whether it
 * is alone or grouped with others.
 *
 * Conventions for every entry point
 *   - Stateless: the library keeps no data between calls; it caches only launch
 *     parameters per process (the GPU's compute-unit count, each kernel's occupancy and
 *     raised LDS limit), so every GPU one process drives must be the same model.
 *   - Threads: entry points may be called from several host threads at once (the caches
 *     are locked; the error string is per thread), each call with its own workspace.
 *   - Every pointer argument except `stream` and the descriptor structs themselves is a
 *     DEVICE pointer owned by the caller, valid until the work enqueued on `stream` has
 *     finished. The descriptor structs (strata_qmat, strata_route_out) are read on the
 *     host during the call only.
 *   - All work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the default
 *     stream). No call allocates, frees or synchronises, so calls may be captured into a
 *     HIP graph.
 *   - Device pointers must be 16-byte aligned; `ws` must be 256-byte aligned.
 *   - Return value: 0 on success, or a negative status (below). On error nothing has
 *     been enqueued, except for STRATA_EHIP, where a launch failed;
 *     strata_window_last_error() then describes the failure (thread-local string).
 *   - prof_events (last argument of each compute entry point): NULL, or an array of
 *     hipEvent_t handles (created by the caller, timing enabled) that the dispatches
 *     themselves record at the start and end of each kernel, for measuring kernel
 *     durations: route {start of its first kernel, end of its last}; moe {gate/up
 *     start, gate/up end, down start, end of the combine}; layer {router GEMV start, end,
 *     gate/up (with the routing) start, end, down start, end of the combine}; head
 *     {start, end}; accept, tier and stream_read {start, end}; stack {start of its first
 *     kernel, end of its last}. A NULL
 *     entry is skipped. Pass NULL while the stream is being captured into a graph.
 *   - Workspace `ws`: at least strata_window_workspace(...) bytes of scratch (partial
 *     sums and intermediates; the first STRATA_WS_COUNTER_BYTES bytes are reserved).
 *     Its contents need no initialisation. Two calls whose work may overlap in time must
 *     not share a workspace.
 *
 * Limits: 1 <= rows <= 8; 1 <= top_k <= 8; top_k <= n_experts <= 256.
 */
#ifndef STRATA_WINDOW_H
#define STRATA_WINDOW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STRATA_WINDOW_ABI_VERSION 6

enum { STRATA_OK = 0, STRATA_EINVAL = -1, STRATA_EUNSUPPORTED = -2, STRATA_EHIP = -3 };
enum { STRATA_F32 = 0, STRATA_BF16 = 1 };       /* activation dtypes                */
enum { STRATA_ROUTE_RENORM = 1 };                /* route flag: divide top-k weights
                                                    by their sum                     */
enum { STRATA_MAX_ROWS = 8, STRATA_MAX_TOPK = 8, STRATA_MAX_EXPERTS = 256 };
enum { STRATA_MAX_FFN = 4096 };                  /* strata_window_moe: widest ffn    */
enum { STRATA_MAX_LAYERS = 1024 };               /* strata_window_stack              */
#define STRATA_WS_COUNTER_BYTES 4096

/*
 * strata_qmat - one block-quantized matrix W[rows][cols] (rows = outputs, cols = inputs),
 * or n_mat of them stacked (the routed experts of one projection).
 *
 * Dequantisation, blocks of 32 consecutive inputs k of one row n, block b = k / 32:
 *   bits 4 or 2 (affine):   W[n][k] = scale[n][b] * q + min[n][b],  q unsigned in [0, 2^bits)
 *   bits 8 (symmetric):     W[n][k] = scale[n][b] * q,              q two's-complement int8
 * scale and min are IEEE binary16.
 *
 * Code layout (per matrix). G = 512 / bits inputs form a k-group (4-bit: 128, 2-bit: 256,
 * 8-bit: 64); rows form tiles of 16. Each (row tile t, k-group g) owns one 1024-byte
 * chunk, chunks ordered t-major: chunk index c = t * (cols / G) + g. Inside a chunk,
 * 64 lanes of 16 bytes; lane L = 16 * j + (n % 16) holds, for row n, the inputs
 * k = G*g + 32*beta + 8*j + i  (beta = block within the group, i in [0,8)),
 * the code of (beta, i) occupying bits [bits*(8*beta + i), bits*(8*beta + i) + bits) of the
 * lane's 128-bit little-endian word. So for weight (n, k):
 *     t = n/16, g = k/G, beta = (k%G)/32, j = (k%32)/8, i = k%8, L = 16*j + n%16
 *     bit = bits*(8*beta + i)
 *     byte offset = (c*64 + L)*16 + bit/8,  code = (byte >> (bit%8)) & (2^bits - 1)
 *
 * Meta layout (per matrix), the same chunk order: chunk c holds 16 rows x (G/32) blocks,
 * row-major: element index = (c*16 + n%16) * (G/32) + beta.
 *     bits 4/2: uint32 per block = scale | (min << 16)      (binary16 bit patterns)
 *     bits 8:   uint16 per block = scale
 *
 * Requirements: rows % 16 == 0, cols % G == 0, bits in {2, 4, 8}.
 * Stacked matrices: matrix m starts at codes + m*mat_stride_codes bytes and at
 * meta element m*mat_stride_meta (strides 0 when n_mat == 1); strides must keep
 * 16-byte alignment.
 */
typedef struct {
  const void* codes;
  const void* meta;
  int32_t rows, cols, bits;
  int32_t n_mat;
  int64_t mat_stride_codes;   /* bytes    */
  int64_t mat_stride_meta;    /* elements */
} strata_qmat;

/*
 * strata_route_out - routing of one window (written by strata_window_route, read by
 * strata_window_moe). All device pointers, sized by the caller (R = rows, k = top_k,
 * E = n_experts, A = min(E, R*k) + 1):
 *   topk_idx [R*k] int32  row r's experts, by descending logit, ties to the lower index
 *   topk_w   [R*k] float  softmax probability of that expert (renormalised over the
 *                         row's k experts with STRATA_ROUTE_RENORM)
 *   n_active [1]   int32  number of active experts, shared expert included
 *   active   [A]   int32  active expert ids ascending; the shared expert (id E) last
 *   offsets  [A+1] int32  entries of active[a] are offsets[a] .. offsets[a+1]-1
 *   entry_row[R*k+R] int32  row of each entry, ascending within an expert
 *   entry_w  [R*k+R] float  routing weight of each entry (1 for the shared expert)
 *   row_mask [E+1] uint8  bit r set when row r uses that expert (entry E: all rows)
 *   entry_pos[R*k+R] int32  position of each entry in its row's list of experts in
 *                         ascending id order (routed 0..k-1, the shared expert k)
 *   row_w  [R*(k+1)] float  row r's weights in that order (row_w[r*(k+1)+k] = 1)
 * Entries past n_active / offsets[n_active] are left untouched. (entry_pos and row_w
 * let strata_window_moe sum each row's experts in the fixed order with no search.)
 */
typedef struct {
  int32_t* topk_idx;
  float*   topk_w;
  int32_t* n_active;
  int32_t* active;
  int32_t* offsets;
  int32_t* entry_row;
  float*   entry_w;
  uint8_t* row_mask;
  int32_t* entry_pos;
  float*   row_w;
} strata_route_out;

/*
 * strata_window_route - router GEMV, softmax, top-k and per-expert row grouping for one
 * window (Strata docs/BATCHING.md, opening paragraph: every routed expert the rows share
 * is fetched a single time per window; the grouping lists the rows of each expert).
 *   x        [rows][hidden], x_dtype STRATA_F32 or STRATA_BF16, row-major
 *   gate_w   [n_experts][hidden] float, row-major
 *   logit_bias [n_experts] float or NULL: added to each row's logits before softmax/top-k
 *   logit[r][e] = sum_h gate_w[e][h] * x[r][h] + bias[e], accumulated in double from
 *   exact products; p = softmax over all experts; the top_k largest logits are selected.
 *   flags: 0 or STRATA_ROUTE_RENORM.
 * Errors: STRATA_EINVAL for a null or misaligned pointer, a bad dtype or flag, sizes
 * outside the limits (hidden must be a multiple of 32), or a workspace smaller than
 * strata_window_workspace(0, ...).
 */
int strata_window_route(void* stream, const void* x, int x_dtype, int rows, int hidden,
                        const float* gate_w, const float* logit_bias, int n_experts,
                        int top_k, int flags, const strata_route_out* out,
                        void* ws, size_t ws_bytes, void* const* prof_events);

/*
 * strata_window_moe - the experts of one window: for every active expert and each of its
 * rows, h = silu(W_gate x) * (W_up x) with silu(z) = z / (1 + exp(-z)), y = W_down h;
 * then for each row r
 *   out[r] = sum over r's entries (ascending expert id) of entry_w * y  +  y_shared
 *            (+ residual[r] when residual != NULL)
 * (Strata docs/BATCHING.md, opening paragraph: the shared expert and the routed experts
 * are fetched a single time per window, whichever rows use them.)
 *   x        [rows][hidden], x_dtype; residual NULL or [rows][hidden] of x_dtype
 *   gate, up: n_mat = n_experts matrices [ffn][hidden]; down: [hidden][ffn]
 *   sh_gate, sh_up, sh_down: the shared expert, n_mat = 1, same shapes and bits
 *   route    the output of strata_window_route for this window (same rows, experts, k)
 *   out      [rows][hidden] float
 *   x_next_bf16 NULL or [rows][hidden] bf16: round-to-nearest-even of out
 * Intermediates stay in float. Bits 4 or 2 (all six matrices alike).
 * Errors: STRATA_EINVAL as for route, or mismatched matrix shapes/bits, or a workspace
 * smaller than strata_window_workspace(1, ...); STRATA_EUNSUPPORTED for bits 8 here, for
 * ffn > STRATA_MAX_FFN, or for a hidden / ffn whose activation image does not fit one
 * compute unit's 160 KB of LDS (about hidden <= 7936 for bf16 x, <= 4480 for float x,
 * ffn <= 4096).
 */
int strata_window_moe(void* stream, const void* x, int x_dtype, int rows, int hidden,
                      int ffn, const strata_qmat* gate, const strata_qmat* up,
                      const strata_qmat* down, const strata_qmat* sh_gate,
                      const strata_qmat* sh_up, const strata_qmat* sh_down,
                      const strata_route_out* route, int n_experts, int top_k,
                      const void* residual, float* out, uint16_t* x_next_bf16,
                      void* ws, size_t ws_bytes, void* const* prof_events);

/*
 * strata_window_layer - the whole MoE layer of one window in one call: what
 * strata_window_route and then strata_window_moe compute, with the same arguments and
 * outputs (route receives the window's routing, as strata_window_route writes it), in
 * four kernels instead of five: the router's GEMV, then gate/up whose every workgroup
 * takes top-k, softmax and grouping from the GEMV's partial sums itself, then down and
 * the combine. Where the activations and the routing tables do not fit one compute
 * unit's LDS together (bf16 activations above about 7,600 hidden, float above about
 * 4,200), the call runs the routing as a kernel of its own, as strata_window_route does,
 * and the plain gate/up: the same results. (Strata docs/BATCHING.md, opening paragraph: the router, the shared expert
 * and each routed expert the rows use are fetched a single time per window.)
 *   ws: at least strata_window_workspace(3, ...) bytes.
 * Errors: those of strata_window_route and strata_window_moe, and a workspace smaller
 * than strata_window_workspace(3, ...).
 */
int strata_window_layer(void* stream, const void* x, int x_dtype, int rows, int hidden, int ffn,
                        const float* gate_w, const float* logit_bias, int flags,
                        const strata_qmat* gate, const strata_qmat* up, const strata_qmat* down,
                        const strata_qmat* sh_gate, const strata_qmat* sh_up,
                        const strata_qmat* sh_down, int n_experts, int top_k,
                        const strata_route_out* route, const void* residual, float* out,
                        uint16_t* x_next_bf16, void* ws, size_t ws_bytes, void* const* prof_events);

/*
 * strata_window_layer_noalloc - strata_window_layer without a workspace argument, for
 * callers that cannot allocate device memory: code being captured into a HIP graph, tight
 * serving loops, and harnesses that forbid allocation. The call itself allocates nothing;
 * its workspace is a fixed array of STRATA_NOALLOC_SCRATCH_BYTES in the library's device
 * memory, one per GPU, held until the process ends (the first call on a device looks up
 * that device's copy). The caller still provides every input and output, as for
 * strata_window_layer, whose arguments, results and errors this call has.
 *   Every call on one GPU uses that GPU's array: calls that may overlap in time on the
 *   same GPU (two streams, two host threads) race on it and must not be made. The array
 *   needs no initialisation and keeps whatever the last call left there.
 * Errors: those of strata_window_layer; STRATA_EINVAL when the shape's workspace
 * (strata_window_workspace(3, ...)) exceeds STRATA_NOALLOC_SCRATCH_BYTES (nothing is
 * enqueued); STRATA_EHIP when the array's address cannot be looked up.
 */
#define STRATA_NOALLOC_SCRATCH_BYTES (2u << 20)
int strata_window_layer_noalloc(void* stream, const void* x, int x_dtype, int rows, int hidden, int ffn,
                                const float* gate_w, const float* logit_bias, int flags,
                                const strata_qmat* gate, const strata_qmat* up, const strata_qmat* down,
                                const strata_qmat* sh_gate, const strata_qmat* sh_up,
                                const strata_qmat* sh_down, int n_experts, int top_k,
                                const strata_route_out* route, const void* residual, float* out,
                                uint16_t* x_next_bf16, void* const* prof_events);

/*
 * strata_window_head - the output head of the window (Strata docs/BATCHING.md, opening
 * paragraph: one fetch of the head serves the whole window; docs/MULTI_GPU.md "What each card
 * holds": the last card runs it): logits[r][v] = sum_h W[v][h] * x[r][h] over an 8-bit
 * block-quantized W [vocab][hidden], then argmax[r] = the lowest v of the largest logit.
 *   logits NULL or [rows][vocab] float; argmax [rows] int32.
 * Errors: STRATA_EINVAL as above (head bits must be 8, rows == vocab, cols == hidden).
 */
int strata_window_head(void* stream, const void* x, int x_dtype, int rows, int hidden,
                       const strata_qmat* head, int vocab, float* logits,
                       int32_t* argmax, void* ws, size_t ws_bytes, void* const* prof_events);

/*
 * strata_window_accept - greedy verification of the window's MTP proposals (Strata
 * docs/BATCHING.md, the --batch-mtp paragraph: each slot verifies one proposal beside its
 * current token, two rows per slot; docs/MULTI_GPU.md, the --pipeline-windows paragraph:
 * a window accepted whole also yields a bonus token).
 *   argmax   [rows] int32: the head's argmax per row (strata_window_head)
 *   mtp = 1: slot s owns rows 2s (its current token) and 2s + 1 (its proposal), so
 *            rows == 2 * n_slots; proposal [n_slots] int32 is the token each proposal row
 *            carries. The proposal is kept when it equals argmax[2s]; the slot then emits
 *            tokens[s] = {proposal, argmax[2s + 1]} (n_tokens 2), else
 *            {argmax[2s], -1} (n_tokens 1).
 *   mtp = 0: rows == n_slots, proposal may be NULL; slot s emits {argmax[s], -1}.
 *   tokens [n_slots][2] int32, n_tokens [n_slots] int32, n_accepted [1] int32 (the kept
 *   proposals of the window): outputs.
 * Errors: STRATA_EINVAL for mtp not 0/1, n_slots outside 1..8/(mtp ? 2 : 1), rows not
 * matching, or a NULL / misaligned pointer. One wave; no workspace.
 */
int strata_window_accept(void* stream, const int32_t* argmax, int rows, int n_slots, int mtp,
                         const int32_t* proposal, int32_t* tokens, int32_t* n_tokens,
                         int32_t* n_accepted, void* const* prof_events);

/*
 * strata_sample_params - one row's sampling parameters (device memory, one per row).
 *   temperature <= 0: greedy (the lowest index of the largest logit); else the logits are
 *               divided by it before the softmax
 *   top_k       candidates: the top_k largest logits (ties to the lower index); clamped to
 *               1 .. min(STRATA_MAX_SAMPLE_TOPK, vocab)
 *   top_p       the shortest prefix of the candidates (by probability, descending) whose
 *               mass reaches top_p of theirs is kept (>= 1: all)
 *   min_p       candidates below min_p times the largest probability are dropped
 *   seed        the request's seed: the key of the draw
 */
typedef struct {
  float temperature;
  int32_t top_k;
  float top_p;
  float min_p;
  uint64_t seed;
} strata_sample_params;
enum { STRATA_MAX_SAMPLE_TOPK = 128 };

/*
 * strata_window_sample - the sampled token of every row of the window (Strata
 * docs/BATCHING.md, "Exactness": sampled requests are drawn row by row with the
 * single-request window's counter-based draw, Philox(seed, position)).
 *   logits   [rows][vocab] float (strata_window_head's logits)
 *   params   [rows] strata_sample_params (device); position [rows] int64 (device): the
 *            token position each row is drawn at (with MTP, a slot's proposal row is at its
 *            token row's position + 1)
 *   tokens   [rows] int32 out
 *   ws       at least strata_window_workspace(5, rows, ..., vocab) bytes of scratch: each
 *            4096-logit chunk's best candidates (contents on entry do not matter)
 * The draw: u in [0, 1) from Philox4x32-10 (Salmon et al., SC'11) with counter (position
 * low word, high word, 0, 0) and key (seed low word, high word), the first two output words
 * as a 53-bit fraction; p_j = exp((l_j - l_0) / temperature) over the candidates (l_0 the
 * largest), in double; the kept candidates are the shorter of the top_p and min_p
 * prefixes (at least one); the token is the first kept candidate whose running sum of p_j
 * exceeds u times their sum. A slot's MTP proposal is verified by strata_window_accept
 * with these tokens in place of the argmax (kept when equal to its token row's draw).
 * Logits must not be NaN (infinities are ordered as values).
 * Errors: STRATA_EINVAL for rows outside 1..8, vocab < 1, a NULL / misaligned pointer, or
 * a workspace smaller than strata_window_workspace(5, ...).
 * Two kernels: one workgroup per (4096-logit chunk, row) keeps the chunk's best top_k, one
 * workgroup per row reduces those to the row's and draws. prof_events: NULL or {start of
 * the first kernel, end of the second}.
 */
int strata_window_sample(void* stream, const float* logits, int rows, int vocab,
                         const strata_sample_params* params, const int64_t* position,
                         int32_t* tokens, void* ws, size_t ws_bytes, void* const* prof_events);

/*
 * strata_window_tier - routing counts of the window and the adaptive tier's swap choice
 * (Strata docs/BATCHING.md, the paragraph on batch windows counting the experts they
 * route to, with --adapt-every, --adapt-decay and --adapt-min-gain: the windows' routing
 * accumulates per-expert counts, and a periodic round exchanges heavily used experts
 * outside the fast tier for lightly used resident ones, each exchange subject to a
 * minimum ratio of the two counts).
 *   row_mask [n_experts + 1] uint8: strata_route_out.row_mask of the window (the shared
 *            expert's entry is not counted)
 *   counts   [n_experts] float, in/out: counts[e] = fmaf(counts[e], decay, number of the
 *            window's rows routed to e); decay in [0, 1]
 *   resident NULL: counting only. Else [n_experts] uint8 in/out (nonzero = in the fast
 *            tier) and a selection round follows the count: the experts outside the tier
 *            by count, largest first, are paired with the resident ones by count,
 *            smallest first (ties: lower expert index first in both); pair i swaps while
 *            every pair up to it has an incoming count > 0 and >= min_gain * outgoing
 *            count (product in float), at most max_swaps pairs.
 *   swaps    [2 * max_swaps] int32 out: (in, out) expert pairs; n_swaps [1] int32 out.
 * Errors: STRATA_EINVAL for n_experts outside 1..256, decay outside [0, 1], max_swaps
 * outside 0..n_experts, a negative or non-finite min_gain, or a NULL / misaligned pointer.
 * One workgroup; no workspace.
 */
int strata_window_tier(void* stream, const uint8_t* row_mask, int n_experts, float* counts, float decay,
                       uint8_t* resident, int max_swaps, float min_gain, int32_t* swaps,
                       int32_t* n_swaps, void* const* prof_events);

/*
 * strata_window_stream_read - a plain streaming read of `bytes` bytes at `src` (16-byte
 * words, non-temporal; every wave one contiguous chunk with 16 loads per lane in flight,
 * 32 waves per compute unit): the bandwidth that HBM
 * actually delivers to a read, against which the layer's kernels are compared (the
 * roofline of the layer is this read of its weights). Measurement only; it computes
 * nothing of the layer.
 *   src   device, 16-byte aligned, bytes a nonzero multiple of 16
 *   sink  device uint32 [1]: written (with magic) only when the xor of the words one
 *         lane reads equals magic, so the caller chooses whether anything is written
 *   prof_events: NULL or {start, end} events recorded by the dispatch.
 * Errors: STRATA_EINVAL for NULL / misaligned pointers or a bad size.
 */
int strata_window_stream_read(void* stream, const void* src, size_t bytes, uint32_t* sink,
                              uint32_t magic, void* const* prof_events);

/*
 * strata_layer - one MoE layer of a stack (host struct, read during the call): its
 * router (gate_w [n_experts][hidden] float, logit_bias [n_experts] float or NULL), its six
 * matrix families as in strata_window_moe, and where its window's routing is written
 * (strata_route_out; layers may share one, since each layer's routing is used before
 * the next layer's is written).
 */
typedef struct {
  const float* gate_w;
  const float* logit_bias;
  strata_qmat gate, up, down, sh_gate, sh_up, sh_down;
  strata_route_out route;
} strata_layer;

/*
 * strata_window_stack - one window through a stack of n_layers MoE layers and then,
 * optionally, the 8-bit head: a pipeline stage's share of the model for one window
 * (Strata docs/MULTI_GPU.md, "What each card holds": a card holds a contiguous range of
 * layers, the last one also the head; PR #1636, "What changed": every stage runs the
 * eight-row verify windows). Layer l computes what strata_window_layer computes with
 * residual = its input x_l, and x_{l+1} = bf16(x_l + out_l) is the next layer's input
 * (x_0 = x, in x_dtype; every later x_l is bf16). The call runs three kernels per layer
 * instead of four: layer l's combine and layer l + 1's router GEMV share one launch, each
 * of its workgroups forming its own 512-input chunk of x_{l+1} before its share of the
 * GEMV. Every layer's routing and x_{l+1} equal those of the same layers run one
 * strata_window_layer call at a time, bit for bit.
 *   layers   host array [n_layers]; every layer has the shapes hidden, ffn, n_experts,
 *            top_k and the same bits
 *   flags    STRATA_ROUTE_RENORM or 0, for every layer
 *   head     NULL, or the 8-bit head [vocab][hidden] (then argmax [rows] int32 is
 *            required and logits [rows][vocab] float is optional, as strata_window_head)
 *   out      NULL or [rows][hidden] float: the last layer's output (residual included)
 *   x_final  [rows][hidden] bf16: the last layer's x_next, the head's input
 *   ws: at least strata_window_workspace(4, ..., vocab) bytes (vocab 0 without a head).
 *   prof_events: NULL or {start of the first kernel, end of the last}.
 * Errors: those of strata_window_layer for any layer and of strata_window_head; n_layers
 * outside 1..STRATA_MAX_LAYERS, layers or x_final NULL, or a layer whose bits differ.
 */
int strata_window_stack(void* stream, const void* x, int x_dtype, int rows, int hidden, int ffn,
                        int n_experts, int top_k, int flags, int n_layers, const strata_layer* layers,
                        const strata_qmat* head, int vocab, float* logits, int32_t* argmax,
                        float* out, uint16_t* x_final, void* ws, size_t ws_bytes,
                        void* const* prof_events);

/* Workspace bytes for which = 0 (route), 1 (moe), 2 (head), 3 (layer), 4 (stack; vocab 0
 * without a head), 5 (sample: rows and vocab only); 0 for invalid arguments. */
size_t strata_window_workspace(int which, int rows, int hidden, int ffn, int n_experts,
                               int top_k, int vocab);

/* Description of the last error on the calling thread ("" if none). */
const char* strata_window_last_error(void);

/* STRATA_WINDOW_ABI_VERSION of the built library. */
int strata_window_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* STRATA_WINDOW_H */
