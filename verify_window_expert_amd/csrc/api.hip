// C ABI of the verify-window MoE layer: argument checks, workspace layout, launches.
// The entry points and their contracts are documented in include/strata_window.h.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>

#include "../../include/strata_window.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr size_t kLdsLimit = 160 * 1024;
constexpr size_t kStaticLds = 2048;   // the kernels' own tables (upper bound)

// ---------------------------------------------------------------- workspace layouts

struct RouteWs { size_t partials, total; };
RouteWs route_ws(int rows, int hidden, int E) {
  const size_t n_hc = (hidden + 511) / 512;
  RouteWs w;
  w.partials = STRATA_WS_COUNTER_BYTES;
  w.total = round_up(w.partials + sizeof(double) * rows * E * n_hc, 256);
  return w;
}

struct MoeWs { size_t h, y, total; };
MoeWs moe_ws(int rows, int hidden, int ffn, int top_k) {
  const size_t ent = (size_t)rows * top_k + rows;
  MoeWs w;
  w.h = STRATA_WS_COUNTER_BYTES;                          // bf16 hi, then bf16 lo, per entry and input
  w.y = round_up(w.h + 4 * ent * ffn, 256);               // the experts' outputs per entry
  w.total = round_up(w.y + 4 * ent * hidden, 256);
  return w;
}

struct LayerWs { MoeWs moe; size_t partials, total; };
LayerWs layer_ws(int rows, int hidden, int ffn, int E, int top_k) {
  LayerWs w;
  w.moe = moe_ws(rows, hidden, ffn, top_k);
  w.partials = w.moe.total;
  w.total = round_up(w.partials + sizeof(double) * rows * E * ((hidden + 511) / 512), 256);
  return w;
}

struct HeadWs { size_t val, idx, total; };
HeadWs head_ws(int rows, int vocab) {
  const size_t n = (size_t)sw::head_workgroups(vocab) * rows;
  HeadWs w;
  w.val = STRATA_WS_COUNTER_BYTES;
  w.idx = round_up(w.val + 4 * n, 256);
  w.total = round_up(w.idx + 4 * n, 256);
  return w;
}

// the sampled draw: each 4096-logit chunk's best 128 keys, their indices, and a lower bound
// of its K-th key, per row
struct SampleWs { size_t key, idx, lo, total; };
SampleWs sample_ws(int rows, int vocab) {
  const size_t nc = (size_t)rows * sw::sample_chunks(vocab), n = nc * 128;
  SampleWs w;
  w.key = STRATA_WS_COUNTER_BYTES;
  w.idx = round_up(w.key + 4 * n, 256);
  w.lo = round_up(w.idx + 4 * n, 256);
  w.total = round_up(w.lo + 4 * nc, 256);
  return w;
}

// the stack: one layer's workspace (reused by every layer), the two bf16 inputs of the
// layers after the first (ping-pong), and the head's
struct StackWs { LayerWs layer; size_t xa, xb, head; HeadWs hw; size_t total; };
StackWs stack_ws(int rows, int hidden, int ffn, int E, int top_k, int vocab) {
  StackWs w;
  w.layer = layer_ws(rows, hidden, ffn, E, top_k);
  w.xa = w.layer.total;
  w.xb = round_up(w.xa + 2 * (size_t)rows * hidden, 256);
  w.head = round_up(w.xb + 2 * (size_t)rows * hidden, 256);
  w.hw = head_ws(rows, vocab > 0 ? vocab : 1);
  w.total = vocab > 0 ? w.head + w.hw.total : w.head;
  return w;
}

// ------------------------------------------------------------------------ checks

int check_common(const void* x, int x_dtype, int rows, int hidden, void* ws) {
  if (!x) return fail(STRATA_EINVAL, "x is NULL");
  if (!aligned(x, 16)) return fail(STRATA_EINVAL, "x is not 16-byte aligned");
  if (x_dtype != STRATA_F32 && x_dtype != STRATA_BF16) return fail(STRATA_EINVAL, "bad x_dtype %d", x_dtype);
  if (rows < 1 || rows > STRATA_MAX_ROWS) return fail(STRATA_EINVAL, "rows %d outside 1..%d", rows, STRATA_MAX_ROWS);
  if (hidden < 1) return fail(STRATA_EINVAL, "hidden %d < 1", hidden);
  if (!ws) return fail(STRATA_EINVAL, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(STRATA_EINVAL, "workspace is not 256-byte aligned");
  return STRATA_OK;
}

int check_experts(int n_experts, int top_k) {
  if (top_k < 1 || top_k > STRATA_MAX_TOPK) return fail(STRATA_EINVAL, "top_k %d outside 1..%d", top_k, STRATA_MAX_TOPK);
  if (n_experts < top_k || n_experts > STRATA_MAX_EXPERTS)
    return fail(STRATA_EINVAL, "n_experts %d outside top_k..%d", n_experts, STRATA_MAX_EXPERTS);
  return STRATA_OK;
}

int check_route_out(const strata_route_out* o) {
  if (!o) return fail(STRATA_EINVAL, "route output descriptor is NULL");
  const void* p[] = {o->topk_idx, o->topk_w, o->n_active, o->active, o->offsets,
                     o->entry_row, o->entry_w, o->row_mask, o->entry_pos, o->row_w};
  const char* nm[] = {"topk_idx", "topk_w", "n_active", "active", "offsets",
                      "entry_row", "entry_w", "row_mask", "entry_pos", "row_w"};
  for (int i = 0; i < 10; i++) {
    if (!p[i]) return fail(STRATA_EINVAL, "route output %s is NULL", nm[i]);
    if (!aligned(p[i], 16)) return fail(STRATA_EINVAL, "route output %s is not 16-byte aligned", nm[i]);
  }
  return STRATA_OK;
}

int check_qmat(const strata_qmat* q, const char* name, int rows, int cols, int n_mat, int bits) {
  if (!q) return fail(STRATA_EINVAL, "%s descriptor is NULL", name);
  if (!q->codes || !q->meta) return fail(STRATA_EINVAL, "%s codes/meta NULL", name);
  if (!aligned(q->codes, 16) || !aligned(q->meta, 16)) return fail(STRATA_EINVAL, "%s codes/meta not 16-byte aligned", name);
  if (q->bits != bits) return fail(STRATA_EINVAL, "%s has %d bits, expected %d", name, q->bits, bits);
  if (q->rows != rows || q->cols != cols)
    return fail(STRATA_EINVAL, "%s is %dx%d, expected %dx%d", name, q->rows, q->cols, rows, cols);
  if (q->n_mat != n_mat) return fail(STRATA_EINVAL, "%s holds %d matrices, expected %d", name, q->n_mat, n_mat);
  const int G = 512 / bits;
  if (rows % 16 || cols % G) return fail(STRATA_EINVAL, "%s: rows %% 16 and cols %% %d must be 0", name, G);
  if (n_mat > 1) {
    const int64_t need_c = (int64_t)rows * cols * bits / 8, need_m = (int64_t)rows * (cols / 32);
    if (q->mat_stride_codes < need_c || q->mat_stride_meta < need_m)
      return fail(STRATA_EINVAL, "%s matrix strides smaller than one matrix", name);
    const int64_t meta_bytes = q->mat_stride_meta * (bits == 8 ? 2 : 4);
    if (q->mat_stride_codes % 16 || meta_bytes % 16)
      return fail(STRATA_EINVAL, "%s matrix strides break 16-byte alignment", name);
  }
  return STRATA_OK;
}

// Whether the fused gate/up (routing core + activation image in one workgroup's LDS)
// fits; else the layer runs the routing core as a kernel of its own and the plain gate/up.
bool fused_fits(int hidden, int x_dtype) {
  return sw::gateup_lds_bytes(hidden, x_dtype) + kStaticLds + sw::route_core_lds_bytes() <= kLdsLimit;
}

int launch_status(int rc, const char* what) {
  if (rc == 0) return STRATA_OK;
  return fail(STRATA_EHIP, "%s launch failed: %s", what, hipGetErrorString((hipError_t)rc));
}

sw::Prof prof(void* const* ev, int i) {
  sw::Prof p;
  if (ev) {
    p.start = (hipEvent_t)ev[i];
    p.stop = (hipEvent_t)ev[i + 1];
  }
  return p;
}

sw::QDev qdev(const strata_qmat* routed, const strata_qmat* shared) {
  sw::QDev d;
  d.codes = (const uint8_t*)routed->codes;
  d.meta = (const uint8_t*)routed->meta;
  d.stride_codes = routed->mat_stride_codes;
  d.stride_meta_bytes = routed->mat_stride_meta * (routed->bits == 8 ? 2 : 4);
  d.sh_codes = (const uint8_t*)shared->codes;
  d.sh_meta = (const uint8_t*)shared->meta;
  return d;
}

// ------------------------------------------------- fixed scratch of the no-allocation call
// strata_window_layer_noalloc's workspace: a file-scope device array, of which every GPU
// holds its own copy. In host code `scratch` is only a stand-in for the symbol: its device
// address is looked up once per device (with that device current) and kept; only that
// address is ever passed to a kernel.
constexpr size_t kScratchBytes = (size_t)STRATA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

// The current device's scratch address, or NULL with *rc set.
void* scratch_ptr(int* rc) {
  static std::mutex m;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  const hipError_t ed = hipGetDevice(&dev);
  if (ed != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *rc = fail(STRATA_EHIP, "no current device for the scratch array (%s)", hipGetErrorString(ed));
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(m);
  if (!ptrs[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *rc = fail(STRATA_EHIP, "scratch array address on device %d: %s", dev, hipGetErrorString(e));
      return nullptr;
    }
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

}  // namespace

extern "C" {

int strata_window_abi_version(void) { return STRATA_WINDOW_ABI_VERSION; }

const char* strata_window_last_error(void) { return g_err; }

size_t strata_window_workspace(int which, int rows, int hidden, int ffn, int n_experts, int top_k, int vocab) {
  if (which == 5) return (rows >= 1 && rows <= STRATA_MAX_ROWS && vocab >= 1) ? sample_ws(rows, vocab).total : 0;
  if (rows < 1 || rows > STRATA_MAX_ROWS || hidden < 1) return 0;
  switch (which) {
    case 0: return n_experts >= 1 ? route_ws(rows, hidden, n_experts).total : 0;
    case 1: return (ffn >= 1 && top_k >= 1) ? moe_ws(rows, hidden, ffn, top_k).total : 0;
    case 2: return vocab >= 1 ? head_ws(rows, vocab).total : 0;
    case 3: return (ffn >= 1 && top_k >= 1 && n_experts >= 1) ? layer_ws(rows, hidden, ffn, n_experts, top_k).total : 0;
    case 4:
      return (ffn >= 1 && top_k >= 1 && n_experts >= 1 && vocab >= 0)
                 ? stack_ws(rows, hidden, ffn, n_experts, top_k, vocab).total
                 : 0;
    default: return 0;
  }
}

}  // extern "C"

namespace {

// Checks of a route call and its argument block (partials at ws + partials_at).
int prepare_route(const void* x, int x_dtype, int rows, int hidden, const float* gate_w, const float* logit_bias,
                  int n_experts, int top_k, int flags, const strata_route_out* out, void* ws,
                  size_t partials_at, sw::RouteArgs& a) {
  int rc;
  if ((rc = check_common(x, x_dtype, rows, hidden, ws))) return rc;
  if ((rc = check_experts(n_experts, top_k))) return rc;
  if (hidden % 32) return fail(STRATA_EINVAL, "hidden %d is not a multiple of 32", hidden);
  if (!gate_w || !aligned(gate_w, 16)) return fail(STRATA_EINVAL, "gate_w NULL or not 16-byte aligned");
  if (logit_bias && !aligned(logit_bias, 16)) return fail(STRATA_EINVAL, "logit_bias not 16-byte aligned");
  if (flags & ~STRATA_ROUTE_RENORM) return fail(STRATA_EINVAL, "unknown route flags 0x%x", flags);
  if ((rc = check_route_out(out))) return rc;
  a.x = x; a.x_dtype = x_dtype; a.rows = rows; a.hidden = hidden;
  a.gate_w = gate_w; a.bias = logit_bias; a.n_experts = n_experts; a.top_k = top_k;
  a.renorm = (flags & STRATA_ROUTE_RENORM) != 0;
  a.partials = (double*)((char*)ws + partials_at);
  a.topk_idx = out->topk_idx; a.topk_w = out->topk_w; a.n_active = out->n_active; a.active = out->active;
  a.offsets = out->offsets; a.entry_row = out->entry_row; a.entry_w = out->entry_w; a.row_mask = out->row_mask;
  a.entry_pos = out->entry_pos; a.row_w = out->row_w;
  return STRATA_OK;
}

// Checks of a moe call and its two argument blocks (intermediates in ws per w).
int prepare_moe(const void* x, int x_dtype, int rows, int hidden, int ffn, const strata_qmat* gate,
                const strata_qmat* up, const strata_qmat* down, const strata_qmat* sh_gate, const strata_qmat* sh_up,
                const strata_qmat* sh_down, const strata_route_out* route, int n_experts, int top_k,
                const void* residual, float* out, uint16_t* x_next_bf16, void* ws, const MoeWs& w,
                sw::GateUpArgs& g, sw::DownArgs& d, int& max_slots, bool out_optional = false) {
  int rc;
  if ((rc = check_common(x, x_dtype, rows, hidden, ws))) return rc;
  if ((rc = check_experts(n_experts, top_k))) return rc;
  if (ffn < 1) return fail(STRATA_EINVAL, "ffn %d < 1", ffn);
  if ((rc = check_route_out(route))) return rc;
  if (!gate) return fail(STRATA_EINVAL, "gate descriptor is NULL");
  const int bits = gate->bits;
  if (bits == 8) return fail(STRATA_EUNSUPPORTED, "8-bit expert matrices are not built (4 or 2 bits)");
  if (bits != 4 && bits != 2) return fail(STRATA_EINVAL, "expert bits %d not in {2, 4}", bits);
  if ((rc = check_qmat(gate, "gate", ffn, hidden, n_experts, bits))) return rc;
  if ((rc = check_qmat(up, "up", ffn, hidden, n_experts, bits))) return rc;
  if ((rc = check_qmat(down, "down", hidden, ffn, n_experts, bits))) return rc;
  if ((rc = check_qmat(sh_gate, "sh_gate", ffn, hidden, 1, bits))) return rc;
  if ((rc = check_qmat(sh_up, "sh_up", ffn, hidden, 1, bits))) return rc;
  if ((rc = check_qmat(sh_down, "sh_down", hidden, ffn, 1, bits))) return rc;
  if ((!out && !out_optional) || (out && !aligned(out, 16)))
    return fail(STRATA_EINVAL, "out NULL or not 16-byte aligned");
  if (residual && !aligned(residual, 16)) return fail(STRATA_EINVAL, "residual not 16-byte aligned");
  if (x_next_bf16 && !aligned(x_next_bf16, 16)) return fail(STRATA_EINVAL, "x_next not 16-byte aligned");
  const size_t lds_gu = sw::gateup_lds_bytes(hidden, x_dtype), lds_dn = sw::down_lds_bytes(ffn);
  if (lds_gu + kStaticLds > kLdsLimit || lds_dn + kStaticLds > kLdsLimit)
    return fail(STRATA_EUNSUPPORTED, "hidden %d / ffn %d need more than %zu bytes of LDS", hidden, ffn, kLdsLimit);
  if (ffn > STRATA_MAX_FFN) return fail(STRATA_EUNSUPPORTED, "ffn %d > %d", ffn, STRATA_MAX_FFN);
  max_slots = std::min(n_experts, rows * top_k) + 1;

  g.x = x; g.x_dtype = x_dtype; g.rows = rows; g.hidden = hidden; g.ffn = ffn; g.bits = bits;
  g.n_experts = n_experts;
  g.gate = qdev(gate, sh_gate); g.up = qdev(up, sh_up);
  g.n_active = route->n_active; g.active = route->active; g.offsets = route->offsets; g.entry_row = route->entry_row;
  g.row_mask = route->row_mask;
  g.max_slots = max_slots;
  const int n_ent = rows * top_k + rows;
  g.h_hi = (uint16_t*)((char*)ws + w.h);
  g.h_lo = g.h_hi + (size_t)n_ent * ffn;

  d.x_res = residual; d.x_dtype = x_dtype; d.rows = rows; d.hidden = hidden; d.ffn = ffn; d.bits = bits;
  d.n_experts = n_experts;
  d.down = qdev(down, sh_down);
  d.n_active = route->n_active; d.active = route->active; d.offsets = route->offsets;
  d.entry_row = route->entry_row; d.entry_pos = route->entry_pos; d.row_w = route->row_w;
  d.h_hi = g.h_hi; d.h_lo = g.h_lo; d.h_entries = n_ent; d.y = (float*)((char*)ws + w.y); d.out = out; d.x_next = x_next_bf16;
  d.max_slots = max_slots; d.top_k = top_k;
  return STRATA_OK;
}

}  // namespace

extern "C" {

int strata_window_route(void* stream, const void* x, int x_dtype, int rows, int hidden, const float* gate_w,
                        const float* logit_bias, int n_experts, int top_k, int flags, const strata_route_out* out,
                        void* ws, size_t ws_bytes, void* const* prof_events) {
  g_err[0] = 0;
  sw::RouteArgs a;
  const RouteWs w = route_ws(rows, hidden, n_experts);
  if (int rc = prepare_route(x, x_dtype, rows, hidden, gate_w, logit_bias, n_experts, top_k, flags, out, ws,
                             w.partials, a))
    return rc;
  if (ws_bytes < w.total) return fail(STRATA_EINVAL, "route workspace %zu < %zu bytes", ws_bytes, w.total);
  const sw::Prof pr = prof(prof_events, 0);
  return launch_status(sw::launch_route(a, (hipStream_t)stream, prof_events ? &pr : nullptr), "route");
}

int strata_window_moe(void* stream, const void* x, int x_dtype, int rows, int hidden, int ffn,
                      const strata_qmat* gate, const strata_qmat* up, const strata_qmat* down,
                      const strata_qmat* sh_gate, const strata_qmat* sh_up, const strata_qmat* sh_down,
                      const strata_route_out* route, int n_experts, int top_k, const void* residual, float* out,
                      uint16_t* x_next_bf16, void* ws, size_t ws_bytes, void* const* prof_events) {
  g_err[0] = 0;
  sw::GateUpArgs g;
  sw::DownArgs d;
  int max_slots = 0;
  const MoeWs w = moe_ws(rows, hidden, ffn, top_k);
  if (int rc = prepare_moe(x, x_dtype, rows, hidden, ffn, gate, up, down, sh_gate, sh_up, sh_down, route, n_experts,
                           top_k, residual, out, x_next_bf16, ws, w, g, d, max_slots))
    return rc;
  if (ws_bytes < w.total) return fail(STRATA_EINVAL, "moe workspace %zu < %zu bytes", ws_bytes, w.total);
  hipStream_t s = (hipStream_t)stream;
  const sw::Prof pg = prof(prof_events, 0), pd = prof(prof_events, 2);
  int rc;
  if ((rc = launch_status(sw::launch_gateup(g, max_slots, s, prof_events ? &pg : nullptr), "gate/up"))) return rc;
  return launch_status(sw::launch_down(d, s, prof_events ? &pd : nullptr), "down");
}

int strata_window_layer(void* stream, const void* x, int x_dtype, int rows, int hidden, int ffn,
                        const float* gate_w, const float* logit_bias, int flags, const strata_qmat* gate,
                        const strata_qmat* up, const strata_qmat* down, const strata_qmat* sh_gate,
                        const strata_qmat* sh_up, const strata_qmat* sh_down, int n_experts, int top_k,
                        const strata_route_out* route, const void* residual, float* out, uint16_t* x_next_bf16,
                        void* ws, size_t ws_bytes, void* const* prof_events) {
  g_err[0] = 0;
  sw::RouteArgs r;
  sw::GateUpArgs g;
  sw::DownArgs d;
  int max_slots = 0;
  const LayerWs w = layer_ws(rows, hidden, ffn > 0 ? ffn : 1, n_experts > 0 ? n_experts : 1, top_k > 0 ? top_k : 1);
  int rc;
  if ((rc = prepare_route(x, x_dtype, rows, hidden, gate_w, logit_bias, n_experts, top_k, flags, route, ws,
                          w.partials, r)))
    return rc;
  if ((rc = prepare_moe(x, x_dtype, rows, hidden, ffn, gate, up, down, sh_gate, sh_up, sh_down, route, n_experts,
                        top_k, residual, out, x_next_bf16, ws, w.moe, g, d, max_slots)))
    return rc;
  if (ws_bytes < w.total) return fail(STRATA_EINVAL, "layer workspace %zu < %zu bytes", ws_bytes, w.total);
  g.route = r;
  hipStream_t s = (hipStream_t)stream;
  const sw::Prof pr = prof(prof_events, 0), pg = prof(prof_events, 2), pd = prof(prof_events, 4);
  if (fused_fits(hidden, x_dtype)) {
    if ((rc = launch_status(sw::launch_route_logits(r, s, prof_events ? &pr : nullptr), "router"))) return rc;
    if ((rc = launch_status(sw::launch_gateup_routed(g, max_slots, s, prof_events ? &pg : nullptr), "gate/up")))
      return rc;
  } else {
    // the activation image leaves no room for the routing core's tables: the routing
    // core runs as a kernel of its own (as strata_window_route), then the plain gate/up
    if ((rc = launch_status(sw::launch_route(r, s, prof_events ? &pr : nullptr), "router"))) return rc;
    if ((rc = launch_status(sw::launch_gateup(g, max_slots, s, prof_events ? &pg : nullptr), "gate/up"))) return rc;
  }
  return launch_status(sw::launch_down(d, s, prof_events ? &pd : nullptr), "down");
}

int strata_window_layer_noalloc(void* stream, const void* x, int x_dtype, int rows, int hidden, int ffn,
                                const float* gate_w, const float* logit_bias, int flags, const strata_qmat* gate,
                                const strata_qmat* up, const strata_qmat* down, const strata_qmat* sh_gate,
                                const strata_qmat* sh_up, const strata_qmat* sh_down, int n_experts, int top_k,
                                const strata_route_out* route, const void* residual, float* out,
                                uint16_t* x_next_bf16, void* const* prof_events) {
  g_err[0] = 0;
  // the shape's workspace must fit the fixed array (checked before any device call)
  const size_t need = strata_window_workspace(3, rows, hidden, ffn, n_experts, top_k, 0);
  if (need == 0)
    return fail(STRATA_EINVAL, "rows %d / hidden %d / ffn %d / n_experts %d / top_k %d out of range", rows, hidden,
                ffn, n_experts, top_k);
  if (need > kScratchBytes)
    return fail(STRATA_EINVAL, "this shape needs %zu bytes of scratch, more than the fixed %zu", need, kScratchBytes);
  int rc = STRATA_OK;
  void* ws = scratch_ptr(&rc);
  if (!ws) return rc;
  return strata_window_layer(stream, x, x_dtype, rows, hidden, ffn, gate_w, logit_bias, flags, gate, up, down,
                             sh_gate, sh_up, sh_down, n_experts, top_k, route, residual, out, x_next_bf16, ws,
                             kScratchBytes, prof_events);
}

int strata_window_stack(void* stream, const void* x, int x_dtype, int rows, int hidden, int ffn, int n_experts,
                        int top_k, int flags, int n_layers, const strata_layer* layers, const strata_qmat* head,
                        int vocab, float* logits, int32_t* argmax, float* out, uint16_t* x_final, void* ws,
                        size_t ws_bytes, void* const* prof_events) {
  g_err[0] = 0;
  if (n_layers < 1 || n_layers > STRATA_MAX_LAYERS)
    return fail(STRATA_EINVAL, "n_layers %d outside 1..%d", n_layers, (int)STRATA_MAX_LAYERS);
  if (!layers) return fail(STRATA_EINVAL, "layers is NULL");
  if (!x_final || !aligned(x_final, 16)) return fail(STRATA_EINVAL, "x_final NULL or not 16-byte aligned");
  if (out && !aligned(out, 16)) return fail(STRATA_EINVAL, "out not 16-byte aligned");
  if (!ws || !aligned(ws, 256)) return fail(STRATA_EINVAL, "ws NULL or not 256-byte aligned");
  if (rows < 1 || rows > STRATA_MAX_ROWS || hidden < 1 || ffn < 1 || n_experts < 1 || top_k < 1)
    return fail(STRATA_EINVAL, "rows %d / hidden %d / ffn %d / n_experts %d / top_k %d out of range", rows, hidden,
                ffn, n_experts, top_k);
  const StackWs w = stack_ws(rows, hidden, ffn, n_experts, top_k, head ? vocab : 0);
  if (ws_bytes < w.total) return fail(STRATA_EINVAL, "stack workspace %zu < %zu bytes", ws_bytes, w.total);
  char* const wb = (char*)ws;
  uint16_t* const xpp[2] = {(uint16_t*)(wb + w.xa), (uint16_t*)(wb + w.xb)};
  // layer l reads x_l and writes x_{l+1}: x_0 = x; the last layer writes x_final, every
  // other one the ping-pong buffer that its input is not in
  auto input = [&](int l) -> const void* { return l == 0 ? x : (const void*)xpp[(l - 1) % 2]; };
  auto input_dtype = [&](int l) { return l == 0 ? x_dtype : (int)STRATA_BF16; };
  auto output = [&](int l) { return l == n_layers - 1 ? x_final : xpp[l % 2]; };

  // every check first (nothing is enqueued on an error), then the launches
  sw::RouteArgs r;
  sw::GateUpArgs g;
  sw::DownArgs d;
  int max_slots = 0, rc;
  for (int l = 0; l < n_layers; l++) {
    const strata_layer& L = layers[l];
    if (L.gate.bits != layers[0].gate.bits)
      return fail(STRATA_EINVAL, "layer %d: bits %d differ from layer 0's %d", l, L.gate.bits, layers[0].gate.bits);
    if ((rc = prepare_route(input(l), input_dtype(l), rows, hidden, L.gate_w, L.logit_bias, n_experts, top_k, flags,
                            &L.route, ws, w.layer.partials, r)) ||
        (rc = prepare_moe(input(l), input_dtype(l), rows, hidden, ffn, &L.gate, &L.up, &L.down, &L.sh_gate, &L.sh_up,
                          &L.sh_down, &L.route, n_experts, top_k, input(l), l == n_layers - 1 ? out : nullptr,
                          output(l), ws, w.layer.moe, g, d, max_slots, true))) {
      char msg[sizeof g_err];
      snprintf(msg, sizeof msg, "%s", g_err);
      return fail(rc, "layer %d: %s", l, msg);
    }
  }
  sw::HeadArgs ha;
  if (head) {
    if (vocab < 1) return fail(STRATA_EINVAL, "vocab %d < 1", vocab);
    if ((rc = check_qmat(head, "head", vocab, hidden, 1, 8))) return rc;
    if (!argmax || !aligned(argmax, 16)) return fail(STRATA_EINVAL, "argmax NULL or not 16-byte aligned");
    if (logits && !aligned(logits, 16)) return fail(STRATA_EINVAL, "logits not 16-byte aligned");
    const size_t lds = (size_t)8 * (hidden + 8) * 2 + (size_t)(hidden / 32) * 64;
    if (lds + kStaticLds > kLdsLimit)
      return fail(STRATA_EUNSUPPORTED, "hidden %d needs more than %zu bytes of LDS", hidden, kLdsLimit);
    ha.x = x_final; ha.x_dtype = STRATA_BF16; ha.rows = rows; ha.hidden = hidden; ha.vocab = vocab;
    ha.codes = (const uint8_t*)head->codes; ha.meta = (const uint8_t*)head->meta;
    ha.logits = logits; ha.argmax = argmax;
    ha.part_val = (float*)(wb + w.head + w.hw.val); ha.part_idx = (int32_t*)(wb + w.head + w.hw.idx);
  }

  hipStream_t s = (hipStream_t)stream;
  // the events: the first launch (layer 0's router) records the start, the last (the
  // head's, else the last layer's combine) the end
  sw::Prof first, last;
  if (prof_events) { first.start = (hipEvent_t)prof_events[0]; last.stop = (hipEvent_t)prof_events[1]; }
  const sw::Prof* p_first = prof_events ? &first : nullptr;
  const sw::Prof* p_last = prof_events ? &last : nullptr;
  for (int l = 0; l < n_layers; l++) {
    const strata_layer& L = layers[l];
    prepare_route(input(l), input_dtype(l), rows, hidden, L.gate_w, L.logit_bias, n_experts, top_k, flags, &L.route,
                  ws, w.layer.partials, r);
    prepare_moe(input(l), input_dtype(l), rows, hidden, ffn, &L.gate, &L.up, &L.down, &L.sh_gate, &L.sh_up,
                &L.sh_down, &L.route, n_experts, top_k, input(l), l == n_layers - 1 ? out : nullptr, output(l), ws,
                w.layer.moe, g, d, max_slots, true);
    g.route = r;
    const bool last_layer = l == n_layers - 1;
    // layer 0's router GEMV here; every later layer's partials come from the hand-over.
    // Where the routing core's tables do not fit beside the activations, the routing
    // core runs as a kernel of its own and gate/up reads its tables.
    const bool fused = fused_fits(hidden, input_dtype(l));
    if (l == 0 && (rc = launch_status(sw::launch_route_logits(r, s, p_first), "router"))) return rc;
    if (!fused && (rc = launch_status(sw::launch_route_final(r, s, nullptr), "routing"))) return rc;
    if ((rc = launch_status(fused ? sw::launch_gateup_routed(g, max_slots, s, nullptr)
                                  : sw::launch_gateup(g, max_slots, s, nullptr), "gate/up")))
      return rc;
    if ((rc = launch_status(sw::launch_down(d, s, last_layer && !head ? p_last : nullptr, last_layer),
                            "down")))
      return rc;
    if (!last_layer) {
      // layer l's combine and layer l + 1's router in one launch
      const strata_layer& N = layers[l + 1];
      sw::RouteArgs rn;
      prepare_route(output(l), STRATA_BF16, rows, hidden, N.gate_w, N.logit_bias, n_experts, top_k, flags, &N.route,
                    ws, w.layer.partials, rn);
      sw::CombineRouteArgs c;
      c.route = rn;
      c.y = d.y; c.row_w = d.row_w; c.top_k = top_k;
      c.x_res = input(l); c.x_next = output(l); c.out = nullptr;
      if ((rc = launch_status(sw::launch_combine_route(c, input_dtype(l) == STRATA_F32, s, nullptr), "combine + router")))
        return rc;
    }
  }
  if (head) return launch_status(sw::launch_head(ha, s, p_last), "head");
  return STRATA_OK;
}

int strata_window_head(void* stream, const void* x, int x_dtype, int rows, int hidden, const strata_qmat* head,
                       int vocab, float* logits, int32_t* argmax, void* ws, size_t ws_bytes,
                       void* const* prof_events) {
  g_err[0] = 0;
  int rc;
  if ((rc = check_common(x, x_dtype, rows, hidden, ws))) return rc;
  if (vocab < 1) return fail(STRATA_EINVAL, "vocab %d < 1", vocab);
  if ((rc = check_qmat(head, "head", vocab, hidden, 1, 8))) return rc;
  if (!argmax || !aligned(argmax, 16)) return fail(STRATA_EINVAL, "argmax NULL or not 16-byte aligned");
  if (logits && !aligned(logits, 16)) return fail(STRATA_EINVAL, "logits not 16-byte aligned");
  const size_t lds = (size_t)(x_dtype == STRATA_F32 ? 16 : 8) * (hidden + 8) * 2 + (size_t)(hidden / 32) * 64;
  if (lds + kStaticLds > kLdsLimit)
    return fail(STRATA_EUNSUPPORTED, "hidden %d needs more than %zu bytes of LDS", hidden, kLdsLimit);
  const HeadWs w = head_ws(rows, vocab);
  if (ws_bytes < w.total) return fail(STRATA_EINVAL, "head workspace %zu < %zu bytes", ws_bytes, w.total);

  sw::HeadArgs a;
  a.x = x; a.x_dtype = x_dtype; a.rows = rows; a.hidden = hidden; a.vocab = vocab;
  a.codes = (const uint8_t*)head->codes; a.meta = (const uint8_t*)head->meta;
  a.logits = logits; a.argmax = argmax;
  a.part_val = (float*)((char*)ws + w.val); a.part_idx = (int32_t*)((char*)ws + w.idx);
  const sw::Prof ph = prof(prof_events, 0);
  return launch_status(sw::launch_head(a, (hipStream_t)stream, prof_events ? &ph : nullptr), "head");
}

int strata_window_accept(void* stream, const int32_t* argmax, int rows, int n_slots, int mtp,
                         const int32_t* proposal, int32_t* tokens, int32_t* n_tokens, int32_t* n_accepted,
                         void* const* prof_events) {
  g_err[0] = 0;
  if (mtp != 0 && mtp != 1) return fail(STRATA_EINVAL, "mtp %d is neither 0 nor 1", mtp);
  if (n_slots < 1 || n_slots > STRATA_MAX_ROWS / (mtp ? 2 : 1))
    return fail(STRATA_EINVAL, "n_slots %d outside 1..%d", n_slots, STRATA_MAX_ROWS / (mtp ? 2 : 1));
  if (rows != n_slots * (mtp ? 2 : 1))
    return fail(STRATA_EINVAL, "rows %d is not %d per slot x %d slots", rows, mtp ? 2 : 1, n_slots);
  const void* p[] = {argmax, tokens, n_tokens, n_accepted};
  const char* nm[] = {"argmax", "tokens", "n_tokens", "n_accepted"};
  for (int i = 0; i < 4; i++)
    if (!p[i] || !aligned(p[i], 16)) return fail(STRATA_EINVAL, "%s NULL or not 16-byte aligned", nm[i]);
  if (mtp && (!proposal || !aligned(proposal, 16)))
    return fail(STRATA_EINVAL, "proposal NULL or not 16-byte aligned");
  sw::AcceptArgs a;
  a.argmax = argmax; a.n_slots = n_slots; a.mtp = mtp; a.proposal = proposal;
  a.tokens = tokens; a.n_tokens = n_tokens; a.n_accepted = n_accepted;
  const sw::Prof pa = prof(prof_events, 0);
  return launch_status(sw::launch_accept(a, (hipStream_t)stream, prof_events ? &pa : nullptr), "accept");
}

int strata_window_sample(void* stream, const float* logits, int rows, int vocab, const strata_sample_params* params,
                         const int64_t* position, int32_t* tokens, void* ws, size_t ws_bytes,
                         void* const* prof_events) {
  g_err[0] = 0;
  if (rows < 1 || rows > STRATA_MAX_ROWS) return fail(STRATA_EINVAL, "rows %d outside 1..%d", rows, STRATA_MAX_ROWS);
  if (vocab < 1) return fail(STRATA_EINVAL, "vocab %d < 1", vocab);
  const void* p[] = {logits, params, position, tokens, ws};
  const char* nm[] = {"logits", "params", "position", "tokens", "ws"};
  for (int i = 0; i < 5; i++)
    if (!p[i] || !aligned(p[i], 16)) return fail(STRATA_EINVAL, "%s NULL or not 16-byte aligned", nm[i]);
  const SampleWs w = sample_ws(rows, vocab);
  if (ws_bytes < w.total) return fail(STRATA_EINVAL, "workspace %zu bytes < %zu", ws_bytes, w.total);
  static_assert(sizeof(strata_sample_params) == sizeof(sw::SampleParams), "parameter layouts");
  sw::SampleArgs a;
  a.logits = logits; a.rows = rows; a.vocab = vocab;
  a.params = (const sw::SampleParams*)params; a.position = position; a.tokens = tokens;
  a.chunks = sw::sample_chunks(vocab);
  a.cand_key = (uint32_t*)((char*)ws + w.key);
  a.cand_idx = (uint32_t*)((char*)ws + w.idx);
  a.cand_lo = (uint32_t*)((char*)ws + w.lo);
  const sw::Prof ps = prof(prof_events, 0);
  return launch_status(sw::launch_sample(a, (hipStream_t)stream, prof_events ? &ps : nullptr), "sample");
}

int strata_window_stream_read(void* stream, const void* src, size_t bytes, uint32_t* sink, uint32_t magic,
                              void* const* prof_events) {
  g_err[0] = 0;
  if (!src || !aligned(src, 16)) return fail(STRATA_EINVAL, "src NULL or not 16-byte aligned");
  if (!sink || !aligned(sink, 4)) return fail(STRATA_EINVAL, "sink NULL or not 4-byte aligned");
  if (bytes == 0 || bytes % 16) return fail(STRATA_EINVAL, "bytes %zu not a nonzero multiple of 16", bytes);
  sw::StreamArgs a;
  a.src = src; a.words = bytes / 16; a.sink = sink; a.magic = magic;
  const sw::Prof pa = prof(prof_events, 0);
  return launch_status(sw::launch_stream_read(a, (hipStream_t)stream, prof_events ? &pa : nullptr), "stream_read");
}

int strata_window_tier(void* stream, const uint8_t* row_mask, int n_experts, float* counts, float decay,
                       uint8_t* resident, int max_swaps, float min_gain, int32_t* swaps, int32_t* n_swaps,
                       void* const* prof_events) {
  g_err[0] = 0;
  if (n_experts < 1 || n_experts > STRATA_MAX_EXPERTS)
    return fail(STRATA_EINVAL, "n_experts %d outside 1..%d", n_experts, STRATA_MAX_EXPERTS);
  if (!row_mask || !aligned(row_mask, 16)) return fail(STRATA_EINVAL, "row_mask NULL or not 16-byte aligned");
  if (!counts || !aligned(counts, 16)) return fail(STRATA_EINVAL, "counts NULL or not 16-byte aligned");
  if (!(decay >= 0.f && decay <= 1.f)) return fail(STRATA_EINVAL, "decay %g outside [0, 1]", (double)decay);
  if (resident) {
    if (!aligned(resident, 16)) return fail(STRATA_EINVAL, "resident not 16-byte aligned");
    if (max_swaps < 0 || max_swaps > n_experts) return fail(STRATA_EINVAL, "max_swaps %d outside 0..%d", max_swaps, n_experts);
    if (!(min_gain >= 0.f && min_gain < 1e30f)) return fail(STRATA_EINVAL, "min_gain %g is not a finite value >= 0", (double)min_gain);
    if (!n_swaps || !aligned(n_swaps, 16)) return fail(STRATA_EINVAL, "n_swaps NULL or not 16-byte aligned");
    if (max_swaps > 0 && (!swaps || !aligned(swaps, 16))) return fail(STRATA_EINVAL, "swaps NULL or not 16-byte aligned");
  }
  sw::TierArgs a;
  a.row_mask = row_mask; a.n_experts = n_experts; a.counts = counts; a.decay = decay;
  a.resident = resident; a.max_swaps = resident ? max_swaps : 0; a.min_gain = min_gain;
  a.swaps = swaps; a.n_swaps = n_swaps;
  const sw::Prof pt = prof(prof_events, 0);
  return launch_status(sw::launch_tier(a, (hipStream_t)stream, prof_events ? &pt : nullptr), "tier");
}

}  // extern "C"
