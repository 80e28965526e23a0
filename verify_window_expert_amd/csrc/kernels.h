// Kernel argument blocks and launchers of the window kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include <mutex>

namespace sw {

struct RouteArgs {
  const void* x; int x_dtype; int rows, hidden;
  const float* gate_w; const float* bias; int n_experts, top_k, renorm;
  double* partials;         // [chunk][row][expert]
  int32_t* topk_idx; float* topk_w; int32_t* n_active; int32_t* active; int32_t* offsets;
  int32_t* entry_row; float* entry_w; uint8_t* row_mask;
  int32_t* entry_pos; float* row_w;
};

// One quantized matrix family: routed experts (stacked) and the shared expert.
struct QDev {
  const uint8_t* codes; const uint8_t* meta;      // routed, matrix 0
  int64_t stride_codes, stride_meta_bytes;        // between routed matrices
  const uint8_t* sh_codes; const uint8_t* sh_meta;
};

struct GateUpArgs {
  RouteArgs route;          // the fused layer: the routing core runs in every workgroup
  const void* x; int x_dtype; int rows, hidden, ffn, bits, n_experts;
  QDev gate, up;
  const int32_t* n_active; const int32_t* active; const int32_t* offsets;
  const int32_t* entry_row; const uint8_t* row_mask;
  uint16_t* h_hi;           // [entries][ffn]: h rounded to bf16, in the permuted order
  uint16_t* h_lo;           // [entries][ffn]: bf16 rounding of h - hi, same order
  int max_slots;            // capacity of the active array (offsets: max_slots + 1)
  int split;                // set by the launcher: waves per item (1 or 2), fixed by the
                            // shapes alone so a row's sums never depend on the window
};

struct DownArgs {
  const void* x_res; int x_dtype; int rows, hidden, ffn, bits, n_experts;
  QDev down;
  const int32_t* n_active; const int32_t* active; const int32_t* offsets;
  const int32_t* entry_row; const int32_t* entry_pos; const float* row_w;
  const uint16_t* h_hi; const uint16_t* h_lo;   // as GateUpArgs
  int h_entries;            // entries the h arrays hold (rows * top_k + rows)
  float* y;                 // [rows][top_k + 1][hidden]: row r's experts in ascending id order
  float* out; uint16_t* x_next;   // either may be NULL
  int max_slots, top_k;     // capacity of the active / offsets arrays; routing top-k
};

struct HeadArgs {
  const void* x; int x_dtype; int rows, hidden, vocab;
  const uint8_t* codes; const uint8_t* meta;
  float* logits;            // nullable
  int32_t* argmax;
  float* part_val; int32_t* part_idx;   // [workgroups][rows]
};

struct AcceptArgs {
  const int32_t* argmax; int n_slots, mtp;
  const int32_t* proposal;  // [n_slots] (mtp only)
  int32_t* tokens; int32_t* n_tokens; int32_t* n_accepted;
};

// One row's sampling parameters (the layout of strata_sample_params).
struct SampleParams {
  float temperature; int32_t top_k; float top_p; float min_p; uint64_t seed;
};

struct SampleArgs {
  const float* logits; int rows, vocab;
  const SampleParams* params;   // [rows]
  const int64_t* position;      // [rows]
  int32_t* tokens;              // [rows]
  int chunks;                   // sample_chunks(vocab)
  uint32_t* cand_key;           // [rows][chunks][128]: each chunk's best keys (workspace)
  uint32_t* cand_idx;           // [rows][chunks][128]: their indices
  uint32_t* cand_lo;            // [rows][chunks]: a key at most each chunk's K-th largest
};

struct TierArgs {
  const uint8_t* row_mask; int n_experts;
  float* counts; float decay;
  uint8_t* resident;        // NULL: counting only
  int max_swaps; float min_gain;
  int32_t* swaps; int32_t* n_swaps;
};

// A stack's hand-over between layers l and l + 1 (one launch): layer l's combine and
// layer l + 1's router GEMV.
struct CombineRouteArgs {
  RouteArgs route;          // layer l + 1's router (its x is formed here, not read)
  const float* y; const float* row_w; int top_k;   // layer l's expert outputs, weights
  const void* x_res;        // layer l's input (the residual); nullable
  uint16_t* x_next;         // [rows][hidden] bf16: layer l + 1's input (written)
  float* out;               // [rows][hidden] float, nullable: layer l's output
};

struct StreamArgs {
  const void* src; size_t words;   // 16-byte words
  uint32_t* sink; uint32_t magic;  // written only if the fold of a wave's words equals magic
  size_t chunk;                    // set by the launcher: bytes per wave
};

// Optional timing events of one launch (both may be null): recorded by the dispatch
// itself at the kernel's start and end (hipExtLaunchKernel).
struct Prof {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Launch `kernel`, with the dispatch recording `p`'s events when given.
template <typename K, typename... Args>
inline void launch(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, const Prof* p, Args... args) {
  if (p && (p->start || p->stop))
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, p->start, p->stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

// Raise a kernel's dynamic LDS limit when its static LDS plus `bytes` of dynamic LDS
// exceed the default 64 KB (once per process and kernel; the attribute only grows).
template <auto kernel>
inline int set_lds(size_t bytes) {
  static std::mutex m;
  static size_t granted = 0;
  std::lock_guard<std::mutex> lock(m);
  if (bytes <= granted) return 0;
  hipFuncAttributes fa;
  if (int e = (int)hipFuncGetAttributes(&fa, (const void*)kernel)) return e;
  if (fa.sharedSizeBytes + bytes > 64 * 1024) {
    const int e = (int)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e) return e;
  }
  granted = bytes;
  return 0;
}

// Launchers return the hipError_t of the launch (0 on success).
int launch_route(const RouteArgs& a, hipStream_t s, const Prof* p);
int launch_gateup(const GateUpArgs& a, int max_slots, hipStream_t s, const Prof* p);
// the fused layer's gate/up: routing from a.route's partials in every workgroup (one more
// workgroup writes the routing outputs), then gate/up as launch_gateup
int launch_gateup_routed(const GateUpArgs& a, int max_slots, hipStream_t s, const Prof* p);
// the router's GEMV alone (the fused layer's first kernel), and the routing core alone
// (top-k, softmax, grouping from the GEMV's partials: one workgroup)
int launch_route_logits(const RouteArgs& a, hipStream_t s, const Prof* p);
int launch_route_final(const RouteArgs& a, hipStream_t s, const Prof* p);
// down, then (combine) the combine kernel
int launch_down(const DownArgs& a, hipStream_t s, const Prof* p, bool combine = true);
// layer l's combine and layer l + 1's router GEMV in one launch (res_f32: layer l's input
// is float)
int launch_combine_route(const CombineRouteArgs& c, int res_f32, hipStream_t s, const Prof* p);
size_t down_lds_bytes(int ffn);
int launch_head(const HeadArgs& a, hipStream_t s, const Prof* p);
int launch_accept(const AcceptArgs& a, hipStream_t s, const Prof* p);
int launch_sample(const SampleArgs& a, hipStream_t s, const Prof* p);
int sample_chunks(int vocab);   // 4096-logit chunks of a row in the sampled draw
int launch_tier(const TierArgs& a, hipStream_t s, const Prof* p);
int launch_stream_read(const StreamArgs& a, hipStream_t s, const Prof* p);
int head_workgroups(int vocab);
// dynamic LDS of the gate/up kernel (the activation image)
size_t gateup_lds_bytes(int hidden, int x_dtype);
size_t route_core_lds_bytes();   // the fused layer's gate/up: the routing core's static LDS

}  // namespace sw
