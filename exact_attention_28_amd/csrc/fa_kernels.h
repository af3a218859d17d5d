// fa_kernels.h - host-side launchers of the gfx950 kernels (internal).
// Arguments have been validated by the C ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  bool causal;
  float s_q, s_k, s_v;  // fp8 per-tensor scales (1 for other dtypes)
  hipStream_t stream;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  bool causal;
  void* ws;  // row sums D and log2-scaled LSE
  hipStream_t stream;
};
size_t bwd_workspace_bytes(int B, int Hq, int Nq);
hipError_t launch_bwd_bf16(const BwdArgs& a);

struct NaiveArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  bool causal;
  void* ws;  // S (fp16), then P (bf16) in place: B*Hq*Nq*Nk * 2 bytes
  hipStream_t stream;
};
size_t naive_workspace_bytes(int B, int Hq, int Nq, int Nk);
hipError_t launch_naive_bf16(const NaiveArgs& a);

hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_fwd_bf16(const FwdArgs& a);
// The bf16 forward over a paged cache: a.k, a.v are the pools, a.Nk unused;
// keys of request b are seq_lens[b] tokens through block_table.
hipError_t launch_paged_prefill_bf16(const FwdArgs& a, const int32_t* bt,
                                     const int32_t* sl, int max_pages,
                                     int num_pages);
hipError_t launch_fwd_fp8(const FwdArgs& a);
// The bf16 forward at d = 128 with the two waves of each SIMD in opposite
// phases (matrix phase written out as inline asm): contiguous K/V, and over
// a paged cache (arguments as launch_paged_prefill_bf16).
hipError_t launch_fwd_bf16_pp(const FwdArgs& a);
hipError_t launch_paged_prefill_bf16_pp(const FwdArgs& a, const int32_t* bt,
                                        const int32_t* sl, int max_pages,
                                        int num_pages);

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int num_pages, B, Hq, Hkv, d, max_pages;
  float scale;
  void* o;
  float* lse;  // may be null
  void* ws;    // page-range bookkeeping and partials
  bool kv_fp8;     // pools hold e4m3 codes with per-tensor scales
  float s_k, s_v;  // the pools' scales (1 for bf16)
  hipStream_t stream;
};

// Work split shared by the workspace-size query and the launch: the batch's
// page list is cut into `ranges` equal ranges per KV head; a workgroup of
// `nw` waves holds `heads_per_wg` KV heads x `waves_per_head` ranges.
struct DecodePlan {
  int nw, heads_per_wg, waves_per_head, head_groups, ranges;
  long grid;
  long off_o, off_l;  // workspace word offsets of partial O and LSE
  size_t workspace_bytes;
};
// Returns false when the requested split count cannot be honoured.
bool plan_decode(int B, int Hq, int Hkv, int d, int max_pages,
                 int num_splits, DecodePlan* plan);

hipError_t launch_paged_decode(const DecodeArgs& a, const DecodePlan& plan);

// Size of the decode's built-in workspace (one per device, for the entry
// point that allocates nothing), and its device address on the current
// device: looked up with hipGetSymbolAddress on the first call per device,
// then reused. Returns the lookup's error, if any.
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace fa
