// Host-side launchers shared by the C ABI (api.cpp) and the kernel sources.
// Arguments reaching these functions have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* kv_seqlens;
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  hipStream_t stream;
  // Packed variable-length sequences (cu_q == nullptr: the [B, H, N, d]
  // layout).  q, o [Hq, total_q, d]; k, v [Hkv, total_k, d]; lse [Hq, total_q];
  // sequence b owns query rows cu_q[b] .. cu_q[b+1]-1 and key rows
  // cu_k[b] .. cu_k[b+1]-1.  Nq then bounds the longest query sequence.
  const int32_t* cu_q = nullptr;
  const int32_t* cu_k = nullptr;
  int total_q = 0, total_k = 0;
};

struct PartialOut {
  float* o_part;    // [B, Hq, S, d]
  float* lse_part;  // [B, Hq, S]
  int num_splits;   // S
};

// bf16 prefill forward on matrix cores.
hipError_t launch_fwd_bf16(const AttnArgs& a);
// float32 forward; with part != nullptr it computes split-KV partials instead
// of the final output (single-token decode in float32).
hipError_t launch_fwd_f32(const AttnArgs& a, const PartialOut* part);
// A paged KV cache: pools k, v [num_pages, Hkv, page_size, d] and a block
// table [B, max_pages] of page indices in key order.
struct PagedKV {
  const int32_t* block_table;
  int page_size, max_pages, num_pages;
};

// bf16 split-KV decode partials on matrix cores (Nq == 1); with paged != null
// the cache is read through the block table (a.Nk = max_pages * page_size).
hipError_t launch_decode_splitkv_bf16(const AttnArgs& a, const PartialOut& part, const PagedKV* paged = nullptr);
// Exact log-sum-exp merge of split partials into o (bf16 or f32) and lse.
hipError_t launch_lse_merge(const float* o_part, const float* lse_part, void* o, float* lse,
                            int rows, int d, int num_splits, bool out_bf16, hipStream_t stream);

// Device address of the static decode scratch (FA_NOALLOC_SCRATCH_BYTES) on
// the current device; looked up once per device.
hipError_t noalloc_scratch(void** ptr);

// FP8 prefill forward (d = 128): q, k, v hold FP8 codes (E4M3, or E5M2 when
// e5m2 != 0) whose real values are descale * value(code); o is bf16.
struct Fp8Scales {
  float q_descale, k_descale, v_descale;
};
hipError_t launch_fwd_fp8(const AttnArgs& a, int e5m2, const Fp8Scales& sc);

// Backward pass (bf16): gradients of fa_fwd's output.
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
  float* rowdot;  // workspace: rowsum(dO * O) per query row, [B, Hq, Nq]
  const int32_t* kv_seqlens;
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  hipStream_t stream;
};
hipError_t launch_bwd_bf16(const BwdArgs& a);

// Split-KV chunk length for a sequence of `len` valid keys.
__host__ __device__ inline int split_chunk(int len, int num_splits, int align) {
  if (len <= 0) return 0;
  int c = (len + num_splits - 1) / num_splits;
  return (c + align - 1) / align * align;
}

}  // namespace fa
