// C ABI of libfa.so: argument validation (before any HIP call), kernel
// selection and launch on the caller's stream.  See include/fa.h for the
// contract of each entry point.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "fa_launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return FA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(FA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t lse_offset(size_t part_bytes) { return (part_bytes + 255) / 256 * 256; }

// Checks shared by the prefill and decode entry points.
int check_common(int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int dtype) {
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0)
    return fail(FA_ERR_INVALID_ARG, "sizes must be non-negative (B=%d Hq=%d Hkv=%d Nq=%d Nk=%d)", B, Hq, Hkv,
                Nq, Nk);
  if (dtype != FA_F32 && dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", d);
  if (Hq > 0 && (Hkv <= 0 || Hq % Hkv != 0))
    return fail(FA_ERR_UNSUPPORTED, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  return FA_OK;
}

int check_ptr(const void* p, size_t align, const char* name) {
  if (p == nullptr) return fail(FA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, align)) return fail(FA_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
  return FA_OK;
}

int check_splits(int num_splits) {
  if (num_splits < 1 || num_splits > FA_MAX_SPLITS)
    return fail(FA_ERR_UNSUPPORTED, "num_splits %d outside [1, %d]", num_splits, FA_MAX_SPLITS);
  return FA_OK;
}

int check_decode_args(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int Nk, int d,
                      float scale, int num_splits, int dtype) {
  int st = check_common(B, Hq, Hkv, 1, Nk, d, scale, dtype);
  if (st != FA_OK) return st;
  if ((st = check_splits(num_splits)) != FA_OK) return st;
  if ((long long)Hkv * ((Hq / (Hkv > 0 ? Hkv : 1) + 31) / 32) > 65535 || B > 65535)
    return fail(FA_ERR_UNSUPPORTED, "decode grid too large (B=%d, Hkv=%d)", B, Hkv);
  if ((long long)B * Hq == 0) return FA_OK;
  if ((st = check_ptr(q, 16, "q")) != FA_OK) return st;
  if (Nk > 0) {
    if ((st = check_ptr(k, 16, "k_cache")) != FA_OK) return st;
    if ((st = check_ptr(v, 16, "v_cache")) != FA_OK) return st;
  }
  return FA_OK;
}

fa::AttnArgs make_args(const void* q, const void* k, const void* v, void* o, float* lse,
                       const int32_t* kv_seqlens, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                       int causal, void* stream) {
  fa::AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.kv_seqlens = kv_seqlens;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk; a.d = d;
  a.scale = scale;
  a.causal = causal;
  a.stream = (hipStream_t)stream;
  return a;
}

// Both decode stages on a workspace the caller validated (or the static
// scratch): partials, then the merge.
int decode_launch(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B, int Hq,
                  int Hkv, int Nk, int d, float scale, const int32_t* kv_seqlens, int num_splits, void* workspace,
                  int dtype, void* stream) {
  const size_t rows = (size_t)B * Hq;
  float* o_part = (float*)workspace;
  float* lse_part = (float*)((char*)workspace + lse_offset(rows * num_splits * d * sizeof(float)));
  fa::AttnArgs a = make_args(q, k_cache, v_cache, nullptr, nullptr, kv_seqlens, B, Hq, Hkv, 1, Nk, d, scale, 0,
                             stream);
  fa::PartialOut part{o_part, lse_part, num_splits};
  hipError_t e = dtype == FA_BF16 ? fa::launch_decode_splitkv_bf16(a, part) : fa::launch_fwd_f32(a, &part);
  if (e != hipSuccess) return hip_status(e, "fa_decode split stage launch");
  return hip_status(fa::launch_lse_merge(o_part, lse_part, o, lse, (int)rows, d, num_splits, dtype == FA_BF16,
                                         (hipStream_t)stream),
                    "fa_decode merge stage launch");
}

}  // namespace

extern "C" {

int fa_version(void) { return 100; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "FA_UNKNOWN_STATUS";
  }
}

const char* fa_last_error(void) { return g_last_error; }

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
           int Nk, int d, float scale, int causal, const int32_t* kv_seqlens, int dtype, void* stream) {
  int st = check_common(B, Hq, Hkv, Nq, Nk, d, scale, dtype);
  if (st != FA_OK) return st;
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if ((long long)B * Hq * Nq == 0) return ok();  // nothing to write
  if ((st = check_ptr(q, 16, "q")) != FA_OK) return st;
  if ((st = check_ptr(o, 16, "o")) != FA_OK) return st;
  if ((st = check_ptr(lse, 4, "lse")) != FA_OK) return st;
  if (Nk > 0) {
    if ((st = check_ptr(k, 16, "k")) != FA_OK) return st;
    if ((st = check_ptr(v, 16, "v")) != FA_OK) return st;
  }
  if (kv_seqlens != nullptr && !aligned(kv_seqlens, 4))
    return fail(FA_ERR_INVALID_ARG, "kv_seqlens is not 4-byte aligned");
  const long long tiles = ((long long)Nq + 127) / 128 * B * Hq;
  if (tiles > 0x7fffffffLL) return fail(FA_ERR_UNSUPPORTED, "problem too large for one launch");
  fa::AttnArgs a = make_args(q, k, v, o, lse, kv_seqlens, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream);
  if (dtype == FA_BF16) return hip_status(fa::launch_fwd_bf16(a), "fa_fwd (bf16) launch");
  return hip_status(fa::launch_fwd_f32(a, nullptr), "fa_fwd (f32) launch");
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
               int Nk, int d, float scale, int causal, const int32_t* kv_seqlens, float q_descale, float k_descale,
               float v_descale, int dtype, void* stream) {
  if (dtype != FA_FP8_E4M3 && dtype != FA_FP8_E5M2)
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd_fp8 takes dtype FA_FP8_E4M3 or FA_FP8_E5M2, got %d", dtype);
  int st = check_common(B, Hq, Hkv, Nq, Nk, d, scale, FA_BF16);
  if (st != FA_OK) return st;
  if (d != 128) return fail(FA_ERR_UNSUPPORTED, "fa_fwd_fp8 supports head dim 128 only (got %d)", d);
  for (float ds : {q_descale, k_descale, v_descale})
    if (!(std::isfinite(ds) && ds > 0.f)) return fail(FA_ERR_INVALID_ARG, "descales must be finite and > 0");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if ((long long)B * Hq * Nq == 0) return ok();
  if ((st = check_ptr(q, 16, "q")) != FA_OK) return st;
  if ((st = check_ptr(o, 16, "o")) != FA_OK) return st;
  if ((st = check_ptr(lse, 4, "lse")) != FA_OK) return st;
  if (Nk > 0) {
    if ((st = check_ptr(k, 16, "k")) != FA_OK) return st;
    if ((st = check_ptr(v, 16, "v")) != FA_OK) return st;
  }
  if (kv_seqlens != nullptr && !aligned(kv_seqlens, 4))
    return fail(FA_ERR_INVALID_ARG, "kv_seqlens is not 4-byte aligned");
  const long long tiles = ((long long)Nq + 255) / 256 * B * Hq;
  if (tiles > 0x7fffffffLL) return fail(FA_ERR_UNSUPPORTED, "problem too large for one launch");
  fa::AttnArgs a = make_args(q, k, v, o, lse, kv_seqlens, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream);
  return hip_status(fa::launch_fwd_fp8(a, dtype == FA_FP8_E5M2, fa::Fp8Scales{q_descale, k_descale, v_descale}),
                    "fa_fwd_fp8 launch");
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens_q,
                  const int32_t* cu_seqlens_k, int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                  int d, float scale, int causal, int dtype, void* stream) {
  int st = check_common(B, Hq, Hkv, total_q, total_k, d, scale, dtype);
  if (st != FA_OK) return st;
  if (max_seqlen_q < 0) return fail(FA_ERR_INVALID_ARG, "max_seqlen_q must be non-negative");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if ((long long)B * Hq * total_q == 0 || max_seqlen_q == 0) return ok();  // nothing to write
  if ((st = check_ptr(cu_seqlens_q, 4, "cu_seqlens_q")) != FA_OK) return st;
  if ((st = check_ptr(cu_seqlens_k, 4, "cu_seqlens_k")) != FA_OK) return st;
  if ((st = check_ptr(q, 16, "q")) != FA_OK) return st;
  if ((st = check_ptr(o, 16, "o")) != FA_OK) return st;
  if ((st = check_ptr(lse, 4, "lse")) != FA_OK) return st;
  if (total_k > 0) {
    if ((st = check_ptr(k, 16, "k")) != FA_OK) return st;
    if ((st = check_ptr(v, 16, "v")) != FA_OK) return st;
  }
  const long long tiles = ((long long)max_seqlen_q + 127) / 128 * B * Hq;
  if (tiles > 0x7fffffffLL) return fail(FA_ERR_UNSUPPORTED, "problem too large for one launch");
  fa::AttnArgs a = make_args(q, k, v, o, lse, nullptr, B, Hq, Hkv, max_seqlen_q, 0, d, scale, causal, stream);
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  a.total_k = total_k;
  if (dtype == FA_BF16) return hip_status(fa::launch_fwd_bf16(a), "fa_fwd_varlen (bf16) launch");
  return hip_status(fa::launch_fwd_f32(a, nullptr), "fa_fwd_varlen (f32) launch");
}

size_t fa_decode_workspace_bytes(int B, int Hq, int d, int num_splits) {
  if (B < 0 || Hq < 0 || (d != 64 && d != 128) || num_splits < 1 || num_splits > FA_MAX_SPLITS) return 0;
  const size_t rows = (size_t)B * Hq * num_splits;
  return lse_offset(rows * d * sizeof(float)) + rows * sizeof(float);
}

int fa_decode_splitkv(const void* q, const void* k_cache, const void* v_cache, float* o_part, float* lse_part,
                      int B, int Hq, int Hkv, int Nk, int d, float scale, const int32_t* kv_seqlens,
                      int num_splits, int dtype, void* stream) {
  int st = check_decode_args(q, k_cache, v_cache, B, Hq, Hkv, Nk, d, scale, num_splits, dtype);
  if (st != FA_OK) return st;
  if ((long long)B * Hq == 0) return ok();
  if ((st = check_ptr(o_part, 16, "o_part")) != FA_OK) return st;
  if ((st = check_ptr(lse_part, 4, "lse_part")) != FA_OK) return st;
  if (kv_seqlens != nullptr && !aligned(kv_seqlens, 4))
    return fail(FA_ERR_INVALID_ARG, "kv_seqlens is not 4-byte aligned");
  fa::AttnArgs a = make_args(q, k_cache, v_cache, nullptr, nullptr, kv_seqlens, B, Hq, Hkv, 1, Nk, d, scale, 0,
                             stream);
  fa::PartialOut part{o_part, lse_part, num_splits};
  if (dtype == FA_BF16) return hip_status(fa::launch_decode_splitkv_bf16(a, part), "fa_decode_splitkv launch");
  return hip_status(fa::launch_fwd_f32(a, &part), "fa_decode_splitkv (f32) launch");
}

int fa_lse_merge(const float* o_part, const float* lse_part, void* o, float* lse, int rows, int d,
                 int num_splits, int dtype, void* stream) {
  if (rows < 0) return fail(FA_ERR_INVALID_ARG, "rows must be non-negative");
  if (dtype != FA_F32 && dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", d);
  int st = check_splits(num_splits);
  if (st != FA_OK) return st;
  if (rows == 0) return ok();
  if ((st = check_ptr(o_part, 16, "o_part")) != FA_OK) return st;
  if ((st = check_ptr(lse_part, 4, "lse_part")) != FA_OK) return st;
  if ((st = check_ptr(o, 16, "o")) != FA_OK) return st;
  if ((st = check_ptr(lse, 4, "lse")) != FA_OK) return st;
  return hip_status(fa::launch_lse_merge(o_part, lse_part, o, lse, rows, d, num_splits, dtype == FA_BF16,
                                         (hipStream_t)stream),
                    "fa_lse_merge launch");
}

int fa_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B, int Hq,
              int Hkv, int Nk, int d, float scale, const int32_t* kv_seqlens, int num_splits, void* workspace,
              size_t workspace_bytes, int dtype, void* stream) {
  int st = check_decode_args(q, k_cache, v_cache, B, Hq, Hkv, Nk, d, scale, num_splits, dtype);
  if (st != FA_OK) return st;
  if ((long long)B * Hq == 0) return ok();
  if ((st = check_ptr(o, 16, "o")) != FA_OK) return st;
  if ((st = check_ptr(lse, 4, "lse")) != FA_OK) return st;
  const size_t need = fa_decode_workspace_bytes(B, Hq, d, num_splits);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!aligned(workspace, 256)) return fail(FA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if (kv_seqlens != nullptr && !aligned(kv_seqlens, 4))
    return fail(FA_ERR_INVALID_ARG, "kv_seqlens is not 4-byte aligned");
  return decode_launch(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Nk, d, scale, kv_seqlens, num_splits, workspace,
                       dtype, stream);
}

int fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B, int Hq,
                      int Hkv, int Nk, int d, float scale, const int32_t* kv_seqlens, int num_splits, int dtype,
                      void* stream) {
  int st = check_decode_args(q, k_cache, v_cache, B, Hq, Hkv, Nk, d, scale, num_splits, dtype);
  if (st != FA_OK) return st;
  if ((long long)B * Hq == 0) return ok();
  if ((st = check_ptr(o, 16, "o")) != FA_OK) return st;
  if ((st = check_ptr(lse, 4, "lse")) != FA_OK) return st;
  if (kv_seqlens != nullptr && !aligned(kv_seqlens, 4))
    return fail(FA_ERR_INVALID_ARG, "kv_seqlens is not 4-byte aligned");
  const size_t need = fa_decode_workspace_bytes(B, Hq, d, num_splits);
  if (need > (size_t)FA_NOALLOC_SCRATCH_BYTES)
    return fail(FA_ERR_WORKSPACE,
                "fa_decode_noalloc: partials of B=%d Hq=%d d=%d num_splits=%d need %zu bytes, more than the "
                "%d-byte static scratch; use fa_decode with a workspace",
                B, Hq, d, num_splits, need, FA_NOALLOC_SCRATCH_BYTES);
  void* scratch = nullptr;
  const hipError_t e = fa::noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "fa_decode_noalloc: static scratch lookup");
  return decode_launch(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Nk, d, scale, kv_seqlens, num_splits, scratch,
                       dtype, stream);
}



int fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table, void* o,
                    float* lse, int B, int Hq, int Hkv, int num_pages, int page_size, int max_pages_per_seq, int d,
                    float scale, const int32_t* kv_seqlens, int num_splits, void* workspace,
                    size_t workspace_bytes, int dtype, void* stream) {
  if (page_size < 1 || max_pages_per_seq < 1 || num_pages < 1)
    return fail(FA_ERR_INVALID_ARG, "page_size, max_pages_per_seq and num_pages must be >= 1 (got %d, %d, %d)",
                page_size, max_pages_per_seq, num_pages);
  if ((long long)page_size * max_pages_per_seq > (1LL << 24))
    return fail(FA_ERR_UNSUPPORTED, "page_size * max_pages_per_seq exceeds 2^24 keys per sequence");
  const int capacity = page_size * max_pages_per_seq;
  int st = check_decode_args(q, k_pages, v_pages, B, Hq, Hkv, capacity, d, scale, num_splits, dtype);
  if (st != FA_OK) return st;
  if (dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "fa_decode_paged supports bf16 only");
  if ((long long)B * Hq == 0) return ok();
  if ((st = check_ptr(block_table, 4, "block_table")) != FA_OK) return st;
  if ((st = check_ptr(kv_seqlens, 4, "kv_seqlens")) != FA_OK) return st;
  if ((st = check_ptr(o, 16, "o")) != FA_OK) return st;
  if ((st = check_ptr(lse, 4, "lse")) != FA_OK) return st;
  const size_t need = fa_decode_workspace_bytes(B, Hq, d, num_splits);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!aligned(workspace, 256)) return fail(FA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  const size_t rows = (size_t)B * Hq;
  float* o_part = (float*)workspace;
  float* lse_part = (float*)((char*)workspace + lse_offset(rows * num_splits * d * sizeof(float)));
  fa::AttnArgs a = make_args(q, k_pages, v_pages, nullptr, nullptr, kv_seqlens, B, Hq, Hkv, 1, capacity, d, scale,
                             0, stream);
  fa::PartialOut part{o_part, lse_part, num_splits};
  fa::PagedKV paged{block_table, page_size, max_pages_per_seq, num_pages};
  hipError_t e = fa::launch_decode_splitkv_bf16(a, part, &paged);
  if (e != hipSuccess) return hip_status(e, "fa_decode_paged split stage launch");
  return hip_status(fa::launch_lse_merge(o_part, lse_part, o, lse, (int)rows, d, num_splits, true,
                                         (hipStream_t)stream),
                    "fa_decode_paged merge stage launch");
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Nq, int d) {
  if (B < 0 || Hq < 0 || Nq < 0 || (d != 64 && d != 128)) return 0;
  return ((size_t)B * Hq * Nq * sizeof(float) + 255) / 256 * 256;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
           const int32_t* kv_seqlens, void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  int st = check_common(B, Hq, Hkv, Nq, Nk, d, scale, dtype);
  if (st != FA_OK) return st;
  if (dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "fa_bwd supports bf16 only");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
  const bool has_q = (long long)B * Hq * Nq > 0, has_k = (long long)B * Hkv * Nk > 0;
  if (!has_q && !has_k) return ok();  // nothing to write
  if (has_q) {
    if ((st = check_ptr(q, 16, "q")) != FA_OK) return st;
    if ((st = check_ptr(o, 16, "o")) != FA_OK) return st;
    if ((st = check_ptr(dout, 16, "dout")) != FA_OK) return st;
    if ((st = check_ptr(lse, 4, "lse")) != FA_OK) return st;
    if ((st = check_ptr(dq, 16, "dq")) != FA_OK) return st;
    const size_t need = fa_bwd_workspace_bytes(B, Hq, Nq, d);
    if (workspace == nullptr || workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    if (!aligned(workspace, 256)) return fail(FA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  }
  if (has_k) {
    if ((st = check_ptr(k, 16, "k")) != FA_OK) return st;
    if ((st = check_ptr(v, 16, "v")) != FA_OK) return st;
    if ((st = check_ptr(dk, 16, "dk")) != FA_OK) return st;
    if ((st = check_ptr(dv, 16, "dv")) != FA_OK) return st;
  }
  if (kv_seqlens != nullptr && !aligned(kv_seqlens, 4))
    return fail(FA_ERR_INVALID_ARG, "kv_seqlens is not 4-byte aligned");
  const long long qtiles = ((long long)Nq + 127) / 128 * B * Hq, ktiles = ((long long)Nk + 127) / 128 * B * Hkv;
  if (qtiles > 0x7fffffffLL || ktiles > 0x7fffffffLL || (long long)B * Hq * Nq > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "problem too large for one launch");
  fa::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.rowdot = (float*)workspace;
  a.kv_seqlens = kv_seqlens;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk; a.d = d;
  a.scale = scale;
  a.causal = causal;
  a.stream = (hipStream_t)stream;
  return hip_status(fa::launch_bwd_bf16(a), "fa_bwd launch");
}

}  // extern "C"
