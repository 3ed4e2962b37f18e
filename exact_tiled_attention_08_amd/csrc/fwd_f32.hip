// float32 forward of exact attention (vector ALU, no reduced precision).
//
// The same blocked online-softmax update as the bf16 kernel (the
// "FlashAttention" concept note, section "是什么"), computed in float32 end to
// end: each thread owns one query row (its q, running max m, running sum l
// and output accumulator stay in registers) and K/V tiles of 32 keys are
// staged in LDS and read by every thread of the work-group.  With a partial
// output it computes split-KV partials for single-token decode instead.
#include "fa.h"
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  float* o_part;
  float* lse_part;
  const int32_t* kv_seqlens;
  const int32_t* cu_q;  // packed variable-length layout when non-null
  const int32_t* cu_k;
  int total_q, total_k;
  int B, Hq, Hkv, Nq, Nk;
  int n_qtiles;
  int S;  // number of splits; 0 = final output
  int causal;
  float scale;
};

template <int D>
__global__ __launch_bounds__(128) void fwd_f32_kernel(F32Params p) {
  constexpr int BQ = 128, BN = 32;
  __shared__ __attribute__((aligned(16))) float k_lds[BN * D];
  __shared__ __attribute__((aligned(16))) float v_lds[BN * D];

  const int tid = threadIdx.x;
  const int nsp = p.S > 0 ? p.S : 1;
  size_t w = blockIdx.x;
  const int qt = (int)(w % p.n_qtiles); w /= p.n_qtiles;
  const int hq = (int)(w % p.Hq); w /= p.Hq;
  const int split = (int)(w % nsp);
  const int b = (int)(w / nsp);
  const int hk = hq / (p.Hq / p.Hkv);

  // Rows of this sequence: dense / padded [B, H, N, d], or packed
  // [H, total, d] with sequence b at rows cu[b] .. cu[b+1]-1.
  int nq = p.Nq, nk = p.Nk, kv_len;
  size_t q_row0, kv_base;
  if (p.cu_q != nullptr) {
    const int2 qr = packed_rows(p.cu_q, b, p.total_q), kr = packed_rows(p.cu_k, b, p.total_k);
    nq = qr.y;
    nk = kv_len = kr.y;
    q_row0 = (size_t)hq * p.total_q + qr.x;
    kv_base = (size_t)hk * p.total_k + kr.x;
  } else {
    kv_len = clamp_len(p.kv_seqlens, b, p.Nk);
    q_row0 = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;
    kv_base = ((size_t)b * p.Hkv + hk) * (size_t)p.Nk;
  }
  int ks = 0, ke = kv_len;
  if (p.S > 0) {
    const int chunk = split_chunk(kv_len, p.S, FA_DECODE_SPLIT_ALIGN);
    ks = min(split * chunk, kv_len);
    ke = min(ks + chunk, kv_len);
  }
  const int diag = nk - nq;
  const int q0 = qt * BQ;
  if (q0 >= nq) return;  // a packed sequence shorter than the longest one
  int kend = ke;
  if (p.causal) kend = min(kend, min(q0 + BQ, nq) - 1 + diag + 1);

  const int qrow = q0 + tid;
  const size_t qo = q_row0 + qrow;
  float q[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qrow < nq ? p.q[qo * D + d] : 0.f;
    o[d] = 0.f;
  }
  const int lim = p.causal ? min(ke, qrow + diag + 1) : ke;  // visible keys: [ks, lim)
  float m = kNegInf, l = 0.f;

  for (int t0 = ks; t0 < kend; t0 += BN) {
    __syncthreads();
    for (int e = tid * 4; e < BN * D; e += BQ * 4) {
      const int row = e / D, col = e - row * D;
      float4 kk = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (t0 + row < kend) {
        kk = *(const float4*)(p.k + (kv_base + t0 + row) * D + col);
        vv = *(const float4*)(p.v + (kv_base + t0 + row) * D + col);
      }
      *(float4*)(k_lds + e) = kk;
      *(float4*)(v_lds + e) = vv;
    }
    __syncthreads();

    float s[BN];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(q[d], k_lds[j * D + d], acc);
      s[j] = (t0 + j < lim) ? acc * p.scale : kNegInf;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = expf(m - m_use);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      const float pj = expf(s[j] - m_use);
      l += pj;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(pj, v_lds[j * D + d], o[d]);
    }
    m = m_new;
  }

  if (qrow >= nq) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse = l > 0.f ? m + logf(l) : kNegInf;
  if (p.S > 0) {
    const size_t row = (((size_t)b * p.Hq + hq) * p.S + split);
#pragma unroll
    for (int d = 0; d < D; ++d) p.o_part[row * D + d] = o[d] * inv;
    p.lse_part[row] = lse;
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d) p.o[qo * D + d] = o[d] * inv;
    p.lse[qo] = lse;
  }
}

hipError_t launch_fwd_f32(const AttnArgs& a, const PartialOut* part) {
  F32Params p;
  p.q = (const float*)a.q;
  p.k = (const float*)a.k;
  p.v = (const float*)a.v;
  p.o = (float*)a.o;
  p.lse = a.lse;
  p.o_part = part ? part->o_part : nullptr;
  p.lse_part = part ? part->lse_part : nullptr;
  p.kv_seqlens = a.kv_seqlens;
  p.cu_q = a.cu_q;
  p.cu_k = a.cu_k;
  p.total_q = a.total_q;
  p.total_k = a.total_k;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk;
  p.n_qtiles = (a.Nq + 127) / 128;
  p.S = part ? part->num_splits : 0;
  p.causal = a.causal;
  p.scale = a.scale;
  const long long grid = (long long)p.n_qtiles * a.Hq * a.B * (p.S > 0 ? p.S : 1);
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.d == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3((unsigned)grid), dim3(128), 0, a.stream, p);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3((unsigned)grid), dim3(128), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace fa
