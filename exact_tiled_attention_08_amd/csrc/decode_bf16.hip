// Split-KV single-token decode (bf16, matrix cores) and the exact LSE merge.
//
// The "FlashAttention" concept note (section "是什么", closing remarks) notes
// that one-token decode is bound by reading the KV cache and needs its own
// kernel and scheduling.  Here each work-group owns one (sequence, KV head,
// key split): it streams that split's keys once and applies them to all the
// query heads that share the KV head (GQA, same section), so every cache byte
// is read exactly once.  The splits' normalised partials (O_s, lse_s) are
// then merged exactly: the same section's online-softmax update with the
// blocks taken to be the splits.
//
// Tile math reuses the prefill conventions (S^T = K Q^T, O^T += V^T P^T on
// 32x32x16 bf16 MFMA): the up to 32 query heads of one KV head form the 32
// query columns, and each of the 4 waves takes its own 32 keys of every
// 128-key tile, keeping a private (m, l, O) that the work-group combines at
// the end.
#include "fa.h"
#include "fa_device.hpp"
#include "fa_launch.hpp"

#include <mutex>

namespace fa {

template <int D>
struct DecTile {
  static constexpr int BN = 128;          // keys per tile (32 per wave)
  static constexpr int THREADS = 256;
  static constexpr int KSTRIDE = D + 8;
  static constexpr int VSTRIDE = D + 32;
  static constexpr int DCH = D / 8;
  static constexpr int CHUNKS = BN * DCH / THREADS;
  static constexpr int STAGE_ELEMS = BN * KSTRIDE + BN * VSTRIDE;  // uint16 elements
};

struct DecParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* o_part;
  float* lse_part;
  const int32_t* kv_seqlens;
  int B, Hq, Hkv, Nk, S;
  int group;      // Hq / Hkv
  int n_qblocks;  // ceil(group / 32)
  float scale_log2;
  // paged cache only: pool [num_pages, Hkv, page_size, D], table [B, max_pages]
  const int32_t* block_table;
  int page_size, max_pages, num_pages;
  float inv_page;  // 1 / page_size
};

// PAGED: key j of sequence b is row j % page_size of page block_table[b][j / page_size]
// (page indices clamped to the pool); otherwise the cache is contiguous BHSD.
// Held to 256 registers so that two work-groups share a CU: twice the loads
// in flight per CU.  The paged cache gains ~30 % from it (its loads wait on
// the block-table reads as well), the contiguous one ~0.5 %.
template <int D, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void decode_splitkv_bf16_kernel(DecParams p) {
  using T = DecTile<D>;
  constexpr int BN = T::BN;
  // Staging area for one K and one V tile; reused for the final combine.
  __shared__ __attribute__((aligned(16))) uint16_t stage[T::STAGE_ELEMS];
  uint16_t* k_lds = stage;
  uint16_t* v_lds = stage + BN * T::KSTRIDE;
  static_assert(4 * 32 * (D + 3) * 4 <= T::STAGE_ELEMS * 2, "combine buffer must fit");

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, hi = lane >> 5;

  const int split = blockIdx.x;
  const int hk = blockIdx.y / p.n_qblocks;
  const int qb = blockIdx.y - hk * p.n_qblocks;
  const int b = blockIdx.z;

  const int kv_len = clamp_len(p.kv_seqlens, b, p.Nk);
  const int chunk = split_chunk(kv_len, p.S, FA_DECODE_SPLIT_ALIGN);
  const int ks = min(split * chunk, kv_len);
  const int ke = min(ks + chunk, kv_len);
  const int n_t = ke > ks ? (ke - ks + BN - 1) / BN : 0;

  const int ncols = min(32, p.group - qb * 32);  // query heads in this block
  const int hq0 = hk * p.group + qb * 32;
  const size_t kv_base = ((size_t)b * p.Hkv + hk) * (size_t)p.Nk;

  bf16x8 qf[D / 16];
  if (li < ncols) {
    const uint16_t* qp = p.q + ((size_t)b * p.Hq + hq0 + li) * D + 8 * hi;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = *(const bf16x8*)(qp + 16 * s);
  } else {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = bf16x8{};
  }

  float m = kNegInf, l = 0.f, lr = 0.f;  // max, weight sum, rounded-weight sum
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};

  uint4 kreg[T::CHUNKS], vreg[T::CHUNKS];
  // Paged cache: the page of each of this thread's rows, fetched two tiles
  // ahead so that the table lookup does not add its latency to the K/V loads.
  // key = page * page_size + rem, from a float reciprocal and a +-1 fix-up
  // (exact for keys < 2^24, which the entry point guarantees).
  int pgr[T::CHUNKS], rem[T::CHUNKS];
  auto fetch_pages = [&](int t) {
#pragma unroll
    for (int c = 0; c < T::CHUNKS; ++c) {
      const int key = ks + t * BN + (tid + c * T::THREADS) / T::DCH;
      int qi = (int)((float)key * p.inv_page);
      int r = key - qi * p.page_size;
      if (r < 0) { --qi; r += p.page_size; }
      if (r >= p.page_size) { ++qi; r -= p.page_size; }
      rem[c] = r;
      pgr[c] = key < ke ? p.block_table[(size_t)b * p.max_pages + qi] : 0;
    }
  };
  auto load_tile = [&](int t) {
#pragma unroll
    for (int c = 0; c < T::CHUNKS; ++c) {
      const int idx = tid + c * T::THREADS;
      const int row = idx / T::DCH, col = idx % T::DCH;
      const int key = ks + t * BN + row;
      if (key < ke) {
        size_t off;
        if (PAGED) {
          const int pg = min(max(pgr[c], 0), p.num_pages - 1);
          off = (((size_t)pg * p.Hkv + hk) * p.page_size + rem[c]) * D + col * 8;
        } else {
          off = (kv_base + key) * D + col * 8;
        }
        // The cache is streamed once: nontemporal loads (measured: a plain
        // streaming read of 8 GiB reaches ~6.2 TB/s, a nontemporal one ~7 TB/s).
        kreg[c] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)(p.k + off)));
        vreg[c] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)(p.v + off)));
      } else {
        kreg[c] = uint4{0, 0, 0, 0};
        vreg[c] = uint4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int c = 0; c < T::CHUNKS; ++c) {
      const int idx = tid + c * T::THREADS;
      const int row = idx / T::DCH, col = idx % T::DCH;
      *(uint4*)(k_lds + row * T::KSTRIDE + col * 8) = kreg[c];
      *(uint4*)(v_lds + row * T::VSTRIDE + col * 8) = vreg[c];
    }
  };

  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int kb = wave;  // this wave's 32-key block of every tile

  if (n_t > 0) {
    if (PAGED) fetch_pages(0);
    load_tile(0);
    if (PAGED && n_t > 1) fetch_pages(1);
  }
  for (int t = 0; t < n_t; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < n_t) {
      load_tile(t + 1);
      if (PAGED && t + 2 < n_t) fetch_pages(t + 2);
    }

    f32x16 s = f32x16{};
    const uint16_t* kp = k_lds + (kb * 32 + li) * T::KSTRIDE + 8 * hi;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) s = mfma32x32x16(*(const bf16x8*)(kp + 16 * st), qf[st], s);

    const int key0 = ks + t * BN + kb * 32;
    if (key0 + 32 > ke) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key0 + 8 * (r >> 2) + 4 * hi + (r & 3) >= ke) s[r] = kNegInf;
    }

    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, wave_xor32(mx));
    const float m_new = fmaxf(m, mx * p.scale_log2);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = fast_exp2(__builtin_fmaf(s[r], p.scale_log2, -m_use));
      rs += s[r];
    }
    l = l * alpha + rs;
    lr *= alpha;
    m = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

    bf16x8 pf[2];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      float tmp[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) tmp[e] = s[8 * mm + e];
      pf[mm] = pack_bf16x8_sum(tmp, lr);
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const uint16_t* vp = v_lds + (kb * 32 + 16 * mm + tr_row) * T::VSTRIDE + db * 32 + tr_col;
        const bf16x8 a = join_bf16x8(lds_read_tr16(vp), lds_read_tr16(vp + 8 * T::VSTRIDE));
        oacc[db] = mfma32x32x16(a, pf[mm], oacc[db]);
      }
  }

  // Combine the 4 waves' states (disjoint key sets) exactly, then write the
  // split's normalised partial.
  __syncthreads();
  float* red = (float*)stage;                 // [4 waves][32 cols][D + 3]
  constexpr int RS = D + 3;
  const float lt = l + wave_xor32(l);
  const float lrt = lr + wave_xor32(lr);
  float* my = red + (wave * 32 + li) * RS;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) my[db * 32 + 8 * (r >> 2) + 4 * hi + (r & 3)] = oacc[db][r];
  if (hi == 0) {
    my[D] = m;
    my[D + 1] = lt;
    my[D + 2] = lrt;
  }
  __syncthreads();
  for (int e = tid; e < ncols * D; e += T::THREADS) {
    const int col = e / D, dd = e - col * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red[(w * 32 + col) * RS + D]);
    const float M_use = (M == kNegInf) ? 0.f : M;
    float acc = 0.f, tot = 0.f, totr = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* rw = red + (w * 32 + col) * RS;
      const float sc = fast_exp2(rw[D] - M_use);
      acc += sc * rw[dd];
      tot += sc * rw[D + 1];
      totr += sc * rw[D + 2];
    }
    const size_t row = ((size_t)b * p.Hq + hq0 + col) * p.S + split;
    p.o_part[row * D + dd] = tot > 0.f ? acc / totr : 0.f;
    if (dd == 0) p.lse_part[row] = tot > 0.f ? (M + __log2f(tot)) * kLn2 : kNegInf;
  }
}

template <int D>
static hipError_t launch_decode_t(const AttnArgs& a, const PartialOut& part, const PagedKV* paged) {
  DecParams p;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k;
  p.v = (const uint16_t*)a.v;
  p.o_part = part.o_part;
  p.lse_part = part.lse_part;
  p.kv_seqlens = a.kv_seqlens;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nk = a.Nk; p.S = part.num_splits;
  p.group = a.Hq / a.Hkv;
  p.n_qblocks = (p.group + 31) / 32;
  p.scale_log2 = a.scale * kLog2e;
  p.block_table = paged ? paged->block_table : nullptr;
  p.page_size = paged ? paged->page_size : 0;
  p.max_pages = paged ? paged->max_pages : 0;
  p.num_pages = paged ? paged->num_pages : 0;
  p.inv_page = paged ? 1.0f / (float)paged->page_size : 0.f;
  const long long gy = (long long)a.Hkv * p.n_qblocks;
  if (gy > 65535 || a.B > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid(part.num_splits, (unsigned)gy, a.B);
  if (paged)
    hipLaunchKernelGGL((decode_splitkv_bf16_kernel<D, true>), grid, dim3(256), 0, a.stream, p);
  else
    hipLaunchKernelGGL((decode_splitkv_bf16_kernel<D, false>), grid, dim3(256), 0, a.stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_splitkv_bf16(const AttnArgs& a, const PartialOut& part, const PagedKV* paged) {
  return a.d == 128 ? launch_decode_t<128>(a, part, paged) : launch_decode_t<64>(a, part, paged);
}

// ---------------------------------------------------------------------------
// Exact merge: per row, M = max_s lse_s, w_s = e^(lse_s - M),
// O = sum_s w_s O_s / sum_s w_s, LSE = M + ln sum_s w_s.
// One wave per row, four rows per work-group: the wave reads the row's S LSEs
// once (lane s, s + 64, ...), reduces M and sum_s w_s across lanes, keeps the
// weights in LDS, and then streams the S partial rows with every lane owning
// D / 64 adjacent outputs (one 8-byte load per split for D = 128).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void lse_merge_kernel(const float* __restrict__ o_part,
                                                       const float* __restrict__ lse_part, void* o, float* lse,
                                                       int S, int rows) {
  constexpr int E = D / 64;  // outputs per lane
  __shared__ float wsh[4][FA_MAX_SPLITS];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row_i = blockIdx.x * 4 + wave;
  const bool live = row_i < rows;
  const size_t row = live ? (size_t)row_i : 0;
  const float* lp = lse_part + row * S;
  float M = kNegInf;
  if (live)
    for (int s = lane; s < S; s += 64) M = fmaxf(M, lp[s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  const float M_use = (M == kNegInf) ? 0.f : M;
  float tot = 0.f;
  if (live)
    for (int s = lane; s < S; s += 64) {
      const float w = fast_exp2((lp[s] - M_use) * kLog2e);
      wsh[wave][s] = w;
      tot += w;
    }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 64);
  __syncthreads();
  if (!live) return;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  const float* op = o_part + row * S * D + lane * E;
#pragma unroll 4
  for (int s = 0; s < S; ++s) {
    const float w = wsh[wave][s];
    if constexpr (E == 2) {
      const float2 x = *(const float2*)(op + (size_t)s * D);
      acc[0] += w * x.x;
      acc[1] += w * x.y;
    } else {
      acc[0] += w * op[(size_t)s * D];
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  if constexpr (BF16) {
    __bf16* ob = (__bf16*)o + row * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) ob[e] = (__bf16)(acc[e] * inv);
  } else {
    float* of = (float*)o + row * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) of[e] = acc[e] * inv;
  }
  if (lane == 0) lse[row] = tot > 0.f ? M_use + __log2f(tot) * kLn2 : kNegInf;
}

hipError_t launch_lse_merge(const float* o_part, const float* lse_part, void* o, float* lse, int rows,
                            int d, int num_splits, bool out_bf16, hipStream_t stream) {
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (d == 128) {
    if (out_bf16)
      hipLaunchKernelGGL((lse_merge_kernel<128, true>), grid, block, 0, stream, o_part, lse_part, o, lse,
                         num_splits, rows);
    else
      hipLaunchKernelGGL((lse_merge_kernel<128, false>), grid, block, 0, stream, o_part, lse_part, o, lse,
                         num_splits, rows);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((lse_merge_kernel<64, true>), grid, block, 0, stream, o_part, lse_part, o, lse,
                         num_splits, rows);
    else
      hipLaunchKernelGGL((lse_merge_kernel<64, false>), grid, block, 0, stream, o_part, lse_part, o, lse,
                         num_splits, rows);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode scratch for callers that cannot allocate (fa_decode_noalloc): the
// split partials live in this file-scope device array instead of a caller
// workspace.  Each GPU holds its own copy for the life of the process.  Host
// code never uses the array's name as an address: its device address is
// looked up once per device (with that device current) and cached.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace fa
