// bf16 prefill forward of exact attention on gfx950 matrix cores.
//
// Method: the tiled forward with online softmax of the "FlashAttention"
// concept note, section "是什么" -- a block of query rows stays on chip, K/V
// blocks stream past it, and a per-row running max m and sum l rescale the
// partial output so the final O equals softmax(scale Q K^T) V.  Masks and the
// GQA head mapping are applied inside the tile, as the same section says;
// tiles that lie wholly above the causal diagonal or beyond a sequence's
// valid length are never loaded.  The FA2 idea of spreading one head over
// many work-groups (one per query block) is the grid; the saiita.com.cn
// explainer, section "二代和三代", credits it for the utilisation gain.
//
// Work-group: 4 waves x 32 query rows = 128 rows.  Each KV tile holds 64
// keys.  Everything per query row lives in one lane pair (lanes i and i+32):
//   S^T = K Q^T      A = K rows from LDS, B = Q^T kept in VGPRs
//   O^T += V^T P^T   A = V^T via ds_read_b64_tr_b16, B = P^T straight from
//                    the S^T accumulators (rounded to bf16)
// so the row max/sum need one cross-half exchange and the rescale of O by
// alpha = 2^(m_old - m_new) is lane-local.  Exponentials run in base 2 with
// scale*log2(e) folded into one FMA.
//
// K/V tiles move HBM -> LDS with direct global_load_lds_dwordx4 copies (no
// VGPR staging) into two LDS buffers: tile t+1 streams in while tile t is
// being consumed, with one barrier per tile.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

template <int D>
struct FwdTile {
  static constexpr int BM = 128;                    // query rows per work-group
  static constexpr int BN = 64;                     // keys per KV tile
  static constexpr int THREADS = 256;               // 4 waves
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;              // rows per wave-wide 1 KiB copy
  static constexpr int TILE = BN * D;               // elements per K (or V) tile
  static constexpr int COPIES = BN / RPI / 4;       // 1 KiB copies per wave per tile per tensor
  static_assert(BN % (4 * RPI) == 0, "tile rows must split evenly over the waves");
};

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* kv_seqlens;
  int B, Hq, Hkv, Nq, Nk;
  int n_qtiles;
  float scale_log2;  // scale * log2(e)
};

template <int D, bool CAUSAL, bool PADDED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void fwd_bf16_kernel(FwdParams p) {
  using T = FwdTile<D>;
  constexpr int BM = T::BM, BN = T::BN;
  // [buffer][K | V][BN rows x D], rows swizzled in 16-byte chunks (swz<D>).
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2][2][T::TILE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, hi = lane >> 5;

  // Work-group -> (query tile, head, batch).  The last (heaviest, under a
  // causal mask) query tiles of every head are dispatched first.
  const int bh_count = p.B * p.Hq;
  const int bh = blockIdx.x % bh_count;
  const int qt = p.n_qtiles - 1 - (int)(blockIdx.x / bh_count);
  const int b = bh / p.Hq, hq = bh - b * p.Hq;
  const int hk = hq / (p.Hq / p.Hkv);

  const int kv_len = PADDED ? clamp_len(p.kv_seqlens, b, p.Nk) : p.Nk;
  const int q0 = qt * BM;
  const int diag = p.Nk - p.Nq;  // key j visible to row i iff j <= i + diag
  int kend = kv_len;
  if (CAUSAL) {
    const int q_last = min(q0 + BM, p.Nq) - 1;
    kend = min(kend, q_last + diag + 1);
  }
  const int n_kt = kend > 0 ? (kend + BN - 1) / BN : 0;

  const size_t q_base = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;
  const size_t kv_base = ((size_t)b * p.Hkv + hk) * (size_t)p.Nk;
  const uint16_t* kg = p.k + kv_base * D;
  const uint16_t* vg = p.v + kv_base * D;

  // Q^T fragment: lane (li, hi) holds row q0 + 32*wave + li, columns
  // 16*s + 8*hi .. +7 for each k-step s.
  const int qrow = q0 + wave * 32 + li;
  bf16x8 qf[D / 16];
  if (qrow < p.Nq) {
    const uint16_t* qp = p.q + (q_base + qrow) * D + 8 * hi;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = *(const bf16x8*)(qp + 16 * s);
  } else {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = bf16x8{};
  }

  float m = kNegInf;  // reference (running) max of scaled scores, base-2 units
  float l = 0.f;      // sum of the weights over this lane's half of each tile
  float lr = 0.f;     // the same sum over the bf16-rounded weights P.V uses
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};

  // Copy plan: wave w fills rows [w*COPIES*RPI, (w+1)*COPIES*RPI) of each
  // tile; in copy i, lane l brings row r = (w*COPIES + i)*RPI + l/CPR, source
  // chunk (l % CPR) ^ swz(r), to LDS position l % CPR of that row.
  int src_row[T::COPIES], src_col[T::COPIES];
#pragma unroll
  for (int i = 0; i < T::COPIES; ++i) {
    const int r = (wave * T::COPIES + i) * T::RPI + lane / T::CPR;
    src_row[i] = r;
    src_col[i] = ((lane % T::CPR) ^ swz<D>(r)) * 8;
  }
  auto issue_tile = [&](int kt, int buf) {
    const int k0 = kt * BN;
    const bool tail = k0 + BN > kv_len;  // rows past the length re-read the last valid row
#pragma unroll
    for (int i = 0; i < T::COPIES; ++i) {
      int row = k0 + src_row[i];
      if (tail) row = min(row, kv_len - 1);
      const size_t off = (size_t)row * D + src_col[i];
      load_lds_16B(kg + off, &lds[buf][0][(wave * T::COPIES + i) * 512]);
      load_lds_16B(vg + off, &lds[buf][1][(wave * T::COPIES + i) * 512]);
    }
  };

  // Per-lane LDS offsets (elements) of the fragment reads.
  //  K: row kb*32 + li, chunk 2*st + hi.
  int k_off[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) k_off[st] = li * D + (((2 * st + hi) ^ swz<D>(li)) * 8);
  //  V (transposed 4x16 reads): row kb*32 + 16*mm + 8*u + 4*hi + (lane&15)/4,
  //  column db*32 + 16*((lane>>4)&1) + 4*(lane&3).
  const int tr_r = 4 * hi + ((lane & 15) >> 2);
  const int tr_cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // chunk within the 32-column block
  const int tr_in = 4 * (lane & 1);                               // element within the chunk
  int v_off[D / 32][2];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = 8 * u + tr_r;
      v_off[db][u] = r * D + (((4 * db + tr_cc) ^ swz<D>(r)) * 8) + tr_in;
    }

  if (n_kt > 0) issue_tile(0, 0);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile kt is in LDS; every wave is done with tile kt-1
    if (kt + 1 < n_kt) issue_tile(kt + 1, buf ^ 1);

    const uint16_t* kl = lds[buf][0];
    const uint16_t* vl = lds[buf][1];

    // S^T[key][query] = K Q^T for the 64 keys of the tile, two 32-key blocks.
    f32x16 s[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
        s[kb] = mfma32x32x16(*(const bf16x8*)(kl + kb * 32 * D + k_off[st]), qf[st], s[kb]);
    }

    // Masks, only on tiles that cross the causal diagonal or the valid length.
    const int k0 = kt * BN;
    const bool need_mask = (k0 + BN > kv_len) || (CAUSAL && k0 + BN - 1 > q0 + diag);
    if (need_mask) {
      const int lim = CAUSAL ? min(kv_len, qrow + diag + 1) : kv_len;  // keys < lim visible
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= lim) s[kb][r] = kNegInf;
        }
    }

    // Online softmax update of (m, l, O) for this lane's query row.  The
    // reference max m only moves when the tile max exceeds it by more than
    // kRescaleSlack (base-2 units): every exponent stays <= kRescaleSlack, the
    // result is unchanged (l and O share the same reference), and the O
    // rescale -- the costliest VALU step -- is skipped on most tiles.
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, wave_xor32(mx)) * p.scale_log2;
    if (__any(mx > m + kRescaleSlack)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - ((m_new == kNegInf) ? 0.f : m_new));
      m = m_new;
      l *= alpha;
      lr *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const float m_use = (m == kNegInf) ? 0.f : m;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], p.scale_log2, -m_use));
        rs += s[kb][r];
      }
    l += rs;

    // P^T fragments (registers 8*mm .. 8*mm+7 of key block kb), rounded to
    // bf16; lr accumulates the rounded weights so that O / lr is a properly
    // normalised average, while the LSE uses the unrounded sum l.
    bf16x8 pf[BN / 16];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        float t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = s[kb][8 * mm + e];
        pf[kb * 2 + mm] = pack_bf16x8_sum(t, lr);
      }

    // O^T[d][query] += V^T P^T.  Element t of either operand pairs with key
    // kb*32 + 16*mm + 8*(t/4) + 4*hi + t%4.
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const uint16_t* vp = vl + (kb * 32 + 16 * mm) * D;
          const bf16x8 a = join_bf16x8(lds_read_tr16(vp + v_off[db][0]), lds_read_tr16(vp + v_off[db][1]));
          oacc[db] = mfma32x32x16(a, pf[kb * 2 + mm], oacc[db]);
        }
  }

  // Epilogue: O = O_acc / lr, LSE = ln2 * (m + log2 l).  Only O and LSE are
  // ever written to memory.
  const float lt = l + wave_xor32(l);
  const float lrt = lr + wave_xor32(lr);
  if (qrow < p.Nq) {
    const float inv = lt > 0.f ? 1.f / lrt : 0.f;
    uint16_t* op = p.o + (q_base + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
        w.y = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *(uint2*)(op + db * 32 + 8 * g + 4 * hi) = w;
      }
    if (hi == 0) p.lse[q_base + qrow] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : kNegInf;
  }
}

template <int D, bool CAUSAL, bool PADDED>
static hipError_t launch_fwd_bf16_t(const AttnArgs& a) {
  using T = FwdTile<D>;
  FwdParams p;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k;
  p.v = (const uint16_t*)a.v;
  p.o = (uint16_t*)a.o;
  p.lse = a.lse;
  p.kv_seqlens = a.kv_seqlens;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk;
  p.n_qtiles = (a.Nq + T::BM - 1) / T::BM;
  p.scale_log2 = a.scale * kLog2e;
  const long long grid = (long long)p.n_qtiles * a.B * a.Hq;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, PADDED>), dim3((unsigned)grid), dim3(T::THREADS), 0,
                     a.stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const AttnArgs& a) {
  const bool padded = a.kv_seqlens != nullptr;
  if (a.d == 128) {
    if (a.causal) return padded ? launch_fwd_bf16_t<128, true, true>(a) : launch_fwd_bf16_t<128, true, false>(a);
    return padded ? launch_fwd_bf16_t<128, false, true>(a) : launch_fwd_bf16_t<128, false, false>(a);
  }
  if (a.causal) return padded ? launch_fwd_bf16_t<64, true, true>(a) : launch_fwd_bf16_t<64, true, false>(a);
  return padded ? launch_fwd_bf16_t<64, false, true>(a) : launch_fwd_bf16_t<64, false, false>(a);
}

}  // namespace fa
