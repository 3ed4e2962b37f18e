// FP8 prefill forward of exact attention on gfx950 (d = 128).
//
// Inputs are 8-bit floating-point codes (OCP E4M3 or E5M2) with one float32
// descale per tensor, so the real inputs are descale * value(code).  The
// attention computed is the definition of the "FlashAttention" concept note,
// section "是什么", by the same blocked online-softmax update as the bf16
// kernel; the 2026 explainer ("二代和三代") credits FP8 matrix units for
// FlashAttention-3's throughput, which is the reason for this path.
//
// What changes against the bf16 ping-pong kernel (fwd_bf16.hip):
//   * S^T = K Q^T runs on the FP8 matrix cores (v_mfma_f32_32x32x64_f8f6f4)
//     and accumulates in float32 registers; the two descales fold into the
//     softmax scale.  Inside one instruction the 64 products are summed at
//     less than float32 precision (measured on MI355X: errors up to ~2^-15 of
//     the sum of |products|), which bounds the score error by that fraction of
//     scale * sum_d |q_d k_d|.
//   * K tiles stay FP8 in LDS (8 KiB per 64 keys, half the bytes).
//   * V is converted exactly to bf16 while it is staged, in the matrix phase
//     (every E4M3 and E5M2 value is a bf16 value), and O^T += V^T P^T stays
//     on the bf16 matrix cores with P rounded to bf16, exactly as in the bf16
//     kernel; v's descale multiplies O once at the end.  P itself is never
//     quantised to FP8, so the only rounding that FP8 adds is the caller's
//     own.
// Everything else -- grid, heaviest-first order, two 4-wave groups one phase
// apart, three rotating buffers, masks, lazy rescale, epilogue -- is the
// bf16 kernel's.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

struct Fp8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* kv_seqlens;
  int B, Hq, Hkv, Nq, Nk;
  int n_qtiles;
  float scale_log2;  // scale * q_descale * k_descale * log2(e)
  float v_descale;
};

struct Fp8Tile {
  static constexpr int D = 128, BM = 256, BN = 64, WAVES = 8, THREADS = 512;
  static constexpr int KTILE = BN * D;   // bytes of an FP8 K tile (8 KiB)
  static constexpr int VTILE = BN * D;   // bf16 elements of a converted V tile (16 KiB)
  static constexpr int V_BASE = 3 * KTILE;  // byte offset of the V buffers in LDS
};

// XOR swizzle of the 16-byte chunks of a 128-byte FP8 K row: chunk c of row r
// sits at position c ^ swz_k8(r).  A fragment read touches one chunk of 16
// consecutive rows per 16 lanes; (r % 2, c ^ swz_k8(r)) then covers all 16
// bank groups of a 256-byte LDS line exactly once.
__device__ __forceinline__ int swz_k8(int r) { return (r >> 1) & 7; }

// Swizzle of the converted bf16 V tiles: the bf16 kernel's swz_v128 (which
// keeps the transposed fragment reads conflict-free) plus a swap of the two
// chunks of each pair in odd rows.  The staging writes store chunk pairs
// (2j, 2j+1) of two adjacent rows in one instruction; with the swap the two
// rows' first chunks fall in different bank halves.  Reads are unaffected:
// the swap stays inside each aligned group of four chunks they touch.
__device__ __forceinline__ int swz_v8(int r) { return 4 * (r & 3) + (r & 1); }

template <int FMT>
__device__ __forceinline__ f32x16 mfma32x32x64_f8(i32x8 a, i32x8 b, f32x16 c) {
  // FMT selects the operand format of both A and B: 0 = E4M3, 1 = E5M2.
  // With zero scale operands the compiler emits the unscaled instruction.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, 0, 0, 0, 0);
}

// Two FP8 codes (byte pair `HI` of w) -> two bf16 values, exactly.
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  if constexpr (FMT == 0) return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  else return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI));
}

template <int FMT, bool CAUSAL, bool PADDED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_fp8_pp_kernel(Fp8Params p) {
  using T = Fp8Tile;
  constexpr int D = T::D, BM = T::BM, BN = T::BN;
  // K buffers 0..2 (FP8, bytes [0, 24 KiB)), V buffers 0..2 (bf16, after them);
  // tile t lives in buffer t % 3.
  __shared__ __attribute__((aligned(1024))) uint8_t lds[T::V_BASE + 3 * T::VTILE * 2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, hi = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool lead = wave_u < 4;  // group 0 leads, group 1 lags one phase

  const int bh_count = p.B * p.Hq;
  const int bh = xcd_grouped_head((int)(blockIdx.x % bh_count), p.B, p.Hq, p.Hkv);
  const int qt = p.n_qtiles - 1 - (int)(blockIdx.x / bh_count);
  const int b = bh / p.Hq, hq = bh - b * p.Hq;
  const int hk = hq / (p.Hq / p.Hkv);

  const int kv_len = PADDED ? clamp_len(p.kv_seqlens, b, p.Nk) : p.Nk;
  const int q0 = qt * BM;
  const int diag = p.Nk - p.Nq;
  int kend = kv_len;
  if (CAUSAL) kend = min(kend, min(q0 + BM, p.Nq) - 1 + diag + 1);
  const int n_kt = kend > 0 ? (kend + BN - 1) / BN : 0;
  const int w_first = q0 + wave_u * 32;
  int w_kend = kv_len;
  if (CAUSAL) w_kend = min(w_kend, min(w_first + 32, p.Nq) - 1 + diag + 1);
  const int w_nkt = w_kend > 0 ? (w_kend + BN - 1) / BN : 0;

  const size_t q_base = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;
  const size_t kv_base = ((size_t)b * p.Hkv + hk) * (size_t)p.Nk;
  const uint8_t* kg = p.k + kv_base * D;
  const uint8_t* vg = p.v + kv_base * D;

  // Q^T fragments (B operand): lane (li, hi) holds query row w_first + li,
  // bytes 64*s + 32*hi .. +31 for k-step s.  The K fragments (A operand) take
  // the same bytes of their key rows, so the k labelling of the two operands
  // agrees whatever order the instruction sums in.
  const int qrow = w_first + li;
  i32x8 qf[2];
  if (qrow < p.Nq) {
    const uint8_t* qp = p.q + (q_base + qrow) * D + 32 * hi;
    qf[0] = *(const i32x8*)(qp);
    qf[1] = *(const i32x8*)(qp + 64);
  } else {
    qf[0] = i32x8{};
    qf[1] = i32x8{};
  }
  // Retire the Q loads before the loop (see the bf16 kernel).
  asm volatile("" : "+v"(qf[0]));
  asm volatile("" : "+v"(qf[1]));

  float m = kNegInf, l = 0.f, lr = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  f32x16 s[BN / 32];
  bf16x8 pf[BN / 16];
#pragma unroll
  for (int kb = 0; kb < BN / 32; ++kb) s[kb] = f32x16{};
#pragma unroll
  for (int i = 0; i < BN / 16; ++i) pf[i] = bf16x8{};

  // K copy plan: wave w moves rows 8w .. 8w+7 of each K tile (1 KiB, one
  // global_load_lds_dwordx4); lane i brings row 8w + i/8, source chunk
  // (i % 8) ^ swz_k8(row), to LDS position i % 8 of that row.  Tiles past the
  // last one are clamped to it (the copy lands in a buffer no phase reads).
  // The lane offsets are the same for every full tile (computed once); only
  // the last tile of a sequence, where rows past the length re-read the last
  // valid row, adjusts them.
  const int st_row = wave_u * 8 + (lane >> 3);
  const int st_chunk = lane & 7;
  int k_cp = st_row * D + ((st_chunk ^ swz_k8(st_row)) << 4);
  int v_ld = st_row * D + st_chunk * 16;
  asm volatile("" : "+v"(k_cp), "+v"(v_ld));
  // rows by which a lane's row moves back in the last tile (0 elsewhere)
  auto tail_shift = [&](int k0) { return (k0 + BN > kv_len) ? max(0, k0 + st_row - (kv_len - 1)) : 0; };
  auto copy_k = [&](int t, int buf) {
    t = min(t, n_kt - 1);
    const int k0 = t * BN;
    int voff = k_cp;
    if (k0 + BN > kv_len) voff -= tail_shift(k0) * D;
    copy16_to_lds(kg + (size_t)k0 * D, voff, lds + buf * T::KTILE + wave_u * 1024);
  };
  // V staging: thread (w, i) loads 16 codes of row 8w + i/8 (columns
  // 16*(i%8) .. +15), converts them to bf16 and writes the two 16-byte
  // chunks 2*(i%8), 2*(i%8)+1 of the bf16 row (swizzled by swz_v8).
  uint4 vstage;
  auto load_v = [&](int t) {
    t = min(t, n_kt - 1);
    const int k0 = t * BN;
    int off = v_ld;
    if (k0 + BN > kv_len) off -= tail_shift(k0) * D;
    vstage = *(const uint4*)(vg + (size_t)k0 * D + off);
  };
  auto store_v = [&](int buf) {
    uint4 lo, hi4;
    lo.x = fp8x2_to_bf16x2<FMT, false>(vstage.x);
    lo.y = fp8x2_to_bf16x2<FMT, true>(vstage.x);
    lo.z = fp8x2_to_bf16x2<FMT, false>(vstage.y);
    lo.w = fp8x2_to_bf16x2<FMT, true>(vstage.y);
    hi4.x = fp8x2_to_bf16x2<FMT, false>(vstage.z);
    hi4.y = fp8x2_to_bf16x2<FMT, true>(vstage.z);
    hi4.z = fp8x2_to_bf16x2<FMT, false>(vstage.w);
    hi4.w = fp8x2_to_bf16x2<FMT, true>(vstage.w);
    const int pos = (2 * st_chunk) ^ swz_v8(st_row);  // chunk 2j; chunk 2j+1 sits at pos ^ 1
    uint16_t* vrow = (uint16_t*)(lds + T::V_BASE) + buf * T::VTILE + st_row * D;
    *(uint4*)(vrow + pos * 8) = lo;
    *(uint4*)(vrow + (pos ^ 1) * 8) = hi4;
  };

  // Per-lane fragment offsets.  K (bytes): row kb*32 + li, chunks 4s + 2hi
  // and 4s + 2hi + 1.  V (bf16 elements): as in the bf16 kernel.
  int k_off[2][2];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int c = 0; c < 2; ++c) k_off[st][c] = li * D + (((4 * st + 2 * hi + c) ^ swz_k8(li)) << 4);
  const int tr_r = 4 * hi + ((lane & 15) >> 2);
  const int tr_cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_in = 4 * (lane & 1);
  int v_off[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
    v_off[db] = tr_r * D + (((4 * db + tr_cc) ^ swz_v8(tr_r)) * 8) + tr_in;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int c = 0; c < 2; ++c) asm volatile("" : "+v"(k_off[st][c]));
#pragma unroll
  for (int db = 0; db < D / 32; ++db) asm volatile("" : "+v"(v_off[db]));
  const uint8_t* kl0 = lds;
  const uint16_t* vl0 = (const uint16_t*)(lds + T::V_BASE);
  int ka[2][2], va[D / 32];

  // Fragment groups, consecutive MFMAs always on different accumulators:
  //   P.V group i (0..3): key slice i (16 keys) for the four d-blocks (bf16)
  //   S group 4 + st:     k-step st (64 bytes of d) for both key blocks (FP8)
  // Fragments are held as raw 16-byte words: a V fragment is one word, a K
  // fragment two.
  auto load_group = [&](int g, uint4* f) {
    if (g < 4) {
      const int c = ((g >> 1) * 32 + 16 * (g & 1)) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        f[db] = __builtin_bit_cast(uint4, join_bf16x8(lds_read_tr16(vl0 + va[db] + c),
                                                      lds_read_tr16(vl0 + va[db] + c + 8 * D)));
    } else {
      const int st = g - 4;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c) f[2 * kb + c] = *(const uint4*)(kl0 + ka[st][c] + kb * 32 * D);
    }
  };
  auto mfma_group = [&](int g, const uint4* f) {
    if (g < 4) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        oacc[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, f[db]), pf[g], oacc[db]);
    } else {
      const int st = g - 4;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const i32x8 a = {(int)f[2 * kb].x,     (int)f[2 * kb].y,     (int)f[2 * kb].z,     (int)f[2 * kb].w,
                         (int)f[2 * kb + 1].x, (int)f[2 * kb + 1].y, (int)f[2 * kb + 1].z, (int)f[2 * kb + 1].w};
        s[kb] = mfma32x32x64_f8<FMT>(a, qf[st], st == 0 ? f32x16{} : s[kb]);
      }
    }
  };
  auto matrix_phase = [&](int kbuf, int vbuf) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int c = 0; c < 2; ++c) ka[st][c] = k_off[st][c] + kbuf * T::KTILE;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) va[db] = v_off[db] + vbuf * T::VTILE;
    uint4 fa[4], fb[4];
    load_group(0, fa);
#pragma unroll
    for (int g = 0; g < 6; ++g) {
      if (g + 1 < 6) load_group(g + 1, (g & 1) ? fa : fb);
      mfma_group(g, (g & 1) ? fb : fa);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Online-softmax update for tile j, as in the bf16 kernel.
  auto softmax_phase = [&](int j) {
    if (j >= w_nkt) {
#pragma unroll
      for (int i = 0; i < BN / 16; ++i) pf[i] = bf16x8{};
      return;
    }
    const int k0 = j * BN;
    const bool need_mask = (k0 + BN > kv_len) || (CAUSAL && k0 + BN - 1 > w_first + diag);
    if (need_mask) {
      const int rel = (CAUSAL ? min(kv_len, qrow + diag + 1) : kv_len) - k0 - 4 * hi;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) >= rel) s[kb][r] = kNegInf;
    }
    float mxp[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mxp[r & 3] = fmaxf(mxp[r & 3], s[kb][r]);
    float mx = fmaxf(fmaxf(mxp[0], mxp[1]), fmaxf(mxp[2], mxp[3]));
    mx = pair_max32(mx) * p.scale_log2;
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
    float rsp[4] = {0.f, 0.f, 0.f, 0.f}, lrp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], p.scale_log2, -m_use));
        rsp[r & 3] += s[kb][r];
      }
    l += (rsp[0] + rsp[1]) + (rsp[2] + rsp[3]);
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        float t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = s[kb][8 * mm + e];
        pf[kb * 2 + mm] = pack_bf16x8_sum(t, lrp[kb * 2 + mm]);
      }
    lr += (lrp[0] + lrp[1]) + (lrp[2] + lrp[3]);
  };

  // Each step issues one V load and one K copy per thread, both in the
  // matrix phase after its products are issued (the vector ALU has room
  // there; the softmax phase is the longer one).  The V load of step j-1
  // (tile j+1) is converted into LDS in the matrix phase of step j, into a
  // buffer no wave reads then: it last held tile j-2, whose last reads ended
  // before the barrier that opened the phase, and tile j+1 is first read in
  // phase 2j+4.  The compiler's own wait for the load also covers the copies
  // issued after it.  Before either barrier of step j every wave leaves at
  // most two memory operations in flight (step j's own V load and K copy):
  // the K copy of step j-1 (tile j+1, read from phase 2j+2 on) is then
  // complete by the barrier that ends phase 2j+1, as in the bf16 kernel.
  auto barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  auto wait_copies = [&]() { asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); };

  // Step 0 multiplies P = 0 by V buffer 2, which nothing has filled yet.
  {
    uint4* v2 = (uint4*)(lds + T::V_BASE + 2 * T::VTILE * 2);
    for (int i = tid; i < T::VTILE / 8; i += T::THREADS) v2[i] = uint4{0, 0, 0, 0};
  }
  if (n_kt > 0) {
    copy_k(0, 0);
    copy_k(1, 1);
    load_v(0);
    store_v(0);
    load_v(1);
    asm volatile("s_waitcnt vmcnt(1)" ::: "memory");  // K_0 and K_1 are in
  }
  barrier();
  if (!lead) barrier();
  if (n_kt > 0) {
    // Step j uses buffers b0 = j % 3, b1 = (j + 1) % 3, b2 = (j + 2) % 3; the
    // loop is unrolled by three so that they are constants.
    auto step = [&](int j, int b0, int b1, int b2) {
      matrix_phase(b0, b2);  // K_j in K buffer b0, V_{j-1} in V buffer b2
      store_v(b1);           // V_{j+1} into V buffer (j + 1) % 3
      load_v(j + 2);
      copy_k(j + 2, b2);
      wait_copies();
      barrier();
      softmax_phase(j);
      wait_copies();
      barrier();
    };
    for (int j = 0; j <= n_kt; j += 3) {
      step(j, 0, 1, 2);
      if (j + 1 > n_kt) break;
      step(j + 1, 1, 2, 0);
      if (j + 2 > n_kt) break;
      step(j + 2, 2, 0, 1);
    }
  }
  if (lead) barrier();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the clamped copies before exit

  const float lt = pair_sum32(l);
  const float lrt = pair_sum32(lr);
  if (qrow < p.Nq) {
    const float inv = lt > 0.f ? p.v_descale / lrt : 0.f;
    uint16_t* op = p.o + (q_base + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) store_row_bf16x32(op + db * 32, oacc[db], inv, hi);
    if (hi == 0) p.lse[q_base + qrow] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : kNegInf;
  }
}

template <int FMT, bool CAUSAL, bool PADDED>
static hipError_t launch_fp8_t(const AttnArgs& a, const Fp8Scales& sc) {
  Fp8Params p;
  p.q = (const uint8_t*)a.q;
  p.k = (const uint8_t*)a.k;
  p.v = (const uint8_t*)a.v;
  p.o = (uint16_t*)a.o;
  p.lse = a.lse;
  p.kv_seqlens = a.kv_seqlens;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk;
  p.n_qtiles = (a.Nq + Fp8Tile::BM - 1) / Fp8Tile::BM;
  p.scale_log2 = a.scale * sc.q_descale * sc.k_descale * kLog2e;
  p.v_descale = sc.v_descale;
  const long long grid = (long long)p.n_qtiles * a.B * a.Hq;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_fp8_pp_kernel<FMT, CAUSAL, PADDED>), dim3((unsigned)grid), dim3(Fp8Tile::THREADS), 0,
                     a.stream, p);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_fmt(const AttnArgs& a, const Fp8Scales& sc) {
  const bool padded = a.kv_seqlens != nullptr;
  if (a.causal) return padded ? launch_fp8_t<FMT, true, true>(a, sc) : launch_fp8_t<FMT, true, false>(a, sc);
  return padded ? launch_fp8_t<FMT, false, true>(a, sc) : launch_fp8_t<FMT, false, false>(a, sc);
}

hipError_t launch_fwd_fp8(const AttnArgs& a, int e5m2, const Fp8Scales& sc) {
  return e5m2 ? launch_fmt<1>(a, sc) : launch_fmt<0>(a, sc);
}

}  // namespace fa
