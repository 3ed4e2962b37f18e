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
// Two kernels.  The ping-pong kernel (fwd_bf16_pp_kernel, below) runs d = 128
// and d = 64; the 4-wave kernel that follows here runs d = 64 under a causal
// mask when the grid is too small for 256-row work-groups to balance (see
// launch_mode).
//
// 4-wave kernel: 4 waves x 32 query rows = 128 rows per work-group.  Each KV
// tile holds 64 keys.  In both kernels everything per query row lives in one
// lane pair (lanes i and i+32):
//   S^T = K Q^T      A = K rows from LDS, B = Q^T kept in VGPRs
//   O^T += V^T P^T   A = V^T via ds_read_b64_tr_b16, B = P^T straight from
//                    the S^T accumulators (rounded to bf16)
// so the row max/sum need one cross-half exchange and the rescale of O by
// alpha = 2^(m_old - m_new) is lane-local.  Exponentials run in base 2 with
// scale*log2(e) folded into one FMA.
//
// K/V tiles move HBM -> LDS with direct global_load_lds_dwordx4 copies (no
// VGPR staging) into two LDS buffers: tile t+1 streams in while tile t is
// being consumed, with one barrier per tile.  The two buffers are distinct
// __shared__ arrays and the tile loop is unrolled by two, so every LDS read
// names its buffer statically and the compiler can tell the in-flight copies
// into the other buffer do not alias it (otherwise it waits for them).
#include <atomic>

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
  const int32_t* cu_q;  // packed layout only
  const int32_t* cu_k;
  int total_q, total_k;
  int B, Hq, Hkv, Nq, Nk;
  int n_qtiles;
  float scale_log2;  // scale * log2(e)
};

// Sequence layouts: dense [B, H, N, d]; the same with per-sequence valid key
// lengths; or packed variable-length sequences (rows of every head
// concatenated along the token axis, [H, total, d], delimited by cumulative
// offsets).
enum SeqMode : int { kDense = 0, kPadded = 1, kPacked = 2 };

// One (sequence, query head) of a forward call: the row index of its first
// query and of its KV head's first key (rows of d elements; the LSE shares
// the query index), its query and key counts, and the keys that may be seen.
struct SeqRows {
  size_t q_row0, kv_row0;
  int nq, nk, kv_len;
};

template <int MODE>
__device__ __forceinline__ SeqRows seq_rows(const FwdParams& p, int b, int hq, int hk) {
  SeqRows r;
  if constexpr (MODE == kPacked) {
    const int2 qr = packed_rows(p.cu_q, b, p.total_q), kr = packed_rows(p.cu_k, b, p.total_k);
    r.q_row0 = (size_t)hq * p.total_q + qr.x;
    r.kv_row0 = (size_t)hk * p.total_k + kr.x;
    r.nq = qr.y;
    r.nk = r.kv_len = kr.y;
  } else {
    r.q_row0 = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;
    r.kv_row0 = ((size_t)b * p.Hkv + hk) * (size_t)p.Nk;
    r.nq = p.Nq;
    r.nk = p.Nk;
    r.kv_len = MODE == kPadded ? clamp_len(p.kv_seqlens, b, p.Nk) : p.Nk;
  }
  return r;
}

template <int D, bool CAUSAL, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void fwd_bf16_kernel(FwdParams p) {
  using T = FwdTile<D>;
  constexpr int BM = T::BM, BN = T::BN;
  // Two buffers of one K and one V tile, BN rows x D, rows swizzled in
  // 16-byte chunks (swz<D>).
  __shared__ __attribute__((aligned(1024))) uint16_t k_s0[T::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_s0[T::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k_s1[T::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_s1[T::TILE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, hi = lane >> 5;

  // Work-group -> (query tile, head, batch).  The heavier half of the query
  // tiles (under a causal mask, the last ones) is dispatched first, heaviest
  // first; the lighter half follows lightest first, so that the work-groups
  // dispatched one grid-half apart, which share a CU when the whole grid is
  // resident at once (this kernel runs small causal grids), carry about the
  // same work together: tiles n-1-s and s.
  const int bh_count = p.B * p.Hq;
  const int bh = xcd_grouped_head((int)(blockIdx.x % bh_count), p.B, p.Hq, p.Hkv);
  const int slot = (int)(blockIdx.x / bh_count), half = (p.n_qtiles + 1) / 2;
  const int qt = !CAUSAL ? p.n_qtiles - 1 - slot : (slot < half ? p.n_qtiles - 1 - slot : slot - half);
  const int b = bh / p.Hq, hq = bh - b * p.Hq;
  const int hk = hq / (p.Hq / p.Hkv);

  const SeqRows sr = seq_rows<MODE>(p, b, hq, hk);
  const int nq = sr.nq, kv_len = sr.kv_len;
  const int q0 = qt * BM;
  if (MODE == kPacked && q0 >= nq) return;  // a sequence shorter than the longest one
  const int diag = sr.nk - nq;  // key j visible to row i iff j <= i + diag
  int kend = kv_len;
  if (CAUSAL) {
    const int q_last = min(q0 + BM, nq) - 1;
    kend = min(kend, q_last + diag + 1);
  }
  const int n_kt = kend > 0 ? (kend + BN - 1) / BN : 0;

  const size_t q_base = sr.q_row0;
  const uint16_t* kg = p.k + sr.kv_row0 * D;
  const uint16_t* vg = p.v + sr.kv_row0 * D;

  // Q^T fragment: lane (li, hi) holds row q0 + 32*wave + li, columns
  // 16*s + 8*hi .. +7 for each k-step s.
  const int qrow = q0 + wave * 32 + li;
  bf16x8 qf[D / 16];
  if (qrow < nq) {
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
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  int src_row[T::COPIES], src_off[T::COPIES];
#pragma unroll
  for (int i = 0; i < T::COPIES; ++i) {
    const int r = (wave * T::COPIES + i) * T::RPI + lane / T::CPR;
    src_row[i] = r;
    src_off[i] = r * D + ((lane % T::CPR) ^ swz<D>(r)) * 8;
  }
  auto issue_tile = [&](int kt, uint16_t* kdst, uint16_t* vdst) {
    const int k0 = kt * BN;
    const uint16_t* kt_k = kg + (size_t)k0 * D;
    const uint16_t* kt_v = vg + (size_t)k0 * D;
    const bool tail = k0 + BN > kv_len;  // rows past the length re-read the last valid row
#pragma unroll
    for (int i = 0; i < T::COPIES; ++i) {
      int off = src_off[i];
      if (tail) off += (min(k0 + src_row[i], kv_len - 1) - (k0 + src_row[i])) * D;
      const int dst = (wave_u * T::COPIES + i) * 512;
      load_lds_16B(kt_k + off, kdst + dst);
      load_lds_16B(kt_v + off, vdst + dst);
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

  // One tile: wait for its copies, start the next tile's copies into the
  // other buffer, then S^T, mask, online softmax and P.V.
  auto tile_step = [&](int kt, const uint16_t* kl, const uint16_t* vl, uint16_t* kn, uint16_t* vn) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile kt is in LDS; every wave is done with tile kt-1
    if (kt + 1 < n_kt) issue_tile(kt + 1, kn, vn);

    // S^T[key][query] = K Q^T for the 64 keys of the tile, two 32-key blocks.
    f32x16 s[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      bf16x8 kf[D / 16];
#pragma unroll
      for (int st = 0; st < D / 16; ++st) kf[st] = *(const bf16x8*)(kl + kb * 32 * D + k_off[st]);
      s[kb] = f32x16{};
#pragma unroll
      for (int st = 0; st < D / 16; ++st) s[kb] = mfma32x32x16(kf[st], qf[st], s[kb]);
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
  };

  if (n_kt > 0) issue_tile(0, k_s0, v_s0);
  for (int kt = 0; kt < n_kt; kt += 2) {
    tile_step(kt, k_s0, v_s0, k_s1, v_s1);
    if (kt + 1 < n_kt) tile_step(kt + 1, k_s1, v_s1, k_s0, v_s0);
  }

  // Epilogue: O = O_acc / lr, LSE = ln2 * (m + log2 l).  Only O and LSE are
  // ever written to memory.
  const float lt = pair_sum32(l);
  const float lrt = pair_sum32(lr);
  if (qrow < nq) {
    const float inv = lt > 0.f ? 1.f / lrt : 0.f;
    uint16_t* op = p.o + (q_base + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) store_row_bf16x32(op + db * 32, oacc[db], inv, hi);
    if (hi == 0) p.lse[q_base + qrow] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// Ping-pong kernel: eight waves in two groups of four, kept one phase apart ("ping
// pong").  Waves w and w+4 share a SIMD.  In every phase one group runs its
// matrix-core work for tile j -- S_j = K_j Q^T and O += V_{j-1} P_{j-1} -- while
// the other group runs the online-softmax update of its previous tile on the
// vector ALU, so the two kinds of work overlap on each SIMD instead of
// alternating inside one wave.  A barrier closes every phase.
//
//   phase 2j   : group 0 matrix(j)      group 1 softmax(j-1)
//   phase 2j+1 : group 0 softmax(j)     group 1 matrix(j)
//
// Both groups run the same program -- matrix(j), barrier, softmax(j),
// barrier -- group 1 simply starting one barrier later.  K and V tiles rotate
// through rings of NBUF LDS buffers each; step j starts copying K_{j+NBUF-1}
// and V_{j+NBUF-2} (the furthest a ring of NBUF buffers allows: one tile more
// and a copy would overwrite a tile the lagging group still reads).  With
// NBUF = 4 every copy has three phases to land before it is waited on.
//
// Under a causal mask query tile i sees i+1 times the keys of tile 0; with
// PAIR a work-group runs tile i and then tile n-1-i, so every work-group of a
// head does the same work and the grid has no long tail.
//
// d = 64 runs the same kernel on 128-key tiles: a tile is again 16 KiB, the
// copy plan and the waits are unchanged, and a step again holds 32 products
// (its softmax covers twice the elements, which at d = 64 outweighs them).
template <int D_>
struct PPTile {
  static constexpr int D = D_, BM = 256, BN = D_ == 128 ? 64 : 128, WAVES = 8, THREADS = 512;
  static constexpr int TILE = BN * D;                 // elements per K or V tile (16 KiB)
  static constexpr int CPR = D / 8, RPI = 64 / CPR;   // 16-byte chunks per row, rows per 1 KiB copy
  static constexpr int COPIES = BN / RPI / WAVES;     // 1 KiB copies per wave per tile (= 2)
};

// Chunk swizzle of the V tiles, which are only read transposed: a half wave
// reads 4 consecutive rows (from a multiple of 4) x 4 consecutive chunks.  At
// d = 128 (256-byte rows) XOR-ing the chunk with 4*(r % 4) spreads them over
// all 64 banks; at d = 64 (128-byte rows) rows r and r+2 share banks, and
// XOR-ing with 4*((r/2) % 2) separates them.  Neither depends on bits above
// the second, so moving 8 or 16 rows on leaves the swizzle unchanged.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  if constexpr (D == 128) return swz_v128(r);
  else return 4 * ((r >> 1) & 1);
}

template <int D, bool CAUSAL, int MODE, int NBUF, bool PAIR>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_bf16_pp_kernel(FwdParams p) {
  using T = PPTile<D>;
  constexpr int BM = T::BM, BN = T::BN;
  constexpr int ST = D / 16, DB = D / 32, NS = BN / 16;  // k-steps, d-blocks, 16-key slices
  static_assert(NBUF == 3 || NBUF == 4, "ring depth");
  constexpr int KAHEAD = NBUF - 1, VAHEAD = NBUF - 2;  // tiles copied ahead of the one being used
  // buffers 0..NBUF-1: K tiles, NBUF..2*NBUF-1: V tiles; tile t lives in buffer t % NBUF.
  __shared__ __attribute__((aligned(1024))) uint16_t kv_lds[2 * NBUF][T::TILE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, hi = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool lead = wave_u < 4;  // group 0 leads, group 1 lags one phase

  const int bh_count = p.B * p.Hq;
  const int bh = xcd_grouped_head((int)(blockIdx.x % bh_count), p.B, p.Hq, p.Hkv);
  const int slot = (int)(blockIdx.x / bh_count);
  const int b = bh / p.Hq, hq = bh - b * p.Hq;
  const int hk = hq / (p.Hq / p.Hkv);

  const SeqRows sr = seq_rows<MODE>(p, b, hq, hk);
  const int nq = sr.nq, kv_len = sr.kv_len;
  const int diag = sr.nk - nq;
  const size_t q_base = sr.q_row0;
  const uint16_t* kg = p.k + sr.kv_row0 * D;
  const uint16_t* vg = p.v + sr.kv_row0 * D;

  // Work-group -> query tiles.  Without PAIR: one tile, the heaviest causal
  // tiles dispatched first.  With PAIR: tiles slot and n-1-slot (one tile
  // when they coincide).
  const int n_tiles_here = PAIR ? ((p.n_qtiles - 1 - slot) > slot ? 2 : 1) : 1;
  for (int ti = 0; ti < n_tiles_here; ++ti) {
    const int qt = PAIR ? (ti == 0 ? slot : p.n_qtiles - 1 - slot) : p.n_qtiles - 1 - slot;
    const int q0 = qt * BM;
    if (MODE == kPacked && q0 >= nq) continue;  // a sequence shorter than the longest one (uniform)
    int kend = kv_len;
    if (CAUSAL) kend = min(kend, min(q0 + BM, nq) - 1 + diag + 1);
    const int n_kt = kend > 0 ? (kend + BN - 1) / BN : 0;
    // tiles this wave's rows can see at all (later tiles are skipped, not masked)
    const int w_first = q0 + wave_u * 32;
    int w_kend = kv_len;
    if (CAUSAL) w_kend = min(w_kend, min(w_first + 32, nq) - 1 + diag + 1);
    const int w_nkt = w_kend > 0 ? (w_kend + BN - 1) / BN : 0;

    const int qrow = w_first + li;
    bf16x8 qf[D / 16];
    if (qrow < nq) {
      const uint16_t* qp = p.q + (q_base + qrow) * D + 8 * hi;
#pragma unroll
      for (int st = 0; st < D / 16; ++st) qf[st] = *(const bf16x8*)(qp + 16 * st);
    } else {
#pragma unroll
      for (int st = 0; st < D / 16; ++st) qf[st] = bf16x8{};
    }
    // Retire the Q loads here.  Their first use is inside the tile loop, and
    // the compiler's wait for them there would be a vmcnt count that, in every
    // later step, also waits for that step's K/V copies.
#pragma unroll
    for (int st = 0; st < D / 16; ++st) asm volatile("" : "+v"(qf[st]));

    // Per-lane LDS offsets of the fragment reads (elements), the same for
    // every tile.  K: row li of a 32-key block, chunk 2*st + hi; V (transposed
    // 4x16 reads): row tr_r (the second read of a pair is 8 rows on).
    int k_off[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st) k_off[st] = li * D + (((2 * st + hi) ^ swz<D>(li)) * 8);
    const int tr_r = 4 * hi + ((lane & 15) >> 2);
    const int tr_cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int tr_in = 4 * (lane & 1);
    int v_off[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)  // V region starts at buffer NBUF
      v_off[db] = NBUF * T::TILE + tr_r * D + (((4 * db + tr_cc) ^ vswz<D>(tr_r)) * 8) + tr_in;
    // Fragment reads address lds0 + (per-step address register) + (a
    // compile-time offset): the step adds its buffer's base to the lane offsets
    // once, so one loop body serves every buffer.  The empty asm hides the lane
    // offsets' known bits, so the compiler keeps the constant parts as additions
    // it can fold into the DS instructions' offset field (the library is built
    // with DS offset folding allowed: these addresses are never negative).
#pragma unroll
    for (int st = 0; st < D / 16; ++st) asm volatile("" : "+v"(k_off[st]));
#pragma unroll
    for (int db = 0; db < D / 32; ++db) asm volatile("" : "+v"(v_off[db]));
    const uint16_t* lds0 = kv_lds[0];

    // Copy plan: wave w moves the 1 KiB copies c = 2w, 2w+1 (rows RPI*c ..
    // RPI*c + RPI-1) of each K and V tile; lane l brings row RPI*c + l/CPR,
    // source chunk (l % CPR) ^ swizzle(row), to LDS position l % CPR (K: swz,
    // V: vswz).
    // The lane offsets of a full tile's copies are the same for every tile:
    // computed once here (bytes; the first copy's carries the +1 KiB bias of
    // copy16x2_to_lds).  Only the last tile of a sequence, where rows past the
    // length re-read the last valid row, adjusts them.
    static_assert(T::COPIES == 2, "copies are issued in pairs");
    const int cp_r0 = (wave_u * T::COPIES) * T::RPI + lane / T::CPR, cp_r1 = cp_r0 + T::RPI;
    const int cp_c = lane % T::CPR;
    int cp_k0 = (cp_r0 * D + ((cp_c ^ swz<D>(cp_r0)) * 8)) * 2 + 1024;
    int cp_k1 = (cp_r1 * D + ((cp_c ^ swz<D>(cp_r1)) * 8)) * 2;
    int cp_v0 = (cp_r0 * D + ((cp_c ^ vswz<D>(cp_r0)) * 8)) * 2 + 1024;
    int cp_v1 = (cp_r1 * D + ((cp_c ^ vswz<D>(cp_r1)) * 8)) * 2;
    asm volatile("" : "+v"(cp_k0), "+v"(cp_k1), "+v"(cp_v0), "+v"(cp_v1));

    float m = kNegInf, l = 0.f, lr = 0.f;
    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    f32x16 s[BN / 32];   // S_j, from its matrix phase to its softmax phase
    bf16x8 pf[BN / 16];  // P_j, from its softmax phase to the next matrix phase
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int i = 0; i < BN / 16; ++i) pf[i] = bf16x8{};

    // Tiles past the last one are clamped to it: the copy then lands in a
    // buffer no phase reads, which keeps exactly four copies per step.
    auto copy_tile = [&](const uint16_t* src, int t, uint16_t* dst, bool is_v) {
      t = min(t, n_kt - 1);
      const int k0 = t * BN;
      const uint16_t* base = src + (size_t)k0 * D;
      int o0 = is_v ? cp_v0 : cp_k0, o1 = is_v ? cp_v1 : cp_k1;
      if (k0 + BN > kv_len) {  // rows past the length re-read the last valid row
        o0 -= max(0, k0 + cp_r0 - (kv_len - 1)) * (2 * D);
        o1 -= max(0, k0 + cp_r1 - (kv_len - 1)) * (2 * D);
      }
      // the wave's two copies are adjacent in LDS: one m0 setting serves both
      copy16x2_to_lds((const char*)base - 1024, o0, o1, dst + wave_u * T::COPIES * 512);
    };

    int ka[D / 16], va[D / 32];  // this step's K / V fragment offsets (elements)
    // Consecutive MFMAs always accumulate into different registers: a chain of
    // dependent MFMAs on one accumulator issues far below the matrix-core rate,
    // two or more interleaved chains keep it busy.  Four groups of four
    // products for S, four for P.V:
    //   S group g (0..3):  key blocks 2*kp, 2*kp+1 (alternating) at k-steps
    //                      2*sp, 2*sp+1, with kp = g / (ST/2), sp = g % (ST/2)
    //   P.V group 4+i:     16-key slices NS/4*i .. (all d-blocks, alternating)
    auto s_item = [](int g, int i, int& kb, int& st) {
      kb = 2 * (g / (ST / 2)) + (i & 1);
      st = 2 * (g % (ST / 2)) + (i >> 1);
    };
    auto pv_item = [](int g, int i, int& sl, int& db) {
      sl = (NS / 4) * (g - 4) + i / DB;
      db = i % DB;
    };
    auto load_group = [&](int g, bf16x8* f) {
      if (g < 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int kb, st;
          s_item(g, i, kb, st);
          f[i] = *(const bf16x8*)(lds0 + ka[st] + kb * 32 * D);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int sl, db;
          pv_item(g, i, sl, db);
          const int c = 16 * sl * D;
          f[i] = join_bf16x8(lds_read_tr16(lds0 + va[db] + c), lds_read_tr16(lds0 + va[db] + c + 8 * D));
        }
      }
    };
    auto mfma_group = [&](int g, const bf16x8* f) {
      if (g < 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int kb, st;
          s_item(g, i, kb, st);
          s[kb] = mfma32x32x16(f[i], qf[st], st == 0 ? f32x16{} : s[kb]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int sl, db;
          pv_item(g, i, sl, db);
          oacc[db] = mfma32x32x16(f[i], pf[sl], oacc[db]);
        }
      }
    };
    // The pipeline alternates P.V groups (G4..G7) and S groups (G0..G3): the
    // P.V groups' transposed V reads move half the bytes per LDS cycle of the
    // S groups' K reads, and alternating the two spreads the LDS demand evenly
    // over the phase.  The first two groups of a matrix phase (P.V on V_{j-1},
    // S on K_j) are loaded at the start of the wave's previous softmax phase,
    // so the phase opens with MFMAs instead of waiting on LDS.  Both tiles were
    // copied at least two steps back; the copy waits below make them complete
    // before that softmax phase in both groups, and no copy in flight then
    // targets their buffers.
    constexpr int PRE = 2;
    bf16x8 fa[4], fb[4];
    auto run_groups = [&]() {
      auto grp = [](int i) { return (i & 1) ? (i >> 1) : 4 + (i >> 1); };
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i + 1 < 8 && i + 1 >= PRE) load_group(grp(i + 1), (i & 1) ? fa : fb);
        mfma_group(grp(i), (i & 1) ? fb : fa);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto preload = [&]() {
      load_group(4, fa);
      load_group(0, fb);
    };
    // Every step runs all eight groups -- one code path keeps the register
    // allocation tight.  Work a wave does not need is harmless: S_j of a tile
    // past the wave's range is never used, and P.V runs with P = 0 (at j = 0,
    // and after a skipped softmax) against finite V data.
    auto set_bufs = [&](int kbuf, int vbuf) {
#pragma unroll
      for (int st = 0; st < D / 16; ++st) ka[st] = k_off[st] + kbuf * T::TILE;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) va[db] = v_off[db] + vbuf * T::TILE;
    };

    // Online-softmax update for tile j (S_j -> P_j), as in the 4-wave kernel.
    auto softmax_phase = [&](int j) {
      if (j >= w_nkt) {
#pragma unroll
        for (int i = 0; i < BN / 16; ++i) pf[i] = bf16x8{};
        return;
      }
      const int k0 = j * BN;
      const bool need_mask = (k0 + BN > kv_len) || (CAUSAL && k0 + BN - 1 > w_first + diag);
      if (need_mask) {
        // key k0 + 4*hi + c(kb, r) is visible iff c < rel.  The sign of
        // c - rel selects the score or -inf bit for bit.  (The element is
        // copied to a scalar first: this compiler's __builtin_bit_cast of a
        // vector element reads element 0 whatever the index.)
        const int rel = (CAUSAL ? min(kv_len, qrow + diag + 1) : kv_len) - k0 - 4 * hi;
        const int ninf = __builtin_bit_cast(int, kNegInf);
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int keep = (kb * 32 + 8 * (r >> 2) + (r & 3) - rel) >> 31;  // all ones iff visible
            const float e = s[kb][r];
            s[kb][r] = __builtin_bit_cast(float, (__builtin_bit_cast(int, e) & keep) | (ninf & ~keep));
          }
      }
      // Row max, exponentials and the two row sums, with the reductions split
      // into four independent partial chains (short dependency chains keep the
      // vector ALU busy).
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
      float rsp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], p.scale_log2, -m_use));
          rsp[r & 3] += s[kb][r];
        }
      l += (rsp[0] + rsp[1]) + (rsp[2] + rsp[3]);
      float lrp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          float t[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) t[e] = s[kb][8 * mm + e];
          pf[kb * 2 + mm] = pack_bf16x8_sum(t, lrp[(kb * 2 + mm) & 3]);
        }
      lr += (lrp[0] + lrp[1]) + (lrp[2] + lrp[3]);
    };

    // Each step issues exactly four copy instructions per wave (K_{j+KAHEAD},
    // V_{j+VAHEAD}), after its matrix work.  Step j's softmax phase reads the
    // early fragments of K_{j+1} and V_j, copied NBUF-2 steps before; for
    // group 0 that phase opens with the barrier in which group 1 ends step
    // j-1.  So every wave waits, before the barrier that ends its step, for
    // all copies older than its last NBUF-3 steps' (vmcnt 0 with three
    // buffers, vmcnt 4 with four): those copies are then complete in both
    // groups before either group reads them.  Before the mid-step barrier the
    // wait allows NBUF-2 steps of copies in flight and is already met.  The
    // loop body stays free of group-dependent code, which stops the compiler
    // from cloning it per group.  lgkmcnt(0) retires this wave's LDS reads
    // before any barrier, so a buffer is free once the barrier after its last
    // use has passed.  (tests/test_schedule_model.py replays this schedule.)
    auto barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
    auto wait_mid = [&]() {
      if constexpr (NBUF == 3) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    };
    auto wait_end = [&]() {
      if constexpr (NBUF == 3) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    };
    auto wait_all_copies = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

    // Step 0 multiplies P = 0 by V buffer NBUF-1 (V_{-1}), which no copy has
    // filled yet: give it finite contents.
    for (int i = tid; i < T::TILE / 8; i += T::THREADS) ((uint4*)kv_lds[2 * NBUF - 1])[i] = uint4{0, 0, 0, 0};
    if (n_kt > 0) {
#pragma unroll
      for (int t = 0; t < KAHEAD; ++t) copy_tile(kg, t, kv_lds[t], false);
#pragma unroll
      for (int t = 0; t < VAHEAD; ++t) copy_tile(vg, t, kv_lds[NBUF + t], true);
      wait_all_copies();  // the first tiles are in before either group reads them
    }
    barrier();
    if (!lead) barrier();
    // Step j: start K_{j+KAHEAD} (into the buffer of K_{j-1}) and V_{j+VAHEAD}
    // (into the buffer of V_{j-2}); matrix work on K_j and V_{j-1}; softmax of
    // S_j.  A work-group with no visible tile (empty sequence, or every row
    // above the causal diagonal) runs no step: its copies would address tile -1.
    if (n_kt > 0) {
      // Step j uses K buffer kb = j % NBUF and V buffer (kb - 1) % NBUF.  The
      // loop is unrolled by NBUF so that every buffer index is a constant and
      // the buffer bases fold into the LDS instructions' offset fields.
      auto step = [&](int j, int kb) {
        run_groups();  // K_j in K buffer kb, V_{j-1} in V buffer kb-1 (set and preloaded before)
        // Copies go out after the matrix work is issued: at the start of the
        // phase all four waves of the group would queue them at once, holding
        // back their first MFMAs.
        copy_tile(kg, j + KAHEAD, kv_lds[(kb + KAHEAD) % NBUF], false);
        copy_tile(vg, j + VAHEAD, kv_lds[NBUF + (kb + VAHEAD) % NBUF], true);
        wait_mid();
        barrier();
        set_bufs((kb + 1) % NBUF, kb);  // step j + 1: K_{j+1} in K buffer kb+1, V_j in V buffer kb
        preload();                      // (after the last step: harmless reads that nothing uses)
        softmax_phase(j);
        wait_end();
        barrier();
      };
      set_bufs(0, NBUF - 1);
      preload();
      // (written out: an unrolled loop with an exit test costs the register
      // allocation some 40 VGPRs)
      for (int j = 0; j <= n_kt; j += NBUF) {
        step(j, 0);
        if (j + 1 > n_kt) break;
        step(j + 1, 1);
        if (j + 2 > n_kt) break;
        step(j + 2, 2);
        if constexpr (NBUF == 4) {
          if (j + 3 > n_kt) break;
          step(j + 3, 3);
        }
      }
    }
    if (lead) barrier();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the clamped copies before the epilogue
    // Before the next tile's LDS writes, every wave's copies of this tile
    // have landed (the last step's may still be in flight at the barrier above).
    if (ti + 1 < n_tiles_here) barrier();

    const float lt = pair_sum32(l);
    const float lrt = pair_sum32(lr);
    if (qrow < nq) {
      const float inv = lt > 0.f ? 1.f / lrt : 0.f;
      uint16_t* op = p.o + (q_base + qrow) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) store_row_bf16x32(op + db * 32, oacc[db], inv, hi);
      if (hi == 0) p.lse[q_base + qrow] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : kNegInf;
    }
  }
}

static FwdParams make_params(const AttnArgs& a, int bm) {
  FwdParams p;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k;
  p.v = (const uint16_t*)a.v;
  p.o = (uint16_t*)a.o;
  p.lse = a.lse;
  p.kv_seqlens = a.kv_seqlens;
  p.cu_q = a.cu_q;
  p.cu_k = a.cu_k;
  p.total_q = a.total_q;
  p.total_k = a.total_k;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk;
  p.n_qtiles = (a.Nq + bm - 1) / bm;
  p.scale_log2 = a.scale * kLog2e;
  return p;
}

template <int D, bool CAUSAL, int MODE, int NBUF = 3, bool PAIR = false>
static hipError_t launch_fwd_bf16_pp(const AttnArgs& a) {
  using T = PPTile<D>;
  const FwdParams p = make_params(a, T::BM);
  const long long slots = PAIR ? (p.n_qtiles + 1) / 2 : p.n_qtiles;
  const long long grid = slots * a.B * a.Hq;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_bf16_pp_kernel<D, CAUSAL, MODE, NBUF, PAIR>), dim3((unsigned)grid), dim3(T::THREADS), 0,
                     a.stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL, int MODE>
static hipError_t launch_fwd_bf16_t(const AttnArgs& a) {
  using T = FwdTile<D>;
  const FwdParams p = make_params(a, T::BM);
  const long long grid = (long long)p.n_qtiles * a.B * a.Hq;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, MODE>), dim3((unsigned)grid), dim3(T::THREADS), 0,
                     a.stream, p);
  return hipGetLastError();
}

// Compute units of the current device (queried once per device).
static int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int MODE>
static hipError_t launch_mode(const AttnArgs& a) {
  if (a.d == 128) return a.causal ? launch_fwd_bf16_pp<128, true, MODE>(a) : launch_fwd_bf16_pp<128, false, MODE>(a);
  if (!a.causal) return launch_fwd_bf16_pp<64, false, MODE>(a);
  // d = 64 under a causal mask: the work of a query tile grows with its index,
  // and a grid of fewer than two 256-row work-groups per CU runs as long as its
  // heaviest tile while the CUs that drew light ones idle.  There the 128-row
  // kernel (several work-groups per CU, half the tile) balances better.
  const long long pp_grid = (long long)((a.Nq + PPTile<64>::BM - 1) / PPTile<64>::BM) * a.B * a.Hq;
  if (pp_grid < 2LL * cu_count()) return launch_fwd_bf16_t<64, true, MODE>(a);
  return launch_fwd_bf16_pp<64, true, MODE>(a);
}

hipError_t launch_fwd_bf16(const AttnArgs& a) {
  if (a.cu_q != nullptr) return launch_mode<kPacked>(a);
  return a.kv_seqlens != nullptr ? launch_mode<kPadded>(a) : launch_mode<kDense>(a);
}

}  // namespace fa
