// Backward pass of exact attention (bf16, matrix cores): dQ, dK, dV.
//
// The pages say that the backward pass recomputes intermediate values instead
// of storing them (Exam deep-dive "Flash Attention 在改善什麼？", section 技術版,
// "Recomputation"; Interview note, section 节省显存，不等于所有内存都变少).  What
// it computes is the derivative of the forward definition of the "FlashAttention"
// concept note, section "是什么".  Per (query i, key j) pair that takes part:
//     P_ij  = 2^(S_ij * scale * log2(e) - LSE_i * log2(e))     (recomputed)
//     dP_ij = dO_i . V_j
//     dS_ij = P_ij (dP_ij - D_i),   D_i = dO_i . O_i
//     dV_j += P_ij dO_i,   dK_j += scale dS_ij Q_i,   dQ_i += scale dS_ij K_j
// Three launches: D (one dot product per query row), dQ (one work-group per
// 128-query block streaming 32-key tiles), then dV and dK together (one
// work-group per 128-key block streaming the 32-query tiles of every query
// head that reads it).  The gradient kernels keep different operands on the
// lanes -- dQ the queries (as in the forward), dV/dK the keys -- so every
// product takes its operands straight from the recomputed tiles: no atomics
// (every result is deterministic) and no extra transposes beyond the
// ds_read_b64_tr_b16 reads already used by the forward.  Per visible (query,
// key) pair the kernels execute seven products: S and dP in both, dQ, dV, dK.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

// Element offset of (row, 16-byte chunk) in a row-major [rows][D] bf16 tile
// whose chunks are XOR-swizzled per row.
template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * D + ((chunk ^ swz<D>(row)) * 8);
}

// Register-staged copy of an R-row tile: load() reads rows [0, nvalid) of a
// row-major [*, D] bf16 tensor (later rows become zeros), store() writes the
// swizzled tile to LDS.  256 threads; consecutive threads take consecutive
// 16-byte chunks of a row.
template <int D, int R>
struct TileStage {
  static constexpr int CPR = D / 8;
  static constexpr int CH = R * CPR / 256;
  static_assert(CH >= 1 && R * CPR % 256 == 0, "tile must split evenly over 256 threads");
  uint4 reg[CH];
  __device__ __forceinline__ void load(const uint16_t* base, int nvalid, int tid) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = tid + c * 256, row = idx / CPR, ch = idx % CPR;
      reg[c] = row < nvalid ? *(const uint4*)(base + (size_t)row * D + ch * 8) : uint4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = tid + c * 256, row = idx / CPR, ch = idx % CPR;
      *(uint4*)(lds + tile_off<D>(row, ch)) = reg[c];
    }
  }
};

// A operand of an MFMA whose rows are the tile's columns (d) and whose k runs
// over 16 tile rows starting at r0: two ds_read_b64_tr_b16 (rows r0 + tr_r and
// r0 + 8 + tr_r).  Lane l supplies d = 32*db + (l % 32); the k order matches
// that of a 32x32 accumulator's registers 8*mm .. 8*mm+7 turned into a bf16x8
// B operand (rows 8*(t/4) + 4*(l/32) + t%4 of the slice), as in the forward.
template <int D>
__device__ __forceinline__ bf16x8 tr_fragment(const uint16_t* tile, int r0, int db, int lane) {
  const int tr_r = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_in = 4 * (lane & 1);
  const int ch = 4 * db + tr_cc;
  return join_bf16x8(lds_read_tr16(tile + tile_off<D>(r0 + tr_r, ch) + tr_in),
                     lds_read_tr16(tile + tile_off<D>(r0 + 8 + tr_r, ch) + tr_in));
}

// ---------------------------------------------------------------------------
// D_i = dO_i . O_i (float32), one row per TPR threads.
template <int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const uint16_t* __restrict__ dout,
                                                          const uint16_t* __restrict__ o, float* __restrict__ rowdot,
                                                          long long rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  const long long row = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int sub = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const uint4 a = *(const uint4*)(dout + row * D + sub * 8);
    const uint4 b = *(const uint4*)(o + row * D + sub * 8);
    const unsigned ua[4] = {a.x, a.y, a.z, a.w}, ub[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      acc = __builtin_fmaf(__uint_as_float(ua[x] << 16), __uint_as_float(ub[x] << 16), acc);
      acc = __builtin_fmaf(__uint_as_float(ua[x] & 0xffff0000u), __uint_as_float(ub[x] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && sub == 0) rowdot[row] = acc;
}

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse;
  const float* rowdot;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const int32_t* kv_seqlens;
  int B, Hq, Hkv, Nq, Nk;
  int n_tiles;       // query blocks (dQ kernel) or key blocks (dK/dV kernel) per head
  float scale;
  float scale_log2;  // scale * log2(e)
};

// LSE in base 2 for the recomputation of P; a row with no visible key (LSE =
// -inf) gets +inf so that every recomputed probability of the row is 0.
__device__ __forceinline__ float lse_base2(float lse) { return lse == kNegInf ? __builtin_inff() : lse * kLog2e; }

// ---------------------------------------------------------------------------
// dQ: 4 waves x 32 query rows per work-group; 32-key tiles.  Per tile and wave
//   S^T  = K Q^T,  dP^T = V dO^T           (A: K / V rows from LDS, B: Q / dO in VGPRs)
//   dS^T = P^T * (dP^T - D)                (P^T recomputed from the LSE)
//   dQ^T += K^T dS^T                       (A: K^T by transposed reads, B: dS^T)
template <int D, bool CAUSAL, bool PADDED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_kernel(BwdParams p) {
  constexpr int BM = 128, BN = 32;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[BN * D];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, li = lane & 31, hi = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int bh_count = p.B * p.Hq;
  const int bh = blockIdx.x % bh_count;
  const int qt = p.n_tiles - 1 - (int)(blockIdx.x / bh_count);  // heaviest (causal) first
  const int b = bh / p.Hq, hq = bh - b * p.Hq;
  const int hk = hq / (p.Hq / p.Hkv);

  const int kv_len = PADDED ? clamp_len(p.kv_seqlens, b, p.Nk) : p.Nk;
  const int q0 = qt * BM;
  const int diag = p.Nk - p.Nq;
  int kend = kv_len;
  if (CAUSAL) kend = min(kend, min(q0 + BM, p.Nq) - 1 + diag + 1);
  const int n_kt = kend > 0 ? (kend + BN - 1) / BN : 0;

  const size_t qrow_base = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;
  const size_t kv_base = ((size_t)b * p.Hkv + hk) * (size_t)p.Nk;
  const int qrow = q0 + wave * 32 + li;
  const bool row_ok = qrow < p.Nq;

  bf16x8 qf[D / 16], dof[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    if (row_ok) {
      qf[st] = *(const bf16x8*)(p.q + (qrow_base + qrow) * D + 16 * st + 8 * hi);
      dof[st] = *(const bf16x8*)(p.dout + (qrow_base + qrow) * D + 16 * st + 8 * hi);
    } else {
      qf[st] = bf16x8{};
      dof[st] = bf16x8{};
    }
  }
  const float lse2 = row_ok ? lse_base2(p.lse[qrow_base + qrow]) : __builtin_inff();
  const float drow = row_ok ? p.rowdot[qrow_base + qrow] : 0.f;

  f32x16 dq_acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq_acc[db] = f32x16{};

  TileStage<D, BN> kst, vst;
  const uint16_t* kg = p.k + kv_base * D;
  const uint16_t* vg = p.v + kv_base * D;
  if (n_kt > 0) {
    kst.load(kg, kv_len, tid);
    vst.load(vg, kv_len, tid);
  }
  for (int t = 0; t < n_kt; ++t) {
    __syncthreads();
    kst.store(k_lds, tid);
    vst.store(v_lds, tid);
    __syncthreads();
    if (t + 1 < n_kt) {
      const int k1 = (t + 1) * BN;
      kst.load(kg + (size_t)k1 * D, kv_len - k1, tid);
      vst.load(vg + (size_t)k1 * D, kv_len - k1, tid);
    }
    const int k0 = t * BN;

    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      s = mfma32x32x16(*(const bf16x8*)(k_lds + tile_off<D>(li, 2 * st + hi)), qf[st], s);
      dp = mfma32x32x16(*(const bf16x8*)(v_lds + tile_off<D>(li, 2 * st + hi)), dof[st], dp);
    }
    // lane l: query qrow; register r: key k0 + 8(r/4) + 4*hi + r%4.  Tiles
    // whose keys are all valid and visible to every row of the wave skip the
    // per-element mask (rows past Nq have LSE +inf, so their P is 0 anyway).
    float ds[16];
    if (k0 + BN <= kv_len && (!CAUSAL || k0 + BN - 1 <= q0 + wave_u * 32 + diag)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = fast_exp2(__builtin_fmaf(s[r], p.scale_log2, -lse2)) * (dp[r] - drow);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        bool vis = key < kv_len;
        if (CAUSAL) vis = vis && key <= qrow + diag;
        const float pr = vis ? fast_exp2(__builtin_fmaf(s[r], p.scale_log2, -lse2)) : 0.f;
        ds[r] = pr * (dp[r] - drow);
      }
    }
    bf16x8 dsf[2];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) dsf[mm] = pack_bf16x8(ds + 8 * mm);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) dq_acc[db] = mfma32x32x16(tr_fragment<D>(k_lds, 16 * mm, db, lane), dsf[mm], dq_acc[db]);
  }

  if (row_ok) {
    uint16_t* op = p.dq + (qrow_base + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = pack_bf16x2(dq_acc[db][4 * g] * p.scale, dq_acc[db][4 * g + 1] * p.scale);
        w.y = pack_bf16x2(dq_acc[db][4 * g + 2] * p.scale, dq_acc[db][4 * g + 3] * p.scale);
        *(uint2*)(op + db * 32 + 8 * g + 4 * hi) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dV and dK in one kernel: 4 waves x 32 keys per work-group (keys on the
// lanes, as above); 32-query tiles of every query head that reads the block.
// Per tile and wave, four products:
//   S  = Q K^T      (A: Q rows from LDS, B: the wave's K rows, kept in VGPRs)
//   dP = dO V^T     (A: dO rows from LDS, B: the block's V rows from LDS)
//   P  = 2^(S scale log2(e) - LSE),  dS = P * (dP - D)
//   dV^T += dO^T P  (A: transposed reads of dO),  dK^T += Q^T dS  (A: Q^T)
// The Q and dO tiles rotate through two LDS buffers, filled by direct
// global->LDS copies one tile ahead (rows past the sequence re-read its last
// row: their LSE is +inf, so they carry no weight); wave 0 stages each tile's
// LSE and row dots.  One barrier per tile (tests/test_schedule_model.py
// replays the schedule).  64.5 KiB of LDS and at most 256 VGPRs, so two
// work-groups share a CU.
template <int D, bool CAUSAL, bool PADDED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_fused_kernel(BwdParams p) {
  constexpr int BK = 128, BQ = 32, TQ = BQ * D;
  constexpr int CPR = D / 8, RPI = 64 / CPR;            // 16-byte chunks per row, rows per 1 KiB copy
  constexpr int QCOPIES = BQ / RPI / 4;                 // 1 KiB copies per wave per Q (or dO) tile
  constexpr int VCOPIES = BK / RPI / 4;                 // ... per wave for the block's V rows
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[BK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t qdo_lds[2][2][TQ];  // [buffer][Q, dO]
  __shared__ __attribute__((aligned(16))) float ld_lds[2][2][BQ];         // [buffer][LSE (base 2), row dot]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, li = lane & 31, hi = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int bh_count = p.B * p.Hkv;
  const int bh = blockIdx.x % bh_count;
  const int kt = (int)(blockIdx.x / bh_count);  // causal: the first key blocks carry the most work
  const int b = bh / p.Hkv, hk = bh - b * p.Hkv;
  const int group = p.Hq / p.Hkv;

  const int kv_len = PADDED ? clamp_len(p.kv_seqlens, b, p.Nk) : p.Nk;
  const int kt0 = kt * BK;
  const int diag = p.Nk - p.Nq;
  const size_t kv_base = ((size_t)b * p.Hkv + hk) * (size_t)p.Nk;
  const int key = kt0 + wave_u * 32 + li;  // this lane's key
  const int key_end = kt0 + wave_u * 32 + 32;

  int qt_first = 0;
  if (CAUSAL) qt_first = max(0, kt0 - diag) / BQ;
  const int n_qt = (p.Nq + BQ - 1) / BQ;
  const int per_head = kt0 < kv_len ? max(0, n_qt - qt_first) : 0;
  const int n_it = per_head * group;

  // Copies: lane l of copy c brings row c*RPI + l/CPR, source chunk
  // (l % CPR) ^ swz(row), to LDS position l % CPR of that row.
  const int cp_row = lane / CPR, cp_chunk = lane % CPR;
  auto copy_rows = [&](const uint16_t* src, int row0, int nvalid, int c, uint16_t* dst) {
    const int r = c * RPI + cp_row;
    const int rs = min(row0 + r, nvalid - 1) - row0;  // rows past the valid ones re-read the last
    const int off = (rs * D + ((cp_chunk ^ swz<D>(r)) * 8)) * 2;
    copy16_to_lds(src + (size_t)row0 * D, off, dst + c * 512);
  };
  // Query tile `it`: head hq, rows q0 .. q0 + 31.
  auto tile_of = [&](int it, int& hq, int& q0) {
    hq = hk * group + it / per_head;
    q0 = (qt_first + it % per_head) * BQ;
  };
  auto issue_tile = [&](int it, int buf) {
    int hq, q0;
    tile_of(it, hq, q0);
    const size_t rb = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;
#pragma unroll
    for (int i = 0; i < QCOPIES; ++i) {
      const int c = wave_u * QCOPIES + i;
      copy_rows(p.q + rb * D, q0, p.Nq, c, qdo_lds[buf][0]);
      copy_rows(p.dout + rb * D, q0, p.Nq, c, qdo_lds[buf][1]);
    }
  };
  // Wave 0 loads the tile's LSE (lanes 0..31) and row dots (lanes 32..63).
  float ld_reg = 0.f;
  auto load_ld = [&](int it) {
    int hq, q0;
    tile_of(it, hq, q0);
    const size_t rb = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;
    const int q = q0 + li;
    if (hi == 0) ld_reg = q < p.Nq ? lse_base2(p.lse[rb + q]) : __builtin_inff();
    else ld_reg = q < p.Nq ? p.rowdot[rb + q] : 0.f;
  };

  // B operand of S: lane (li, hi) holds K of key `key`, columns 16*st + 8*hi .. +7
  // (zeros past the sequence's length).
  bf16x8 kf[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
    kf[st] = key < kv_len ? *(const bf16x8*)(p.k + (kv_base + key) * D + 16 * st + 8 * hi) : bf16x8{};
#pragma unroll
  for (int st = 0; st < D / 16; ++st) asm volatile("" : "+v"(kf[st]));

  f32x16 acc_dv[D / 32], acc_dk[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc_dv[db] = acc_dk[db] = f32x16{};

  if (n_it > 0) {
    const uint16_t* vsrc = p.v + kv_base * D;
#pragma unroll
    for (int i = 0; i < VCOPIES; ++i) copy_rows(vsrc, kt0, kv_len, wave_u * VCOPIES + i, v_lds);
    issue_tile(0, 0);
    if (wave_u == 0) load_ld(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (wave_u == 0) ld_lds[0][hi][li] = ld_reg;
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  for (int it = 0; it < n_it; ++it) {
    const int buf = it & 1;
    if (it + 1 < n_it) {
      issue_tile(it + 1, buf ^ 1);
      if (wave_u == 0) load_ld(it + 1);
    }
    int hq_unused, q0;
    tile_of(it, hq_unused, q0);
    const uint16_t* qt = qdo_lds[buf][0];
    const uint16_t* dt = qdo_lds[buf][1];

    // One k-step's fragments at a time (the scheduling barriers keep the
    // compiler from hoisting every read, which would not fit the register
    // budget); the other work-group on the SIMD covers the read latency.
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      const bf16x8 fq = *(const bf16x8*)(qt + tile_off<D>(li, 2 * st + hi));
      const bf16x8 fd = *(const bf16x8*)(dt + tile_off<D>(li, 2 * st + hi));
      const bf16x8 fv = *(const bf16x8*)(v_lds + tile_off<D>(wave_u * 32 + li, 2 * st + hi));
      s = mfma32x32x16(fq, kf[st], s);
      dp = mfma32x32x16(fd, fv, dp);
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane l: key `key`; register r: query q0 + 8(r/4) + 4*hi + r%4.  Tiles
    // whose queries all see every key of the wave skip the per-element mask.
    const bool full = key_end <= kv_len && (!CAUSAL || key_end - 1 <= q0 + diag);
    // P and dS for eight queries (registers 8*mm .. 8*mm+7) at a time, packed
    // to bf16 at once, so only half of them are ever live in float32.
    bf16x8 pf[2], dsf[2];
    auto half = [&](int mm, bool masked) {
      float pv[8], dsv[8];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * mm + jj;
        const float4 l4 = *(const float4*)(&ld_lds[buf][0][8 * j + 4 * hi]);
        const float4 d4 = *(const float4*)(&ld_lds[buf][1][8 * j + 4 * hi]);
        const float lse4[4] = {l4.x, l4.y, l4.z, l4.w}, dr4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 4 * j + x;
          bool vis = true;
          if (masked) {
            const int q = q0 + 8 * j + 4 * hi + x;
            vis = key < kv_len && q < p.Nq;
            if (CAUSAL) vis = vis && key <= q + diag;
          }
          const float pr = vis ? fast_exp2(__builtin_fmaf(s[r], p.scale_log2, -lse4[x])) : 0.f;
          pv[4 * jj + x] = pr;
          dsv[4 * jj + x] = pr * (dp[r] - dr4[x]);
        }
      }
      pf[mm] = pack_bf16x8(pv);
      dsf[mm] = pack_bf16x8(dsv);
    };
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      if (full) half(mm, false);
      else half(mm, true);
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        acc_dv[db] = mfma32x32x16(tr_fragment<D>(dt, 16 * mm, db, lane), pf[mm], acc_dv[db]);
        acc_dk[db] = mfma32x32x16(tr_fragment<D>(qt, 16 * mm, db, lane), dsf[mm], acc_dk[db]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the next tile's copies and LSE/row dots
    if (wave_u == 0 && it + 1 < n_it) ld_lds[buf ^ 1][hi][li] = ld_reg;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  if (key < p.Nk) {
    uint16_t* dvp = p.dv + (kv_base + key) * D;
    uint16_t* dkp = p.dk + (kv_base + key) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        uint2 w;
        w.x = pack_bf16x2(acc_dv[db][4 * g4], acc_dv[db][4 * g4 + 1]);
        w.y = pack_bf16x2(acc_dv[db][4 * g4 + 2], acc_dv[db][4 * g4 + 3]);
        *(uint2*)(dvp + db * 32 + 8 * g4 + 4 * hi) = w;
        w.x = pack_bf16x2(acc_dk[db][4 * g4] * p.scale, acc_dk[db][4 * g4 + 1] * p.scale);
        w.y = pack_bf16x2(acc_dk[db][4 * g4 + 2] * p.scale, acc_dk[db][4 * g4 + 3] * p.scale);
        *(uint2*)(dkp + db * 32 + 8 * g4 + 4 * hi) = w;
      }
  }
}

template <int D, bool CAUSAL, bool PADDED>
static hipError_t launch_bwd_t(const BwdArgs& a) {
  BwdParams p;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k;
  p.v = (const uint16_t*)a.v;
  p.dout = (const uint16_t*)a.dout;
  p.lse = a.lse;
  p.rowdot = a.rowdot;
  p.dq = (uint16_t*)a.dq;
  p.dk = (uint16_t*)a.dk;
  p.dv = (uint16_t*)a.dv;
  p.kv_seqlens = a.kv_seqlens;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk;
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  const long long rows = (long long)a.B * a.Hq * a.Nq;
  if (rows > 0) {
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL(bwd_rowdot_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, a.stream,
                       (const uint16_t*)a.dout, (const uint16_t*)a.o, a.rowdot, rows);
    p.n_tiles = (a.Nq + 127) / 128;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, PADDED>), dim3((unsigned)((long long)p.n_tiles * a.B * a.Hq)),
                       dim3(256), 0, a.stream, p);
  }
  const long long krows = (long long)a.B * a.Hkv * a.Nk;
  if (krows > 0) {
    p.n_tiles = (a.Nk + 127) / 128;
    const dim3 grid((unsigned)((long long)p.n_tiles * a.B * a.Hkv));
    hipLaunchKernelGGL((bwd_dkdv_fused_kernel<D, CAUSAL, PADDED>), grid, dim3(256), 0, a.stream, p);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a) {
  const bool padded = a.kv_seqlens != nullptr;
  if (a.causal) return padded ? launch_bwd_t<D, true, true>(a) : launch_bwd_t<D, true, false>(a);
  return padded ? launch_bwd_t<D, false, true>(a) : launch_bwd_t<D, false, false>(a);
}

hipError_t launch_bwd_bf16(const BwdArgs& a) { return a.d == 128 ? launch_bwd_d<128>(a) : launch_bwd_d<64>(a); }

}  // namespace fa
