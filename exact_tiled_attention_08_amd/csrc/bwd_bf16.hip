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
// Two launches: dQ (one work-group per 128-query block streaming 32-key
// tiles; it also forms the row dots D = dO . O), then dV and dK together (one
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

// Direct global->LDS copy c of a [BN, D] bf16 tile (see the prefill kernels):
// lane l brings row c*RPI + l/CPR of the tensor rows starting at row0, source
// chunk (l % CPR) ^ swz(row), to LDS position l % CPR of that tile row; rows
// at or past nvalid re-read row nvalid - 1 (callers guarantee row0 < nvalid).
template <int D>
__device__ __forceinline__ void copy_tile_rows(const uint16_t* src, int row0, int nvalid, int c, uint16_t* dst,
                                               int lane) {
  constexpr int CPR = D / 8, RPI = 64 / CPR;
  const int r = c * RPI + lane / CPR;
  const int rs = min(row0 + r, nvalid - 1) - row0;
  const int off = (rs * D + (((lane % CPR) ^ swz<D>(r)) * 8)) * 2;
  copy16_to_lds(src + (size_t)row0 * D, off, dst + c * 512);
}

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

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const uint16_t* o;
  const float* lse;
  float* rowdot;  // D_i = dO_i . O_i, written by the dQ kernel, read by the dK/dV kernel
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
// The kernel first forms each of its rows' D = dO . O (and stores it for the
// dK/dV kernel); K and V tiles rotate through two LDS buffers filled by
// direct global->LDS copies one tile ahead, one barrier per tile (the
// schedule of the dK/dV kernel, replayed in tests/test_schedule_model.py).
template <int D, bool CAUSAL, bool PADDED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(BwdParams p) {
  constexpr int BM = 128, BN = 32, TK = BN * D;
  constexpr int RPI = 64 / (D / 8), COPIES = BN / RPI / 4;  // 1 KiB copies per wave per K (or V) tile
  __shared__ __attribute__((aligned(1024))) uint16_t kv_lds[3][2][TK];  // [buffer][K, V]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, li = lane & 31, hi = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int bh_count = p.B * p.Hq;
  const int bh = xcd_grouped_head((int)(blockIdx.x % bh_count), p.B, p.Hq, p.Hkv);  // a KV head's heads on one XCD
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
  const int qrow = q0 + wave_u * 32 + li;
  const bool row_ok = qrow < p.Nq;

  // Q and dO of this lane's row (columns 16*st + 8*hi .. +7), and the row's
  // D = dO . O from the same half rows and the partner lane's.
  bf16x8 qf[D / 16], dof[D / 16];
  float dpart = 0.f;
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    if (row_ok) {
      const size_t off = (qrow_base + qrow) * D + 16 * st + 8 * hi;
      qf[st] = *(const bf16x8*)(p.q + off);
      dof[st] = *(const bf16x8*)(p.dout + off);
      const bf16x8 of = *(const bf16x8*)(p.o + off);
      const uint4 ud = __builtin_bit_cast(uint4, dof[st]), uo = __builtin_bit_cast(uint4, of);
      const unsigned d4[4] = {ud.x, ud.y, ud.z, ud.w}, o4[4] = {uo.x, uo.y, uo.z, uo.w};
#pragma unroll
      for (int x = 0; x < 4; ++x)
        dpart = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d4[x]), __builtin_bit_cast(bf16x2, o4[x]),
                                                dpart, false);
    } else {
      qf[st] = bf16x8{};
      dof[st] = bf16x8{};
    }
  }
  const float drow = pair_sum32(dpart);
  if (row_ok && hi == 0) p.rowdot[qrow_base + qrow] = drow;
  const float lse2 = row_ok ? lse_base2(p.lse[qrow_base + qrow]) : __builtin_inff();

  f32x16 dq_acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq_acc[db] = f32x16{};

  const uint16_t* kg = p.k + kv_base * D;
  const uint16_t* vg = p.v + kv_base * D;
  auto issue = [&](int t, int buf) {
#pragma unroll
    for (int i = 0; i < COPIES; ++i) {
      const int c = wave_u * COPIES + i;
      copy_tile_rows<D>(kg, t * BN, kv_len, c, kv_lds[buf][0], lane);
      copy_tile_rows<D>(vg, t * BN, kv_len, c, kv_lds[buf][1], lane);
    }
  };
  // S^T = K Q^T and dP^T = V dO^T of the tile in buffer `buf`, fragments read
  // one k-step ahead.
  auto sdp = [&](int buf, f32x16& s, f32x16& dp) {
    const uint16_t* kl = kv_lds[buf][0];
    const uint16_t* vl = kv_lds[buf][1];
    s = f32x16{};
    dp = f32x16{};
    bf16x8 fk[2], fv[2];
    fk[0] = *(const bf16x8*)(kl + tile_off<D>(li, hi));
    fv[0] = *(const bf16x8*)(vl + tile_off<D>(li, hi));
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      if (st + 1 < D / 16) {
        fk[(st + 1) & 1] = *(const bf16x8*)(kl + tile_off<D>(li, 2 * (st + 1) + hi));
        fv[(st + 1) & 1] = *(const bf16x8*)(vl + tile_off<D>(li, 2 * (st + 1) + hi));
      }
      s = mfma32x32x16(fk[st & 1], qf[st], s);
      dp = mfma32x32x16(fv[st & 1], dof[st], dp);
    }
  };

  // Software pipeline over 32-key tiles in a ring of three LDS buffers:
  // iteration t starts the copy of tile t+2, computes S and dP of tile t+1
  // (matrix cores) beside the softmax of tile t (vector ALU), then dQ += K^T
  // dS of tile t.  Tile t+1 was copied one iteration earlier and waited for
  // before the barrier that ended it; buffer (t+2) % 3 last held tile t-1,
  // whose last reads were retired before that barrier.  (tests/
  // test_schedule_model.py replays this schedule.)
  f32x16 s_cur = f32x16{}, dp_cur = f32x16{};
  if (n_kt > 0) {
    issue(0, 0);
    if (n_kt > 1) issue(1, 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (n_kt > 0) sdp(0, s_cur, dp_cur);

  int b_cur = 0;  // buffer of tile t
  for (int t = 0; t < n_kt; ++t) {
    const int b_nxt = b_cur == 2 ? 0 : b_cur + 1, b_far = b_nxt == 2 ? 0 : b_nxt + 1;
    if (t + 2 < n_kt) issue(t + 2, b_far);
    // S, dP of tile t+1 (after the last tile: finite data nothing uses).
    f32x16 s_nxt, dp_nxt;
    sdp(b_nxt, s_nxt, dp_nxt);

    // lane l: query qrow; register r: key k0 + 8(r/4) + 4*hi + r%4.  The
    // exponential runs for every element (rows past Nq have LSE +inf, keys
    // past the length read finite rows); tiles that are not all valid and
    // visible to every row of the wave then zero what is not, in a branch of
    // their own so the common path stays one straight-line block.
    const int k0 = t * BN;
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = fast_exp2(__builtin_fmaf(s_cur[r], p.scale_log2, -lse2)) * (dp_cur[r] - drow);
    if (!(k0 + BN <= kv_len && (!CAUSAL || k0 + BN - 1 <= q0 + wave_u * 32 + diag))) {
      asm volatile("");
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        bool vis = key < kv_len;
        if (CAUSAL) vis = vis & (key <= qrow + diag);
        ds[r] = vis ? ds[r] : 0.f;
      }
    }
    bf16x8 dsf[2];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) dsf[mm] = pack_bf16x8(ds + 8 * mm);
    // Key slice mm outermost: consecutive products accumulate into different
    // d-blocks (a product that waits for the previous one's accumulator
    // stalls the matrix core).
    const uint16_t* kl = kv_lds[b_cur][0];
    constexpr int NF = 2 * (D / 32);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int mm = f / (D / 32), db = f % (D / 32);
      dq_acc[db] = mfma32x32x16(tr_fragment<D>(kl, 16 * mm, db, lane), dsf[mm], dq_acc[db]);
    }
    s_cur = s_nxt;
    dp_cur = dp_nxt;
    b_cur = b_nxt;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile t+2's copies
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  if (row_ok) {
    uint16_t* op = p.dq + (qrow_base + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) store_row_bf16x32(op + db * 32, dq_acc[db], p.scale, hi);
  }
}

// ---------------------------------------------------------------------------
// dV and dK in one kernel: 4 waves x 32 keys per work-group (keys on the
// lanes); 32-query tiles of every query head that reads the block.  Per tile
// and wave, four products:
//   S  = Q K^T      (A: Q rows from LDS, B: the wave's K rows, kept in VGPRs)
//   dP = dO V^T     (A: dO rows from LDS, B: the wave's V rows from LDS)
//   P  = 2^(S scale log2(e) - LSE),  dS = P * (dP - D)
//   dV^T += dO^T P  (A: transposed reads of dO),  dK^T += Q^T dS  (A: Q^T)
// The Q and dO tiles rotate through two LDS buffers, filled by direct
// global->LDS copies one tile ahead (rows past the sequence re-read its last
// row: their LSE is +inf, so they carry no weight); waves 0 and 1 stage each
// tile's LSE and row dots.  One barrier per tile (tests/test_schedule_model.py
// replays the schedule).  The per-lane LDS offsets are computed once and the
// (head, query tile) walk advances by counters, so a tile costs no divisions.
// 64.5 KiB of LDS and at most 256 VGPRs, so two work-groups share a CU.
template <int D, bool CAUSAL, bool PADDED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_fused_kernel(BwdParams p) {
  constexpr int BK = 128, BQ = 32, TQ = BQ * D;
  constexpr int RPI = 64 / (D / 8);
  constexpr int QCOPIES = BQ / RPI / 4;  // 1 KiB copies per wave per Q (or dO) tile
  constexpr int VCOPIES = BK / RPI / 4;  // ... per wave for the block's V rows
  // LDS (elements): V rows [0, BK*D); Q, dO of buffer 0; Q, dO of buffer 1.
  constexpr int V_OFF = 0, QDO_OFF = BK * D;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[BK * D + 4 * TQ];
  __shared__ __attribute__((aligned(16))) float ld_lds[2][2][BQ];  // [buffer][LSE (base 2), row dot]
  auto q_off = [](int buf) { return QDO_OFF + 2 * buf * TQ; };
  auto do_off = [](int buf) { return QDO_OFF + (2 * buf + 1) * TQ; };

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

  // Per-lane LDS offsets (elements), computed once; the empty asm keeps the
  // compiler from recomputing them at every use.  Rows of a tile: row li (row 32*wave + li of the V rows),
  // chunk 2*st + hi.  Transposed reads: rows tr_r + 8u, chunk 4*db + tr_cc
  // (rows 16 on share the swizzle).
  int rd[D / 16], vrd[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    rd[st] = tile_off<D>(li, 2 * st + hi);
    vrd[st] = V_OFF + tile_off<D>(wave_u * 32 + li, 2 * st + hi);
  }
  const int tr_r = 4 * hi + ((lane & 15) >> 2), tr_cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  int tro[D / 32][2];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int u = 0; u < 2; ++u) tro[db][u] = tile_off<D>(tr_r + 8 * u, 4 * db + tr_cc) + 4 * (lane & 1);
#pragma unroll
  for (int st = 0; st < D / 16; ++st) asm volatile("" : "+v"(rd[st]), "+v"(vrd[st]));
#pragma unroll
  for (int db = 0; db < D / 32; ++db) asm volatile("" : "+v"(tro[db][0]), "+v"(tro[db][1]));
  auto frag = [&](int base, int off) { return *(const bf16x8*)(lds + base + off); };
  auto tfrag = [&](int base, int mm, int db) {
    return join_bf16x8(lds_read_tr16(lds + base + 16 * mm * D + tro[db][0]),
                       lds_read_tr16(lds + base + 16 * mm * D + tro[db][1]));
  };

  // The query tiles in order: head hq = hk*group + h, tile qt_first .. n_qt-1.
  // (next_h, next_qt) walk them one ahead of the compute.
  int next_h = 0, next_qt = qt_first;
  auto issue_next = [&](int buf) {
    const int hq = hk * group + next_h, q0 = next_qt * BQ;
    const size_t rb = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;
#pragma unroll
    for (int i = 0; i < QCOPIES; ++i) {
      const int c = wave_u * QCOPIES + i;
      copy_tile_rows<D>(p.q + rb * D, q0, p.Nq, c, lds + q_off(buf), lane);
      copy_tile_rows<D>(p.dout + rb * D, q0, p.Nq, c, lds + do_off(buf), lane);
    }
    if (++next_qt == n_qt) {
      next_qt = qt_first;
      ++next_h;
    }
  };
  // The row data of the tile (next_h, next_qt), as stored: even waves load
  // the LSE, odd waves the row dots (a wave-uniform choice), one row per lane
  // (rows past the query count, and the tile after the last one, re-read a
  // valid row).  Waves 0 and 1 put them in LDS after the tile's wait for its
  // copies.  The loaded value is read nowhere before that wait, so no wait
  // the compiler places for it falls inside the tile, where it would also
  // wait for the copies just issued.
  int ld_q = 0;  // row of the lane's loaded value (for the validity test)
  auto ld_load = [&]() {
    const int hq = hk * group + min(next_h, group - 1);
    ld_q = next_qt * BQ + li;
    const float* src = (wave_u & 1) ? p.rowdot : p.lse;
    return src[((size_t)b * p.Hq + hq) * (size_t)p.Nq + min(ld_q, p.Nq - 1)];
  };
  // LDS slot of a tile's row li: the LSE in base 2 (+inf for a row with no
  // visible key or past the query count: every P of the row is then 0), or
  // the row dot (0 past the query count).
  auto ld_store = [&](int buf, float raw) {
    if (wave_u < 2 && hi == 0) {
      const bool ok = ld_q < p.Nq;
      ld_lds[buf][wave_u][li] = wave_u == 0 ? (ok ? lse_base2(raw) : __builtin_inff()) : (ok ? raw : 0.f);
    }
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

  float ld_reg = 0.f;
  if (n_it > 0) {
    const uint16_t* vsrc = p.v + kv_base * D;
#pragma unroll
    for (int i = 0; i < VCOPIES; ++i) copy_tile_rows<D>(vsrc, kt0, kv_len, wave_u * VCOPIES + i, lds + V_OFF, lane);
    ld_reg = ld_load();
    issue_next(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    ld_store(0, ld_reg);
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  int cur_qt = qt_first;  // query tile being computed
  auto tile = [&](int it, int buf) {
    ld_reg = ld_load();
    if (it + 1 < n_it) issue_next(buf ^ 1);
    const int q0 = cur_qt * BQ;
    if (++cur_qt == n_qt) cur_qt = qt_first;
    // Tiles whose queries all see every key of the wave skip the mask.
    const bool masked = !(key_end <= kv_len && (!CAUSAL || key_end - 1 <= q0 + diag));

    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      s = mfma32x32x16(frag(q_off(buf), rd[st]), kf[st], s);
      dp = mfma32x32x16(frag(do_off(buf), rd[st]), frag(0, vrd[st]), dp);
    }
    // lane l: key `key`; register r: query q0 + 8(r/4) + 4*hi + r%4.  P and
    // dS for eight queries (registers 8*mm .. 8*mm+7) at a time, so only
    // half of them are ever live in float32.  The exponential runs for every
    // element (masked-out ones are finite here -- zero K rows, re-read Q rows
    // -- or have LSE +inf); masked tiles then zero what is not visible, in a
    // branch of their own so the common path stays one straight-line block.
    auto half = [&](int mm, float (&pv)[8], float (&dsv)[8]) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * mm + jj;
        const float4 l4 = *(const float4*)(&ld_lds[buf][0][8 * j + 4 * hi]);
        const float4 d4 = *(const float4*)(&ld_lds[buf][1][8 * j + 4 * hi]);
        const float lse4[4] = {l4.x, l4.y, l4.z, l4.w}, dr4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 4 * j + x;
          const float pr = fast_exp2(__builtin_fmaf(s[r], p.scale_log2, -lse4[x]));
          pv[4 * jj + x] = pr;
          dsv[4 * jj + x] = pr * (dp[r] - dr4[x]);
        }
      }
      if (masked) {
        // Element e holds query q0 + 4*hi + c with c = 8*(2mm + e/4) + e%4,
        // visible iff lo <= c < hi_q (lo from the causal diagonal, hi_q from
        // the query count; an empty range for keys past the sequence).  The
        // empty asm keeps this a branch taken by masked tiles only.
        asm volatile("");
        int lo = CAUSAL ? key - diag - 4 * hi - q0 : INT_MIN / 2;
        int hi_q = p.Nq - q0 - 4 * hi;
        if (key >= kv_len) hi_q = lo;
        const unsigned range = (unsigned)(hi_q - lo);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = 8 * (2 * mm + e / 4) + e % 4;
          const bool vis = (unsigned)(c - lo) < range && hi_q > lo;
          pv[e] = vis ? pv[e] : 0.f;
          dsv[e] = vis ? dsv[e] : 0.f;
        }
      }
    };
    auto grads = [&](int mm, bf16x8 pf, bf16x8 dsf) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        acc_dv[db] = mfma32x32x16(tfrag(do_off(buf), mm, db), pf, acc_dv[db]);
        acc_dk[db] = mfma32x32x16(tfrag(q_off(buf), mm, db), dsf, acc_dk[db]);
      }
    };
    float pv[8], dsv[8];
    half(0, pv, dsv);
    const bf16x8 pf0 = pack_bf16x8(pv), dsf0 = pack_bf16x8(dsv);
    // The first half's dV/dK products and the forming of the second half
    // share one straight-line block, so they can overlap.
    grads(0, pf0, dsf0);
    half(1, pv, dsv);
    grads(1, pack_bf16x8(pv), pack_bf16x8(dsv));

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the next tile's copies and LSE/row dots
    if (it + 1 < n_it) ld_store(buf ^ 1, ld_reg);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  for (int it = 0; it < n_it; ++it) tile(it, it & 1);

  if (key < p.Nk) {
    uint16_t* dvp = p.dv + (kv_base + key) * D;
    uint16_t* dkp = p.dk + (kv_base + key) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      store_row_bf16x32(dvp + db * 32, acc_dv[db], 1.f, hi);
      store_row_bf16x32(dkp + db * 32, acc_dk[db], p.scale, hi);
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
  p.o = (const uint16_t*)a.o;
  const long long rows = (long long)a.B * a.Hq * a.Nq;
  if (rows > 0) {  // dQ (and the row dots D the dK/dV kernel reads)
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
