// Backward pass of the fused exact attention for AMD Instinct MI355X (gfx950).
//
// Given Q, K, V, the forward output O and its LSE, and the output gradient
// dO, computes dQ, dK, dV of L = sum(dO * O).  The LSE is what the forward
// returns it for (the CuTe DSL example's docstring: the log-sum-exp is kept
// for training); the algorithm is the FlashAttention-2 backward the pages
// cite: P is recomputed tile by tile from the scores and the LSE, never
// stored, with
//
//   D_i   = dO_i . O_i                       (= sum_j P_ij dP_ij)
//   dP_ij = dO_i . V_j
//   dS_ij = P_ij (dP_ij - D_i)
//   dV_j  = sum_i P_ij dO_i
//   dQ_i  = scale sum_j dS_ij K_j,   dK_j = scale sum_i dS_ij Q_i
//
// Three launches on one stream:
//   prep   D_i and lse_i * log2(e) per query row (memory-bound),
//   dq     query-row outer, like the forward: one wave owns 32 query rows
//          (at d = 192, and up to 128 on grids of at most 256 workgroups of
//          128 rows, two waves, each over half the keys of every tile),
//          K and V tiles stream through LDS, dQ^T = K^T dS^T accumulates in
//          registers,
//   dkdv   key outer: two waves own 32 keys of one kv head (each half of
//          the rows of every query tile; above d = 128 two more, one wave of
//          each pair summing dV and the other dK), the Q and dO tiles of
//          every query row (and every query head of the GQA group) that sees
//          them stream through LDS, dK^T = Q^T dS and dV^T = dO^T P
//          accumulate in registers and the two halves are added at the end.
// Each gradient element is written once by one lane: no atomics, and the
// results do not depend on scheduling.
//
// The MFMA layouts follow the forward kernel: a 32x32x16 accumulator of a
// product whose rows were fed in the sigma order is, converted to 16 bit,
// directly the B operand of the next product over those rows; operands with
// the tile's rows as the contraction come from ds_read_b64_tr_b16.

#include "attn_common.h"

namespace {

constexpr float LOG2E = 1.44269504088896340736f;

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dvec;  // D_i, [B][Hq][Sq]
  float* l2;    // lse_i * log2(e), +inf for rows that see no key, [B][Hq][Sq]
  int B, Sq, Sk, Hq, Hkv;
  int d;        // head size: rows hold d elements; the kernels are built for
                // D >= d, columns past d read as zeros and are not written
  int group, gh, hsub, rows_wg, qtiles, ncols, xcd_cols;  // dq launch (forward plan)
  int off;      // Sk - Sq
  float scale, scale_log2;
};

// ------------------------------------------------------------ prep
// Eight threads per query row, each over 16-byte chunks t, t + 8, ... of the
// row, then a reduction over the eight lanes.  Rows are taken in memory
// order (b, i, h), so consecutive rows are contiguous.
template <int DT, int D>
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(BwdParams p) {
  constexpr int CH = D / 8;  // 16-byte chunks per row
  const int t = threadIdx.x & 7;
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int64_t rows = (int64_t)p.B * p.Sq * p.Hq;
  const bool valid = row < rows;
  float acc = 0.f;
  if (valid) {
    const uint16_t* orow = p.o + row * p.d;
    const uint16_t* drow = p.dout + row * p.d;
    for (int c = t; c < CH && 8 * c < p.d; c += 8) {
      const u32x4 a = *(const u32x4*)(orow + 8 * c);
      const u32x4 g = *(const u32x4*)(drow + 8 * c);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float a0, a1, g0, g1;
        if constexpr (DT == ATTN_DTYPE_BF16) {
          a0 = __uint_as_float(a[w] << 16);
          a1 = __uint_as_float(a[w] & 0xffff0000u);
          g0 = __uint_as_float(g[w] << 16);
          g1 = __uint_as_float(g[w] & 0xffff0000u);
        } else {
          a0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(a[w] & 0xffffu));
          a1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(a[w] >> 16));
          g0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(g[w] & 0xffffu));
          g1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(g[w] >> 16));
        }
        acc = __builtin_fmaf(a0, g0, acc);
        acc = __builtin_fmaf(a1, g1, acc);
      }
    }
  }
  acc += __shfl_xor(acc, 1, 8);
  acc += __shfl_xor(acc, 2, 8);
  acc += __shfl_xor(acc, 4, 8);
  if (valid && t == 0) {
    const int h = (int)(row % p.Hq);
    const int64_t bi = row / p.Hq;
    const int i = (int)(bi % p.Sq);
    const int b = (int)(bi / p.Sq);
    const int64_t at = ((int64_t)b * p.Hq + h) * p.Sq + i;
    const float l = p.lse[at];
    p.dvec[at] = acc;
    p.l2[at] = l > -INFINITY ? l * LOG2E : INFINITY;
  }
}

// ------------------------------------------------------------ dQ
// KH = 2, NWD = 8 (at d = 192): 8 waves, 4 row waves x 2 key halves.  Wave w takes
// the rows of row wave w & 3 and the 32 keys w >> 2 of every tile, so a wave
// holds S and dP of one 32-key block: its Q and dO fragments, dQ sums and
// one key block fit two waves per SIMD, where all 64 keys left one.  The
// second half's dQ sums are added to the first's through LDS at the end.
// With 4 waves and KH = 2 (up to d = 128): 2 row waves x 2 key halves over
// 64-row workgroups (the forward's key-halves plan), twice as many.
template <int DT, int D, bool CAUSAL, int KH, int NWD>
__global__ __launch_bounds__(64 * NWD, D > 128 && KH == 1 ? 1 : 2) void attn_bwd_dq_kernel(
    BwdParams p) {
  using T = Ty<DT>;
  constexpr int CB = D / 32;
  constexpr int KK = D / 16;
  constexpr int TB = 64 * D * 2;
  constexpr int KB = 2 / KH;  // 32-key blocks per wave and tile
  constexpr int NF = 2 * KB;  // 16-key dS fragments per wave and tile
  static_assert(KH == 1 || KH == 2, "one or two key halves");
  static_assert(NWD == 4 * KH || (NWD == 4 && KH == 2 && D <= 128), "4 or 8 waves");
  static_assert(KH == 1 || CB * 16 * 64 * 4 <= TB, "a half's dQ sums fit one tile buffer");
  __shared__ __attribute__((aligned(1024))) char lds_k0[TB], lds_k1[TB], lds_v0[TB], lds_v1[TB];
  ATTN_POISON_LDS_ARRAY(lds_k0);
  ATTN_POISON_LDS_ARRAY(lds_k1);
  ATTN_POISON_LDS_ARRAY(lds_v0);
  ATTN_POISON_LDS_ARRAY(lds_v1);
  ATTN_POISON_LDS_DONE();
  auto kbuf = [&](int n) { return (n & 1) ? (LDS_PTR(char))lds_k1 : (LDS_PTR(char))lds_k0; };
  auto vbuf = [&](int n) { return (n & 1) ? (LDS_PTR(char))lds_v1 : (LDS_PTR(char))lds_v0; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int RW = NWD / KH;  // row waves
  const int wave = wv & (RW - 1);  // row wave
  const int kh = KH == 2 ? wv / RW : 0;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // work decode: the forward's (heaviest row blocks first, XCD-grouped)
  int qt, col;
  {
    const int L = blockIdx.x;
    if (p.xcd_cols > 0) {
      const int xcd = L & 7;
      const int k = L >> 3;
      qt = p.qtiles - 1 - k / p.xcd_cols;
      col = xcd * p.xcd_cols + k % p.xcd_cols;
    } else {
      qt = p.qtiles - 1 - L / p.ncols;
      col = L % p.ncols;
    }
  }
  const int hs = col % p.hsub;
  const int kvh = (col / p.hsub) % p.Hkv;
  const int b = col / (p.hsub * p.Hkv);
  const int hq = kvh * p.group + hs * p.gh + wave % p.gh;
  const int q0wg = qt * p.rows_wg;
  const int q0w = q0wg + (wave / p.gh) * 32;

  const int n_end = block_tiles(q0wg, p.rows_wg, p.Sq, p.Sk, p.off, CAUSAL);
  int n_full = p.Sk / 64;
  if (CAUSAL) {
    const int lim = q0wg + p.off + 1;
    n_full = min(n_full, lim > 0 ? lim / 64 : 0);
  }

  const uint32_t rbkv = (uint32_t)p.Hkv * p.d * 2;
  const char* kslice = (const char*)(p.k + ((int64_t)b * p.Sk * p.Hkv + kvh) * p.d);
  const char* vslice = (const char*)(p.v + ((int64_t)b * p.Sk * p.Hkv + kvh) * p.d);

  // this lane's query row: Q and dO fragments (B operands, d as k)
  const int qi = q0w + l32;
  const bool ok = qi < p.Sq;
  i16x8 qf[KK], dof[KK];
  {
    const int64_t r = ((int64_t)b * p.Sq + (ok ? qi : 0)) * p.Hq + hq;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (ok && kk * 16 + hh * 8 < p.d) {  // columns past d stay zero
        x = *(const u32x4*)(p.q + r * p.d + kk * 16 + hh * 8);
        y = *(const u32x4*)(p.dout + r * p.d + kk * 16 + hh * 8);
      }
      qf[kk] = __builtin_bit_cast(i16x8, x);
      dof[kk] = __builtin_bit_cast(i16x8, y);
    }
  }
  float lse2 = INFINITY, drow = 0.f;
  if (ok) {
    const int64_t at = ((int64_t)b * p.Hq + hq) * p.Sq + qi;
    lse2 = p.l2[at];
    drow = p.dvec[at];
  }
  int lim_row = p.Sk - 1;
  if (CAUSAL) lim_row = min(lim_row, qi + p.off);

  uint32_t rbase[2], tbase[2];
  row_frag_bases(lane, rbase);
  tr_frag_bases(lane, tbase);

  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;

  // the tile loads, spread over 4 waves: with 8 waves the first half's
  // waves load K and the second half's V
  auto load_kv = [&](int n) {
    if (NWD == 4 || kh == 0) load_tile<D>(kslice, rbkv, n, p.Sk, p.d, kbuf(n), wv & 3, lane);
    if (NWD == 4 || kh == 1) load_tile<D>(vslice, rbkv, n, p.Sk, p.d, vbuf(n), wv & 3, lane);
  };
  if (n_end > 0) {
    load_kv(0);
    for (int j = 0; j < n_end; ++j) {
      // tile j has landed (this wave's loads) and every wave is done with
      // tile j - 1, whose buffers now take tile j + 1
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (j + 1 < n_end) load_kv(j + 1);
      // this wave's key rows of the tile: 32 kh KB .. + 32 KB
      LDS_PTR(char) const kt = kbuf(j) + kh * KB * 32 * 64;
      LDS_PTR(char) const vt = vbuf(j) + kh * KB * 32 * 64;
      // S^T = K Q^T and dP^T = V dO^T for the wave's keys of the tile
      // (the fragments of the next step are read during the current one)
      f32x16 S[KB], dP[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          S[kb][r] = 0.f;
          dP[kb][r] = 0.f;
        }
      if constexpr (KH == 2) {
        // one fragment in flight (K for S, then V for dP of the same kk):
        // the registers of two waves per SIMD leave no room for two
        constexpr int NS = 2 * KK;  // steps (kk, S or dP)
        auto rd = [&](int st) { return read_row_frag(st & 1 ? vt : kt, rbase, 0, st >> 1); };
        i16x8 fa = rd(0), fb;
#pragma unroll
        for (int st = 0; st < NS; st += 2) {
          fb = rd(st + 1);
          __builtin_amdgcn_sched_barrier(0);
          S[0] = T::mfma(fa, qf[st >> 1], S[0]);
          if (st + 2 < NS) fa = rd(st + 2);
          __builtin_amdgcn_sched_barrier(0);
          dP[0] = T::mfma(fb, dof[st >> 1], dP[0]);
        }
      } else {
        constexpr int NS = KB * KK;  // steps (kb, kk)
        auto rd = [&](int st, i16x8 (&f)[2]) {
          f[0] = read_row_frag(kt, rbase, st / KK, st % KK);
          f[1] = read_row_frag(vt, rbase, st / KK, st % KK);
        };
        i16x8 fa[2], fb[2];
        rd(0, fa);
#pragma unroll
        for (int st = 0; st < NS; st += 2) {
          rd(st + 1, fb);
          __builtin_amdgcn_sched_barrier(0);
          S[st / KK] = T::mfma(fa[0], qf[st % KK], S[st / KK]);
          dP[st / KK] = T::mfma(fa[1], dof[st % KK], dP[st / KK]);
          if (st + 2 < NS) rd(st + 2, fa);
          __builtin_amdgcn_sched_barrier(0);
          S[(st + 1) / KK] = T::mfma(fb[0], qf[(st + 1) % KK], S[(st + 1) / KK]);
          dP[(st + 1) / KK] = T::mfma(fb[1], dof[(st + 1) % KK], dP[(st + 1) / KK]);
        }
      }
      if (j >= n_full) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int L = lim_row - j * 64 - (kh * KB + kb) * 32 - 8 * hh;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (key_of_reg(r) > L) S[kb][r] = -INFINITY;
        }
      }
      // dS^T = P^T (dP^T - D), rounded to 16 bit: registers 8t'..8t'+7 are
      // keys 16t' + 8hh + 0..7, the B operand of the next product
      i16x8 dsf[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        f32x8 e;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float s = S[f >> 1][8 * (f & 1) + r];
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s, p.scale_log2, -lse2));
          e[r] = pr * (dP[f >> 1][8 * (f & 1) + r] - drow);
        }
        dsf[f] = T::cvt(e);
      }
      // dQ^T += K^T dS^T (fragments one step ahead)
      {
        constexpr int NS = NF * CB;  // steps (f, cb)
        i16x8 fa = read_tr_frag(kt, tbase, 0, 0), fb;
#pragma unroll
        for (int st = 0; st < NS; st += 2) {
          fb = read_tr_frag(kt, tbase, (st + 1) / CB, (st + 1) % CB);
          __builtin_amdgcn_sched_barrier(0);
          acc[st % CB] = T::mfma(fa, dsf[st / CB], acc[st % CB]);
          if (st + 2 < NS) fa = read_tr_frag(kt, tbase, (st + 2) / CB, (st + 2) % CB);
          __builtin_amdgcn_sched_barrier(0);
          acc[(st + 1) % CB] = T::mfma(fb, dsf[(st + 1) / CB], acc[(st + 1) % CB]);
        }
      }
    }
  }

  if constexpr (KH == 2) {
    // the second half's sums go through the tile buffer of its row wave
    // (lane-major, conflict free), once every wave is done with the tiles
    __syncthreads();
    LDS_PTR(float) const xs = (LDS_PTR(float))(wave == 0   ? (LDS_PTR(char))lds_k0
                                               : wave == 1 ? (LDS_PTR(char))lds_k1
                                               : wave == 2 ? (LDS_PTR(char))lds_v0
                                                           : (LDS_PTR(char))lds_v1);
    if (kh == 1) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) xs[(cb * 16 + r) * 64 + lane] = acc[cb][r];
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[cb][r] += xs[(cb * 16 + r) * 64 + lane];
  }

  if (ok) {
    uint16_t* row = p.dq + (((int64_t)b * p.Sq + qi) * p.Hq + hq) * p.d;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x8 x;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] = acc[cb][4 * g + r] * p.scale;
          x[r + 4] = 0.f;
        }
        const i16x8 y = T::cvt(x);
        const u32x2 w = {(unsigned)(uint16_t)y[0] | ((unsigned)(uint16_t)y[1] << 16),
                         (unsigned)(uint16_t)y[2] | ((unsigned)(uint16_t)y[3] << 16)};
        if (cb * 32 + 8 * g + 4 * hh < p.d) *(u32x2*)(row + cb * 32 + 8 * g + 4 * hh) = w;
      }
  }
}

// ------------------------------------------------------------ dK, dV
//
// Workgroup: 8 waves over 32 * KG keys of one (batch, kv head).  Each wave
// owns the 32 keys of its key group kg and, of every 64-row query tile, the
// 32 rows of its row half qh; the dK/dV partial sums of the two row halves
// are added through LDS at the end.  The keys' K and V rows stay in LDS for
// the whole walk (the B operands of S and dP, read as row fragments).  The
// walk covers the query tiles that see any of the keys, for every query
// head of the kv head's group; tile t sits in LDS buffer t % NB (Q and dO
// double-buffered up to d = 192, with the rows' lse * log2(e) and D).
//
// Up to d = 128 (KG = 4, 128 keys): wave w is key group w & 3, row half
// w >> 2, and sums both dK and dV; the two waves of a key group share a SIMD
// (one's softmax beside the other's MFMAs).
//
// Above 128 a wave's dK and dV sums alone would take 2 x (D / 32) x 16
// registers, leaving one wave per SIMD.  There the workgroup has 2 key groups
// (64 keys) x 2 row halves x 2 roles: a dV wave computes S, P and
// dV^T += dO^T P; a dK wave computes S, dP, dS and dK^T += Q^T dS.  S is
// computed by both (5 products per row block and key group instead of 4),
// but each wave holds one set of sums, so two waves share each SIMD again.
// At 256 there is one Q/dO buffer (K and V of 64 keys plus two Q/dO buffers
// would take 192 KiB of the CU's 160): the next tile is then loaded after
// the current one has been used, behind a second barrier.
template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv_kernel(BwdParams p) {
  using T = Ty<DT>;
  constexpr int CB = D / 32;
  constexpr int KK = D / 16;
  constexpr int TB = 64 * D * 2;
  constexpr bool ROLES = D > 128;      // a wave sums dK or dV, not both
  constexpr int KG = ROLES ? 2 : 4;    // key groups of 32 keys
  constexpr int NR = ROLES ? 2 : 1;    // roles per key group and row half
  constexpr int KT = KG / 2;           // 64-key tiles of K (and of V)
  constexpr int NB = D > 192 ? 1 : 2;  // Q/dO tile buffers
  constexpr int LW = KG * NR;          // waves per row half
  constexpr int VW = 4 / LW;           // 16-row load slices per wave of a 64-row tile
  static_assert(2 * LW == 8, "eight waves");
  __shared__ __attribute__((aligned(1024))) char lds_q0[TB], lds_q1[NB > 1 ? TB : 16],
      lds_o0[TB], lds_o1[NB > 1 ? TB : 16];
  __shared__ __attribute__((aligned(1024))) char lds_k[KT][TB], lds_v[KT][TB];
  __shared__ __attribute__((aligned(256))) float lds_l2[NB][64], lds_d[NB][64];
  ATTN_POISON_LDS_ARRAY(lds_q0);
  ATTN_POISON_LDS_ARRAY(lds_q1);
  ATTN_POISON_LDS_ARRAY(lds_o0);
  ATTN_POISON_LDS_ARRAY(lds_o1);
  ATTN_POISON_LDS_ARRAY(lds_k);
  ATTN_POISON_LDS_ARRAY(lds_v);
  ATTN_POISON_LDS_ARRAY(lds_l2);
  ATTN_POISON_LDS_ARRAY(lds_d);
  ATTN_POISON_LDS_DONE();
  // a wave's dK (or dV) partial sums, CB x 16 floats per lane, fill exactly
  // one tile buffer
  static_assert(CB * 16 * 64 * 4 == TB, "reduction area = tile area");
  auto qbuf = [&](int n) {
    return (NB > 1 && (n & 1)) ? (LDS_PTR(char))lds_q1 : (LDS_PTR(char))lds_q0;
  };
  auto obuf = [&](int n) {
    return (NB > 1 && (n & 1)) ? (LDS_PTR(char))lds_o1 : (LDS_PTR(char))lds_o0;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave % KG;          // key group
  const int qh = (wave / KG) & 1;    // row half of each query tile
  const int role = wave / (2 * KG);  // with roles: 0 sums dV, 1 sums dK
  const int lw = kg + KG * role;     // the wave's place among its row half's
  // a 64-row tile loaded by the LW waves of one row half: each takes VW of
  // the four 16-row slices of the shared tile loader
  auto load64 = [&](const char* slice, uint32_t row_bytes, int n, int nrows, LDS_PTR(char) dst) {
#pragma unroll
    for (int s = 0; s < VW; ++s) load_tile<D>(slice, row_bytes, n, nrows, p.d, dst, lw * VW + s, lane);
  };
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // key blocks in order (the first ones see the most query rows when causal)
  const int ncol = p.B * p.Hkv;
  const int kblk = blockIdx.x / ncol;
  const int col = blockIdx.x % ncol;
  const int b = col / p.Hkv;
  const int kvh = col % p.Hkv;
  const int k0 = kblk * 32 * KG;
  const int kj = k0 + kg * 32 + l32;  // this lane's key
  const bool kok = kj < p.Sk;

  // K rows (row half 0) and V rows (row half 1) of the block's 32 * KG keys
  // into LDS, as KT 64-row tiles each; a tile wholly past Sk is zeroed instead
  {
    const uint32_t rbk = (uint32_t)p.Hkv * p.d * 2;
    const char* slice =
        (const char*)((qh == 0 ? p.k : p.v) + ((int64_t)b * p.Sk * p.Hkv + kvh) * p.d);
#pragma unroll
    for (int i = 0; i < KT; ++i) {
      LDS_PTR(char) const dst = (LDS_PTR(char))(qh == 0 ? lds_k[i] : lds_v[i]);
      if (k0 + 64 * i < p.Sk) {
        load64(slice, rbk, KT * kblk + i, p.Sk, dst);
      } else {
        LDS_PTR(u32x4) z = (LDS_PTR(u32x4))dst;
        for (int e = lw * 64 + lane; e < TB / 16; e += LW * 64) z[e] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
  }

  // query tiles that see a key of the block: i + off >= k0 when causal
  const int nqt = (p.Sq + 63) / 64;
  int qt0 = 0;
  if (CAUSAL) {
    const int first = k0 - p.off;
    qt0 = first > 0 ? first / 64 : 0;
  }
  const int per_head = nqt > qt0 ? nqt - qt0 : 0;
  const int steps = per_head * p.group;
  const uint32_t rbq = (uint32_t)p.Hq * p.d * 2;

  // tile t: Q by row half 0's waves, dO by row half 1's, and the 64 rows'
  // lse * log2(e) and D (the first wave of each), rows clamped to Sq - 1
  // (rows past Sq are masked below)
  // walk position of the next tile to load: query head kvh * group + nh,
  // tile qt0 + nq (counters, not divisions: the scalar unit is busy enough)
  int nh = 0, nq = 0;
  auto issue = [&](int t) {
    const int h = kvh * p.group + nh;
    const int qt = qt0 + nq;
    const int64_t head0 = (int64_t)b * p.Sq * p.Hq + h;
    load64((const char*)((qh == 0 ? p.q : p.dout) + head0 * p.d), rbq, qt, p.Sq,
           qh == 0 ? qbuf(t) : obuf(t));
    if (lw == 0) {
      const float* src = (qh == 0 ? p.l2 : p.dvec) + ((int64_t)b * p.Hq + h) * p.Sq;
      const uint32_t r = (uint32_t)min(qt * 64 + lane, p.Sq - 1);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, p.Sq * 4, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (LDS_PTR(void))(qh == 0 ? &lds_l2[t % NB][0] : &lds_d[t % NB][0]), 4, r * 4, 0,
          0, 0);
    }
  };
  // the next tile's loads: into the other buffer while this tile is
  // computed (two buffers), or after every wave is done with the one buffer
  auto next = [&](int t) {
    if (++nq == per_head) {
      nq = 0;
      ++nh;
    }
    issue(t + 1);
  };

  uint32_t rbase[2], tbase[2], kbase[2];
  row_frag_bases(lane, rbase);
  tr_frag_bases(lane, tbase);
  {
    // row fragments of the keys in natural order: lane l32 reads key row
    // 32 (kg & 1) + l32 of K (V) tile kg >> 1, so its S and dP column is key kj
    const int sw = (l32 >> 2) & 3;
#pragma unroll
    for (int par = 0; par < 2; ++par)
      kbase[par] = (uint32_t)(l32 * 64 + (((2 * par + hh) ^ sw) << 4));
  }
  LDS_PTR(char) const ktile = (LDS_PTR(char))lds_k[kg >> 1];
  LDS_PTR(char) const vtile = (LDS_PTR(char))lds_v[kg >> 1];

  if (steps > 0) issue(0);

  // The walk, the row-half reduction and the stores of one kind of wave:
  // M = 0 sums dV, 1 sums dK, 2 both.  Only the sums a wave keeps are
  // declared in its instance, so a role's registers hold one set.
  auto run = [&](auto mode) {
    constexpr int M = decltype(mode)::value;
    constexpr bool DV = M != 1;
    constexpr bool DK = M != 0;
    f32x16 adk[DK ? CB : 1], adv[DV ? CB : 1];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (DK) adk[cb][r] = 0.f;
        if constexpr (DV) adv[cb][r] = 0.f;
      }

    // tile t's contributions of the wave's 32 query rows to its 32 keys
    auto body = [&](int t, int qt) {
      const int i0 = qt * 64 + 32 * qh;  // first query row of this wave
      // rows that see none of the wave's keys, or lie past Sq: nothing to add
      if (i0 >= p.Sq || (CAUSAL && i0 + 31 + p.off < k0 + 32 * kg)) return;
      LDS_PTR(char) const qtile = qbuf(t);
      LDS_PTR(char) const otile = obuf(t);
      LDS_PTR(const float) const l2t = (LDS_PTR(const float)) & lds_l2[t % NB][0];
      LDS_PTR(const float) const dtt = (LDS_PTR(const float)) & lds_d[t % NB][0];
      // rows need masking: a causal row that does not see every key of the
      // wave, or a row past Sq
      const int kmax = k0 + 32 * kg + 31;
      const bool edge = (CAUSAL && i0 + p.off < kmax) || i0 + 32 > p.Sq;
      // S = Q K^T and dP = dO V^T: rows = the wave's 32 query rows in the
      // sigma order, columns = its 32 keys (lane)
      f32x16 S, dP;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        S[r] = 0.f;
        dP[r] = 0.f;
      }
      {
        // fragments of step kk + 1 are read while the MFMAs of step kk run
        auto rd = [&](int kk, i16x8 (&f)[4]) {
          const uint32_t ko = row_frag_off(kbase, kg & 1, kk);
          f[0] = read_row_frag(qtile, rbase, qh, kk);
          f[1] = *(LDS_PTR(const i16x8))(ktile + ko);
          if constexpr (DK) {
            f[2] = read_row_frag(otile, rbase, qh, kk);
            f[3] = *(LDS_PTR(const i16x8))(vtile + ko);
          }
        };
        i16x8 fa[4], fb[4];
        rd(0, fa);
#pragma unroll
        for (int kk = 0; kk < KK; kk += 2) {
          rd(kk + 1, fb);
          __builtin_amdgcn_sched_barrier(0);
          S = T::mfma(fa[0], fa[1], S);
          if constexpr (DK) dP = T::mfma(fa[2], fa[3], dP);
          if (kk + 2 < KK) rd(kk + 2, fa);
          __builtin_amdgcn_sched_barrier(0);
          S = T::mfma(fb[0], fb[1], S);
          if constexpr (DK) dP = T::mfma(fb[2], fb[3], dP);
        }
      }
      // register r holds query row 32 qh + key_of_reg(r) + 8 hh of the tile;
      // registers 4g .. 4g+3 are 4 consecutive rows
      i16x8 pf[2], dsf[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        f32x8 pe, de;
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          const int g = 2 * f + g2;
          const int row0 = 32 * qh + key_of_reg(4 * g) + 8 * hh;
          const f32x4 l4 = *(LDS_PTR(const f32x4))(l2t + row0);
          f32x4 d4 = {0.f, 0.f, 0.f, 0.f};
          if constexpr (DK) d4 = *(LDS_PTR(const f32x4))(dtt + row0);
#pragma unroll
          for (int r3 = 0; r3 < 4; ++r3) {
            const int r = 4 * g + r3;
            const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], p.scale_log2, -l4[r3]));
            pe[4 * g2 + r3] = pr;
            de[4 * g2 + r3] = DK ? pr * (dP[r] - d4[r3]) : 0.f;
          }
        }
        // masked rows and keys, in one branch per 8 scores (a test per score
        // would cut the body into a branch per score); the empty volatile asm
        // keeps it a branch, so that tiles without masked scores skip the
        // compares instead of running them under a select
        if (edge) {
          asm volatile("" ::: "memory");
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int qi = qt * 64 + 32 * qh + key_of_reg(4 * (2 * f + e / 4)) + 8 * hh + e % 4;
            if (qi >= p.Sq || (CAUSAL && kj > qi + p.off)) {
              pe[e] = 0.f;
              de[e] = 0.f;
            }
          }
        }
        if constexpr (DV) pf[f] = T::cvt(pe);
        if constexpr (DK) dsf[f] = T::cvt(de);
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the 32 rows (two 16-row
      // steps); the fragments of the next step are read during the current one
      {
        constexpr int NS = 2 * CB;
        auto rd = [&](int st, i16x8 (&f)[2]) {
          if constexpr (DV) f[0] = read_tr_frag(otile, tbase, 2 * qh + st / CB, st % CB);
          if constexpr (DK) f[1] = read_tr_frag(qtile, tbase, 2 * qh + st / CB, st % CB);
        };
        i16x8 fa[2], fb[2];
        rd(0, fa);
#pragma unroll
        for (int st = 0; st < NS; st += 2) {
          rd(st + 1, fb);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (DV) adv[st % CB] = T::mfma(fa[0], pf[st / CB], adv[st % CB]);
          if constexpr (DK) adk[st % CB] = T::mfma(fa[1], dsf[st / CB], adk[st % CB]);
          if (st + 2 < NS) rd(st + 2, fa);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (DV)
            adv[(st + 1) % CB] = T::mfma(fb[0], pf[(st + 1) / CB], adv[(st + 1) % CB]);
          if constexpr (DK)
            adk[(st + 1) % CB] = T::mfma(fb[1], dsf[(st + 1) / CB], adk[(st + 1) % CB]);
        }
      }
    };

    int cq = 0;  // tile index within its head of the tile being computed
    for (int t = 0; t < steps; ++t) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (NB > 1 && t + 1 < steps) next(t);
      body(t, qt0 + cq);
      if (++cq == per_head) cq = 0;
      if (NB == 1 && t + 1 < steps) {
        __syncthreads();
        next(t);
      }
    }

    // add the row halves: the waves of row half 1 hand their sums to those
    // of row half 0 through LDS (lane-contiguous 16-byte slots).  Both sums
    // (KG = 4): dK into the K/V area, dV into the Q/dO area.  Roles: one
    // area per key group and role, K and V (dV of key groups 0, 1), then Q
    // and dO (dK).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    LDS_PTR(char) red_k;
    LDS_PTR(char) red_v;
    if constexpr (M == 2) {
      red_k = (LDS_PTR(char))(kg < KT ? lds_k[kg % KT] : lds_v[kg % KT]);
      red_v = kg < KT    ? (kg == 0 ? (LDS_PTR(char))lds_q0 : (LDS_PTR(char))lds_q1)
              : kg == KT ? (LDS_PTR(char))lds_o0
                         : (LDS_PTR(char))lds_o1;
    } else {
      static_assert(KT == 1, "roles: one K and one V tile");
      const int slot = kg + 2 * M;
      LDS_PTR(char) const area = slot == 0   ? (LDS_PTR(char))lds_k[0]
                                 : slot == 1 ? (LDS_PTR(char))lds_v[0]
                                 : slot == 2 ? (LDS_PTR(char))lds_q0
                                             : (LDS_PTR(char))lds_o0;
      red_k = area;
      red_v = area;
    }
    if (qh == 1) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t o = (uint32_t)(((cb * 4 + g) * 64 + lane) * 16);
          if constexpr (DK)
            *(LDS_PTR(f32x4))(red_k + o) = (f32x4){adk[cb][4 * g], adk[cb][4 * g + 1],
                                                   adk[cb][4 * g + 2], adk[cb][4 * g + 3]};
          if constexpr (DV)
            *(LDS_PTR(f32x4))(red_v + o) = (f32x4){adv[cb][4 * g], adv[cb][4 * g + 1],
                                                   adv[cb][4 * g + 2], adv[cb][4 * g + 3]};
        }
    }
    __syncthreads();
    if (qh == 0 && kok) {
      const int64_t r = ((int64_t)b * p.Sk + kj) * p.Hkv + kvh;
      uint16_t* dkrow = p.dk + r * p.d;
      uint16_t* dvrow = p.dv + r * p.d;
      auto pack = [](const i16x8& x) {
        return (u32x2){(unsigned)(uint16_t)x[0] | ((unsigned)(uint16_t)x[1] << 16),
                       (unsigned)(uint16_t)x[2] | ((unsigned)(uint16_t)x[3] << 16)};
      };
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t o = (uint32_t)(((cb * 4 + g) * 64 + lane) * 16);
          const bool col_ok = cb * 32 + 8 * g + 4 * hh < p.d;
          if constexpr (DK) {
            const f32x4 ok = *(LDS_PTR(const f32x4))(red_k + o);
            f32x8 x;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              x[r4] = (adk[cb][4 * g + r4] + ok[r4]) * p.scale;
              x[r4 + 4] = 0.f;
            }
            const u32x2 wk = pack(T::cvt(x));
            if (col_ok) *(u32x2*)(dkrow + cb * 32 + 8 * g + 4 * hh) = wk;
          }
          if constexpr (DV) {
            const f32x4 ov = *(LDS_PTR(const f32x4))(red_v + o);
            f32x8 y;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              y[r4] = adv[cb][4 * g + r4] + ov[r4];
              y[r4 + 4] = 0.f;
            }
            const u32x2 wv = pack(T::cvt(y));
            if (col_ok) *(u32x2*)(dvrow + cb * 32 + 8 * g + 4 * hh) = wv;
          }
        }
    }
  };

  if constexpr (ROLES) {
    if (role == 0)
      run(std::integral_constant<int, 0>{});
    else
      run(std::integral_constant<int, 1>{});
  } else {
    run(std::integral_constant<int, 2>{});
  }
}

// ------------------------------------------------------------ host side
attn_status validate_bwd(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                         int Sq, int Sk, int Hq, int Hkv, int d, float scale, int causal,
                         int dtype) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_INVALID_ARG;
  if (!sizes_ok(B, Sq, Sk, Hq, Hkv) || d < 1) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout |
       (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv) & 15u)
    return ATTN_ERR_INVALID_ARG;
  if (((uintptr_t)lse) & 3u) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_DTYPE_F16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED;
  // any multiple of 8 up to 256, padded to 32, 64, 96, 128, 192 or 256
  if (!head_size_ok(d)) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)Sq + Sk >= (1ll << 30)) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)Hq * d * 2 * 64 >= (1ll << 31)) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * Sq * Hq >= (1ll << 31) || (int64_t)B * Sk * Hkv >= (1ll << 31))
    return ATTN_ERR_INVALID_ARG;
  if ((int64_t)Sq * 4 >= (1ll << 31)) return ATTN_ERR_INVALID_ARG;
  const Plan pl = make_plan(B, Sq, Sk, Hq, Hkv, d, causal);
  if (pl.grid <= 0) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

size_t bwd_workspace_bytes(int B, int Sq, int Hq) {
  const size_t n = (size_t)B * Hq * Sq;
  return 2 * ((n * 4 + 255) & ~(size_t)255);
}

template <int DT, int D, bool CAUSAL>
hipError_t launch_bwd_t(const Plan& pl, const BwdParams& p, hipStream_t st) {
  const long long rows = (long long)p.B * p.Sq * p.Hq;
  hipLaunchKernelGGL((attn_bwd_prep_kernel<DT, D>), dim3((unsigned)((rows + 31) / 32)), dim3(256),
                     0, st, p);
  // dQ: key halves (two waves over the same rows, each over half the keys
  // of every tile): at d = 192 8 waves (two per SIMD); up to 128, when the
  // grid leaves each CU at most one workgroup, the forward's key-halves plan
  // (64-row workgroups of 4 waves, twice as many); 4 waves otherwise (one per
  // SIMD at 256)
  if constexpr (D == 192) {
    hipLaunchKernelGGL((attn_bwd_dq_kernel<DT, D, CAUSAL, 2, 8>), dim3(pl.grid), dim3(512), 0, st,
                       p);
  } else {
    const Plan kp = D <= 128 && pl.grid <= 256
                        ? make_plan(p.B, p.Sq, p.Sk, p.Hq, p.Hkv, p.d, CAUSAL, 2, 4)
                        : Plan{};
    bool launched = false;
    if constexpr (D <= 128) {
      if (kp.grid > 0) {
        BwdParams pq = p;
        pq.gh = kp.gh;
        pq.hsub = pq.group / kp.gh;
        pq.rows_wg = kp.rows_wg;
        pq.qtiles = kp.qtiles;
        pq.ncols = kp.ncols;
        pq.xcd_cols = kp.xcd_cols;
        hipLaunchKernelGGL((attn_bwd_dq_kernel<DT, D, CAUSAL, 2, 4>), dim3(kp.grid), dim3(256), 0,
                           st, pq);
        launched = true;
      }
    }
    if (!launched) {
      hipLaunchKernelGGL((attn_bwd_dq_kernel<DT, D, CAUSAL, 1, 4>), dim3(pl.grid), dim3(256), 0,
                         st, p);
    }
  }
  // 8 waves over 32 keys per key group: 4 groups up to d = 128, 2 above
  constexpr int KG = D > 128 ? 2 : 4;
  const long long kgrid = (long long)p.B * p.Hkv * ((p.Sk + 32 * KG - 1) / (32 * KG));
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DT, D, CAUSAL>), dim3((unsigned)kgrid), dim3(512), 0,
                     st, p);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_bwd_c(bool causal, const Plan& pl, const BwdParams& p, hipStream_t st) {
  return causal ? launch_bwd_t<DT, D, true>(pl, p, st) : launch_bwd_t<DT, D, false>(pl, p, st);
}

template <int DT>
hipError_t launch_bwd_d(int d, bool causal, const Plan& pl, const BwdParams& p, hipStream_t st) {
  switch (padded_head(d)) {
    case 32: return launch_bwd_c<DT, 32>(causal, pl, p, st);
    case 64: return launch_bwd_c<DT, 64>(causal, pl, p, st);
    case 96: return launch_bwd_c<DT, 96>(causal, pl, p, st);
    case 128: return launch_bwd_c<DT, 128>(causal, pl, p, st);
    case 192: return launch_bwd_c<DT, 192>(causal, pl, p, st);
    default: return launch_bwd_c<DT, 256>(causal, pl, p, st);
  }
}

}  // namespace

extern "C" {

attn_status attn_bwd_check(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int B, int Sq, int Sk, int Hq, int Hkv, int d, float scale,
                           int causal, int dtype) {
  return validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Sq, Sk, Hq, Hkv, d, scale, causal,
                      dtype);
}

attn_status attn_bwd_workspace(int B, int Sq, int Hq, size_t* bytes) {
  if (bytes == nullptr || B < 1 || Sq < 1 || Hq < 1) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * Sq * Hq >= (1ll << 31)) return ATTN_ERR_INVALID_ARG;
  *bytes = bwd_workspace_bytes(B, Sq, Hq);
  return ATTN_OK;
}

}  // extern "C"

namespace {

// The three launches for causal offset `off` (query i sees key j <= i + off;
// Sk - Sq for attn_bwd), after validation.
attn_status run_bwd(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                    int Sq, int Sk, int Hq, int Hkv, int d, float scale, int causal, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream, int off) {
  const size_t need = bwd_workspace_bytes(B, Sq, Hq);
  if (workspace == nullptr || ((uintptr_t)workspace & 255u) || workspace_bytes < need)
    return ATTN_ERR_INVALID_ARG;
  const Plan pl = make_plan(B, Sq, Sk, Hq, Hkv, d, causal);
  BwdParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (const uint16_t*)o;
  p.dout = (const uint16_t*)dout;
  p.lse = lse;
  p.dq = (uint16_t*)dq;
  p.dk = (uint16_t*)dk;
  p.dv = (uint16_t*)dv;
  p.dvec = (float*)workspace;
  p.l2 = (float*)((char*)workspace + need / 2);
  p.B = B;
  p.Sq = Sq;
  p.Sk = Sk;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.d = d;
  p.group = Hq / Hkv;
  p.gh = pl.gh;
  p.hsub = p.group / pl.gh;
  p.rows_wg = pl.rows_wg;
  p.qtiles = pl.qtiles;
  p.ncols = pl.ncols;
  p.xcd_cols = pl.xcd_cols;
  p.off = off;
  p.scale = scale;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = dtype == ATTN_DTYPE_BF16 ? launch_bwd_d<ATTN_DTYPE_BF16>(d, causal != 0, pl, p, hs)
                                          : launch_bwd_d<ATTN_DTYPE_F16>(d, causal != 0, pl, p, hs);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                     int Sq, int Sk, int Hq, int Hkv, int d, float scale, int causal, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  attn_status st = validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Sq, Sk, Hq, Hkv, d, scale,
                                causal, dtype);
  if (st != ATTN_OK) return st;
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Sq, Sk, Hq, Hkv, d, scale, causal, dtype,
                 workspace, workspace_bytes, stream, Sk - Sq);
}

attn_status attn_bwd_causal_offset_check(const void* q, const void* k, const void* v,
                                         const void* o, const float* lse, const void* dout,
                                         void* dq, void* dk, void* dv, int B, int Sq, int Sk,
                                         int Hq, int Hkv, int d, float scale,
                                         long long causal_offset, int dtype) {
  attn_status st = validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Sq, Sk, Hq, Hkv, d, scale,
                                1, dtype);
  if (st != ATTN_OK) return st;
  if (causal_offset <= -(1ll << 30) || causal_offset >= (1ll << 30)) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

attn_status attn_bwd_causal_offset(const void* q, const void* k, const void* v, const void* o,
                                   const float* lse, const void* dout, void* dq, void* dk,
                                   void* dv, int B, int Sq, int Sk, int Hq, int Hkv, int d,
                                   float scale, long long causal_offset, int dtype,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  attn_status st = attn_bwd_causal_offset_check(q, k, v, o, lse, dout, dq, dk, dv, B, Sq, Sk, Hq,
                                                Hkv, d, scale, causal_offset, dtype);
  if (st != ATTN_OK) return st;
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Sq, Sk, Hq, Hkv, d, scale, 1, dtype,
                 workspace, workspace_bytes, stream, (int)causal_offset);
}

}  // extern "C"
