// Decode-shaped attention forward for AMD Instinct MI355X (gfx950): a few new
// query rows per sequence (g * Sq <= 128 rows per kv head, g = Hq / Hkv)
// over a long K/V cache.
//
// The MiniPaged-Qwen page (section 19) sets decode apart from prefill: the
// query side has almost no parallelism and the work becomes reading the K/V
// cache.  The computation is the forward's (online softmax over K/V tiles,
// personal-notes page section "Online Softmax"), mapped for that regime:
//
// * All g * Sq query rows of one (batch, kv head) -- every query head of the
//   GQA group and every new token -- are the 32 rows of ONE wave: row r is
//   query head h0 + r / Sq, token r % Sq.  The prefill kernel would give each
//   query head its own 32-row wave, mostly empty.  More than 32 such rows
//   are cut into 32-row groups, each a workgroup of its own over the same
//   keys (placed on one XCD, so that the K/V tiles are read from HBM once).
// * The DEC_WAVES (4) waves of a workgroup walk different 32-key tiles of the
//   key range (tile w, w + 4, ...), each with its own softmax state, and the
//   states are merged through LDS at the end (the online-softmax rescale).
//   A key range can further be cut into pieces over workgroups, merged by
//   the merge kernel, when (batch, kv head) pairs are too few to fill the GPU.
// * The work is bound by reading K and V: K rows go straight from global
//   memory into registers as the A operand of S^T = K Q^T (lane l loads key
//   row sigma(l & 31)); V tiles go to LDS by buffer DMA for the transposed
//   reads of O^T += V^T P^T.  Each wave keeps the next tile's K and V in
//   flight while it computes the current one; two workgroups per CU.
//
// Rounding and normalisation follow the prefill kernel: P rounded to the
// input type before P V (fp16 as hi + lo), O normalised by the sum of the
// rounded P, LSE from the fp32 sum (bf16) or the hi + lo sum (fp16).

#include "attn_common.h"

namespace {

constexpr int DBC = 32;                    // keys per tile
constexpr float DEC_RESCALE_TAU = 8.0f;    // lazy max update, as the prefill kernel

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(DEC_WAVES * 64, D > 128 ? 1 : 8 / DEC_WAVES) void attn_decode_kernel(
    DecodeArgs p) {
  using T = Ty<DT>;
  constexpr int CB = D / 32;
  constexpr int KK = D / 16;
  constexpr int VBLK = DBC * 64;           // bytes per 32-column block of a V tile
  constexpr int VTB = DBC * D * 2;         // bytes per V tile
  constexpr int NW = DEC_WAVES;
  // per wave: two V tile stages; reused at the end for the merge (NW x 32
  // rows x D floats = exactly the same size)
  __shared__ __attribute__((aligned(1024))) char lds_v[NW][2][VTB];
  __shared__ float lds_m[NW][32], lds_lr[NW][32], lds_lf[NW][32];
  ATTN_POISON_LDS_ARRAY(lds_v);
  ATTN_POISON_LDS_ARRAY(lds_m);
  ATTN_POISON_LDS_ARRAY(lds_lr);
  ATTN_POISON_LDS_ARRAY(lds_lf);
  ATTN_POISON_LDS_DONE();
  static_assert(NW * 2 * VTB == NW * 32 * D * 4, "merge area = tile area");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // workgroup -> (piece, batch, kv head, row group); with several row
  // groups, those of one (batch, kv head) sit 8 ids apart (one XCD)
  const int piece = blockIdx.x / p.ucols;
  const int u = blockIdx.x % p.ucols;
  int col = u, rg = 0;
  if (p.rgroups > 1) {
    const int chunk = 8 * p.rgroups;
    col = (u / chunk) * 8 + u % 8;
    rg = (u % chunk) / 8;
    if (col >= p.B * p.Hkv) return;  // padding of the last chunk
  }
  const int b = col / p.Hkv;
  const int kvh = col % p.Hkv;
  const int g = p.Hq / p.Hkv;
  // this workgroup's query rows: rows 32 rg .. 32 rg + M - 1 of the
  // g * Sq rows of the kv head (row R is head kvh * g + R / Sq, token R % Sq)
  const int r0g = 32 * rg;
  const int M = min(32, g * p.Sq - r0g);
  // keys of this sequence (paged cache: its own length, at most Sk, which
  // the host keeps within the block table)
  int Sk = p.Sk;
  if (p.seqlens != nullptr) Sk = max(0, min(p.seqlens[b], p.Sk));

  // this lane's query row
  const int r = l32;
  const bool rok = r < M;
  const int hq = kvh * g + (rok ? (r0g + r) / p.Sq : 0);
  const int qi = rok ? (r0g + r) % p.Sq : 0;
  i16x8 qf[KK];
  {
    const uint16_t* qrow = p.q + (int64_t)b * p.q_sb + (int64_t)qi * p.q_ss + (int64_t)hq * p.q_sh;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};  // columns past d stay zero
      if (rok && kk * 16 + hh * 8 < p.d) x = *(const u32x4*)(qrow + kk * 16 + hh * 8);
      qf[kk] = __builtin_bit_cast(i16x8, x);
    }
  }
  // keys this row sees: j < Sk, and j <= qi + off when causal (off = Sk - Sq
  // for the last Sq positions of a sequence, or the caller's offset)
  const int off = p.seqlens != nullptr ? Sk - p.Sq : p.off;
  int lim = Sk - 1;
  if (CAUSAL) lim = min(lim, qi + off);
  if (!rok) lim = -1;

  // the piece's tiles [t_lo, t_hi); this wave takes t_lo + wave, + NW, ...
  const int ntiles = (Sk + DBC - 1) / DBC;
  const int t_lo = piece * p.piece_tiles;
  const int t_hi = min(ntiles, t_lo + p.piece_tiles);
  // last key seen by any row (tiles past it are skipped): the last query
  // row's limit when causal
  int last_key = Sk - 1;
  if (CAUSAL) last_key = min(last_key, p.Sq - 1 + off);
  const int t_end = last_key >= 0 ? min(t_hi, last_key / DBC + 1) : 0;

  const bool paged = p.block_table != nullptr;
  const char* kbase =
      (const char*)(p.k + (paged ? 0 : (int64_t)b * p.k_sb) + (int64_t)kvh * p.k_sh);
  const char* vbase =
      (const char*)(p.v + (paged ? 0 : (int64_t)b * p.v_sb) + (int64_t)kvh * p.v_sh);
  const uint32_t rbk = (uint32_t)(p.k_ss * 2);
  const uint32_t rbv = (uint32_t)(p.v_ss * 2);
  // Rows (of the K and V row arrays) of the two 16-key halves of tile n:
  // each half is 16 consecutive rows (block_size is a multiple of 16).  r1
  // is meaningful only when the second half holds a key below Sk.  A table
  // entry is read through the constant address space with a wave-uniform
  // index, so it is a scalar load: a vector load would join the vmcnt queue
  // of the K/V tiles in flight and force a wait on all of them.
  struct TileRows {
    int64_t r0, r1;
  };
  using const_int = const __attribute__((address_space(4))) int;
  auto row_of = [&](int t) -> int64_t {  // paged: pool row of token t
    const int idx = __builtin_amdgcn_readfirstlane(b * p.max_blocks + t / p.block_size);
    int blk = ((const_int*)p.block_table)[idx];
    blk = min(max(blk, 0), p.num_blocks - 1);
    return (int64_t)blk * p.block_size + t % p.block_size;
  };
  auto tile_rows = [&](int n) -> TileRows {
    const int t0 = n * DBC;
    if (!paged) return {(int64_t)t0, (int64_t)t0 + 16};
    if (t0 > Sk - 1) return {0, 0};  // a tile past the sequence: no table read
    const int64_t r0 = row_of(t0);
    if (t0 + 16 > Sk - 1) return {r0, r0};              // no key in the second half
    if (t0 % p.block_size + 16 < p.block_size) return {r0, r0 + 16};  // same block
    return {r0, row_of(t0 + 16)};
  };

  // K fragments of tile n: key row sigma(l32) of the tile (the last key for
  // lanes past Sk), chunks kk
  auto load_k = [&](int n, const TileRows& tr, i16x8 (&kf)[KK]) {
    const int kidx = min(n * DBC + sigma(l32), Sk - 1) - n * DBC;  // 0 .. 31
    const int64_t row = (kidx >= 16 ? tr.r1 : tr.r0) + (kidx & 15);
    const uint16_t* krow = (const uint16_t*)(kbase + row * (int64_t)rbk);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};  // columns past d: zeros, not read
      if (kk * 16 + hh * 8 < p.d) x = *(const u32x4*)(krow + kk * 16 + hh * 8);
      kf[kk] = __builtin_bit_cast(i16x8, x);
    }
  };
  // V tile n -> this wave's LDS stage: column-blocked, 32 rows x 64 bytes per
  // block, chunk c of row r at slot c ^ ((r >> 2) & 3); round u covers block
  // u >> 1, rows 16 (u & 1) + lane / 4
  // (rows past Sk re-read the last key's row, whose values are finite)
  // (chunks past d, in the column blocks from full_col_blocks(D) on, load
  // zeros: an offset past the descriptor's end)
  constexpr int FULL = full_col_blocks(D);
  auto load_v = [&](int n, const TileRows& tr, LDS_PTR(char) buf) {
    const int row = lane >> 2;
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    const int last = Sk - 1 - n * DBC;  // last key of the tile, relative (>= 0)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      // half h2 from its own 16 rows, or (second half wholly past Sk) the
      // first half's last key
      const bool own = h2 == 0 || last >= 16;
      const int64_t base = (h2 == 0 || !own) ? tr.r0 : tr.r1;
      const int rr = own ? min(row, last - 16 * h2) : last;
      const uint32_t off = (uint32_t)rr * rbv + (uint32_t)chunk * 16;
      // the descriptor spans the 16 rows' bytes, 15 strides + one row of D
      // elements (a stride below D, or 0, still reads whole rows)
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(vbase + base * (int64_t)rbv), 0, (int)(15 * rbv + p.d * 2), 0x00020000);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const uint32_t o = cb < FULL || 32 * cb + chunk * 8 < p.d ? off : OOB_OFFSET;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_PTR(void))(buf + cb * VBLK + h2 * 1024),
                                                 16, o, 64 * cb, 0, 0);
      }
    }
  };
  // transposed V fragment (A operand of O^T += V^T P^T): rows 16t + 8hh ..
  // +7 of column 32cb + l32
  uint32_t tb[2];
  {
    const int g16 = lane >> 4;
    const int s16 = lane & 15;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = 8 * (g16 >> 1) + 4 * half + (s16 >> 2);
      const int cc = 16 * (g16 & 1) + 4 * (s16 & 3);
      tb[half] = (uint32_t)(row * 64 + ((((cc >> 3) ^ ((row >> 2) & 3))) << 4) + (cc & 7) * 2);
    }
  }
  auto read_vt = [&](LDS_PTR(char) buf, int t, int cb) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (LDS_PTR(i16x4))(buf + (cb * VBLK + t * 16 * 64 + tb[0])));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (LDS_PTR(i16x4))(buf + (cb * VBLK + t * 16 * 64 + tb[1])));
    return (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[cb][q] = 0.f;
  float m_run = -1e30f, l_rnd = 0.f, l_fp32 = 0.f;

  LDS_PTR(char) const vb0 = (LDS_PTR(char))lds_v[wave][0];
  LDS_PTR(char) const vb1 = (LDS_PTR(char))lds_v[wave][1];
  int n = t_lo + wave;
  i16x8 kA[KK], kB[KK];
  if (n < t_end) {
    const TileRows tr = tile_rows(n);
    load_k(n, tr, kA);
    load_v(n, tr, vb0);
  }
  // one tile: kf holds K(n), vbuf V(n); the next tile's loads are in flight
  auto tile = [&](int nn, const i16x8 (&kf)[KK], LDS_PTR(char) vbuf) {
    f32x16 S;
#pragma unroll
    for (int q = 0; q < 16; ++q) S[q] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) S = T::mfma(kf[kk], qf[kk], S);
    // mask keys past this row's limit (ragged end, causal tail)
    if (nn * DBC + DBC - 1 > min(lim, Sk - 1) || !rok) {
      const int L = lim - nn * DBC - 8 * hh;
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (key_of_reg(q) > L) S[q] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < 16; ++q) mx = fmaxf(mx, S[q]);
    mx = other_half_max(mx) * p.scale_log2;
    const bool resc = __builtin_amdgcn_ballot_w64(mx > m_run + DEC_RESCALE_TAU) != 0;
    float alpha = 1.f;
    if (resc) {
      const float m_new = fmaxf(m_run, mx);
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
    }
    float ls = 0.f, lr = 0.f;
    i16x8 ph[2], pl[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      f32x8 e;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        e[q] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[8 * f + q], p.scale_log2, -m_run));
        ls += e[q];
      }
      ph[f] = T::cvt(e);
      lr = T::sum8(ph[f], lr);
      if constexpr (T::SPLIT_P) {
        pl[f] = T::cvt(e - T::widen(ph[f]));
        lr = T::sum8(pl[f], lr);
      }
    }
    if (resc) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[cb][q] *= alpha;
    }
    l_rnd = l_rnd * alpha + lr;
    l_fp32 = l_fp32 * alpha + ls;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const i16x8 vf = read_vt(vbuf, t, cb);
        acc[cb] = T::mfma(vf, ph[t], acc[cb]);
        if constexpr (T::SPLIT_P) acc[cb] = T::mfma(vf, pl[t], acc[cb]);
      }
  };
  // s_waitcnt immediate for vmcnt(KK + 2 CB), expcnt and lgkmcnt untouched
  // (gfx9 encoding: vmcnt bits 3:0 and 15:14)
  constexpr int VMN = KK + 2 * CB;
  constexpr int VM_NEXT = 0x0F70 | (VMN & 15) | ((VMN >> 4) << 14);
  static_assert(VMN < 64, "vmcnt range");
  // tiles n, n + NW, ... alternate between the (kA, stage 0) and (kB,
  // stage 1) register/LDS sets, so the loop body is unrolled by two
  // The pool rows of a tile (table reads, when paged) are looked up one
  // tile before its loads are issued, so the scalar loads land during the
  // tile in between.
  TileRows trB = tile_rows(n + NW < t_end ? n + NW : n);
  for (; n < t_end; n += 2 * NW) {
    if (n + NW < t_end) {
      load_k(n + NW, trB, kB);
      load_v(n + NW, trB, vb1);
    }
    const TileRows trA = tile_rows(n + 2 * NW < t_end ? n + 2 * NW : n);
    // K(n) and V(n) (issued one tile earlier) have landed: wait for all but
    // the loads just issued
    if (n + NW < t_end)
      __builtin_amdgcn_s_waitcnt(VM_NEXT);  // vmcnt(KK + 2 CB)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    tile(n, kA, vb0);
    if (n + NW >= t_end) break;
    if (n + 2 * NW < t_end) {
      load_k(n + 2 * NW, trA, kA);
      load_v(n + 2 * NW, trA, vb0);
      __builtin_amdgcn_s_waitcnt(VM_NEXT);
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    trB = tile_rows(n + 3 * NW < t_end ? n + 3 * NW : n);
    tile(n + NW, kB, vb1);
  }

  // ---- merge the NW waves' states through LDS
  auto pair_sum = [](float x) {
    auto rr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                               false);
    return __uint_as_float(rr[0]) + __uint_as_float(rr[1]);
  };
  const float lr_tot = pair_sum(l_rnd);
  const float lf_tot = T::LSE_FROM_FP32_SUM ? pair_sum(l_fp32) : lr_tot;
  __syncthreads();  // every wave is done with its V stages: reuse them
  // [wave][row][D] floats; the float4 at column c of row r sits at column
  // c ^ 4 (r % 16) (c ^ 4 (r % 8) when D is not a multiple of 64, so that
  // the column stays inside the row), so that 16 rows written at one
  // column, and one row read by 16 lanes, fill the 64 banks evenly
  float* mo = (float*)&lds_v[0][0][0];
  constexpr int SWZ = D % 64 == 0 ? 15 : 7;
  auto mo_at = [&](int row, int c) { return mo + row * D + (c ^ ((row & SWZ) << 2)); };
  if (hh == 0) {
    lds_m[wave][l32] = m_run;
    lds_lr[wave][l32] = lr_tot;
    lds_lf[wave][l32] = lf_tot;
  }
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      // acc[cb] register 4 g4 + q is row d = 32 cb + 8 g4 + 4 hh + q of O^T
      f32x4 x;
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = acc[cb][4 * g4 + q];
      *(f32x4*)mo_at(wave * 32 + l32, 32 * cb + 8 * g4 + 4 * hh) = x;
    }
  __syncthreads();
  // thread: rows tid / 16 (+ 4 NW per pass), float4 columns 4 (tid % 16) + 64 j
  const int l16 = tid & 15;
  constexpr int RPP = 4 * NW;  // rows per pass
#pragma unroll
  for (int pass = 0; pass < 32 / RPP; ++pass) {
    const int rr = (tid >> 4) + RPP * pass;
    if (rr < M) {
      float mmax = -1e30f;
#pragma unroll
      for (int w = 0; w < NW; ++w) mmax = fmaxf(mmax, lds_m[w][rr]);
      float wgt[NW], lr_s = 0.f, lf_s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        wgt[w] = __builtin_amdgcn_exp2f(lds_m[w][rr] - mmax);
        lr_s += wgt[w] * lds_lr[w][rr];
        lf_s += wgt[w] * lds_lf[w][rr];
      }
      const bool has = lr_s > 0.f;
      const float inv = has ? 1.f / lr_s : 0.f;
      const float lse = has ? (mmax + __builtin_amdgcn_logf(lf_s)) * LN2 : -INFINITY;
      const int h = kvh * g + (r0g + rr) / p.Sq;
      const int i = (r0g + rr) % p.Sq;
      uint16_t* orow = p.o + (int64_t)b * p.o_sb + (int64_t)i * p.o_ss + (int64_t)h * p.o_sh;
      // a piece of a split key range writes its fp32 state normalised over
      // its keys instead
      float* prow = p.part_o == nullptr
                        ? nullptr
                        : p.part_o + ((((int64_t)piece * p.B + b) * p.Sq + i) * p.Hq + h) * D;
#pragma unroll
      for (int j = 0; j < (D + 63) / 64; ++j) {
        const int c = 4 * l16 + 64 * j;
        if (c >= p.d) continue;  // columns past d (and past D) are not written
        f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const f32x4 y = *(const f32x4*)mo_at(w * 32 + rr, c);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc4[e] += wgt[w] * y[e];
        }
        if (prow == nullptr) {
          f32x8 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = acc4[e] * inv;
            x[e + 4] = 0.f;
          }
          const i16x8 hv = T::cvt(x);
          const u32x2 w2 = {(unsigned)(uint16_t)hv[0] | ((unsigned)(uint16_t)hv[1] << 16),
                            (unsigned)(uint16_t)hv[2] | ((unsigned)(uint16_t)hv[3] << 16)};
          *(u32x2*)(orow + c) = w2;
        } else {
          *(f32x4*)(prow + c) = acc4 * inv;
        }
      }
      if (l16 == 0) {
        if (prow == nullptr) {
          if (p.lse != nullptr) p.lse[((int64_t)b * p.Hq + h) * p.Sq + i] = lse;
        } else {
          p.part_lse[(((int64_t)piece * p.B + b) * p.Hq + h) * p.Sq + i] = lse;
        }
      }
    }
  }
}

template <int DT, int D>
hipError_t launch_decode_d(bool causal, const DecodeArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.grid), block(DEC_WAVES * 64);
  if (causal)
    hipLaunchKernelGGL((attn_decode_kernel<DT, D, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_decode_kernel<DT, D, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

__attribute__((visibility("hidden"))) hipError_t attn_detail::launch_decode(
    int dtype, int d, int causal, const DecodeArgs& a, hipStream_t st) {
  const bool c = causal != 0;
  if (dtype == ATTN_DTYPE_BF16) {
    switch (padded_head(d)) {
      case 32: return launch_decode_d<ATTN_DTYPE_BF16, 32>(c, a, st);
      case 64: return launch_decode_d<ATTN_DTYPE_BF16, 64>(c, a, st);
      case 96: return launch_decode_d<ATTN_DTYPE_BF16, 96>(c, a, st);
      case 128: return launch_decode_d<ATTN_DTYPE_BF16, 128>(c, a, st);
      case 192: return launch_decode_d<ATTN_DTYPE_BF16, 192>(c, a, st);
      default: return launch_decode_d<ATTN_DTYPE_BF16, 256>(c, a, st);
    }
  }
  switch (padded_head(d)) {
    case 32: return launch_decode_d<ATTN_DTYPE_F16, 32>(c, a, st);
    case 64: return launch_decode_d<ATTN_DTYPE_F16, 64>(c, a, st);
    case 96: return launch_decode_d<ATTN_DTYPE_F16, 96>(c, a, st);
    case 128: return launch_decode_d<ATTN_DTYPE_F16, 128>(c, a, st);
    case 192: return launch_decode_d<ATTN_DTYPE_F16, 192>(c, a, st);
    default: return launch_decode_d<ATTN_DTYPE_F16, 256>(c, a, st);
  }
}
