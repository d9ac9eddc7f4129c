// Fused exact-attention forward for AMD Instinct MI355X (gfx950, CDNA4).
//
//   O = softmax(scale * Q K^T + M) V,   LSE = log of the softmax denominator
//
// The method is the tiled online-softmax evaluation described on the pages
// ("MiniPaged-Qwen: Qwen3 prefill FlashAttention", sections 3-5 and 13;
// "FlashAttention personal implementation notes", sections "Online Softmax"
// and "FlashAttention"; the cuTile write-up's main loop, causal and GQA
// sections): Q is tiled by query rows, K and V stream through on-chip memory
// tile by tile, each query row keeps a running max m, a running denominator l
// and an unnormalised accumulator, and the score matrix never leaves the chip.
//
// gfx950 mapping (the pages' CUDA designs are prior art; this is the CDNA4
// layout):
//
// * One wave (64 lanes) owns QB blocks of 32 query rows of one query head.
//   Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16
//   (K tile rows as the A operand, Q rows as the B operand).  In the 32x32
//   accumulator layout lane l holds column l%32, i.e. ONE query row, and 16 of
//   the 32 keys; lanes l and l+32 hold the other 16 keys of the same row.
//   Row max and row sum are therefore in-lane plus one v_permlane32_swap, and
//   the rescale factor of the accumulator is a per-lane scalar.
// * The K rows of each 32-key block are fed to the MFMA in a permuted order
//   (sigma below) chosen so that the S^T accumulator, converted to 16 bit, is
//   already the B operand of the second product O^T += V^T P^T: P never
//   leaves registers.
// * V^T fragments come straight from the row-major V tile in LDS through the
//   gfx950 transpose read ds_read_b64_tr_b16.
// * K and V tiles are double-buffered in LDS with a 16-byte XOR swizzle that
//   keeps both the row reads of K and the transposed reads of V free of bank
//   conflicts.  Tiles go global -> LDS with gfx950 direct-to-LDS loads
//   (global_load_lds_dwordx4), so the prefetch holds no registers.
// * Online softmax runs in the log2 domain (exp2 with scale*log2(e) folded
//   into one FMA, as in the cuTile write-up's fast-math step).  The running
//   max is only moved when a tile's max exceeds it by more than RESCALE_TAU
//   (2^8): the result is mathematically identical, because numerator and
//   denominator use the same stale max, and most tiles then skip the
//   rescaling of the accumulator.  With bf16 (whose exponent range is
//   fp32's) the max is taken on a row block's first tile only; a later tile
//   whose probabilities against it overshoot a bound is redone with its own
//   max (DEFER_SUM_LIMIT).
// * The softmax denominator sums the very 16-bit probabilities that multiply
//   V (v_dot2 against 1.0: exact products, fp32 accumulation), so the
//   normalisation O = sum P~ V / sum P~ uses one consistent set of rounded
//   weights; for fp16 inputs P is carried as a hi + lo pair.
// * Causal masking is applied only on the tiles that straddle the diagonal or
//   the ragged end of K (the cuTile write-up's K-loop split); tiles above the
//   diagonal are never visited (its causal loop bound).
// * GQA: the waves of a workgroup are different query heads of one kv group
//   (and/or consecutive row blocks), so every K/V tile loaded into LDS serves
//   all of them.
// * Work items are ordered heaviest-first (causal row blocks near the end of
//   the sequence first) and, when the counts allow, grouped per XCD so that
//   the workgroups sharing a kv head land on the same L2.
// * Key split (attn_fwd_split): when the row blocks are too few to fill the
//   chip, the K/V tiles of a row block are cut into pieces of a fixed number
//   of tiles, one workgroup per piece.  A piece writes its row states in fp32
//   (output normalised over its own keys, and the log-sum-exp of those keys)
//   and a second kernel merges the pieces with the online-softmax rescale
//   (personal-notes page, section "Online Softmax", applied to whole pieces).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "attn.h"
#include "attn_common.h"

namespace {

constexpr float RESCALE_TAU = 8.0f; // log2 headroom before the max is moved
// bf16: after the first tile of a row block the running max is not taken per
// tile; a tile whose probabilities against it sum past this bound in a lane
// (some score more than about 2^35 above the max, or an overflow to inf) is
// redone with its true max.  bf16 has the fp32 exponent range, so
// probabilities up to 2^40 round with the same relative error as those up to
// 1.  A lane's sum then grows by less than 2^40 per 32 keys, so a row's sum
// stays below 2^35 Sk and its accumulators below 2^35 Sk max|V|: finite in
// fp32 while Sk max|V| < 2^93.
constexpr float DEFER_SUM_LIMIT = 1099511627776.0f;  // 2^40

// ------------------------------------------------------------ parameters
struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  // element strides of (batch, seq, head); d is contiguous.  Every row
  // starts 16-byte aligned (host-checked).
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int B, Sq, Sk, Hq, Hkv;
  int d;         // head size: the kernel is built for D >= d, columns past d
                 // read as zeros and are not written
  int group;     // Hq / Hkv
  int gh;        // query heads per workgroup (divides group and the wave count)
  int hsub;      // group / gh
  int rows_wg;   // query rows per workgroup (per head)
  int qtiles;    // ceil(Sq / rows_wg)
  int ncols;     // B * Hkv * hsub
  int xcd_cols;  // columns per XCD when the grid is XCD-ordered, else 0
  int xcd_qsplit;  // > 0: XCDs per (batch, kv head) (query blocks dealt out)
  int off;       // Sk - Sq
  float scale_log2;  // scale * log2(e)
  // key split: K/V tiles per piece (even; 0 = no split).  A row block with
  // more tiles than that is cut into pieces; the pieces write fp32 partial
  // states for rows q_split.. Sq-1 (sq_split = Sq - q_split rows):
  //   part_o  [piece][b][i - q_split][hq][D], normalised over the piece's keys
  //   part_lse[piece][b][hq][i - q_split], natural log (-inf: no key seen)
  int chunk;
  int q_split, sq_split;
  float* part_o;
  float* part_lse;
};



// ------------------------------------------------------------ the kernel
//
// One wave = 32 query rows of one head; the waves of a workgroup share every
// K/V tile.  The work of a tile is skewed across loop iterations so that each
// iteration hands the vector ALU and the matrix core independent work:
//
//   iteration j:  softmax(S(j)) -> P(j)            [VALU: max, exp2, convert]
//                 O += V(j-1)^T P(j-1)             [MFMA, previous tile]
//                 S(j+1) = K(j+1) Q^T              [MFMA, next tile]
//
// The three streams have no dependencies among them inside the iteration, so
// the compiler interleaves exp/convert instructions between the MFMAs of the
// same wave, and two waves per SIMD fill each other's LDS waits.  K runs one
// tile ahead of V: iteration j reads K(j+1) and V(j-1) while K(j+2) and V(j)
// stream in, so two K and two V buffers live in LDS.
//
// The thresholded max update is decided at the start of an iteration from
// S(j) (bf16: on the first tile, or at the end of an iteration whose P(j)
// overshot); the rescale of the accumulators by alpha(j) is applied at the
// END of the iteration, after O has absorbed V(j-1)^T P(j-1), whose
// probabilities were taken against the previous max.
template <typename PT, int N>
struct PFrag {
  PT hi[N];
  PT lo[N];  // fp16 only (hi + lo split); unused for bf16
};

// NG groups of 4 waves per workgroup.  With NG = 2 (grids of at most one
// workgroup per CU: short sequences, few heads), the two groups walk
// alternate K/V tiles of the same query rows, two waves per SIMD, each with
// its own tile buffers and online-softmax state; at the end group 1 hands
// its state (running max, sums, unnormalised O) to group 0 through LDS and
// group 0 combines the two with the online-softmax rescale (personal-notes
// page, section "Online Softmax", applied to the two key subsets).
//
// KH = 2 (key halves, NG = 1): the 4 waves are 2 row waves x 2 key halves.
// Both waves of a row wave take the same 32 query rows, one the first and
// one the second 32-key block of every tile, each with its own online-
// softmax state, merged through LDS at the end as the two groups are.  A
// workgroup then holds 64 rows instead of 128 with the same tile buffers,
// so a launch that would leave most CUs with one workgroup has twice as
// many workgroups, two per CU, and the snake order below puts a long row
// block and a short one on each CU.
//
// NW = 8 (key halves at d = 192, where a workgroup's tile buffers leave one
// workgroup per CU): 4 row waves x 2 key halves over the same tiles, so that
// two waves share each SIMD; the two halves of the waves load alternate
// column blocks of a tile.
template <int DT, int D, bool CAUSAL, int NG, int KH, int NW>
__global__ __launch_bounds__(NG * NW * 64, (D > 128 || NG > 1 || NW > 4) ? 1 : 2) void
attn_fwd_pipe_kernel(Params p) {
  using T = Ty<DT>;
  static_assert(NW == 4 || (NW == 8 && KH == 2 && NG == 1), "8 waves run as key halves");
  constexpr int NT = NW * 64;         // threads per group
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int CPT = BC * CPR / NT;  // direct loads per lane per tile
  constexpr int KB = BC / 32;         // 32-key blocks per tile
  constexpr int KBW = KB / KH;        // ... per wave
  constexpr int CB = D / 32;
  constexpr int KK = D / 16;
  constexpr int NP = BC / 16 / KH;    // 16-key P fragments per wave
  constexpr int TB = BC * D * 2;      // bytes per K or V tile buffer
  static_assert(CPT * NT == BC * CPR, "tile must split evenly over threads");
  static_assert(CPT * (NW / 4) == CB, "one load round per 32-column block and wave quad");
  // bf16 up to d = 128: the running max is taken on a row block's first tile
  // and then only for a tile whose probabilities overshoot (DEFER_SUM_LIMIT);
  // above 128 the redo finds no registers
  constexpr bool DEFER_MAX = DT == ATTN_DTYPE_BF16 && D <= 128;
  static_assert(!DEFER_MAX || !T::SPLIT_P, "the deferred max redoes a single-part P");

  // Two K and two V tile buffers, each its own LDS object: the compiler's
  // alias analysis then separates the direct loads into one buffer from the
  // reads of another, so no read waits for an unrelated tile load (with one
  // LDS array every read of a tile waited for all loads in flight).
  // (one set per group)
  __shared__ __attribute__((aligned(1024))) char lds_k0[NG][TB], lds_k1[NG][TB], lds_v0[NG][TB],
      lds_v1[NG][TB];
  ATTN_POISON_LDS_ARRAY(lds_k0);
  ATTN_POISON_LDS_ARRAY(lds_k1);
  ATTN_POISON_LDS_ARRAY(lds_v0);
  ATTN_POISON_LDS_ARRAY(lds_v1);
  ATTN_POISON_LDS_DONE();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: SGPR
  const int grp = NG > 1 ? wave_all >> 2 : 0;  // group
  const int wave = wave_all & (NW - 1);       // wave within the group
  static_assert(KH == 1 || (KH == 2 && NG == 1), "key halves run as one group");
  const int kh = KH > 1 ? (wave & 1) : 0;        // key half of every tile
  const int rw = KH > 1 ? (wave >> 1) : wave;    // row wave: 32 rows of one head
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  auto kbuf_of = [&](int n) {
    return (n & 1) ? (LDS_PTR(char))lds_k1[grp] : (LDS_PTR(char))lds_k0[grp];
  };
  auto vbuf_of = [&](int n) {
    return (n & 1) ? (LDS_PTR(char))lds_v1[grp] : (LDS_PTR(char))lds_v0[grp];
  };

  // ---- work decode: heaviest row blocks first, optionally grouped per XCD;
  // with a key split, all first pieces, then all second pieces, ...
  int qt, col, piece;
  {
    int L = blockIdx.x;
    // Snake order (key halves): a grid of two workgroups per CU places
    // workgroup k + 256 on the CU of workgroup k (k + 32 and k within one
    // XCD's ids), so every other run of 256 (32 per XCD) is taken in reverse
    // order of weight: the heaviest block shares its CU with the lightest.
    // The order only moves work between CUs; any placement gives the same
    // results.
    auto snake = [](int k, int n, int s) {
      const int base = k / s * s;
      if (!((k / s) & 1)) return k;
      return base + min(s, n - base) - 1 - (k - base);
    };
    if (KH > 1 && NW == 4) {
      const int n = (int)gridDim.x;
      if (p.xcd_qsplit > 0 || p.xcd_cols > 0)
        L = (snake(L >> 3, n >> 3, kCUCount / 8) << 3) | (L & 7);
      else
        L = snake(L, n, kCUCount);
    }
    int u;
    if (p.xcd_qsplit > 0) {
      // XCD x: (batch, kv head) x / xcd_qsplit, every head subset, query
      // blocks x % xcd_qsplit, + xcd_qsplit, ... heaviest first (no key split)
      const int xcd = L & 7;
      const int k = L >> 3;
      const int hs0 = k % p.hsub;
      u = (k / p.hsub) * p.xcd_qsplit + xcd % p.xcd_qsplit;
      col = (xcd / p.xcd_qsplit) * p.hsub + hs0;
    } else if (p.xcd_cols > 0) {
      const int xcd = L & 7;
      const int k = L >> 3;
      u = k / p.xcd_cols;
      col = xcd * p.xcd_cols + k % p.xcd_cols;
    } else {
      u = L / p.ncols;
      col = L % p.ncols;
    }
    piece = u / p.qtiles;
    qt = p.qtiles - 1 - (u - piece * p.qtiles);
  }
  const int hs = col % p.hsub;
  const int kvh = (col / p.hsub) % p.Hkv;
  const int b = col / (p.hsub * p.Hkv);
  const int head_in_wg = rw % p.gh;
  const int rowblk = rw / p.gh;
  const int hq = kvh * p.group + hs * p.gh + head_in_wg;
  const int q0wg = qt * p.rows_wg;
  const int q0w = q0wg + rowblk * 32;

  // ---- KV tile range of the workgroup: tiles [j_lo, j_hi) of the row
  // block's n_end.  Group g walks tiles j_lo + g, j_lo + g + NG, ...: its
  // local tile i (buffer i & 1) is tile_of(i).  Both groups run n_loc
  // iterations so that they pass the same barriers; a group with one tile
  // fewer runs a filler tile past j_hi whose keys are all masked.
  const int n_end = block_tiles(q0wg, p.rows_wg, p.Sq, p.Sk, p.off, CAUSAL);
  const int pieces = block_pieces(n_end, p.chunk);
  if (piece >= pieces) return;  // an empty piece: uniform over the workgroup
  const bool split = pieces > 1;
  const int j_lo = piece * p.chunk;
  const int j_hi = split ? min(n_end, j_lo + p.chunk) : n_end;
  const int n_loc = j_hi > j_lo ? (j_hi - j_lo + NG - 1) / NG : 0;
  auto tile_of = [&](int i) { return j_lo + grp + NG * i; };
  // the tile a load reads: a filler tile reads the block's last tile (its
  // keys are masked), so that no load addresses memory past the tensors
  auto load_of = [&](int i) { return min(tile_of(i), j_hi - 1); };
  int n_full = p.Sk / BC;
  if (CAUSAL) {
    const int lim = q0wg + p.off + 1;
    n_full = min(n_full, lim > 0 ? lim / BC : 0);
  }
  n_full = min(n_full, n_end);

  // K and V rows of this (batch, kv head): byte slices whose rows (keys) are
  // k_ss * 2 and v_ss * 2 bytes apart
  const uint32_t rbk = (uint32_t)(p.k_ss * 2);
  const uint32_t rbv = (uint32_t)(p.v_ss * 2);
  const char* kslice = (const char*)(p.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh);
  const char* vslice = (const char*)(p.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh);

  // ---- LDS tile layout of this kernel: column-blocked.  A K or V tile is
  // stored as D/32 blocks of 32 columns; block cb holds the 64 rows of those
  // columns, 64 bytes (four 16-byte chunks) per row, and chunk c of row r
  // sits at slot c ^ ((r >> 2) & 3).  Every fragment address is then a
  // per-lane base plus compile-time offsets for the column block and the row
  // group, and both read patterns are free of bank conflicts: the 16 rows of
  // a K fragment row read land on 16 distinct 16-byte slots of one 256-byte
  // bank cycle, and the 4 rows x 64 bytes of a V transpose read of 32 lanes
  // fill one bank cycle exactly.
  constexpr int BLK = 64 * 64;  // bytes per column block of a tile
  // K fragment (kb, kk): row 32kb + sigma(l32), logical chunk 2kk + hh, i.e.
  // block kk/2, in-block chunk 2(kk&1) + hh.  kb counts the wave's own key
  // blocks, which start at block kh * KBW of the tile.
  uint32_t kbase_lds[2];
  {
    const int row = 32 * KBW * kh + sigma(l32);
    const int sw = (row >> 2) & 3;
#pragma unroll
    for (int par = 0; par < 2; ++par)
      kbase_lds[par] = (uint32_t)(row * 64 + (((2 * par + hh) ^ sw) << 4));
  }
  // V^T fragment (t, cb, half): transpose read of rows 16t + 8(g16>>1) +
  // 4half + (s16>>2), columns 32cb + 16(g16&1) + 4(s16&3).  t counts the
  // wave's own 16-key groups, which start at group kh * NP of the tile.
  uint32_t vbase_lds[2];
  {
    const int g16 = lane >> 4;
    const int s16 = lane & 15;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = 16 * NP * kh + 8 * (g16 >> 1) + 4 * half + (s16 >> 2);
      const int cc = 16 * (g16 & 1) + 4 * (s16 & 3);  // column inside the block
      vbase_lds[half] =
          (uint32_t)(row * 64 + ((((cc >> 3) ^ ((row >> 2) & 3))) << 4) + (cc & 7) * 2);
    }
  }
  auto k_addr = [&](LDS_PTR(char) kbuf, int kb, int kk) {
    return kbuf + ((kk >> 1) * BLK + kb * 32 * 64 + kbase_lds[kk & 1]);
  };
  auto v_addr = [&](LDS_PTR(char) vbuf, int t, int cb, int half) {
    return vbuf + (cb * BLK + t * 16 * 64 + vbase_lds[half]);
  };
  // Direct global -> LDS load round u of a wave writes column block
  // cbk = u * (NW / 4) + wave / 4 of the tile, LDS bytes
  // [(cbk * 4 + wave % 4) * 1024, +1024): rows 16 * (wave % 4) + lane / 4,
  // slot lane % 4.
  const int wq = NW == 8 ? wave & 3 : wave;   // wave within its quad
  const int wh = NW == 8 ? wave >> 2 : 0;     // quad
  const int ld_row = 16 * wq + (lane >> 2);
  const int ld_chunk = (lane & 3) ^ ((ld_row >> 2) & 3);
  const int ld_col = ld_chunk * 8;  // + 32 * u: the column block of round u

  // Tile loads are MUBUF loads to LDS through a buffer descriptor of the
  // tile: the tile base and record count live in SGPRs, the per-lane offset
  // is the same for every full tile, and the column round goes in the scalar
  // offset, so a tile costs no per-lane address arithmetic.  (The FLAT-encoded
  // global load to LDS would also do, but the compiler then assumes it may
  // count on the LDS counter and waits for every outstanding LDS read at
  // each dependency.)  Rows past Sk in the ragged last tile re-read row
  // Sk - 1 (their keys are masked).  The descriptor spans the bytes the
  // tile's rows occupy, (BC - 1) * (row stride) + one row of D elements, so
  // a row stride below D (overlapping or broadcast K/V views, stride 0
  // included) still reads every row whole.  Host validation keeps BC * (row
  // stride) below 2^31.
  const uint32_t ld_off_k = (uint32_t)ld_row * rbk + (uint32_t)ld_col * 2;
  const uint32_t ld_off_v = (uint32_t)ld_row * rbv + (uint32_t)ld_col * 2;
  // The column rounds from full_col_blocks(D) on may hold columns that a
  // padded head size lacks: those lanes load from past the descriptor's end,
  // which fills zeros.
  constexpr int FULL = full_col_blocks(D);
  // The ragged last tile of K/V (if any): its lanes' offsets, computed once
  // (rows past Sk re-read row Sk - 1), so that a tile load selects an offset
  // instead of branching.
  const int n_rag = p.Sk % BC ? p.Sk / BC : -1;
  const uint32_t rag_row = (uint32_t)(min(n_rag * BC + ld_row, p.Sk - 1) - n_rag * BC);
  const uint32_t ld_off_k_rag = rag_row * rbk + (uint32_t)ld_col * 2;
  const uint32_t ld_off_v_rag = rag_row * rbv + (uint32_t)ld_col * 2;
  auto issue_rows = [&](const char* slice, uint32_t row_bytes, uint32_t ld_off,
                        uint32_t ld_off_rag, int n, LDS_PTR(char) buf) {
    const char* tile = slice + (int64_t)n * BC * row_bytes;
    const uint32_t off = n == n_rag ? ld_off_rag : ld_off;
    // raw buffer, 32-bit data format (word 3 of the descriptor)
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)tile, 0, (int)((BC - 1) * row_bytes + p.d * 2),
                                          0x00020000);
    // the wave's LDS offset, opaque here, so that each load's destination is
    // a scalar add at the load instead of a loop-invariant value the compiler
    // would keep (and, short of scalar registers, reload from a VGPR lane)
    uint32_t wofs = (uint32_t)wq * 1024;
    asm volatile("" : "+s"(wofs));
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int cbk = u * (NW / 4) + wh;  // column block (uniform)
      const uint32_t o = cbk < FULL || 32 * cbk + ld_col < p.d ? off : OOB_OFFSET;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (LDS_PTR(void))(buf + cbk * 4096 + wofs), 16, o, 64 * cbk, 0, 0);
    }
  };

  // ---- Q fragments, kept in registers
  i16x8 qf[KK];
  {
    const int qi = q0w + l32;
    const bool ok = qi < p.Sq;
    const uint16_t* qrow =
        p.q + (int64_t)b * p.q_sb + (int64_t)(ok ? qi : 0) * p.q_ss + (int64_t)hq * p.q_sh;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};  // columns past d stay zero
      if (ok && kk * 16 + hh * 8 < p.d) x = *(const u32x4*)(qrow + kk * 16 + hh * 8);
      qf[kk] = __builtin_bit_cast(i16x8, x);
    }
  }

  // ---- state: O^T, running max, and per-lane partial row sums (the lane
  // holds half of its row's keys; lanes l and l+32 are combined at the end):
  // l_rnd sums exactly the 16-bit P that multiply V, so O is normalised by a
  // consistent set of weights; l_fp32 sums the unrounded P for the LSE.
  f32x16 acc_o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[cb][r] = 0.f;
  float m_run = -1e30f;
  float l_rnd = 0.f;
  float l_fp32 = 0.f;
  int lim_row;
  {
    const int qi = q0w + l32;
    lim_row = p.Sk - 1;
    if (CAUSAL) lim_row = min(lim_row, qi + p.off);
  }
  // S^T = K(kbuf) Q^T
  auto qk = [&](f32x16 (&S)[KBW], LDS_PTR(char) kbuf) {
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) S[kb][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const i16x8 kf = *(LDS_PTR(const i16x8))(k_addr(kbuf, kb, kk));
        S[kb] = T::mfma(kf, qf[kk], S[kb]);
      }
    }
  };
  // O^T += V(vbuf)^T P^T
  auto pv = [&](const PFrag<i16x8, NP>& P, LDS_PTR(char) vbuf) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int t = 0; t < NP; ++t) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_PTR(i16x4))(v_addr(vbuf, t, cb, 0)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_PTR(i16x4))(v_addr(vbuf, t, cb, 1)));
        const i16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc_o[cb] = T::mfma(vf, P.hi[t], acc_o[cb]);
        if constexpr (T::SPLIT_P) acc_o[cb] = T::mfma(vf, P.lo[t], acc_o[cb]);
      }
    }
  };

  f32x16 SA[KBW], SB[KBW];
  PFrag<i16x8, NP> PA, PB;
#pragma unroll
  for (int t = 0; t < NP; ++t) {
    PB.hi[t] = (i16x8){0, 0, 0, 0, 0, 0, 0, 0};
    PB.lo[t] = (i16x8){0, 0, 0, 0, 0, 0, 0, 0};
  }

  // One iteration.  Sc = S(j) on entry, Sn receives S(j+1); Pp = P(j-1),
  // Pc receives P(j).  PAR = j & 1 fixes every LDS buffer address at compile
  // time.
  //
  // The main block is scheduled by hand as a list of steps (16 for the P V
  // product, 16 for the next tile's S at d = 128): each step issues the LDS
  // reads of the step LA places ahead, one MFMA (two for the fp16 hi/lo pair)
  // and the softmax work (argument, exp2, row sums, conversion) of one or
  // two scores of this tile, skewed as below.  sched_barrier
  // keeps the steps in order, so LDS reads run ahead of their MFMAs and the
  // vector ALU works beside the matrix core.
  constexpr int NPV = CB * NP;   // O^T += V^T P^T steps (t, cb)
  constexpr int NQK = KBW * KK;  // S^T = K Q^T steps (kb, kk)
  constexpr int NOPS = NPV + NQK;
  constexpr int NSC = KBW * 16;  // scores per lane
  constexpr int LA = 3;          // read-ahead, in steps
  // Steps that issue the tile loads.  With two key blocks per wave at
  // d = 128 (32 steps) the K load goes a quarter and the V load three
  // quarters into the list, apart from each other and from the top of the
  // iteration (measured: 1.2-1.4 % on the 8K GQA workload, none on the 16K
  // one); the key halves' lone waves keep them at the front, where the loads
  // have the most time to land (V three quarters in: +3 % on 2 x 1024
  // causal fp16).
  constexpr bool LD_SPREAD = D == 128 && KBW == 2;
  // Above d = 128 the step list has no registers to spare for the loads'
  // address arithmetic: there they are issued at the top of the iteration
  // (inside the steps the d = 256 kernel spilled into scratch and ran ten
  // times slower).
  constexpr bool LD_IN_STEPS = D <= 128;
  constexpr int LD_STEP_K = LD_SPREAD ? NOPS / 4 : 1;
  constexpr int LD_STEP_V = LD_SPREAD ? 3 * NOPS / 4 : 3;
  static_assert(LD_STEP_K < NOPS && LD_STEP_V < NOPS, "the loads are issued inside the step list");
  // Softmax work per step: the scores of key block 0 of S(j) are spread over
  // the P V steps and those of key block 1 over the first QK steps (those of
  // key block 0 of S(j+1)), so each block of S(j) is dead before the MFMAs
  // of the same block of S(j+1) start and both tiles share one register set.
  // With one key block per wave (key halves) S(j) and S(j+1) have registers
  // of their own, and its scores are spread over the whole step list, QK
  // steps included.  score_lo(i) is the first score of step i.
  constexpr int SK = D <= 128 ? 1 : 0;  // softmax skew, in steps
  // step after the last scores' arguments
  constexpr int SC_END = KBW > 1 ? NPV + KK : NOPS - 2 * SK;
  auto score_lo = [&](int i) {
    if (KBW == 1) return i <= SC_END ? 16 * i / SC_END : NSC;
    if (i <= NPV) return 16 * i / NPV;
    if (i <= NPV + KK) return 16 + 16 * (i - NPV) / KK;
    return NSC;
  };
  static_assert(KB == 2, "two 32-key blocks per tile");
  static_assert(SC_END + 2 * SK <= NOPS, "the skewed softmax ends inside the step list");

  // (i: the group's local tile index; j: the tile)
  auto iter = [&](auto par, int i, f32x16 (&Sc)[KBW], f32x16 (&Sn)[KBW],
                  const PFrag<i16x8, NP>& Pp, PFrag<i16x8, NP>& Pc) {
    constexpr int PAR = decltype(par)::value;
    const int j = tile_of(i);
    LDS_PTR(char) const K_NEXT = kbuf_of(PAR ^ 1);  // K(j+1)
    LDS_PTR(char) const V_PREV = vbuf_of(PAR ^ 1);  // V(j-1)
    LDS_PTR(char) const K_LOAD = kbuf_of(PAR);      // K(j+2)
    LDS_PTR(char) const V_LOAD = vbuf_of(PAR);      // V(j)
    const int it = i;  // the group's local tile index (the step loop reuses i)
    if constexpr (!LD_IN_STEPS) {
      issue_rows(kslice, rbk, ld_off_k, ld_off_k_rag, load_of(it + 2), K_LOAD);
      issue_rows(vslice, rbv, ld_off_v, ld_off_v_rag, load_of(it), V_LOAD);
    }
    // mask the straddling tiles (and a filler tile past j_hi, wholly), then
    // the row max and the max update
    auto mask = [&](f32x16 (&S)[KBW]) {
      if (j >= n_full || j >= j_hi) {
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
          const int L = j >= j_hi ? -BC : lim_row - j * BC - (KBW * kh + kb) * 32 - 8 * hh;
          // key_of_reg(r) > L: the sign of L - key_of_reg(r), spread over the
          // word, selects -inf bit by bit (v_bfi_b32), with no compare mask in
          // scalar registers
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t sel = (uint32_t)((L - key_of_reg(r)) >> 31);
            S[kb][r] = __uint_as_float((sel & 0xff800000u) | (~sel & __float_as_uint(S[kb][r])));
          }
        }
      }
    };
    // the row max of S (scaled to log2 units) and the thresholded max update;
    // alpha: the factor the accumulators take
    float alpha = 1.f;
    bool resc = false;
    auto max_update = [&](const f32x16 (&S)[KBW], float tau) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][r]);
      mx = other_half_max(mx) * p.scale_log2;
      const float m_new = fmaxf(m_run, mx);
      // move the max only past the threshold: alpha = 1 (no rescale) otherwise
      if (__builtin_amdgcn_ballot_w64(mx > m_run + tau) != 0) {
        alpha *= __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        resc = true;
      }
    };
    mask(Sc);
    // bf16: the max is taken on the first tile only (a tile that overshoots
    // it is redone below)
    if (!DEFER_MAX || i == 0) max_update(Sc, RESCALE_TAU);
    const float neg_m = -m_run;
    float ls = 0.f;   // unrounded P (LSE)
    float lr = 0.f;   // rounded P (normalisation of O)
    f32x8 e;
    float xa[NSC];
    i16x8 fr[LA + 1];
    // LDS reads of step i into fragment slot i % (LA + 1)
    auto read_step = [&](int i) {
      if (i < NPV) {
        const int t = i / CB, cb = i % CB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_PTR(i16x4))(v_addr(V_PREV, t, cb, 0)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_PTR(i16x4))(v_addr(V_PREV, t, cb, 1)));
        fr[i % (LA + 1)] = (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        const int q = i - NPV, kb = q / KK, kk = q % KK;
        fr[i % (LA + 1)] = *(LDS_PTR(const i16x8))(k_addr(K_NEXT, kb, kk));
      }
    };
#pragma unroll
    for (int i = 0; i < LA; ++i) read_step(i);
    // raised wave priority for the step block: on a SIMD shared by two
    // waves, the one in its MFMA + softmax steps issues ahead of one in its
    // serial part (row max, rescale, barrier) (measured: 1-1.5 % on the
    // long GQA workloads)
    __builtin_amdgcn_s_setprio(2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NOPS; ++i) {
      if (i + LA < NOPS) read_step(i + LA);
      const i16x8 f = fr[i % (LA + 1)];
      if (i < NPV) {  // O^T += V(j-1)^T P(j-1)
        // key block t outer: P(j-1) fragment t dies after step CB*t + CB-1,
        // before P(j) fragments take registers, and consecutive MFMAs go to
        // different accumulators
        const int t = i / CB, cb = i % CB;
        acc_o[cb] = T::mfma(f, Pp.hi[t], acc_o[cb]);
        if constexpr (T::SPLIT_P) acc_o[cb] = T::mfma(f, Pp.lo[t], acc_o[cb]);
      } else {  // S(j+1)^T = K(j+1) Q^T
        const int q = i - NPV, kb = q / KK, kk = q % KK;
        if (kk == 0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) Sn[kb][r] = 0.f;
        }
        Sn[kb] = T::mfma(f, qf[kk], Sn[kb]);
      }
      // the tile loads of K(j+2) and V(j), issued beside the first MFMAs:
      // their address arithmetic and descriptors then overlap the matrix
      // core instead of delaying the first step
      // (past the group's last tiles the K load re-reads its last tile into
      // a buffer no later step reads, so that the step has no branch)
      if (LD_IN_STEPS && i == LD_STEP_K)
        issue_rows(kslice, rbk, ld_off_k, ld_off_k_rag, load_of(it + 2), K_LOAD);
      if (LD_IN_STEPS && i == LD_STEP_V)
        issue_rows(vslice, rbv, ld_off_v, ld_off_v_rag, load_of(it), V_LOAD);
      // P(j) = exp2(S(j) * c - m), skewed over three steps (SK = 1): the
      // argument of this step's scores, the exp2 of the previous step's,
      // the sums and conversion of the one before, so that no op of a step
      // waits on the op just before it (measured: 1.5-2 % on the long GQA
      // workloads).  The last scores (step NPV + KK - 1) finish two steps
      // later, inside the QK steps of key block 1.  Head sizes above 128
      // have no registers to spare for the values in flight (SK = 0).
#pragma unroll
      for (int sc = score_lo(i); sc < score_lo(i + 1); ++sc) {
        const int kb = sc / 16, r = sc % 16;
        xa[sc] = __builtin_fmaf(Sc[kb][r], p.scale_log2, neg_m);
      }
#pragma unroll
      for (int sc = (i >= SK ? score_lo(i - SK) : 0); sc < (i >= SK ? score_lo(i - SK + 1) : 0);
           ++sc)
        xa[sc] = __builtin_amdgcn_exp2f(xa[sc]);
#pragma unroll
      for (int sc = (i >= 2 * SK ? score_lo(i - 2 * SK) : 0);
           sc < (i >= 2 * SK ? score_lo(i - 2 * SK + 1) : 0); ++sc) {
        {
          e[sc % 8] = xa[sc];
          if constexpr (T::LSE_FROM_FP32_SUM) {
            ls += e[sc % 8];
            // pinned here: sunk to its use after the block, the sum would
            // keep every exp2 result of the tile alive
            asm volatile("" : "+v"(ls));
          }
          if (sc % 8 == 7) {
            const i16x8 h = T::cvt(e);
            Pc.hi[sc / 8] = h;
            lr = T::sum8(h, lr);
            asm volatile("" : "+v"(lr));
            // an empty asm use pins the conversion (and the exp2s feeding
            // it) to this step; the compiler would otherwise sink them to
            // their use in the next iteration
            asm volatile("" ::"v"(h));
            if constexpr (T::SPLIT_P) {
              const i16x8 lo = T::cvt(e - T::widen(h));
              Pc.lo[sc / 8] = lo;
              lr = T::sum8(lo, lr);
              asm volatile("" ::"v"(lo));
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (DEFER_MAX) {
      // A lane whose probabilities of this tile sum past the bound (a score
      // far above the running max, or an overflow to inf): the wave takes
      // S(j) again, from K(j) in global memory (its LDS buffer is already
      // taking K(j+2)), moves the max to the tile's max and redoes P(j) and
      // its sums.  The accumulators take the factor at the end of the
      // iteration, as with the per-tile max.
      if (__builtin_amdgcn_ballot_w64(ls > DEFER_SUM_LIMIT) != 0) {
        f32x16 S[KBW];
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
          // key row 32 (KBW kh + kb) + sigma(l32) of tile j (rows past Sk
          // re-read row Sk - 1 and are masked), columns 16 kk + 8 hh .. +7
          const int krow = min(j * BC + 32 * (KBW * kh + kb) + sigma(l32), p.Sk - 1);
          const char* src = kslice + (int64_t)krow * rbk + hh * 16;
#pragma unroll
          for (int r = 0; r < 16; ++r) S[kb][r] = 0.f;
          u32x4 x[KK];
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            x[kk] = (u32x4){0u, 0u, 0u, 0u};  // columns past d are zeros
            if (kk * 16 + hh * 8 < p.d) x[kk] = *(const u32x4*)(src + kk * 32);
          }
#pragma unroll
          for (int kk = 0; kk < KK; ++kk)
            S[kb] = T::mfma(__builtin_bit_cast(i16x8, x[kk]), qf[kk], S[kb]);
          // one key block's fragments at a time (a cold path, kept out of
          // the register peak of the steps)
          __builtin_amdgcn_sched_barrier(0);
        }
        mask(S);
        max_update(S, 0.f);
        ls = 0.f;
        lr = 0.f;
#pragma unroll
        for (int sc = 0; sc < NSC; ++sc) {
          e[sc % 8] = __builtin_amdgcn_exp2f(
              __builtin_fmaf(S[sc / 16][sc % 16], p.scale_log2, -m_run));
          ls += e[sc % 8];
          if (sc % 8 == 7) {
            const i16x8 h = T::cvt(e);
            Pc.hi[sc / 8] = h;
            lr = T::sum8(h, lr);
          }
        }
      }
    }
    l_rnd = l_rnd * alpha + lr;
    if constexpr (T::LSE_FROM_FP32_SUM) l_fp32 = l_fp32 * alpha + ls;
    // rescale after O has absorbed V(j-1)^T P(j-1) (taken against the old max)
    if (resc) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[cb][r] *= alpha;
    }
    // the tile loads of this wave must have landed before the barrier
    // publishes them to the other waves
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  if (n_loc > 0) {
    // prologue: the group's first two K tiles in flight; the V buffer read
    // for the tile before the first in the first iteration is cleared so
    // that 0 * V stays 0.
    issue_rows(kslice, rbk, ld_off_k, ld_off_k_rag, load_of(0), kbuf_of(0));
    if (n_loc > 1) issue_rows(kslice, rbk, ld_off_k, ld_off_k_rag, load_of(1), kbuf_of(1));
    {
      LDS_PTR(u32x4) z = (LDS_PTR(u32x4))vbuf_of(1);
      for (int x = tid & (NT - 1); x < TB / 16; x += NT) z[x] = (u32x4){0u, 0u, 0u, 0u};
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // K(0), K(1) landed
    __syncthreads();
    qk(SA, kbuf_of(0));
    __syncthreads();  // every wave has read K(0) before K(2) overwrites it
    int i = 0;
    for (; i + 1 < n_loc; i += 2) {
      iter(std::integral_constant<int, 0>{}, i, SA, SB, PB, PA);
      iter(std::integral_constant<int, 1>{}, i + 1, SB, SA, PA, PB);
    }
    if (i < n_loc) {
      iter(std::integral_constant<int, 0>{}, i, SA, SB, PB, PA);
      pv(PA, vbuf_of(0));  // drain: the last tile's P is in PA
    } else {
      pv(PB, vbuf_of(1));  // drain: the last tile's P is in PB
    }
  }

  // Key halves with two or more column blocks: both waves of a row wave
  // finish its rows, key half h the column blocks from h * (CB / 2) on.
  constexpr bool KH_SPLIT_END = KH > 1 && CB >= 2;
  auto mine = [&](int cb) { return !KH_SPLIT_END || ((cb >= CB / 2) == (kh == 1)); };
  if constexpr (NG > 1 || (KH > 1 && !KH_SPLIT_END)) {
    // group 1's state to group 0 (key halves: key half 1's to key half 0 of
    // the same row wave): the handing wave writes its O^T accumulators into
    // a tile buffer of its own (free once every wave is past the loop),
    // lane-contiguous 16-byte slots; its max and partial sums go to a small
    // array.  The receiving wave combines: m = max(m0, m1),
    // a_g = 2^(m_g - m), O = a0 O0 + a1 O1, l = a0 l0 + a1 l1.
    __shared__ float lds_state[4][3][64];
    ATTN_POISON_LDS_ARRAY(lds_state);  // before the barrier below
    __syncthreads();
    const int slot = NG > 1 ? wave : rw;  // the pair's buffer and state row
    const bool hands = NG > 1 ? grp == 1 : kh == 1;
    LDS_PTR(char) const mbuf = slot == 0   ? (LDS_PTR(char))lds_k0[NG - 1]
                               : slot == 1 ? (LDS_PTR(char))lds_k1[NG - 1]
                               : slot == 2 ? (LDS_PTR(char))lds_v0[NG - 1]
                                           : (LDS_PTR(char))lds_v1[NG - 1];
    static_assert(CB * 4 * 1024 <= TB, "a wave's accumulators fit one tile buffer");
    if (hands) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(LDS_PTR(f32x4))(mbuf + ((cb * 4 + g) * 64 + lane) * 16) =
              (f32x4){acc_o[cb][4 * g], acc_o[cb][4 * g + 1], acc_o[cb][4 * g + 2],
                      acc_o[cb][4 * g + 3]};
      lds_state[slot][0][lane] = m_run;
      lds_state[slot][1][lane] = l_rnd;
      lds_state[slot][2][lane] = l_fp32;
    }
    __syncthreads();
    if (hands) return;  // the receiving wave finishes the rows
    const float m1 = lds_state[slot][0][lane];
    const float m = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - m);
    const float a1 = __builtin_amdgcn_exp2f(m1 - m);
    m_run = m;
    l_rnd = a0 * l_rnd + a1 * lds_state[slot][1][lane];
    l_fp32 = a0 * l_fp32 + a1 * lds_state[slot][2][lane];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 y = *(LDS_PTR(const f32x4))(mbuf + ((cb * 4 + g) * 64 + lane) * 16);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc_o[cb][4 * g + r] = a0 * acc_o[cb][4 * g + r] + a1 * y[r];
      }
  }
  if constexpr (KH_SPLIT_END) {
    // Each key half writes the column blocks the other one finishes into
    // its own slot (a tile buffer, free once every wave is past the loop)
    // and its max and partial sums into a small array; then both combine
    // the two states the same way, in the order (key half 0, key half 1),
    // so that both get the same sums and the same LSE.
    // [row wave][key half][m, l_rnd, l_fp32][lane]
    __shared__ float lds_st[NW / 2][2][3][64];
    ATTN_POISON_LDS_ARRAY(lds_st);  // before the barrier below
    __syncthreads();
    // slot x = 2 rw + key half: a tile buffer each with 4 waves, half of one
    // with 8 (an even number of column blocks)
    constexpr int SLOT = (CB + 1) / 2 * 4 * 1024;
    static_assert(SLOT * (NW / 4) <= TB, "a slot of half a wave's accumulators fits");
    auto xbuf = [&](int slot) {
      const int x = 2 * rw + slot;
      const int bx = NW == 8 ? x >> 1 : x;
      LDS_PTR(char) const base = bx == 0   ? (LDS_PTR(char))lds_k0[0]
                                 : bx == 1 ? (LDS_PTR(char))lds_k1[0]
                                 : bx == 2 ? (LDS_PTR(char))lds_v0[0]
                                           : (LDS_PTR(char))lds_v1[0];
      return NW == 8 ? base + (x & 1) * SLOT : base;
    };
    // column block cb's place in a slot
    auto cslot = [](int cb) { return cb >= CB / 2 ? cb - CB / 2 : cb; };
    {
      LDS_PTR(char) const w = xbuf(kh);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        if (mine(cb)) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(LDS_PTR(f32x4))(w + ((cslot(cb) * 4 + g) * 64 + lane) * 16) =
              (f32x4){acc_o[cb][4 * g], acc_o[cb][4 * g + 1], acc_o[cb][4 * g + 2],
                      acc_o[cb][4 * g + 3]};
      }
      lds_st[rw][kh][0][lane] = m_run;
      lds_st[rw][kh][1][lane] = l_rnd;
      lds_st[rw][kh][2][lane] = l_fp32;
    }
    __syncthreads();
    const float m0 = lds_st[rw][0][0][lane];
    const float m1 = lds_st[rw][1][0][lane];
    const float m = fmaxf(m0, m1);
    const float a0 = __builtin_amdgcn_exp2f(m0 - m);
    const float a1 = __builtin_amdgcn_exp2f(m1 - m);
    m_run = m;
    l_rnd = a0 * lds_st[rw][0][1][lane] + a1 * lds_st[rw][1][1][lane];
    l_fp32 = a0 * lds_st[rw][0][2][lane] + a1 * lds_st[rw][1][2][lane];
    const float a_own = kh ? a1 : a0;
    const float a_oth = kh ? a0 : a1;
    LDS_PTR(const char) const rbuf = xbuf(kh ^ 1);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      if (!mine(cb)) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 y = *(LDS_PTR(const f32x4))(rbuf + ((cslot(cb) * 4 + g) * 64 + lane) * 16);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc_o[cb][4 * g + r] = a_own * acc_o[cb][4 * g + r] + a_oth * y[r];
      }
    }
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l)
  {
    const int qi = q0w + l32;
    // lanes l and l+32 hold the two halves of the row's keys (all lanes active)
    auto pair_sum = [](float x) {
      auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                false, false);
      return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    };
    const float l_tot = pair_sum(l_rnd);
    const bool has = l_tot > 0.f;
    const float inv = has ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
    float l_lse = l_tot;
    if constexpr (T::LSE_FROM_FP32_SUM) l_lse = pair_sum(l_fp32);
    if (split && qi < p.Sq) {
      // fp32 partial state of this piece (rows of a split block are >= q_split)
      const int ii = qi - p.q_split;
      float* prow = p.part_o +
                    ((((int64_t)piece * p.B + b) * p.sq_split + ii) * p.Hq + hq) * D;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        if (!mine(cb)) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 x;
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] = acc_o[cb][4 * g + r] * inv;
          if (cb * 32 + 8 * g + 4 * hh < p.d) *(f32x4*)(prow + cb * 32 + 8 * g + 4 * hh) = x;
        }
      }
      if (hh == 0 && kh == 0) {
        const float lse = has ? (m_run + __builtin_amdgcn_logf(l_lse)) * LN2 : -INFINITY;
        p.part_lse[(((int64_t)piece * p.B + b) * p.Hq + hq) * p.sq_split + ii] = lse;
      }
    } else if (qi < p.Sq) {
      uint16_t* orow = p.o + (int64_t)b * p.o_sb + (int64_t)qi * p.o_ss + (int64_t)hq * p.o_sh;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        if (!mine(cb)) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x8 x;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x[r] = acc_o[cb][4 * g + r] * inv;
            x[r + 4] = 0.f;
          }
          const i16x8 y = T::cvt(x);
          const u32x2 w = {(unsigned)(uint16_t)y[0] | ((unsigned)(uint16_t)y[1] << 16),
                           (unsigned)(uint16_t)y[2] | ((unsigned)(uint16_t)y[3] << 16)};
          if (cb * 32 + 8 * g + 4 * hh < p.d) *(u32x2*)(orow + cb * 32 + 8 * g + 4 * hh) = w;
        }
      }
      if (p.lse != nullptr && hh == 0 && kh == 0) {
        const float lse = has ? (m_run + __builtin_amdgcn_logf(l_lse)) * LN2 : -INFINITY;
        p.lse[((int64_t)b * p.Hq + hq) * p.Sq + qi] = lse;
      }
    }
  }
}

// ------------------------------------------------------------ merge kernel
//
// Combines partial row states over disjoint key subsets into the state of
// their union: with M = max_p lse_p and w_p = e^(lse_p - M),
//   O = sum_p w_p O_p / sum_p w_p,   LSE = M + ln sum_p w_p.
// This is the online-softmax update of the personal-notes page (section
// "Online Softmax": new max, the factor e^(m_old - m_new) on the old
// denominator and output) with a whole normalised part (O_p, lse_p), i.e. the
// state m = lse_p, l = 1, in the place of a tile.  A part with lse = -inf saw
// no key and gets weight 0; a row that no part saw gets O = 0, LSE = -inf.
//
// Memory-bound: each thread owns 4 consecutive elements of one row (D / 4
// threads per row), so the reads of a part row and the write of O are
// contiguous across the row's threads.
struct MergeParams {
  const void* parts;      // part p, row r: parts + (p * rows + r) * pstride elements
  const float* parts_lse; // part p, (b, h, i): + p * rows + (b * Hq + h) * sq_rows + i - q_first
  uint16_t* o;            // (B, Sq, Hq, D) through the strides below
  int64_t o_sb, o_ss, o_sh;
  float* lse;             // (B, Hq, Sq) or null
  int B, Sq, Hq;
  int d;        // head size (columns written); the kernel is built for D >= d
  int pstride;  // elements per part row: D for a key split's workspace, d for
                // attn_merge's dense parts
  int n_parts;  // parts per row; 0 = the piece count of a key split (below)
  int q_first;  // first merged query row; rows are (b, q_first.. Sq-1, h)
  int sq_rows;  // Sq - q_first
  int64_t rows; // B * sq_rows * Hq
  // key split (n_parts == 0): row i has block_pieces(block_tiles(...)) parts
  int rows_wg, chunk, Sk, off, causal;
};

template <int PDT>
__device__ __forceinline__ f32x4 load_part4(const void* base, int64_t elem) {
  if constexpr (PDT == ATTN_DTYPE_F32) {
    return *(const f32x4*)((const float*)base + elem);
  } else {
    const u32x2 w = *(const u32x2*)((const uint16_t*)base + elem);
    f32x4 x;
    if constexpr (PDT == ATTN_DTYPE_BF16) {
      x[0] = __uint_as_float(w[0] << 16);
      x[1] = __uint_as_float(w[0] & 0xffff0000u);
      x[2] = __uint_as_float(w[1] << 16);
      x[3] = __uint_as_float(w[1] & 0xffff0000u);
    } else {
      // one half at a time: reading both halves of w[1] through a bit cast of
      // the vector element to a two-half vector was compiled to a reuse of
      // w[0] (one dword loaded instead of two)
      x[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[0] & 0xffffu));
      x[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[0] >> 16));
      x[2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[1] & 0xffffu));
      x[3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[1] >> 16));
    }
    return x;
  }
}

template <int PDT, int ODT, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeParams p) {
  constexpr int TPR = D / 4;        // threads per row
  constexpr int RPB = 256 / TPR;    // rows per workgroup
  constexpr float LOG2E = 1.44269504088896340736f;
  if ((int)threadIdx.x >= RPB * TPR) return;  // d = 96: 240 of 256 threads
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  if (r >= p.rows) return;
  const int c = (threadIdx.x % TPR) * 4;
  const bool col_ok = c < p.d;  // columns past a padded head size: no loads, no store
  const int hq = (int)(r % p.Hq);
  const int64_t t = r / p.Hq;
  const int ii = (int)(t % p.sq_rows);
  const int b = (int)(t / p.sq_rows);
  const int qi = p.q_first + ii;
  int n = p.n_parts;
  if (n == 0) {
    const int q0 = (qi / p.rows_wg) * p.rows_wg;
    n = block_pieces(block_tiles(q0, p.rows_wg, p.Sq, p.Sk, p.off, p.causal != 0), p.chunk);
    if (n == 1) return;  // a block that was not split wrote O itself
  }
  const int64_t lrow = ((int64_t)b * p.Hq + hq) * p.sq_rows + ii;
  // one pass over the pieces, MB at a time: the loads of a batch are all in
  // flight together (a decode row can have 16 or more pieces, and few rows
  // give the kernel few waves to hide a round trip per piece), and the
  // running max M rescales the sums when a batch raises it.  MB follows the
  // piece count (2, 4, 8 or 16) so that short merges load no empty slots.
  float M = -INFINITY;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float W = 0.f;
  auto merge = [&](auto mb) {
    constexpr int MB = decltype(mb)::value;
    for (int q0 = 0; q0 < n; q0 += MB) {
      float l[MB];
      f32x4 x[MB];
#pragma unroll
      for (int e = 0; e < MB; ++e) {
        const int q = q0 + e;
        l[e] = -INFINITY;
        x[e] = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (q < n) {
          l[e] = p.parts_lse[(int64_t)q * p.rows + lrow];
          if (col_ok) x[e] = load_part4<PDT>(p.parts, ((int64_t)q * p.rows + r) * p.pstride + c);
        }
      }
      float m = M;
#pragma unroll
      for (int e = 0; e < MB; ++e) m = fmaxf(m, l[e]);
      if (m > -INFINITY) {
        const float a = __builtin_amdgcn_exp2f((M - m) * LOG2E);  // 0 while M = -inf
        W *= a;
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] *= a;
#pragma unroll
        for (int e = 0; e < MB; ++e) {
          const float w = __builtin_amdgcn_exp2f((l[e] - m) * LOG2E);
          W += w;
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[k] = __builtin_fmaf(w, x[e][k], acc[k]);
        }
        M = m;
      }
    }
  };
  if (n <= 2)
    merge(std::integral_constant<int, 2>{});
  else if (n <= 4)
    merge(std::integral_constant<int, 4>{});
  else if (n <= 8)
    merge(std::integral_constant<int, 8>{});
  else
    merge(std::integral_constant<int, 16>{});
  const float inv = W > 0.f ? 1.f / W : 0.f;
  f32x8 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y[e] = acc[e] * inv;
    y[e + 4] = 0.f;
  }
  const i16x8 h = Ty<ODT>::cvt(y);
  const u32x2 w2 = {(unsigned)(uint16_t)h[0] | ((unsigned)(uint16_t)h[1] << 16),
                    (unsigned)(uint16_t)h[2] | ((unsigned)(uint16_t)h[3] << 16)};
  if (col_ok)
    *(u32x2*)(p.o + (int64_t)b * p.o_sb + (int64_t)qi * p.o_ss + (int64_t)hq * p.o_sh + c) = w2;
  if (p.lse != nullptr && c == 0)
    p.lse[((int64_t)b * p.Hq + hq) * p.Sq + qi] =
        W > 0.f ? M + __builtin_amdgcn_logf(W) * LN2 : -INFINITY;
}

// ------------------------------------------------------------ host side
attn_status validate(const void* q, const void* k, const void* v, void* o,
                     const float* lse, int B, int Sq, int Sk, int Hq, int Hkv,
                     int d, float scale, int causal, int dtype) {
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARG;
  if (!sizes_ok(B, Sq, Sk, Hq, Hkv) || d < 1) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u)
    return ATTN_ERR_INVALID_ARG;
  if (((uintptr_t)lse) & 3u) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_DTYPE_F16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!head_size_ok(d)) return ATTN_ERR_UNSUPPORTED;
  // index-space limits: positions and per-tensor row counts stay in int32
  // arithmetic inside the kernel; element offsets are 64-bit.
  if ((int64_t)Sq + Sk >= (1ll << 30)) return ATTN_ERR_INVALID_ARG;
  // a K/V tile (64 rows of Hkv * d * 2 bytes) spans less than 2^31 bytes
  if ((int64_t)Hkv * d * 2 * 64 >= (1ll << 31)) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * Sq * Hq >= (1ll << 31) || (int64_t)B * Sk * Hkv >= (1ll << 31))
    return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

// Element strides (batch, seq, head) of q, k, v, o, in that order.
struct Strides {
  int64_t s[12];
};

Strides dense_strides(int Sq, int Sk, int Hq, int Hkv, int d) {
  const int64_t q[3] = {(int64_t)Sq * Hq * d, (int64_t)Hq * d, d};
  const int64_t k[3] = {(int64_t)Sk * Hkv * d, (int64_t)Hkv * d, d};
  return Strides{{q[0], q[1], q[2], k[0], k[1], k[2], k[0], k[1], k[2], q[0], q[1], q[2]}};
}

// The rows of an output view (sizes n[3], element strides s[3], rows of d
// contiguous elements) are pairwise disjoint: taking the dimensions of more
// than one index by increasing stride, each stride reaches past everything
// the smaller ones span.  (Sufficient, not necessary: a view that fails it
// may still be disjoint, but every dense or sliced layout passes.)
bool rows_disjoint(const int64_t* n, const int64_t* s, int64_t d) {
  int idx[3] = {0, 1, 2};
  for (int a = 0; a < 3; ++a)
    for (int b = a + 1; b < 3; ++b)
      if (s[idx[b]] < s[idx[a]]) {
        const int t = idx[a];
        idx[a] = idx[b];
        idx[b] = t;
      }
  int64_t extent = d;  // elements spanned by the dimensions taken so far
  for (int a = 0; a < 3; ++a) {
    const int i = idx[a];
    if (n[i] <= 1) continue;
    if (s[i] < extent) return false;
    extent += s[i] * (n[i] - 1);
  }
  return true;
}

// Strides: non-negative multiples of 8 elements (16-byte aligned rows), a K
// or V tile (64 key rows) within 2^31 bytes of its first row, and output rows
// that do not overlap (two rows written to one address would race).  q, k
// and v are only read: any strides, 0 (a broadcast) included.
attn_status validate_strides(const int64_t* st, int B, int Sq, int Hq, int d) {
  if (st == nullptr) return ATTN_ERR_INVALID_ARG;
  for (int i = 0; i < 12; ++i)
    if (st[i] < 0 || (st[i] & 7) != 0) return ATTN_ERR_INVALID_ARG;
  if (st[4] * 2 * 64 >= (1ll << 31) || st[7] * 2 * 64 >= (1ll << 31)) return ATTN_ERR_INVALID_ARG;
  const int64_t n_o[3] = {B, Sq, Hq};
  if (!rows_disjoint(n_o, st + 9, d)) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

// Key split.  One workgroup of the attention kernel already draws most of a
// CU's matrix throughput (a second one on the same CU mostly shares it), so
// the automatic choice splits only when the query blocks leave CUs idle
// (fewer blocks than kCUs), and then takes the smallest even piece length
// whose pieces still number at most kCUs: the longest piece sets the time,
// and every piece beyond one per CU would share a CU with another.
constexpr int kCUs = 256;

struct SplitPlan {
  Plan base;
  int chunk;           // tiles per piece, even; 0 = no split
  int npieces;         // pieces of the longest row block
  int q_first;         // first query row of a split block (Sq if none)
  long long grid;      // attention workgroups
  long long merge_rows;
  long long merge_grid;
  size_t lse_offset;   // byte offset of part_lse in the workspace
  size_t ws_bytes;     // workspace bytes (0 = none)
};

// off: the causal offset (query i sees key j <= i + off), Sk - Sq unless
// the caller gives another (a key shard of a longer sequence).  The plan of
// 4-wave workgroups of 32 rows per wave: one or two groups (kh = 1), or
// key halves (kh = 2: 2 row waves x 2 key halves), key split as asked
// (kv_split > 1), automatic (0) or none (1).
SplitPlan make_split_plan_rows(int B, int Sq, int Sk, int Hq, int Hkv, int d, int causal,
                               int kv_split, int off, int kh = 1, int nw = 4) {
  SplitPlan sp{};
  sp.base = make_plan(B, Sq, Sk, Hq, Hkv, d, causal, kh, nw);
  const Plan& pl = sp.base;
  sp.chunk = 0;
  sp.npieces = 1;
  sp.q_first = Sq;
  sp.grid = pl.grid;
  if (pl.grid <= 0) return sp;
  // tiles of the longest row block (the last one: causal rows see the most keys)
  const int nmax = block_tiles((pl.qtiles - 1) * pl.rows_wg, pl.rows_wg, Sq, Sk, off, causal != 0);
  sp.base.ng = kh == 1 && two_groups(pl.grid, d, nmax) ? 2 : 1;
  if (kv_split == 1) return sp;
  int chunk;
  if (kv_split == 0) {
    if ((long long)pl.qtiles * pl.ncols >= kCUs) return sp;
    // the piece count falls as the piece length grows: bisect over even
    // lengths c = 2h for the smallest one with at most kCUs pieces
    auto fits = [&](int c) {
      long long pieces = 0;
      for (int qt = 0; qt < pl.qtiles; ++qt)
        pieces += block_pieces(block_tiles(qt * pl.rows_wg, pl.rows_wg, Sq, Sk, off, causal != 0), c);
      return pieces * pl.ncols <= kCUs;
    };
    int lo = 1, hi = (nmax + 1) / 2;  // fits(2 * hi) holds: one piece per block
    while (lo < hi) {
      const int mid = (lo + hi) / 2;
      if (fits(2 * mid)) hi = mid;
      else lo = mid + 1;
    }
    chunk = 2 * lo;
  } else {
    chunk = (nmax + kv_split - 1) / kv_split;
  }
  chunk += chunk & 1;  // even: a piece starts on buffer 0 of the tile ring
  if (chunk < 2) chunk = 2;
  if (chunk >= nmax) return sp;
  sp.chunk = chunk;
  sp.npieces = block_pieces(nmax, chunk);
  int qt0 = 0;
  while (block_pieces(block_tiles(qt0 * pl.rows_wg, pl.rows_wg, Sq, Sk, off, causal != 0),
                      chunk) == 1)
    ++qt0;  // ends: the last block has npieces > 1 pieces
  sp.q_first = qt0 * pl.rows_wg;
  sp.grid = (long long)sp.npieces * pl.qtiles * pl.ncols;
  {
    long long active = 0;  // workgroups with a piece to run
    for (int qt = 0; qt < pl.qtiles; ++qt)
      active += block_pieces(block_tiles(qt * pl.rows_wg, pl.rows_wg, Sq, Sk, off, causal != 0),
                             chunk);
    sp.base.ng = kh == 1 && two_groups(active * pl.ncols, d, chunk) ? 2 : 1;
  }
  sp.merge_rows = (long long)B * (Sq - sp.q_first) * Hq;
  const int D = padded_head(d);
  const int rpb = 256 / (D / 4);
  sp.merge_grid = (sp.merge_rows + rpb - 1) / rpb;
  const size_t parts = (size_t)sp.npieces * (size_t)sp.merge_rows;
  sp.lse_offset = ((parts * (size_t)D * 4) + 255) & ~(size_t)255;
  sp.ws_bytes = sp.lse_offset + parts * 4;
  if (sp.grid > 0x7fffffffll || sp.merge_grid > 0x7fffffffll) sp.grid = -1;
  return sp;
}

// The launch plan of a forward call.  In the regime of the two groups (at
// most one 4-wave workgroup per CU, at least 8 tiles in the longest block)
// an unsplit call takes the key halves, and so does an automatic one unless
// the key split would cut the longest block into kSplitOverKeyHalves pieces
// or more.  Measured on MI355X against the plan without key halves (one or
// two groups, automatic split): 2 x 1024 causal fp16 23.5 against 28.9 us,
// bf16 19.1 against 22.9, 1280 x 1536 causal 27.8 against 33.0 (2 pieces),
// 1100 x 1100 causal (8 heads) 19.5 against 24.1 (5 pieces), 200 x 520 (GQA,
// 2 x 4 heads) 11.2 against 13.4 (5 pieces); but 512 x 2048 non-causal
// (8 heads) 30.6 against 24.5 and d = 40 1000 x 1000 causal (4 heads) 13.5
// against 12.1, whose split takes 8 pieces: many short pieces and the merge
// beat one long chain of half tiles.
constexpr int kSplitOverKeyHalves = 6;
//
// fp16 at padded head sizes 192 and 256 runs key halves (8 and 4 waves),
// split or not: the 4-wave kernel's hi + lo P halves leave it short of
// registers there, and it spilled into scratch (measured on MI355X, 8K GQA
// heads at d = 256: 14.4 ms against 1.9 ms with key halves, bf16 keeping the
// 4-wave kernel at 1.19 ms, against 1.64 with key halves; 1280 x 1536 causal
// at d = 192 cut into 2 key pieces: 471 us against 50 us unsplit).
SplitPlan make_split_plan(int B, int Sq, int Sk, int Hq, int Hkv, int d, int causal,
                          int kv_split, int off, int dtype) {
  const bool f16_wide = dtype == ATTN_DTYPE_F16 && padded_head(d) > 128;
  const int kh0 = f16_wide ? 2 : 1;
  const int nw0 = f16_wide && padded_head(d) == 192 ? 8 : 4;
  const SplitPlan sp =
      make_split_plan_rows(B, Sq, Sk, Hq, Hkv, d, causal, kv_split, off, kh0, nw0);
  if (sp.grid > 0 && sp.chunk == 0 && padded_head(d) == 192) {
    // unsplit at d = 192: the same grid in 8-wave workgroups of key halves
    SplitPlan e = sp;
    e.base = make_plan(B, Sq, Sk, Hq, Hkv, d, causal, 2, 8);
    e.base.ng = 1;
    e.grid = e.base.grid;
    return e;
  }
  if (kv_split > 1 || sp.grid <= 0 || sp.npieces >= kSplitOverKeyHalves) return sp;
  const Plan pl = make_plan(B, Sq, Sk, Hq, Hkv, d, causal);
  const int nmax = block_tiles((pl.qtiles - 1) * pl.rows_wg, pl.rows_wg, Sq, Sk, off, causal != 0);
  if (!key_halves(pl.grid, d, nmax)) return sp;
  SplitPlan k{};
  k.base = make_plan(B, Sq, Sk, Hq, Hkv, d, causal, 2);
  if (k.base.grid <= 0) return sp;
  k.base.ng = 1;
  k.chunk = 0;
  k.npieces = 1;
  k.q_first = Sq;
  k.grid = k.base.grid;
  return k;
}

template <int PDT, int ODT>
hipError_t launch_merge(int d, long long grid, const MergeParams& mp, hipStream_t st) {
  const dim3 g((unsigned)grid), b(256);
  switch (padded_head(d)) {
    case 32: hipLaunchKernelGGL((attn_merge_kernel<PDT, ODT, 32>), g, b, 0, st, mp); break;
    case 64: hipLaunchKernelGGL((attn_merge_kernel<PDT, ODT, 64>), g, b, 0, st, mp); break;
    case 96: hipLaunchKernelGGL((attn_merge_kernel<PDT, ODT, 96>), g, b, 0, st, mp); break;
    case 128: hipLaunchKernelGGL((attn_merge_kernel<PDT, ODT, 128>), g, b, 0, st, mp); break;
    case 192: hipLaunchKernelGGL((attn_merge_kernel<PDT, ODT, 192>), g, b, 0, st, mp); break;
    default: hipLaunchKernelGGL((attn_merge_kernel<PDT, ODT, 256>), g, b, 0, st, mp); break;
  }
  return hipGetLastError();
}

hipError_t launch_merge_any(int parts_dtype, int dtype, int d, long long grid,
                            const MergeParams& mp, hipStream_t st) {
  if (dtype == ATTN_DTYPE_BF16) {
    if (parts_dtype == ATTN_DTYPE_F32) return launch_merge<ATTN_DTYPE_F32, ATTN_DTYPE_BF16>(d, grid, mp, st);
    if (parts_dtype == ATTN_DTYPE_BF16) return launch_merge<ATTN_DTYPE_BF16, ATTN_DTYPE_BF16>(d, grid, mp, st);
    return launch_merge<ATTN_DTYPE_F16, ATTN_DTYPE_BF16>(d, grid, mp, st);
  }
  if (parts_dtype == ATTN_DTYPE_F32) return launch_merge<ATTN_DTYPE_F32, ATTN_DTYPE_F16>(d, grid, mp, st);
  if (parts_dtype == ATTN_DTYPE_BF16) return launch_merge<ATTN_DTYPE_BF16, ATTN_DTYPE_F16>(d, grid, mp, st);
  return launch_merge<ATTN_DTYPE_F16, ATTN_DTYPE_F16>(d, grid, mp, st);
}

template <int DT, int D, bool CAUSAL>
hipError_t launch_t(const Plan& pl, long long nwg, const Params& p, hipStream_t st) {
  const dim3 grid((unsigned)nwg), block(pl.ng * pl.nw * 64);
  // the tile buffers are static LDS (pl.lds_bytes reports their size)
  if constexpr (D <= 128) {
    if (pl.ng == 2) {
      hipLaunchKernelGGL((attn_fwd_pipe_kernel<DT, D, CAUSAL, 2, 1, 4>), grid, block, 0, st, p);
      return hipGetLastError();
    }
    if (pl.kh == 2 && pl.nw == 4) {
      hipLaunchKernelGGL((attn_fwd_pipe_kernel<DT, D, CAUSAL, 1, 2, 4>), grid, block, 0, st, p);
      return hipGetLastError();
    }
  }
  if constexpr (D == 256) {
    if (pl.kh == 2 && pl.nw == 4) {
      hipLaunchKernelGGL((attn_fwd_pipe_kernel<DT, D, CAUSAL, 1, 2, 4>), grid, block, 0, st, p);
      return hipGetLastError();
    }
  }
  if constexpr (D == 192) {
    if (pl.kh == 2 && pl.nw == 8) {
      hipLaunchKernelGGL((attn_fwd_pipe_kernel<DT, D, CAUSAL, 1, 2, 8>), grid, block, 0, st, p);
      return hipGetLastError();
    }
  }
  if constexpr (DT == ATTN_DTYPE_F16 && D > 128) {
    // fp16 above 128 always plans key halves; the 4-wave kernel is not built
    return hipErrorInvalidConfiguration;
  } else {
    hipLaunchKernelGGL((attn_fwd_pipe_kernel<DT, D, CAUSAL, 1, 1, 4>), grid, block, 0, st, p);
    return hipGetLastError();
  }
}

template <int DT, int D>
hipError_t launch_c(bool causal, const Plan& pl, long long nwg, const Params& p,
                    hipStream_t st) {
  return causal ? launch_t<DT, D, true>(pl, nwg, p, st) : launch_t<DT, D, false>(pl, nwg, p, st);
}

template <int DT>
hipError_t launch_d(int d, bool causal, const Plan& pl, long long nwg, const Params& p,
                    hipStream_t st) {
  switch (padded_head(d)) {
    case 32: return launch_c<DT, 32>(causal, pl, nwg, p, st);
    case 64: return launch_c<DT, 64>(causal, pl, nwg, p, st);
    case 96: return launch_c<DT, 96>(causal, pl, nwg, p, st);
    case 128: return launch_c<DT, 128>(causal, pl, nwg, p, st);
    case 192: return launch_c<DT, 192>(causal, pl, nwg, p, st);
    default: return launch_c<DT, 256>(causal, pl, nwg, p, st);
  }
}

Params fill_params(const Plan& pl, const void* q, const void* k, const void* v, void* o,
                   float* lse, int B, int Sq, int Sk, int Hq, int Hkv, int d, float scale,
                   const Strides& st, int off) {
  Params p{};
  p.q_sb = st.s[0], p.q_ss = st.s[1], p.q_sh = st.s[2];
  p.k_sb = st.s[3], p.k_ss = st.s[4], p.k_sh = st.s[5];
  p.v_sb = st.s[6], p.v_ss = st.s[7], p.v_sh = st.s[8];
  p.o_sb = st.s[9], p.o_ss = st.s[10], p.o_sh = st.s[11];
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)o;
  p.lse = lse;
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
  p.xcd_qsplit = pl.xcd_qsplit;
  p.off = off;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  p.chunk = 0;
  p.q_split = Sq;
  p.sq_split = 0;
  p.part_o = nullptr;
  p.part_lse = nullptr;
  return p;
}

hipError_t launch_attn(int dtype, int d, int causal, const Plan& pl, long long nwg,
                       const Params& p, hipStream_t st) {
  return dtype == ATTN_DTYPE_BF16 ? launch_d<ATTN_DTYPE_BF16>(d, causal != 0, pl, nwg, p, st)
                                  : launch_d<ATTN_DTYPE_F16>(d, causal != 0, pl, nwg, p, st);
}

// The forward pass with strides and an optional key split.  Arguments are
// validated by the callers.
// Decode shapes (every query row of a kv head fits one wave): the decode
// kernel, with its key range cut into pieces over workgroups when the
// (batch, kv head) pairs are too few, merged by the merge kernel.
//
// A paged K/V cache (pg != null) replaces the dense key range of each
// sequence by a block table and a length; Sk is then the longest length the
// plan covers.
struct PagedKV {
  const int* block_table;
  const int* seqlens;
  int num_blocks, block_size, max_blocks;
};

attn_status run_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int Sq, int Sk, int Hq, int Hkv, int d, float scale, int causal,
                       int dtype, const Strides& st, int kv_split, void* workspace,
                       size_t workspace_bytes, hipStream_t hs, const PagedKV* pg, int off) {
  const DecodePlan dp = make_decode_plan(B, Sq, Sk, Hq, Hkv, d, kv_split);
  if (dp.grid <= 0) return ATTN_ERR_INVALID_ARG;
  if (dp.pieces > 1 && (workspace == nullptr || ((uintptr_t)workspace & 255u) ||
                        workspace_bytes < dp.ws_bytes))
    return ATTN_ERR_INVALID_ARG;
  DecodeArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.q_sb = st.s[0], a.q_ss = st.s[1], a.q_sh = st.s[2];
  a.k_sb = st.s[3], a.k_ss = st.s[4], a.k_sh = st.s[5];
  a.v_sb = st.s[6], a.v_ss = st.s[7], a.v_sh = st.s[8];
  a.o_sb = st.s[9], a.o_ss = st.s[10], a.o_sh = st.s[11];
  a.B = B;
  a.Sq = Sq;
  a.Sk = Sk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.off = off;
  a.piece_tiles = dp.piece_tiles;
  a.rgroups = dp.rgroups;
  a.ucols = dp.ucols;
  a.grid = dp.grid;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  if (pg != nullptr) {
    a.block_table = pg->block_table;
    a.seqlens = pg->seqlens;
    a.num_blocks = pg->num_blocks;
    a.block_size = pg->block_size;
    a.max_blocks = pg->max_blocks;
  }
  if (dp.pieces > 1) {
    a.part_o = (float*)workspace;
    a.part_lse = (float*)((char*)workspace + dp.lse_offset);
  }
  hipError_t e = launch_decode(dtype, d, causal, a, hs);
  if (e != hipSuccess) return ATTN_ERR_LAUNCH;
  if (dp.pieces == 1) return ATTN_OK;
  MergeParams mp{};
  mp.parts = a.part_o;
  mp.parts_lse = a.part_lse;
  mp.o = (uint16_t*)o;
  mp.o_sb = a.o_sb, mp.o_ss = a.o_ss, mp.o_sh = a.o_sh;
  mp.lse = lse;
  mp.B = B;
  mp.Sq = Sq;
  mp.Hq = Hq;
  mp.d = d;
  mp.pstride = padded_head(d);
  mp.n_parts = dp.pieces;
  mp.q_first = 0;
  mp.sq_rows = Sq;
  mp.rows = (long long)B * Sq * Hq;
  const int rpb = 256 / (padded_head(d) / 4);
  e = launch_merge_any(ATTN_DTYPE_F32, dtype, d, (mp.rows + rpb - 1) / rpb, mp, hs);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status run_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Sq, int Sk, int Hq, int Hkv, int d, float scale, int causal,
                        int dtype, const Strides& st, int kv_split, void* workspace,
                        size_t workspace_bytes, hipStream_t hs, int off) {
  if (decode_eligible(Sq, Hq, Hkv, d))
    return run_decode(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, scale, causal, dtype, st, kv_split,
                      workspace, workspace_bytes, hs, nullptr, off);
  const SplitPlan sp = make_split_plan(B, Sq, Sk, Hq, Hkv, d, causal, kv_split, off, dtype);
  if (sp.grid <= 0) return ATTN_ERR_INVALID_ARG;
  if (sp.chunk > 0 && (workspace == nullptr || ((uintptr_t)workspace & 255u) ||
                       workspace_bytes < sp.ws_bytes))
    return ATTN_ERR_INVALID_ARG;
  Params p = fill_params(sp.base, q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, scale, st, off);
  if (sp.chunk == 0) {
    hipError_t e = launch_attn(dtype, d, causal, sp.base, sp.grid, p, hs);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
  }
  p.chunk = sp.chunk;
  if (p.xcd_qsplit > 0) {  // pieces follow the column-major order
    p.xcd_qsplit = 0;
    p.xcd_cols = (p.ncols % 8 == 0) ? p.ncols / 8 : 0;
  }
  p.q_split = sp.q_first;
  p.sq_split = Sq - sp.q_first;
  p.part_o = (float*)workspace;
  p.part_lse = (float*)((char*)workspace + sp.lse_offset);
  hipError_t e = launch_attn(dtype, d, causal, sp.base, sp.grid, p, hs);
  if (e != hipSuccess) return ATTN_ERR_LAUNCH;
  MergeParams mp{};
  mp.parts = p.part_o;
  mp.parts_lse = p.part_lse;
  mp.o = (uint16_t*)o;
  mp.o_sb = p.o_sb, mp.o_ss = p.o_ss, mp.o_sh = p.o_sh;
  mp.lse = lse;
  mp.B = B;
  mp.Sq = Sq;
  mp.Hq = Hq;
  mp.d = d;
  mp.pstride = padded_head(d);
  mp.n_parts = 0;
  mp.q_first = sp.q_first;
  mp.sq_rows = Sq - sp.q_first;
  mp.rows = sp.merge_rows;
  mp.rows_wg = sp.base.rows_wg;
  mp.chunk = sp.chunk;
  mp.Sk = Sk;
  mp.off = off;
  mp.causal = causal;
  e = launch_merge_any(ATTN_DTYPE_F32, dtype, d, sp.merge_grid, mp, hs);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// ------------------------------------------------------------ static scratch
//
// attn_fwd_split_noalloc keeps the key split's partial states in this
// library-owned device array instead of a caller workspace.  Each GPU the
// library runs on holds its own copy until the process ends.  Host code
// never uses the array's name as a device address: at the first call on a
// device, with that device current, hipGetSymbolAddress gives that device's
// address, which is kept per device and passed to the kernels.
constexpr size_t kScratchBytes = ATTN_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the device that runs `stream` (the current device
// for the null stream), looked up once per device.
attn_status scratch_for_stream(hipStream_t stream, void** out) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return ATTN_ERR_LAUNCH;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return ATTN_ERR_LAUNCH;
  }
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> guard(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return ATTN_ERR_LAUNCH;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return ATTN_ERR_LAUNCH;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || ptr == nullptr) return ATTN_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o,
                                   float* lse, int B, int Sq, int Sk, int Hq, int Hkv, int d,
                                   float scale, int causal, int dtype, int kv_split,
                                   void* stream) {
  attn_status st = attn_fwd_check(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, scale, causal, dtype);
  if (st != ATTN_OK) return st;
  if (kv_split < 0) return ATTN_ERR_INVALID_ARG;
  size_t need = 0;
  st = attn_fwd_split_workspace(B, Sq, Sk, Hq, Hkv, d, causal, dtype, kv_split, &need);
  if (st != ATTN_OK) return st;
  if (need > kScratchBytes) return ATTN_ERR_SCRATCH;  // before any device call
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_for_stream((hipStream_t)stream, &ws);
    if (st != ATTN_OK) return st;
  }
  return run_forward(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, scale, causal, dtype,
                     dense_strides(Sq, Sk, Hq, Hkv, d), kv_split, ws, need, (hipStream_t)stream,
                     Sk - Sq);
}

attn_status attn_fwd_check(const void* q, const void* k, const void* v, void* o,
                           float* lse, int B, int Sq, int Sk, int Hq, int Hkv,
                           int d, float scale, int causal, int dtype) {
  attn_status st = validate(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, scale, causal, dtype);
  if (st != ATTN_OK) return st;
  const Plan pl = make_plan(B, Sq, Sk, Hq, Hkv, d, causal);
  if (pl.grid <= 0) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

attn_status attn_fwd_plan(int B, int Sq, int Sk, int Hq, int Hkv, int d,
                          int causal, int dtype, int* out, int n) {
  // validation with stand-in aligned pointers (sizes only)
  static const uint64_t dummy[2] = {0, 0};
  const void* pp = (const void*)(((uintptr_t)dummy + 15) & ~(uintptr_t)15);
  attn_status st = attn_fwd_check(pp, pp, pp, (void*)pp, nullptr, B, Sq, Sk, Hq,
                                  Hkv, d, 1.0f, causal, dtype);
  if (st != ATTN_OK) return st;
  // attn_fwd: no key split
  const Plan pl = make_split_plan(B, Sq, Sk, Hq, Hkv, d, causal, 1, Sk - Sq, dtype).base;
  int vals[11] = {pl.grid, pl.ng * pl.nw * 64, pl.rows_wg, BC, pl.gh, 32 * pl.qb,
                  pl.ng * pl.lds_bytes, pl.xcd_cols > 0 || pl.xcd_qsplit > 0 ? 1 : 0,
                  pl.pipelined, 0, pl.kh == 2 ? 1 : 0};
  if (decode_eligible(Sq, Hq, Hkv, d)) {
    // the decode kernel, unsplit: a workgroup per (batch, kv head) with all
    // g * Sq rows in one wave, DEC_WAVES waves over the keys
    const int g = Hq / Hkv;
    const DecodePlan dp = make_decode_plan(B, Sq, Sk, Hq, Hkv, d, 1);
    if (dp.grid <= 0) return ATTN_ERR_INVALID_ARG;
    const int vals_dec[10] = {(int)dp.grid, DEC_WAVES * 64, Sq, 32, g, 32,
                              DEC_WAVES * 2 * 32 * padded_head(d) * 2, 0, 0, 1};
    for (int i = 0; i < 10; ++i) vals[i] = vals_dec[i];
    vals[10] = 0;
  }
  for (int i = 0; i < n && i < 11; ++i) out[i] = vals[i];
  return ATTN_OK;
}

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o,
                     float* lse, int B, int Sq, int Sk, int Hq, int Hkv, int d,
                     float scale, int causal, int dtype, void* stream) {
  attn_status st = attn_fwd_check(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, scale, causal, dtype);
  if (st != ATTN_OK) return st;
  return run_forward(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, scale, causal, dtype,
                     dense_strides(Sq, Sk, Hq, Hkv, d), 1, nullptr, 0, (hipStream_t)stream, Sk - Sq);
}

attn_status attn_fwd_split_plan(int B, int Sq, int Sk, int Hq, int Hkv, int d, int causal,
                                int dtype, int kv_split, int* out, int n) {
  if (kv_split < 0) return ATTN_ERR_INVALID_ARG;
  int base[9];
  attn_status st = attn_fwd_plan(B, Sq, Sk, Hq, Hkv, d, causal, dtype, base, 9);
  if (st != ATTN_OK) return st;
  if (decode_eligible(Sq, Hq, Hkv, d)) {
    const DecodePlan dp = make_decode_plan(B, Sq, Sk, Hq, Hkv, d, kv_split);
    if (dp.grid <= 0) return ATTN_ERR_INVALID_ARG;
    const long long mrows = (long long)B * Sq * Hq;
    const int rpb = 256 / (padded_head(d) / 4);
    const int vals[7] = {(int)dp.grid, dp.pieces, dp.pieces > 1 ? dp.piece_tiles * 32 : 0,
                         dp.pieces > 1 ? 0 : Sq,
                         dp.pieces > 1 ? (int)((mrows + rpb - 1) / rpb) : 0, DEC_WAVES * 64, 0};
    for (int i = 0; i < n && i < 7; ++i) out[i] = vals[i];
    return ATTN_OK;
  }
  const SplitPlan sp = make_split_plan(B, Sq, Sk, Hq, Hkv, d, causal, kv_split, Sk - Sq, dtype);
  if (sp.grid <= 0) return ATTN_ERR_INVALID_ARG;
  const int vals[7] = {(int)sp.grid, sp.npieces, sp.chunk * BC, sp.q_first,
                       (int)sp.merge_grid, sp.base.ng * sp.base.nw * 64,
                       sp.base.kh == 2 ? 1 : 0};
  for (int i = 0; i < n && i < 7; ++i) out[i] = vals[i];
  return ATTN_OK;
}

attn_status attn_fwd_split_workspace(int B, int Sq, int Sk, int Hq, int Hkv, int d,
                                     int causal, int dtype, int kv_split, size_t* bytes) {
  if (bytes == nullptr) return ATTN_ERR_INVALID_ARG;
  int out[5];
  attn_status st = attn_fwd_split_plan(B, Sq, Sk, Hq, Hkv, d, causal, dtype, kv_split, out, 5);
  if (st != ATTN_OK) return st;
  *bytes = decode_eligible(Sq, Hq, Hkv, d)
               ? make_decode_plan(B, Sq, Sk, Hq, Hkv, d, kv_split).ws_bytes
               : make_split_plan(B, Sq, Sk, Hq, Hkv, d, causal, kv_split, Sk - Sq, dtype).ws_bytes;
  return ATTN_OK;
}

attn_status attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Sq, int Sk, int Hq, int Hkv, int d, float scale,
                           int causal, int dtype, int kv_split, void* workspace,
                           size_t workspace_bytes, void* stream) {
  attn_status st = attn_fwd_check(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, scale, causal, dtype);
  if (st != ATTN_OK) return st;
  if (kv_split < 0) return ATTN_ERR_INVALID_ARG;
  return run_forward(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, scale, causal, dtype,
                     dense_strides(Sq, Sk, Hq, Hkv, d), kv_split, workspace, workspace_bytes,
                     (hipStream_t)stream, Sk - Sq);
}

attn_status attn_fwd_strided_check(const void* q, const void* k, const void* v, void* o,
                                   float* lse, int B, int Sq, int Sk, int Hq, int Hkv, int d,
                                   float scale, int causal, int dtype,
                                   const long long* strides) {
  attn_status st = attn_fwd_check(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, scale, causal, dtype);
  if (st != ATTN_OK) return st;
  return validate_strides((const int64_t*)strides, B, Sq, Hq, d);
}

attn_status attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int Sq, int Sk, int Hq, int Hkv, int d, float scale,
                             int causal, int dtype, const long long* strides, int kv_split,
                             void* workspace, size_t workspace_bytes, void* stream) {
  attn_status st = attn_fwd_strided_check(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, scale, causal,
                                          dtype, strides);
  if (st != ATTN_OK) return st;
  if (kv_split < 0) return ATTN_ERR_INVALID_ARG;
  Strides sv;
  for (int i = 0; i < 12; ++i) sv.s[i] = strides[i];
  return run_forward(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, scale, causal, dtype, sv, kv_split,
                     workspace, workspace_bytes, (hipStream_t)stream, Sk - Sq);
}

attn_status attn_fwd_causal_offset_check(const void* q, const void* k, const void* v, void* o,
                                         float* lse, int B, int Sq, int Sk, int Hq, int Hkv,
                                         int d, float scale, long long causal_offset, int dtype,
                                         const long long* strides) {
  attn_status st = attn_fwd_check(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, scale, 1, dtype);
  if (st != ATTN_OK) return st;
  if (causal_offset <= -(1ll << 30) || causal_offset >= (1ll << 30)) return ATTN_ERR_INVALID_ARG;
  return strides != nullptr ? validate_strides((const int64_t*)strides, B, Sq, Hq, d) : ATTN_OK;
}

attn_status attn_fwd_causal_offset_workspace(int B, int Sq, int Sk, int Hq, int Hkv, int d,
                                             long long causal_offset, int dtype, int kv_split,
                                             size_t* bytes) {
  if (bytes == nullptr || kv_split < 0) return ATTN_ERR_INVALID_ARG;
  int out[1];
  attn_status st = attn_fwd_plan(B, Sq, Sk, Hq, Hkv, d, 1, dtype, out, 1);
  if (st != ATTN_OK) return st;
  if (causal_offset <= -(1ll << 30) || causal_offset >= (1ll << 30)) return ATTN_ERR_INVALID_ARG;
  if (decode_eligible(Sq, Hq, Hkv, d)) {
    const DecodePlan dp = make_decode_plan(B, Sq, Sk, Hq, Hkv, d, kv_split);
    if (dp.grid <= 0) return ATTN_ERR_INVALID_ARG;
    *bytes = dp.ws_bytes;
    return ATTN_OK;
  }
  const SplitPlan sp = make_split_plan(B, Sq, Sk, Hq, Hkv, d, 1, kv_split, (int)causal_offset, dtype);
  if (sp.grid <= 0) return ATTN_ERR_INVALID_ARG;
  *bytes = sp.ws_bytes;
  return ATTN_OK;
}

attn_status attn_fwd_causal_offset(const void* q, const void* k, const void* v, void* o,
                                   float* lse, int B, int Sq, int Sk, int Hq, int Hkv, int d,
                                   float scale, long long causal_offset, int dtype,
                                   const long long* strides, int kv_split, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  attn_status st = attn_fwd_causal_offset_check(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, scale,
                                                causal_offset, dtype, strides);
  if (st != ATTN_OK) return st;
  if (kv_split < 0) return ATTN_ERR_INVALID_ARG;
  Strides sv = dense_strides(Sq, Sk, Hq, Hkv, d);
  if (strides != nullptr)
    for (int i = 0; i < 12; ++i) sv.s[i] = strides[i];
  return run_forward(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, scale, 1, dtype, sv, kv_split,
                     workspace, workspace_bytes, (hipStream_t)stream, (int)causal_offset);
}

attn_status attn_merge_check(const void* o_parts, const float* lse_parts, int n_parts,
                             int parts_dtype, int B, int Sq, int Hq, int d, void* o,
                             float* lse, int dtype) {
  if (!o_parts || !lse_parts || !o) return ATTN_ERR_INVALID_ARG;
  if (n_parts < 1 || B < 1 || Sq < 1 || Hq < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
  if (parts_dtype != ATTN_DTYPE_F32 && parts_dtype != ATTN_DTYPE_F16 &&
      parts_dtype != ATTN_DTYPE_BF16)
    return ATTN_ERR_UNSUPPORTED;
  if (dtype != ATTN_DTYPE_F16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!head_size_ok(d)) return ATTN_ERR_UNSUPPORTED;
  const uintptr_t need = parts_dtype == ATTN_DTYPE_F32 ? 15u : 7u;
  if (((uintptr_t)o_parts & need) || ((uintptr_t)o & 7u) || ((uintptr_t)lse_parts & 3u) ||
      ((uintptr_t)lse & 3u))
    return ATTN_ERR_INVALID_ARG;
  const long long rows = (long long)B * Sq * Hq;
  if (rows >= (1ll << 31) || rows * n_parts >= (1ll << 40)) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

attn_status attn_merge(const void* o_parts, const float* lse_parts, int n_parts,
                       int parts_dtype, int B, int Sq, int Hq, int d, void* o, float* lse,
                       int dtype, void* stream) {
  attn_status st = attn_merge_check(o_parts, lse_parts, n_parts, parts_dtype, B, Sq, Hq, d, o,
                                    lse, dtype);
  if (st != ATTN_OK) return st;
  MergeParams mp{};
  mp.parts = o_parts;
  mp.parts_lse = lse_parts;
  mp.o = (uint16_t*)o;
  mp.o_sb = (int64_t)Sq * Hq * d, mp.o_ss = (int64_t)Hq * d, mp.o_sh = d;
  mp.lse = lse;
  mp.B = B;
  mp.Sq = Sq;
  mp.Hq = Hq;
  mp.d = d;
  mp.pstride = d;
  mp.n_parts = n_parts;
  mp.q_first = 0;
  mp.sq_rows = Sq;
  mp.rows = (long long)B * Sq * Hq;
  const int rpb = 256 / (padded_head(d) / 4);
  const long long grid = (mp.rows + rpb - 1) / rpb;
  hipError_t e = launch_merge_any(parts_dtype, dtype, d, grid, mp, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status attn_decode_paged_check(const void* q, const void* k_cache, const void* v_cache,
                                    const int* block_table, const int* seqlens, void* o,
                                    float* lse, int B, int Sq, int Hq, int Hkv, int d,
                                    int num_blocks, int block_size, int max_blocks,
                                    int max_seqlen, float scale, int causal, int dtype) {
  if (!q || !k_cache || !v_cache || !block_table || !seqlens || !o) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Sq < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (num_blocks < 1 || max_blocks < 1 || block_size < 16 || block_size % 16 != 0)
    return ATTN_ERR_INVALID_ARG;
  if (max_seqlen < 1 || (long long)max_seqlen > (long long)max_blocks * block_size)
    return ATTN_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)o) & 15u)
    return ATTN_ERR_INVALID_ARG;
  if (((uintptr_t)block_table | (uintptr_t)seqlens | (uintptr_t)lse) & 3u)
    return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_DTYPE_F16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!head_size_ok(d) || !decode_eligible(Sq, Hq, Hkv, d)) return ATTN_ERR_UNSUPPORTED;
  // index space: query rows (merge), block-table entries, pool elements
  if ((long long)B * Sq * Hq >= (1ll << 31) || (long long)B * max_blocks >= (1ll << 31) ||
      (long long)num_blocks * block_size >= (1ll << 31) ||
      (long long)Hkv * d * 2 * 64 >= (1ll << 31))
    return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

attn_status attn_decode_paged_workspace(int B, int Sq, int Hq, int Hkv, int d, int max_seqlen,
                                        int kv_split, size_t* bytes) {
  if (bytes == nullptr || kv_split < 0 || B < 1 || Sq < 1 || Hkv < 1 || Hq < 1 ||
      Hq % Hkv != 0 || max_seqlen < 1)
    return ATTN_ERR_INVALID_ARG;
  if (!head_size_ok(d) || !decode_eligible(Sq, Hq, Hkv, d)) return ATTN_ERR_UNSUPPORTED;
  const DecodePlan dp = make_decode_plan(B, Sq, max_seqlen, Hq, Hkv, d, kv_split);
  if (dp.grid <= 0) return ATTN_ERR_INVALID_ARG;
  *bytes = dp.ws_bytes;
  return ATTN_OK;
}

attn_status attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                              const int* block_table, const int* seqlens, void* o, float* lse,
                              int B, int Sq, int Hq, int Hkv, int d, int num_blocks,
                              int block_size, int max_blocks, int max_seqlen, float scale,
                              int causal, int dtype, int kv_split, void* workspace,
                              size_t workspace_bytes, void* stream) {
  attn_status st = attn_decode_paged_check(q, k_cache, v_cache, block_table, seqlens, o, lse, B,
                                           Sq, Hq, Hkv, d, num_blocks, block_size, max_blocks,
                                           max_seqlen, scale, causal, dtype);
  if (st != ATTN_OK) return st;
  if (kv_split < 0) return ATTN_ERR_INVALID_ARG;
  // q, o dense (B, Sq, Hq, d); pool rows (block, slot) hold Hkv heads of d
  Strides sv = dense_strides(Sq, 1, Hq, Hkv, d);
  sv.s[3] = 0, sv.s[4] = (int64_t)Hkv * d, sv.s[5] = d;
  sv.s[6] = 0, sv.s[7] = (int64_t)Hkv * d, sv.s[8] = d;
  const PagedKV pg{block_table, seqlens, num_blocks, block_size, max_blocks};
  return run_decode(q, k_cache, v_cache, o, lse, B, Sq, max_seqlen, Hq, Hkv, d, scale, causal,
                    dtype, sv, kv_split, workspace, workspace_bytes, (hipStream_t)stream, &pg,
                    max_seqlen - Sq);
}

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head size or dtype";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_SCRATCH:
      return "the key split needs more than the library's static scratch (16 MiB)";
    default: return "unknown status";
  }
}

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

}  // extern "C"
