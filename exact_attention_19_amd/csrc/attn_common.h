// Device and host pieces shared by the forward and backward attention
// kernels for gfx950 (CDNA4): vector types, the 16-bit MFMA wrappers, the
// key order that lets an S^T accumulator feed the next MFMA as its B operand,
// the column-blocked LDS tile layout with its two fragment read patterns and
// the direct-to-LDS tile load, and the query-block launch plan.
//
// Internal header of the library (not part of the C ABI in attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn.h"

// ------------------------------------------------------------ decode path
// Arguments of the decode kernel (attn_decode.hip): g * Sq <= 32 query rows
// per kv head, all in one wave.  In a named namespace: the launcher is
// shared between translation units.
namespace attn_detail {
struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int B, Sq, Sk, Hq, Hkv;
  int d;             // head size; the kernel is built for D >= d (padded)
  int off;           // causal: query i sees key j <= i + off (dense keys;
                     // a paged sequence of length L uses L - Sq)
  int piece_tiles;   // 32-key tiles per piece
  int rgroups;       // 32-row groups per kv head: ceil(g * Sq / 32)
  int ucols;         // workgroups per piece: B * Hkv, or with several row
                     // groups B * Hkv rounded up to 8, times rgroups
  long long grid;    // ucols * pieces
  float scale_log2;
  float* part_o;     // pieces > 1: [piece][b][i][h][d] fp32, else null
  float* part_lse;   // pieces > 1: [piece][b][h][i]
  // paged K/V cache (block_table != null): K and V rows of token t of
  // sequence b are row (block_table[b][t / block_size] * block_size +
  // t % block_size) of the pools, whose rows are k_ss / v_ss elements apart
  // (k_sb, v_sb unused); sequence b has min(seqlens[b], Sk) keys, and Sk
  // is at most max_blocks * block_size; block_size is a multiple of 16
  const int* block_table;  // [B][max_blocks]
  const int* seqlens;      // [B]
  int block_size, max_blocks, num_blocks;
};

// Launch of the decode kernel (defined in attn_decode.hip).
__attribute__((visibility("hidden"))) hipError_t launch_decode(int dtype, int d, int causal,
                                                               const DecodeArgs& a,
                                                               hipStream_t st);
}  // namespace attn_detail

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

#define LDS_PTR(T) __attribute__((address_space(3))) T*

// LDS poison (debug builds, -DATTN_POISON_LDS): every kernel starts by filling
// each of its LDS arrays with 0xFF bytes, a NaN in fp32, fp16 and bf16 alike,
// so that a read of LDS the kernel has not written first shows up as NaN in
// its outputs.  Product builds compile it away.  Four-byte stores: every LDS
// array is a whole number of words, whatever its alignment.
#ifdef ATTN_POISON_LDS
template <int BYTES>
__device__ __forceinline__ void poison_lds(LDS_PTR(char) p) {
  static_assert(BYTES % 4 == 0, "LDS arrays are whole words");
  for (int i = (int)threadIdx.x * 4; i < BYTES; i += (int)blockDim.x * 4)
    *(LDS_PTR(unsigned))(p + i) = ~0u;
}
#define ATTN_POISON_LDS_ARRAY(a) poison_lds<sizeof(a)>((LDS_PTR(char))(a))
#define ATTN_POISON_LDS_DONE() __syncthreads()
#else
#define ATTN_POISON_LDS_ARRAY(a) ((void)0)
#define ATTN_POISON_LDS_DONE() ((void)0)
#endif
#define GLOBAL_PTR(T) __attribute__((address_space(1))) T*

constexpr int BC = 64;              // keys per K/V tile
constexpr float LN2 = 0.693147180559945309417f;

// ------------------------------------------------------------ head sizes
// Any head size d that is a multiple of 8 from 8 to 256 runs on the kernels
// built for the next size up in this list (the CuTe DSL example pads its
// head size up to a multiple of 32 the same way): the tile layout, the MFMA
// steps and the LDS buffers take the padded size D, the columns past d are
// loaded as zeros (Q, K, V) and never stored (O).
inline bool head_size_ok(int d) { return d >= 8 && d <= 256 && d % 8 == 0; }
inline int padded_head(int d) {
  return d <= 32 ? 32 : d <= 64 ? 64 : d <= 96 ? 96 : d <= 128 ? 128 : d <= 192 ? 192 : 256;
}
// The 32-column blocks below every head size that runs on the kernel built
// for D (d > the next smaller built size): loads of blocks from this one on
// must check their columns against d.
constexpr int full_col_blocks(int D) {
  return D == 32 ? 0 : D == 64 ? 1 : D == 96 ? 2 : D == 128 ? 3 : D == 192 ? 4 : 6;
}
// A buffer-load offset past any record count the host allows (< 2^31): the
// load returns zeros, which is how the padded columns of a tile are filled.
constexpr uint32_t OOB_OFFSET = 0x80000000u;

// ---------------------------------------------------------------- dtypes
template <int DT>
struct Ty;

template <>
struct Ty<ATTN_DTYPE_BF16> {
  static __device__ __forceinline__ f32x16 mfma(i16x8 a, i16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32)
  static __device__ __forceinline__ i16x8 cvt(f32x8 x) {
    return __builtin_bit_cast(i16x8, __builtin_convertvector(x, bf16x8));
  }
  // acc + the sum of the 8 bf16 values of x (v_dot2_f32_bf16 against 1.0:
  // exact products, fp32 accumulate)
  static __device__ __forceinline__ float sum8(i16x8 x, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(
          __builtin_bit_cast(bf16x2, (short __attribute__((ext_vector_type(2)))){x[2 * i], x[2 * i + 1]}),
          one, acc, false);
    return acc;
  }
  static constexpr bool SPLIT_P = false;
  // The sum of the bf16-rounded P normalises O, but one rounded dominant
  // weight can move it by 2^-9 relative: the LSE uses an fp32 sum of the
  // unrounded P instead.
  static constexpr bool LSE_FROM_FP32_SUM = true;
};

template <>
struct Ty<ATTN_DTYPE_F16> {
  static __device__ __forceinline__ f32x16 mfma(i16x8 a, i16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(
        __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // fp32 -> fp16, round to nearest even (v_cvt_pk_f16_f32)
  static __device__ __forceinline__ i16x8 cvt(f32x8 x) {
    return __builtin_bit_cast(i16x8, __builtin_convertvector(x, f16x8));
  }
  static __device__ __forceinline__ f32x8 widen(i16x8 x) {
    return __builtin_convertvector(__builtin_bit_cast(f16x8, x), f32x8);
  }
  // acc + the sum of the 8 fp16 values of x (v_dot2_f32_f16 against 1.0)
  static __device__ __forceinline__ float sum8(i16x8 x, float acc) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2(
          __builtin_bit_cast(f16x2, (short __attribute__((ext_vector_type(2)))){x[2 * i], x[2 * i + 1]}),
          one, acc, false);
    return acc;
  }
  // fp16 probabilities are carried as hi + lo halves (P = hi + lo to about
  // 22 bits), so the P V product keeps fp32-level accuracy: the fp16
  // tolerance leaves almost no room beside the output rounding of |O| >= 4.
  static constexpr bool SPLIT_P = true;
  static constexpr bool LSE_FROM_FP32_SUM = false;  // hi + lo sum is exact enough
};

// Position of accumulator row m (of a 32x32 MFMA block) in the key order.
// m = 8g + 4h + r  ->  key 16(g>>1) + 8h + 4(g&1) + r.  With this order the
// 8 registers 8t'..8t'+7 of the S^T accumulator hold, in lane half h, keys
// 16t' + 8h + 0..7: exactly the B-operand layout of a 32x32x16 MFMA over the
// 16 keys 16t'..16t'+15.
__device__ __forceinline__ int sigma(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

// Key offset (inside a 32-key block, minus 8*h) of accumulator register
// 4g + r: the compile-time part of sigma.
__device__ __forceinline__ constexpr int key_of_reg(int reg) {
  return 16 * ((reg >> 2) >> 1) + 4 * ((reg >> 2) & 1) + (reg & 3);
}

// Max over the lane pair (l, l + 32): v_permlane32_swap(x, x) returns {x of
// lanes 0-31 in both halves, x of lanes 32-63 in both halves}.
__device__ __forceinline__ float other_half_max(float x) {
  // v_permlane32_swap(x, x) returns {x of lanes 0-31 in both halves,
  // x of lanes 32-63 in both halves}: their max is the max over the lane pair.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ------------------------------------------------------------ causal range
// K/V tiles visited by the query rows [q0, q0 + rows) (clipped to Sq): the
// causal limit of the last row, or all of K.
__host__ __device__ inline int block_tiles(int q0, int rows, int Sq, int Sk, int off,
                                           bool causal) {
  const int q_last = (q0 + rows < Sq ? q0 + rows : Sq) - 1;
  int kv_end = Sk;
  if (causal && q_last + off + 1 < kv_end) kv_end = q_last + off + 1;
  return kv_end > 0 ? (kv_end + BC - 1) / BC : 0;
}

// Pieces of a row block of `tiles` tiles under a split of `chunk` tiles per
// piece (a block that fits one piece is not split).
__host__ __device__ inline int block_pieces(int tiles, int chunk) {
  return (chunk > 0 && tiles > chunk) ? (tiles + chunk - 1) / chunk : 1;
}

// ------------------------------------------------------------ LDS tiles
//
// A 64-row tile of d columns (16-bit) is stored as d/32 column blocks; block
// cb holds the 64 rows of those 32 columns, 64 bytes (four 16-byte chunks)
// per row, and chunk c of row r sits at slot c ^ ((r >> 2) & 3).  Both read
// patterns below are free of bank conflicts: the 16 rows of a row-fragment
// read land on 16 distinct 16-byte slots of one 256-byte bank cycle, and the
// 4 rows x 64 bytes of a transposed read of 32 lanes fill one bank cycle.
constexpr int TILE_BLK = 64 * 64;  // bytes per column block of a tile

// Row fragment (A or B operand with the d dimension as k): rows
// 32 rb + sigma(l32) of the tile, 16-column chunk kk, lane half hh taking
// columns 16 kk + 8 hh .. +7.  Per-lane bases for the two parities of kk.
__device__ __forceinline__ void row_frag_bases(int lane, uint32_t (&base)[2]) {
  const int row = sigma(lane & 31);
  const int sw = (row >> 2) & 3;
#pragma unroll
  for (int par = 0; par < 2; ++par)
    base[par] = (uint32_t)(row * 64 + (((2 * par + (lane >> 5)) ^ sw) << 4));
}
__device__ __forceinline__ uint32_t row_frag_off(const uint32_t (&base)[2], int rb, int kk) {
  return (uint32_t)((kk >> 1) * TILE_BLK + rb * 32 * 64) + base[kk & 1];
}

// Transposed fragment (A or B operand with the tile's rows as k):
// ds_read_b64_tr_b16 of rows 16t + 8(g16>>1) + 4half + (s16>>2) and columns
// 32cb + 16(g16&1) + 4(s16&3) gives lane l the 4 rows of one column; the two
// halves together are the 8 consecutive rows 16t + 8(l>>5) .. +7 of column
// 32cb + (l&31).
__device__ __forceinline__ void tr_frag_bases(int lane, uint32_t (&base)[2]) {
  const int g16 = lane >> 4;
  const int s16 = lane & 15;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 8 * (g16 >> 1) + 4 * half + (s16 >> 2);
    const int cc = 16 * (g16 & 1) + 4 * (s16 & 3);
    base[half] = (uint32_t)(row * 64 + ((((cc >> 3) ^ ((row >> 2) & 3))) << 4) + (cc & 7) * 2);
  }
}
__device__ __forceinline__ i16x8 read_tr_frag(LDS_PTR(char) tile, const uint32_t (&base)[2],
                                              int t, int cb) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (LDS_PTR(i16x4))(tile + (cb * TILE_BLK + t * 16 * 64 + base[0])));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (LDS_PTR(i16x4))(tile + (cb * TILE_BLK + t * 16 * 64 + base[1])));
  return (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ i16x8 read_row_frag(LDS_PTR(char) tile, const uint32_t (&base)[2],
                                               int rb, int kk) {
  return *(LDS_PTR(const i16x8))(tile + row_frag_off(base, rb, kk));
}

// Direct global -> LDS load of tile rows [64 n, 64 n + 64) of a row-strided
// slice (row_bytes apart, d <= D contiguous elements per row) by the 4 waves
// of a workgroup: round u of a wave writes LDS bytes [(4u + wave) * 1024,
// +1024), i.e. column block (4u + wave) / 4, rows 16 ((4u + wave) % 4) +
// lane / 4, slot lane % 4.  Rows at or past nrows re-read row nrows - 1
// (finite values; the caller masks them); columns at or past d are zeros
// (their loads aim past the descriptor's end).  MUBUF loads through a buffer
// descriptor of the tile's bytes (63 rows x row_bytes + one row, which the
// host keeps below 2^31).
template <int D>
__device__ __forceinline__ void load_tile(const char* slice, uint32_t row_bytes, int n, int nrows,
                                          int d, LDS_PTR(char) buf, int wave, int lane) {
  constexpr int CB = D / 32;
  constexpr int FULL = full_col_blocks(D);
  const int ld_row = 16 * wave + (lane >> 2);
  const int ld_chunk = (lane & 3) ^ ((ld_row >> 2) & 3);
  const int r = min(64 * n + ld_row, nrows - 1) - 64 * n;
  const uint32_t off = (uint32_t)r * row_bytes + (uint32_t)ld_chunk * 16;
  const char* tile = slice + (int64_t)n * 64 * row_bytes;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)tile, 0, (int)(63 * row_bytes + (uint32_t)d * 2), 0x00020000);
#pragma unroll
  for (int u = 0; u < CB; ++u) {
    const uint32_t o = u < FULL || 32 * u + 8 * ld_chunk < d ? off : OOB_OFFSET;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_PTR(void))(buf + (u * 4 + wave) * 1024), 16,
                                             o, 64 * u, 0, 0);
  }
}

// ------------------------------------------------------------ launch plan
struct Plan {
  int nw, qb, gh, rows_wg, qtiles, ncols, xcd_cols, grid, lds_bytes, pipelined;
  int xcd_qsplit;  // > 0: XCDs sharing one (batch, kv head), each taking every
                   // xcd_qsplit-th query block of all its head subsets
  int ng;          // groups of nw waves per workgroup walking alternate
                   // K/V tiles of the same rows (1 or 2)
  int kh;          // 2: the waves are row waves x 2 key halves of each
                   // tile (nw / 2 row waves per workgroup); else 1
};

bool sizes_ok(int B, int Sq, int Sk, int Hq, int Hkv) {
  return B >= 1 && Sq >= 1 && Sk >= 1 && Hq >= 1 && Hkv >= 1;
}

Plan make_plan(int B, int Sq, int Sk, int Hq, int Hkv, int d, int causal, int kh = 1,
               int nw = 4) {
  (void)Sk;
  (void)causal;
  Plan pl{};
  pl.nw = nw;
  pl.kh = kh;
  const int rwaves = pl.nw / kh;  // waves with rows of their own
  const int group = Hq / Hkv;
  int gh = 1;
  while (gh * 2 <= rwaves && group % (gh * 2) == 0) gh *= 2;
  pl.gh = gh;
  const int hsub = group / gh;
  pl.ncols = B * Hkv * hsub;
  pl.qb = 1;
  pl.pipelined = 1;
  pl.rows_wg = (rwaves / gh) * 32;
  const long long qt = (Sq + pl.rows_wg - 1) / pl.rows_wg;
  pl.qtiles = qt > 0x7fffffffll ? -1 : (int)qt;
  pl.xcd_cols = (pl.ncols % 8 == 0) ? pl.ncols / 8 : 0;
  // Fewer (batch, kv head) pairs than XCDs, each split into head subsets: the
  // subsets of a pair go to one XCD (they read the same K/V tiles at the same
  // time, so the second read hits that XCD's L2), and the pair's query blocks
  // are dealt to 8 / (B * Hkv) XCDs.
  pl.xcd_qsplit = 0;
  {
    const int bh = B * Hkv;
    if (hsub > 1 && bh < 8 && 8 % bh == 0 && qt % (8 / bh) == 0) {
      pl.xcd_qsplit = 8 / bh;
      pl.xcd_cols = 0;
    }
  }
  const long long grid = qt * pl.ncols;
  pl.grid = (grid > 0x7fffffffll || pl.qtiles < 0) ? -1 : (int)grid;
  pl.lds_bytes = 4 * BC * padded_head(d) * 2;
  pl.ng = 1;  // set by the caller that knows the key split (two_groups)
  return pl;
}

// Two groups of 4 waves per workgroup, taking alternate K/V tiles of the same
// query rows, when the workgroups with work number at most one per CU (256 on
// MI355X): a lone 4-wave workgroup then leaves each SIMD one wave, and a
// second group's softmax runs beside the first one's matrix products.  Their
// tile buffers take twice the LDS (128 KiB at d = 128), so padded head sizes
// above 128 keep one group.  Measured on MI355X (f16, d = 128): two waves
// per SIMD finish a tile pair about 14 % sooner than one wave does a tile
// each, while the second group's first loads and the merge of the two states
// add about 3 us per workgroup; below 8 tiles in the longest workgroup (4 per
// group) that costs more than it saves.
constexpr int kCUCount = 256;
constexpr int kTwoGroupMinTiles = 8;
inline bool two_groups(long long active_workgroups, int d, int max_tiles) {
  return active_workgroups <= kCUCount && padded_head(d) <= 128 &&
         max_tiles >= kTwoGroupMinTiles;
}

// Key halves instead, for an unsplit launch in the same regime (at most one
// 4-wave workgroup per CU, at least 8 tiles in the longest block): 64-row
// workgroups, twice as many, whose two key-half waves per row wave run on
// different SIMDs, so the longest block's rows spread over two CUs.
inline bool key_halves(long long workgroups, int d, int max_tiles) {
  return workgroups <= kCUCount && padded_head(d) <= 128 && max_tiles >= kTwoGroupMinTiles;
}

using attn_detail::DecodeArgs;
using attn_detail::launch_decode;

// Waves per decode workgroup, each walking its own key tiles.  Measured on
// MI355X: 4 (two workgroups per CU) stream K and V at 5.5 TB/s; 8 (one
// workgroup of two waves per SIMD) were 1-5 % slower.
constexpr int DEC_WAVES = 4;

// Shapes the decode kernel takes: the query rows of a kv head (g * Sq) fit
// one 32-row wave, or, up to four 32-row groups (each its own workgroup over
// the same keys), when Sq <= 8.  Measured on MI355X (32 sequences x 8192
// keys): with few tokens per head the prefill kernel, whose waves hold 32
// rows of one head, leaves most rows empty (g 16, Sq 4: 302 us against 146
// us); from about 9 tokens on it is the faster one (g 4, Sq 16: 245 us
// against 288 us).
constexpr int DEC_MAX_ROWS = 128;
constexpr int DEC_MAX_SQ_GROUPED = 8;

inline bool decode_eligible(int Sq, int Hq, int Hkv, int d) {
  (void)d;  // every head size (padded up to a built one)
  const long long rows = (long long)(Hq / Hkv) * Sq;
  return rows <= 32 || (rows <= DEC_MAX_ROWS && Sq <= DEC_MAX_SQ_GROUPED);
}

struct DecodePlan {
  int pieces;
  int piece_tiles;
  int rgroups, ucols;
  long long grid;
  size_t lse_offset;  // workspace: part_o then part_lse (256-byte aligned)
  size_t ws_bytes;
};

// Pieces per (batch, kv head): kv_split 1 = none; k > 1 = k; 0 = the
// library's choice.  Measured on MI355X: one decode workgroup per CU already
// streams K and V at the chip's practical rate (5.5 TB/s with 256 of them; a
// second workgroup per CU was slower), and each piece adds to the merge, so
// the choice splits only when there are fewer than 256 workgroups, into
// about 256 workgroups with at least 8 tiles (256 keys) each.  128
// workgroups left half the CUs idle: 32K keys of one sequence took 35.5 us
// in 16 pieces and 30.4 us in 32, 16 sequences of 8K 148 us unsplit and
// 107 us in 2 pieces, and short sequences gain down to about 8 tiles per
// piece (4K keys: 14.6 us in 8 pieces, 12.0 us in 16).
//
// With more than 32 query rows per kv head, each 32-row group is its own
// workgroup; the groups of one (batch, kv head) are placed 8 workgroup ids
// apart, which puts them on one XCD (ids are dealt to the 8 XCDs in turn), so
// the second read of the same K and V tiles finds them in that XCD's L2.
inline DecodePlan make_decode_plan(int B, int Sq, int Sk, int Hq, int Hkv, int d, int kv_split) {
  DecodePlan dp{};
  const int ntiles = (Sk + 31) / 32;
  dp.rgroups = (int)(((long long)(Hq / Hkv) * Sq + 31) / 32);
  const long long bh = (long long)B * Hkv;
  const long long ucols = dp.rgroups > 1 ? ((bh + 7) / 8) * 8 * dp.rgroups : bh;
  if (ucols > 0x7fffffffll) {
    dp.grid = -1;
    return dp;
  }
  dp.ucols = (int)ucols;
  const long long cols = bh * dp.rgroups;
  long long pieces = 1;
  if (kv_split == 0) {
    if (cols < 256) pieces = (256 + cols - 1) / cols;
    const long long most = ntiles / 8 > 1 ? ntiles / 8 : 1;
    if (pieces > most) pieces = most;
  } else if (kv_split > 1) {
    pieces = kv_split;
  }
  if (pieces > ntiles) pieces = ntiles;
  dp.piece_tiles = (int)((ntiles + pieces - 1) / pieces);
  dp.pieces = (ntiles + dp.piece_tiles - 1) / dp.piece_tiles;
  dp.grid = ucols * dp.pieces;
  if (dp.pieces > 1) {
    const size_t rows = (size_t)B * Sq * Hq;
    dp.lse_offset = ((size_t)dp.pieces * rows * padded_head(d) * 4 + 255) & ~(size_t)255;
    dp.ws_bytes = dp.lse_offset + (size_t)dp.pieces * rows * 4;
  }
  if (dp.grid > 0x7fffffffll) dp.grid = -1;
  return dp;
}

}  // namespace

