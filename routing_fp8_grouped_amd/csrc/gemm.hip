// Grouped FP8 GEMM of the SwiGLU experts (the "DeepSeek-V3" summary page,
// section 6 (a)-(c); the book's chapter 16 "Scales along the GEMM inner
// dimension" and "Periodic high-precision promotion", chapter 17 "SwiGLU
// recomputation" and "FP8 dispatch, BF16 combine").
//
// Both expert GEMMs use one persistent kernel template:
//   stage 1  [rows, d] x W13[g]^T -> G, U  (K = d), epilogue h = SiLU(G) * U,
//            1x128 requantisation of h -> E4M3 codes + FP32 scales
//   stage 2  [rows, f] x W2[g]^T  -> Y     (K = f), epilogue BF16
// Tiles are 256 rows x 256 weight rows; in stage 1 the 256 weight rows are the
// 128 gate rows and the matching 128 up rows of one 128-wide slice of f, so one
// tile yields complete 1x128 tiles of h.  K advances in 128-wide blocks, the
// granularity of both scales: one v_mfma_scale_f32_16x16x128_f8f6f4 per 16x16
// sub-tile computes the block's partial sum, which is promoted into the FP32
// accumulator with the product of the row's activation scale and the weight
// block's scale.  (The pages' H800 kernel promoted every four WGMMAs; on gfx950
// a single MFMA spans exactly one scale block.)
//
// Per workgroup: 512 threads = 8 waves, two per SIMD, in a 4 x 2 grid.  Wave
// (wm, wn) owns rows wm*64 .. +63 and 128 weight-tile rows, i.e. 4 x 8 MFMA
// sub-tiles: in stage 1 the gate rows wn*64 .. +63 and the up rows of the same
// 64 h columns (so SiLU(G) * U is formed in registers and only the row amax of
// the 1x128 requantisation crosses waves), in stage 2 rows wn*128 .. +127.
// The weight fragment is the MFMA's first operand, so each lane holds four
// consecutive output columns of one row, and the promotion factor (row scale x
// weight-block scale) is one register per lane and sub-tile row block.  With
// two waves per SIMD the promotion FMAs of one wave issue while the other
// wave's MFMAs run; within a wave each promotion follows two MFMAs after its
// own (one in the second GEMM, whose register budget is tighter), so its FMAs
// do not wait for the MFMA result.
//
// Operands stream HBM -> LDS through a two-stage ring filled by direct
// global->LDS loads (no VGPR round trip).  Each K block has one barrier, placed
// after the wave's last LDS read of the block: past it the block's stage is
// refilled with the block two ahead, and the first fragments of the next block
// are read while the last MFMAs of this block run.  The epilogues need no LDS
// staging, so the ring keeps loading the next tile while they run.
//
// Power-of-two variant (E8M0): when every activation, weight and H scale is a
// power of two (the quantisers' power-of-two rule), the scales go into the
// instruction's hardware block-scale operands (the E8M0 code is the FP32
// exponent field) and the accumulator is chained through the MFMA: no partial
// sums, no promotion FMAs.  H is then requantised with the same rule.
//
// Work distribution: the tile list (group, m super-block of 4 m-tiles, n-tile,
// m-tile) is built on the device from the group offsets, so nothing waits on
// the host for the ragged row counts.  Workgroup b runs on XCD b % 8 and takes
// tiles of its XCD's contiguous eighth of the list, so the workgroups sharing a
// weight tile or an activation tile run together behind one L2.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int BM = 256;   // rows per tile
constexpr int BN = 256;   // weight rows per tile
constexpr int BK = 128;   // K block (scale block)
constexpr int NTHR = 512;
constexpr int MAX_GROUPS = 1024;
constexpr int SUPER_M = 4;   // m-tiles per super-block of the tile order

struct GemmArgs {
  const uint8_t* a;         // [a_rows, K] E4M3
  const float* as;          // [a_rows, K/128]
  int a_rows;
  const int32_t* row_src;   // [total rows] source row of each row, or null (identity)
  int n_groups;
  int total_rows;           // rows of h / y (and of row_src)
  int K;
  int N;                    // weight rows per group
  int n_tiles_n;
  const uint8_t* b;         // [n_groups, N, K] E4M3
  const float* bs;          // [n_groups, N/128, K/128]
  int f;                    // stage 1: intermediate width (N = 2f)
  uint8_t* h;               // stage 1 out [rows, f]
  float* hs;                // stage 1 out [rows, f/128]
  uint16_t* y;              // stage 2 out [rows, N]
  uint8_t* gu;              // stage 1, optional: FP8 cache of [G, U] [rows, 2f] (1x128 tiles)
  float* gus;               // its scales [rows, 2f/128]
};

// LDS layout of a 128-byte operand row r: its 16-byte chunk c sits at chunk
// position c ^ swz(r).  A fragment read (ds_read_b128) has lanes 0..15 on rows
// r0..r0+15 at one chunk; swz gives rows r0..r0+7 eight different positions
// and gives the even rows and the odd rows of r0..r0+15 eight positions each,
// so the read is conflict-free whether 8 or 16 lanes are served per cycle.
__device__ __forceinline__ int swz(int r) { return op_swz(r); }
__device__ __forceinline__ int op_off(int r, int c) { return r * BK + ((c ^ swz(r)) << 4); }

// ---- LDS ring: two K blocks, filled by direct global->LDS loads ----
constexpr int ST_A = BM * BK;                   // activation tile, 32 KB
constexpr int ST_B = BN * BK;                   // weight tile, 32 KB
constexpr int ST_SA = BM * 4;                   // activation scales of the 256 rows
constexpr int ST_SW = 256;                      // weight scales: [0] wave column 0, [1] column 1
constexpr int STG = ST_A + ST_B + ST_SA + ST_SW;

// Barrier for LDS data only: waits for this wave's LDS operations, not for the
// direct loads in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt unconstrained
  asm volatile("s_barrier" ::: "memory");
}

struct Tile {
  int g, n, row0, rows_valid;
};

// Tile l of the list: groups in order; inside a group, super-blocks of
// SUPER_M m-tiles; inside a super-block n-tiles, and m-tiles fastest.
__device__ __forceinline__ Tile decode_tile(const GemmArgs& p, const int32_t* __restrict__ offsets,
                                            const int* smTile, int NT, int l) {
  const int q = l / NT;
  int a = 0, b = p.n_groups - 1;
  while (a < b) {
    const int mid = (a + b + 1) >> 1;
    if (smTile[mid] <= q) a = mid; else b = mid - 1;
  }
  a = __builtin_amdgcn_readfirstlane(a);   // uniform: offsets come through scalar loads
  const int mt = __builtin_amdgcn_readfirstlane(smTile[a + 1] - smTile[a]);
  const int local = l - smTile[a] * NT;
  const int sb = local / (SUPER_M * NT);
  const int rem = local - sb * SUPER_M * NT;
  const int msb = min(SUPER_M, mt - sb * SUPER_M);
  Tile t;
  t.g = a;
  t.n = rem / msb;
  const int m = sb * SUPER_M + (rem - t.n * msb);
  // the group's rows split evenly over its mt tiles (multiples of 16), so the
  // tiles sharing a weight panel take equally long and stay together in L2
  // (a short remainder tile would run ahead and make the others fetch the
  // panel again).  Used by the first GEMM and by any K of 32 blocks or more;
  // with the second GEMM's 16 blocks the drift is too short to matter.
  const int R = offsets[a + 1] - offsets[a];
  const int rpt = (p.h || p.K >= 32 * BK) ? min(BM, ((R + mt - 1) / mt + 15) / 16 * 16) : BM;
  t.row0 = offsets[a] + m * rpt;
  // rows past total_rows (only possible with malformed offsets) are never touched
  t.rows_valid = max(0, min(rpt, min(offsets[a + 1], p.total_rows) - t.row0));
  return t;
}

// Row of p.a's row space holding tile row r (rows past the group's end repeat
// its last row; they are multiplied but never stored).
__device__ __forceinline__ int tile_row(const GemmArgs& p, const Tile& t, int r) {
  return min(max(t.row0 + min(r, t.rows_valid - 1), 0), p.total_rows - 1);
}

// Per-lane global sources of one wave's direct loads for a tile, kept in LDS
// (9 words per lane: [0..3] activation rows, [4..7] weight rows, [8] a scale
// row) so that no register holds them across the multiply; the K block offset
// is added at issue time.  Instruction i of wave w writes 1 KB at (4 w + i) KB
// of its operand region: lane l writes 16 bytes at 16 l, i.e. tile row
// 8 (4 w + i) + l / 8, physical chunk l % 8, which holds the logical chunk
// (l % 8) ^ swz(row) (the swizzle is applied on the source side).  Waves 0..3
// also load the activation scales of rows 64 w .. 64 w + 63 (word 8 is a byte
// offset into p.as), wave 4 the weight scales (word 8 is a byte offset into
// p.bs; lane parity selects the scale block of wave column 0 or 1).
constexpr int SRC_WORDS = 9;

// Weight row (within the group) held by row rr of the LDS weight tile.
template <bool SWIGLU>
__device__ __forceinline__ int weight_row(const GemmArgs& p, int n, int rr) {
  if (SWIGLU) return rr < 128 ? n * 128 + rr : p.f + n * 128 + (rr - 128);
  return n * BN + rr;
}

// LDS weight-tile row of sub-tile column ns of wave column wn.  In stage 1 a
// wave takes 64 gate rows (ns 0..3) and the matching 64 up rows (ns 4..7), so
// SiLU(G) * U is formed in registers; in stage 2 it takes 128 consecutive rows.
template <bool SWIGLU>
__device__ __forceinline__ int brow(int wn, int ns) {
  if (SWIGLU) return (ns < 4 ? 0 : 128) + wn * 64 + (ns & 3) * 16;
  return wn * 128 + ns * 16;
}

// Gather indices of a tile's 256 rows, loaded into an LDS table one tile ahead
// (waves 0..3, lane l: tile row 64 w + l), so no register waits on them.
__device__ __forceinline__ void dma_tile_rows(const GemmArgs& p, const Tile& t, int wave, int lane,
                                              int* table) {
  if (wave < 4) {
    const int r = wave * 64 + lane;
    dma4(p.row_src, (uint32_t)tile_row(p, t, r) * 4u, lds_addr(table + wave * 64));
  }
}

template <bool SWIGLU>
__device__ __forceinline__ void build_sources(const GemmArgs& p, const Tile& t, const int* table,
                                              int wave, int lane, uint32_t* srcw) {
  const int KS = p.K / BK;
  const int pc = lane & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (wave * 4 + i) * 8 + (lane >> 3);
    const int c = pc ^ swz(r);
    int row = p.row_src ? table[r] : tile_row(p, t, r);
    row = min(max(row, 0), p.a_rows - 1);
    // rows past the end of a partial tile are not loaded (their LDS rows are
    // multiplied but never stored); an odd offset marks them
    srcw[i * 64 + lane] = r < t.rows_valid ? (uint32_t)row * (uint32_t)p.K + c * 16 : 1u;
    int wr = weight_row<SWIGLU>(p, t.n, r);
    if (wr >= p.N) wr = 0;   // padding rows of a partial tile: any valid row, never stored
    srcw[(4 + i) * 64 + lane] = (uint32_t)wr * (uint32_t)p.K + c * 16;
  }
  uint32_t so;
  if (wave < 4) {
    const int rs = wave * 64 + lane;
    int row = p.row_src ? table[rs] : tile_row(p, t, rs);
    row = min(max(row, 0), p.a_rows - 1);
    so = (uint32_t)row * (uint32_t)(KS * 4);
  } else {
    const int nsb = p.N / 128;
    int sb;
    if (SWIGLU) sb = (lane & 1) ? p.f / 128 + t.n : t.n;
    else sb = min(2 * t.n + (lane & 1), nsb - 1);
    so = (uint32_t)(t.g * nsb + sb) * (uint32_t)(KS * 4);
  }
  srcw[8 * 64 + lane] = so;
}

__device__ __forceinline__ void issue_stage(const GemmArgs& p, const uint8_t* bbase, const uint32_t* srcw,
                                            int kb, int wave, int lane, unsigned char* stage) {
  const uint32_t base = lds_addr(stage);
  const uint8_t* a = p.a + (size_t)kb * BK;
  const uint8_t* b = bbase + (size_t)kb * BK;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t src = srcw[i * 64 + lane];
    if (!(src & 1u)) dma16(a, src, base + (wave * 4 + i) * 1024);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) dma16(b, srcw[(4 + i) * 64 + lane], base + ST_A + (wave * 4 + i) * 1024);
  if (wave < 4) dma4(p.as + kb, srcw[8 * 64 + lane], base + ST_A + ST_B + wave * 256);
  else if (wave == 4) dma4(p.bs + kb, srcw[8 * 64 + lane], base + ST_A + ST_B + ST_SA);
}

// MFMA operand fragment: rows r (this lane's row r16 added by the caller),
// K bytes [g16 * 32, g16 * 32 + 32).
__device__ __forceinline__ v8i frag(const unsigned char* T, int r, int g16) {
  const uint4 lo = *reinterpret_cast<const uint4*>(T + op_off(r, g16 * 2));
  const uint4 hi = *reinterpret_cast<const uint4*>(T + op_off(r, g16 * 2 + 1));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// ---- epilogues ----
// With the weight fragment as the MFMA's first operand, lane (g16, r16) holds
// in acc[ms][ns] row ms*16 + r16 of the wave's 64 rows and the 4 consecutive
// columns brow(wn, ns) + 4*g16 + e of the weight tile.

// 1x128 quantisation of the 64 x 64 block acc[.][j0 .. j0+3] of each wave, whose
// partner wave (wn ^ 1) holds the other 64 columns of the same 1x128 tiles:
// row amax over the lane's 16 values, the 4 lanes of the row and, through
// smAmax, the partner; then the E4M3 codes, 4 per 32-bit store.  `out` points
// at the wave's first column of tile row 0, rows `ld` bytes apart; the scale of
// tile row r goes to sout[(row0 + r) * sld] (written by wave column 0).
template <bool POW2>
__device__ __forceinline__ void quantise_rows(const v4f (&acc)[4][8], int j0, float (*smAmax)[BM], int wm,
                                              int wn, int g16, int r16, const Tile& cur, uint8_t* out,
                                              size_t ld, float* sout, int sld) {
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) a = fmaxf(a, fabsf(acc[ms][j0 + j][e]));
    a = fmaxf(a, __shfl_xor(a, 16));
    a = fmaxf(a, __shfl_xor(a, 32));
    if (g16 == 0) smAmax[wn][wm * 64 + ms * 16 + r16] = a;
  }
  lds_barrier();
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) {
    const int rt = wm * 64 + ms * 16 + r16;
    const float sc = tile_scale<POW2>(fmaxf(smAmax[0][rt], smAmax[1][rt]));
    const Divider div(sc);
    const bool ok = rt < cur.rows_valid;
    if (wn == 0 && g16 == 0 && ok) sout[(size_t)(cur.row0 + rt) * sld] = sc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4f v = acc[ms][j0 + j];
      // correctly rounded FP32 quotients, as in the activation quantiser
      const uint32_t q = f32x4_to_e4m3(div(v[0]), div(v[1]), div(v[2]), div(v[3]));
      if (ok) *reinterpret_cast<uint32_t*>(out + (size_t)(cur.row0 + rt) * ld + j * 16) = q;
    }
  }
  lds_barrier();   // every wave has read smAmax before it is written again
}

// Stage 1: the optional FP8 cache of G and U (1x128 tiles, the forward's
// rule), then h = SiLU(G) * U in place of G and its 1x128 requantisation.
// The wave's columns of the tile's 128-wide slice of f are wn*64 .. +63.
template <bool POW2>
__device__ __forceinline__ void epilogue_swiglu(const GemmArgs& p, const Tile& cur, v4f (&acc)[4][8],
                                                float (*smAmax)[BM], int wm, int wn, int lane) {
  const int g16 = lane >> 4, r16 = lane & 15;
  const int nhs = p.f / 128;
  const size_t col = (size_t)cur.n * 128 + wn * 64 + 4 * g16;
  if (p.gu) {
    quantise_rows<POW2>(acc, 0, smAmax, wm, wn, g16, r16, cur, p.gu + col, 2 * (size_t)p.f, p.gus + cur.n,
                        2 * nhs);
    quantise_rows<POW2>(acc, 4, smAmax, wm, wn, g16, r16, cur, p.gu + p.f + col, 2 * (size_t)p.f,
                        p.gus + nhs + cur.n, 2 * nhs);
  }
#pragma unroll
  for (int ms = 0; ms < 4; ++ms)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[ms][j][e] = swiglu_f32(acc[ms][j][e], acc[ms][4 + j][e]);
  quantise_rows<POW2>(acc, 0, smAmax, wm, wn, g16, r16, cur, p.h + col, (size_t)p.f, p.hs + cur.n, nhs);
}

// Stage 2: BF16 from registers.  Lane pairs (l, l + 16) trade halves with
// v_permlane16_swap so that each lane holds 8 consecutive columns: sub-tile
// column ns in the even 16-lane rows, ns + 1 in the odd ones.  Each store
// then writes 16 bytes per lane and 64 contiguous bytes per row.
__device__ __forceinline__ void epilogue_bf16(const GemmArgs& p, const Tile& cur, v4f (&acc)[4][8], int wm,
                                              int wn, int lane) {
  const int g16 = lane >> 4, r16 = lane & 15;
  const int col0 = cur.n * BN + wn * 128;
  if (col0 >= p.N) return;
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) {
    const int rt = wm * 64 + ms * 16 + r16;
    uint16_t* yr = p.y + (size_t)(cur.row0 + rt) * p.N + col0 + (g16 & 1) * 16 + (g16 >> 1) * 8;
#pragma unroll
    for (int ns = 0; ns < 8; ns += 2) {
      const v4f a = acc[ms][ns], b = acc[ms][ns + 1];
      const uint32_t a0 = (uint32_t)f32_to_bf16(a[0]) | ((uint32_t)f32_to_bf16(a[1]) << 16);
      const uint32_t a1 = (uint32_t)f32_to_bf16(a[2]) | ((uint32_t)f32_to_bf16(a[3]) << 16);
      const uint32_t b0 = (uint32_t)f32_to_bf16(b[0]) | ((uint32_t)f32_to_bf16(b[1]) << 16);
      const uint32_t b1 = (uint32_t)f32_to_bf16(b[2]) | ((uint32_t)f32_to_bf16(b[3]) << 16);
      const auto x = __builtin_amdgcn_permlane16_swap(a0, b0, false, false);
      const auto z = __builtin_amdgcn_permlane16_swap(a1, b1, false, false);
      const uint4 v = {x[0], z[0], x[1], z[1]};
      if (rt < cur.rows_valid) *reinterpret_cast<uint4*>(yr + ns * 16) = v;
    }
  }
}

// Loader: issues the K blocks of this workgroup's tiles into the ring, one
// block per call.  When it starts a tile it builds the tile's sources from the
// gather table and loads the gather indices of its next tile into the other
// table; every ring barrier waits for all direct loads, so those land before
// they are used.
template <bool SWIGLU>
struct Loader {
  const GemmArgs& p;
  const int32_t* __restrict__ offsets;
  const int* smTile;
  int (*smRows)[BM];
  int NT, KB, wave, lane, nslot;
  int hi;
  int L;
  int kb, par;
  bool more;
  uint32_t* srcw;          // this wave's source table in LDS
  Tile tile;
  const uint8_t* bbase;    // the loader tile's group weights (uniform)

  __device__ __forceinline__ void issue(unsigned char* stage) {
    if (kb == 0) {
      build_sources<SWIGLU>(p, tile, smRows[par], wave, lane, srcw);
      bbase = p.b + (size_t)tile.g * p.N * p.K;
      if (p.row_src && L + nslot < hi)
        dma_tile_rows(p, decode_tile(p, offsets, smTile, NT, L + nslot), wave, lane, smRows[par ^ 1]);
    }
    issue_stage(p, bbase, srcw, kb, wave, lane, stage);
    if (++kb == KB) {
      kb = 0;
      L += nslot;
      par ^= 1;
      more = L < hi;
      if (more) tile = decode_tile(p, offsets, smTile, NT, L);
    }
  }
};

// Per-wave register state of the multiply.
struct Frags {
  v8i af[4];       // activation fragments of the block (rows ms*16 .. +15)
  v8i bq[2];       // weight fragments, column ns in slot ns & 1
  float cs[2][4];  // activation scale of this lane's row of fragment ms x weight scale ([1]: up rows)
  int ea[4];       // E8M0 variant: scale code of this lane's activation row of fragment ms
  int eb[2];       // E8M0 variant: scale code of the wave's weight block ([1]: up rows)
};

template <bool SWIGLU, bool E8M0>
__device__ __forceinline__ void load_scales(Frags& F, const unsigned char* stage, int wm, int wn, int r16) {
  const unsigned char* B_ = stage + ST_A;
  if (E8M0) {
    const uint32_t* SA_ = reinterpret_cast<const uint32_t*>(B_ + ST_B);
    const uint32_t* SW_ = reinterpret_cast<const uint32_t*>(B_ + ST_B + ST_SA);
    F.eb[0] = (int)(SW_[SWIGLU ? 0 : wn] >> 23);
    if (SWIGLU) F.eb[1] = (int)(SW_[1] >> 23);
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) F.ea[ms] = (int)(SA_[wm * 64 + ms * 16 + r16] >> 23);
    return;
  }
  const float* SA_ = reinterpret_cast<const float*>(B_ + ST_B);
  const float* SW_ = reinterpret_cast<const float*>(B_ + ST_B + ST_SA);
  const float s0 = SW_[SWIGLU ? 0 : wn];
  const float s1 = SW_[1];
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) {
    const float sa = SA_[wm * 64 + ms * 16 + r16];
    F.cs[0][ms] = sa * s0;
    if (SWIGLU) F.cs[1][ms] = sa * s1;
  }
}

template <bool SWIGLU, bool E8M0>
__device__ __forceinline__ void load_first(Frags& F, const unsigned char* stage, int wm, int wn, int g16,
                                           int r16) {
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) F.af[ms] = frag(stage, wm * 64 + ms * 16 + r16, g16);
  F.bq[0] = frag(stage + ST_A, brow<SWIGLU>(wn, 0) + r16, g16);
  load_scales<SWIGLU, E8M0>(F, stage, wm, wn, r16);
}

// One K block on stage `cur`: MFMA i = (ns, ms) in ns-major order, each
// partial promoted after the next MFMA has been issued; the weight fragment of
// column ns + 1 is read while column ns is multiplied.  After the last read of
// `cur` (column 7's fragment) comes the ring barrier; unless LAST, the stage
// is then refilled (the loader's next block) and the first fragments of the
// next block are read from `nxt` while column 7 is multiplied.
//
// A wave whose 64 rows all lie past the end of a partial tile (`active` false)
// skips the reads and the arithmetic but keeps the barrier and the loads.
//
// E8M0: the MFMA takes the block scales and accumulates into acc directly.
template <bool SWIGLU, bool LAST, bool E8M0>
__device__ __forceinline__ void k_block(v4f (&acc)[4][8], Frags& F, Loader<SWIGLU>& ld,
                                        unsigned char* cur, const unsigned char* nxt, int wm, int wn,
                                        int g16, int r16, bool active) {
  if (!active) {
    ring_barrier();
    if (!LAST && ld.more) ld.issue(cur);
    return;
  }
  const unsigned char* Bc = cur + ST_A;
  // each partial sum is promoted PD MFMAs after its own, so the FMAs never
  // wait for an MFMA in flight
  constexpr int PD = SWIGLU ? 2 : 1;
  v4f part[PD + 1];
#pragma unroll
  for (int ns = 0; ns < 8; ++ns) {
    // the register budget holds two weight fragments: no LDS read moves across
    // columns (an empty asm with a memory clobber pins them in order)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (ns < 7) F.bq[(ns + 1) & 1] = frag(Bc, brow<SWIGLU>(wn, ns + 1) + r16, g16);
    if (ns == 7) {
      ring_barrier();
      if (!LAST) {
        if (ld.more) ld.issue(cur);
        F.bq[0] = frag(nxt + ST_A, brow<SWIGLU>(wn, 0) + r16, g16);
      }
    }
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      const int i = ns * 4 + ms;
      if (E8M0) {
        acc[ms][ns] = mfma_fp8_16x16x128_scaled(F.bq[ns & 1], F.af[ms], acc[ms][ns],
                                                F.eb[SWIGLU ? (ns >> 2) : 0], F.ea[ms]);
        if (i >= 1) {
          const int pi = i - 1;
          asm volatile("" : "+v"(acc[pi & 3][pi >> 2]));
        }
      } else {
        part[i % (PD + 1)] = mfma_fp8_16x16x128(F.bq[ns & 1], F.af[ms], v4f{0.f, 0.f, 0.f, 0.f});
        // MFMA i is issued before the promotion of partial i - PD (the
        // compiler would otherwise move the promotion up to its own MFMA and
        // stall the wave for that MFMA's latency)
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!E8M0 && i >= PD) {
        const int pi = i - PD, pms = pi & 3, pns = pi >> 2;
        const float c = F.cs[SWIGLU ? (pns >> 2) : 0][pms];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[pms][pns][e] = fmaf(part[pi % (PD + 1)][e], c, acc[pms][pns][e]);
        // pins the promotion (and so the MFMAs before it) at this point: the
        // compiler would otherwise sink the block's arithmetic past the ring
        // barrier and hold every weight fragment at once
        asm volatile("" : "+v"(acc[pms][pns]));
      }
      if (ns == 7 && !LAST) {
        // the next block's fragment ms replaces this one once its last MFMA is issued
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        F.af[ms] = frag(nxt, wm * 64 + ms * 16 + r16, g16);
      }
    }
  }
  if (!E8M0)
#pragma unroll
    for (int pi = 32 - PD; pi < 32; ++pi) {
      const int pms = pi & 3, pns = pi >> 2;
      const float c = F.cs[SWIGLU ? (pns >> 2) : 0][pms];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[pms][pns][e] = fmaf(part[pi % (PD + 1)][e], c, acc[pms][pns][e]);
    }
  if (!LAST) load_scales<SWIGLU, E8M0>(F, nxt, wm, wn, r16);
}

template <bool SWIGLU, bool E8M0>
__global__ __launch_bounds__(NTHR, 1) void grouped_gemm_kernel(GemmArgs p,
                                                              const int32_t* __restrict__ offsets) {
  __shared__ __attribute__((aligned(16))) unsigned char sm[2 * STG];
  __shared__ int smTile[MAX_GROUPS + 1];
  __shared__ __attribute__((aligned(16))) int smRows[2][BM];   // gather indices, by tile parity
  __shared__ float smAmax[2][BM];
  __shared__ uint32_t smSrc[NTHR / 64][SRC_WORDS * 64];   // per-wave source tables

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int KB = p.K / BK;
  const int NT = p.n_tiles_n;

  // ---- tile list: m-tiles per group, exclusive prefix in LDS ----
  if (wave == 0) {
    int carry = 0;
    for (int base = 0; base < p.n_groups; base += 64) {
      const int g = base + lane;
      int mt = 0;
      if (g < p.n_groups) mt = (offsets[g + 1] - offsets[g] + BM - 1) / BM;
      int v = mt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o);
        if (lane >= o) v += u;
      }
      if (g < p.n_groups) smTile[g + 1] = carry + v;
      carry += __shfl(v, 63);
    }
    if (lane == 0) smTile[0] = 0;
  }
  __syncthreads();
  // the host guarantees fewer than 2^31 / 8 tiles
  const int total = smTile[p.n_groups] * NT;
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int nslot = gridDim.x >> 3;
  const int lo = total * xcd / 8, hi = total * (xcd + 1) / 8;
  if (lo + slot >= hi) return;

  Loader<SWIGLU> ld{p, offsets, smTile, smRows, NT, KB, wave, lane, nslot, hi, lo + slot, 0, 0, true,
                    smSrc[wave]};
  ld.tile = decode_tile(p, offsets, smTile, NT, ld.L);
  if (p.row_src) {
    dma_tile_rows(p, ld.tile, wave, lane, smRows[0]);
    ring_barrier();
  }
  // prologue: blocks 0 and 1 in flight, block 0 landed
  ld.issue(sm);
  ring_barrier();
  if (ld.more) ld.issue(sm + STG);

  Frags F;
  int S = 0;   // ring stage of the block being multiplied
  for (int L = lo + slot; L < hi; L += nslot) {
    const Tile cur = decode_tile(p, offsets, smTile, NT, L);
    v4f acc[4][8];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
      for (int ns = 0; ns < 8; ++ns) acc[ms][ns] = v4f{0.f, 0.f, 0.f, 0.f};
    // rows wm*64 .. +63 hold data (uniform per wave)
    const bool active = wm * 64 < cur.rows_valid;
    if (active) load_first<SWIGLU, E8M0>(F, sm + S * STG, wm, wn, g16, r16);
    for (int kb = 0; kb < KB - 1; ++kb) {
      k_block<SWIGLU, false, E8M0>(acc, F, ld, sm + S * STG, sm + (S ^ 1) * STG, wm, wn, g16, r16, active);
      S ^= 1;
    }
    k_block<SWIGLU, true, E8M0>(acc, F, ld, sm + S * STG, sm + (S ^ 1) * STG, wm, wn, g16, r16, active);

    // ---- epilogue.  Every wave has finished reading stage S (the ring
    // barrier of the last block followed the last read); the next tile's
    // first block is in stage S ^ 1 (landed at that barrier) ----
    unsigned char* E = sm + S * STG;
    // the epilogues work in registers: stage S is refilled before them
    if (ld.more) ld.issue(E);
    if (SWIGLU) epilogue_swiglu<E8M0>(p, cur, acc, smAmax, wm, wn, lane);
    else epilogue_bf16(p, cur, acc, wm, wn, lane);
    S ^= 1;
  }
}

static int g_num_cus[64];

static int num_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (g_num_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_num_cus[dev] = n;
  }
  return g_num_cus[dev];
}

hipError_t launch_gemm_up(const uint8_t* aq, const float* as, int a_rows, const int32_t* row_src,
                          const int32_t* offsets, int n_groups, int total_rows, int d, int f,
                          const uint8_t* w13, const float* w13_s, uint8_t* h, float* hs,
                          bool e8m0, hipStream_t stream, uint8_t* gu, float* gus) {
  // few rows per group: stream the weights (the tiled kernel alone writes the
  // [G, U] cache)
  if (total_rows <= 16 * n_groups && gu == nullptr && d <= kSmallMaxK)
    return launch_gemm_up_small(aq, as, a_rows, row_src, offsets, n_groups, total_rows, d, f, w13,
                                w13_s, h, hs, e8m0, stream);
  const int grid = ((num_cus() + 7) / 8) * 8;
  GemmArgs s1{};
  s1.a = aq;
  s1.as = as;
  s1.a_rows = a_rows;
  s1.row_src = row_src;
  s1.n_groups = n_groups;
  s1.total_rows = total_rows;
  s1.K = d;
  s1.N = 2 * f;
  s1.n_tiles_n = f / 128;
  s1.b = w13;
  s1.bs = w13_s;
  s1.f = f;
  s1.h = h;
  s1.hs = hs;
  s1.gu = gu;
  s1.gus = gus;
  if (e8m0)
    hipLaunchKernelGGL((grouped_gemm_kernel<true, true>), dim3(grid), dim3(NTHR), 0, stream, s1, offsets);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<true, false>), dim3(grid), dim3(NTHR), 0, stream, s1, offsets);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const uint8_t* h, const float* hs, const int32_t* offsets, int n_groups,
                            int total_rows, int d, int f, const uint8_t* w2, const float* w2_s,
                            uint16_t* y, bool e8m0, hipStream_t stream) {
  // few rows per group: the weight-streaming kernel, whose software promotion
  // is exact with power-of-two scales
  if (total_rows <= 16 * n_groups && f <= kSmallMaxK)
    return launch_gemm_down_small(h, hs, offsets, n_groups, total_rows, d, f, w2, w2_s, y, stream);
  const int grid = ((num_cus() + 7) / 8) * 8;
  GemmArgs s2{};
  s2.a = h;
  s2.as = hs;
  s2.a_rows = total_rows;
  s2.row_src = nullptr;
  s2.n_groups = n_groups;
  s2.total_rows = total_rows;
  s2.K = f;
  s2.N = d;
  s2.n_tiles_n = (d + BN - 1) / BN;
  s2.b = w2;
  s2.bs = w2_s;
  s2.f = f;
  s2.y = y;
  if (e8m0)
    hipLaunchKernelGGL((grouped_gemm_kernel<false, true>), dim3(grid), dim3(NTHR), 0, stream, s2, offsets);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<false, false>), dim3(grid), dim3(NTHR), 0, stream, s2, offsets);
  return hipGetLastError();
}

}  // namespace moe
