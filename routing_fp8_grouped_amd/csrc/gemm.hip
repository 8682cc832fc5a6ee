// Grouped FP8 GEMM of the SwiGLU experts (the "DeepSeek-V3" summary page,
// section 6 (a)-(c); the book's chapter 16 "Scales along the GEMM inner
// dimension" and "Periodic high-precision promotion", chapter 17 "SwiGLU
// recomputation" and "FP8 dispatch, BF16 combine").
//
// Both expert GEMMs use one persistent kernel template:
//   stage 1  [rows, d] x W13[g]^T -> G, U  (K = d), epilogue h = SiLU(G) * U,
//            1x128 requantisation of h -> E4M3 codes + FP32 scales
//   stage 2  [rows, f] x W2[g]^T  -> Y     (K = f), epilogue BF16
// Tiles are 128 rows x 256 weight rows; in stage 1 the 256 weight rows are the
// 128 gate rows and the matching 128 up rows of one 128-wide slice of f, so one
// tile yields one complete 1x128 tile of h.  K advances in 128-wide blocks, the
// granularity of both scales: one v_mfma_scale_f32_16x16x128_f8f6f4 per 16x16
// sub-tile computes the block's partial sum, which is promoted into the FP32
// accumulator with the product of the row's activation scale and the weight
// block's scale.  (The pages' H800 kernel promoted every four WGMMAs; on gfx950
// a single MFMA spans exactly one scale block.)
//
// Work distribution: the tile list (group, n-tile, m-tile), m fastest, is built
// on the device from the group offsets, so nothing waits on the host for the
// ragged row counts.  Workgroup b runs on XCD b % 8 and takes the tiles of its
// XCD's contiguous eighth of the list, so the workgroups sharing a weight tile
// (consecutive m-tiles) run together behind one L2.
//
// Per workgroup: 256 threads = 4 waves in a 2 x 2 grid, each wave 64 rows x 128
// weight rows (4 x 8 MFMA sub-tiles).  Operands are double-buffered in LDS
// (16-byte chunks XOR-swizzled by row); the next K block (possibly of the next
// tile) is loaded into registers while the current one is multiplied.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int GM = 128;   // rows per tile
constexpr int GNB = 256;  // weight rows per tile
constexpr int GK = 128;   // K block (scale block)
constexpr int G_THREADS = 256;
constexpr int G_MAX_GROUPS = 1024;

struct GemmArgs {
  const uint8_t* a;         // [a_rows, K] E4M3
  const float* as;          // [a_rows, K/128]
  int a_rows;
  const int32_t* row_src;   // [total rows] source row of each row, or null (identity)
  const int32_t* offsets;   // [n_groups + 1]
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
};

// LDS layout of a 128-byte operand row r: its 16-byte chunk c sits at chunk
// position c ^ swz(r).  A fragment read (ds_read_b128) has lanes 0..15 on rows
// r0..r0+15 at one chunk; swz gives rows r0..r0+7 eight different positions
// (conflict-free when 8 lanes are served per cycle) and gives the even rows
// and the odd rows of r0..r0+15 eight positions each (conflict-free when 16
// lanes are served per cycle over 64 banks).
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }
__device__ __forceinline__ int op_off(int r, int c) { return r * GK + ((c ^ swz(r)) << 4); }

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct Tile {
  int g, n, row0, rows_valid;
};

// Weight row (within the group) held by row rr of the LDS weight tile.
template <bool SWIGLU>
__device__ __forceinline__ int weight_row(const GemmArgs& p, int n, int rr) {
  if (SWIGLU) return rr < 128 ? n * 128 + rr : p.f + n * 128 + (rr - 128);
  return n * GNB + rr;
}

// LDS weight-tile row of sub-tile ns for wave column wn.
template <bool SWIGLU>
__device__ __forceinline__ int frag_row(int wn, int ns) {
  if (SWIGLU) return ns < 4 ? wn * 64 + ns * 16 : 128 + wn * 64 + (ns - 4) * 16;
  return wn * 128 + ns * 16;
}

// ---- LDS ring: NSTAGE K blocks in flight, filled by direct global->LDS loads ----
constexpr int NSTAGE = 3;
constexpr int ST_A = GM * GK;                   // activation tile, 16 KB
constexpr int ST_B = GNB * GK;                  // weight tile, 32 KB
constexpr int ST_SA = 256 * 4;                  // activation scales (rows 0..127; 128..255 spare)
constexpr int ST_SW = 4 * 256;                  // per wave: its two weight-block scales
constexpr int ST_BYTES = ST_A + ST_B + ST_SA + ST_SW;
// DMA instructions per wave per K block: 4 (A) + 8 (B) + 1 (SA) + 1 (SW).
constexpr int DMA_PER_STAGE = 14;

// Direct global->LDS loads.  Lane l of the wave writes its 16 (or 4) bytes at
// LDS byte address lds + 16 l (4 l); the source address is per lane.  They are
// issued from inline assembly so that the compiler does not track them: it
// would otherwise make every later LDS read wait for all of them, which would
// drain the pipeline each K block.  The instructions have no register outputs
// (the data goes to LDS); every LDS read of their data follows an explicit
// vmcnt wait and a barrier below, and every reuse of a ring slot follows a
// barrier.  M0 carries the LDS address; the compiler does not allocate it.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}
// base: wave-uniform global address; off: per-lane byte offset (32 bits).
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(uniform_ptr(base)), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(off), "s"(uniform_ptr(base)), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | (((N >> 4) & 3) << 14));
}

__device__ __forceinline__ Tile decode_tile(const GemmArgs& p, const int32_t* __restrict__ offsets,
                                            const int* smTile, int NT, long l) {
  const int q = (int)(l / NT);
  int a = 0, b = p.n_groups - 1;
  while (a < b) {
    const int mid = (a + b + 1) >> 1;
    if (smTile[mid] <= q) a = mid; else b = mid - 1;
  }
  a = __builtin_amdgcn_readfirstlane(a);   // uniform: offsets come through scalar loads
  Tile t;
  t.g = a;
  const int mtg = __builtin_amdgcn_readfirstlane(smTile[a + 1] - smTile[a]);
  const int local = (int)(l - (long)smTile[a] * NT);
  t.n = local / mtg;
  const int m = local - t.n * mtg;
  t.row0 = offsets[a] + m * GM;
  // rows past total_rows (only possible with malformed offsets) are never touched
  t.rows_valid = min(GM, min(offsets[a + 1], p.total_rows) - t.row0);
  return t;
}

// Per-lane global sources of one wave's DMA instructions for a tile; the K block
// offset is added at issue time.  LDS destinations are fixed: instruction i of
// wave w writes 1 KB at (w * n_i + i) KB of its region, lane l 16 bytes at
// 16 l, i.e. row 8 (w * n_i + i) + l / 8, physical chunk l % 8, which holds the
// logical chunk (l % 8) ^ swz(row) (the swizzle is applied on the
// source side).
struct TileSrc {
  uint32_t a[4];          // byte offsets into p.a
  uint32_t b[8];          // byte offsets into the group's weights
  uint32_t sa;            // byte offset into p.as
  uint32_t sw;            // byte offset into p.bs
  const uint8_t* bbase;   // the group's weights (uniform)
};

// Source rows (in p.a) of this lane's 4 activation DMA rows and its scale row.
struct TileRows {
  int a[4];
  int sa;
};

// Row of p.a holding tile row r (rows past the group's end repeat its last row).
__device__ __forceinline__ int tile_row(const GemmArgs& p, const Tile& t, int r) {
  return min(max(t.row0 + min(r, t.rows_valid - 1), 0), p.total_rows - 1);
}

// Gather indices of a tile's 128 rows, DMA'd into an LDS table one tile ahead
// (lane l of wave w fetches row_src of tile row (w & 1) * 64 + l; waves 2 and 3
// repeat waves 0 and 1), so no register ever waits on them.
__device__ __forceinline__ void dma_tile_rows(const GemmArgs& p, const Tile& t, int wave, int lane,
                                              unsigned char* table) {
  const int r = (wave & 1) * 64 + lane;
  dma4(p.row_src, (uint32_t)tile_row(p, t, r) * 4u, lds_addr(table + (wave & 1) * 256));
}

__device__ __forceinline__ TileRows tile_rows(const GemmArgs& p, const Tile& t, const int* table,
                                              int wave, int lane) {
  TileRows r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = (wave * 4 + i) * 8 + (lane >> 3);
    r.a[i] = p.row_src ? table[rr] : tile_row(p, t, rr);
  }
  const int rs = (wave & 1) * 64 + lane;
  r.sa = p.row_src ? table[rs] : tile_row(p, t, rs);
  return r;
}

template <bool SWIGLU>
__device__ __forceinline__ TileSrc tile_sources(const GemmArgs& p, const Tile& t, const TileRows& rows,
                                                int wave, int lane) {
  TileSrc s;
  const int KS = p.K / GK;
  const int pc = lane & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (wave * 4 + i) * 8 + (lane >> 3);
    const int c = pc ^ swz(r);
    const int row = min(max(rows.a[i], 0), p.a_rows - 1);
    s.a[i] = (uint32_t)row * (uint32_t)p.K + c * 16;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rr = (wave * 8 + i) * 8 + (lane >> 3);
    const int c = pc ^ swz(rr);
    int wr = weight_row<SWIGLU>(p, t.n, rr);
    if (wr >= p.N) wr = 0;   // padding rows of a partial tile: any valid row, never stored
    s.b[i] = (uint32_t)wr * (uint32_t)p.K + c * 16;
  }
  s.bbase = p.b + (size_t)t.g * p.N * p.K;
  s.sa = (uint32_t)min(max(rows.sa, 0), p.a_rows - 1) * (uint32_t)(KS * 4);
  {
    // even lanes: this wave's first weight-scale block, odd lanes: its second
    const int nsb = p.N / 128;
    const int wn = wave & 1;
    int sb;
    if (SWIGLU) sb = (lane & 1) ? p.f / 128 + t.n : t.n;
    else sb = min(2 * t.n + wn, nsb - 1);
    s.sw = (uint32_t)(t.g * nsb + sb) * (uint32_t)(KS * 4);
  }
  return s;
}

__device__ __forceinline__ void issue_stage(const GemmArgs& p, const TileSrc& s, int kb, int wave,
                                            unsigned char* stage) {
  const uint32_t base = lds_addr(stage);
  const uint8_t* a = p.a + (size_t)kb * GK;
  const uint8_t* b = s.bbase + (size_t)kb * GK;
#pragma unroll
  for (int i = 0; i < 4; ++i) dma16(a, s.a[i], base + (wave * 4 + i) * 1024);
#pragma unroll
  for (int i = 0; i < 8; ++i) dma16(b, s.b[i], base + ST_A + (wave * 8 + i) * 1024);
  dma4(p.as + kb, s.sa, base + ST_A + ST_B + (wave & 1) * 256);
  dma4(p.bs + kb, s.sw, base + ST_A + ST_B + ST_SA + wave * 256);
}

// Barrier for LDS data only: waits for this wave's LDS operations, not for the
// DMA loads in flight (a __syncthreads() fence would drain those too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
}

template <bool SWIGLU>
__global__ __launch_bounds__(G_THREADS, 1) void grouped_gemm_kernel(GemmArgs p,
                                                                    const int32_t* __restrict__ offsets) {
  __shared__ __attribute__((aligned(16))) unsigned char sm[NSTAGE * ST_BYTES];
  __shared__ float smAmax[2][GM];
  __shared__ int smTile[G_MAX_GROUPS + 1];
  __shared__ __attribute__((aligned(16))) int smRows[2][GM];   // gather indices, by tile parity

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int KB = p.K / GK;
  const int NT = p.n_tiles_n;

  // ---- tile list: m-tiles per group, exclusive prefix in LDS ----
  if (wave == 0) {
    int carry = 0;
    for (int base = 0; base < p.n_groups; base += 64) {
      const int g = base + lane;
      int mt = 0;
      if (g < p.n_groups) mt = (offsets[g + 1] - offsets[g] + GM - 1) / GM;
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
  const long total = (long)smTile[p.n_groups] * NT;
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int nslot = gridDim.x >> 3;
  const long lo = total * xcd / 8, hi = total * (xcd + 1) / 8;
  if (lo + slot >= hi) return;

  // Loader state runs up to two K blocks ahead of the multiply.  When it starts
  // a tile it builds the tile's DMA sources from the gather table and DMAs the
  // gather indices of its next tile into the other table; those land before the
  // next tile starts (every wait below covers all DMAs older than the block
  // about to be multiplied, and the barrier publishes them to all waves).
  long ld_L = lo + slot;
  int ld_kb = 0;
  int ld_par = 0;
  bool ld_more = true;   // is there a (tile, K block) at the loader position?
  Tile ld_tile = decode_tile(p, offsets, smTile, NT, ld_L);
  TileSrc src;
  if (p.row_src) {
    dma_tile_rows(p, ld_tile, wave, lane, reinterpret_cast<unsigned char*>(smRows[0]));
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  }
#define LOADER_ISSUE(dst)                                                              \
  do {                                                                                 \
    if (ld_kb == 0) {                                                                  \
      src = tile_sources<SWIGLU>(p, ld_tile, tile_rows(p, ld_tile, smRows[ld_par], wave, lane), \
                                 wave, lane);                                          \
      if (p.row_src && ld_L + nslot < hi)                                              \
        dma_tile_rows(p, decode_tile(p, offsets, smTile, NT, ld_L + nslot), wave, lane,         \
                      reinterpret_cast<unsigned char*>(smRows[ld_par ^ 1]));           \
    }                                                                                  \
    issue_stage(p, src, ld_kb, wave, (dst));                                              \
    if (++ld_kb == KB) {                                                               \
      ld_kb = 0;                                                                       \
      ld_L += nslot;                                                                   \
      ld_par ^= 1;                                                                     \
      ld_more = ld_L < hi;                                                             \
      if (ld_more) ld_tile = decode_tile(p, offsets, smTile, NT, ld_L);                         \
    }                                                                                  \
  } while (0)

  // prologue: blocks 0 and 1 in flight
  LOADER_ISSUE(sm);
  bool next_issued = false;
  if (ld_more) {
    LOADER_ISSUE(sm + ST_BYTES);
    next_issued = true;
  }

  v4f acc[4][8];
#pragma unroll
  for (int ms = 0; ms < 4; ++ms)
#pragma unroll
    for (int ns = 0; ns < 8; ++ns) acc[ms][ns] = v4f{0.f, 0.f, 0.f, 0.f};

  long L = lo + slot;
  Tile cur = decode_tile(p, offsets, smTile, NT, L);
  int kb = 0;
  int st = 0;   // ring slot of the block being multiplied

  while (true) {
    // block `st` has landed once at most the next block's DMAs are outstanding
    if (next_issued) wait_vmcnt<DMA_PER_STAGE>(); else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();   // all lanes' DMAs visible; slot st+2 free again
    bool issued2 = false;
    if (ld_more) {
      LOADER_ISSUE(sm + ((st + 2) % NSTAGE) * ST_BYTES);
      issued2 = true;
    }

    // ---- multiply block `st` ----
    {
      const unsigned char* A = sm + st * ST_BYTES;
      const unsigned char* B = A + ST_A;
      const float* SA = reinterpret_cast<const float*>(B + ST_B);
      const float* SW = reinterpret_cast<const float*>(B + ST_B + ST_SA + wave * 256);
      const float sw0 = SW[0], sw1 = SW[1];
      float sv[4][4], c[4][4];
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        const float4 s4 = *reinterpret_cast<const float4*>(&SA[wm * 64 + ms * 16 + g16 * 4]);
        sv[ms][0] = s4.x; sv[ms][1] = s4.y; sv[ms][2] = s4.z; sv[ms][3] = s4.w;
#pragma unroll
        for (int i = 0; i < 4; ++i) c[ms][i] = sv[ms][i] * sw0;
      }
      v8i af[4];
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        const int r = wm * 64 + ms * 16 + r16;
        const uint4 lo4 = *reinterpret_cast<const uint4*>(A + op_off(r, g16 * 2));
        const uint4 hi4 = *reinterpret_cast<const uint4*>(A + op_off(r, g16 * 2 + 1));
        af[ms] = v8i{(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w,
                     (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
      }
      v4f part[2][4];
#pragma unroll
      for (int ns = 0; ns < 8; ++ns) {
        const int r = frag_row<SWIGLU>(wn, ns) + r16;
        const uint4 lo4 = *reinterpret_cast<const uint4*>(B + op_off(r, g16 * 2));
        const uint4 hi4 = *reinterpret_cast<const uint4*>(B + op_off(r, g16 * 2 + 1));
        const v8i bf = v8i{(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w,
                           (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
          part[ns & 1][ms] = mfma_fp8_16x16x128(af[ms], bf, v4f{0.f, 0.f, 0.f, 0.f});
        // promote the previous sub-tile column while this one is in the MFMA pipe
        if (ns > 0) {
          const int pn = ns - 1;
          if (pn == 4) {   // sub-tiles 4..7 use the second weight-scale block
#pragma unroll
            for (int ms = 0; ms < 4; ++ms)
#pragma unroll
              for (int i = 0; i < 4; ++i) c[ms][i] = sv[ms][i] * sw1;
          }
#pragma unroll
          for (int ms = 0; ms < 4; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[ms][pn][i] = fmaf(part[pn & 1][ms][i], c[ms][i], acc[ms][pn][i]);
        }
      }
#pragma unroll
      for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[ms][7][i] = fmaf(part[1][ms][i], c[ms][i], acc[ms][7][i]);
    }

    // ---- epilogue at the end of a tile ----
    if (kb == KB - 1) {
      lds_barrier();   // every wave has finished reading slot st
      unsigned char* E = sm + st * ST_BYTES + wave * 4096;
      if (SWIGLU) {
        // h = SiLU(g) * u; g in sub-tiles 0..3, u in 4..7 (same columns)
        float amax[4][4];
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
#pragma unroll
          for (int i = 0; i < 4; ++i) amax[ms][i] = 0.0f;
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float gv = acc[ms][c][i], uv = acc[ms][4 + c][i];
              const float hv = gv / (1.0f + expf(-gv)) * uv;
              acc[ms][c][i] = hv;
              amax[ms][i] = fmaxf(amax[ms][i], fabsf(hv));
            }
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = amax[ms][i];
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
            amax[ms][i] = v;
            if (r16 == 0) smAmax[wn][wm * 64 + ms * 16 + g16 * 4 + i] = v;
          }
        lds_barrier();
        const int hcol0 = cur.n * 128 + wn * 64;
        const int nhs = p.f / 128;
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
          float sc[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rt = wm * 64 + ms * 16 + g16 * 4 + i;
            sc[i] = scale_from_amax(fmaxf(smAmax[0][rt], smAmax[1][rt]));
            if (wn == 0 && r16 == 0 && rt < cur.rows_valid)
              p.hs[(size_t)(cur.row0 + rt) * nhs + cur.n] = sc[i];
          }
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t q = f32x2_to_e4m3(acc[ms][c][i] / sc[i], 0.0f) & 0xFFu;
              E[(g16 * 4 + i) * 64 + c * 16 + r16] = (unsigned char)q;
            }
          wave_sync_lds();
          const int rl = lane >> 2, cq = lane & 3;
          const int rt = wm * 64 + ms * 16 + rl;
          const uint4 v = *reinterpret_cast<const uint4*>(E + rl * 64 + cq * 16);
          if (rt < cur.rows_valid)
            *reinterpret_cast<uint4*>(p.h + (size_t)(cur.row0 + rt) * p.f + hcol0 + cq * 16) = v;
          wave_sync_lds();
        }
      } else {
        const int col0 = cur.n * GNB + wn * 128;
        const bool col_ok = col0 < p.N;
        uint16_t* E16 = reinterpret_cast<uint16_t*>(E);
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
#pragma unroll
          for (int ns = 0; ns < 8; ++ns)
#pragma unroll
            for (int i = 0; i < 4; ++i) E16[(g16 * 4 + i) * 128 + ns * 16 + r16] = f32_to_bf16(acc[ms][ns][i]);
          wave_sync_lds();
          const int rl = lane >> 2, q = lane & 3;
          const int rt = wm * 64 + ms * 16 + rl;
          if (col_ok && rt < cur.rows_valid) {
            uint16_t* dst = p.y + (size_t)(cur.row0 + rt) * p.N + col0 + q * 32;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              reinterpret_cast<uint4*>(dst)[j] = *reinterpret_cast<const uint4*>(E16 + rl * 128 + q * 32 + j * 8);
          }
          wave_sync_lds();
        }
      }
#pragma unroll
      for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int ns = 0; ns < 8; ++ns) acc[ms][ns] = v4f{0.f, 0.f, 0.f, 0.f};
    }

    // ---- next block ----
    if (++kb == KB) {
      kb = 0;
      L += nslot;
      if (L >= hi) break;
      cur = decode_tile(p, offsets, smTile, NT, L);
    }
    next_issued = issued2;
    st = (st + 1) % NSTAGE;
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
                          hipStream_t stream) {
  const int grid = ((num_cus() + 7) / 8) * 8;
  GemmArgs s1{};
  s1.a = aq;
  s1.as = as;
  s1.a_rows = a_rows;
  s1.row_src = row_src;
  s1.offsets = offsets;
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
  hipLaunchKernelGGL(grouped_gemm_kernel<true>, dim3(grid), dim3(G_THREADS), 0, stream, s1, offsets);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const uint8_t* h, const float* hs, const int32_t* offsets, int n_groups,
                            int total_rows, int d, int f, const uint8_t* w2, const float* w2_s,
                            uint16_t* y, hipStream_t stream) {
  const int grid = ((num_cus() + 7) / 8) * 8;
  GemmArgs s2{};
  s2.a = h;
  s2.as = hs;
  s2.a_rows = total_rows;
  s2.row_src = nullptr;
  s2.offsets = offsets;
  s2.n_groups = n_groups;
  s2.total_rows = total_rows;
  s2.K = f;
  s2.N = d;
  s2.n_tiles_n = (d + GNB - 1) / GNB;
  s2.b = w2;
  s2.bs = w2_s;
  s2.f = f;
  s2.y = y;
  hipLaunchKernelGGL(grouped_gemm_kernel<false>, dim3(grid), dim3(G_THREADS), 0, stream, s2, offsets);
  return hipGetLastError();
}

}  // namespace moe
