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

__device__ __forceinline__ int op_off(int r, int c) { return r * GK + ((c ^ ((r >> 1) & 7)) << 4); }

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

// Source pointers of one thread's load slots for the current tile.
struct TileSrc {
  const uint8_t* a[4];   // activation rows: 4 16-byte chunks per K block
  const uint8_t* b[8];   // weight rows: 8 16-byte chunks per K block
  const float* sa;       // activation scales of row tid (tid < 128)
  const float* sw0;      // weight scales of this wave's two 128-row blocks
  const float* sw1;
  uint32_t b_ok;         // bit it: weight row of slot it exists
};

// Registers holding one K block in flight between global memory and LDS.
struct Stage {
  uint4 a[4];
  uint4 b[8];
  float sa, sw0, sw1;
};

__device__ __forceinline__ Tile decode_tile(const GemmArgs& p, const int* smTile, int NT, long l) {
  const int q = (int)(l / NT);
  int a = 0, b = p.n_groups - 1;
  while (a < b) {
    const int mid = (a + b + 1) >> 1;
    if (smTile[mid] <= q) a = mid; else b = mid - 1;
  }
  Tile t;
  t.g = a;
  const int mtg = smTile[a + 1] - smTile[a];
  const int local = (int)(l - (long)smTile[a] * NT);
  t.n = local / mtg;
  const int m = local - t.n * mtg;
  t.row0 = p.offsets[a] + m * GM;
  // rows past total_rows (only possible with malformed offsets) are never touched
  t.rows_valid = min(GM, min(p.offsets[a + 1], p.total_rows) - t.row0);
  return t;
}

template <bool SWIGLU>
__device__ __forceinline__ TileSrc tile_sources(const GemmArgs& p, const Tile& t, int tid, int wn) {
  TileSrc s;
  const int KS = p.K / GK;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = (tid + G_THREADS * it) >> 3, c = (tid + G_THREADS * it) & 7;
    int row = min(max(t.row0 + min(r, t.rows_valid - 1), 0), p.total_rows - 1);
    if (p.row_src) row = p.row_src[row];
    row = min(max(row, 0), p.a_rows - 1);
    s.a[it] = p.a + (size_t)row * p.K + c * 16;
  }
  {
    int srow = min(max(t.row0 + min(tid & (GM - 1), t.rows_valid - 1), 0), p.total_rows - 1);
    if (p.row_src) srow = p.row_src[srow];
    srow = min(max(srow, 0), p.a_rows - 1);
    s.sa = p.as + (size_t)srow * KS;
  }
  s.b_ok = 0;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int rr = (tid + G_THREADS * it) >> 3, c = (tid + G_THREADS * it) & 7;
    const int wr = weight_row<SWIGLU>(p, t.n, rr);
    const bool ok = wr < p.N;
    s.b_ok |= (ok ? 1u : 0u) << it;
    s.b[it] = p.b + ((size_t)t.g * p.N + (ok ? wr : 0)) * p.K + c * 16;
  }
  const int nsb = p.N / 128;
  int sb0, sb1;
  if (SWIGLU) {
    sb0 = t.n;
    sb1 = p.f / 128 + t.n;
  } else {
    sb0 = sb1 = min(2 * t.n + wn, nsb - 1);
  }
  s.sw0 = p.bs + ((size_t)t.g * nsb + sb0) * KS;
  s.sw1 = p.bs + ((size_t)t.g * nsb + sb1) * KS;
  return s;
}

__device__ __forceinline__ void issue_loads(const TileSrc& s, int kb, int tid, Stage& st) {
  const size_t off = (size_t)kb * GK;
#pragma unroll
  for (int it = 0; it < 4; ++it) st.a[it] = *reinterpret_cast<const uint4*>(s.a[it] + off);
#pragma unroll
  for (int it = 0; it < 8; ++it)
    st.b[it] = ((s.b_ok >> it) & 1u) ? *reinterpret_cast<const uint4*>(s.b[it] + off)
                                     : make_uint4(0, 0, 0, 0);
  st.sa = s.sa[kb];
  st.sw0 = s.sw0[kb];
  st.sw1 = s.sw1[kb];
}

__device__ __forceinline__ void commit_stage(const Stage& st, int tid, unsigned char* A,
                                             unsigned char* B, float* SA) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = (tid + G_THREADS * it) >> 3, c = (tid + G_THREADS * it) & 7;
    *reinterpret_cast<uint4*>(A + op_off(r, c)) = st.a[it];
  }
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int rr = (tid + G_THREADS * it) >> 3, c = (tid + G_THREADS * it) & 7;
    *reinterpret_cast<uint4*>(B + op_off(rr, c)) = st.b[it];
  }
  if (tid < GM) SA[tid] = st.sa;
}

template <bool SWIGLU>
__global__ __launch_bounds__(G_THREADS, 1) void grouped_gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) unsigned char smA[2][GM * GK];
  __shared__ __attribute__((aligned(16))) unsigned char smB[2][GNB * GK];
  __shared__ float smSA[2][GM];
  __shared__ __attribute__((aligned(16))) unsigned char smE[4][4096];
  __shared__ float smAmax[2][GM];
  __shared__ int smTile[G_MAX_GROUPS + 1];

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
      if (g < p.n_groups) mt = (p.offsets[g + 1] - p.offsets[g] + GM - 1) / GM;
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
  long L = lo + slot;
  if (L >= hi) return;

  v4f acc[4][8];
#pragma unroll
  for (int ms = 0; ms < 4; ++ms)
#pragma unroll
    for (int ns = 0; ns < 8; ++ns) acc[ms][ns] = v4f{0.f, 0.f, 0.f, 0.f};

  Tile cur = decode_tile(p, smTile, NT, L);
  TileSrc src = tile_sources<SWIGLU>(p, cur, tid, wn);
  Stage st;
  issue_loads(src, 0, tid, st);
  float sw0 = st.sw0, sw1 = st.sw1;
  commit_stage(st, tid, smA[0], smB[0], smSA[0]);
  __syncthreads();
  int buf = 0, kb = 0;

  while (true) {
    // ---- issue the loads of the next (tile, K block) ----
    int nkb = kb + 1;
    long nL = L;
    bool has_next = true;
    Tile nxt = cur;
    if (nkb == KB) {
      nkb = 0;
      nL = L + nslot;
      has_next = nL < hi;
      if (has_next) {
        nxt = decode_tile(p, smTile, NT, nL);
        src = tile_sources<SWIGLU>(p, nxt, tid, wn);
      }
    }
    if (has_next) issue_loads(src, nkb, tid, st);

    // ---- multiply the current K block ----
    {
      const unsigned char* A = smA[buf];
      const unsigned char* B = smB[buf];
      float c0[4][4], c1[4][4];
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        const float4 s4 = *reinterpret_cast<const float4*>(&smSA[buf][wm * 64 + ms * 16 + g16 * 4]);
        const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c0[ms][i] = sv[i] * sw0;
          c1[ms][i] = sv[i] * sw1;
        }
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
#pragma unroll
      for (int ns = 0; ns < 8; ++ns) {
        const int r = frag_row<SWIGLU>(wn, ns) + r16;
        const uint4 lo4 = *reinterpret_cast<const uint4*>(B + op_off(r, g16 * 2));
        const uint4 hi4 = *reinterpret_cast<const uint4*>(B + op_off(r, g16 * 2 + 1));
        const v8i bf = v8i{(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w,
                           (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
          const v4f part = mfma_fp8_16x16x128(af[ms], bf, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[ms][ns][i] = fmaf(part[i], ns < 4 ? c0[ms][i] : c1[ms][i], acc[ms][ns][i]);
        }
      }
    }

    // ---- epilogue at the end of a tile ----
    if (kb == KB - 1) {
      unsigned char* E = smE[wave];
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
        __syncthreads();
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

    if (!has_next) break;
    commit_stage(st, tid, smA[buf ^ 1], smB[buf ^ 1], smSA[buf ^ 1]);
    sw0 = st.sw0;
    sw1 = st.sw1;
    __syncthreads();
    buf ^= 1;
    kb = nkb;
    L = nL;
    cur = nxt;
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
  hipLaunchKernelGGL(grouped_gemm_kernel<true>, dim3(grid), dim3(G_THREADS), 0, stream, s1);
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
  hipLaunchKernelGGL(grouped_gemm_kernel<false>, dim3(grid), dim3(G_THREADS), 0, stream, s2);
  return hipGetLastError();
}

}  // namespace moe
