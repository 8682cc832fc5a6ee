// Grouped FP8 GEMM of the SwiGLU experts for few rows per expert (decode-sized
// batches): the same computation as grouped_gemm_kernel (the "DeepSeek-V3"
// summary page, section 6; the book's chapter 16 "Periodic high-precision
// promotion", chapter 17), organised for streaming the expert weights from HBM
// rather than for reuse.
//
// A tile is at most 16 rows of one group (an "m-chunk") against 256 weight
// rows.  Each of the 8 waves owns 32 weight rows and streams their FP8 codes
// from global memory straight into registers, SM_D K blocks ahead, with no
// LDS ring and no barrier inside the K loop.  The tile's 16 activation rows
// (shared by the waves and by every weight block of the group, so they come
// from L2) are staged in LDS once per tile, which keeps the memory pipeline
// for the weight stream; this bounds K at kSmallMaxK.  In stage 1
// wave w owns the gate rows w*16 .. +15 and the matching up rows, so SiLU(g)*u
// is formed in registers; the 1x128 amax across the 8 waves goes through LDS.
// Scales: the rows' activation scales and the two weight-scale columns of the
// tile are staged in LDS once per tile.  Promotion as in the large kernel: one
// 16x16x128 MFMA per K block and output block, its partial sum multiplied by
// activation scale x weight scale and added to an FP32 accumulator.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int SM_M = 16;          // rows per m-chunk
constexpr int SM_THREADS = 512;   // 8 waves
constexpr int SM_D = 4;           // K blocks of weight loads in flight per wave
constexpr int SM_MAX_KB = kSmallMaxK / 128;
constexpr int SM_AROW = kSmallMaxK + 16;   // LDS bytes per staged activation row (padded)
constexpr int SM_MAX_GROUPS = 1024;

struct SmallArgs {
  const uint8_t* a;         // [a_rows, K] E4M3
  const float* as;          // [a_rows, K/128]
  int a_rows;
  const int32_t* row_src;   // [total rows] or null (identity)
  int n_groups;
  int total_rows;
  int K;
  int N;                    // weight rows per group
  int n_tiles_n;            // 256-row weight blocks per group
  const uint8_t* b;         // [n_groups, N, K]
  const float* bs;          // [n_groups, N/128, K/128]
  int f;                    // stage 1: N = 2f
  uint8_t* h;
  float* hs;
  uint16_t* y;
};

// Weight fragments are loaded as whole 128-byte lines: for a fragment of 16
// weight rows R .. R+15 (one K block), lane (g, j) (g = lane / 16, j = lane % 16)
// loads 16 bytes of chunk c = 2g + (j >= 8) from row R + j % 8 (load x) and from
// row R + 8 + j % 8 (load y), so each load instruction reads 8 rows entirely,
// with non-temporal loads (the weights are read once per launch).  Streaming
// whole lines this way is faster than the fragment's own layout, in which a
// line is split between two instructions.  Two DPP moves per register
// (rotate each 16-lane row by 8, write only half of its lanes) then give lane
// (g, j) chunks 2g and 2g + 1 of row R + j, the MFMA's operand layout:
//   frag lo = x, with lanes 8..15 of each row taken from y's lanes 0..7
//   frag hi = y, with lanes 0..7 of each row taken from x's lanes 8..15
typedef int i32x4 __attribute__((ext_vector_type(4)));

struct LinePair {
  i32x4 x, y;
};

__device__ __forceinline__ LinePair load_lines(const uint8_t* x_src, const uint8_t* y_src) {
  return {__builtin_nontemporal_load(reinterpret_cast<const i32x4*>(x_src)),
          __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(y_src))};
}

__device__ __forceinline__ v8i lines_to_frag(const LinePair& l) {
  constexpr int ROW_ROR8 = 0x128;
  v8i f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = __builtin_amdgcn_update_dpp(l.x[i], l.y[i], ROW_ROR8, 0xF, 0xC, false);
    f[4 + i] = __builtin_amdgcn_update_dpp(l.y[i], l.x[i], ROW_ROR8, 0xF, 0x3, false);
  }
  return f;
}

struct Frag2 {
  LinePair b0, b1;
};

// Activation fragment of row r16, K bytes kb*128 + g16*32 .. +31, from the
// tile's rows staged in LDS (row stride SM_AROW: consecutive rows start 16
// bytes apart in the banks, so the 16 rows of a read hit different banks).
__device__ __forceinline__ v8i lds_frag(const uint8_t* sA, int r16, int g16, int kb) {
  const uint8_t* q = sA + r16 * SM_AROW + kb * 128 + g16 * 32;
  const uint4 lo = *reinterpret_cast<const uint4*>(q);
  const uint4 hi = *reinterpret_cast<const uint4*>(q + 16);
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// POW2: H is requantised with the power-of-two scale rule (the variant whose
// scales are all powers of two; with such scales the promotion is exact).
template <bool SWIGLU, bool POW2>
__global__ __launch_bounds__(SM_THREADS, 1) void grouped_gemm_small_kernel(
    SmallArgs p, const int32_t* __restrict__ offsets) {
  __shared__ int smTile[SM_MAX_GROUPS + 1];        // m-chunk prefix over groups
  __shared__ __attribute__((aligned(16))) float sSA[SM_MAX_KB][SM_M];   // [kb][row]
  __shared__ float sSW[2][SM_MAX_KB];              // weight scales of column sets 0 / 1
  __shared__ float sAmax[SM_THREADS / 64][SM_M];
  __shared__ int sRow[SM_M];
  __shared__ __attribute__((aligned(16))) uint8_t sA[SM_M * SM_AROW];   // the tile's activation rows

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int KB = p.K / 128;
  const int NT = p.n_tiles_n;

  if (wave == 0) {
    int carry = 0;
    for (int base = 0; base < p.n_groups; base += 64) {
      const int g = base + lane;
      int mt = 0;
      if (g < p.n_groups) mt = (offsets[g + 1] - offsets[g] + SM_M - 1) / SM_M;
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

  for (int l = lo + slot; l < hi; l += nslot) {
    // tile l: group by binary search over the m-chunk prefix, then n-major,
    // m-chunk fastest (the chunks sharing a weight block run together)
    const int q = l / NT;
    int ga = 0, gb = p.n_groups - 1;
    while (ga < gb) {
      const int mid = (ga + gb + 1) >> 1;
      if (smTile[mid] <= q) ga = mid; else gb = mid - 1;
    }
    const int g = __builtin_amdgcn_readfirstlane(ga);
    const int mt = __builtin_amdgcn_readfirstlane(smTile[g + 1] - smTile[g]);
    const int local = l - smTile[g] * NT;
    const int n = local / mt;
    const int m = local - n * mt;
    const int row0 = offsets[g] + m * SM_M;
    const int rows_valid = min(SM_M, min(offsets[g + 1], p.total_rows) - row0);

    // ---- stage the rows' sources and scales ----
    if (tid < SM_M) {
      const int rr = min(max(row0 + min(tid, rows_valid - 1), 0), p.total_rows - 1);
      int src = p.row_src ? p.row_src[rr] : rr;
      sRow[tid] = min(max(src, 0), p.a_rows - 1);
    }
    __syncthreads();
    for (int i = tid; i < KB * SM_M; i += SM_THREADS) {
      const int r = i / KB, kb = i - r * KB;
      sSA[kb][r] = p.as[(size_t)sRow[r] * KB + kb];
    }
    const int nsb = p.N / 128;
    for (int i = tid; i < 2 * KB; i += SM_THREADS) {
      const int c = i / KB, kb = i - c * KB;
      int sb;
      if (SWIGLU) sb = c ? p.f / 128 + n : n;
      else sb = min(2 * n + c, nsb - 1);
      sSW[c][kb] = p.bs[(size_t)(g * nsb + sb) * KB + kb];
    }
    // the tile's 16 activation rows, once per tile (they come from L2: every
    // weight block of the group reads the same rows); the waves then read
    // their fragments from LDS instead of each loading them per K block
    {
      const int c16 = p.K / 16;
      for (int i = tid; i < SM_M * c16; i += SM_THREADS) {
        const int r = i / c16, c = i - r * c16;
        *reinterpret_cast<uint4*>(&sA[r * SM_AROW + c * 16]) =
            *reinterpret_cast<const uint4*>(p.a + (size_t)sRow[r] * p.K + c * 16);
      }
    }
    __syncthreads();

    // ---- this wave's operands: activation row r16 of the tile (in LDS); weight
    // rows of the two 16-column blocks (stage 1: gate and up of h columns wave*16 .. +15;
    // stage 2: rows wave*32 .. +31 of the 256-row block) ----
    int wr0, wr1;
    if (SWIGLU) {
      wr0 = n * 128 + wave * 16 + r16;
      wr1 = p.f + n * 128 + wave * 16 + r16;
    } else {
      wr0 = n * 256 + wave * 32 + r16;
      wr1 = wr0 + 16;
    }
    const bool col0_ok = SWIGLU || wr0 - r16 < p.N;
    const bool col1_ok = SWIGLU || wr1 - r16 < p.N;
    // whole-line loads: this lane reads chunk 2 g16 + (r16 >= 8) of rows
    // base + r16 % 8 and base + 8 + r16 % 8 of each fragment (rows past the
    // group's weights, in a partial last block, read its last row instead;
    // their columns are never stored)
    const uint8_t* gb_ = p.b + (size_t)g * p.N * p.K;
    const int lr = r16 & 7, lc = (2 * g16 + (r16 >> 3)) * 16;
    const int fb0 = wr0 - r16, fb1 = wr1 - r16;
    const uint8_t* pb0x = gb_ + (size_t)min(fb0 + lr, p.N - 1) * p.K + lc;
    const uint8_t* pb0y = gb_ + (size_t)min(fb0 + 8 + lr, p.N - 1) * p.K + lc;
    const uint8_t* pb1x = gb_ + (size_t)min(fb1 + lr, p.N - 1) * p.K + lc;
    const uint8_t* pb1y = gb_ + (size_t)min(fb1 + 8 + lr, p.N - 1) * p.K + lc;
    // stage 2: waves 0..3 lie in weight-scale block 2n, waves 4..7 in 2n+1
    const int swc0 = SWIGLU ? 0 : (wave >= 4 ? 1 : 0);
    const int swc1 = SWIGLU ? 1 : swc0;

    v4f acc0 = v4f{0.f, 0.f, 0.f, 0.f}, acc1 = v4f{0.f, 0.f, 0.f, 0.f};
    Frag2 buf[SM_D];
#pragma unroll
    for (int j = 0; j < SM_D; ++j) {
      if (j < KB) {
        buf[j].b0 = load_lines(pb0x + j * 128, pb0y + j * 128);
        buf[j].b1 = load_lines(pb1x + j * 128, pb1y + j * 128);
      }
    }
    v8i a_next = lds_frag(sA, r16, g16, 0);
    for (int kb0 = 0; kb0 < KB; kb0 += SM_D) {
#pragma unroll
      for (int j = 0; j < SM_D; ++j) {
        const int kb = kb0 + j;
        if (kb < KB) {
          const v8i af = a_next;
          if (kb + 1 < KB) a_next = lds_frag(sA, r16, g16, kb + 1);
          const v4f p0 = mfma_fp8_16x16x128(af, lines_to_frag(buf[j].b0), v4f{0.f, 0.f, 0.f, 0.f});
          const v4f p1 = mfma_fp8_16x16x128(af, lines_to_frag(buf[j].b1), v4f{0.f, 0.f, 0.f, 0.f});
          if (kb + SM_D < KB) {
            const int o = (kb + SM_D) * 128;
            buf[j].b0 = load_lines(pb0x + o, pb0y + o);
            buf[j].b1 = load_lines(pb1x + o, pb1y + o);
          }
          const float4 sa = *reinterpret_cast<const float4*>(&sSA[kb][g16 * 4]);
          const float s0 = sSW[swc0][kb], s1 = sSW[swc1][kb];
          acc0[0] = fmaf(p0[0], sa.x * s0, acc0[0]);
          acc0[1] = fmaf(p0[1], sa.y * s0, acc0[1]);
          acc0[2] = fmaf(p0[2], sa.z * s0, acc0[2]);
          acc0[3] = fmaf(p0[3], sa.w * s0, acc0[3]);
          acc1[0] = fmaf(p1[0], sa.x * s1, acc1[0]);
          acc1[1] = fmaf(p1[1], sa.y * s1, acc1[1]);
          acc1[2] = fmaf(p1[2], sa.z * s1, acc1[2]);
          acc1[3] = fmaf(p1[3], sa.w * s1, acc1[3]);
        }
      }
    }

    // ---- epilogue: lane holds rows g16*4 + i, column r16 of its blocks ----
    if (SWIGLU) {
      float hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gv = acc0[i], uv = acc1[i];
        hv[i] = swiglu_f32(gv, uv);
        float a = fabsf(hv[i]);
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
        if (r16 == 0) sAmax[wave][g16 * 4 + i] = a;
      }
      __syncthreads();
      const int nhs = p.f / 128;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = g16 * 4 + i;
        float a = sAmax[0][r];
#pragma unroll
        for (int w = 1; w < SM_THREADS / 64; ++w) a = fmaxf(a, sAmax[w][r]);
        const float sc = tile_scale<POW2>(a);
        if (r < rows_valid) {
          const float qv = Divider(sc)(hv[i]);   // correctly rounded FP32 quotient
          p.h[(size_t)(row0 + r) * p.f + n * 128 + wave * 16 + r16] =
              (uint8_t)(f32x2_to_e4m3(qv, 0.0f) & 0xFFu);
          if (wave == 0 && r16 == 0) p.hs[(size_t)(row0 + r) * nhs + n] = sc;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = g16 * 4 + i;
        if (r < rows_valid) {
          uint16_t* dst = p.y + (size_t)(row0 + r) * p.N + n * 256 + wave * 32 + r16;
          if (col0_ok) dst[0] = f32_to_bf16(acc0[i]);
          if (col1_ok) dst[16] = f32_to_bf16(acc1[i]);
        }
      }
    }
    __syncthreads();   // sRow, sSA, sSW, sAmax are rewritten by the next tile
  }
}

static int g_num_cus_small[64];

static int num_cus_small() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (g_num_cus_small[dev] == 0) {
    int nc = 0;
    if (hipDeviceGetAttribute(&nc, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || nc <= 0)
      nc = 256;
    g_num_cus_small[dev] = nc;
  }
  return g_num_cus_small[dev];
}

hipError_t launch_gemm_up_small(const uint8_t* aq, const float* as, int a_rows,
                                const int32_t* row_src, const int32_t* offsets, int n_groups,
                                int total_rows, int d, int f, const uint8_t* w13,
                                const float* w13_s, uint8_t* h, float* hs, bool pow2,
                                hipStream_t stream) {
  SmallArgs s{};
  s.a = aq; s.as = as; s.a_rows = a_rows; s.row_src = row_src; s.n_groups = n_groups;
  s.total_rows = total_rows; s.K = d; s.N = 2 * f; s.n_tiles_n = f / 128; s.b = w13; s.bs = w13_s;
  s.f = f; s.h = h; s.hs = hs;
  const int grid = ((num_cus_small() + 7) / 8) * 8;   // persistent: one workgroup per CU
  if (pow2)
    hipLaunchKernelGGL((grouped_gemm_small_kernel<true, true>), dim3(grid), dim3(SM_THREADS), 0, stream, s,
                       offsets);
  else
    hipLaunchKernelGGL((grouped_gemm_small_kernel<true, false>), dim3(grid), dim3(SM_THREADS), 0, stream, s,
                       offsets);
  return hipGetLastError();
}

hipError_t launch_gemm_down_small(const uint8_t* h, const float* hs, const int32_t* offsets,
                                  int n_groups, int total_rows, int d, int f, const uint8_t* w2,
                                  const float* w2_s, uint16_t* y, hipStream_t stream) {
  SmallArgs s{};
  s.a = h; s.as = hs; s.a_rows = total_rows; s.row_src = nullptr; s.n_groups = n_groups;
  s.total_rows = total_rows; s.K = f; s.N = d; s.n_tiles_n = (d + 255) / 256; s.b = w2; s.bs = w2_s;
  s.f = f; s.y = y;
  const int grid = ((num_cus_small() + 7) / 8) * 8;   // persistent: one workgroup per CU
  hipLaunchKernelGGL((grouped_gemm_small_kernel<false, false>), dim3(grid), dim3(SM_THREADS), 0, stream, s,
                     offsets);
  return hipGetLastError();
}

}  // namespace moe
