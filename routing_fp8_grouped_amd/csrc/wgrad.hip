// Weight-gradient GEMM of the experts (the "DeepSeek-V3" summary page, section
// 6: Wgrad in FP8; the book's chapter 17 "One linear layer creates three
// GEMMs" and the 128x1 regrouping with power-of-two scales).
//
// For every expert e and its padded row range [k0, k0 + Ke) of the K-major
// operands (see backward.hip):
//   dW[e][m][n] = sum_{kk < Ke} A[m][k0 + kk] * B[n][k0 + kk] * sA[kb][m] * sB[kb][n]
// with A [M, Kp], B [N, Kp] E4M3 codes and power-of-two scales per row and
// 128-wide K block (kb = (k0 + kk) / 128).  Both scales go into the
// block-scaled MFMA as E8M0 codes (lane l of a fragment supplies the code of
// its own A row or B row), so the accumulator is chained through the
// instruction.  Output FP32 [G][M][N]; an expert without rows gets zeros.
//
// Two forms.  When M and N are multiples of 256 (the V3 shapes), wgrad256_kernel
// (below): 256 x 256 output tiles, each walked across the experts of a slice.
// Otherwise wgrad_kernel: one workgroup per 128 x 128 output tile of one
// expert, 4 waves in a 2 x 2 arrangement, 64 x 64 each (4 x 4 MFMA tiles).
// Both stage K blocks through a double-buffered LDS tile (A and B: 128 bytes
// per row) with the next block's global loads in registers while the current
// one is multiplied, and sum each output element's K blocks in the same
// order, so they give the same results.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int WG_MAX_GROUPS = 1024;

__device__ __forceinline__ void wg_block_prefix(const int32_t* __restrict__ offsets, int n_groups, int* pb,
                                                int lane) {
  int carry = 0;
  for (int base = 0; base < n_groups; base += 64) {
    const int g = base + lane;
    int nb = 0;
    if (g < n_groups) nb = (offsets[g + 1] - offsets[g] + 127) >> 7;
    int v = nb;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(v, o);
      if (lane >= o) v += u;
    }
    if (g < n_groups) pb[g + 1] = carry + v;
    carry += __shfl(v, 63);
  }
  if (lane == 0) pb[0] = 0;
}

__device__ __forceinline__ int wg_off(int r, int c) { return r * 128 + ((c ^ op_swz(r)) << 4); }

__device__ __forceinline__ v8i wg_frag(const unsigned char* T, int r, int g16) {
  const uint4 lo = *reinterpret_cast<const uint4*>(T + wg_off(r, g16 * 2));
  const uint4 hi = *reinterpret_cast<const uint4*>(T + wg_off(r, g16 * 2 + 1));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Chunk i (< 4) of thread tid: row (tid + 256 i) / 8, 16-byte chunk (tid + 256 i) % 8.
#define WG_CHUNK(i) const int r##i = (tid + 256 * i) >> 3, c##i = (tid + 256 * i) & 7
#define WG_LOAD(i, kblk)                                                                            \
  ra##i = *reinterpret_cast<const uint4*>(A + (size_t)(m0 + r##i) * Kp + (size_t)(kblk) * 128 + c##i * 16); \
  rb##i = *reinterpret_cast<const uint4*>(B + (size_t)(n0 + r##i) * Kp + (size_t)(kblk) * 128 + c##i * 16)
#define WG_STORE(i)                                                \
  *reinterpret_cast<uint4*>(tA + wg_off(r##i, c##i)) = ra##i;      \
  *reinterpret_cast<uint4*>(tB + wg_off(r##i, c##i)) = rb##i

__global__ __launch_bounds__(256) void wgrad_kernel(const uint8_t* __restrict__ A, const float* __restrict__ sA,
                                                    const uint8_t* __restrict__ B, const float* __restrict__ sB,
                                                    const int32_t* __restrict__ offsets, int n_groups, int M,
                                                    int N, int Kp, float* __restrict__ out) {
  __shared__ int pb[WG_MAX_GROUPS + 1];
  __shared__ __attribute__((aligned(16))) unsigned char sm[2][2][128 * 128];   // [buffer][A|B]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1, g16 = lane >> 4, r16 = lane & 15;
  const int e = blockIdx.y;
  const int tiles_n = N / 128;
  const int m0 = (blockIdx.x / tiles_n) * 128, n0 = (blockIdx.x % tiles_n) * 128;
  if (wave == 0) wg_block_prefix(offsets, n_groups, pb, lane);
  __syncthreads();
  const int kb0 = pb[e], nkb = pb[e + 1] - pb[e];
  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  // global -> register staging: thread t moves 16-byte chunks t + 256 i
  // (i < 4) of the A tile and of the B tile
  WG_CHUNK(0); WG_CHUNK(1); WG_CHUNK(2); WG_CHUNK(3);
  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
  if (nkb > 0) {
    WG_LOAD(0, kb0); WG_LOAD(1, kb0); WG_LOAD(2, kb0); WG_LOAD(3, kb0);
  }
  for (int kb = 0; kb < nkb; ++kb) {
    unsigned char* tA = sm[kb & 1][0];
    unsigned char* tB = sm[kb & 1][1];
    WG_STORE(0); WG_STORE(1); WG_STORE(2); WG_STORE(3);
    __syncthreads();
    if (kb + 1 < nkb) {
      WG_LOAD(0, kb0 + kb + 1); WG_LOAD(1, kb0 + kb + 1); WG_LOAD(2, kb0 + kb + 1); WG_LOAD(3, kb0 + kb + 1);
    }
    const size_t srow = (size_t)(kb0 + kb);
    int ea[4], eb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ea[i] = (int)(__float_as_uint(sA[srow * M + m0 + wm * 64 + i * 16 + r16]) >> 23);
      eb[i] = (int)(__float_as_uint(sB[srow * N + n0 + wn * 64 + i * 16 + r16]) >> 23);
    }
    v8i af[4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) af[ms] = wg_frag(tA, wm * 64 + ms * 16 + r16, g16);
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const v8i bf = wg_frag(tB, wn * 64 + ns * 16 + r16, g16);
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) acc[ms][ns] = mfma_fp8_16x16x128_scaled(af[ms], bf, acc[ms][ns], ea[ms], eb[ns]);
    }
  }
  float* o = out + (size_t)e * M * N;
#pragma unroll
  for (int ms = 0; ms < 4; ++ms)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[(size_t)(m0 + wm * 64 + ms * 16 + g16 * 4 + i) * N + n0 + wn * 64 + ns * 16 + r16] = acc[ms][ns][i];
}

// ---- 256 x 256 tiles (M and N multiples of 256) ----
// Half the operand bytes per FLOP of the 128 x 128 form: a workgroup of 8
// waves (4 x 2, each 64 rows x 128 columns, 4 x 8 MFMA tiles) owns one 256 x
// 256 output tile and walks the experts of its slice (e = slice, slice + S,
// ...) as one stream of K blocks, the next block's operands and scales loaded
// into registers while the current one is multiplied.  The MFMA takes B as
// its first operand, so a lane holds four consecutive output columns of one
// row and stores them with one 16-byte store.
constexpr int W2_THREADS = 512;
constexpr int W2_T = 256;

#define W2_CHUNK(i) const int q##i = (tid + 512 * i) >> 3, k##i = (tid + 512 * i) & 7
#define W2_LOAD(i, kblk)                                                                            \
  ra##i = *reinterpret_cast<const uint4*>(A + (size_t)(m0 + q##i) * Kp + (size_t)(kblk) * 128 + k##i * 16); \
  rb##i = *reinterpret_cast<const uint4*>(B + (size_t)(n0 + q##i) * Kp + (size_t)(kblk) * 128 + k##i * 16)
#define W2_STORE(i)                                                \
  *reinterpret_cast<uint4*>(tA + wg_off(q##i, k##i)) = ra##i;      \
  *reinterpret_cast<uint4*>(tB + wg_off(q##i, k##i)) = rb##i
#define W2_LOAD_SCALES(kblk)                                                        \
  _Pragma("unroll") for (int i = 0; i < 4; ++i)                                     \
      na[i] = sA[(size_t)(kblk) * M + m0 + wm * 64 + i * 16 + r16];                 \
  _Pragma("unroll") for (int i = 0; i < 8; ++i)                                     \
      nb[i] = sB[(size_t)(kblk) * N + n0 + wn * 128 + i * 16 + r16]

// Lane l of wave (wm, wn), MFMA tile (ms, ns): output row 64 wm + 16 ms + l % 16,
// columns 128 wn + 16 ns + 4 (l / 16) + [0, 4) of the tile at o (row stride N).
template <bool ZERO>
__device__ __forceinline__ void w2_store(float* __restrict__ o, int N, uint32_t lane_off, const v4f (&acc)[4][8]) {
  asm volatile("" : "+v"(lane_off));   // the 32 addresses are formed here, not held across the K loop
  const v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) {
    float* row = o + (size_t)(ms * 16) * N + lane_off;
#pragma unroll
    for (int ns = 0; ns < 8; ++ns) *reinterpret_cast<v4f*>(row + ns * 16) = ZERO ? z : acc[ms][ns];
  }
}

__global__ __launch_bounds__(W2_THREADS) void wgrad256_kernel(const uint8_t* __restrict__ A,
                                                              const float* __restrict__ sA,
                                                              const uint8_t* __restrict__ B,
                                                              const float* __restrict__ sB,
                                                              const int32_t* __restrict__ offsets,
                                                              int n_groups, int M, int N, int Kp,
                                                              float* __restrict__ out) {
  __shared__ int pb[WG_MAX_GROUPS + 1];
  __shared__ __attribute__((aligned(16))) unsigned char sm[2][2][W2_T * 128];   // [buffer][A|B]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1, g16 = lane >> 4, r16 = lane & 15;
  const int slice = blockIdx.y, S = gridDim.y;
  const int tiles_n = N / W2_T;
  const int m0 = (blockIdx.x / tiles_n) * W2_T, n0 = (blockIdx.x % tiles_n) * W2_T;
  if (wave == 0) wg_block_prefix(offsets, n_groups, pb, lane);
  __syncthreads();
  const uint32_t lane_off = (uint32_t)(wm * 64 + r16) * N + wn * 128 + g16 * 4;
  float* const tile0 = out + (size_t)m0 * N + n0;
  v4f acc[4][8];
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = zero;
  W2_CHUNK(0); W2_CHUNK(1); W2_CHUNK(2); W2_CHUNK(3);
  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
  float na[4], nb[8];
  int le = slice;   // expert of the next block to load; experts without rows get zeros on the way
  for (; le < n_groups && pb[le + 1] == pb[le]; le += S) w2_store<true>(tile0 + (size_t)le * M * N, N, lane_off, acc);
  int lkb = 0;
  if (le < n_groups) {
    W2_LOAD(0, pb[le]); W2_LOAD(1, pb[le]); W2_LOAD(2, pb[le]); W2_LOAD(3, pb[le]);
    W2_LOAD_SCALES(pb[le]);
  }
  int buf = 0;
  while (le < n_groups) {   // uniform: pb and the iterators are the same in every thread
    const int ce = le;
    unsigned char* tA = sm[buf][0];
    unsigned char* tB = sm[buf][1];
    W2_STORE(0); W2_STORE(1); W2_STORE(2); W2_STORE(3);
    int ea[4], eb[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) ea[i] = (int)(__float_as_uint(na[i]) >> 23);
#pragma unroll
    for (int i = 0; i < 8; ++i) eb[i] = (int)(__float_as_uint(nb[i]) >> 23);
    if (++lkb == pb[le + 1] - pb[le]) {
      lkb = 0;
      le = n_groups;   // no next block unless the search finds one
      for (int e = ce + S; e < n_groups; e += S)
        if (pb[e + 1] > pb[e]) { le = e; break; }
    }
    __syncthreads();
    if (le < n_groups) {
      const int kb = pb[le] + lkb;
      W2_LOAD(0, kb); W2_LOAD(1, kb); W2_LOAD(2, kb); W2_LOAD(3, kb);
      W2_LOAD_SCALES(kb);
    }
    v8i af[4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) af[ms] = wg_frag(tA, wm * 64 + ms * 16 + r16, g16);
#pragma unroll
    for (int ns = 0; ns < 8; ++ns) {
      const v8i bf = wg_frag(tB, wn * 128 + ns * 16 + r16, g16);
#pragma unroll
      for (int ms = 0; ms < 4; ++ms)
        acc[ms][ns] = mfma_fp8_16x16x128_scaled(bf, af[ms], acc[ms][ns], eb[ns], ea[ms]);
    }
    if (le != ce) {   // last block of expert ce
      w2_store<false>(tile0 + (size_t)ce * M * N, N, lane_off, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = zero;
      for (int e = ce + S; e < le; e += S) w2_store<true>(tile0 + (size_t)e * M * N, N, lane_off, acc);
    }
    buf ^= 1;
  }
}

hipError_t launch_wgrad(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                        const int32_t* offsets, int n_groups, int M, int N, int Kp, float* out,
                        hipStream_t stream) {
  if (M % W2_T == 0 && N % W2_T == 0) {
    // one workgroup per CU (128 KB of LDS): slices so that every CU gets several
    const int tiles = (M / W2_T) * (N / W2_T);
    const int S = std::min(n_groups, std::max(1, (2048 + tiles - 1) / tiles));
    hipLaunchKernelGGL(wgrad256_kernel, dim3(tiles, S), dim3(W2_THREADS), 0, stream, A, sA, B, sB, offsets,
                       n_groups, M, N, Kp, out);
    return hipGetLastError();
  }
  const dim3 grid((M / 128) * (N / 128), n_groups);
  hipLaunchKernelGGL(wgrad_kernel, grid, dim3(256), 0, stream, A, sA, B, sB, offsets, n_groups, M, N, Kp, out);
  return hipGetLastError();
}

}  // namespace moe
