// Backward of the MoE layer around the expert GEMMs (the "DeepSeek-V3" summary
// page, section 6 "FP8 mixed-precision training": Fprop, Dgrad and Wgrad all in
// FP8; the book's chapter 17 "One linear layer creates three GEMMs", "SwiGLU
// recomputation", and the regrouping of 1x128 tiles into 128x1 tiles with
// power-of-two scales; chapter 16 "Why transposition is not trivial").
//
//   transpose_blocks_kernel   FP8 weights [N, K] -> [K, N] with their 128x128
//                             block scales (once, offline): Dgrad multiplies
//                             by W rather than W^T
//   combine_backward_kernel   dY rows of the experts and the gate gradients
//   regroup_128x1_kernel      a per-expert 128x1 (along rows), power-of-two,
//                             transposed FP8 copy of an operand of Wgrad
//   swiglu_backward_kernel    SiLU(g)*u recomputed from the forward's FP8 cache
//                             of [G, U]; dG, dU; their 1x128 FP8 copy for Dgrad
//                             and the transposed 128x1 copies of [dG, dU] and H
//                             for Wgrad
//
// Transposed operands of Wgrad ("K-major" layout): row c holds column c of the
// original for all rows of all experts, expert e occupying the 128-aligned
// column range [128 pb[e], 128 pb[e+1]) with pb[e] = sum over earlier experts of
// ceil(rows / 128); padding columns are zero codes.  Their scales are
// [Kp/128, C]: one per column and 128-row block.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int BW_MAX_GROUPS = 1024;

// E4M3 code -> FP32 (exact; the code is OCP E4M3FN as written by the quantisers).
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// pb[e] = sum over groups e' < e of ceil(rows(e') / 128), pb[n_groups] = total.
// One wave computes it into LDS; the caller synchronises.
__device__ __forceinline__ void padded_block_prefix(const int32_t* __restrict__ offsets, int n_groups,
                                                    int* pb, int lane) {
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

// Group holding padded block blk (pb non-decreasing; empty groups are skipped).
__device__ __forceinline__ int block_group(const int* pb, int n_groups, int blk) {
  int a = 0, b = n_groups - 1;
  while (a < b) {
    const int mid = (a + b + 1) >> 1;
    if (pb[mid] <= blk) a = mid; else b = mid - 1;
  }
  return a;
}

// ---- weights: [G][N][K] -> [G][K][N], scales [G][N/128][K/128] -> [G][K/128][N/128]
__global__ __launch_bounds__(256) void transpose_blocks_kernel(const uint8_t* __restrict__ w,
                                                               const float* __restrict__ ws, int N,
                                                               int K, uint8_t* __restrict__ wt,
                                                               float* __restrict__ wts) {
  __shared__ uint8_t tile[128][129];
  const int kb = blockIdx.x, nb = blockIdx.y, g = blockIdx.z, t = threadIdx.x;
  const size_t src0 = (size_t)g * N * K + (size_t)nb * 128 * K + (size_t)kb * 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int chunk = t + 256 * i, r = chunk >> 3, c16 = chunk & 7;
    const uint4 v = *reinterpret_cast<const uint4*>(w + src0 + (size_t)r * K + c16 * 16);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 16; ++j) tile[r][c16 * 16 + j] = (uint8_t)(u[j >> 2] >> (8 * (j & 3)));
  }
  __syncthreads();
  const size_t dst0 = (size_t)g * N * K + (size_t)kb * 128 * N + (size_t)nb * 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int chunk = t + 256 * i, rr = chunk >> 3, c16 = chunk & 7;
    uint32_t u[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 16; ++j) u[j >> 2] |= (uint32_t)tile[c16 * 16 + j][rr] << (8 * (j & 3));
    *reinterpret_cast<uint4*>(wt + dst0 + (size_t)rr * N + c16 * 16) = make_uint4(u[0], u[1], u[2], u[3]);
  }
  if (t == 0)
    wts[((size_t)g * (K / 128) + kb) * (N / 128) + nb] = ws[((size_t)g * (N / 128) + nb) * (K / 128) + kb];
}

// ---- combine backward: one workgroup per token ----
// dy[pos[t][j]] = BF16(w[t][j] * dout[t]); dy[shared_row0 + t] = dout[t];
// dw[t][j] = sum_c dout[t][c] * y[pos[t][j]][c] in FP32.
// Q: also the 1x128 power-of-two FP8 copy of every dY row written (dyq, dys),
// the same arithmetic as fp8_quant_1x128_pow2 on dy: the 16 threads of a 1x128
// tile hold 8 consecutive elements each (256 threads cover 16 whole tiles).
__device__ __forceinline__ void quant_chunk_pow2(const uint32_t (&o)[4], uint8_t* __restrict__ q, float* sq,
                                                 bool first) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(static_cast<uint16_t>(o[i] & 0xFFFFu));
    v[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(o[i] >> 16));
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o2 = 8; o2 > 0; o2 >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o2));
  const float sc = tile_scale<true>(amax);
  uint2 out;
  out.x = f32x4_to_e4m3(v[0] / sc, v[1] / sc, v[2] / sc, v[3] / sc);
  out.y = f32x4_to_e4m3(v[4] / sc, v[5] / sc, v[6] / sc, v[7] / sc);
  *reinterpret_cast<uint2*>(q) = out;
  if (first) *sq = sc;
}

template <bool Q>
__global__ __launch_bounds__(256) void combine_backward_kernel(
    const uint16_t* __restrict__ dout, const uint16_t* __restrict__ y, const int32_t* __restrict__ pos,
    const float* __restrict__ w, int k, int d, int rows, int shared_row0, uint16_t* __restrict__ dy,
    float* __restrict__ dw, uint8_t* __restrict__ dyq, float* __restrict__ dys) {
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t* go = dout + (size_t)t * d;
  const int n8 = d / 8;
  for (int j = 0; j < k; ++j) {
    const int row = pos[t * k + j];
    const float wt = w[t * k + j];
    // a slot outside the rows (an unassigned one, pos < 0) has no expert
    // output: its gate gradient is 0 and no dY row is written (uniform branch)
    if (row < 0 || row >= rows) {
      if (tid == 0) dw[t * k + j] = 0.0f;
      continue;
    }
    float part = 0.0f;
    for (int c = tid; c < n8; c += 256) {
      const uint4 a = *reinterpret_cast<const uint4*>(go + c * 8);
      const uint4 b = *reinterpret_cast<const uint4*>(y + (size_t)row * d + c * 8);
      const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a0 = bf16_to_f32((uint16_t)(av[i] & 0xFFFFu)), a1 = bf16_to_f32((uint16_t)(av[i] >> 16));
        const float b0 = bf16_to_f32((uint16_t)(bv[i] & 0xFFFFu)), b1 = bf16_to_f32((uint16_t)(bv[i] >> 16));
        part = fmaf(a0, b0, part);
        part = fmaf(a1, b1, part);
        o[i] = (uint32_t)f32_to_bf16(wt * a0) | ((uint32_t)f32_to_bf16(wt * a1) << 16);
      }
      *reinterpret_cast<uint4*>(dy + (size_t)row * d + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
      if (Q) quant_chunk_pow2(o, dyq + (size_t)row * d + c * 8, dys + (size_t)row * (d / 128) + (c >> 4),
                              (c & 15) == 0);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if (lane == 0) red[wave] = part;
    __syncthreads();
    if (tid == 0) dw[t * k + j] = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
  }
  if (shared_row0 >= 0)
    for (int c = tid; c < n8; c += 256) {
      const uint4 v = *reinterpret_cast<const uint4*>(go + c * 8);
      const size_t row = (size_t)(shared_row0 + t);
      *reinterpret_cast<uint4*>(dy + row * d + c * 8) = v;
      if (Q) {
        const uint32_t o[4] = {v.x, v.y, v.z, v.w};
        quant_chunk_pow2(o, dyq + row * d + c * 8, dys + row * (d / 128) + (c >> 4), (c & 15) == 0);
      }
    }
}

// ---- 128x1 regrouping into the K-major layout ----
// Workgroup (cb, blk): columns [128 cb, 128 cb + 128) of padded block blk.
// FP8IN: the source is a 1x128 FP8 tensor (codes + scales) whose row r of the
// grouped order is row row_src[r] (or r when row_src is null); otherwise a BF16
// tensor in grouped order.  The tile is kept in LDS in its input form (FP8
// codes with their row scales, or BF16), 19 or 35 KB, so several workgroups
// share a CU; each column thread rebuilds its 64 FP32 values exactly (code x
// scale in FP32, or the BF16 value), takes the column's 128-row amax, a
// power-of-two scale, and codes E4M3(x / scale), staged in LDS (over the tile)
// for whole 128-byte output rows.
template <bool FP8IN>
__global__ __launch_bounds__(256) void regroup_128x1_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs, const uint16_t* __restrict__ xb,
    const int32_t* __restrict__ row_src, const int32_t* __restrict__ offsets, int n_groups, int C,
    int Kp, uint8_t* __restrict__ out, float* __restrict__ out_s) {
  constexpr int ROWB = FP8IN ? 144 : 272;   // padded row bytes of the input tile
  __shared__ int pb[BW_MAX_GROUPS + 1];
  __shared__ __attribute__((aligned(16))) uint8_t tile[128 * ROWB];   // input tile, then [column][row] codes
  __shared__ float rscale[FP8IN ? 128 : 1];
  __shared__ float colmax[2][128];
  const int tid = threadIdx.x, cb = blockIdx.x, blk = blockIdx.y;
  if (tid < 64) padded_block_prefix(offsets, n_groups, pb, tid);
  __syncthreads();
  if (blk >= pb[n_groups]) return;   // uniform
  const int e = block_group(pb, n_groups, blk);
  const int row0 = offsets[e] + (blk - pb[e]) * 128;
  const int nrows = min(128, offsets[e + 1] - row0);
  {
    const int r = tid >> 1, half = tid & 1;
    if (FP8IN) {
      uint4 q[4];
      float sc = 0.0f;
      if (r < nrows) {
        const int src = row_src ? row_src[row0 + r] : row0 + r;
        sc = xs[(size_t)src * (C / 128) + cb];
        const uint8_t* p = xq + (size_t)src * C + cb * 128 + half * 64;
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = *reinterpret_cast<const uint4*>(p + i * 16);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = make_uint4(0u, 0u, 0u, 0u);   // zero rows pad the block
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&tile[r * ROWB + half * 64 + i * 16]) = q[i];
      if (half == 0) rscale[r] = sc;
    } else {
      uint4 q[8];
      if (r < nrows) {
        const uint16_t* p = xb + (size_t)(row0 + r) * C + cb * 128 + half * 64;
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = *reinterpret_cast<const uint4*>(p + i * 8);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(&tile[r * ROWB + half * 128 + i * 16]) = q[i];
    }
  }
  __syncthreads();
  // column phase: thread (c, part) holds rows [64 part, 64 part + 64) of column c
  const int c = tid & 127, part = tid >> 7;
  float w[64];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    const int rr = part * 64 + i;
    if (FP8IN)
      w[i] = e4m3_to_f32(tile[rr * ROWB + c]) * rscale[rr];
    else
      w[i] = bf16_to_f32(*reinterpret_cast<const uint16_t*>(&tile[rr * ROWB + 2 * c]));
    amax = fmaxf(amax, fabsf(w[i]));
  }
  colmax[part][c] = amax;
  __syncthreads();   // every read of the tile is done: its memory now holds the codes
  const float s = scale_from_amax_pow2(fmaxf(colmax[0][c], colmax[1][c]));
  const float inv = 1.0f / s;   // exact: s is a power of two
  uint32_t pk[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    pk[j] = f32x4_to_e4m3(w[4 * j] * inv, w[4 * j + 1] * inv, w[4 * j + 2] * inv, w[4 * j + 3] * inv);
  if (part == 0) out_s[(size_t)blk * C + cb * 128 + c] = s;
  uint8_t(*tq)[144] = reinterpret_cast<uint8_t(*)[144]>(&tile[0]);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint4*>(&tq[c][part * 64 + i * 16]) = make_uint4(pk[4 * i], pk[4 * i + 1], pk[4 * i + 2], pk[4 * i + 3]);
  __syncthreads();
  // full 128-byte output rows: 8 lanes per row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int cc = (tid >> 3) + 32 * i, ch = tid & 7;
    *reinterpret_cast<uint4*>(out + (size_t)(cb * 128 + cc) * Kp + (size_t)blk * 128 + ch * 16) =
        *reinterpret_cast<const uint4*>(&tq[cc][ch * 16]);
  }
}

// ---- SwiGLU backward ----
// Workgroup (cb, blk): h-columns [128 cb, 128 cb + 128) of padded block blk.
// From the cache, g and u are the codes times their 1x128 scales (FP32);
// s = sigmoid(g), h = g s u, dG = dH u s (1 + g (1 - s)), dU = dH g s are
// evaluated in FP64 and rounded once to FP32.  Outputs: [dG, dU] with 1x128
// power-of-two scales in row order (the Dgrad operand), and the K-major 128x1
// copies of [dG, dU] ([2f, Kp]) and of h ([f, Kp]) (the Wgrad operands).
struct SwigluVals {
  float h, dg, du;
};

__device__ __forceinline__ SwigluVals swiglu_bwd_vals(float g, float u, float dh) {
  const double gd = g, ud = u, dhd = dh;
  const double s = 1.0 / (1.0 + exp(-gd));
  SwigluVals r;
  r.h = (float)(gd * s * ud);
  r.dg = (float)(dhd * ud * s * (1.0 + gd * (1.0 - s)));
  r.du = (float)(dhd * gd * s);
  return r;
}

// Four threads (4r .. 4r+3, one wave) own row r of the tile, 32 columns each:
// h, dG, dU are evaluated once (FP64) and kept in registers; a row's amax is
// in-thread plus two shuffles; a column's amax goes through an LDS table, one
// quantity at a time; the transposed codes are staged in LDS.  Division by a
// power-of-two scale is a multiplication by its exact inverse.
constexpr int SWB_THREADS = 512;

__global__ __launch_bounds__(SWB_THREADS) void swiglu_backward_kernel(
    const uint8_t* __restrict__ guq, const float* __restrict__ gus, const uint16_t* __restrict__ dh,
    const int32_t* __restrict__ offsets, int n_groups, int f, int Kp, uint8_t* __restrict__ dguq,
    float* __restrict__ dgus, uint8_t* __restrict__ dgut, float* __restrict__ dguts,
    uint8_t* __restrict__ ht, float* __restrict__ hts) {
  __shared__ int pb[BW_MAX_GROUPS + 1];
  __shared__ __attribute__((aligned(16))) float red[128][129];   // values, then [column][row] codes
  __shared__ float part_max[4][128];
  const int tid = threadIdx.x, cb = blockIdx.x, blk = blockIdx.y;
  if (tid < 64) padded_block_prefix(offsets, n_groups, pb, tid);
  __syncthreads();
  if (blk >= pb[n_groups]) return;   // uniform
  const int e = block_group(pb, n_groups, blk);
  const int row0 = offsets[e] + (blk - pb[e]) * 128;
  const int nrows = min(128, offsets[e + 1] - row0);
  const int nsc = 2 * f / 128;
  const int r = tid >> 2, qt = tid & 3, col0 = qt * 32;
  const bool valid = r < nrows;
  const size_t rowi = (size_t)(row0 + r);
  float vh[32], vg[32], vu[32];
  {
    uint32_t gw[8], uw[8], dw[16];
    if (valid) {
      const uint8_t* pg = guq + rowi * 2 * f + cb * 128 + col0;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint4 a = *reinterpret_cast<const uint4*>(pg + i * 16);
        const uint4 b = *reinterpret_cast<const uint4*>(pg + f + i * 16);
        gw[4 * i] = a.x; gw[4 * i + 1] = a.y; gw[4 * i + 2] = a.z; gw[4 * i + 3] = a.w;
        uw[4 * i] = b.x; uw[4 * i + 1] = b.y; uw[4 * i + 2] = b.z; uw[4 * i + 3] = b.w;
      }
      const uint16_t* pd = dh + rowi * f + cb * 128 + col0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 q = *reinterpret_cast<const uint4*>(pd + i * 8);
        dw[4 * i] = q.x; dw[4 * i + 1] = q.y; dw[4 * i + 2] = q.z; dw[4 * i + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) gw[i] = uw[i] = 0u;
#pragma unroll
      for (int i = 0; i < 16; ++i) dw[i] = 0u;
    }
    const float gs = valid ? gus[rowi * nsc + cb] : 0.0f;
    const float us = valid ? gus[rowi * nsc + f / 128 + cb] : 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float g = e4m3_to_f32((gw[i >> 2] >> (8 * (i & 3))) & 0xFFu) * gs;
      const float u = e4m3_to_f32((uw[i >> 2] >> (8 * (i & 3))) & 0xFFu) * us;
      const float d = bf16_to_f32((uint16_t)(dw[i >> 1] >> (16 * (i & 1))));
      const SwigluVals v = swiglu_bwd_vals(g, u, d);
      vh[i] = v.h;
      vg[i] = v.dg;
      vu[i] = v.du;
      // materialise the three FP32 results here, so that no FP64 temporaries
      // are carried into the quantisation passes
      asm volatile("" : "+v"(vh[i]), "+v"(vg[i]), "+v"(vu[i]));
    }
  }
  // ---- [dG, dU] in row order: 1x128 tiles, power-of-two scales ----
  {
    float mg = 0.0f, mu = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      mg = fmaxf(mg, fabsf(vg[i]));
      mu = fmaxf(mu, fabsf(vu[i]));
    }
    mg = fmaxf(mg, __shfl_xor(mg, 1));
    mu = fmaxf(mu, __shfl_xor(mu, 1));
    mg = fmaxf(mg, __shfl_xor(mg, 2));
    mu = fmaxf(mu, __shfl_xor(mu, 2));
    const float sg = scale_from_amax_pow2(mg), su = scale_from_amax_pow2(mu);
    const float ig = 1.0f / sg, iu = 1.0f / su;
    if (valid) {
      uint8_t* og = dguq + rowi * 2 * f + cb * 128 + col0;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint32_t a[4], b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = 16 * i + 4 * j;
          a[j] = f32x4_to_e4m3(vg[c] * ig, vg[c + 1] * ig, vg[c + 2] * ig, vg[c + 3] * ig);
          b[j] = f32x4_to_e4m3(vu[c] * iu, vu[c + 1] * iu, vu[c + 2] * iu, vu[c + 3] * iu);
        }
        *reinterpret_cast<uint4*>(og + i * 16) = make_uint4(a[0], a[1], a[2], a[3]);
        *reinterpret_cast<uint4*>(og + f + i * 16) = make_uint4(b[0], b[1], b[2], b[3]);
      }
      if (qt == 0) {
        dgus[rowi * nsc + cb] = sg;
        dgus[rowi * nsc + f / 128 + cb] = su;
      }
    }
  }
  // ---- K-major 128x1 copies: h -> ht, dG -> dgut rows [0, f), dU -> dgut rows [f, 2f) ----
  uint8_t(*tq)[144] = reinterpret_cast<uint8_t(*)[144]>(&red[0][0]);   // aliases red
  auto pass = [&](const float(&v)[32], int q) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 32; ++i) red[r][col0 + i] = v[i];
    __syncthreads();
    // column phase: thread (c, rq) holds rows [32 rq, 32 rq + 32) of column c
    const int c = tid & 127, rq = tid >> 7;
    float w[32];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      w[j] = red[rq * 32 + j][c];
      m = fmaxf(m, fabsf(w[j]));
    }
    part_max[rq][c] = m;
    __syncthreads();   // every read of red is done: its memory now holds the codes
    m = fmaxf(fmaxf(part_max[0][c], part_max[1][c]), fmaxf(part_max[2][c], part_max[3][c]));
    const float sc = scale_from_amax_pow2(m);
    const float inv = 1.0f / sc;   // exact: sc is a power of two
    if (rq == 0) {
      if (q == 0) hts[(size_t)blk * f + cb * 128 + c] = sc;
      else dguts[(size_t)blk * 2 * f + (q - 1) * f + cb * 128 + c] = sc;
    }
    uint32_t pk[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      pk[j] = f32x4_to_e4m3(w[4 * j] * inv, w[4 * j + 1] * inv, w[4 * j + 2] * inv, w[4 * j + 3] * inv);
    *reinterpret_cast<uint4*>(&tq[c][rq * 32]) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    *reinterpret_cast<uint4*>(&tq[c][rq * 32 + 16]) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
    __syncthreads();
    // full 128-byte output rows: 8 lanes per row
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int cc = (tid >> 3) + 64 * i, ch = tid & 7;
      uint8_t* dst = q == 0 ? ht + (size_t)(cb * 128 + cc) * Kp
                            : dgut + (size_t)((q - 1) * f + cb * 128 + cc) * Kp;
      *reinterpret_cast<uint4*>(dst + (size_t)blk * 128 + ch * 16) = *reinterpret_cast<const uint4*>(&tq[cc][ch * 16]);
    }
    __syncthreads();   // before the next pass overwrites red
  };
  pass(vh, 0);
  pass(vg, 1);
  pass(vu, 2);
}

hipError_t launch_transpose_blocks(const uint8_t* w, const float* ws, int G, int N, int K, uint8_t* wt,
                                   float* wts, hipStream_t stream) {
  hipLaunchKernelGGL(transpose_blocks_kernel, dim3(K / 128, N / 128, G), dim3(256), 0, stream, w, ws, N, K,
                     wt, wts);
  return hipGetLastError();
}

hipError_t launch_combine_backward(const uint16_t* dout, const uint16_t* y, const int32_t* pos,
                                   const float* w, int T, int k, int d, int shared_row0, uint16_t* dy,
                                   float* dw, uint8_t* dyq, float* dys, hipStream_t stream) {
  // rows of y / dy (the same bound as the forward combine's)
  const int rlim = shared_row0 >= 0 ? shared_row0 + T : T * k;
  if (dyq)
    hipLaunchKernelGGL(combine_backward_kernel<true>, dim3(T), dim3(256), 0, stream, dout, y, pos, w, k, d,
                       rlim, shared_row0, dy, dw, dyq, dys);
  else
    hipLaunchKernelGGL(combine_backward_kernel<false>, dim3(T), dim3(256), 0, stream, dout, y, pos, w, k, d,
                       rlim, shared_row0, dy, dw, nullptr, nullptr);
  return hipGetLastError();
}

int wgrad_blocks_bound(int total_rows, int n_groups) { return total_rows / 128 + n_groups; }

hipError_t launch_regroup_128x1(const uint8_t* xq, const float* xs, const uint16_t* xb,
                                const int32_t* row_src, const int32_t* offsets, int n_groups,
                                int total_rows, int C, int Kp, uint8_t* out, float* out_s,
                                hipStream_t stream) {
  const dim3 grid(C / 128, wgrad_blocks_bound(total_rows, n_groups));
  if (xq)
    hipLaunchKernelGGL(regroup_128x1_kernel<true>, grid, dim3(256), 0, stream, xq, xs, xb, row_src, offsets,
                       n_groups, C, Kp, out, out_s);
  else
    hipLaunchKernelGGL(regroup_128x1_kernel<false>, grid, dim3(256), 0, stream, xq, xs, xb, row_src, offsets,
                       n_groups, C, Kp, out, out_s);
  return hipGetLastError();
}

hipError_t launch_swiglu_backward(const uint8_t* guq, const float* gus, const uint16_t* dh,
                                  const int32_t* offsets, int n_groups, int total_rows, int f, int Kp,
                                  uint8_t* dguq, float* dgus, uint8_t* dgut, float* dguts, uint8_t* ht,
                                  float* hts, hipStream_t stream) {
  const dim3 grid(f / 128, wgrad_blocks_bound(total_rows, n_groups));
  hipLaunchKernelGGL(swiglu_backward_kernel, grid, dim3(SWB_THREADS), 0, stream, guq, gus, dh, offsets, n_groups, f,
                     Kp, dguq, dgus, dgut, dguts, ht, hts);
  return hipGetLastError();
}

}  // namespace moe
