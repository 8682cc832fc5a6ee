// Router of the MoE layer: sigmoid affinity, selection-only bias, group-limited
// top-k and normalised gates (the "DeepSeek-V3" summary page, section 1
// "DeepSeekMoE" and "Node-limited routing", section 2; the book's chapter 7
// "The router's affinity scores", "Selecting and combining experts", and
// chapter 8 "V3's routing-only bias", "Restricting target nodes").
//
// One workgroup routes 64 tokens against all (<= 256) experts:
//   1. logits: BF16 MFMA 16x16x32 with FP32 accumulation over each 128-wide K
//      chunk, chunks summed in FP64 registers.  The token tile is staged in
//      LDS; each wave streams the centroid rows of its 64 experts straight from
//      global memory (they are shared by every workgroup and stay in L2/MALL).
//   2. selection, one token per wave at a time, in FP64: per-group sum of the
//      k/M largest biased scores, top-M groups and top-k experts by wavefront
//      argmax reductions (ties to the lower index), gates from the unbiased
//      affinity.  Gating is kept in higher precision because top-k has
//      discrete boundaries (book chapter 17 "Router precision has discrete
//      consequences").
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int RT_TOK = 64;
constexpr int RT_EXP = 256;
constexpr int RT_KC = 128;

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wavefront argmax over (value, index): larger value wins, equal values go to
// the smaller index.  Every lane returns the same pair.
__device__ __forceinline__ void wave_argmax(double& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double ov = __shfl_xor(v, o);
    const int oi = __shfl_xor(i, o);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
    }
  }
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int a_lds_off(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }

__global__ __launch_bounds__(256) void route_kernel(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ wg,
                                                    const float* __restrict__ bias, int T, int d,
                                                    int E, int G, int M, int k, double route_scale,
                                                    int32_t* __restrict__ idx,
                                                    float* __restrict__ wout) {
  __shared__ __attribute__((aligned(16))) unsigned char a_lds[RT_TOK * RT_KC * 2];
  __shared__ double logit[RT_TOK][RT_EXP + 1];
  __shared__ double zbuf[4][RT_EXP];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int t0 = blockIdx.x * RT_TOK;
  const int n_kc = d / RT_KC;

  // Token-tile loads: thread owns 4 16-byte chunks of the 64 x 256-byte tile.
  const uint16_t* a_src[4];
  int a_dst[4];
  bool a_ok[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int id = threadIdx.x + 256 * it;
    const int r = id >> 4, c = id & 15;
    a_ok[it] = (t0 + r) < T;
    a_src[it] = x + (size_t)(a_ok[it] ? t0 + r : 0) * d + c * 8;
    a_dst[it] = a_lds_off(r, c);
  }
  // Centroid rows of this wave's experts: lane reads 32 BF16 of row e per chunk.
  const uint16_t* b_src[4];
  bool b_ok[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int e = 64 * wave + 16 * nt + r16;
    b_ok[nt] = e < E;
    b_src[nt] = wg + (size_t)(b_ok[nt] ? e : 0) * d + g16 * 32;
  }

  double acc64[4][4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc64[mt][nt][i] = 0.0;

  uint4 a_next[4];
  uint4 b_next[4][4];
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int it = 0; it < 4; ++it)
    a_next[it] = a_ok[it] ? *reinterpret_cast<const uint4*>(a_src[it]) : zero4;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      b_next[nt][q] = b_ok[nt] ? *reinterpret_cast<const uint4*>(b_src[nt] + q * 8) : zero4;

  for (int kc = 0; kc < n_kc; ++kc) {
    __syncthreads();  // every wave is done reading the previous token tile
#pragma unroll
    for (int it = 0; it < 4; ++it) *reinterpret_cast<uint4*>(a_lds + a_dst[it]) = a_next[it];
    uint4 b_cur[4][4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) b_cur[nt][q] = b_next[nt][q];
    __syncthreads();
    if (kc + 1 < n_kc) {
      const size_t off = (size_t)(kc + 1) * RT_KC;
#pragma unroll
      for (int it = 0; it < 4; ++it)
        a_next[it] = a_ok[it] ? *reinterpret_cast<const uint4*>(a_src[it] + off) : zero4;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          b_next[nt][q] = b_ok[nt] ? *reinterpret_cast<const uint4*>(b_src[nt] + off + q * 8) : zero4;
    }
    v4f acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      v8bf af[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int r = mt * 16 + r16;
        af[mt] = *reinterpret_cast<const v8bf*>(a_lds + a_lds_off(r, g16 * 4 + kk));
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const v8bf bf = __builtin_bit_cast(v8bf, b_cur[nt][kk]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = mfma_bf16_16x16x32(af[mt], bf, acc[mt][nt]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc64[mt][nt][i] += (double)acc[mt][nt][i];
  }

#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        logit[mt * 16 + g16 * 4 + i][64 * wave + 16 * nt + r16] = acc64[mt][nt][i];
  __syncthreads();

  // ---- selection: wave `wave` routes tokens wave, wave+4, ... of the tile ----
  const int per = E / G;
  const int n_top = k / M;
  const double NEG_INF = -__builtin_huge_val();
  for (int tt = wave; tt < RT_TOK; tt += 4) {
    const int t = t0 + tt;
    if (t >= T) break;
    double zc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      zc[j] = NEG_INF;
      if (e < E) {
        const double s = 1.0 / (1.0 + exp(-logit[tt][e]));
        const double z = s + (bias ? (double)bias[e] : 0.0);
        zbuf[wave][e] = z;
        zc[j] = z;
      }
    }
    wave_sync_lds();
    // group scores: lane g sums the n_top largest biased scores of group g
    double gv = NEG_INF;
    if (lane < G) {
      double top[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) top[i] = NEG_INF;
      for (int e = lane * per; e < (lane + 1) * per; ++e) {
        double v = zbuf[wave][e];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (i < n_top && v > top[i]) {
            const double tmp = top[i];
            top[i] = v;
            v = tmp;
          }
        }
      }
      gv = 0.0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < n_top) gv += top[i];
    }
    wave_sync_lds();  // zbuf is rewritten by the next token
    uint64_t gmask = 0;
    for (int r = 0; r < M; ++r) {
      double v = gv;
      int i = lane;
      wave_argmax(v, i);
      gmask |= 1ull << i;
      if (lane == i) gv = NEG_INF;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e < E && !((gmask >> (e / per)) & 1ull)) zc[j] = NEG_INF;
    }
    int sel[16];
    bool taken[4] = {false, false, false, false};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sel[r] = 0x7fffffff;
      if (r < k) {
        double bv = NEG_INF;
        int be = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = lane + 64 * j;
          if (e < E && !taken[j] && zc[j] != NEG_INF && (zc[j] > bv || (zc[j] == bv && e < be))) {
            bv = zc[j];
            be = e;
          }
        }
        wave_argmax(bv, be);
        sel[r] = be;
        if (be < E && (be & 63) == lane) taken[be >> 6] = true;
      }
    }
    // lane j < k: expert sel[j], its rank among the selected ids, its gate
    int my_e = 0x7fffffff;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (r == lane) my_e = sel[r];
    int rank = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (r < k && sel[r] < my_e) ++rank;
    double s = 0.0;
    const bool mine = lane < k && my_e < E;
    if (mine) s = 1.0 / (1.0 + exp(-logit[tt][my_e]));
    const double ssum = wave_sum(s);
    if (mine) {
      idx[(size_t)t * k + rank] = my_e;
      wout[(size_t)t * k + rank] = (float)(route_scale * s / ssum);
    }
  }
}

hipError_t launch_route(const uint16_t* x, const uint16_t* wg, const float* bias, int T, int d,
                        int E, int G, int M, int k, float route_scale, int32_t* idx, float* w,
                        hipStream_t stream) {
  const int blocks = (T + RT_TOK - 1) / RT_TOK;
  hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(256), 0, stream, x, wg, bias, T, d, E, G, M,
                     k, (double)route_scale, idx, w);
  return hipGetLastError();
}

}  // namespace moe
