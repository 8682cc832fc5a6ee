// Router of the MoE layer: sigmoid affinity, selection-only bias, group-limited
// top-k and normalised gates (the "DeepSeek-V3" summary page, section 1
// "DeepSeekMoE" and "Node-limited routing", section 2; the book's chapter 7
// "The router's affinity scores", "Selecting and combining experts", and
// chapter 8 "V3's routing-only bias", "Restricting target nodes").
//
// One workgroup (8 waves) routes 64 tokens against all (<= 256) experts:
//   1. logits: BF16 MFMA 16x16x32, FP32 partial sums over each 128-wide chunk
//      of d, chunks summed in FP64 registers.  Token rows and centroid rows
//      stream through a three-stage LDS ring (64 elements of d per stage, so
//      every direct global->LDS load fetches whole 128-byte lines; the kernel
//      is bound by its request rate); wave w owns experts 32 w .. 32 w + 31.  The
//      FP64 logits are stored to LDS rounded to FP32 (relative 6e-8: the
//      biased scores move by < 1e-7, far inside the 1e-6 near-tie band).
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
constexpr int RT_THREADS = 512;
constexpr int RT_KS = 64;                              // d elements per ring stage
constexpr int RT_ROWB = RT_KS * 2;                     // 128-byte rows: whole cache lines
constexpr int RT_A = RT_TOK * RT_ROWB;                 // token rows of a stage, 8 KB
constexpr int RT_STG = (RT_TOK + RT_EXP) * RT_ROWB;    // 40 KB
constexpr int RT_NST = 3;                              // ring depth
constexpr int RT_LSTRIDE = RT_EXP + 1;                 // FP32 logit table row stride
constexpr int RT_MAXG = 64;

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS layout of a 128-byte row r: its 16-byte chunk c sits at c ^ op_swz(r),
// the operand layout of the expert GEMMs (a fragment read, 16 lanes on rows
// r0..r0+15 at one chunk, spreads over the banks).
__device__ __forceinline__ int rt_off(int r, int c) { return r * RT_ROWB + ((c ^ op_swz(r)) << 4); }

__device__ __forceinline__ v8bf rt_frag(const unsigned char* T, int r, int c) {
  return *reinterpret_cast<const v8bf*>(T + rt_off(r, c));
}

// s_waitcnt vmcnt(N) only (gfx9 encoding)
template <int N>
__device__ __forceinline__ void rt_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | (((N >> 4) & 3) << 14));
}

__device__ __forceinline__ float sigmoid32(float l) {
  return __builtin_amdgcn_rcpf(1.0f + expf(-l));
}

// Selection for 8 groups of 32 experts and k <= 8 (the V3 shape), with the
// results of the general code below: member m of a token's team owns group m
// and keeps its 32 biased scores in registers; the group score sums the n_top
// largest in descending order; the top-k are taken in k rounds of a per-member
// argmax (ties to the lower id) and a team argmax (larger score, then lower
// id), i.e. in the order of the general merge; member m then computes the gate
// of the m-th selected expert in FP64, the team sums them by the same
// shuffles.
__device__ __forceinline__ void route_select_g8(const float* L, const float* sbias, float (*gscore)[RT_TOK],
                                                int tt, int t, int T, int M, int k, int n_top,
                                                double route_scale, int32_t* __restrict__ idx,
                                                float* __restrict__ wout, int mem) {
  const float NEG = -__builtin_huge_valf();
  constexpr int NONE = 0x7fffffff;
  float z[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) z[i] = sigmoid32(L[mem * 32 + i]) + sbias[mem * 32 + i];
  {
    float top[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) top[i] = NEG;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      float v = z[e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i < n_top && v > top[i]) {
          const float tmp = top[i];
          top[i] = v;
          v = tmp;
        }
      }
    }
    float gs = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < n_top) gs += top[i];
    gscore[mem][tt] = gs;
  }
  wave_sync_lds();
  uint32_t gmask = 0;
  for (int r = 0; r < M; ++r) {
    float bv = NEG;
    int bg = -1;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const float v = gscore[g][tt];
      if (!((gmask >> g) & 1u) && (bg < 0 || v > bv)) {
        bv = v;
        bg = g;
      }
    }
    gmask |= 1u << bg;
  }
  const bool kept = (gmask >> mem) & 1u;
  uint32_t taken = 0;
  int sel[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    sel[r] = NONE;
    if (r < k) {
      float bv = NEG;
      int bi = NONE;
      if (kept) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          if (!((taken >> i) & 1u) && (bi == NONE || z[i] > bv)) {
            bv = z[i];
            bi = mem * 32 + i;
          }
        }
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        const bool take = (oi != NONE) && (bi == NONE || ov > bv || (ov == bv && oi < bi));
        if (take) {
          bv = ov;
          bi = oi;
        }
      }
      sel[r] = bi;
      if ((bi >> 5) == mem) taken |= 1u << (bi & 31);
    }
  }
  int mine = sel[0];
#pragma unroll
  for (int r = 1; r < 8; ++r)
    if (mem == r) mine = sel[r];
  double s_mine = 0.0;
  if (mem < k) s_mine = 1.0 / (1.0 + exp(-(double)L[mine]));
  double ssum = 0.0 + s_mine;
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) ssum += __shfl_xor(ssum, o);
  if (t < T && mem < k) {
    int rank = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k && sel[j] < mine) ++rank;
    idx[(size_t)t * k + rank] = mine;
    wout[(size_t)t * k + rank] = (float)(route_scale * s_mine / ssum);
  }
}

// Selection and gates of 64 tokens from their FP32 logit table in LDS
// (token-major, row stride RT_LSTRIDE): called by all 512 threads.
__device__ __forceinline__ void route_select_tile(const float* logit, const float* sbias,
                                                  float (*gscore)[RT_TOK], int t0, int T, int E, int G,
                                                  int M, int k, double route_scale,
                                                  int32_t* __restrict__ idx, float* __restrict__ wout,
                                                  int wave, int lane) {
  // ---- selection: a team of 8 lanes per token (wave w, lanes 8 j .. 8 j + 7
  // route token 8 w + j); member m handles the groups g = m mod 8 ----
  // Biased scores z = sigmoid(l) + b in FP32 (within ~1e-7 of the exact
  // value, far inside the 1e-6 near-tie band); the gates use the FP64
  // affinity of the selected experts.
  const int tt = wave * 8 + (lane >> 3);
  const int mem = lane & 7;
  const int t = t0 + tt;
  const float* L = logit + tt * RT_LSTRIDE;
  const int per = E / G;
  const int n_top = k / M;
  const float NEG = -__builtin_huge_valf();
  if (G == 8 && per == 32 && k <= 8) {   // uniform: the V3 shape
    route_select_g8(L, sbias, gscore, tt, t, T, M, k, n_top, route_scale, idx, wout, mem);
    return;
  }
  // 1. group scores: sum of the n_top (<= k <= 16) largest biased scores of each group
  for (int g = mem; g < G; g += 8) {
    float top[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) top[i] = NEG;
    for (int e = g * per; e < (g + 1) * per; ++e) {
      float v = sigmoid32(L[e]) + sbias[e];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i < n_top && v > top[i]) {
          const float tmp = top[i];
          top[i] = v;
          v = tmp;
        }
      }
    }
    float gs = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i < n_top) gs += top[i];
    gscore[g][tt] = gs;
  }
  wave_sync_lds();
  // 2. the M best groups (ties to the lower group index), on every member
  uint64_t gmask = 0;
  for (int r = 0; r < M; ++r) {
    float bv = NEG;
    int bg = -1;
    for (int g = 0; g < G; ++g) {
      const float v = gscore[g][tt];
      if (!((gmask >> g) & 1ull) && (bg < 0 || v > bv)) {
        bv = v;
        bg = g;
      }
    }
    gmask |= 1ull << bg;
  }
  // 3. each member: the k best experts of its kept groups, best first (ties
  // to the lower id: experts are visited in ascending order and only a
  // strictly larger score moves an entry down)
  float sv[16];
  int si[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    sv[i] = NEG;
    si[i] = 0x7fffffff;
  }
  for (int g = mem; g < G; g += 8) {
    if (!((gmask >> g) & 1ull)) continue;
    for (int e = g * per; e < (g + 1) * per; ++e) {
      float v = sigmoid32(L[e]) + sbias[e];
      int vi = e;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i < k && (si[i] == 0x7fffffff || v > sv[i])) {
          const float tv = sv[i];
          const int ti = si[i];
          sv[i] = v;
          si[i] = vi;
          v = tv;
          vi = ti;
        }
      }
    }
  }
  // 4. merge the 8 sorted lists: k rounds of a team argmax over the heads
  // (larger score, then lower id); the winner's list moves up by one
  int sel[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    sel[r] = 0x7fffffff;
    if (r < k) {
      float bv = sv[0];
      int bi = si[0];
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        const bool take = (oi != 0x7fffffff) && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi));
        if (take) {
          bv = ov;
          bi = oi;
        }
      }
      sel[r] = bi;
      if (si[0] == bi) {
#pragma unroll
        for (int i = 0; i < 15; ++i) {
          sv[i] = sv[i + 1];
          si[i] = si[i + 1];
        }
        sv[15] = NEG;
        si[15] = 0x7fffffff;
      }
    }
  }
  // 5. ascending ids with their gates w = route_scale * s / sum(s) in FP64;
  // member m computes the entries r = m, m + 8
  double s_part = 0.0;
  double s_mine[2] = {0.0, 0.0};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (r == mem + 8 * h && r < k) {
        s_mine[h] = 1.0 / (1.0 + exp(-(double)L[sel[r]]));
        s_part += s_mine[h];
      }
    }
  }
  double ssum = s_part;
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) ssum += __shfl_xor(ssum, o);
  if (t < T) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (r == mem + 8 * h && r < k) {
          int rank = 0;
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (j < k && sel[j] < sel[r]) ++rank;
          idx[(size_t)t * k + rank] = sel[r];
          wout[(size_t)t * k + rank] = (float)(route_scale * s_mine[h] / ssum);
        }
      }
    }
  }
}

__global__ __launch_bounds__(RT_THREADS) void route_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wg,
                                                           const float* __restrict__ bias, int T,
                                                           int d, int E, int G, int M, int k,
                                                           double route_scale,
                                                           int32_t* __restrict__ idx,
                                                           float* __restrict__ wout) {
  // ring of RT_NST stages; after the logits it holds the FP32 logit table
  __shared__ __attribute__((aligned(16))) unsigned char ring[RT_NST * RT_STG];
  __shared__ float gscore[RT_MAXG][RT_TOK];
  __shared__ float sbias[RT_EXP];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int t0 = blockIdx.x * RT_TOK;
  const int n_ks = d / RT_KS;
  if (threadIdx.x < RT_EXP) sbias[threadIdx.x] = (bias && (int)threadIdx.x < E) ? bias[threadIdx.x] : 0.0f;

  // ---- logits ----
  // Direct loads of whole 128-byte lines: an instruction writes 1 KB = 8 rows;
  // lane l fills row 8 i + l / 8, physical chunk l % 8 with the logical chunk
  // (l % 8) ^ op_swz(row).  Wave w loads expert rows 32 w .. 32 w + 31 (its own
  // experts, 4 loads) and token rows 8 w .. 8 w + 7 (1 load); rows past T or
  // E repeat the last valid row (their results are never used).
  const int pc = lane & 7;
  uint32_t a_off, b_off[4];
  {
    const int r = wave * 8 + (lane >> 3);
    const int t = min(t0 + r, T - 1);
    a_off = (uint32_t)t * (uint32_t)d * 2u + (uint32_t)((pc ^ op_swz(r)) * 16);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 32 + i * 8 + (lane >> 3);
    const int e = min(r, E - 1);
    b_off[i] = (uint32_t)e * (uint32_t)d * 2u + (uint32_t)((pc ^ op_swz(r)) * 16);
  }
  const uint32_t ring0 = lds_addr(ring);
#define RT_ISSUE(ks_)                                                                        \
  do {                                                                                       \
    const int ks__ = (ks_);                                                                  \
    const uint32_t base__ = ring0 + (ks__ % RT_NST) * RT_STG;                                \
    dma16(x + (size_t)ks__ * RT_KS, a_off, base__ + wave * 1024);                            \
    _Pragma("unroll") for (int i__ = 0; i__ < 4; ++i__)                                      \
      dma16(wg + (size_t)ks__ * RT_KS, b_off[i__], base__ + RT_A + (wave * 4 + i__) * 1024); \
  } while (0)

  double acc64[4][2][4];
  v4f acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) acc64[mt][nt][i] = 0.0;
    }

  // stages 0 .. RT_NST-2 in flight (d >= 128, so n_ks >= 2)
  for (int ks = 0; ks < RT_NST - 1 && ks < n_ks; ++ks) RT_ISSUE(ks);
  for (int ks = 0; ks < n_ks; ++ks) {
    // stage ks has landed once at most the younger stages (5 loads each) are
    // outstanding
    const int younger = min(RT_NST - 2, n_ks - 1 - ks);
    if (younger >= RT_NST - 2) {
      rt_wait_vmcnt<5 * (RT_NST - 2)>();
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the tail of the loop
    }
    asm volatile("s_barrier" ::: "memory");   // all waves' loads visible; stage ks-1 free
    if (ks + RT_NST - 1 < n_ks) RT_ISSUE(ks + RT_NST - 1);
    const unsigned char* A = ring + (ks % RT_NST) * RT_STG;
    const unsigned char* B = A + RT_A;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {   // two 32-wide halves of the stage's 64 elements of d
      v8bf af[4], bf[2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) af[mt] = rt_frag(A, mt * 16 + r16, kk * 4 + g16);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) bf[nt] = rt_frag(B, wave * 32 + nt * 16 + r16, kk * 4 + g16);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = mfma_bf16_16x16x32(af[mt], bf[nt], acc[mt][nt]);
    }
    if ((ks & 1) == 1) {   // a 128-wide chunk of d is complete: promote to FP64
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc64[mt][nt][i] += (double)acc[mt][nt][i];
          acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
        }
    }
  }
#undef RT_ISSUE
  __syncthreads();   // every wave is done with the ring

  // FP32 logit table [token][expert] over the ring
  float* logit = reinterpret_cast<float*>(ring);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        logit[(mt * 16 + g16 * 4 + i) * RT_LSTRIDE + wave * 32 + nt * 16 + r16] = (float)acc64[mt][nt][i];
  __syncthreads();

  route_select_tile(logit, sbias, gscore, t0, T, E, G, M, k, route_scale, idx, wout, wave, lane);
}

hipError_t launch_route(const uint16_t* x, const uint16_t* wg, const float* bias, int T, int d,
                        int E, int G, int M, int k, float route_scale, int32_t* idx, float* w,
                        hipStream_t stream) {
  const int blocks = (T + RT_TOK - 1) / RT_TOK;
  hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(RT_THREADS), 0, stream, x, wg, bias, T, d, E, G, M,
                     k, (double)route_scale, idx, w);
  return hipGetLastError();
}

// ---- two-kernel form for small batches (a workspace holds the logits) ----
// route_logits_kernel: workgroup (token block of TM, expert block of EN) computes
// those logits over all of d, so a batch of few tokens spreads the centroid
// stream over E / EN workgroups instead of one.  The arithmetic per logit is
// that of route_kernel: 16x16x32 BF16 MFMAs in d order, the FP32 partial of
// each 128-wide chunk added to an FP64 sum in chunk order, the sum rounded
// once to FP32; so both forms give the same logits.  Stages of 128 elements
// of d (256-byte rows, 16-byte chunk c of row r at c ^ (r & 15)).
constexpr int RL_KS = 128;                    // d elements per stage
constexpr int RL_ROWB = RL_KS * 2;            // 256-byte rows
constexpr int RL_NST = 4;                     // ring depth

__device__ __forceinline__ int rl_off(int r, int c) { return r * RL_ROWB + ((c ^ (r & 15)) << 4); }

template <int TM, int EN, int NW>
__global__ __launch_bounds__(NW * 64) void route_logits_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ wg, int T,
                                                                 int d, int E, float* __restrict__ logits) {
  constexpr int ROWS = TM + EN;
  constexpr int STG = ROWS * RL_ROWB;
  constexpr int NINSTR = ROWS / 4;            // 1 KB direct loads per stage: 4 rows each
  constexpr int NTE = EN / 16;                // expert tiles
  constexpr int TPW = (TM / 16) * NTE / NW;   // 16x16 tiles per wave
  static_assert(TPW >= 1 && (TM / 16) * NTE == TPW * NW, "tile split");
  __shared__ __attribute__((aligned(16))) unsigned char ring[RL_NST * STG];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int t0 = blockIdx.x * TM, e0 = blockIdx.y * EN;
  const int n_ks = d / RL_KS;
  // this lane's source rows: instruction i (of this wave) fills rows 4 j .. 4 j + 3
  // with j = wave + NW * i; lane l writes row 4 j + l / 16, physical chunk l % 16
  constexpr int IPW = (NINSTR + NW - 1) / NW;
  uint32_t src[IPW];
  const uint16_t* base[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int j = wave + NW * i;
    const int r = 4 * j + (lane >> 4);
    const int lc = (lane & 15) ^ (r & 15);
    if (r < TM) {
      base[i] = x;
      src[i] = (uint32_t)min(t0 + r, T - 1) * (uint32_t)d * 2u + lc * 16;
    } else {
      base[i] = wg;
      src[i] = (uint32_t)min(e0 + r - TM, E - 1) * (uint32_t)d * 2u + lc * 16;
    }
  }
  const uint32_t ring0 = lds_addr(ring);
  auto issue = [&](int ks) {
    const uint32_t st = ring0 + (ks % RL_NST) * STG;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int j = wave + NW * i;
      if (j < NINSTR) dma16(base[i] + (size_t)ks * RL_KS, src[i], st + j * 1024);
    }
  };
  v4f acc[TPW];
  double acc64[TPW][4];
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc64[q][i] = 0.0;
  }
  for (int ks = 0; ks < RL_NST - 1 && ks < n_ks; ++ks) issue(ks);
  for (int ks = 0; ks < n_ks; ++ks) {
    // stage ks has landed once this wave's loads of it are done (the younger
    // stages may stay in flight); the barrier makes every wave's visible
    const int younger = min(RL_NST - 2, n_ks - 1 - ks);
    if (younger == RL_NST - 2) {
      constexpr int OUT = (RL_NST - 2) * IPW;   // upper bound of this wave's younger loads
      rt_wait_vmcnt<OUT>();
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    }
    asm volatile("s_barrier" ::: "memory");
    if (ks + RL_NST - 1 < n_ks) issue(ks + RL_NST - 1);
    const unsigned char* S = ring + (ks % RL_NST) * STG;
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      const int id = wave * TPW + q;
      const int mt = id / NTE, nt = id - (id / NTE) * NTE;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const v8bf af = *reinterpret_cast<const v8bf*>(S + rl_off(mt * 16 + r16, kk * 4 + g16));
        const v8bf bf = *reinterpret_cast<const v8bf*>(S + rl_off(TM + nt * 16 + r16, kk * 4 + g16));
        acc[q] = mfma_bf16_16x16x32(af, bf, acc[q]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) acc64[q][i] += (double)acc[q][i];
      acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int id = wave * TPW + q;
    const int mt = id / NTE, nt = id - (id / NTE) * NTE;
    const int e = e0 + nt * 16 + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + mt * 16 + g16 * 4 + i;
      if (t < T && e < E) logits[(size_t)t * E + e] = (float)acc64[q][i];
    }
  }
}

// Selection of 64 tokens from the logits of route_logits_kernel.
__global__ __launch_bounds__(RT_THREADS) void route_select_kernel(const float* __restrict__ logits,
                                                                  const float* __restrict__ bias, int T,
                                                                  int E, int G, int M, int k,
                                                                  double route_scale,
                                                                  int32_t* __restrict__ idx,
                                                                  float* __restrict__ wout) {
  __shared__ float logit[RT_TOK * RT_LSTRIDE];
  __shared__ float gscore[RT_MAXG][RT_TOK];
  __shared__ float sbias[RT_EXP];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * RT_TOK;
  if (threadIdx.x < RT_EXP) sbias[threadIdx.x] = (bias && (int)threadIdx.x < E) ? bias[threadIdx.x] : 0.0f;
  // all of a thread's loads in flight at once (the table was just written by
  // workgroups on other XCDs: every load is a far miss)
  constexpr int PER = RT_TOK * RT_EXP / RT_THREADS;
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x + j * RT_THREADS;
    const int r = i / E, e = i - r * E;
    v[j] = i < RT_TOK * E ? logits[(size_t)min(t0 + r, T - 1) * E + e] : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x + j * RT_THREADS;
    const int r = i / E, e = i - r * E;
    if (i < RT_TOK * E) logit[r * RT_LSTRIDE + e] = v[j];
  }
  __syncthreads();
  route_select_tile(logit, sbias, gscore, t0, T, E, G, M, k, route_scale, idx, wout, wave, lane);
}

// Token counts up to which the two-kernel form is used, and its tile shapes.
constexpr int RS_SMALL_T = 1024;   // 16 tokens x 32 experts per workgroup
constexpr int RS_MAX_T = 8192;     // 64 tokens x 64 experts per workgroup

size_t route_workspace_bytes(int T, int E) {
  if (T <= 0 || T > RS_MAX_T) return 0;
  return ((size_t)T * (size_t)E * 4 + 255) & ~(size_t)255;
}

hipError_t launch_route_ws(const uint16_t* x, const uint16_t* wg, const float* bias, int T, int d, int E,
                           int G, int M, int k, float route_scale, int32_t* idx, float* w, float* logits,
                           hipStream_t stream) {
  if (T > RS_MAX_T || logits == nullptr)
    return launch_route(x, wg, bias, T, d, E, G, M, k, route_scale, idx, w, stream);
  if (T <= RS_SMALL_T)
    hipLaunchKernelGGL((route_logits_kernel<16, 32, 2>), dim3((T + 15) / 16, (E + 31) / 32), dim3(128), 0,
                       stream, x, wg, T, d, E, logits);
  else
    hipLaunchKernelGGL((route_logits_kernel<64, 64, 8>), dim3((T + 63) / 64, (E + 63) / 64), dim3(512), 0,
                       stream, x, wg, T, d, E, logits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_select_kernel, dim3((T + RT_TOK - 1) / RT_TOK), dim3(RT_THREADS), 0, stream, logits,
                     bias, T, E, G, M, k, (double)route_scale, idx, w);
  return hipGetLastError();
}

}  // namespace moe
