// Backward pass for every size the forward accepts that the MFMA backward
// kernels (chunk_bwd.hip and the adjoint modes of the grouped kernels) do not
// cover: float32, and bfloat16 with a head size other than 64 or a state size
// other than 64, 128 or 256 (512 included).  The pages publish no backward
// pass (disconfirmai.com "Jane Street ML Engineers Map Mamba-2 Recurrent State
// Computation to Tensor Cores with cuTile", lead paragraph: training needs
// one); the formulas are the vector-Jacobian product of the chunked forward
// (devotd.net news item on the Mamba-2 CUDA Tile forward-pass kernels,
// section 2), per (batch, chunk c, head), with M[i, j] = 2^(cs_i - cs_j) for
// j <= i (cs in log2 units, cl = cs of the chunk's last step), CB = C B^T of
// the group, h the chunk-start state and g the gradient reaching the
// chunk-end state:
//     E_c   = sum_i 2^cs_i dy_i (outer) C_i,  r_c = 2^cl r_{c+1} + E_c,
//             r_nc = dfinal, g_c = r_{c+1}, dinit = r_0
//     dU_j  = sum_{i>=j} M_ij CB_ij dy_i + 2^(cl - cs_j) g B_j
//     dx_j  = dt_j dU_j + D dy_j
//     W_ij  = dt_j (dy_i . x_j)
//     dC_i += sum_{j<=i} M_ij W_ij B_j + 2^cs_i dy_i h
//     dB_j += sum_{i>=j} M_ij W_ij C_i + 2^(cl - cs_j) dt_j x_j g
//     dq_k  = sum_{i>=k>j} M_ij CB_ij W_ij + sum_{i>=k} 2^cs_i dy_i . (h C_i)
//             + sum_{j<k} 2^(cl - cs_j) dt_j x_j . (g B_j) + 2^cl <g, h>
//     ddt_k = x_k . dU_k + A dq_k,  dA = sum_k dt_k dq_k,  dD = sum dy . x
// (dq_k is the gradient of the step's log decay A dt_k; dB and dC sum the
// heads of each group).  The rectangle sum over i >= k > j is formed as
// sum_{m<k} (colsum_m - rowsum_m) of the strictly lower triangle, in float64.
//
// Every contraction runs on the vector ALU in float32 as 64 x 64 output tiles
// of 256 threads (4 x 4 outputs each) with operands staged through LDS in
// steps of 16; inputs are read as bfloat16 or float32 and the gradients of
// x, dt, B and C are written in the input dtype.  Positions past L are zero
// input (dt = 0, x = 0), as in the forward.
#include "common.h"
#include "launch.h"

namespace m2 {

namespace {

constexpr int kT = 64;        // output tile
constexpr int kKB = 16;       // reduction step staged per pass
constexpr int kLS = kT + 4;   // LDS row stride of a staged operand (floats)

struct Stage {
  float a[kKB][kLS];
  float b[kKB][kLS];
};

__device__ __forceinline__ float ld(const bf16* p) { return bf2f(*p); }
__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ void st(bf16* p, float v) { *p = f2bf(v); }
__device__ __forceinline__ void st(float* p, float v) { *p = v; }

// acc[a][b] += sum_{k in [k0, k1)} la(4 tr + a, k) * lb(4 tc + b, k), with
// tr = thread / 16, tc = thread % 16 (row and column inside the 64 x 64
// tile).  la(r, k), lb(r, k) return operand elements (0 outside the data);
// KA / KB: whether consecutive threads stage consecutive k (the operand is
// contiguous along k) or consecutive rows.  Every thread of the block calls
// this with the same arguments.
template <bool KA, bool KB, class LA, class LB>
__device__ __forceinline__ void mm(float (&acc)[4][4], int k0, int k1, LA la, LB lb, Stage& s) {
  const int t = threadIdx.x, tr = t >> 4, tc = t & 15;
  for (int kb = k0; kb < k1; kb += kKB) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = t + 256 * e;
      {
        const int r = KA ? idx >> 4 : idx & 63, k = KA ? idx & 15 : idx >> 6;
        s.a[k][r] = kb + k < k1 ? la(r, kb + k) : 0.f;
      }
      {
        const int r = KB ? idx >> 4 : idx & 63, k = KB ? idx & 15 : idx >> 6;
        s.b[k][r] = kb + k < k1 ? lb(r, kb + k) : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kKB; ++k) {
      const f32x4 av = *(const f32x4*)&s.a[k][4 * tr];
      const f32x4 bv = *(const f32x4*)&s.b[k][4 * tc];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_fmaf(av[a], bv[b], acc[a][b]);
    }
  }
}

__device__ __forceinline__ void zero(float (&acc)[4][4]) {
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
}

// Sum of v over the 16 lanes of this thread's tile row (lanes 16 q .. 16 q + 15
// of the wave hold the same tile rows), the same value on each of them.
__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 16);
  return v;
}

struct Chunk {
  int64_t b, c, h, g, t0;
  int Lc;  // valid steps of the chunk
};

__device__ __forceinline__ Chunk chunk_of(int64_t bh, int64_t c, int64_t H, int64_t G, int64_t L,
                                          int Q) {
  Chunk k;
  k.b = bh / H;
  k.h = bh % H;
  k.g = k.h / (H / G);
  k.c = c;
  k.t0 = c * Q;
  const int64_t rem = L - k.t0;
  k.Lc = (int)(rem < Q ? rem : Q);
  return k;
}

// The chunk's cumulative sums and dt into LDS (Q floats each).
__device__ __forceinline__ void load_cs(float* cs, float* dt, const float* __restrict__ dA_cs,
                                        const float* __restrict__ dt_T, int64_t b, int64_t h,
                                        int64_t c, int64_t H, int64_t nc, int Q) {
  const int64_t o = ((b * H + h) * nc + c) * Q;
  for (int i = threadIdx.x; i < Q; i += 256) {
    cs[i] = dA_cs[o + i];
    dt[i] = dt_T[o + i];
  }
}

// E[b, c, h] = sum_i 2^cs_i dy_i (outer) C_i over the chunk's valid steps.
// Grid: (p tiles x n tiles, nc, B H).
template <typename T>
__global__ void __launch_bounds__(256) gb_adjoint_kernel(
    const T* __restrict__ dy, const T* __restrict__ Cm, const float* __restrict__ dA_cs,
    const float* __restrict__ dt_T, float* __restrict__ E, int64_t L, int64_t H, int64_t G,
    int64_t P, int64_t N, int64_t nc, int Q, int nNt) {
  __shared__ Stage s;
  __shared__ float cs[256], dts[256];
  const Chunk k = chunk_of(blockIdx.z, blockIdx.y, H, G, L, Q);
  const int64_t p0 = (int64_t)(blockIdx.x / nNt) * kT, n0 = (int64_t)(blockIdx.x % nNt) * kT;
  load_cs(cs, dts, dA_cs, dt_T, k.b, k.h, k.c, H, nc, Q);
  __syncthreads();
  for (int i = threadIdx.x; i < Q; i += 256) cs[i] = fast_exp2(cs[i]);
  float acc[4][4];
  zero(acc);
  const T* dyb = dy + ((k.b * L + k.t0) * H + k.h) * P;
  const T* cb = Cm + ((k.b * L + k.t0) * G + k.g) * N;
  mm<false, false>(
      acc, 0, k.Lc,
      [&](int r, int i) { return p0 + r < P ? cs[i] * ld(dyb + (int64_t)i * H * P + p0 + r) : 0.f; },
      [&](int r, int i) { return n0 + r < N ? ld(cb + (int64_t)i * G * N + n0 + r) : 0.f; }, s);
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
  float* out = E + ((k.b * nc + k.c) * H + k.h) * P * N;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t p = p0 + 4 * tr + a, n = n0 + 4 * tc + b;
      if (p < P && n < N) out[p * N + n] = acc[a][b];
    }
}

// Reverse jump, in place: E[b, c, h] becomes g_c (the gradient at chunk c's
// end), dinit = r_0.  Per block also the part of <g_c, h_c> over its entries
// (ghp[b, h, c, block]).  Grid: (entry blocks, H, B).
__global__ void __launch_bounds__(256) gb_reverse_kernel(
    float* __restrict__ E, const float* __restrict__ hs, const float* __restrict__ dA_cs,
    const float* __restrict__ dfinal, float* __restrict__ dinit, float* __restrict__ ghp,
    int64_t H, int64_t PN, int64_t nc, int Q) {
  __shared__ float red[256];
  const int64_t h = blockIdx.y, b = blockIdx.z, nblk = gridDim.x;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool in = e < PN;
  const int64_t bh = b * H + h;
  float r = (in && dfinal) ? dfinal[bh * PN + e] : 0.f;
  for (int64_t c = nc - 1; c >= 0; --c) {
    const int64_t idx = ((b * nc + c) * H + h) * PN + e;
    float prod = 0.f;
    if (in) {
      const float ev = E[idx];
      E[idx] = r;
      prod = r * hs[idx];
      r = fast_exp2(dA_cs[(bh * nc + c) * Q + Q - 1]) * r + ev;
    }
    red[threadIdx.x] = prod;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
      __syncthreads();
    }
    if (threadIdx.x == 0) ghp[(bh * nc + c) * nblk + blockIdx.x] = red[0];
    __syncthreads();
  }
  if (in && dinit) dinit[bh * PN + e] = r;
}

// Vg[b, c, h][j, p] = sum_n B_j[n] g_c[p, n] and the per-p-tile parts of
// T^h_i = 2^cs_i sum_p dy_i[p] sum_n C_i[n] h_c[p, n] (thp[b, c, h, pt, i]).
// Grid: (q tiles x p tiles, nc, B H).
template <typename T>
__global__ void __launch_bounds__(256) gb_vy_kernel(
    const T* __restrict__ dy, const T* __restrict__ Bm, const T* __restrict__ Cm,
    const float* __restrict__ hs, const float* __restrict__ gs, const float* __restrict__ dA_cs,
    const float* __restrict__ dt_T, float* __restrict__ Vg, float* __restrict__ thp, int64_t L,
    int64_t H, int64_t G, int64_t P, int64_t N, int64_t nc, int Q, int nPt) {
  __shared__ Stage s;
  __shared__ float cs[256], dts[256];
  const Chunk k = chunk_of(blockIdx.z, blockIdx.y, H, G, L, Q);
  const int64_t i0 = (int64_t)(blockIdx.x / nPt) * kT;
  const int pt = blockIdx.x % nPt;
  const int64_t p0 = (int64_t)pt * kT;
  load_cs(cs, dts, dA_cs, dt_T, k.b, k.h, k.c, H, nc, Q);
  const int64_t sidx = ((k.b * nc + k.c) * H + k.h) * P * N;
  const T* bb = Bm + ((k.b * L + k.t0) * G + k.g) * N;
  const T* cb = Cm + ((k.b * L + k.t0) * G + k.g) * N;
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
  const int Lc = k.Lc;
  float acc[4][4];
  zero(acc);
  mm<true, true>(
      acc, 0, (int)N,
      [&](int r, int n) { return i0 + r < Lc ? ld(bb + (i0 + r) * G * N + n) : 0.f; },
      [&](int r, int n) { return p0 + r < P ? gs[sidx + (p0 + r) * N + n] : 0.f; }, s);
  float* vg = Vg + ((k.b * nc + k.c) * H + k.h) * Q * P;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t i = i0 + 4 * tr + a, p = p0 + 4 * tc + b;
      if (i < Q && p < P) vg[i * P + p] = acc[a][b];
    }
  zero(acc);
  mm<true, true>(
      acc, 0, (int)N,
      [&](int r, int n) { return i0 + r < Lc ? ld(cb + (i0 + r) * G * N + n) : 0.f; },
      [&](int r, int n) { return p0 + r < P ? hs[sidx + (p0 + r) * N + n] : 0.f; }, s);
  const T* dyb = dy + ((k.b * L + k.t0) * H + k.h) * P;
  float* th = thp + (((k.b * nc + k.c) * H + k.h) * nPt + pt) * Q;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t i = i0 + 4 * tr + a;
    float v = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t p = p0 + 4 * tc + b;
      if (i < Lc && p < P) v += acc[a][b] * ld(dyb + i * H * P + p);
    }
    v = row16_sum(v);
    if (tc == 0 && i < Q) th[i] = i < Lc ? fast_exp2(cs[i]) * v : 0.f;
  }
}

// CB[b, c, g][i, j] = C_i . B_j on and below the diagonal tiles.
// Grid: (q tiles x q tiles, nc, B G).
template <typename T>
__global__ void __launch_bounds__(256) gb_cb_kernel(const T* __restrict__ Bm,
                                                    const T* __restrict__ Cm,
                                                    float* __restrict__ CB, int64_t L, int64_t G,
                                                    int64_t N, int64_t nc, int Q, int nQt) {
  __shared__ Stage s;
  const int it = blockIdx.x / nQt, jt = blockIdx.x % nQt;
  if (jt > it) return;
  const int64_t b = blockIdx.z / G, g = blockIdx.z % G, c = blockIdx.y;
  const int64_t t0 = c * Q, rem = L - t0;
  const int Lc = (int)(rem < Q ? rem : Q);
  const int64_t i0 = (int64_t)it * kT, j0 = (int64_t)jt * kT;
  const T* bb = Bm + ((b * L + t0) * G + g) * N;
  const T* cb = Cm + ((b * L + t0) * G + g) * N;
  float acc[4][4];
  zero(acc);
  mm<true, true>(
      acc, 0, (int)N,
      [&](int r, int n) { return i0 + r < Lc ? ld(cb + (i0 + r) * G * N + n) : 0.f; },
      [&](int r, int n) { return j0 + r < Lc ? ld(bb + (j0 + r) * G * N + n) : 0.f; }, s);
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
  float* out = CB + ((b * nc + c) * G + g) * (int64_t)Q * Q;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int bb2 = 0; bb2 < 4; ++bb2) {
      const int64_t i = i0 + 4 * tr + a, j = j0 + 4 * tc + bb2;
      if (i < Q && j < Q) out[i * Q + j] = acc[a][bb2];
    }
}

// dU_j = sum_{i>=j} M_ij CB_ij dy_i + 2^(cl - cs_j) Vg_j; writes dx and the
// per-p-tile parts of x_j . dU_j (xup[b, c, h, pt, j]).
// Grid: (q tiles x p tiles, nc, B H).
template <typename T>
__global__ void __launch_bounds__(256) gb_du_kernel(
    const T* __restrict__ x, const T* __restrict__ dy, const float* __restrict__ CB,
    const float* __restrict__ Vg, const float* __restrict__ dA_cs, const float* __restrict__ dt_T,
    const float* __restrict__ D, T* __restrict__ dx, float* __restrict__ xup, int64_t L,
    int64_t H, int64_t G, int64_t P, int64_t nc, int Q, int nPt) {
  __shared__ Stage s;
  __shared__ float cs[256], dts[256];
  const Chunk k = chunk_of(blockIdx.z, blockIdx.y, H, G, L, Q);
  const int64_t j0 = (int64_t)(blockIdx.x / nPt) * kT;
  const int pt = blockIdx.x % nPt;
  const int64_t p0 = (int64_t)pt * kT;
  load_cs(cs, dts, dA_cs, dt_T, k.b, k.h, k.c, H, nc, Q);
  __syncthreads();
  const int Lc = k.Lc;
  const float* cbm = CB + ((k.b * nc + k.c) * G + k.g) * (int64_t)Q * Q;
  const T* dyb = dy + ((k.b * L + k.t0) * H + k.h) * P;
  const T* xb = x + ((k.b * L + k.t0) * H + k.h) * P;
  float acc[4][4];
  zero(acc);
  if (j0 < Lc)
    mm<false, false>(
        acc, (int)j0, Lc,
        [&](int r, int i) {
          const int64_t j = j0 + r;
          return (j < Lc && i >= j) ? fast_exp2(cs[i] - cs[j]) * cbm[i * Q + j] : 0.f;
        },
        [&](int r, int i) { return p0 + r < P ? ld(dyb + (int64_t)i * H * P + p0 + r) : 0.f; },
        s);
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
  const float cl = cs[Q - 1];
  const float dd = D ? D[k.h] : 0.f;
  const float* vg = Vg + ((k.b * nc + k.c) * H + k.h) * Q * P;
  float* xu = xup + (((k.b * nc + k.c) * H + k.h) * nPt + pt) * Q;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t j = j0 + 4 * tr + a;
    float v = 0.f;
    if (j < Lc) {
      const float sj = fast_exp2(cl - cs[j]);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t p = p0 + 4 * tc + b;
        if (p < P) {
          const float du = acc[a][b] + sj * vg[j * P + p];
          const int64_t o = j * H * P + p;
          st(dx + ((k.b * L + k.t0) * H + k.h) * P + o, dts[j] * du + dd * ld(dyb + o));
          v += ld(xb + o) * du;
        }
      }
    }
    v = row16_sum(v);
    if (tc == 0 && j < Q) xu[j] = v;
  }
}

// dq_k and ddt_k of one (batch, chunk, head); the chunk's parts of dA and dD.
// One block per (chunk, batch x head).  Grid: (nc, B H).
template <typename T>
__global__ void __launch_bounds__(256) gb_dq_kernel(
    const T* __restrict__ x, const T* __restrict__ dy, const float* __restrict__ CB,
    const float* __restrict__ Vg, const float* __restrict__ thp, const float* __restrict__ xup,
    const float* __restrict__ ghp, const float* __restrict__ dA_cs,
    const float* __restrict__ dt_T, const float* __restrict__ A, T* __restrict__ ddt,
    float* __restrict__ dA_part, float* __restrict__ dD_part, int64_t L, int64_t H, int64_t G,
    int64_t P, int64_t nc, int Q, int nPt, int nQt, int ngh) {
  __shared__ Stage s;
  __shared__ float cs[256], dts[256];
  __shared__ double colsum[256], rowsum[256], dq[256];
  __shared__ float part[16][kT];
  __shared__ float red[256];
  const Chunk k = chunk_of(blockIdx.y, blockIdx.x, H, G, L, Q);
  load_cs(cs, dts, dA_cs, dt_T, k.b, k.h, k.c, H, nc, Q);
  for (int i = threadIdx.x; i < 256; i += 256) colsum[i] = rowsum[i] = 0.0;
  __syncthreads();
  const int Lc = k.Lc;
  const float* cbm = CB + ((k.b * nc + k.c) * G + k.g) * (int64_t)Q * Q;
  const T* dyb = dy + ((k.b * L + k.t0) * H + k.h) * P;
  const T* xb = x + ((k.b * L + k.t0) * H + k.h) * P;
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
  // T_ij = M_ij CB_ij dt_j (dy_i . x_j) over the strictly lower triangle:
  // row sums and column sums, tile by tile in a fixed order
  for (int it = 0; it < nQt; ++it)
    for (int jt = 0; jt <= it; ++jt) {
      const int64_t i0 = (int64_t)it * kT, j0 = (int64_t)jt * kT;
      if (i0 >= Lc) continue;
      float acc[4][4];
      zero(acc);
      mm<true, true>(
          acc, 0, (int)P,
          [&](int r, int p) { return i0 + r < Lc ? ld(dyb + (i0 + r) * H * P + p) : 0.f; },
          [&](int r, int p) { return j0 + r < Lc ? ld(xb + (j0 + r) * H * P + p) : 0.f; }, s);
      float cpart[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int64_t i = i0 + 4 * tr + a;
        float rp = 0.f;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int64_t j = j0 + 4 * tc + b;
          float t = 0.f;
          if (i < Lc && j < i) t = fast_exp2(cs[i] - cs[j]) * cbm[i * Q + j] * dts[j] * acc[a][b];
          rp += t;
          cpart[b] += t;
        }
        rp = row16_sum(rp);
        if (tc == 0 && i < Q) rowsum[i] += (double)rp;
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) part[tr][4 * tc + b] = cpart[b];
      __syncthreads();
      if (threadIdx.x < kT && j0 + threadIdx.x < Q) {
        float v = 0.f;
        for (int q = 0; q < 16; ++q) v += part[q][threadIdx.x];
        colsum[j0 + threadIdx.x] += (double)v;
      }
      __syncthreads();
    }
  // per-step terms: T^h_i (summed over p tiles), T^S_j, x_j . dU_j, dy . x
  const float cl = cs[Q - 1];
  const float* vg = Vg + ((k.b * nc + k.c) * H + k.h) * Q * P;
  const int64_t base = ((k.b * nc + k.c) * H + k.h) * nPt;
  float ddx = 0.f;
  for (int i = threadIdx.x; i < Q; i += 256) {
    double th = 0.0, xu = 0.0;
    for (int q = 0; q < nPt; ++q) {
      th += thp[(base + q) * Q + i];
      xu += xup[(base + q) * Q + i];
    }
    float ts = 0.f, dyx = 0.f;
    if (i < Lc) {
      for (int64_t p = 0; p < P; ++p) {
        const float xv = ld(xb + (int64_t)i * H * P + p);
        ts += xv * vg[(int64_t)i * P + p];
        dyx += xv * ld(dyb + (int64_t)i * H * P + p);
      }
      ts *= fast_exp2(cl - cs[i]) * dts[i];
    }
    ddx += dyx;
    // stash: dq holds T^h for now; part[0..3] rows reused for T^S and x.dU
    dq[i] = th;
    ((float*)part)[i] = ts;
    ((float*)part)[256 + i] = (float)xu;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double gh = 0.0;
    const float* gp = ghp + ((k.b * H + k.h) * nc + k.c) * ngh;
    for (int q = 0; q < ngh; ++q) gh += gp[q];
    const double carried = (double)fast_exp2(cl) * gh;
    // suffix sums of T^h, prefix sums of T^S and of colsum - rowsum
    double suf = 0.0;
    for (int i = Q - 1; i >= 0; --i) {
      suf += dq[i];
      dq[i] = suf;
    }
    double pre = 0.0, rect = 0.0;
    for (int i = 0; i < Q; ++i) {
      dq[i] += pre + rect + carried;
      pre += (double)((float*)part)[i];
      rect += colsum[i] - rowsum[i];
    }
  }
  __syncthreads();
  const float a = A[k.h];
  float dap = 0.f;
  for (int i = threadIdx.x; i < Lc; i += 256) {
    const float q = (float)dq[i];
    st(ddt + (k.b * L + k.t0 + i) * H + k.h, ((float*)part)[256 + i] + a * q);
    dap += dts[i] * q;
  }
  // block sums of dap and ddx, fixed order
  red[threadIdx.x] = dap;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) dA_part[(k.b * nc + k.c) * H + k.h] = red[0];
  __syncthreads();
  red[threadIdx.x] = ddx;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) dD_part[(k.b * nc + k.c) * H + k.h] = red[0];
}

// (M o W) of tile (i0, j0) into LDS: mw[r][q] = M_ij dt_j (dy_i . x_j) for
// i = i0 + r >= j = j0 + q, both valid; 0 elsewhere.
template <typename T>
__device__ __forceinline__ void mw_tile(float (*mw)[kT + 1], int64_t i0, int64_t j0, int Lc,
                                        const T* dyb, const T* xb, int64_t HP, int64_t P,
                                        const float* cs, const float* dts, Stage& s) {
  float acc[4][4];
  zero(acc);
  mm<true, true>(
      acc, 0, (int)P,
      [&](int r, int p) { return i0 + r < Lc ? ld(dyb + (i0 + r) * HP + p) : 0.f; },
      [&](int r, int p) { return j0 + r < Lc ? ld(xb + (j0 + r) * HP + p) : 0.f; }, s);
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t i = i0 + 4 * tr + a, j = j0 + 4 * tc + b;
      mw[4 * tr + a][4 * tc + b] =
          (i < Lc && j <= i) ? fast_exp2(cs[i] - cs[j]) * dts[j] * acc[a][b] : 0.f;
    }
}

// dC (DB = false) or dB (DB = true) of one (batch, chunk, group) row tile and
// up to kNG state-column tiles, summed over the group's heads:
//   dC_i = sum_h [sum_{j<=i} (M o W)_ij B_j + 2^cs_i dy_i h]
//   dB_j = sum_h [sum_{i>=j} (M o W)_ij C_i + 2^(cl - cs_j) dt_j x_j g]
// Per head the (M o W) tiles that meet the row tile are formed once into LDS
// and used for every column tile (kNG accumulator tiles per thread).
// Grid: (q tiles x column-tile groups, nc, B G).
constexpr int kNG = 2;

template <typename T, bool DB>
__global__ void __launch_bounds__(256) gb_dbdc_kernel(
    const T* __restrict__ x, const T* __restrict__ dy, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const float* __restrict__ st_, const float* __restrict__ dA_cs,
    const float* __restrict__ dt_T, T* __restrict__ out, int64_t L, int64_t H, int64_t G,
    int64_t P, int64_t N, int64_t nc, int Q, int nNt, int nQt) {
  __shared__ Stage s;
  __shared__ float cs[256], dts[256];
  __shared__ float mw[4][kT][kT + 1];  // Q <= 256: at most four tiles meet a row tile
  const int nNg = (nNt + kNG - 1) / kNG;
  const int64_t b = blockIdx.z / G, g = blockIdx.z % G, c = blockIdx.y;
  const int rt = blockIdx.x / nNg, ng = blockIdx.x % nNg;
  const int64_t r0 = (int64_t)rt * kT;
  const int nt0 = ng * kNG;
  const int64_t t0 = c * Q, rem = L - t0;
  const int Lc = (int)(rem < Q ? rem : Q);
  const int64_t HG = H / G, HP = H * P;
  // the other operand of the in-chunk term: B rows for dC, C rows for dB
  const T* ob = (DB ? Cm : Bm) + ((b * L + t0) * G + g) * N;
  const int lo = DB ? rt : 0, hi = DB ? nQt - 1 : rt;
  float acc[kNG][4][4];
#pragma unroll
  for (int u = 0; u < kNG; ++u) zero(acc[u]);
  if (r0 < Lc) {
    for (int64_t hh = 0; hh < HG; ++hh) {
      const int64_t h = g * HG + hh;
      __syncthreads();
      load_cs(cs, dts, dA_cs, dt_T, b, h, c, H, nc, Q);
      __syncthreads();
      const float cl = cs[Q - 1];
      const T* dyb = dy + ((b * L + t0) * H + h) * P;
      const T* xb = x + ((b * L + t0) * H + h) * P;
      const float* sm = st_ + ((b * nc + c) * H + h) * P * N;  // h_c (dC) or g_c (dB)
      // this head's (M o W) tiles against the row tile
      for (int ot = lo; ot <= hi; ++ot) {
        const int64_t o0 = (int64_t)ot * kT;
        if (o0 >= Lc) break;
        if (DB)
          mw_tile(mw[ot - lo], o0, r0, Lc, dyb, xb, HP, P, cs, dts, s);  // rows i, columns j
        else
          mw_tile(mw[ot - lo], r0, o0, Lc, dyb, xb, HP, P, cs, dts, s);
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kNG; ++u) {
        if (nt0 + u >= nNt) break;  // uniform
        const int64_t n0 = (int64_t)(nt0 + u) * kT;
        // state term over p
        mm<true, false>(
            acc[u], 0, (int)P,
            [&](int r, int p) {
              const int64_t i = r0 + r;
              if (i >= Lc) return 0.f;
              return DB ? fast_exp2(cl - cs[i]) * dts[i] * ld(xb + i * HP + p)
                        : fast_exp2(cs[i]) * ld(dyb + i * HP + p);
            },
            [&](int r, int p) { return n0 + r < N ? sm[(int64_t)p * N + n0 + r] : 0.f; }, s);
        // in-chunk term, tile by tile of the other index
        for (int ot = lo; ot <= hi; ++ot) {
          const int64_t o0 = (int64_t)ot * kT;
          if (o0 >= Lc) break;
          const float(*m)[kT + 1] = mw[ot - lo];
          mm<false, false>(
              acc[u], 0, kT, [&](int r, int q) { return DB ? m[q][r] : m[r][q]; },
              [&](int r, int q) {
                const int64_t t = o0 + q;
                return (t < Lc && n0 + r < N) ? ld(ob + t * G * N + n0 + r) : 0.f;
              },
              s);
        }
      }
    }
  }
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
#pragma unroll
  for (int u = 0; u < kNG; ++u) {
    if (nt0 + u >= nNt) break;
    const int64_t n0 = (int64_t)(nt0 + u) * kT;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int64_t r = r0 + 4 * tr + a, n = n0 + 4 * tc + bb;
        if (r < Lc && n < N) st(out + ((b * L + t0 + r) * G + g) * N + n, acc[u][a][bb]);
      }
  }
}

template <typename T>
hipError_t launch_generic(const Dims& d, const void* x, const void* dy, const void* B,
                          const void* C, const float* dA_cs, const float* dt_T, float* hs,
                          float* E, const float* dfinal, float* dinit, const float* A,
                          const float* D, void* dx, void* ddt, void* dB, void* dC,
                          const GenericBwdScratch& w, hipStream_t s) {
  const int Q = (int)d.Q;
  const int nPt = (int)((d.P + kT - 1) / kT), nNt = (int)((d.N + kT - 1) / kT);
  const int nQt = (Q + kT - 1) / kT;
  const unsigned nc = (unsigned)d.nc, BH = (unsigned)(d.B * d.H), BG = (unsigned)(d.B * d.G);
  const int64_t PN = d.P * d.N;
  const int ngh = (int)((PN + 255) / 256);
  const T* xt = (const T*)x;
  const T* dyt = (const T*)dy;
  const T* Bt = (const T*)B;
  const T* Ct = (const T*)C;
  gb_adjoint_kernel<T><<<dim3(nPt * nNt, nc, BH), 256, 0, s>>>(
      dyt, Ct, dA_cs, dt_T, E, d.L, d.H, d.G, d.P, d.N, d.nc, Q, nNt);
  gb_reverse_kernel<<<dim3(ngh, (unsigned)d.H, (unsigned)d.B), 256, 0, s>>>(
      E, hs, dA_cs, dfinal, dinit, w.ghp, d.H, PN, d.nc, Q);
  gb_vy_kernel<T><<<dim3(nQt * nPt, nc, BH), 256, 0, s>>>(dyt, Bt, Ct, hs, E, dA_cs, dt_T, w.vg,
                                                          w.thp, d.L, d.H, d.G, d.P, d.N, d.nc,
                                                          Q, nPt);
  gb_cb_kernel<T><<<dim3(nQt * nQt, nc, BG), 256, 0, s>>>(Bt, Ct, w.cb, d.L, d.G, d.N, d.nc, Q,
                                                          nQt);
  gb_du_kernel<T><<<dim3(nQt * nPt, nc, BH), 256, 0, s>>>(
      xt, dyt, w.cb, w.vg, dA_cs, dt_T, D, (T*)dx, w.xup, d.L, d.H, d.G, d.P, d.nc, Q, nPt);
  gb_dq_kernel<T><<<dim3(nc, BH), 256, 0, s>>>(
      xt, dyt, w.cb, w.vg, w.thp, w.xup, w.ghp, dA_cs, dt_T, A, (T*)ddt, w.dA_part, w.dD_part,
      d.L, d.H, d.G, d.P, d.nc, Q, nPt, nQt, ngh);
  const unsigned nNg = (unsigned)((nNt + kNG - 1) / kNG);
  gb_dbdc_kernel<T, false><<<dim3(nQt * nNg, nc, BG), 256, 0, s>>>(
      xt, dyt, Bt, Ct, hs, dA_cs, dt_T, (T*)dC, d.L, d.H, d.G, d.P, d.N, d.nc, Q, nNt, nQt);
  gb_dbdc_kernel<T, true><<<dim3(nQt * nNg, nc, BG), 256, 0, s>>>(
      xt, dyt, Bt, Ct, E, dA_cs, dt_T, (T*)dB, d.L, d.H, d.G, d.P, d.N, d.nc, Q, nNt, nQt);
  return hipGetLastError();
}

}  // namespace

GenericBwdSizes generic_backward_sizes(const Dims& d) {
  GenericBwdSizes z;
  const int64_t nPt = (d.P + kT - 1) / kT;
  z.vg = (size_t)(d.B * d.nc * d.H * d.Q * d.P);
  z.thp = z.xup = (size_t)(d.B * d.nc * d.H * nPt * d.Q);
  z.ghp = (size_t)(d.B * d.H * d.nc * ((d.P * d.N + 255) / 256));
  z.cb = (size_t)(d.B * d.nc * d.G * d.Q * d.Q);
  z.part = (size_t)(d.B * d.nc * d.H);
  return z;
}

hipError_t launch_backward_generic(const Dims& d, const void* x, const void* dy, const void* B,
                                   const void* C, const float* dA_cs, const float* dt_T,
                                   float* hs, float* E, const float* dfinal, float* dinit,
                                   const float* A, const float* D, void* dx, void* ddt, void* dB,
                                   void* dC, const GenericBwdScratch& w, hipStream_t s) {
  if (d.Q > 256) return hipErrorInvalidValue;  // the per-chunk LDS arrays hold 256 steps
  return d.bf16 ? launch_generic<bf16>(d, x, dy, B, C, dA_cs, dt_T, hs, E, dfinal, dinit, A, D,
                                       dx, ddt, dB, dC, w, s)
                : launch_generic<float>(d, x, dy, B, C, dA_cs, dt_T, hs, E, dfinal, dinit, A, D,
                                        dx, ddt, dB, dC, w, s);
}

}  // namespace m2
