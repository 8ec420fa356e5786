// chunk_scan = compute_out: outputs of each chunk from its start state, fused
// so that the chunk x chunk interaction matrix stays on chip (devotd.net news
// item on the Mamba-2 CUDA Tile forward-pass kernels, section 2: compute_out
// keeps the intermediate matrix in registers instead of global memory;
// disconfirmai.com "Jane Street ML Engineers Map Mamba-2 Recurrent State
// Computation to Tensor Cores with cuTile", abstract: carried-state term,
// decayed causally masked interaction matrix and skip connection in one tiled
// kernel).  For token i of chunk c, head h (group g):
//     y[i,p] = 2^cs_i sum_n C[i,n] h[p,n]                          (carried state)
//            + sum_{j<=i} G[j,i] 2^(cs_i - cs_j) dt_j x[j,p]        (in-chunk)
//            + D x[i,p]                                            (skip)
//     G[j,i] = sum_n B[j,n] C[i,n]
//
// bfloat16 path (MFMA, fp32 accumulation).  Everything is computed
// transposed, Y^T[p, i], so that the accumulator of G^T = B C^T (lane holds
// one column i and four consecutive rows j) can be masked, decayed, rounded
// to bf16 and fed straight back as the B operand of the next MFMA without
// leaving registers.  The K order of that MFMA is permuted to match: element
// e of lane group q stands for j = 32 jp + 4q + e (e < 4) or
// 32 jp + 16 + 4q + (e - 4).  The x operand follows the same permutation
// through two LDS transpose reads.  Output rows are permuted the same way in
// every contraction, MFMA row m of p-tile pt (PT = P/16 tiles) standing for
// p = 4 PT (m/4) + 4 pt + m%4, so each lane finally holds 4 PT consecutive p
// of one token and writes them with 16-byte stores.  The skip term rides on the diagonal of the masked
// matrix (j == i), where the decay is exactly 1.
//
// Work split: one workgroup per (b, c, h) with Q/32 waves; wave w owns the
// 16-row i-tiles w and Q/16-1-w, which balances the causal triangle.  C, B
// and the start state stream through LDS in blocks of NB state columns.
//
// float32 path: one thread per output element, plain loops.
#include "common.h"
#include "launch.h"

namespace m2 {

namespace {

template <int P, int Q, int NB>
struct ScanCfg {
  static constexpr int QT = Q / 16;       // 16-row tiles per chunk
  static constexpr int NW = Q / 32;       // waves
  static constexpr int PT = P / 16;       // p tiles
  static constexpr int XS = P + 8;        // LDS row strides (elements)
  static constexpr int CS = NB + 8;
  static constexpr int HS = NB + 8;
  static constexpr size_t lds_bytes =
      (size_t)Q * XS * 2 + 2 * (size_t)Q * CS * 2 + (size_t)P * HS * 2 + 2 * (size_t)Q * 4;
};

// Output-row permutation: MFMA row m of p-tile pt stands for this p.
template <int PT>
__device__ __forceinline__ int prow(int m, int pt) { return 4 * PT * (m >> 2) + 4 * pt + (m & 3); }

// Finishes one 16-row i-tile t of a wave: scales the carried-state part by
// 2^cs_i, adds the masked in-chunk contraction over the j-tiles 0..t held in
// Gt (accumulators of G^T[j, i]), and stores y rows i < valid.
template <int NG, int P, int Q>
__device__ __forceinline__ void tile_out(f32x4 (&Gt)[NG], f32x4 (&Yt)[P / 16], int t,
                                         const float* css, const float* dts, const bf16* Xs,
                                         float Dh, bf16* __restrict__ y, int64_t ybase, int H,
                                         int64_t valid) {
  constexpr int PT = P / 16, XS = P + 8;
  const int lane = lane_id();
  const int L16 = lane & 15, grp = lane >> 4;
  const int i = 16 * t + L16;
  const float csi = css[i];
  const float sc = fast_exp2(csi);
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) Yt[pt] *= sc;
#pragma unroll
  for (int jp = 0; jp < (NG + 1) / 2; ++jp) {
    if (2 * jp > t) break;
    bf16x8 gm;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int jt = 2 * jp + half;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float gv = 0.f;
        if (jt < NG && jt <= t) {
          const int j = 16 * jt + 4 * grp + r;
          if (j <= i) gv = Gt[jt < NG ? jt : 0][r] * fast_exp2(csi - css[j]) * dts[j];
          if (j == i) gv += Dh;
        }
        gm[half * 4 + r] = f2bf(gv);
      }
    }
    const int ka = 32 * jp + 4 * grp + (L16 >> 2);
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      const bf16* p0 = Xs + ka * XS + 4 * PT * (L16 & 3) + 4 * pt;
      const bf16x8 xop = cat(lds_read_tr(p0), lds_read_tr(p0 + 16 * XS));
      Yt[pt] = mfma16x16x32(xop, gm, Yt[pt]);
    }
  }
  if (i < valid) {
    bf16* dst = y + (ybase + (int64_t)i * H) * P + 4 * PT * grp;
    if constexpr (PT % 2 == 0) {  // 16-byte stores
#pragma unroll
      for (int pt = 0; pt < PT; pt += 2) {
        bf16x8 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          o[r] = f2bf(Yt[pt][r]);
          o[4 + r] = f2bf(Yt[pt + 1][r]);
        }
        *(bf16x8*)(dst + 4 * pt) = o;
      }
    } else {  // an odd tile count leaves the lane's run 8-byte aligned only
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        bf16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = f2bf(Yt[pt][r]);
        *(bf16x4*)(dst + 4 * pt) = o;
      }
    }
  }
}

template <int P, int Q, int NB>
__global__ void __launch_bounds__(Q * 2) chunk_scan_bf16_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ Bm, const bf16* __restrict__ Cm,
    const float* __restrict__ dA_cs, const float* __restrict__ dt_T,
    const float* __restrict__ states, const float* __restrict__ Dv, bf16* __restrict__ y, int L,
    int H, int G, int N, int nc) {
  using K = ScanCfg<P, Q, NB>;
  constexpr int QT = K::QT, PT = K::PT, XS = K::XS, CS = K::CS, HS = K::HS;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16* Xs = (bf16*)smem;            // [Q][XS]   x rows of the chunk
  bf16* Cs = Xs + Q * XS;            // [Q][CS]   C rows, one NB column block
  bf16* Bs = Cs + Q * CS;            // [Q][CS]   B rows, one NB column block
  bf16* Hs = Bs + Q * CS;            // [P][HS]   start state, one NB column block
  float* css = (float*)(Hs + P * HS);  // [Q]
  float* dts = css + Q;                // [Q]

  const int bid = blockIdx.x;
  const int h = bid % H;
  const int c = (bid / H) % nc;
  const int b = bid / (H * nc);
  const int g = h / (H / G);
  const int tid = threadIdx.x;
  constexpr int nthr = Q * 2;
  const int lane = lane_id();
  const int w = wave_id();
  const int L16 = lane & 15, grp = lane >> 4;
  const int t0 = w, t1 = QT - 1 - w;  // this wave's i-tiles (t0 < t1)
  const int64_t tok0 = (int64_t)c * Q;

  const int64_t cbase = ((int64_t)b * H + h) * nc + c;
  for (int j = tid; j < Q; j += nthr) {
    css[j] = dA_cs[cbase * Q + j];
    dts[j] = dt_T[cbase * Q + j];
  }
  for (int idx = tid; idx < Q * (P / 8); idx += nthr) {
    const int r = idx / (P / 8), c8 = (idx % (P / 8)) * 8;
    const int64_t t = tok0 + r;
    bf16x8 v;
    if (t < L) {
      v = *(const bf16x8*)(x + ((((int64_t)b * L + t) * H + h) * P + c8));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = f2bf(0.f);
    }
    *(bf16x8*)(Xs + r * XS + c8) = v;
  }

  f32x4 G0[QT / 2], G1[QT];
  f32x4 Y[2][PT];
#pragma unroll
  for (int a = 0; a < QT / 2; ++a) G0[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int a = 0; a < QT; ++a) G1[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int a = 0; a < PT; ++a) Y[0][a] = Y[1][a] = f32x4{0.f, 0.f, 0.f, 0.f};

  // State columns in blocks of NB; a last block reaching past N (N is a
  // multiple of 16) is zero beyond it in all three tiles, so it adds nothing.
  const float* hsrc = states + (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
  for (int nb = 0; nb < N; nb += NB) {
    __syncthreads();
    for (int idx = tid; idx < Q * (NB / 8); idx += nthr) {
      const int r = idx / (NB / 8), c8 = (idx % (NB / 8)) * 8;
      const int64_t t = tok0 + r;
      bf16x8 vc, vb;
      if (t < L && nb + c8 < N) {
        const int64_t off = (((int64_t)b * L + t) * G + g) * N + nb + c8;
        vc = *(const bf16x8*)(Cm + off);
        vb = *(const bf16x8*)(Bm + off);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) vc[e] = vb[e] = f2bf(0.f);
      }
      *(bf16x8*)(Cs + r * CS + c8) = vc;
      *(bf16x8*)(Bs + r * CS + c8) = vb;
    }
    for (int idx = tid; idx < P * (NB / 4); idx += nthr) {
      const int p = idx / (NB / 4), c4 = (idx % (NB / 4)) * 4;
      const f32x4 v = nb + c4 < N ? *(const f32x4*)(hsrc + (int64_t)p * N + nb + c4)
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
      bf16x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = f2bf(v[e]);
      *(bf16x4*)(Hs + p * HS + c4) = o;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < NB / 32; ++kk) {
      const int koff = kk * 32 + grp * 8;
      const bf16x8 c0op = *(const bf16x8*)(Cs + (16 * t0 + L16) * CS + koff);
      const bf16x8 c1op = *(const bf16x8*)(Cs + (16 * t1 + L16) * CS + koff);
#pragma unroll
      for (int jt = 0; jt < QT; ++jt) {
        if (jt <= t1) {
          const bf16x8 bop = *(const bf16x8*)(Bs + (16 * jt + L16) * CS + koff);
          if (jt < QT / 2 && jt <= t0) G0[jt] = mfma16x16x32(bop, c0op, G0[jt]);
          G1[jt] = mfma16x16x32(bop, c1op, G1[jt]);
        }
      }
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const bf16x8 hop = *(const bf16x8*)(Hs + prow<PT>(L16, pt) * HS + koff);
        Y[0][pt] = mfma16x16x32(hop, c0op, Y[0][pt]);
        Y[1][pt] = mfma16x16x32(hop, c1op, Y[1][pt]);
      }
    }
  }

  const float Dh = Dv ? Dv[h] : 0.f;
  const int64_t ybase = ((int64_t)b * L + tok0) * H + h;
  tile_out<QT / 2, P, Q>(G0, Y[0], t0, css, dts, Xs, Dh, y, ybase, H, L - tok0);
  tile_out<QT, P, Q>(G1, Y[1], t1, css, dts, Xs, Dh, y, ybase, H, L - tok0);
}

// float32: one thread per (b, t, h, p).
__global__ void __launch_bounds__(256) chunk_scan_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ Bm, const float* __restrict__ Cm,
    const float* __restrict__ dA_cs, const float* __restrict__ dt_T,
    const float* __restrict__ states, const float* __restrict__ Dv, float* __restrict__ y,
    int64_t total, int L, int H, int G, int P, int N, int Q, int nc) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int p = (int)(gid % P);
  const int h = (int)((gid / P) % H);
  const int64_t t = (gid / ((int64_t)P * H)) % L;
  const int b = (int)(gid / ((int64_t)P * H * L));
  const int g = h / (H / G);
  const int c = (int)(t / Q), i = (int)(t % Q);
  const int64_t cbase = ((int64_t)b * H + h) * nc + c;
  const float* cs = dA_cs + cbase * Q;
  const float* dtc = dt_T + cbase * Q;
  const float* Ci = Cm + (((int64_t)b * L + t) * G + g) * N;
  const float* hp = states + ((((int64_t)b * nc + c) * H + h) * P + p) * N;
  float inter = 0.f;
  for (int n = 0; n < N; ++n) inter += Ci[n] * hp[n];
  float acc = exp2f(cs[i]) * inter;
  for (int j = 0; j <= i; ++j) {
    const int64_t tj = (int64_t)c * Q + j;
    const float* Bj = Bm + (((int64_t)b * L + tj) * G + g) * N;
    float cb = 0.f;
    for (int n = 0; n < N; ++n) cb += Ci[n] * Bj[n];
    acc += cb * exp2f(cs[i] - cs[j]) * dtc[j] * x[(((int64_t)b * L + tj) * H + h) * P + p];
  }
  if (Dv) acc += Dv[h] * x[gid];
  y[gid] = acc;
}

template <int P, int Q, int NB>
hipError_t launch_bf16(const Dims& d, const void* x, const void* B, const void* C,
                       const float* dA_cs, const float* dt_T, const float* states, const float* D,
                       void* y, hipStream_t s) {
  using K = ScanCfg<P, Q, NB>;
  auto kern = chunk_scan_bf16_kernel<P, Q, NB>;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)K::lds_bytes);
  if (attr != hipSuccess) return attr;
  kern<<<(unsigned)(d.B * d.nc * d.H), Q * 2, K::lds_bytes, s>>>(
      (const bf16*)x, (const bf16*)B, (const bf16*)C, dA_cs, dt_T, states, D, (bf16*)y,
      (int)d.L, (int)d.H, (int)d.G, (int)d.N, (int)d.nc);
  return hipGetLastError();
}

template <int P>
hipError_t launch_bf16_q(const Dims& d, const void* x, const void* B, const void* C,
                         const float* dA_cs, const float* dt_T, const float* states,
                         const float* D, void* y, hipStream_t s) {
  constexpr int NB = P > 64 ? 32 : 64;
  switch (d.Q) {
    case 64: return launch_bf16<P, 64, NB>(d, x, B, C, dA_cs, dt_T, states, D, y, s);
    case 128: return launch_bf16<P, 128, NB>(d, x, B, C, dA_cs, dt_T, states, D, y, s);
    case 256: return launch_bf16<P, 256, NB>(d, x, B, C, dA_cs, dt_T, states, D, y, s);
    default: return hipErrorInvalidValue;
  }
}

// The same float32 arithmetic, in the same order, with one workgroup per
// (b, c, h) for sizes where the chunk fits in LDS: the chunk's C, B and x
// rows, its start state, cumulative sums and dt are staged once, then the
// decayed in-chunk weights W[i][j] = (C_i . B_j) 2^(cs_i - cs_j) dt_j (j <= i)
// are formed once per chunk by the whole workgroup, and each output is the
// carried-state dot product plus one pass over W's row.  The plain kernel
// above reloads C, B and x rows from global memory inside its inner loops
// and recomputes C_i . B_j for every output column.
__global__ void __launch_bounds__(256) chunk_scan_f32_lds_kernel(
    const float* __restrict__ x, const float* __restrict__ Bm, const float* __restrict__ Cm,
    const float* __restrict__ dA_cs, const float* __restrict__ dt_T,
    const float* __restrict__ states, const float* __restrict__ Dv, float* __restrict__ y, int L,
    int H, int G, int P, int N, int Q, int nc) {
  extern __shared__ float sm[];
  const int NS = N + 1;      // C and B row stride: neighbouring rows in different banks
  float* Cs = sm;            // [Q][NS]
  float* Bs = Cs + Q * NS;   // [Q][NS]
  float* Xs = Bs + Q * NS;   // [Q][P]
  float* Hs = Xs + Q * P;    // [P][N]
  float* css = Hs + P * N;   // [Q]
  float* dts = css + Q;      // [Q]
  float* W = dts + Q;        // [Q][Q], lower triangle used
  const int h = blockIdx.x % H;
  const int c = (blockIdx.x / H) % nc;
  const int b = blockIdx.x / (H * nc);
  const int g = h / (H / G);
  const int64_t tok0 = (int64_t)c * Q;
  const int valid = (int)min((int64_t)Q, (int64_t)L - tok0);
  const int tid = threadIdx.x;
  for (int idx = tid; idx < valid * N; idx += blockDim.x) {
    const int r = idx / N, n = idx % N;
    const int64_t off = (((int64_t)b * L + tok0 + r) * G + g) * N + n;
    Cs[r * NS + n] = Cm[off];
    Bs[r * NS + n] = Bm[off];
  }
  for (int idx = tid; idx < valid * P; idx += blockDim.x) {
    const int r = idx / P, p = idx % P;
    Xs[idx] = x[(((int64_t)b * L + tok0 + r) * H + h) * P + p];
  }
  const float* hsrc = states + (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
  for (int idx = tid; idx < P * N; idx += blockDim.x) Hs[idx] = hsrc[idx];
  const int64_t cbase = (((int64_t)b * H + h) * nc + c) * Q;
  for (int idx = tid; idx < valid; idx += blockDim.x) {
    css[idx] = dA_cs[cbase + idx];
    dts[idx] = dt_T[cbase + idx];
  }
  __syncthreads();
  for (int idx = tid; idx < valid * valid; idx += blockDim.x) {
    const int i = idx / valid, j = idx % valid;
    if (j > i) continue;
    const float* Ci = Cs + i * NS;
    const float* Bj = Bs + j * NS;
    float cb = 0.f;
    for (int n = 0; n < N; ++n) cb += Ci[n] * Bj[n];
    W[i * Q + j] = cb * exp2f(css[i] - css[j]) * dts[j];
  }
  __syncthreads();
  const float Dh = Dv ? Dv[h] : 0.f;
  for (int o = tid; o < valid * P; o += blockDim.x) {
    const int i = o / P, p = o % P;
    const float* Ci = Cs + i * NS;
    const float* hp = Hs + p * N;
    float inter = 0.f;
    for (int n = 0; n < N; ++n) inter += Ci[n] * hp[n];
    float acc = exp2f(css[i]) * inter;
    for (int j = 0; j <= i; ++j) acc += W[i * Q + j] * Xs[j * P + p];
    if (Dv) acc += Dh * Xs[i * P + p];
    y[(((int64_t)b * L + tok0 + i) * H + h) * P + p] = acc;
  }
}

// LDS bytes the staged float32 kernel needs, if it fits in 64 KB (else 0).
size_t f32_lds_bytes(const Dims& d) {
  const int64_t n = 2 * d.Q * (d.N + 1) + d.Q * d.P + d.P * d.N + 2 * d.Q + d.Q * d.Q;
  return n * 4 <= 64 * 1024 ? (size_t)n * 4 : 0;
}

}  // namespace

hipError_t launch_chunk_scan(const Dims& d, const void* x, const void* B, const void* C,
                             const float* dA_cs, const float* dt_T, const float* states,
                             const float* D, void* y, hipStream_t s) {
  if (d.bf16) {
    switch (d.P) {
      case 16: return launch_bf16_q<16>(d, x, B, C, dA_cs, dt_T, states, D, y, s);
      case 32: return launch_bf16_q<32>(d, x, B, C, dA_cs, dt_T, states, D, y, s);
      case 48: return launch_bf16_q<48>(d, x, B, C, dA_cs, dt_T, states, D, y, s);
      case 64: return launch_bf16_q<64>(d, x, B, C, dA_cs, dt_T, states, D, y, s);
      case 80: return launch_bf16_q<80>(d, x, B, C, dA_cs, dt_T, states, D, y, s);
      case 96: return launch_bf16_q<96>(d, x, B, C, dA_cs, dt_T, states, D, y, s);
      case 112: return launch_bf16_q<112>(d, x, B, C, dA_cs, dt_T, states, D, y, s);
      case 128: return launch_bf16_q<128>(d, x, B, C, dA_cs, dt_T, states, D, y, s);
      default: return hipErrorInvalidValue;
    }
  }
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)chunk_scan_f32_lds_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
      64 * 1024);
  if (const size_t lds = attr == hipSuccess ? f32_lds_bytes(d) : 0) {
    chunk_scan_f32_lds_kernel<<<(unsigned)(d.B * d.nc * d.H), 256, lds, s>>>(
        (const float*)x, (const float*)B, (const float*)C, dA_cs, dt_T, states, D, (float*)y,
        (int)d.L, (int)d.H, (int)d.G, (int)d.P, (int)d.N, (int)d.Q, (int)d.nc);
    return hipGetLastError();
  }
  const int64_t total = d.B * d.L * d.H * d.P;
  chunk_scan_f32_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
      (const float*)x, (const float*)B, (const float*)C, dA_cs, dt_T, states, D, (float*)y, total,
      (int)d.L, (int)d.H, (int)d.G, (int)d.P, (int)d.N, (int)d.Q, (int)d.nc);
  return hipGetLastError();
}

}  // namespace m2
