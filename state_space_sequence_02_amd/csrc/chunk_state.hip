// chunk_state: the state each chunk reaches from a zero start, the per-chunk
// B X^T contraction of fwd_pass_state (disconfirmai.com "Jane Street ML
// Engineers Map Mamba-2 Recurrent State Computation to Tensor Cores with
// cuTile", body: without decay the jump over a chunk is h + B X^T, a matrix
// product; with decay, rows are pre-scaled by exponentials of the log-space
// cumulative sum).  For chunk c, head h (group g):
//     S[p, n] = sum_j w_j x[j, p] B[j, n],   w_j = 2^(cs[Q-1] - cs[j]) dt_j
//
// bfloat16 path (MFMA): the kernel computes S^T = B^T (w X), M = n, N = p,
// K = time.  Both operands are stored in LDS in their natural row-major
// [time][feature] layout (x rows scaled by w_j while staged) and read with
// the gfx950 LDS transpose read, which hands each lane the four consecutive
// time steps an MFMA operand needs.  Wave w owns 16*NTW state columns n;
// inside a wave the MFMA row m of n-tile nt stands for
//     n = n0 + 4*NTW*(m/4) + 4*nt + m%4,
// so every lane ends up holding 4*NTW consecutive n of one row p and stores
// them with 16-byte writes.
//
// float32 path: one thread per state entry, plain FMA loop over the chunk.
#include "common.h"
#include "launch.h"

namespace m2 {

namespace {

constexpr int kJB = 64;    // time steps staged per block
constexpr int kXPad = 8;   // LDS row padding (elements)
constexpr int kBPad = 8;

// N is any multiple of 16: the waves cover Npad columns (N rounded up to the
// waves' 16 NTW-column tiles); B columns past N are zero in LDS and their
// state columns are not stored.
template <int P, int NTW>
__global__ void __launch_bounds__(1024) chunk_state_bf16_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ Bm, const float* __restrict__ dA_cs,
    const float* __restrict__ dt_T, float* __restrict__ states, int L, int H, int G, int N,
    int Npad, int Q, int nc) {
  constexpr int PT = P / 16;
  constexpr int XS = P + kXPad;  // LDS row stride of Xs (elements)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int BS = Npad + kBPad;
  bf16* Xs = (bf16*)smem;                  // [kJB][XS]
  bf16* Bs = Xs + kJB * XS;                // [kJB][BS]
  float* wq = (float*)(Bs + kJB * BS);     // [Q]

  const int bid = blockIdx.x;              // (b, c, h) with h fastest
  const int h = bid % H;
  const int c = (bid / H) % nc;
  const int b = bid / (H * nc);
  const int g = h / (H / G);
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = lane_id();
  const int w = wave_id();
  const int L16 = lane & 15, grp = lane >> 4;
  const int n0 = w * 16 * NTW;

  const int64_t cbase = ((int64_t)b * H + h) * nc + c;
  const float* cs = dA_cs + cbase * Q;
  const float* dtc = dt_T + cbase * Q;
  const float cs_last = cs[Q - 1];
  for (int j = tid; j < Q; j += nthr) wq[j] = fast_exp2(cs_last - cs[j]) * dtc[j];

  f32x4 acc[NTW][PT];
#pragma unroll
  for (int a = 0; a < NTW; ++a)
#pragma unroll
    for (int q = 0; q < PT; ++q) acc[a][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t t0 = (int64_t)c * Q;
  for (int jb = 0; jb < Q; jb += kJB) {
    __syncthreads();  // wq ready / previous block consumed
    // Stage w-scaled x rows: kJB x P, 8 elements per 16-byte chunk.
    for (int idx = tid; idx < kJB * (P / 8); idx += nthr) {
      const int r = idx / (P / 8), c8 = (idx % (P / 8)) * 8;
      const int64_t t = t0 + jb + r;
      bf16x8 v;
      if (t < L) {
        const bf16x8 raw = *(const bf16x8*)(x + ((((int64_t)b * L + t) * H + h) * P + c8));
        const float s = wq[jb + r];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = f2bf(bf2f(raw[e]) * s);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = f2bf(0.f);
      }
      *(bf16x8*)(Xs + r * XS + c8) = v;
    }
    // Stage B rows: kJB x Npad (zero past N).
    const int nch = Npad / 8;
    for (int idx = tid; idx < kJB * nch; idx += nthr) {
      const int r = idx / nch, c8 = (idx % nch) * 8;
      const int64_t t = t0 + jb + r;
      bf16x8 v;
      if (t < L && c8 < N) {
        v = *(const bf16x8*)(Bm + ((((int64_t)b * L + t) * G + g) * N + c8));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = f2bf(0.f);
      }
      *(bf16x8*)(Bs + r * BS + c8) = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kJB / 32; ++kk) {
      const int k0 = kk * 32 + grp * 8 + (L16 >> 2);
      bf16x8 aop[NTW], bop[PT];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const bf16* p0 = Bs + k0 * BS + n0 + 4 * NTW * (L16 & 3) + 4 * nt;
        aop[nt] = cat(lds_read_tr(p0), lds_read_tr(p0 + 4 * BS));
      }
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const bf16* p0 = Xs + k0 * XS + 16 * pt + 4 * (L16 & 3);
        bop[pt] = cat(lds_read_tr(p0), lds_read_tr(p0 + 4 * XS));
      }
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[nt][pt] = mfma16x16x32(aop[nt], bop[pt], acc[nt][pt]);
    }
  }

  // acc[nt][pt][r] = S[p = 16 pt + L16][n = n0 + 4 NTW grp + 4 nt + r]
  float* out = states + (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
  const int nl = n0 + 4 * NTW * grp;
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) {
    float* row = out + (int64_t)(16 * pt + L16) * N + nl;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
      if (nl + 4 * nt < N) *(f32x4*)(row + 4 * nt) = acc[nt][pt];
  }
}

// float32: one thread per (b, c, h, p, n).
__global__ void __launch_bounds__(256) chunk_state_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ Bm, const float* __restrict__ dA_cs,
    const float* __restrict__ dt_T, float* __restrict__ states, int64_t total, int L, int H,
    int G, int P, int N, int Q, int nc) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int n = (int)(gid % N);
  const int p = (int)((gid / N) % P);
  const int64_t bch = gid / ((int64_t)P * N);  // ((b * nc + c) * H + h)
  const int h = (int)(bch % H);
  const int c = (int)((bch / H) % nc);
  const int b = (int)(bch / ((int64_t)H * nc));
  const int g = h / (H / G);
  const int64_t cbase = ((int64_t)b * H + h) * nc + c;
  const float* cs = dA_cs + cbase * Q;
  const float* dtc = dt_T + cbase * Q;
  const float cs_last = cs[Q - 1];
  float acc = 0.f;
  for (int j = 0; j < Q; ++j) {
    const int64_t t = (int64_t)c * Q + j;
    if (t >= L) break;
    const float wj = exp2f(cs_last - cs[j]) * dtc[j];
    acc += wj * x[(((int64_t)b * L + t) * H + h) * P + p] * Bm[(((int64_t)b * L + t) * G + g) * N + n];
  }
  states[gid] = acc;
}

// The same float32 arithmetic, in the same order, with one workgroup per
// (b, c, h): the chunk's x and B rows and the row weights w_j are staged in
// LDS once, where they fit, instead of being reloaded by every thread.
__global__ void __launch_bounds__(256) chunk_state_f32_lds_kernel(
    const float* __restrict__ x, const float* __restrict__ Bm, const float* __restrict__ dA_cs,
    const float* __restrict__ dt_T, float* __restrict__ states, int L, int H, int G, int P,
    int N, int Q, int nc) {
  extern __shared__ float sm[];
  float* Xs = sm;            // [Q][P]
  float* Bs = Xs + Q * P;    // [Q][N]
  float* ws = Bs + Q * N;    // [Q]
  const int h = blockIdx.x % H;
  const int c = (blockIdx.x / H) % nc;
  const int b = blockIdx.x / (H * nc);
  const int g = h / (H / G);
  const int64_t tok0 = (int64_t)c * Q;
  const int valid = (int)min((int64_t)Q, (int64_t)L - tok0);
  const int tid = threadIdx.x;
  for (int idx = tid; idx < valid * P; idx += blockDim.x) {
    const int r = idx / P, p = idx % P;
    Xs[idx] = x[(((int64_t)b * L + tok0 + r) * H + h) * P + p];
  }
  for (int idx = tid; idx < valid * N; idx += blockDim.x) {
    const int r = idx / N, n = idx % N;
    Bs[idx] = Bm[(((int64_t)b * L + tok0 + r) * G + g) * N + n];
  }
  const int64_t cbase = (((int64_t)b * H + h) * nc + c) * Q;
  const float cs_last = dA_cs[cbase + Q - 1];
  for (int j = tid; j < valid; j += blockDim.x)
    ws[j] = exp2f(cs_last - dA_cs[cbase + j]) * dt_T[cbase + j];
  __syncthreads();
  float* out = states + (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
  for (int o = tid; o < P * N; o += blockDim.x) {
    const int p = o / N, n = o % N;
    float acc = 0.f;
    for (int j = 0; j < valid; ++j) acc += ws[j] * Xs[j * P + p] * Bs[j * N + n];
    out[o] = acc;
  }
}

// LDS bytes the staged float32 kernel needs, if it fits in 64 KB (else 0).
size_t f32_state_lds_bytes(const Dims& d) {
  const int64_t n = d.Q * d.P + d.Q * d.N + d.Q;
  return n * 4 <= 64 * 1024 ? (size_t)n * 4 : 0;
}

template <int P, int NTW>
hipError_t launch_bf16(const Dims& d, const void* x, const void* B, const float* dA_cs,
                       const float* dt_T, float* states, hipStream_t s) {
  const int64_t cols = 16 * NTW;  // state columns per wave
  const int64_t npad = (d.N + cols - 1) / cols * cols;
  const int threads = (int)(64 * (npad / cols));
  if (threads > 1024) return hipErrorInvalidValue;
  const size_t lds = (size_t)kJB * (P + kXPad) * 2 + (size_t)kJB * (npad + kBPad) * 2 +
                     (size_t)d.Q * 4;
  auto kern = chunk_state_bf16_kernel<P, NTW>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  kern<<<(unsigned)(d.B * d.nc * d.H), threads, lds, s>>>(
      (const bf16*)x, (const bf16*)B, dA_cs, dt_T, states, (int)d.L, (int)d.H, (int)d.G,
      (int)d.N, (int)npad, (int)d.Q, (int)d.nc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_state(const Dims& d, const void* x, const void* B, const float* dA_cs,
                              const float* dt_T, float* states, hipStream_t s) {
  if (d.bf16) {
    // 4 column tiles per wave up to headdim 64, 2 above (accumulators NTW x P/16)
    switch (d.P) {
      case 16: return launch_bf16<16, 4>(d, x, B, dA_cs, dt_T, states, s);
      case 32: return launch_bf16<32, 4>(d, x, B, dA_cs, dt_T, states, s);
      case 48: return launch_bf16<48, 4>(d, x, B, dA_cs, dt_T, states, s);
      case 64: return launch_bf16<64, 4>(d, x, B, dA_cs, dt_T, states, s);
      case 80: return launch_bf16<80, 2>(d, x, B, dA_cs, dt_T, states, s);
      case 96: return launch_bf16<96, 2>(d, x, B, dA_cs, dt_T, states, s);
      case 112: return launch_bf16<112, 2>(d, x, B, dA_cs, dt_T, states, s);
      case 128: return launch_bf16<128, 2>(d, x, B, dA_cs, dt_T, states, s);
      default: return hipErrorInvalidValue;
    }
  }
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)chunk_state_f32_lds_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
      64 * 1024);
  if (const size_t lds = attr == hipSuccess ? f32_state_lds_bytes(d) : 0) {
    chunk_state_f32_lds_kernel<<<(unsigned)(d.B * d.nc * d.H), 256, lds, s>>>(
        (const float*)x, (const float*)B, dA_cs, dt_T, states, (int)d.L, (int)d.H, (int)d.G,
        (int)d.P, (int)d.N, (int)d.Q, (int)d.nc);
    return hipGetLastError();
  }
  const int64_t total = d.B * d.nc * d.H * d.P * d.N;
  chunk_state_f32_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
      (const float*)x, (const float*)B, dA_cs, dt_T, states, total, (int)d.L, (int)d.H,
      (int)d.G, (int)d.P, (int)d.N, (int)d.Q, (int)d.nc);
  return hipGetLastError();
}

}  // namespace m2
