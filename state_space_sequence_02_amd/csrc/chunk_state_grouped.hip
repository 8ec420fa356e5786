// chunk_state, grouped variant used by the fused forward pass.  Each chunk's
// state from a zero start is the jump formula's B X^T product with the rows
// of X pre-scaled by exponentials of the log-space cumulative sum
// (disconfirmai.com "Jane Street ML Engineers Map Mamba-2 Recurrent State
// Computation to Tensor Cores with cuTile", body):
//     S[p, n] = sum_j w_j x[j, p] B[j, n],   w_j = 2^(cs[Q-1] - cs[j]) dt_j.
// B depends only on the (batch, chunk, group), so one workgroup serves a run
// of that group's heads: its B^T operands are read once (through LDS, with
// the gfx950 transpose read) and stay in registers for every head.  Per head
// only x moves: it arrives by direct-to-LDS loads into a double buffer
// (head k+1 lands while head k computes), is scaled by w_j in place, and is
// read as the MFMA B operand with the transpose read.  The float32 result,
// the kernel's dominant traffic, leaves as 16-byte stores issued after the
// next head's bytes have been waited for, so they drain during the next
// head's work.
//
// The same kernel forms the adjoint chunk states of the backward pass (ADJ):
//     E[p, n] = sum_i 2^cs[i] dy[i, p] C[i, n]
// the gradient that chunk's outputs send back into its start state, from the
// state term y_i += 2^cs[i] (h C_i) of the forward pass; only the row weights
// differ (rows past the sequence end weigh 0).
//
// State size 512 runs as two launches over halves of the state columns (each
// column of S depends only on the same column of B): each launch holds 256
// columns of B^T operands, the register budget of state size 256, and
// writes its half of every row of the [.., P, 512] states.
//
// Layout: N/32 waves; wave w owns the 32 state columns n0 = 32 w .. 32 w + 31
// as NTW = 2 MFMA tiles, MFMA row m of tile nt standing for
// n = n0 + 4 NTW (m/4) + 4 nt + m%4, so each lane stores 4 NTW consecutive n
// of one row p.
#include "common.h"
#include "launch.h"

namespace m2 {

namespace {

template <int P, int Q, int N>
struct SCfg {
  static constexpr int NTW = 2, NW = N / (16 * NTW), NT = 64 * NW, PT = P / 16, KS = Q / 32;
  // Workgroups per CU the register budget is sized for: one 8-wave workgroup
  // (its B^T operands need ~140 VGPRs per lane), else two.
  static constexpr int OCC = NW >= 8 ? 1 : 2;
  static constexpr int WPE = (OCC * NW + 3) / 4;
  static constexpr int XS_BYTES = Q * P * 2;
  static constexpr int CS_BYTES = Q * 4;
  static constexpr int BUF = XS_BYTES + 2 * CS_BYTES;
  static constexpr int BROW = N + 8;              // staging row stride (elements)
  static constexpr int STG = 64 * BROW * 2;       // 64 rows of B per staging pass
  static constexpr int LDS = BUF + (BUF > STG ? BUF : STG);
  static_assert(P == 64, "grouped chunk_state is specialised for headdim 64");
  static_assert(N == 64 || N == 128 || N == 256, "state size must be 64, 128 or 256");
};

// Position of 16-byte chunk c in x row r (8 chunks per row); an involution.
__device__ __forceinline__ int xswz(int r, int c) { return c ^ (r & 7); }

template <int P, int Q, int N>
__device__ __forceinline__ void load_x(uint32_t buf, const bf16* __restrict__ x,
                                       const float* __restrict__ dA_cs,
                                       const float* __restrict__ dt_T, int b, int c, int h,
                                       int L, int H, int nc) {
  using K = SCfg<P, Q, N>;
  const int lane = lane_id();
  const int w = wave_id();
  constexpr int XI = Q / 8 / K::NW;  // wave-loads of 8 rows (1 KB) per wave
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int k = w + K::NW * i;
    const int s = k * 64 + lane;
    const int r = s >> 3, pos = s & 7;
    int64_t t = (int64_t)c * Q + r;
    if (t > L - 1) t = L - 1;  // rows past L get w = 0 below
    dma16(x + (((int64_t)b * L + t) * H + h) * P + xswz(r, pos) * 8, buf + k * 1024);
  }
  const uint32_t cs = buf + K::XS_BYTES;
  const int64_t cb = (((int64_t)b * H + h) * nc + c) * Q;
  if (w < 2 && lane < Q / 4) dma16((w == 0 ? dA_cs : dt_T) + cb + lane * 4, cs + w * K::CS_BYTES);
}

template <int P, int Q, int N, bool ADJ>
__global__ void __launch_bounds__((SCfg<P, Q, N>::NT), (SCfg<P, Q, N>::WPE)) chunk_state_grouped_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ Bm, const float* __restrict__ dA_cs,
    const float* __restrict__ dt_T, float* __restrict__ states, int L, int H, int G, int nc,
    int hpw, int slices, int ldn, int ncol0) {
  // rows of B and of the states hold ldn columns; this launch covers
  // columns ncol0 .. ncol0 + N - 1
  using K = SCfg<P, Q, N>;
  constexpr int NTW = K::NTW, PT = K::PT, KS = K::KS, BROW = K::BROW;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  bf16* Bs = (bf16*)(smem + K::BUF);  // staging aliases buffer 1

  int bid = blockIdx.x;
  const int slice = bid % slices;
  bid /= slices;
  const int g = bid % G;
  bid /= G;
  const int c = bid % nc;
  const int b = bid / nc;
  const int HG = H / G;
  const int h0 = g * HG + slice * hpw;
  const int nh = min(hpw, HG - slice * hpw);

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = wave_id();
  const int L16 = lane & 15, grp = lane >> 4;
  const int n0 = w * 16 * NTW;
  const int64_t tok0 = (int64_t)c * Q;

  // each workgroup walks its heads from a different one, so the workgroups
  // in flight touch different heads' slices of the token rows; the c / 8
  // term spreads the start heads of one XCD's chunks (c = XCD mod 8) too
  const int rot = nh > 0 ? (c + (c >> 3)) % nh : 0;
  const uint32_t sbase = lds_addr(smem);
  load_x<P, Q, N>(sbase, x, dA_cs, dt_T, b, c, h0 + rot, L, H, nc);

  // ---- Phase A: B^T operands of this wave's columns, 64 time steps at a time;
  // the rows pass through registers, block jb + 1's loads issued before
  // block jb's operand reads so that their latency overlaps.
  bf16x8 Bop[NTW][KS];
  constexpr int SIT = (64 * (N / 8) + K::NT - 1) / K::NT;  // 16-byte pieces per thread and block
  bf16x8 sv[SIT];
  auto stage_load = [&](int jb) {
#pragma unroll
    for (int it = 0; it < SIT; ++it) {
      const int idx = tid + it * K::NT;
      const int r = idx / (N / 8), c8 = (idx % (N / 8)) * 8;
      const int64_t t = tok0 + jb * 64 + r;
      if (idx < 64 * (N / 8) && t < L) {
        sv[it] = *(const bf16x8*)(Bm + (((int64_t)b * L + t) * G + g) * ldn + ncol0 + c8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[it][e] = f2bf(0.f);
      }
    }
  };
  stage_load(0);
#pragma unroll
  for (int jb = 0; jb < Q / 64; ++jb) {
    lds_barrier();
#pragma unroll
    for (int it = 0; it < SIT; ++it) {
      const int idx = tid + it * K::NT;
      if (idx < 64 * (N / 8)) {
        const int r = idx / (N / 8), c8 = (idx % (N / 8)) * 8;
        *(bf16x8*)(Bs + r * BROW + c8) = sv[it];
      }
    }
    if (jb + 1 < Q / 64) stage_load(jb + 1);
    lds_barrier();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int k0 = kk * 32 + grp * 8 + (L16 >> 2);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const bf16* p0 = Bs + k0 * BROW + n0 + 4 * NTW * (L16 & 3) + 4 * nt;
        Bop[nt][jb * 2 + kk] = cat(lds_read_tr(p0), lds_read_tr(p0 + 4 * BROW));
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();

  // ---- Phase B: heads.
  for (int k = 0; k < nh; ++k) {
    const int kr = k + rot < nh ? k + rot : k + rot - nh;
    const int h = h0 + kr;
    unsigned char* cur = smem + (k & 1) * K::BUF;
    if (k + 1 < nh)
      load_x<P, Q, N>(sbase + ((k + 1) & 1) * K::BUF, x, dA_cs, dt_T, b, c,
                      h0 + (kr + 1 < nh ? kr + 1 : kr + 1 - nh), L, H, nc);
    // Scale x rows by w_j in place (each 16-byte slot belongs to row s / 8).
    {
      const float* css = (const float*)(cur + K::XS_BYTES);
      const float* dts = css + Q;
      const float cs_last = css[Q - 1];
      // every read first, then every write: interleaved, each write would
      // order the next read behind it (one LDS round trip per slot)
      constexpr int NS = Q * 8 / K::NT;
      bf16x8 v[NS];
      float wr[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int s = tid + K::NT * i;
        const int r = s >> 3;
        v[i] = *(const bf16x8*)(cur + s * 16);
        if constexpr (ADJ)
          wr[i] = (tok0 + r < L) ? fast_exp2(css[r]) : 0.f;
        else
          wr[i] = fast_exp2(cs_last - css[r]) * dts[r];
      }
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = f2bf(bf2f(v[i][e]) * wr[i]);
        *(bf16x8*)(cur + (tid + K::NT * i) * 16) = o;
      }
    }
    lds_barrier();  // scaled x visible; next head's loads stay in flight
    f32x4 acc[NTW][PT];
#pragma unroll
    for (int a = 0; a < NTW; ++a)
#pragma unroll
      for (int q = 0; q < PT; ++q) acc[a][q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int ra = kk * 32 + grp * 8 + (L16 >> 2), rb = ra + 4;
      bf16x8 xop[PT];
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const int col = 16 * pt + 4 * (L16 & 3);
        const int ch = col >> 3, off = (col & 7) * 2;
        const bf16* pa = (const bf16*)(cur + ra * (P * 2) + (xswz(ra, ch) << 4) + off);
        const bf16* pb = (const bf16*)(cur + rb * (P * 2) + (xswz(rb, ch) << 4) + off);
        xop[pt] = cat(lds_read_tr(pa), lds_read_tr(pb));
      }
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[nt][pt] = mfma16x16x32(Bop[nt][kk], xop[pt], acc[nt][pt]);
    }
    __builtin_amdgcn_s_waitcnt(0);  // next head's x landed; older stores drained
    // acc[nt][pt][r] = S[p = 16 pt + L16][n = n0 + 4 NTW grp + 4 nt + r]
    float* out = states + (((int64_t)b * nc + c) * H + h) * (int64_t)P * ldn + ncol0;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      float* row = out + (int64_t)(16 * pt + L16) * ldn + n0 + 4 * NTW * grp;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) *(f32x4*)(row + 4 * nt) = acc[nt][pt];
    }
    lds_barrier();
  }
}

int cu_count_state() {
  static const int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    return v;
  }();
  return n;
}

template <int P, int Q, int N, bool ADJ>
hipError_t launch_grouped(const Dims& d, const void* x, const void* B, const float* dA_cs,
                          const float* dt_T, float* states, int ncol0, hipStream_t s) {
  using K = SCfg<P, Q, N>;
  auto kern = chunk_state_grouped_kernel<P, Q, N, ADJ>;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, K::LDS);
  if (attr != hipSuccess) return attr;
  // Enough workgroups to fill every CU at the intended occupancy, as many
  // heads per workgroup as that allows (B^T is read once per workgroup).
  const int64_t HG = d.H / d.G;
  int64_t hpw = (d.B * d.nc * d.H) / (K::OCC * cu_count_state());
  if (hpw < 1) hpw = 1;
  if (hpw > HG) hpw = HG;
  const int64_t slices = (HG + hpw - 1) / hpw;
  hpw = (HG + slices - 1) / slices;
  const int64_t grid = d.B * d.nc * d.G * slices;
  kern<<<(unsigned)grid, K::NT, K::LDS, s>>>((const bf16*)x, (const bf16*)B, dA_cs, dt_T, states,
                                           (int)d.L, (int)d.H, (int)d.G, (int)d.nc, (int)hpw,
                                           (int)slices, (int)d.N, ncol0);
  return hipGetLastError();
}

template <int Q, bool ADJ>
hipError_t launch_grouped_n(const Dims& d, const void* x, const void* B, const float* dA_cs,
                            const float* dt_T, float* states, hipStream_t s) {
  switch (d.N) {
    case 64: return launch_grouped<64, Q, 64, ADJ>(d, x, B, dA_cs, dt_T, states, 0, s);
    case 128: return launch_grouped<64, Q, 128, ADJ>(d, x, B, dA_cs, dt_T, states, 0, s);
    case 256: return launch_grouped<64, Q, 256, ADJ>(d, x, B, dA_cs, dt_T, states, 0, s);
    case 512: {
      const hipError_t e = launch_grouped<64, Q, 256, ADJ>(d, x, B, dA_cs, dt_T, states, 0, s);
      if (e != hipSuccess) return e;
      return launch_grouped<64, Q, 256, ADJ>(d, x, B, dA_cs, dt_T, states, 256, s);
    }
    default: return hipErrorInvalidValue;
  }
}

template <bool ADJ>
hipError_t launch_grouped_q(const Dims& d, const void* x, const void* B, const float* dA_cs,
                            const float* dt_T, float* states, hipStream_t s) {
  switch (d.Q) {
    case 64: return launch_grouped_n<64, ADJ>(d, x, B, dA_cs, dt_T, states, s);
    case 128: return launch_grouped_n<128, ADJ>(d, x, B, dA_cs, dt_T, states, s);
    case 256: return launch_grouped_n<256, ADJ>(d, x, B, dA_cs, dt_T, states, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool grouped_state_supported(const Dims& d) {
  return d.bf16 && d.P == 64 && (d.N == 64 || d.N == 128 || d.N == 256 || d.N == 512) &&
         (d.Q == 64 || d.Q == 128 || d.Q == 256);
}

hipError_t launch_chunk_state_grouped(const Dims& d, const void* x, const void* B,
                                      const float* dA_cs, const float* dt_T, float* states,
                                      hipStream_t s) {
  return launch_grouped_q<false>(d, x, B, dA_cs, dt_T, states, s);
}

hipError_t launch_chunk_state_adjoint(const Dims& d, const void* dy, const void* C,
                                      const float* dA_cs, const float* dt_T, float* states,
                                      hipStream_t s) {
  return launch_grouped_q<true>(d, dy, C, dA_cs, dt_T, states, s);
}

}  // namespace m2
