// span_scan: the replay of fwd_pass_state over a span of chunks fused with
// compute_out, so that the chunk-start states are handed to the output
// contraction on chip and never reach memory (devotd.net news item on the
// Mamba-2 CUDA Tile forward-pass kernels, section 2: compute_out reads the
// state at each chunk start, and fusion keeps the intermediate matrix out of
// global memory; disconfirmai.com "Jane Street ML Engineers Map Mamba-2
// Recurrent State Computation to Tensor Cores with cuTile", body: the jump
// h <- decay h + B X^T with the rows of X pre-scaled by exponentials of the
// log-space cumulative sum).
//
// Used for state sizes 64 and 128.  One workgroup per (batch, span of K
// chunks, run of R heads of one B/C group) starts from the span's start
// state (float32, written by the jump across spans) and walks the span in
// blocks of 32 time steps.  For block
// b .. e of chunk c (cs: the chunk's cumulative sums in log2 units, cs[b-1]
// = 0 at the chunk start) and each head, with h the state after step b - 1:
//     y_i = 2^(cs_i - cs[b-1]) C_i . h
//         + sum_{b <= j <= i} (C_i . B_j) 2^(cs_i - cs_j) dt_j x_j + D x_i
//     h  <- 2^(cs_e - cs[b-1]) h + sum_{b <= j <= e} 2^(cs_e - cs_j) dt_j x_j (outer) B_j
// The exponents are differences within one block and never positive, so no
// factor overflows whatever the decay (the memoryless limit included).  The
// state is kept as 2^lam acc with one scalar lam per head: a block's decay
// adds to lam, and acc is rescaled only when lam would fall below -64.
//
// Work split: 8 waves; wave w holds p-tile w & 3 (16 rows of P = 64) of the
// whole state (all N columns) of HPW = R / 2 heads, so neither contraction
// needs a sum across waves:
//   * state tiles D[n, p] (float32 MFMA accumulators), MFMA row m of n-tile nt
//     standing for n = 32 (nt / 2) + 8 (m / 4) + 4 (nt % 2) + m % 4, so that a
//     lane's two accumulators of tiles 2k, 2k + 1 hold n = 32 k + 8 q .. + 7
//     (q = lane / 16): rounded to bfloat16 they are directly the A operand of
//     the carried-state product Y^T[p, i] += h[p, n] C[i, n], whose C operand
//     is a plain 16-byte row read;
//   * G^T[j, i] = B_j . C_i of the block (three 16 x 16 tiles on and below the
//     diagonal), formed by every wave from the same C operands, so the masked,
//     decayed weights never leave registers; their accumulator rows give the
//     in-chunk product's K order: element e of lane group q is step
//     j = 4 q + e (e < 4) or 16 + 4 q + (e - 4);
//   * x^T, read transposed in that K order, is the in-chunk A operand and,
//     scaled by the state weights in registers, the B operand of the state
//     update D[n, p] += B^T[n, j] (w x)[j, p].
// B, C, the heads' x rows, cumulative sums and dt of each block arrive by
// direct-to-LDS loads into a ring of NBUF buffers, NBUF - 1 blocks ahead;
// every vector memory operation in the loop is such a load or a y store, so
// each wave waits with exact counts (they retire in issue order) and one
// barrier per block orders the ring.  Workgroup ids place every run of a
// (batch, span, group) on one XCD, so the span's B and C rows reach that
// XCD's L2 once.
#include "common.h"
#include "launch.h"

namespace m2 {

namespace {

template <int Q, int N, int HPW>
struct ScanSpanCfg {
  static constexpr int P = 64, RB = 32, NW = 8, NT = 64 * NW;
  static constexpr int R = 2 * HPW;          // heads per workgroup
  static constexpr int NTL = N / 16;         // state n-tiles per head
  static constexpr int KS = N / 32;          // k-steps over the state columns
  static constexpr int XH = RB * P * 2;      // one head's x rows of a block (4 KB)
  static constexpr int XS = R * XH;
  static constexpr int BS = RB * N * 2;      // B rows of a block (C rows likewise)
  static constexpr int SM = 1024;            // per head 32 cumulative sums, then 32 dt
  static constexpr int BUF = XS + 2 * BS + SM;
  static constexpr int BPC = Q / RB;         // blocks per chunk
  static constexpr int XT = XS / 1024, BT = BS / 1024;
  static constexpr int TOT = XT + 2 * BT + 1;  // direct-to-LDS loads per block (workgroup)
  static constexpr int NJ = (TOT + NW - 1) / NW;  // most loads per wave per block
  static constexpr int STORES = 2 * HPW;     // y stores per wave per block
  // per wave, per head: a block's decay tables (96 floats), after the ring
  static constexpr int TABW = HPW * 96 * 4;
  static constexpr int TAB = NW * TABW;
  static constexpr int depth() {
    int nb = (160 * 1024 - TAB) / BUF;
    if (nb > 4) nb = 4;
    while (nb > 3 && NJ * (nb - 2) + STORES * (nb - 1) > 62) --nb;
    return nb;
  }
  static constexpr int NBUF = depth();
  static constexpr int LDS = NBUF * BUF + TAB;
  static_assert(HPW == 1 || HPW == 2, "heads per wave");
  static_assert(N == 64 || N == 128, "state size");
  static_assert(NBUF >= 3 && NJ * (NBUF - 2) + STORES * (NBUF - 1) <= 62, "ring depth");
  static_assert(Q % RB == 0 && BPC >= 2, "chunk size");
};

// 16-byte chunk positions inside LDS rows (involutions).  x rows hold 8
// chunks: the transposed x reads touch rows 4 q + d (d = 0..3) at two
// chunks, which (r & 7) spreads over distinct banks.  B and C rows hold N/8
// chunks and are read both along rows (16 consecutive rows, one chunk) and
// transposed (rows 4 q + d, four consecutive chunks): 4 (r % 4) + (r / 4) % 4
// takes 16 distinct values on 16 consecutive rows and, on rows 4 q + d, moves
// the four chunks of each row to their own group of four.
__device__ __forceinline__ int ss_x(int r, int c) { return c ^ (r & 7); }
template <int N>
__device__ __forceinline__ int ss_bc(int r, int c) {
  return c ^ ((4 * (r & 3) + ((r >> 2) & 3)) & (N / 8 - 1));
}

typedef float f32x8 __attribute__((ext_vector_type(8)));

// Eight floats to bfloat16 (round to nearest even).
__device__ __forceinline__ bf16x8 to_bf8(f32x4 lo, f32x4 hi) {
  const f32x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_convertvector(v, bf16x8);
}

// 16-byte direct-to-LDS load from a wave-uniform base plus this lane's
// 32-bit byte offset (saddr form: the base stays in scalar registers);
// otherwise as dma16.  A vector memory instruction that reads an SGPR a
// VALU instruction wrote needs 5 wait states in between (gfx9 hazard), and
// the compiler does not insert them ahead of inline asm: when it reloads a
// spilled base with v_readlane right before the load, the load would read
// a stale base.  The s_nop 4 provides them whatever precedes the load.
__device__ __forceinline__ void dma16_so(const void* base, uint32_t voff, uint32_t lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "{m0}"(m0)
               : "memory");
}

// Load slot plan: slot j of this wave is load k = j * NW + wave of every
// block.  x, B and C slots keep a wave-uniform block-0 base (scalar) and the
// lane's byte offset from it; the sums slot (cumulative sums on lanes q < 8,
// dt on the others: two arrays) keeps a full per-lane address.  Every slot
// moves by 32 time steps per block (cumulative sums and dt are
// time-contiguous across chunk boundaries in [nc][Q]).  Every load is issued
// by all 64 lanes (lanes past the run's heads load a duplicate into unused
// LDS), so a block costs each wave exactly `nj` vector memory operations.
template <int Q, int N, int HPW>
struct SpanScanLoads {
  using C = ScanSpanCfg<Q, N, HPW>;
  static constexpr int KSUM = C::XT + 2 * C::BT;  // the sums slot
  const char* base[C::NJ];
  uint32_t voff[C::NJ];
  const char* sum_ptr;
  int nj;

  // Slot k of a block: token row (within the block) and element offset
  // (within the token's row of x, B or C) of this lane's 16 bytes; kind 0 x,
  // 1 B, 2 C, 3 sums.
  __device__ __forceinline__ static int slot(int k, int lane, int h0, int g, int* row, int* col) {
    if (k < C::XT) {
      const int r = k >> 2, s = (k & 3) * 64 + lane;
      *row = s >> 3;
      *col = 8 * ss_x(*row, s & 7) + (h0 + r) * C::P;
      return 0;
    }
    if (k < KSUM) {
      const bool isC = k >= C::XT + C::BT;
      const int s = (k - C::XT - (isC ? C::BT : 0)) * 64 + lane;
      *row = s / (N / 8);
      *col = 8 * ss_bc<N>(*row, s % (N / 8)) + g * N;
      return isC ? 2 : 1;
    }
    *row = *col = 0;
    return 3;
  }
  __device__ __forceinline__ static uint32_t dst(int k) {
    if (k < C::XT) return (k >> 2) * C::XH + (k & 3) * 1024;
    if (k < KSUM) return C::XS + (k - C::XT) * 1024;  // B slots, then C slots
    return C::XS + 2 * C::BS;
  }
  __device__ __forceinline__ static int64_t stride(int k, int H, int G) {
    if (k < C::XT) return (int64_t)C::RB * H * C::P * 2;
    if (k < KSUM) return (int64_t)C::RB * G * N * 2;
    return (int64_t)C::RB * 4;
  }

  __device__ __forceinline__ void init(const bf16* x, const bf16* Bm, const bf16* Cm,
                                       const float* dA_cs, const float* dt_T, int c0, int b,
                                       int h0, int g, int L, int H, int G, int nc) {
    const int lane = lane_id();
    const int w = wave_id();
    const int64_t tok0 = (int64_t)c0 * Q;
    nj = 0;
    sum_ptr = (const char*)dA_cs;
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      const int k = j * C::NW + w;
      base[j] = (const char*)dA_cs;
      voff[j] = 0;
      if (k < C::TOT) nj = j + 1;
      if (k >= C::TOT) continue;
      int row, col, row0, col0;
      const int kind = slot(k, lane, h0, g, &row, &col);
      slot(k, 0, h0, g, &row0, &col0);  // lane 0: the uniform part
      if (kind == 0) {
        base[j] = (const char*)(x + ((int64_t)b * L + tok0) * H * C::P);
        voff[j] = (uint32_t)(((int64_t)row * H * C::P + col) * 2);
      } else if (kind != 3) {
        base[j] = (const char*)((kind == 2 ? Cm : Bm) + ((int64_t)b * L + tok0) * G * N);
        voff[j] = (uint32_t)(((int64_t)row * G * N + col) * 2);
      } else {
        const int r = lane >> 4, q = lane & 15;
        const int rr = r < C::R ? r : 0;
        const int64_t o = (((int64_t)b * H + h0 + rr) * nc + c0) * Q + 4 * (q & 7);
        sum_ptr = (const char*)((q < 8 ? dA_cs : dt_T) + o);
      }
    }
  }

  // Block i of the span (all rows inside the sequence).
  __device__ __forceinline__ void issue(uint32_t buf, int i, int H, int G) const {
    const int w = wave_id();
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      const int k = j * C::NW + w;
      if (j < nj) {
        if (k == KSUM)
          dma16(sum_ptr + i * stride(k, H, G), buf + dst(k));
        else
          dma16_so(base[j] + i * stride(k, H, G), voff[j], buf + dst(k));
      }
    }
  }

  // Block i whose rows reach past the sequence end: token rows clamped to
  // L - 1 (their dt is zero, so they carry no weight).
  __device__ __forceinline__ void issue_clamped(uint32_t buf, int i, const bf16* x,
                                                const bf16* Bm, const bf16* Cm, int c0, int b,
                                                int h0, int g, int L, int H, int G) const {
    const int lane = lane_id();
    const int w = wave_id();
    const int64_t tok0 = (int64_t)c0 * Q + (int64_t)i * C::RB;
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      if (j < nj) {
        const int k = j * C::NW + w;
        int row, col;
        const int kind = slot(k, lane, h0, g, &row, &col);
        int64_t t = tok0 + row;
        if (t > L - 1) t = L - 1;
        const char* src = kind == 0 ? (const char*)(x + ((int64_t)b * L + t) * H * C::P + col)
                        : kind == 1 ? (const char*)(Bm + ((int64_t)b * L + t) * G * N + col)
                        : kind == 2 ? (const char*)(Cm + ((int64_t)b * L + t) * G * N + col)
                                    : sum_ptr + i * stride(k, H, G);
        dma16(src, buf + dst(k));
      }
    }
  }
};

template <int Q, int N, int HPW>
__global__ void __launch_bounds__(512) span_scan_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ Bm, const bf16* __restrict__ Cm,
    const float* __restrict__ dA_cs, const float* __restrict__ dt_T,
    const float* __restrict__ span_states, const float* __restrict__ Dv, bf16* __restrict__ y,
    int L, int H, int G, int nc, int K, int ng, int BNGG) {
  using C = ScanSpanCfg<Q, N, HPW>;
  constexpr int R = C::R, NTL = C::NTL, KS = C::KS, N2 = 2 * N;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  // id = 8 r + xcd: every run of a (batch, span, group) on one XCD
  const int HG = H / G, RG = HG / R;
  const int xcd = blockIdx.x & 7, rq = blockIdx.x >> 3;
  const int run = rq % RG;
  const int bsg = (rq / RG) * 8 + xcd;
  if (bsg >= BNGG) return;
  const int g = bsg % G;
  const int b = bsg / G / ng, s = (bsg / G) % ng;
  const int h0 = g * HG + run * R;
  const int c0 = s * K, c1 = min(c0 + K, nc);
  const int nblk = (c1 - c0) * C::BPC;

  const int lane = lane_id();
  const int w = wave_id();
  const int L16 = lane & 15, q = lane >> 4;
  const int pt = w & 3;                  // this wave's 16 rows of P
  const int hs = (w >> 2) * HPW;         // its first head within the run
  const int p = 16 * pt + L16;

  // state tiles: acc[k][nt][e] = h[p][32 (nt / 2) + 8 q + 4 (nt % 2) + e]
  f32x4 acc[HPW][NTL];
  float Dh[HPW];
#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    const int h = h0 + hs + k;
    const float* sst = span_states + (((int64_t)b * ng + s) * H + h) * 64 * N + (int64_t)p * N;
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt)
      acc[k][nt] = *(const f32x4*)(sst + 32 * (nt >> 1) + 8 * q + 4 * (nt & 1));
    Dh[k] = Dv ? Dv[h] : 0.f;
  }
  __builtin_amdgcn_s_waitcnt(0);  // start states and D are in registers

  const uint32_t sbase = lds_addr(smem);
  SpanScanLoads<Q, N, HPW> ld;
  ld.init(x, Bm, Cm, dA_cs, dt_T, c0, b, h0, g, L, H, G, nc);
  // blocks from `nfull` on reach past the sequence end
  const int nfull = min(nblk, (int)(((int64_t)L - (int64_t)c0 * Q) / C::RB));
#pragma unroll
  for (int j = 0; j < C::NBUF - 1; ++j) {
    if (j < nfull)
      ld.issue(sbase + j * C::BUF, j, H, G);
    else if (j < nblk)
      ld.issue_clamped(sbase + j * C::BUF, j, x, Bm, Cm, c0, b, h0, g, L, H, G);
  }

  // Lane-constant LDS byte offsets inside a buffer.
  // C and B rows along the row (G^T and carried-state operands): row
  // 16 t + L16, chunk 4 k + q; the swizzle of row 16 t + L16 equals that of L16.
  const int rsw = (4 * (L16 & 3) + ((L16 >> 2) & 3)) & (N / 8 - 1);
  const int rrow = L16 * N2 + 16 * (q ^ (rsw & 3));
  // transposed B reads (state update): rows 4 q + (L16 / 4) and 16 + 4 q + (L16 / 4)
  const int trow = 4 * q + (L16 >> 2);
  const int tsw = (4 * (L16 >> 2) + q) & (N / 8 - 1);  // swizzle of both transposed rows
  const int trw = trow * N2 + 16 * ((L16 & 3) ^ (tsw & 3));
  // transposed x reads: same rows, p-tile chunk 2 pt + (L16 & 3) / 2
  const int xch = 2 * pt + ((L16 & 3) >> 1);
  const int xoff0 = trow * 128 + (ss_x(trow, xch) << 4) + 8 * (L16 & 1);
  const int xoff1 = (trow + 16) * 128 + (ss_x(trow + 16, xch) << 4) + 8 * (L16 & 1);

  // Per head: cs at the step before the block (0 at a chunk start), and the
  // state's scale: the state is 2^lam acc, so a block's decay adds to lam
  // instead of scaling every accumulator; acc is rescaled (lam back to 0)
  // only when lam would fall below -kLamMin, which bounds every factor below
  // by 2^kLamMin (acc and the weighted x stay far inside float32 and bfloat16).
  constexpr float kLamMin = 64.f;
  // this wave's decay tables, per head: XW[j] = 2^(cs_e - cs_j) dt_j and
  // YS[i] = 2^(cs_i - prev) for the block's 32 steps, then F[j] =
  // 2^(cs_15 - cs_j) dt_j (j < 16) and E[i] = 2^(cs_i - cs_15) (i >= 16), the
  // two factors of the off-diagonal G^T tile's weights.  Every exponent is a
  // difference of cumulative sums in time order, never positive, so no
  // factor overflows.  Formed by the wave's lanes once per block (two
  // exponentials each) instead of by every lane for its own steps.
  float* const tab = (float*)(smem + C::NBUF * C::BUF) + w * (HPW * 96);
  float prev[HPW], lam[HPW];
#pragma unroll
  for (int k = 0; k < HPW; ++k) prev[k] = lam[k] = 0.f;

  for (int i = 0; i < nblk; ++i) {
    const int jb = i % C::BPC;
    const int c = c0 + i / C::BPC;
    // operations issued after block i's loads: the loads of later blocks
    // already issued, and (if every block they belong to was full) the y
    // stores of the blocks since; counting fewer only waits longer
    int newer = ld.nj * (min(i + C::NBUF - 2, nblk - 1) - i);
    const int s0 = max(0, i - C::NBUF + 1);
    if (i - 1 < nfull) newer += C::STORES * (i - s0);
    asm volatile("" ::: "memory");
    wait_vm(newer);
    __builtin_amdgcn_s_barrier();  // block i landed for every wave; block i - 1 fully read
    asm volatile("" ::: "memory");
    if (i + C::NBUF - 1 < nblk) {
      const int jn = i + C::NBUF - 1;
      const uint32_t nb = sbase + (jn % C::NBUF) * C::BUF;
      if (jn < nfull)
        ld.issue(nb, jn, H, G);
      else
        ld.issue_clamped(nb, jn, x, Bm, Cm, c0, b, h0, g, L, H, G);
    }
    const unsigned char* cur = smem + (i % C::NBUF) * C::BUF;
    const unsigned char* Bs = cur + C::XS;
    const unsigned char* Cs = Bs + C::BS;
    const float* sums = (const float*)(Cs + C::BS);

    // ---- carried-state product and G^T over the state columns
    f32x4 Y[HPW][2], G00, G01, G11;
#pragma unroll
    for (int k = 0; k < HPW; ++k) Y[k][0] = Y[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    G00 = G01 = G11 = f32x4{0.f, 0.f, 0.f, 0.f};
    // C rows of both i-tiles along the row (16 bytes), one k-step ahead; the
    // B rows of both j-tiles read at their k-step
    // chunk (4 kk + q) ^ rsw = 4 ((kk % 4) ^ (rsw / 4)) + (q ^ rsw % 4) + 16 (kk / 4)
    // (rsw < 16): four lane offsets, the rest an immediate
    auto roff = [&](int kk) {
      return rrow + 64 * ((kk & 3) ^ ((rsw >> 2) & ((N / 32 - 1) & 3))) + 256 * (kk >> 2);
    };
    auto cops = [&](int kk, bf16x8 (&o)[2]) {
      o[0] = *(const bf16x8*)(Cs + roff(kk));
      o[1] = *(const bf16x8*)(Cs + 16 * N2 + roff(kk));
    };
    bf16x8 cr[2][2];
    cops(0, cr[0]);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if (kk + 1 < KS) cops(kk + 1, cr[(kk + 1) & 1]);
      const bf16x8(&o)[2] = cr[kk & 1];
      const bf16x8 b0 = *(const bf16x8*)(Bs + roff(kk));
      const bf16x8 b1 = *(const bf16x8*)(Bs + 16 * N2 + roff(kk));
#pragma unroll
      for (int k = 0; k < HPW; ++k) {
        const bf16x8 ha = to_bf8(acc[k][2 * kk], acc[k][2 * kk + 1]);
        Y[k][0] = mfma16x16x32(ha, o[0], Y[k][0]);
        Y[k][1] = mfma16x16x32(ha, o[1], Y[k][1]);
      }
      G00 = mfma16x16x32(b0, o[0], G00);
      G01 = mfma16x16x32(b0, o[1], G01);
      G11 = mfma16x16x32(b1, o[1], G11);
      // keep the next k-step's reads where they are (the scheduler would
      // otherwise hoist every read of the unrolled loop)
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- in-chunk term, skip term, y; then the weighted x rows
    const int64_t tok0 = (int64_t)c * Q + jb * C::RB;
    const int64_t valid = (int64_t)L - tok0;
    const bool update = i + 1 < nblk;  // the span's last block needs no state update
    bf16x8 wx[HPW];
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
      const float* cs = sums + (hs + k) * 64;
      const float* dt = cs + 32;
      const f32x4 csa = *(const f32x4*)(cs + 4 * q), csb = *(const f32x4*)(cs + 16 + 4 * q);
      const f32x4 dta = *(const f32x4*)(dt + 4 * q), dtb = *(const f32x4*)(dt + 16 + 4 * q);
      const float cse = cs[31];
      const float ci0 = cs[L16], ci1 = cs[16 + L16];
      float* const tb = tab + k * 96;
      {
        const int li = lane & 31;
        const bool lo = lane < 32, mid = !lo && lane < 48;
        const float c15 = cs[15], csl = cs[li];
        const float a0 = lo ? cse - csl : (mid ? c15 - csl : csl - c15);
        const float m0 = (lo || mid) ? dt[li] : 1.f;
        tb[lo ? li : 64 + li] = fast_exp2(a0) * m0;
        const float ys = fast_exp2(csl - prev[k]);
        if (lo) tb[32 + li] = ys;
      }
      const f32x4 xw0 = *(const f32x4*)(tb + 4 * q), xw1 = *(const f32x4*)(tb + 16 + 4 * q);
      const f32x4 f01 = *(const f32x4*)(tb + 64 + 4 * q);
      const float ys0 = tb[32 + L16], ys1 = tb[48 + L16], e01 = tb[80 + L16];
      // carried-state part: h = 2^lam acc, decayed from the step before the block
      const float sl = fast_exp2(lam[k]);
      Y[k][0] *= ys0 * sl;
      Y[k][1] *= ys1 * sl;
      // weights G^T[j, i] 2^(cs_i - cs_j) dt_j, causal mask, D on the
      // diagonal; this lane's steps are j = 4 q + e (i-tiles 0 and 1) and
      // 16 + 4 q + e (i-tile 1).  Inside the diagonal tiles the exponent is
      // formed per element (never positive where the mask keeps it); the
      // off-diagonal tile takes E[i] F[j].
      f32x4 w0a, w1a, w1b;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 4 * q + e;
        float v0 = j <= L16 ? G00[e] * (fast_exp2(ci0 - csa[e]) * dta[e]) : 0.f;
        if (j == L16) v0 += Dh[k];
        w0a[e] = v0;
        w1a[e] = G01[e] * (e01 * f01[e]);
        float v1 = j <= L16 ? G11[e] * (fast_exp2(ci1 - csb[e]) * dtb[e]) : 0.f;
        if (j == L16) v1 += Dh[k];
        w1b[e] = v1;
      }
      const unsigned char* xs = cur + (hs + k) * C::XH;
      const bf16x8 xop = cat(lds_read_tr((const bf16*)(xs + xoff0)),
                             lds_read_tr((const bf16*)(xs + xoff1)));
      const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
      Y[k][0] = mfma16x16x32(xop, to_bf8(w0a, zero), Y[k][0]);
      Y[k][1] = mfma16x16x32(xop, to_bf8(w1a, w1b), Y[k][1]);
      // y rows of this block: the lane holds token 16 it + L16, p = 16 pt + 4 q .. + 3
      const int h = h0 + hs + k;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int ii = 16 * it + L16;
        if (ii < valid) {
          const bf16x8 o8 = to_bf8(Y[k][it], zero);
          *(bf16x4*)(y + (((int64_t)b * L + tok0 + ii) * H + h) * 64 + 16 * pt + 4 * q) =
              __builtin_shufflevector(o8, o8, 0, 1, 2, 3);
        }
      }
      // the block's decay joins the scale; the weighted x rows (the state
      // update's B operand, same K order) carry 2^(cs_e - cs_j - lam) dt_j
      float lnew = lam[k] + (cse - prev[k]);
      if (update && lnew < -kLamMin) {  // wave-uniform: rescale to lam = 0
        const float r = fast_exp2(lnew);
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) acc[k][nt] *= r;
        lnew = 0.f;
      }
      lam[k] = lnew;
      const float sx = fast_exp2(-lnew);
      f32x4 xa, xb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xa[e] = bf2f(xop[e]) * (xw0[e] * sx);
        xb[e] = bf2f(xop[4 + e]) * (xw1[e] * sx);
      }
      wx[k] = to_bf8(xa, xb);
      prev[k] = jb == C::BPC - 1 ? 0.f : cse;
    }

    // ---- state update: acc[n, p] += B^T[n, j] (w x)[j, p] 2^-lam
    if (update) {
      // chunk (4 a + L16 % 4) ^ tsw, a = nt / 2: four lane offsets by a % 4,
      // the rest an immediate
      auto bt_at = [&](int nt) {
        const int a = nt >> 1;
        const int off = trw + 64 * ((a & 3) ^ ((tsw >> 2) & ((N / 32 - 1) & 3))) + 256 * (a >> 2) +
                        8 * (nt & 1);
        return cat(lds_read_tr((const bf16*)(Bs + off)),
                   lds_read_tr((const bf16*)(Bs + 16 * N2 + off)));
      };
      bf16x8 bt[2];
      bt[0] = bt_at(0);
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt) {
        if (nt + 1 < NTL) bt[(nt + 1) & 1] = bt_at(nt + 1);
#pragma unroll
        for (int k = 0; k < HPW; ++k) acc[k][nt] = mfma16x16x32(bt[nt & 1], wx[k], acc[k][nt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

int cu_count_scan() {
  static const int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    return v;
  }();
  return n;
}

template <int Q, int N, int HPW>
hipError_t launch_ss(const Dims& d, int K, const void* x, const void* B, const void* C,
                     const float* dA_cs, const float* dt_T, const float* span_states,
                     const float* D, void* y, hipStream_t s) {
  using Cf = ScanSpanCfg<Q, N, HPW>;
  auto kern = span_scan_kernel<Q, N, HPW>;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, Cf::LDS);
  if (attr != hipSuccess) return attr;
  const int64_t ng = (d.nc + K - 1) / K;
  const int64_t BNGG = d.B * ng * d.G;
  const int64_t grid = (BNGG + 7) / 8 * 8 * (d.H / d.G / Cf::R);
  kern<<<(unsigned)grid, Cf::NT, Cf::LDS, s>>>(
      (const bf16*)x, (const bf16*)B, (const bf16*)C, dA_cs, dt_T, span_states, D, (bf16*)y,
      (int)d.L, (int)d.H, (int)d.G, (int)d.nc, K, (int)ng, (int)BNGG);
  return hipGetLastError();
}

template <int HPW>
hipError_t launch_ss_qn(const Dims& d, int K, const void* x, const void* B, const void* C,
                        const float* dA_cs, const float* dt_T, const float* span_states,
                        const float* D, void* y, hipStream_t s) {
#define M2_SS(QQ, NN)                                                                      \
  if (d.Q == QQ && d.N == NN)                                                              \
    return launch_ss<QQ, NN, HPW>(d, K, x, B, C, dA_cs, dt_T, span_states, D, y, s);
  M2_SS(64, 64) M2_SS(128, 64) M2_SS(256, 64)
  M2_SS(64, 128) M2_SS(128, 128) M2_SS(256, 128)
#undef M2_SS
  return hipErrorInvalidValue;
}

}  // namespace

int span_scan_heads(const Dims& d, int K) {
  // State size 256 is not taken.  With one head per wave every wave reads the
  // block's whole B and C rows for a single head (about 6 KB of LDS reads per
  // token and head against 2.4 KB for the replay plus the grouped chunk_scan),
  // and it measured slower than those two kernels (400 us against 354 us at
  // L = 64K).  Two heads per wave (four per workgroup) fill all 256 registers
  // and measured slower still (442 us against 355 us).
  if (!(d.bf16 && d.P == 64 && (d.N == 64 || d.N == 128) &&
        (d.Q == 64 || d.Q == 128 || d.Q == 256) && K > 0))
    return 0;
  const int64_t HG = d.H / d.G, ng = (d.nc + K - 1) / K;
  // four heads per workgroup (two per wave) where that still gives every CU
  // a workgroup, else two; an odd number of heads per group is not covered
  if (HG % 4 == 0 && d.B * ng * d.H / 4 >= cu_count_scan()) return 4;
  if (HG % 2 == 0) return 2;
  return 0;
}

int span_scan_chunks(const Dims& d) {
  // At state size 64 span_scan carries most of the step, so its grid
  // decides: the longest span (8, 4 or 2 chunks) whose span_scan grid
  // still gives every CU a workgroup (L = 8K, H = 32: spans of 2 instead of
  // 4, twice the workgroups, 0.103 -> 0.068 ms per step).  0 elsewhere, and
  // where no span length does (span_end's rule, span_chunks, then decides).
  // At state size 128 the same rule measured no faster (L = 8K: 0.1106 ->
  // 0.1113 ms; span_scan's throughput there did not grow with its grid),
  // nor did spans of one chunk in place of the split path (L = 4K, N = 64:
  // 0.0433 -> 0.0437 ms).
  if (!(d.bf16 && d.P == 64 && d.N == 64 && (d.Q == 64 || d.Q == 128 || d.Q == 256)))
    return 0;
  const int64_t HG = d.H / d.G;
  if (HG % 2 != 0) return 0;
  const int64_t cus = cu_count_scan();
  for (int K = 8; K >= 2; K /= 2) {
    if (d.nc < K) continue;
    const int64_t ng = (d.nc + K - 1) / K;
    const int64_t R = (HG % 4 == 0 && d.B * ng * d.H / 4 >= cus) ? 4 : 2;
    if (d.B * ng * d.H / R >= cus) return K;
  }
  return 0;
}

hipError_t launch_span_scan(const Dims& d, int K, int R, const void* x, const void* B,
                            const void* C, const float* dA_cs, const float* dt_T,
                            const float* span_states, const float* D, void* y, hipStream_t s) {
  switch (R) {
    case 2: return launch_ss_qn<1>(d, K, x, B, C, dA_cs, dt_T, span_states, D, y, s);
    case 4: return launch_ss_qn<2>(d, K, x, B, C, dA_cs, dt_T, span_states, D, y, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace m2
