// fwd_pass_state over spans of chunks: the decayed jump (devotd.net news item
// on the Mamba-2 CUDA Tile forward-pass kernels, section 2: fwd_pass_state
// yields the state at every chunk start and after the last chunk, keeping
// chunk order while independent parts of the state run in parallel;
// disconfirmai.com "Jane Street ML Engineers Map Mamba-2 Recurrent State
// Computation to Tensor Cores with cuTile", body: the jump formula, B X^T with
// the rows of X pre-scaled by exponentials of the log-space cumulative sum)
// applied span by span, so that the float32 per-chunk states never reach
// memory.
//
// The chunks of a sequence are cut into spans of K consecutive chunks.
//   1. span_end (this file, REPLAY = false): per (batch, span, head), the
//      state after the span from a zero start, walking the span's chunks in
//      order with the running state in float32 MFMA accumulators:
//          run = 2^(cs_c[Q-1]) run + sum_j w_j x_j (outer) B_j,
//          w_j = 2^(cs_c[Q-1] - cs_c[j]) dt_j,
//      and the span's log2 decay, the sum of its chunks' cs_c[Q-1].
//   2. span_passing: the same jump across spans (state_passing with spans
//      for chunks): the state at every span start, and the final state.
//   3. span_replay (REPLAY = true): per (batch, span, head), the span walked
//      again from its start state, writing the bfloat16 state at every chunk
//      start.  The span's last chunk needs no contraction.
// Per chunk and head this moves x twice and the bfloat16 start state once,
// where chunk_state + state_passing write and re-read a float32 state.
//
// Work split of steps 1 and 3: one workgroup per (batch, span, run of R
// heads of one group) holding those heads' whole P x N states: N/32 waves,
// wave w owning the 32 state columns 32 w .. 32 w + 31 for all P = 64 rows
// as 2 x 4 MFMA tiles per head (D[n, p] += B^T[n, j] (w x)[j, p]).  The run's
// heads share every B row.  Per block of 32 time steps, the B rows, the R
// heads' x rows and their cumulative sums and dt arrive by direct-to-LDS
// loads into a ring of NBUF buffers, NBUF - 1 blocks ahead of use: B rows are
// four times as wide as x rows (N = 256), so only a deep ring keeps enough
// bytes in flight per CU.  x is scaled by w_j in place and both operands are
// read back with the transpose read.  Every vector memory operation in the
// loop is a direct-to-LDS load or a store, so each wave waits with exact
// counts (vector memory operations retire in issue order).  Workgroup ids
// place every run of a (batch, span, group) on one XCD (id % 8), so the
// span's B rows are fetched into that XCD's L2 once.
#include "common.h"
#include "launch.h"

namespace m2 {

namespace {

// Most heads per workgroup, and workgroups per CU the LDS ring and the
// register budget are sized for by default.
constexpr int kSpanHeads = 4;
constexpr int kSpanOcc = 1;

template <int Q, int N, int R, int OCCT = kSpanOcc>
struct SpanCfg {
  static constexpr int P = 64, RB = 32, NW = N / 32, NT = 64 * NW, PT = P / 16;
  static constexpr int XH = RB * P * 2;      // one head's x rows of a block (4 KB)
  static constexpr int XS = R * XH;
  static constexpr int BS = RB * N * 2;      // B rows of a block, 2N bytes each
  static constexpr int CS = 1024;            // per head: 32 cumulative sums, 32 dt
  // per head (16 bytes each): cs[Q-4 .. Q-1] of the block's chunk; sized for
  // all 64 lanes of its load, so that load needs no lane mask
  static constexpr int CL = 1024;
  static constexpr int BUF = XS + BS + CS + CL;
  // workgroups per CU: the target, if two buffers each still fit
  static constexpr int OCC = (160 * 1024 / (2 * BUF)) < OCCT ? (160 * 1024 / (2 * BUF)) : OCCT;
  static constexpr int WPE = (OCC * NW + 3) / 4;  // waves per SIMD to fit
  static constexpr int BPC = Q / RB;         // blocks per chunk
  static constexpr int XT = XS / 1024, BT = BS / 1024;
  static constexpr int TOT = XT + BT + 2;    // direct-to-LDS loads per block (workgroup)
  // Ring depth: as many buffers as LDS holds (at most 8) while a wave's
  // outstanding operations (the loads of NBUF - 2 later blocks and the
  // start-state stores since) still fit the counter's wait field.
  static constexpr int newest(int nb) {
    return (TOT + NW - 1) / NW * (nb - 2) + 4 * R * ((nb - 1 + BPC - 1) / BPC);
  }
  static constexpr int depth() {
    int nb = (160 * 1024 / OCC / BUF) < 8 ? (160 * 1024 / OCC / BUF) : 8;
    while (nb > 2 && newest(nb) > 62) --nb;
    return nb;
  }
  static constexpr int NBUF = depth();
  static constexpr int LDS = NBUF * BUF;
  static constexpr int SLOTS = XS / 16;      // 16-byte x slots of a block
  static_assert(R == 1 || R == 2 || R == 4, "heads per workgroup");
  static_assert(NBUF >= 2 && newest(NBUF) <= 62, "ring depth");
  static_assert(Q % RB == 0 && BPC >= 2, "chunk size");
};

// 16-byte chunk positions inside LDS rows (involutions).  The LDS has 64
// banks of 4 bytes and serves an 8-byte (transposed) read 32 lanes at a
// time, so those 32 lanes must address 32 distinct 8-byte bank slots.  x rows
// hold 8 chunks: a transposed read of x touches rows 8 g + d (+ 4), d =
// 0..3, g = 0, 1, at two chunks, both halves; (r & 7) places them on 32
// distinct slots.  B rows hold N/8 chunks: a transposed read of B touches the
// same rows at one pair of chunks (both halves of each); the pair moves by an
// even amount distinct for each of those 8 rows (2 (r % 4) + 8 ((r / 8) % 2)),
// or, with 8 chunks per row (N = 64, where odd and even rows already fall on
// different halves of the bank period), by 2 ((r / 2) % 2) + 4 ((r / 8) % 2).
__device__ __forceinline__ int sx(int r, int c) { return c ^ (r & 7); }
// That needs each B tile to hold 16 consecutive state columns (ALT), which
// leaves a lane's accumulators of the two tiles 16 columns apart, so the
// replay, which stores a bfloat16 state at every chunk start, keeps tiles of
// interleaved columns instead (8 contiguous columns per lane, one 16-byte
// store) at the price of 2-way conflicted B reads: all lanes read the same
// half of their chunks, and (4 (r % 4)) spreads the rows over 16 chunks.
template <int N, bool ALT>
__device__ __forceinline__ int sb(int r, int c) {
  if constexpr (!ALT) return c ^ (((r & 3) << 2) & (N / 8 - 1));
  if constexpr (N == 64) return c ^ (2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1));
  return c ^ ((2 * (r & 3) + 8 * ((r >> 3) & 1)) & (N / 8 - 1));
}
// Column of accumulator (nt, e) of lane group grp within a wave's 32-column
// group: ALT tiles 16 nt + 4 grp + e, else 8 grp + 4 nt + e.
template <bool ALT>
__device__ __forceinline__ int acc_col(int nt, int grp) {
  return ALT ? 16 * nt + 4 * grp : 8 * grp + 4 * nt;
}

// Direct-to-LDS loads of block `blk` (time steps tok0 .. tok0 + 31 of chunk
// c) into buffer `buf` (an LDS byte address): load k of the block goes to
// wave k % NW.  Rows past L are clamped to L - 1: their weight is 0 (dt is
// zero-padded).
template <int Q, int N, int R, int LDN, bool ALT>
__device__ __forceinline__ void issue_block(uint32_t buf, const bf16* __restrict__ x,
                                            const bf16* __restrict__ Bm,
                                            const float* __restrict__ dA_cs,
                                            const float* __restrict__ dt_T, int c, int jb, int b,
                                            int h0, int g, int L, int H, int G, int nc, int ncol0) {
  using C = SpanCfg<Q, N, R>;
  const int lane = lane_id();
  const int w = wave_id();
  const int64_t tok0 = (int64_t)c * Q + jb * C::RB;
#pragma unroll
  for (int k0 = 0; k0 < C::TOT; k0 += C::NW) {
    const int k = k0 + w;
    if (k < C::XT) {
      const int r = k >> 2, s = (k & 3) * 64 + lane;
      const int row = s >> 3, pos = s & 7;
      int64_t t = tok0 + row;
      if (t > L - 1) t = L - 1;
      dma16(x + (((int64_t)b * L + t) * H + h0 + r) * C::P + 8 * sx(row, pos),
            buf + r * C::XH + s * 16);
    } else if (k < C::XT + C::BT) {
      const int s = (k - C::XT) * 64 + lane;
      const int row = s / (N / 8), pos = s % (N / 8);
      int64_t t = tok0 + row;
      if (t > L - 1) t = L - 1;
      dma16(Bm + (((int64_t)b * L + t) * G + g) * LDN + ncol0 + 8 * sb<N, ALT>(row, pos),
            buf + C::XS + s * 16);
    } else if (k == C::XT + C::BT) {  // cumulative sums and dt of the R heads
      const int r = lane >> 4, q = lane & 15;
      const int rr = r < R ? r : 0;
      const int64_t o = (((int64_t)b * H + h0 + rr) * nc + c) * Q + jb * C::RB + 4 * (q & 7);
      if (r < R) dma16((q < 8 ? dA_cs : dt_T) + o, buf + C::XS + C::BS + lane * 16);
    } else if (k == C::XT + C::BT + 1) {  // last cumulative sums of the chunk
      const int rr = lane < R ? lane : 0;
      const int64_t o = (((int64_t)b * H + h0 + rr) * nc + c) * Q + Q - 4;
      if (lane < R) dma16(dA_cs + o, buf + C::XS + C::BS + C::CS + lane * 16);
    }
  }
}

// The same loads with the per-lane addresses formed once per workgroup: for
// load slot j of this wave, the address of block 0 (p[j]), the LDS offset
// (dst[j]) and the slot's strides per block and per chunk (the last
// cumulative sums move once per chunk).  The slot's kind only decides those
// values at set-up: every load is issued the same way, with all 64 lanes
// (lanes past the heads load a valid duplicate into unused LDS), so issuing
// a block takes no lane masks or branches on the kind.  Valid while the
// block lies inside the sequence (no clamping needed).
template <int Q, int N, int R, int LDN, bool ALT>
struct DmaPlan {
  using C = SpanCfg<Q, N, R>;
  static constexpr int NJ = (C::TOT + C::NW - 1) / C::NW;
  const char* p[NJ];
  uint32_t dst[NJ];
  int64_t st[NJ], sc[NJ];
  int nj;  // slots this wave issues

  __device__ __forceinline__ void init(const bf16* __restrict__ x, const bf16* __restrict__ Bm,
                                       const float* __restrict__ dA_cs,
                                       const float* __restrict__ dt_T, int c0, int b, int h0,
                                       int g, int L, int H, int G, int nc, int ncol0) {
    const int lane = lane_id();
    const int w = wave_id();
    const int64_t tok0 = (int64_t)c0 * Q;
    nj = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int k = j * C::NW + w;
      p[j] = (const char*)dA_cs;
      dst[j] = 0;
      st[j] = sc[j] = 0;
      if (k < C::TOT) nj = j + 1;
      if (k < C::XT) {
        const int r = k >> 2, s = (k & 3) * 64 + lane;
        const int row = s >> 3, pos = s & 7;
        p[j] = (const char*)(x + (((int64_t)b * L + tok0 + row) * H + h0 + r) * C::P + 8 * sx(row, pos));
        dst[j] = r * C::XH + (k & 3) * 1024;
        st[j] = (int64_t)C::RB * H * C::P * 2;
      } else if (k < C::XT + C::BT) {
        const int s = (k - C::XT) * 64 + lane;
        const int row = s / (N / 8), pos = s % (N / 8);
        p[j] = (const char*)(Bm + (((int64_t)b * L + tok0 + row) * G + g) * LDN + ncol0 +
                             8 * sb<N, ALT>(row, pos));
        dst[j] = C::XS + (k - C::XT) * 1024;
        st[j] = (int64_t)C::RB * G * LDN * 2;
      } else if (k == C::XT + C::BT) {
        const int r = lane >> 4, q = lane & 15;
        const int rr = r < R ? r : 0;
        const int64_t o = (((int64_t)b * H + h0 + rr) * nc + c0) * Q + 4 * (q & 7);
        p[j] = (const char*)((q < 8 ? dA_cs : dt_T) + o);
        dst[j] = C::XS + C::BS;
        st[j] = (int64_t)C::RB * 4;
      } else if (k == C::XT + C::BT + 1) {
        const int rr = lane < R ? lane : 0;
        p[j] = (const char*)(dA_cs + (((int64_t)b * H + h0 + rr) * nc + c0) * Q + Q - 4);
        dst[j] = C::XS + C::BS + C::CS;
        sc[j] = (int64_t)Q * 4;
      }
    }
  }

  __device__ __forceinline__ void issue(uint32_t buf, int i) const {
    const int ic = i / C::BPC;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (j < nj) dma16(p[j] + i * st[j] + ic * sc[j], buf + dst[j]);
  }
};

// Which part of the run's states tile m of wave w holds: R tiles of 32 state
// columns each (all 64 rows as 2 x 4 MFMA tiles).  With R <= NW the NW / R
// waves of a head split its N columns, so a wave contracts one head's x rows.
// More heads than waves (a wave holding R / NW heads whole) is supported by
// these helpers, though the launchers instantiate only the head counts the
// host's rule picks (at most 1 head per workgroup at N = 64, 2 at N = 128),
// which never exceed the waves.
template <int NW, int R>
__device__ __forceinline__ int tile_head(int w, int m) {
  return NW >= R ? w / (NW / R) : w * (R / NW) + m / NW;
}
template <int NW, int R>
__device__ __forceinline__ int tile_cols(int w, int m) {  // 32-column group
  return NW >= R ? (w % (NW / R)) * R + m : m % NW;
}

template <int Q, int N, int R, int LDN>
__device__ __forceinline__ void store_hst(bf16* __restrict__ hst, const f32x4 (&acc)[R][2][4],
                                          int b, int c, int h0, int H, int nc, int L16,
                                          int grp, int w, int ncol0) {
  using C = SpanCfg<Q, N, R>;
#pragma unroll
  for (int m = 0; m < R; ++m) {
    const int r = tile_head<C::NW, R>(w, m);
    const int ncol = 32 * tile_cols<C::NW, R>(w, m) + 8 * grp;  // interleaved tiles
    bf16* dst = hst + ((((int64_t)b * nc + c) * H + h0 + r) * 64 + L16) * LDN + ncol0 + ncol;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = f2bf(acc[m][0][pt][e]);
        o[4 + e] = f2bf(acc[m][1][pt][e]);
      }
      *(bf16x8*)(dst + (int64_t)16 * pt * LDN) = o;
    }
  }
}

template <int Q, int N, int R, bool REPLAY, int LDN, int OCCT>
__global__ void __launch_bounds__((SpanCfg<Q, N, R, OCCT>::NT), (SpanCfg<Q, N, R, OCCT>::WPE)) chunk_state_span_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ Bm, const float* __restrict__ dA_cs,
    const float* __restrict__ dt_T, float* __restrict__ span_states,
    float* __restrict__ span_decay, bf16* __restrict__ hst, int L, int H, int G, int nc, int K,
    int ng, int BNGG, int ncol0_arg) {
  // Rows of B, of the span states and of the chunk-start states hold LDN
  // columns; a workgroup covers columns ncol0 .. ncol0 + N - 1 (ncol0_arg
  // when there is one column half, from the workgroup id when two).
  using C = SpanCfg<Q, N, R, OCCT>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  // Every run of a (batch, span, group), and at LDN = 2N both column halves
  // of it, on one XCD, so the span's B rows and x rows are fetched into that
  // XCD's L2 once: id = 8 r + xcd, r = NH RG q + NH run + half,
  // (batch, span, group) index 8 q + xcd.
  constexpr int NH = LDN / N;
  const int HG = H / G, RG = HG / R;
  const int xcd = blockIdx.x & 7, rq = blockIdx.x >> 3;
  const int rh = rq % (RG * NH);
  const int run = rh / NH;
  const int ncol0 = NH == 1 ? ncol0_arg : (rh % NH) * N;
  const int bsg = (rq / (RG * NH)) * 8 + xcd;
  if (bsg >= BNGG) return;
  const int g = bsg % G;
  const int b = bsg / G / ng, s = (bsg / G) % ng;
  const int h0 = g * HG + run * R;
  const int c0 = s * K, c1 = min(c0 + K, nc);
  const int cend = REPLAY ? c1 - 1 : c1;  // chunks whose contraction is needed
  const int nblk = (cend - c0) * C::BPC;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = wave_id();
  const int L16 = lane & 15, grp = lane >> 4;
  // this wave's direct-to-LDS loads per block
  const int nw = C::TOT / C::NW + (w < C::TOT % C::NW ? 1 : 0);

  // acc[m][nt][pt][e] = state of head h0 + tile_head(w, m) at
  // [p = 16 pt + L16][n = 32 tile_cols(w, m) + acc_col(nt, grp) + e]
  constexpr bool ALT = !REPLAY;
  f32x4 acc[R][2][4];
#pragma unroll
  for (int m = 0; m < R; ++m) {
    const int r = tile_head<C::NW, R>(w, m);
    const int ncol = 32 * tile_cols<C::NW, R>(w, m);
    const float* sst = span_states + (((int64_t)b * ng + s) * H + h0 + r) * 64 * LDN + ncol0;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        acc[m][nt][pt] = REPLAY ? *(const f32x4*)(sst + (16 * pt + L16) * LDN + ncol +
                                                  acc_col<ALT>(nt, grp))
                                : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float dsum[R];
#pragma unroll
  for (int r = 0; r < R; ++r) dsum[r] = 0.f;

  const uint32_t sbase = lds_addr(smem);
  __builtin_amdgcn_s_waitcnt(0);  // the start states are in registers
  DmaPlan<Q, N, R, LDN, ALT> plan;
  plan.init(x, Bm, dA_cs, dt_T, c0, b, h0, g, L, H, G, nc, ncol0);
  // blocks from `nfast` on reach past the sequence end: their rows are clamped
  const int nfast = min(nblk, (int)(((int64_t)L - (int64_t)c0 * Q) / C::RB));
#pragma unroll
  for (int j = 0; j < C::NBUF - 1; ++j) {
    if (j < nfast)
      plan.issue(sbase + j * C::BUF, j);
    else if (j < nblk)
      issue_block<Q, N, R, LDN, ALT>(sbase + j * C::BUF, x, Bm, dA_cs, dt_T, c0 + j / C::BPC,
                                j % C::BPC, b, h0, g, L, H, G, nc, ncol0);
  }

  // x rows of the block in buffer `bp` scaled by w_j in place: slot s is
  // head s / 256, row (s % 256) / 8
  auto scale_x = [&](unsigned char* bp) {
    const float* sb_ = (const float*)(bp + C::XS + C::BS);
    const float* cl_ = (const float*)(bp + C::XS + C::BS + C::CS);
#pragma unroll
    for (int s0 = 0; s0 < C::SLOTS; s0 += C::NT) {
      const int sl = s0 + tid;
      if (C::SLOTS % C::NT == 0 || sl < C::SLOTS) {
        const int r = sl >> 8, row = (sl & 255) >> 3;
        const bf16x8 v = *(const bf16x8*)(bp + sl * 16);
        const float wr = fast_exp2(cl_[4 * r + 3] - sb_[64 * r + row]) * sb_[64 * r + 32 + row];
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = f2bf(bf2f(v[e]) * wr);
        *(bf16x8*)(bp + sl * 16) = o;
      }
    }
  };
  // Software pipeline: block i + 1 is scaled while block i's MFMAs run (they
  // touch different buffers), so each block needs one barrier.  Block 0 is
  // scaled first.
  static_assert(C::NBUF >= 3, "the block being scaled, the block being read and the one loading");
  if (nblk > 0) {
    asm volatile("" ::: "memory");
    wait_vm(nw * min(C::NBUF - 2, nblk - 1));
    __builtin_amdgcn_s_barrier();  // block 0 landed for every wave
    asm volatile("" ::: "memory");
    scale_x(smem);
  }

  for (int i = 0; i < nblk; ++i) {
    const int c = c0 + i / C::BPC, jb = i % C::BPC;
    // operations newer than block i + 1's loads: the loads of the blocks after
    // it already issued, and the start-state stores issued since (after the
    // last block nothing is left to wait for but this wave's LDS writes)
    int newer = 0;
    if (i + 1 < nblk) {
      newer = nw * (min(i + C::NBUF - 2, nblk - 1) - (i + 1));
      if (REPLAY) {
        const int j0 = max(0, i + 2 - C::NBUF);
        const int starts = (i - 1) / C::BPC - (j0 - 1 + C::BPC) / C::BPC + 1;  // j0 <= j <= i-1, j % BPC == 0
        newer += 4 * R * (i > j0 ? max(starts, 0) : 0);  // store_hst: 4 per head tile
      }
    }
    asm volatile("" ::: "memory");
    wait_vm(newer);
    // block i + 1 landed and block i scaled, for every wave; block i - 1 fully read
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (i + C::NBUF - 1 < nblk) {
      const int j = i + C::NBUF - 1;
      if (j < nfast)
        plan.issue(sbase + (j % C::NBUF) * C::BUF, j);
      else
        issue_block<Q, N, R, LDN, ALT>(sbase + (j % C::NBUF) * C::BUF, x, Bm, dA_cs, dt_T,
                                  c0 + j / C::BPC, j % C::BPC, b, h0, g, L, H, G, nc, ncol0);
    }
    unsigned char* cur = smem + (i % C::NBUF) * C::BUF;
    const float* cl = (const float*)(cur + C::XS + C::BS + C::CS);
    if (jb == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) dsum[r] += cl[4 * r + 3];
      if (REPLAY) store_hst<Q, N, R, LDN>(hst, acc, b, c, h0, H, nc, L16, grp, w, ncol0);
#pragma unroll
      for (int m = 0; m < R; ++m) {
        const float dec = fast_exp2(cl[4 * tile_head<C::NW, R>(w, m) + 3]);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          acc[m][0][pt] *= dec;
          acc[m][1][pt] *= dec;
        }
      }
    }
    if (i + 1 < nblk) scale_x(smem + ((i + 1) % C::NBUF) * C::BUF);
    const unsigned char* bsm = cur + C::XS;
    const int ra = 8 * grp + (L16 >> 2), rb = ra + 4;
    constexpr int HPW = R > C::NW ? R / C::NW : 1;  // heads per wave
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const unsigned char* xs = cur + tile_head<C::NW, R>(w, hh * (R / HPW)) * C::XH;
      bf16x8 xop[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int ch = 2 * pt + ((L16 & 3) >> 1), off = 8 * (L16 & 1);
        const bf16* pa = (const bf16*)(xs + ra * 128 + sx(ra, ch) * 16 + off);
        const bf16* pb = (const bf16*)(xs + rb * 128 + sx(rb, ch) * 16 + off);
        xop[pt] = cat(lds_read_tr(pa), lds_read_tr(pb));
      }
#pragma unroll
      for (int v = 0; v < R / HPW; ++v) {
        const int m = hh * (R / HPW) + v;
        // tile nt, MFMA row i: ALT n = 32 tile_cols + 16 nt + i (lane L16
        // points at chunk 4 tile_cols + 2 nt + (L16 % 4) / 2, half L16 % 2);
        // else n = 32 tile_cols + 8 (i / 4) + 4 nt + i % 4 (chunk
        // 4 tile_cols + L16 % 4, half nt)
        bf16x8 bop[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int bc = ALT ? 4 * tile_cols<C::NW, R>(w, m) + 2 * nt + ((L16 & 3) >> 1)
                             : 4 * tile_cols<C::NW, R>(w, m) + (L16 & 3);
          const int hb = ALT ? 8 * (L16 & 1) : 8 * nt;
          const bf16* pa = (const bf16*)(bsm + ra * (2 * N) + sb<N, ALT>(ra, bc) * 16 + hb);
          const bf16* pb = (const bf16*)(bsm + rb * (2 * N) + sb<N, ALT>(rb, bc) * 16 + hb);
          bop[nt] = cat(lds_read_tr(pa), lds_read_tr(pb));
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int pt = 0; pt < 4; ++pt)
            acc[m][nt][pt] = mfma16x16x32(bop[nt], xop[pt], acc[m][nt][pt]);
      }
    }
  }

  if (REPLAY) {  // start state of the span's last chunk
    store_hst<Q, N, R, LDN>(hst, acc, b, c1 - 1, h0, H, nc, L16, grp, w, ncol0);
  } else {
#pragma unroll
    for (int m = 0; m < R; ++m) {
      const int r = tile_head<C::NW, R>(w, m);
      const int ncol = 32 * tile_cols<C::NW, R>(w, m);
      float* sst = span_states + (((int64_t)b * ng + s) * H + h0 + r) * 64 * LDN + ncol0;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          *(f32x4*)(sst + (16 * pt + L16) * LDN + ncol + acc_col<ALT>(nt, grp)) = acc[m][nt][pt];
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (tid == 0 && ncol0 == 0) span_decay[((int64_t)b * H + h0 + r) * ng + s] = dsum[r];
  }
}

// The jump across spans: st holds the span-end states [B, ng, H, P*N/4] on
// entry and the span-start states on exit (in place); decay [B, H, ng] is
// each span's log2 decay.  One thread per 4 consecutive state entries.
constexpr int kSpanDepth = 8;

__global__ void __launch_bounds__(256) span_passing_kernel(f32x4* __restrict__ st,
                                                           const float* __restrict__ decay,
                                                           const f32x4* __restrict__ init,
                                                           f32x4* __restrict__ final_state,
                                                           int64_t H, int64_t PNv, int64_t bph,
                                                           int ng) {
  const int64_t bh = (int64_t)blockIdx.x / bph;
  const int64_t gid = ((int64_t)blockIdx.x % bph) * 256 + threadIdx.x;
  if (gid >= PNv) return;
  const int64_t b = bh / H, h = bh % H;
  const int64_t stride = H * PNv;
  f32x4* base = st + (b * ng * H + h) * PNv + gid;
  const float* dec = decay + bh * ng;
  f32x4 run = init ? init[bh * PNv + gid] : f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 buf[kSpanDepth];
#pragma unroll
  for (int k = 0; k < kSpanDepth; ++k)
    if (k < ng) buf[k] = __builtin_nontemporal_load(base + (int64_t)k * stride);
  for (int s0 = 0; s0 < ng; s0 += kSpanDepth) {
#pragma unroll
    for (int k = 0; k < kSpanDepth; ++k) {
      const int s = s0 + k;
      if (s < ng) {
        const f32x4 cur = buf[k];
        if (s + kSpanDepth < ng)
          buf[k] = __builtin_nontemporal_load(base + (int64_t)(s + kSpanDepth) * stride);
        base[(int64_t)s * stride] = run;
        run = fast_exp2(dec[s]) * run + cur;
      }
    }
  }
  if (final_state) final_state[bh * PNv + gid] = run;
}

int cu_count_span() {
  static const int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    return v;
  }();
  return n;
}

// Heads per workgroup: as many as share B (a divisor of the group's heads)
// while the grid still gives every CU a workgroup: up to 4 at N >= 256, 2 at
// N = 128 and 1 at N = 64, where a workgroup has only N/32 waves and several
// workgroups must share a CU to keep about eight waves on it.
int span_heads(const Dims& d, int K) {
  const int64_t HG = d.H / d.G, ng = (d.nc + K - 1) / K;
  const int maxR = d.N == 64 ? 1 : d.N == 128 ? 2 : kSpanHeads;
  for (int R = maxR; R > 1; R /= 2)
    if (HG % R == 0 && d.B * ng * d.H / R >= cu_count_span()) return R;
  return 1;
}

template <int Q, int N, int R, bool REPLAY, int LDN, int OCCT>
hipError_t launch_span_occ(const Dims& d, int K, const void* x, const void* B,
                           const float* dA_cs, const float* dt_T, float* span_states,
                           float* span_decay, void* hst, hipStream_t s) {
  using C = SpanCfg<Q, N, R, OCCT>;
  auto kern = chunk_state_span_kernel<Q, N, R, REPLAY, LDN, OCCT>;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
  if (attr != hipSuccess) return attr;
  const int64_t ng = (d.nc + K - 1) / K;
  const int64_t BNGG = d.B * ng * d.G;
  const int64_t grid = (BNGG + 7) / 8 * 8 * (d.H / d.G / R) * (LDN / N);
  kern<<<(unsigned)grid, C::NT, C::LDS, s>>>((const bf16*)x, (const bf16*)B, dA_cs, dt_T,
                                           span_states, span_decay, (bf16*)hst, (int)d.L,
                                           (int)d.H, (int)d.G, (int)d.nc, K, (int)ng, (int)BNGG,
                                           0);
  return hipGetLastError();
}

// Workgroups per CU the LDS ring is sized for.  One by default (the ring
// takes the whole LDS); where the grid is larger than the device and the
// kernel is small enough for several workgroups per CU (one head per
// workgroup, about 112 VGPRs; or N <= 128, at most 4 waves per workgroup), a
// ring sized for two, or four at N = 64, lets more of the grid run at once.
template <int Q, int N, int R, bool REPLAY, int LDN>
hipError_t launch_span(const Dims& d, int K, const void* x, const void* B, const float* dA_cs,
                       const float* dt_T, float* span_states, float* span_decay, void* hst,
                       hipStream_t s) {
  if constexpr (kSpanOcc == 1 && (R == 1 || (N == 128 && R == 2))) {
    const int64_t ng = (d.nc + K - 1) / K;
    const int64_t grid = (d.B * ng * d.G + 7) / 8 * 8 * (d.H / d.G / R) * (LDN / N);
    const int64_t cus = cu_count_span();
    if constexpr (N == 64) {
      if (grid > 2 * cus)
        return launch_span_occ<Q, N, R, REPLAY, LDN, 4>(d, K, x, B, dA_cs, dt_T, span_states,
                                                        span_decay, hst, s);
    }
    if (grid > cus)
      return launch_span_occ<Q, N, R, REPLAY, LDN, 2>(d, K, x, B, dA_cs, dt_T, span_states,
                                                      span_decay, hst, s);
  }
  return launch_span_occ<Q, N, R, REPLAY, LDN, kSpanOcc>(d, K, x, B, dA_cs, dt_T, span_states,
                                                         span_decay, hst, s);
}

template <int R, bool REPLAY>
hipError_t launch_span_qn(const Dims& d, int K, const void* x, const void* B, const float* dA_cs,
                          const float* dt_T, float* span_states, float* span_decay, void* hst,
                          hipStream_t s) {
#define M2_SPAN(QQ, NN)                                                                    \
  if (d.Q == QQ && d.N == NN)                                                              \
    return launch_span<QQ, NN, R, REPLAY, NN>(d, K, x, B, dA_cs, dt_T, span_states,         \
                                              span_decay, hst, s);
  // only the head counts span_heads can pick: 1 at N = 64, up to 2 at N = 128
  if constexpr (R == 1) {
    M2_SPAN(64, 64) M2_SPAN(128, 64) M2_SPAN(256, 64)
  }
  if constexpr (R <= 2) {
    M2_SPAN(64, 128) M2_SPAN(128, 128) M2_SPAN(256, 128)
  }
  M2_SPAN(64, 256) M2_SPAN(128, 256) M2_SPAN(256, 256)
#undef M2_SPAN
  // state size 512: both halves of the state columns in one launch (each
  // column of the state evolves on its own)
#define M2_SPAN512(QQ)                                                                       \
  if (d.Q == QQ && d.N == 512)                                                               \
    return launch_span<QQ, 256, R, REPLAY, 512>(d, K, x, B, dA_cs, dt_T, span_states,        \
                                                span_decay, hst, s);
  M2_SPAN512(64) M2_SPAN512(128) M2_SPAN512(256)
#undef M2_SPAN512
  return hipErrorInvalidValue;
}

template <bool REPLAY>
hipError_t launch_span_r(const Dims& d, int K, int R, const void* x, const void* B,
                         const float* dA_cs, const float* dt_T, float* span_states,
                         float* span_decay, void* hst, hipStream_t s) {
  switch (R) {
    case 1: return launch_span_qn<1, REPLAY>(d, K, x, B, dA_cs, dt_T, span_states, span_decay, hst, s);
    case 2: return launch_span_qn<2, REPLAY>(d, K, x, B, dA_cs, dt_T, span_states, span_decay, hst, s);
    case 4: return launch_span_qn<4, REPLAY>(d, K, x, B, dA_cs, dt_T, span_states, span_decay, hst, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int span_chunks(const Dims& d) {
  if (!(d.bf16 && d.P == 64 && (d.N == 64 || d.N == 128 || d.N == 256 || d.N == 512) &&
        (d.Q == 64 || d.Q == 128 || d.Q == 256)))
    return 0;
  // Spans of 8 chunks when that gives every CU two (batch, span, head)
  // units, else spans of 4 if they do (each workgroup then walks half as many
  // blocks in sequence), else the longest span that gives every CU one;
  // shorter spans save too little of the state traffic.
  const int64_t cus = cu_count_span();
  for (int64_t want = 2 * cus; want >= cus; want -= cus)
    for (int K = 8; K >= 4; K /= 2) {
      const int64_t ng = (d.nc + K - 1) / K;
      if (d.nc >= K && d.B * d.H * ng >= want) return K;
    }
  return 0;
}

size_t span_states_bytes(const Dims& d, int K) {
  const int64_t ng = (d.nc + K - 1) / K;
  return (size_t)(d.B * ng * d.H * d.P * d.N) * sizeof(float);
}

hipError_t launch_fwd_pass_state_span(const Dims& d, int K, const void* x, const void* B,
                                      const float* dA_cs, const float* dt_T, const float* init,
                                      float* span_states, float* span_decay, void* hst,
                                      float* final_state, hipStream_t s, hipEvent_t mid,
                                      bool replay) {
  const int R = span_heads(d, K);
  hipError_t e =
      launch_span_r<false>(d, K, R, x, B, dA_cs, dt_T, span_states, span_decay, hst, s);
  if (e != hipSuccess) return e;
  if (mid) {
    e = hipEventRecord(mid, s);
    if (e != hipSuccess) return e;
  }
  const int64_t ng = (d.nc + K - 1) / K;
  const int64_t PNv = d.P * d.N / 4, bph = (PNv + 255) / 256;
  span_passing_kernel<<<(unsigned)(d.B * d.H * bph), 256, 0, s>>>(
      (f32x4*)span_states, span_decay, (const f32x4*)init, (f32x4*)final_state, d.H, PNv, bph,
      (int)ng);
  e = hipGetLastError();
  if (e != hipSuccess || !replay) return e;
  return launch_span_r<true>(d, K, R, x, B, dA_cs, dt_T, span_states, span_decay, hst, s);
}

}  // namespace m2
