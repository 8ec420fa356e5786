// C ABI of the SSD forward pass: argument checks on the host, workspace
// carving, and stream-ordered launches of the stage kernels.  Declarations and
// the contract of every entry point are in include/mamba2_ssd.h.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "launch.h"
#include "mamba2_ssd.h"

// Workspace of mamba2_ssd_forward_noalloc: one copy per GPU, held for the
// process's lifetime.  Host code never uses this name as an address (it is a
// host-side stand-in there); it uses the device address looked up below.
static __device__ __align__(256) unsigned char scratch[MAMBA2_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return MAMBA2_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Upper bounds that keep every index and grid size inside the kernels' types.
constexpr int64_t kMaxSeq = (int64_t)1 << 30;
constexpr int64_t kMaxUnits = (int64_t)1 << 26;   // B * nc * H workgroups
constexpr int64_t kMaxElems = (int64_t)1 << 40;   // elements of any tensor

int validate(const mamba2_dims* d, m2::Dims* out) {
  if (!d) return fail(MAMBA2_ERR_NULL, "dims is NULL");
  if (d->dtype != MAMBA2_DTYPE_F32 && d->dtype != MAMBA2_DTYPE_BF16)
    return fail(MAMBA2_ERR_DTYPE, "unknown dtype code %d", (int)d->dtype);
  if (d->reserved != 0) return fail(MAMBA2_ERR_SHAPE, "dims.reserved must be 0");
  if (d->batch < 1 || d->seqlen < 1 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 ||
      d->ngroups < 1 || d->chunk_size < 1)
    return fail(MAMBA2_ERR_SHAPE,
                "sizes must be >= 1 (batch=%lld seqlen=%lld nheads=%lld headdim=%lld "
                "dstate=%lld ngroups=%lld chunk_size=%lld)",
                (long long)d->batch, (long long)d->seqlen, (long long)d->nheads,
                (long long)d->headdim, (long long)d->dstate, (long long)d->ngroups,
                (long long)d->chunk_size);
  if (d->nheads % d->ngroups != 0)
    return fail(MAMBA2_ERR_SHAPE, "nheads (%lld) is not a multiple of ngroups (%lld)",
                (long long)d->nheads, (long long)d->ngroups);
  const int64_t Q = d->chunk_size;
  const bool bf = d->dtype == MAMBA2_DTYPE_BF16;
  if (bf) {
    if (Q != 64 && Q != 128 && Q != 256)
      return fail(MAMBA2_ERR_UNSUPPORTED, "bfloat16 chunk_size must be 64, 128 or 256 (got %lld)",
                  (long long)Q);
    if (d->headdim % 16 != 0 || d->headdim > 128)
      return fail(MAMBA2_ERR_UNSUPPORTED,
                  "bfloat16 headdim must be a multiple of 16 and at most 128 (got %lld)",
                  (long long)d->headdim);
    if (d->dstate % 16 != 0 || d->dstate > 512)
      return fail(MAMBA2_ERR_UNSUPPORTED,
                  "bfloat16 dstate must be a multiple of 16 and at most 512 (got %lld)",
                  (long long)d->dstate);
  } else {
    if (Q != 16 && Q != 32 && Q != 64 && Q != 128 && Q != 256)
      return fail(MAMBA2_ERR_UNSUPPORTED,
                  "float32 chunk_size must be 16, 32, 64, 128 or 256 (got %lld)", (long long)Q);
    if (d->headdim > 1024 || d->dstate > 4096)
      return fail(MAMBA2_ERR_UNSUPPORTED, "float32 headdim <= 1024 and dstate <= 4096 required");
  }
  if (d->seqlen > kMaxSeq || d->nheads > 65536 || d->batch > 65536)
    return fail(MAMBA2_ERR_UNSUPPORTED, "sizes beyond the supported range");
  const int64_t nc = (d->seqlen + Q - 1) / Q;
  const double units = (double)d->batch * (double)nc * (double)d->nheads;
  const double st = units * (double)d->headdim * (double)d->dstate;
  const double xs = (double)d->batch * (double)d->seqlen * (double)d->nheads * (double)d->headdim;
  if (units > (double)kMaxUnits || st > (double)kMaxElems || xs > (double)kMaxElems)
    return fail(MAMBA2_ERR_UNSUPPORTED, "problem too large for one call");
  if (out) {
    out->B = d->batch;
    out->L = d->seqlen;
    out->H = d->nheads;
    out->P = d->headdim;
    out->N = d->dstate;
    out->G = d->ngroups;
    out->Q = Q;
    out->nc = nc;
    out->bf16 = bf;
  }
  return MAMBA2_OK;
}

int need(const void* p, const char* name) {
  if (!p) return fail(MAMBA2_ERR_NULL, "%s is NULL", name);
  if (!aligned16(p)) return fail(MAMBA2_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return MAMBA2_OK;
}

int maybe(const void* p, const char* name) {
  if (p && !aligned16(p)) return fail(MAMBA2_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return MAMBA2_OK;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(MAMBA2_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace of mamba2_ssd_forward, exactly what its path uses (256-byte
// aligned pieces): dA_cs and dt_T [B,H,nc,Q] f32; then
//   split path: the per-chunk states [B,nc,H,P,N] f32, (grouped output
//     stage) the chunk-start states as bf16 and (state size 512) the first
//     column half's y as bf16;
//   span path (K > 0): the span states [B,ng,H,P,N] f32 and span log2 decays
//     [B,H,ng], then, unless span_scan runs, the bf16 chunk-start states and
//     (state size 512) the first column half's y.
// The opt-in one-kernel forward (mamba2_ssd_forward_fused) carves its own
// layout (three [B,H,nc,Q] f32 arrays and the bf16 chunk-start states) from
// the same workspace, so `total` covers that too where it is supported.
struct Workspace {
  bool grouped;
  int K, Rs;  // span length (0: split path) and span_scan heads (0: replay)
  size_t cs_bytes, st_bytes, span_bytes, hst_bytes, part_bytes, total;
};

Workspace plan(const m2::Dims& d) {
  Workspace w;
  w.grouped = m2::grouped_scan_supported(d);
  w.K = 0;
  if (w.grouped) {
    w.K = m2::span_scan_chunks(d);
    if (!w.K) w.K = m2::span_chunks(d);
  }
  w.Rs = w.K ? m2::span_scan_heads(d, w.K) : 0;
  w.cs_bytes = round256((size_t)(d.B * d.H * d.nc * d.Q) * sizeof(float));
  const size_t hst = round256((size_t)(d.B * d.nc * d.H * d.P * d.N) * 2);
  if (w.K) {
    const int64_t ng = (d.nc + w.K - 1) / w.K;
    w.span_bytes = round256(m2::span_states_bytes(d, w.K));
    w.st_bytes = w.span_bytes + round256((size_t)(d.B * d.H * ng) * sizeof(float));
    w.hst_bytes = w.Rs ? 0 : hst;
    w.part_bytes = w.Rs ? 0 : round256(m2::grouped_scan_part_bytes(d));
  } else {
    w.span_bytes = 0;
    w.st_bytes = round256((size_t)(d.B * d.nc * d.H * d.P * d.N) * sizeof(float));
    w.hst_bytes = w.grouped ? hst : 0;
    w.part_bytes = w.grouped ? round256(m2::grouped_scan_part_bytes(d)) : 0;
  }
  w.total = 2 * w.cs_bytes + w.st_bytes + w.hst_bytes + w.part_bytes;
  if (m2::fused_state_supported(d)) {
    const size_t fused = 3 * w.cs_bytes + hst;
    if (fused > w.total) w.total = fused;
  }
  return w;
}

// Enqueues the four stages; when `ev` is non-null, records ev[0..4] around them.
int enqueue_forward(const m2::Dims& d, const void* x, const void* dt, const float* A,
                    const void* B, const void* C, const float* D, const float* init_state,
                    void* y, float* final_state, void* workspace, hipStream_t s,
                    hipEvent_t* ev) {
  const Workspace w = plan(d);
  char* ws = (char*)workspace;
  float* dA_cs = (float*)ws;
  float* dt_T = (float*)(ws + w.cs_bytes);
  float* states = (float*)(ws + 2 * w.cs_bytes);
  void* hst = ws + 2 * w.cs_bytes + w.st_bytes;
  void* part = w.part_bytes ? (void*)(ws + 2 * w.cs_bytes + w.st_bytes + w.hst_bytes) : nullptr;
  hipError_t e = hipSuccess;
  if (ev) e = hipEventRecord(ev[0], s);
  if (e == hipSuccess) e = m2::launch_chunk_cumsum(d, dt, A, dA_cs, dt_T, s);
  if (e != hipSuccess) return hip_status(e, "chunk_cumsum launch");
  if (ev) e = hipEventRecord(ev[1], s);
  const int K = w.K;
  if (K) {
    // fwd_pass_state over spans: span-end states (stage slot 1), then the
    // jump across spans and the replay that writes the chunk-start states
    // (stage slot 2); or, where span_scan covers the sizes, the jump alone
    // (slot 2) and span_scan, the replay fused with the output stage (slot 3)
    float* span_decay = (float*)((char*)states + w.span_bytes);
    const int Rs = w.Rs;
    if (e == hipSuccess)
      e = m2::launch_fwd_pass_state_span(d, K, x, B, dA_cs, dt_T, init_state, states, span_decay,
                                         hst, final_state, s, ev ? ev[2] : nullptr, Rs == 0);
    if (e != hipSuccess) return hip_status(e, "fwd_pass_state launch");
    if (ev) e = hipEventRecord(ev[3], s);
    if (e == hipSuccess)
      e = Rs ? m2::launch_span_scan(d, K, Rs, x, B, C, dA_cs, dt_T, states, D, y, s)
             : m2::launch_chunk_scan_grouped(d, x, B, C, dA_cs, dt_T, hst, D, y, part, s);
    if (e != hipSuccess) return hip_status(e, "chunk_scan launch");
    if (ev) e = hipEventRecord(ev[4], s);
    return hip_status(e, "event record");
  }
  if (e == hipSuccess)
    e = m2::grouped_state_supported(d) ? m2::launch_chunk_state_grouped(d, x, B, dA_cs, dt_T, states, s)
                                       : m2::launch_chunk_state(d, x, B, dA_cs, dt_T, states, s);
  if (e != hipSuccess) return hip_status(e, "chunk_state launch");
  if (ev) e = hipEventRecord(ev[2], s);
  if (e == hipSuccess)
    e = w.grouped ? m2::launch_state_passing_bf16(d, states, dA_cs, init_state, hst, final_state, s)
                  : m2::launch_state_passing(d, states, dA_cs, init_state, final_state, s);
  if (e != hipSuccess) return hip_status(e, "state_passing launch");
  if (ev) e = hipEventRecord(ev[3], s);
  if (e == hipSuccess)
    e = w.grouped ? m2::launch_chunk_scan_grouped(d, x, B, C, dA_cs, dt_T, hst, D, y, part, s)
                  : m2::launch_chunk_scan(d, x, B, C, dA_cs, dt_T, states, D, y, s);
  if (e != hipSuccess) return hip_status(e, "chunk_scan launch");
  if (ev) e = hipEventRecord(ev[4], s);
  return hip_status(e, "event record");
}

int check_forward_args(const mamba2_dims* dims, m2::Dims* d, const void* x, const void* dt,
                       const float* A, const void* B, const void* C, const float* D,
                       const float* init_state, void* y, float* final_state, void* workspace,
                       size_t workspace_bytes);

#define CHECK(expr)               \
  do {                            \
    const int rc_ = (expr);       \
    if (rc_ != MAMBA2_OK) return rc_; \
  } while (0)

int check_forward_args(const mamba2_dims* dims, m2::Dims* d, const void* x, const void* dt,
                       const float* A, const void* B, const void* C, const float* D,
                       const float* init_state, void* y, float* final_state, void* workspace,
                       size_t workspace_bytes) {
  CHECK(validate(dims, d));
  CHECK(need(x, "x"));
  CHECK(need(dt, "dt"));
  CHECK(need(A, "A"));
  CHECK(need(B, "B"));
  CHECK(need(C, "C"));
  CHECK(maybe(D, "D"));
  CHECK(maybe(init_state, "init_state"));
  CHECK(need(y, "y"));
  CHECK(maybe(final_state, "final_state"));
  const Workspace w = plan(*d);
  if (!workspace) return fail(MAMBA2_ERR_WORKSPACE, "workspace is NULL");
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(MAMBA2_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < w.total)
    return fail(MAMBA2_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes,
                w.total);
  return MAMBA2_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MAMBA2_ERR_HIP, "device %d is beyond the %d devices the scratch table covers", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p || ((uintptr_t)p & 255u) != 0)
      return fail(MAMBA2_ERR_HIP, "scratch has no 256-byte aligned device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MAMBA2_OK;
}

// Workspace of the backward pass: the forward quantities it recomputes
// (dA_cs, dt_T, per-chunk states reused for the adjoint states, bf16 start
// states, final state) and its own (bf16 end-of-chunk gradients, carried-state
// and boundary dot-product parts, the groups' summed interaction matrices,
// per-chunk dA and dD parts).
// Backward workspace.  MFMA path (backward_supported): dA_cs, dt_T, the
// float32 per-chunk states (then the adjoint states), bf16 chunk-start
// states and chunk-end gradients, the recomputed final state, and the
// kernels' partial sums.  Generic path: dA_cs, dt_T, the float32 chunk-start
// states and adjoint states / chunk-end gradients, then the scratch of
// generic_backward_sizes (float32).
struct BwdWorkspace {
  bool fast;
  size_t cs, st, hst, fin, th, wsum, rsum, dots, part, total;
  int64_t wph;
  m2::GenericBwdSizes gen;
};

BwdWorkspace plan_backward(const m2::Dims& d) {
  BwdWorkspace w = {};
  w.fast = m2::backward_supported(d);
  w.cs = round256((size_t)(d.B * d.H * d.nc * d.Q) * sizeof(float));
  w.st = round256((size_t)(d.B * d.nc * d.H * d.P * d.N) * sizeof(float));
  if (!w.fast) {
    w.gen = m2::generic_backward_sizes(d);
    const m2::GenericBwdSizes& g = w.gen;
    w.total = 2 * w.cs + 2 * w.st +
              round256(g.vg * 4) + round256(g.thp * 4) + round256(g.xup * 4) +
              round256(g.ghp * 4) + round256(g.cb * 4) + 2 * round256(g.part * 4);
    return w;
  }
  w.wph = m2::state_reverse_waves_per_head(d);
  w.hst = round256((size_t)(d.B * d.nc * d.H * d.P * d.N) * 2);
  w.fin = round256((size_t)(d.B * d.H * d.P * d.N) * sizeof(float));
  w.th = round256((size_t)(d.B * d.nc * d.H * (d.N / 64) * d.Q) * sizeof(float));
  w.wsum = round256((size_t)(d.B * d.nc * d.G) * (size_t)(d.Q * (d.Q + 16) / 2) * 2);
  w.rsum = w.cs;
  w.dots = round256((size_t)(d.B * d.H * d.nc * w.wph) * sizeof(float));
  w.part = round256((size_t)(d.B * d.nc * d.H) * sizeof(float));
  w.total = 2 * w.cs + w.st + 2 * w.hst + w.fin + w.th + w.wsum + w.rsum + w.dots + 2 * w.part;
  return w;
}

// The generic backward: the forward's per-chunk states recomputed (float32
// chunk-start states), then chunk_bwd_generic.hip.
int enqueue_backward_generic(const m2::Dims& d, const BwdWorkspace& w, const void* x,
                             const void* dt, const float* A, const void* B, const void* C,
                             const float* D, const float* init_state, const void* dy,
                             const float* dfinal, void* dx, void* ddt, float* dA, void* dB,
                             void* dC, float* dD, float* dinit, void* workspace, hipStream_t s) {
  char* p = (char*)workspace;
  float* dA_cs = (float*)p;
  p += w.cs;
  float* dt_T = (float*)p;
  p += w.cs;
  float* hs = (float*)p;
  p += w.st;
  float* E = (float*)p;
  p += w.st;
  m2::GenericBwdScratch g;
  auto take = [&](size_t n) {
    float* q = (float*)p;
    p += round256(n * 4);
    return q;
  };
  g.vg = take(w.gen.vg);
  g.thp = take(w.gen.thp);
  g.xup = take(w.gen.xup);
  g.ghp = take(w.gen.ghp);
  g.cb = take(w.gen.cb);
  g.dA_part = take(w.gen.part);
  g.dD_part = take(w.gen.part);
  hipError_t e = m2::launch_chunk_cumsum(d, dt, A, dA_cs, dt_T, s);
  if (e == hipSuccess)
    e = m2::grouped_state_supported(d) ? m2::launch_chunk_state_grouped(d, x, B, dA_cs, dt_T, hs, s)
                                       : m2::launch_chunk_state(d, x, B, dA_cs, dt_T, hs, s);
  if (e == hipSuccess) e = m2::launch_state_passing(d, hs, dA_cs, init_state, nullptr, s);
  if (e == hipSuccess)
    e = m2::launch_backward_generic(d, x, dy, B, C, dA_cs, dt_T, hs, E, dfinal, dinit, A, D, dx,
                                    ddt, dB, dC, g, s);
  if (e == hipSuccess)
    e = m2::launch_bwd_param_sums(d, g.dA_part, g.dD_part, dA, D ? dD : nullptr, s);
  return hip_status(e, "backward launch");
}

constexpr int kBwdStages = 8;

int enqueue_backward(const m2::Dims& d, const void* x, const void* dt, const float* A,
                     const void* B, const void* C, const float* D, const float* init_state,
                     const void* dy, const float* dfinal, void* dx, void* ddt, float* dA,
                     void* dB, void* dC, float* dD, float* dinit, void* workspace,
                     hipStream_t s, hipEvent_t* ev) {
  const BwdWorkspace w = plan_backward(d);
  if (!w.fast) {
    if (ev) {  // one stage: the whole generic pass
      hipError_t e = hipEventRecord(ev[0], s);
      int rc = e == hipSuccess ? MAMBA2_OK : hip_status(e, "event record");
      if (rc == MAMBA2_OK)
        rc = enqueue_backward_generic(d, w, x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt,
                                      dA, dB, dC, dD, dinit, workspace, s);
      for (int i = 1; i <= kBwdStages && rc == MAMBA2_OK; ++i) {
        e = hipEventRecord(ev[i], s);
        if (e != hipSuccess) rc = hip_status(e, "event record");
      }
      return rc;
    }
    return enqueue_backward_generic(d, w, x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt, dA,
                                    dB, dC, dD, dinit, workspace, s);
  }
  char* p = (char*)workspace;
  float* dA_cs = (float*)p;
  p += w.cs;
  float* dt_T = (float*)p;
  p += w.cs;
  float* st = (float*)p;
  p += w.st;
  void* hst = p;
  p += w.hst;
  void* gst = p;
  p += w.hst;
  float* fin = (float*)p;
  p += w.fin;
  float* th = (float*)p;
  p += w.th;
  void* wsum = p;
  p += w.wsum;
  float* rsum = (float*)p;
  p += w.rsum;
  float* dots = (float*)p;
  p += w.dots;
  float* dA_part = (float*)p;
  p += w.part;
  float* dD_part = (float*)p;
  hipError_t e = hipSuccess;
  int stage = 0;
  auto mark = [&]() {
    if (ev && e == hipSuccess) e = hipEventRecord(ev[stage], s);
    ++stage;
  };
  mark();
  e = e == hipSuccess ? m2::launch_chunk_cumsum(d, dt, A, dA_cs, dt_T, s) : e;
  mark();
  // the forward's bf16 chunk-start states: over spans of chunks where the
  // forward takes that path (the span states and decays borrow the float32
  // state slot, which the adjoint states fill afterwards), else chunk_state
  // then state_passing; the profile's two stages are span_end and the jump
  // plus the replay there
  const int K = m2::span_chunks(d);
  if (K) {
    hipEvent_t mid = (ev && e == hipSuccess) ? ev[stage] : nullptr;
    float* sdec = (float*)((char*)st + round256(m2::span_states_bytes(d, K)));
    e = e == hipSuccess ? m2::launch_fwd_pass_state_span(d, K, x, B, dA_cs, dt_T, init_state, st,
                                                         sdec, hst, fin, s, mid, true)
                        : e;
    ++stage;
  } else {
    e = e == hipSuccess ? m2::launch_chunk_state_grouped(d, x, B, dA_cs, dt_T, st, s) : e;
    mark();
    e = e == hipSuccess ? m2::launch_state_passing_bf16(d, st, dA_cs, init_state, hst, fin, s)
                        : e;
  }
  mark();
  e = e == hipSuccess ? m2::launch_chunk_state_adjoint(d, dy, C, dA_cs, dt_T, st, s) : e;
  mark();
  e = e == hipSuccess
          ? m2::launch_state_passing_reverse(d, st, dA_cs, dfinal, hst, gst, dinit, dots, s)
          : e;
  mark();
  e = e == hipSuccess
          ? m2::launch_chunk_bwd_dbdc(d, x, dy, B, C, dA_cs, dt_T, hst, gst, wsum, rsum, dB, dC,
                                      th, s)
          : e;
  mark();
  // above N = 256 the state term of dU is formed first, into the float32
  // state slot (no longer read once the reverse pass has run; it holds
  // P N >= Q P floats per (chunk, head))
  float* dus = nullptr;
  if (m2::backward_state_term_separate(d)) {
    dus = st;
    e = e == hipSuccess ? m2::launch_chunk_bwd_dus(d, B, gst, dus, s) : e;
  }
  e = e == hipSuccess ? m2::launch_chunk_bwd_dx(d, x, dy, B, C, dA_cs, dt_T, gst, dots,
                                                (int)w.wph, th, rsum, A, D, dx, ddt, dA_part,
                                                dD_part, dus, s)
                      : e;
  mark();
  e = e == hipSuccess ? m2::launch_bwd_param_sums(d, dA_part, dD_part, dA, D ? dD : nullptr, s)
                      : e;
  mark();
  return hip_status(e, "backward launch");
}

int check_backward_args(const mamba2_dims* dims, m2::Dims* d, const void* x, const void* dt,
                        const float* A, const void* B, const void* C, const float* D,
                        const float* init_state, const void* dy, const float* dfinal,
                        void* dx, void* ddt, float* dA, void* dB, void* dC, float* dD,
                        float* dinit, void* workspace, size_t workspace_bytes) {
  CHECK(validate(dims, d));
  CHECK(need(x, "x"));
  CHECK(need(dt, "dt"));
  CHECK(need(A, "A"));
  CHECK(need(B, "B"));
  CHECK(need(C, "C"));
  CHECK(maybe(D, "D"));
  CHECK(maybe(init_state, "init_state"));
  CHECK(need(dy, "dy"));
  CHECK(maybe(dfinal, "dfinal"));
  CHECK(need(dx, "dx"));
  CHECK(need(ddt, "ddt"));
  CHECK(need(dA, "dA"));
  CHECK(need(dB, "dB"));
  CHECK(need(dC, "dC"));
  if (D) CHECK(need(dD, "dD"));
  CHECK(maybe(dinit, "dinit"));
  const BwdWorkspace w = plan_backward(*d);
  if (w.fast && w.wph > 128)  // the dx kernel's LDS holds at most 128 boundary parts
    return fail(MAMBA2_ERR_UNSUPPORTED, "state too large for the backward pass");
  if (!workspace) return fail(MAMBA2_ERR_WORKSPACE, "workspace is NULL");
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(MAMBA2_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < w.total)
    return fail(MAMBA2_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes,
                w.total);
  return MAMBA2_OK;
}

}  // namespace

extern "C" {

int mamba2_fwd_pass_state(const mamba2_dims* dims, const void* x, const void* B,
                          const float* dA_cs, const float* dt_T, const float* init_state,
                          float* w_T, void* chunk_start_states, float* final_state,
                          void* stream) {
  m2::Dims d;
  CHECK(validate(dims, &d));
  if (!m2::fused_state_supported(d))
    return fail(MAMBA2_ERR_UNSUPPORTED,
                "fwd_pass_state needs bfloat16, headdim 64, dstate 64/128/256 and chunk_size "
                "64/128/256");
  CHECK(need(x, "x"));
  CHECK(need(B, "B"));
  CHECK(need(dA_cs, "dA_cs"));
  CHECK(need(dt_T, "dt_T"));
  CHECK(maybe(init_state, "init_state"));
  CHECK(need(w_T, "w_T"));
  CHECK(need(chunk_start_states, "chunk_start_states"));
  CHECK(need(final_state, "final_state"));
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = m2::launch_chunk_weights(d, dA_cs, dt_T, w_T, s);
  if (e == hipSuccess)
    e = m2::launch_fwd_pass_state(d, x, B, dA_cs, w_T, init_state, chunk_start_states,
                                  final_state, s);
  return hip_status(e, "fwd_pass_state launch");
}

int mamba2_ssd_forward_fused(const mamba2_dims* dims, const void* x, const void* dt,
                             const float* A, const void* B, const void* C, const float* D,
                             const float* init_state, void* y, float* final_state,
                             void* workspace, size_t workspace_bytes, void* stream) {
  m2::Dims d;
  CHECK(check_forward_args(dims, &d, x, dt, A, B, C, D, init_state, y, final_state, workspace,
                           workspace_bytes));
  if (!m2::fused_state_supported(d))
    return fail(MAMBA2_ERR_UNSUPPORTED,
                "the one-kernel fwd_pass_state needs bfloat16, headdim 64, dstate 64/128/256 "
                "and chunk_size 64/128/256");
  if (!final_state) return fail(MAMBA2_ERR_NULL, "final_state is NULL");
  // workspace: dA_cs, dt_T, w_T [B,H,nc,Q] f32, then the bf16 chunk-start
  // states (inside the default forward's workspace size)
  const Workspace w = plan(d);
  char* ws = (char*)workspace;
  float* dA_cs = (float*)ws;
  float* dt_T = (float*)(ws + w.cs_bytes);
  float* w_T = (float*)(ws + 2 * w.cs_bytes);
  void* hst = ws + 3 * w.cs_bytes;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = m2::launch_chunk_cumsum(d, dt, A, dA_cs, dt_T, s);
  if (e == hipSuccess) e = m2::launch_chunk_weights(d, dA_cs, dt_T, w_T, s);
  if (e == hipSuccess)
    e = m2::launch_fwd_pass_state(d, x, B, dA_cs, w_T, init_state, hst, final_state, s);
  if (e == hipSuccess)
    e = m2::launch_chunk_scan_grouped(d, x, B, C, dA_cs, dt_T, hst, D, y, nullptr, s);
  return hip_status(e, "ssd_forward_fused launch");
}

size_t mamba2_ssd_backward_workspace_bytes(const mamba2_dims* dims) {
  m2::Dims d;
  if (validate(dims, &d) != MAMBA2_OK) return 0;
  return plan_backward(d).total;
}

int mamba2_ssd_backward(const mamba2_dims* dims, const void* x, const void* dt, const float* A,
                        const void* B, const void* C, const float* D, const float* init_state,
                        const void* dy, const float* dfinal, void* dx, void* ddt, float* dA,
                        void* dB, void* dC, float* dD, float* dinit, void* workspace,
                        size_t workspace_bytes, void* stream) {
  m2::Dims d;
  CHECK(check_backward_args(dims, &d, x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt, dA, dB,
                            dC, dD, dinit, workspace, workspace_bytes));
  return enqueue_backward(d, x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt, dA, dB, dC, dD,
                          dinit, workspace, (hipStream_t)stream, nullptr);
}

int mamba2_ssd_backward_profile(const mamba2_dims* dims, const void* x, const void* dt,
                                const float* A, const void* B, const void* C, const float* D,
                                const float* init_state, const void* dy, const float* dfinal,
                                void* dx, void* ddt, float* dA, void* dB, void* dC, float* dD,
                                float* dinit, void* workspace, size_t workspace_bytes,
                                void* stream, float* stage_ms) {
  m2::Dims d;
  CHECK(check_backward_args(dims, &d, x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt, dA, dB,
                            dC, dD, dinit, workspace, workspace_bytes));
  if (!stage_ms) return fail(MAMBA2_ERR_NULL, "stage_ms is NULL");
  hipEvent_t ev[kBwdStages + 1] = {};
  hipError_t e = hipSuccess;
  for (int i = 0; i <= kBwdStages && e == hipSuccess; ++i) e = hipEventCreate(&ev[i]);
  int rc = (e == hipSuccess) ? MAMBA2_OK : hip_status(e, "event create");
  if (rc == MAMBA2_OK)
    rc = enqueue_backward(d, x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt, dA, dB, dC, dD,
                          dinit, workspace, (hipStream_t)stream, ev);
  if (rc == MAMBA2_OK) {
    e = hipEventSynchronize(ev[kBwdStages]);
    for (int i = 0; i < kBwdStages && e == hipSuccess; ++i)
      e = hipEventElapsedTime(&stage_ms[i], ev[i], ev[i + 1]);
    rc = hip_status(e, "event timing");
  }
  for (int i = 0; i <= kBwdStages; ++i)
    if (ev[i]) (void)hipEventDestroy(ev[i]);
  return rc;
}


int mamba2_validate(const mamba2_dims* dims) {
  CHECK(validate(dims, nullptr));
  return ok();
}

int mamba2_chunk_cumsum(const mamba2_dims* dims, const void* dt, const float* A, float* dA_cs,
                        float* dt_T, void* stream) {
  m2::Dims d;
  CHECK(validate(dims, &d));
  CHECK(need(dt, "dt"));
  CHECK(need(A, "A"));
  CHECK(need(dA_cs, "dA_cs"));
  CHECK(need(dt_T, "dt_T"));
  return hip_status(m2::launch_chunk_cumsum(d, dt, A, dA_cs, dt_T, (hipStream_t)stream),
                    "chunk_cumsum launch");
}

int mamba2_chunk_state(const mamba2_dims* dims, const void* x, const void* B, const float* dA_cs,
                       const float* dt_T, float* states, void* stream) {
  m2::Dims d;
  CHECK(validate(dims, &d));
  CHECK(need(x, "x"));
  CHECK(need(B, "B"));
  CHECK(need(dA_cs, "dA_cs"));
  CHECK(need(dt_T, "dt_T"));
  CHECK(need(states, "states"));
  const hipError_t e =
      m2::grouped_state_supported(d)
          ? m2::launch_chunk_state_grouped(d, x, B, dA_cs, dt_T, states, (hipStream_t)stream)
          : m2::launch_chunk_state(d, x, B, dA_cs, dt_T, states, (hipStream_t)stream);
  return hip_status(e, "chunk_state launch");
}

int mamba2_state_passing(const mamba2_dims* dims, float* states, const float* dA_cs,
                         const float* init_state, float* final_state, void* stream) {
  m2::Dims d;
  CHECK(validate(dims, &d));
  CHECK(need(states, "states"));
  CHECK(need(dA_cs, "dA_cs"));
  CHECK(maybe(init_state, "init_state"));
  CHECK(maybe(final_state, "final_state"));
  return hip_status(
      m2::launch_state_passing(d, states, dA_cs, init_state, final_state, (hipStream_t)stream),
      "state_passing launch");
}

int mamba2_chunk_scan(const mamba2_dims* dims, const void* x, const void* B, const void* C,
                      const float* dA_cs, const float* dt_T, const float* states, const float* D,
                      void* y, void* stream) {
  m2::Dims d;
  CHECK(validate(dims, &d));
  CHECK(need(x, "x"));
  CHECK(need(B, "B"));
  CHECK(need(C, "C"));
  CHECK(need(dA_cs, "dA_cs"));
  CHECK(need(dt_T, "dt_T"));
  CHECK(need(states, "states"));
  CHECK(maybe(D, "D"));
  CHECK(need(y, "y"));
  return hip_status(
      m2::launch_chunk_scan(d, x, B, C, dA_cs, dt_T, states, D, y, (hipStream_t)stream),
      "chunk_scan launch");
}

size_t mamba2_ssd_workspace_bytes(const mamba2_dims* dims) {
  m2::Dims d;
  if (validate(dims, &d) != MAMBA2_OK) return 0;
  return plan(d).total;
}

int mamba2_ssd_forward(const mamba2_dims* dims, const void* x, const void* dt, const float* A,
                       const void* B, const void* C, const float* D, const float* init_state,
                       void* y, float* final_state, void* workspace, size_t workspace_bytes,
                       void* stream) {
  m2::Dims d;
  CHECK(check_forward_args(dims, &d, x, dt, A, B, C, D, init_state, y, final_state, workspace,
                           workspace_bytes));
  return enqueue_forward(d, x, dt, A, B, C, D, init_state, y, final_state, workspace,
                         (hipStream_t)stream, nullptr);
}

int mamba2_ssd_forward_noalloc(const mamba2_dims* dims, const void* x, const void* dt,
                               const float* A, const void* B, const void* C, const float* D,
                               const float* init_state, void* y, float* final_state,
                               void* stream) {
  m2::Dims d;
  CHECK(validate(dims, &d));
  const size_t need_bytes = plan(d).total;
  if (need_bytes > MAMBA2_NOALLOC_SCRATCH_BYTES)
    return fail(MAMBA2_ERR_WORKSPACE,
                "these sizes need %zu bytes of workspace; the static scratch holds %zu",
                need_bytes, (size_t)MAMBA2_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  CHECK(scratch_on_current_device(&ws));
  CHECK(check_forward_args(dims, &d, x, dt, A, B, C, D, init_state, y, final_state, ws,
                           MAMBA2_NOALLOC_SCRATCH_BYTES));
  return enqueue_forward(d, x, dt, A, B, C, D, init_state, y, final_state, ws,
                         (hipStream_t)stream, nullptr);
}

int mamba2_ssd_forward_profile(const mamba2_dims* dims, const void* x, const void* dt,
                               const float* A, const void* B, const void* C, const float* D,
                               const float* init_state, void* y, float* final_state,
                               void* workspace, size_t workspace_bytes, void* stream,
                               float* stage_ms) {
  m2::Dims d;
  CHECK(check_forward_args(dims, &d, x, dt, A, B, C, D, init_state, y, final_state, workspace,
                           workspace_bytes));
  if (!stage_ms) return fail(MAMBA2_ERR_NULL, "stage_ms is NULL");
  hipEvent_t ev[5] = {};
  hipError_t e = hipSuccess;
  for (int i = 0; i < 5 && e == hipSuccess; ++i) e = hipEventCreate(&ev[i]);
  int rc = (e == hipSuccess) ? MAMBA2_OK : hip_status(e, "event create");
  if (rc == MAMBA2_OK)
    rc = enqueue_forward(d, x, dt, A, B, C, D, init_state, y, final_state, workspace,
                         (hipStream_t)stream, ev);
  if (rc == MAMBA2_OK) {
    e = hipEventSynchronize(ev[4]);
    for (int i = 0; i < 4 && e == hipSuccess; ++i) e = hipEventElapsedTime(&stage_ms[i], ev[i], ev[i + 1]);
    rc = hip_status(e, "event timing");
  }
  for (int i = 0; i < 5; ++i)
    if (ev[i]) (void)hipEventDestroy(ev[i]);
  return rc;
}

int mamba2_decode_step(const mamba2_dims* dims, const void* x, const void* dt, const float* A,
                       const void* B, const void* C, const float* D, float* state, void* y,
                       void* stream) {
  m2::Dims d;
  CHECK(validate(dims, &d));
  if (d.L != 1)
    return fail(MAMBA2_ERR_SHAPE, "decode_step advances one token: seqlen must be 1 (got %lld)",
                (long long)d.L);
  CHECK(need(x, "x"));
  CHECK(need(dt, "dt"));
  CHECK(need(A, "A"));
  CHECK(need(B, "B"));
  CHECK(need(C, "C"));
  CHECK(maybe(D, "D"));
  CHECK(need(state, "state"));
  CHECK(need(y, "y"));
  return hip_status(m2::launch_decode_step(d, x, dt, A, B, C, D, state, y, (hipStream_t)stream),
                    "decode_step launch");
}

const char* mamba2_status_string(int status) {
  switch (status) {
    case MAMBA2_OK: return "ok";
    case MAMBA2_ERR_NULL: return "a required pointer is NULL";
    case MAMBA2_ERR_SHAPE: return "invalid sizes";
    case MAMBA2_ERR_DTYPE: return "unknown dtype";
    case MAMBA2_ERR_UNSUPPORTED: return "sizes not supported by this library";
    case MAMBA2_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MAMBA2_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MAMBA2_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

const char* mamba2_last_error(void) { return g_last_error; }

}  // extern "C"
