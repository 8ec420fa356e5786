// Host-side launchers of the SSD kernels.  Sizes are validated by the C ABI
// layer before any of these is called; each launcher only enqueues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m2 {

struct Dims {
  int64_t B, L, H, P, N, G, Q, nc;
  bool bf16;
};

hipError_t launch_chunk_cumsum(const Dims& d, const void* dt, const float* A, float* dA_cs,
                               float* dt_T, hipStream_t s);
hipError_t launch_chunk_state(const Dims& d, const void* x, const void* B, const float* dA_cs,
                              const float* dt_T, float* states, hipStream_t s);
hipError_t launch_state_passing(const Dims& d, float* states, const float* dA_cs,
                                const float* init, float* final_state, hipStream_t s);
hipError_t launch_chunk_scan(const Dims& d, const void* x, const void* B, const void* C,
                             const float* dA_cs, const float* dt_T, const float* states,
                             const float* D, void* y, hipStream_t s);

// Fused-forward variants: state_passing that leaves the chunk-start states as
// bfloat16 in a separate buffer (the float32 per-chunk states are read once),
// and the grouped chunk_scan that consumes them.
hipError_t launch_state_passing_bf16(const Dims& d, const float* states, const float* dA_cs,
                                     const float* init, void* hst, float* final_state,
                                     hipStream_t s);
bool grouped_scan_supported(const Dims& d);
bool grouped_state_supported(const Dims& d);
hipError_t launch_chunk_state_grouped(const Dims& d, const void* x, const void* B,
                                      const float* dA_cs, const float* dt_T, float* states,
                                      hipStream_t s);
// State size 512 runs as two passes over column halves and needs `part`, a
// bfloat16 [B, L, H, P] scratch of grouped_scan_part_bytes(d) (else NULL).
size_t grouped_scan_part_bytes(const Dims& d);
hipError_t launch_chunk_scan_grouped(const Dims& d, const void* x, const void* B, const void* C,
                                     const float* dA_cs, const float* dt_T, const void* hst,
                                     const float* D, void* y, void* part, hipStream_t s);

// Backward pass (bfloat16, P = 64, N in {64, 128, 256}, Q in {64, 128, 256}).
bool backward_supported(const Dims& d);
// E[B,nc,H,P,N] f32: per-chunk adjoint states sum_i 2^cs_i dy_i C_i^T.
hipError_t launch_chunk_state_adjoint(const Dims& d, const void* dy, const void* C,
                                      const float* dA_cs, const float* dt_T, float* states,
                                      hipStream_t s);
// Reverse jump over E: gst[B,nc,H,P,N] bf16 (gradient at each chunk's end),
// dh0 (nullable), dots[B,H,nc,wph] (parts of 2^cs_last <g_c, h_c>).
int64_t state_reverse_waves_per_head(const Dims& d);
hipError_t launch_state_passing_reverse(const Dims& d, const float* E, const float* dA_cs,
                                        const float* dfinal, const void* hst, void* gst,
                                        float* dh0, float* dots, hipStream_t s);
// dB, dC, and th[B,nc,H,N/64,Q]: per state-column tile parts of
// 2^cs_i dy_i . (h_c C_i), the carried-state term of y_i weighted by dy_i.
// wsum: [B,nc,G] blocks of Q(Q+16)/2 bf16 (the group's summed W triangle);
// rsum [B,H,nc,Q] f32: the rectangle sums of the log-decay gradient.
hipError_t launch_chunk_bwd_dbdc(const Dims& d, const void* x, const void* dy, const void* B,
                                 const void* C, const float* dA_cs, const float* dt_T,
                                 const void* hst, const void* gst, void* wsum, float* rsum,
                                 void* dB, void* dC, float* th, hipStream_t s);
hipError_t launch_chunk_bwd_dx(const Dims& d, const void* x, const void* dy, const void* B,
                               const void* C, const float* dA_cs, const float* dt_T,
                               const void* gst, const float* dots, int wph, const float* th,
                               const float* rsum, const float* A, const float* D, void* dx,
                               void* ddt, float* dA_part, float* dD_part, const float* dus,
                               hipStream_t s);
// Above N = 256 (backward_state_term_separate): the state term of dU before
// its row decay, dus[B,L,H,P] f32 = B g^T per (chunk, head), which
// launch_chunk_bwd_dx then reads (dus non-NULL) instead of forming it.
bool backward_state_term_separate(const Dims& d);
hipError_t launch_chunk_bwd_dus(const Dims& d, const void* B, const void* gst, float* dus,
                                hipStream_t s);
hipError_t launch_bwd_param_sums(const Dims& d, const float* dA_part, const float* dD_part,
                                 float* dA, float* dD, hipStream_t s);

// Backward pass for the sizes backward_supported() rejects (chunk_bwd_generic.hip):
// float32 arithmetic on the vector ALU, any size the forward accepts with
// Q <= 256.  hs: the float32 chunk-start states [B,nc,H,P,N] (from
// chunk_state + state_passing); E: [B,nc,H,P,N] float32 scratch (left holding
// the gradient at every chunk end); the scratch below in float32 elements.
struct GenericBwdSizes {
  size_t vg, thp, xup, ghp, cb, part;
};
GenericBwdSizes generic_backward_sizes(const Dims& d);
struct GenericBwdScratch {
  float *vg, *thp, *xup, *ghp, *cb, *dA_part, *dD_part;
};
hipError_t launch_backward_generic(const Dims& d, const void* x, const void* dy, const void* B,
                                   const void* C, const float* dA_cs, const float* dt_T,
                                   float* hs, float* E, const float* dfinal, float* dinit,
                                   const float* A, const float* D, void* dx, void* ddt, void* dB,
                                   void* dC, const GenericBwdScratch& w, hipStream_t s);

// fwd_pass_state as one kernel (bfloat16, P = 64, N in {64, 128, 256},
// Q in {64, 128, 256}): chunk-start states to hst (bf16 [B,nc,H,P,N]) and the
// final state, from the weights w_T = 2^(cs_last - cs_j) dt_j [B,H,nc,Q].
// fwd_pass_state over spans of chunks (state_span.hip): span_chunks gives the
// span length K (0 = this path does not apply to these sizes).  span_states
// [B, ng, H, P, N] float32 and span_decay [B, H, ng] are scratch
// (ng = ceil(nc / K)); hst receives the bfloat16 chunk-start states.  `mid`
// (may be null) is recorded after the span-end kernel.
int span_chunks(const Dims& d);
size_t span_states_bytes(const Dims& d, int K);
// replay = false stops after the jump across spans (span_states then hold
// every span's start state, for span_scan).
hipError_t launch_fwd_pass_state_span(const Dims& d, int K, const void* x, const void* B,
                                      const float* dA_cs, const float* dt_T, const float* init,
                                      float* span_states, float* span_decay, void* hst,
                                      float* final_state, hipStream_t s, hipEvent_t mid,
                                      bool replay);

// span_scan (span_scan.hip): the replay of each span fused with compute_out,
// from the span start states the jump leaves in span_states; y only.
// span_scan_heads gives the heads per workgroup (0 = not covered: the replay
// and the grouped chunk_scan run instead).
int span_scan_heads(const Dims& d, int K);
// The forward's span length where span_scan runs (0 = span_chunks decides).
int span_scan_chunks(const Dims& d);
hipError_t launch_span_scan(const Dims& d, int K, int R, const void* x, const void* B,
                            const void* C, const float* dA_cs, const float* dt_T,
                            const float* span_states, const float* D, void* y, hipStream_t s);

bool fused_state_supported(const Dims& d);
hipError_t launch_chunk_weights(const Dims& d, const float* dA_cs, const float* dt_T, float* w_T,
                                hipStream_t s);
hipError_t launch_fwd_pass_state(const Dims& d, const void* x, const void* B, const float* dA_cs,
                                 const float* w_T, const float* init, void* hst,
                                 float* final_state, hipStream_t s);

// One-token recurrent step, in place on the float32 state [B,H,P,N];
// x, y [B,H,P], dt [B,H], B, C [B,G,N].
hipError_t launch_decode_step(const Dims& d, const void* x, const void* dt, const float* A,
                              const void* B, const void* C, const float* D, float* state,
                              void* y, hipStream_t s);

}  // namespace m2
