// Internal launch interface between the C ABI (api.hip) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Gate inputs: when A is null, log_alpha and beta hold log alpha and beta;
// otherwise they hold the raw pre-activations a and b, turned into gates
// in-kernel with the per-head A and b_alpha (b_alpha may be null: zero).
//
// Decode: n_tok tokens per (sequence, head), applied in order. Token inputs
// are [N, n_tok, H, d]. State slots: sequence n reads slot
// read_idx[n * r_stride] (read_idx null: slot n). write_idx null: the final
// state goes back to the slot it came from; otherwise the state after token
// j goes to slot write_idx[n * w_stride + j] when that is in [0, n_slots)
// and is not written elsewhere. A read slot outside [0, n_slots) marks a
// padding entry: nothing is written but y = 0.
struct DecodeArgs {
  const void *q, *k, *v;
  const float *log_alpha, *beta;
  const float *A = nullptr, *b_alpha = nullptr;
  float *S;
  const int32_t *read_idx = nullptr;
  int r_stride = 1;
  const int32_t *write_idx = nullptr;
  int w_stride = 1;
  int n_slots = 0;
  void *y;
  int N, H, dk, dv;
  int n_tok = 1;
  int in_dtype, out_dtype;  // 0 = f32, 1 = bf16, 2 = f16
  hipStream_t stream;
  // Fused decode only (front end and output gate in the same kernel): q, k,
  // v are then the raw projections, y receives o, and conv_state holds per
  // slot and head the three previous raw rows of each stream,
  // [slots, H, 3 (q, k, v), 3 (oldest first), d] in in_dtype, read from the
  // start slot and written wherever the state is.
  const float *conv_w = nullptr;  // [3][H*d][4]
  void *conv_state = nullptr;
  const void *z = nullptr;        // [N, n_tok, H, d] in in_dtype
  const float *norm_w = nullptr;  // [d] or null
  float l2_eps = 0.0f, rms_eps = 0.0f;
};

// most tokens one decode call applies per (sequence, head)
constexpr int kDecodeMaxTok = 8;

// Controls for the runs of the segment-parallel prefill, whose "sequences"
// are segments; the defaults make every sequence an ordinary prefill. All
// are uniform per workgroup.
struct SegCtl {
  int y_nseq = 0x7fffffff;   // sequences n < y_nseq write y
  int s0_nseq = 0x7fffffff;  // sequences n < s0_nseq start from S0[n], the others from zero
  int s0_ident = 0;          // every sequence starts from the identity (dk == dv)
  int v_zero = 0;            // v is read as zeros (the pointer is still a valid buffer)
  int st_first = 0;          // sequences n >= st_first write S_T[n - st_first]
  bool plain() const {
    return y_nseq == 0x7fffffff && s0_nseq == 0x7fffffff && !s0_ident && !v_zero && !st_first;
  }
};

struct ChunkArgs {
  const void *q, *k, *v;
  const float *log_alpha, *beta;
  const float *A = nullptr, *b_alpha = nullptr;
  const float *S0;  // may be null (zeros)
  void *y;
  float *S_T;       // may be null
  const int32_t *cu_seqlens;  // may be null
  int N, T, H, dk, dv;
  int in_dtype, out_dtype;
  hipStream_t stream;
  // launch_chunk_fwd_states only: chunk-start states in the backward
  // workspace's tile order
  float *states = nullptr;
  SegCtl seg;
};

struct FrontendArgs {
  const void *xq, *xk, *xv;  // raw projections [rows, H, d]
  const float *conv_w;       // [3][H*d][4]
  const int32_t *cu_seqlens; // may be null
  int N, T;                  // sequences; tokens per sequence when cu_seqlens is null
  int64_t rows;
  int H, d;
  float eps;
  void *q, *k, *v;
  int in_dtype, out_dtype;
  hipStream_t stream;
};

struct GateArgs {
  const void *y, *z;  // [rows, d]
  const float *norm_w;  // [d] or null
  float eps;
  void *o;
  int64_t rows;
  int d;
  int in_dtype, z_dtype, out_dtype;
  hipStream_t stream;
};

// Chunked backward pass: gradients of <dy, y> + <dS_T, S_T>.
struct BwdArgs {
  const void *q, *k, *v;          // in_dtype
  const float *log_alpha, *beta;
  const float *S0;                // may be null (zeros)
  const void *dy;                 // grad_dtype, [rows, H, dv]
  const float *dS_T;              // may be null (zeros)
  const int32_t *cu_seqlens;      // may be null
  int N, T, H, dk_size, dv_size;
  int64_t rows;
  void *dq, *dk, *dv;             // grad_dtype
  float *dlog_alpha, *dbeta;      // [rows, H]
  float *dS0;                     // may be null
  float *ws_states, *ws_part;     // workspace (see chunk_bwd_workspace_size)
  // Runs: the sweep, reduction and head sums run `runs` times, run = runs - 1
  // first. With run_rows == 0 run j covers chunks floor(j nc / runs) ..
  // floor((j + 1) nc / runs) - 1 of every sequence (nc its chunk count), so
  // that every run has work for every long sequence; otherwise it covers the
  // chunks whose first row lies in [j run_rows, (j + 1) run_rows). A run's
  // partial sums are kept for part_rows rows, sequence after sequence: with
  // one run at the sequence's own rows, else from sequence n's offset in
  // row j of run_off ([runs][N + 1], the last entry the run's row count;
  // varlen) or from n times the run's common row count (equal lengths).
  // ws_carry holds the state gradient of every (sequence, head, column
  // tile) from one run to the next.
  int runs = 1, run = 0;
  int64_t run_rows = 0;
  int32_t *run_off = nullptr;
  int64_t part_rows = 0;
  float *ws_carry = nullptr;
  // raw gates: log_alpha / beta then hold a / b, dlog_alpha / dbeta receive
  // da / db, and dA, db_alpha [H] the per-head sums
  const float *A = nullptr, *b_alpha = nullptr;
  float *dA = nullptr, *db_alpha = nullptr;
  int in_dtype, grad_dtype;
  hipStream_t stream;
};

// Convolution cache of the fused decode from a prefill's raw projections.
struct ConvStateArgs {
  const void *xq, *xk, *xv;       // raw projections [rows, H, d]
  const int32_t *cu_seqlens;      // may be null
  const int32_t *slot_idx;        // [N] or null (slot n)
  int N, T, H, d, n_slots;
  int elem_bytes;
  void *conv_state;               // [n_slots, H, 3, 3, d]
  hipStream_t stream;
};

hipError_t launch_conv_state(const ConvStateArgs &a);

// Bookkeeping of the segment-parallel prefill (segment.hip): segment bounds
// (N x (P + 1)), initial states of the zero-start runs (N x (P - 1) states,
// the first of each sequence the caller's S0), n_ident identity matrices and
// vzero_bytes of zeros (the values of the transition runs).
struct SegPrepArgs {
  const int32_t *cu_seqlens;  // may be null
  int N, T, P;
  int32_t *cu_seg;            // [N][P + 1] segment bounds
  hipStream_t stream;
};
hipError_t launch_seg_prep(const SegPrepArgs &a);
// The chain of one sequence's segment summaries into initial states.
hipError_t launch_seg_combine(const float *Nst, const float *Mst, float *Sin, int H, int dk,
                              int dv, int P, hipStream_t stream);
hipError_t launch_decode_step(const DecodeArgs &a);
hipError_t launch_chunk_bwd(const BwdArgs &a);
size_t chunk_bwd_workspace_size(int64_t rows, int N, int H, int dk, int dv, int in_dtype);
size_t chunk_bwd_states_bytes(int64_t rows, int N, int H, int dk, int dv, int in_dtype);
// Runs of the backward sweep (see BwdArgs::runs).
struct BwdSegPlan {
  int runs;           // number of runs
  int64_t run_rows;   // 0: proportional runs; else rows per run
  int64_t part_rows;  // rows of partial sums kept per run
};
BwdSegPlan bwd_seg_plan(int64_t rows, int N, int H, int dk, int dv);
// byte offsets of the workspace's parts: partial sums, carried state
// gradients, run offsets (each 256-byte aligned)
struct BwdLayout {
  size_t part, carry, table, total;
};
BwdLayout chunk_bwd_layout(int64_t rows, int N, int H, int dk, int dv, int in_dtype);
hipError_t launch_decode_fused(const DecodeArgs &a);  // dk == dv
hipError_t launch_frontend(const FrontendArgs &a);
hipError_t launch_output_gate(const GateArgs &a);
hipError_t launch_chunk_fwd(const ChunkArgs &a);      // dispatches on in_dtype
hipError_t launch_chunk_fwd_f32(const ChunkArgs &a);  // fp32 inputs
hipError_t launch_chunk_fwd_bf16(const ChunkArgs &a); // bf16 inputs
// 16-bit inputs: chunk-start states only (a.states; y and S_T not written)
hipError_t launch_chunk_fwd_states(const ChunkArgs &a);
// state columns per workgroup of the plain prefill for a's shape and dtype
int chunk_fwd_state_columns(const ChunkArgs &a);

}  // namespace gdn
