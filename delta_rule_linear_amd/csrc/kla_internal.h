// Internal launcher interface between the C-ABI layer (kla_api.cpp) and the
// HIP kernel translation units.  Arguments are already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kla {

struct PrefillArgs {
  const void *q, *k, *v;
  // bf16 prefill only, nullable: the lo plane of a split query (q + q_lo)
  const void *q_lo = nullptr;
  const float *alpha, *eta;   // alpha nullable (alpha = 1)
  const int32_t *cu_seqlens;  // device, or nullptr for dense
  int32_t n_seqs;
  int64_t seq_len_dense;      // tokens per sequence when cu_seqlens == nullptr
  int32_t H, D;               // D = dk = dv
  float eps;
  int beta_direct;            // 1: beta = eta; 0: beta = eta / (|k|^2 + eps)
  const float *initial_state; // nullable
  float *o;
  float *final_state;         // nullable
  // split-sequence passes (0: whole sequences; 1: segment maps; 2: outputs)
  int seg_mode = 0;
  int n_splits = 1;
  float *ws_a = nullptr, *ws_b = nullptr;  // [n_seqs, H, P-1, D, D]
  const float *ws_s = nullptr;             // [n_seqs, H, P, D, D]
  float *ws_ckpt = nullptr;                // states-only pass: chunk-start state slots
  // bf16 prefill: 1 stores o write-back (for a caller that reads it straight
  // back); 0 stores it non-temporal (the output is not read by this work)
  int o_write_back = 0;
  // whole-sequence passes: sequence indices by decreasing length (device,
  // written by launch_seq_order), or null for the given order
  const int32_t *seq_order = nullptr;
};

struct DecodeArgs {
  const void *q, *k, *v;
  const float *alpha, *eta;   // alpha nullable (alpha = 1)
  float *state, *o;
  int32_t n_seqs, H, D;
  float eps;
  int beta_direct;            // 1: beta = eta; 0: beta = eta / (|k|^2 + eps)
  int channel_decay = 0;      // 1: alpha [n_seqs, H, D], one decay per key channel
};

// Curvature-conditioned read: query cleaning before the KLA read.
struct CcqArgs {
  const void *q, *k;          // [tokens, H, D], bf16 or fp32
  const float *lambda;        // [tokens, H]
  const int32_t *cu_seqlens;  // prefill only (nullptr: dense)
  int32_t n_seqs;
  int64_t seq_len_dense;
  int32_t H, D;
  bool bf16_inputs;
  const float *ccq_in;        // prefill: start sums or nullptr
  float *ccq_out;             // end sums or nullptr
  void *qh, *ql;              // cleaned query: fp32 in qh, or bf16 hi / lo planes (bf16)
  // bf16 only, nullable: [total_tok, H, D] fp32 scratch (free during the
  // pass) for the sums of the first halves of long sequences; when set, each
  // long sequence is cleaned as two halves in parallel
  float *half_sums = nullptr;
};

// Curvature-conditioned decode step, one kernel: the sums take the new key,
// q_clean is formed (and written to q_clean), and the KLA decode step reads
// with it.
struct CcqDecodeArgs {
  const void *q, *k, *v;               // [n_seqs, H, D], bf16 or fp32
  const float *lambda, *alpha, *eta;   // [n_seqs, H]; alpha nullable (alpha = 1)
  float *ccq_state;                    // the sums, updated in place
  float *state, *o;                    // fp32 state (in place), o [n_seqs, H, D]
  float *q_clean;                      // [n_seqs, H, D] fp32
  int32_t n_seqs, H, D;
  float eps;
  int beta_direct;
  bool bf16_inputs;
};

// Backward of the prefill (gradients of o and of the final state).
struct BwdParams {
  const void *q, *k, *v;      // [total_tok, H, D], bf16 or fp32
  const float *alpha, *eta;   // alpha nullable (alpha = 1)
  const int32_t *cu_seqlens;  // device, or nullptr for dense
  int32_t n_seqs;
  int64_t seq_len_dense;
  int64_t total_tok;
  int32_t H, D;
  float eps;
  int beta_direct;
  const float *initial_state;  // nullable
  const float *d_o;            // [total_tok, H, D] fp32
  const float *d_final;        // nullable
  float *dq, *dk, *dv;         // [total_tok, H, D] fp32
  float *d_alpha;              // [total_tok, H], written when alpha is set
  float *d_eta;                // [total_tok, H]
  float *d_initial;            // nullable
  // workspace: chunk-start states [floor(tok/64) + n_seqs, H, D, D], the
  // column slices' dq, dk [D/16, tok, H, D], dbeta, c [D/16, tok, H], |k|^2 [tok, H]
  float *ws_ckpt, *ws_dq, *ws_dk, *ws_db, *ws_c, *ws_kk;
  // final states [n_seqs, H, D, D]; when set, ws_ckpt already holds the
  // chunk-start states (written by the states-only prefill) and the
  // backward kernel skips its own forward sweep
  float *ws_fin = nullptr;
};

// Each returns the HIP status of the launch.
// order[0..n_seqs) <- the sequences of cu_seqlens by decreasing length
// (ties by index); n_seqs <= kla::kSeqOrderMax.
constexpr int kSeqOrderMax = 1024;
hipError_t launch_seq_order(const int32_t *cu_seqlens, int n_seqs, int32_t *order, hipStream_t s);
hipError_t launch_prefill_bf16(const PrefillArgs &a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs &a, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs &a, hipStream_t s);
// Split-sequence helpers: ws_a <- identity per (sequence, head, segment <
// P-1); then the scan S_0 = initial state (or 0), S_{p+1} = A_p S_p + B_p,
// written to ws_s for p = 0..P-1.
hipError_t launch_split_identity(const PrefillArgs &a, hipStream_t s);
hipError_t launch_split_scan(const PrefillArgs &a, hipStream_t s);
// Device address, on the current device, of the library's static scratch
// array (KLA_NOALLOC_SCRATCH_BYTES, kla_split.hip), taken once per device
// with hipGetSymbolAddress and kept.
hipError_t noalloc_scratch(void **ptr);
hipError_t launch_decode_f32(const DecodeArgs &a, hipStream_t s);
// CCQ: the prefill pre-pass (q_clean for every token) and the fused decode
// step.
hipError_t launch_ccq_query(const CcqArgs &a, hipStream_t s);
hipError_t launch_ccq_decode_step(const CcqDecodeArgs &a, hipStream_t s);
// Per-channel decay prefill (alpha [total_tok, H, D]); whole sequences only.
hipError_t launch_prefill_kda(const PrefillArgs &a, bool bf16_inputs, hipStream_t s);
// bf16 prefill without output (whole sequences): every chunk-start state to
// its slot of ws_ckpt (sequence s, chunk c: slot floor(bos_s / 64) + s + c,
// each [H, D, D]) and the final state to final_state.  o is not written.
hipError_t launch_prefill_states(const PrefillArgs &a, hipStream_t s);
// Backward: the two-sweep kernel, then the reduction over column slices.
hipError_t launch_bwd(const BwdParams &p, bool bf16_inputs, hipStream_t s);

}  // namespace kla
