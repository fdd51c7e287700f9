// KLA chunkwise-parallel prefill for gfx950 (CDNA4).
//
// Method: the KLA technical summary ("Resumo Tecnico: Atencao Linear
// Kaczmarz (KLA)", gist.science/pt/paper/2605.08587) keeps Gated
// DeltaNet's chunk-parallel algorithm and changes only the diagonal
// coefficient matrix B = Diag(beta) of the chunk solver (section
// "Implementacao"), with beta_t = eta_t / (|k_t|^2 + eps) (section
// "A Regra de Atualizacao KLA").  With beta_direct the step is beta_t =
// eta_t, the learned scalar of Gated DeltaNet that KLA replaces (same
// summary, introduction); without alpha the decay is 1 (DeltaNet, "Linear
// Attention Architectures: Mechanisms, Trade-offs, and Cross-Layer Routing",
// section "Notacao Unificada").  For a chunk of n <= 64 tokens with
// chunk-start state S (dk x dv), g_r = sum_{i<=r} log alpha_i:
//
//   L     = strictly-lower( Diag(beta) (K K^T o Gam) ),  Gam_rs = e^{g_r-g_s}
//   T     = (I + L)^{-1} Diag(beta)                      (UT transform)
//   R     = V - Diag(e^g) K S                            (residual vs S)
//   Delta = T R
//   O     = Diag(e^g) Q S + lower(Q K^T o Gam) Delta
//   S'    = e^{g_n} S + K^T Diag(e^{g_n - g}) Delta
//
// This is the WY form U - W S with U = T V, W = T Diag(e^g) K, regrouped so
// W is never formed (one dk-long contraction less per chunk).  T itself is
// never formed either: with 16-row blocks b, Ahat = K K^T o Gam and
// Y_bb = (I + Diag(beta_b) Ahat_bb)^{-1} Diag(beta_b) (a 16x16 block inverse),
// Delta follows by block forward substitution
//   Delta_b = Y_bb (R_b - sum_{m<b} Ahat_bm Delta_m),
// which is (I + L) Delta = Diag(beta) R solved blockwise.
//
// Mapping.  One workgroup of 4 waves per (sequence, head, 64-column block of
// dv); each wave owns 16 columns of the state and keeps them in MFMA
// accumulator registers for the whole sequence.  Per chunk:
//   1. all waves stage K, Q, V in LDS; row norms |k|^2 are reduced on the way
//      in and wave 0 scans the log-decays;
//   2. wave 0 computes the diagonal K K^T tiles and inverts the four 16x16
//      diagonal blocks, while waves 1-3 compute the other Gram tiles; then
//      every wave forms Q S, K S and R for its columns;
//   3. every wave runs the substitution for Delta, the output, and the
//      state update on its own columns.
// A state (or Delta) tile in accumulator layout feeds the next MFMA directly
// as its B operand: the contraction index is permuted consistently on the A
// side, so those tiles never go through LDS.  K^T for the state update is
// read from the row-major K tile with the transposing LDS read.
//
// Precision.  bf16 inputs enter MFMA exactly.  Every fp32 intermediate
// (S, R, Y, Ahat, M, Delta) enters as a hi+lo pair of bf16
// (x = hi + lo + O(2^-17 x)); products of two split operands use
// hi*hi + hi*lo + lo*hi.  fp32 inputs use the fp32 MFMA
// (v_mfma_f32_16x16x4_f32) throughout.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kla_device.h"
#include "kla_internal.h"

namespace kla {
namespace {

template <typename E, int D>
struct Cfg {
  static constexpr bool BF = std::is_same<E, bf16>::value;
  using P = typename std::conditional<BF, bf16, float>::type;  // operand-plane type
  static constexpr int LDK = D + (BF ? 8 : 4);    // K, Q rows (elements)
  static constexpr int LDV = DVB + (BF ? 8 : 4);  // V rows
  static constexpr int LDP = BF ? C + 8 : C + 4;  // Ahat, M operand planes (64x64)
  static constexpr int LDY = 20;                  // Y diagonal blocks (16x16)
  static constexpr int NST = D / 16;              // state tiles per wave (dk direction)
};

template <typename E, int D>
struct Smem {
  using CF = Cfg<E, D>;
  using P = typename CF::P;
  // Every member starts on a 16-byte boundary (128-bit LDS accesses).
  alignas(16) E Kr[C * CF::LDK];
  alignas(16) E Qr[C * CF::LDK];
  alignas(16) E Vs[C * CF::LDV];
  alignas(16) P Ah[C * CF::LDP];  // -Ahat below the block diagonal
  alignas(16) P Al[CF::BF ? C * CF::LDP : 8];
  alignas(16) P Mh[C * CF::LDP];  // M = lower(Q K^T o Gam)
  alignas(16) P Ml[CF::BF ? C * CF::LDP : 8];
  alignas(16) P Yh[4 * 16 * CF::LDY];
  alignas(16) P Yl[CF::BF ? 4 * 16 * CF::LDY : 8];
  alignas(16) float Ld[4 * 16 * 20];  // -Diag(beta) Ahat below the diagonal of the diagonal blocks, [block][col][row]
  alignas(16) float kk[C];
  alignas(16) float et[C];
  alignas(16) float beta[C];
  alignas(16) float g2[C];    // cumulative log2 decay
  alignas(16) float gam[C];   // 2^g2
  alignas(16) float rgam[C];  // 2^(g2_last - g2)
};

// A operand matching join()'s row order: from a row-major source row
// (pointer at column kb), columns kb+4j..kb+4j+3 and kb+16+4j..kb+16+4j+3.
__device__ inline bf16x8 lda_perm(const bf16 *row, int j) {
  const bf16x4 x = *reinterpret_cast<const bf16x4 *>(row + 4 * j);
  const bf16x4 y = *reinterpret_cast<const bf16x4 *>(row + 16 + 4 * j);
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ inline bf16x4 lda4(const bf16 *p) { return *reinterpret_cast<const bf16x4 *>(p); }


__device__ inline void store_split(bf16 *h, bf16 *l, int idx, float x) {
  const bf16 hv = static_cast<bf16>(x);
  h[idx] = hv;
  l[idx] = static_cast<bf16>(x - static_cast<float>(hv));
}
__device__ inline void store_split(float *h, float *, int idx, float x) { h[idx] = x; }

// What one workgroup computes.  Mode 0: one (sequence, head, 64-column block
// of dv) over the whole sequence.  Mode 0 deals the (sequence, head) pairs
// out longest sequence first (sp.order: sequence indices by decreasing
// length, or null for the given order), round-robin over the eight XCDs:
// workgroup i runs on XCD i % 8, and the (i / 8)-th workgroup of an XCD
// takes column block (i / 8) % NB of pair 8 ((i / 8) / NB) + i % 8, so both
// column blocks of a pair share one XCD's L2 and each XCD gets an equal
// share of the long sequences.  The grid is padded to a multiple of 8 NB;
// the padding workgroups do nothing.  The split-sequence path cuts every
// sequence into n_splits segments on chunk boundaries; the state map of a
// segment is affine, S_end = A S_start + B, and the same kernels run it in
// two passes around a scan of those maps:
//   mode 1, segments 0..P-2: the state pass from the start [I | 0] with V
//     read as [0 | V].  Column blocks 0..NB-1 give A (start and end in ws_a,
//     set to I beforehand), blocks NB..2NB-1 give B (zero start, end in
//     ws_b).  No output.
//   mode 2, all segments: each from its start state in ws_s (written by the
//     scan), writing o; the last segment writes the final state.
//   mode 3, whole sequences, states only (the OUT = false instance): each
//     chunk-start state goes to its slot of ckpt (sequence s, chunk c: slot
//     floor(bos_s / 64) + s + c, each [H, D, D]) and the final state to Sfin.
struct SegParams {
  int mode, n_splits;
  int64_t n_pairs;       // n_seqs * H
  const int32_t *order;  // mode 0: sequences by decreasing length, or null
  float *ws_a, *ws_b;   // [n_seqs, H, P-1, D, D]
  const float *ws_s;    // [n_seqs, H, P, D, D]
  float *ckpt;          // mode 3: chunk-start state slots
  int o_wb;             // 1: o with write-back stores (read back right away), else non-temporal
};
struct Work {
  int h, nb, vb;        // head, state column block, V column block (-1: V read as zero)
  int64_t bos, eos;     // token range of this workgroup
  const float *s0;      // start state (D x D row-major) or null for zero
  float *sfin;          // end state destination or null
  float *ck;            // mode 3: this (sequence, head)'s first chunk-start slot
  bool out;             // write o
};
template <int NB, int D>
__device__ inline Work resolve_work(const SegParams &sp, const int32_t *cu_seqlens,
                                    int64_t seq_len_dense, int H, const float *S0, float *Sfin) {
  const int64_t lb = logical_block();
  const int P = sp.n_splits;
  Work wk;
  int64_t shi, p = 0;
  if (sp.mode == 0) {
    const int64_t kx = (int64_t)blockIdx.x / 8, pair = (kx / NB) * 8 + blockIdx.x % 8;
    wk.nb = wk.vb = (int)(kx % NB);
    wk.out = true;
    wk.ck = nullptr;
    if (pair >= sp.n_pairs) {  // grid padding: no tokens, no state
      wk.h = 0;
      wk.bos = wk.eos = 0;
      wk.s0 = nullptr;
      wk.sfin = nullptr;
      return wk;
    }
    const int64_t r = pair / H;
    wk.h = (int)(pair % H);
    const int64_t s = sp.order ? sp.order[r] : r, sh = s * H + wk.h;
    wk.bos = cu_seqlens ? cu_seqlens[s] : s * seq_len_dense;
    wk.eos = cu_seqlens ? cu_seqlens[s + 1] : wk.bos + seq_len_dense;
    constexpr int64_t DD0 = (int64_t)D * D;
    wk.s0 = S0 ? S0 + sh * DD0 : nullptr;
    wk.sfin = Sfin ? Sfin + sh * DD0 : nullptr;
    return wk;
  }
  if (sp.mode == 1) {
    const int cb = (int)(lb % (2 * NB));
    const int64_t r = lb / (2 * NB);
    p = r % (P - 1);
    shi = r / (P - 1);
    wk.nb = cb < NB ? cb : cb - NB;
    wk.vb = cb < NB ? -1 : cb - NB;
  } else {
    wk.nb = wk.vb = (int)(lb % NB);
    const int64_t r = lb / NB;
    p = sp.mode == 2 ? r % P : 0;
    shi = sp.mode == 2 ? r / P : r;
  }
  wk.h = (int)(shi % H);
  const int64_t s = shi / H, sh = shi;
  int64_t bos, eos;
  if (cu_seqlens) {
    bos = cu_seqlens[s];
    eos = cu_seqlens[s + 1];
  } else {
    bos = s * seq_len_dense;
    eos = bos + seq_len_dense;
  }
  constexpr int64_t DD = (int64_t)D * D;
  wk.out = sp.mode != 1;
  wk.ck = nullptr;
  if (sp.mode == 3) {
    wk.bos = bos;
    wk.eos = eos;
    wk.s0 = S0 ? S0 + sh * DD : nullptr;
    wk.sfin = Sfin ? Sfin + sh * DD : nullptr;
    if (sp.mode == 3) wk.ck = sp.ckpt + ((bos / C + s) * H + wk.h) * DD;
    return wk;
  }
  const int64_t nch = (eos - bos + C - 1) / C, per = (nch + P - 1) / P;
  const int64_t c0 = p * per < nch ? p * per : nch, c1 = (p + 1) * per < nch ? (p + 1) * per : nch;
  wk.bos = bos + c0 * C;
  wk.eos = bos + c1 * C < eos ? bos + c1 * C : eos;
  if (sp.mode == 1) {
    const int64_t m = (sh * (P - 1) + p) * DD;
    wk.s0 = wk.vb < 0 ? sp.ws_a + m : nullptr;
    wk.sfin = wk.vb < 0 ? sp.ws_a + m : sp.ws_b + m;
  } else {
    wk.s0 = sp.ws_s + (sh * P + p) * DD;
    wk.sfin = (p == P - 1 && Sfin) ? Sfin + sh * DD : nullptr;
  }
  return wk;
}

// 16x16 Gram tile G[r][s] = sum_d A[r0+r][d] B[s0+s][d] (rows of A, B in LDS).
template <typename E, int D, int LDK = Cfg<E, D>::LDK>
__device__ inline f32x4 gram_tile(const E *A, const E *B, int r0, int s0, int j, int c16) {
  using CF = Cfg<E, D>;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (CF::BF) {
    // all operands first, then the MFMA chain
    bf16x8 a[D / 32], b[D / 32];
#pragma unroll
    for (int u = 0; u < D / 32; ++u) {
      a[u] = *reinterpret_cast<const bf16x8 *>(&A[(r0 + c16) * LDK + 32 * u + 8 * j]);
      b[u] = *reinterpret_cast<const bf16x8 *>(&B[(s0 + c16) * LDK + 32 * u + 8 * j]);
    }
#pragma unroll
    for (int u = 0; u < D / 32; ++u) acc = mma(a[u], b[u], acc);
  } else {
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 4)
      acc = mma(A[(r0 + c16) * LDK + k0 + j], B[(s0 + c16) * LDK + k0 + j], acc);
  }
  return acc;
}

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void prefill_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ eta,
    const int32_t *__restrict__ cu_seqlens, int64_t seq_len_dense, int H, float eps, int beta_direct,
    const float *__restrict__ S0, float *__restrict__ o, float *__restrict__ Sfin, SegParams sp) {
  using CF = Cfg<E, D>;
  using P = typename CF::P;
  constexpr bool BF = CF::BF;
  constexpr int NB = D / DVB;
  constexpr int NST = CF::NST;
  constexpr int SEG_EL = 16 / sizeof(E);  // elements per 16-byte segment
  constexpr int SEG_ROW = D / SEG_EL;     // segments per K/Q row
  constexpr int SEG_VROW = DVB / SEG_EL;  // segments per V row (this block)
  static_assert(kThreads % SEG_ROW == 0, "row segments must not straddle waves");

  __shared__ Smem<E, D> sm;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int l = tid & 63;
  const int j = l >> 4, c16 = l & 15;

  const Work wk = resolve_work<NB, D>(sp, cu_seqlens, seq_len_dense, H, S0, Sfin);
  const int nb = wk.nb, h = wk.h;
  const int64_t bos = wk.bos, eos = wk.eos;
  const int col = nb * DVB + 16 * w + c16;  // this lane's state/output column

  // M above the block diagonal is read as zero.
  for (int i = tid; i < C * CF::LDP; i += kThreads) {
    sm.Mh[i] = P(0.f);
    if constexpr (BF) sm.Ml[i] = P(0.f);
  }

  // State tiles: tile t holds rows 16t+4j+i (i<4), column `col`.  A null
  // start state is an empty buffer range: every load returns zero.
  f32x4 S[NST];
  {
    const rsrc_t rs = make_rsrc(wk.s0 ? wk.s0 : o, wk.s0 ? (int64_t)D * D * 4 : 0);
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[t][i] = buf_ld4(rs, ((16 * t + 4 * j + i) * D + col) * 4);
  }

  // Chunk inputs are loaded one chunk ahead into registers, so their HBM
  // latency overlaps the previous chunk's compute.
  constexpr int NSEG = C * SEG_ROW / kThreads;   // K (and Q) segments per thread
  constexpr int NVSEG = C * SEG_VROW / kThreads; // V segments per thread
  static_assert(NSEG * kThreads == C * SEG_ROW && NVSEG * kThreads == C * SEG_VROW, "tiling");
  uint4 kreg[NSEG], qreg[NSEG], vreg[NVSEG];
  float areg = 1.f, ereg = 0.f;
  auto fetch = [&](int64_t t0) {
    // rows past the end of the sequence fall outside the descriptors: zeros
    const int64_t nn = (eos - t0) < C ? (eos - t0) : C;
    const int64_t rowb = (int64_t)H * D * sizeof(E);
    const rsrc_t rk = make_rsrc(k + t0 * H * (int64_t)D, nn * rowb);
    const rsrc_t rq = make_rsrc(q + t0 * H * (int64_t)D, nn * rowb);
    const rsrc_t rv = make_rsrc(v + t0 * H * (int64_t)D, wk.vb >= 0 ? nn * rowb : 0);  // V = 0 for A blocks
#pragma unroll
    for (int u = 0; u < NSEG; ++u) {
      const int sg = u * kThreads + tid, r = sg / SEG_ROW, cs = sg % SEG_ROW;
      const uint32_t off = (uint32_t)((r * H + h) * D + cs * SEG_EL) * sizeof(E);
      kreg[u] = buf_ld16(rk, off);
      qreg[u] = buf_ld16(rq, off);
    }
#pragma unroll
    for (int u = 0; u < NVSEG; ++u) {
      const int sg = u * kThreads + tid, r = sg / SEG_VROW, cs = sg % SEG_VROW;
      vreg[u] = buf_ld16(rv, (uint32_t)((r * H + h) * D + wk.vb * DVB + cs * SEG_EL) * sizeof(E));
    }
    if (w == 0) {
      // no alpha: an empty range (the scan then takes log alpha = 0)
      const rsrc_t ra = make_rsrc(alpha ? alpha + t0 * H : eta, alpha ? nn * H * 4 : 0);
      const rsrc_t re = make_rsrc(eta + t0 * H, nn * H * 4);
      areg = buf_ld4(ra, (uint32_t)(l * H + h) * 4);  // zero past the end
      ereg = buf_ld4(re, (uint32_t)(l * H + h) * 4);
    }
  };
  // Copy the prefetched chunk starting at t0 into LDS, with |k|^2 per row
  // and (wave 0) the scanned log2-decays.
  auto stage = [&](int64_t t0) {
#pragma unroll
    for (int u = 0; u < NSEG; ++u) {
      const int sg = u * kThreads + tid, r = sg / SEG_ROW, cs = sg % SEG_ROW;
      *reinterpret_cast<uint4 *>(&sm.Kr[r * CF::LDK + cs * SEG_EL]) = kreg[u];
      *reinterpret_cast<uint4 *>(&sm.Qr[r * CF::LDK + cs * SEG_EL]) = qreg[u];
      // |k_r|^2: this segment's share, reduced over the SEG_ROW lanes of row r
      const E *ke = reinterpret_cast<const E *>(&kreg[u]);
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < SEG_EL; ++e) {
        const float x = static_cast<float>(ke[e]);
        part += x * x;
      }
      part = group_sum<SEG_ROW>(part);
      if (cs == 0) sm.kk[r] = part;
    }
#pragma unroll
    for (int u = 0; u < NVSEG; ++u) {
      const int sg = u * kThreads + tid, r = sg / SEG_VROW, cs = sg % SEG_VROW;
      *reinterpret_cast<uint4 *>(&sm.Vs[r * CF::LDV + cs * SEG_EL]) = vreg[u];
    }
    if (w == 0) {
      // cumulative log2-decay over the chunk (rows past the end: alpha = 1, eta = 0)
      sm.et[l] = ereg;
      const float g = wave_scan(alpha && l < eos - t0 ? log2f(areg) : 0.f);  // alpha = 1 past the end
      const float glast = __shfl(g, 63, 64);
      sm.g2[l] = g;
      sm.gam[l] = exp2f(g);
      sm.rgam[l] = exp2f(glast - g);
    }
  };

  fetch(bos);
  stage(bos);
  for (int64_t tok0 = bos; tok0 < eos; tok0 += C) {
    const int n = (int)((eos - tok0) < C ? (eos - tok0) : C);
    lds_barrier();  // chunk tok0 is staged
    // Prefetch the next chunk (past the end the descriptors are empty and the
    // loads return zeros without touching memory).
    fetch(tok0 + C);

    // ---- 2. Gram tiles, diagonal block inverses, Q S, K S, R --------------
    if (w == 0) {
      const float b_l = beta_direct ? sm.et[l] : sm.et[l] / (sm.kk[l] + eps);
      sm.beta[l] = b_l;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // diagonal K K^T tiles -> -Diag(beta) Ahat on the diagonal blocks (strictly lower)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const f32x4 acc = gram_tile<E, D>(sm.Kr, sm.Kr, 16 * b, 16 * b, j, c16);
        const float gS = sm.g2[16 * b + c16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * j + i, R = 16 * b + r;
          const float v = -sm.beta[R] * acc[i] * exp2f(fminf(sm.g2[R] - gS, 0.f));
          sm.Ld[(b * 16 + c16) * 20 + r] = r > c16 ? v : 0.f;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // lane (block j, column c16): x = (I + L_jj)^{-1} e_c by substitution,
      // column-oriented: once x_t is final it is eliminated from every later
      // row.  Each lane holds column c16 of -L_jj; -L[r][t] reaches the whole
      // row of lanes by a DPP broadcast from lane t.
      {
        float lc[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 v4 = *reinterpret_cast<const float4 *>(&sm.Ld[(j * 16 + c16) * 20 + 4 * q4]);
          lc[4 * q4] = v4.x;
          lc[4 * q4 + 1] = v4.y;
          lc[4 * q4 + 2] = v4.z;
          lc[4 * q4 + 3] = v4.w;
        }
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == c16) ? 1.f : 0.f;
        solve_steps(x, lc, std::make_integer_sequence<int, 15>{});
        // Y = X Diag(beta): column c16 scaled by beta of that column
        const float bc = sm.beta[16 * j + c16];
#pragma unroll
        for (int r = 0; r < 16; ++r) store_split(sm.Yh, sm.Yl, (j * 16 + r) * CF::LDY + c16, x[r] * bc);
      }
    } else {
      // waves 1, 2, 3 take jobs [0,5), [5,10), [10,16): straight-line code,
      // plane and mask chosen arithmetically so the jobs can overlap.
      const int q0 = 5 * (w - 1);
      auto job = [&](int qj) {
        const Job jb = job_of(qj);
        const bool qk = jb.qk;
        const f32x4 acc = gram_tile<E, D>(qk ? sm.Qr : sm.Kr, sm.Kr, 16 * jb.bi, 16 * jb.bj, j, c16);
        P *ph = qk ? sm.Mh : sm.Ah;
        P *pl = qk ? sm.Ml : sm.Al;
        const float sgn = qk ? 1.f : -1.f;
        const int Sc = 16 * jb.bj + c16;
        const float gS = sm.g2[Sc];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int R = 16 * jb.bi + 4 * j + i;
          const float v = sgn * acc[i] * exp2f(fminf(sm.g2[R] - gS, 0.f));
          store_split(ph, pl, R * CF::LDP + Sc, R >= Sc ? v : 0.f);
        }
      };
#pragma unroll
      for (int u = 0; u < 5; ++u) job(q0 + u);
      if (w == 3) job(15);
    }

    // Q S and K S for this wave's columns, then R = V - diag(gamma) K S
    f32x4 QS[4], R[4];
    if constexpr (BF) {
      Split8 Sf[NST / 2];
#pragma unroll
      for (int kk = 0; kk < NST / 2; ++kk) Sf[kk] = join(split4(S[2 * kk]), split4(S[2 * kk + 1]));
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        f32x4 aq = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NST / 2; ++kk) {
          const bf16x8 a1 = lda_perm(&sm.Qr[(16 * bi + c16) * CF::LDK + 32 * kk], j);
          const bf16x8 a2 = lda_perm(&sm.Kr[(16 * bi + c16) * CF::LDK + 32 * kk], j);
          aq = mma(a1, Sf[kk].hi, aq);
          aq = mma(a1, Sf[kk].lo, aq);
          ak = mma(a2, Sf[kk].hi, ak);
          ak = mma(a2, Sf[kk].lo, ak);
        }
        QS[bi] = aq;
        R[bi] = ak;
      }
    } else {
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        f32x4 aq = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NST; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int a_off = (16 * bi + c16) * CF::LDK + 16 * t + 4 * j + i;
            aq = mma(sm.Qr[a_off], S[t][i], aq);
            ak = mma(sm.Kr[a_off], S[t][i], ak);
          }
        QS[bi] = aq;
        R[bi] = ak;
      }
    }
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * bi + 4 * j + i;
        R[bi][i] = static_cast<float>(sm.Vs[r * CF::LDV + 16 * w + c16]) - sm.gam[r] * R[bi][i];
      }
    lds_barrier();

    // ---- 3. Delta by block substitution, output, state update -------------
    f32x4 Dl[4];
    if constexpr (BF) {
      Split4 Ds[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        f32x4 acc = R[b];
#pragma unroll
        for (int m = 0; m < b; ++m) {
          const int off = (16 * b + c16) * CF::LDP + 16 * m + 4 * j;
          const bf16x4 ah = lda4(&sm.Ah[off]), al = lda4(&sm.Al[off]);
          acc = mma(ah, Ds[m].hi, acc);
          acc = mma(ah, Ds[m].lo, acc);
          acc = mma(al, Ds[m].hi, acc);
        }
        const Split4 as = split4(acc);
        const int yo = (b * 16 + c16) * CF::LDY + 4 * j;
        const bf16x4 yh = lda4(&sm.Yh[yo]), yl = lda4(&sm.Yl[yo]);
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
        d = mma(yh, as.hi, d);
        d = mma(yh, as.lo, d);
        d = mma(yl, as.hi, d);
        Dl[b] = d;
        Ds[b] = split4(d);
      }
      const Split8 Df[2] = {join(Ds[0], Ds[1]), join(Ds[2], Ds[3])};
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = sm.gam[16 * bi + 4 * j + i] * QS[bi][i];
#pragma unroll
        for (int kk = 0; kk <= bi / 2; ++kk) {
          const int off = (16 * bi + c16) * CF::LDP + 32 * kk;
          const bf16x8 ah = lda_perm(&sm.Mh[off], j), al = lda_perm(&sm.Ml[off], j);
          acc = mma(ah, Df[kk].hi, acc);
          acc = mma(ah, Df[kk].lo, acc);
          acc = mma(al, Df[kk].hi, acc);
        }
        QS[bi] = acc;  // now the output tile
      }
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        f32x4 acc = R[b];
#pragma unroll
        for (int m = 0; m < b; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc = mma(sm.Ah[(16 * b + c16) * CF::LDP + 16 * m + 4 * j + i], Dl[m][i], acc);
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) d = mma(sm.Yh[(b * 16 + c16) * CF::LDY + 4 * j + i], acc[i], d);
        Dl[b] = d;
      }
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = sm.gam[16 * bi + 4 * j + i] * QS[bi][i];
#pragma unroll
        for (int mt = 0; mt <= bi; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc = mma(sm.Mh[(16 * bi + c16) * CF::LDP + 16 * mt + 4 * j + i], Dl[mt][i], acc);
        QS[bi] = acc;
      }
    }

    // output rows < n (rows past the end fall outside the descriptor)
    {
      const rsrc_t ro = make_rsrc(wk.out ? o + tok0 * H * (int64_t)D : o, wk.out ? (int64_t)n * H * D * 4 : 0);
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float val = QS[bi][i];
          buf_st4(ro, (uint32_t)(((16 * bi + 4 * j + i) * H + h) * D + col) * 4, val);
        }
    }

    // S' = 2^{g2_last} S + K^T Diag(2^{g2_last - g2}) Delta
    const float glast = sm.gam[C - 1];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int i = 0; i < 4; ++i) Dl[bi][i] *= sm.rgam[16 * bi + 4 * j + i];
#pragma unroll
    for (int t = 0; t < NST; ++t) S[t] *= glast;
    if constexpr (BF) {
      const Split8 Hf[2] = {join(split4(Dl[0]), split4(Dl[1])), join(split4(Dl[2]), split4(Dl[3]))};
#pragma unroll
      for (int t = 0; t < NST; ++t)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          // K^T rows 16t.., tokens 32kk+4j+e and 32kk+16+4j+e (join() order)
          const bf16 *base = &sm.Kr[16 * t + 4 * (c16 & 3)];
          const bf16x4 x0 = ld_tr(base + (32 * kk + 4 * j + (c16 >> 2)) * CF::LDK);
          const bf16x4 x1 = ld_tr(base + (32 * kk + 16 + 4 * j + (c16 >> 2)) * CF::LDK);
          const bf16x8 a = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
          S[t] = mma(a, Hf[kk].hi, S[t]);
          S[t] = mma(a, Hf[kk].lo, S[t]);
        }
    } else {
#pragma unroll
      for (int t = 0; t < NST; ++t)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            S[t] = mma(sm.Kr[(16 * mt + 4 * j + i) * CF::LDK + 16 * t + c16], Dl[mt][i], S[t]);
    }
    lds_barrier();  // everyone is done with this chunk's LDS
    stage(tok0 + C);
  }

  {
    const rsrc_t rs = make_rsrc(wk.sfin ? wk.sfin : o, wk.sfin ? (int64_t)D * D * 4 : 0);
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float val = S[t][i];
        buf_st4(rs, ((16 * t + 4 * j + i) * D + col) * 4, val);
      }
  }
}

// ===========================================================================
// bf16 prefill with producer and consumer waves.
//
// Eight waves per workgroup.  Waves 0-3 (consumers) own 16 state columns
// each and run the state-dependent chain of chunk c; waves 4-7 (producers)
// stage the chunks and build their Gram tiles and diagonal-block inverses.
// Each SIMD hosts one consumer and one producer.  Per chunk c:
//   segment A: consumers form Q S, K S and R for chunk c;
//              producers stage K of chunk c+1 and scan its decays, and
//              build chunk c's M = lower(Q K^T o Gam) planes;
//   barrier;
//   segment B: consumers run the substitution, output and state update of c;
//              producers build chunk c+1's -Ahat planes and diagonal-block
//              inverses, and stage Q and V of chunk c+1;
//   barrier.
// K, the -Ahat and Y planes and the gates live in two slots (chunk parity);
// Q, V and the M planes have one buffer each: Q and V of chunk c are read
// only in segment A of c and chunk c+1's are staged in segment B, and M of
// chunk c is built in segment A of c and read in segment B of c.
//
// QLO: the query is a pair of bf16 planes, q + q_lo (a split fp32 query).
// The lo plane enters Q S as q_lo S_hi and the M planes as q_lo K^T; its
// share of the output is about 2^-8 of the whole, so the terms dropped
// (q_lo S_lo) are below 2^-16 of the output.
// ===========================================================================

// SQ (single query buffer, the two-plane read): Q, its lo plane, V and the
// M planes have one buffer each; otherwise they live in the two slots with
// K, the -Ahat and Y planes and the gates.
template <int D, bool OUT, bool SQ>
struct PSlot {
  using CF = Cfg<bf16, D>;
  static constexpr bool PER_SLOT = OUT && !SQ;
  static constexpr int LDA = 20;  // compact 16x16 blocks of -Ahat and Y
  // Row pitches (elements) of K, Q and the M planes: 2 * LDK and 2 * LDP
  // bytes are 32 more than a multiple of 128, which keeps the consumers'
  // row-per-lane 16-byte reads and the transposing K^T reads free of LDS
  // bank conflicts.
  static constexpr int LDK = D + 16;
  static constexpr int LDP = C + 16;
  alignas(16) bf16 Kr[C * LDK];
  alignas(16) bf16 Qr[PER_SLOT ? C * LDK : 8];
  alignas(16) bf16 Vs[SQ ? 8 : C * CF::LDV];
  alignas(16) bf16 Ah[6 * 16 * LDA];  // -Ahat blocks (b, m), m < b, index b(b-1)/2 + m
  alignas(16) bf16 Al[6 * 16 * LDA];
  alignas(16) bf16 Mh[PER_SLOT ? C * LDP : 8];  // M = lower(Q K^T o Gam), zero above the block diagonal
  alignas(16) bf16 Ml[PER_SLOT ? C * LDP : 8];
  static constexpr int LDYT = 24;     // Y^T rows: 16 values + pad, 16-byte aligned
  alignas(16) bf16 Yh[4 * 16 * LDYT];  // Y_bb^T, Y_bb = (I + L_bb)^{-1} Diag(beta_b)
  alignas(16) bf16 Yl[4 * 16 * LDYT];
  alignas(16) float gam[C];
  alignas(16) float rgam[C];
  alignas(16) float g2[C];            // cumulative log2-decay
};
template <int D, bool OUT, bool SQ>
struct PSmem {
  using CF = Cfg<bf16, D>;
  using SL = PSlot<D, OUT, SQ>;
  SL slot[2];
  alignas(16) bf16 Qr[SQ ? C * SL::LDK : 8];
  alignas(16) bf16 Qlr[SQ ? C * SL::LDK : 8];
  alignas(16) bf16 Vs[SQ ? C * CF::LDV : 8];
  alignas(16) bf16 Mh[SQ ? C * SL::LDP : 8];
  alignas(16) bf16 Ml[SQ ? C * SL::LDP : 8];
  // producer scratch for the chunk being prepared
  alignas(16) float kk[C];
  alignas(16) float et[C];
  alignas(16) float beta[C];
};

// OUT = false: the segment-map pass, which writes no output and so needs
// neither Q nor M (only K, V, the gates and the -Ahat, Y planes).
template <int D, bool OUT, bool QLO>
__global__ __launch_bounds__(512) void prefill_pc_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ q_lo, const bf16 *__restrict__ k,
    const bf16 *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ eta,
    const int32_t *__restrict__ cu_seqlens, int64_t seq_len_dense, int H, float eps, int beta_direct,
    const float *__restrict__ S0, float *__restrict__ o, float *__restrict__ Sfin, SegParams sp) {
  using CF = Cfg<bf16, D>;
  using SL = PSlot<D, OUT, QLO>;
  constexpr int LDA = SL::LDA;
  constexpr int NB = D / DVB;
  constexpr int NST = CF::NST;
  constexpr int SEG_EL = 8;               // bf16 per 16-byte segment
  constexpr int SEG_ROW = D / SEG_EL;     // segments per K/Q row
  constexpr int SEG_VROW = DVB / SEG_EL;  // segments per V row (this block)
  constexpr int PT = 256;                 // producer threads
  constexpr int NSEG = C * SEG_ROW / PT;
  constexpr int NVSEG = C * SEG_VROW / PT;
  static_assert(NSEG * PT == C * SEG_ROW && NVSEG * PT == C * SEG_VROW, "tiling");

  static_assert(OUT || !QLO, "a second query plane needs the output");
  __shared__ PSmem<D, OUT, QLO> sm;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const bool producer = w >= 4;
  const int pw = w - 4;                                    // producer wave 0..3
  const int ptid = tid - PT;
  const int l = tid & 63;
  const int j = l >> 4, c16 = l & 15;

  const Work wk = resolve_work<NB, D>(sp, cu_seqlens, seq_len_dense, H, S0, Sfin);
  const int nb = wk.nb, h = wk.h;
  const int64_t bos = wk.bos, eos = wk.eos;
  const int col = nb * DVB + 16 * w + c16;  // consumer lane's state/output column

  // Q, V and M of a chunk: in its slot, or in the single buffers (QLO)
  auto QB = [&](SL &sl) __attribute__((always_inline)) -> bf16 * {
    if constexpr (QLO) return sm.Qr; else return sl.Qr;
  };
  auto VB = [&](SL &sl) __attribute__((always_inline)) -> bf16 * {
    if constexpr (QLO) return sm.Vs; else return sl.Vs;
  };
  auto MHB = [&](SL &sl) __attribute__((always_inline)) -> bf16 * {
    if constexpr (QLO) return sm.Mh; else return sl.Mh;
  };
  auto MLB = [&](SL &sl) __attribute__((always_inline)) -> bf16 * {
    if constexpr (QLO) return sm.Ml; else return sl.Ml;
  };
  // M above the block diagonal is read as zero.
  if constexpr (OUT) {
    for (int i = tid; i < C * SL::LDP; i += 512) {
      MHB(sm.slot[0])[i] = bf16(0.f);
      MLB(sm.slot[0])[i] = bf16(0.f);
      MHB(sm.slot[1])[i] = bf16(0.f);
      MLB(sm.slot[1])[i] = bf16(0.f);
    }
  }

  // ---- producer pieces ------------------------------------------------------
  // K and the gates of a chunk are fetched into registers two chunks ahead
  // of their consumption and staged in segment A; Q (and its lo plane) and
  // V likewise, staged in segment B.
  uint4 kreg[NSEG], qreg[NSEG], qlreg[QLO ? NSEG : 1], vreg[NVSEG];
  float areg = 1.f, ereg = 0.f;
  auto fetch_k = [&](int64_t t0) __attribute__((always_inline)) {  // HBM -> registers (zeros past the end)
    const int64_t nn = (eos - t0) < C ? (eos - t0) : C;
    const rsrc_t rk = make_rsrc(k + t0 * H * (int64_t)D, nn * (int64_t)H * D * 2);
#pragma unroll
    for (int u = 0; u < NSEG; ++u) {
      const int sg = u * PT + ptid, r = sg / SEG_ROW, cs = sg % SEG_ROW;
      kreg[u] = buf_ld16(rk, (uint32_t)((r * H + h) * D + cs * SEG_EL) * 2);
    }
    if (pw == 0) {
      // no alpha: an empty range (the scan then takes log alpha = 0)
      const rsrc_t ra = make_rsrc(alpha ? alpha + t0 * H : eta, alpha ? nn * H * 4 : 0);
      const rsrc_t re = make_rsrc(eta + t0 * H, nn * H * 4);
      areg = buf_ld4(ra, (uint32_t)(l * H + h) * 4);  // zero past the end
      ereg = buf_ld4(re, (uint32_t)(l * H + h) * 4);
    }
  };
  auto fetch_qv = [&](int64_t t0) __attribute__((always_inline)) {
    const int64_t nn = (eos - t0) < C ? (eos - t0) : C;
    const int64_t rowb = (int64_t)H * D * 2;
    const rsrc_t rv = make_rsrc(v + t0 * H * (int64_t)D, wk.vb >= 0 ? nn * rowb : 0);  // V = 0 for A blocks
    if constexpr (OUT) {
      const rsrc_t rq = make_rsrc(q + t0 * H * (int64_t)D, nn * rowb);
      const rsrc_t rql = make_rsrc(QLO ? q_lo + t0 * H * (int64_t)D : q, QLO ? nn * rowb : 0);
#pragma unroll
      for (int u = 0; u < NSEG; ++u) {
        const int sg = u * PT + ptid, r = sg / SEG_ROW, cs = sg % SEG_ROW;
        const uint32_t off = (uint32_t)((r * H + h) * D + cs * SEG_EL) * 2;
        qreg[u] = buf_ld16(rq, off);
        if constexpr (QLO) qlreg[u] = buf_ld16(rql, off);
      }
    }
#pragma unroll
    for (int u = 0; u < NVSEG; ++u) {
      const int sg = u * PT + ptid, r = sg / SEG_VROW, cs = sg % SEG_VROW;
      vreg[u] = buf_ld16(rv, (uint32_t)((r * H + h) * D + wk.vb * DVB + cs * SEG_EL) * 2);
    }
  };
  // a 16-byte segment of a K or Q row (logical columns 8cs..8cs+7) into its
  // two places in the LDS column order
  auto put_row_seg = [&](bf16 *rowp, int cs, const uint4 &x) __attribute__((always_inline)) {
    *reinterpret_cast<uint2 *>(&rowp[pcol(cs * SEG_EL)]) = uint2{x.x, x.y};
    *reinterpret_cast<uint2 *>(&rowp[pcol(cs * SEG_EL + 4)]) = uint2{x.z, x.w};
  };
  auto stage_k = [&](SL &sl, int64_t t0) __attribute__((always_inline)) {  // K and the decays into a slot
#pragma unroll
    for (int u = 0; u < NSEG; ++u) {
      const int sg = u * PT + ptid, r = sg / SEG_ROW, cs = sg % SEG_ROW;
      put_row_seg(&sl.Kr[r * SL::LDK], cs, kreg[u]);
    }
    if (pw == 0) {
      sm.et[l] = ereg;
      const float g = wave_scan(alpha && l < eos - t0 ? flog2_rate(areg) : 0.f);  // alpha = 1 past the end
      const float glast = __shfl(g, 63, 64);
      sl.g2[l] = g;
      sl.gam[l] = fexp2(g);
      sl.rgam[l] = fexp2(glast - g);
    }
  };
  auto stage_qv = [&](SL &sl) __attribute__((always_inline)) {  // Q (+ lo plane) and V
    if constexpr (OUT) {
      bf16 *qb = QB(sl);
#pragma unroll
      for (int u = 0; u < NSEG; ++u) {
        const int sg = u * PT + ptid, r = sg / SEG_ROW, cs = sg % SEG_ROW;
        put_row_seg(&qb[r * SL::LDK], cs, qreg[u]);
        if constexpr (QLO) put_row_seg(&sm.Qlr[r * SL::LDK], cs, qlreg[u]);
      }
    }
    bf16 *vb = VB(sl);
#pragma unroll
    for (int u = 0; u < NVSEG; ++u) {
      const int sg = u * PT + ptid, r = sg / SEG_VROW, cs = sg % SEG_VROW;
      *reinterpret_cast<uint4 *>(&vb[r * CF::LDV + cs * SEG_EL]) = vreg[u];
    }
  };
  auto wave_sync = [&]() __attribute__((always_inline)) {  // order this wave's LDS writes before its reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // Gram jobs q0 .. q0+nj-1 of a slot's chunk (numbering of job_of: 0-5 the
  // -Ahat blocks, 6-15 the M blocks).  Each tile is computed transposed,
  // C[s][r] = K[s] . (Q or K)[r], so a lane holds four consecutive s of one
  // row r and writes them as one 8-byte store per plane.  Operands of the
  // next job are loaded first.
  auto jobs = [&](SL &sl, int q0, int nj) __attribute__((always_inline)) {
    bf16 *const qb = QB(sl);
    bf16x8 opa[2][D / 32], opb[2][D / 32], opl[2][QLO ? D / 32 : 1];
    float grb[2];
    f32x4 gsb[2];
    auto ldjob = [&](int u) __attribute__((always_inline)) {  // operands and gates of job u
      const Job jb = job_of(q0 + u);
      const bf16 *B = jb.qk ? qb : sl.Kr;
      grb[u & 1] = sl.g2[16 * jb.bi + c16];
      gsb[u & 1] = *reinterpret_cast<const f32x4 *>(&sl.g2[16 * jb.bj + 4 * j]);
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        opa[u & 1][t] = *reinterpret_cast<const bf16x8 *>(&sl.Kr[(16 * jb.bj + c16) * SL::LDK + 32 * t + 8 * j]);
        opb[u & 1][t] = *reinterpret_cast<const bf16x8 *>(&B[(16 * jb.bi + c16) * SL::LDK + 32 * t + 8 * j]);
        if constexpr (QLO) {
          if (jb.qk) opl[u & 1][t] = *reinterpret_cast<const bf16x8 *>(&sm.Qlr[(16 * jb.bi + c16) * SL::LDK + 32 * t + 8 * j]);
        }
      }
    };
    if (nj > 0) ldjob(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u < nj) {
        if (u + 1 < nj) ldjob(u + 1);
        sched_fence();
        const Job jb = job_of(q0 + u);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < D / 32; ++t) acc = mma(opa[u & 1][t], opb[u & 1][t], acc);
        if constexpr (QLO) {
          if (jb.qk) {
#pragma unroll
            for (int t = 0; t < D / 32; ++t) acc = mma(opa[u & 1][t], opl[u & 1][t], acc);
          }
        }
        sched_fence();
        const int r = 16 * jb.bi + c16;  // this lane's row
        const float gr = grb[u & 1];
        const f32x4 gsv = gsb[u & 1];
        f32x4 vals;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int sc = 16 * jb.bj + 4 * j + i;
          const float val = acc[i] * fexp2(fminf(gr - gsv[i], 0.f));
          vals[i] = jb.qk ? (r >= sc ? val : 0.f) : -val;
        }
        const Split4 sp = split4(vals);
        if (jb.qk) {
          const int off = r * SL::LDP + pcol(16 * jb.bj + 4 * j);
          *reinterpret_cast<bf16x4 *>(&MHB(sl)[off]) = sp.hi;
          *reinterpret_cast<bf16x4 *>(&MLB(sl)[off]) = sp.lo;
        } else {
          const int off = ((jb.bi * (jb.bi - 1) / 2 + jb.bj) * 16 + c16) * LDA + 4 * j;
          *reinterpret_cast<bf16x4 *>(&sl.Ah[off]) = sp.hi;
          *reinterpret_cast<bf16x4 *>(&sl.Al[off]) = sp.lo;
        }
      }
    }
  };
  // The diagonal blocks of a slot's chunk (producer wave 0): the diagonal
  // K K^T tiles, |k|^2 off their diagonal, beta, -L on the diagonal blocks
  // and the four 16x16 inverses Y_bb (one DPP column substitution per lane:
  // lane (j, c16) solves column c16 of block j).
  auto diag = [&](SL &sl) __attribute__((always_inline)) {
    f32x4 dg[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) dg[b] = gram_tile<bf16, D, SL::LDK>(sl.Kr, sl.Kr, 16 * b, 16 * b, j, c16);
    // |k_r|^2 is the diagonal: row 16b + c16 sits in lane (c16 / 4, c16), element c16 % 4
    if ((c16 >> 2) == j) {
      const int e = c16 & 3;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        sm.kk[16 * b + c16] = e == 0 ? dg[b][0] : e == 1 ? dg[b][1] : e == 2 ? dg[b][2] : dg[b][3];
    }
    wave_sync();
    sm.beta[l] = beta_direct ? sm.et[l] : sm.et[l] / (sm.kk[l] + eps);
    wave_sync();
    // every gate and beta this lane needs first, then -L: lane (j, c16)
    // holds rows 4j..4j+3 of column c16 of each diagonal block b
    f32x4 gr[4], br[4];
    float gc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      gr[b] = *reinterpret_cast<const f32x4 *>(&sl.g2[16 * b + 4 * j]);
      br[b] = *reinterpret_cast<const f32x4 *>(&sm.beta[16 * b + 4 * j]);
      gc[b] = sl.g2[16 * b + c16];
    }
    f32x4 val[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = -br[b][i] * dg[b][i] * fexp2(fminf(gr[b][i] - gc[b], 0.f));
        val[b][i] = 4 * j + i > c16 ? x : 0.f;  // -L below the diagonal
      }
    // The solve wants lane (b, c16) to hold all of column c16 of block b:
    // for each i, a 4x4 transpose of (16-lane row, block register), by
    // swapping the upper 32 lanes of blocks 0, 1 with the lower 32 of
    // blocks 2, 3, then the odd rows of blocks 0, 2 with the even rows of
    // blocks 1, 3.  Afterwards lc[4r + i] = -L_b[4r + i][c16].
    float lc[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(val[0][i]), __float_as_uint(val[2][i]), false, false);
      const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(val[1][i]), __float_as_uint(val[3][i]), false, false);
      const auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
      const auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
      lc[i] = __uint_as_float(s01[0]);
      lc[4 + i] = __uint_as_float(s01[1]);
      lc[8 + i] = __uint_as_float(s23[0]);
      lc[12 + i] = __uint_as_float(s23[1]);
    }
    // The solve reads lc through DPP, which needs two wait states after a
    // VALU write of the register (the compiler adds none before inline asm):
    // every lc passes through this one statement, whose s_nop provides them.
    asm volatile("s_nop 2"
                 : "+v"(lc[0]), "+v"(lc[1]), "+v"(lc[2]), "+v"(lc[3]), "+v"(lc[4]), "+v"(lc[5]),
                   "+v"(lc[6]), "+v"(lc[7]), "+v"(lc[8]), "+v"(lc[9]), "+v"(lc[10]), "+v"(lc[11]),
                   "+v"(lc[12]), "+v"(lc[13]), "+v"(lc[14]), "+v"(lc[15]));
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (r == c16) ? 1.f : 0.f;
    solve_steps(x, lc, std::make_integer_sequence<int, 15>{});
    const float bc = sm.beta[16 * j + c16];
    // column c16 of Y_jj, contiguous in Y^T: two 16-byte writes per plane
    Split4 yq[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      yq[q4] = split4(f32x4{x[4 * q4] * bc, x[4 * q4 + 1] * bc, x[4 * q4 + 2] * bc, x[4 * q4 + 3] * bc});
    const int yo = (j * 16 + c16) * SL::LDYT;
    *reinterpret_cast<bf16x8 *>(&sl.Yh[yo]) = __builtin_shufflevector(yq[0].hi, yq[1].hi, 0, 1, 2, 3, 4, 5, 6, 7);
    *reinterpret_cast<bf16x8 *>(&sl.Yh[yo + 8]) = __builtin_shufflevector(yq[2].hi, yq[3].hi, 0, 1, 2, 3, 4, 5, 6, 7);
    *reinterpret_cast<bf16x8 *>(&sl.Yl[yo]) = __builtin_shufflevector(yq[0].lo, yq[1].lo, 0, 1, 2, 3, 4, 5, 6, 7);
    *reinterpret_cast<bf16x8 *>(&sl.Yl[yo + 8]) = __builtin_shufflevector(yq[2].lo, yq[3].lo, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // Where the Gram jobs of a chunk run (numbering of job_of).  Any job of
  // chunk c may run in segment B of the trip before c or in segment A of
  // c's trip; the split balances the two segments.
  //   two slots:  segment B before c: wave 0 the diagonal blocks, waves 1-3
  //               jobs 0-3, 4-7, 8-11 (only the -Ahat jobs 0-5 without
  //               output: 0-1, 2-3, 4-5); segment A of c: jobs 12-15, one
  //               per wave;
  //   single Q (QLO): Q of c is staged in segment B before c, so its M
  //               jobs wait for segment A of c: wave 0 job 6, waves 1-3
  //               jobs 7-9, 10-12, 13-15; segment B before c: wave 0 the
  //               diagonal blocks, waves 1-3 two -Ahat jobs each.
  auto seg_a_jobs = [&](SL &cs) __attribute__((always_inline)) {
    if constexpr (QLO)
      jobs(cs, pw == 0 ? 6 : 4 + 3 * pw, pw == 0 ? 1 : 3);
    else if constexpr (OUT)
      jobs(cs, 12 + pw, 1);
  };
  auto seg_b_jobs = [&](SL &nx) __attribute__((always_inline)) {
    if (pw == 0)
      diag(nx);
    else if constexpr (OUT && !QLO)
      jobs(nx, 4 * (pw - 1), 4);
    else
      jobs(nx, 2 * (pw - 1), 2);
  };

  // The two roles run separate loops with the same number of barriers, so
  // neither role's loop-carried registers are live in the other's code.
  if (producer) {
    // prologue: chunk 0 (K, gates, Q, V) staged and its segment-B jobs;
    // chunk 1 fetched
    fetch_k(bos);
    fetch_qv(bos);
    stage_k(sm.slot[0], bos);
    stage_qv(sm.slot[0]);
    fetch_k(bos + C);
    fetch_qv(bos + C);
    lds_barrier();
    if (bos < eos) seg_b_jobs(sm.slot[0]);
    lds_barrier();
    int cur = 0;
    for (int64_t tok0 = bos; tok0 < eos; tok0 += C, cur ^= 1) {
      SL &cs = sm.slot[cur], &nx = sm.slot[cur ^ 1];
      // segment A: chunk c+1's K (with Q and V in the two-slot layout), then
      // chunk c's remaining jobs
      stage_k(nx, tok0 + C);
      fetch_k(tok0 + 2 * C);
      if constexpr (!QLO) {
        stage_qv(nx);
        fetch_qv(tok0 + 2 * C);
      }
      seg_a_jobs(cs);
      lds_barrier();
      // segment B: (QLO: chunk c+1's Q and V, then) chunk c+1's first jobs
      if constexpr (QLO) {
        stage_qv(nx);
        fetch_qv(tok0 + 2 * C);
      }
      if (tok0 + C < eos) seg_b_jobs(nx);
      lds_barrier();
    }
    return;
  }

  // ---- consumers ---------------------------------------------------------
  f32x4 S[NST];
  {
    const rsrc_t rs = make_rsrc(wk.s0 ? wk.s0 : o, wk.s0 ? (int64_t)D * D * 4 : 0);
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[t][i] = buf_ld4(rs, ((16 * t + 4 * j + i) * D + col) * 4);
  }
  lds_barrier();
  lds_barrier();

  // One chunk: Sin is the state entering it, Sout receives the state after
  // it.  The loop runs two chunks per trip, alternating the two state
  // arrays and the two LDS slots, so slot addresses are constants and the
  // update needs no copy back into the entering array.
  f32x4 S2[NST];
  auto cstep = [&](SL &sl, int64_t tok0, f32x4 (&Sin)[NST], f32x4 (&Sout)[NST])
                   __attribute__((always_inline)) {

    // ---- segment A: Q S, K S, R = V - Diag(gamma) K S -----------------------
    f32x4 QS[4], R[4];
    {
      constexpr int NK = NST / 2, NSTEP = 4 * NK;
      Split8 Sf[NK];
      // the decayed state for this chunk's update first, so the split below
      // may consume Sin in place
      const float glast = sl.gam[C - 1];
#pragma unroll
      for (int t = 0; t < NST; ++t) Sout[t] = Sin[t] * glast;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) Sf[kk] = join(split4(Sin[2 * kk]), split4(Sin[2 * kk + 1]));
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        QS[bi] = f32x4{0.f, 0.f, 0.f, 0.f};
        R[bi] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // steps run kk-major so consecutive MFMAs update different tiles; the
      // A operands are loaded two steps ahead
      bf16x8 qa[3], ka[3], qla[QLO ? 3 : 1];
      auto ld = [&](int st) {
        const int kk = st / 4, bi = st % 4;
        const int off = (16 * bi + c16) * SL::LDK + 32 * kk + 8 * j;
        if constexpr (OUT) qa[st % 3] = *reinterpret_cast<const bf16x8 *>(&QB(sl)[off]);
        if constexpr (QLO) qla[st % 3] = *reinterpret_cast<const bf16x8 *>(&sm.Qlr[off]);
        ka[st % 3] = *reinterpret_cast<const bf16x8 *>(&sl.Kr[off]);
      };
      ld(0);
      ld(1);
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) {
        if (st + 2 < NSTEP) ld(st + 2);
        sched_fence();
        const int kk = st / 4, bi = st % 4;
        // Q S is formed transposed, (Q S)^T = S^T Q^T: the state fragments
        // serve as the A operand, so the output tile holds four consecutive
        // dv values of one token per lane (16-byte stores below)
        if constexpr (OUT) QS[bi] = mma(Sf[kk].hi, qa[st % 3], QS[bi]);
        R[bi] = mma(ka[st % 3], Sf[kk].hi, R[bi]);
        if constexpr (OUT) QS[bi] = mma(Sf[kk].lo, qa[st % 3], QS[bi]);
        R[bi] = mma(ka[st % 3], Sf[kk].lo, R[bi]);
        if constexpr (QLO) QS[bi] = mma(Sf[kk].hi, qla[st % 3], QS[bi]);
        sched_fence();
      }
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        // V rows 16bi+4j..+3 of this lane's column, one transposing read
        const bf16x4 vv = ld_tr(&VB(sl)[(16 * bi + 4 * j + (c16 >> 2)) * CF::LDV + 16 * w + 4 * (c16 & 3)]);
        const f32x4 gv = *reinterpret_cast<const f32x4 *>(&sl.gam[16 * bi + 4 * j]);
#pragma unroll
        for (int i = 0; i < 4; ++i) R[bi][i] = static_cast<float>(vv[i]) - gv[i] * R[bi][i];
      }
    }
    lds_barrier();

    // ---- segment B: Delta, output, state update -----------------------------
    {
      const int n = (int)((eos - tok0) < C ? (eos - tok0) : C);
      // every operand of the substitution up front: the chain is latency-bound
      bf16x4 yh[4], yl[4], ah[6], al[6];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        // Y[c16][4j..4j+3] from Y^T (row-major, 16 + pad per row) by the
        // transposing read: lane c addresses row 4j + c/4, columns 4(c%4)..
        const int yo = (b * 16 + 4 * j + (c16 >> 2)) * SL::LDYT + 4 * (c16 & 3);
        yh[b] = ld_tr(&sl.Yh[yo]);
        yl[b] = ld_tr(&sl.Yl[yo]);
      }
#pragma unroll
      for (int qb = 0; qb < 6; ++qb) {
        const int off = (qb * 16 + c16) * LDA + 4 * j;
        ah[qb] = lda4(&sl.Ah[off]);
        al[qb] = lda4(&sl.Al[off]);
      }
      f32x4 Dl[4];
      Split4 Ds[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        f32x4 acc = R[b];
#pragma unroll
        for (int m = 0; m < b; ++m) {
          const int qb = b * (b - 1) / 2 + m;
          acc = mma(ah[qb], Ds[m].hi, acc);
          acc = mma(ah[qb], Ds[m].lo, acc);
          acc = mma(al[qb], Ds[m].hi, acc);
        }
        const Split4 as = split4(acc);
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
        d = mma(yh[b], as.hi, d);
        d = mma(yh[b], as.lo, d);
        d = mma(yl[b], as.hi, d);
        Dl[b] = d;
        Ds[b] = split4(d);
      }
      const Split8 Df[2] = {join(Ds[0], Ds[1]), join(Ds[2], Ds[3])};
      if constexpr (OUT) {
        // O = Diag(gamma) Q S + M Delta: steps (kk, bi), bi >= 2 kk, kk-major
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) QS[bi] *= sl.gam[16 * bi + c16];  // token column c16
        {
          constexpr int NSTEP = 6;
          bf16x8 mh[3], ml[3];
          auto ld = [&](int st) {
            const int kk = st < 4 ? 0 : 1, bi = st < 4 ? st : st - 2;
            const int off = (16 * bi + c16) * SL::LDP + 32 * kk + 8 * j;
            mh[st % 3] = *reinterpret_cast<const bf16x8 *>(&MHB(sl)[off]);
            ml[st % 3] = *reinterpret_cast<const bf16x8 *>(&MLB(sl)[off]);
          };
          ld(0);
          ld(1);
#pragma unroll
          for (int st = 0; st < NSTEP; ++st) {
            if (st + 2 < NSTEP) ld(st + 2);
            sched_fence();
            const int kk = st < 4 ? 0 : 1, bi = st < 4 ? st : st - 2;
            // (M Delta)^T = Delta^T M^T, accumulated into the transposed output
            QS[bi] = mma(Df[kk].hi, mh[st % 3], QS[bi]);
            QS[bi] = mma(Df[kk].lo, mh[st % 3], QS[bi]);
            QS[bi] = mma(Df[kk].hi, ml[st % 3], QS[bi]);
            sched_fence();
          }
        }
      }
      // S' = 2^{g2_last} S + K^T Diag(2^{g2_last - g2}) Delta
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int i = 0; i < 4; ++i) Dl[bi][i] *= sl.rgam[16 * bi + 4 * j + i];
      const Split8 Hf[2] = {join(split4(Dl[0]), split4(Dl[1])), join(split4(Dl[2]), split4(Dl[3]))};
      {
        // steps (kk, t), kk-major; K^T operands by transposing reads, two ahead
        constexpr int NSTEP = 2 * NST;
        bf16x8 kt[3];
        auto ld = [&](int st) {
          const int kk = st / NST, t = st % NST;
          const bf16 *base = &sl.Kr[pcol(16 * t + 4 * (c16 & 3))];
          const bf16x4 x0 = ld_tr(base + (32 * kk + 4 * j + (c16 >> 2)) * SL::LDK);
          const bf16x4 x1 = ld_tr(base + (32 * kk + 16 + 4 * j + (c16 >> 2)) * SL::LDK);
          kt[st % 3] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        ld(0);
        ld(1);
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
          if (st + 2 < NSTEP) ld(st + 2);
          sched_fence();
          const int kk = st / NST, t = st % NST;
          Sout[t] = mma(kt[st % 3], Hf[kk].hi, Sout[t]);
          Sout[t] = mma(kt[st % 3], Hf[kk].lo, Sout[t]);
          sched_fence();
        }
      }
      // the output last, so the M Delta products have drained during the
      // state update
      if constexpr (OUT) {
        const rsrc_t ro = make_rsrc(wk.out ? o + tok0 * H * (int64_t)D : o, wk.out ? (int64_t)n * H * D * 4 : 0);
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)  // token 16bi + c16, dv 16w + 4j..+3; rows past the end are dropped
        {
          const uint32_t off = (uint32_t)(((16 * bi + c16) * H + h) * D + nb * DVB + 16 * w + 4 * j) * 4;
          if (sp.o_wb)
            buf_st16(ro, off, QS[bi]);
          else
            buf_st16_nt(ro, off, QS[bi]);
        }
      }
    }
    lds_barrier();
  };
  // states-only pass: the state entering each chunk to its slot
  auto store_ck = [&](const f32x4 (&Sx)[NST], int64_t t0) __attribute__((always_inline)) {
    if constexpr (!OUT) {
      if (wk.ck) {
        const int64_t DD = (int64_t)D * D;
        const rsrc_t rc = make_rsrc(wk.ck + ((t0 - bos) / C) * H * DD, DD * 4);
#pragma unroll
        for (int t = 0; t < NST; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) buf_st4(rc, ((16 * t + 4 * j + i) * D + col) * 4, Sx[t][i]);
      }
    }
  };
  int64_t tok0 = bos;
  bool in_s2 = false;  // the current state is in S2
  while (tok0 < eos) {
    store_ck(S, tok0);
    cstep(sm.slot[0], tok0, S, S2);
    tok0 += C;
    if (tok0 >= eos) {
      in_s2 = true;
      break;
    }
    store_ck(S2, tok0);
    cstep(sm.slot[1], tok0, S2, S);
    tok0 += C;
  }
  if (in_s2) {
#pragma unroll
    for (int t = 0; t < NST; ++t) S[t] = S2[t];
  }

  {
    const rsrc_t rs = make_rsrc(wk.sfin ? wk.sfin : o, wk.sfin ? (int64_t)D * D * 4 : 0);
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float val = S[t][i];
        buf_st4(rs, ((16 * t + 4 * j + i) * D + col) * 4, val);
      }
  }
}

// Workgroups of one launch: (sequence, head) x [segment] x column block.
inline int64_t grid_of(const PrefillArgs &a, int NB) {
  const int64_t sh = (int64_t)a.n_seqs * a.H;
  if (a.seg_mode == 1) return sh * (a.n_splits - 1) * 2 * NB;
  if (a.seg_mode == 2) return sh * a.n_splits * NB;
  if (a.seg_mode == 0) return (sh + 7) / 8 * 8 * NB;  // padded: 8 XCDs x whole pairs
  return sh * NB;
}
inline SegParams seg_of(const PrefillArgs &a) {
  SegParams sp;
  sp.mode = a.seg_mode;
  sp.n_splits = a.n_splits;
  sp.n_pairs = (int64_t)a.n_seqs * a.H;
  sp.order = a.seq_order;
  sp.ws_a = a.ws_a;
  sp.ws_b = a.ws_b;
  sp.ws_s = a.ws_s;
  sp.ckpt = a.ws_ckpt;
  sp.o_wb = a.o_write_back;
  return sp;
}

template <int D>
hipError_t launch_pc(const PrefillArgs &a, hipStream_t st) {
  const int64_t grid = grid_of(a, D / DVB);
  auto kern = a.seg_mode == 1 ? prefill_pc_kernel<D, false, false>
              : a.q_lo        ? prefill_pc_kernel<D, true, true>
                              : prefill_pc_kernel<D, true, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), 0, st,
                     static_cast<const bf16 *>(a.q), static_cast<const bf16 *>(a.q_lo),
                     static_cast<const bf16 *>(a.k), static_cast<const bf16 *>(a.v), a.alpha,
                     a.eta, a.cu_seqlens, a.seq_len_dense, a.H, a.eps, a.beta_direct,
                     a.initial_state, a.o, a.final_state, seg_of(a));
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_d(const PrefillArgs &a, hipStream_t st) {
  const int64_t grid = grid_of(a, D / DVB);
  hipLaunchKernelGGL((prefill_kernel<E, D>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                     static_cast<const E *>(a.q), static_cast<const E *>(a.k),
                     static_cast<const E *>(a.v), a.alpha, a.eta, a.cu_seqlens, a.seq_len_dense,
                     a.H, a.eps, a.beta_direct, a.initial_state, a.o, a.final_state, seg_of(a));
  return hipGetLastError();
}

// Longest-first order of packed sequences: order[rank] = s, rank = the
// number of sequences longer than s, or as long with a smaller index (a
// stable sort by decreasing length; deterministic).  One workgroup; the
// lengths are staged in LDS.
constexpr int kOrderMax = 1024;
__global__ __launch_bounds__(kOrderMax) void seq_order_kernel(const int32_t *__restrict__ cu,
                                                              int n, int32_t *__restrict__ order) {
  __shared__ int32_t len[kOrderMax];
  const int s = threadIdx.x;
  if (s < n) len[s] = cu[s + 1] - cu[s];
  __syncthreads();
  if (s >= n) return;
  const int ls = len[s];
  int rank = 0;
  for (int t = 0; t < n; ++t) rank += (len[t] > ls) | ((len[t] == ls) & (t < s));
  order[rank] = s;
}

}  // namespace

hipError_t launch_seq_order(const int32_t *cu_seqlens, int n_seqs, int32_t *order, hipStream_t st) {
  if (n_seqs > kOrderMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(seq_order_kernel, dim3(1), dim3(kOrderMax), 0, st, cu_seqlens, n_seqs, order);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16(const PrefillArgs &a, hipStream_t s) {
  return a.D == 128 ? launch_pc<128>(a, s) : launch_pc<64>(a, s);
}
hipError_t launch_prefill_states(const PrefillArgs &a, hipStream_t st) {
  // whole sequences (mode 3), no output: the chunk-start states and the final state
  PrefillArgs b = a;
  b.seg_mode = 3;
  b.n_splits = 1;
  const int64_t grid = (int64_t)a.n_seqs * a.H * (a.D / DVB);
  auto kern = a.D == 128 ? prefill_pc_kernel<128, false, false> : prefill_pc_kernel<64, false, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), 0, st,
                     static_cast<const bf16 *>(b.q), static_cast<const bf16 *>(nullptr),
                     static_cast<const bf16 *>(b.k), static_cast<const bf16 *>(b.v), b.alpha, b.eta,
                     b.cu_seqlens, b.seq_len_dense, b.H, b.eps, b.beta_direct, b.initial_state, b.o,
                     b.final_state, seg_of(b));
  return hipGetLastError();
}
hipError_t launch_prefill_f32(const PrefillArgs &a, hipStream_t s) {
  return a.D == 128 ? launch_d<float, 128>(a, s) : launch_d<float, 64>(a, s);
}

}  // namespace kla
