// KLA prefill with a per-channel decay (Kimi Delta Attention's gate) for
// gfx950.
//
// The linear-attention survey page ("Linear Attention Architectures:
// Mechanisms, Trade-offs, and Cross-Layer Routing", section "Metodologia e
// Estrutura") describes Kimi Delta Attention's decay as a vector with one
// rate per feature channel.  The state's rows are the key channels, so the
// decayed state is S~ = Diag(a_t) S_{t-1}; the residual, the KLA step
// beta_t = eta_t / (|k_t|^2 + eps) (or beta_t = eta_t) and the write are
// those of the scalar kernels (KLA technical summary, "Resumo Tecnico:
// Atencao Linear Kaczmarz (KLA)", sections "A Regra de Atualizacao KLA" and
// "Implementacao").
//
// Chunk form.  Inside a chunk of n <= 64 tokens let G_t be the cumulative
// log2-decay vector (one entry per key channel).  Every scalar decay factor
// of the chunk solver becomes a per-channel one:
//   Ahat_ts = sum_i k_t[i] k_s[i] 2^{G_t[i] - G_s[i]}        (t > s)
//   M_ts    = sum_i q_t[i] k_s[i] 2^{G_t[i] - G_s[i]}        (t >= s)
//   R       = V - (K o 2^G) S,  Delta = (I + StrictLower(Diag(beta) Ahat))^{-1} Diag(beta) R
//   O       = (Q o 2^G) S + M Delta
//   S'      = Diag(2^{G_n}) S + (K o 2^{G_n - G})^T Delta
// The channel factor cannot be pulled out of the contraction, so the
// operands carry it.  To keep every operand bounded, decays are measured
// from ref_b = G just before 16-row block b:
//   E_t = 2^{G_t - ref_b(t)} <= 1,   F_s = 2^{ref_b(s) - G_s} >= 1 (at most
//   16 tokens of growth),  P_bc = 2^{ref_b - ref_c} <= 1 (b > c),
//   Ahat_ts = sum_i (k_t E_t)[i] P_b(t)b(s)[i] (k_s F_s)[i],
//   (K o 2^G)_t = (k_t E_t) o 2^{ref_b(t)},  (K o 2^{G_n-G})_s = (k_s F_s) o 2^{G_n - ref_b(s)}.
// F stays below 2^100 as long as, inside every 16-token block, the product
// of each channel's rates stays above 2^-100 (every rate above ~0.013
// suffices); products that underflow lose terms below 2^-26 of their
// factor's scale.  A chunk where some channel's rates multiply below 2^-100
// inside a block (the scan flags it) takes an exact path instead: its Gram
// tiles are summed directly, sum_i x_t[i] k_s[i] 2^{G_t[i] - G_s[i]} with
// every factor <= 1, and its operands carry the absolute factors 2^{G_t}
// and 2^{G_n - G_s} (also <= 1), so nothing overflows for any rates in
// (0, 1].
//
// Mapping.  One workgroup of 4 waves per (sequence, head, 64 columns of dv),
// every operand in fp32 LDS and every contraction on the fp32 MFMA
// (v_mfma_f32_16x16x4_f32).  Per chunk:
//   stage  -> K, Q, V, log2(a) in LDS (from registers prefetched a chunk ahead)
//   scan   -> G per channel (threads < dk), block references, factor vectors
//   form   -> k o E, k o F, q o E in place
//   gram   -> wave 0: diagonal Ahat tiles, 16x16 inverses, Y planes;
//             waves 1-3: the 16 other Ahat / M tiles (kept in registers);
//             every wave: Q S and K S for its columns, R
//   write  -> -Ahat and M over the k o E and q o E space; k o F *= 2^{G_n - ref}
//   state  -> substitution, output, state update (as the scalar fp32 kernel)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kla_device.h"
#include "kla_internal.h"

namespace kla {
namespace {

template <int D>
struct KdaCfg {
  static constexpr int LDK = D + 4;    // fp32 rows of the K, Q operands
  static constexpr int LDV = DVB + 4;  // V rows (this workgroup's columns)
  static constexpr int LDP = C + 4;    // -Ahat and M planes (64 x 64)
  static constexpr int LDY = 20;       // Y diagonal blocks (16 x 16)
  static constexpr int NST = D / 16;   // state tiles per wave (dk direction)
  static_assert(C * LDP <= C * LDK, "planes must fit in the operand space");
};

template <int D>
struct KdaSmem {
  using CF = KdaCfg<D>;
  alignas(16) float KE[C * CF::LDK];  // k o E; after the Gram phase -Ahat [C][LDP]
  alignas(16) float KF[C * CF::LDK];  // log2 a -> G while scanning; then k o F; then k o 2^{G_n - G}
  alignas(16) float QE[C * CF::LDK];  // q o E; after the Gram phase M [C][LDP]
  alignas(16) float Vs[C * CF::LDV];
  alignas(16) float Yh[4 * 16 * CF::LDY];  // Y_bb = (I + L_bb)^{-1} Diag(beta_b)
  alignas(16) float Ld[4 * 16 * 20];       // -Diag(beta) Ahat in the diagonal blocks, [block][col][row]
  alignas(16) float kk[C];
  alignas(16) float et[C];
  alignas(16) float beta[C];
  alignas(16) float ref[4][D];  // G just before block b (0 for b = 0)
  alignas(16) float Z[4][D];    // 2^{ref_b}
  alignas(16) float W[4][D];    // 2^{G_n - ref_b}
  alignas(16) float P[6][D];    // 2^{ref_b - ref_c}, b > c, index b(b-1)/2 + c
  alignas(16) float Zn[D];      // 2^{G_n}
  alignas(16) float Gn[D];      // G_n
  int deep;                     // this chunk takes the exact path
};

__device__ inline f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ inline void st4(float *p, f32x4 x) { *reinterpret_cast<f32x4 *>(p) = x; }

// 16-byte segment (8 bf16 or 4 fp32) -> fp32 values
__device__ inline void to_f32(const uint4 &u, __bf16, float (&x)[8]) {
  const bf16x8 b = __builtin_bit_cast(bf16x8, u);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(b[e]);
}
__device__ inline void to_f32(const uint4 &u, float, float (&x)[4]) {
  x[0] = __uint_as_float(u.x);
  x[1] = __uint_as_float(u.y);
  x[2] = __uint_as_float(u.z);
  x[3] = __uint_as_float(u.w);
}

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void prefill_kda_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ eta,
    const int32_t *__restrict__ cu_seqlens, int64_t seq_len_dense, int H, float eps,
    int beta_direct, const float *__restrict__ S0, float *__restrict__ o,
    float *__restrict__ Sfin) {
  using CF = KdaCfg<D>;
  constexpr int NB = D / DVB;
  constexpr int NST = CF::NST;
  constexpr int LDK = CF::LDK, LDV = CF::LDV, LDP = CF::LDP, LDY = CF::LDY;
  constexpr int SEG_EL = 16 / sizeof(E);  // elements per 16-byte segment
  constexpr int SEG_ROW = D / SEG_EL;     // segments per K/Q row
  constexpr int SEG_VROW = DVB / SEG_EL;  // segments per V row (this block)
  constexpr int SEG_AROW = D / 4;         // fp32 segments per decay row
  constexpr int NSEG = C * SEG_ROW / kThreads;
  constexpr int NVSEG = C * SEG_VROW / kThreads;
  constexpr int NASEG = C * SEG_AROW / kThreads;
  static_assert(NSEG * kThreads == C * SEG_ROW && NVSEG * kThreads == C * SEG_VROW &&
                    NASEG * kThreads == C * SEG_AROW, "staging tiling");
  static_assert(kThreads % SEG_ROW == 0, "row segments must not straddle waves");

  __shared__ KdaSmem<D> sm;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int j = l >> 4, c16 = l & 15;

  const int64_t lb = logical_block();
  const int nb = (int)(lb % NB);
  const int64_t sh = lb / NB;
  const int h = (int)(sh % H);
  const int64_t s = sh / H;
  const int64_t bos = cu_seqlens ? (int64_t)cu_seqlens[s] : s * seq_len_dense;
  const int64_t eos = cu_seqlens ? (int64_t)cu_seqlens[s + 1] : bos + seq_len_dense;
  const int col = nb * DVB + 16 * w + c16;  // this lane's state/output column
  constexpr int64_t DD = (int64_t)D * D;

  f32x4 S[NST];
  {
    const rsrc_t rs = make_rsrc(S0 ? S0 + sh * DD : o, S0 ? DD * 4 : 0);
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[t][i] = buf_ld4(rs, ((16 * t + 4 * j + i) * D + col) * 4);
  }

  // ---- chunk inputs, one chunk ahead in registers ---------------------------
  uint4 kreg[NSEG], qreg[NSEG], vreg[NVSEG], areg[NASEG];
  float ereg = 0.f;
  auto fetch = [&](int64_t t0) {
    // rows past the end of the sequence fall outside the descriptors: zeros
    const int64_t nn = (eos - t0) < C ? (eos - t0) : C;
    const int64_t rowb = (int64_t)H * D * sizeof(E);
    const rsrc_t rk = make_rsrc(k + t0 * H * (int64_t)D, nn * rowb);
    const rsrc_t rq = make_rsrc(q + t0 * H * (int64_t)D, nn * rowb);
    const rsrc_t rv = make_rsrc(v + t0 * H * (int64_t)D, nn * rowb);
    const rsrc_t ra = make_rsrc(alpha + t0 * H * (int64_t)D, nn * (int64_t)H * D * 4);
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
      vreg[u] = buf_ld16(rv, (uint32_t)((r * H + h) * D + nb * DVB + cs * SEG_EL) * sizeof(E));
    }
#pragma unroll
    for (int u = 0; u < NASEG; ++u) {
      const int sg = u * kThreads + tid, r = sg / SEG_AROW, cs = sg % SEG_AROW;
      areg[u] = buf_ld16(ra, (uint32_t)((r * H + h) * D + 4 * cs) * 4);
    }
    if (w == 0) {
      const rsrc_t re = make_rsrc(eta + t0 * H, nn * H * 4);
      ereg = buf_ld4(re, (uint32_t)(l * H + h) * 4);  // zero past the end
    }
  };
  // registers -> LDS: K, Q, V as fp32, log2 of the rates (0 past the end:
  // rate 1), row norms |k|^2 from the raw keys, eta
  auto stage = [&](int64_t t0) {
    const int64_t n = (eos - t0) < C ? (eos - t0) : C;
#pragma unroll
    for (int u = 0; u < NSEG; ++u) {
      const int sg = u * kThreads + tid, r = sg / SEG_ROW, cs = sg % SEG_ROW;
      float kx[SEG_EL], qx[SEG_EL];
      to_f32(kreg[u], E(), kx);
      to_f32(qreg[u], E(), qx);
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < SEG_EL; e += 4) {
        st4(&sm.KE[r * LDK + cs * SEG_EL + e], f32x4{kx[e], kx[e + 1], kx[e + 2], kx[e + 3]});
        st4(&sm.QE[r * LDK + cs * SEG_EL + e], f32x4{qx[e], qx[e + 1], qx[e + 2], qx[e + 3]});
      }
#pragma unroll
      for (int e = 0; e < SEG_EL; ++e) part += kx[e] * kx[e];
      part = group_sum<SEG_ROW>(part);
      if (cs == 0) sm.kk[r] = part;
    }
#pragma unroll
    for (int u = 0; u < NVSEG; ++u) {
      const int sg = u * kThreads + tid, r = sg / SEG_VROW, cs = sg % SEG_VROW;
      float vx[SEG_EL];
      to_f32(vreg[u], E(), vx);
#pragma unroll
      for (int e = 0; e < SEG_EL; e += 4)
        st4(&sm.Vs[r * LDV + cs * SEG_EL + e], f32x4{vx[e], vx[e + 1], vx[e + 2], vx[e + 3]});
    }
#pragma unroll
    for (int u = 0; u < NASEG; ++u) {
      const int sg = u * kThreads + tid, r = sg / SEG_AROW, cs = sg % SEG_AROW;
      const bool in = r < n;
      f32x4 g;
      g[0] = in ? flog2_rate(__uint_as_float(areg[u].x)) : 0.f;
      g[1] = in ? flog2_rate(__uint_as_float(areg[u].y)) : 0.f;
      g[2] = in ? flog2_rate(__uint_as_float(areg[u].z)) : 0.f;
      g[3] = in ? flog2_rate(__uint_as_float(areg[u].w)) : 0.f;
      st4(&sm.KF[r * LDK + 4 * cs], g);
    }
    if (w == 0) sm.et[l] = ereg;
    if (tid == 0) sm.deep = 0;
  };

  fetch(bos);
  stage(bos);
  for (int64_t tok0 = bos; tok0 < eos; tok0 += C) {
    const int n = (int)((eos - tok0) < C ? (eos - tok0) : C);
    lds_barrier();  // chunk tok0 is staged
    fetch(tok0 + C);

    // ---- scan: G per channel, block references and factor vectors ----------
    if (tid < D) {
      const int ch = tid;
      float g = 0.f, rf[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        rf[b] = g;  // G just before block b
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) {
          const int t = 16 * b + tt;
          g += sm.KF[t * LDK + ch];
          sm.KF[t * LDK + ch] = g;
        }
      }
      // g = G_n (the rates past the end are 1); a block whose rates multiply
      // below 2^-100 in this channel sends the chunk down the exact path
      bool deep = false;
#pragma unroll
      for (int b = 0; b < 4; ++b) deep |= rf[b] - (b < 3 ? rf[b + 1] : g) > 100.f;
      if (deep) sm.deep = 1;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        sm.ref[b][ch] = rf[b];
        sm.Z[b][ch] = fexp2(rf[b]);
        sm.W[b][ch] = fexp2(g - rf[b]);
      }
#pragma unroll
      for (int b = 1; b < 4; ++b)
#pragma unroll
        for (int c = 0; c < b; ++c) sm.P[b * (b - 1) / 2 + c][ch] = fexp2(rf[b] - rf[c]);
      sm.Zn[ch] = fexp2(g);
      sm.Gn[ch] = g;
    }
    lds_barrier();

    // uniform (written before the last barrier): read as a scalar so the
    // branches on it are scalar
    const bool deep = __builtin_amdgcn_readfirstlane(sm.deep) != 0;

    // ---- form k o E, k o F, q o E in place -----------------------------------
    // (exact path: k o 2^G, q o 2^G and k o 2^{G_n - G}, with Z = W = 1)
    auto form = [&](bool exact) __attribute__((always_inline)) {
      constexpr int Q4 = D / 4;            // float4 per row
      constexpr int RPP = kThreads / Q4;   // rows per pass
      const int c4 = 4 * (tid % Q4);
#pragma unroll
      for (int r = tid / Q4; r < C; r += RPP) {
        const f32x4 G = ld4(&sm.KF[r * LDK + c4]);
        const f32x4 rf = ld4(&sm.ref[r >> 4][c4]);
        const f32x4 gn = ld4(&sm.Gn[c4]);
        const f32x4 kx = ld4(&sm.KE[r * LDK + c4]);
        const f32x4 qx = ld4(&sm.QE[r * LDK + c4]);
        f32x4 ke, kf, qe;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float Ev = exact ? fexp2(G[e]) : fexp2(G[e] - rf[e]);
          const float Fv = exact ? fexp2(fminf(gn[e] - G[e], 0.f)) : fexp2(rf[e] - G[e]);
          ke[e] = kx[e] * Ev;
          kf[e] = kx[e] * Fv;
          qe[e] = qx[e] * Ev;
        }
        st4(&sm.KE[r * LDK + c4], ke);
        st4(&sm.KF[r * LDK + c4], kf);
        st4(&sm.QE[r * LDK + c4], qe);
      }
    };
    // exact Gram element: sum_i X_t[i] K_s[i] 2^{G_t[i] - G_s[i]} for t >= s
    // (raw X = Q or K and G still in LDS), else 0
    auto exact_tile = [&](bool qk, int bi, int bj) __attribute__((always_inline)) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const int sc = 16 * bj + c16;
      const float *X = qk ? sm.QE : sm.KE;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * bi + 4 * j + i;
        if (t >= sc) {
          float a = 0.f;
#pragma unroll 1
          for (int ch = 0; ch < D; ch += 4) {
            const f32x4 x = ld4(&X[t * LDK + ch]), kv = ld4(&sm.KE[sc * LDK + ch]);
            const f32x4 gt = ld4(&sm.KF[t * LDK + ch]), gs = ld4(&sm.KF[sc * LDK + ch]);
#pragma unroll
            for (int e = 0; e < 4; ++e) a += x[e] * kv[e] * fexp2(fminf(gt[e] - gs[e], 0.f));
          }
          acc[i] = a;
        }
      }
      return acc;
    };
    // ---- Gram tiles, diagonal inverses; Q S, K S, R --------------------------
    f32x4 jt[6];  // waves 1-3: their Gram tiles until the operand space is free
    auto gram = [&](bool exact) __attribute__((always_inline)) {
    if (w == 0) {
      sm.beta[l] = beta_direct ? sm.et[l] : sm.et[l] / (sm.kk[l] + eps);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // diagonal tiles -> -Diag(beta) Ahat below the diagonal of each block
      // (acc[i] = Ahat[16b + 4j + i][16b + c16])
      auto ld_write = [&](int b, const f32x4 &acc) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * j + i;
          sm.Ld[(b * 16 + c16) * 20 + r] = r > c16 ? -sm.beta[16 * b + r] * acc[i] : 0.f;
        }
      };
      if (exact) {
#pragma unroll 1
        for (int b = 0; b < 4; ++b) {
          const f32x4 acc = exact_tile(false, b, b);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * j + i;
            sm.Ld[(b * 16 + c16) * 20 + r] = r > c16 ? -sm.beta[16 * b + r] * acc[i] : 0.f;
          }
        }
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k0 = 0; k0 < D; k0 += 4)
            acc = mma(sm.KE[(16 * b + c16) * LDK + k0 + j], sm.KF[(16 * b + c16) * LDK + k0 + j], acc);
          ld_write(b, acc);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // lane (block j, column c16): column c16 of (I + L_jj)^{-1}
      float lc[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v4 = ld4(&sm.Ld[(j * 16 + c16) * 20 + 4 * q4]);
        lc[4 * q4] = v4[0];
        lc[4 * q4 + 1] = v4[1];
        lc[4 * q4 + 2] = v4[2];
        lc[4 * q4 + 3] = v4[3];
      }
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = (r == c16) ? 1.f : 0.f;
      solve_steps(x, lc, std::make_integer_sequence<int, 15>{});
      const float bc = sm.beta[16 * j + c16];
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.Yh[(j * 16 + r) * LDY + c16] = x[r] * bc;
    } else {
      // waves 1, 2, 3: jobs [0,5), [5,10), [10,16)
      const int q0 = 5 * (w - 1);
      const int nj = w == 3 ? 6 : 5;
      if (exact) {
#pragma unroll
        for (int u = 0; u < 6; ++u) {
          if (u < nj) {
            const Job jb = job_of(q0 + u);
            jt[u] = exact_tile(jb.qk, jb.bi, jb.bj);
          }
        }
        return;
      }
#pragma unroll
      for (int u = 0; u < 6; ++u) {
        if (u < nj) {
          const Job jb = job_of(q0 + u);
          const float *A = jb.qk ? sm.QE : sm.KE;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          if (jb.bi == jb.bj) {
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += 4)
              acc = mma(A[(16 * jb.bi + c16) * LDK + k0 + j], sm.KF[(16 * jb.bj + c16) * LDK + k0 + j], acc);
          } else {
            const float *Pv = sm.P[jb.bi * (jb.bi - 1) / 2 + jb.bj];
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += 4)
              acc = mma(A[(16 * jb.bi + c16) * LDK + k0 + j] * Pv[k0 + j],
                        sm.KF[(16 * jb.bj + c16) * LDK + k0 + j], acc);
          }
          jt[u] = acc;
        }
      }
    }
    };
    // fast path: operands, then the Gram tiles on the MFMA; exact path: the
    // Gram tiles from the raw inputs, then the operands with absolute
    // factors (Z = W = 1)
    if (!deep) form(false);
    lds_barrier();
    gram(deep);
    if (deep) {
      lds_barrier();  // every read of the raw inputs is done
      if (tid < D) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          sm.Z[b][tid] = 1.f;
          sm.W[b][tid] = 1.f;
        }
      }
      form(true);
      lds_barrier();
    }

    // Q S and K S with the state rows scaled by 2^{ref_bi}: (q o 2^G) S = (q o E) (Diag(2^{ref}) S)
    f32x4 QS[4], R[4];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      f32x4 Sz[NST];
#pragma unroll
      for (int t = 0; t < NST; ++t) Sz[t] = S[t] * ld4(&sm.Z[bi][16 * t + 4 * j]);
      f32x4 aq = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < NST; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int a_off = (16 * bi + c16) * LDK + 16 * t + 4 * j + i;
          aq = mma(sm.QE[a_off], Sz[t][i], aq);
          ak = mma(sm.KE[a_off], Sz[t][i], ak);
        }
      QS[bi] = aq;
#pragma unroll
      for (int i = 0; i < 4; ++i) R[bi][i] = sm.Vs[(16 * bi + 4 * j + i) * LDV + 16 * w + c16] - ak[i];
    }
    lds_barrier();  // every read of k o E and q o E is done

    // ---- planes over the operand space; k o F -> k o 2^{G_n - G} ------------
    if (w != 0) {
      const int q0 = 5 * (w - 1);
      const int nj = w == 3 ? 6 : 5;
#pragma unroll
      for (int u = 0; u < 6; ++u) {
        if (u < nj) {
          const Job jb = job_of(q0 + u);
          const int Sc = 16 * jb.bj + c16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int Rr = 16 * jb.bi + 4 * j + i;
            if (jb.qk)
              sm.QE[Rr * LDP + Sc] = Rr >= Sc ? jt[u][i] : 0.f;  // M, lower incl. diagonal
            else
              sm.KE[Rr * LDP + Sc] = -jt[u][i];                  // -Ahat, below the diagonal blocks
          }
        }
      }
    }
    {
      constexpr int Q4 = D / 4, RPP = kThreads / Q4;
      const int c4 = 4 * (tid % Q4);
#pragma unroll
      for (int r = tid / Q4; r < C; r += RPP)
        st4(&sm.KF[r * LDK + c4], ld4(&sm.KF[r * LDK + c4]) * ld4(&sm.W[r >> 4][c4]));
    }
    lds_barrier();

    // ---- Delta by block substitution, output, state update ------------------
    const float *Ah = sm.KE;
    const float *Mh = sm.QE;
    f32x4 Dl[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      f32x4 acc = R[b];
#pragma unroll
      for (int m = 0; m < b; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = mma(Ah[(16 * b + c16) * LDP + 16 * m + 4 * j + i], Dl[m][i], acc);
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) d = mma(sm.Yh[(b * 16 + c16) * LDY + 4 * j + i], acc[i], d);
      Dl[b] = d;
    }
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      f32x4 acc = QS[bi];
#pragma unroll
      for (int mt = 0; mt <= bi; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = mma(Mh[(16 * bi + c16) * LDP + 16 * mt + 4 * j + i], Dl[mt][i], acc);
      QS[bi] = acc;  // now the output tile
    }
    {
      const rsrc_t ro = make_rsrc(o + tok0 * H * (int64_t)D, (int64_t)n * H * D * 4);
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          buf_st4(ro, (uint32_t)(((16 * bi + 4 * j + i) * H + h) * D + col) * 4, QS[bi][i]);
    }
    // S' = Diag(2^{G_n}) S + (k o 2^{G_n - G})^T Delta
#pragma unroll
    for (int t = 0; t < NST; ++t) S[t] *= ld4(&sm.Zn[16 * t + 4 * j]);
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[t] = mma(sm.KF[(16 * mt + 4 * j + i) * LDK + 16 * t + c16], Dl[mt][i], S[t]);
    lds_barrier();  // everyone is done with this chunk's LDS
    stage(tok0 + C);
  }

  {
    const rsrc_t rs = make_rsrc(Sfin ? Sfin + sh * DD : o, Sfin ? DD * 4 : 0);
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) buf_st4(rs, ((16 * t + 4 * j + i) * D + col) * 4, S[t][i]);
  }
}

// ---- bf16 inputs: the contractions on the bf16 MFMA ------------------------
// The same chunk form, exact path and substitution as above, with the fast
// path's decays referenced per channel to the chunk's midpoint decay
// r = G_n / 2 instead of per 16-token block: E'_t = 2^{G_t - r} and
// F'_s = 2^{r - G_s} = 1 / E'_s, so every Gram tile is a plain product
// (k o E' or q o E' against k o F'), Q S and K S take the state scaled by
// 2^r (split once for all row blocks), and the state update is
// S' = 2^r o (2^r o S + (k o F')^T Delta), with no rescaled copy of k o F.
// E' and F' stay within 2^{+-100} when the chunk's decay in every channel is
// at least 2^-200; a chunk below that, or with a 16-token block below
// 2^-100, takes the exact path.  E'_t is the running product of the rates
// in t's block times 2^{ref_b - r} (block totals in log2).  The contractions
// run on v_mfma_f32_16x16x32_bf16: the Gram tiles, Q S and K S, the
// substitution, M Delta and the state update.  Every fp32 factor there enters as a bf16 pair
// hi = bf16(x), lo = bf16(x - hi), and a product of two split factors is the
// three MFMAs hi*hi + hi*lo + lo*hi (the lo*lo term is below 2^-16 of the
// product).  The operand planes are kept as bf16 hi and lo planes in the
// pcol column order, so a state fragment pair or a Gram operand is one
// 16-byte read.
//
// LDS: the k o E' and q o E' planes (hi, lo); the k o F' planes share their
// rows with the raw rates and the exact path's log-decays G (D + 8 floats a
// row); E' waits as fp32 in the lo planes, each row in that row's bytes, so
// each row is formed by the one wave that read it, E' first.
// Gram jobs of the bf16 kernel with NW waves (the first four own the state
// columns).  The K K^T diagonal blocks and their inverses go to one wave
// (kda_diag_wave); the off-diagonal block pairs of (1,0) (2,0) (2,1) (3,0)
// (3,1) (3,2), each as its K K^T tile (-Ahat, u even) and its Q K^T tile (M,
// u odd), which share the k o F' operand, and then the diagonal M
// blocks go to the others:
//   NW = 4: wave 0 the diagonal blocks; waves 1-3 two pairs each
//           (2(w-1), 2(w-1)+1); diagonal M blocks: wave 1 blocks 0 and 1,
//           wave 2 block 2, wave 3 block 3;
//   NW = 8: wave 4 the diagonal blocks; waves 5-7 two pairs each
//           (2(w-5), 2(w-5)+1); diagonal M blocks: wave 5 blocks 0 and 1,
//           wave 6 block 2, wave 7 block 3 (waves 0-3 form Q S and K S for
//           their columns meanwhile).
template <int NW>
constexpr int kda_diag_wave() { return NW == 4 ? 0 : 4; }
template <int NW>
__device__ inline int kda_npairs(int w) {
  if constexpr (NW == 4) return w >= 1 ? 2 : 0;
  else return w >= 5 ? 2 : 0;
}
template <int NW>
__device__ inline int kda_njobs(int w) {
  if constexpr (NW == 4) return w == 0 ? 0 : (w == 1 ? 6 : 5);
  else return w >= 5 ? (w == 5 ? 6 : 5) : 0;
}
template <int NW>
__device__ inline Job kda_job(int w, int u) {
  Job jb;
  if (u < 2 * kda_npairs<NW>(w)) {
    const int pp = (NW == 4 ? 2 * (w - 1) : 2 * (w - 5)) + (u >> 1);
    jb.bi = pp == 0 ? 1 : pp < 3 ? 2 : 3;
    jb.bj = pp - jb.bi * (jb.bi - 1) / 2;
    jb.qk = (u & 1) != 0;
  } else {
    jb.qk = true;
    if constexpr (NW == 4) jb.bi = w == 1 ? u - 4 : w;
    else jb.bi = w == 5 ? u - 4 : w - 4;
    jb.bj = jb.bi;
  }
  return jb;
}
template <int NW>
constexpr int kda_maxjobs() { return 6; }

template <int D>
struct KdaBfSmem {
  static constexpr int LDB = D + 16;      // k o E, q o E rows (bf16; 2 LDB bytes = 32 mod 128)
  static constexpr int LDR = 2 * D + 16;  // k o F rows (bf16): hi at 0, lo at LO; 2 LDR bytes = 32 mod 128
  static constexpr int LO = D + 8;
  static constexpr int LDG = D + 8;       // the same rows as fp32 G
  static constexpr int LDV = DVB + 8;     // V rows (bf16)
  static constexpr int LDA = 20;          // -Ahat blocks (bf16 hi, lo; 16 x 16 each, transposed)
  static constexpr int LDP = C + 16;      // M planes (bf16 hi, lo; pcol order)
  static constexpr int LDYT = 24;         // Y^T rows (bf16 hi, lo)
  alignas(16) bf16 KE[2 * C * LDB];  // hi plane then lo plane; raw k in the hi plane until formed, E' in the lo plane
  alignas(16) bf16 QE[2 * C * LDB];  // the same for q
  alignas(16) bf16 KF[C * LDR];
  alignas(16) bf16 Vs[C * LDV];
  alignas(16) bf16 AP[2 * 6 * 16 * LDA];  // -Ahat planes (hi, lo), written as the Gram jobs finish
  alignas(16) bf16 MP[2 * C * LDP];       // M planes (hi, lo)
  alignas(16) bf16 Yh[4 * 16 * LDYT];  // Y_bb^T, Y_bb = (I + L_bb)^{-1} Diag(beta_b)
  alignas(16) bf16 Yl[4 * 16 * LDYT];
  alignas(16) float Ld[4 * 16 * 20];
  alignas(16) float kk[C];
  alignas(16) float et[C];
  alignas(16) float beta[C];
  // per channel, by chunk parity: the B-side scale of Q S and K S and the
  // update's post-scale 2^{G_n / 2} (1 on the exact path), and the state's
  // pre-scale 2^{G_n / 2} (2^{G_n} on the exact path)
  alignas(16) float Zr[2][D];
  alignas(16) float Yp[2][D];
  alignas(16) float Gn[D];
  int deep;
  int mode;  // 0: the chunk's decays are staged; 1: deep; 2: not scanned
};

__device__ inline f32x4 to_f32x4(bf16x4 x) {
  return f32x4{static_cast<float>(x[0]), static_cast<float>(x[1]), static_cast<float>(x[2]),
               static_cast<float>(x[3])};
}
__device__ inline Split8 split8(f32x4 a, f32x4 b) { return join(split4(a), split4(b)); }
__device__ inline bf16x4 half_lo(bf16x8 x) { return __builtin_shufflevector(x, x, 0, 1, 2, 3); }
__device__ inline bf16x4 half_hi(bf16x8 x) { return __builtin_shufflevector(x, x, 4, 5, 6, 7); }
// hi*hi + hi*lo + lo*hi on the 32-deep bf16 MFMA
__device__ inline f32x4 mma3(const Split8 &a, const Split8 &b, f32x4 c) {
  c = mma(a.hi, b.hi, c);
  c = mma(a.hi, b.lo, c);
  return mma(a.lo, b.hi, c);
}

// A copy of a lane index that the compiler cannot hoist out of the chunk
// loop: the addresses derived from it are recomputed where they are used
// instead of being held in registers across the loop.
__device__ inline int fresh_lane(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void prefill_kda_bf_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ eta,
    const int32_t *__restrict__ cu_seqlens, int64_t seq_len_dense, int H, float eps,
    int beta_direct, const float *__restrict__ S0, float *__restrict__ o,
    float *__restrict__ Sfin) {
  using SM = KdaBfSmem<D>;
  // NW waves; the first NCW = 4 own 16 state columns each (DVB in all), the
  // others (NW = 8) share only the chunk-wide phases: staging, scan, operand
  // forming, the Gram tiles and their planes
  constexpr int KT = 64 * NW, NCW = 4, DIAGW = kda_diag_wave<NW>();
  // with helper waves, they scan the next chunk's rates during the
  // substitution (from registers), and its decays are staged with it
  constexpr bool AHEAD = NW != NCW;
  static_assert(16 * NCW == DVB, "column waves");
  constexpr int NB = D / DVB;
  constexpr int NST = D / 16;
  constexpr int LDB = SM::LDB, LDR = SM::LDR, LO = SM::LO, LDG = SM::LDG, LDV = SM::LDV,
                LDA = SM::LDA, LDP = SM::LDP, LDYT = SM::LDYT;
  constexpr int SEG_EL = 8;               // bf16 per 16-byte segment
  constexpr int SEG_ROW = D / SEG_EL;     // segments per K/Q row
  constexpr int SEG_VROW = DVB / SEG_EL;  // segments per V row (this block)
  constexpr int SEG_AROW = D / 4;         // fp32 segments per decay row
  constexpr int NSEG = C * SEG_ROW / KT;
  constexpr int NVSEG = C * SEG_VROW / KT;
  constexpr int NASEG = C * SEG_AROW / KT;
  static_assert(NSEG * KT == C * SEG_ROW && NVSEG * KT == C * SEG_VROW &&
                    NASEG * KT == C * SEG_AROW, "staging tiling");
  static_assert(KT % SEG_ROW == 0, "row segments must not straddle waves");
  constexpr int Q4 = D / 4;           // 4-column groups per row
  constexpr int RPP = KT / Q4;  // rows per pass of the element-wise phases
  static_assert(64 % Q4 == 0, "a row of the element-wise phases stays inside one wave");

  __shared__ SM sm;
  bf16 *const KEh = sm.KE, *const KEl = sm.KE + C * LDB;
  bf16 *const QEh = sm.QE, *const QEl = sm.QE + C * LDB;
  float *const Gp = reinterpret_cast<float *>(sm.KF);
  // E' (the fast path's decays) as fp32 in the lo planes of k o E'
  // (channels 0 .. D/2-1) and q o E' (the others), row r in their row r,
  // rotated by 8 floats per group of 8 rows so that lanes writing rows 8
  // apart use different banks; the lo planes are free from the Gram phase's
  // last read to the next forming
  auto eptr = [&](int r, int c) __attribute__((always_inline)) {
    return reinterpret_cast<float *>(c < D / 2 ? KEl : QEl) + r * (LDB / 2) +
           (((c & (D / 2 - 1)) + 8 * (r >> 3)) & (D / 2 - 1));
  };
  static_assert(2 * D <= LDB * 2 * 2 && (LDB / 2) % 4 == 0, "E rows in the lo planes");

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int j = l >> 4, c16 = l & 15;

  const int64_t lb = logical_block();
  const int nb = (int)(lb % NB);
  const int64_t sh = lb / NB;
  const int h = (int)(sh % H);
  const int64_t s = sh / H;
  const int64_t bos = cu_seqlens ? (int64_t)cu_seqlens[s] : s * seq_len_dense;
  const int64_t eos = cu_seqlens ? (int64_t)cu_seqlens[s + 1] : bos + seq_len_dense;
  const int col = nb * DVB + 16 * w + c16;  // this lane's state/output column
  constexpr int64_t DD = (int64_t)D * D;

  f32x4 S[NST];
  if (w < NCW) {
    const rsrc_t rs = make_rsrc(S0 ? S0 + sh * DD : o, S0 ? DD * 4 : 0);
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[t][i] = buf_ld4(rs, ((16 * t + 4 * j + i) * D + col) * 4);
  }

  // ---- chunk inputs, one chunk ahead in registers ---------------------------
  uint4 kreg[NSEG], qreg[NSEG], vreg[NVSEG], areg[NASEG];
  float ereg = 0.f;
  auto fetch = [&](int64_t t0) {
    const int tid = fresh_lane(threadIdx.x), l = tid & 63;
    const int64_t nn = (eos - t0) < C ? (eos - t0) : C;
    const int64_t rowb = (int64_t)H * D * 2;
    const rsrc_t rk = make_rsrc(k + t0 * H * (int64_t)D, nn * rowb);
    const rsrc_t rq = make_rsrc(q + t0 * H * (int64_t)D, nn * rowb);
    const rsrc_t rv = make_rsrc(v + t0 * H * (int64_t)D, nn * rowb);
#pragma unroll
    for (int u = 0; u < NSEG; ++u) {
      const int sg = u * KT + tid, r = sg / SEG_ROW, cs = sg % SEG_ROW;
      const uint32_t off = (uint32_t)((r * H + h) * D + cs * SEG_EL) * 2;
      kreg[u] = buf_ld16(rk, off);
      qreg[u] = buf_ld16(rq, off);
    }
#pragma unroll
    for (int u = 0; u < NVSEG; ++u) {
      const int sg = u * KT + tid, r = sg / SEG_VROW, cs = sg % SEG_VROW;
      vreg[u] = buf_ld16(rv, (uint32_t)((r * H + h) * D + nb * DVB + cs * SEG_EL) * 2);
    }
    if (w == 0) {
      const rsrc_t re = make_rsrc(eta + t0 * H, nn * H * 4);
      ereg = buf_ld4(re, (uint32_t)(l * H + h) * 4);  // zero past the end
    }
  };
  // the rates (the largest input): without helper waves fetched half a chunk
  // later, so their registers are free during the Gram and Q S / K S phase;
  // with them, only for a chunk the helpers have not scanned
  auto fetch_a = [&](int64_t t0) {
    const int tid = fresh_lane(threadIdx.x);
    const int64_t nn = (eos - t0) < C ? (eos - t0) : C;
    const rsrc_t ra = make_rsrc(alpha + t0 * H * (int64_t)D, nn * (int64_t)H * D * 4);
#pragma unroll
    for (int u = 0; u < NASEG; ++u) {
      const int sg = u * KT + tid, r = sg / SEG_AROW, cs = sg % SEG_AROW;
      areg[u] = buf_ld16(ra, (uint32_t)((r * H + h) * D + 4 * cs) * 4);
    }
  };
  // registers -> LDS: the rates (1 past the end)
  auto stage_rates = [&](int64_t t0) {
    const int tid = fresh_lane(threadIdx.x);
    const int64_t n = (eos - t0) < C ? (eos - t0) : C;
#pragma unroll
    for (int u = 0; u < NASEG; ++u) {
      const int sg = u * KT + tid, r = sg / SEG_AROW, cs = sg % SEG_AROW;
      const bool in = r < n;
      f32x4 g;
      g[0] = in ? __uint_as_float(areg[u].x) : 1.f;
      g[1] = in ? __uint_as_float(areg[u].y) : 1.f;
      g[2] = in ? __uint_as_float(areg[u].z) : 1.f;
      g[3] = in ? __uint_as_float(areg[u].w) : 1.f;
      st4(&Gp[r * LDG + 4 * cs], g);
    }
  };
  // registers -> LDS: raw K and Q (bf16, pcol order) in the hi planes, V as
  // fp32, the rates (without helper waves), |k|^2, eta
  auto stage = [&](int64_t t0) {
    const int tid = fresh_lane(threadIdx.x), l = tid & 63;
    const int64_t n = (eos - t0) < C ? (eos - t0) : C;
#pragma unroll
    for (int u = 0; u < NSEG; ++u) {
      const int sg = u * KT + tid, r = sg / SEG_ROW, cs = sg % SEG_ROW;
      const uint4 kx = kreg[u], qx = qreg[u];
      *reinterpret_cast<uint2 *>(&KEh[r * LDB + pcol(cs * SEG_EL)]) = uint2{kx.x, kx.y};
      *reinterpret_cast<uint2 *>(&KEh[r * LDB + pcol(cs * SEG_EL + 4)]) = uint2{kx.z, kx.w};
      *reinterpret_cast<uint2 *>(&QEh[r * LDB + pcol(cs * SEG_EL)]) = uint2{qx.x, qx.y};
      *reinterpret_cast<uint2 *>(&QEh[r * LDB + pcol(cs * SEG_EL + 4)]) = uint2{qx.z, qx.w};
      const bf16x8 kb = __builtin_bit_cast(bf16x8, kx);
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < SEG_EL; ++e) {
        const float x = static_cast<float>(kb[e]);
        part += x * x;
      }
      part = group_sum<SEG_ROW>(part);
      if (cs == 0) sm.kk[r] = part;
    }
#pragma unroll
    for (int u = 0; u < NVSEG; ++u) {
      const int sg = u * KT + tid, r = sg / SEG_VROW, cs = sg % SEG_VROW;
      *reinterpret_cast<uint4 *>(&sm.Vs[r * LDV + cs * SEG_EL]) = vreg[u];
    }
    if constexpr (!AHEAD) stage_rates(t0);
    if (w == 0) sm.et[l] = ereg;
    if (tid == 0) sm.deep = 0;
  };

  // -Ahat blocks (b, m), m < b, transposed (row 16b + c16 of a lane holds
  // columns 4j..4j+3), index b(b-1)/2 + m; M in the pcol column order, its
  // two blocks above the diagonal that the 32-deep products read, (0, 1) and
  // (2, 3), zero (set once: no job writes them)
  bf16 *const Ah = sm.AP, *const Al = sm.AP + 6 * 16 * LDA;
  bf16 *const Mh = sm.MP, *const Ml = sm.MP + C * LDP;
  for (int e = tid; e < 256; e += KT) {
    // one 4-column group of one row of one plane per thread: rows 0-15 x
    // columns 16-31 and rows 32-47 x columns 48-63
    const int zr = (e >> 3) & 15, zg = e & 3, zs = (e >> 2) & 1, zp = (e >> 7) & 1;
    const int row = zs ? 32 + zr : zr, c = (zs ? 48 : 16) + 4 * zg;
    *reinterpret_cast<uint2 *>(&(zp ? Ml : Mh)[row * LDP + pcol(c)]) = uint2{0u, 0u};
  }

  fetch(bos);
  if constexpr (!AHEAD) fetch_a(bos);
  stage(bos);
  if (tid == 0) sm.mode = 2;
  for (int64_t tok0 = bos; tok0 < eos; tok0 += C) {
    // lane indices (and the addresses from them) recomputed in every chunk
    const int tid = fresh_lane(threadIdx.x), l = tid & 63, j = l >> 4, c16 = l & 15;
    const int col = nb * DVB + 16 * w + c16;
    const int n = (int)((eos - tok0) < C ? (eos - tok0) : C);
    lds_barrier();  // chunk tok0 is staged
    const int mode = AHEAD ? __builtin_amdgcn_readfirstlane(sm.mode) : 2;
    const int cur = (int)(((tok0 - bos) / C) & 1);  // factor slot of this chunk
    fetch(tok0 + C);
    bool deep = false;
    if (mode != 0) {
    if constexpr (AHEAD) {
      // the decays were not staged (first chunk) or the chunk is deep:
      // the rates from memory, then the scan below
      fetch_a(tok0);
      stage_rates(tok0);
      if (tid == 0) sm.deep = 0;
      lds_barrier();
    }

    // ---- scan: decays per channel, E' and the scales ------------------------
    // Four adjacent lanes share a channel, lane `part` with 16-token block
    // `part`: the running product of the block's rates in registers, the
    // blocks' totals in log2 by DPP, then E' = product * 2^{ref_b - r}.  A
    // block below 2^-100 or a chunk below 2^-200 sends the chunk down the
    // exact path, which takes the log-decays G from the raw rates, still in
    // this lane's registers.
    static_assert(KT / D == 4, "one 16-token block of one channel per lane");
    const int sch = tid >> 2, spart = tid & 3;
    float xr[16];
    {
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) xr[tt] = Gp[(16 * spart + tt) * LDG + sch];
      float e[16], run = 1.f;
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        run *= xr[tt];
        e[tt] = run;
      }
      // block totals in log2, the references ref_b (G before block b) and
      // the midpoint r = G_n / 2
      const float lt = __builtin_amdgcn_logf(run);
      const float L0 = dpp<0x00>(lt), L1 = dpp<0x55>(lt), L2 = dpp<0xAA>(lt), L3 = dpp<0xFF>(lt);
      const float ref = spart == 0 ? 0.f : spart == 1 ? L0 : spart == 2 ? L0 + L1 : (L0 + L1) + L2;
      const float gn = ((L0 + L1) + L2) + L3, rm = 0.5f * gn;
      const float T0 = dpp<0x00>(run), T1 = dpp<0x55>(run), T2 = dpp<0xAA>(run),
                  T3 = dpp<0xFF>(run);
      if (T0 < 0x1p-100f || T1 < 0x1p-100f || T2 < 0x1p-100f || T3 < 0x1p-100f || !(gn >= -200.f))
        sm.deep = 1;
      const float fac = fexp2(ref - rm);
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) *eptr(16 * spart + tt, sch) = e[tt] * fac;
      if (spart == 0) {
        const float zr = fexp2(rm);
        sm.Zr[cur][sch] = zr;
        sm.Yp[cur][sch] = zr;
      }
    }
    lds_barrier();
    deep = __builtin_amdgcn_readfirstlane(sm.deep) != 0;
    if (deep) {
      // G_t = log2 of the product of the chunk's rates up to t (rates below
      // 2^-126 taken as 2^-126, so every log is finite), and G_n
      float run = 0.f;
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        run += flog2_rate(xr[tt]);
        xr[tt] = run;
      }
      const float T0 = dpp<0x00>(run), T1 = dpp<0x55>(run), T2 = dpp<0xAA>(run),
                  T3 = dpp<0xFF>(run);
      const float off = spart == 0 ? 0.f : spart == 1 ? T0 : spart == 2 ? T0 + T1 : (T0 + T1) + T2;
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) Gp[(16 * spart + tt) * LDG + sch] = off + xr[tt];
      if (spart == 0) sm.Gn[sch] = ((T0 + T1) + T2) + T3;
      lds_barrier();
    }
    }  // mode != 0

    // ---- form k o E', k o F', q o E' as hi/lo planes ------------------------
    // (exact path: k o 2^G, q o 2^G and k o 2^{G_n - G}, with the state
    // scales set to match).  A row's E' (or G) is read by this wave before
    // any of the row is written.
    auto form = [&](bool exact) __attribute__((always_inline)) {
      // this lane's rows r0 + u RPP: every read first (a row is read and
      // written only by this wave), then the products, splits and writes
      constexpr int NFR = C / RPP;
      static_assert(NFR * RPP == C, "forming rows");
      const int c4 = 4 * (tid % Q4), r0 = tid / Q4;
      f32x4 Gv[NFR], kxv[NFR], qxv[NFR];
      const f32x4 gn = ld4(&sm.Gn[c4]);
#pragma unroll
      for (int u = 0; u < NFR; ++u) {
        const int r = r0 + u * RPP;
        Gv[u] = exact ? ld4(&Gp[r * LDG + c4]) : ld4(eptr(r, c4));  // G or E'
        kxv[u] = to_f32x4(*reinterpret_cast<const bf16x4 *>(&KEh[r * LDB + pcol(c4)]));
        qxv[u] = to_f32x4(*reinterpret_cast<const bf16x4 *>(&QEh[r * LDB + pcol(c4)]));
      }
      asm volatile("" ::: "memory");  // the reads above, the writes below
#pragma unroll
      for (int u = 0; u < NFR; ++u) {
        const int r = r0 + u * RPP;
        const f32x4 G = Gv[u], kx = kxv[u], qx = qxv[u];
        f32x4 ke, kf, qe;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float Ev = exact ? fexp2(G[e]) : G[e];
          const float Fv = exact ? fexp2(fminf(gn[e] - G[e], 0.f)) : __builtin_amdgcn_rcpf(G[e]);
          ke[e] = kx[e] * Ev;
          kf[e] = kx[e] * Fv;
          qe[e] = qx[e] * Ev;
        }
        const Split4 sk = split4(ke), sf = split4(kf), sq = split4(qe);
        *reinterpret_cast<bf16x4 *>(&KEh[r * LDB + pcol(c4)]) = sk.hi;
        *reinterpret_cast<bf16x4 *>(&KEl[r * LDB + pcol(c4)]) = sk.lo;
        *reinterpret_cast<bf16x4 *>(&QEh[r * LDB + pcol(c4)]) = sq.hi;
        *reinterpret_cast<bf16x4 *>(&QEl[r * LDB + pcol(c4)]) = sq.lo;
        *reinterpret_cast<bf16x4 *>(&sm.KF[r * LDR + pcol(c4)]) = sf.hi;
        *reinterpret_cast<bf16x4 *>(&sm.KF[r * LDR + LO + pcol(c4)]) = sf.lo;
      }
      asm volatile("" ::: "memory");
    };
    // exact Gram element: sum_i X_t[i] K_s[i] 2^{G_t[i] - G_s[i]} for t >= s
    // (raw X = Q or K in the hi planes, G still in LDS), else 0
    // (transposed: element i of lane (j, c16) is row 16bi + c16, column
    // 16bj + 4j + i; else row 16bi + 4j + i, column 16bj + c16)
    auto exact_tile = [&](bool qk, int bi, int bj, bool tr) __attribute__((always_inline)) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const bf16 *X = qk ? QEh : KEh;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tr ? 16 * bi + c16 : 16 * bi + 4 * j + i;
        const int sc = tr ? 16 * bj + 4 * j + i : 16 * bj + c16;
        if (t >= sc) {
          float a = 0.f;
#pragma unroll 1
          for (int ch = 0; ch < D; ch += 4) {
            const f32x4 x = to_f32x4(*reinterpret_cast<const bf16x4 *>(&X[t * LDB + pcol(ch)]));
            const f32x4 kv = to_f32x4(*reinterpret_cast<const bf16x4 *>(&KEh[sc * LDB + pcol(ch)]));
            const f32x4 gt = ld4(&Gp[t * LDG + ch]), gs = ld4(&Gp[sc * LDG + ch]);
#pragma unroll
            for (int e = 0; e < 4; ++e) a += x[e] * kv[e] * fexp2(fminf(gt[e] - gs[e], 0.f));
          }
          acc[i] = a;
        }
      }
      return acc;
    };
    // Gram tile on the bf16 MFMA: rows 16bi.. of A (k o E' or q o E') against
    // rows 16bj.. of k o F' (E'_t F'_s = 2^{G_t - G_s} for any block pair)
    auto bf_tile = [&](bool qk, int bi, int bj, bool tr) __attribute__((always_inline)) {
      const bf16 *Ah = qk ? QEh : KEh, *Al = qk ? QEl : KEl;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < D / 32; ++u) {
        const int ao = (16 * bi + c16) * LDB + 32 * u + 8 * j;
        const int bo = (16 * bj + c16) * LDR + 32 * u + 8 * j;
        Split8 a, b;
        a.hi = *reinterpret_cast<const bf16x8 *>(&Ah[ao]);
        a.lo = *reinterpret_cast<const bf16x8 *>(&Al[ao]);
        b.hi = *reinterpret_cast<const bf16x8 *>(&sm.KF[bo]);
        b.lo = *reinterpret_cast<const bf16x8 *>(&sm.KF[bo + LO]);
        acc = tr ? mma3(b, a, acc) : mma3(a, b, acc);
      }
      return acc;
    };
    // both transposed tiles of an off-diagonal pair (bi, bj): -Ahat from the
    // k o E' rows and M from the q o E' rows against rows 16bj.. of k o F'
    // (read once for both)
    auto bf_pair = [&](int bi, int bj, f32x4 &tk, f32x4 &tq) __attribute__((always_inline)) {
      tk = f32x4{0.f, 0.f, 0.f, 0.f};
      tq = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < D / 32; ++u) {
        const int ao = (16 * bi + c16) * LDB + 32 * u + 8 * j;
        const int bo = (16 * bj + c16) * LDR + 32 * u + 8 * j;
        Split8 ka, qa, f;
        ka.hi = *reinterpret_cast<const bf16x8 *>(&KEh[ao]);
        ka.lo = *reinterpret_cast<const bf16x8 *>(&KEl[ao]);
        qa.hi = *reinterpret_cast<const bf16x8 *>(&QEh[ao]);
        qa.lo = *reinterpret_cast<const bf16x8 *>(&QEl[ao]);
        f.hi = *reinterpret_cast<const bf16x8 *>(&sm.KF[bo]);
        f.lo = *reinterpret_cast<const bf16x8 *>(&sm.KF[bo + LO]);
        tk = mma3(f, ka, tk);
        tq = mma3(f, qa, tq);
      }
    };
    // ---- Gram tiles, diagonal inverses; Q S, K S, R --------------------------
    f32x4 jt[kda_maxjobs<NW>()];  // a wave's Gram tiles until they are written as planes
    auto gram = [&](bool exact) __attribute__((always_inline)) {
      if (w == DIAGW) {
        if constexpr (!AHEAD) {
          sm.beta[l] = beta_direct ? sm.et[l] : sm.et[l] / (sm.kk[l] + eps);
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        // diagonal tiles -> -Diag(beta) Ahat below the diagonal of each block
        // (acc[i] = Ahat[16b + 4j + i][16b + c16])
        if (exact) {
#pragma unroll 1
          for (int b = 0; b < 4; ++b) {
            const f32x4 acc = exact_tile(false, b, b, false);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 4 * j + i;
              sm.Ld[(b * 16 + c16) * 20 + r] = r > c16 ? -sm.beta[16 * b + r] * acc[i] : 0.f;
            }
          }
        } else {
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const f32x4 acc = bf_tile(false, b, b, false);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 4 * j + i;
              sm.Ld[(b * 16 + c16) * 20 + r] = r > c16 ? -sm.beta[16 * b + r] * acc[i] : 0.f;
            }
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // lane (block j, column c16): column c16 of (I + L_jj)^{-1}
        float lc[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v4 = ld4(&sm.Ld[(j * 16 + c16) * 20 + 4 * q4]);
          lc[4 * q4] = v4[0];
          lc[4 * q4 + 1] = v4[1];
          lc[4 * q4 + 2] = v4[2];
          lc[4 * q4 + 3] = v4[3];
        }
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == c16) ? 1.f : 0.f;
        solve_steps(x, lc, std::make_integer_sequence<int, 15>{});
        // column c16 of Y_jj, contiguous in Y^T: two 16-byte writes per plane
        const float bc = sm.beta[16 * j + c16];
        Split4 yq[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          yq[q4] = split4(f32x4{x[4 * q4] * bc, x[4 * q4 + 1] * bc, x[4 * q4 + 2] * bc, x[4 * q4 + 3] * bc});
        const int yo = (j * 16 + c16) * LDYT;
        *reinterpret_cast<bf16x8 *>(&sm.Yh[yo]) = __builtin_shufflevector(yq[0].hi, yq[1].hi, 0, 1, 2, 3, 4, 5, 6, 7);
        *reinterpret_cast<bf16x8 *>(&sm.Yh[yo + 8]) = __builtin_shufflevector(yq[2].hi, yq[3].hi, 0, 1, 2, 3, 4, 5, 6, 7);
        *reinterpret_cast<bf16x8 *>(&sm.Yl[yo]) = __builtin_shufflevector(yq[0].lo, yq[1].lo, 0, 1, 2, 3, 4, 5, 6, 7);
        *reinterpret_cast<bf16x8 *>(&sm.Yl[yo + 8]) = __builtin_shufflevector(yq[2].lo, yq[3].lo, 0, 1, 2, 3, 4, 5, 6, 7);
      } else {
        // the other waves: the jobs of kda_job
        const int nj = kda_njobs<NW>(w), np = kda_npairs<NW>(w);
        if (exact) {
#pragma unroll
          for (int u = 0; u < kda_maxjobs<NW>(); ++u) {
            if (u < nj) {
              const Job jb = kda_job<NW>(w, u);
              jt[u] = exact_tile(jb.qk, jb.bi, jb.bj, true);
            }
          }
          return;
        }
#pragma unroll
        for (int u = 0; u < 4; u += 2) {
          if (u < 2 * np) {
            const Job jb = kda_job<NW>(w, u);
            bf_pair(jb.bi, jb.bj, jt[u], jt[u + 1]);
          }
        }
#pragma unroll
        for (int u = 0; u < kda_maxjobs<NW>(); ++u) {
          if (u >= 2 * np && u < nj) {
            const Job jb = kda_job<NW>(w, u);
            jt[u] = bf_tile(true, jb.bi, jb.bj, true);
          }
        }
      }
    };
    // the jobs' tiles as planes (-Ahat negated; M masked to t >= s)
    auto write_planes = [&]() __attribute__((always_inline)) {
      const int nj = kda_njobs<NW>(w);
#pragma unroll
      for (int u = 0; u < kda_maxjobs<NW>(); ++u) {
        if (u < nj) {
          const Job jb = kda_job<NW>(w, u);
          const int r = 16 * jb.bi + c16;  // this lane's row
          f32x4 vals;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int sc = 16 * jb.bj + 4 * j + i;
            vals[i] = jb.qk ? (r >= sc ? jt[u][i] : 0.f) : -jt[u][i];
          }
          const Split4 sp = split4(vals);
          if (jb.qk) {
            const int off = r * LDP + pcol(16 * jb.bj + 4 * j);
            *reinterpret_cast<bf16x4 *>(&Mh[off]) = sp.hi;
            *reinterpret_cast<bf16x4 *>(&Ml[off]) = sp.lo;
          } else {
            const int off = ((jb.bi * (jb.bi - 1) / 2 + jb.bj) * 16 + c16) * LDA + 4 * j;
            *reinterpret_cast<bf16x4 *>(&Ah[off]) = sp.hi;
            *reinterpret_cast<bf16x4 *>(&Al[off]) = sp.lo;
          }
        }
      }
    };
    // fast path: operands, then the Gram tiles on the MFMA; exact path: the
    // Gram tiles from the raw inputs, then the operands with absolute
    // factors (and the state scales set to match)
    if (!deep) form(false);
    // with helper waves, beta on wave 0 (done forming first) for the
    // diagonal wave
    if constexpr (AHEAD) {
      if (w == 0) sm.beta[l] = beta_direct ? sm.et[l] : sm.et[l] / (sm.kk[l] + eps);
    }
    lds_barrier();
    // the next chunk's rates (helper waves), a phase ahead of their scan:
    // lane (quad cq, part p) holds channels 4cq..4cq+3 of tokens 8p..8p+7
    uint4 ra[8];
    if constexpr (AHEAD) {
      if (w >= NCW) {
        const int hl = tid - 64 * NCW, cq = hl >> 3, p8 = hl & 7;
        const int64_t t1 = tok0 + C;
        const int64_t n1 = (eos - t1) < C ? (eos - t1) : C;
        const rsrc_t rr = make_rsrc(alpha + t1 * H * (int64_t)D, n1 * (int64_t)H * D * 4);
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
          ra[tt] = buf_ld16(rr, (uint32_t)(((8 * p8 + tt) * H + h) * D + 4 * cq) * 4);
        if (hl == 0) sm.mode = 0;
      }
    }
    gram(deep);
    write_planes();
    if (deep) {
      lds_barrier();  // every read of the raw inputs is done
      if (tid < D) {
        sm.Zr[cur][tid] = 1.f;
        sm.Yp[cur][tid] = fexp2(sm.Gn[tid]);
      }
      form(true);
      lds_barrier();
    }

    // Q S and K S: (q o 2^G) S = (q o E') (Diag(2^{G_n / 2}) S), the scaled
    // state split once for every row block (the B operand)
    f32x4 QS[4], R[4];
    if (w < NCW) {
      Split8 Sf[NST / 2];
#pragma unroll
      for (int kk = 0; kk < NST / 2; ++kk)
        Sf[kk] = split8(S[2 * kk] * ld4(&sm.Zr[cur][32 * kk + 4 * j]),
                        S[2 * kk + 1] * ld4(&sm.Zr[cur][32 * kk + 16 + 4 * j]));
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        f32x4 aq = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NST / 2; ++kk) {
          const int ao = (16 * bi + c16) * LDB + 32 * kk + 8 * j;
          Split8 qa, ka;
          qa.hi = *reinterpret_cast<const bf16x8 *>(&QEh[ao]);
          qa.lo = *reinterpret_cast<const bf16x8 *>(&QEl[ao]);
          ka.hi = *reinterpret_cast<const bf16x8 *>(&KEh[ao]);
          ka.lo = *reinterpret_cast<const bf16x8 *>(&KEl[ao]);
          aq = mma3(qa, Sf[kk], aq);
          ak = mma3(ka, Sf[kk], ak);
        }
        QS[bi] = aq;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          R[bi][i] = static_cast<float>(sm.Vs[(16 * bi + 4 * j + i) * LDV + 16 * w + c16]) - ak[i];
      }
    }
    lds_barrier();  // every read of k o E and q o E is done
    if constexpr (!AHEAD) fetch_a(tok0 + C);

    if (w < NCW) {
    // ---- Delta by block substitution, output ---------------------------------
    // Delta_b = Y_bb (R_b - sum_{m<b} Ahat_bm Delta_m) on the 16-deep bf16 MFMA,
    // every factor split; then O = Q S + M Delta and the state update on the
    // 32-deep MFMA with the same split Delta
    bf16x4 yh[4], yl[4], ah[6], al[6];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int yo = (bb * 16 + 4 * j + (c16 >> 2)) * LDYT + 4 * (c16 & 3);
      yh[bb] = ld_tr(&sm.Yh[yo]);
      yl[bb] = ld_tr(&sm.Yl[yo]);
    }
#pragma unroll
    for (int qb = 0; qb < 6; ++qb) {
      const int off = (qb * 16 + c16) * LDA + 4 * j;
      ah[qb] = *reinterpret_cast<const bf16x4 *>(&Ah[off]);
      al[qb] = *reinterpret_cast<const bf16x4 *>(&Al[off]);
    }
    Split4 Ds[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      f32x4 acc = R[bb];
#pragma unroll
      for (int m = 0; m < bb; ++m) {
        const int qb = bb * (bb - 1) / 2 + m;
        acc = mma(ah[qb], Ds[m].hi, acc);
        acc = mma(ah[qb], Ds[m].lo, acc);
        acc = mma(al[qb], Ds[m].hi, acc);
      }
      const Split4 as = split4(acc);
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
      d = mma(yh[bb], as.hi, d);
      d = mma(yh[bb], as.lo, d);
      d = mma(yl[bb], as.hi, d);
      Ds[bb] = split4(d);
    }
    const Split8 Df[2] = {join(Ds[0], Ds[1]), join(Ds[2], Ds[3])};
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      f32x4 acc = QS[bi];
#pragma unroll
      for (int kk = 0; kk <= bi / 2; ++kk) {
        const int off = (16 * bi + c16) * LDP + 32 * kk + 8 * j;
        Split8 m8;
        m8.hi = *reinterpret_cast<const bf16x8 *>(&Mh[off]);
        m8.lo = *reinterpret_cast<const bf16x8 *>(&Ml[off]);
        acc = mma3(m8, Df[kk], acc);
      }
      QS[bi] = acc;  // now the output tile
    }
    {
      const rsrc_t ro = make_rsrc(o + tok0 * H * (int64_t)D, (int64_t)n * H * D * 4);
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          buf_st4(ro, (uint32_t)(((16 * bi + 4 * j + i) * H + h) * D + col) * 4, QS[bi][i]);
    }
    // S' = Diag(2^{G_n}) S + (k o 2^{G_n - G})^T Delta = Diag(2^{G_n / 2})
    // (Diag(2^{G_n / 2}) S + (k o F')^T Delta) (exact path: pre-scale 2^{G_n},
    // post-scale 1, k o F' = k o 2^{G_n - G}); the A operand by transposing
    // reads of the k o F' planes
#pragma unroll
    for (int t = 0; t < NST; ++t) S[t] *= ld4(&sm.Yp[cur][16 * t + 4 * j]);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int t = 0; t < NST; ++t) {
        const bf16 *base = &sm.KF[pcol(16 * t + 4 * (c16 & 3))];
        const int r0 = (32 * kk + 4 * j + (c16 >> 2)) * LDR, r1 = (32 * kk + 16 + 4 * j + (c16 >> 2)) * LDR;
        Split8 kt;
        kt.hi = __builtin_shufflevector(ld_tr(base + r0), ld_tr(base + r1), 0, 1, 2, 3, 4, 5, 6, 7);
        kt.lo = __builtin_shufflevector(ld_tr(base + LO + r0), ld_tr(base + LO + r1), 0, 1, 2, 3, 4, 5, 6, 7);
        S[t] = mma3(kt, Df[kk], S[t]);
      }
#pragma unroll
    for (int t = 0; t < NST; ++t) S[t] *= ld4(&sm.Zr[cur][16 * t + 4 * j]);
    } else if constexpr (AHEAD) {
      // the next chunk's scan (fast path): running products over each lane's
      // eight tokens, joined per 16-token block with the partner lane's, the
      // block totals in log2 across the lane's group of eight, E' = product
      // * 2^{ref_b - G_n / 2} to the lo planes (free now), the scales into
      // the other chunk slot
      static_assert(D == 128 && KT - 64 * NCW == 256, "helper scan layout");
      const int hl = tid - 64 * NCW, cq = hl >> 3, p8 = hl & 7;
      const int64_t t1 = tok0 + C;
      const int n1 = (int)((eos - t1) < C ? (eos - t1) : C);
      f32x4 e[8], run = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const bool in = 8 * p8 + tt < n1;
        const f32x4 x = {in ? __uint_as_float(ra[tt].x) : 1.f, in ? __uint_as_float(ra[tt].y) : 1.f,
                         in ? __uint_as_float(ra[tt].z) : 1.f, in ? __uint_as_float(ra[tt].w) : 1.f};
        run *= x;
        e[tt] = run;
      }
      f32x4 prev, L, Lq0, Lq1, O0, O1;
#pragma unroll
      for (int i = 0; i < 4; ++i) prev[i] = dpp<kQuadXor1>(run[i]);  // the partner part's total
      if (p8 & 1) {
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) e[tt] *= prev;
      }
      const f32x4 tb = (p8 & 1) ? prev * run : run * prev;  // the block's total
      bool deepb = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        deepb |= tb[i] < 0x1p-100f;
        L[i] = __builtin_amdgcn_logf(tb[i]);
        Lq0[i] = dpp<0x00>(L[i]);  // blocks 2 (p8 >> 2) and 2 (p8 >> 2) + 1
        Lq1[i] = dpp<0xAA>(L[i]);
        O0[i] = dpp<kHalfMirror>(Lq0[i]);  // the other quad's two blocks
        O1[i] = dpp<kHalfMirror>(Lq1[i]);
      }
      const bool hiq = (p8 & 4) != 0;
      const f32x4 L0 = hiq ? O0 : Lq0, L1 = hiq ? O1 : Lq1, L2 = hiq ? Lq0 : O0, L3 = hiq ? Lq1 : O1;
      const f32x4 gn = ((L0 + L1) + L2) + L3, rm = 0.5f * gn;
      const int bk = p8 >> 1;
      const f32x4 ref = bk == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : bk == 1 ? L0 : bk == 2 ? L0 + L1 : (L0 + L1) + L2;
      f32x4 fac, zr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        deepb |= !(gn[i] >= -200.f);
        fac[i] = fexp2(ref[i] - rm[i]);
        zr[i] = fexp2(rm[i]);
      }
      if (deepb) sm.mode = 1;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) st4(eptr(8 * p8 + tt, 4 * cq), e[tt] * fac);
      if (p8 == 0) {
        st4(&sm.Zr[cur ^ 1][4 * cq], zr);
        st4(&sm.Yp[cur ^ 1][4 * cq], zr);
      }
    }
    lds_barrier();  // everyone is done with this chunk's LDS
    stage(tok0 + C);
  }

  if (w < NCW) {
    const rsrc_t rs = make_rsrc(Sfin ? Sfin + sh * DD : o, Sfin ? DD * 4 : 0);
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) buf_st4(rs, ((16 * t + 4 * j + i) * D + col) * 4, S[t][i]);
  }
}

template <int D>
hipError_t launch_kda_bf(const PrefillArgs &a, hipStream_t st) {
  // d = 128: four more waves for the chunk-wide phases
  constexpr int NW = D == 128 ? 8 : 4;
  const int64_t grid = (int64_t)a.n_seqs * a.H * (D / DVB);
  hipLaunchKernelGGL((prefill_kda_bf_kernel<D, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, st,
                     static_cast<const bf16 *>(a.q), static_cast<const bf16 *>(a.k),
                     static_cast<const bf16 *>(a.v), a.alpha, a.eta, a.cu_seqlens, a.seq_len_dense,
                     a.H, a.eps, a.beta_direct, a.initial_state, a.o, a.final_state);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_kda(const PrefillArgs &a, hipStream_t st) {
  const int64_t grid = (int64_t)a.n_seqs * a.H * (D / DVB);
  hipLaunchKernelGGL((prefill_kda_kernel<E, D>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                     static_cast<const E *>(a.q), static_cast<const E *>(a.k),
                     static_cast<const E *>(a.v), a.alpha, a.eta, a.cu_seqlens, a.seq_len_dense,
                     a.H, a.eps, a.beta_direct, a.initial_state, a.o, a.final_state);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_kda(const PrefillArgs &a, bool bf16_inputs, hipStream_t s) {
  if (bf16_inputs) return a.D == 128 ? launch_kda_bf<128>(a, s) : launch_kda_bf<64>(a, s);
  return a.D == 128 ? launch_kda<float, 128>(a, s) : launch_kda<float, 64>(a, s);
}

}  // namespace kla
