// KLA chunkwise-parallel prefill for gfx950 (CDNA4).
//
// Method: the KLA technical summary ("Resumo Tecnico: Atencao Linear
// Kaczmarz (KLA)", gist.science/pt/paper/2605.08587) keeps Gated
// DeltaNet's chunk-parallel algorithm and changes only the diagonal
// coefficient matrix B = Diag(beta) of the chunk solver (section
// "Implementacao"), with beta_t = eta_t / (|k_t|^2 + eps) (section
// "A Regra de Atualizacao KLA").  For a chunk of n <= 64 tokens with
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
// W is never formed (one dk-long contraction less per chunk).
//
// Mapping.  One workgroup of 4 waves per (sequence, head, 64-column block of
// dv); each wave owns 16 columns of the state and keeps them in MFMA
// accumulator registers for the whole sequence.  Per chunk all waves stage
// K, Q, V and the gates in LDS, compute the Gram tiles on MFMA, solve T in
// fp32, and then each wave runs the state-dependent chain on its own
// columns.  A state tile in accumulator layout feeds the next MFMA directly
// as its B operand: the contraction index is permuted consistently on the A
// side, so the state never goes through LDS.
//
// Precision.  bf16 inputs enter MFMA exactly.  Every fp32 intermediate
// (S, T, R, M, Delta) enters as a hi+lo pair of bf16 (x = hi + lo + O(2^-17 x));
// products of two split operands use hi*hi + hi*lo + lo*hi.  fp32 inputs use
// the fp32 MFMA (v_mfma_f32_16x16x4_f32) throughout.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kla_internal.h"

namespace kla {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;         // chunk length
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int DVB = 16 * kWaves;  // dv columns per workgroup

// Lower-triangular 16x16 tile list of a 64x64 matrix (row block, col block).
__constant__ int8_t kTri[10][2] = {{0, 0}, {1, 0}, {1, 1}, {2, 0}, {2, 1},
                                   {2, 2}, {3, 0}, {3, 1}, {3, 2}, {3, 3}};

template <typename E, int D>
struct Cfg {
  static constexpr bool BF = std::is_same<E, bf16>::value;
  using P = typename std::conditional<BF, bf16, float>::type;  // operand-plane type
  static constexpr int LDK = D + (BF ? 8 : 4);   // K, Q rows (elements)
  static constexpr int LDKT = C + 8;             // K^T rows (bf16 only)
  static constexpr int LDV = DVB + (BF ? 8 : 4); // V rows
  static constexpr int LDF = C + 4;              // fp32 64x64 work matrices
  static constexpr int LDP = BF ? C + 8 : C + 4; // T, M operand planes
  static constexpr int NST = D / 16;             // state tiles per wave (dk direction)
};

template <typename E, int D>
struct Smem {
  using CF = Cfg<E, D>;
  using P = typename CF::P;
  // Every member starts on a 16-byte boundary (128-bit LDS accesses).
  alignas(16) E Kr[C * CF::LDK];
  alignas(16) E Qr[C * CF::LDK];
  alignas(16) E Kt[CF::BF ? D * CF::LDKT : 8];
  alignas(16) E Vs[C * CF::LDV];
  alignas(16) float Lf[C * CF::LDF];
  alignas(16) float Xf[C * CF::LDF];
  alignas(16) P Th[C * CF::LDP];
  alignas(16) P Tl[CF::BF ? C * CF::LDP : 8];
  alignas(16) P Mh[C * CF::LDP];
  alignas(16) P Ml[CF::BF ? C * CF::LDP : 8];
  alignas(16) float tmp[3 * 256];
  alignas(16) float g[C];
  alignas(16) float beta[C];
  alignas(16) float gam[C];
  alignas(16) float rgam[C];
  alignas(16) float al[C];
  alignas(16) float et[C];
};

__device__ inline f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct Split8 {
  bf16x8 hi, lo;
};

// B operand of a 32-deep bf16 MFMA taken from two accumulator tiles that
// cover contraction rows [0,16) and [16,32): element i of lane-group j holds
// row 4j+i (i<4) or 16+4j+(i-4) (i>=4).  Each value is split into hi + lo.
__device__ inline Split8 split_tiles(f32x4 c0, f32x4 c1) {
  Split8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bf16 h0 = static_cast<bf16>(c0[i]);
    bf16 h1 = static_cast<bf16>(c1[i]);
    r.hi[i] = h0;
    r.lo[i] = static_cast<bf16>(c0[i] - static_cast<float>(h0));
    r.hi[4 + i] = h1;
    r.lo[4 + i] = static_cast<bf16>(c1[i] - static_cast<float>(h1));
  }
  return r;
}

// A operand matching split_tiles' row order: from a row-major source row
// (pointer at column kb), columns kb+4j..kb+4j+3 and kb+16+4j..kb+16+4j+3.
__device__ inline bf16x8 lda_perm(const bf16 *row, int j) {
  bf16x4 x = *reinterpret_cast<const bf16x4 *>(row + 4 * j);
  bf16x4 y = *reinterpret_cast<const bf16x4 *>(row + 16 + 4 * j);
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ inline void store_split(bf16 *h, bf16 *l, int idx, float x) {
  bf16 hv = static_cast<bf16>(x);
  h[idx] = hv;
  l[idx] = static_cast<bf16>(x - static_cast<float>(hv));
}
__device__ inline void store_split(float *h, float *, int idx, float x) { h[idx] = x; }

// XCD-aware workgroup order: consecutive logical ids land on one XCD so the
// dv-blocks of one (sequence, head) share that XCD's L2.  Bijective for any
// grid size, whatever the hardware dispatch order.
__device__ inline int64_t logical_block() {
  const int64_t G = gridDim.x, i = blockIdx.x;
  const int64_t q = G / 8, r = G % 8, x = i % 8, kx = i / 8;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + kx;
}

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void prefill_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ eta,
    const int32_t *__restrict__ cu_seqlens, int64_t seq_len_dense, int H, float eps,
    const float *__restrict__ S0, float *__restrict__ o, float *__restrict__ Sfin) {
  using CF = Cfg<E, D>;
  using P = typename CF::P;
  constexpr bool BF = CF::BF;
  constexpr int NB = D / DVB;
  constexpr int NST = CF::NST;
  constexpr int SEG_EL = 16 / sizeof(E);       // elements per 16-byte segment
  constexpr int SEG_ROW = D / SEG_EL;          // segments per K/Q row
  constexpr int SEG_VROW = DVB / SEG_EL;       // segments per V row (this block)

  __shared__ Smem<E, D> sm;

  const int tid = threadIdx.x;
  const int w = tid / 64, l = tid % 64;
  const int j = l / 16, c16 = l % 16;

  const int64_t lb = logical_block();
  const int nb = (int)(lb % NB);
  const int64_t shi = lb / NB;
  const int h = (int)(shi % H);
  const int64_t s = shi / H;
  int64_t bos, eos;
  if (cu_seqlens) {
    bos = cu_seqlens[s];
    eos = cu_seqlens[s + 1];
  } else {
    bos = s * seq_len_dense;
    eos = bos + seq_len_dense;
  }
  const int col = nb * DVB + 16 * w + c16;  // this lane's state/output column

  // Planes of T and M above the block diagonal are read as zeros.
  for (int i = tid; i < C * CF::LDP; i += kThreads) {
    sm.Th[i] = P(0.f);
    sm.Mh[i] = P(0.f);
    if constexpr (BF) {
      sm.Tl[i] = P(0.f);
      sm.Ml[i] = P(0.f);
    }
  }

  // State tiles: tile t holds rows 16t+4j+i (i<4), column `col`.
  f32x4 S[NST];
  {
    const float *src = S0 ? S0 + ((s * H + h) * (int64_t)D) * D : nullptr;
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[t][i] = src ? src[(16 * t + 4 * j + i) * D + col] : 0.f;
  }

  for (int64_t tok0 = bos; tok0 < eos; tok0 += C) {
    const int n = (int)((eos - tok0) < C ? (eos - tok0) : C);

    // ---- stage the chunk in LDS (rows >= n are zero) ----------------------
    __syncthreads();  // previous chunk's readers are done with LDS
    for (int sg = tid; sg < C * SEG_ROW; sg += kThreads) {
      const int r = sg / SEG_ROW, cs = sg % SEG_ROW;
      uint4 kv = {0, 0, 0, 0}, qv = {0, 0, 0, 0};
      if (r < n) {
        const int64_t off = ((tok0 + r) * H + h) * (int64_t)D + cs * SEG_EL;
        kv = *reinterpret_cast<const uint4 *>(k + off);
        qv = *reinterpret_cast<const uint4 *>(q + off);
      }
      *reinterpret_cast<uint4 *>(&sm.Kr[r * CF::LDK + cs * SEG_EL]) = kv;
      *reinterpret_cast<uint4 *>(&sm.Qr[r * CF::LDK + cs * SEG_EL]) = qv;
      if constexpr (BF) {
        const bf16 *ke = reinterpret_cast<const bf16 *>(&kv);
#pragma unroll
        for (int e = 0; e < SEG_EL; ++e) sm.Kt[(cs * SEG_EL + e) * CF::LDKT + r] = ke[e];
      }
    }
    for (int sg = tid; sg < C * SEG_VROW; sg += kThreads) {
      const int r = sg / SEG_VROW, cs = sg % SEG_VROW;
      uint4 vv = {0, 0, 0, 0};
      if (r < n)
        vv = *reinterpret_cast<const uint4 *>(v + ((tok0 + r) * H + h) * (int64_t)D +
                                              nb * DVB + cs * SEG_EL);
      *reinterpret_cast<uint4 *>(&sm.Vs[r * CF::LDV + cs * SEG_EL]) = vv;
    }
    if (tid < C) {
      const bool in = tid < n;
      sm.al[tid] = in ? alpha[(tok0 + tid) * H + h] : 1.f;
      sm.et[tid] = in ? eta[(tok0 + tid) * H + h] : 0.f;
    }
    __syncthreads();

    // ---- gates: beta, cumulative log-decay g (wave 0, one lane per row) ---
    if (w == 0) {
      float kk = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) {
        const float x = static_cast<float>(sm.Kr[l * CF::LDK + d]);
        kk += x * x;
      }
      const float b = l < n ? sm.et[l] / (kk + eps) : 0.f;
      float g = l < n ? logf(sm.al[l]) : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(g, off, 64);
        if (l >= off) g += y;
      }
      const float glast = __shfl(g, 63, 64);
      sm.g[l] = g;
      sm.beta[l] = b;
      sm.gam[l] = expf(g);
      sm.rgam[l] = expf(glast - g);
    }
    __syncthreads();

    // ---- Gram tiles on MFMA: L (fp32, for the solve) and M (operand) -----
    for (int job = w; job < 20; job += kWaves) {
      const int bi = kTri[job % 10][0], bj = kTri[job % 10][1];
      const E *A = job < 10 ? sm.Kr : sm.Qr;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF) {
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += 32) {
          bf16x8 a = *reinterpret_cast<const bf16x8 *>(&A[(16 * bi + c16) * CF::LDK + k0 + 8 * j]);
          bf16x8 b =
              *reinterpret_cast<const bf16x8 *>(&sm.Kr[(16 * bj + c16) * CF::LDK + k0 + 8 * j]);
          acc = mma(a, b, acc);
        }
      } else {
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += 4)
          acc = mma(A[(16 * bi + c16) * CF::LDK + k0 + j], sm.Kr[(16 * bj + c16) * CF::LDK + k0 + j],
                    acc);
      }
      const int sc = 16 * bj + c16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * bi + 4 * j + i;
        const float dec = expf(fminf(sm.g[r] - sm.g[sc], 0.f));
        if (job < 10)
          sm.Lf[r * CF::LDF + sc] = r > sc ? sm.beta[r] * acc[i] * dec : 0.f;
        else
          store_split(sm.Mh, sm.Ml, r * CF::LDP + sc, r >= sc ? acc[i] * dec : 0.f);
      }
    }

    // ---- state-dependent products that do not need T: QS, KS, R ---------
    f32x4 QS[4], R[4];
    if constexpr (BF) {
      Split8 Sf[NST / 2];
#pragma unroll
      for (int kk = 0; kk < NST / 2; ++kk) Sf[kk] = split_tiles(S[2 * kk], S[2 * kk + 1]);
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
    // R = V - diag(gamma) K S  (rows 16bi+4j+i, local column 16w+c16)
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * bi + 4 * j + i;
        R[bi][i] = static_cast<float>(sm.Vs[r * CF::LDV + 16 * w + c16]) - sm.gam[r] * R[bi][i];
      }
    __syncthreads();

    // ---- T = (I + L)^{-1} Diag(beta): blocked forward substitution --------
    // Diagonal 16x16 blocks: wave 0, lane (block j, column c16) solves
    // (I + L_jj) x = e_c by substitution down the rows.
    if (w == 0) {
      float x[16];
      const int b0 = 16 * j;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = (r == c16) ? 1.f : 0.f;
#pragma unroll
        for (int t = 0; t < r; ++t) acc -= sm.Lf[(b0 + r) * CF::LDF + b0 + t] * x[t];
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.Xf[(b0 + r) * CF::LDF + b0 + c16] = x[r];
    }
    __syncthreads();
    // Off-diagonal blocks by distance d from the diagonal:
    //   X_ij = -X_ii * sum_{m=j}^{i-1} L_im X_mj,  i - j = d.
    {
      const int rr = tid / 16, cc = tid % 16;
      for (int d = 1; d < 4; ++d) {
        for (int qb = 0; qb < 4 - d; ++qb) {
          const int i = d + qb, jb = qb;
          float acc = 0.f;
          for (int m = jb; m < i; ++m)
#pragma unroll
            for (int t = 0; t < 16; ++t)
              acc += sm.Lf[(16 * i + rr) * CF::LDF + 16 * m + t] *
                     sm.Xf[(16 * m + t) * CF::LDF + 16 * jb + cc];
          sm.tmp[qb * 256 + tid] = acc;
        }
        __syncthreads();
        for (int qb = 0; qb < 4 - d; ++qb) {
          const int i = d + qb, jb = qb;
          float acc = 0.f;
#pragma unroll
          for (int t = 0; t < 16; ++t)
            acc += sm.Xf[(16 * i + rr) * CF::LDF + 16 * i + t] * sm.tmp[qb * 256 + t * 16 + cc];
          sm.Xf[(16 * i + rr) * CF::LDF + 16 * jb + cc] = -acc;
        }
        __syncthreads();
      }
      // T = X Diag(beta) on the lower block triangle, as MFMA operand planes.
#pragma unroll
      for (int tt = 0; tt < 10; ++tt) {
        const int r = 16 * kTri[tt][0] + rr, sc = 16 * kTri[tt][1] + cc;
        store_split(sm.Th, sm.Tl, r * CF::LDP + sc, sm.Xf[r * CF::LDF + sc] * sm.beta[sc]);
      }
    }
    __syncthreads();

    // ---- chain: Delta = T R, O = diag(gamma) QS + M Delta, state update ---
    f32x4 Dl[4];
    if constexpr (BF) {
      Split8 Rf[2];
      Rf[0] = split_tiles(R[0], R[1]);
      Rf[1] = split_tiles(R[2], R[3]);
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk <= bi / 2; ++kk) {
          const int off = (16 * bi + c16) * CF::LDP + 32 * kk;
          const bf16x8 ah = lda_perm(&sm.Th[off], j), al = lda_perm(&sm.Tl[off], j);
          acc = mma(ah, Rf[kk].hi, acc);
          acc = mma(ah, Rf[kk].lo, acc);
          acc = mma(al, Rf[kk].hi, acc);
        }
        Dl[bi] = acc;
      }
      Split8 Df[2];
      Df[0] = split_tiles(Dl[0], Dl[1]);
      Df[1] = split_tiles(Dl[2], Dl[3]);
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
      for (int bi = 0; bi < 4; ++bi) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int mt = 0; mt <= bi; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc = mma(sm.Th[(16 * bi + c16) * CF::LDP + 16 * mt + 4 * j + i], R[mt][i], acc);
        Dl[bi] = acc;
      }
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = sm.gam[16 * bi + 4 * j + i] * QS[bi][i];
        for (int mt = 0; mt <= bi; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc = mma(sm.Mh[(16 * bi + c16) * CF::LDP + 16 * mt + 4 * j + i], Dl[mt][i], acc);
        QS[bi] = acc;
      }
    }

    // output rows < n
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * bi + 4 * j + i;
        if (r < n) o[((tok0 + r) * H + h) * (int64_t)D + col] = QS[bi][i];
      }

    // S' = e^{g_n} S + K^T Diag(e^{g_n - g}) Delta
    const float glast = sm.gam[C - 1];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int i = 0; i < 4; ++i) Dl[bi][i] *= sm.rgam[16 * bi + 4 * j + i];
#pragma unroll
    for (int t = 0; t < NST; ++t) S[t] *= glast;
    if constexpr (BF) {
      Split8 Hf[2];
      Hf[0] = split_tiles(Dl[0], Dl[1]);
      Hf[1] = split_tiles(Dl[2], Dl[3]);
#pragma unroll
      for (int t = 0; t < NST; ++t)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 a = lda_perm(&sm.Kt[(16 * t + c16) * CF::LDKT + 32 * kk], j);
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
  }

  if (Sfin) {
    float *dst = Sfin + ((s * H + h) * (int64_t)D) * D;
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(16 * t + 4 * j + i) * D + col] = S[t][i];
  }
}

template <typename E, int D>
hipError_t launch_d(const PrefillArgs &a, hipStream_t st) {
  const int64_t grid = (int64_t)a.n_seqs * a.H * (D / DVB);
  hipLaunchKernelGGL((prefill_kernel<E, D>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                     static_cast<const E *>(a.q), static_cast<const E *>(a.k),
                     static_cast<const E *>(a.v), a.alpha, a.eta, a.cu_seqlens, a.seq_len_dense,
                     a.H, a.eps, a.initial_state, a.o, a.final_state);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs &a, hipStream_t s) {
  return a.D == 128 ? launch_d<bf16, 128>(a, s) : launch_d<bf16, 64>(a, s);
}
hipError_t launch_prefill_f32(const PrefillArgs &a, hipStream_t s) {
  return a.D == 128 ? launch_d<float, 128>(a, s) : launch_d<float, 64>(a, s);
}

}  // namespace kla
