// KLA single-token decode step for gfx950.
//
// Per (sequence, head) the step is the KLA write followed by the read
// (KLA technical summary, "Resumo Tecnico: Atencao Linear Kaczmarz (KLA)",
// section "A Regra de Atualizacao KLA"), regrouped so the fp32 state is read
// from HBM once and written once:
//   x = S^T k,  y = S^T q                 (one sweep over S)
//   beta = eta / (k.k + eps),  e = v - alpha x
//   o = alpha y + beta (k.q) e            (= S_new^T q)
//   S_new = alpha S + beta k e^T
// With beta_direct the step is beta = eta, the learned scalar of Gated
// DeltaNet that KLA replaces (same summary, introduction); without alpha the
// decay is 1 (DeltaNet, "Linear Attention Architectures: Mechanisms,
// Trade-offs, and Cross-Layer Routing", section "Notacao Unificada").  With
// the per-channel decay of Kimi Delta Attention (same page, section
// "Metodologia e Estrutura") row r of the state decays by a[r]:
//   x = S^T (a o k),  y = S^T (a o q),  e = v - x,  o = y + beta (k.q) e,
//   S_new = Diag(a) S + beta k e^T.
// The kernel is bound by HBM bandwidth (0.75 flop/byte).  Every column of
// the state is independent given k and q (x and y are column sums over the
// rows), so one workgroup of 512 threads takes one (sequence, head) and 64
// state columns; each thread holds RPT = D / 32 rows x 4 columns of the state
// in registers between the read and the write.  The new state goes
// out with non-temporal stores: nothing reads it before the next step, and
// the stores then keep the caches for the loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kla_internal.h"

namespace kla {
namespace {

constexpr int kDecCols = 64;      // state columns per workgroup
constexpr int kDecThreads = 512;
typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(__bf16 x) { return static_cast<float>(x); }

template <typename E, int D, bool CH, int COLS = kDecCols, int NT = kDecThreads>
__global__ __launch_bounds__(NT) void decode_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ eta, float *__restrict__ state,
    float *__restrict__ o, float eps, int beta_direct) {
  constexpr int NQ = COLS / 4;           // float4 column groups per row (this block)
  constexpr int NRG = NT / NQ;           // row groups
  constexpr int RPT = D / NRG;           // rows per thread
  static_assert(NQ * NRG == NT && RPT * NRG == D, "decode tiling");
  constexpr int NCB = D / COLS;

  __shared__ float sq[D], sk[D], sv[COLS], se[COLS], sa[CH ? D : 1];
  __shared__ float px[NRG][COLS], py[NRG][COLS];

  const int64_t sh = blockIdx.x / NCB;  // (sequence, head) pair
  const int cb = (int)(blockIdx.x % NCB), c0 = cb * COLS;
  const int t = threadIdx.x;
  const int cq = t % NQ, rg = t / NQ;
  float *Sg = state + sh * (int64_t)(D * D) + c0;

  // Issue the state loads first: they carry all the bytes.
  float4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    s[i] = *reinterpret_cast<const float4 *>(Sg + (rg + NRG * i) * D + 4 * cq);

  for (int i = t; i < D; i += NT) {
    sq[i] = to_f32(q[sh * D + i]);
    sk[i] = to_f32(k[sh * D + i]);
    if constexpr (CH) sa[i] = alpha[sh * D + i];
  }
  if (t < COLS) sv[t] = to_f32(v[sh * D + c0 + t]);
  const float a = CH ? 1.f : (alpha ? alpha[sh] : 1.f);  // scalar decay (CH: per row below)
  const float et = eta[sh];
  __syncthreads();

  // k.k and k.q: every wave reduces its own copy (fixed order, no barrier).
  float kk = 0.f, kq = 0.f;
  {
    const int l = t & 63;
#pragma unroll
    for (int i = l; i < D; i += 64) {
      kk += sk[i] * sk[i];
      kq += sk[i] * sq[i];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      kk += __shfl_xor(kk, off, 64);
      kq += __shfl_xor(kq, off, 64);
    }
  }
  const float beta = beta_direct ? et : et / (kk + eps);

  float4 xs = {0.f, 0.f, 0.f, 0.f}, ys = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const float ar = CH ? sa[rg + NRG * i] : 1.f;
    const float kr = ar * sk[rg + NRG * i], qr = ar * sq[rg + NRG * i];
    xs.x += s[i].x * kr; xs.y += s[i].y * kr; xs.z += s[i].z * kr; xs.w += s[i].w * kr;
    ys.x += s[i].x * qr; ys.y += s[i].y * qr; ys.z += s[i].z * qr; ys.w += s[i].w * qr;
  }
  *reinterpret_cast<float4 *>(&px[rg][4 * cq]) = xs;
  *reinterpret_cast<float4 *>(&py[rg][4 * cq]) = ys;
  __syncthreads();

  if (t < COLS) {
    float x = 0.f, y = 0.f;
#pragma unroll
    for (int r = 0; r < NRG; ++r) {
      x += px[r][t];
      y += py[r][t];
    }
    const float e = sv[t] - a * x;
    se[t] = e;
    o[sh * D + c0 + t] = a * y + beta * kq * e;
  }
  __syncthreads();

  const float4 e4 = *reinterpret_cast<const float4 *>(&se[4 * cq]);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const float bk = beta * sk[rg + NRG * i];
    const float ar = CH ? sa[rg + NRG * i] : a;
    const f32x4v r = {ar * s[i].x + bk * e4.x, ar * s[i].y + bk * e4.y, ar * s[i].z + bk * e4.z,
                      ar * s[i].w + bk * e4.w};
    __builtin_nontemporal_store(r, reinterpret_cast<f32x4v *>(Sg + (rg + NRG * i) * D + 4 * cq));
  }
}

template <typename E>
hipError_t launch(const DecodeArgs &a, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.n_seqs * a.H * (a.D / kDecCols))), block(kDecThreads);
  const E *q = static_cast<const E *>(a.q), *k = static_cast<const E *>(a.k),
          *v = static_cast<const E *>(a.v);
  auto kern = a.D == 128 ? (a.channel_decay ? decode_kernel<E, 128, true> : decode_kernel<E, 128, false>)
                        : (a.channel_decay ? decode_kernel<E, 64, true> : decode_kernel<E, 64, false>);
  hipLaunchKernelGGL(kern, grid, block, 0, st, q, k, v, a.alpha, a.eta, a.state, a.o, a.eps,
                     a.beta_direct);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs &a, hipStream_t s) { return launch<__bf16>(a, s); }
hipError_t launch_decode_f32(const DecodeArgs &a, hipStream_t s) { return launch<float>(a, s); }

}  // namespace kla
