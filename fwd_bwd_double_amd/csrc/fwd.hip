// Forward pass: O = softmax(scale * Q K^T + mask) V and the row LSE.
//
// Tiled online softmax as on the FlashAttention explainer page (marketmaker.cc,
// flash-attention-trading-models), sections "The Flash Attention algorithm"
// and "The online softmax recurrence": a workgroup owns 128 query rows (32 per
// wave, one query per lane), streams 64-key tiles of K and V through LDS and
// keeps per row a running raw-score max m, a running sum l and an fp32 output
// accumulator, rescaling both by exp(scale*(m_old - m_new)) whenever the max
// grows.  The division by l happens once, after the last tile.  The exponent
// is formed as (S - m) * scale: subtracting the max before scaling makes the
// largest weight exactly 1 (GProj page, rit.work
// flashattention-bf16-gradient-gproj, section "Why the error shows up at the
// end of training").  Key tiles entirely in the future of the workgroup's rows
// are never loaded (explainer page, section "Causal masking is where trading
// gets a discount").
#include "launch.hpp"
#include "tile.hpp"

namespace fbd {

template <class T, int BN, bool CAUSAL>
__global__ __launch_bounds__(NT) void fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                 const T* __restrict__ V, T* __restrict__ O,
                                                 float* __restrict__ LSE, int N, int BH, int nblk,
                                                 float scale) {
  constexpr int RS = Lay<T>::RS;
  using Stage = TileStage<T, BN>;
  constexpr int TS = Stage::TS;
  __shared__ __attribute__((aligned(16))) T Ks[BN * RS];
  __shared__ __attribute__((aligned(16))) T Vt[HD * TS];

  const Work wk = row_work(BH, nblk);
  const size_t hoff = (size_t)wk.head * N * HD;
  const T* Qh = Q + hoff;
  const T* Kh = K + hoff;
  const T* Vh = V + hoff;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q0 = wk.blk * BLK;
  const int qw = q0 + wave * WROWS;
  const int my_i = qw + (lane & 31);
  const int h = lane >> 5;
  const float sl2 = scale * LOG2E;

  Frag<T> qf[4];
  ld_frags(Qh, N, qw, lane, qf);

  float m = -INFINITY, l = 0.f;
  f32x16 o0 = zero16(), o1 = zero16();

  const int jend = CAUSAL ? min(N, q0 + BLK) : N;
  const int ntiles = (jend + BN - 1) / BN;
  Stage sk, sv;
  sk.load(Kh, N, 0, tid);
  sv.load(Vh, N, 0, tid);
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * BN;
    __syncthreads();
    sk.store_rows(Ks, tid);
    sv.store_tr(Vt, tid);
    __syncthreads();
    if (t + 1 < ntiles) {
      sk.load(Kh, N, j0 + BN, tid);
      sv.load(Vh, N, j0 + BN, tid);
    }
#pragma unroll
    for (int jb = 0; jb < BN; jb += 32) {
      // Every wave computes every sub-block of the workgroup's key range; keys
      // after a row (causal) or past N are masked to -inf.  Keeping the waves'
      // control flow identical keeps the accumulators in fixed registers.
      const int js = j0 + jb;
      f32x16 sacc = zero16();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mma(sacc, ld_row(Ks, jb, kb, lane), qf[kb]);
      float s[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = sacc[v];
      if (CAUSAL ? (js + 31 > qw) : (js + 32 > N)) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = js + 8 * (v >> 2) + 4 * h + (v & 3);
          s[v] = (CAUSAL ? (j > my_i) : (j >= N)) ? -INFINITY : s[v];
        }
      }
      float mt = s[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mt = fmaxf(mt, s[v]);
      mt = fmaxf(mt, other_half(mt));
      // the first sub-block (key 0) is visible to every row, so m is finite
      // from then on and a fully masked sub-block leaves it unchanged
      const float mn = fmaxf(m, mt);
      if (__any(mn > m)) {
        const float alpha = __builtin_amdgcn_exp2f((m - mn) * sl2);
        l *= alpha;
        o0 *= alpha;
        o1 *= alpha;
        m = mn;
      }
      float p[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        p[v] = __builtin_amdgcn_exp2f((s[v] - mn) * sl2);
        l += p[v];
      }
      const Frag<T> pf0 = pack8<T>(p), pf1 = pack8<T>(p + 8);
      const int jt = jb / 16;
      mma(o0, ld_tr(Vt, TS, 0, jt, lane), pf0);
      mma(o0, ld_tr(Vt, TS, 0, jt + 1, lane), pf1);
      mma(o1, ld_tr(Vt, TS, 32, jt, lane), pf0);
      mma(o1, ld_tr(Vt, TS, 32, jt + 1, lane), pf1);
    }
  }
  l += other_half(l);
  const float inv = 1.f / l;
  float out[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) out[v] = o0[v] * inv;
  st_cols(O + hoff, N, qw, 0, lane, out);
#pragma unroll
  for (int v = 0; v < 16; ++v) out[v] = o1[v] * inv;
  st_cols(O + hoff, N, qw, 32, lane, out);
  if (h == 0 && my_i < N)
    LSE[(size_t)wk.head * N + my_i] = scale * m + __builtin_amdgcn_logf(l) * LN2;
}

template <class T, bool CAUSAL>
static hipError_t launch_fwd_t(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               int BH, int N, float scale, hipStream_t st) {
  constexpr int BN = 64;
  const int nblk = (N + BLK - 1) / BLK;
  hipLaunchKernelGGL((fwd_kernel<T, BN, CAUSAL>), dim3(nblk * BH), dim3(NT), 0, st, (const T*)Q,
                     (const T*)K, (const T*)V, (T*)O, LSE, N, BH, nblk, scale);
  return hipGetLastError();
}

hipError_t launch_fwd(int dt, const void* Q, const void* K, const void* V, void* O, float* LSE,
                      int BH, int N, int causal, float scale, hipStream_t st) {
  if (dt == 0) {
    if (causal) return launch_fwd_t<bf16, true>(Q, K, V, O, LSE, BH, N, scale, st);
    return launch_fwd_t<bf16, false>(Q, K, V, O, LSE, BH, N, scale, st);
  }
  if (causal) return launch_fwd_t<float, true>(Q, K, V, O, LSE, BH, N, scale, st);
  return launch_fwd_t<float, false>(Q, K, V, O, LSE, BH, N, scale, st);
}

}  // namespace fbd
