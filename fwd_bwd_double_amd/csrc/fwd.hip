// Forward pass: O = softmax(scale * Q K^T + mask) V and the row LSE.
//
// Tiled online softmax as on the FlashAttention explainer page (marketmaker.cc,
// flash-attention-trading-models), sections "The Flash Attention algorithm"
// and "The online softmax recurrence": a workgroup owns 128 query rows, streams
// 64-key tiles of K and V through LDS, and keeps per row a running raw-score
// max m, a running sum l and an fp32 output accumulator, rescaling both by
// exp(scale*(m_old - m_new)) when the max grows (once per tile; a wave skips
// the rescale when none of its rows' max moved).  The division by l happens
// once, after the last tile.  The exponent is formed as (S - m) * scale:
// subtracting the max before scaling makes the largest weight exactly 1 (GProj
// page, rit.work flashattention-bf16-gradient-gproj, section "Why the error
// shows up at the end of training", on fusing the scale and the max into one
// operation).  fp32 operands keep that order exactly: the score MFMAs start
// from -m in their accumulator, so they arrive as S - m, and only a row whose
// max grew inside a tile subtracts the growth before the scaling.  For bf16
// the score MFMAs start from zero (no accumulator image of -m to rebuild per
// tile) and the subtraction and the scaling share the FMA that forms the
// exponent, (S - m) * scale * log2(e) as one rounding of S * c - m * c: the
// weight at the max is then 2^e with |e| at most half an ulp of m * c, which
// the bf16 rounding of P (the value both l and P V use) takes to exactly 1
// while |m * c * log2(e)| < 2^16.  A wave with a row at 2^15 or beyond there
// subtracts the max first instead (one more VALU operation per weight, only
// in such tiles), so the largest weight is exactly 1 always.  Key tiles
// entirely in the future of the workgroup's rows are never loaded (explainer page, section
// "Causal masking is where trading gets a discount").
//
// K and V tiles reach LDS by buffer -> LDS DMA into two alternating buffers:
// the copy of tile t+1 runs while tile t is computed.  V is read along the
// key index with the transposing LDS read, so both stay row-major.
//
// Layout: NW waves per workgroup, FWD_G groups of 32 queries per wave,
// one query per lane in each group (4 x 1 measured fastest on MI355X: more
// groups per wave halve LDS reads per FLOP but cost occupancy).  The row sum
// l adds the bf16-rounded probabilities -- the values the P V product uses --
// with v_dot2_f32_bf16.
#include <type_traits>

#include "launch.hpp"
#include "tile.hpp"

namespace fbd {

constexpr int FWD_G = FBD_FWD_G;   // 32-query groups per wave

// NW waves per workgroup: 4 (128 query rows), or 8 (256 rows) for long
// sequences without a block mask
template <class T, int BN, int NW, bool CAUSAL, bool DOCS, bool BMASK>
__global__ __launch_bounds__(64 * NW, FBD_FWD_OCC) void fwd_kernel(const T* __restrict__ Q,
                                                     const T* __restrict__ K,
                                                     const T* __restrict__ V, T* __restrict__ O,
                                                     float* __restrict__ LSE, int N, int BH,
                                                     int H, int grp, int win,
                                                     const int* __restrict__ DS,
                                                     const uint8_t* __restrict__ BMK, int nblk,
                                                     float scale) {
  constexpr int FWD_WAVES = NW;
  constexpr int FWD_BLK = FWD_WAVES * FWD_G * WROWS;   // query rows per workgroup
  static_assert(!BMASK || FWD_BLK == 128,
                "a workgroup owns one 128-row block of the block-sparse mask");
  // two buffers as separate objects, used in a loop unrolled by two, so the
  // compiler can tell the copy of the next tile never aliases the reads of
  // the current one (and places no wait between them)
  __shared__ __attribute__((aligned(16))) T K0[BN * HD];
  __shared__ __attribute__((aligned(16))) T V0[BN * HD];
  __shared__ __attribute__((aligned(16))) T K1[BN * HD];
  __shared__ __attribute__((aligned(16))) T V1[BN * HD];

  const Work wk = row_work(BH, nblk);
  const size_t hoff = (size_t)wk.head * N * HD;
  const size_t kvoff = (size_t)kv_head(wk.head, H, grp) * N * HD;
  const uint32_t hbytes = (uint32_t)N * HD * sizeof(T);
  const auto rk = make_rsrc(K + kvoff, hbytes);
  const auto rv = make_rsrc(V + kvoff, hbytes);
  // the wave index as a scalar, so the DMA's LDS addresses stay in SGPRs
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q0 = wk.blk * FWD_BLK;
  const int qw = q0 + wave * FWD_G * WROWS;
  const int h = lane >> 5;
  const float sl2 = scale * LOG2E;

  // Per query group: running max m (raw score units), running sum l and the
  // output accumulator o.  fp32: the score products of a tile start from -m
  // in the MFMA accumulator (negm) and arrive as x = S - m.  bf16: they start
  // from zero and arrive as x = S.  The max, and with it the rescale of o and
  // l, is updated once per key tile.  `seen` marks rows that have met a
  // visible key (until then m is a placeholder 0 and nothing is
  // accumulated): with a sliding window a row's first visible key can lie
  // beyond the block's first tile.
  constexpr bool ACC_M = sizeof(T) == 4;   // scores arrive as S - m
  Frag<T> qf[FWD_G][4];
  float m[FWD_G], l[FWD_G];
  bool seen[FWD_G];
  f32x16 o[FWD_G][2], negm[FWD_G];
#pragma unroll
  for (int g = 0; g < FWD_G; ++g) {
    ld_frags(Q + hoff, N, qw + g * WROWS, lane, qf[g]);
    m[g] = 0.f;
    l[g] = 0.f;
    seen[g] = false;
    o[g][0] = zero16();
    o[g][1] = zero16();
    negm[g] = zero16();
  }

  // keys of the block's rows: causal j <= i, from each row's start (sliding
  // window, document); the block's first row has the smallest start
  // (documents only: the window alone is a fixed offset from each row)
  const int* ds = DOCS ? DS + (size_t)(wk.head / H) * N : nullptr;
  int rs[FWD_G], rs_w[FWD_G];   // this lane's row start; the wave's largest
#pragma unroll
  for (int g = 0; g < FWD_G; ++g) {
    rs[g] = DOCS ? row_start(ds, qw + g * WROWS + (lane & 31), win, N) : 0;
    rs_w[g] = DOCS ? __builtin_amdgcn_readlane(rs[g], 31) : 0;
  }
  const int rs0 = DOCS ? row_start(ds, q0, win, N) : q0 - win + 1;
  const int jbeg = CAUSAL ? min(max(0, rs0), q0) / BN * BN : 0;
  const int jend = CAUSAL ? min(N, q0 + FWD_BLK) : N;
  const int ntiles = (jend - jbeg + BN - 1) / BN;
  constexpr int NS = BN / 32;   // 32-key sub-blocks per tile
  // block-sparse mask (a compile-time variant, so the unmasked kernel keeps
  // its registers): the workgroup's row of 128 x 128 blocks; tiles in a
  // dropped block are never loaded
  const int nbm = (N + 127) >> 7;
  const uint8_t* bmr = BMASK ? BMK + ((size_t)(wk.head / H) * nbm + (q0 >> 7)) * nbm : nullptr;
  auto kept = [&](int t) { return !BMASK || bmr[(jbeg + t * BN) >> 7] != 0; };

  // the loop visits every tile index, keeping its counted form; a tile of a
  // dropped block is neither loaded nor computed
  auto tile = [&](int t, const T* Ks, const T* Vs, T* Kn, T* Vn) {
    const int j0 = jbeg + t * BN;
    wait_dma();
    __syncthreads();   // tile t is in (Ks, Vs); every wave is done with (Kn, Vn)
    if (t + 1 < ntiles && kept(t + 1)) {
      dma_tile<T, BN, FWD_WAVES>(rk, j0 + BN, Kn, wave, lane);
      dma_tile<T, BN, FWD_WAVES>(rv, j0 + BN, Vn, wave, lane);
    }
    if (!kept(t)) return;
    // Every wave computes every 32-key sub-block of the tile; keys after a
    // row (causal) or past N are masked to -inf.  Identical control flow in
    // all waves keeps the accumulators in fixed registers.
    f32x16 x[NS][FWD_G];
#pragma unroll
    for (int sb = 0; sb < NS; ++sb) {
      Frag<T> kr[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) kr[kb] = ld_row(Ks, sb * 32, kb, lane);
#pragma unroll
      for (int g = 0; g < FWD_G; ++g) {
        x[sb][g] = ACC_M ? negm[g] : zero16();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mma(x[sb][g], kr[kb], qf[g][kb]);
      }
    }
    // Online-softmax update per query group.  On the first tile there is no
    // history: m becomes the exact tile max.  fp32: later, base = max(x) > 0
    // where a row's max grew; subtracting base before scaling gives the new
    // row max weight exactly 1.  bf16: m becomes max(m, max(x)) and the
    // exponent subtracts m * scale (nb).
    float base[FWD_G], nb[FWD_G];
    bool sub[FWD_G];
#pragma unroll
    for (int g = 0; g < FWD_G; ++g) {
      const int qg = qw + g * WROWS;
      const int my_i = qg + (lane & 31);
#pragma unroll
      for (int sb = 0; sb < NS; ++sb) {
        const int js = j0 + sb * 32;
        if (CAUSAL ? (js + 31 > qg || (DOCS ? js < rs_w[g] : js <= qg + 31 - win))
                   : (js + 32 > N)) {
          // causal without documents: key j is visible iff my_i - win < j <=
          // my_i, i.e. (unsigned)(my_i - j) < win, one compare per element
          const int d0 = my_i - js - 4 * h;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int j = js + 8 * (v >> 2) + 4 * h + (v & 3);
            bool hide;
            if constexpr (!CAUSAL) hide = j >= N;
            else if constexpr (DOCS) hide = j > my_i || j < rs[g];
            else hide = (unsigned)(d0 - 8 * (v >> 2) - (v & 3)) >= (unsigned)win;
            x[sb][g][v] = hide ? -INFINITY : x[sb][g][v];
          }
        }
      }
      float xm = x[0][g][0];
#pragma unroll
      for (int sb = 0; sb < NS; ++sb)
#pragma unroll
        for (int v = 0; v < 16; ++v) xm = vmax(xm, x[sb][g][v]);
      xm = half_max(xm);
      // a row meeting its first visible key takes that tile's max as m; a row
      // already seen moves m by the growth of its max and rescales; a row
      // with no visible key yet keeps everything zero
      const bool fresh = !seen[g] && xm > -INFINITY;
      if constexpr (ACC_M) {
        base[g] = seen[g] ? vmax(xm, 0.f) : (fresh ? xm : 0.f);
        if (__any(seen[g] && xm > 0.f)) {
          const float alpha = seen[g] ? __builtin_amdgcn_exp2f(-base[g] * sl2) : 1.f;
          l[g] *= alpha;
          o[g][0] *= alpha;
          o[g][1] *= alpha;
        }
        m[g] += base[g];
        sub[g] = __any(base[g] != 0.f);
      } else {
        const float mn = seen[g] ? vmax(m[g], xm) : (fresh ? xm : 0.f);
        if (__any(seen[g] && xm > m[g])) {
          const float alpha = seen[g] ? __builtin_amdgcn_exp2f((m[g] - mn) * sl2) : 1.f;
          l[g] *= alpha;
          o[g][0] *= alpha;
          o[g][1] *= alpha;
        }
        m[g] = mn;
        nb[g] = -mn * sl2;
        // the one-FMA exponent errs at the max by up to half an ulp of
        // m * c * log2(e); below 2^15 that rounds away in bf16, beyond it a
        // wave subtracts first (rare: scores of that size are extreme)
        sub[g] = __any(!(__builtin_fabsf(nb[g]) < 32768.f));
      }
      seen[g] = seen[g] || fresh;
    }
#pragma unroll
    for (int sb = 0; sb < NS; ++sb) {
      Frag<T> pf[FWD_G][2];
#pragma unroll
      for (int g = 0; g < FWD_G; ++g) {
        float p[16];
        if (!ACC_M && !sub[g]) {
          // one FMA per weight: the weight at the max is 2^e with |e| at
          // most half an ulp of m * sl2 (< 2^15), which the bf16 rounding
          // below takes to exactly 1, so l and P V still see the exact 1
#pragma unroll
          for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(fmaf(x[sb][g][v], sl2, nb[g]));
        } else if (!ACC_M) {
          // subtract, then scale: exactly 2^0 at the max
#pragma unroll
          for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f((x[sb][g][v] - m[g]) * sl2);
        } else if (sub[g]) {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            p[v] = __builtin_amdgcn_exp2f((x[sb][g][v] - base[g]) * sl2);
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(x[sb][g][v] * sl2);
        }
        pf[g][0] = pack8<T>(p);
        pf[g][1] = pack8<T>(p + 8);
        l[g] = frag_acc_sum(pf[g][0], l[g]);
        l[g] = frag_acc_sum(pf[g][1], l[g]);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const Frag<T> v0 = ld_tr(Vs, 0, 2 * sb + tt, lane);
        const Frag<T> v1 = ld_tr(Vs, 32, 2 * sb + tt, lane);
#pragma unroll
        for (int g = 0; g < FWD_G; ++g) {
          mma(o[g][0], v0, pf[g][tt]);
          mma(o[g][1], v1, pf[g][tt]);
        }
      }
    }
    if constexpr (ACC_M) {
#pragma unroll
      for (int g = 0; g < FWD_G; ++g) negm[g] = zero16() - m[g];
    }
  };
  if (!BMASK || (ntiles > 0 && kept(0))) {
    dma_tile<T, BN, FWD_WAVES>(rk, jbeg, K0, wave, lane);
    dma_tile<T, BN, FWD_WAVES>(rv, jbeg, V0, wave, lane);
  }
  for (int t = 0; t < ntiles; t += 2) {
    tile(t, K0, V0, K1, V1);
    if (t + 1 < ntiles) tile(t + 1, K1, V1, K0, V0);
  }
  // a row left with no visible key (possible only under a block mask) gets
  // O = 0 and LSE = -inf
#pragma unroll
  for (int g = 0; g < FWD_G; ++g) {
    const int qg = qw + g * WROWS;
    const int my_i = qg + (lane & 31);
    const float lt = half_sum(l[g]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float out[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) out[v] = o[g][0][v] * inv;
    st_cols(O + hoff, N, qg, 0, lane, out);
#pragma unroll
    for (int v = 0; v < 16; ++v) out[v] = o[g][1][v] * inv;
    st_cols(O + hoff, N, qg, 32, lane, out);
    if (h == 0 && my_i < N)
      LSE[(size_t)wk.head * N + my_i] =
          lt > 0.f ? scale * m[g] + __builtin_amdgcn_logf(lt) * LN2 : -INFINITY;
  }
}

template <class T, bool CAUSAL>
static hipError_t launch_fwd_t(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               int BH, int H, int grp, int win, const int* ds,
                               const uint8_t* bm, int N, float scale, hipStream_t st) {
  constexpr int BN = sizeof(T) == 2 ? FBD_FWD_BN : 64;
  auto run = [&](auto nw, auto docs, auto bmask) {
    constexpr int NW = decltype(nw)::value;
    constexpr int ROWS = NW * FWD_G * WROWS;
    const int nblk = (N + ROWS - 1) / ROWS;
    hipLaunchKernelGGL(
        (fwd_kernel<T, BN, NW, CAUSAL, decltype(docs)::value, decltype(bmask)::value>),
        dim3(nblk * BH), dim3(64 * NW), 0, st, (const T*)Q, (const T*)K, (const T*)V, (T*)O, LSE,
        N, BH, H, grp, win, ds, bm, nblk, scale);
  };
  using Y = std::true_type;
  using F = std::false_type;
  using W4 = std::integral_constant<int, 4>;
  using W8 = std::integral_constant<int, 8>;
  // without a block mask, bf16 operands and long sequences: 8-wave workgroups
  auto run_unmasked = [&](auto docs) {
    if constexpr (sizeof(T) == 2) {
      if (N >= FBD_WIDE_N) {
        run(W8{}, docs, F{});
        return;
      }
    }
    run(W4{}, docs, F{});
  };
  if constexpr (CAUSAL) {
    if (ds) {
      if (bm) run(W4{}, Y{}, Y{});
      else run_unmasked(Y{});
      return hipGetLastError();
    }
  }
  if (bm) run(W4{}, F{}, Y{});
  else run_unmasked(F{});
  return hipGetLastError();
}

hipError_t launch_fwd(int dt, const void* Q, const void* K, const void* V, void* O, float* LSE,
                      int BH, int H, int grp, int win, const int* ds, const uint8_t* bm, int N,
                      int causal, float scale, hipStream_t st) {
  if (dt == 0) {
    if (causal)
      return launch_fwd_t<bf16, true>(Q, K, V, O, LSE, BH, H, grp, win, ds, bm, N, scale, st);
    return launch_fwd_t<bf16, false>(Q, K, V, O, LSE, BH, H, grp, win, ds, bm, N, scale, st);
  }
  if (causal)
    return launch_fwd_t<float, true>(Q, K, V, O, LSE, BH, H, grp, win, ds, bm, N, scale, st);
  return launch_fwd_t<float, false>(Q, K, V, O, LSE, BH, H, grp, win, ds, bm, N, scale, st);
}

}  // namespace fbd
