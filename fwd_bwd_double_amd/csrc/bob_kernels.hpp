#pragma once
// Backward-over-backward: the vector-Jacobian product of the first backward
// map (Q, K, V, dO) -> (dQ, dK, dV) with cotangents (A, Bk, C) =
// (g_dQ, g_dK, g_dV), computed in two passes as on the FlashBoB page
// (rit.work, flashbob-second-order-attention, section "Two scalar states
// replace quadratic tensors").
//
// With P, dP = dO V^T, D = rowsum(dO o O) and dS = P o (dP - D) as in the
// first backward, and
//   W = scale (A K^T + Q Bk^T),  U = dO C^T,
//   alpha_i = sum_j P_ij W_ij,
//   G = W o (dP - D) - alpha o dP + U,   beta_i = sum_j P_ij G_ij,
//   Sh = P o (G - beta),  H = P o (W - alpha),
// the result is
//   gQ = scale (Sh K + dS Bk),   gK = scale (Sh^T Q + dS^T A),
//   gV = H^T dO,                 gdO = H V + P C.
// (The pages state the operation, not these formulas; they follow from the
// definition by differentiating <A, dQ> + <Bk, dK> + <C, dV>.)
//
// Row pass (lane = query i).  alpha_i and beta_i need the whole row, but
// everything else is linear in them, so the pass accumulates four fp32
// d-vectors per row
//   XE = sum_j R(P (W (dP - D) + U)) K_j + R(dS) Bk_j,   Y = sum_j R(P) K_j,
//   Z  = sum_j R(dS) K_j,   FG = sum_j R(P W) V_j + R(P) C_j,
// plus the row sums alpha_i and x_i = sum_j P (W (dP - D) + U) (the fp32
// values whose bf16 roundings feed XE), and after the last key block applies
// the corrections once:
//   beta_i = b_i - 2 alpha_i D_i = x_i - alpha_i D_i   (b_i = sum_j P (W dP + U)),
//   kappa_i = alpha_i D_i + beta_i,
//   gQ = scale (XE - alpha Z - kappa Y),   gdO = FG - alpha O
// (sum_j P_ij V_j = O_i).  The alpha term of gQ is alpha sum_j P dP K_j; since
// P dP = dS + D P it is taken as alpha (Z + D Y), with the D Y part joining
// beta's Y term as kappa.  The Z operand is then the dS values the Bk product
// packs anyway, and dS, unlike P dP, sums to zero over a row.  The pass
// writes gQ, gdO and the row states D, alpha, beta, -kappa.
//
// Fused with the first backward's row pass (EMIT: when the cotangents are
// known before the backward runs, as in a Hessian-vector product), Z and Y
// are exactly the backward row pass's two accumulators, so the same
// registers also give
//   dQ = scale (Z - r Y)  with GProj (r_i = sum_j R(dS_ij)),  scale Z without,
// for one row sum of the packed bf16 dS values per tile.
//
// GProj for g_Q (PROJ; the GProj page's projection, section "How a zero sum
// turns into a false gradient", carried over to this pass).  The K-side
// weights of g_Q, Sh = P (W (dP - D) + U) - alpha dS - kappa P, sum to
// exactly zero over a row (sum_j dS = 0, sum_j P = 1, sum_j P (W (dP - D) + U)
// = beta + alpha D = kappa), but the pass feeds their three parts to the
// matrix cores as separate bf16 operands and combines them after the sums;
// the residual row sum of those operands,
//   r_Sh = sum R(x) - alpha r - kappa sum R(P),
// carries a false multiple of the keys' mean into g_Q, large when the keys
// share a large mean and rows are near one-hot.  With PROJ it is removed
// along R(P) K:
//   g_Q = scale (XE - alpha Z - (kappa + r_Sh) Y).
// g_dO's weights of V, P (W - alpha), sum to zero over a row as well; the pass
// forms g_dO = sum R(P W) V + R(P) C - alpha O, so their residual is
// r_H = sum R(P W) - alpha, removed along O:  g_dO = FG - (alpha + r_H) O.
// Four v_dot2 row sums over operands the pass packs anyway.
//
// Column pass (lane = key j).  K, V, Bk, C of the workgroup's keys stay in
// registers; query blocks stream past them with their row states, and
// gK, gV are accumulated and written once.
//
// Streamed tiles reach LDS by buffer -> LDS DMA into two alternating buffers
// (the copy of tile t+1 runs while tile t is computed) and are stored once,
// row-major; products over the sequence index read them with the transposing
// LDS read.
#include "launch.hpp"
#include "tile.hpp"

#include <type_traits>

namespace fbd {

// Resident workgroups per CU of the row pass.  The bf16 causal forms run two
// (two waves per SIMD): their Q, dO and g_dQ fragments then sit in LDS (48 KB
// per workgroup, 80 KB with the tile buffers) and are read for each product,
// a latency the other wave hides.  The other forms keep those fragments in
// registers at one wave per SIMD: without the causal mask the two-wave kernel
// spills hundreds of registers, and with the fragments in LDS but one wave
// per SIMD the pass is slower.
template <class T, bool CAUSAL, bool BMASK>
constexpr int bob_row_occ() {
  return (sizeof(T) == 2 && CAUSAL) ? 2 : FBD_BOB_ROW_OCC;
}

// EMIT: also write the first backward's dQ and its GProj row sums r (Rws);
// PROJ: project the residual row sum of g_Q's K-side weights (above)
template <class T, int BN, bool CAUSAL, bool DOCS, bool BMASK, bool EMIT, bool PROJ>
__global__ __launch_bounds__(NT, (bob_row_occ<T, CAUSAL, BMASK>())) void bob_row_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ O, const float* __restrict__ LSE, const T* __restrict__ dO,
    const T* __restrict__ A, const T* __restrict__ Bk, const T* __restrict__ C,
    T* __restrict__ gQ, T* __restrict__ gdO, float* __restrict__ Dws, float* __restrict__ Aws,
    float* __restrict__ Bws, float* __restrict__ Lws, float* __restrict__ Kws, int N, int BH,
    int H, int grp, int win, const int* __restrict__ DS, const uint8_t* __restrict__ BMK,
    int nblk, float scale, T* __restrict__ dQ, float* __restrict__ Rws, int gproj) {
  // two buffers as separate objects (loop unrolled by two): the copy of the
  // next tile provably never aliases the reads of the current one
  struct Buf {
    T k[BN * HD], v[BN * HD], b[BN * HD], c[BN * HD];
  };
  __shared__ __attribute__((aligned(16))) Buf B0;
  __shared__ __attribute__((aligned(16))) Buf B1;
  // the Q, dO, g_dQ fragments of the two-wave form: [operand][wave][kb][lane]
  constexpr bool OPS_LDS = bob_row_occ<T, CAUSAL, BMASK>() == 2;
  __shared__ __attribute__((aligned(16))) Frag<T> Ops[OPS_LDS ? 3 : 1][NT / 64][4][64];

  const Work wk = row_work(BH, nblk);
  const size_t hoff = (size_t)wk.head * N * HD;
  const size_t kvoff = (size_t)kv_head(wk.head, H, grp) * N * HD;
  const size_t soff = (size_t)wk.head * N;
  const uint32_t hbytes = (uint32_t)N * HD * sizeof(T);
  const auto rk = make_rsrc(K + kvoff, hbytes);
  const auto rv = make_rsrc(V + kvoff, hbytes);
  const auto rb = make_rsrc(Bk + kvoff, hbytes);
  const auto rc = make_rsrc(C + kvoff, hbytes);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q0 = wk.blk * BLK;
  const int qw = q0 + wave * WROWS;
  const int my_i = qw + (lane & 31);
  const int h = lane >> 5;
  const float sl2 = scale * LOG2E;

  Frag<T> qf[4], dof[4], af[4];
  ld_frags(Q + hoff, N, qw, lane, qf);
  ld_frags(dO + hoff, N, qw, lane, dof);
  ld_frags(A + hoff, N, qw, lane, af);
  if constexpr (OPS_LDS) {
    // each lane reads back only what it wrote: no barrier needed
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      Ops[0][wave][kb][lane] = qf[kb];
      Ops[1][wave][kb][lane] = dof[kb];
      Ops[2][wave][kb][lane] = af[kb];
    }
  }
  auto opq = [&](int kb) -> const Frag<T>& {
    if constexpr (OPS_LDS) return Ops[0][wave][kb][lane];
    else return qf[kb];
  };
  auto opdo = [&](int kb) -> const Frag<T>& {
    if constexpr (OPS_LDS) return Ops[1][wave][kb][lane];
    else return dof[kb];
  };
  auto opa = [&](int kb) -> const Frag<T>& {
    if constexpr (OPS_LDS) return Ops[2][wave][kb][lane];
    else return af[kb];
  };
  float Di;
  {
    Frag<T> of[4];
    ld_frags(O + hoff, N, qw, lane, of);
    Di = row_dot(dof, of);
  }
  const float lse2 = my_i < N ? LSE[soff + my_i] * LOG2E : 0.f;

  f32x16 X0 = zero16(), X1 = zero16(), Y0 = zero16(), Y1 = zero16();
  f32x16 Z0 = zero16(), Z1 = zero16(), F0 = zero16(), F1 = zero16();
  float alpha = 0.f, xsum = 0.f, r = 0.f;
  float sx = 0.f, sp = 0.f, sf = 0.f;   // row sums of the bf16 operands (PROJ)

  // keys of the block's rows: causal j <= i, from each row's start (sliding
  // window, document); the block's first row has the smallest start
  // (documents only: the window alone is a fixed offset from each row)
  const int* ds = DOCS ? DS + (size_t)(wk.head / H) * N : nullptr;
  const int rs = DOCS ? row_start(ds, my_i, win, N) : 0;              // this lane's row
  const int rs_w = DOCS ? __builtin_amdgcn_readlane(rs, 31) : 0;      // the wave's largest
  const int rs0 = DOCS ? row_start(ds, q0, win, N) : q0 - win + 1;
  const int jbeg = CAUSAL ? min(max(0, rs0), q0) / BN * BN : 0;
  const int jend = CAUSAL ? min(N, q0 + BLK) : N;
  const int ntiles = (jend - jbeg + BN - 1) / BN;
  // block-sparse mask: the workgroup's row of 128 x 128 blocks
  const int nbm = (N + 127) >> 7;
  // (a compile-time variant, so the unmasked kernel keeps its registers)
  const uint8_t* bmr = BMASK ? BMK + ((size_t)(wk.head / H) * nbm + (q0 >> 7)) * nbm : nullptr;
  auto kept = [&](int t) { return !BMASK || bmr[(jbeg + t * BN) >> 7] != 0; };
  auto stage = [&](int j0, Buf& bf) {
    dma_tile<T, BN, NT / 64>(rk, j0, bf.k, wave, lane);
    dma_tile<T, BN, NT / 64>(rv, j0, bf.v, wave, lane);
    dma_tile<T, BN, NT / 64>(rb, j0, bf.b, wave, lane);
    dma_tile<T, BN, NT / 64>(rc, j0, bf.c, wave, lane);
  };
  // the loop visits every tile index so that it keeps its counted form; a
  // tile of a dropped block is neither loaded nor computed
  auto tile = [&](int t, const Buf& cb, Buf& nb) {
    const int j0 = jbeg + t * BN;
    wait_dma();
    __syncthreads();   // tile t is in cb; every wave is done with nb
    if (t + 1 < ntiles && kept(t + 1)) stage(j0 + BN, nb);
    if (!kept(t)) return;
    const T* Ks = cb.k;
    const T* Vs = cb.v;
    const T* Bs = cb.b;
    const T* Cs = cb.c;
#pragma unroll
    for (int jb = 0; jb < BN; jb += 32) {
      const int js = j0 + jb;   // all waves compute all sub-blocks; dead keys masked
      // one straight-line body per case, so the scheduler can interleave the
      // whole sub-block's matrix and vector work
      auto sub = [&](auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        // the compiler's single-wave interleave of matrix products and LDS
        // reads: at one wave per SIMD (no other wave hides latency) 3% faster
        // than its default schedule; in the two-wave form, whose score
        // products read their query-side operand from LDS, the default
        // schedule is more than twice as slow
        __builtin_amdgcn_iglp_opt(1);
      f32x16 s = zero16(), dp = zero16(), w = zero16(), u = zero16();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const Frag<T> kr = ld_row(Ks, jb, kb, lane);
        mma(s, kr, opq(kb));
        mma(w, kr, opa(kb));
        mma(w, ld_row(Bs, jb, kb, lane), opq(kb));
        const Frag<T> vr = ld_row(Vs, jb, kb, lane);
        mma(dp, vr, opdo(kb));
        mma(u, ld_row(Cs, jb, kb, lane), opdo(kb));
      }
      float xs[16], ps[16], es[16], fs[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) ps[v] = __builtin_amdgcn_exp2f(s[v] * sl2 - lse2);
      if constexpr (MASK) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = js + 8 * (v >> 2) + 4 * h + (v & 3);
          ps[v] = (CAUSAL ? (j > my_i || (DOCS ? j < rs : j <= my_i - win)) : (j >= N)) ? 0.f : ps[v];
        }
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pv = ps[v];
        const float W = scale * w[v];
        const float dpd = dp[v] - Di;
        const float pw = pv * W;
        alpha += pw;
        xs[v] = pv * (W * dpd + u[v]);
        xsum += xs[v];
        es[v] = pv * dpd;
        fs[v] = pw;
      }
      const int jt = jb / 16;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const Frag<T> xf = pack8<T>(xs + 8 * tt), pf = pack8<T>(ps + 8 * tt);
        const Frag<T> ef = pack8<T>(es + 8 * tt);
        const Frag<T> ff = pack8<T>(fs + 8 * tt);
        if constexpr (EMIT || PROJ) r = frag_acc_sum(ef, r);   // v_dot2 on the bf16 pairs
        if constexpr (PROJ) {
          sx = frag_acc_sum(xf, sx);
          sp = frag_acc_sum(pf, sp);
          sf = frag_acc_sum(ff, sf);
        }
        {
          const Frag<T> a0 = ld_tr(Ks, 0, jt + tt, lane), a1 = ld_tr(Ks, 32, jt + tt, lane);
          mma(X0, a0, xf);
          mma(X1, a1, xf);
          mma(Y0, a0, pf);
          mma(Y1, a1, pf);
          mma(Z0, a0, ef);
          mma(Z1, a1, ef);
        }
        {
          const Frag<T> a0 = ld_tr(Bs, 0, jt + tt, lane), a1 = ld_tr(Bs, 32, jt + tt, lane);
          mma(X0, a0, ef);
          mma(X1, a1, ef);
        }
        {
          const Frag<T> a0 = ld_tr(Vs, 0, jt + tt, lane), a1 = ld_tr(Vs, 32, jt + tt, lane);
          mma(F0, a0, ff);
          mma(F1, a1, ff);
        }
        {
          const Frag<T> a0 = ld_tr(Cs, 0, jt + tt, lane), a1 = ld_tr(Cs, 32, jt + tt, lane);
          mma(F0, a0, pf);
          mma(F1, a1, pf);
        }
      }
      };
      if (CAUSAL ? (js + 31 > qw || (DOCS ? js < rs_w : js <= qw + 31 - win)) : (js + 32 > N))
        sub(std::true_type());
      else
        sub(std::false_type());
    }
  };
  if (!BMASK || (ntiles > 0 && kept(0))) stage(jbeg, B0);
  for (int t = 0; t < ntiles; t += 2) {
    tile(t, B0, B1);
    if (t + 1 < ntiles) tile(t + 1, B1, B0);
  }
  alpha = half_sum(alpha);
  // b = sum_j P (W dP + U) = sum_j x + alpha D, so beta = b - 2 alpha D = sum_j x - alpha D
  xsum = half_sum(xsum);
  // beta and kappa = alpha D + beta as explicit fused multiply-adds, so that
  // every variant of the pass rounds them alike (the column pass reads -kappa)
  const float beta = __builtin_fmaf(-alpha, Di, xsum);
  const float kappa = __builtin_fmaf(alpha, Di, beta);
  if constexpr (EMIT || PROJ) r = half_sum(r);
  float ycoef = kappa;   // Z over R(dS)
  float ocoef = alpha;                 // coefficient of O in g_dO
  if constexpr (PROJ) {
    ycoef += half_sum(sx) - alpha * r - ycoef * half_sum(sp);
    ocoef = half_sum(sf);               // alpha + r_H
  }
  float out[16], ov[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) out[v] = scale * (X0[v] - alpha * Z0[v] - ycoef * Y0[v]);
  st_cols(gQ + hoff, N, qw, 0, lane, out);
#pragma unroll
  for (int v = 0; v < 16; ++v) out[v] = scale * (X1[v] - alpha * Z1[v] - ycoef * Y1[v]);
  st_cols(gQ + hoff, N, qw, 32, lane, out);
  if constexpr (EMIT) {
    if (gproj) {
#pragma unroll
      for (int v = 0; v < 16; ++v) out[v] = scale * (Z0[v] - r * Y0[v]);
      st_cols(dQ + hoff, N, qw, 0, lane, out);
#pragma unroll
      for (int v = 0; v < 16; ++v) out[v] = scale * (Z1[v] - r * Y1[v]);
      st_cols(dQ + hoff, N, qw, 32, lane, out);
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) out[v] = scale * Z0[v];
      st_cols(dQ + hoff, N, qw, 0, lane, out);
#pragma unroll
      for (int v = 0; v < 16; ++v) out[v] = scale * Z1[v];
      st_cols(dQ + hoff, N, qw, 32, lane, out);
    }
  }
  ld_cols(O + hoff, N, qw, 0, lane, ov);
#pragma unroll
  for (int v = 0; v < 16; ++v) out[v] = F0[v] - ocoef * ov[v];
  st_cols(gdO + hoff, N, qw, 0, lane, out);
  ld_cols(O + hoff, N, qw, 32, lane, ov);
#pragma unroll
  for (int v = 0; v < 16; ++v) out[v] = F1[v] - ocoef * ov[v];
  st_cols(gdO + hoff, N, qw, 32, lane, out);
  if (h == 0 && my_i < N) {
    Dws[soff + my_i] = Di;
    Aws[soff + my_i] = alpha;
    Bws[soff + my_i] = beta;
    Lws[soff + my_i] = -lse2;
    Kws[soff + my_i] = -kappa;   // the column pass's U starts there
    if constexpr (EMIT) Rws[soff + my_i] = r;
  }
}

template <class T, int BM, bool CAUSAL, bool DOCS, bool BMASK>
__global__ __launch_bounds__(NT, FBD_BOB_COL_OCC) void bob_col_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ Lws, const T* __restrict__ dO, const T* __restrict__ A,
    const T* __restrict__ Bk, const T* __restrict__ C, const float* __restrict__ Dws,
    const float* __restrict__ Aws, const float* __restrict__ Kws, T* __restrict__ gK,
    T* __restrict__ gV, int N, int BH, int H, int grp, int win, const int* __restrict__ DS,
    const uint8_t* __restrict__ BMK, float scale, int nsl, float* __restrict__ Part) {
  static_assert(BM % 64 == 0, "row statistics move in 64-row DMA instructions");
  // two buffers as separate objects (loop unrolled by two); each holds the
  // Q, dO, g_dQ tiles and the -LSE*log2(e), D, alpha, -kappa of the tile's rows
  struct Buf {
    T q[BM * HD], dO[BM * HD], a[BM * HD];
    float nl[BM], D[BM], al[BM], ka[BM];
    int ds[DOCS ? BM : 4];   // first visible key of each row (document masks)
  };
  __shared__ __attribute__((aligned(16))) Buf B0;
  __shared__ __attribute__((aligned(16))) Buf B1;

  // workgroup = (key block, key/value head, slice of its query heads); the
  // slice's query heads stream past in turn, accumulating into the same gK,
  // gV (one slice: the whole group, written as the result; several: fp32
  // partial sums, added up afterwards)
  const Work wk = col_work(BH / grp * nsl);
  const int kvh = wk.head / nsl, sl = wk.head - kvh * nsl;
  const int hps = grp / nsl;                      // query heads per slice
  const size_t hoff = (size_t)kvh * N * HD;       // key-side tensors
  const int qh0 = first_q_head(kvh, H, grp) + sl * hps;
  const uint32_t hbytes = (uint32_t)N * HD * sizeof(T);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k0 = wk.blk * BLK;
  const int kw = k0 + wave * WROWS;
  const int my_j = kw + (lane & 31);
  const int h = lane >> 5;
  const float sl2 = scale * LOG2E;

  Frag<T> kf[4], vf[4], bf[4], cf[4];
  ld_frags(K + hoff, N, kw, lane, kf);
  ld_frags(V + hoff, N, kw, lane, vf);
  ld_frags(Bk + hoff, N, kw, lane, bf);
  ld_frags(C + hoff, N, kw, lane, cf);
  f32x16 gk0 = zero16(), gk1 = zero16(), gv0 = zero16(), gv1 = zero16();

  const int istart = CAUSAL ? k0 : 0;
  // queries of the block's keys: causal i >= j, within the window i < j + win,
  // and with documents up to the first row whose document starts past the
  // block (rows of one batch: the group's query heads share it)
  const int* ds = DOCS ? DS + (size_t)(qh0 / H) * N : nullptr;
  const int kmax = k0 + BLK - 1;
  int iend = CAUSAL ? min(N, kmax + win) : N;
  if (CAUSAL && DOCS) iend = min(iend, first_above(ds, min(N, k0 + BLK), N, kmax, lane));
  const int ntiles = iend > istart ? (iend - istart + BM - 1) / BM : 0;
  const int nsteps = ntiles * hps;      // (query head, query tile) steps
  // block-sparse mask (a compile-time variant): the workgroup's column of
  // 128 x 128 blocks; every step index is visited, and a step whose query
  // tile lies in a dropped block is neither loaded nor computed
  const int nbm = (N + 127) >> 7;
  const uint8_t* bmc = BMASK ? BMK + (size_t)(qh0 / H) * nbm * nbm + (k0 >> 7) : nullptr;
  auto kept = [&](int u) {
    return !BMASK || bmc[(size_t)((istart + (u % ntiles) * BM) >> 7) * nbm] != 0;
  };
  // stage step u: query tile u % ntiles of query head qh0 + u / ntiles
  auto stage = [&](int u, Buf& b) {
    const int qh = qh0 + u / ntiles;
    const int i0 = istart + (u % ntiles) * BM;
    const size_t qoff = (size_t)qh * N * HD, soff = (size_t)qh * N;
    const uint32_t sbytes = (uint32_t)N * 4u;
    dma_tile<T, BM, NT / 64>(make_rsrc(Q + qoff, hbytes), i0, b.q, wave, lane);
    dma_tile<T, BM, NT / 64>(make_rsrc(dO + qoff, hbytes), i0, b.dO, wave, lane);
    dma_tile<T, BM, NT / 64>(make_rsrc(A + qoff, hbytes), i0, b.a, wave, lane);
#pragma unroll
    for (int k = 0; k < BM / 64; ++k) {
      if (wave == 0) dma_rows_f32(make_rsrc(Lws + soff, sbytes), i0, b.nl, k, lane);
      if (wave == 1) dma_rows_f32(make_rsrc(Dws + soff, sbytes), i0, b.D, k, lane);
      if (wave == 2) dma_rows_f32(make_rsrc(Aws + soff, sbytes), i0, b.al, k, lane);
      if (wave == 3) dma_rows_f32(make_rsrc(Kws + soff, sbytes), i0, b.ka, k, lane);
      if (DOCS && wave == 0)
        dma_rows_f32(make_rsrc(ds, sbytes), i0, reinterpret_cast<float*>(b.ds), k, lane);
    }
  };
  auto tile = [&](int u, const Buf& cb, Buf& nb) {
    const int i0 = istart + (u % ntiles) * BM;
    wait_dma();
    __syncthreads();   // step u is in cb; every wave is done with nb
    if (u + 1 < nsteps && kept(u + 1)) stage(u + 1, nb);
    if (!kept(u)) return;
    const T* Qs = cb.q;
    const T* dOs = cb.dO;
    const T* As = cb.a;
    const float* sL = cb.nl;
    const float* sD = cb.D;
    const float* sA = cb.al;
    const float* sK = cb.ka;
    const int* sDS = cb.ds;
#pragma unroll
    for (int ib = 0; ib < BM; ib += 32) {
      const int is = i0 + ib;
      // all waves compute all sub-blocks: rows before a key (causal) and rows
      // past N are masked below.  The four score-type products are formed
      // one after another, each consumed as soon as it is complete, to keep
      // few of them live at once.
      const int it = ib / 16;
      float ps[16];
      {
        f32x16 s = zero16();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mma(s, ld_row(Qs, ib, kb, lane), kf[kb]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sL[ib + 8 * q + 4 * h]);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            ps[4 * q + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * q + r], sl2, l4[r]));
        }
        if ((CAUSAL && (is <= kw || is + 31 >= kw + win || (DOCS && sDS[ib + 31] > kw))) ||
            is + 32 > N) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int i = is + 8 * (v >> 2) + 4 * h + (v & 3);
            const bool doc = DOCS && sDS[ib + 8 * (v >> 2) + 4 * h + (v & 3)] > my_j;
            ps[v] = ((CAUSAL && (my_j > i || i >= my_j + win || doc)) || i >= N) ? 0.f : ps[v];
          }
        }
      }
      // dS = P o (dP - D): gK += dS^T A
      f32x16 dpd = zero16();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mma(dpd, ld_row(dOs, ib, kb, lane), vf[kb]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sD[ib + 8 * q + 4 * h]);
#pragma unroll
        for (int r = 0; r < 4; ++r) dpd[4 * q + r] -= d4[r];
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ds[e] = ps[8 * tt + e] * dpd[8 * tt + e];
        const Frag<T> dsf = pack8<T>(ds);
        mma(gk0, ld_tr(As, 0, it + tt, lane), dsf);
        mma(gk1, ld_tr(As, 32, it + tt, lane), dsf);
      }
      // h = scale W - alpha with W = Q Bk^T + A K^T:  gV += (P o h)^T dO
      f32x16 hv = zero16();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        mma(hv, ld_row(Qs, ib, kb, lane), bf[kb]);
        mma(hv, ld_row(As, ib, kb, lane), kf[kb]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(&sA[ib + 8 * q + 4 * h]);
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[4 * q + r] = __builtin_fmaf(scale, hv[4 * q + r], -a4[r]);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float hs[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) hs[e] = ps[8 * tt + e] * hv[8 * tt + e];
        const Frag<T> hf = pack8<T>(hs);
        mma(gv0, ld_tr(dOs, 0, it + tt, lane), hf);
        mma(gv1, ld_tr(dOs, 32, it + tt, lane), hf);
      }
      // Sh = P o (W (dP - D) + U - alpha dP - beta) = P o (h (dP - D) + U - kappa)
      // with U = dO C^T and kappa = alpha D + beta per row:  gK += Sh^T Q.
      // The U product starts from the rows' -kappa, so no subtraction remains.
      f32x16 u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 k4 = *reinterpret_cast<const f32x4*>(&sK[ib + 8 * q + 4 * h]);
#pragma unroll
        for (int r = 0; r < 4; ++r) u[4 * q + r] = k4[r];
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mma(u, ld_row(dOs, ib, kb, lane), cf[kb]);
#pragma unroll
      for (int v = 0; v < 16; ++v) u[v] = ps[v] * __builtin_fmaf(hv[v], dpd[v], u[v]);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float sh[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) sh[e] = u[8 * tt + e];
        const Frag<T> shf = pack8<T>(sh);
        mma(gk0, ld_tr(Qs, 0, it + tt, lane), shf);
        mma(gk1, ld_tr(Qs, 32, it + tt, lane), shf);
      }
    }
  };
  if (nsteps > 0 && kept(0)) stage(0, B0);
  for (int u = 0; u < nsteps; u += 2) {
    tile(u, B0, B1);
    if (u + 1 < nsteps) tile(u + 1, B1, B0);
  }
  float out[16];
  T* const ok = gK + hoff;
  T* const ov = gV + hoff;
  float* const pk = nsl > 1 ? Part + ((size_t)sl * (BH / grp) + kvh) * N * HD : nullptr;
  float* const pv = nsl > 1 ? pk + (size_t)nsl * (BH / grp) * N * HD : nullptr;
#pragma unroll
  for (int v = 0; v < 16; ++v) out[v] = scale * gk0[v];
  if (nsl == 1) st_cols(ok, N, kw, 0, lane, out);
  else st_cols(pk, N, kw, 0, lane, out);
#pragma unroll
  for (int v = 0; v < 16; ++v) out[v] = scale * gk1[v];
  if (nsl == 1) st_cols(ok, N, kw, 32, lane, out);
  else st_cols(pk, N, kw, 32, lane, out);
#pragma unroll
  for (int v = 0; v < 16; ++v) out[v] = gv0[v];
  if (nsl == 1) st_cols(ov, N, kw, 0, lane, out);
  else st_cols(pv, N, kw, 0, lane, out);
#pragma unroll
  for (int v = 0; v < 16; ++v) out[v] = gv1[v];
  if (nsl == 1) st_cols(ov, N, kw, 32, lane, out);
  else st_cols(pv, N, kw, 32, lane, out);
}

// Row pass (EMIT: fused with the first backward's row pass, writing dQ and r;
// proj: the g_Q projection, bf16 only: fp32 operands are not rounded).
template <class T, bool CAUSAL, bool DOCS, bool EMIT>
static hipError_t launch_bob_row_t(const void* Q, const void* K, const void* V, const void* O,
                                   const float* LSE, const void* dO, const void* gdQ,
                                   const void* gdK, const void* gdV, void* gQ, void* gdO,
                                   float* Dws, float* Aws, float* Bws, float* Lws, float* Kws,
                                   int BH, int H, int grp, int win, const int* ds,
                                   const uint8_t* bm, int N, float scale, void* dQ, float* Rws,
                                   int gproj, int proj, hipStream_t st) {
  // fp32 operands take twice the LDS per row: they keep the smallest tiles
  constexpr int BN = sizeof(T) == 2 ? FBD_BOB_BN : 32;
  const int nblk = (N + BLK - 1) / BLK;
  auto row = [&](auto bmask, auto pj) {
    hipLaunchKernelGGL(
        (bob_row_kernel<T, BN, CAUSAL, DOCS, decltype(bmask)::value, EMIT, decltype(pj)::value>),
        dim3(nblk * BH), dim3(NT), 0, st, (const T*)Q, (const T*)K, (const T*)V, (const T*)O, LSE,
        (const T*)dO, (const T*)gdQ, (const T*)gdK, (const T*)gdV, (T*)gQ, (T*)gdO, Dws, Aws, Bws,
        Lws, Kws, N, BH, H, grp, win, ds, bm, nblk, scale, (T*)dQ, Rws, gproj);
  };
  using Y = std::true_type;
  using F = std::false_type;
  if (sizeof(T) == 2 && proj) {
    if constexpr (sizeof(T) == 2) {
      if (bm) row(Y{}, Y{});
      else row(F{}, Y{});
    }
  } else {
    if (bm) row(Y{}, F{});
    else row(F{}, F{});
  }
  return hipGetLastError();
}

template <class T, bool CAUSAL, bool DOCS>
static hipError_t launch_bob_t(const void* Q, const void* K, const void* V, const void* O,
                               const float* LSE, const void* dO, const void* gdQ, const void* gdK,
                               const void* gdV, void* gQ, void* gK, void* gV, void* gdO,
                               float* Dws, float* Aws, float* Bws, float* Lws, float* Kws, int BH,
                               int H, int grp, int win, const int* ds, const uint8_t* bm, int N,
                               float scale, int passes, int nsl, float* Part, int proj,
                               hipStream_t st) {
  constexpr int BM = sizeof(T) == 2 ? FBD_BOB_BM : 64;
  const int nblk = (N + BLK - 1) / BLK;
  if (passes & 1) {
    hipError_t e = launch_bob_row_t<T, CAUSAL, DOCS, false>(
        Q, K, V, O, LSE, dO, gdQ, gdK, gdV, gQ, gdO, Dws, Aws, Bws, Lws, Kws, BH, H, grp, win, ds,
        bm, N, scale, nullptr, nullptr, 0, proj, st);
    if (e != hipSuccess) return e;
  }
  if (!(passes & 2)) return hipSuccess;
  auto col = [&](auto bmask) {
    hipLaunchKernelGGL((bob_col_kernel<T, BM, CAUSAL, DOCS, decltype(bmask)::value>),
                       dim3(nblk * (BH / grp) * nsl), dim3(NT), 0, st, (const T*)Q,
                       (const T*)K, (const T*)V, (const float*)Lws, (const T*)dO,
                       (const T*)gdQ, (const T*)gdK, (const T*)gdV, (const float*)Dws,
                       (const float*)Aws, (const float*)Kws, (T*)gK, (T*)gV, N, BH, H, grp, win,
                       ds, bm, scale, nsl, Part);
  };
  if (bm) col(std::true_type{});
  else col(std::false_type{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsl == 1) return e;
  return launch_sum_slices(sizeof(T) == 2 ? 0 : 1, Part, nsl, BH / grp, N, gK, gV, st);
}

}  // namespace fbd
