// Backward pass with optional GProj.
//
// Recompute instead of store (FlashAttention explainer page, marketmaker.cc
// flash-attention-trading-models, section "Backward pass: recompute instead of
// store"): only O and the row LSE are kept from the forward; every tile of P
// is recomputed as exp(scale * S - LSE) from Q and K.
//
//   row pass    (lane = query i): D_i = sum_d dO_id O_id,
//               dS = P o (dO V^T - D),  dQ = scale * R(dS) K
//   column pass (lane = key j):  dV = R(P)^T dO,  dK = scale * R(dS)^T Q
//
// R() is the rounding of an operand to bf16 for the matrix cores (identity for
// fp32 inputs).  With GProj (GProj page, rit.work
// flashattention-bf16-gradient-gproj, section "How a zero sum turns into a
// false gradient") the row pass also accumulates r_i = sum_j R(dS_ij) over
// exactly those bf16 values and R(P) K, and finishes
//   dQ = scale * (R(dS) K - r_i R(P) K);
// the column pass reads r and adds the key correction
//   dK = scale * (R(dS)^T Q - Q^T R(r o P))
// as a separate fp32-accumulated product; the projected dS is never re-rounded.
// Tiles reach LDS by buffer -> LDS DMA into two alternating buffers, and the
// operands contracted over the sequence index are read with the transposing
// LDS read, so every tile is stored once, row-major.
// Each output block is written once by one workgroup; there are no atomics.
#include <type_traits>

#include "launch.hpp"
#include "tile.hpp"

namespace fbd {

// NW waves per workgroup: 4 (128 query rows), or 8 (256 rows) for long
// sequences without a block mask
template <class T, int BN, int NW, bool GPROJ, bool CAUSAL, bool DOCS, bool BMASK>
__global__ __launch_bounds__(64 * NW, FBD_BWD_ROW_OCC) void bwd_row_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ O, const float* __restrict__ LSE, const T* __restrict__ dO,
    T* __restrict__ dQ, float* __restrict__ Dws, float* __restrict__ Rws, float* __restrict__ Lws,
    int N, int BH, int H, int grp, int win, const int* __restrict__ DS,
    const uint8_t* __restrict__ BMK, int nblk, float scale) {
  constexpr int ROWS = NW * WROWS;   // query rows per workgroup
  static_assert(!BMASK || ROWS == 128, "a workgroup owns one 128-row block of the block-sparse mask");
  // two buffers as separate objects (loop unrolled by two): the copy of the
  // next tile provably never aliases the reads of the current one
  __shared__ __attribute__((aligned(16))) T K0[BN * HD];
  __shared__ __attribute__((aligned(16))) T V0[BN * HD];
  __shared__ __attribute__((aligned(16))) T K1[BN * HD];
  __shared__ __attribute__((aligned(16))) T V1[BN * HD];

  const Work wk = row_work(BH, nblk);
  const size_t hoff = (size_t)wk.head * N * HD;
  const size_t kvoff = (size_t)kv_head(wk.head, H, grp) * N * HD;
  const size_t soff = (size_t)wk.head * N;
  const uint32_t hbytes = (uint32_t)N * HD * sizeof(T);
  const auto rk = make_rsrc(K + kvoff, hbytes);
  const auto rv = make_rsrc(V + kvoff, hbytes);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q0 = wk.blk * ROWS;
  const int qw = q0 + wave * WROWS;
  const int my_i = qw + (lane & 31);
  const int h = lane >> 5;
  const float sl2 = scale * LOG2E;

  Frag<T> qf[4], dof[4];
  ld_frags(Q + hoff, N, qw, lane, qf);
  ld_frags(dO + hoff, N, qw, lane, dof);
  float Di;
  {
    Frag<T> of[4];
    ld_frags(O + hoff, N, qw, lane, of);
    Di = row_dot(dof, of);
  }
  const float lse2 = my_i < N ? LSE[soff + my_i] * LOG2E : 0.f;

  f32x16 dq0 = zero16(), dq1 = zero16();
  f32x16 pk0 = zero16(), pk1 = zero16();
  float r = 0.f;

  // keys of the block's rows: causal j <= i, from each row's start (sliding
  // window, document); the block's first row has the smallest start
  // (documents only: the window alone is a fixed offset from each row)
  const int* ds = DOCS ? DS + (size_t)(wk.head / H) * N : nullptr;
  const int rs = DOCS ? row_start(ds, my_i, win, N) : 0;              // this lane's row
  const int rs_w = DOCS ? __builtin_amdgcn_readlane(rs, 31) : 0;      // the wave's largest
  const int rs0 = DOCS ? row_start(ds, q0, win, N) : q0 - win + 1;
  const int jbeg = CAUSAL ? min(max(0, rs0), q0) / BN * BN : 0;
  const int jend = CAUSAL ? min(N, q0 + ROWS) : N;
  const int ntiles = (jend - jbeg + BN - 1) / BN;
  // block-sparse mask (a compile-time variant): the workgroup's row of
  // 128 x 128 blocks; the loop visits every tile index, and a tile of a
  // dropped block is neither loaded nor computed
  const int nbm = (N + 127) >> 7;
  const uint8_t* bmr = BMASK ? BMK + ((size_t)(wk.head / H) * nbm + (q0 >> 7)) * nbm : nullptr;
  auto kept = [&](int t) { return !BMASK || bmr[(jbeg + t * BN) >> 7] != 0; };
  auto tile = [&](int t, const T* Ks, const T* Vs, T* Kn, T* Vn) {
    const int j0 = jbeg + t * BN;
    wait_dma();
    __syncthreads();   // tile t is in (Ks, Vs); every wave is done with (Kn, Vn)
    if (t + 1 < ntiles && kept(t + 1)) {
      dma_tile<T, BN, NW>(rk, j0 + BN, Kn, wave, lane);
      dma_tile<T, BN, NW>(rv, j0 + BN, Vn, wave, lane);
    }
    if (!kept(t)) return;
#pragma unroll
    for (int jb = 0; jb < BN; jb += 32) {
      const int js = j0 + jb;   // all waves compute all sub-blocks; dead keys masked
      // S and dP are formed one after the other; P is packed (and its
      // GProj product issued) before dP is formed, so few values are live
      const int jt = jb / 16;
      float p[16];
      {
        f32x16 sacc = zero16();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mma(sacc, ld_row(Ks, jb, kb, lane), qf[kb]);
#pragma unroll
        for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(sacc[v] * sl2 - lse2);
        if (CAUSAL ? (js + 31 > qw || (DOCS ? js < rs_w : js <= qw + 31 - win)) : (js + 32 > N)) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int j = js + 8 * (v >> 2) + 4 * h + (v & 3);
            p[v] = (CAUSAL ? (j > my_i || (DOCS ? j < rs : j <= my_i - win)) : (j >= N)) ? 0.f : p[v];
          }
        }
      }
      if constexpr (GPROJ) {
        // PK += R(P) K
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const Frag<T> pf = pack8<T>(p + 8 * tt);
          mma(pk0, ld_tr(Ks, 0, jt + tt, lane), pf);
          mma(pk1, ld_tr(Ks, 32, jt + tt, lane), pf);
        }
      }
      // dS = P o (dP - D):  dQ += R(dS) K,  r += sum of exactly those bf16 values
      f32x16 ds = zero16();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mma(ds, ld_row(Vs, jb, kb, lane), dof[kb]);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float e[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) e[k] = p[8 * tt + k] * (ds[8 * tt + k] - Di);
        const Frag<T> df = pack8<T>(e);
        if constexpr (GPROJ) r = frag_acc_sum(df, r);   // v_dot2 on the bf16 pairs
        mma(dq0, ld_tr(Ks, 0, jt + tt, lane), df);
        mma(dq1, ld_tr(Ks, 32, jt + tt, lane), df);
      }
    }
  };
  if (!BMASK || (ntiles > 0 && kept(0))) {
    dma_tile<T, BN, NW>(rk, jbeg, K0, wave, lane);
    dma_tile<T, BN, NW>(rv, jbeg, V0, wave, lane);
  }
  for (int t = 0; t < ntiles; t += 2) {
    tile(t, K0, V0, K1, V1);
    if (t + 1 < ntiles) tile(t + 1, K1, V1, K0, V0);
  }
  float out[16];
  if constexpr (GPROJ) {
    r = half_sum(r);
#pragma unroll
    for (int v = 0; v < 16; ++v) out[v] = scale * (dq0[v] - r * pk0[v]);
    st_cols(dQ + hoff, N, qw, 0, lane, out);
#pragma unroll
    for (int v = 0; v < 16; ++v) out[v] = scale * (dq1[v] - r * pk1[v]);
    st_cols(dQ + hoff, N, qw, 32, lane, out);
  } else {
#pragma unroll
    for (int v = 0; v < 16; ++v) out[v] = scale * dq0[v];
    st_cols(dQ + hoff, N, qw, 0, lane, out);
#pragma unroll
    for (int v = 0; v < 16; ++v) out[v] = scale * dq1[v];
    st_cols(dQ + hoff, N, qw, 32, lane, out);
  }
  if (h == 0 && my_i < N) {
    Dws[soff + my_i] = Di;
    Lws[soff + my_i] = -lse2;
    if constexpr (GPROJ) Rws[soff + my_i] = r;
  }
}

template <class T, int BM, bool GPROJ, bool CAUSAL, bool DOCS, bool BMASK>
__global__ __launch_bounds__(NT, FBD_BWD_COL_OCC) void bwd_col_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ Lws, const T* __restrict__ dO, const float* __restrict__ Dws,
    const float* __restrict__ Rws, T* __restrict__ dK, T* __restrict__ dV, int N, int BH, int H,
    int grp, int win, const int* __restrict__ DS, const uint8_t* __restrict__ BMK, float scale,
    int nsl, float* __restrict__ Part) {
  static_assert(BM % 64 == 0, "row statistics move in 64-row DMA instructions");
  // two buffers as separate objects (loop unrolled by two); each holds the
  // Q and dO tiles and the -LSE*log2(e), D (, r) of the tile's rows
  struct Buf {
    T q[BM * HD];
    T dO[BM * HD];
    float nl[BM], D[BM], r[GPROJ ? BM : 4];   // -LSE*log2(e), D, r
    int ds[DOCS ? BM : 4];                               // first visible key (document masks)
  };
  __shared__ __attribute__((aligned(16))) Buf B0;
  __shared__ __attribute__((aligned(16))) Buf B1;

  // workgroup = (key block, key/value head, slice of its query heads); the
  // slice's query heads stream past in turn and their contributions
  // accumulate into the same dK, dV registers (one slice: the whole group,
  // written as the result; several: fp32 partial sums, added up afterwards)
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

  Frag<T> kf[4], vf[4];
  ld_frags(K + hoff, N, kw, lane, kf);
  ld_frags(V + hoff, N, kw, lane, vf);
  f32x16 dk0 = zero16(), dk1 = zero16(), dv0 = zero16(), dv1 = zero16();

  const int istart = CAUSAL ? k0 : 0;   // k0 is a multiple of BM
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
    dma_tile<T, BM, NT / 64>(make_rsrc(Q + qoff, hbytes), i0, b.q, wave, lane);
    dma_tile<T, BM, NT / 64>(make_rsrc(dO + qoff, hbytes), i0, b.dO, wave, lane);
#pragma unroll
    for (int k = 0; k < BM / 64; ++k) {
      if (wave == 0) dma_rows_f32(make_rsrc(Lws + soff, (uint32_t)N * 4u), i0, b.nl, k, lane);
      if (wave == 1) dma_rows_f32(make_rsrc(Dws + soff, (uint32_t)N * 4u), i0, b.D, k, lane);
      if (GPROJ && wave == 2)
        dma_rows_f32(make_rsrc(Rws + soff, (uint32_t)N * 4u), i0, b.r, k, lane);
      if (DOCS && wave == 3)
        dma_rows_f32(make_rsrc(ds, (uint32_t)N * 4u), i0, reinterpret_cast<float*>(b.ds), k, lane);
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
    const float* sL = cb.nl;
    const float* sD = cb.D;
    const float* sR = cb.r;
    const int* sDS = cb.ds;
#pragma unroll
    for (int ib = 0; ib < BM; ib += 32) {
      const int is = i0 + ib;
      // all waves compute all sub-blocks: rows before a key (causal) and rows
      // past N are masked below
      // S and dP are formed one after the other and each is consumed at
      // once (P -> dV, then dS -> dK), so few values are live together
      const int it = ib / 16;
      float p[16];
      {
        f32x16 sacc = zero16();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mma(sacc, ld_row(Qs, ib, kb, lane), kf[kb]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sL[ib + 8 * q + 4 * h]);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            p[4 * q + u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[4 * q + u], sl2, l4[u]));
        }
        if ((CAUSAL && (is <= kw || is + 31 >= kw + win || (DOCS && sDS[ib + 31] > kw))) ||
            is + 32 > N) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int i = is + 8 * (v >> 2) + 4 * h + (v & 3);
            const bool doc = DOCS && sDS[ib + 8 * (v >> 2) + 4 * h + (v & 3)] > my_j;
            p[v] = ((CAUSAL && (my_j > i || i >= my_j + win || doc)) || i >= N) ? 0.f : p[v];
          }
        }
      }
      // dV += R(P)^T dO
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const Frag<T> pf = pack8<T>(p + 8 * tt);
        mma(dv0, ld_tr(dOs, 0, it + tt, lane), pf);
        mma(dv1, ld_tr(dOs, 32, it + tt, lane), pf);
      }
      // dS = P o (dP - D):  dK += R(dS)^T Q  (+ GProj key correction
      // - R(P)^T (r o Q) as Q^T R(-r o P), a separate fp32-accumulated
      // product, so the projected dS is never re-rounded)
      f32x16 ds = zero16();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mma(ds, ld_row(dOs, ib, kb, lane), vf[kb]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sD[ib + 8 * q + 4 * h]);
#pragma unroll
        for (int u = 0; u < 4; ++u) ds[4 * q + u] = p[4 * q + u] * (ds[4 * q + u] - d4[u]);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float e[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) e[k] = ds[8 * tt + k];
        const Frag<T> df = pack8<T>(e);
        const Frag<T> qa = ld_tr(Qs, 0, it + tt, lane), qb = ld_tr(Qs, 32, it + tt, lane);
        mma(dk0, qa, df);
        mma(dk1, qb, df);
        if constexpr (GPROJ) {
          float rp[8];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const f32x4 r4 = *reinterpret_cast<const f32x4*>(&sR[ib + 16 * tt + 8 * q + 4 * h]);
#pragma unroll
            for (int u = 0; u < 4; ++u) rp[4 * q + u] = -r4[u] * p[8 * tt + 4 * q + u];
          }
          const Frag<T> rf = pack8<T>(rp);
          mma(dk0, qa, rf);
          mma(dk1, qb, rf);
        }
      }
    }
  };
  if (nsteps > 0 && kept(0)) stage(0, B0);
  for (int u = 0; u < nsteps; u += 2) {
    tile(u, B0, B1);
    if (u + 1 < nsteps) tile(u + 1, B1, B0);
  }
  float out[16];
  if (nsl == 1) {
#pragma unroll
    for (int v = 0; v < 16; ++v) out[v] = scale * dk0[v];
    st_cols(dK + hoff, N, kw, 0, lane, out);
#pragma unroll
    for (int v = 0; v < 16; ++v) out[v] = scale * dk1[v];
    st_cols(dK + hoff, N, kw, 32, lane, out);
#pragma unroll
    for (int v = 0; v < 16; ++v) out[v] = dv0[v];
    st_cols(dV + hoff, N, kw, 0, lane, out);
#pragma unroll
    for (int v = 0; v < 16; ++v) out[v] = dv1[v];
    st_cols(dV + hoff, N, kw, 32, lane, out);
  } else {
    float* pk = Part + ((size_t)sl * (BH / grp) + kvh) * N * HD;
    float* pv = pk + (size_t)nsl * (BH / grp) * N * HD;
#pragma unroll
    for (int v = 0; v < 16; ++v) out[v] = scale * dk0[v];
    st_cols(pk, N, kw, 0, lane, out);
#pragma unroll
    for (int v = 0; v < 16; ++v) out[v] = scale * dk1[v];
    st_cols(pk, N, kw, 32, lane, out);
#pragma unroll
    for (int v = 0; v < 16; ++v) out[v] = dv0[v];
    st_cols(pv, N, kw, 0, lane, out);
#pragma unroll
    for (int v = 0; v < 16; ++v) out[v] = dv1[v];
    st_cols(pv, N, kw, 32, lane, out);
  }
}

// Sum of the nsl fp32 partial key-side gradients of the split column passes:
// Part holds nsl (B*Hkv, N, 64) blocks for K, then nsl for V; n4 = B*Hkv*N*16
// groups of four values.  One thread per group, slices added in order.
template <class T>
__global__ __launch_bounds__(256) void sum_slices_kernel(const float* __restrict__ Part, int nsl,
                                                         size_t n4, T* __restrict__ gK,
                                                         T* __restrict__ gV) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4* p = reinterpret_cast<const f32x4*>(Part);
  f32x4 a = p[i], b = p[(size_t)nsl * n4 + i];
  for (int s = 1; s < nsl; ++s) {
    a += p[(size_t)s * n4 + i];
    b += p[(size_t)(nsl + s) * n4 + i];
  }
  if constexpr (sizeof(T) == 2) {
    reinterpret_cast<bf16x4*>(gK)[i] = bf16x4{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
    reinterpret_cast<bf16x4*>(gV)[i] = bf16x4{(bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
  } else {
    reinterpret_cast<f32x4*>(gK)[i] = a;
    reinterpret_cast<f32x4*>(gV)[i] = b;
  }
}

hipError_t launch_sum_slices(int dt, const float* Part, int nsl, int BHkv, int N, void* gK,
                             void* gV, hipStream_t st) {
  const size_t n4 = (size_t)BHkv * N * (HD / 4);
  const dim3 grid((unsigned)((n4 + 255) / 256));
  if (dt == 0)
    hipLaunchKernelGGL(sum_slices_kernel<bf16>, grid, dim3(256), 0, st, Part, nsl, n4, (bf16*)gK,
                       (bf16*)gV);
  else
    hipLaunchKernelGGL(sum_slices_kernel<float>, grid, dim3(256), 0, st, Part, nsl, n4,
                       (float*)gK, (float*)gV);
  return hipGetLastError();
}

template <class T, bool GPROJ, bool CAUSAL, bool DOCS>
static hipError_t launch_bwd_t(const void* Q, const void* K, const void* V, const void* O,
                               const float* LSE, const void* dO, void* dQ, void* dK, void* dV,
                               float* Dws, float* Rws, float* Lws, int BH, int H, int grp,
                               int win, const int* ds, const uint8_t* bm, int N, float scale, int passes,
                               int nsl, float* Part, hipStream_t st) {
  // fp32 operands take twice the LDS per row: they keep the smallest tiles
  constexpr int BN = sizeof(T) == 2 ? FBD_BWD_BN : 64, BM = sizeof(T) == 2 ? FBD_BWD_BM : 64;
  const int nblk = (N + BLK - 1) / BLK;
  // the block mask selects a compile-time kernel variant; without one, bf16
  // row passes over long sequences take 8-wave workgroups
  auto row = [&](auto nw, auto bmask) {
    constexpr int NW = decltype(nw)::value;
    const int nrb = (N + NW * WROWS - 1) / (NW * WROWS);
    hipLaunchKernelGGL((bwd_row_kernel<T, BN, NW, GPROJ, CAUSAL, DOCS, decltype(bmask)::value>),
                       dim3(nrb * BH), dim3(64 * NW), 0, st, (const T*)Q, (const T*)K,
                       (const T*)V, (const T*)O, LSE, (const T*)dO, (T*)dQ, Dws, Rws, Lws, N, BH,
                       H, grp, win, ds, bm, nrb, scale);
  };
  using W4 = std::integral_constant<int, 4>;
  using W8 = std::integral_constant<int, 8>;
  auto col = [&](auto bmask) {
    hipLaunchKernelGGL((bwd_col_kernel<T, BM, GPROJ, CAUSAL, DOCS, decltype(bmask)::value>),
                       dim3(nblk * (BH / grp) * nsl), dim3(NT), 0, st, (const T*)Q,
                       (const T*)K, (const T*)V, (const float*)Lws, (const T*)dO,
                       (const float*)Dws, (const float*)Rws, (T*)dK, (T*)dV, N, BH, H, grp, win,
                       ds, bm, scale, nsl, Part);
  };
  if (passes & 1) {
    bool wide = false;
    if constexpr (sizeof(T) == 2) wide = !bm && N >= FBD_WIDE_N;
    if (bm) row(W4{}, std::true_type{});
    else if (!wide) row(W4{}, std::false_type{});
    else if constexpr (sizeof(T) == 2) row(W8{}, std::false_type{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(passes & 2)) return hipSuccess;
  if (bm) col(std::true_type{});
  else col(std::false_type{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsl == 1) return e;
  return launch_sum_slices(sizeof(T) == 2 ? 0 : 1, Part, nsl, BH / grp, N, dK, dV, st);
}

template <class T, bool GPROJ>
static hipError_t launch_bwd_c(int causal, const void* Q, const void* K, const void* V,
                               const void* O, const float* LSE, const void* dO, void* dQ,
                               void* dK, void* dV, float* Dws, float* Rws, float* Lws, int BH,
                               int H, int grp, int win, const int* ds, const uint8_t* bm, int N, float scale,
                               int passes, int nsl, float* Part, hipStream_t st) {
  if (causal)
    return ds ? launch_bwd_t<T, GPROJ, true, true>(Q, K, V, O, LSE, dO, dQ, dK, dV, Dws, Rws, Lws, BH, H, grp, win, ds, bm, N, scale, passes, nsl, Part, st)
              : launch_bwd_t<T, GPROJ, true, false>(Q, K, V, O, LSE, dO, dQ, dK, dV, Dws, Rws, Lws, BH, H, grp, win, ds, bm, N, scale, passes, nsl, Part, st);
  return launch_bwd_t<T, GPROJ, false, false>(Q, K, V, O, LSE, dO, dQ, dK, dV, Dws, Rws, Lws, BH, H, grp, win, ds, bm, N, scale, passes, nsl, Part, st);
}

hipError_t launch_bwd(int dt, const void* Q, const void* K, const void* V, const void* O,
                      const float* LSE, const void* dO, void* dQ, void* dK, void* dV, float* Dws,
                      float* Rws, float* Lws, int BH, int H, int grp, int win, const int* ds,
                      const uint8_t* bm, int N,
                      int causal, float scale, int gproj, int passes, int nsl, float* Part,
                      hipStream_t st) {
  if (dt == 0) {
    if (gproj)
      return launch_bwd_c<bf16, true>(causal, Q, K, V, O, LSE, dO, dQ, dK, dV, Dws, Rws, Lws, BH, H, grp, win, ds, bm, N, scale, passes, nsl, Part, st);
    return launch_bwd_c<bf16, false>(causal, Q, K, V, O, LSE, dO, dQ, dK, dV, Dws, Rws, Lws, BH, H, grp, win, ds, bm, N, scale, passes, nsl, Part, st);
  }
  if (gproj)
    return launch_bwd_c<float, true>(causal, Q, K, V, O, LSE, dO, dQ, dK, dV, Dws, Rws, Lws, BH, H, grp, win, ds, bm, N, scale, passes, nsl, Part, st);
  return launch_bwd_c<float, false>(causal, Q, K, V, O, LSE, dO, dQ, dK, dV, Dws, Rws, Lws, BH, H, grp, win, ds, bm, N, scale, passes, nsl, Part, st);
}

}  // namespace fbd
