// FP8 (OCP E4M3) forward with optional incoherent processing.
//
// The FlashAttention explainer page (marketmaker.cc,
// flash-attention-trading-models), section "FA3: the Hopper mechanics", item
// 3, describes FP8 attention.  Naive block quantisation suffers from
// outliers, so the vectors are first multiplied by a random orthogonal
// matrix, which spreads an outlier over all coordinates.  Here the matrix is
// R = diag(s) H / 8, where H is the 64 x 64 Sylvester Hadamard matrix and s
// is a vector of signs given as a 64-bit mask.  R is orthogonal, so
// (Q R)(K R)^T = Q K^T.  R is applied to the rows of Q and K only.
//
// Two stages:
//  * a quantisation pre-pass (three launches) writes E4M3 codes and power-of-two scales 2^e,
//    with e = floor(log2 amax) - 7.  Q and K get one scale per 64 rows of a
//    head; V gets one per column of a head, because P V accumulates each
//    output column over all keys and so needs only one multiply at the end.
//    The rotation is the fast Walsh-Hadamard transform in fp32: strides 1,
//    2, ..., 32, each pair (a, b) -> (a + b, a - b), then times 1/8.
//  * the forward streams 64-key tiles of the K codes and of the transposed
//    V codes through LDS.  Each product is one v_mfma_f32_32x32x64_f8f6f4
//    per 32 x 32 block: S^T = K Q^T contracts over the head dimension (64),
//    and O^T = V^T P^T over the tile's 64 keys.  The online softmax is the
//    bf16 kernel's, in the units of the tile's scale product 2^(eq + ek).
//    The probabilities go to E4M3 as 256 P: the factor 2^8, folded into the
//    exponent, keeps small weights out of the subnormal range.  l sums the
//    unrounded values, and LSE removes the 2^8 again.
//
// Code layouts (all per head, bytes):
//   Q8, K8  N x 64 row-major codes;
//   V8T     64 x NP, NP = N rounded up to 64: row d holds column d of V.
//           Within each 64-key group the sixteen 4-key words are stored
//           evens first: stored word w holds keys 4s .. 4s+3, where
//           s = 2 (w % 8) + w / 8.  Keys at or past N hold zero codes.
//   EQ, EK  int32 exponent per 64-row block; EV int32 exponent per column.
// The word order makes one lane's 32 contiguous bytes of a V^T row the 32 keys
// of its half of the probability operand.  That operand comes from the score
// result's register layout (lane half h holds keys 8a + 4h + b of each
// 32-key sub-block), so no register shuffle is needed.
#include <type_traits>

#include "launch.hpp"
#include "tile.hpp"

namespace fbd {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Four fp32 values as four E4M3 bytes, first value in the low byte
// (v_cvt_pk_fp8_f32: round to nearest even).
__device__ __forceinline__ int f8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// floor(log2 a) - 7 for finite a > 0, 0 otherwise: a / 2^e lies in [128, 256).
__device__ __forceinline__ int blk_exp(float a) {
  return a > 0.f ? __builtin_amdgcn_frexp_expf(a) - 8 : 0;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

// ---------------------------------------------------------------------------
// Pre-pass.
// ---------------------------------------------------------------------------

// Q and K in one launch: one wave per 64-row block of one head, one row per
// lane; blocks [0, nqb) are Q's, the rest K's.  Workgroup 0 also clears the
// nvmax column maxima that the V kernels accumulate next on the stream.
template <class T>
__global__ __launch_bounds__(64) void fp8_quant_rows_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, uint8_t* __restrict__ Q8,
    uint8_t* __restrict__ K8, int* __restrict__ EQ, int* __restrict__ EK,
    uint32_t* __restrict__ VMAX, int nvmax, int N, int nb, int nqb, int rotate, uint32_t s_lo,
    uint32_t s_hi) {
  const bool isq = (int)blockIdx.x < nqb;
  const int bid = isq ? blockIdx.x : blockIdx.x - nqb;
  const T* X = isq ? Q : K;
  uint8_t* X8 = isq ? Q8 : K8;
  int* E = isq ? EQ : EK;
  const int head = bid / nb, blk = bid % nb;
  const int lane = threadIdx.x;
  if (blockIdx.x == 0)
    for (int i = lane; i < nvmax; i += 64) VMAX[i] = 0u;
  const int row = blk * 64 + lane;
  const bool ok = row < N;
  float x[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) x[i] = 0.f;
  if (ok) {
    const T* p = X + ((size_t)head * N + row) * HD;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, reinterpret_cast<const uint4*>(p)[c]);
#pragma unroll
        for (int s = 0; s < 8; ++s) x[8 * c + s] = (float)b[s];
      }
    } else {
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const f32x4 f = reinterpret_cast<const f32x4*>(p)[c];
#pragma unroll
        for (int s = 0; s < 4; ++s) x[4 * c + s] = f[s];
      }
    }
  }
  if (rotate) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const uint32_t bit = ((i < 32 ? s_lo >> i : s_hi >> (i - 32)) & 1u) << 31;
      x[i] = __uint_as_float(__float_as_uint(x[i]) ^ bit);
    }
#pragma unroll
    for (int hs = 1; hs < 64; hs *= 2)
#pragma unroll
      for (int i = 0; i < 64; ++i)
        if ((i & hs) == 0) {
          const float a = x[i], b = x[i + hs];
          x[i] = a + b;
          x[i + hs] = a - b;
        }
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] *= 0.125f;
  }
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) am = fmaxf(am, fabsf(x[i]));
  const int e = blk_exp(wave_max(am));
  if (lane == 0) E[(size_t)head * nb + blk] = e;
  if (ok) {
    i32x4* out = reinterpret_cast<i32x4*>(X8 + ((size_t)head * N + row) * HD);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      i32x4 w;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 16 * c + 4 * q;
        w[q] = f8x4(__builtin_amdgcn_ldexpf(x[i], -e), __builtin_amdgcn_ldexpf(x[i + 1], -e),
                    __builtin_amdgcn_ldexpf(x[i + 2], -e), __builtin_amdgcn_ldexpf(x[i + 3], -e));
      }
      out[c] = w;
    }
  }
}

// Column maxima of V: one workgroup per 256 rows of one head, 16-byte loads
// (a wave reads whole rows), folded into VMAX with an atomic max on the bit
// patterns (non-negative floats order like their bits).
template <class T>
__global__ __launch_bounds__(256) void fp8_vmax_kernel(const T* __restrict__ V,
                                                       uint32_t* __restrict__ VMAX, int N,
                                                       int nch) {
  constexpr int EPL = 16 / (int)sizeof(T);   // elements per 16-byte load
  constexpr int LPR = HD / EPL;               // lanes per row
  constexpr int RPI = 256 / LPR;              // rows per workgroup iteration
  __shared__ float red[4][HD];
  const int head = blockIdx.x / nch, ch = blockIdx.x % nch;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cg = tid % LPR, r0 = tid / LPR;
  const T* p = V + (size_t)head * N * HD + cg * EPL;
  float m[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) m[e] = 0.f;
#pragma unroll
  for (int i = 0; i < 256 / RPI; ++i) {
    const int r = ch * 256 + r0 + i * RPI;
    if (r < N) {
      const uint4 u = *reinterpret_cast<const uint4*>(p + (size_t)r * HD);
      if constexpr (sizeof(T) == 2) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, u);
#pragma unroll
        for (int e = 0; e < EPL; ++e) m[e] = fmaxf(m[e], fabsf((float)b[e]));
      } else {
        const f32x4 f = __builtin_bit_cast(f32x4, u);
#pragma unroll
        for (int e = 0; e < EPL; ++e) m[e] = fmaxf(m[e], fabsf(f[e]));
      }
    }
  }
#pragma unroll
  for (int off = LPR; off < 64; off *= 2)
#pragma unroll
    for (int e = 0; e < EPL; ++e) m[e] = fmaxf(m[e], __shfl_xor(m[e], off, 64));
  if (lane < LPR)
#pragma unroll
    for (int e = 0; e < EPL; ++e) red[wave][cg * EPL + e] = m[e];
  __syncthreads();
  if (tid < HD) {
    const float am = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
    atomicMax(&VMAX[(size_t)head * HD + tid], __float_as_uint(am));
  }
}

// V codes, transposed: one workgroup per 64-key tile of one head.  The tile's
// sixteen 4-key words per column are stored in the order stored word w holds
// source word 2 (w % 8) + w / 8.
template <class T>
__global__ __launch_bounds__(256) void fp8_quant_v_kernel(const T* __restrict__ V,
                                                          const uint32_t* __restrict__ VMAX,
                                                          uint8_t* __restrict__ V8T,
                                                          int* __restrict__ EV, int N, int NP,
                                                          int ntile) {
  // workgroup: one 64-key tile of one head.  Loads are row-major and whole
  // rows wide (a lane takes 4 keys x 4 columns; the 16 lanes of a key group
  // cover one 128-byte bf16 row per instruction); each lane packs its column
  // codes into 4-key words, the words meet in LDS as a 64 x 16 word tile of
  // V^T in stored order, and each lane then writes 16 contiguous bytes of
  // one V^T row
  __shared__ uint32_t sw[HD][17];   // [column][stored word], padded
  const int head = blockIdx.x / ntile, t = blockIdx.x % ntile;
  const int tid = threadIdx.x, lane = tid & 63;
  const int dg = lane & 15, s = (lane >> 4) + 4 * (tid >> 6);   // columns 4dg.., key group s
  const int d0 = 4 * dg;
  int e[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) e[c] = blk_exp(__uint_as_float(VMAX[(size_t)head * HD + d0 + c]));
  if (t == 0 && s == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) EV[(size_t)head * HD + d0 + c] = e[c];
  }
  const T* p = V + (size_t)head * N * HD + d0;
  float x[4][4];   // [key][column]
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int key = t * 64 + 4 * s + b;
    if constexpr (sizeof(T) == 2) {
      const uint2 u = key < N ? *reinterpret_cast<const uint2*>(p + (size_t)key * HD)
                              : make_uint2(0, 0);
      const bf16x4 v4 = __builtin_bit_cast(bf16x4, u);
#pragma unroll
      for (int c = 0; c < 4; ++c) x[b][c] = (float)v4[c];
    } else {
      const f32x4 v4 = key < N ? *reinterpret_cast<const f32x4*>(p + (size_t)key * HD)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) x[b][c] = v4[c];
    }
  }
  // key group s is stored as word 8 (s & 1) + (s >> 1) of its 64-key group
  const int w = 8 * (s & 1) + (s >> 1);
#pragma unroll
  for (int c = 0; c < 4; ++c)
    sw[d0 + c][w] = (uint32_t)f8x4(__builtin_amdgcn_ldexpf(x[0][c], -e[c]),
                                   __builtin_amdgcn_ldexpf(x[1][c], -e[c]),
                                   __builtin_amdgcn_ldexpf(x[2][c], -e[c]),
                                   __builtin_amdgcn_ldexpf(x[3][c], -e[c]));
  __syncthreads();
  const int d = tid >> 2, part = tid & 3;
  const uint4 o = make_uint4(sw[d][4 * part], sw[d][4 * part + 1], sw[d][4 * part + 2],
                             sw[d][4 * part + 3]);
  *reinterpret_cast<uint4*>(V8T + ((size_t)head * HD + d) * NP + t * 64 + 16 * part) = o;
}

// ---------------------------------------------------------------------------
// Forward.
// ---------------------------------------------------------------------------

// LDS tile: 64 rows x 64 bytes; the four 16-byte chunks of row r are XOR-
// swizzled by (r >> 2) & 3, so the 16 lanes a ds_read_b128 serves per cycle
// (16 consecutive rows, one chunk) hit 16 different bank groups.
__device__ __forceinline__ int swz8(int r) { return (r >> 2) & 3; }

// DMA of one tile: source row r at byte off0 + r * stride (4 waves, one
// 1 KB instruction each).  Bytes past the resource's end read as zero.
__device__ __forceinline__ void dma8(__amdgpu_buffer_rsrc_t rs, uint32_t off0, uint32_t stride,
                                     uint8_t* tile, int wave, int lane) {
  const int L = wave * 64 + lane;
  const int r = L >> 2, cl = L & 3;
  const uint32_t voff = off0 + (uint32_t)r * stride + (uint32_t)((cl ^ swz8(r)) << 4);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + wave * 1024), 16, voff, 0, 0,
                                           0);
}

// Operand of a 32x32x64 fp8 product from a tile: lane -> row r, bytes
// 32h .. 32h + 31 of the row (h = lane >> 5).
__device__ __forceinline__ i32x8 ld8(const uint8_t* tile, int r, int h) {
  const i32x4 a = *reinterpret_cast<const i32x4*>(tile + r * 64 + (((2 * h) ^ swz8(r)) << 4));
  const i32x4 b = *reinterpret_cast<const i32x4*>(tile + r * 64 + (((2 * h + 1) ^ swz8(r)) << 4));
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ f32x16 mma8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ f32x16 splat16(float x) {
  f32x16 r;
#pragma unroll
  for (int v = 0; v < 16; ++v) r[v] = x;
  return r;
}

constexpr int F8_BLK = 128;   // query rows per workgroup: 4 waves x 32

template <class T, bool CAUSAL, bool DOCS, bool BMASK>
__global__ __launch_bounds__(256, FBD_FP8_OCC) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8,
    const uint8_t* __restrict__ V8T, const int* __restrict__ EQ, const int* __restrict__ EK,
    const int* __restrict__ EV, T* __restrict__ O, float* __restrict__ LSE, int N, int NP,
    int nb, int BH, int H, int grp, int win, const int* __restrict__ DS,
    const uint8_t* __restrict__ BMK, int nblk, float scale) {
  __shared__ __attribute__((aligned(16))) uint8_t K0[64 * 64];
  __shared__ __attribute__((aligned(16))) uint8_t V0[64 * 64];
  __shared__ __attribute__((aligned(16))) uint8_t K1[64 * 64];
  __shared__ __attribute__((aligned(16))) uint8_t V1[64 * 64];

  const Work wk = row_work(BH, nblk);
  const int kvh = kv_head(wk.head, H, grp);
  const auto rk = make_rsrc(K8 + (size_t)kvh * N * HD, (uint32_t)N * HD);
  const auto rv = make_rsrc(V8T + (size_t)kvh * HD * NP, (uint32_t)HD * NP);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6),
            h = lane >> 5;
  const int q0 = wk.blk * F8_BLK;
  const int qw = q0 + wave * WROWS;
  const int my_i = qw + (lane & 31);
  const float sl2 = scale * LOG2E;

  i32x8 qf;
  {
    const i32x4 z = {0, 0, 0, 0};
    const i32x4* p = reinterpret_cast<const i32x4*>(Q8 + ((size_t)wk.head * N + my_i) * HD + 32 * h);
    const i32x4 a = my_i < N ? p[0] : z, b = my_i < N ? p[1] : z;
    qf = i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  // the wave's 32 rows lie in one 64-row scale block
  const int eq = qw < N ? EQ[(size_t)wk.head * nb + qw / 64] : 0;
  const int* ek = EK + (size_t)kvh * nb;

  // m: running max of the raw score (unscaled units); l: running sum of
  // 256 * exp(scale * (S - m)); o: unnormalised output (in V's code units).
  float m = 0.f, l = 0.f;
  bool seen = false;
  f32x16 o0 = zero16(), o1 = zero16();

  // the masks of the bf16 forward: keys from each row's start (sliding
  // window, document), block-sparse tiles skipped (a compile-time variant)
  const int* ds = DOCS ? DS + (size_t)(wk.head / H) * N : nullptr;
  const int rs = DOCS ? row_start(ds, my_i, win, N) : 0;           // this lane's row
  const int rs_w = DOCS ? __builtin_amdgcn_readlane(rs, 31) : 0;   // the wave's largest
  const int rs0 = DOCS ? row_start(ds, q0, win, N) : q0 - win + 1;
  const int jbeg = CAUSAL ? min(max(0, rs0), q0) / 64 * 64 : 0;
  const int jend = CAUSAL ? min(N, q0 + F8_BLK) : N;
  const int ntiles = (jend - jbeg + 63) / 64;
  const int nbm = (N + 127) >> 7;
  const uint8_t* bmr = BMASK ? BMK + ((size_t)(wk.head / H) * nbm + (q0 >> 7)) * nbm : nullptr;
  auto kept = [&](int t) { return !BMASK || bmr[(jbeg + t * 64) >> 7] != 0; };

  auto tile = [&](int t, const uint8_t* Ks, const uint8_t* Vs, uint8_t* Kn, uint8_t* Vn) {
    const int j0 = jbeg + t * 64;
    wait_dma();
    __syncthreads();   // tile t is in (Ks, Vs); every wave is done with (Kn, Vn)
    if (t + 1 < ntiles && kept(t + 1)) {
      dma8(rk, (uint32_t)(j0 + 64) * HD, HD, Kn, wave, lane);
      dma8(rv, (uint32_t)(j0 + 64), (uint32_t)NP, Vn, wave, lane);
    }
    if (!kept(t)) return;
    // scores in units of 2^et: x = S / 2^et - m / 2^et (the accumulator
    // starts from -m / 2^et, exact: a power-of-two scaling)
    const int et = eq + ek[j0 >> 6];
    const float c = __builtin_amdgcn_ldexpf(1.f, et);
    const float sl2c = sl2 * c;
    f32x16 x[2];
    const f32x16 nm = splat16(-__builtin_amdgcn_ldexpf(m, -et));
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) x[sb] = mma8(ld8(Ks, sb * 32 + (lane & 31), h), qf, nm);
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int js = j0 + sb * 32;
      if (CAUSAL ? (js + 31 > qw || (DOCS ? js < rs_w : js <= qw + 31 - win)) : (js + 32 > N)) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = js + 8 * (v >> 2) + 4 * h + (v & 3);
          bool hide;
          if constexpr (!CAUSAL) hide = j >= N;
          else if constexpr (DOCS) hide = j > my_i || j < rs;
          else hide = (unsigned)(my_i - j) >= (unsigned)win;
          x[sb][v] = hide ? -INFINITY : x[sb][v];
        }
      }
    }
    float xm = x[0][0];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int v = 0; v < 16; ++v) xm = vmax(xm, x[sb][v]);
    xm = half_max(xm);
    const bool fresh = !seen && xm > -INFINITY;
    const float base = seen ? vmax(xm, 0.f) : (fresh ? xm : 0.f);
    if (__any(seen && xm > 0.f)) {
      const float alpha = seen ? __builtin_amdgcn_exp2f(-base * sl2c) : 1.f;
      l *= alpha;
      o0 *= alpha;
      o1 *= alpha;
    }
    m += base * c;
    seen = seen || fresh;
    // 256 P (at most 256: x - base <= 0), four keys per word, sub-block
    // sb's registers 4a .. 4a+3 in word 4 sb + a
    float p[2][16];
    if (__any(base != 0.f)) {
      // one FMA: the weight at the max is 256 * 2^e with |e| < 2^-10, which
      // the E4M3 rounding takes to exactly 256
      const float off = fmaf(-base, sl2c, 8.f);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          p[sb][v] = __builtin_amdgcn_exp2f(fmaf(x[sb][v], sl2c, off));
    } else {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int v = 0; v < 16; ++v) p[sb][v] = __builtin_amdgcn_exp2f(fmaf(x[sb][v], sl2c, 8.f));
    }
    i32x8 pb;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        pb[4 * sb + a] = f8x4(p[sb][4 * a], p[sb][4 * a + 1], p[sb][4 * a + 2], p[sb][4 * a + 3]);
        l += (p[sb][4 * a] + p[sb][4 * a + 1]) + (p[sb][4 * a + 2] + p[sb][4 * a + 3]);
      }
    o0 = mma8(ld8(Vs, lane & 31, h), pb, o0);
    o1 = mma8(ld8(Vs, 32 + (lane & 31), h), pb, o1);
  };
  if (!BMASK || (ntiles > 0 && kept(0))) {
    dma8(rk, (uint32_t)jbeg * HD, HD, K0, wave, lane);
    dma8(rv, (uint32_t)jbeg, (uint32_t)NP, V0, wave, lane);
  }
  for (int t = 0; t < ntiles; t += 2) {
    tile(t, K0, V0, K1, V1);
    if (t + 1 < ntiles) tile(t + 1, K1, V1, K0, V0);
  }
  // a row left with no visible key (block masks only): O = 0, LSE = -inf
  const float lt = half_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int* ev = EV + (size_t)kvh * HD;
#pragma unroll
  for (int mf = 0; mf < 2; ++mf) {
    const f32x16& acc = mf ? o1 : o0;
    float out[16];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const i32x4 e = *reinterpret_cast<const i32x4*>(ev + 32 * mf + 8 * a + 4 * h);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        out[4 * a + b] = __builtin_amdgcn_ldexpf(acc[4 * a + b] * inv, e[b]);
    }
    st_cols(O + (size_t)wk.head * N * HD, N, qw, 32 * mf, lane, out);
  }
  if (h == 0 && my_i < N)
    LSE[(size_t)wk.head * N + my_i] =
        lt > 0.f ? scale * m + (__builtin_amdgcn_logf(lt) - 8.f) * LN2 : -INFINITY;
}

hipError_t launch_fp8_quantize(int dt, const void* Q, const void* K, const void* V, uint8_t* Q8,
                               uint8_t* K8, uint8_t* V8T, int* EQ, int* EK, int* EV,
                               uint32_t* VMAX, int BH, int BHkv, int N, int rotate,
                               uint64_t signs, hipStream_t st) {
  const int nb = (N + 63) / 64, NP = nb * 64, nch = (N + 255) / 256;
  const uint32_t lo = (uint32_t)signs, hi = (uint32_t)(signs >> 32);
  auto run = [&](auto tag) -> hipError_t {
    using T = decltype(tag);
    hipLaunchKernelGGL(fp8_quant_rows_kernel<T>, dim3((BH + BHkv) * nb), dim3(64), 0, st,
                       (const T*)Q, (const T*)K, Q8, K8, EQ, EK, VMAX, BHkv * HD, N, nb, BH * nb,
                       rotate, lo, hi);
    hipLaunchKernelGGL(fp8_vmax_kernel<T>, dim3(BHkv * nch), dim3(256), 0, st, (const T*)V, VMAX,
                       N, nch);
    hipLaunchKernelGGL(fp8_quant_v_kernel<T>, dim3(BHkv * nb), dim3(256), 0, st, (const T*)V,
                       (const uint32_t*)VMAX, V8T, EV, N, NP, nb);
    return hipGetLastError();
  };
  return dt == 0 ? run(bf16{}) : run(float{});
}

hipError_t launch_fwd_fp8(int dt, const uint8_t* Q8, const uint8_t* K8, const uint8_t* V8T,
                          const int* EQ, const int* EK, const int* EV, void* O, float* LSE,
                          int BH, int H, int grp, int win, const int* ds, const uint8_t* bm, int N,
                          int causal, float scale, hipStream_t st) {
  const int nb = (N + 63) / 64, NP = nb * 64;
  const int nblk = (N + F8_BLK - 1) / F8_BLK;
  auto run = [&](auto tag, auto cz, auto dz, auto bz) -> hipError_t {
    using T = decltype(tag);
    hipLaunchKernelGGL((fwd_fp8_kernel<T, decltype(cz)::value, decltype(dz)::value,
                                       decltype(bz)::value>),
                       dim3(nblk * BH), dim3(256), 0, st, Q8, K8, V8T, EQ, EK, EV, (T*)O, LSE, N,
                       NP, nb, BH, H, grp, win, ds, bm, nblk, scale);
    return hipGetLastError();
  };
  auto masks = [&](auto tag) -> hipError_t {
    using Y = std::true_type;
    using F = std::false_type;
    if (!causal) return bm ? run(tag, F{}, F{}, Y{}) : run(tag, F{}, F{}, F{});
    if (ds) return bm ? run(tag, Y{}, Y{}, Y{}) : run(tag, Y{}, Y{}, F{});
    return bm ? run(tag, Y{}, F{}, Y{}) : run(tag, Y{}, F{}, F{});
  };
  return dt == 0 ? masks(bf16{}) : masks(float{});
}

}  // namespace fbd
