// Device building blocks shared by the attention kernels (gfx950 / CDNA4).
//
// Matrix products use the 32x32 MFMA family: v_mfma_f32_32x32x16_bf16 for
// bf16 operands and v_mfma_f32_32x32x2_f32 for fp32 ones, always with fp32
// accumulation.  Lane l of a wave feeds operand row/column (l & 31) and the
// eight contraction slots 8*(l >> 5) + s, s = 0..7 (for fp32 the eight slots
// go through eight 32x32x2 instructions, so both element types present one
// "Frag" of eight values per lane and one logical K = 16 step).  The 32x32
// fp32 result lives in 16 registers per lane: register v of lane l holds
// row 8*(v/4) + 4*(l/32) + v%4 and column l % 32.
//
// Every kernel computes its score tiles with the *stored* operand in the
// row slot and the register-resident operand in the column slot, so a lane
// owns one query (row passes) or one key (column passes) and the other index
// runs down its registers.  Products that contract over that other index
// then take the probability tile straight from registers as the B operand;
// the A operand must be the streamed tile read along its row index, which is
// why streamed tiles are kept in LDS twice: row-major (for contractions over
// d) and transposed (for contractions over the sequence).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fbd {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int HD = 64;        // head dimension
constexpr int NT = 256;       // threads per workgroup (4 waves)
constexpr int WROWS = 32;     // rows (queries or keys) owned by one wave
constexpr int BLK = NT / 64 * WROWS;   // rows owned by one workgroup: 128
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

template <class T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x8 v; };

template <class T> struct Lay;
// Row-major LDS tiles: row stride in elements.  The padding keeps the 16-lane
// groups of an operand read on distinct banks.
template <> struct Lay<bf16> { static constexpr int RS = HD + 8; static constexpr int TP = 4; };
template <> struct Lay<float> { static constexpr int RS = HD + 4; static constexpr int TP = 4; };

__device__ __forceinline__ void mma(f32x16& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[s], b.v[s], acc, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int v = 0; v < 16; ++v) z[v] = 0.f;
  return z;
}

// Value held by lane l ^ 32.
__device__ __forceinline__ float other_half(float x) { return __shfl_xor(x, 32, 64); }

// Combine a value across the two half-waves (lanes l and l ^ 32) with
// v_permlane32_swap: the swap of x with itself returns lanes 0..31 of x in
// both halves of the first result and lanes 32..63 in both halves of the
// second, so op(first, second) is the same in every lane of a pair.
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum of the eight element-type values of an operand fragment, added to acc
// (bf16: four v_dot2_f32_bf16 against (1, 1)).
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float frag_acc_sum(const Frag<bf16>& f, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x2 pr = {f.v[2 * k], f.v[2 * k + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
  }
  return acc;
}
__device__ __forceinline__ float frag_acc_sum(const Frag<float>& f, float acc) {
#pragma unroll
  for (int k = 0; k < 8; ++k) acc += f.v[k];
  return acc;
}

// Round to the element type and back (round-to-nearest-even for bf16).
__device__ __forceinline__ float rnd(float x, bf16*) { return (float)(bf16)x; }
__device__ __forceinline__ float rnd(float x, float*) { return x; }

// Eight fp32 values (registers 8t .. 8t+7 of a 32x32 result) as an operand.
__device__ __forceinline__ Frag<bf16> pack8(const float* x, bf16*) {
  Frag<bf16> f;
#pragma unroll
  for (int s = 0; s < 8; ++s) f.v[s] = (bf16)x[s];
  return f;
}
__device__ __forceinline__ Frag<float> pack8(const float* x, float*) {
  Frag<float> f;
#pragma unroll
  for (int s = 0; s < 8; ++s) f.v[s] = x[s];
  return f;
}
template <class T>
__device__ __forceinline__ Frag<T> pack8(const float* x) { return pack8(x, (T*)nullptr); }

// Sum of the element-type values of a fragment, in fp32.
__device__ __forceinline__ float frag_sum(const Frag<bf16>& f) {
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += (float)f.v[k];
  return s;
}
__device__ __forceinline__ float frag_sum(const Frag<float>& f) {
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += f.v[k];
  return s;
}

// Operand for a contraction over d, read from a row-major LDS tile:
// lane -> tile row r0 + (l & 31), slots d = 16*kb + 8*(l >> 5) + s.
template <class T>
__device__ __forceinline__ Frag<T> ld_row(const T* tile, int r0, int kb, int lane) {
  const T* p = tile + (r0 + (lane & 31)) * Lay<T>::RS + kb * 16 + 8 * (lane >> 5);
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    f.v = *reinterpret_cast<const bf16x8*>(p);
  } else {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    f.v = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  return f;
}

// Operand for a contraction over the sequence index, read from a transposed
// LDS tile Xt[d][j] with row stride ts: lane -> d = d0 + (l & 31); its slots
// are the sequence positions 16*jt + {4h .. 4h+3, 8+4h .. 8+4h+3} (h = l>>5),
// which are exactly the positions that registers 8t .. 8t+7 of a 32x32 result
// hold for the sub-block's 16-row group t (jt = sub-block/16 + t).
template <class T>
__device__ __forceinline__ Frag<T> ld_tr(const T* tileT, int ts, int d0, int jt, int lane) {
  const T* p = tileT + (d0 + (lane & 31)) * ts + jt * 16 + 4 * (lane >> 5);
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
    bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 8);
    f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  } else {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 8);
    f.v = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  return f;
}

// Register-resident operand straight from global memory (one head's N x 64
// matrix): lane -> row r0 + (l & 31), slots d = 16*kb + 8*(l >> 5) + s.
// Rows at or beyond n read as zero.
template <class T>
__device__ __forceinline__ void ld_frags(const T* X, int n, int r0, int lane, Frag<T> (&f)[4]) {
  const int row = r0 + (lane & 31);
  const bool ok = row < n;
  const T* p = X + (size_t)row * HD + 8 * (lane >> 5);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    if constexpr (sizeof(T) == 2) {
      uint4 u = ok ? *reinterpret_cast<const uint4*>(p + kb * 16) : make_uint4(0, 0, 0, 0);
      f[kb].v = __builtin_bit_cast(bf16x8, u);
    } else {
      f32x4 a = ok ? *reinterpret_cast<const f32x4*>(p + kb * 16) : f32x4{0, 0, 0, 0};
      f32x4 b = ok ? *reinterpret_cast<const f32x4*>(p + kb * 16 + 4) : f32x4{0, 0, 0, 0};
      f[kb].v = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
  }
}

// Sum over d of x*y for two fragments sets holding the same rows: each lane
// covers half of d, the two half-waves are combined.
template <class T>
__device__ __forceinline__ float row_dot(const Frag<T> (&x)[4], const Frag<T> (&y)[4]) {
  float s = 0.f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int k = 0; k < 8; ++k) s += (float)x[kb].v[k] * (float)y[kb].v[k];
  return half_sum(s);
}

// Store a wave's 32 rows x 32 columns block of a result held in the
// register layout of a 32x32 product whose *columns* are the rows of the
// output (lane -> output row r0 + (l & 31); register v -> output column
// c0 + 8*(v/4) + 4*(l/32) + v%4): four consecutive columns per store.
template <class T>
__device__ __forceinline__ void st_cols(T* X, int n, int r0, int c0, int lane, const float* vals) {
  const int row = r0 + (lane & 31);
  if (row >= n) return;
  T* p = X + (size_t)row * HD + c0 + 4 * (lane >> 5);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if constexpr (sizeof(T) == 2) {
      bf16x4 o{(bf16)vals[4 * q], (bf16)vals[4 * q + 1], (bf16)vals[4 * q + 2], (bf16)vals[4 * q + 3]};
      *reinterpret_cast<bf16x4*>(p + 8 * q) = o;
    } else {
      *reinterpret_cast<f32x4*>(p + 8 * q) =
          f32x4{vals[4 * q], vals[4 * q + 1], vals[4 * q + 2], vals[4 * q + 3]};
    }
  }
}

// Load of the same layout (used for O in the BoB row-pass epilogue).
template <class T>
__device__ __forceinline__ void ld_cols(const T* X, int n, int r0, int c0, int lane, float* vals) {
  const int row = r0 + (lane & 31);
  const T* p = X + (size_t)row * HD + c0 + 4 * (lane >> 5);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (row < n) {
      if constexpr (sizeof(T) == 2) {
        bf16x4 o = *reinterpret_cast<const bf16x4*>(p + 8 * q);
#pragma unroll
        for (int r = 0; r < 4; ++r) vals[4 * q + r] = (float)o[r];
      } else {
        f32x4 o = *reinterpret_cast<const f32x4*>(p + 8 * q);
#pragma unroll
        for (int r = 0; r < 4; ++r) vals[4 * q + r] = o[r];
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) vals[4 * q + r] = 0.f;
    }
  }
}

// Global -> registers -> LDS staging of an R x 64 tile (R rows of one head's
// matrix starting at row r0; rows >= n are zero).  A unit is a pair of rows
// (2p, 2p+1) times one 16-byte column chunk c; the thread holds both rows'
// chunks so that the transposed store can write two sequence positions per
// 32-bit word (bf16) or 64-bit word (fp32).
template <class T, int R, int NTH = NT>
struct TileStage {
  static constexpr int E = 16 / sizeof(T);          // elements per chunk
  static constexpr int CPR = HD / E;                 // chunks per row
  static constexpr int UNITS = (R / 2) * CPR;
  static constexpr int U = (UNITS + NTH - 1) / NTH;  // units per thread
  uint4 a[U], b[U];

  __device__ __forceinline__ void load(const T* X, int n, int r0, int tid) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int unit = tid + NTH * u;
      const int p = unit % (R / 2), c = unit / (R / 2);
      const int row = r0 + 2 * p;
      a[u] = make_uint4(0, 0, 0, 0);
      b[u] = make_uint4(0, 0, 0, 0);
      if (unit < UNITS) {
        const T* src = X + (size_t)row * HD + c * E;
        if (row < n) a[u] = *reinterpret_cast<const uint4*>(src);
        if (row + 1 < n) b[u] = *reinterpret_cast<const uint4*>(src + HD);
      }
    }
  }

  // Multiply every element of both rows by a per-row factor (rounded back to
  // the element type).  Used for the GProj key correction term.
  __device__ __forceinline__ void scale_rows(const float* fac2, int u) {
    T* pa = reinterpret_cast<T*>(&a[u]);
    T* pb = reinterpret_cast<T*>(&b[u]);
#pragma unroll
    for (int k = 0; k < E; ++k) {
      pa[k] = (T)((float)pa[k] * fac2[0]);
      pb[k] = (T)((float)pb[k] * fac2[1]);
    }
  }

  __device__ __forceinline__ void store_rows(T* tile, int tid) const {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int unit = tid + NTH * u;
      if (unit < UNITS) {
        const int p = unit % (R / 2), c = unit / (R / 2);
        *reinterpret_cast<uint4*>(tile + (2 * p) * Lay<T>::RS + c * E) = a[u];
        *reinterpret_cast<uint4*>(tile + (2 * p + 1) * Lay<T>::RS + c * E) = b[u];
      }
    }
  }

  // tileT[d][row] with row stride TS = R + Lay<T>::TP.
  static constexpr int TS = R + Lay<T>::TP;
  __device__ __forceinline__ void store_tr(T* tileT, int tid) const {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int unit = tid + NTH * u;
      if (unit < UNITS) {
        const int p = unit % (R / 2), c = unit / (R / 2);
        if constexpr (sizeof(T) == 2) {
          const uint32_t* wa = reinterpret_cast<const uint32_t*>(&a[u]);
          const uint32_t* wb = reinterpret_cast<const uint32_t*>(&b[u]);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t lo = (k & 1) ? (wa[k >> 1] >> 16) : (wa[k >> 1] & 0xffffu);
            const uint32_t hi = (k & 1) ? (wb[k >> 1] & 0xffff0000u) : (wb[k >> 1] << 16);
            *reinterpret_cast<uint32_t*>(tileT + (c * 8 + k) * TS + 2 * p) = lo | hi;
          }
        } else {
          const float* fa = reinterpret_cast<const float*>(&a[u]);
          const float* fb = reinterpret_cast<const float*>(&b[u]);
#pragma unroll
          for (int k = 0; k < 4; ++k)
            *reinterpret_cast<f32x2*>(tileT + (c * 4 + k) * TS + 2 * p) = f32x2{fa[k], fb[k]};
        }
      }
    }
  }
};

// Work-item order shared by all launches: a 1-D grid of nblk * BH workgroups
// with the heads varying fastest, so the first wave of workgroups takes the
// same position in every head.  Row passes go from the last row block (the
// most key blocks under the causal mask) to the first; column passes from the
// first key block (seen by the most queries) to the last.
struct Work {
  int head, blk;
};
__device__ __forceinline__ Work row_work(int bh, int nblk) {
  const int L = blockIdx.x;
  return Work{L % bh, nblk - 1 - L / bh};
}
__device__ __forceinline__ Work col_work(int bh) {
  const int L = blockIdx.x;
  return Work{L % bh, L / bh};
}

}  // namespace fbd
