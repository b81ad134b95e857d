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
// their A operand is the streamed tile read along its sequence index, which
// the transposing LDS read (ds_read_b64_tr_b16) delivers from the same
// row-major tile the contractions over d read.
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
// Maximum of two scores.  The NaN-propagating maximum lowers to
// v_maximum3_f32 on gfx950 with no canonicalising moves of its inputs (fmaxf's
// NaN-ignoring form adds one v_max_f32 x, x per operand read from an MFMA
// result); scores are finite or -inf, where the two agree.
__device__ __forceinline__ float vmax(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

// ---------------------------------------------------------------------------
// LDS tiles.  A tile holds R consecutive rows (sequence positions) of one
// head's N x 64 matrix, row-major and unpadded (128 B per row for bf16, 256 B
// for fp32).  Within a row the 16-byte chunks are XOR-swizzled by a function
// of the row so that both operand reads below are spread over all banks.
// Tiles are filled by buffer -> LDS DMA (no register staging): rows at or past
// N read as zero because the buffer resource covers exactly the head's N rows.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

template <class T> struct TileFmt {
  static constexpr int CPR = HD * (int)sizeof(T) / 16;   // 16-byte chunks per row
  static constexpr int ROWB = CPR * 16;                    // bytes per row
};
// bf16: the LDS serves 256 bytes (two 128-byte rows) per cycle.  A row read
// (ds_read_b128, 16 lanes per cycle on 16 consecutive rows, one chunk column)
// is conflict-free when the 8 rows of each parity get distinct swizzles; a
// transposing read (ds_read_b64_tr_b16, 32 lanes per cycle on 4 aligned rows,
// 4 chunks each) is conflict-free when rows r and r+2 differ in bit 2 of the
// swizzle.  The bit-reversal of (row >> 1) & 7 meets both (measured on
// MI355X: 4.2 and 3.0 cycles per wave instruction, against 4.5 and 5.3 for
// (row >> 1) & 7, which fails the second).
template <class T> __device__ __forceinline__ int swz(int row) {
  if constexpr (sizeof(T) == 2)
    return (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
  else return row & 15;
}
template <class T> __device__ __forceinline__ int chunk_off(int row, int chunk) {
  return row * TileFmt<T>::ROWB + ((chunk ^ swz<T>(row)) << 4);
}

// Buffer resource over `bytes` bytes at `base`; loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Issue the DMA of rows [r0, r0 + R) of a head's matrix into `tile`.  The NW
// waves of the workgroup share the work; each wave instruction moves 64
// chunks (1 KB).  Completion: s_waitcnt vmcnt(0) in every wave, then a barrier.
template <class T, int R, int NW>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, int r0, T* tile, int wave,
                                         int lane) {
  constexpr int CPR = TileFmt<T>::CPR;
  constexpr int INSTR = R * CPR / 64;
  static_assert(INSTR % NW == 0, "tile must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < INSTR / NW; ++i) {
    const int k = wave + NW * i;
    const int L = k * 64 + lane;
    const int r = L / CPR, cl = L % CPR;
    const uint32_t voff = (uint32_t)((r0 + r) * CPR + (cl ^ swz<T>(r))) * 16u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)((char*)tile + k * 1024), 16, voff, 0,
                                             0, 0);
  }
}

// DMA of `n64` x 64 consecutive fp32 row statistics starting at row r0 (one
// wave instruction per 64 rows).
__device__ __forceinline__ void dma_rows_f32(__amdgpu_buffer_rsrc_t rs, int r0, float* dst,
                                             int k, int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + 64 * k), 4,
                                           (uint32_t)(r0 + 64 * k + lane) * 4u, 0, 0, 0);
}

__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0f70); }   // vmcnt(0)

// Operand for a contraction over d from a tile: lane -> tile row r0 + (l & 31),
// slots d = 16*kb + 8*(l >> 5) + s.
template <class T>
__device__ __forceinline__ Frag<T> ld_row(const T* tile, int r0, int kb, int lane) {
  const int r = r0 + (lane & 31);
  const char* base = reinterpret_cast<const char*>(tile);
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    f.v = *reinterpret_cast<const bf16x8*>(base + chunk_off<T>(r, 2 * kb + (lane >> 5)));
  } else {
    const int c = 4 * kb + 2 * (lane >> 5);
    const f32x4 a = *reinterpret_cast<const f32x4*>(base + chunk_off<T>(r, c));
    const f32x4 b = *reinterpret_cast<const f32x4*>(base + chunk_off<T>(r, c + 1));
    f.v = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  return f;
}

// Operand for a contraction over the sequence index from a tile: lane -> d =
// d0 + (l & 31); its slots are the sequence positions 16*jt + {4h .. 4h+3,
// 8+4h .. 8+4h+3} (h = l >> 5) -- exactly the positions registers 8t .. 8t+7
// of a 32x32 result hold for the sub-block's 16-row group t (jt = sub/16 + t).
// bf16: two ds_read_b64_tr_b16.  Within each 16-lane group that instruction
// hands result lane p, slot k, element p%4 of the 8 bytes source lane p/4+4k
// addressed; so source lane q addresses row (base + q/4) at columns
// d0 + 16*(group%2) + 4*(q%4) .. +3, and lane l receives four consecutive
// sequence positions of column d0 + (l & 31).  fp32: eight scalar reads.
typedef bf16 bf16x4v __attribute__((ext_vector_type(4)));
template <class T>
__device__ __forceinline__ Frag<T> ld_tr(const T* tile, int d0, int jt, int lane) {
  const char* base = reinterpret_cast<const char*>(tile);
  const int h = lane >> 5;
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    const int q = lane & 15;
    const int d = d0 + 16 * ((lane >> 4) & 1) + 4 * (q & 3);
    const int ra = 16 * jt + 4 * h + (q >> 2), rb = ra + 8;
    const int off = (d & 7) * 2;
    const bf16x4v x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4v*)(base + chunk_off<T>(ra, d >> 3) + off));
    const bf16x4v y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4v*)(base + chunk_off<T>(rb, d >> 3) + off));
    f.v = bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  } else {
    const int d = d0 + (lane & 31);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int pos = 16 * jt + 8 * (s >> 2) + 4 * h + (s & 3);
      f.v[s] = *reinterpret_cast<const float*>(base + chunk_off<T>(pos, d >> 2) + (d & 3) * 4);
    }
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

// Work-item order shared by all launches: a 1-D grid of nblk * BH workgroups
// with the heads varying fastest, so the first wave of workgroups takes the
// same position in every head.  Row passes go from the last row block (the
// most key blocks under the causal mask) to the first; column passes from the
// first key block (seen by the most queries) to the last.
// Document masks: ds is one batch's row of first visible keys, non-decreasing
// with ds[i] <= i (packed documents: each query sees only keys of its own
// document).  Returns the first i in [lo, hi) with ds[i] > kmax, or hi, the
// same in every lane: each round the 64 lanes probe 64 evenly spaced rows and
// a ballot narrows the range 64-fold, so N = 2^18 takes three rounds.  Every
// probe stays below hi (callers pass hi <= N) and the range shrinks every
// round, so it ends for any contents of ds.
__device__ __forceinline__ int first_above(const int* __restrict__ ds, int lo, int hi, int kmax,
                                           int lane) {
  int a = lo, b = hi;   // the answer lies in [a, b]
  while (a < b) {
    const int s = (b - a + 63) / 64;
    const int p = a + lane * s;
    const bool pred = p < b && ds[p] > kmax;
    const unsigned long long m = __ballot(pred);
    if (m == 0) {
      const int last = a + s * min(63, (b - 1 - a) / s);
      a = last + 1;
    } else {
      const int f = __builtin_ctzll(m);
      b = a + f * s;
      a = f == 0 ? b : a + (f - 1) * s + 1;
    }
  }
  return a;
}

// Block-sparse masks: a (B, nb, nb) byte array over 128 x 128 blocks of
// (query, key) positions, nb = ceil(N / 128), row-major by query block; a zero
// drops the block.  A row pass reads its 128-row block's row of the array, a
// column pass its 128-key block's column (stride nb).  The kernels take the
// mask as a compile-time variant and keep their counted tile loops: every
// tile index is visited, and a tile of a dropped block is neither loaded
// (its prefetch is skipped) nor computed.

// First visible key of query row i under the causal mask: i - win + 1 for a
// sliding window, raised to the row's document start when ds is given (row
// index clamped into the head for padding rows past N).
__device__ __forceinline__ int row_start(const int* __restrict__ ds, int i, int win, int N) {
  int r = i - win + 1;
  if (ds) r = max(r, ds[min(i, N - 1)]);
  return r;
}

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
// Key/value head used by query head `head` (of BH = batch * H): groups of grp
// consecutive query heads share one key/value head.
__device__ __forceinline__ int kv_head(int head, int H, int grp) {
  return (head / H) * (H / grp) + (head % H) / grp;
}
// First query head of key/value head `kvh`.
__device__ __forceinline__ int first_q_head(int kvh, int H, int grp) {
  const int hkv = H / grp;
  return (kvh / hkv) * H + (kvh % hkv) * grp;
}

}  // namespace fbd
