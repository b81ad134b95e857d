// Internal launch entry points of the attention kernels (host side).  The
// public C ABI in include/fbd.h validates every argument and then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Streamed tile sizes (rows of the streamed operand per LDS stage): keys per
// tile for the row passes (BN), queries per tile for the column passes (BM).
#ifndef FBD_FWD_BN
#define FBD_FWD_BN 64
#endif
// forward: 32-query groups per wave
#ifndef FBD_FWD_G
#define FBD_FWD_G 1
#endif
// Sequence length from which the forward and the backward row pass run
// 8-wave workgroups over 256-row blocks (no block mask, bf16): each streamed
// key tile then serves twice the queries, which halves the L2-miss traffic
// of the long key streams (measured 5% and 3% faster at N = 262144; slower
// below N = 32768, where fewer, longer workgroups leave a longer tail).
#ifndef FBD_WIDE_N
#define FBD_WIDE_N 65536
#endif
// forward: minimum waves per SIMD the register budget must allow.  At 4 the
// bf16 kernel fits 128 registers without spilling (the compiler alone picks
// 138 and 3 waves); the fp32 kernel is held to 2 workgroups per CU by its
// 64 KB of LDS tiles either way.
#ifndef FBD_FWD_OCC
#define FBD_FWD_OCC 4
#endif
// FP8 forward: minimum waves per SIMD (1: the compiler's choice, 132
// registers and 3 waves; 4 waves measured no faster)
#ifndef FBD_FP8_OCC
#define FBD_FP8_OCC 1
#endif
#ifndef FBD_BWD_BN
#define FBD_BWD_BN 64
#endif
#ifndef FBD_BWD_BM
#define FBD_BWD_BM 64
#endif
#ifndef FBD_BOB_BN
#define FBD_BOB_BN 32
#endif
#ifndef FBD_BOB_BM
#define FBD_BOB_BM 64
#endif
// Minimum resident workgroups per CU the compiler must allow for (register
// budget); a 256-thread workgroup at 1 per CU may use 512 registers per lane.
#ifndef FBD_BWD_ROW_OCC
#define FBD_BWD_ROW_OCC 1
#endif
#ifndef FBD_BWD_COL_OCC
#define FBD_BWD_COL_OCC 1
#endif
#ifndef FBD_BOB_ROW_OCC
#define FBD_BOB_ROW_OCC 1
#endif
#ifndef FBD_BOB_COL_OCC
#define FBD_BOB_COL_OCC 2
#endif

namespace fbd {

// dt: 0 = bf16, 1 = fp32.  BH = batch * query heads, H = query heads per
// batch, grp = query heads per key/value head (1: multi-head; H: multi-query).
// Query-side tensors (Q, O, dO, dQ, g_dQ, g_Q, g_dO, LSE, workspaces) have BH
// heads, key-side tensors (K, V, dK, dV, g_dK, g_dV, g_K, g_V) BH / grp; query
// head h of a batch uses key head h / grp.  win: causal sliding window, key j
// visible to query i iff i - win < j <= i (a value >= N is plain causal).
// ds: nullptr, or (B, N) int32 first visible key of each query row (document
// masks: key j visible to query i of batch b iff ds[b][i] <= j <= i).
// bm: nullptr, or a (B, nb, nb) byte block-sparse mask, nb = ceil(N / 128):
// bm[b][qb][kb] == 0 drops queries 128 qb .. and keys 128 kb .. of batch b
// (on top of the other masks); dropped blocks are never loaded.
// Pointers are device pointers.
// passes (backward and BoB): bit 0 = row pass, bit 1 = column pass.
hipError_t launch_fwd(int dt, const void* Q, const void* K, const void* V, void* O, float* LSE,
                      int BH, int H, int grp, int win, const int* ds, const uint8_t* bm, int N,
                      int causal, float scale, hipStream_t st);

// Column-pass slices (backward and BoB): nsl divides grp.  With nsl == 1 a
// column-pass workgroup owns a (key block, key head) pair and writes its
// key-side results once; with nsl > 1 it owns a (key block, key head, slice of
// grp / nsl query heads) triple and writes fp32 partial sums into Part
// (2 * nsl * (BH / grp) * N * 64 floats: the nsl key-gradient blocks, then the
// nsl value-gradient blocks), which a second kernel adds up, in slice order,
// into the outputs.  Part is unused (may be null) when nsl == 1.
//
// Backward workspace: D, r, and -LSE*log2(e) per row (written by the row pass,
// read by the column pass).
hipError_t launch_bwd(int dt, const void* Q, const void* K, const void* V, const void* O,
                      const float* LSE, const void* dO, void* dQ, void* dK, void* dV, float* Dws,
                      float* Rws, float* Lws, int BH, int H, int grp, int win, const int* ds,
                      const uint8_t* bm, int N, int causal, float scale, int gproj, int passes,
                      int nsl, float* Part, hipStream_t st);

// BoB workspace: D, alpha, beta, -LSE*log2(e) and -kappa = -(alpha*D + beta) per row.
// proj != 0 projects g_Q's residual row sum (bf16 operands only).
hipError_t launch_bob(int dt, const void* Q, const void* K, const void* V, const void* O,
                      const float* LSE, const void* dO, const void* gdQ, const void* gdK,
                      const void* gdV, void* gQ, void* gK, void* gV, void* gdO, float* Dws,
                      float* Aws, float* Bws, float* Lws, float* Kws, int BH, int H, int grp,
                      int win, const int* ds, const uint8_t* bm, int N, int causal, float scale,
                      int passes, int nsl, float* Part, int proj, hipStream_t st);

// BoB's row pass fused with the first backward's row pass, for bf16 operands
// whose BoB cotangents are known before the backward runs (a Hessian-vector
// product): the row pass of launch_bob, which also writes the backward's dQ
// (with GProj when gproj != 0) and the GProj row sums r into Rws.  Dws and Lws
// are then the backward column pass's D and -LSE*log2(e), Rws its r; proj as
// for launch_bob.
hipError_t launch_bob_row_grad(const void* Q, const void* K, const void* V, const void* O,
                               const float* LSE, const void* dO, const void* gdQ, const void* gdK,
                               const void* gdV, void* gQ, void* gdO, void* dQ, float* Dws,
                               float* Aws, float* Bws, float* Lws, float* Kws, float* Rws, int BH,
                               int H, int grp, int win, const int* ds, const uint8_t* bm, int N,
                               int causal, float scale, int gproj, int proj, hipStream_t st);

// The fp32 half of launch_bob (same arguments, dt implied).
hipError_t launch_bob_f32(const void* Q, const void* K, const void* V, const void* O,
                          const float* LSE, const void* dO, const void* gdQ, const void* gdK,
                          const void* gdV, void* gQ, void* gK, void* gV, void* gdO, float* Dws,
                          float* Aws, float* Bws, float* Lws, float* Kws, int BH, int H, int grp,
                          int win, const int* ds, const uint8_t* bm, int N, int causal,
                          float scale, int passes, int nsl, float* Part, hipStream_t st);

// Adds the nsl slices of Part (layout above, BHkv = BH / grp key heads) into
// gK and gV of type dt.
hipError_t launch_sum_slices(int dt, const float* Part, int nsl, int BHkv, int N, void* gK,
                             void* gV, hipStream_t st);

// FP8 forward.  Quantisation pre-pass: E4M3 codes of Q and K (optionally
// rotated by diag(signs) H / 8 when rotate != 0) with one power-of-two scale
// exponent per 64 rows of a head, and of V transposed with one exponent per
// column; VMAX is scratch for the column maxima (BHkv x 64).  The forward
// reads only the codes and exponents.  Layouts are described in fp8.hip.
hipError_t launch_fp8_quantize(int dt, const void* Q, const void* K, const void* V, uint8_t* Q8,
                               uint8_t* K8, uint8_t* V8T, int* EQ, int* EK, int* EV,
                               uint32_t* VMAX, int BH, int BHkv, int N, int rotate,
                               uint64_t signs, hipStream_t st);
hipError_t launch_fwd_fp8(int dt, const uint8_t* Q8, const uint8_t* K8, const uint8_t* V8T,
                          const int* EQ, const int* EK, const int* EV, void* O, float* LSE,
                          int BH, int H, int grp, int win, const int* ds, const uint8_t* bm, int N,
                          int causal, float scale, hipStream_t st);

}  // namespace fbd
