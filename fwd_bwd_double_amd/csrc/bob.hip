// Backward-over-backward launches for bf16 operands (the kernels are in
// bob_kernels.hpp).  The fp32 instantiations live in bob_f32.hip, a
// translation unit of their own that is compiled without the flag that keeps
// MFMA results in architectural registers: with it, the compiler fails on the
// fp32 row kernel, which is larger than the bf16 one.
#include "bob_kernels.hpp"

namespace fbd {

hipError_t launch_bob(int dt, const void* Q, const void* K, const void* V, const void* O,
                      const float* LSE, const void* dO, const void* gdQ, const void* gdK,
                      const void* gdV, void* gQ, void* gK, void* gV, void* gdO, float* Dws,
                      float* Aws, float* Bws, float* Lws, float* Kws, int BH, int H, int grp,
                      int win, const int* ds, const uint8_t* bm, int N, int causal, float scale,
                      int passes, int nsl, float* Part, int proj, hipStream_t st) {
  if (dt != 0)
    return launch_bob_f32(Q, K, V, O, LSE, dO, gdQ, gdK, gdV, gQ, gK, gV, gdO, Dws, Aws, Bws,
                          Lws, Kws, BH, H, grp, win, ds, bm, N, causal, scale, passes, nsl,
                          Part, st);
#define FBD_BOB_ARGS Q, K, V, O, LSE, dO, gdQ, gdK, gdV, gQ, gK, gV, gdO, Dws, Aws, Bws, Lws, Kws, \
                     BH, H, grp, win, ds, bm, N, scale, passes, nsl, Part, proj, st
  if (!causal) return launch_bob_t<bf16, false, false>(FBD_BOB_ARGS);
  return ds ? launch_bob_t<bf16, true, true>(FBD_BOB_ARGS)
            : launch_bob_t<bf16, true, false>(FBD_BOB_ARGS);
#undef FBD_BOB_ARGS
}

hipError_t launch_bob_row_grad(const void* Q, const void* K, const void* V, const void* O,
                               const float* LSE, const void* dO, const void* gdQ, const void* gdK,
                               const void* gdV, void* gQ, void* gdO, void* dQ, float* Dws,
                               float* Aws, float* Bws, float* Lws, float* Kws, float* Rws, int BH,
                               int H, int grp, int win, const int* ds, const uint8_t* bm, int N,
                               int causal, float scale, int gproj, int proj, hipStream_t st) {
#define FBD_BOB_ARGS Q, K, V, O, LSE, dO, gdQ, gdK, gdV, gQ, gdO, Dws, Aws, Bws, Lws, Kws, BH, H, \
                     grp, win, ds, bm, N, scale, dQ, Rws, gproj, proj, st
  if (!causal) return launch_bob_row_t<bf16, false, false, true>(FBD_BOB_ARGS);
  return ds ? launch_bob_row_t<bf16, true, true, true>(FBD_BOB_ARGS)
            : launch_bob_row_t<bf16, true, false, true>(FBD_BOB_ARGS);
#undef FBD_BOB_ARGS
}

}  // namespace fbd
