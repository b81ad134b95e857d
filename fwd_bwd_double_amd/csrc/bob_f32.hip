// Backward-over-backward launches for fp32 operands (kernels in
// bob_kernels.hpp; see bob.hip for why this is a separate translation unit).
#include "bob_kernels.hpp"

namespace fbd {

hipError_t launch_bob_f32(const void* Q, const void* K, const void* V, const void* O,
                          const float* LSE, const void* dO, const void* gdQ, const void* gdK,
                          const void* gdV, void* gQ, void* gK, void* gV, void* gdO, float* Dws,
                          float* Aws, float* Bws, float* Lws, float* Kws, int BH, int H, int grp,
                          int win, const int* ds, const uint8_t* bm, int N, int causal,
                          float scale, int passes, int nsl, float* Part, hipStream_t st) {
#define FBD_BOB_ARGS Q, K, V, O, LSE, dO, gdQ, gdK, gdV, gQ, gK, gV, gdO, Dws, Aws, Bws, Lws, Kws, \
                     BH, H, grp, win, ds, bm, N, scale, passes, nsl, Part, 0, st
  if (!causal) return launch_bob_t<float, false, false>(FBD_BOB_ARGS);
  return ds ? launch_bob_t<float, true, true>(FBD_BOB_ARGS)
            : launch_bob_t<float, true, false>(FBD_BOB_ARGS);
#undef FBD_BOB_ARGS
}

}  // namespace fbd
