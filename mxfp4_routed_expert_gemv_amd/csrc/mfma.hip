// Host-side rules of the matrix-core path class: which shapes take the
// scaled-MXFP4 grouped GEMMs and the shared experts' bf16 matrix-core GEMMs
// (shared_gemm.hip), the persistent grid size, and the routed GEMMs' m-tile
// height.
//
// The pages keep two shared experts resident beside the routed ones (the
// kimi-k3-in-c review, "at a glance" table; the README's shard census); every
// token goes through both: S = sum_j Wd_j (silu(Wg_j x) * (Wu_j x)).
#include "internal.h"

namespace k3 {

int grouped_grid() { return (cu_count() + 7) / 8 * 8; }

// Rows per m-tile from the expected pairs per expert (T k / E), with some
// headroom so that most experts fit one tile.
int pick_mf(const k3moe_shape& s, int max_mf) {
  const double ppe = (double)s.T * s.k / s.E * 1.15;
  int mf = (int)((ppe + 15.0) / 16.0);
  if (mf < 1) mf = 1;
  if (mf > max_mf) mf = max_mf;
  return mf;
}


// The shared experts take the matrix-core kernels only inside the MFMA path
// class (so a token's bits change at no other batch size than the class
// boundary), and only when their width fits the kernels' 128-feature tiles;
// otherwise they stay GEMVs at every batch size.
bool shared_mfma_ok(const k3moe_shape& s) { return use_mfma(s) && s.f_shared % 128 == 0; }

hipError_t launch_shared_mfma(const k3moe_shape& s, const k3moe_expert_bank& b, const void* x,
                              float* h, float* y, hipStream_t st, const CombineArgs& comb) {
  // (in this class the combine stays a kernel of its own: folded into the
  // down's epilogue its scattered reads cost more than they save)
  if (comb.y_perm || !shared_lds_ok(s)) return hipErrorInvalidValue;
  return launch_shared_lds(s, b, x, h, y, st);
}

bool mfma_shape_ok(const k3moe_shape& s) {
  // the scaled-MXFP4 grouped GEMMs take 128-element stages in groups of 4
  return s.x_dtype == K3MOE_BF16 && s.d % 512 == 0 && s.f % 512 == 0;
}

}  // namespace k3
