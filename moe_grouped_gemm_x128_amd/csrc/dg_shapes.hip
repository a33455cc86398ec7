// dg_shapes.hip -- host-side queries on the GEMM kernel's tile instances
// (no device code): which instances exist, and the threads and LDS bytes of a
// workgroup of each, which the planner in dg_api.hip uses for occupancy.
#include "dg_shapes.h"

namespace dg {

bool has_instance(int kind, const TileShape& s) {
  if (kind < KIND_DENSE || kind > KIND_MASKED_BF16) return false;
#define X(BM, BN, WM, WN, S) \
  if (s.bm == BM && s.bn == BN && s.wm == WM && s.wn == WN) return !excluded(BM, BN, WM, kind);
  DG_SHAPES(X)
#undef X
  return false;
}

int threads_of(const TileShape& s) { return s.wm * s.wn * 64; }

// The ring of S stages (A and B tiles plus their scales per stage), the sink
// for padding DMAs, and the bf16 epilogue's staging rows where the kernel
// uses them (the fused SwiGLU epilogue: the waves' per-row maxima instead).
// The contiguous FP8 kinds' two-stage tiles keep A's row scales out of the
// stages, in two group buffers of 16 bytes per tile row.
int lds_bytes_of(int kind, const TileShape& s) {
  const bool row_sb = (kind == KIND_WGRAD || kind == KIND_KGROUPED);
  const bool swiglu = kind == KIND_CONTIG_SWIGLU;
  const bool sa_groups = swiglu || (layout_of(kind) == KIND_CONTIGUOUS && !bf16_kind(kind));
  const int sa_n = ((s.bm + 63) / 64) * 64;
  const int sb_n = row_sb ? ((s.bn + 63) / 64) * 64 : 64;
  const int stage = (s.bm + s.bn) * kBlockK + 4 * (sa_n + sb_n);
  const int wtn = s.bn / s.wn;
  const bool staged = !row_sb && !swiglu && (wtn == 64 || wtn == 32);
  const int out = swiglu ? s.bm * s.wn * 4 : staged ? s.wm * s.wn * 16 * (wtn * 2 + 16) : 16;
  const int groups = 2 * ((s.bm + 15) / 16) * 16 * 16;
#define X(BM, BN, WM, WN, S)                                                                    \
  if (s.bm == BM && s.bn == BN && s.wm == WM && s.wn == WN)                                     \
    return (sa_groups && S == 2) ? S * (stage - 4 * sa_n) + 1024 + groups + out : S * stage + 1024 + out;
  DG_SHAPES(X)
#undef X
  return 0;
}

}  // namespace dg
