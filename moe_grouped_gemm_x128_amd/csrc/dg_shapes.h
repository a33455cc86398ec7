// dg_shapes.h -- the GEMM kernel's tile instances (one table for the kernel
// dispatch in dg_kernels.hip and the host-side queries in dg_shapes.hip).
#pragma once

#include "dg_kernel.h"

namespace dg {

constexpr int kBlockK = 128;  // K block = scale granularity

// (BM, BN, waves along M, waves along N, LDS ring stages)
#define DG_SHAPES(X)      \
  X(256, 256, 1, 8, 2)    \
  X(256, 32, 4, 1, 4)     \
  X(256, 16, 4, 1, 4)     \
  X(256, 224, 4, 2, 2)    \
  X(192, 256, 2, 4, 2)    \
  X(224, 256, 1, 8, 2)    \
  X(256, 128, 1, 8, 3)    \
  X(256, 64, 1, 4, 3)     \
  X(256, 128, 1, 4, 3)    \
  X(256, 128, 2, 2, 3)    \
  X(256, 256, 2, 4, 2)    \
  X(128, 128, 2, 2, 4)    \
  X(128, 64, 2, 2, 4)     \
  X(64, 128, 1, 4, 4)     \
  X(64, 64, 1, 4, 4)      \
  X(64, 32, 2, 2, 4)

// Instances left out: the 256x256 tile with 2x4 waves needs more than the
// register file for the fp32 read-modify-write epilogue of the weight-gradient
// kinds (it would spill); those kinds use the 1x8 layout of that tile.  The
// fused SwiGLU epilogue exists for the 256x256 tile only (on 2x4 or 1x8
// waves): its 128 gate and 128 up columns give 128 output columns, exactly
// one 1x128 scale group, and each wave holds the gate and the matching up
// columns of its rows.
constexpr bool excluded(int bm, int bn, int wm, int kind) {
  if (kind == KIND_CONTIG_SWIGLU) return !(bm == 256 && bn == 256 && (wm == 1 || wm == 2));
  // the power-of-two kinds have their fp32-scale kind's instances
  kind = layout_of(kind);
  // 192-row tiles: dense layouts only (a grouped layout's 128-row blocks would
  // straddle them); 224-row tiles: the weight gradient only (7168 = 32 x 224
  // rows of D, so 7168 x 2048 is 256 tiles of 224 x 256 on 256 CUs: 5% faster
  // warm, equal cold; the K-grouped kind's four D were 9% slower cold with it)
  if (bm == 192) return !(kind == KIND_DENSE || kind == KIND_BF16);
  if (bm == 224) return kind != KIND_WGRAD;
  return bm == 256 && bn == 256 && wm == 2 && (kind == KIND_WGRAD || kind == KIND_KGROUPED);
}

}  // namespace dg
