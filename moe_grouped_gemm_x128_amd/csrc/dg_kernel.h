// dg_kernel.h -- kernel parameter block and launch interface shared by the
// host dispatcher (dg_api.hip) and the gfx950 kernels (dg_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dg.h"

namespace dg {

// Problem kinds; the kernel template is specialised on these.
enum Kind : int {
  KIND_DENSE = 0,       // C bf16 [M,N];      B scales per 128x128 block
  KIND_CONTIGUOUS = 1,  // C bf16 [M_tot,N];  expert per row from m_indices
  KIND_MASKED = 2,      // C bf16 [G,Mx,N];   rows < masked_m[g]
  KIND_WGRAD = 3,       // D fp32 [M,N] +=;   B scales per row
  KIND_KGROUPED = 4,    // D fp32 [G,M,N] +=; per-group K ranges
  KIND_DENSE_POW2 = 5,  // C bf16 [M,N]; power-of-two scales applied by the block-scaled MFMA
  KIND_BF16 = 6,        // C bf16 [M,N] = A bf16 [M,K] . B bf16 [N,K]^T; no scales; a "K block" is
                        // 128 bytes = 64 values (lda = 2K bytes, kbs = K/64)
  KIND_CONTIG_SWIGLU = 7,  // contiguous layout with B [G,2I,K] (gate rows, then up rows); the
                           // epilogue applies SwiGLU to the bf16-rounded pair and writes
                           // fp8 q [M_tot,I] with 1x128 scales [M_tot,I/128] (out, out_scale)
  KIND_CONTIG_POW2 = 8,    // KIND_CONTIGUOUS with power-of-two scales applied by the block-scaled MFMA
  KIND_MASKED_POW2 = 9,    // KIND_MASKED with power-of-two scales applied by the block-scaled MFMA
  KIND_CONTIG_BF16 = 10,   // KIND_CONTIGUOUS with bf16 operands and no scales (as KIND_BF16)
  KIND_MASKED_BF16 = 11,   // KIND_MASKED with bf16 operands and no scales (as KIND_BF16)
};

// The operand layout and scheduling of a kind (the power-of-two and the
// grouped bf16 kinds share their fp32-scale kind's; the dense bf16 kind
// keeps its own).
constexpr int layout_of(int kind) {
  return kind == KIND_DENSE_POW2                                 ? KIND_DENSE
         : kind == KIND_CONTIG_POW2 || kind == KIND_CONTIG_BF16 ? KIND_CONTIGUOUS
         : kind == KIND_MASKED_POW2 || kind == KIND_MASKED_BF16 ? KIND_MASKED
                                                                 : kind;
}
constexpr bool bf16_kind(int kind) {
  return kind == KIND_BF16 || kind == KIND_CONTIG_BF16 || kind == KIND_MASKED_BF16;
}
constexpr bool pow2_kind(int kind) {
  return kind == KIND_DENSE_POW2 || kind == KIND_CONTIG_POW2 || kind == KIND_MASKED_POW2;
}

constexpr int kMaxKGroups = 256;

struct Params {
  const uint8_t* a;      // fp8 LHS (row stride lda bytes)
  const float* sa;       // LHS scales, row stride sks words
  const uint8_t* b;      // fp8 RHS, [G][N][lda]
  const float* sb;       // RHS scales: [G][NB][kbs] (block) or [N][kbs] (row)
  void* out;             // bf16 C or fp32 D (fused SwiGLU: fp8 codes)
  float* out_scale;      // fused SwiGLU: the codes' 1x128 scales
  const int32_t* ctrl;   // m_indices (contiguous) or masked_m (masked)
  int m;                 // rows per group: M, M_total or M_max
  int n;                 // N
  int lda;               // bytes per operand row: K, or total tokens T
  int kbs;               // K blocks per operand row (lda / 128)
  int sks;               // scale row stride in 4-byte words: kbs (fp32 scales) or
                         // ceil(kbs / 4) (packed UE8M0: four exponent bytes per word)
  int spk;               // log2 of the K blocks per scale word: 0 or 2 (packed)
  int groups;            // G (1 for dense and wgrad)
  int tiles_m;           // ceil(m / BM)
  int tiles_n;           // ceil(n / BN)
  int tiles;             // tile count (upper bound for the masked layout)
  int vec_out;           // 1 if 4 consecutive outputs may be stored as one vector
  // split-K (dense and masked): `splits` workgroups share one output tile,
  // split s covering K blocks [s*kchunk, min(kbs, (s+1)*kchunk)) and writing
  // its fp32 partial tile to ws + s*ws_stride (same row/column indexing as
  // the output); the reduction kernel then sums the partials in split order.
  int splits;            // 1 = no split
  int kchunk;            // K blocks per split
  float* ws;             // fp32 partials [splits][rows of all groups][n]
  int64_t ws_stride;     // floats per split
  int kg_min_blocks;     // K-grouped: fewest K blocks of any non-empty group
  int kb_begin[kMaxKGroups + 1];  // K-grouped: first 128-block of each group
};

struct TileShape {
  int bm, bn, wm, wn;
};

// Launches the kernel instance for (kind, shape) on `stream`.  Returns
// hipErrorInvalidValue if no instance exists for that shape.
hipError_t launch(int kind, const TileShape& shape, const Params& p, int grid,
                  hipStream_t stream);

// Sums the split-K partials of p.ws in split order and writes bf16 p.out
// (dense: every row; masked: rows below masked_m of each group).
hipError_t launch_splitk_reduce(int kind, const Params& p, hipStream_t stream);

// FP8 quantiser (dg_quant.hip).  mode 0: x [rows,cols] -> 1x128 groups
// along cols; 1: 128x128 blocks; 2: x [rows=T, cols=F] -> q [F,T] with 1x128
// groups along T; 3, 4: modes 0, 1 with power-of-two scales written as packed
// UE8M0 bytes (s then points to int32 words).  num_cus sizes the grid.
hipError_t launch_swiglu_quantize(const uint16_t* c, uint8_t* q, float* s, int rows, int half_cols, int num_cus,
                                  hipStream_t stream);
hipError_t launch_quantize(int mode, const float* x, uint8_t* q, float* s, int rows, int cols, int num_cus,
                           hipStream_t stream);

// The masked-layout GEMM (dg_grouped_fp8_masked's contract) with split-K
// partials from the library's pool (scratch == nullptr) or from the device
// buffer of scratch_floats floats that scratch() returns, asked for only when
// K is split, after the arguments are validated (no allocation; split K is
// kept under graph capture; DG_ERROR_WORKSPACE if the partials do not fit).
dg_status grouped_masked(const void* a, const float* sa, const void* b, const float* sb, void* c,
                         const int32_t* masked_m, int num_groups, int m_max, int n, int k, hipStream_t stream,
                         float* (*scratch)(), size_t scratch_floats);

// True if an instance exists for (kind, shape).
bool has_instance(int kind, const TileShape& shape);

// Threads per workgroup (64 per wave) and LDS bytes per workgroup of an
// instance; 0 if there is none.
int threads_of(const TileShape& shape);
int lds_bytes_of(int kind, const TileShape& shape);

}  // namespace dg
