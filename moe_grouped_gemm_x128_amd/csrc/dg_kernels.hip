// dg_kernels.hip -- FP8 (e4m3) fine-grained-scaled NT GEMM kernels for gfx950.
//
// One kernel template serves every layout (DeepGEMM pages, "简洁的代码设计":
// a single core GEMM kernel); the layouts differ only in how a tile id maps
// to (group, rows, columns, K range) and in the epilogue.
//
// Per workgroup tile (BM x BN outputs, 4 waves of 64 lanes):
//   * operands go HBM -> registers -> LDS, 128-wide K block at a time, double
//     buffered: the next block's global loads are in flight while the current
//     block is multiplied;
//   * each 16x16 output subtile of a K block is one v_mfma_f32_16x16x128_f8f6f4
//     with a zero accumulator: the exact fp32 block partial (DeepGEMM pages,
//     "主要特点": tensor-core FP8 accumulation alone is imprecise);
//   * the partial is promoted into the fp32 main accumulator with one VALU
//     FMA by sa[m,kb]*sb[n/128,kb] (the pages' two-level accumulation);
//   * the epilogue rounds to bf16 (or adds into fp32 D) with row/column masks.
//
// The MFMA is fed B rows as its first operand and A rows as its second, so a
// lane ends up holding 4 consecutive output columns of one output row: one
// row scale per lane and contiguous 8-byte bf16 stores.
//
// Tiles are walked by a persistent grid.  Workgroup w runs on XCD w % 8;
// the walk hands each XCD a contiguous range of tile ids so tiles that share
// A rows or B columns meet in the same L2.
#include "dg_kernel.h"

namespace dg {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBK = 128;      // K block = scale granularity
constexpr int kGroupM = 8;    // tile rows per raster group

// LDS row = 128 bytes = 8 chunks of 16 bytes.  Chunk c of row r is stored at
// chunk position c ^ swz(r).  A wave's 16-lane phase of ds_read_b128 reads one
// chunk from each of 16 consecutive rows; this swizzle spreads them over all
// banks for both a 32-bank (8 rows per phase) and a 64-bank (16 rows) view.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 h = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

struct TileInfo {
  int g;          // group (expert)
  int m0, n0;     // first row (within the group) and column
  int rows;       // valid rows from m0 (<= BM)
  int kb0, kb1;   // K block range
  int64_t a_row0; // absolute LHS row of m0
  int64_t out_row0;  // absolute output row of m0
};

template <int BM>
__device__ __forceinline__ void raster(int L, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group = kGroupM * tiles_n;
  const int gid = L / group;
  const int first = gid * kGroupM;
  const int gm = min(tiles_m - first, kGroupM);
  const int r = L - gid * group;
  tm = first + r % gm;
  tn = r / gm;
}

template <int BM, int BN, int WM, int WN, int KIND>
__global__ __launch_bounds__(kThreads) void fp8_gemm_kernel(const Params p) {
  constexpr int WTM = BM / WM;   // wave tile rows
  constexpr int WTN = BN / WN;   // wave tile columns
  constexpr int FM = WTM / 16;   // 16-row fragments per wave
  constexpr int FN = WTN / 16;   // 16-column fragments per wave
  constexpr bool kRowScaleB = (KIND == KIND_WGRAD || KIND == KIND_KGROUPED);
  constexpr bool kFp32Out = kRowScaleB;
  // the columns of one wave tile sit inside one 128-block: one sb per wave
  constexpr bool kWaveUniformSb = !kRowScaleB && (kBK % WTN == 0) && (BN % WTN == 0);
  static_assert(WM * WN == 4, "4 waves per workgroup");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile is a multiple of 16");
  constexpr int A_CH = BM * 8;  // 16-byte chunks per stage
  constexpr int B_CH = BN * 8;
  constexpr int A_PT = (A_CH + kThreads - 1) / kThreads;
  constexpr int B_PT = (B_CH + kThreads - 1) / kThreads;

  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * kBK];
  __shared__ float sSA[2][BM];
  __shared__ float sSB[2][BN];
  __shared__ int sRowOk[KIND == KIND_CONTIGUOUS ? BM : 1];
  __shared__ int sExpert;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int l16 = lane & 15;
  const int lq = lane >> 4;

  // ---- tile count (masked: from masked_m on the device, no host sync) ----
  int T = p.tiles;
  if constexpr (KIND == KIND_MASKED) {
    T = 0;
    for (int g = 0; g < p.groups; ++g) {
      int v = min(max(p.ctrl[g], 0), p.m);
      T += ((v + BM - 1) / BM) * p.tiles_n;
    }
  }
  const int per_xcd = (T + 7) >> 3;

  for (int t = blockIdx.x; t < per_xcd * 8; t += gridDim.x) {
    const int L = (t & 7) * per_xcd + (t >> 3);
    if (L >= T) continue;

    // ---- decode tile ----
    TileInfo ti;
    ti.kb0 = 0;
    ti.kb1 = p.kbs;
    if constexpr (KIND == KIND_MASKED) {
      int rem = L, g = 0, mt = 0, v = 0;
      for (; g < p.groups; ++g) {
        v = min(max(p.ctrl[g], 0), p.m);
        mt = (v + BM - 1) / BM;
        const int cnt = mt * p.tiles_n;
        if (rem < cnt) break;
        rem -= cnt;
      }
      if (g >= p.groups) continue;  // unreachable for L < T
      ti.g = g;
      ti.m0 = (rem % mt) * BM;   // m fastest: tiles sharing a B tile run together
      ti.n0 = (rem / mt) * BN;
      ti.rows = min(BM, v - ti.m0);
      ti.a_row0 = (int64_t)g * p.m + ti.m0;
      ti.out_row0 = ti.a_row0;
    } else if constexpr (KIND == KIND_KGROUPED) {
      const int per_g = p.tiles_m * p.tiles_n;
      const int g = L / per_g;
      int tm, tn;
      raster<BM>(L - g * per_g, p.tiles_m, p.tiles_n, tm, tn);
      ti.g = g;
      ti.m0 = tm * BM;
      ti.n0 = tn * BN;
      ti.rows = min(BM, p.m - ti.m0);
      ti.kb0 = p.kb_begin[g];
      ti.kb1 = p.kb_begin[g + 1];
      ti.a_row0 = ti.m0;
      ti.out_row0 = (int64_t)g * p.m + ti.m0;
    } else {
      int tm, tn;
      raster<BM>(L, p.tiles_m, p.tiles_n, tm, tn);
      ti.g = 0;
      ti.m0 = tm * BM;
      ti.n0 = tn * BN;
      ti.rows = min(BM, p.m - ti.m0);
      ti.a_row0 = ti.m0;
      ti.out_row0 = ti.m0;
    }
    if (ti.kb0 >= ti.kb1) continue;  // empty K range: D unchanged

    if constexpr (KIND == KIND_CONTIGUOUS) {
      // expert of this 128-aligned row block: the (single) valid id in it
      __syncthreads();  // previous tile's epilogue is done with sRowOk
      if (tid == 0) sExpert = -1;
      __syncthreads();
      for (int r = tid; r < BM; r += kThreads) {
        const int id = p.ctrl[ti.m0 + r];
        if (id >= 0 && id < p.groups) atomicMax(&sExpert, id);
      }
      __syncthreads();
      const int e = sExpert;
      for (int r = tid; r < BM; r += kThreads) sRowOk[r] = (p.ctrl[ti.m0 + r] == e);
      if (e < 0) continue;  // block-uniform: all padding
      ti.g = e;
    }

    const uint8_t* gA = p.a + ti.a_row0 * (int64_t)p.lda;
    const float* gSA = p.sa + ti.a_row0 * (int64_t)p.kbs;
    // K-grouped weight gradients share one B [N,T]; the group picks the K range
    const int bg = (KIND == KIND_KGROUPED) ? 0 : ti.g;
    const uint8_t* gB = p.b + ((int64_t)bg * p.n + ti.n0) * (int64_t)p.lda;
    const int nb_rows = (p.n + kBK - 1) / kBK;
    const int a_last = max(ti.rows, 1) - 1;     // clamp rows beyond the valid ones
    const int b_last = min(BN, p.n - ti.n0) - 1;

    uint4 ra[A_PT], rb[B_PT];
    float rsa[(BM + kThreads - 1) / kThreads], rsb[(BN + kThreads - 1) / kThreads];

    auto load_stage = [&](int kb) {
#pragma unroll
      for (int q = 0; q < A_PT; ++q) {
        const int c = tid + q * kThreads;
        if (A_CH % kThreads == 0 || c < A_CH) {
          const int row = min(c >> 3, a_last);
          ra[q] = *reinterpret_cast<const uint4*>(gA + (int64_t)row * p.lda + kb * kBK + (c & 7) * 16);
        }
      }
#pragma unroll
      for (int q = 0; q < B_PT; ++q) {
        const int c = tid + q * kThreads;
        if (B_CH % kThreads == 0 || c < B_CH) {
          const int row = min(c >> 3, b_last);
          rb[q] = *reinterpret_cast<const uint4*>(gB + (int64_t)row * p.lda + kb * kBK + (c & 7) * 16);
        }
      }
#pragma unroll
      for (int q = 0; q < (BM + kThreads - 1) / kThreads; ++q) {
        const int r = tid + q * kThreads;
        if (r < BM) rsa[q] = gSA[(int64_t)min(r, a_last) * p.kbs + kb];
      }
#pragma unroll
      for (int q = 0; q < (BN + kThreads - 1) / kThreads; ++q) {
        const int c = tid + q * kThreads;
        if (c < BN) {
          const int n = ti.n0 + min(c, b_last);
          if constexpr (kRowScaleB)
            rsb[q] = p.sb[(int64_t)n * p.kbs + kb];
          else
            rsb[q] = p.sb[((int64_t)ti.g * nb_rows + n / kBK) * p.kbs + kb];
        }
      }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
      for (int q = 0; q < A_PT; ++q) {
        const int c = tid + q * kThreads;
        if (A_CH % kThreads == 0 || c < A_CH) {
          const int row = c >> 3;
          *reinterpret_cast<uint4*>(&sA[buf][row * kBK + (((c & 7) ^ swz(row)) << 4)]) = ra[q];
        }
      }
#pragma unroll
      for (int q = 0; q < B_PT; ++q) {
        const int c = tid + q * kThreads;
        if (B_CH % kThreads == 0 || c < B_CH) {
          const int row = c >> 3;
          *reinterpret_cast<uint4*>(&sB[buf][row * kBK + (((c & 7) ^ swz(row)) << 4)]) = rb[q];
        }
      }
#pragma unroll
      for (int q = 0; q < (BM + kThreads - 1) / kThreads; ++q) {
        const int r = tid + q * kThreads;
        if (r < BM) sSA[buf][r] = rsa[q];
      }
#pragma unroll
      for (int q = 0; q < (BN + kThreads - 1) / kThreads; ++q) {
        const int c = tid + q * kThreads;
        if (c < BN) sSB[buf][c] = rsb[q];
      }
    };

    v4f acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    load_stage(ti.kb0);
    store_stage(0);
    __syncthreads();

    for (int kb = ti.kb0; kb < ti.kb1; ++kb) {
      const int cur = (kb - ti.kb0) & 1;
      const bool more = kb + 1 < ti.kb1;
      if (more) load_stage(kb + 1);

      // fragments: lane (l16, lq) takes row l16 of a 16-row slice and the
      // 32 bytes [32*lq, 32*lq+32) of the K block.  Both operands use the
      // same (lane, byte) -> k assignment, so the MFMA sums exactly the 128
      // products of the block.
      v8i bfr[FN], afr[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int row = wn * WTN + 16 * i + l16;
        const uint8_t* base = &sB[cur][row * kBK];
        const uint4 lo = *reinterpret_cast<const uint4*>(base + (((2 * lq) ^ swz(row)) << 4));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + (((2 * lq + 1) ^ swz(row)) << 4));
        bfr[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int row = wm * WTM + 16 * j + l16;
        const uint8_t* base = &sA[cur][row * kBK];
        const uint4 lo = *reinterpret_cast<const uint4*>(base + (((2 * lq) ^ swz(row)) << 4));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + (((2 * lq + 1) ^ swz(row)) << 4));
        afr[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      float sav[FM];
#pragma unroll
      for (int j = 0; j < FM; ++j) sav[j] = sSA[cur][wm * WTM + 16 * j + l16];

      if constexpr (kWaveUniformSb) {
        const float sbw = sSB[cur][wn * WTN];
        float s[FM];
#pragma unroll
        for (int j = 0; j < FM; ++j) s[j] = sav[j] * sbw;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
          for (int j = 0; j < FM; ++j) {
            const v4f pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                bfr[i], afr[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(s[j], pr[r], acc[i][j][r]);
          }
      } else if constexpr (!kRowScaleB) {
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const float sbi = sSB[cur][wn * WTN + 16 * i];
#pragma unroll
          for (int j = 0; j < FM; ++j) {
            const v4f pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                bfr[i], afr[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
            const float s = sav[j] * sbi;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(s, pr[r], acc[i][j][r]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          float sbr[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) sbr[r] = sSB[cur][wn * WTN + 16 * i + 4 * lq + r];
#pragma unroll
          for (int j = 0; j < FM; ++j) {
            const v4f pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                bfr[i], afr[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[i][j][r] = __builtin_fmaf(sav[j] * sbr[r], pr[r], acc[i][j][r]);
          }
        }
      }

      if (more) store_stage(cur ^ 1);
      __syncthreads();
    }

    // ---- epilogue ----
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int ml = wm * WTM + 16 * j + l16;
      bool row_ok;
      if constexpr (KIND == KIND_CONTIGUOUS)
        row_ok = sRowOk[ml] != 0;
      else
        row_ok = ml < ti.rows;
      if (!row_ok) continue;
      const int64_t orow = ti.out_row0 + ml;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int n = ti.n0 + wn * WTN + 16 * i + 4 * lq;
        if (n >= p.n) continue;
        if constexpr (kFp32Out) {
          float* d = static_cast<float*>(p.out) + orow * p.n + n;
          if (p.vec_out && n + 3 < p.n) {
            float4 v = *reinterpret_cast<float4*>(d);
            v.x += acc[i][j][0];
            v.y += acc[i][j][1];
            v.z += acc[i][j][2];
            v.w += acc[i][j][3];
            *reinterpret_cast<float4*>(d) = v;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < p.n) d[r] += acc[i][j][r];
          }
        } else {
          uint16_t* c = static_cast<uint16_t*>(p.out) + orow * p.n + n;
          if (p.vec_out && n + 3 < p.n) {
            const uint32_t lo = (uint32_t)f32_to_bf16(acc[i][j][0]) | ((uint32_t)f32_to_bf16(acc[i][j][1]) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16(acc[i][j][2]) | ((uint32_t)f32_to_bf16(acc[i][j][3]) << 16);
            *reinterpret_cast<uint2*>(c) = uint2{lo, hi};
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < p.n) c[r] = f32_to_bf16(acc[i][j][r]);
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_shape(int kind, const Params& p, int grid, hipStream_t stream) {
  dim3 g(grid), b(kThreads);
  switch (kind) {
    case KIND_DENSE:
      hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, WM, WN, KIND_DENSE>), g, b, 0, stream, p);
      break;
    case KIND_CONTIGUOUS:
      hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, WM, WN, KIND_CONTIGUOUS>), g, b, 0, stream, p);
      break;
    case KIND_MASKED:
      hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, WM, WN, KIND_MASKED>), g, b, 0, stream, p);
      break;
    case KIND_WGRAD:
      hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, WM, WN, KIND_WGRAD>), g, b, 0, stream, p);
      break;
    case KIND_KGROUPED:
      hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, WM, WN, KIND_KGROUPED>), g, b, 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

#define DG_SHAPES(X) \
  X(128, 128, 2, 2)  \
  X(128, 64, 2, 2)   \
  X(64, 128, 1, 4)   \
  X(64, 64, 1, 4)    \
  X(64, 32, 2, 2)

}  // namespace

bool has_instance(int kind, const TileShape& s) {
  if (kind < KIND_DENSE || kind > KIND_KGROUPED) return false;
#define X(BM, BN, WM, WN) \
  if (s.bm == BM && s.bn == BN && s.wm == WM && s.wn == WN) return true;
  DG_SHAPES(X)
#undef X
  return false;
}

hipError_t launch(int kind, const TileShape& s, const Params& p, int grid, hipStream_t stream) {
#define X(BM, BN, WM, WN) \
  if (s.bm == BM && s.bn == BN && s.wm == WM && s.wn == WN) return launch_shape<BM, BN, WM, WN>(kind, p, grid, stream);
  DG_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace dg
