// dg_kernels.hip -- FP8 (e4m3) fine-grained-scaled NT GEMM kernels for gfx950.
//
// One kernel template serves every layout (DeepGEMM pages, "简洁的代码设计":
// a single core GEMM kernel); the layouts differ only in how a tile id maps
// to (group, rows, columns, K range) and in the epilogue.
//
// Per workgroup tile (BM x BN outputs, WM x WN waves of 64 lanes):
//   * operands and their scales move HBM -> LDS with the gfx950 LDS-DMA loads
//     (global_load_lds_dwordx4 / _dword): no staging registers, and the loads
//     for the next S-1 K blocks stay in flight while the current one is
//     multiplied (an S-stage ring, one barrier per 128-wide K block).  The
//     DMA writes each wave's 1 KB piece contiguously, so the XOR bank swizzle
//     is applied on the global side: the lane that lands on LDS chunk c of row
//     r fetches logical chunk c ^ swz(r);
//   * each 16x16 output subtile of a K block is one v_mfma_f32_16x16x128_f8f6f4
//     with a zero accumulator: the exact fp32 block partial (DeepGEMM pages,
//     "主要特点": tensor-core FP8 accumulation alone is imprecise);
//   * the partial is promoted into the fp32 main accumulator with one VALU
//     FMA by sa[m,kb]*sb[n/128,kb] (the pages' two-level accumulation); the
//     promotion of one fragment group is placed after the MFMAs of the next,
//     so the vector unit works while the matrix unit is busy;
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

constexpr int kBK = 128;      // K block = scale granularity
constexpr int kGroupM = 8;    // tile rows per raster group

// LDS row = 128 bytes = 8 chunks of 16 bytes; logical chunk c of row r sits
// at chunk position c ^ swz(r).  A 16-lane phase of ds_read_b128 reads one
// chunk from each of 16 consecutive rows; the swizzle spreads them over all
// banks for both a 32-bank (8 rows per phase) and a 64-bank (16 rows) view.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 h = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

__device__ __forceinline__ const uint8_t* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(((uint64_t)hi << 32) | lo);
}

// LDS DMA.  Lane i's bytes go to LDS address m0 + i*size.  Issued through
// inline asm so the compiler's wait-count pass does not treat every later
// LDS read as dependent on every in-flight DMA; the waits are explicit below.
// Nothing else in these kernels uses m0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(uint32_t lds, const uint8_t* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t lds, const uint8_t* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that also orders LDS accesses for the compiler.
__device__ __forceinline__ void barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void raster(int L, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group = kGroupM * tiles_n;
  const int gid = L / group;
  const int first = gid * kGroupM;
  const int gm = min(tiles_m - first, kGroupM);
  const int r = L - gid * group;
  tm = first + r % gm;
  tn = r / gm;
}

__device__ __forceinline__ v8i load_frag(const uint8_t* tile, int row, int lq) {
  const uint8_t* base = tile + row * kBK;
  const uint4 lo = *reinterpret_cast<const uint4*>(base + (((2 * lq) ^ swz(row)) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(base + (((2 * lq + 1) ^ swz(row)) << 4));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__device__ __forceinline__ v4f mfma_block(const v8i& b_rows, const v8i& a_rows) {
  // D[n][m] = sum over the 128 k of the block; both operands use the same
  // (lane, byte) -> k assignment, so the sum covers exactly the block.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b_rows, a_rows, v4f{0.f, 0.f, 0.f, 0.f},
                                                          0, 0, 0, 0, 0, 0);
}

template <int BM, int BN, int WM, int WN, int S, int KIND>
__global__ __launch_bounds__(WM * WN * 64) void fp8_gemm_kernel(const Params p) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM;   // wave tile rows
  constexpr int WTN = BN / WN;   // wave tile columns
  constexpr int FM = WTM / 16;   // 16-row fragments per wave
  constexpr int FN = WTN / 16;   // 16-column fragments per wave
  constexpr bool kRowScaleB = (KIND == KIND_WGRAD || KIND == KIND_KGROUPED);
  constexpr bool kFp32Out = kRowScaleB;
  // the columns of one wave tile sit inside one 128-block: one sb per wave
  constexpr bool kWaveUniformSb = !kRowScaleB && (kBK % WTN == 0) && (BN % WTN == 0);
  constexpr bool kStreamM = FM >= FN;  // keep the smaller fragment set resident
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile is a multiple of 16");
  static_assert(S >= 2, "at least double buffering");

  // ---- LDS stage layout and DMA pieces ----
  constexpr int SA_N = ((BM + 63) / 64) * 64;                   // floats
  constexpr int SB_N = kRowScaleB ? ((BN + 63) / 64) * 64 : 64;  // floats
  constexpr int OFF_A = 0;
  constexpr int OFF_B = BM * kBK;
  constexpr int OFF_SA = OFF_B + BN * kBK;
  constexpr int OFF_SB = OFF_SA + SA_N * 4;
  constexpr int STAGE = OFF_SB + SB_N * 4;
  constexpr int PA = BM / 8, PB = BN / 8, PSA = SA_N / 64, PSB = SB_N / 64;  // pieces
  constexpr int P = PA + PB + PSA + PSB;
  constexpr int DMAX = (P + NW - 1) / NW;  // pieces per wave (some waves one fewer)
  constexpr int DMIN = P / NW;
  static_assert(BM % 8 == 0 && BN % 8 == 0, "1 KB DMA pieces");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];
  __shared__ int sRowOk[KIND == KIND_CONTIGUOUS ? BM : 1];
  __shared__ int sExpert;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int l16 = lane & 15;
  const int lq = lane >> 4;
  const uint32_t smem_lds = lds_addr(smem);

  // ---- tile count (masked: from masked_m on the device, no host sync) ----
  int T = p.tiles;
  if constexpr (KIND == KIND_MASKED) {
    T = 0;
    for (int g = 0; g < p.groups; ++g) {
      const int v = min(max(p.ctrl[g], 0), p.m);
      T += ((v + BM - 1) / BM) * p.tiles_n;
    }
  }
  const int per_xcd = (T + 7) >> 3;
  const int nb_rows = (p.n + kBK - 1) / kBK;

  for (int t = blockIdx.x; t < per_xcd * 8; t += gridDim.x) {
    const int L = (t & 7) * per_xcd + (t >> 3);
    if (L >= T) continue;

    // ---- decode tile ----
    int g = 0, m0, n0, rows, kb0 = 0, kb1 = p.kbs;
    int64_t a_row0, out_row0;
    if constexpr (KIND == KIND_MASKED) {
      int rem = L, mt = 0, v = 0;
      for (; g < p.groups; ++g) {
        v = min(max(p.ctrl[g], 0), p.m);
        mt = (v + BM - 1) / BM;
        const int cnt = mt * p.tiles_n;
        if (rem < cnt) break;
        rem -= cnt;
      }
      if (g >= p.groups) continue;  // unreachable for L < T
      m0 = (rem % mt) * BM;        // m fastest: tiles sharing a B tile run together
      n0 = (rem / mt) * BN;
      rows = min(BM, v - m0);
      a_row0 = (int64_t)g * p.m + m0;
      out_row0 = a_row0;
    } else if constexpr (KIND == KIND_KGROUPED) {
      const int per_g = p.tiles_m * p.tiles_n;
      g = L / per_g;
      int tm, tn;
      raster(L - g * per_g, p.tiles_m, p.tiles_n, tm, tn);
      m0 = tm * BM;
      n0 = tn * BN;
      rows = min(BM, p.m - m0);
      kb0 = p.kb_begin[g];
      kb1 = p.kb_begin[g + 1];
      a_row0 = m0;
      out_row0 = (int64_t)g * p.m + m0;
    } else {
      int tm, tn;
      raster(L, p.tiles_m, p.tiles_n, tm, tn);
      m0 = tm * BM;
      n0 = tn * BN;
      rows = min(BM, p.m - m0);
      a_row0 = m0;
      out_row0 = m0;
    }
    const int nkb = kb1 - kb0;
    if (nkb <= 0) continue;  // empty K range: D unchanged

    if constexpr (KIND == KIND_CONTIGUOUS) {
      // expert of this 128-aligned row block: the (single) valid id in it
      barrier();  // previous tile's epilogue is done with sRowOk
      if (tid == 0) sExpert = -1;
      barrier();
      for (int r = tid; r < BM; r += NW * 64) {
        const int id = p.ctrl[m0 + r];
        if (id >= 0 && id < p.groups) atomicMax(&sExpert, id);
      }
      barrier();
      const int e = sExpert;
      for (int r = tid; r < BM; r += NW * 64) sRowOk[r] = (p.ctrl[m0 + r] == e);
      if (e < 0) continue;  // block-uniform: all padding
      g = e;
    }

    // ---- per-tile DMA addressing ----
    // K-grouped weight gradients share one B [N,T]; the group picks the K range
    const int bg = (KIND == KIND_KGROUPED) ? 0 : g;
    const uint8_t* gA = uniform_ptr(p.a + a_row0 * (int64_t)p.lda);
    const uint8_t* gB = uniform_ptr(p.b + ((int64_t)bg * p.n + n0) * (int64_t)p.lda);
    const uint8_t* gSA = uniform_ptr(p.sa + a_row0 * (int64_t)p.kbs);
    const uint8_t* gSB = kRowScaleB ? uniform_ptr(p.sb + (int64_t)n0 * p.kbs)
                                    : uniform_ptr(p.sb + (int64_t)g * nb_rows * p.kbs);
    const int a_last = max(rows, 1) - 1;       // rows past the valid ones re-read the last
    const int b_last = min(BN, p.n - n0) - 1;
    uint32_t voff[DMAX];
#pragma unroll
    for (int q = 0; q < DMAX; ++q) {
      const int pc = wave + NW * q;
      uint32_t v = 0;
      if (pc < PA) {
        const int r = pc * 8 + (lane >> 3);
        v = (uint32_t)min(r, a_last) * p.lda + (((lane & 7) ^ swz(r)) << 4);
      } else if (pc < PA + PB) {
        const int r = (pc - PA) * 8 + (lane >> 3);
        v = (uint32_t)min(r, b_last) * p.lda + (((lane & 7) ^ swz(r)) << 4);
      } else if (pc < PA + PB + PSA) {
        const int r = (pc - PA - PB) * 64 + lane;
        v = (uint32_t)min(r, a_last) * p.kbs * 4;
      } else if (pc < P) {
        if constexpr (kRowScaleB) {
          const int c = (pc - PA - PB - PSA) * 64 + lane;
          v = (uint32_t)min(c, b_last) * p.kbs * 4;
        } else {
          const int nb = min(n0 / kBK + lane, nb_rows - 1);
          v = (uint32_t)nb * p.kbs * 4;
        }
      }
      voff[q] = v;
    }
    // this wave's DMAs for K block kb0 + rel into ring stage `st`
    auto issue = [&](int rel, int st) {
      const int kb = kb0 + rel;
      const uint32_t base = smem_lds + st * STAGE;
#pragma unroll
      for (int q = 0; q < DMAX; ++q) {
        const int pc = wave + NW * q;
        if (pc < PA)
          dma16(base + OFF_A + pc * 1024, gA + kb * kBK, voff[q]);
        else if (pc < PA + PB)
          dma16(base + OFF_B + (pc - PA) * 1024, gB + kb * kBK, voff[q]);
        else if (pc < PA + PB + PSA)
          dma4(base + OFF_SA + (pc - PA - PB) * 256, gSA + kb * 4, voff[q]);
        else if (pc < P)
          dma4(base + OFF_SB + (pc - PA - PB - PSA) * 256, gSB + kb * 4, voff[q]);
      }
    };

    v4f acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // prologue: the first S-1 K blocks in flight
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < nkb) issue(s, s);

    for (int rel = 0; rel < nkb; ++rel) {
      const int st = rel % S;
      // this wave's DMAs for block `rel` are done once at most
      // (blocks issued after it) x DMIN of its operations remain in flight
      const int later = min(S - 2, nkb - 1 - rel);
      if constexpr (S == 2) {
        wait_vm<0>();
      } else if constexpr (S == 3) {
        if (later >= 1) wait_vm<DMIN>(); else wait_vm<0>();
      } else {
        static_assert(S == 4, "ring depth 2..4");
        if (later >= 2) wait_vm<2 * DMIN>(); else if (later == 1) wait_vm<DMIN>(); else wait_vm<0>();
      }
      barrier();  // every wave's block `rel` landed; every wave is done with rel-1
      if (rel + S - 1 < nkb) issue(rel + S - 1, (rel + S - 1) % S);

      const uint8_t* sA = smem + st * STAGE + OFF_A;
      const uint8_t* sB = smem + st * STAGE + OFF_B;
      const float* sSA = reinterpret_cast<const float*>(smem + st * STAGE + OFF_SA);
      const float* sSB = reinterpret_cast<const float*>(smem + st * STAGE + OFF_SB);

      float sav[FM];
#pragma unroll
      for (int j = 0; j < FM; ++j) sav[j] = sSA[wm * WTM + 16 * j + l16];
      // per n-fragment B scale (block scales) or per column quad (row scales)
      float sbv[FN];
      v4f sbq[kRowScaleB ? FN : 1];
      if constexpr (kRowScaleB) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
          sbq[i] = *reinterpret_cast<const v4f*>(&sSB[wn * WTN + 16 * i + 4 * lq]);
      } else if constexpr (kWaveUniformSb) {
        const float s = sSB[(n0 + wn * WTN) / kBK - n0 / kBK];
#pragma unroll
        for (int i = 0; i < FN; ++i) sbv[i] = s;
      } else {
#pragma unroll
        for (int i = 0; i < FN; ++i) sbv[i] = sSB[(n0 + wn * WTN + 16 * i) / kBK - n0 / kBK];
      }

      auto promote = [&](int i, int j, const v4f& pr) {
        if constexpr (kRowScaleB) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(sav[j] * sbq[i][r], pr[r], acc[i][j][r]);
        } else {
          const float s = sav[j] * sbv[i];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(s, pr[r], acc[i][j][r]);
        }
      };

      if constexpr (kStreamM) {
        // resident: the FN column fragments; streamed: the FM row fragments
        v8i bres[FN];
#pragma unroll
        for (int i = 0; i < FN; ++i) bres[i] = load_frag(sB, wn * WTN + 16 * i + l16, lq);
        v8i acur = load_frag(sA, wm * WTM + l16, lq);
        v4f part[2][FN];
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          v8i anext = acur;
          if (j + 1 < FM) anext = load_frag(sA, wm * WTM + 16 * (j + 1) + l16, lq);
#pragma unroll
          for (int i = 0; i < FN; ++i) part[j & 1][i] = mfma_block(bres[i], acur);
          if (j > 0) {
#pragma unroll
            for (int i = 0; i < FN; ++i) promote(i, j - 1, part[(j - 1) & 1][i]);
          }
          acur = anext;
        }
#pragma unroll
        for (int i = 0; i < FN; ++i) promote(i, FM - 1, part[(FM - 1) & 1][i]);
      } else {
        // resident: the FM row fragments; streamed: the FN column fragments
        v8i ares[FM];
#pragma unroll
        for (int j = 0; j < FM; ++j) ares[j] = load_frag(sA, wm * WTM + 16 * j + l16, lq);
        v8i bcur = load_frag(sB, wn * WTN + l16, lq);
        v4f part[2][FM];
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          v8i bnext = bcur;
          if (i + 1 < FN) bnext = load_frag(sB, wn * WTN + 16 * (i + 1) + l16, lq);
#pragma unroll
          for (int j = 0; j < FM; ++j) part[i & 1][j] = mfma_block(bcur, ares[j]);
          if (i > 0) {
#pragma unroll
            for (int j = 0; j < FM; ++j) promote(i - 1, j, part[(i - 1) & 1][j]);
          }
          bcur = bnext;
        }
#pragma unroll
        for (int j = 0; j < FM; ++j) promote(FN - 1, j, part[(FN - 1) & 1][j]);
      }
    }
    barrier();  // all waves are done with the ring before the next tile refills it

    // ---- epilogue ----
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int ml = wm * WTM + 16 * j + l16;
      bool row_ok;
      if constexpr (KIND == KIND_CONTIGUOUS)
        row_ok = sRowOk[ml] != 0;
      else
        row_ok = ml < rows;
      if (!row_ok) continue;
      const int64_t orow = out_row0 + ml;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int n = n0 + wn * WTN + 16 * i + 4 * lq;
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

template <int BM, int BN, int WM, int WN, int S>
hipError_t launch_shape(int kind, const Params& p, int grid, hipStream_t stream) {
  dim3 g(grid), b(WM * WN * 64);
  switch (kind) {
    case KIND_DENSE:
      hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, WM, WN, S, KIND_DENSE>), g, b, 0, stream, p);
      break;
    case KIND_CONTIGUOUS:
      hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, WM, WN, S, KIND_CONTIGUOUS>), g, b, 0, stream, p);
      break;
    case KIND_MASKED:
      hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, WM, WN, S, KIND_MASKED>), g, b, 0, stream, p);
      break;
    case KIND_WGRAD:
      hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, WM, WN, S, KIND_WGRAD>), g, b, 0, stream, p);
      break;
    case KIND_KGROUPED:
      hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, WM, WN, S, KIND_KGROUPED>), g, b, 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// (BM, BN, waves along M, waves along N, LDS ring stages)
#define DG_SHAPES(X)      \
  X(256, 128, 2, 2, 3)    \
  X(256, 256, 2, 4, 2)    \
  X(128, 128, 2, 2, 4)    \
  X(128, 64, 2, 2, 4)     \
  X(64, 128, 1, 4, 4)     \
  X(64, 64, 1, 4, 4)      \
  X(64, 32, 2, 2, 4)

}  // namespace

bool has_instance(int kind, const TileShape& s) {
  if (kind < KIND_DENSE || kind > KIND_KGROUPED) return false;
#define X(BM, BN, WM, WN, S) \
  if (s.bm == BM && s.bn == BN && s.wm == WM && s.wn == WN) return true;
  DG_SHAPES(X)
#undef X
  return false;
}

int threads_of(const TileShape& s) { return s.wm * s.wn * 64; }

int lds_bytes_of(int kind, const TileShape& s) {
  const bool row_sb = (kind == KIND_WGRAD || kind == KIND_KGROUPED);
  const int sa_n = ((s.bm + 63) / 64) * 64;
  const int sb_n = row_sb ? ((s.bn + 63) / 64) * 64 : 64;
  const int stage = (s.bm + s.bn) * kBK + 4 * (sa_n + sb_n);
#define X(BM, BN, WM, WN, S) \
  if (s.bm == BM && s.bn == BN && s.wm == WM && s.wn == WN) return S * stage + 4 * BM + 64;
  DG_SHAPES(X)
#undef X
  return 0;
}

hipError_t launch(int kind, const TileShape& s, const Params& p, int grid, hipStream_t stream) {
#define X(BM, BN, WM, WN, S) \
  if (s.bm == BM && s.bn == BN && s.wm == WM && s.wn == WN) return launch_shape<BM, BN, WM, WN, S>(kind, p, grid, stream);
  DG_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace dg
