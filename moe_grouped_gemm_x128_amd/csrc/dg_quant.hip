// dg_quant.hip -- FP8 (e4m3) quantiser with fine-grained fp32 scales for
// gfx950: it makes the GEMM's operands.
//
// The DeepGEMM pages (DeepSeek DeepGEMM 中文讲解, "注意事项") ask for dynamic
// scale factors from amax; their usage example ("使用示例") fixes the
// granularity: one fp32 scale per row and 128-wide K group for activations
// ([M, K/128]) and one per 128x128 block for weights ([ceil(N/128), K/128]).
// Per group:
//   amax = max |x|,  s = amax / 448 (1 for an all-zero group),
//   q    = e4m3 nearest-even( clamp(x / s, -448, 448) )
// with both divisions equal to IEEE fp32 division (round to nearest even),
// so the codes match a scalar fp32 evaluation bit for bit.
//
// The work is a stream (4 bytes read, 1 byte + a few scale bytes written per
// element), bound by HBM; every input byte is read from HBM once, and each
// thread keeps its values in registers until its group's amax is known.
//   * 1x128 (x [M, K]): the groups are consecutive 512-byte runs of the flat
//     array, so each wave streams 16 consecutive groups (8 KB) per step and
//     the 32 lanes of a group reduce its amax by lane shuffles;
//   * 128x128 and 1x128 transposed: one 512-thread workgroup owns a 128 x 128
//     tile; thread t loads float4 number t of each of the tile's 8 strips of
//     16 rows (32 lanes cover one 512-byte row segment).  128x128: amax over
//     the tile (wave shuffles, then 8 waves through LDS).  Transposed (x [T, F]
//     -> q [F, T], s [F, T/128], the token-contiguous operands of the weight-
//     gradient GEMM): amax per column over the tile's 128 rows (in-thread, lane
//     l with l + 32, then 8 waves through LDS), and the codes are transposed
//     through an LDS byte tile so each store writes 16 consecutive tokens of
//     one feature.
// The quotient x / s is computed without a full division per element (see
// quotient()): one division per group for RN(1/s), then multiplies and FMAs
// that reproduce the IEEE quotient bit for bit.
#include "dg_fp8_codec.h"
#include "dg_kernel.h"

namespace dg {
namespace {

constexpr int kQ = 128;          // group / tile edge
constexpr int kQThreads = 512;   // 8 waves
constexpr int kQStrips = 8;      // float4 loads per thread: 128 rows x 32 float4 / 512
using codec::kE4m3Max;
using codec::scale_of;
using codec::encode4;
using codec::silu;

enum QuantMode : int { Q_ROWS = 0, Q_BLOCKS = 1, Q_TRANSPOSED = 2, Q_ROWS_UE8M0 = 3, Q_BLOCKS_UE8M0 = 4 };

// Power-of-two (UE8M0) scales (DeepGEMM pages, aikraft.ru support table:
// packed UE8M0, four values in one torch.int): a group's scale is the
// smallest 2^(E - 127), E in [0, 254], not below s0 = scale_of(amax), read off
// s0's fp32 fields -- an exact power keeps its exponent field, anything above
// it takes the next; a subnormal s0 is at most 2^-127 (E = 0, the field 0
// with mantissa 2^22) or below 2^-126 (E = 1).  The quotient by 2^(E - 127)
// is exact, so the codes are those of an exact division.  E goes to byte
// (group mod 4) of word group/4 of the row's packed words; a row's last group
// also zeroes the bytes past it.
__device__ __forceinline__ uint32_t ue8m0_code(float amax) {
  const uint32_t b = __float_as_uint(scale_of(amax));
  const uint32_t ex = b >> 23, man = b & 0x7fffffu;
  if (ex == 0) return man > 0x400000u ? 1u : 0u;
  return min(ex + (man != 0u ? 1u : 0u), 254u);
}
__device__ __forceinline__ float ue8m0_value(uint32_t e) {
  return __uint_as_float(e == 0 ? 0x400000u : e << 23);
}
// byte `g` of a row of `kw` packed words, plus the row's padding bytes when g
// is its last group
__device__ __forceinline__ void put_code(uint8_t* row_bytes, int g, int groups, int kw, uint32_t e) {
  row_bytes[g] = (uint8_t)e;
  if (g == groups - 1)
    for (int p = groups; p < 4 * kw; ++p) row_bytes[p] = 0;
}


// x / s, equal to the IEEE fp32 quotient: y0 = x * RN(1/s), then two
// residual corrections y += RN(1/s) * (x - y*s) with the residual exact in an
// FMA (Markstein's scheme).  A group whose scale is below 2^-60 is first
// rescaled by 2^64 (x and s alike, exactly) so the residuals stay in the
// normal range; the sign is copied from x so that -0 stays -0.
__device__ __forceinline__ float quotient(float x, float s) {
  const float k = s < 0x1p-60f ? 0x1p64f : 1.0f;
  x *= k;
  s *= k;
  const float r = 1.0f / s;
  float y = x * r;
  float e = __builtin_fmaf(-y, s, x);
  y = __builtin_fmaf(e, r, y);
  e = __builtin_fmaf(-y, s, x);
  y = __builtin_copysignf(__builtin_fmaf(e, r, y), x);
  return fminf(fmaxf(y, -kE4m3Max), kE4m3Max);
}

__device__ __forceinline__ float max_xor(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask, 64)); }
// Every byte is touched once: loads and stores carry the nontemporal
// (streaming) hint, so they do not displace other data in the caches
// (measured: 15% faster on [65536, 7168], 40% on [4096, 7168]).
typedef float f4nt __attribute__((ext_vector_type(4)));
typedef unsigned u4nt __attribute__((ext_vector_type(4)));
typedef unsigned u2nt __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float4 load_nt(const float* p) {
  const f4nt t = __builtin_nontemporal_load(reinterpret_cast<const f4nt*>(p));
  return float4{t[0], t[1], t[2], t[3]};
}

// 128 x 128 tiles: MODE is Q_BLOCKS, Q_BLOCKS_UE8M0 or Q_TRANSPOSED
template <int MODE>
__global__ __launch_bounds__(kQThreads) void quant_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                                                          float* __restrict__ s, int rows, int cols, int64_t tiles,
                                                          int col_tiles) {
  constexpr bool kUe8m0 = MODE == Q_BLOCKS_UE8M0;
  // Q_BLOCKS / Q_TRANSPOSED: per-wave partial maxima; Q_TRANSPOSED: byte tile
  __shared__ float sMax[8][kQ];
  __shared__ __attribute__((aligned(16))) uint8_t sT[MODE == Q_TRANSPOSED ? kQ : 1][kQ + 16];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int c4 = t & 31;       // float4 column of the thread in the tile
  const int rsub = t >> 5;     // row of the thread within each 16-row strip

  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int64_t tr = tile / col_tiles;
    const int tc = (int)(tile - tr * col_tiles);
    const int64_t r0 = tr * kQ;
    const int c0 = tc * kQ;
    const int col = c0 + 4 * c4;
    // load: strip i covers tile rows 16i .. 16i+15
    float4 v[kQStrips];
#pragma unroll
    for (int i = 0; i < kQStrips; ++i) {
      const int64_t r = r0 + 16 * i + rsub;
      const bool ok = r < rows && (MODE != Q_TRANSPOSED || col < cols);
      v[i] = ok ? load_nt(x + r * cols + col) : float4{0.f, 0.f, 0.f, 0.f};
    }
    auto amax4 = [](const float4& a) { return fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))); };

    if constexpr (MODE == Q_BLOCKS || MODE == Q_BLOCKS_UE8M0) {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < kQStrips; ++i) m = fmaxf(m, amax4(v[i]));
      m = max_xor(m, 32);
      m = max_xor(m, 16);
      m = max_xor(m, 8);
      m = max_xor(m, 4);
      m = max_xor(m, 2);
      m = max_xor(m, 1);
      __syncthreads();  // the previous tile's readers of sMax are done
      if (lane == 0) sMax[wave][0] = m;
      __syncthreads();
      float mm = sMax[0][0];
#pragma unroll
      for (int w = 1; w < 8; ++w) mm = fmaxf(mm, sMax[w][0]);
      float sc;
      if constexpr (kUe8m0) {
        const uint32_t e = ue8m0_code(mm);
        sc = ue8m0_value(e);
        const int kw = (col_tiles + 3) / 4;
        if (t == 0) put_code(reinterpret_cast<uint8_t*>(s) + tr * (4 * kw), tc, col_tiles, kw, e);
      } else {
        sc = scale_of(mm);
        if (t == 0) s[tr * col_tiles + tc] = sc;
      }
#pragma unroll
      for (int i = 0; i < kQStrips; ++i) {
        const int64_t r = r0 + 16 * i + rsub;
        if (r < rows)
          __builtin_nontemporal_store(
              encode4(quotient(v[i].x, sc), quotient(v[i].y, sc), quotient(v[i].z, sc), quotient(v[i].w, sc)),
              reinterpret_cast<uint32_t*>(q + r * cols + col));
      }
    } else {
      // columns are features, rows are tokens; groups run down a column
      float4 m = float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < kQStrips; ++i) {
        m.x = fmaxf(m.x, fabsf(v[i].x));
        m.y = fmaxf(m.y, fabsf(v[i].y));
        m.z = fmaxf(m.z, fabsf(v[i].z));
        m.w = fmaxf(m.w, fabsf(v[i].w));
      }
      m.x = max_xor(m.x, 32);
      m.y = max_xor(m.y, 32);
      m.z = max_xor(m.z, 32);
      m.w = max_xor(m.w, 32);
      __syncthreads();  // the previous tile's readers of sMax and sT are done
      if (lane < 32) *reinterpret_cast<float4*>(&sMax[wave][4 * c4]) = m;
      __syncthreads();
      float4 a = *reinterpret_cast<const float4*>(&sMax[0][4 * c4]);
#pragma unroll
      for (int w = 1; w < 8; ++w) {
        const float4 b = *reinterpret_cast<const float4*>(&sMax[w][4 * c4]);
        a.x = fmaxf(a.x, b.x);
        a.y = fmaxf(a.y, b.y);
        a.z = fmaxf(a.z, b.z);
        a.w = fmaxf(a.w, b.w);
      }
      const float sx = scale_of(a.x), sy = scale_of(a.y), sz = scale_of(a.z), sw = scale_of(a.w);
      const int kg = rows / kQ;  // token groups per feature
      if (t < 32) {
        const float sv[4] = {sx, sy, sz, sw};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (col + j < cols) s[(int64_t)(col + j) * kg + tr] = sv[j];
      }
      // codes into the byte tile [feature][token]
#pragma unroll
      for (int i = 0; i < kQStrips; ++i) {
        const uint32_t w = encode4(quotient(v[i].x, sx), quotient(v[i].y, sy), quotient(v[i].z, sz),
                                   quotient(v[i].w, sw));
        const int tok = 16 * i + rsub;
        sT[4 * c4 + 0][tok] = (uint8_t)(w & 0xffu);
        sT[4 * c4 + 1][tok] = (uint8_t)((w >> 8) & 0xffu);
        sT[4 * c4 + 2][tok] = (uint8_t)((w >> 16) & 0xffu);
        sT[4 * c4 + 3][tok] = (uint8_t)(w >> 24);
      }
      __syncthreads();
      // 8 lanes write one feature's 128 tokens (a whole 128-byte line)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int f = 64 * k + (t >> 3);
        const int ch = t & 7;
        if (c0 + f < cols)
          __builtin_nontemporal_store(*reinterpret_cast<const u4nt*>(&sT[f][16 * ch]),
                                      reinterpret_cast<u4nt*>(q + (int64_t)(c0 + f) * rows + r0 + 16 * ch));
      }
    }
  }
}

// 1x128 groups of a row-major [M, K] array (K % 128 == 0) are consecutive
// 512-byte runs of the flat array: each wave streams 16 consecutive groups
// (8 KB) per step, lane l holding float4 number l + 64j (group 2j + l/32).
// kUe8m0: power-of-two scales, packed (`gpr` groups per row).
template <bool kUe8m0>
__global__ __launch_bounds__(kQThreads) void quant_rows_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                                                               float* __restrict__ s, int64_t groups, int gpr) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (kQThreads / 64);
  const int64_t chunks = (groups + 15) / 16;
  for (int64_t c = (int64_t)blockIdx.x * (kQThreads / 64) + (threadIdx.x >> 6); c < chunks; c += waves) {
    const int64_t g0 = c * 16;
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t g = g0 + 2 * j + (lane >> 5);
      v[j] = g < groups ? load_nt(x + g0 * kQ + 256 * j + 4 * lane) : float4{0.f, 0.f, 0.f, 0.f};
    }
    // power-of-two scales whose rows have a multiple of 4 groups: the packed
    // codes have no padding, so the step's 16 groups are 16 consecutive bytes
    // -- written as 4 words by lanes 0-3 after the loop instead of 16 byte stores
    const bool whole = kUe8m0 && (gpr % 4 == 0) && g0 + 16 <= groups;
    uint32_t ecode[8];  // code of this lane's group in pass j
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float m = fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w)));
      m = max_xor(m, 16);
      m = max_xor(m, 8);
      m = max_xor(m, 4);
      m = max_xor(m, 2);
      m = max_xor(m, 1);
      const int64_t g = g0 + 2 * j + (lane >> 5);
      float sc;
      uint32_t e = 0;
      if constexpr (kUe8m0) {
        e = ue8m0_code(m);
        sc = ue8m0_value(e);
      } else {
        sc = scale_of(m);
      }
      ecode[j] = e;
      if (g < groups) {
        if ((lane & 31) == 0) {
          if constexpr (kUe8m0) {
            if (!whole) {
              const int64_t row = g / gpr;
              const int kw = (gpr + 3) / 4;
              put_code(reinterpret_cast<uint8_t*>(s) + row * (4 * kw), (int)(g - row * gpr), gpr, kw, e);
            }
          } else {
            s[g] = sc;
          }
        }
        __builtin_nontemporal_store(
            encode4(quotient(v[j].x, sc), quotient(v[j].y, sc), quotient(v[j].z, sc), quotient(v[j].w, sc)),
            reinterpret_cast<uint32_t*>(q + g0 * kQ + 256 * j + 4 * lane));
      }
    }
    if constexpr (kUe8m0) {
      // group 2j + h (h = lane / 32) of the step has code ecode[j] in lane
      // half h; word w holds groups 4w .. 4w + 3 = passes 2w, 2w + 1, both halves
      uint32_t other[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) other[j] = (uint32_t)__shfl_xor((int)ecode[j], 32, 64);
      uint32_t word = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo = lane < 32 ? ecode[2 * w] : other[2 * w];          // group 4w
        const uint32_t hi = lane < 32 ? other[2 * w] : ecode[2 * w];          // group 4w + 1
        const uint32_t lo2 = lane < 32 ? ecode[2 * w + 1] : other[2 * w + 1];  // group 4w + 2
        const uint32_t hi2 = lane < 32 ? other[2 * w + 1] : ecode[2 * w + 1];  // group 4w + 3
        const uint32_t vw = lo | (hi << 8) | (lo2 << 16) | (hi2 << 24);
        word = (lane == w) ? vw : word;
      }
      if (whole && lane < 4) reinterpret_cast<uint32_t*>(s)[(g0 >> 2) + lane] = word;
    }
  }
}

// ---- SwiGLU on the first linear's output, then the 1x128 rule ----------
// c [M, 2I] bf16 holds the gate projection in columns [0, I) and the up
// projection in [I, 2I); h = silu(gate) * up [M, I] is quantised in 1x128
// groups, which are consecutive 128-byte runs of the flat q [M, I].  16 lanes
// share a group, each with 8 gate and 8 up values (one 16-byte load of each),
// so a wave covers 4 groups per pass and 16 per step (16 KB in flight).
// Per element the work is about 20 VALU cycles (two of them transcendental
// at quarter rate), close to the ~24 per element that HBM speed allows.
// h carries the exp unit's error (a few fp32 ulp), so the quotient is
// h * RN(1/s) instead of the exact division of the plain quantiser: codes
// differ from exact evaluation only where h / s lies within a few ulp of a
// rounding midpoint between two e4m3 values.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__global__ __launch_bounds__(kQThreads) void swiglu_quant_kernel(const uint16_t* __restrict__ c,
                                                                 uint8_t* __restrict__ q, float* __restrict__ s,
                                                                 int64_t groups, int64_t groups_per_row) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & 15;
  const int64_t half = groups_per_row * kQ;  // I, in elements
  const int64_t waves = (int64_t)gridDim.x * (kQThreads / 64);
  const int64_t chunks = (groups + 15) / 16;
  for (int64_t ch = (int64_t)blockIdx.x * (kQThreads / 64) + (threadIdx.x >> 6); ch < chunks; ch += waves) {
    u4nt gv[4], uv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t g = ch * 16 + 4 * j + (lane >> 4);
      if (g < groups) {
        // row r's gate group gi starts at r * 2I + gi * 128 = (g + r * I/128) * 128
        const uint16_t* p = c + (g + g / groups_per_row * groups_per_row) * kQ + sub * 8;
        gv[j] = __builtin_nontemporal_load(reinterpret_cast<const u4nt*>(p));
        uv[j] = __builtin_nontemporal_load(reinterpret_cast<const u4nt*>(p + half));
      } else {
        gv[j] = u4nt{0u, 0u, 0u, 0u};
        uv[j] = u4nt{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float h[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        h[2 * t] = silu(bf16_lo(gv[j][t])) * bf16_lo(uv[j][t]);
        h[2 * t + 1] = silu(bf16_hi(gv[j][t])) * bf16_hi(uv[j][t]);
      }
      float m = 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(h[t]));
      m = max_xor(m, 8);
      m = max_xor(m, 4);
      m = max_xor(m, 2);
      m = max_xor(m, 1);
      const float sc = scale_of(m);
      const codec::GroupRecip gr = codec::group_recip(sc);
      float y[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) y[t] = codec::scaled(h[t], gr);
      const int64_t g = ch * 16 + 4 * j + (lane >> 4);
      if (g < groups) {
        if (sub == 0) s[g] = sc;
        const u2nt w = {encode4(y[0], y[1], y[2], y[3]), encode4(y[4], y[5], y[6], y[7])};
        __builtin_nontemporal_store(w, reinterpret_cast<u2nt*>(q + g * kQ + sub * 8));
      }
    }
  }
}

}  // namespace

hipError_t launch_swiglu_quantize(const uint16_t* c, uint8_t* q, float* s, int rows, int half_cols, int num_cus,
                                  hipStream_t stream) {
  const int64_t gpr = half_cols / kQ;
  const int64_t groups = (int64_t)rows * gpr;
  if (groups <= 0) return hipSuccess;
  const int64_t wgs = (groups + 16 * (kQThreads / 64) - 1) / (16 * (kQThreads / 64));
  const int64_t cap = (int64_t)(num_cus > 0 ? num_cus : 256) * 8;
  const int grid = (int)(wgs < cap ? wgs : cap);
  hipLaunchKernelGGL(swiglu_quant_kernel, dim3(grid), dim3(kQThreads), 0, stream, c, q, s, groups, gpr);
  return hipGetLastError();
}

hipError_t launch_quantize(int mode, const float* x, uint8_t* q, float* s, int rows, int cols, int num_cus,
                           hipStream_t stream) {
  const int64_t row_tiles = (rows + kQ - 1) / kQ;
  const int col_tiles = (cols + kQ - 1) / kQ;
  const int64_t tiles = row_tiles * col_tiles;
  // enough workgroups to keep eight resident per CU; each walks tiles with a
  // grid stride
  const int64_t cap = (int64_t)(num_cus > 0 ? num_cus : 256) * 8;
  const int grid = (int)(tiles < cap ? tiles : cap);
  if (grid <= 0) return hipSuccess;
  switch (mode) {
    case Q_ROWS:
    case Q_ROWS_UE8M0: {
      const int64_t groups = (int64_t)rows * (cols / kQ);
      const int64_t wgs = (groups + 16 * (kQThreads / 64) - 1) / (16 * (kQThreads / 64));
      const int g2 = (int)(wgs < cap ? wgs : cap);
      if (mode == Q_ROWS)
        hipLaunchKernelGGL(quant_rows_kernel<false>, dim3(g2), dim3(kQThreads), 0, stream, x, q, s, groups, cols / kQ);
      else
        hipLaunchKernelGGL(quant_rows_kernel<true>, dim3(g2), dim3(kQThreads), 0, stream, x, q, s, groups, cols / kQ);
      break;
    }
    case Q_BLOCKS:
      hipLaunchKernelGGL(quant_kernel<Q_BLOCKS>, dim3(grid), dim3(kQThreads), 0, stream, x, q, s, rows, cols, tiles,
                         col_tiles);
      break;
    case Q_BLOCKS_UE8M0:
      hipLaunchKernelGGL(quant_kernel<Q_BLOCKS_UE8M0>, dim3(grid), dim3(kQThreads), 0, stream, x, q, s, rows, cols,
                         tiles, col_tiles);
      break;
    case Q_TRANSPOSED:
      hipLaunchKernelGGL(quant_kernel<Q_TRANSPOSED>, dim3(grid), dim3(kQThreads), 0, stream, x, q, s, rows, cols,
                         tiles, col_tiles);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dg
