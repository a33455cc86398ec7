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
#include <type_traits>

#include "dg_fp8_codec.h"
#include "dg_kernel.h"
#include "dg_rsrc.h"
#include "dg_shapes.h"

namespace dg {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f4nt __attribute__((ext_vector_type(4)));
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

// LDS DMA through buffer loads.  Lane i's bytes go to LDS address m0 +
// i*size; the address is rsrc.base + voffset + soffset, and bytes at or past
// rsrc.num_records (range-checked on the per-lane offset) read as zero, so
// rows and columns past the tile's valid ones need no clamping.  The K-block
// offset moves the resource base (soffset stays 0): since that offset is
// less than one row, the range check still ends at the first invalid row.  Issued
// through inline asm so the compiler's wait-count pass does not treat every
// later LDS read as dependent on every in-flight DMA; the waits are explicit
// below.  Nothing else in these kernels uses m0.
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

// Raw buffer resource: 48-bit base, stride 0, byte range, 32-bit data format.
// Kept as four wave-uniform scalars (scalar-unit arithmetic) and packed into
// the 128-bit instruction operand only at the DMA.
struct Rsrc {
  uint32_t lo, hi, num, flags;
};

__device__ __forceinline__ Rsrc buffer_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t b = (uint64_t)base;
  return Rsrc{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b),
              (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) & 0xffffu,
              (uint32_t)__builtin_amdgcn_readfirstlane(num_bytes), 0x00020000u};
}

// The resource moved `bytes` further along, with its range cut to zero unless
// `live` and bytes < num: the range check still ends where the original one
// did, and a dead or exhausted resource reads zeros without touching memory
// (the range never wraps below zero).
__device__ __forceinline__ v4i at(const Rsrc& r, uint32_t bytes, bool live) {
  uint32_t lo, hi;
  base_moved(r.lo, r.hi, bytes, &lo, &hi);
  const uint32_t num = __builtin_amdgcn_readfirstlane(range_after(r.num, bytes, live));  // wave-uniform
  return v4i{(int)lo, (int)hi, (int)num, (int)r.flags};
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(uint32_t lds, v4i rsrc, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc) : "memory", "m0");
}
// The same with the nontemporal (streaming) cache policy, for operands read
// once per output tile row or column (see kStreamB).
__device__ __forceinline__ void dma16_nt(uint32_t lds, v4i rsrc, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :: "s"(lds), "v"(voff), "s"(rsrc) : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t lds, v4i rsrc, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc) : "memory", "m0");
}
#pragma clang diagnostic pop

// An opaque copy: keeps the compiler from hoisting (and keeping live) values
// that are cheaper to recompute next to their use.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait for the oldest of the ring's in-flight K blocks: `later` blocks (at
// most L) were issued after it, each D operations per wave, so at most
// min(later, L) * D operations may stay in flight.
template <int L, int D>
__device__ __forceinline__ void wait_blocks(int later) {
  if constexpr (L == 0) {
    wait_vm<0>();
  } else {
    if (later >= L) wait_vm<L * D>(); else wait_blocks<L - 1, D>(later);
  }
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

// A lane reads two 16-byte chunks of row (16f + l16) of a 16-row fragment f.
// Fragments start on multiples of 16 rows, so the swizzle of the row is
// swz(l16) and the lane's two in-fragment offsets are fixed: `lo` and `hi`.
__device__ __forceinline__ v8i load_frag(const uint8_t* frag_base, uint32_t lo, uint32_t hi) {
  const uint4 a = *reinterpret_cast<const uint4*>(frag_base + lo);
  const uint4 b = *reinterpret_cast<const uint4*>(frag_base + hi);
  return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// Power-of-two scales (UE8M0): the block-scaled MFMA multiplies each 32-wide
// K chunk of an operand row by 2^(E - 127), E being the 8-bit scale byte the
// lane holding that chunk supplies (byte 0 of its scale operand), and adds
// srcC: acc + sb * sa * (block sum), with the scaling applied inside the matrix
// unit and no vector-unit promotion.  A positive power-of-two fp32 scale
// 2^(E-127) has E as its exponent field (shift 23); a packed word holds the
// bytes E of four consecutive K blocks, K block 4w + i in byte i (shift 8i).
__device__ __forceinline__ int ue8m0_of(float s, uint32_t shift) {
  return (int)((__builtin_bit_cast(uint32_t, s) >> shift) & 0xffu);
}

__device__ __forceinline__ v4f mfma_block_scaled(const v8i& b_rows, const v8i& a_rows, const v4f& acc, int sb_e,
                                                 int sa_e) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b_rows, a_rows, acc, 0, 0, 0, sb_e, 0, sa_e);
}

// BF16: a lane's 32 fragment bytes are 16 bf16 values of its row; the two
// halves feed two 16x16x32 bf16 MFMAs that accumulate into `acc` (both
// operands use the same lane -> k assignment, so the pair covers the 64 values
// of the 128-byte K block).
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v4f mfma_block_bf16(const v8i& b_rows, const v8i& a_rows, const v4f& acc) {
  const v8bf b0 = __builtin_bit_cast(v8bf, v4i{b_rows[0], b_rows[1], b_rows[2], b_rows[3]});
  const v8bf b1 = __builtin_bit_cast(v8bf, v4i{b_rows[4], b_rows[5], b_rows[6], b_rows[7]});
  const v8bf a0 = __builtin_bit_cast(v8bf, v4i{a_rows[0], a_rows[1], a_rows[2], a_rows[3]});
  const v8bf a1 = __builtin_bit_cast(v8bf, v4i{a_rows[4], a_rows[5], a_rows[6], a_rows[7]});
  const v4f d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0, a0, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1, a1, d, 0, 0, 0);
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
  constexpr int LAYOUT = layout_of(KIND);            // dense, contiguous or masked scheduling
  constexpr bool kPow2 = pow2_kind(KIND);             // scales applied by the MFMA
  constexpr bool kBf16 = bf16_kind(KIND);              // bf16 operands, no scales at all
  // contiguous layout with the SwiGLU + re-quantise epilogue: the tile's B
  // rows are 128 gate rows and the 128 matching up rows, in LDS order
  // [pair][gate 16 | up 16], so a wave's fragments 2q and 2q+1 hold the gate
  // and the up value of the same output element in the same lane
  constexpr bool kSwiGLU = (KIND == KIND_CONTIG_SWIGLU);
  constexpr bool kContig = (LAYOUT == KIND_CONTIGUOUS) || kSwiGLU;
  static_assert(!kSwiGLU || (BM == 256 && BN == 256 && ((WM == 1 && WN == 8) || (WM == 2 && WN == 4))),
                "fused SwiGLU tile");
  // B loaded with the streaming (nontemporal) cache policy by the instances
  // whose launches read each B tile with one row of tiles: the dense tiles of
  // at most 128 rows (the heuristic's choice for M <= 128) and the masked
  // layout's tall tiles (one tile covers a group's rows).  Measured faster
  // there (dense M=64 x 7168 x 16384 +60%, masked decode +17-24%) and slower
  // where several row tiles re-read the same B (large-M dense -5 to -13%,
  // contiguous -4%).  Decided per instance at compile time: a runtime choice
  // in the DMA loop cost the 256x256 instances registers (spills in the loop).
  constexpr bool kStreamB =
      ((LAYOUT == KIND_DENSE || KIND == KIND_BF16) && BM <= 128) || LAYOUT == KIND_MASKED;
  constexpr bool kDirectAcc = kPow2 || kBf16;         // MFMAs accumulate into acc: no promotion
  constexpr bool kFp32Out = kRowScaleB;
  // the columns of one wave tile sit inside one 128-block: one sb per wave
  constexpr bool kWaveUniformSb = !kRowScaleB && !kSwiGLU && (kBK % WTN == 0) && (BN % WTN == 0);
  constexpr bool kStreamM = FM >= FN;  // keep the smaller fragment set resident
  // Masked layout with tall tiles: a wave whose rows run past the group's
  // valid rows skips those row fragments (no LDS read, no MFMA; their zero
  // partials keep the promotion rotation unchanged), so one tile can cover
  // every row of a group and B is streamed once per group.
  constexpr bool kSkipRows = (LAYOUT == KIND_MASKED) && kStreamM && (FM > 4) && (FM % 4 == 0) && (FM <= 16);
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile is a multiple of 16");
  static_assert(S >= 2, "at least double buffering");

  // ---- LDS stage layout and DMA pieces ----
  // Row scales of A in groups of kGrp K blocks (contiguous layout, two-stage
  // rings): a tile's sa for its K blocks 4g .. 4g+3 is fetched once, at the
  // start of the block before 4g, into one of two group buffers after the
  // ring.  Each lane of a group piece reads one scale word of row l/4 (16
  // rows x 4 words per piece), so a piece touches 16 rows' cache lines
  // instead of 64 and each row once per four K blocks instead of every
  // block.  A per-block sa piece touches one line per row (rows K/128 words
  // apart), which costs the texture path more than the operand pieces' whole
  // lines where sa misses the L2: the contiguous layout's sa (all tokens'
  // rows) is 4-8x the dense shapes'.  Measured: contiguous G=8, N=4096,
  // K=7168 4-5% faster; the dense shapes, whose sa stays in the L2 when
  // warm, 4-5% slower warm (3-5% faster cold), so they keep per-block
  // pieces, and so do deeper rings (a group buffer would still be read when
  // the next tile's first group lands in it).
  constexpr bool kSaGrp = (S == 2) && !kBf16 && kContig;
  constexpr int kGrp = 4;
  constexpr int SAG_ROWS = ((BM + 15) / 16) * 16;
  constexpr int SAG_BYTES = SAG_ROWS * 16;                       // [row][4 words]
  constexpr int PSAG = kSaGrp ? SAG_ROWS / 16 : 0;               // group pieces
  constexpr int QSAG = (PSAG + NW - 1) / NW;
  constexpr int SA_N = kSaGrp ? 0 : ((BM + 63) / 64) * 64;      // floats per stage
  constexpr int SB_N = kRowScaleB ? ((BN + 63) / 64) * 64 : 64;  // floats
  constexpr int OFF_A = 0;
  constexpr int OFF_B = BM * kBK;
  constexpr int OFF_SA = OFF_B + BN * kBK;
  constexpr int OFF_SB = OFF_SA + SA_N * 4;
  constexpr int STAGE = OFF_SB + SB_N * 4;
  // DMA pieces per stage: 1 KB operand pieces (8 LDS rows) and 256 B scale
  // pieces.  Wave w issues operand pieces w, w+NW, ... (the same count on
  // every wave) and scale pieces w, w+NW, ... (some waves one fewer).
  constexpr int PA = BM / 8, PB = BN / 8, PSA = SA_N / 64, PSB = SB_N / 64;
  constexpr int PS = PSA + PSB;
  // (a block width or height that is not a multiple of 8 * NW rows, e.g.
  // 224, leaves some waves one piece short: they issue a dead piece into the
  // sink instead)
  constexpr int QA = (PA + NW - 1) / NW, QB = (PB + NW - 1) / NW, QS = (PS + NW - 1) / NW;
  // every wave issues QA + QB + QS DMAs per stage: scale pieces past PS are
  // padding that reads nothing and lands in a sink slot after the ring
  constexpr int DMIN = QA + QB + QS;
  static_assert(BN % 16 == 0, "whole 16-column fragments");

  // + padding-DMA sink (1 KB) + the two sa group buffers
  constexpr int OFF_G = S * STAGE + 1024;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[OFF_G + (kSaGrp ? 2 * SAG_BYTES : 0)];
  // bf16 epilogue staging: a wave's 16-row fragment row goes through LDS so
  // that each store covers whole (64 columns) or half (32 columns) 128-byte
  // lines; rows padded by 16 bytes against bank conflicts
  constexpr bool kStage = !kFp32Out && !kSwiGLU && (WTN == 64 || WTN == 32);
  constexpr int kStageRow = WTN * 2 + 16;
  __shared__ __attribute__((aligned(16))) uint8_t sOut[kStage ? NW : 1][kStage ? 16 * kStageRow : 16];
  // fused SwiGLU: each wave's |h| maximum over its columns, per tile row
  __shared__ __attribute__((aligned(16))) float sRowMax[kSwiGLU ? BM : 1][kSwiGLU ? WN : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int l16 = lane & 15;
  const int lq = lane >> 4;
  const uint32_t smem_lds = lds_addr(smem);
  const uint32_t frag_lo = l16 * kBK + (((2 * lq) ^ swz(l16)) << 4);
  const uint32_t frag_hi = l16 * kBK + (((2 * lq + 1) ^ swz(l16)) << 4);

  // ---- tile count (masked: from masked_m on the device, no host sync) ----
  int T = p.tiles;
  if constexpr (LAYOUT == KIND_MASKED) {
    T = 0;
    for (int g = 0; g < p.groups; ++g) {
      const int v = min(max(p.ctrl[g], 0), p.m);
      T += ((v + BM - 1) / BM) * p.tiles_n;
    }
  }
  // split-K: `splits` consecutive work items share one output tile
  constexpr bool kCanSplit = (LAYOUT == KIND_DENSE || LAYOUT == KIND_MASKED || KIND == KIND_BF16);
  const int splits = kCanSplit ? p.splits : 1;
  const int TS = T * splits;
  const int per_xcd = (TS + 7) >> 3;
  const int nb_rows = (p.n + kBK - 1) / kBK;

  // ---- work items ----
  // Item t (a grid-stride index, remapped so each XCD gets a contiguous run
  // of items) is one (output tile, K split) pair.  decode() gives its Tile;
  // live == 0: no work (past the end, an empty K range, or -- contiguous -- a
  // block of padding rows).
  // contiguous: bit i of rmask[i / 64] says whether row wm * WTM + i of the
  // tile carries the tile's expert (this wave's rows only)
  constexpr int RMW = kContig ? (WTM + 63) / 64 : 1;
  struct Tile {
    int live, g, m0, n0, rows, kb0, nkb, split;
    int64_t a_row0, out_row0;
    uint64_t rmask[RMW];
  };
  const int t_end = per_xcd * 8;
  auto decode = [&](int t) -> Tile {
    Tile x{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, {}};
    const int LS = (t & 7) * per_xcd + (t >> 3);
    if (t >= t_end || LS >= TS) return x;
    const int L = splits > 1 ? LS / splits : LS;
    x.split = LS - L * splits;
    int kb1 = p.kbs;
    if constexpr (LAYOUT == KIND_MASKED) {
      int rem = L, mt = 0, v = 0, g = 0;
      for (; g < p.groups; ++g) {
        v = min(max(p.ctrl[g], 0), p.m);
        mt = (v + BM - 1) / BM;
        const int cnt = mt * p.tiles_n;
        if (rem < cnt) break;
        rem -= cnt;
      }
      if (g >= p.groups) return x;  // unreachable for L < T
      x.g = g;
      x.m0 = (rem % mt) * BM;       // m fastest: tiles sharing a B tile run together
      x.n0 = (rem / mt) * BN;
      x.rows = min(BM, v - x.m0);
      x.a_row0 = (int64_t)g * p.m + x.m0;
      x.out_row0 = x.a_row0;
    } else if constexpr (KIND == KIND_KGROUPED) {
      // the group is the fastest index: every XCD's contiguous run of items
      // holds all groups alike, whose K ranges (work per tile) differ
      const int g = L % p.groups;
      int tm, tn;
      raster(L / p.groups, p.tiles_m, p.tiles_n, tm, tn);
      x.g = g;
      x.m0 = tm * BM;
      x.n0 = tn * BN;
      x.rows = min(BM, p.m - x.m0);
      x.kb0 = p.kb_begin[g];
      kb1 = p.kb_begin[g + 1];
      x.a_row0 = x.m0;
      x.out_row0 = (int64_t)g * p.m + x.m0;
    } else {
      int tm, tn;
      raster(L, p.tiles_m, p.tiles_n, tm, tn);
      x.m0 = tm * BM;
      x.n0 = tn * (kSwiGLU ? BN / 2 : BN);  // fused SwiGLU: the first output (gate) column
      x.rows = min(BM, p.m - x.m0);
      x.a_row0 = x.m0;
      x.out_row0 = x.m0;
    }
    if (kCanSplit && splits > 1) {
      x.kb0 = x.split * p.kchunk;
      kb1 = min(p.kbs, x.kb0 + p.kchunk);
    }
    x.nkb = kb1 - x.kb0;
    x.live = x.nkb > 0;
    return x;
  };
  // contiguous: the expert of each 128-aligned row block of the tile (the
  // largest id in [0, G) in it: a block holds one expert, the rest is -1
  // padding).  Every wave reads the ids itself (no LDS, no barrier) and keeps
  // the rows of its own that carry the tile's expert as bit masks.  A
  // 256-row tile whose two blocks belong to different experts is computed
  // twice, once per expert (the second pass is queued in `pend`); each pass
  // stores only its expert's rows.
  auto wave_max = [](int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
    return __builtin_amdgcn_readfirstlane(v);
  };
  auto row_id = [&](const Tile& x, int r) { return r < x.rows ? p.ctrl[x.m0 + r] : -1; };
  // rows of this wave with id `e` in a block whose expert is `e` (blocks
  // 0 and 1 qualify per lo / hi)
  auto mark_rows = [&](Tile& x, int e, bool lo, bool hi) {
#pragma unroll
    for (int c = 0; c < RMW; ++c) {
      const int r = wm * WTM + 64 * c + lane;
      const bool in = lane < WTM - 64 * c;
      const bool ok = in && (r < 128 ? lo : hi) && row_id(x, r) == e;
      x.rmask[c] = __ballot(ok);
    }
  };
  int pend_t = -1, pend_g = -1;  // item and expert of a queued second pass
  auto find_expert = [&](Tile& x, int t) {
    int m0v = -1, m1v = -1;
#pragma unroll
    for (int i = 0; i < BM / 64; ++i) {
      const int r = 64 * i + lane;
      const int id = row_id(x, r);
      const int v = (id >= 0 && id < p.groups) ? id : -1;
      if (r < 128) m0v = max(m0v, v); else m1v = max(m1v, v);
    }
    const int e0 = wave_max(m0v);
    const int e1 = BM > 128 ? wave_max(m1v) : -1;
    const int e = e0 >= 0 ? e0 : e1;
    mark_rows(x, e, e0 == e, e1 == e);
    x.g = e;
    x.live = e >= 0;
    if (e0 >= 0 && e1 >= 0 && e1 != e0) {
      pend_t = t;
      pend_g = e1;
    }
  };
  // the first live item at or after `t` (or a queued second pass); `t`
  // moves past it
  auto next_live = [&](int& t) -> Tile {
    if constexpr (kContig) {
      if (pend_t >= 0) {
        Tile x = decode(pend_t);
        x.g = pend_g;
        pend_t = -1;
        mark_rows(x, x.g, false, true);  // the second block's expert
        return x;
      }
    }
    Tile x = decode(t_end);
    while (t < t_end) {
      x = decode(t);
      if constexpr (kContig)
        if (x.live) find_expert(x, t);
      t += gridDim.x;
      if (x.live) break;
    }
    return x;
  };
  // DMA sources of a tile at its first K block (a dead tile's read nothing):
  // the operand resources (the same on every wave) and the resource of each
  // of this wave's scale pieces -- sa rows or sb rows (row-scaled B) / 128-column
  // blocks, moved to the piece's first row, or empty -- so that a K block
  // only moves the bases.
  struct Res {
    Rsrc a, b;
    Rsrc s[QS];
    Rsrc sa;   // sa rows of the tile (grouped sa)
    int kb0, nkb;
    int gpar;  // group buffer of the tile's first sa group
  };
  // r advanced by `bytes` with its range cut where it ended (empty if that is
  // past the end or !on); wave-uniform
  auto moved = [](const Rsrc& r, uint32_t bytes, bool on) {
    uint32_t lo, hi;
    base_moved(r.lo, r.hi, bytes, &lo, &hi);
    return Rsrc{(uint32_t)__builtin_amdgcn_readfirstlane(lo), (uint32_t)__builtin_amdgcn_readfirstlane(hi),
                (uint32_t)__builtin_amdgcn_readfirstlane(range_after(r.num, bytes, on)), r.flags};
  };
  auto make_res = [&](const Tile& x) -> Res {
    const int bg = (KIND == KIND_KGROUPED) ? 0 : x.g;  // K-grouped: one B [N,T]
    const int bcols = max(0, min(BN, p.n - x.n0));      // valid B rows (output columns)
    const uint32_t on = x.live ? 1u : 0u;
    const uint32_t son = kBf16 ? 0u : on;  // BF16: the scale pieces read nothing
    Res r;
    r.a = buffer_rsrc(p.a + x.a_row0 * (int64_t)p.lda, on * (uint32_t)x.rows * p.lda);
    // fused SwiGLU: gate rows n0.. and up rows I + n0.. (I = N/2), one range
    const uint32_t brows = kSwiGLU ? (uint32_t)(p.n / 2 + BN / 2) : (uint32_t)bcols;
    r.b = buffer_rsrc(p.b + ((int64_t)bg * p.n + x.n0) * (int64_t)p.lda, on * brows * p.lda);
    const Rsrc sa = buffer_rsrc(p.sa + x.a_row0 * (int64_t)p.sks, son * (uint32_t)x.rows * p.sks * 4);
    Rsrc sb;
    if constexpr (kRowScaleB) {
      sb = buffer_rsrc(p.sb + (int64_t)x.n0 * p.sks, on * (uint32_t)bcols * p.sks * 4);
    } else {
      // only the 128-column blocks the tile touches
      // (fused SwiGLU: the gate block n0/128 through the up block (I + n0)/128)
      const int nb0 = x.n0 / kBK;
      const int nbt = kSwiGLU ? p.n / 2 / kBK + 1
                              : min(nb_rows - nb0, (x.n0 - nb0 * kBK + BN + kBK - 1) / kBK);  // a tile may straddle blocks
      sb = buffer_rsrc(p.sb + ((int64_t)x.g * nb_rows + nb0) * p.sks, son * (uint32_t)max(nbt, 0) * p.sks * 4);
    }
    const uint32_t prow = 64u * p.sks * 4;  // bytes of 64 scale rows
#pragma unroll
    for (int q = 0; q < QS; ++q) {
      const int sp = wave + NW * q;  // scale piece: sa rows 64*sp.., then sb
      const bool is_a = sp < PSA;
      const uint32_t rowoff = (uint32_t)(is_a ? sp : sp - PSA) * prow;
      const Rsrc src{is_a ? sa.lo : sb.lo, is_a ? sa.hi : sb.hi, is_a ? sa.num : sb.num, sa.flags};
      r.s[q] = moved(src, rowoff, sp < PS);
    }
    r.sa = sa;
    r.kb0 = x.kb0;
    r.nkb = x.live ? x.nkb : 0;
    r.gpar = 0;
    return r;
  };
  // Cross-tile prefetch: the DMAs of the next tile's first S-1 K blocks are
  // issued during the current tile's last S-1 blocks, so a tile starts with
  // its data in flight and its epilogue overlaps them.  Needs every tile to
  // have at least S-1 K blocks (K-grouped ranges can be empty or short).
  // (K-grouped: groups with no tokens have no live tiles and are never in
  // the ring, so the shortest non-empty group decides)
  const int min_nkb = (KIND == KIND_KGROUPED)       ? p.kg_min_blocks
                      : (kCanSplit && splits > 1) ? min(p.kchunk, p.kbs - (splits - 1) * p.kchunk)
                                                  : p.kbs;
  const bool xfer = min_nkb >= S - 1;

  // bf16 output (or split-K partials) in whole 4-column vectors, offsets that
  // fit the 32-bit buffer range: the epilogue's stores have a fixed count
  // staged bf16: 16 B per lane, (WTN*2*16)/1024 stores per fragment row
  constexpr int kStageStores = FM * (WTN * 2 * 16 / 1024);
  constexpr int kStores = kStage ? kStageStores : FM * FN;
  constexpr bool kExactFits = (S - 2) * DMIN + kStores <= 63;  // vmcnt range
  // (not for the fp32 D kinds: their row-scale registers leave no room for
  // it; staged layouts: bf16 with N % 8 == 0 only, split-K partials take the
  // per-fragment path with the conservative wait)
  const bool staged = kStage && !(kCanSplit && splits > 1) && p.vec_out && (p.n % 8 == 0);
  const bool exact_stores = kExactFits && (kStage ? staged : (!kFp32Out || (kCanSplit && splits > 1))) &&
                            p.vec_out && (int64_t)BM * p.n * 4 < 0x7fffffffLL;
  bool stores_pending = false;  // the previous tile's epilogue stores may be in flight

  int t_next = blockIdx.x;
  Tile cur = next_live(t_next);
  int qbase = 0;        // ring stage of the current tile's first K block
  int gpar = 0;         // sa group buffer of the current tile's first group
  bool first = true;
  while (cur.live) {
    // the next tile: looked up (with cross-tile prefetch) only before the
    // current tile's last S-1 K blocks, so its state is not live in the main
    // part of the K loop (registers)
    Tile nxt = decode(t_end);
    Res rc = make_res(cur);
    rc.gpar = gpar;
    const int n0 = cur.n0, rows = cur.rows, nkb = cur.nkb, split = cur.split;
    const int64_t out_row0 = cur.out_row0;

    // Lane l of operand piece q lands on LDS row 8*(wave + NW*q) + l/8, chunk
    // l%8.  Row steps between a wave's pieces are multiples of 16, so the
    // swizzle term is fixed per lane; only the row step changes with q.
    const int r0 = wave * 8 + (lane >> 3);
    const uint32_t voff0 = (uint32_t)r0 * p.lda + (((lane & 7) ^ swz(r0)) << 4);
    const uint32_t step = (uint32_t)(NW * 8) * p.lda;  // bytes between a wave's pieces
    // fused SwiGLU: LDS row j of B is gate row n0 + 16 (j / 32) + j % 16 when
    // (j / 16) is even, else the up row I + n0 + ...; a wave's pieces are 64
    // LDS rows = 32 source rows apart
    const uint32_t voffb0 =
        kSwiGLU ? (uint32_t)(((r0 >> 4) & 1) * (p.n / 2) + 16 * (r0 >> 5) + (r0 & 15)) * p.lda +
                      (((lane & 7) ^ swz(r0)) << 4)
                : voff0;
    const uint32_t stepb = kSwiGLU ? (uint32_t)(NW * 4) * p.lda : step;
    // scale pieces: 64 rows (or columns / 128-blocks) each, one float per lane
    const uint32_t svoff = (uint32_t)lane * p.sks * 4;
    // fused SwiGLU: the B scale piece's lane 1 reads the up block I/128 blocks
    // on, so the stage holds sb(gate) at 0 and sb(up) at 1
    const uint32_t svoff_b = kSwiGLU && lane == 1 ? (uint32_t)(p.n / 2 / kBK) * p.sks * 4 : svoff;
    // sa group pieces: lane l reads word l%4 of the group in row l/4 of the
    // piece (rows 16*pg .. 16*pg+15 of the tile)
    const uint32_t gvoff = (uint32_t)((lane >> 2) + 16 * wave) * p.sks * 4 + (uint32_t)(lane & 3) * 4;
    const uint32_t gstep = (uint32_t)(16 * NW) * p.sks * 4;  // rows between a wave's pieces

    // The DMAs of one K block: each source moved to the block (empty past
    // the tile's K range or for a dead tile: such a block reads zeros and
    // touches no memory, into a stage no live block of the ring needs) and
    // the ring stage it lands in.  Built once per block; `issue` then only
    // sends pieces [lo, hi) of it (A pieces first, then B, then scales), so a
    // block's DMAs can be spread over the fragment groups of the previous
    // block instead of stalling every wave at the same point.
    struct Blk {
      v4i a, b, s[QS];
      v4i g;  // sa rows of the tile at the group's first word (a group's first block only)
      uint32_t base, gbase;
      bool grp;
    };
    // A source moved to K byte offset `koff` of its rows (scalar arithmetic):
    // a non-empty range holds at least one row, which is longer than any K
    // offset, so the range stays positive; a dead block or source reads
    // nothing.
    auto at_k = [](const Rsrc& r, uint32_t koff, bool live) {
      uint32_t lo, hi;
      base_moved(r.lo, r.hi, koff, &lo, &hi);
      return v4i{(int)__builtin_amdgcn_readfirstlane(lo), (int)__builtin_amdgcn_readfirstlane(hi),
                 (int)__builtin_amdgcn_readfirstlane(range_at_k(r.num, koff, live)), (int)r.flags};
    };
    auto blk_of = [&](const Res& r, int rel, int st) -> Blk {
      const bool live = rel < r.nkb;
      const uint32_t kb = (uint32_t)(r.kb0 + rel);
      Blk d;
      d.a = at_k(r.a, kb * kBK, live);
      d.b = at_k(r.b, kb * kBK, live);
#pragma unroll
      for (int q = 0; q < QS; ++q) d.s[q] = at_k(r.s[q], (kb >> p.spk) * 4, live);
      d.base = __builtin_amdgcn_readfirstlane(smem_lds + st * STAGE);
      d.grp = false;
      d.gbase = 0;
      if constexpr (kSaGrp) {
        // the group's words: fp32 scales of blocks kb .. kb+3, or the packed
        // words from the one holding block kb on (a group of four blocks
        // spans at most two of them)
        d.grp = live && (rel % kGrp) == 0;
        d.g = at_k(r.sa, (p.spk ? (kb >> 2) : kb) * 4, d.grp);
        d.gbase = __builtin_amdgcn_readfirstlane(smem_lds + OFF_G + ((r.gpar + rel / kGrp) & 1) * SAG_BYTES);
      }
      return d;
    };
    constexpr int ND = QA + QB + QS;
    // Piece order within a block: A, B, then the scale pieces -- except for
    // the masked layout, whose scale pieces go first.  The wave's DMAs
    // complete in issue order as far as its waits can tell, and a scale
    // piece (one row per lane, a cache line each) takes longer than an
    // operand piece (whole lines): issued last it holds up the wait for the
    // whole block.  Measured: the masked decode G=16 7-10% faster; the dense
    // small-M tiles mixed (-4% to +9%), the large tiles equal, so only the
    // masked layout reorders.
    constexpr bool kScalesFirst = (LAYOUT == KIND_MASKED);
    constexpr int iA = kScalesFirst ? QS : 0, iB = iA + QA, iS = kScalesFirst ? 0 : QA + QB;
    auto issue = [&](const Blk& d, int lo, int hi) {
      auto scales = [&]() {
#pragma unroll
        for (int q = 0; q < QS; ++q) {
          if (iS + q < lo || iS + q >= hi) continue;
          const int sp = wave + NW * q;
          dma4(sp < PS ? d.base + OFF_SA + sp * 256 : smem_lds + S * STAGE, d.s[q], sp < PSA ? svoff : svoff_b);
        }
      };
      if constexpr (kScalesFirst) scales();
#pragma unroll
      for (int q = 0; q < QA; ++q)
        if (iA + q >= lo && iA + q < hi) {
          if constexpr (PA % NW == 0) {
            dma16(d.base + OFF_A + (wave + NW * q) * 1024, d.a, voff0 + q * step);
          } else {
            // past the last A piece: read nothing into the sink
            const bool real = wave + NW * q < PA;
            v4i rq = d.a;
            rq[2] = real ? d.a[2] : 0;
            dma16(real ? d.base + OFF_A + (wave + NW * q) * 1024 : smem_lds + S * STAGE, rq, voff0 + q * step);
          }
        }
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        if (iB + q < lo || iB + q >= hi) continue;
        const int pi = wave + NW * q;
        if constexpr (PB % NW == 0) {
          if constexpr (kStreamB)
            dma16_nt(d.base + OFF_B + pi * 1024, d.b, voffb0 + q * stepb);
          else
            dma16(d.base + OFF_B + pi * 1024, d.b, voffb0 + q * stepb);
        } else {
          // past the last B piece: read nothing into the sink
          const bool real = pi < PB;
          v4i rq = d.b;
          rq[2] = real ? d.b[2] : 0;
          dma16(real ? d.base + OFF_B + pi * 1024 : smem_lds + S * STAGE, rq, voff0 + q * step);
        }
      }
      if constexpr (!kScalesFirst) scales();
      if (lo < 0 && kSaGrp) {
        // the block's sa group (issue(d, -1, -1) at a block start, not
        // spread over the fragment groups: a branch among the MFMAs costs
        // registers); pieces past the tile's rows read nothing into the sink
#pragma unroll
        for (int q = 0; q < QSAG; ++q) {
          const int pg = wave + NW * q;
          const bool real = PSAG % NW == 0 || pg < PSAG;
          v4i rq = d.g;
          rq[2] = real ? d.g[2] : 0;
          dma4(real ? d.gbase + pg * 256 : smem_lds + S * STAGE, rq, gvoff + q * gstep);
        }
      }
    };
    const int qs = qbase % S;

    v4f acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    if constexpr (kFp32Out) {
      // D += ...: the accumulators start from D, loaded here so the loads
      // overlap the tile's first K blocks and the epilogue only stores
      // (lane indices opaque: see the epilogue)
      const int lane = (int)opaque(threadIdx.x & 63u);
      const int l16 = lane & 15;
      const int lq = lane >> 4;
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int ml = wm * WTM + 16 * j + l16;
        if (ml >= rows) continue;
        const float* d = static_cast<const float*>(p.out) + (out_row0 + ml) * p.n;
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const int n = n0 + wn * WTN + 16 * i + 4 * lq;
          if (n >= p.n) continue;
          if (p.vec_out && n + 3 < p.n) {
            // D is read once and written once per tile: streaming (nontemporal)
            // accesses keep it from displacing the operands (weight gradient +6%,
            // K-grouped +10%; the same for bf16 C stores made other kinds slower)
            const f4nt t = __builtin_nontemporal_load(reinterpret_cast<const f4nt*>(d + n));
            const float4 v = float4{t[0], t[1], t[2], t[3]};
            acc[i][j] = v4f{v.x, v.y, v.z, v.w};
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < p.n) acc[i][j][r] = d[n + r];
          }
        }
      }
    }

    // Fragments: NR resident ones are read once per K block, NO streamed
    // ones one at a time.  MFMA M(o, r) multiplies streamed fragment o by
    // resident fragment r into part[r]; its promotion F(o, r) (one FMA per
    // element by sa*sb) is issued NR-1 MFMAs later, in the rotation
    //   M(o,0) F(o-1,1) M(o,1) F(o-1,2) ... M(o,NR-1) F(o,0) M(o+1,0) ...
    // so every FMA finds its partial ready and every MFMA finds its part
    // register already consumed.  The rotation runs on across K blocks: the
    // last group's F(NO-1, 1..NR-1) follow the next block's first MFMAs.
    constexpr int NO = kStreamM ? FM : FN;
    constexpr int NR = kStreamM ? FN : FM;
    // zero partials and scales make the carried-over promotions of the first
    // K block exact no-ops (fma(0, 0, acc) == acc), so they need no branch
    v4f part[NR];
    float pend[NR];  // scales of the group still being promoted
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      part[r] = v4f{0.f, 0.f, 0.f, 0.f};
      pend[r] = 0.f;
    }
    auto acc_at = [&](int o, int r) -> v4f& { return kStreamM ? acc[r][o] : acc[o][r]; };
    auto fma4 = [&](v4f& a, float s, const v4f& pr) {
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = __builtin_fmaf(s, pr[e], a[e]);
    };
    // row-scaled B (weight gradients): the scale differs per output column
    v4f pendq[kRowScaleB ? NR : 1];
#pragma unroll
    for (int r = 0; r < (kRowScaleB ? NR : 1); ++r) pendq[r] = v4f{0.f, 0.f, 0.f, 0.f};
    auto fma4q = [&](v4f& a, float s, const v4f& q, const v4f& pr) {
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = __builtin_fmaf(s * q[e], pr[e], a[e]);
    };

    // The K loop for NOV live streamed fragments per wave (NOV == NO except
    // for the masked layout, whose waves skip the row quarters past the
    // group's valid rows; the rotation then ends at fragment NOV-1).
    auto k_loop = [&](auto nov_c) {
    constexpr int NOV = decltype(nov_c)::value;
      // prologue: the first S-1 K blocks in flight (with cross-tile prefetch
      // only for a workgroup's first tile; later tiles' were issued ahead)
      if (first || !xfer) {
  #pragma unroll
        for (int s = 0; s < S - 1; ++s)
          if (s < nkb) {
            const Blk d0 = blk_of(rc, s, (qs + s) % S);
            issue(d0, 0, ND);
            if constexpr (kSaGrp) issue(d0, -1, -1);  // (s == 0 starts a group)
          }
      }

      // one K block; `dma` is the block issued during it (S-1 ahead)
      auto block = [&](int rel, const Blk& dma) {
        const int st = (qs + rel) % S;
        // power-of-two scales: where this block's exponent byte sits in the
        // scale words read from LDS (fp32 exponent field, or packed byte)
        const uint32_t esh = p.spk ? 8u * ((uint32_t)(rc.kb0 + rel) & 3u) : 23u;
        // this wave's DMAs for block `rel` are done once at most
        // (blocks issued after it) x DMIN of its operations remain in flight;
        // with cross-tile prefetch S-2 blocks always follow (epilogue stores
        // in between only make the wait stricter)
        const int later = xfer ? S - 2 : min(S - 2, nkb - 1 - rel);
        // the previous epilogue's kStores stores were issued after blocks
        // 0..S-2 of this tile, so they too may stay in flight while waiting
        // for those blocks
        if (stores_pending && rel < S - 1) {
          if constexpr (kExactFits) wait_vm<(S - 2) * DMIN + kStores>(); else wait_vm<0>();
        } else {
          wait_blocks<S - 2, DMIN>(later);
        }
        barrier();  // every wave's block `rel` landed; every wave is done with rel-1

        const uint8_t* sA = smem + st * STAGE + OFF_A;
        const uint8_t* sB = smem + st * STAGE + OFF_B;
        const float* sSA = reinterpret_cast<const float*>(smem + st * STAGE + OFF_SA);
        // grouped sa: this block's word of each row in its group's buffer
        const float* sSG = reinterpret_cast<const float*>(smem + OFF_G + ((rc.gpar + rel / kGrp) & 1) * SAG_BYTES);
        const int kbr = rc.kb0 + rel;
        const int gw = p.spk ? (kbr >> 2) - ((kbr - rel % kGrp) >> 2) : rel % kGrp;
        auto sa_row = [&](int r) -> float { return kSaGrp ? sSG[4 * r + gw] : sSA[r]; };
        const float* sSB = reinterpret_cast<const float*>(smem + st * STAGE + OFF_SB);
        const uint8_t* wA = sA + wm * WTM * kBK;  // this wave's first A row
        const uint8_t* wB = sB + wn * WTN * kBK;  // this wave's first B row
        auto frag_a = [&](int j) { return load_frag(wA + j * 16 * kBK, frag_lo, frag_hi); };
        auto frag_b = [&](int i) { return load_frag(wB + i * 16 * kBK, frag_lo, frag_hi); };
        auto load_s = [&](int o) -> v8i { return kStreamM ? frag_a(o) : frag_b(o); };  // streamed fragment o
        // the first MFMA's two fragments are read first (and kept first by
        // the scheduling fence), so it waits only for them, not for every
        // resident fragment of the block
        v8i res[NR];
        res[0] = NOV > 0 ? (kStreamM ? frag_b(0) : frag_a(0)) : v8i{0, 0, 0, 0, 0, 0, 0, 0};
        v8i cur = NOV > 0 ? load_s(0) : v8i{0, 0, 0, 0, 0, 0, 0, 0};
        __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
        for (int r = 1; r < NR; ++r)
          res[r] = NOV > 0 ? (kStreamM ? frag_b(r) : frag_a(r)) : v8i{0, 0, 0, 0, 0, 0, 0, 0};

        // row scales: when A is the streamed operand, group o's scale is read
        // one group ahead, with group o's fragment (so no group waits on an
        // LDS read it has just issued; only three scales are live);
        // otherwise all FM (resident, few) are read up front
        float sav[kStreamM ? 1 : FM];
        float sa_next = (kStreamM && NOV > 0) ? sa_row(wm * WTM + l16) : 0.f;
        if constexpr (!kStreamM) {
  #pragma unroll
          for (int j = 0; j < FM; ++j) sav[j] = sa_row(wm * WTM + 16 * j + l16);
        }
        float sa_prev = 0.f, sa_cur = 0.f;
        // B scale per n-fragment (block scales) or per column quad (row scales)
        float sbv[FN];
        v4f sbq[kRowScaleB ? FN : 1];
        if constexpr (kRowScaleB) {
  #pragma unroll
          for (int i = 0; i < FN; ++i)
            sbq[i] = *reinterpret_cast<const v4f*>(&sSB[wn * WTN + 16 * i + 4 * lq]);
        } else if constexpr (kWaveUniformSb) {
          const float sb = sSB[(n0 + wn * WTN) / kBK - n0 / kBK];
  #pragma unroll
          for (int i = 0; i < FN; ++i) sbv[i] = sb;
        } else if constexpr (kSwiGLU) {
  #pragma unroll
          for (int i = 0; i < FN; ++i) sbv[i] = sSB[i & 1];  // gate block, up block, ...
        } else {
  #pragma unroll
          for (int i = 0; i < FN; ++i) sbv[i] = sSB[(n0 + wn * WTN + 16 * i) / kBK - n0 / kBK];
        }
        // F(o, r) of this block (o is the current or the previous group)
        auto promote = [&](int o, int r, bool previous) {
          const int j = kStreamM ? o : r, i = kStreamM ? r : o;
          const float sa = kStreamM ? (previous ? sa_prev : sa_cur) : sav[kStreamM ? 0 : j];
          if constexpr (kRowScaleB)
            fma4q(acc[i][j], sa, sbq[i], part[r]);
          else
            fma4(acc[i][j], sa * sbv[i], part[r]);
        };
        // F(NOV-1, r) of the previous block
        auto promote_pending = [&](int r) {
          if constexpr (kRowScaleB)
            fma4q(acc_at(NOV - 1, r), pend[r], pendq[r], part[r]);
          else
            fma4(acc_at(NOV - 1, r), pend[r], part[r]);
        };
        if constexpr (kSaGrp)
          if (dma.grp) issue(dma, -1, -1);
        if constexpr (NOV == 0) issue(dma, 0, ND);  // no groups to spread over

  #pragma unroll
        for (int o = 0; o < NOV; ++o) {
          v8i nxt = cur;
          if (o + 1 < NOV) nxt = load_s(o + 1);
          if constexpr (kStreamM) {
            sa_cur = sa_next;
            if (o + 1 < NOV) sa_next = sa_row(wm * WTM + 16 * (o + 1) + l16);
          }
  #pragma unroll
          for (int r = 0; r < NR; ++r) {
            if constexpr (kBf16) {
              acc_at(o, r) = kStreamM ? mfma_block_bf16(res[r], cur, acc_at(o, r))
                                      : mfma_block_bf16(cur, res[r], acc_at(o, r));
            } else if constexpr (kPow2) {
              // B fragment i carries sb, A fragment j carries its rows' sa
              const int j = kStreamM ? o : r, i = kStreamM ? r : o;
              const float sa = kStreamM ? sa_cur : sav[kStreamM ? 0 : j];
              acc_at(o, r) = kStreamM ? mfma_block_scaled(res[r], cur, acc_at(o, r), ue8m0_of(sbv[i], esh),
                                                          ue8m0_of(sa, esh))
                                      : mfma_block_scaled(cur, res[r], acc_at(o, r), ue8m0_of(sbv[i], esh),
                                                          ue8m0_of(sa, esh));
            } else {
              part[r] = kStreamM ? mfma_block(res[r], cur) : mfma_block(cur, res[r]);
              if (r + 1 < NR) {
                if (o > 0)
                  promote(o - 1, r + 1, true);
                else
                  promote_pending(r + 1);
              }
            }
          }
          // this group's share of the next block's DMAs (spread over the first
          // half of the groups so they still land in time)
          constexpr int kSpread = NOV / 2 > 0 ? NOV / 2 : 1;
          if (o < kSpread)
            issue(dma, (o * ND) / kSpread, ((o + 1) * ND) / kSpread);
          if constexpr (!kDirectAcc) promote(o, 0, false);
          sa_prev = sa_cur;
          cur = nxt;
          // keep each group's loads, MFMAs and FMAs together: no fragment
          // reads hoisted further ahead (register pressure)
          __builtin_amdgcn_sched_barrier(0);
        }
        // the rest of the last group is promoted during the next block
  #pragma unroll
        for (int r = 0; r < NR && NOV > 0 && !kDirectAcc; ++r) {
          const int j = kStreamM ? NOV - 1 : r, i = kStreamM ? r : NOV - 1;
          const float sa = kStreamM ? sa_prev : sav[kStreamM ? 0 : j];
          if constexpr (kRowScaleB) {
            pend[r] = sa;
            pendq[r] = sbq[i];
          } else {
            pend[r] = sa * sbv[i];
          }
        }
      };
      // main part: the DMAs are this tile's own blocks
      const int tail = max(0, nkb - (S - 1));
  #pragma unroll 1
      for (int rel = 0; rel < tail; ++rel) block(rel, blk_of(rc, rel + S - 1, (qs + rel + S - 1) % S));
      // last S-1 blocks: the DMAs are the next tile's first blocks (cross-tile
      // prefetch), else dead blocks
      if (xfer) nxt = next_live(t_next);
      Res rn = make_res(nxt);
      rn.gpar = (gpar + (nkb + kGrp - 1) / kGrp) & 1;
  #pragma unroll 1
      for (int rel = tail; rel < nkb; ++rel) block(rel, blk_of(rn, rel + S - 1 - nkb, (qs + rel + S - 1) % S));
  #pragma unroll
      for (int r = 1; r < NR && NOV > 0 && !kDirectAcc; ++r) {
        if constexpr (kRowScaleB)
          fma4q(acc_at(NOV - 1, r), pend[r], pendq[r], part[r]);
        else
          fma4(acc_at(NOV - 1, r), pend[r], part[r]);
      }
    };
    if constexpr (kSkipRows) {
      const int quarters = min(NO / 4, max(0, (rows - wm * WTM + 63) / 64));
      switch (quarters) {
        case 0: k_loop(std::integral_constant<int, 0>{}); break;
        case 1: k_loop(std::integral_constant<int, (NO >= 4 ? 4 : NO)>{}); break;
        case 2: k_loop(std::integral_constant<int, (NO >= 8 ? 8 : NO)>{}); break;
        case 3: k_loop(std::integral_constant<int, (NO >= 12 ? 12 : NO)>{}); break;
        default: k_loop(std::integral_constant<int, NO>{}); break;
      }
    } else {
      k_loop(std::integral_constant<int, NO>{});
    }
    if (!xfer) {
      wait_vm<0>();  // dead DMAs of the last blocks have landed
      barrier();     // all waves are done with the ring before the next prologue refills it
    }

    // ---- epilogue ----
    // The lane's indices made anew, opaque to the compiler: otherwise it
    // computes the epilogue's lane-dependent offsets and masks once before
    // the first tile and keeps them in registers through every K loop.
    const int lane = (int)opaque(threadIdx.x & 63u);
    const int l16 = lane & 15;
    const int lq = lane >> 4;
    // contiguous: does row 16*j + r of this wave's rows carry the tile's expert
    // (j a compile-time fragment row, r < 16)
    auto rbit = [&](int j, int r) -> bool {
      return ((cur.rmask[((16 * j) / 64) % RMW] >> (uint32_t)(16 * (j % 4) + r)) & 1u) != 0;
    };
    if constexpr (kSwiGLU) {
      // h = silu(gate) * up on the bf16-rounded GEMM outputs (what the unfused
      // path stores and its SwiGLU kernel reads), then the 1x128 rule over the
      // tile's 128 output columns [n0, n0 + 128) of each row: the waves' |h|
      // maxima over their columns meet in LDS.  A wave's fragments 2q and
      // 2q+1 are the gate and up values of its column pair q: lane (l16, lq)
      // of fragment row j holds output columns n0 + (WTN/2) wn + 16 q + 4 lq
      // .. + 3 of tile row wm WTM + 16 j + l16.
      constexpr int NP = FN / 2;  // gate/up fragment pairs per wave
      static_assert(FN % 2 == 0 && WN % 4 == 0, "SwiGLU pairs and row-maximum vectors");
      const int half = p.n / 2;
      auto bf16r = [](float x) { return __uint_as_float((uint32_t)f32_to_bf16(x) << 16); };
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        float m = 0.f;
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          float h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            h[e] = codec::silu(bf16r(acc[2 * q][j][e])) * bf16r(acc[2 * q + 1][j][e]);
            m = fmaxf(m, fabsf(h[e]));
          }
          acc[2 * q][j] = v4f{h[0], h[1], h[2], h[3]};
        }
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (lq == 0) sRowMax[wm * WTM + 16 * j + l16][wn] = m;
      }
      barrier();  // every wave's maxima are in LDS
      uint8_t* qo = static_cast<uint8_t*>(p.out);
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int r = wm * WTM + 16 * j + l16;
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < WN; c += 4) {
          const float4 a = *reinterpret_cast<const float4*>(&sRowMax[r][c]);
          amax = fmaxf(amax, fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w)));
        }
        const float sc = codec::scale_of(amax);
        const codec::GroupRecip gr = codec::group_recip(sc);
        if (rbit(j, l16)) {
          const int64_t orow = out_row0 + r;
#pragma unroll
          for (int q = 0; q < NP; ++q) {
            const uint32_t w = codec::encode4(codec::scaled(acc[2 * q][j][0], gr), codec::scaled(acc[2 * q][j][1], gr),
                                              codec::scaled(acc[2 * q][j][2], gr), codec::scaled(acc[2 * q][j][3], gr));
            *reinterpret_cast<uint32_t*>(qo + orow * half + n0 + (WTN / 2) * wn + 16 * q + 4 * lq) = w;
          }
          if (wn == 0 && lq == 0) p.out_scale[orow * (half / kBK) + n0 / kBK] = sc;
        }
      }
    } else if (kStage && staged) {
      // fragment row j: lanes write their 4 bf16 per column fragment into the
      // wave's LDS rows, then read 16 contiguous bytes each along the rows
      constexpr int kLanesPerRow = WTN * 2 / 16;    // 8 (64 columns) or 4 (32)
      constexpr int kRowsPerRound = 64 / kLanesPerRow;
      constexpr int kRounds = 16 / kRowsPerRound;   // 2 or 1
      uint8_t* so = sOut[kStage ? wave : 0];
      const uint32_t sbase = lds_addr(so);
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(static_cast<uint16_t*>(p.out) + out_row0 * p.n), (short)0, (int)((uint32_t)BM * p.n * 2), 0x00020000);
      const int rl = lane / kLanesPerRow, cb = (lane % kLanesPerRow) * 16;  // read-back row and byte
#pragma unroll
      for (int j = 0; j < FM; ++j) {
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const uint32_t lo = (uint32_t)f32_to_bf16(acc[i][j][0]) | ((uint32_t)f32_to_bf16(acc[i][j][1]) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16(acc[i][j][2]) | ((uint32_t)f32_to_bf16(acc[i][j][3]) << 16);
          *reinterpret_cast<uint2*>(so + l16 * kStageRow + (16 * i + 4 * lq) * 2) = uint2{lo, hi};
        }
#pragma unroll
        for (int h = 0; h < kRounds; ++h) {
          const int r = h * kRowsPerRound + rl;
          const uint4 v = *reinterpret_cast<const uint4*>(so + r * kStageRow + cb);
          const int ml = wm * WTM + 16 * j + r;
          bool row_ok;
          if constexpr (kContig)
            row_ok = rbit(j, r);
          else
            row_ok = ml < rows;
          const int n = n0 + wn * WTN + cb / 2;  // 8 columns, all valid or none (N % 8 == 0)
          const uint32_t off = (row_ok && n < p.n) ? ((uint32_t)ml * p.n + n) * 2u : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, ro, off, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);  // one fragment row at a time (registers)
      }
      (void)sbase;
    } else if (exact_stores) {
      // One buffer store per fragment pair, issued whether or not its lanes
      // are valid: a lane whose row or columns fall outside the output gets
      // an offset past the resource's range and the store drops it.  The
      // wave's store count is then fixed (FM * FN), so the next tile's first
      // waits can leave exactly these stores in flight.
      // fp32 split-K partials, else bf16 C
      const bool part = kCanSplit && splits > 1;
      const bool f32 = part;
      const uint32_t esz = f32 ? 4u : 2u;
      void* obase = part ? (void*)(p.ws + split * p.ws_stride + out_row0 * p.n)
                         : (void*)(static_cast<uint16_t*>(p.out) + out_row0 * p.n);
      const __amdgpu_buffer_rsrc_t ro =
          __builtin_amdgcn_make_buffer_rsrc(obase, (short)0, (int)((uint32_t)BM * p.n * esz), 0x00020000);
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int ml = wm * WTM + 16 * j + l16;
        bool row_ok;
        if constexpr (kContig)
          row_ok = rbit(j, l16);
        else
          row_ok = ml < rows;
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const int n = n0 + wn * WTN + 16 * i + 4 * lq;
          const uint32_t off = (row_ok && n < p.n) ? ((uint32_t)ml * p.n + n) * esz : 0x80000000u;
          if (f32) {
            // (bit-cast the whole vector: a bit-cast of one element of an
            // ext_vector_type is miscompiled to element 0 by this clang)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, acc[i][j]), ro, off, 0, 0);
          } else {
            const uint32_t lo = (uint32_t)f32_to_bf16(acc[i][j][0]) | ((uint32_t)f32_to_bf16(acc[i][j][1]) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16(acc[i][j][2]) | ((uint32_t)f32_to_bf16(acc[i][j][3]) << 16);
            __builtin_amdgcn_raw_buffer_store_b64(v2i{(int)lo, (int)hi}, ro, off, 0, 0);
          }
        }
      }
    } else {
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int ml = wm * WTM + 16 * j + l16;
      bool row_ok;
      if constexpr (kContig)
        row_ok = rbit(j, l16);
      else
        row_ok = ml < rows;
      if (!row_ok) continue;
      const int64_t orow = out_row0 + ml;
      if (kCanSplit && splits > 1) {
        // this split's fp32 partial tile (plain stores, summed later)
        float* w = p.ws + split * p.ws_stride + orow * p.n;
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const int n = n0 + wn * WTN + 16 * i + 4 * lq;
          if (n >= p.n) continue;
          if (p.vec_out && n + 3 < p.n) {
            *reinterpret_cast<float4*>(w + n) = float4{acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < p.n) w[n + r] = acc[i][j][r];
          }
        }
        continue;
      }
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int n = n0 + wn * WTN + 16 * i + 4 * lq;
        if (n >= p.n) continue;
        if constexpr (kFp32Out) {
          float* d = static_cast<float*>(p.out) + orow * p.n + n;
          if (p.vec_out && n + 3 < p.n) {
            __builtin_nontemporal_store(f4nt{acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]},
                                        reinterpret_cast<f4nt*>(d));
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < p.n) d[r] = acc[i][j][r];  // acc started from D
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
    stores_pending = xfer && exact_stores && !kSwiGLU;

    // ---- next tile ----
    if (!xfer) nxt = next_live(t_next);
    qbase += nkb;
    gpar = (gpar + (nkb + kGrp - 1) / kGrp) & 1;
    cur = nxt;
    first = false;
  }
  wait_vm<0>();  // no DMA (dead blocks included) outlives the workgroup
}

template <int BM, int BN, int WM, int WN, int S, int KIND>
void launch_kind(dim3 g, dim3 b, hipStream_t stream, const Params& p) {
  if constexpr (!excluded(BM, BN, WM, KIND))
    hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, WM, WN, S, KIND>), g, b, 0, stream, p);
}

template <int BM, int BN, int WM, int WN, int S>
hipError_t launch_shape(int kind, const Params& p, int grid, hipStream_t stream) {
  dim3 g(grid), b(WM * WN * 64);
  if (excluded(BM, BN, WM, kind)) return hipErrorInvalidValue;
  switch (kind) {
    case KIND_DENSE:
      launch_kind<BM, BN, WM, WN, S, KIND_DENSE>(g, b, stream, p);
      break;
    case KIND_CONTIGUOUS:
      launch_kind<BM, BN, WM, WN, S, KIND_CONTIGUOUS>(g, b, stream, p);
      break;
    case KIND_MASKED:
      launch_kind<BM, BN, WM, WN, S, KIND_MASKED>(g, b, stream, p);
      break;
    case KIND_WGRAD:
      launch_kind<BM, BN, WM, WN, S, KIND_WGRAD>(g, b, stream, p);
      break;
    case KIND_KGROUPED:
      launch_kind<BM, BN, WM, WN, S, KIND_KGROUPED>(g, b, stream, p);
      break;
    case KIND_DENSE_POW2:
      launch_kind<BM, BN, WM, WN, S, KIND_DENSE_POW2>(g, b, stream, p);
      break;
    case KIND_BF16:
      launch_kind<BM, BN, WM, WN, S, KIND_BF16>(g, b, stream, p);
      break;
    case KIND_CONTIG_SWIGLU:
      launch_kind<BM, BN, WM, WN, S, KIND_CONTIG_SWIGLU>(g, b, stream, p);
      break;
    case KIND_CONTIG_POW2:
      launch_kind<BM, BN, WM, WN, S, KIND_CONTIG_POW2>(g, b, stream, p);
      break;
    case KIND_MASKED_POW2:
      launch_kind<BM, BN, WM, WN, S, KIND_MASKED_POW2>(g, b, stream, p);
      break;
    case KIND_CONTIG_BF16:
      launch_kind<BM, BN, WM, WN, S, KIND_CONTIG_BF16>(g, b, stream, p);
      break;
    case KIND_MASKED_BF16:
      launch_kind<BM, BN, WM, WN, S, KIND_MASKED_BF16>(g, b, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Split-K reduction: C = bf16(sum of the fp32 partials in split order).  One
// thread per 4 consecutive outputs of a row, one 16-byte load per split; the
// masked layout skips rows at or past masked_m of their group, which the
// GEMM kernel did not write either.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const Params p, int masked) {
  const int nq = (p.n + 3) / 4;
  const int64_t items = (int64_t)p.groups * p.m * nq;
  for (int64_t it = blockIdx.x * 256LL + threadIdx.x; it < items; it += (int64_t)gridDim.x * 256) {
    const int64_t row = it / nq;
    const int c = (int)(it - row * nq) * 4;
    if (masked) {
      const int g = (int)(row / p.m);
      if (row - (int64_t)g * p.m >= min(max(p.ctrl[g], 0), p.m)) continue;
    }
    const float* w = p.ws + row * p.n + c;
    uint16_t* o = static_cast<uint16_t*>(p.out) + row * p.n + c;
    if (p.vec_out && c + 3 < p.n) {
      float4 v = *reinterpret_cast<const float4*>(w);
      for (int sp = 1; sp < p.splits; ++sp) {
        const float4 u = *reinterpret_cast<const float4*>(w + sp * p.ws_stride);
        v.x += u.x;
        v.y += u.y;
        v.z += u.z;
        v.w += u.w;
      }
      const uint32_t lo = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16);
      *reinterpret_cast<uint2*>(o) = uint2{lo, hi};
    } else {
      for (int r = 0; r < 4 && c + r < p.n; ++r) {
        float v = w[r];
        for (int sp = 1; sp < p.splits; ++sp) v += w[sp * p.ws_stride + r];
        o[r] = f32_to_bf16(v);
      }
    }
  }
}

}  // namespace

hipError_t launch_splitk_reduce(int kind, const Params& p, hipStream_t stream) {
  const int layout = layout_of(kind);
  if (layout != KIND_DENSE && layout != KIND_MASKED && kind != KIND_BF16) return hipErrorInvalidValue;
  const int64_t items = (int64_t)p.groups * p.m * ((p.n + 3) / 4);
  const int64_t blocks = (items + 255) / 256;
  const int grid = (int)(blocks < 4096 ? (blocks > 0 ? blocks : 1) : 4096);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid), dim3(256), 0, stream, p, layout == KIND_MASKED ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch(int kind, const TileShape& s, const Params& p, int grid, hipStream_t stream) {
#define X(BM, BN, WM, WN, S) \
  if (s.bm == BM && s.bn == BN && s.wm == WM && s.wn == WN) return launch_shape<BM, BN, WM, WN, S>(kind, p, grid, stream);
  DG_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace dg
