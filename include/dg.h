/*
 * dg.h -- C ABI of the MI355X (gfx950) FP8 fine-grained-scaled NT GEMM library.
 *
 * The operation (DeepSeek DeepGEMM 中文讲解, "主要特点": FP8 GEMM with
 * fine-grained scaling, two-level accumulation on the vector units;
 * "使用示例": operands are (fp8 [M,K], fp32 [M,K/128]) and
 * (fp8 [N,K], fp32 [ceil(N/128),K/128]), output bf16 [M,N] allocated by the
 * caller; "适用条件": K must be a multiple of 128):
 *
 *     C[m,n] = bf16( sum_kb sa[m,kb] * sb[n/128,kb] * sum_{k in kb} A[m,k]*B[n,k] )
 *
 * with kb running over the 128-wide K blocks.  "NT" means both A and B are
 * stored K-contiguous (row-major A [M,K], B [N,K]).
 *
 * Conventions shared by every entry point:
 *   - every tensor pointer is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or keeps the caller's memory;
 *   - split K: for shapes with too few output tiles to occupy every compute
 *     unit (few rows, long K), the dense and masked calls split K over several
 *     workgroups and add the fp32 partials in a second kernel, in a fixed
 *     order (results are deterministic).  The partials (splits * rows * N * 4
 *     bytes, at most 256 MB) live in a workspace the library keeps per (device,
 *     stream) -- calls on one stream are ordered, so they share it -- taken
 *     from a memory pool the library owns per device and grown in the
 *     stream's order (no device synchronisation); it is the one piece of
 *     device memory the library holds beyond the caller's tensors, kept until
 *     the process ends.  At most 64 streams keep one; a call on any further
 *     stream takes a buffer for itself and returns it to the pool after its
 *     kernels.  If no buffer can be had the call runs without a split.  A call
 *     made while `stream` is being captured into a HIP graph never splits, so
 *     it allocates nothing and records only the GEMM kernel
 *     (dg_grouped_fp8_masked_noalloc keeps the split there, see below);
 *   - tensors are row-major with the last dimension contiguous;
 *   - fp8 = OCP E4M3FN bytes (what torch calls float8_e4m3fn); scales fp32;
 *   - K_b = K/128, NB = ceil(N/128);
 *   - a and b must be 16-byte aligned, scales 4-byte aligned, c 2-byte
 *     aligned (bf16) or d 4-byte aligned (fp32);
 *   - work is enqueued on `stream` and the call returns without waiting;
 *   - arguments are validated on the host BEFORE any HIP call; a bad argument
 *     returns a status and enqueues nothing.  No call aborts or throws.
 *   - device-resident control data (m_indices, masked_m) cannot be checked on
 *     the host; out-of-range values mean "skip": a row whose expert id is not
 *     in [0, G) is left untouched, masked_m[g] is clamped to [0, M_max].
 *   - environment overrides for tests and tuning, read at each call:
 *     DG_FORCE_TILE=BMxBNxWMxWN forces a tile instance (UNSUPPORTED if the kind
 *     has none), DG_FORCE_SPLITS=s forces s K splits where splitting is
 *     allowed, DG_LOG=1 prints each plan to stderr.  Results stay within the
 *     same accuracy bound either way.
 */
#ifndef DG_MI355X_H
#define DG_MI355X_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DG_SUCCESS = 0,
  DG_ERROR_INVALID_VALUE = 1, /* null pointer, a size <= 0, G <= 0           */
  DG_ERROR_UNSUPPORTED = 2,   /* K % 128 != 0, misalignment, layout limits   */
  DG_ERROR_LAUNCH = 3,        /* the HIP runtime reported a launch failure   */
  DG_ERROR_WORKSPACE = 4      /* a call's split-K partials exceed the fixed
                                 scratch of an allocation-free entry point   */
} dg_status;

/* Dense FP8 NT GEMM (DeepGEMM pages, "使用示例": the normal FP8 GEMM call).
 *   a  [M,K] fp8,  sa [M,K_b] fp32  (one scale per row and 128-wide K block)
 *   b  [N,K] fp8,  sb [NB,K_b] fp32 (one scale per 128x128 block)
 *   c  [M,N] bf16, every element written.
 * M, N >= 1; K >= 128 and K % 128 == 0. */
dg_status dg_gemm_fp8_nt(const void* a, const float* sa, const void* b, const float* sb,
                         void* c, int m, int n, int k, hipStream_t stream);

/* Dense FP8 NT GEMM with power-of-two (UE8M0) scales (DeepGEMM pages,
 * aikraft.ru support table: the newer architecture's scale format is packed
 * UE8M0, i.e. an 8-bit exponent).  Same operands, layouts and result as
 * dg_gemm_fp8_nt, but every scale in sa and sb must be an exact power of two
 * 2^e with -127 <= e <= 127 (stored as fp32): the block-scaled MFMA then
 * applies sa*sb inside the matrix unit and accumulates in fp32, with no
 * vector-unit promotion.  Only the exponent field of each scale is read; a
 * scale that is not such a power of two gives wrong results (no error). */
dg_status dg_gemm_fp8_nt_ue8m0(const void* a, const float* sa, const void* b, const float* sb,
                               void* c, int m, int n, int k, hipStream_t stream);

/* The same GEMM with the scales in the packed UE8M0 format (DeepGEMM pages,
 * aikraft.ru support table: packed UE8M0, four values in one torch.int).
 * Each int32 word holds the 8-bit biased exponents E of four consecutive
 * 128-wide K blocks, K block 4w + i in byte i (bits 8i..8i+7) of word w; the
 * scale is 2^(E - 127), E in 0..254 (E = 255 is the E8M0 NaN code and makes
 * the outputs it touches NaN).  Layouts, with K_w = ceil(K/512):
 *   sa [M, K_w] int32 (row r, word w: K blocks 4w..4w+3 of row r)
 *   sb [ceil(N/128), K_w] int32 (one exponent per 128x128 block)
 * The bytes of the last word past K/128 blocks are ignored.  The result is
 * bit-identical to dg_gemm_fp8_nt_ue8m0 with the fp32 scales 2^(E - 127).
 * sa, sb 4-byte aligned; the rest as dg_gemm_fp8_nt. */
dg_status dg_gemm_fp8_nt_ue8m0_packed(const void* a, const int32_t* sa, const void* b,
                                      const int32_t* sb, void* c, int m, int n, int k,
                                      hipStream_t stream);

/* Dense BF16 NT GEMM (DeepGEMM pages: aikraft.ru lists BF16 GEMM beside FP8
 * in its support table; DeepSeek DeepGEMM 中文讲解, "未来计划": BF16 support).
 * The same scheduler, operand staging and layouts as the FP8 path, with bf16
 * MFMAs accumulating in fp32 and no scales:
 *   a [M,K] bf16, b [N,K] bf16, c [M,N] bf16 = round-to-nearest-even(sum_k a*b),
 *   every element written.
 * M, N >= 1; K >= 64, K % 64 == 0 and K <= 2^22. */
dg_status dg_gemm_bf16_nt(const void* a, const void* b, void* c, int m, int n, int k,
                          hipStream_t stream);

/* The two grouped layouts in BF16 (the BF16 GEMM of dg_gemm_bf16_nt on the
 * grouped calls' scheduling): bf16 operands, fp32 accumulation, no scales,
 * round-to-nearest-even bf16 output.  Row rules, layout limits and results as
 * dg_grouped_fp8_contiguous / dg_grouped_fp8_masked:
 *   contiguous: a [M_total,K], b [G,N,K], c [M_total,N], m_indices [M_total]
 *   masked:     a [G,M_max,K], b [G,N,K], c [G,M_max,N], masked_m [G]
 * K >= 64, K % 64 == 0 and K <= 2^22; a, b 16-byte aligned. */
dg_status dg_grouped_bf16_contiguous(const void* a, const void* b, void* c, const int32_t* m_indices,
                                     int m_total, int n, int k, int num_groups, hipStream_t stream);
dg_status dg_grouped_bf16_masked(const void* a, const void* b, void* c, const int32_t* masked_m,
                                 int num_groups, int m_max, int n, int k, hipStream_t stream);

/* MoE grouped GEMM, contiguous layout (DeepGEMM pages, "分组 GEMM": training
 * forward and inference prefill; "使用示例": m_indices gives each LHS row its
 * group).  The rows of all experts are stacked into one LHS:
 *   a  [M_total,K] fp8, sa [M_total,K_b] fp32
 *   b  [G,N,K] fp8,     sb [G,NB,K_b] fp32
 *   m_indices [M_total] int32 (device): expert of each row, -1 = padding row
 *   c  [M_total,N] bf16: rows with an id in [0,G) are written, others untouched.
 * Layout limit: M_total % 128 == 0 and every aligned 128-row block holds rows
 * of at most one expert (each expert's segment padded to a multiple of 128
 * with -1 rows); rows of any other expert inside such a block are skipped. */
dg_status dg_grouped_fp8_contiguous(const void* a, const float* sa, const void* b,
                                    const float* sb, void* c, const int32_t* m_indices,
                                    int m_total, int n, int k, int num_groups,
                                    hipStream_t stream);

/* MoE grouped GEMM, contiguous layout, fused with SwiGLU and the FP8
 * re-quantise of its output (the Russian overview of the DeepGEMM pages,
 * "Ключевые функции: Mega MoE и индексация": Mega MoE fuses an expert's first
 * linear layer with the SwiGLU activation; the second FP8 GEMM takes its input
 * with 1x128 scales).  Same operands and row rules as
 * dg_grouped_fp8_contiguous, with the first linear layer's stacked projection
 * as B:
 *   b [G,N,K] fp8 with N = 2I: rows [0,I) are the gate projection, rows
 *     [I,2I) the up projection (the column layout of
 *     dg_swiglu_quantize_fp8_1x128); sb [G,N/128,K_b] fp32
 *   q [M_total,I] fp8 e4m3, s [M_total,I/128] fp32: for every row with an id
 *     in [0,G), exactly what dg_grouped_fp8_contiguous into a bf16 C
 *     [M_total,N] followed by dg_swiglu_quantize_fp8_1x128 on C gives, bit for
 *     bit (the bf16 rounding of C included); other rows untouched.
 * The bf16 C is never written to memory.  N % 256 == 0 (I % 128 == 0),
 * (N/2 + 128) * K < 2^32, q and s 4-byte aligned.  Inputs must keep h finite
 * in fp32. */
dg_status dg_grouped_fp8_contiguous_swiglu(const void* a, const float* sa, const void* b,
                                           const float* sb, void* q, float* s,
                                           const int32_t* m_indices, int m_total, int n, int k,
                                           int num_groups, hipStream_t stream);

/* MoE grouped GEMM, masked layout (DeepGEMM pages, "分组 GEMM": inference
 * decode, the graph-captured case -- the valid row counts stay on the device
 * and no host synchronisation happens).
 *   a  [G,M_max,K] fp8, sa [G,M_max,K_b] fp32
 *   b  [G,N,K] fp8,     sb [G,NB,K_b] fp32
 *   masked_m [G] int32 (device): rows r < min(max(masked_m[g],0), M_max) of
 *            group g are computed
 *   c  [G,M_max,N] bf16: only those rows are written, others untouched. */
dg_status dg_grouped_fp8_masked(const void* a, const float* sa, const void* b,
                                const float* sb, void* c, const int32_t* masked_m,
                                int num_groups, int m_max, int n, int k, hipStream_t stream);

/* The masked-layout GEMM above for callers that cannot allocate device memory
 * (code being captured into a HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, layouts and results as
 * dg_grouped_fp8_masked; the call allocates nothing: when K is split, the
 * fp32 partials go to a fixed scratch array of 64 MB that the library holds
 * on each GPU it runs on until the process ends (so split K is kept under
 * capture, where dg_grouped_fp8_masked drops it).  Every call on a GPU
 * shares that GPU's scratch: calls that overlap on one GPU (other streams,
 * or graphs replayed concurrently) race and must be ordered by the caller.
 * A call whose partials (splits * G * M_max * N * 4 bytes for the planned
 * split) exceed the scratch returns DG_ERROR_WORKSPACE and enqueues nothing. */
dg_status dg_grouped_fp8_masked_noalloc(const void* a, const float* sa, const void* b,
                                        const float* sb, void* c, const int32_t* masked_m,
                                        int num_groups, int m_max, int n, int k,
                                        hipStream_t stream);

/* The two grouped layouts with packed UE8M0 scales (the format of
 * dg_gemm_fp8_nt_ue8m0_packed: int32 words holding the biased exponents E of
 * four consecutive 128-wide K blocks, K block 4w + i in byte i; scale
 * 2^(E - 127), E = 255 NaN; bytes past the last K block ignored), applied
 * inside the block-scaled MFMA.  Operands, row rules, results and alignment
 * as dg_grouped_fp8_contiguous / dg_grouped_fp8_masked, with K_w = ceil(K/512):
 *   contiguous: sa [M_total,K_w] int32, sb [G,ceil(N/128),K_w] int32
 *   masked:     sa [G,M_max,K_w] int32, sb [G,ceil(N/128),K_w] int32
 * (the masked call may split K like dg_grouped_fp8_masked, with the same
 * workspace rules). */
dg_status dg_grouped_fp8_contiguous_ue8m0_packed(const void* a, const int32_t* sa, const void* b,
                                                 const int32_t* sb, void* c,
                                                 const int32_t* m_indices, int m_total, int n,
                                                 int k, int num_groups, hipStream_t stream);
dg_status dg_grouped_fp8_masked_ue8m0_packed(const void* a, const int32_t* sa, const void* b,
                                             const int32_t* sb, void* c,
                                             const int32_t* masked_m, int num_groups,
                                             int m_max, int n, int k, hipStream_t stream);

/* Weight-gradient FP8 GEMM with fp32 output accumulated into D (DeepGEMM
 * pages, "反向传播中的梯度计算": dW from FP8 inputs, fp32 result without an
 * explicit cast).  K is the token dimension; both operands are token-
 * contiguous and scaled per row and per 128 tokens:
 *   a [M,K] fp8, sa [M,K_b] fp32;  b [N,K] fp8, sb [N,K_b] fp32
 *   d [M,N] fp32, updated in place: d += sum_kb sa[m,kb]*sb[n,kb]*block sum. */
dg_status dg_wgrad_fp8_nt(const void* a, const float* sa, const void* b, const float* sb,
                          float* d, int m, int n, int k, hipStream_t stream);

/* K-grouped weight gradient (same passage: per-expert gradients in one call).
 * The token ranges of the G groups are concatenated along K:
 *   a [M,T] fp8, sa [M,T/128]; b [N,T] fp8, sb [N,T/128]; T = sum ks[g]
 *   ks_host [G] int32 on the HOST: token count of each group, each a
 *           multiple of 128 (0 allowed: that group's D is left as it is)
 *   d [G,M,N] fp32, d[g] += the weight gradient over group g's tokens.
 * Layout limit: G <= 256. */
dg_status dg_k_grouped_wgrad_fp8_nt(const void* a, const float* sa, const void* b,
                                    const float* sb, float* d, const int32_t* ks_host,
                                    int num_groups, int m, int n, hipStream_t stream);

/* ---- FP8 quantiser: makes the operands above from fp32 ------------------
 * DeepGEMM pages (DeepSeek DeepGEMM 中文讲解, "注意事项": FP8 needs dynamic
 * scale factors from amax; "使用示例": scale granularity [M, K/128] for
 * activations and [ceil(N/128), K/128] for weights).  For each group:
 *     amax = max |x|,  s = amax / 448 (s = 1 for an all-zero group),
 *     q    = e4m3 round-to-nearest-even( clamp(x / s, -448, 448) )
 * with both divisions in IEEE fp32.  Inputs must be finite (a NaN or
 * infinity gives unspecified codes and scales for its group, no error), and
 * a group's amax must be 0 or at least 2^-140 (below that s would underflow
 * to zero; such a group gets unspecified codes).
 * x must be 16-byte aligned, s 4-byte aligned; every output element is
 * written.  Sizes must fit the 32-bit arguments. */

/* Activations: one scale per row and 128 consecutive columns.
 *   x [M,K] fp32 -> q [M,K] fp8 (4-byte aligned), s [M,K/128] fp32.
 * M >= 1; K >= 128 and K % 128 == 0. */
dg_status dg_quantize_fp8_1x128(const float* x, void* q, float* s, int m, int k,
                                hipStream_t stream);

/* Weights: one scale per 128x128 block (the last row block holds the rows
 * that exist).
 *   x [N,K] fp32 -> q [N,K] fp8 (4-byte aligned), s [ceil(N/128),K/128] fp32.
 * N >= 1; K >= 128 and K % 128 == 0. */
dg_status dg_quantize_fp8_128x128(const float* x, void* q, float* s, int n, int k,
                                  hipStream_t stream);

/* Both rules with power-of-two scales in the packed UE8M0 format that the
 * *_ue8m0_packed GEMMs take (DeepGEMM pages, aikraft.ru support table: packed
 * UE8M0, four values in one torch.int).  The pages give no rule for choosing
 * such a scale; taken: the smallest 2^(E - 127), E in [0, 254], not below the
 * fp32 rule's s = amax / 448 (1 for an all-zero group), so
 *     q = e4m3 round-to-nearest-even( clamp(x / 2^(E - 127), -448, 448) )
 * with an exact quotient.  The codes E are packed four per int32 word along
 * K, group 4w + i in byte i of word w; the bytes past the last group are 0:
 *   1x128:   x [M,K] fp32 -> q [M,K] fp8, s [M, ceil(K/512)] int32
 *   128x128: x [N,K] fp32 -> q [N,K] fp8, s [ceil(N/128), ceil(K/512)] int32
 * Sizes, alignment and error rules as the fp32-scale calls above. */
dg_status dg_quantize_fp8_1x128_ue8m0(const float* x, void* q, int32_t* s, int m, int k,
                                      hipStream_t stream);
dg_status dg_quantize_fp8_128x128_ue8m0(const float* x, void* q, int32_t* s, int n, int k,
                                        hipStream_t stream);

/* Token-contiguous operands of the weight-gradient GEMMs (DeepGEMM pages,
 * "反向传播中的梯度计算"): the 1x128 rule applied to the transpose of x, i.e.
 * groups of 128 consecutive tokens of one feature.
 *   x [T,F] fp32 (tokens x features) -> q [F,T] fp8 (16-byte aligned),
 *   s [F,T/128] fp32.
 * T >= 128 and T % 128 == 0; F >= 1 and F % 4 == 0. */
dg_status dg_quantize_fp8_1x128_transposed(const float* x, void* q, float* s, int t, int f,
                                           hipStream_t stream);

/* ---- SwiGLU + FP8 re-quantise between an expert's two linear layers -----
 * DeepGEMM pages (the Russian overview, "Ключевые функции: Mega MoE и
 * индексация": Mega MoE fuses an expert's first linear layer, SwiGLU and the
 * second linear layer; the second FP8 GEMM needs its input re-quantised with
 * 1x128 scales).  The column layout is a reading, the pages give none:
 *   c [M, 2I] bf16, the first GEMM's output: gate = c[:, 0:I], up = c[:, I:2I]
 *   h = silu(gate) * up = gate / (1 + e^-gate) * up, in fp32
 *   q [M, I] fp8 e4m3, s [M, I/128] fp32: the 1x128 rule of
 *   dg_quantize_fp8_1x128 applied to h (amax / 448, s = 1 for a zero group).
 * h is within a few fp32 ulp of exact for every gate and the quotient is
 * h * RN(1/s), so a code can differ from exact evaluation only where h / s
 * lies within about 2^-20 (relative) of the midpoint between two e4m3 values;
 * the scales match exact evaluation to within the same relative margin.
 * Every row is independent (grouped layouts pass their whole row range;
 * padding rows get codes of whatever they hold).  Inputs must keep h finite
 * in fp32.  c 16-byte aligned, q 8-byte, s 4-byte.  M >= 1; I >= 128,
 * I % 128 == 0, 2I fits an int.  Every output element is written. */
dg_status dg_swiglu_quantize_fp8_1x128(const void* c, void* q, float* s, int m, int i,
                                       hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char* dg_status_string(dg_status s);

/* ---- introspection (host only, no GPU needed) ---------------------------- */

typedef enum {
  DG_KIND_DENSE = 0,
  DG_KIND_CONTIGUOUS = 1,
  DG_KIND_MASKED = 2,
  DG_KIND_WGRAD = 3,
  DG_KIND_K_GROUPED_WGRAD = 4,
  DG_KIND_DENSE_POW2 = 5,     /* dg_gemm_fp8_nt_ue8m0, dg_gemm_fp8_nt_ue8m0_packed */
  DG_KIND_BF16 = 6,           /* dg_gemm_bf16_nt (k counts bf16 values) */
  DG_KIND_CONTIGUOUS_SWIGLU = 7, /* dg_grouped_fp8_contiguous_swiglu (n = 2I) */
  DG_KIND_CONTIGUOUS_POW2 = 8,   /* dg_grouped_fp8_contiguous_ue8m0_packed */
  DG_KIND_MASKED_POW2 = 9,       /* dg_grouped_fp8_masked_ue8m0_packed */
  DG_KIND_CONTIGUOUS_BF16 = 10,  /* dg_grouped_bf16_contiguous (k counts bf16 values) */
  DG_KIND_MASKED_BF16 = 11       /* dg_grouped_bf16_masked (k counts bf16 values) */
} dg_kind;

/* Tile configuration the per-shape heuristic picks (DeepGEMM pages: block
 * sizes and wave counts are chosen automatically per shape; non-power-of-two
 * block sizes raise GPU utilisation).  `m` is the rows per group (M, M_total,
 * M_max), `k` the K (or total tokens) and `num_cus` the compute-unit count the
 * persistent grid is sized for. */
typedef struct {
  int block_m;      /* output rows per workgroup tile                        */
  int block_n;      /* output columns per workgroup tile                     */
  int waves_m;      /* waves along M (waves_m * waves_n is 4 or 8)           */
  int waves_n;      /* waves along N                                         */
  int tiles;        /* tile count (an upper bound for the masked layout)     */
  int grid;         /* persistent workgroups launched                        */
  int k_splits;     /* workgroups sharing one output tile along K (1 = none) */
  int kernel;       /* always 0: every layout runs on the general kernel    */
} dg_tile_config;

dg_status dg_select_config(int kind, int m, int n, int k, int num_groups, int num_cus,
                           dg_tile_config* out);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int dg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DG_MI355X_H */
