// Internal launch interface between the host library (bpt_api.cpp) and the
// gfx950 kernels. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bpt {

// BPT_OK if the current HIP device is a gfx950, else BPT_ERR_DEVICE (cached
// per device).
int check_device();

// Epilogue kinds of the GEMM kernels.
enum Epi : int {
  EPI_QK = 0,    // + bias, scatter into head-major Q and K   [b, nh, s, d]
  EPI_VT = 1,    // + bias, scatter into transposed V          [b, nh, d, s'] (s' = key-permuted)
  EPI_RESID = 2, // out = acc + bias + resid                   [M, N] row-major
  EPI_RELU = 3,  // out = max(0, acc + bias)                   [M, N] row-major
  EPI_QKV = 4,   // fp32 path: + bias, scatter into Q, K, V    [b, nh, s, d]
  EPI_RESID_DROP = 5, // out = resid + dropout(acc + bias)         [M, N] row-major
  EPI_MASK = 6,  // out = (acc + bias) where resid > 0, else 0     [M, N] row-major
  EPI_ACC32 = 7, // fp32 out (+)= acc + bias                    [M, N] row-major fp32
};

struct GemmEpilogue {
  const void *bias = nullptr;  // indexed by the output column n
  const void *resid = nullptr; // [M, ld_resid]
  void *out = nullptr;         // [M, ld_out]
  int64_t ld_out = 0, ld_resid = 0;
  // scatter targets (EPI_QK / EPI_VT / EPI_QKV)
  void *q = nullptr, *k = nullptr, *v = nullptr;
  int64_t seq = 0, heads = 0, head_dim = 0, hidden = 0;
  float q_scale = 1.f; // EPI_QK: factor applied to the Q columns before rounding
  // EPI_RESID_DROP: training-mode dropout of the branch acc + bias. Row m of
  // the product is token row0 + m; element (token, column) is dropped iff
  // its 16-bit uniform of site drop_site under drop_seed is below
  // drop_threshold, and kept values are multiplied by drop_scale.
  uint64_t drop_seed = 0;
  uint32_t drop_site = 0;
  uint32_t drop_threshold = 0;
  float drop_scale = 1.f;
  int64_t row0 = 0;
  // EPI_ACC32: add to the fp32 output instead of overwriting it
  int accumulate = 0;
  // EPI_ACC32 launched with gridDim.y = splits > 1: workgroup layer z covers
  // K range [z·K, (z+1)·K) of A and Bt and writes its own fp32 output at
  // out + z·split_stride
  int64_t split_stride = 0;
  // token-major EPI_ACC32 (launch_gemm_acc32_tok): the number of valid K rows
  int64_t mn_rows = 0;
};

// Keep flags of dropout site `site` for tokens token0 .. token0+tokens-1 and
// channels 0..channels-1 (channels % 16 == 0), one byte per element (1 =
// kept), row-major [tokens, channels].
hipError_t launch_dropout_keep(uint8_t *keep, int64_t tokens, int64_t channels, int64_t token0,
                               uint64_t seed, uint32_t site, uint32_t threshold, hipStream_t stream);

// out = in ∘ keep · scale for bf16 [rows, cols] (row stride ld elements,
// cols % 16 == 0): row r is token token0 + r of dropout site `site`; each
// result rounded to bf16 once. in and out must not overlap.
hipError_t launch_dropout_scale_bf16(const void *in, void *out, int64_t rows, int64_t cols,
                                     int64_t ld, int64_t token0, uint64_t seed, uint32_t site,
                                     uint32_t threshold, float scale, hipStream_t stream);

// C[M, N] = A[M, K] · Bt[N, K]^T on MFMA (bf16 in, fp32 accumulate), then the
// epilogue. Requires K % 64 == 0, N % 64 == 0; M arbitrary.
hipError_t launch_gemm_bf16(int epi, const void *A, int64_t lda, const void *Bt, int64_t ldb,
                            int64_t M, int64_t N, int64_t K, const GemmEpilogue &ep,
                            hipStream_t stream);

// fp32 weight-gradient product out[M, N] (+)= A·Btᵀ (A [M, K], Bt [N, K]
// K-contiguous) with the K range split over `splits` workgroup layers that
// write partial products to part [splits, M, N]; a second kernel adds them
// in a fixed order (so the result does not depend on timing). splits = 1 is
// the plain EPI_ACC32 product. K % (32·splits) == 0; out is dense (ld = N).
hipError_t launch_gemm_acc32_split(const void *A, int64_t lda, const void *Bt, int64_t ldb, int64_t M,
                                   int64_t N, int64_t K, int splits, float *part, float *out,
                                   int accumulate, const void *zero_bias, hipStream_t stream);
// The same product from token-major operands, out[M, N] (+)= Aᵀ·B with
// A [K, M] and B [K, N] (row strides lda >= M, ldb >= N, multiples of 8):
// no transposed copies; any K (rows past K read as zero); the K range is
// split over `splits` layers of round_up(K, 32) / splits rows each
// (round_up(K, 32) % (32·splits) == 0).
hipError_t launch_gemm_acc32_tok(const void *A, int64_t lda, const void *Bt, int64_t ldb, int64_t M,
                                 int64_t N, int64_t K, int splits, float *part, float *out,
                                 int accumulate, const void *zero_bias, hipStream_t stream);
// out[i] (+)= Σ_k part[k·n + i], k = 0..nparts-1 in order
hipError_t launch_sum_parts(const float *part, int64_t nparts, int64_t n, float *out, int accumulate,
                            hipStream_t stream);

// Layer backward helpers (attn_bwd.hip).
// dQ, dK, dV of the blockwise attention into dQKV [b, s, 3h] (columns
// [0, h), [h, 2h), [2h, 3h)): Qs (pre-scaled as for the forward), K, V, dO
// head-major [b·nh, s, d]; dOT the key-permuted transpose of dO [b·nh, d, sp]
// (zero past s, sp % 64 == 0); nlse = -lse from the forward; nDq = -rowsum(dO ∘ O)
// [b·nh, s]; s % 16 == 0.
hipError_t launch_attention_bwd_bf16(const void *Qs, const void *K, const void *V, const void *dO,
                                     const void *dOT, const float *nlse, const float *nDq, void *dQKV,
                                     int64_t batch, int64_t seq, int64_t sp, int64_t heads,
                                     int64_t head_dim, int causal, hipStream_t stream);
// X [nb, s, d] -> XT [nb, d, sp], key-permuted positions, zero past s
hipError_t launch_transpose_perm(const void *X, void *XT, int64_t nb, int64_t seq, int64_t sp,
                                 int64_t head_dim, hipStream_t stream);
// The inverse for the forward's V^T: XT [nb, D, seq] (row stride seq, position
// p holding token vt_perm(p)) -> X [nb, seq, D]. seq % 16 == 0, D % 32 == 0.
hipError_t launch_untranspose_perm(const void *XT, void *X, int64_t nb, int64_t seq,
                                   int64_t head_dim, hipStream_t stream);
// nDq[bh, q] = -Σ_i dO[bh, q, i] · O[b, q, head·d + i] (dO head-major, O token-major)
hipError_t launch_attention_delta(const void *dO, const void *O, float *nDq, int64_t batch,
                                  int64_t seq, int64_t heads, int64_t head_dim, hipStream_t stream);
// bf16 X [R, C] (row stride ldx) -> XT [C, Rp], columns R .. Rp-1 zero;
// C and ldx multiples of 64 and 8, Rp >= R a multiple of 8
hipError_t launch_transpose_bf16(const void *X, int64_t ldx, void *XT, int64_t R, int64_t C,
                                 int64_t Rp, hipStream_t stream);
// the same, and out[c] (+)= Σ_r X[r, c] in fp32 in a fixed order (per
// 64-row tile, then over the tiles); part holds transpose_row_tiles(Rp) × C
// floats of scratch
int64_t transpose_row_tiles(int64_t Rp);
// out[c] (+)= Σ_r X[r, c] alone (the same passes, no transposed copy); part
// holds transpose_row_tiles(R rounded up to 8) × C floats
hipError_t launch_colsum(const void *X, int64_t ldx, int64_t R, int64_t C, float *part, float *out,
                         int accumulate, hipStream_t stream);
hipError_t launch_transpose_colsum(const void *X, int64_t ldx, void *XT, int64_t R, int64_t C,
                                   int64_t Rp, float *part, float *out, int accumulate,
                                   hipStream_t stream);
hipError_t launch_fill_u32(void *p, int64_t n, uint32_t v, hipStream_t stream);

// fp32 path: C[M, N] = A[M, K] · Bt[N, K]^T on the vector ALU in fp32.
hipError_t launch_gemm_f32(int epi, const float *A, int64_t lda, const float *Bt, int64_t ldb,
                           int64_t M, int64_t N, int64_t K, const GemmEpilogue &ep,
                           hipStream_t stream);

// Blockwise attention, bf16: Q, K [b·nh, s, d], Vt [b·nh, d, s'] -> A [b, s, nh·d].
// Q must already be multiplied by attention_q_scale(d) = log2(e)/sqrt(d).
// rows: query rows per workgroup (16, 32, 64, 128 or 256); keys: keys per
// LDS stage (16, 32 or 64). nlse (optional, fp32 [b·nh, s], rows 256 and
// keys 64 only): each row's log2-sum-exp2 of its scores, negated.
hipError_t launch_attention_bf16(const void *Q, const void *K, const void *Vt, void *A,
                                 int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                                 int causal, hipStream_t stream, float *nlse = nullptr,
                                 int rows = 256, int keys = 64);
// The attention tile of block sizes B_q, B_kv: the largest of 256, 128, 64,
// 32, 16 query rows that divides B_q (a query block is B_q / rows
// workgroups), and the largest of 64, 32, 16 keys that divides B_kv (a
// key/value block is B_kv / keys stages).
int attention_tile_rows(int64_t B_q);
int attention_stage_keys(int64_t B_kv);

// The fp32 attention's fixed tile: query rows per workgroup, keys per LDS
// stage (one thread per query row; B_q and B_kv do not change it).
constexpr int kF32AttnRows = 64, kF32AttnKeys = 32;

// Blockwise attention, fp32: Q, K, V [b·nh, s, d] -> A [b, s, nh·d].
hipError_t launch_attention_f32(const float *Q, const float *K, const float *V, float *A,
                                int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                                int causal, hipStream_t stream);

inline float attention_q_scale(int64_t head_dim) {
  return 1.4426950408889634f / __builtin_sqrtf((float)head_dim);
}

} // namespace bpt
