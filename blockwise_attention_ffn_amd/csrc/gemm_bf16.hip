// bf16 GEMM on CDNA4 matrix cores with fused epilogues.
//
// Serves the four dense contractions of the BPT layer (BPT paper review, §三
// "核心公式" and Algorithm 1): the fused QKV projection over the whole sequence
// (epilogue: bias, split into heads), the output projection with the first
// residual, the FFN up-projection with bias and ReLU, and the FFN
// down-projection with the second residual.
//
// C[M, N] = A[M, K] · Bt[N, K]^T. Both operands are K-contiguous, which is
// what the v_mfma_f32_32x32x16_bf16 operand layout wants (each lane holds 8
// consecutive K values of one row of A and one column of B).
//
// Tiling: 256×256 output tile per workgroup of 4 waves (2×2), each wave a
// 128×128 sub-tile = 4×4 MFMA blocks of 32×32 (256 fp32 accumulators per
// lane, held in the AGPR half of the unified register file). K advances by 64
// per step through two LDS buffers (2 × 64 KiB): global loads of step k+1 are
// in flight while step k runs on the matrix cores. LDS rows are 128 B; the
// 16-byte chunk index is XOR-swizzled with (row & 7) so that both the staging
// stores and the fragment loads hit 8 distinct chunks per 8 lanes.
//
// Orientation: with SWAP the MFMA computes Bt·A^T blocks, so each lane holds
// one output ROW and 4 consecutive output COLUMNS per register group, which
// turns row-major epilogue stores into 8-byte vector stores. Without SWAP a
// lane holds 4 consecutive ROWS of one column, which is what the transposed-V
// scatter needs.
#include "bpt_internal.h"

namespace bpt {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 256, TN = 256, TK = 64;
constexpr int NT = 256;
constexpr int TILE_ELEMS = TM * TK; // one operand tile in LDS (bf16 elements)

// Key position inside a 16-key group in the transposed-V layout: bits 2 and 3
// swapped, so that the 8 keys one lane feeds to the P·V MFMA are contiguous.
__device__ __forceinline__ int64_t vt_perm(int64_t t) {
  return (t & ~int64_t(12)) | ((t & 4) << 1) | ((t & 8) >> 1);
}

__device__ __forceinline__ float bf2f(bf16 v) { return (float)v; }

template <int EPI, bool SWAP>
__global__ __launch_bounds__(NT, 1) void gemm_bf16_kernel(const bf16 *__restrict__ A, int64_t lda,
                                                          const bf16 *__restrict__ Bt, int64_t ldb,
                                                          int M, int N, int K, GemmEpilogue ep) {
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * 2 * TILE_ELEMS];

  const int tiles_m = (M + TM - 1) / TM;
  const int tiles_n = (N + TN - 1) / TN;
  const int total = tiles_m * tiles_n;

  // Workgroups go round-robin to the 8 XCDs; give each XCD a contiguous run
  // of logical tiles so that its L2 sees neighbouring A and B panels.
  int bid = blockIdx.x;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  // Grouped ordering: 8 tile-rows share each B panel sweep.
  constexpr int GROUP = 8;
  const int in_group = GROUP * tiles_n;
  const int group = bid / in_group;
  const int first_m = group * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (bid % in_group) % gsz;
  const int tn = (bid % in_group) / gsz;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, g = lane >> 5;

  // staging: thread -> (row lr + 32 i, 16-byte chunk lc)
  const int lc = tid & 7;
  const int lr = tid >> 3;
  const bf16 *a_src[8];
  const bf16 *b_src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int ra = min(tm * TM + lr + 32 * i, M - 1);
    int rb = min(tn * TN + lr + 32 * i, N - 1);
    a_src[i] = A + (int64_t)ra * lda + lc * 8;
    b_src[i] = Bt + (int64_t)rb * ldb + lc * 8;
  }
  u32x4 ra[8], rb[8];

  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ra[i] = *reinterpret_cast<const u32x4 *>(a_src[i] + kt * TK);
      rb[i] = *reinterpret_cast<const u32x4 *>(b_src[i] + kt * TK);
    }
  };
  auto sstore = [&](int buf) {
    bf16 *As = smem + buf * 2 * TILE_ELEMS;
    bf16 *Bs = As + TILE_ELEMS;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = lr + 32 * i;
      const int off = row * TK + ((lc ^ (row & 7)) << 3);
      *reinterpret_cast<u32x4 *>(As + off) = ra[i];
      *reinterpret_cast<u32x4 *>(Bs + off) = rb[i];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = K / TK;
  gload(0);
  sstore(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const bf16 *As = smem + buf * 2 * TILE_ELEMS;
    const bf16 *Bs = As + TILE_ELEMS;
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      const int kc = ks * 2 + g;
      bf16x8 af[4], bfv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + l32;
        af[i] = *reinterpret_cast<const bf16x8 *>(As + row * TK + ((kc ^ (row & 7)) << 3));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wn * 128 + j * 32 + l32;
        bfv[j] = *reinterpret_cast<const bf16x8 *>(Bs + row * TK + ((kc ^ (row & 7)) << 3));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (SWAP)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfv[j], af[i], acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfv[j], acc[i][j], 0, 0, 0);
        }
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  const bf16 *bias = reinterpret_cast<const bf16 *>(ep.bias);
  if constexpr (SWAP) {
    // lane: output row m, 4 consecutive columns n .. n+3 per register group
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = tm * TM + wm * 128 + i * 32 + l32;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int n = tn * TN + wn * 128 + j * 32 + r4 * 8 + g * 4;
          if (n >= N) continue;
          float v[4];
          const bf16x4 bv = *reinterpret_cast<const bf16x4 *>(bias + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][r4 * 4 + e] + bf2f(bv[e]);
          bf16 *dst;
          if constexpr (EPI == EPI_QK) {
            const int64_t h = ep.hidden, D = ep.head_dim, s = ep.seq;
            const int64_t which = n / h, rem = n - which * h;
            const int64_t head = rem / D, d = rem - head * D;
            const int64_t bi = m / s, t = m - bi * s;
            bf16 *base = reinterpret_cast<bf16 *>(which == 0 ? ep.q : ep.k);
            dst = base + ((bi * ep.heads + head) * s + t) * D + d;
          } else if constexpr (EPI == EPI_RESID) {
            const bf16x4 rv = *reinterpret_cast<const bf16x4 *>(
                reinterpret_cast<const bf16 *>(ep.resid) + (int64_t)m * ep.ld_resid + n);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += bf2f(rv[e]);
            dst = reinterpret_cast<bf16 *>(ep.out) + (int64_t)m * ep.ld_out + n;
          } else { // EPI_RELU
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], 0.f);
            dst = reinterpret_cast<bf16 *>(ep.out) + (int64_t)m * ep.ld_out + n;
          }
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
          *reinterpret_cast<bf16x4 *>(dst) = o;
        }
      }
    }
  } else {
    // lane: output column n, 4 consecutive rows m .. m+3 per register group
    static_assert(EPI == EPI_VT, "the non-swapped orientation serves the V^T scatter");
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = tn * TN + wn * 128 + j * 32 + l32;
      if (n >= N) continue;
      const float bn = bf2f(bias[n]);
      const int64_t D = ep.head_dim, s = ep.seq;
      const int64_t head = n / D, d = n - head * D;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int m = tm * TM + wm * 128 + i * 32 + r4 * 8 + g * 4;
          if (m >= M) continue;
          const int64_t bi = m / s, t = m - bi * s;
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)(acc[i][j][r4 * 4 + e] + bn);
          bf16 *dst = reinterpret_cast<bf16 *>(ep.v) + ((bi * ep.heads + head) * D + d) * s +
                      vt_perm(t);
          *reinterpret_cast<bf16x4 *>(dst) = o;
        }
      }
    }
  }
}

} // namespace

hipError_t launch_gemm_bf16(int epi, const void *A, int64_t lda, const void *Bt, int64_t ldb,
                            int64_t M, int64_t N, int64_t K, const GemmEpilogue &ep,
                            hipStream_t stream) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  if (K % TK != 0 || N % 64 != 0) return hipErrorInvalidValue;
  const int64_t tiles = ((M + TM - 1) / TM) * ((N + TN - 1) / TN);
  if (tiles > INT32_MAX || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
    return hipErrorInvalidValue;
  dim3 grid((unsigned)tiles), block(NT);
  const bf16 *a = reinterpret_cast<const bf16 *>(A);
  const bf16 *b = reinterpret_cast<const bf16 *>(Bt);
  switch (epi) {
  case EPI_QK:
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI_QK, true>), grid, block, 0, stream, a, lda, b, ldb,
                       (int)M, (int)N, (int)K, ep);
    break;
  case EPI_VT:
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI_VT, false>), grid, block, 0, stream, a, lda, b, ldb,
                       (int)M, (int)N, (int)K, ep);
    break;
  case EPI_RESID:
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI_RESID, true>), grid, block, 0, stream, a, lda, b,
                       ldb, (int)M, (int)N, (int)K, ep);
    break;
  case EPI_RELU:
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI_RELU, true>), grid, block, 0, stream, a, lda, b, ldb,
                       (int)M, (int)N, (int)K, ep);
    break;
  default:
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

} // namespace bpt
