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
// lane, in the AGPR half of the unified register file). K advances by 64 per
// step through two LDS buffers (2 × 64 KiB). Tiles are staged with
// global_load_lds_dwordx4 (HBM/L2 -> LDS without passing through registers):
// each wave instruction fills one contiguous KiB of LDS, lane L writing bytes
// 16L..16L+15, so the XOR swizzle of the 16-byte chunk index (chunk ^
// ((row >> 1) & 7), rows of 128 B: the 16 lanes of one LDS cycle hit 16
// distinct 16-byte bank groups) is applied by choosing which global chunk each
// lane fetches. Fragment loads of the next k-substep are issued before the MFMAs
// of the current one, and the loads of the next K step before the MFMAs of
// the current step.
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

constexpr int TM = 256, TN = 256, TK = 64;
constexpr int NT = 256;
constexpr int TILE_ELEMS = TM * TK;      // one operand tile in LDS (bf16 elements)
constexpr int LOADS_PER_WAVE = TM * TK * 2 / 1024 / 4; // KiB blocks per operand per wave = 8

// Key position inside a 16-key group in the transposed-V layout: bits 2 and 3
// swapped, so that the 8 keys one lane feeds to the P·V MFMA are contiguous.
__device__ __forceinline__ int vt_perm(int t) {
  return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1);
}

__device__ __forceinline__ float bf2f(bf16 v) { return (float)v; }

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void load_lds16(const void *g, bf16 *lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)lds_base, 16, 0, 0);
}

template <int EPI, bool SWAP>
__global__ __launch_bounds__(NT, 1) void gemm_bf16_kernel(const bf16 *__restrict__ A, int64_t lda,
                                                          const bf16 *__restrict__ Bt, int64_t ldb,
                                                          int M, int N, int K, GemmEpilogue ep) {
  __shared__ __attribute__((aligned(1024))) bf16 smem[2 * 2 * TILE_ELEMS];

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

  // staging: wave w fills LDS KiB-blocks w*8 .. w*8+7 of each operand tile;
  // block b = rows 8b .. 8b+7; lane -> (row 8b + lane/8, LDS chunk lane%8),
  // fetching global chunk (lane%8) ^ ((row >> 1) & 7).
  const bf16 *a_src[LOADS_PER_WAVE];
  const bf16 *b_src[LOADS_PER_WAVE];
#pragma unroll
  for (int i = 0; i < LOADS_PER_WAVE; ++i) {
    const int row = (wave * LOADS_PER_WAVE + i) * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ ((row >> 1) & 7);
    const int ra = min(tm * TM + row, M - 1);
    const int rb = min(tn * TN + row, N - 1);
    a_src[i] = A + (int64_t)ra * lda + ch * 8;
    b_src[i] = Bt + (int64_t)rb * ldb + ch * 8;
  }
  auto stage = [&](int kt, int buf) {
    bf16 *As = smem + buf * 2 * TILE_ELEMS;
    bf16 *Bs = As + TILE_ELEMS;
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i) {
      const int blk = (wave * LOADS_PER_WAVE + i) * 512; // 1 KiB = 512 bf16
      load_lds16(a_src[i] + kt * TK, As + blk);
      load_lds16(b_src[i] + kt * TK, Bs + blk);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment read offsets (elements) inside an operand tile, per k-substep
  int a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm * 128 + i * 32 + l32;
    const int rb = wn * 128 + i * 32 + l32;
    a_off[i] = ra * TK;
    b_off[i] = rb * TK;
  }
  const int swz_a = (l32 >> 1) & 7; // ((row >> 1) & 7) for row = 32*i + l32

  auto read_frags = [&](const bf16 *As, const bf16 *Bs, int ks, bf16x8 *af, bf16x8 *bfv) {
    const int kc = ((ks * 2 + g) ^ swz_a) << 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const bf16x8 *>(As + a_off[i] + kc);
#pragma unroll
    for (int j = 0; j < 4; ++j) bfv[j] = *reinterpret_cast<const bf16x8 *>(Bs + b_off[j] + kc);
  };

  const int KT = K / TK;
  stage(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0): the direct-to-LDS writes have landed
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    const bf16 *As = smem + buf * 2 * TILE_ELEMS;
    const bf16 *Bs = As + TILE_ELEMS;
    bf16x8 af[2][4], bfv[2][4];
    read_frags(As, Bs, 0, af[0], bfv[0]);
    // the last step re-stages its own tile into the idle buffer, keeping the
    // step free of branches (nothing reads that buffer afterwards)
    stage(min(kt + 1, KT - 1), buf ^ 1);
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < TK / 16) read_frags(As, Bs, ks + 1, af[cur ^ 1], bfv[cur ^ 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (SWAP)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfv[cur][j], af[cur][i], acc[i][j],
                                                                0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfv[cur][j], acc[i][j],
                                                                0, 0, 0);
        }
      // 8 fragment reads of the next substep spread over the 16 MFMAs
      if (ks + 1 < TK / 16) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // DS read
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0); // MFMA
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  const bf16 *bias = reinterpret_cast<const bf16 *>(ep.bias);
  if constexpr (SWAP) {
    // lane: output row m, 4 consecutive columns n .. n+3 per register group
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nb = tn * TN + wn * 128 + j * 32; // 32-column block, wave-uniform
      if (nb >= N) continue;
      // scatter target of this column block (one head of Q or K)
      bf16 *qk_base = nullptr;
      int d0 = 0;
      if constexpr (EPI == EPI_QK) {
        const int h = (int)ep.hidden, D = (int)ep.head_dim;
        const int which = nb / h, rem = nb - which * h;
        const int head = rem / D;
        d0 = rem - head * D;
        qk_base = reinterpret_cast<bf16 *>(which == 0 ? ep.q : ep.k) +
                  (int64_t)head * ep.seq * ep.head_dim;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = tm * TM + wm * 128 + i * 32 + l32;
        if (m >= M) continue;
        bf16 *row_dst;
        const bf16 *row_res = nullptr;
        if constexpr (EPI == EPI_QK) {
          const int s = (int)ep.seq;
          const int bi = m / s, t = m - bi * s;
          row_dst = qk_base + ((int64_t)bi * ep.heads * s + t) * ep.head_dim + d0;
        } else {
          row_dst = reinterpret_cast<bf16 *>(ep.out) + (int64_t)m * ep.ld_out + nb;
          if constexpr (EPI == EPI_RESID)
            row_res = reinterpret_cast<const bf16 *>(ep.resid) + (int64_t)m * ep.ld_resid + nb;
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int c = r4 * 8 + g * 4; // column offset inside the block
          const bf16x4 bv = *reinterpret_cast<const bf16x4 *>(bias + nb + c);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][r4 * 4 + e] + bf2f(bv[e]);
          if constexpr (EPI == EPI_RESID) {
            const bf16x4 rv = *reinterpret_cast<const bf16x4 *>(row_res + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += bf2f(rv[e]);
          } else if constexpr (EPI == EPI_RELU) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], 0.f);
          }
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
          *reinterpret_cast<bf16x4 *>(row_dst + c) = o;
        }
      }
    }
  } else {
    // lane: output column n, 4 consecutive rows m .. m+3 per register group
    static_assert(EPI == EPI_VT, "the non-swapped orientation serves the V^T scatter");
    const int s = (int)ep.seq, D = (int)ep.head_dim;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = tn * TN + wn * 128 + j * 32 + l32;
      if (n >= N) continue;
      const float bn = bf2f(bias[n]);
      const int head = n / D, d = n - head * D;
      bf16 *col_base = reinterpret_cast<bf16 *>(ep.v) + ((int64_t)head * D + d) * s;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int m = tm * TM + wm * 128 + i * 32 + r4 * 8 + g * 4;
          if (m >= M) continue;
          const int bi = m / s, t = m - bi * s;
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)(acc[i][j][r4 * 4 + e] + bn);
          bf16 *dst = col_base + (int64_t)bi * ep.heads * D * s + vt_perm(t);
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
  if ((epi == EPI_QK || epi == EPI_VT) && (ep.head_dim % 32 != 0 || ep.hidden % 32 != 0))
    return hipErrorInvalidValue;
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
