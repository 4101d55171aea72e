// fp32 path of the BPT layer forward: every product and sum in fp32 on the
// vector ALU (gfx950 has no reduced-precision shortcut that would keep the
// fp32 result within 1e-4, so no MFMA bf16/xf32 here).
//
// Same schedule as the bf16 path (BPT paper review, Algorithm 1): the QKV
// projection over the whole sequence, then per query block an inner loop over
// key/value stages with running max / sum statistics (§三 Eq. 3 "Scaling"),
// then the output projection, residual, ReLU FFN and second residual over a
// bounded group of query blocks.
#include "bpt_internal.h"
#include "philox.h"

#include <math.h>

namespace bpt {
namespace {

// ---------------------------------------------------------------------------
// GEMM: C[M, N] = A[M, K] · Bt[N, K]^T, 64×64 tile, 256 threads × (4×4); both
// operands K-contiguous (Bt is a weight in the [out, in] layout).
constexpr int FT = 64, FK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float *__restrict__ A, int64_t lda,
                                                       const float *__restrict__ Bt, int64_t ldb,
                                                       int M, int N, int K, GemmEpilogue ep) {
  __shared__ float As[FK][FT + 4];
  __shared__ float Bs[FK][FT + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * FT, n0 = blockIdx.x * FT;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 4, kk = idx & 15;
      const int gm = m0 + r, gk = k0 + kk;
      As[kk][r] = (gm < M && gk < K) ? A[(int64_t)gm * lda + gk] : 0.f;
      const int gn = n0 + r;
      Bs[kk][r] = (gn < N && gk < K) ? Bt[(int64_t)gn * ldb + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const float *bias = reinterpret_cast<const float *>(ep.bias);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
    // EPI_RESID_DROP: this thread's 4 columns lie in one 16-column block of
    // the dropout generator (n0 is a multiple of 64)
    uint32_t keep = 0;
    if constexpr (EPI == EPI_RESID_DROP)
      keep = dev::dropout_keep16(ep.drop_seed, ep.drop_site, (uint64_t)(ep.row0 + m),
                                 (uint64_t)((n0 + tx * 4) >> 4), ep.drop_threshold);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float v = acc[i][j] + bias[n];
      if constexpr (EPI == EPI_QKV) {
        const int64_t h = ep.hidden, D = ep.head_dim, s = ep.seq;
        const int64_t which = n / h, rem = n - which * h;
        const int64_t head = rem / D, d = rem - head * D;
        const int64_t bi = m / s, t = m - bi * s;
        float *base = reinterpret_cast<float *>(which == 0 ? ep.q : (which == 1 ? ep.k : ep.v));
        base[((bi * ep.heads + head) * s + t) * D + d] = v;
      } else if constexpr (EPI == EPI_RESID || EPI == EPI_RESID_DROP) {
        if constexpr (EPI == EPI_RESID_DROP) v = ((keep >> (n & 15)) & 1u) ? v * ep.drop_scale : 0.f;
        v += reinterpret_cast<const float *>(ep.resid)[(int64_t)m * ep.ld_resid + n];
        reinterpret_cast<float *>(ep.out)[(int64_t)m * ep.ld_out + n] = v;
      } else {
        reinterpret_cast<float *>(ep.out)[(int64_t)m * ep.ld_out + n] = fmaxf(v, 0.f);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Attention: one thread per query row, 64 rows per workgroup, keys in LDS
// stages of 32 with the running (max, sum) update after each stage.
constexpr int AQ = kF32AttnRows, AK = kF32AttnKeys;

template <int D>
__global__ __launch_bounds__(AQ) void attn_f32_kernel(const float *__restrict__ Q,
                                                      const float *__restrict__ K,
                                                      const float *__restrict__ V,
                                                      float *__restrict__ Aout, int s, int heads,
                                                      int causal, float scale) {
  __shared__ float Ks[AK][D];
  __shared__ float Vs[AK][D];
  const int bh = blockIdx.x;
  const int n_qt = gridDim.y;
  const int q0 = (n_qt - 1 - (int)blockIdx.y) * AQ;
  const int bi = bh / heads, head = bh - bi * heads;
  const int tid = threadIdx.x;
  const int qi = q0 + tid;
  const float *Qh = Q + (int64_t)bh * s * D;
  const float *Kh = K + (int64_t)bh * s * D;
  const float *Vh = V + (int64_t)bh * s * D;

  float q[D], o[D];
  const int qa = min(qi, s - 1);
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = Qh[(int64_t)qa * D + e] * scale;
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kv_end = causal ? min(s, q0 + AQ) : s;
  for (int k0 = 0; k0 < kv_end; k0 += AK) {
    __syncthreads();
    for (int idx = tid; idx < AK * D; idx += AQ) {
      const int r = idx / D, e = idx - r * D;
      const int kr = min(k0 + r, s - 1);
      Ks[r][e] = Kh[(int64_t)kr * D + e];
      Vs[r][e] = Vh[(int64_t)kr * D + e];
    }
    __syncthreads();
    float sc[AK];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < AK; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) acc = __builtin_fmaf(q[e], Ks[j][e], acc);
      const int key = k0 + j;
      const bool dead = key >= s || (causal && key > qi);
      sc[j] = dead ? -INFINITY : acc;
      mx = fmaxf(mx, sc[j]);
    }
    const float m_new = fmaxf(m, mx);
    if (m_new == -INFINITY) continue; // every key of this stage is masked for this row
    const float alpha = expf(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < AK; ++j) {
      const float p = expf(sc[j] - m_new);
      l += p;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] = __builtin_fmaf(p, Vs[j][e], o[e]);
    }
  }
  if (qi < s) {
    const float inv = 1.f / l;
    float *dst = Aout + ((int64_t)bi * s + qi) * ((int64_t)heads * D) + (int64_t)head * D;
#pragma unroll
    for (int e = 0; e < D; ++e) dst[e] = o[e] * inv;
  }
}

} // namespace

hipError_t launch_gemm_f32(int epi, const float *A, int64_t lda, const float *Bt, int64_t ldb,
                           int64_t M, int64_t N, int64_t K, const GemmEpilogue &ep,
                           hipStream_t stream) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  const int64_t gm = (M + FT - 1) / FT, gn = (N + FT - 1) / FT;
  if (gm > 65535 || gn > INT32_MAX || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
    return hipErrorInvalidValue;
  dim3 grid((unsigned)gn, (unsigned)gm), block(256);
  switch (epi) {
  case EPI_QKV:
    hipLaunchKernelGGL(gemm_f32_kernel<EPI_QKV>, grid, block, 0, stream, A, lda, Bt, ldb, (int)M,
                       (int)N, (int)K, ep);
    break;
  case EPI_RESID:
    hipLaunchKernelGGL(gemm_f32_kernel<EPI_RESID>, grid, block, 0, stream, A, lda, Bt, ldb,
                       (int)M, (int)N, (int)K, ep);
    break;
  case EPI_RELU:
    hipLaunchKernelGGL(gemm_f32_kernel<EPI_RELU>, grid, block, 0, stream, A, lda, Bt, ldb, (int)M,
                       (int)N, (int)K, ep);
    break;
  case EPI_RESID_DROP:
    hipLaunchKernelGGL(gemm_f32_kernel<EPI_RESID_DROP>, grid, block, 0, stream, A, lda, Bt, ldb,
                       (int)M, (int)N, (int)K, ep);
    break;
  default:
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention_f32(const float *Q, const float *K, const float *V, float *A,
                                int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                                int causal, hipStream_t stream) {
  if (batch <= 0 || seq <= 0) return hipSuccess;
  const int64_t n_qt = (seq + AQ - 1) / AQ;
  const int64_t bh = batch * heads;
  if (bh > INT32_MAX || n_qt > 65535 || seq > INT32_MAX) return hipErrorInvalidValue;
  dim3 grid((unsigned)bh, (unsigned)n_qt), block(AQ);
  const float scale = 1.f / sqrtf((float)head_dim);
  switch (head_dim) {
  case 32:
    hipLaunchKernelGGL(attn_f32_kernel<32>, grid, block, 0, stream, Q, K, V, A, (int)seq,
                       (int)heads, causal, scale);
    break;
  case 64:
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, block, 0, stream, Q, K, V, A, (int)seq,
                       (int)heads, causal, scale);
    break;
  case 128:
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, block, 0, stream, Q, K, V, A, (int)seq,
                       (int)heads, causal, scale);
    break;
  default:
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

} // namespace bpt
