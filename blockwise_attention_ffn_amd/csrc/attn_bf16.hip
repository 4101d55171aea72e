// Fused blockwise attention, bf16 in / fp32 statistics, for CDNA4.
//
// What it computes: for every (batch, head) and every query row q,
//   A[q] = softmax_k( Q[q]·K[k] / sqrt(d) ) V[k],   causal: only k <= q,
// by the BPT schedule (BPT paper review, §三 Eq. 3 "Scaling" and Algorithm 1):
// an outer, parallel loop over query blocks and an inner loop over key/value
// blocks that keeps a running row maximum m and row sum l and rescales the
// partial output by exp(m_old - m_new) whenever m grows. No score matrix is
// ever written to memory.
//
// GPU mapping:
//  * one workgroup = 256 query rows of one (batch, head); 4 waves × 64 rows;
//    query blocks of the method larger than 256 rows span several
//    workgroups, smaller ones share one (the result does not depend on it);
//  * the inner loop walks the keys in stages of 64 (the running statistics
//    are folded once per stage, a partition of every key/value block of 64
//    or more keys; the online update is exact for any partition);
//  * K and V^T stages are double-buffered in LDS (2 × 32 KiB) and loaded with
//    coalesced 16-byte loads while the previous stage computes;
//  * scores are computed transposed, S^T = K·Q^T, on v_mfma_f32_32x32x16_bf16
//    with Q held in registers as the B operand. Each lane then owns one query
//    column: its row max / row sum need one exchange with the lane 32 apart,
//    and the rescale of its output column is a per-lane scalar;
//  * O^T = V^T·P^T on the same MFMA, fed straight from the score registers
//    (rounded to bf16); V is stored transposed with keys permuted inside each
//    16-key group so that a lane's 8 keys are one 16-byte LDS load;
//  * exp2 with the factor log2(e)/sqrt(d) folded into one FMA per score;
//  * causal: stages entirely after a wave's last query are skipped, only
//    stages crossing the diagonal are masked, and the longest query tiles
//    are dispatched first; each head's workgroups land on one XCD (head
//    index % 8) so that the K/V stream is shared through that XCD's L2.
#include "bpt_internal.h"

#include <math.h>

namespace bpt {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BQ = 256; // query rows per workgroup
constexpr int KB = 64;  // keys per stage
constexpr int NT = 256;

template <int D>
__global__ __launch_bounds__(NT, 1) void attn_fwd_bf16_kernel(const bf16 *__restrict__ Q,
                                                              const bf16 *__restrict__ K,
                                                              const bf16 *__restrict__ Vt,
                                                              bf16 *__restrict__ Aout, int s,
                                                              int heads, int causal, float c_log2,
                                                              int n_qt) {
  constexpr int DK = D / 16; // MFMA k-steps over the head dim for S^T
  constexpr int DB = D / 32; // 32-row blocks of O^T
  constexpr int KCH = D / 8; // 16-byte chunks per K row
  constexpr int KSW = (KCH >= 8 ? 8 : KCH) - 1; // XOR swizzle mask of the K chunk index
  constexpr int LD_PER_T = (KB * D / 8) / NT; // 16-byte chunks per thread per operand stage
  static_assert(LD_PER_T >= 1, "stage too small for the workgroup");

  __shared__ __attribute__((aligned(16))) bf16 Ks[2][KB * D];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][D * KB];

  const int bh = blockIdx.x;
  const int qt = n_qt - 1 - (int)blockIdx.y; // longest (causal) first
  const int q0 = qt * BQ;
  const int bi = bh / heads, head = bh - bi * heads;
  const bf16 *Qh = Q + (int64_t)bh * s * D;
  const bf16 *Kh = K + (int64_t)bh * s * D;
  const bf16 *Vh = Vt + (int64_t)bh * D * s;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  // Q^T fragments (B operand): query row qrow[u], head-dim chunk ks*16 + g*8
  bf16x8 qf[2][DK];
  int qrow[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    qrow[u] = q0 + wave * 64 + u * 32 + l32;
    const int qa = min(qrow[u], s - 1);
#pragma unroll
    for (int ks = 0; ks < DK; ++ks)
      qf[u][ks] = *reinterpret_cast<const bf16x8 *>(Qh + (int64_t)qa * D + ks * 16 + g * 8);
  }

  f32x16 o[2][DB];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[u][db][r] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  const int kv_end = causal ? min(s, q0 + BQ) : s;
  const int nst = (kv_end + KB - 1) / KB;
  const int wq_first = q0 + wave * 64;
  const int wq_last = min(q0 + wave * 64 + 63, s - 1);

  // staging registers
  u32x4 rk[LD_PER_T], rv[LD_PER_T];
  auto gload = [&](int st) {
    const int k0 = st * KB;
#pragma unroll
    for (int i = 0; i < LD_PER_T; ++i) {
      const int idx = tid + NT * i;
      const int key = idx / KCH, ch = idx - key * KCH;
      const int krow = min(k0 + key, s - 1);
      rk[i] = *reinterpret_cast<const u32x4 *>(Kh + (int64_t)krow * D + ch * 8);
      const int drow = idx >> 3, vch = idx & 7;
      const int kc = min(k0 + vch * 8, s - 8); // keys >= s are masked; read finite data
      rv[i] = *reinterpret_cast<const u32x4 *>(Vh + (int64_t)drow * s + kc);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LD_PER_T; ++i) {
      const int idx = tid + NT * i;
      const int key = idx / KCH, ch = idx - key * KCH;
      *reinterpret_cast<u32x4 *>(&Ks[buf][key * D + ((ch ^ (key & KSW)) << 3)]) = rk[i];
      const int drow = idx >> 3, vch = idx & 7;
      *reinterpret_cast<u32x4 *>(&Vs[buf][drow * KB + ((vch ^ (drow & 7)) << 3)]) = rv[i];
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) gload(st + 1);
    const int k0 = st * KB;
    const bool has_work = !causal || k0 <= wq_last;
    if (has_work) {
      // ---- S^T = K · Q^T : [64 keys] x [2 x 32 queries]
      f32x16 sacc[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][u][r] = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = kb * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
          const int ch = ks * 2 + g;
          const bf16x8 kf =
              *reinterpret_cast<const bf16x8 *>(&Ks[buf][key * D + ((ch ^ (key & KSW)) << 3)]);
#pragma unroll
          for (int u = 0; u < 2; ++u)
            sacc[kb][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[u][ks], sacc[kb][u], 0, 0, 0);
        }
      }
      // ---- mask: keys after the query (causal) or past the sequence end
      const bool need_mask = (causal && k0 + KB - 1 > wq_first) || (k0 + KB > s);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
              const bool dead = key >= s || (causal && key > qrow[u]);
              if (dead) sacc[kb][u][r] = -INFINITY;
            }
      }
      // ---- online softmax update per query column
      bf16x8 pf[2][2][2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][u][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[u], mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run[u] - m_new) * c_log2);
        m_run[u] = m_new;
        const float mc = m_new * c_log2;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][u][r], c_log2, -mc));
            const bf16 pb = (bf16)p;
            rs += (float)pb; // the normaliser sums exactly the weights the MFMA uses
            pf[u][kb][r >> 3][r & 7] = pb;
          }
        l_run[u] = l_run[u] * alpha + rs;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[u][db][r] *= alpha;
      }
      // ---- O^T += V^T · P^T
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int drow = db * 32 + l32;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int ch = kb * 4 + hf * 2 + g;
            const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(
                &Vs[buf][drow * KB + ((ch ^ (drow & 7)) << 3)]);
#pragma unroll
            for (int u = 0; u < 2; ++u)
              o[u][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[u][kb][hf], o[u][db], 0, 0, 0);
          }
      }
    }
    if (st + 1 < nst) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and write A[b, s, heads*D] (token-major, head at column head*D)
  const int64_t h = (int64_t)heads * D;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float l_tot = l_run[u] + __shfl_xor(l_run[u], 32);
    const float inv = 1.f / l_tot;
    if (qrow[u] >= s) continue;
    bf16 *dst = Aout + ((int64_t)bi * s + qrow[u]) * h + (int64_t)head * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(o[u][db][r4 * 4 + e] * inv);
        *reinterpret_cast<bf16x4 *>(dst + db * 32 + r4 * 8 + g * 4) = v;
      }
  }
}

} // namespace

hipError_t launch_attention_bf16(const void *Q, const void *K, const void *Vt, void *A,
                                 int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                                 int causal, hipStream_t stream) {
  if (batch <= 0 || seq <= 0) return hipSuccess;
  if (seq % 16 != 0 || seq > INT32_MAX / 2) return hipErrorInvalidValue;
  const int64_t n_qt = (seq + BQ - 1) / BQ;
  const int64_t bh = batch * heads;
  if (bh > INT32_MAX || n_qt > 65535) return hipErrorInvalidValue;
  dim3 grid((unsigned)bh, (unsigned)n_qt), block(NT);
  const float c_log2 = 1.4426950408889634f / sqrtf((float)head_dim);
  const bf16 *q = reinterpret_cast<const bf16 *>(Q);
  const bf16 *k = reinterpret_cast<const bf16 *>(K);
  const bf16 *v = reinterpret_cast<const bf16 *>(Vt);
  bf16 *a = reinterpret_cast<bf16 *>(A);
  switch (head_dim) {
  case 32:
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<32>, grid, block, 0, stream, q, k, v, a, (int)seq,
                       (int)heads, causal, c_log2, (int)n_qt);
    break;
  case 64:
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, grid, block, 0, stream, q, k, v, a, (int)seq,
                       (int)heads, causal, c_log2, (int)n_qt);
    break;
  case 128:
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, grid, block, 0, stream, q, k, v, a, (int)seq,
                       (int)heads, causal, c_log2, (int)n_qt);
    break;
  default:
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

} // namespace bpt
