// Fused blockwise attention, bf16 in / fp32 statistics, for CDNA4.
//
// What it computes: for every (batch, head) and every query row q,
//   A[q] = softmax_k( Q[q]·K[k] / sqrt(d) ) V[k],   causal: only k <= q,
// by the BPT schedule (BPT paper review, §三 Eq. 3 "Scaling" and Algorithm 1):
// an outer, parallel loop over query blocks and an inner loop over key/value
// blocks that keeps a running row maximum m and row sum l and rescales the
// partial output by exp(m_old - m_new) when m grows. No score matrix is ever
// written to memory.
//
// GPU mapping:
//  * one workgroup = 256 query rows of one (batch, head); 8 waves × 32 rows,
//    two waves per SIMD; query blocks of the method larger than 256 rows span
//    several workgroups, smaller ones share one;
//  * the inner loop walks the keys in stages of 64 and folds the running
//    statistics once per stage: a regrouping of the method's key/value
//    blocks, which the online update computes exactly for any partition of
//    the keys;
//  * K and V^T stages of 64 keys go HBM/L2 -> LDS with buffer_load_dwordx4
//    ... lds (no register staging), four buffers deep, K three stages ahead
//    and V^T two;
//  * scores are computed transposed, S^T = K·Q^T, on v_mfma_f32_32x32x16_bf16
//    with Q held in registers as the B operand. Each lane then owns one query
//    column: its row max / row sum need one permlane32 swap with the lane 32
//    apart, and the rescale of its output column is a per-lane scalar;
//  * O^T = V^T·P^T on the same MFMA, fed straight from the score registers
//    rounded to bf16; V is stored transposed with keys permuted inside each
//    16-key group so that a lane's 8 keys are one 16-byte LDS load;
//  * software pipeline inside each wave: each step issues the score MFMAs
//    of stage j+1, then the P·V MFMAs of stage j, one MFMA per issue slot
//    with LDS fragment reads three slots ahead; the exponentials of a stage
//    are split between the P·V half of the step before and the score half
//    of its own step, so the matrix core and the vector ALU are busy
//    together in both halves; the second wave of each SIMD fills the
//    remaining gaps; all per-wave state (Q, O, scores, weights) stays in
//    VGPRs;
//  * Q arrives scaled by log2(e)/sqrt(d) (applied in the projection's
//    epilogue) and the score MFMAs start from -m_used, a reference max held
//    in registers, so each weight is one v_exp_f32 of a score. m_used is set
//    by the first stage and moved only when a stage's weights exceed 2^32 in
//    some row: each lane's row-sum partial bounds every weight it summed
//    (weights are >= 0, and an overflowed one makes it inf), so one compare
//    replaces the per-stage row maximum. The rare rescale of O and l is by
//    an exact factor;
//  * row sums with v_dot2_f32_bf16 on the packed bf16 weights, i.e. exactly
//    the weights the P·V product uses;
//  * causal: stages after a wave's last query are skipped, only stages
//    crossing the diagonal are masked, the longest query tiles are
//    dispatched first, and a head's workgroups land on one XCD (head % 8) so
//    its K/V stream is shared through that XCD's L2.
#include "bpt_internal.h"
#include "lds_dma.h"

#include <math.h>

namespace bpt {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BQ = 256; // query rows per workgroup
constexpr int KB = 64;  // keys per stage
constexpr int NT = 512; // 8 waves, two per SIMD
constexpr int NSTAGE = 4; // LDS buffers: stage st in st % 4, loads two stages ahead
constexpr float WEIGHT_LIMIT = 0x1p32f; // largest weight before the reference max moves

using dev::i32x4;
using dev::load_lds16;
using dev::make_rsrc;

__device__ __forceinline__ void wait_vmem() { dev::wait_vm<0>(); }

// Barrier between stages that keeps the youngest stage's loads in flight:
// wait until this wave's LDS reads are done and at most VM of its loads
// into LDS are outstanding, then s_barrier.
template <int VM> __device__ __forceinline__ void stage_barrier() { dev::barrier_vm<VM>(); }

// max / sum of a value and its copy in the lane 32 apart
__device__ __forceinline__ float xhalf_max(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <int D> struct AttnCfg {
  static constexpr int DK = D / 16;              // MFMA k-steps over the head dim (S^T)
  static constexpr int DB = D / 32;              // 32-row blocks of O^T
  // K is laid out in LDS as panels of up to 64 head-dim columns, so that
  // rows are at most 128 B: [panel][key][<=64 d], 16-byte chunks swizzled
  // with (key >> 1) & (NC - 1).
  static constexpr int PW = D < 64 ? D : 64;     // panel width (elements)
  static constexpr int NC = PW / 8;              // 16-byte chunks per panel row
  static constexpr int NPANEL = D / PW;
  static constexpr int KPB = 1024 / (PW * 2);    // keys per KiB block
  static constexpr int BPP = KB / KPB;           // KiB blocks per panel
  static constexpr int NBLK = D / 8;             // KiB blocks per K (and per V^T) stage
  static constexpr int LOADS = (NBLK + 7) / 8;    // most loads one wave issues per operand stage
};

// LSE: also write each row's negated log-sum-exp, -(m_used + log2(l)) in the
// log2 units of the pre-scaled scores, to nlse[(b·heads + head)·s + row] (for
// the backward pass, which recomputes the weights as exp2(score - nlse) from
// products that start at -nlse: stored negated, it loads straight into them).
template <int D, bool LSE>
__global__ __launch_bounds__(NT, 1) void attn_fwd_bf16_kernel(const bf16 *__restrict__ Q,
                                                              const bf16 *__restrict__ K,
                                                              const bf16 *__restrict__ Vt,
                                                              bf16 *__restrict__ Aout, int s,
                                                              int heads, int causal, int n_qt,
                                                              float *__restrict__ nlse) {
  using C = AttnCfg<D>;
  constexpr int DK = C::DK, DB = C::DB, PW = C::PW, NC = C::NC;

  __shared__ __attribute__((aligned(1024))) bf16 Ks[NSTAGE][KB * D];
  __shared__ __attribute__((aligned(1024))) bf16 Vs[NSTAGE][D * KB];

  // workgroup and work-item ids through the builtins: this file is compiled
  // with IEEE mode off, which the device library's id functions do not
  // share, so blockIdx / threadIdx would become out-of-line calls (with a
  // call stack in scratch memory)
  const int bh = (int)__builtin_amdgcn_workgroup_id_x();
  const int qt = n_qt - 1 - (int)__builtin_amdgcn_workgroup_id_y(); // longest (causal) first
  const int q0 = qt * BQ;
  const int bi = bh / heads, head = bh - bi * heads;
  const bf16 *Qh = Q + (int64_t)bh * s * D;
  const bf16 *Kh = K + (int64_t)bh * s * D;
  const bf16 *Vh = Vt + (int64_t)bh * D * s;
  // one head's K and V^T, s·D bf16 each (the host keeps s·D·2 below 2^31)
  const i32x4 krsrc = make_rsrc(Kh, (unsigned)s * D * 2u);
  const i32x4 vrsrc = make_rsrc(Vh, (unsigned)s * D * 2u);

  const int tid = (int)__builtin_amdgcn_workitem_id_x();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // wave-uniform, in an SGPR
  __builtin_assume(wave < 8);
  const int l32 = lane & 31, g = lane >> 5;

  // ---- this wave's 32 queries; Q^T fragments (B operand), head-dim chunk ks*16 + g*8
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  bf16x8 qf[DK];
  {
    const int qa = min(qrow, s - 1);
#pragma unroll
    for (int ks = 0; ks < DK; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8 *>(Qh + (int64_t)qa * D + ks * 16 + g * 8);
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  // Q arrives multiplied by log2(e)/sqrt(d), so scores are in log2 units.
  // Scores are kept relative to m_used, the reference max of the
  // exponentials: the score MFMAs start from -m_used, and a weight is
  // exp2(score) with no further arithmetic.
  float m_used = 0.f;
  float l_run = 0.f; // lane-partial row sum
  f32x16 minit; // -m_used in every element: the C operand of the score MFMAs
#pragma unroll
  for (int r = 0; r < 16; ++r) minit[r] = 0.f;

  const int kv_end = causal ? min(s, q0 + BQ) : s;
  const int n_st = (kv_end + KB - 1) / KB; // stages the workgroup stages through LDS
  const int wq_last = min(qw0 + 31, s - 1);
  // stages this wave computes: those holding a key <= its last query
  const int nw = causal ? min(n_st, wq_last / KB + 1) : n_st;

  // ---- staging into LDS buffers (stage x of K in Ks[x % 4], of V^T in
  // Vs[x % 4]). A KiB block of K holds KPB keys of one panel; a KiB block of
  // V^T holds 8 head-dim rows of 64 keys. Lane L writes LDS bytes
  // 16L..16L+15 of the block, so it fetches the global chunk that the
  // swizzle puts there. koff / voff: byte offsets of this lane's chunks in
  // stage 0; stage st adds st·KB·D·2 (K) or st·KB·2 (V^T). A K row at or past
  // s lies outside the K buffer, which reads it as zeros (its scores are
  // masked); a V^T chunk past s holds finite data of the next head-dim row,
  // or zeros past the buffer, and meets a zero weight.
  unsigned koff[C::LOADS], voff[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int blk = wave + 8 * i;
    const int panel = blk / C::BPP;
    const int key = (blk % C::BPP) * C::KPB + lane / NC;
    const int kch = (lane % NC) ^ ((key >> 1) & (NC - 1));
    koff[i] = (unsigned)(key * D + panel * PW + kch * 8) * 2u;
    const int drow = blk * 8 + (lane >> 3);
    const int vch = (lane & 7) ^ ((drow >> 1) & 7);
    voff[i] = (unsigned)(drow * s + vch * 8) * 2u;
  }
  auto issue_k1 = [&](int st, int i) __attribute__((always_inline)) {
    if (wave + 8 * i < C::NBLK)
      load_lds16(krsrc, koff[i] + (unsigned)st * (unsigned)(KB * D * 2),
                 &Ks[st % NSTAGE][(wave + 8 * i) * 512]);
  };
  auto issue_v1 = [&](int st, int i) __attribute__((always_inline)) {
    if (wave + 8 * i < C::NBLK)
      load_lds16(vrsrc, voff[i] + (unsigned)st * (unsigned)(KB * 2),
                 &Vs[st % NSTAGE][(wave + 8 * i) * 512]);
  };
  auto issue_k = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) issue_k1(st, i);
  };
  auto issue_v = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) issue_v1(st, i);
  };

  const int kswz = (l32 >> 1) & (NC - 1); // K chunk swizzle for key = kb*32 + l32
  const int vswz = (l32 >> 1) & 7;        // V^T chunk swizzle for drow = db*32 + l32
  const bf16x2 ones = {(bf16)1.f, (bf16)1.f};

  // S^T - m_used of stage st (64 keys x this wave's 32 queries)
  auto scores = [&](int st, f32x16 (&sa)[2]) __attribute__((always_inline)) {
    const bf16 *kbase = &Ks[st % NSTAGE][l32 * PW];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        const int gc = ks * 2 + g; // global 16-byte chunk of the head dim
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(
            kbase + kb * 32 * PW + (gc / NC) * (KB * PW) + (((gc % NC) ^ kswz) << 3));
        sa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], ks == 0 ? minit : sa[kb], 0,
                                                         0, 0);
      }
    }
  };
  auto mask_if_needed = [&](int st, f32x16 (&sa)[2]) __attribute__((always_inline)) {
    const int k0 = st * KB;
    if ((causal && k0 + KB - 1 > qw0) || k0 + KB > s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= s || (causal && key > qrow)) sa[kb][r] = -INFINITY;
        }
    }
  };
  auto row_max = [&](const f32x16 (&sa)[2]) __attribute__((always_inline)) {
    float a = fmaxf(sa[0][0], sa[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) a = fmaxf(fmaxf(a, sa[0][r]), sa[1][r]); // v_max3 chain
    return xhalf_max(a);
  };
  // unit u (0..15) of a stage's weights: two bf16 weights exp2(score) of
  // score block kb = u / 8 into pf, and their sum into the row-sum partial
  // rs[u & 1] (added to, not reset). Units 0..7 read only score block 0.
  auto unit = [&](const f32x16 (&sa)[2], bf16x8 (&pf)[2][2], float (&rs)[2], int u) __attribute__((always_inline)) {
    const int kb = u >> 3, r = (u & 7) * 2;
    bf16x2 pp;
    pp[0] = (bf16)__builtin_amdgcn_exp2f(sa[kb][r]);
    pp[1] = (bf16)__builtin_amdgcn_exp2f(sa[kb][r + 1]);
    pf[kb][r >> 3][r & 7] = pp[0];
    pf[kb][r >> 3][(r & 7) + 1] = pp[1];
    rs[u & 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, rs[u & 1], false);
  };
  // all weights of one stage
  auto weights_rs = [&](const f32x16 (&sa)[2], bf16x8 (&pf)[2][2], float (&rs)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 16; ++u) unit(sa, pf, rs, u);
  };
  // Rare path, after a stage's weights exceeded WEIGHT_LIMIT in some row
  // (the row-sum partials bound every weight, which are >= 0; an overflowed
  // weight makes its partial inf): move the reference max up to the
  // stage's row max, rescale O and l by the exact factor, shift this stage's
  // and the next stage's relative scores, and recompute the weights.
  auto rescale_stage = [&](f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2], bf16x8 (&pf)[2][2],
                           float (&rs)[2]) __attribute__((always_inline)) {
    const float delta = fmaxf(row_max(s_cur), 0.f); // a row masked here has max -inf
    const float alpha = __builtin_amdgcn_exp2f(-delta);
    m_used += delta;
#pragma unroll
    for (int r = 0; r < 16; ++r) minit[r] = -m_used;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s_cur[kb][r] -= delta;
        s_nxt[kb][r] -= delta; // (unused after the last stage)
      }
    rs[0] = rs[1] = 0.f;
    weights_rs(s_cur, pf, rs);
  };
  auto over_limit = [&](const float (&rs)[2]) __attribute__((always_inline)) { return __any(rs[0] + rs[1] > WEIGHT_LIMIT); };
  // O^T += V^T · P^T for stage st
  auto pv_stage = [&](int st, const bf16x8 (&pf)[2][2]) __attribute__((always_inline)) {
    const bf16 *vbase = &Vs[st % NSTAGE][l32 * KB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int ch = kb * 4 + hf * 2 + g;
          const bf16x8 vf =
              *reinterpret_cast<const bf16x8 *>(vbase + db * 32 * KB + ((ch ^ vswz) << 3));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][hf], o[db], 0, 0, 0);
        }
  };

  // ---- the general step (stages that need a mask, and the last ones):
  // scores of stage st+1, then the weights, limit check and P·V of stage st
  auto step = [&](int st, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2]) __attribute__((always_inline)) {
    if (st + 3 < n_st) issue_k(st + 3);
    if (st + 2 < n_st) issue_v(st + 2);
    if (st < nw) {
      const bool has_next = st + 1 < nw;
      if (has_next) {
        scores(st + 1, s_nxt);
        mask_if_needed(st + 1, s_nxt);
      }
      bf16x8 pf[2][2];
      float rs[2] = {0.f, 0.f};
      weights_rs(s_cur, pf, rs);
      if (over_limit(rs)) rescale_stage(s_cur, s_nxt, pf, rs);
      l_run += rs[0] + rs[1];
      pv_stage(st, pf);
    }
    // the next step needs K(st+2) and V(st+1), issued one step earlier; the
    // loads issued in this step (both, V only, or none) may stay in flight
    if (st + 3 < n_st)
      stage_barrier<2 * C::LOADS>();
    else if (st + 2 < n_st)
      stage_barrier<C::LOADS>();
    else
      stage_barrier<0>();
  };

  // ---- the step for the bulk of the stages, where stage st+1 exists and
  // needs no mask. It is written as NS + NP issue slots of one MFMA each:
  // slots 0..NS-1 hold the score MFMAs of stage st+1 (kb-major) beside the
  // exponentials, bf16 packing and row sums of stage st; after the weight
  // limit check, slots NS.. hold the P·V MFMAs of stage st. Fragment reads
  // from LDS run LA slots ahead through a ring of LA+1 registers, and a
  // scheduling fence after every slot keeps that order, so an MFMA never
  // waits on a read issued just before it.
  constexpr int NS = 2 * DK, NP = 4 * DB, LA = 3;
  // The step's loads into LDS are spread over its slots (load j at slot
  // 1 + j·(NS+NP)/(2·LOADS)) rather than issued together after the barrier,
  // where all eight waves would queue theirs at the texture unit at once.
  constexpr int NLD = 2 * C::LOADS;
  // The weights of a stage come in two halves: units 0..7 (score block 0,
  // complete half-way through the score MFMAs) during the P·V half of the
  // previous step, units 8..15 during the score half of the stage's own
  // step, so each half of a step carries half of the exponentials. On entry
  // pf[0][*] and rs hold units 0..7 of stage st; the step leaves units 0..7
  // of stage st+1 in pf_n[0][*] and rs_n.
  auto step_bulk = [&](int st, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2], bf16x8 (&pf)[2][2],
                       float (&rs)[2], bf16x8 (&pf_n)[2][2], float (&rs_n)[2]) __attribute__((always_inline)) {
    // V(st+2) always exists here (st+2 < n_um); K(st+3) may be one stage past
    // the last, which lands in a free buffer and is never read
    const bf16 *kbase = &Ks[(st + 1) % NSTAGE][l32 * PW];
    const bf16 *vbase = &Vs[st % NSTAGE][l32 * KB];
    // read r < NS: K fragment of score MFMA r; else V^T fragment of P·V MFMA r - NS
    auto frag = [&](int r) __attribute__((always_inline)) -> bf16x8 {
      if (r < NS) {
        const int kb = r / DK, gc = (r % DK) * 2 + g;
        return *reinterpret_cast<const bf16x8 *>(kbase + kb * 32 * PW + (gc / NC) * (KB * PW) +
                                                 (((gc % NC) ^ kswz) << 3));
      }
      const int j = r - NS, db = j >> 2, kb = (j >> 1) & 1, hf = j & 1;
      const int ch = kb * 4 + hf * 2 + g;
      return *reinterpret_cast<const bf16x8 *>(vbase + db * 32 * KB + ((ch ^ vswz) << 3));
    };
    bf16x8 ring[LA + 1];
#pragma unroll
    for (int r = 0; r < LA; ++r) ring[r] = frag(r);
    rs_n[0] = rs_n[1] = 0.f;
    // one issue slot: its loads, its MFMA, the read LA slots ahead, and a
    // share of the weights: units 8..15 of stage st in the score half, units
    // 0..7 of stage st+1 in the P·V half
    auto slot_work = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < NLD; ++j)
        if (slot == 1 + j * (NS + NP) / NLD) {
          if (j < C::LOADS)
            issue_k1(st + 3, j);
          else
            issue_v1(st + 2, j - C::LOADS);
        }
      const bf16x8 fr = ring[slot % (LA + 1)];
      if (slot < NS) {
        const int kb = slot / DK, ks = slot % DK;
        s_nxt[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr, qf[ks], ks == 0 ? minit : s_nxt[kb],
                                                            0, 0, 0);
      } else {
        const int j = slot - NS, db = j >> 2, kb = (j >> 1) & 1, hf = j & 1;
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr, pf[kb][hf], o[db], 0, 0, 0);
      }
      if (slot + LA < NS + NP) ring[(slot + LA) % (LA + 1)] = frag(slot + LA);
      if (slot < NS) {
#pragma unroll
        for (int u = slot * 8 / NS; u < (slot + 1) * 8 / NS; ++u) unit(s_cur, pf, rs, 8 + u);
      } else {
#pragma unroll
        for (int u = (slot - NS) * 8 / NP; u < (slot - NS + 1) * 8 / NP; ++u) unit(s_nxt, pf_n, rs_n, u);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int slot = 0; slot < NS; ++slot) slot_work(slot);
    // all weights of stage st are in pf: check them before its P·V
    if (over_limit(rs)) rescale_stage(s_cur, s_nxt, pf, rs);
    l_run += rs[0] + rs[1];
#pragma unroll
    for (int slot = NS; slot < NS + NP; ++slot) slot_work(slot);
    stage_barrier<2 * C::LOADS>();
  };
  // stages before n_um need no mask (all keys <= the wave's first query and < s)
  const int n_um = min(nw, min(causal ? (qw0 + 1) / KB : s / KB, s / KB));

  // ---- prologue: K(0..2), V(0..1) into LDS; scores and max of stage 0
  issue_k(0);
  issue_v(0);
  if (n_st > 1) {
    issue_k(1);
    issue_v(1);
  }
  if (n_st > 2) issue_k(2);
  wait_vmem();
  __syncthreads();
  f32x16 sA[2], sB[2];
  scores(0, sA); // m_used = 0: the raw scores
  mask_if_needed(0, sA);
  // the reference max starts at stage 0's row max (finite: key 0 is never
  // masked), so every row's largest weight is at least 1
  m_used = row_max(sA);
#pragma unroll
  for (int r = 0; r < 16; ++r) minit[r] = -m_used;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) sA[kb][r] -= m_used;
  // units 0..7 of stage 0, carried into the first bulk step (a general step
  // recomputes all of its weights)
  bf16x8 pfA[2][2], pfB[2][2];
  float rsA[2] = {0.f, 0.f}, rsB[2] = {0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 8; ++u) unit(sA, pfA, rsA, u);

  // every wave takes n_st steps (one barrier each): bulk steps while the
  // next stage is unmasked, then the general step
  int st = 0;
  for (; st + 2 < n_um; st += 2) {
    step_bulk(st, sA, sB, pfA, rsA, pfB, rsB);
    step_bulk(st + 1, sB, sA, pfB, rsB, pfA, rsA);
  }
  for (; st < n_st; st += 2) {
    step(st, sA, sB);
    if (st + 1 < n_st) step(st + 1, sB, sA);
  }
  wait_vmem(); // no load into LDS outlives the loop

  // ---- normalise and write A[b, s, heads*D] (token-major, head at column head*D)
  const float lsum = xhalf_sum(l_run);
  const float inv = 1.f / lsum;
  if constexpr (LSE) {
    if (qrow < s && g == 0) nlse[(int64_t)bh * s + qrow] = -(m_used + __log2f(lsum));
  }
  if (qrow < s) {
    bf16 *dst = Aout + ((int64_t)bi * s + qrow) * ((int64_t)heads * D) + (int64_t)head * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(o[db][r4 * 4 + e] * inv);
        *reinterpret_cast<bf16x4 *>(dst + db * 32 + r4 * 8 + g * 4) = v;
      }
  }
}

} // namespace

hipError_t launch_attention_bf16(const void *Q, const void *K, const void *Vt, void *A,
                                 int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                                 int causal, hipStream_t stream, float *nlse) {
  if (batch <= 0 || seq <= 0) return hipSuccess;
  if (seq % 16 != 0 || seq * head_dim > ((int64_t)1 << 30)) return hipErrorInvalidValue;
  const int64_t n_qt = (seq + BQ - 1) / BQ;
  const int64_t bh = batch * heads;
  if (bh > INT32_MAX || n_qt > 65535) return hipErrorInvalidValue;
  dim3 grid((unsigned)bh, (unsigned)n_qt), block(NT);
  const bf16 *q = reinterpret_cast<const bf16 *>(Q);
  const bf16 *k = reinterpret_cast<const bf16 *>(K);
  const bf16 *v = reinterpret_cast<const bf16 *>(Vt);
  bf16 *a = reinterpret_cast<bf16 *>(A);
#define BPT_ATTN_LAUNCH(DD)                                                                        \
  if (nlse)                                                                                         \
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<DD, true>), grid, block, 0, stream, q, k, v, a,       \
                       (int)seq, (int)heads, causal, (int)n_qt, nlse);                              \
  else                                                                                             \
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<DD, false>), grid, block, 0, stream, q, k, v, a,      \
                       (int)seq, (int)heads, causal, (int)n_qt, nlse);
  switch (head_dim) {
  case 32:
    BPT_ATTN_LAUNCH(32)
    break;
  case 64:
    BPT_ATTN_LAUNCH(64)
    break;
  case 128:
    BPT_ATTN_LAUNCH(128)
    break;
  default:
    return hipErrorInvalidValue;
  }
#undef BPT_ATTN_LAUNCH
  return hipGetLastError();
}

} // namespace bpt
