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
// Block sizes. A workgroup owns ROWS query rows of one (batch, head) (a
// query block of the method is B_q / ROWS workgroups), as WQ waves of 32
// query columns each (ROWS = 16 uses half of one wave's columns: the MFMA
// tile is 32 wide). The inner loop walks the keys in stages of KB (16, 32
// or 64) and folds the running statistics once per stage; a key/value block
// of the method is B_kv / KB stages, so a stage never straddles a block
// boundary (the online update is exact for any partition of the keys).
//
// GPU mapping:
//  * one workgroup = ROWS query rows of one (batch, head): WQ waves × 32
//    rows, at most two waves per SIMD;
//  * K and V^T stages of KB keys go HBM/L2 -> LDS with buffer_load_dwordx4
//    ... lds (no register staging), four buffers deep, K three stages ahead
//    and V^T two;
//  * scores are computed transposed, S^T = K·Q^T, on v_mfma_f32_32x32x16_bf16
//    with Q held in registers as the B operand. Each lane then owns one query
//    column: its row max / row sum need one permlane32 swap with the lane 32
//    apart, and the rescale of its output column is a per-lane scalar. A
//    16-key stage fills rows 0..15 of the 32-row score block; the other rows
//    are never used;
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
//    crossing the diagonal are masked, and each workgroup takes a long and a
//    short query tile of one head (n_qt-1-p, then p), so that all
//    workgroups carry the same number of stages;
//  * an XCD's CUs work on one (batch, head) at a time (XCD x takes x, x+8,
//    ... in turn), so its L2 serves that head's K/V stream to every CU that
//    reads it.
#pragma once

#include "bpt_internal.h"
#include "lds_dma.h"

#include <math.h>

namespace bpt {
namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int NSTAGE = 4; // LDS buffers: stage st in st % 4, K three stages ahead, V^T two
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

template <int D, int WQ, int KB> struct AttnCfg {
  static_assert(D == 32 || D == 64 || D == 128, "head dim");
  static_assert(WQ == 1 || WQ == 2 || WQ == 4 || WQ == 8, "waves per workgroup");
  static_assert(KB == 16 || KB == 32 || KB == 64, "keys per stage");
  static constexpr int NT = 64 * WQ;              // threads per workgroup
  static constexpr int DK = D / 16;              // MFMA k-steps over the head dim (S^T)
  static constexpr int DB = D / 32;              // 32-row blocks of O^T
  // K is laid out in LDS as panels of up to 64 head-dim columns, so that
  // rows are at most 128 B: [panel][key][<=64 d], 16-byte chunks swizzled
  // with (key >> 1) & (NC - 1).
  static constexpr int PW = D < 64 ? D : 64;     // panel width (elements)
  static constexpr int NC = PW / 8;              // 16-byte chunks per panel row
  static constexpr int KPB = 1024 / (PW * 2);    // keys per KiB block of K
  static constexpr int BPP = KB / KPB;           // KiB blocks per panel
  static constexpr int NBLK = KB * D * 2 / 1024; // KiB blocks per K (and per V^T) stage
  // V^T is laid out as [d][KB keys], VC 16-byte chunks per row, chunk c of
  // row r at c ^ ((r >> 1) & (VC - 1))
  static constexpr int VC = KB / 8;
  static constexpr int VRPB = 64 / VC;           // V^T rows per KiB block
  static constexpr int LOADS = (NBLK + WQ - 1) / WQ; // most loads one wave issues per operand stage
  static constexpr int NKB = KB >= 32 ? KB / 32 : 1; // 32-key score blocks per stage
  static constexpr int RV = KB >= 32 ? 16 : 8;   // score registers of a block that hold keys
  static constexpr int NU = KB / 4;              // weight units per stage (2 weights per lane)
  static constexpr int NPV = KB / 16;            // P·V k-steps per 32-row block of O^T
  static_assert(BPP >= 1 && NBLK >= 1, "stage geometry");
  // waves per SIMD the compiler targets: two, or what the LDS of the K and
  // V^T rings (16·KB·D bytes per workgroup, 160 KiB per CU) allows
  static constexpr int WG_PER_CU = 163840 / (16 * KB * D);
  static constexpr int OCC = WG_PER_CU * WQ >= 8 ? 2 : 1;
};

// LSE: also write each row's negated log-sum-exp, -(m_used + log2(l)) in the
// log2 units of the pre-scaled scores, to nlse[(b·heads + head)·s + row] (for
// the backward pass, which recomputes the weights as exp2(score - nlse) from
// products that start at -nlse: stored negated, it loads straight into them).
// rows: query rows per workgroup (32·WQ, or 16 when WQ = 1).
template <int D, bool LSE, int WQ, int KB>
__global__ __launch_bounds__(64 * WQ, (AttnCfg<D, WQ, KB>::OCC)) void attn_fwd_bf16_kernel(
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ Vt,
    bf16 *__restrict__ Aout, int s, int heads, int n_bh, int causal, int n_qt, int rows,
    float *__restrict__ nlse) {
  using C = AttnCfg<D, WQ, KB>;
  constexpr int DK = C::DK, DB = C::DB, PW = C::PW, NC = C::NC, NKB = C::NKB, RV = C::RV;
  constexpr int NU = C::NU, NPV = C::NPV, VC = C::VC;

  __shared__ __attribute__((aligned(1024))) bf16 Ks[NSTAGE][KB * D];
  __shared__ __attribute__((aligned(1024))) bf16 Vs[NSTAGE][D * KB];

  // workgroup and work-item ids through the builtins: these files are
  // compiled with IEEE mode off, which the device library's id functions do
  // not share, so blockIdx / threadIdx would become out-of-line calls (with
  // a call stack in scratch memory).
  //
  // Work of a workgroup: causal (and more than one wave), the query tiles
  // n_qt-1-p and p of one (batch, head) in turn (one tile when they
  // coincide), so every workgroup walks n_qt + 1 tiles' worth of key stages
  // and the workgroups of a dispatch round start, stream K/V and finish
  // together; otherwise tile n_qt-1-p (the loop over two tiles spills SGPRs
  // in the one-wave instances with 64-key stages). Workgroups go to the 8 XCDs
  // round-robin in dispatch order; when n_bh is a multiple of 8, XCD x takes
  // the (batch, head)s x, x+8, ... one after the other, so all its CUs read
  // one head's K/V stream at a time through its L2.
  const unsigned wg = __builtin_amdgcn_workgroup_id_x();
  const bool paired = WQ > 1 && causal && n_qt > 1;
  const int npw = paired ? (n_qt + 1) / 2 : n_qt; // workgroups per (batch, head)
  int bh, p;
  if ((n_bh & 7) == 0) {
    const int k = (int)(wg >> 3), hl = k / npw;
    bh = hl * 8 + (int)(wg & 7u);
    p = k - hl * npw;
  } else {
    bh = (int)(wg % (unsigned)n_bh);
    p = (int)(wg / (unsigned)n_bh);
  }
  // the tiles, in turn: qt_first, then qt_last when it differs
  const int qt_first = n_qt - 1 - p;
  const int qt_last = paired ? p : qt_first;
  const int bi = bh / heads, head = bh - bi * heads;
  const bf16 *Qh = Q + (int64_t)bh * s * D;
  const bf16 *Kh = K + (int64_t)bh * s * D;
  const bf16 *Vh = Vt + (int64_t)bh * D * s;
  // one head's K and V^T, s·D bf16 each (the host keeps s·D·2 below 2^31)
  const i32x4 krsrc = make_rsrc(Kh, (unsigned)s * D * 2u);
  const i32x4 vrsrc = make_rsrc(Vh, (unsigned)s * D * 2u);

  const int tid = (int)__builtin_amdgcn_workitem_id_x();

#pragma nounroll
  for (int qt = qt_first;; qt = qt_last) {
    // (the ids pass through an empty asm at each tile, so that nothing
    // derived from them is hoisted out of this loop and held across both
    // tiles in registers)
    int tid_ = tid;
    asm volatile("" : "+v"(tid_));
    const int lane = tid_ & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid_ >> 6); // wave-uniform, in an SGPR
    __builtin_assume(wave < WQ);
    const int l32 = lane & 31, g = lane >> 5;
    const int q0 = qt * rows;
    const int row_end = min(s, q0 + rows); // rows of this tile: q0 .. row_end - 1
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

    const int kv_end = causal ? row_end : s;
    const int n_st = (kv_end + KB - 1) / KB; // stages the workgroup stages through LDS
    const int wq_last = min(qw0 + 31, row_end - 1);
    // stages this wave computes: those holding a key <= its last query
    // (a wave past row_end, possible only in a partial last tile, computes
    // none but still takes every step's barrier)
    const int nw = wq_last < qw0 ? 0 : (causal ? min(n_st, wq_last / KB + 1) : n_st);

    // ---- staging into LDS buffers (stage x of K in Ks[x % 4], of V^T in
    // Vs[x % 4]). A KiB block of K holds KPB keys of one panel; a KiB block of
    // V^T holds VRPB head-dim rows of KB keys. Lane L writes LDS bytes
    // 16L..16L+15 of the block, so it fetches the global chunk that the
    // swizzle puts there. koff / voff: byte offsets of this lane's chunks in
    // stage 0; stage st adds st·KB·D·2 (K) or st·KB·2 (V^T). A K row at or past
    // s lies outside the K buffer, which reads it as zeros (its scores are
    // masked); a V^T chunk past s holds finite data of the next head-dim row,
    // or zeros past the buffer, and meets a zero weight.
    // The offsets of a wave's first HOLD loads per operand are held in
    // registers; a wave with more loads per stage (fewer waves per
    // workgroup) computes the rest when it issues them.
    auto k_offset = [&](int blk) __attribute__((always_inline)) {
      const int panel = blk / C::BPP;
      const int key = (blk % C::BPP) * C::KPB + lane / NC;
      const int kch = (lane % NC) ^ ((key >> 1) & (NC - 1));
      return (unsigned)(key * D + panel * PW + kch * 8) * 2u;
    };
    auto v_offset = [&](int blk) __attribute__((always_inline)) {
      const int drow = blk * C::VRPB + lane / VC;
      const int vch = (lane % VC) ^ ((drow >> 1) & (VC - 1));
      return (unsigned)(drow * s + vch * 8) * 2u;
    };
    constexpr int HOLD = C::LOADS < 2 ? C::LOADS : 2;
    unsigned koff[HOLD], voff[HOLD];
#pragma unroll
    for (int i = 0; i < HOLD; ++i) {
      koff[i] = k_offset(wave + WQ * i);
      voff[i] = v_offset(wave + WQ * i);
    }
    auto issue_k1 = [&](int st, int i) __attribute__((always_inline)) {
      if (wave + WQ * i < C::NBLK)
        load_lds16(krsrc, (i < HOLD ? koff[i < HOLD ? i : 0] : k_offset(wave + WQ * i)) +
                              (unsigned)st * (unsigned)(KB * D * 2),
                   &Ks[st % NSTAGE][(wave + WQ * i) * 512]);
    };
    auto issue_v1 = [&](int st, int i) __attribute__((always_inline)) {
      if (wave + WQ * i < C::NBLK)
        load_lds16(vrsrc, (i < HOLD ? voff[i < HOLD ? i : 0] : v_offset(wave + WQ * i)) +
                              (unsigned)st * (unsigned)(KB * 2),
                   &Vs[st % NSTAGE][(wave + WQ * i) * 512]);
    };
    auto issue_k = [&](int st) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) issue_k1(st, i);
    };
    auto issue_v = [&](int st) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) issue_v1(st, i);
    };

    // K row this lane's A fragments come from: key l32 of a 32-key block (a
    // 16-key stage has 16 rows; lanes 16..31 re-read rows 0..15 into score
    // rows that are never used)
    const int krow = KB >= 32 ? l32 : (l32 & (KB - 1));
    const int kswz = (krow >> 1) & (NC - 1); // K chunk swizzle of that row
    const int vswz = (l32 >> 1) & (VC - 1);  // V^T chunk swizzle for drow = db*32 + l32
    const bf16x2 ones = {(bf16)1.f, (bf16)1.f};

    // S^T - m_used of stage st (KB keys x this wave's 32 queries)
    auto scores = [&](int st, f32x16 (&sa)[NKB]) __attribute__((always_inline)) {
      const bf16 *kbase = &Ks[st % NSTAGE][krow * PW];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
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
    auto mask_if_needed = [&](int st, f32x16 (&sa)[NKB]) __attribute__((always_inline)) {
      const int k0 = st * KB;
      if ((causal && k0 + KB - 1 > qw0) || k0 + KB > s) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < RV; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= s || (causal && key > qrow)) sa[kb][r] = -INFINITY;
          }
      }
    };
    auto row_max = [&](const f32x16 (&sa)[NKB]) __attribute__((always_inline)) {
      float a = sa[0][0];
      if constexpr (NKB == 2) {
        a = fmaxf(sa[0][0], sa[1][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) a = fmaxf(fmaxf(a, sa[0][r]), sa[1][r]); // v_max3 chain
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < RV; ++r) a = fmaxf(a, sa[kb][r]);
      }
      return xhalf_max(a);
    };
    // unit u (0..NU-1) of a stage's weights: two bf16 weights exp2(score) of
    // score block kb = u / 8 into pf, and their sum into the row-sum partial
    // rs[u & 1] (added to, not reset). Units 0..7 read only score block 0.
    auto unit = [&](const f32x16 (&sa)[NKB], bf16x8 (&pf)[NKB][2], float (&rs)[2], int u) __attribute__((always_inline)) {
      const int kb = u >> 3, r = (u & 7) * 2;
      bf16x2 pp;
      pp[0] = (bf16)__builtin_amdgcn_exp2f(sa[kb][r]);
      pp[1] = (bf16)__builtin_amdgcn_exp2f(sa[kb][r + 1]);
      pf[kb][r >> 3][r & 7] = pp[0];
      pf[kb][r >> 3][(r & 7) + 1] = pp[1];
      rs[u & 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, rs[u & 1], false);
    };
    // all weights of one stage
    auto weights_rs = [&](const f32x16 (&sa)[NKB], bf16x8 (&pf)[NKB][2], float (&rs)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < NU; ++u) unit(sa, pf, rs, u);
    };
    // Rare path, after a stage's weights exceeded WEIGHT_LIMIT in some row
    // (the row-sum partials bound every weight, which are >= 0; an overflowed
    // weight makes its partial inf): move the reference max up to the
    // stage's row max, rescale O and l by the exact factor, shift this stage's
    // and the next stage's relative scores, and recompute the weights.
    auto rescale_stage = [&](f32x16 (&s_cur)[NKB], f32x16 (&s_nxt)[NKB], bf16x8 (&pf)[NKB][2],
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
      for (int kb = 0; kb < NKB; ++kb)
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
    auto pv_stage = [&](int st, const bf16x8 (&pf)[NKB][2]) __attribute__((always_inline)) {
      const bf16 *vbase = &Vs[st % NSTAGE][l32 * KB];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < NPV; ++j) {
          const int kb = j >> 1, hf = j & 1;
          const int ch = kb * 4 + hf * 2 + g;
          const bf16x8 vf =
              *reinterpret_cast<const bf16x8 *>(vbase + db * 32 * KB + ((ch ^ vswz) << 3));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][hf], o[db], 0, 0, 0);
        }
    };

    // ---- the general step (stages that need a mask, and the last ones):
    // scores of stage st+1, then the weights, limit check and P·V of stage st
    auto step = [&](int st, f32x16 (&s_cur)[NKB], f32x16 (&s_nxt)[NKB]) __attribute__((always_inline)) {
      if (st + 3 < n_st) issue_k(st + 3);
      if (st + 2 < n_st) issue_v(st + 2);
      if (st < nw) {
        const bool has_next = st + 1 < nw;
        if (has_next) {
          scores(st + 1, s_nxt);
          mask_if_needed(st + 1, s_nxt);
        }
        bf16x8 pf[NKB][2];
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
    constexpr int NS = NKB * DK, NP = NPV * DB, LA = 3;
    // The step's loads into LDS are spread over its slots (load j at slot
    // 1 + j·(NS+NP)/(2·LOADS), the last slot at most: small tiles have fewer
    // slots than loads) rather than issued together after the barrier, where
    // all waves would queue theirs at the texture unit at once.
    constexpr int NLD = 2 * C::LOADS;
    constexpr auto load_slot = [](int j) {
      const int sl = 1 + j * (NS + NP) / NLD;
      return sl < NS + NP - 1 ? sl : NS + NP - 1;
    };
    static_assert(load_slot(NLD - 1) < NS + NP && load_slot(0) >= 0, "every load has a slot");
    // The weights of a stage come in two halves: units 0..H-1 during the P·V
    // half of the previous step, units H..NU-1 during the score half of the
    // stage's own step, so each half of a step carries half of the
    // exponentials. On entry pf and rs hold units 0..H-1 of stage st; the step
    // leaves units 0..H-1 of stage st+1 in pf_n and rs_n.
    constexpr int H = NU / 2;
    auto step_bulk = [&](int st, f32x16 (&s_cur)[NKB], f32x16 (&s_nxt)[NKB], bf16x8 (&pf)[NKB][2],
                         float (&rs)[2], bf16x8 (&pf_n)[NKB][2], float (&rs_n)[2]) __attribute__((always_inline)) {
      // V(st+2) always exists here (st+2 < n_um); K(st+3) may be one stage past
      // the last, which lands in a free buffer and is never read
      const bf16 *kbase = &Ks[(st + 1) % NSTAGE][krow * PW];
      const bf16 *vbase = &Vs[st % NSTAGE][l32 * KB];
      // read r < NS: K fragment of score MFMA r; else V^T fragment of P·V MFMA r - NS
      auto frag = [&](int r) __attribute__((always_inline)) -> bf16x8 {
        if (r < NS) {
          const int kb = r / DK, gc = (r % DK) * 2 + g;
          return *reinterpret_cast<const bf16x8 *>(kbase + kb * 32 * PW + (gc / NC) * (KB * PW) +
                                                   (((gc % NC) ^ kswz) << 3));
        }
        const int j = r - NS, db = j / NPV, jj = j % NPV, kb = jj >> 1, hf = jj & 1;
        const int ch = kb * 4 + hf * 2 + g;
        return *reinterpret_cast<const bf16x8 *>(vbase + db * 32 * KB + ((ch ^ vswz) << 3));
      };
      bf16x8 ring[LA + 1];
#pragma unroll
      for (int r = 0; r < LA; ++r) ring[r] = frag(r);
      rs_n[0] = rs_n[1] = 0.f;
      // one issue slot: its loads, its MFMA, the read LA slots ahead, and a
      // share of the weights: units H..NU-1 of stage st in the score half,
      // units 0..H-1 of stage st+1 in the P·V half
      auto slot_work = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NLD; ++j)
          if (slot == load_slot(j)) {
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
          const int j = slot - NS, db = j / NPV, jj = j % NPV, kb = jj >> 1, hf = jj & 1;
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr, pf[kb][hf], o[db], 0, 0, 0);
        }
        if (slot + LA < NS + NP) ring[(slot + LA) % (LA + 1)] = frag(slot + LA);
        if (slot < NS) {
#pragma unroll
          for (int u = slot * H / NS; u < (slot + 1) * H / NS; ++u) unit(s_cur, pf, rs, H + u);
        } else {
#pragma unroll
          for (int u = (slot - NS) * H / NP; u < (slot - NS + 1) * H / NP; ++u) unit(s_nxt, pf_n, rs_n, u);
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
    f32x16 sA[NKB], sB[NKB];
    scores(0, sA); // m_used = 0: the raw scores
    mask_if_needed(0, sA);
    // the reference max starts at stage 0's row max (finite: key 0 is never
    // masked), so every row's largest weight is at least 1
    m_used = row_max(sA);
#pragma unroll
    for (int r = 0; r < 16; ++r) minit[r] = -m_used;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sA[kb][r] -= m_used;
    // units 0..H-1 of stage 0, carried into the first bulk step (a general step
    // recomputes all of its weights)
    bf16x8 pfA[NKB][2], pfB[NKB][2];
    float rsA[2] = {0.f, 0.f}, rsB[2] = {0.f, 0.f};
#pragma unroll
    for (int u = 0; u < H; ++u) unit(sA, pfA, rsA, u);

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
      if (qrow < row_end && g == 0) nlse[(int64_t)bh * s + qrow] = -(m_used + __log2f(lsum));
    }
    if (qrow < row_end) {
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
    if (qt == qt_last) break;
  }
}

// Launch for one head dim: rows per workgroup in {16, 32, 64, 128, 256}
// (256 and keys 64 also with the log-sum-exp output), keys per stage in
// {16, 32, 64}.
template <int D>
hipError_t launch_d(const void *Q, const void *K, const void *Vt, void *A, int64_t batch,
                    int64_t seq, int64_t heads, int causal, int rows, int keys, hipStream_t stream,
                    float *nlse) {
  const int64_t n_qt = (seq + rows - 1) / rows;
  const int64_t bh = batch * heads;
  // workgroups per (batch, head): causal ones of more than one wave take two
  // tiles (see the kernel)
  const int64_t npw = rows > 32 && causal && n_qt > 1 ? (n_qt + 1) / 2 : n_qt;
  if (bh * npw > (int64_t)UINT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(bh * npw));
  const bf16 *q = reinterpret_cast<const bf16 *>(Q);
  const bf16 *k = reinterpret_cast<const bf16 *>(K);
  const bf16 *v = reinterpret_cast<const bf16 *>(Vt);
  bf16 *a = reinterpret_cast<bf16 *>(A);
  if (nlse) {
    if (rows != 256 || keys != 64) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, true, 8, 64>), grid, dim3(512), 0, stream, q, k, v,
                       a, (int)seq, (int)heads, (int)bh, causal, (int)n_qt, rows, nlse);
    return hipGetLastError();
  }
#define BPT_ATTN_CASE(WQ_, KB_)                                                                    \
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false, WQ_, KB_>), grid, dim3(64 * WQ_), 0, stream,  \
                     q, k, v, a, (int)seq, (int)heads, (int)bh, causal, (int)n_qt, rows, nlse)
#define BPT_ATTN_KEYS(WQ_)                                                                         \
  switch (keys) {                                                                                  \
  case 16: BPT_ATTN_CASE(WQ_, 16); break;                                                          \
  case 32: BPT_ATTN_CASE(WQ_, 32); break;                                                          \
  case 64: BPT_ATTN_CASE(WQ_, 64); break;                                                          \
  default: return hipErrorInvalidValue;                                                            \
  }
  switch (rows) {
  case 16:
  case 32: BPT_ATTN_KEYS(1) break;
  case 64: BPT_ATTN_KEYS(2) break;
  case 128: BPT_ATTN_KEYS(4) break;
  case 256: BPT_ATTN_KEYS(8) break;
  default: return hipErrorInvalidValue;
  }
#undef BPT_ATTN_KEYS
#undef BPT_ATTN_CASE
  return hipGetLastError();
}

} // namespace attn
} // namespace bpt
