// bf16 GEMM on CDNA4 matrix cores with fused epilogues.
//
// Serves the four dense contractions of the BPT layer (BPT paper review, §三
// "核心公式" and Algorithm 1): the fused QKV projection over the whole sequence
// (epilogue: bias, split into heads, Q multiplied by log2(e)/sqrt(d) for the
// attention's exp2), the output projection with the first
// residual, the FFN up-projection with bias and ReLU, and the FFN
// down-projection with the second residual. The layer backward uses two more:
// the ReLU mask of the FFN's hidden gradient and fp32 (accumulated) weight
// gradients.
//
// C[M, N] = A[M, K] · Bt[N, K]^T. Both operands are K-contiguous, which is
// what the v_mfma_f32_32x32x16_bf16 operand layout wants (each lane holds 8
// consecutive K values of one row of A and one column of B).
//
// Tiling: 256×256 output tile per workgroup of 4 waves (2×2), each wave a
// 128×128 sub-tile = 4×4 MFMA blocks of 32×32 (256 fp32 accumulators per
// lane, in the AGPR half of the unified register file). K advances by 32 per
// step through four LDS stages (4 × 32 KiB), loaded three steps ahead so that
// HBM/L2 latency is covered by two steps of MFMA work. Tiles are staged with
// buffer_load_dwordx4 ... lds (memory -> LDS without passing through
// registers): each wave instruction fills one contiguous KiB of LDS, lane L
// writing bytes 16L..16L+15, so the XOR swizzle of the 16-byte chunk index
// (chunk ^ ((row >> 2) & 3) for rows of 64 B: the 16 lanes of one LDS cycle
// hit 16 distinct 16-byte bank groups) is applied by choosing which global
// chunk each lane fetches. Each step is one barrier and 32 issue slots of one
// MFMA each: fragment reads of the next step (double-buffered in registers)
// and the loads of a later stage are spread over the slots.
//
// Orientation: with SWAP the MFMA computes Bt·A^T blocks, so each lane holds
// one output ROW and 4 consecutive output COLUMNS per register group, which
// turns row-major epilogue stores into 8-byte vector stores. Without SWAP a
// lane holds 4 consecutive ROWS of one column, which is what the transposed-V
// scatter needs.
#include "bpt_internal.h"
#include "lds_dma.h"
#include "philox.h"

#include <type_traits>

namespace bpt {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 256, TN = 256, TK = 32;
constexpr int NT = 256;
constexpr int NSTAGE = 4, AHEAD = 3;
constexpr int TILE_ELEMS = TM * TK;      // one operand tile in LDS (bf16 elements)
constexpr int LOADS_PER_WAVE = TM * TK * 2 / 1024 / 4; // KiB blocks per operand per wave = 4
constexpr int ROWS_PER_BLK = 1024 / (TK * 2);          // 16 rows of 64 B per KiB
// The ReLU and Q|K epilogues stage each wave's 128 x 128 sub-tile in LDS
// of its own: 64 rows at a time, rows padded to WS_ROW floats (4 waves:
// 132 KiB). (The same staging measured slower for the residual epilogues,
// whose residual loads favour whole 512-byte rows.)
template <int EPI, bool SWAP> constexpr bool WAVE_STAGED = SWAP && (EPI == EPI_RELU || EPI == EPI_QK);
constexpr int WS_ROW = 132;
constexpr int WS_ELEMS = 4 * 64 * WS_ROW * 2; // in bf16 elements

// Key position inside a 16-key group in the transposed-V layout: bits 2 and 3
// swapped, so that the 8 keys one lane feeds to the P·V MFMA are contiguous.
__device__ __forceinline__ int vt_perm(int t) {
  return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1);
}

__device__ __forceinline__ float bf2f(bf16 v) { return (float)v; }

typedef __attribute__((address_space(4))) const uint32_t *const_u32p;

using dev::i32x4;
using dev::load_lds16;
using dev::make_rsrc;

// MN (EPI_ACC32 only): both operands token-major, A [K, M] and Bt [K, N]
// (row strides lda, ldb), i.e. the product out = Aᵀ·Bt over K tokens, read
// without a transposed copy: each stage holds 32 rows of K × 256 columns
// (chunk c of row r at c ^ 4·(r & 3)), and the fragments come out of it by
// transposing LDS reads (see frag_tr). Rows at or past ep.mn_rows read zero.
template <int EPI, bool SWAP, bool MN = false>
__global__ __launch_bounds__(NT, 1) void gemm_bf16_kernel(const bf16 *__restrict__ A, int64_t lda,
                                                          const bf16 *__restrict__ Bt, int64_t ldb,
                                                          int M, int N, int K, GemmEpilogue ep) {
  __shared__ __attribute__((aligned(1024))) bf16 smem[WAVE_STAGED<EPI, SWAP> ? WS_ELEMS : NSTAGE * 2 * TILE_ELEMS];

  const int tiles_m = (M + TM - 1) / TM;
  const int tiles_n = (N + TN - 1) / TN;
  const int total = tiles_m * tiles_n;
  // K-split layer (EPI_ACC32 only; gridDim.y is 1 otherwise)
  if constexpr (EPI == EPI_ACC32) {
    if constexpr (MN) {
      A += (int64_t)blockIdx.y * K * lda;
      Bt += (int64_t)blockIdx.y * K * ldb;
    } else {
      A += (int64_t)blockIdx.y * K;
      Bt += (int64_t)blockIdx.y * K;
    }
  }

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // wave-uniform
  __builtin_assume(wave < 4);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, g = lane >> 5;

  // staging: wave w fills LDS KiB-blocks w*4 .. w*4+3 of each operand tile;
  // block b = rows 16b .. 16b+15; lane -> (row 16b + lane/4, LDS chunk
  // lane%4), fetching global chunk (lane%4) ^ ((row >> 2) & 3). The buffer
  // descriptors span this tile's valid rows of A and Bt only, so the rows of
  // a partial tile past M (or N) read as zeros; a_goff / b_goff are the byte
  // offsets of this lane's chunks at k = 0, and step kt adds kt·TK·2.
  i32x4 a_rsrc, b_rsrc;
  uint32_t a_goff[LOADS_PER_WAVE], b_goff[LOADS_PER_WAVE];
  if constexpr (MN) {
    // KiB block b of a stage = rows 2b, 2b+1 (512 bytes each); lane L fills
    // chunk L % 32 of row 2b + L / 32 from global chunk (L % 32) ^ 4·(row & 3).
    // The descriptors start at this tile's first column and end with this
    // layer's last valid row (past it everything reads as zero; a partial
    // tile's columns past the row wrap into the next row, whose products only
    // reach outputs that are never stored).
    const int64_t kz = (int64_t)ep.mn_rows - (int64_t)blockIdx.y * K;
    const int64_t rows_k = kz < K ? kz : K;
    a_rsrc = make_rsrc(A + (int64_t)tm * TM, (uint32_t)((rows_k * lda - (int64_t)tm * TM) * 2));
    b_rsrc = make_rsrc(Bt + (int64_t)tn * TN, (uint32_t)((rows_k * ldb - (int64_t)tn * TN) * 2));
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i) {
      const int row = 2 * (wave * LOADS_PER_WAVE + i) + (lane >> 5);
      const int ch = (lane & 31) ^ (4 * (row & 3));
      a_goff[i] = (uint32_t)(row * lda + ch * 8) * 2u;
      b_goff[i] = (uint32_t)(row * ldb + ch * 8) * 2u;
    }
  } else {
    const int rows_a = min(TM, M - tm * TM), rows_b = min(TN, N - tn * TN);
    a_rsrc = make_rsrc(A + (int64_t)tm * TM * lda, (uint32_t)(rows_a * lda * 2));
    b_rsrc = make_rsrc(Bt + (int64_t)tn * TN * ldb, (uint32_t)(rows_b * ldb * 2));
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i) {
      const int row = (wave * LOADS_PER_WAVE + i) * ROWS_PER_BLK + (lane >> 2);
      const int ch = (lane & 3) ^ ((row >> 2) & 3);
      a_goff[i] = (uint32_t)(row * lda + ch * 8) * 2u;
      b_goff[i] = (uint32_t)(row * ldb + ch * 8) * 2u;
    }
  }
  // load i of a stage: i < 4 the A block i of this wave, else the B block i-4
  auto stage_one = [&](int kt, int buf, int i) {
    bf16 *As = smem + buf * 2 * TILE_ELEMS;
    const uint32_t ko_a = MN ? (uint32_t)kt * (uint32_t)(TK * lda * 2) : (uint32_t)kt * (TK * 2);
    const uint32_t ko_b = MN ? (uint32_t)kt * (uint32_t)(TK * ldb * 2) : (uint32_t)kt * (TK * 2);
    if (i < LOADS_PER_WAVE)
      load_lds16(a_rsrc, a_goff[i] + ko_a, As + (wave * LOADS_PER_WAVE + i) * 512);
    else
      load_lds16(b_rsrc, b_goff[i - LOADS_PER_WAVE] + ko_b,
                 As + TILE_ELEMS + (wave * LOADS_PER_WAVE + i - LOADS_PER_WAVE) * 512);
  };
  auto stage = [&](int kt, int buf) {
#pragma unroll
    for (int i = 0; i < 2 * LOADS_PER_WAVE; ++i) stage_one(kt, buf, i);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment read offsets (elements) inside an operand tile
  int a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (MN) {
      // transposing reads: within each 16-lane group lane j addresses row
      // kb + j/4, columns c0 + 4·(j % 4) .. +3 and receives rows kb .. kb+3
      // of column c0 + (j of the receiving lane); here kb = 16·ks + 8g (+4)
      // and c0 = the block's column + 16·((lane >> 4) & 1). Rows kb + j/4
      // have (row & 3) = (j >> 2) & 3, so the swizzle is lane-constant.
      const int j = lane & 15, sw = 4 * ((j >> 2) & 3);
      const int ca = wm * 128 + i * 32 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
      const int cb = wn * 128 + i * 32 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
      const int r = 8 * g + (j >> 2);
      a_off[i] = r * TM + (((ca >> 3) ^ sw) << 3) + (ca & 7);
      b_off[i] = r * TN + (((cb >> 3) ^ sw) << 3) + (cb & 7);
    } else {
      a_off[i] = (wm * 128 + i * 32 + l32) * TK;
      b_off[i] = (wn * 128 + i * 32 + l32) * TK;
    }
  }
  const int swz = (l32 >> 2) & 3; // ((row >> 2) & 3) for row = 32*i + l32
  // MN: the fragment of k-substep ks at offset o: rows 16·ks + {0..3, 4..7}
  // past the lane's base row, two transposing reads
  auto frag_tr = [&](const bf16 *T, int o, int ks) __attribute__((always_inline)) {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    typedef __bf16 b16x4 __attribute__((ext_vector_type(4)));
    const bf16 *p = T + o + ks * 16 * TM;
    const b16x4 lo = __builtin_bit_cast(b16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p));
    const b16x4 hi = __builtin_bit_cast(b16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 4 * TM)));
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = lo[e];
      f[4 + e] = hi[e];
    }
    return f;
  };

  // all fragments of one K step: [k-substep][block]
  struct Frags {
    bf16x8 a[TK / 16][4], b[TK / 16][4];
  };
  auto read_step = [&](int kt, Frags &f) {
    const bf16 *As = smem + (kt % NSTAGE) * 2 * TILE_ELEMS;
    const bf16 *Bs = As + TILE_ELEMS;
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      const int kc = ((ks * 2 + g) ^ swz) << 3;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (MN) {
          f.a[ks][i] = frag_tr(As, a_off[i], ks);
          f.b[ks][i] = frag_tr(Bs, b_off[i], ks);
        } else {
          f.a[ks][i] = *reinterpret_cast<const bf16x8 *>(As + a_off[i] + kc);
          f.b[ks][i] = *reinterpret_cast<const bf16x8 *>(Bs + b_off[i] + kc);
        }
      }
    }
  };
  // fragment r of a step (r < 16: k-substep r / 8; A block r % 8 for
  // r % 8 < 4, else B block r % 8 - 4)
  auto read_one = [&](int kt, Frags &f, int r) {
    const bf16 *As = smem + (kt % NSTAGE) * 2 * TILE_ELEMS;
    const int ks = r / 8, q = r % 8;
    const int kc = ((ks * 2 + g) ^ swz) << 3;
    if constexpr (MN) {
      if (q < 4)
        f.a[ks][q] = frag_tr(As, a_off[q], ks);
      else
        f.b[ks][q - 4] = frag_tr(As + TILE_ELEMS, b_off[q - 4], ks);
    } else {
      if (q < 4)
        f.a[ks][q] = *reinterpret_cast<const bf16x8 *>(As + a_off[q] + kc);
      else
        f.b[ks][q - 4] = *reinterpret_cast<const bf16x8 *>(As + TILE_ELEMS + b_off[q - 4] + kc);
    }
  };
  auto mfma_one = [&](const Frags &f, int q) {
    const int ks = q / 16, i = (q / 4) % 4, j = q % 4;
    if constexpr (SWAP)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[ks][j], f.a[ks][i], acc[i][j], 0, 0, 0);
    else
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[ks][i], f.b[ks][j], acc[i][j], 0, 0, 0);
  };

  const int KT = K / TK;
  // One K step, after a barrier at which stage kt+1 has landed (only the
  // loads of stage kt+2 may still be in flight) and every wave has finished
  // reading stage kt-1. Then 32 issue slots of one MFMA each on the
  // fragments of step kt; every second slot also reads one fragment of step
  // kt+1 into the other register set, and every fourth slot issues one load
  // of stage kt+AHEAD into the buffer of stage kt-1, so that neither the LDS
  // reads nor the loads arrive as a burst. A scheduling fence after each
  // slot keeps this order. The last AHEAD steps have no stage to load.
  constexpr int NLOAD = 2 * LOADS_PER_WAVE; // loads per wave per stage
  static_assert(NLOAD == 8 && (TK / 16) * 16 == 32, "slot plan: 32 MFMAs, 16 reads, 8 loads");
  // The barrier does not wait for LDS reads: those of step kt+1 feed the
  // MFMAs of the next step, which wait for them; a wave passes the barrier
  // of step kt+2, where their buffer is refilled, only after those MFMAs.
  // A step's barrier leaves in flight the loads issued after the last one of
  // the stage it needs: those of the previous step (NLOAD), or none when the
  // previous step loaded nothing.
  auto body = [&](int kt, const Frags &cur, Frags &nxt, auto load_c, auto wait_c) {
    constexpr bool LOAD = decltype(load_c)::value;
    dev::barrier_vm_only<decltype(wait_c)::value>();
    const int ld_kt = kt + AHEAD, ld_buf = (kt + AHEAD) % NSTAGE;
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      mfma_one(cur, q);
      // (after the last step this reads a stale buffer; never used)
      if ((q & 1) == 0) read_one(kt + 1, nxt, q >> 1);
      if constexpr (LOAD) {
        if ((q & 3) == 1) stage_one(ld_kt, ld_buf, q >> 2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using Load = std::true_type;
  using NoLoad = std::false_type;
  using WaitPrev = std::integral_constant<int, NLOAD>;
  using WaitAll = std::integral_constant<int, 0>;

  // prologue: stages 0 .. AHEAD-1 (a short K re-stages its last tile; the
  // spare copies are never read), then the fragments of step 0 once stage 0
  // has landed
#pragma unroll
  for (int p = 0; p < AHEAD; ++p) stage(min(p, KT - 1), p);
  dev::barrier_vm<(AHEAD - 1) * NLOAD>();
  Frags f0, f1;
  read_step(0, f0);
  // steps 0 .. KL-1 load stage kt+AHEAD; the last min(KT, AHEAD) steps load
  // nothing (the first of them still follows a loading step, or the
  // prologue's last stage)
  const int KL = KT - AHEAD;
  int kt = 0;
  for (; kt + 1 < KL; kt += 2) {
    body(kt, f0, f1, Load{}, WaitPrev{});
    body(kt + 1, f1, f0, Load{}, WaitPrev{});
  }
  if (kt < KL) {
    body(kt, f0, f1, Load{}, WaitPrev{});
    ++kt;
    f0 = f1; // the fragments of step kt (register moves, once per tile)
  }
  body(kt, f0, f1, NoLoad{}, WaitPrev{});
  if (kt + 1 < KT) body(kt + 1, f1, f0, NoLoad{}, WaitAll{});
  if (kt + 2 < KT) body(kt + 2, f0, f1, NoLoad{}, WaitAll{});
  // no load into LDS outlives the loop (already so unless K is one step)
  dev::wait_vm<0>();

  // ---------------------------------------------------------------- epilogue
  // The finished tile goes out through LDS (the stage ring is free now).
  if constexpr (WAVE_STAGED<EPI, SWAP>) {
    // Each wave stages its own 128 x 128 sub-tile through its own LDS, 64
    // rows at a time as fp32 (written straight from the accumulators), and
    // reads it back as rows, lanes 0-31 one row and 32-63 the next, 4
    // columns per lane: no workgroup barrier after the one that frees the
    // stage ring, so one wave's stores overlap another's staging. Rows are
    // padded to WS_ROW floats: the 16 rows of a write phase and the 16
    // chunks of a row read fall on distinct 16-byte bank groups, and every
    // offset but the lane's is an immediate. Bias and ReLU (or the Q scale,
    // with the head scatter) are applied in fp32 on the way out and rounded
    // once.
    float *ws = reinterpret_cast<float *>(smem) + wave * 64 * WS_ROW;
    const bf16 *bias = reinterpret_cast<const bf16 *>(ep.bias);
    const int nc = tn * TN + wn * 128 + l32 * 4; // this lane's 4 output columns
    bf16x4 bw = {};
    if (nc < N) bw = *reinterpret_cast<const bf16x4 *>(bias + nc);
    // EPI_QK: the lane's 4 columns lie in one head of Q or K
    bf16 *qk_base = nullptr;
    float qs = 1.f;
    if constexpr (EPI == EPI_QK) {
      const int h = (int)ep.hidden, dlog = __builtin_ctz((unsigned)ep.head_dim);
      const int which = nc >= h, rem = nc - which * h;
      if (which == 0) qs = ep.q_scale;
      qk_base = reinterpret_cast<bf16 *>(which == 0 ? ep.q : ep.k) +
                (int64_t)(rem >> dlog) * ep.seq * ep.head_dim + (rem & ((1 << dlog) - 1));
    }
    __syncthreads(); // every wave is done with the stage ring
    float b4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) b4[e] = bf2f(bw[e]);
    float *wr = ws + l32 * WS_ROW + g * 4;       // write base: row l32, chunk g
    const float *rd = ws + g * WS_ROW + l32 * 4; // read base: row g, chunk l32
    const int64_t step = 2 * ep.ld_out;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * hh + ii;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            f32x4 v = {acc[i][j][r4 * 4 + 0], acc[i][j][r4 * 4 + 1], acc[i][j][r4 * 4 + 2],
                       acc[i][j][r4 * 4 + 3]};
            *reinterpret_cast<f32x4 *>(wr + ii * 32 * WS_ROW + j * 32 + r4 * 8) = v;
          }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); // this wave's rows are in LDS
      if (nc < N) {
        const int row0 = tm * TM + wm * 128 + hh * 64 + g; // rows row0 + 2·it
        bf16 *dst = reinterpret_cast<bf16 *>(ep.out) + (int64_t)row0 * ep.ld_out + nc;
        auto row_out = [&](int it) __attribute__((always_inline)) {
          const f32x4 v = *reinterpret_cast<const f32x4 *>(rd + it * 2 * WS_ROW);
          bf16x4 ov;
          if constexpr (EPI == EPI_QK) {
#pragma unroll
            for (int e = 0; e < 4; ++e) ov[e] = (bf16)((v[e] + b4[e]) * qs);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) ov[e] = (bf16)fmaxf(v[e] + b4[e], 0.f);
          }
          return ov;
        };
        if constexpr (EPI == EPI_QK) {
          // rows rb .. rb+63 of this half; token t of batch element bi at rb
          const int rb = row0 - g, sq = (int)ep.seq;
          const int bi = rb / sq, t = rb - bi * sq;
          const int64_t hd = ep.head_dim;
          if (t + 64 <= sq && rb + 64 <= M) {
            // one batch element, all rows valid: two tokens per step
            bf16 *q = qk_base + ((int64_t)bi * ep.heads * sq + t + g) * hd;
#pragma unroll
            for (int it = 0; it < 32; ++it) {
              *reinterpret_cast<bf16x4 *>(q) = row_out(it);
              q += 2 * hd;
            }
          } else {
            for (int it = 0; it < 32; ++it) {
              const int m = row0 + 2 * it;
              if (m < M) {
                const int b2 = m / sq, t2 = m - b2 * sq;
                *reinterpret_cast<bf16x4 *>(qk_base + ((int64_t)b2 * ep.heads * sq + t2) * hd) = row_out(it);
              }
            }
          }
        } else if (row0 - g + 64 <= M) {
#pragma unroll
          for (int it = 0; it < 32; ++it) {
            *reinterpret_cast<bf16x4 *>(dst) = row_out(it);
            dst += step;
          }
        } else {
#pragma unroll
          for (int it = 0; it < 32; ++it) {
            if (row0 + 2 * it < M) *reinterpret_cast<bf16x4 *>(dst) = row_out(it);
            dst += step;
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); // reads done before the next half's writes
    }
    return;
  }
  // The other epilogues: the 256×256 tile in two halves of 128 rows held as
  // fp32: the waves that own a half write their accumulators, then every
  // wave streams whole rows out, so that each store instruction writes 512
  // contiguous bytes. Bias, Q scale, residual, mask and dropout are applied
  // in fp32 on the way out and rounded once.
  float *cs = reinterpret_cast<float *>(smem); // 128 KiB: 128 × 256 fp32 (or 256 × 128)
  const bf16 *bias = reinterpret_cast<const bf16 *>(ep.bias);
  // The bias (and for EPI_RESID the residual rows of both halves) is loaded
  // once, before the staging: its latency overlaps the staging of the first
  // half, and the second half waits for no load issued after the first
  // half's stores (memory operations complete in order).
  // (kept as loaded, converted where used, so that nothing waits for them here)
  const int n4 = tn * TN + lane * 4; // SWAP: this lane's 4 output columns
  bf16x4 bv = {};
  bf16x4 rv[2][32];
  if constexpr (SWAP && EPI != EPI_RESID_DROP) {
    if (n4 < N) bv = *reinterpret_cast<const bf16x4 *>(bias + n4);
  }
  // (EPI_MASK reads its mask the same way, from ep.resid)
  if constexpr (EPI == EPI_RESID || EPI == EPI_MASK) {
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int rr = 0; rr < 32; ++rr) {
        const int m = tm * TM + half * 128 + wave * 32 + rr;
        rv[half][rr] = bf16x4{};
        if (m < M && n4 < N)
          rv[half][rr] = *reinterpret_cast<const bf16x4 *>(reinterpret_cast<const bf16 *>(ep.resid) +
                                                          (int64_t)m * ep.ld_resid + n4);
      }
  }
  // EPI_RESID_DROP: a lane takes 16 consecutive columns (one mask block of the
  // dropout generator); their bias
  const int n16 = tn * TN + (lane & 15) * 16;
  bf16x8 bd[2] = {};
  if constexpr (EPI == EPI_RESID_DROP) {
    if (n16 < N) {
      bd[0] = *reinterpret_cast<const bf16x8 *>(bias + n16);
      bd[1] = *reinterpret_cast<const bf16x8 *>(bias + n16 + 8);
    }
  }
  // EPI_VT: the biases of this wave's 64 columns through scalar loads (the
  // address is wave-uniform): dword cc holds columns 2cc and 2cc + 1
  uint32_t bcol[32];
  if constexpr (EPI == EPI_VT) {
    if (tn * TN + wave * 64 < N) {
      const_u32p bp = (const_u32p)(uintptr_t)(bias + tn * TN + wave * 64);
#pragma unroll
      for (int cc = 0; cc < 32; ++cc) bcol[cc] = bp[cc];
    }
  }
  __syncthreads();
  // (the dropout epilogue is too large to write out twice)
  constexpr int HALF_UNROLL = EPI == EPI_RESID_DROP ? 1 : 2;
#pragma unroll HALF_UNROLL
  for (int half = 0; half < 2; ++half) {
    if constexpr (SWAP) {
      const int n = n4;
      // EPI_RESID_DROP: rows wave*32 + 4·pass + lane/16 of the half; the
      // residual is loaded in one batch per half
      bf16x8 rvd[8][2];
      if constexpr (EPI == EPI_RESID_DROP) {
#pragma unroll
        for (int pass = 0; pass < 8; ++pass) {
          const int m = tm * TM + half * 128 + wave * 32 + pass * 4 + (lane >> 4);
          rvd[pass][0] = rvd[pass][1] = bf16x8{};
          if (m < M && n16 < N) {
            const bf16 *src = reinterpret_cast<const bf16 *>(ep.resid) + (int64_t)m * ep.ld_resid + n16;
            rvd[pass][0] = *reinterpret_cast<const bf16x8 *>(src);
            rvd[pass][1] = *reinterpret_cast<const bf16x8 *>(src + 8);
          }
        }
      }
      // rows-major half tile: cs[r][c], r < 128, c < 256; 16-byte chunk
      // index (c/4) XORed with (r & 15) so 16 consecutive rows spread over
      // 16 bank groups
      if (wm == half) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = i * 32 + l32;
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const int c4 = (wn * 128 + j * 32 + r4 * 8 + g * 4) >> 2;
              f32x4 v = {acc[i][j][r4 * 4 + 0], acc[i][j][r4 * 4 + 1], acc[i][j][r4 * 4 + 2],
                         acc[i][j][r4 * 4 + 3]};
              *reinterpret_cast<f32x4 *>(cs + r * 256 + ((c4 ^ (r & 15)) << 2)) = v;
            }
        }
      }
      __syncthreads();
      if constexpr (EPI == EPI_RESID_DROP) {
        // out = resid + dropout(acc + bias): the keep flags of the lane's 16
        // columns in a row are one draw of the generator
        if (n16 < N) {
          float b16[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) b16[e] = bf2f(bd[e >> 3][e & 7]);
          const int c4_0 = (lane & 15) * 4; // the lane's first 16-byte chunk of a staged row
#pragma unroll
          for (int pass = 0; pass < 8; ++pass) {
            const int r = wave * 32 + pass * 4 + (lane >> 4);
            const int m = tm * TM + half * 128 + r;
            if (m < M) {
              float v[16];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const f32x4 x4 = *reinterpret_cast<const f32x4 *>(cs + r * 256 + (((c4_0 + q) ^ (r & 15)) << 2));
#pragma unroll
                for (int e = 0; e < 4; ++e) v[q * 4 + e] = x4[e];
              }
              const uint32_t keep = dev::dropout_keep16(ep.drop_seed, ep.drop_site,
                                                        (uint64_t)(ep.row0 + m), (uint64_t)(n16 >> 4),
                                                        ep.drop_threshold);
              bf16x8 o0, o1;
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                float o = v[i] + b16[i];
                o = ((keep >> i) & 1u) ? o * ep.drop_scale : 0.f;
                o += bf2f(rvd[pass][i >> 3][i & 7]);
                if (i < 8)
                  o0[i] = (bf16)o;
                else
                  o1[i - 8] = (bf16)o;
              }
              bf16 *dst = reinterpret_cast<bf16 *>(ep.out) + (int64_t)m * ep.ld_out + n16;
              *reinterpret_cast<bf16x8 *>(dst) = o0;
              *reinterpret_cast<bf16x8 *>(dst + 8) = o1;
            }
          }
        }
      } else if (n < N) {
        float b4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) b4[e] = bf2f(bv[e]);
        // scatter target of this lane's columns (EPI_QK): one head of Q or K.
        // The row's (batch, token) pair advances with the row instead of a
        // division per row: the wave's rows are consecutive and uniform.
        bf16 *qk_base = nullptr;
        float qs = 1.f; // Q columns: scaled for the attention's exp2
        int bi = 0, t = 0;
        if constexpr (EPI == EPI_QK) {
          const int h = (int)ep.hidden, dlog = __builtin_ctz((unsigned)ep.head_dim);
          const int which = n >= h, rem = n - which * h;
          if (which == 0) qs = ep.q_scale;
          const int head = rem >> dlog, d = rem & ((1 << dlog) - 1);
          qk_base = reinterpret_cast<bf16 *>(which == 0 ? ep.q : ep.k) +
                    (int64_t)head * ep.seq * ep.head_dim + d;
          const int m0 = tm * TM + half * 128 + wave * 32;
          bi = m0 / (int)ep.seq;
          t = m0 - bi * (int)ep.seq;
        }
        // one output row of this wave (rr-th); for EPI_QK, qk_off is the row's
        // element offset (token t of batch bi) inside one head's [s, d] block
        auto emit_row = [&](int rr, int64_t qk_off) __attribute__((always_inline)) {
          const int r = wave * 32 + rr;
          const int m = tm * TM + half * 128 + r;
          const f32x4 v = *reinterpret_cast<const f32x4 *>(cs + r * 256 + ((lane ^ (r & 15)) << 2));
          float o4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = v[e] + b4[e];
          if constexpr (EPI == EPI_QK) {
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] *= qs;
          }
          if constexpr (EPI == EPI_ACC32) {
            // fp32 output, added to what it holds when ep.accumulate
            float *fd = reinterpret_cast<float *>(ep.out) + (int64_t)blockIdx.y * ep.split_stride +
                        (int64_t)m * ep.ld_out + n;
            f32x4 r = {o4[0], o4[1], o4[2], o4[3]};
            if (ep.accumulate) r += *reinterpret_cast<const f32x4 *>(fd);
            *reinterpret_cast<f32x4 *>(fd) = r;
            return;
          }
          bf16 *dst;
          if constexpr (EPI == EPI_QK) {
            dst = qk_base + qk_off;
          } else {
            dst = reinterpret_cast<bf16 *>(ep.out) + (int64_t)m * ep.ld_out + n;
            if constexpr (EPI == EPI_RESID) {
#pragma unroll
              for (int e = 0; e < 4; ++e) o4[e] += bf2f(rv[half][rr][e]);
            } else if constexpr (EPI == EPI_RELU) {
#pragma unroll
              for (int e = 0; e < 4; ++e) o4[e] = fmaxf(o4[e], 0.f);
            } else if constexpr (EPI == EPI_MASK) {
#pragma unroll
              for (int e = 0; e < 4; ++e) o4[e] = bf2f(rv[half][rr][e]) > 0.f ? o4[e] : 0.f;
            }
          }
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = (bf16)o4[e];
          *reinterpret_cast<bf16x4 *>(dst) = ov;
        };
        // advance (token, offset) to the next row with selects, no branch: d
        // elements within a batch, the jump to the next batch's token 0 at
        // the wrap
        int64_t qk_off = 0, qk_jump = 0;
        if constexpr (EPI == EPI_QK) {
          qk_off = ((int64_t)bi * ep.heads * ep.seq + t) * ep.head_dim;
          qk_jump = ((int64_t)(ep.heads - 1) * ep.seq + 1) * ep.head_dim;
        }
        auto next_row = [&]() __attribute__((always_inline)) {
          if constexpr (EPI == EPI_QK) {
            const int t1 = t + 1, wrap = t1 == (int)ep.seq;
            t = wrap ? 0 : t1;
            qk_off += wrap ? qk_jump : (int64_t)ep.head_dim;
          }
        };
        if (tm * TM + half * 128 + 128 <= M) {
          // the whole half lies inside M: no row checks, so the LDS reads of
          // all rows can be issued together
#pragma unroll
          for (int rr = 0; rr < 32; ++rr) {
            emit_row(rr, qk_off);
            next_row();
          }
        } else {
          for (int rr = 0; rr < 32; ++rr) {
            if (tm * TM + half * 128 + wave * 32 + rr < M) emit_row(rr, qk_off);
            next_row();
          }
        }
      }
    } else {
      // EPI_VT: columns-major half tile: cs[c][r], c < 256, r < 128; chunk
      // index (r/4) XORed with (c & 15)
      static_assert(EPI == EPI_VT, "the non-swapped orientation serves the V^T scatter");
      if (wm == half) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = wn * 128 + j * 32 + l32;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const int q4 = (i * 32 + r4 * 8 + g * 4) >> 2;
              f32x4 v = {acc[i][j][r4 * 4 + 0], acc[i][j][r4 * 4 + 1], acc[i][j][r4 * 4 + 2],
                         acc[i][j][r4 * 4 + 3]};
              *reinterpret_cast<f32x4 *>(cs + c * 128 + ((q4 ^ (c & 15)) << 2)) = v;
            }
        }
      }
      __syncthreads();
      // each wave: 64 columns (V^T rows), two per instruction: lanes 0-31 the
      // even column, 32-63 the odd one, 4 consecutive tokens per lane
      const int s = (int)ep.seq, D = (int)ep.head_dim, dlog = __builtin_ctz((unsigned)D);
      const int q4 = lane & 31;
      const int m = tm * TM + half * 128 + q4 * 4;
      // N is a multiple of 64, so this wave's 64 columns are all valid or
      // all past N: one uniform check, none per column
      if (m < M && tn * TN + wave * 64 < N) {
        const int bi = m / s, t = m - bi * s;
#pragma unroll
        for (int cc = 0; cc < 32; ++cc) {
          const int c = wave * 64 + cc * 2 + g;
          const int n = tn * TN + c;
          const f32x4 v = *reinterpret_cast<const f32x4 *>(cs + c * 128 + ((q4 ^ (c & 15)) << 2));
          const float bn = __uint_as_float(g ? bcol[cc] & 0xFFFF0000u : bcol[cc] << 16);
          const int head = n >> dlog, d = n & (D - 1);
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = (bf16)(v[e] + bn);
          bf16 *dst = reinterpret_cast<bf16 *>(ep.v) + (((int64_t)bi * ep.heads + head) * D + d) * s +
                      vt_perm(t);
          *reinterpret_cast<bf16x4 *>(dst) = ov;
        }
      }
    }
    __syncthreads();
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
  case EPI_MASK:
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI_MASK, true>), grid, block, 0, stream, a, lda, b, ldb,
                       (int)M, (int)N, (int)K, ep);
    break;
  case EPI_ACC32:
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI_ACC32, true>), grid, block, 0, stream, a, lda, b, ldb,
                       (int)M, (int)N, (int)K, ep);
    break;
  case EPI_RESID_DROP:
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI_RESID_DROP, true>), grid, block, 0, stream, a, lda, b,
                       ldb, (int)M, (int)N, (int)K, ep);
    break;
  default:
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_acc32_split(const void *A, int64_t lda, const void *Bt, int64_t ldb, int64_t M,
                                   int64_t N, int64_t K, int splits, float *part, float *out,
                                   int accumulate, const void *zero_bias, hipStream_t stream) {
  GemmEpilogue ep;
  ep.bias = zero_bias;
  if (splits <= 1) {
    ep.out = out;
    ep.ld_out = N;
    ep.accumulate = accumulate;
    return launch_gemm_bf16(EPI_ACC32, A, lda, Bt, ldb, M, N, K, ep, stream);
  }
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  if (K % ((int64_t)TK * splits) != 0 || N % 64 != 0 || splits > 65535) return hipErrorInvalidValue;
  const int64_t tiles = ((M + TM - 1) / TM) * ((N + TN - 1) / TN);
  if (tiles > INT32_MAX || M > INT32_MAX || N > INT32_MAX) return hipErrorInvalidValue;
  ep.out = part;
  ep.ld_out = N;
  ep.split_stride = M * N;
  dim3 grid((unsigned)tiles, (unsigned)splits), block(NT);
  hipLaunchKernelGGL((gemm_bf16_kernel<EPI_ACC32, true>), grid, block, 0, stream,
                     reinterpret_cast<const bf16 *>(A), lda, reinterpret_cast<const bf16 *>(Bt), ldb,
                     (int)M, (int)N, (int)(K / splits), ep);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_sum_parts(part, splits, M * N, out, accumulate, stream);
}

hipError_t launch_gemm_acc32_tok(const void *A, int64_t lda, const void *Bt, int64_t ldb, int64_t M,
                                 int64_t N, int64_t K, int splits, float *part, float *out,
                                 int accumulate, const void *zero_bias, hipStream_t stream) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  const int64_t Kp = (K + TK - 1) / TK * TK;
  if (splits < 1 || Kp % ((int64_t)TK * splits) != 0 || N % 64 != 0 || lda % 8 != 0 || ldb % 8 != 0 ||
      lda < M || ldb < N || splits > 65535)
    return hipErrorInvalidValue;
  const int64_t tiles = ((M + TM - 1) / TM) * ((N + TN - 1) / TN), Kc = Kp / splits;
  if (tiles > INT32_MAX || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX ||
      Kc * (lda > ldb ? lda : ldb) * 2 > (int64_t)UINT32_MAX)
    return hipErrorInvalidValue;
  GemmEpilogue ep;
  ep.bias = zero_bias;
  ep.mn_rows = K;
  ep.ld_out = N;
  if (splits == 1) {
    ep.out = out;
    ep.accumulate = accumulate;
  } else {
    ep.out = part;
    ep.split_stride = M * N;
  }
  dim3 grid((unsigned)tiles, (unsigned)splits), block(NT);
  hipLaunchKernelGGL((gemm_bf16_kernel<EPI_ACC32, true, true>), grid, block, 0, stream,
                     reinterpret_cast<const bf16 *>(A), lda, reinterpret_cast<const bf16 *>(Bt), ldb,
                     (int)M, (int)N, (int)Kc, ep);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return launch_sum_parts(part, splits, M * N, out, accumulate, stream);
}

} // namespace bpt
