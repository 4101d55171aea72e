// Backward pass of the blockwise attention on CDNA4 matrix cores, and the
// small data-movement kernels the layer backward needs.
//
// The BPT review (section 三, memory of the blockwise layer, and its remark
// that the method composes with rematerialisation) trains the layer by
// recomputing each block in the backward pass instead of storing it; here the
// forward's per-row log-sum-exp is the only statistic kept, and every score
// block is recomputed from Q and K. With Z = Q Kᵀ/√d, P = softmax_rows(Z),
// O = P V and upstream dO:
//   D = rowsum(dO ∘ O),  dP = dO Vᵀ,  dZ = P ∘ (dP − D),
//   dV = Pᵀ dO,  dK = dZᵀ Q / √d,  dQ = dZ K / √d.
// Three kernels, so that no output needs atomics: one wave per 32 keys walks
// the query blocks for dV, another for dK; one wave per 32 queries walks the
// key blocks for dQ.
//
// MFMA layouts (v_mfma_f32_32x32x16_bf16, D[i][j] += Σ_k A[i][k] B[k][j];
// lane (l32, g) feeds A[l32][8g..8g+7] and B[8g..8g+7][l32] and holds
// D[8r4 + 4g + e][l32] in element 4·r4 + e):
//   * a score block D[q][key] (or D[key][q]) comes out with the key (query)
//     on the lane, so its 16 values per lane are the next product's A operand
//     rows without moving: element rows 2c and 2c+1 (8 values) form the
//     k-slots of the c-th 16-wide product, in the order q = 16c + {4g..4g+3,
//     8+4g..8+4g+3};
//   * the matching B operands (the same 8 tokens, for one column) are read
//     straight out of the token-major row blocks in LDS with CDNA4's
//     transposing LDS read (ds_read_b64_tr_b16), so no transposed copy of
//     Q, K or dO is made.
// Q arrives multiplied by log2(e)/√d (the forward's scaling), so scores are in
// log2 units and P = exp2(score − lse).
#include "bpt_internal.h"
#include "lds_dma.h"

namespace bpt {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two weights rounded to one packed bf16 dword, held at this point of the
// issue order: the empty asm consumes the dword here, so that the
// exponentials and the conversion stay in the issue slot that computes them
// (the next step's MFMAs are their only users, and without this the compiler
// moves them behind the step's barrier, where they run back to back instead
// of beside the MFMAs).
__device__ __forceinline__ bf16x2 pack_here(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  asm volatile("" : "+v"(v));
  return v;
}
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned long long u64x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994531f;

// position of token t inside its 16-group in the key-permuted layout (and
// back: the map is its own inverse)
__device__ __forceinline__ int vt_perm(int t) {
  return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---- operand staging in LDS. A workgroup's 4 waves share each block's
// operands: row-major [32 rows][D] blocks (rows of 2D bytes, 16-byte chunk c
// of row r at c ^ rsw(r)), and (dV) transposed [D][32 positions] blocks (rows
// of 64 bytes, chunk c of row r at c ^ ((r >> 2) & 3)). Loads go memory ->
// LDS (buffer_load_dwordx4 ... lds), 1 KiB per wave instruction, lane L
// writing bytes 16L.. of it; the swizzle is applied by choosing the source
// chunk.
// rsw spreads both kinds of read of a row block over the 64 banks (256 bytes
// of LDS per cycle):
//  * a fragment read (16 bytes per lane, 16 lanes per cycle) takes one chunk
//    of 16 consecutive rows, so rsw is a bijection on the chunk slots of each
//    aligned 16 rows;
//  * a transposing read (8 bytes per lane, 32 lanes per cycle) takes 4
//    consecutive rows (aligned to 4) × 4 chunks, so the 4 rows' values of
//    rsw >> 2 (at D = 64: of the rows sharing a 256-byte line) differ.
// With q the row's 256-byte line (r / (128 / D)), rsw = q ^ (q << 2) in
// D / 8 chunk slots does both (q alone, the plain line index, put all 16
// chunks of a transposing read on 4 slots at D = 128).
template <int D> __device__ __forceinline__ int rsw(int r) {
  const int q = r / (128 / D);
  return (q ^ (q << 2)) & (D / 8 - 1);
}

// 1 KiB piece pc of a row-major [32][D] block whose first row is at byte
// offset g0 (row stride 2D bytes) of the descriptor's buffer
template <int D>
__device__ __forceinline__ void load_rows(const dev::i32x4 &rsrc, uint32_t g0, int pc, bf16 *lds, int lane) {
  constexpr int RPK = 512 / D; // rows per KiB
  const int r = pc * RPK + lane / (D / 8), c = lane % (D / 8);
  // the row's 256-byte line is q = 4·pc + lane / 16 (a bit-or), so c ^ rsw(r)
  // is a per-lane value XOR a constant of the piece
  const int L = lane >> 4;
  const int cx = (c ^ ((L ^ (L << 2)) & (D / 8 - 1))) ^ (((4 * pc) ^ (16 * pc)) & (D / 8 - 1));
  const uint32_t off = g0 + (uint32_t)(r * D + (cx << 3)) * 2u;
  dev::load_lds16(rsrc, off, lds + pc * 512);
}
// 1 KiB piece pc (16 rows) of a transposed [D][32] block: row d at byte
// offset g0 + d·rowb of the descriptor's buffer
__device__ __forceinline__ void load_cols(const dev::i32x4 &rsrc, uint32_t g0, uint32_t rowb, int pc, bf16 *lds,
                                          int lane) {
  const int d = pc * 16 + (lane >> 2), c = lane & 3;
  const uint32_t off = g0 + (uint32_t)d * rowb + (uint32_t)((c ^ ((d >> 2) & 3)) << 4);
  dev::load_lds16(rsrc, off, lds + pc * 512);
}
// A-operand fragment: row `row`, 16-byte chunk `chunk` of a row block
template <int D> __device__ __forceinline__ bf16x8 frag_rows(const bf16 *blk, int row, int chunk) {
  return *reinterpret_cast<const bf16x8 *>(blk + row * D + ((chunk ^ rsw<D>(row)) << 3));
}

// B-operand fragment from a transposed [D][32] block: row d, chunk `chunk`
__device__ __forceinline__ bf16x8 frag_cols(const bf16 *blk, int d, int chunk) {
  return *reinterpret_cast<const bf16x8 *>(blk + d * 32 + ((chunk ^ ((d >> 2) & 3)) << 3));
}


typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// B-operand fragment of a product whose B matrix is a row block (32 tokens ×
// D, rows = the product's k): k-slots 16c + 4g + {0..3} then 16c + 8 + 4g +
// {0..3} (the order of an A fragment packed from a score block), column
// nb·32 + l32. Two transposing LDS reads (ds_read_b64_tr_b16): within each
// 16-lane group, lane j addresses row kb + j/4, columns n0 + 4·(j % 4) .. +3
// (8 bytes inside one 16-byte chunk, so the row swizzle applies per lane),
// and lane i receives rows kb .. kb+3 of column n0 + i.
// The row-block layout packs row, 16-byte chunk and byte into disjoint bit
// fields, and rsw(r + 8) = rsw(r) ^ D/16, rsw(r + 16) = rsw(r) for the rows
// 0..7 a lane starts from, so every read's byte offset is the lane's offset
// for (nb 0, c 0, first half), tr_off0, XOR an immediate (column block nb:
// chunk bits nb << 2; second half: row bit 3 and chunk bit D/16), plus 32·D
// bytes per k-chunk c: one address add per read pair (tests/test_lds_layout.py
// checks the identity for every lane and case at D = 32, 64, 128).
template <int D> __device__ __forceinline__ uint32_t tr_off0(int lane) {
  const int j = lane & 15, g = lane >> 5;
  const int col = 16 * ((lane >> 4) & 1) + 4 * (j & 3), r = 4 * g + (j >> 2);
  return (uint32_t)(r * D + (((col >> 3) ^ rsw<D>(r)) << 3) + (col & 7)) * 2u;
}
typedef __attribute__((address_space(3))) char lds_char;
template <int D>
__device__ __forceinline__ bf16x8 frag_rows_tr(const bf16 *blk, int nb, int c, uint32_t o0) {
  const lds_char *b = (const lds_char *)blk + c * 32 * D;
  const uint32_t o1 = o0 ^ (uint32_t)(nb << 6);
  const uint32_t o2 = o1 ^ (uint32_t)(((D / 16) << 4) | 16 * D);
  const bf16x4 x = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(b + o1)));
  const bf16x4 y = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(b + o2)));
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = x[e];
    f[4 + e] = y[e];
  }
  return f;
}

// s_waitcnt vmcnt(n) (at most 63) lgkmcnt(0), then s_barrier
template <int N> __device__ __forceinline__ void barrier_vm() {
  static_assert(N < 64, "vmcnt holds 6 bits");
  dev::barrier_vm<N>();
}

// LDS stages: during step t the blocks t (score side) and t-1 (gradient side)
// are read while the next two blocks load.
constexpr int BW_NST = 4;
// a ring slot known at compile time: its LDS base then goes into the
// immediate offset of every fragment read instead of a per-read address add
template <int N> struct Slot {
  static constexpr int v = N;
};

// ---- dV (DK = false) or dK (DK = true): wave w of block (bh, y) owns keys
// k0 = 128y + 32w .. k0+31; the 4 waves walk the same query blocks of 32
// (from the workgroup's first key when causal), staged in LDS: Qs rows and
// dOT columns (dV) or Qs and dO rows (dK), and the block's 32 log-sum-exps
// (and D values), one word per lane of a 64-lane load, lanes 32..63 and rows
// past s reading zero. dV's B operand comes from the dOT columns (one 16-byte
// read per fragment: its product is short, and two transposing reads per
// fragment cost it more than the transposed copy), dK's is Qs read transposed. dV needs P = exp2(score − lse) only;
// dK needs dZ = P ∘ (dP − D) too. Splitting the two recomputes the score
// product once more (dV: 2 products per block, dK: 3) and lets each kernel
// keep its accumulators, its two blocks of scores and its MFMA operands in
// registers.
// Software pipeline, one MFMA per issue slot: step t issues the score (and
// dP) products of block t, then block t-1's gradient products beside the
// exponentials of block t (whose A fragments the next step uses); LDS
// fragments are read LA slots ahead. One block of scores and two of A
// fragments are live, little enough for two waves per SIMD.
// Qs, K, V, dO: [b·nh, s, D] (Qs pre-scaled); dOT: [b·nh, D, sp] key-permuted
// and zero beyond s; nlse, nDq: [b·nh, s], -lse and -D. Writes dK (×ln 2, see the
// header) into columns h + head·D, or dV into columns 2h + head·D, of dQKV
// [b, s, 3h].
template <int D, bool DK>
__global__ __launch_bounds__(256) void attn_bwd_dkv_kernel(
    const bf16 *__restrict__ Qs, const bf16 *__restrict__ K, const bf16 *__restrict__ V,
    const bf16 *__restrict__ dO, const bf16 *__restrict__ dOT, const float *__restrict__ nlse,
    const float *__restrict__ nDq, bf16 *__restrict__ dQKV, int s, int sp, int heads, int causal) {
  constexpr int KK = D / 16, NB = D / 32;
  constexpr int BLK = 32 * D;                 // bf16 elements of one operand block
  constexpr int NOP = 2;                      // operand blocks: Qs rows, then dOT (dV) or dO rows (dK)
  constexpr int STG = NOP * BLK + 256;        // operand blocks, then lse and D (64 floats each)
  constexpr int NPC = D / 16;                 // KiB pieces per operand block
  constexpr int NLO = (NOP * NPC + 3) / 4;    // operand loads per wave per block
  constexpr int NL = NLO + 1;                 // + lse or D
  constexpr int NS = (DK ? 2 : 1) * KK;       // score-side MFMAs per block
  constexpr int NG = 2 * NB;                  // gradient-side MFMAs per block
  // fragment reads in flight ahead of their MFMA: 4 at d = 128 (0.3% on the
  // backward over 3, no extra registers for dK); 3 below, where a fourth would
  // cost the d = 64 dV kernel a wave per SIMD
  constexpr int LA = D == 128 ? 4 : 3;
  constexpr int NST = BW_NST, AHEAD = NST - 2; // LDS stages, blocks loading during a step
  __shared__ __attribute__((aligned(1024))) bf16 smem[NST * STG];

  const int bh = blockIdx.x, bi = bh / heads, head = bh - bi * heads;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  __builtin_assume(wave >= 0 && wave < 4); // 256 threads: the staging's piece choice folds
  const int l32 = lane & 31, g = lane >> 5;
  const int K0 = (int)blockIdx.y * 128, k0 = K0 + wave * 32;
  const int64_t hs = (int64_t)bh * s;
  const bf16 *Kh = K + hs * D, *Vh = V + hs * D;
  const dev::i32x4 qr = dev::make_rsrc(Qs + hs * D, (uint32_t)(s * D * 2));
  const dev::i32x4 orr = dev::make_rsrc(dO + hs * D, (uint32_t)(s * D * 2));
  const dev::i32x4 ot = dev::make_rsrc(dOT + (int64_t)bh * D * sp, (uint32_t)(D * sp * 2));
  // dK: waves 0 and 2 stage the log-sum-exps, waves 1 and 3 the D values;
  // dV: every wave stages the log-sum-exps (the same words to the same
  // place, so that every wave issues NL loads)
  const bool st_d = DK && (wave & 1);
  const dev::i32x4 st = dev::make_rsrc(st_d ? nDq + hs : nlse + hs, (uint32_t)(s * 4));
  const uint32_t st_lane = lane < 32 ? (uint32_t)lane * 4u : 0x80000000u;

  const int qfirst = causal ? K0 : 0;
  const int nblk = (s - qfirst + 31) / 32; // query blocks the workgroup walks (>= 1)
  // load i (0..NOP·NPC-1) of query block j goes to wave i % 4; waves with
  // fewer re-issue one of their pieces
  auto stage = [&](int j) __attribute__((always_inline)) {
    const int q0 = qfirst + j * 32;
    bf16 *S = smem + (j % NST) * STG;
    // (the per-lane parts of the offsets are the same at every call, and the
    // compiler holds them across the loop)
    int ln = lane;
#pragma unroll
    for (int t = 0; t < NLO; ++t) {
      int i = t * 4 + wave;
      if (i >= NOP * NPC) i = wave % (NOP * NPC);
      const int o = i / NPC, pc = i % NPC;
      if (o == 0)
        load_rows<D>(qr, (uint32_t)(q0 * D * 2), pc, S, ln);
      else if (DK)
        load_rows<D>(orr, (uint32_t)(q0 * D * 2), pc, S + BLK, ln);
      else
        load_cols(ot, (uint32_t)(q0 * 2), (uint32_t)(sp * 2), pc, S + BLK, ln);
    }
    dev::load_lds4(st, st_lane | (uint32_t)(q0 * 4), S + NOP * BLK + (st_d ? 128 : 0));
  };

  const int key = k0 + l32;
  const int krow = min(key, s - 1);
  bf16x8 kf[KK], vf[DK ? KK : 1];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    kf[kk] = *reinterpret_cast<const bf16x8 *>(Kh + (int64_t)krow * D + kk * 16 + g * 8);
    if (DK) vf[kk] = *reinterpret_cast<const bf16x8 *>(Vh + (int64_t)krow * D + kk * 16 + g * 8);
  }
  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[nb][r] = 0.f;
  // the fragments have arrived before any load into LDS is issued, so that no
  // wait for them inside the loop is ordered behind those loads
  dev::wait_vm<0>();
  // K and V fragments are only ever MFMA B operands: keep them in AGPRs
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    asm volatile("" : "+a"(kf[kk]));
    if (DK) asm volatile("" : "+a"(vf[kk]));
  }

  // Every wave walks every block of the workgroup: blocks before the wave's
  // first key (causal) and keys past s come out fully masked (P = dZ = 0),
  // which costs at most 3 blocks per wave and keeps the loop free of
  // per-wave branches.
  // score / dP element 4·r4 + e: query q0 + 8r4 + 4g + e, key k0 + l32
  // block j sits in ring slot j % NST; the step functions take the slot as
  // a compile-time tag (the loop below is unrolled NST times)
  static_assert(NST == 4, "the main loop is unrolled over the 4 ring slots");
  auto block = [&](auto sl) __attribute__((always_inline)) { return smem + decltype(sl)::v * STG; };
  // the products of block j start from -lse (and -D), loaded as stored; a
  // score above the causal diagonal or past s starts from -inf instead, so
  // that its P is 0
  auto init = [&](int j, auto sl, f32x16 &sc, f32x16 &dp) __attribute__((always_inline)) {
    const int q0 = qfirst + j * 32;
    const float *Sst = reinterpret_cast<const float *>(block(sl) + NOP * BLK);
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 L4 = *reinterpret_cast<const f32x4 *>(Sst + 8 * r4 + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[4 * r4 + e] = L4[e];
      if (DK) {
        const f32x4 D4 = *reinterpret_cast<const f32x4 *>(Sst + 64 + 8 * r4 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[4 * r4 + e] = D4[e];
      }
    }
    if ((causal && q0 < k0 + 31) || q0 + 31 >= s || k0 + 31 >= s) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = q0 + 8 * (r >> 2) + 4 * g + (r & 3);
        const bool ok = q < s && key < s && (!causal || key <= q);
        sc[r] = ok ? sc[r] : -INFINITY;
      }
    }
  };
  // score-side fragment r: Qs row chunk (dV: chunk r; dK: even r, chunk r/2)
  // or dO row chunk (dK: odd r)
  auto sfrag = [&](const bf16 *S, int r) __attribute__((always_inline)) {
    if (DK) return frag_rows<D>(S + (r & 1) * BLK, l32, 2 * (r >> 1) + g);
    return frag_rows<D>(S, l32, 2 * r + g);
  };
  auto score_mfma = [&](int r, const bf16x8 &fr, f32x16 &sc, f32x16 &dp) __attribute__((always_inline)) {
    if (DK) {
      if (r & 1)
        dp = mfma(fr, vf[r >> 1], dp);
      else
        sc = mfma(fr, kf[r >> 1], sc);
    } else {
      sc = mfma(fr, kf[r], sc);
    }
  };
  // gradient-side fragment i = c·NB + nb: columns nb·32.., k-chunk c, from
  // the dOT block (dV) or Qs read transposed (dK)
  const uint32_t toff = tr_off0<D>(lane);
  auto gfrag = [&](const bf16 *S, int i) __attribute__((always_inline)) {
    if (DK) return frag_rows_tr<D>(S, i % NB, i / NB, toff);
    return frag_cols(S + BLK, (i % NB) * 32 + l32, 2 * (i / NB) + g);
  };
  // unit u (0..7): elements 2u, 2u+1 -> the A fragment (P for dV, dZ for dK)
  auto unit = [&](const f32x16 &sc, const f32x16 &dp, bf16x8 (&fa)[2], int u) __attribute__((always_inline)) {
    const float p0 = __builtin_amdgcn_exp2f(sc[2 * u]), p1 = __builtin_amdgcn_exp2f(sc[2 * u + 1]);
    const int c = u >> 2, k = (u & 3) * 2;
    const bf16x2 v = DK ? pack_here(p0 * dp[2 * u], p1 * dp[2 * u + 1]) : pack_here(p0, p1);
    fa[c][k] = v[0];
    fa[c][k + 1] = v[1];
  };
  auto score_only = [&](int j, auto sl, f32x16 &sc, f32x16 &dp) __attribute__((always_inline)) {
    const bf16 *S = block(sl);
    init(j, sl, sc, dp);
#pragma unroll
    for (int r = 0; r < NS; ++r) score_mfma(r, sfrag(S, r), sc, dp);
  };
  auto grad_only = [&](auto sl, const bf16x8 (&fa)[2]) __attribute__((always_inline)) {
    const bf16 *S = block(sl);
#pragma unroll
    for (int i = 0; i < NG; ++i) acc[i % NB] = mfma(fa[i / NB], gfrag(S, i), acc[i % NB]);
  };
  // step j (in slot sl): the score products of block j into (sc, dp), then
  // block j-1's gradient products from fa_o beside the exponentials of block j
  // into fa_n
  auto step_bulk = [&](int j, auto sl, const bf16x8 (&fa_o)[2], bf16x8 (&fa_n)[2], f32x16 &sc, f32x16 &dp)
      __attribute__((always_inline)) {
    const bf16 *Sn = block(sl), *So = block(Slot<(decltype(sl)::v + NST - 1) % NST>{});
    auto frag = [&](int r) __attribute__((always_inline)) { return r < NS ? sfrag(Sn, r) : gfrag(So, r - NS); };
    bf16x8 ring[LA + 1];
#pragma unroll
    for (int r = 0; r < LA; ++r) ring[r] = frag(r);
    init(j, sl, sc, dp);
    auto slot = [&](int r) __attribute__((always_inline)) {
      const bf16x8 fr = ring[r % (LA + 1)];
      if (r < NS) {
        score_mfma(r, fr, sc, dp);
      } else {
        const int i = r - NS;
        acc[i % NB] = mfma(fa_o[i / NB], fr, acc[i % NB]);
      }
      if (r + LA < NS + NG) ring[(r + LA) % (LA + 1)] = frag(r + LA);
      if (r >= NS) {
#pragma unroll
        for (int u = (r - NS) * 8 / NG; u < (r - NS + 1) * 8 / NG; ++u) unit(sc, dp, fa_n, u);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int r = 0; r < NS + NG; ++r) slot(r);
  };
  // before step t: block t has landed (blocks t+1 .. t+AHEAD-1 may still be
  // loading); block t+AHEAD goes into the buffer of block t-2, which every
  // wave finished in step t-1
  auto sync = [&](int t) __attribute__((always_inline)) {
    if (AHEAD > 1 && t + AHEAD - 1 < nblk)
      barrier_vm<(AHEAD - 1) * NL>();
    else
      barrier_vm<0>();
    if (t + AHEAD < nblk) stage(t + AHEAD);
  };

#pragma unroll
  for (int j = 0; j < AHEAD; ++j)
    if (j < nblk) stage(j);
  f32x16 sc, dp;
  bf16x8 fA[2], fB[2];
  sync(0);
  score_only(0, Slot<0>{}, sc, dp);
#pragma unroll
  for (int u = 0; u < 8; ++u) unit(sc, dp, fA, u);
  // steps 1, 2, ...: block t in slot t % 4; the A fragments alternate
  // between fA (even t) and fB (odd t)
  int t = 1;
  for (; t + 3 < nblk; t += 4) {
    sync(t);
    step_bulk(t, Slot<1>{}, fA, fB, sc, dp);
    sync(t + 1);
    step_bulk(t + 1, Slot<2>{}, fB, fA, sc, dp);
    sync(t + 2);
    step_bulk(t + 2, Slot<3>{}, fA, fB, sc, dp);
    sync(t + 3);
    step_bulk(t + 3, Slot<0>{}, fB, fA, sc, dp);
  }
  // 0 to 3 steps left (t % 4 == 1), then the last block's gradient products
  if (t < nblk) {
    sync(t);
    step_bulk(t, Slot<1>{}, fA, fB, sc, dp);
    if (t + 1 < nblk) {
      sync(t + 1);
      step_bulk(t + 1, Slot<2>{}, fB, fA, sc, dp);
      if (t + 2 < nblk) {
        sync(t + 2);
        step_bulk(t + 2, Slot<3>{}, fA, fB, sc, dp);
        grad_only(Slot<3>{}, fB);
      } else {
        grad_only(Slot<2>{}, fA);
      }
    } else {
      grad_only(Slot<1>{}, fB);
    }
  } else {
    grad_only(Slot<0>{}, fA);
  }
  dev::wait_vm<0>(); // no load into LDS outlives the kernel
  if (k0 >= s) return;
  // acc element 4·r4 + e: key k0 + 8r4 + 4g + e, head dim nb·32 + l32
  const int64_t h = (int64_t)heads * D;
  const float scale = DK ? kLn2 : 1.f;
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kr = k0 + 8 * r4 + 4 * g + e;
      if (kr < s) {
        bf16 *row = dQKV + ((int64_t)bi * s + kr) * 3 * h + (DK ? h : 2 * h) + head * D + l32;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) row[nb * 32] = (bf16)(acc[nb][r4 * 4 + e] * scale);
      }
    }
}

// 16 floats, each the low (= high) half of x, written by eight 64-bit moves
// (from plain code the compiler emits sixteen 32-bit moves, even for a
// splat of 64-bit values); no memory access
__device__ __forceinline__ f32x16 splat_pairs(unsigned long long x) {
  unsigned long long a0, a1, a2, a3, a4, a5, a6, a7;
  asm volatile("v_mov_b64 %0, %8\n\tv_mov_b64 %1, %8\n\tv_mov_b64 %2, %8\n\tv_mov_b64 %3, %8\n\t"
               "v_mov_b64 %4, %8\n\tv_mov_b64 %5, %8\n\tv_mov_b64 %6, %8\n\tv_mov_b64 %7, %8"
               : "=v"(a0), "=v"(a1), "=v"(a2), "=v"(a3), "=v"(a4), "=v"(a5), "=v"(a6), "=v"(a7)
               : "v"(x));
  return __builtin_bit_cast(f32x16, (u64x8){a0, a1, a2, a3, a4, a5, a6, a7});
}

// unit u (0..7) of a block's element-wise work in the dQ kernel: elements
// 2u and 2u+1 of the score and dP blocks, which arrive as score − lse and
// dP − D (the products start from those values; masked scores are -inf) ->
// dZ = exp2(score − lse)·(dP − D), rounded to bf16 into dword u % 4 of
// A-operand fragment u / 4 (fragment c holds element rows 2c and 2c+1, see
// the header)
__device__ __forceinline__ void z_unit(const f32x16 &sc, const f32x16 &dp, bf16x8 (&za)[2], int u) {
  const float p0 = __builtin_amdgcn_exp2f(sc[2 * u]), p1 = __builtin_amdgcn_exp2f(sc[2 * u + 1]);
  const int c = u >> 2, k = (u & 3) * 2;
  const bf16x2 v = pack_here(p0 * dp[2 * u], p1 * dp[2 * u + 1]);
  za[c][k] = v[0];
  za[c][k + 1] = v[1];
}

// ---- dQ: wave w of block (bh, y) owns queries q0 = 128y + 32w .. q0+31;
// the 4 waves walk the same key blocks of 32 (up to the workgroup's last
// query when causal), staged in LDS: K and V rows (the B operand of dQ is K
// read transposed); the same software pipeline as the dV/dK kernel (the
// score and dP^T products of block t, then block t-1's dQ products beside
// the dZ work of block t). Causal query tiles go out longest first. Writes
// dQ into columns head·D of dQKV.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(
    const bf16 *__restrict__ Qs, const bf16 *__restrict__ K, const bf16 *__restrict__ V,
    const bf16 *__restrict__ dO, const float *__restrict__ nlse, const float *__restrict__ nDq,
    bf16 *__restrict__ dQKV, int s, int heads, int causal) {
  constexpr int KK = D / 16, NB = D / 32;
  constexpr int BLK = 32 * D;
  constexpr int STG = 2 * BLK;                 // K, V rows
  constexpr int NPC = D / 16;
  constexpr int NL = (2 * NPC + 3) / 4;        // loads per wave per block
  constexpr int NS = 2 * KK, NG = 2 * NB, LA = D == 128 ? 4 : 3; // (as in the dV/dK kernel)
  constexpr int NST = BW_NST, AHEAD = NST - 2;
  __shared__ __attribute__((aligned(1024))) bf16 smem[NST * STG];

  const int bh = blockIdx.x, bi = bh / heads, head = bh - bi * heads;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  __builtin_assume(wave >= 0 && wave < 4); // 256 threads: the staging's piece choice folds
  const int l32 = lane & 31, g = lane >> 5;
  // causal: query tile y walks 4(y+1) key blocks, so the tiles go out in
  // decreasing y, longest first
  const int Q0 = (int)(causal ? gridDim.y - 1 - blockIdx.y : blockIdx.y) * 128, q0 = Q0 + wave * 32;
  const int64_t hs = (int64_t)bh * s;
  const bf16 *Qh = Qs + hs * D, *dOh = dO + hs * D;
  const dev::i32x4 kr_ = dev::make_rsrc(K + hs * D, (uint32_t)(s * D * 2));
  const dev::i32x4 vr_ = dev::make_rsrc(V + hs * D, (uint32_t)(s * D * 2));

  const int kend = causal ? (Q0 + 128 < s ? Q0 + 128 : s) : s;
  const int nblk = (kend + 31) / 32;
  // load i (0..2·NPC-1) goes to wave i % 4; waves with fewer re-issue one of
  // their pieces (the same bytes to the same place), so that every wave
  // issues NL loads per block
  auto stage = [&](int j) __attribute__((always_inline)) {
    const int k0 = j * 32;
    bf16 *S = smem + (j % NST) * STG;
    int ln = lane;
#pragma unroll
    for (int t = 0; t < NL; ++t) {
      int i = t * 4 + wave;
      if (i >= 2 * NPC) i = wave % (2 * NPC);
      const int o = i / NPC, pc = i % NPC;
      if (o == 0)
        load_rows<D>(kr_, (uint32_t)(k0 * D * 2), pc, S, ln);
      else
        load_rows<D>(vr_, (uint32_t)(k0 * D * 2), pc, S + BLK, ln);
    }
  };

  const int q = q0 + l32;
  const int qrow = min(q, s - 1);
  bf16x8 qf[KK], of[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qf[kk] = *reinterpret_cast<const bf16x8 *>(Qh + (int64_t)qrow * D + kk * 16 + g * 8);
    of[kk] = *reinterpret_cast<const bf16x8 *>(dOh + (int64_t)qrow * D + kk * 16 + g * 8);
  }
  // -lse and -D, each twice in a 64-bit pair (8 pair moves fill a product's
  // 16 start values)
  const unsigned long long nL2 = __float_as_uint(nlse[hs + qrow]) * 0x100000001ull;
  const unsigned long long nD2 = __float_as_uint(nDq[hs + qrow]) * 0x100000001ull;
  f32x16 dq[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[nb][r] = 0.f;
  dev::wait_vm<0>(); // (as in the dV/dK kernel)
  // Q and dO fragments are only ever MFMA B operands: keep them in AGPRs
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+a"(qf[kk]), "+a"(of[kk]));

  // every wave walks every key block of the workgroup; keys after the wave's
  // last query (causal) come out fully masked, at most 3 blocks per wave
  // element 4·r4 + e: key k0 + 8r4 + 4g + e, query q0 + l32
  // (ring slots as compile-time tags, as in the dV/dK kernel)
  static_assert(NST == 4, "the main loop is unrolled over the 4 ring slots");
  auto block = [&](auto sl) __attribute__((always_inline)) { return smem + decltype(sl)::v * STG; };
  // the products start from -lse and -D (one row per lane); a score above the
  // causal diagonal or past s starts from -inf
  auto init = [&](int j, f32x16 &sc, f32x16 &dp) __attribute__((always_inline)) {
    const int k0 = j * 32;
    // (written at each use: a loop-invariant 16-wide copy of each would hold
    // 32 VGPRs)
    sc = splat_pairs(nL2);
    dp = splat_pairs(nD2);
    if ((causal && k0 + 31 > q0) || k0 + 31 >= s || q0 + 31 >= s) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = k0 + 8 * (r >> 2) + 4 * g + (r & 3);
        const bool ok = kr < s && q < s && (!causal || kr <= q);
        sc[r] = ok ? sc[r] : -INFINITY;
      }
    }
  };
  // score-side fragment r (even: K row chunk, odd: V row chunk)
  auto sfrag = [&](const bf16 *S, int r) __attribute__((always_inline)) {
    return frag_rows<D>(S + (r & 1) * BLK, l32, 2 * (r >> 1) + g);
  };
  // gradient-side fragment i = c·NB + nb: columns nb·32.. of K read
  // transposed, k-chunk c
  const uint32_t toff = tr_off0<D>(lane);
  auto gfrag = [&](const bf16 *S, int i) __attribute__((always_inline)) {
    return frag_rows_tr<D>(S, i % NB, i / NB, toff);
  };
  auto score_mfma = [&](int r, const bf16x8 &fr, f32x16 &sc, f32x16 &dp) __attribute__((always_inline)) {
    if (r & 1)
      dp = mfma(fr, of[r >> 1], dp);
    else
      sc = mfma(fr, qf[r >> 1], sc);
  };
  auto score_only = [&](int j, auto sl, f32x16 &sc, f32x16 &dp) __attribute__((always_inline)) {
    const bf16 *S = block(sl);
    init(j, sc, dp);
#pragma unroll
    for (int r = 0; r < NS; ++r) score_mfma(r, sfrag(S, r), sc, dp);
  };
  auto grad_only = [&](auto sl, const bf16x8 (&za)[2]) __attribute__((always_inline)) {
    const bf16 *S = block(sl);
#pragma unroll
    for (int i = 0; i < NG; ++i) dq[i % NB] = mfma(za[i / NB], gfrag(S, i), dq[i % NB]);
  };
  // (the dK kernel's schedule)
  auto step_bulk = [&](int j, auto sl, const bf16x8 (&za_o)[2], bf16x8 (&za_n)[2], f32x16 &sc, f32x16 &dp)
      __attribute__((always_inline)) {
    const bf16 *Sn = block(sl), *So = block(Slot<(decltype(sl)::v + NST - 1) % NST>{});
    auto frag = [&](int r) __attribute__((always_inline)) { return r < NS ? sfrag(Sn, r) : gfrag(So, r - NS); };
    bf16x8 ring[LA + 1];
#pragma unroll
    for (int r = 0; r < LA; ++r) ring[r] = frag(r);
    init(j, sc, dp);
    auto slot = [&](int r) __attribute__((always_inline)) {
      const bf16x8 fr = ring[r % (LA + 1)];
      if (r < NS) {
        score_mfma(r, fr, sc, dp);
      } else {
        const int i = r - NS;
        dq[i % NB] = mfma(za_o[i / NB], fr, dq[i % NB]);
      }
      if (r + LA < NS + NG) ring[(r + LA) % (LA + 1)] = frag(r + LA);
      if (r >= NS) {
#pragma unroll
        for (int u = (r - NS) * 8 / NG; u < (r - NS + 1) * 8 / NG; ++u) z_unit(sc, dp, za_n, u);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int r = 0; r < NS + NG; ++r) slot(r);
  };
  // (as in the dV/dK kernel)
  auto sync = [&](int t) __attribute__((always_inline)) {
    if (AHEAD > 1 && t + AHEAD - 1 < nblk)
      barrier_vm<(AHEAD - 1) * NL>();
    else
      barrier_vm<0>();
    if (t + AHEAD < nblk) stage(t + AHEAD);
  };

#pragma unroll
  for (int j = 0; j < AHEAD; ++j)
    if (j < nblk) stage(j);
  f32x16 sc, dp;
  bf16x8 zA[2], zB[2];
  sync(0);
  score_only(0, Slot<0>{}, sc, dp);
#pragma unroll
  for (int u = 0; u < 8; ++u) z_unit(sc, dp, zA, u);
  // (the dV/dK kernel's loop and tail)
  int t = 1;
  for (; t + 3 < nblk; t += 4) {
    sync(t);
    step_bulk(t, Slot<1>{}, zA, zB, sc, dp);
    sync(t + 1);
    step_bulk(t + 1, Slot<2>{}, zB, zA, sc, dp);
    sync(t + 2);
    step_bulk(t + 2, Slot<3>{}, zA, zB, sc, dp);
    sync(t + 3);
    step_bulk(t + 3, Slot<0>{}, zB, zA, sc, dp);
  }
  if (t < nblk) {
    sync(t);
    step_bulk(t, Slot<1>{}, zA, zB, sc, dp);
    if (t + 1 < nblk) {
      sync(t + 1);
      step_bulk(t + 1, Slot<2>{}, zB, zA, sc, dp);
      if (t + 2 < nblk) {
        sync(t + 2);
        step_bulk(t + 2, Slot<3>{}, zA, zB, sc, dp);
        grad_only(Slot<3>{}, zB);
      } else {
        grad_only(Slot<2>{}, zA);
      }
    } else {
      grad_only(Slot<1>{}, zB);
    }
  } else {
    grad_only(Slot<0>{}, zA);
  }
  dev::wait_vm<0>();
  if (q0 >= s) return;
  // dq element 4·r4 + e: query q0 + 8r4 + 4g + e, head dim nb·32 + l32
  const float rs = 1.f / __builtin_sqrtf((float)D);
  const int64_t h = (int64_t)heads * D;
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int qr = q0 + 8 * r4 + 4 * g + e;
      if (qr < s) {
        bf16 *row = dQKV + ((int64_t)bi * s + qr) * 3 * h + head * D + l32;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) row[nb * 32] = (bf16)(dq[nb][r4 * 4 + e] * rs);
      }
    }
}

// ---- D[bh, q] = Σ_d dO[bh, q, d] · O[b, q, head·D + d] (dO head-major, O
// token-major): D/8 lanes per row, 16 bytes of each operand per lane, the
// lane sums combined by a butterfly of lane exchanges
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(const bf16 *__restrict__ dO,
                                                             const bf16 *__restrict__ O,
                                                             float *__restrict__ nDq, int s, int heads,
                                                             int64_t rows) {
  constexpr int LPR = D / 8, RPB = 256 / LPR; // lanes per row, rows per workgroup
  const int64_t i = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int l = threadIdx.x % LPR;
  float acc = 0.f;
  if (i < rows) {
    const int64_t bh = i / s;
    const int q = (int)(i - bh * s);
    const int64_t bi = bh / heads, head = bh - bi * heads;
    const bf16x8 x = *reinterpret_cast<const bf16x8 *>(dO + i * D + l * 8);
    const bf16x8 y = *reinterpret_cast<const bf16x8 *>(O + (bi * s + q) * heads * D + head * D + l * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)x[e] * (float)y[e];
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (i < rows && l == 0) nDq[i] = -acc; // stored negated, as the products start from -D
}

// ---- X [nb, s, D] -> XT [nb, D, sp]: position p of a row holds token
// vt_perm(p); positions of tokens >= s are zero. 64 positions × 32 dims per
// workgroup (sp % 64 == 0, D % 32 == 0): one 16-byte load of 8 dims and one
// 16-byte store of 8 positions per thread, through LDS.
__global__ __launch_bounds__(256) void transpose_perm_kernel(const bf16 *__restrict__ X,
                                                             bf16 *__restrict__ XT, int s, int sp,
                                                             int D) {
  __shared__ __attribute__((aligned(16))) bf16 tile[64][40]; // rows padded to 80 bytes
  const int p0 = blockIdx.x * 64, d0 = blockIdx.y * 32;
  const int64_t bh = blockIdx.z;
  const bf16 *Xh = X + bh * s * D;
  bf16 *XTh = XT + bh * D * sp;
  const int t = threadIdx.x;
  {
    const int r = t >> 2, ch = (t & 3) * 8; // token p0 + r, dims d0 + ch ..
    bf16x8 v = {};
    if (p0 + r < s) v = *reinterpret_cast<const bf16x8 *>(Xh + (int64_t)(p0 + r) * D + d0 + ch);
    *reinterpret_cast<bf16x8 *>(&tile[r][ch]) = v;
  }
  __syncthreads();
  {
    const int dr = t >> 3, pc = (t & 7) * 8; // dim d0 + dr, positions p0 + pc ..
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[vt_perm(pc + e)][dr];
    *reinterpret_cast<bf16x8 *>(XTh + (int64_t)(d0 + dr) * sp + p0 + pc) = v;
  }
}

// ---- the inverse for the forward's V^T: XT [nb, D, s] (row stride s,
// position p of a row holding token vt_perm(p)) -> X [nb, s, D]. 64 positions
// × 32 dims per workgroup: one 16-byte load of 8 positions and one 16-byte
// store of 8 dims per thread, through LDS. s % 16 == 0, so an 8-position
// chunk lies wholly inside or wholly past the row, and the tokens of a chunk
// inside it are too (vt_perm stays within groups of 16).
__global__ __launch_bounds__(256) void untranspose_perm_kernel(const bf16 *__restrict__ XT,
                                                               bf16 *__restrict__ X, int s, int D) {
  __shared__ __attribute__((aligned(16))) bf16 tile[64][40]; // [token][dim], rows padded to 80 bytes
  const int p0 = blockIdx.x * 64, d0 = blockIdx.y * 32;
  const int64_t bh = blockIdx.z;
  const bf16 *XTh = XT + bh * D * s;
  bf16 *Xh = X + bh * s * D;
  const int t = threadIdx.x;
  {
    const int dr = t >> 3, pc = (t & 7) * 8; // dim d0 + dr, positions p0 + pc ..
    bf16x8 v = {};
    if (p0 + pc < s) v = *reinterpret_cast<const bf16x8 *>(XTh + (int64_t)(d0 + dr) * s + p0 + pc);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[vt_perm(pc + e)][dr] = v[e];
  }
  __syncthreads();
  {
    const int r = t >> 2, ch = (t & 3) * 8; // token p0 + r, dims d0 + ch ..
    if (p0 + r < s)
      *reinterpret_cast<bf16x8 *>(Xh + (int64_t)(p0 + r) * D + d0 + ch) =
          *reinterpret_cast<const bf16x8 *>(&tile[r][ch]);
  }
}

// ---- X [R, C] (row stride ldx; C, ldx % 64 == 0) -> XT [C, Rp] (row stride
// Rp >= R, Rp % 8 == 0; columns R .. Rp-1 zero); 64 × 64 tiles through LDS
// with 16-byte loads and stores. With colpart, each tile also writes its
// column sums in fp32: colpart[blockIdx.y·C + c] = Σ over the tile's rows of
// X[r, c] (the fixed-order first pass of a column sum). XT may be null: then
// only the column sums are written.
__global__ __launch_bounds__(256) void transpose_kernel(const bf16 *__restrict__ X, int64_t ldx,
                                                        bf16 *__restrict__ XT, int64_t R, int64_t C,
                                                        int64_t Rp, float *__restrict__ colpart) {
  __shared__ __attribute__((aligned(16))) bf16 tile[64][72]; // rows padded to 144 bytes
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int t = threadIdx.x;
  // 512 loads of 8 columns: load i covers row i / 8, columns 8·(i % 8)..
  for (int i = t; i < 512; i += 256) {
    const int r = i >> 3, ch = (i & 7) * 8;
    bf16x8 v = {};
    if (r0 + r < R) v = *reinterpret_cast<const bf16x8 *>(X + (r0 + r) * ldx + c0 + ch);
    *reinterpret_cast<bf16x8 *>(&tile[r][ch]) = v;
  }
  __syncthreads();
  if (colpart != nullptr && t < 64) {
    float acc = 0.f;
    for (int r = 0; r < 64; ++r) acc += (float)tile[r][t];
    colpart[(int64_t)blockIdx.y * C + c0 + t] = acc;
  }
  if (XT == nullptr) return; // (column sums only)
  // 512 stores of 8 positions: store i covers XT row c0 + i / 8, positions
  // r0 + 8·(i % 8).. (all in or all past Rp, as Rp % 8 == 0)
  for (int i = t; i < 512; i += 256) {
    const int c = i >> 3, rk = (i & 7) * 8;
    if (r0 + rk < Rp) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = tile[rk + e][c];
      *reinterpret_cast<bf16x8 *>(XT + (c0 + c) * Rp + r0 + rk) = v;
    }
  }
}

// ---- the same sum for at most 8 parts (the K-split products' partials, and
// column sums of few row tiles), bandwidth-bound: four columns per thread in
// 16-byte accesses, a grid-stride loop. Bit for bit the result of
// colsum_final_kernel, which then adds out (or 0), part 0, part 1, ... in
// this order; the two differ only in the sign of a zero on the way (that
// kernel adds 0 + part k, never -0), and the +0 added last makes every zero
// result +0, as there.
__global__ __launch_bounds__(256) void sum_parts_few_kernel(const f32x4 *__restrict__ part, int nparts,
                                                            int64_t n4, f32x4 *__restrict__ out,
                                                            int accumulate) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    f32x4 t = accumulate ? out[i] : (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < nparts; ++k) t += part[k * n4 + i];
    t += (f32x4){0.f, 0.f, 0.f, 0.f};
    out[i] = t;
  }
}

// ---- out[c] (+)= Σ_k part[k, c], k in order: the second pass of a column
// sum, and the sum of K-split partial products
// 32 columns per workgroup, 8 threads per column: thread group k sums parts
// k, k+8, k+16, ..., then the 8 sums are added in order of k
__global__ __launch_bounds__(256) void colsum_final_kernel(const float *__restrict__ part,
                                                           int64_t nparts, int64_t C,
                                                           float *__restrict__ out, int accumulate) {
  __shared__ float red[8][32];
  const int cl = threadIdx.x & 31, k0 = threadIdx.x >> 5;
  const int64_t c = (int64_t)blockIdx.x * 32 + cl;
  float acc = 0.f;
  if (c < C)
    for (int64_t k = k0; k < nparts; k += 8) acc += part[k * C + c];
  red[k0][cl] = acc;
  __syncthreads();
  if (k0 == 0 && c < C) {
    float t = accumulate ? out[c] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) t += red[j][cl];
    out[c] = t;
  }
}

__global__ void fill_u32_kernel(uint32_t *__restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

} // namespace

hipError_t launch_attention_bwd_bf16(const void *Qs, const void *K, const void *V, const void *dO,
                                     const void *dOT, const float *nlse, const float *nDq, void *dQKV,
                                     int64_t batch, int64_t seq, int64_t sp, int64_t heads,
                                     int64_t head_dim, int causal, hipStream_t stream) {
  if (batch <= 0 || seq <= 0) return hipSuccess;
  if (seq % 16 != 0 || sp % 64 != 0 || sp < seq) return hipErrorInvalidValue;
  const int64_t bh = batch * heads;
  const int64_t nblk = (seq + 127) / 128;
  if (bh > INT32_MAX || nblk > 65535) return hipErrorInvalidValue;
  dim3 grid((unsigned)bh, (unsigned)nblk), block(256);
  const bf16 *q = (const bf16 *)Qs, *k = (const bf16 *)K, *v = (const bf16 *)V, *o = (const bf16 *)dO;
  const bf16 *ot = (const bf16 *)dOT;
  bf16 *out = (bf16 *)dQKV;
#define BPT_BWD_LAUNCH(DD)                                                                         \
  hipLaunchKernelGGL((attn_bwd_dkv_kernel<DD, false>), grid, block, 0, stream, q, k, v, o, ot, nlse, \
                     nDq, out, (int)seq, (int)sp, (int)heads, causal);                               \
  hipLaunchKernelGGL((attn_bwd_dkv_kernel<DD, true>), grid, block, 0, stream, q, k, v, o, ot, nlse,  \
                     nDq, out, (int)seq, (int)sp, (int)heads, causal);                               \
  hipLaunchKernelGGL((attn_bwd_dq_kernel<DD>), grid, block, 0, stream, q, k, v, o, nlse, nDq, out,    \
                     (int)seq, (int)heads, causal);
  switch (head_dim) {
  case 32:
    BPT_BWD_LAUNCH(32)
    break;
  case 64:
    BPT_BWD_LAUNCH(64)
    break;
  case 128:
    BPT_BWD_LAUNCH(128)
    break;
  default:
    return hipErrorInvalidValue;
  }
#undef BPT_BWD_LAUNCH
  return hipGetLastError();
}

hipError_t launch_attention_delta(const void *dO, const void *O, float *nDq, int64_t batch,
                                  int64_t seq, int64_t heads, int64_t head_dim, hipStream_t stream) {
  const int64_t rows = batch * heads * seq;
  if (rows <= 0) return hipSuccess;
  const int rpb = 256 / (int)(head_dim / 8);
  const int64_t blocks = (rows + rpb - 1) / rpb;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
#define BPT_DELTA_LAUNCH(DD)                                                                       \
  hipLaunchKernelGGL(attn_bwd_delta_kernel<DD>, dim3((unsigned)blocks), dim3(256), 0, stream,      \
                     (const bf16 *)dO, (const bf16 *)O, nDq, (int)seq, (int)heads, rows);
  switch (head_dim) {
  case 32:
    BPT_DELTA_LAUNCH(32)
    break;
  case 64:
    BPT_DELTA_LAUNCH(64)
    break;
  case 128:
    BPT_DELTA_LAUNCH(128)
    break;
  default:
    return hipErrorInvalidValue;
  }
#undef BPT_DELTA_LAUNCH
  return hipGetLastError();
}

hipError_t launch_transpose_perm(const void *X, void *XT, int64_t nb, int64_t seq, int64_t sp,
                                 int64_t head_dim, hipStream_t stream) {
  if (nb <= 0 || seq <= 0) return hipSuccess;
  if (head_dim % 32 != 0 || sp % 64 != 0 || nb > 65535) return hipErrorInvalidValue;
  dim3 grid((unsigned)(sp / 64), (unsigned)(head_dim / 32), (unsigned)nb);
  hipLaunchKernelGGL(transpose_perm_kernel, grid, dim3(256), 0, stream, (const bf16 *)X, (bf16 *)XT,
                     (int)seq, (int)sp, (int)head_dim);
  return hipGetLastError();
}

hipError_t launch_untranspose_perm(const void *XT, void *X, int64_t nb, int64_t seq,
                                   int64_t head_dim, hipStream_t stream) {
  if (nb <= 0 || seq <= 0) return hipSuccess;
  if (head_dim % 32 != 0 || seq % 16 != 0 || nb > 65535 || seq > INT32_MAX)
    return hipErrorInvalidValue;
  dim3 grid((unsigned)((seq + 63) / 64), (unsigned)(head_dim / 32), (unsigned)nb);
  hipLaunchKernelGGL(untranspose_perm_kernel, grid, dim3(256), 0, stream, (const bf16 *)XT,
                     (bf16 *)X, (int)seq, (int)head_dim);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const void *X, int64_t ldx, void *XT, int64_t R, int64_t C,
                                 int64_t Rp, hipStream_t stream) {
  return launch_transpose_colsum(X, ldx, XT, R, C, Rp, nullptr, nullptr, 0, stream);
}

int64_t transpose_row_tiles(int64_t Rp) { return (Rp + 63) / 64; }

hipError_t launch_transpose_colsum(const void *X, int64_t ldx, void *XT, int64_t R, int64_t C,
                                   int64_t Rp, float *part, float *out, int accumulate,
                                   hipStream_t stream) {
  if (Rp <= 0 || C <= 0) return hipSuccess;
  if (Rp < R || Rp % 8 != 0 || C % 64 != 0 || ldx % 8 != 0) return hipErrorInvalidValue;
  const int64_t gy = transpose_row_tiles(Rp), gx = C / 64;
  if (gy > 65535 || gx > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream,
                     (const bf16 *)X, ldx, (bf16 *)XT, R, C, Rp, out ? part : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || out == nullptr) return e;
  return launch_sum_parts(part, gy, C, out, accumulate, stream);
}

hipError_t launch_colsum(const void *X, int64_t ldx, int64_t R, int64_t C, float *part, float *out,
                         int accumulate, hipStream_t stream) {
  if (R <= 0 || C <= 0) return hipSuccess;
  if (C % 64 != 0 || ldx % 8 != 0) return hipErrorInvalidValue;
  const int64_t Rp = (R + 7) / 8 * 8, gy = transpose_row_tiles(Rp), gx = C / 64;
  if (gy > 65535 || gx > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream,
                     (const bf16 *)X, ldx, (bf16 *)nullptr, R, C, Rp, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_sum_parts(part, gy, C, out, accumulate, stream);
}

hipError_t launch_sum_parts(const float *part, int64_t nparts, int64_t n, float *out, int accumulate,
                            hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (nparts >= 1 && nparts <= 8 && n % 4 == 0 && ((uintptr_t)part | (uintptr_t)out) % 16 == 0) {
    const int64_t n4 = n / 4, want = (n4 + 255) / 256;
    hipLaunchKernelGGL(sum_parts_few_kernel, dim3((unsigned)(want < 8192 ? want : 8192)), dim3(256), 0, stream,
                       (const f32x4 *)part, (int)nparts, n4, (f32x4 *)out, accumulate);
    return hipGetLastError();
  }
  const int64_t blocks = (n + 31) / 32;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(colsum_final_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part, nparts, n,
                     out, accumulate);
  return hipGetLastError();
}

hipError_t launch_fill_u32(void *p, int64_t n, uint32_t v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint32_t *)p, n,
                     v);
  return hipGetLastError();
}

} // namespace bpt
