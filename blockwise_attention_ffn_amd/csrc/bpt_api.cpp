// Host side of the BPT layer forward C ABI (include/bpt.h): argument
// validation, the workspace plan, and the launch schedule on one stream.
//
// Schedule of one layer (BPT paper review, Algorithm 1):
//   1. the QKV projection of the whole sequence (two launches of the MFMA
//      GEMM: Q|K into head-major [b, nh, s, d], V into transposed
//      [b, nh, d, s']);
//   2. blockwise attention over every (batch, head, query block), writing
//      A [b, s, h];
//   3. y = x + A·Woᵀ + bo for all tokens (into out);
//   4. for each group of G consecutive query blocks (G·B_q rows of the
//      flattened token axis): H = max(0, y·W1ᵀ + b1) (bounded scratch of
//      G·B_q × f), out = y + H·W2ᵀ + b2.
// The weights arrive in the [out, in] layout, which is the K-contiguous B
// operand every GEMM here reads. Only step 4's scratch depends on f, and it
// is independent of s.
#include "../../include/bpt.h"
#include "bpt_internal.h"

#include <atomic>
#include <math.h>
#include <string.h>

namespace {

using namespace bpt;

constexpr size_t kAlign = 256;
constexpr int64_t kEpilogueRowsBf16 = 8192; // target rows per FFN group
constexpr int64_t kEpilogueRowsF32 = 1024;

struct Plan {
  int64_t b, s, h, nh, f, d;
  int dtype;
  size_t esize;
  int64_t rows_per_group;
  int attn_rows, attn_keys; // the attention's tile: query rows per workgroup, keys per stage
  // byte offsets into the workspace
  size_t off_q, off_k, off_v, off_a, off_h;
  size_t total;
};

inline bool mul_ok(size_t a, size_t b, size_t *r) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *r = a * b;
  return true;
}

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int check_shape(const bpt_shape *sh) {
  if (!sh) return BPT_ERR_NULL;
  if (sh->dtype != BPT_F32 && sh->dtype != BPT_BF16) return BPT_ERR_DTYPE;
  if (sh->batch < 1 || sh->seq < 16 || sh->seq % 16 != 0) return BPT_ERR_SHAPE;
  if (sh->hidden < 64 || sh->hidden % 64 != 0) return BPT_ERR_SHAPE;
  if (sh->ffn < 64 || sh->ffn % 64 != 0) return BPT_ERR_SHAPE;
  if (sh->heads < 1 || sh->hidden % sh->heads != 0) return BPT_ERR_SHAPE;
  const int64_t d = sh->hidden / sh->heads;
  if (d != 32 && d != 64 && d != 128) return BPT_ERR_SHAPE;
  // index arithmetic inside the kernels is 32-bit per dimension
  if (sh->seq > (int64_t)1 << 28 || sh->hidden > (int64_t)1 << 20 || sh->ffn > (int64_t)1 << 22 ||
      sh->batch > (int64_t)1 << 20)
    return BPT_ERR_SHAPE;
  if (sh->batch * sh->seq > (int64_t)1 << 30) return BPT_ERR_SHAPE;
  // one head's K or V (seq·d elements) is addressed with 32-bit byte offsets
  if (sh->seq * d > (int64_t)1 << 30) return BPT_ERR_SHAPE;
  return BPT_OK;
}

int check_block(const bpt_shape *sh, int64_t B) {
  if (B < 16 || B > sh->seq || B % 16 != 0 || sh->seq % B != 0) return BPT_ERR_BLOCK;
  return BPT_OK;
}

int make_plan(const bpt_shape *sh, int64_t B_q, int64_t B_kv, Plan *p, int64_t ffn_rows = 0) {
  int st = check_shape(sh);
  if (st) return st;
  if ((st = check_block(sh, B_q)) || (st = check_block(sh, B_kv))) return st;
  if (ffn_rows < 0 || (ffn_rows > 0 && (ffn_rows % B_q != 0 || ffn_rows > sh->batch * sh->seq)))
    return BPT_ERR_BLOCK;
  p->b = sh->batch;
  p->s = sh->seq;
  p->h = sh->hidden;
  p->nh = sh->heads;
  p->f = sh->ffn;
  p->d = p->h / p->nh;
  p->dtype = sh->dtype;
  p->esize = sh->dtype == BPT_BF16 ? 2 : 4;
  const int64_t tokens = p->b * p->s;
  const int64_t target = sh->dtype == BPT_BF16 ? kEpilogueRowsBf16 : kEpilogueRowsF32;
  int64_t G = (target + B_q - 1) / B_q;
  if (G < 1) G = 1;
  int64_t rows = G * B_q;
  if (rows > tokens) rows = tokens; // tokens is a multiple of B_q
  if (ffn_rows > 0) rows = ffn_rows;
  p->rows_per_group = rows;
  p->attn_rows = sh->dtype == BPT_BF16 ? attention_tile_rows(B_q) : kF32AttnRows;
  p->attn_keys = sh->dtype == BPT_BF16 ? attention_stage_keys(B_kv) : kF32AttnKeys;

  size_t off = 0, sz;
  auto region = [&](size_t elems, size_t *o) -> bool {
    if (!mul_ok(elems, p->esize, &sz)) return false;
    *o = off;
    if (sz > SIZE_MAX - off - kAlign) return false;
    off = align_up(off + sz);
    return true;
  };
  const size_t h = p->h, f = p->f, bsh = (size_t)tokens * h;
  bool ok = true;
  ok = ok && region(bsh, &p->off_q) && region(bsh, &p->off_k) && region(bsh, &p->off_v) &&
       region(bsh, &p->off_a) && region((size_t)rows * f, &p->off_h);
  if (!ok) return BPT_ERR_SIZE;
  p->total = off;
  return BPT_OK;
}

struct Range {
  uintptr_t lo, hi;
};
inline bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

} // namespace

namespace bpt {
int check_device() {
  static std::atomic<int> cache[64]; // 0 unknown, 1 ok, 2 not gfx950
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return BPT_ERR_DEVICE;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 1) return BPT_OK;
    if (c == 2) return BPT_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BPT_ERR_DEVICE;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? BPT_OK : BPT_ERR_DEVICE;
}
} // namespace bpt

namespace {

struct LayerArgs {
  const void *x, *Wqkv, *bqkv, *Wo, *bo, *W1, *b1, *W2, *b2;
  void *out;
};

// Validate pointers of a full layer call. `need_ffn`: Wo..b2 and out are used.
int check_pointers(const Plan &p, const LayerArgs &a, bool need_ffn, void *ws, size_t ws_bytes,
                   void *extra_out) {
  if (!a.x || !a.Wqkv || !a.bqkv || !ws) return BPT_ERR_NULL;
  if (need_ffn && (!a.Wo || !a.bo || !a.W1 || !a.b1 || !a.W2 || !a.b2 || !a.out))
    return BPT_ERR_NULL;
  if (!need_ffn && !extra_out) return BPT_ERR_NULL;
  const void *ptrs[] = {a.x, a.Wqkv, a.bqkv, a.Wo, a.bo, a.W1, a.b1, a.W2, a.b2, a.out, ws,
                        extra_out};
  for (const void *q : ptrs)
    if (q && (reinterpret_cast<uintptr_t>(q) & 15u)) return BPT_ERR_ALIGN;
  if (ws_bytes < p.total) return BPT_ERR_WORKSPACE;

  const size_t e = p.esize, h = p.h, f = p.f, bsh = (size_t)(p.b * p.s) * h;
  auto R = [](const void *q, size_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(q);
    return Range{lo, lo + bytes};
  };
  Range inputs[9] = {R(a.x, bsh * e),      R(a.Wqkv, 3 * h * h * e), R(a.bqkv, 3 * h * e),
                     R(a.Wo, h * h * e),   R(a.bo, h * e),           R(a.W1, h * f * e),
                     R(a.b1, f * e),       R(a.W2, f * h * e),       R(a.b2, h * e)};
  const int n_in = need_ffn ? 9 : 3;
  const Range wsr = R(ws, p.total);
  for (int i = 0; i < n_in; ++i)
    if (overlap(wsr, inputs[i])) return BPT_ERR_ALIAS;
  if (need_ffn) {
    const Range o = R(a.out, bsh * e);
    if (overlap(o, wsr)) return BPT_ERR_ALIAS;
    for (int i = 0; i < 9; ++i) {
      if (i == 0 && a.out == a.x) continue; // in place is allowed
      if (overlap(o, inputs[i])) return BPT_ERR_ALIAS;
    }
  }
  if (extra_out) {
    const Range o = R(extra_out, bsh * e);
    if (overlap(o, wsr)) return BPT_ERR_ALIAS;
    for (int i = 0; i < n_in; ++i)
      if (overlap(o, inputs[i])) return BPT_ERR_ALIAS;
    if (need_ffn && overlap(o, R(a.out, bsh * e))) return BPT_ERR_ALIAS;
  }
  return BPT_OK;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? BPT_OK : BPT_ERR_HIP; }

#define BPT_TRY(expr)                                                                              \
  do {                                                                                             \
    hipError_t e_ = (expr);                                                                        \
    if (e_ != hipSuccess) return BPT_ERR_HIP;                                                      \
  } while (0)

// Steps 1 (Wqkv only) to 3. A_dst: where attention writes A.
int run_attention_part(const Plan &p, const LayerArgs &a, int causal, bool run_qkv, void *A_dst,
                       char *ws, hipStream_t stream) {
  const int64_t tokens = p.b * p.s, h = p.h;
  void *Q = ws + p.off_q, *K = ws + p.off_k, *V = ws + p.off_v;
  if (p.dtype == BPT_BF16) {
    if (run_qkv) {
      // Wqkv is [3h, h]: rows 0..2h-1 give Q|K, rows 2h..3h-1 give V
      GemmEpilogue ep;
      ep.bias = a.bqkv;
      ep.q = Q;
      ep.k = K;
      ep.seq = p.s;
      ep.heads = p.nh;
      ep.head_dim = p.d;
      ep.hidden = h;
      ep.q_scale = attention_q_scale(p.d);
      BPT_TRY(launch_gemm_bf16(EPI_QK, a.x, h, a.Wqkv, h, tokens, 2 * h, h, ep, stream));
      GemmEpilogue ev = ep;
      ev.bias = reinterpret_cast<const char *>(a.bqkv) + 2 * h * 2;
      ev.v = V;
      BPT_TRY(launch_gemm_bf16(EPI_VT, a.x, h,
                               reinterpret_cast<const char *>(a.Wqkv) + 2 * h * h * 2, h, tokens,
                               h, h, ev, stream));
    }
    BPT_TRY(launch_attention_bf16(Q, K, V, A_dst, p.b, p.s, p.nh, p.d, causal, stream, nullptr,
                                  p.attn_rows, p.attn_keys));
  } else {
    if (run_qkv) {
      GemmEpilogue ep;
      ep.bias = a.bqkv;
      ep.q = Q;
      ep.k = K;
      ep.v = V;
      ep.seq = p.s;
      ep.heads = p.nh;
      ep.head_dim = p.d;
      ep.hidden = h;
      BPT_TRY(launch_gemm_f32(EPI_QKV, (const float *)a.x, h, (const float *)a.Wqkv, h, tokens,
                              3 * h, h, ep, stream));
    }
    BPT_TRY(launch_attention_f32((const float *)Q, (const float *)K, (const float *)V,
                                 (float *)A_dst, p.b, p.s, p.nh, p.d, causal, stream));
  }
  return BPT_OK;
}

// Training-mode dropout of the two residual branches (threshold T of the
// 16-bit uniforms, scale 65536 / (65536 - T)); nullptr: inference.
struct Dropout {
  uint64_t seed;
  uint32_t threshold;
  float scale;
};

// T = round(p·65536) for p in [0, 1); false for anything else (NaN included)
bool dropout_threshold(double p, uint32_t *threshold) {
  if (!(p >= 0.0 && p < 1.0)) return false;
  *threshold = (uint32_t)llround(p * 65536.0);
  return *threshold < 65536u;
}

// the branch epilogue (EPI_RESID, or EPI_RESID_DROP for a dropout site)
int branch_epi(const Dropout *drop, uint32_t site, int64_t row0, GemmEpilogue &e) {
  if (!drop || drop->threshold == 0) return EPI_RESID;
  e.drop_seed = drop->seed;
  e.drop_site = site;
  e.drop_threshold = drop->threshold;
  e.drop_scale = drop->scale;
  e.row0 = row0;
  return EPI_RESID_DROP;
}

int run_layer(const Plan &p, const LayerArgs &a, int causal, void *A_out, void *y_out, char *ws,
              hipStream_t stream, const Dropout *drop = nullptr, void *H_out = nullptr) {
  const int64_t tokens = p.b * p.s, h = p.h, f = p.f;
  const size_t e = p.esize;
  char *Aws = ws + p.off_a;
  char *Hws = ws + p.off_h;
  int st = run_attention_part(p, a, causal, true, Aws, ws, stream);
  if (st) return st;
  if (A_out) BPT_TRY(hipMemcpyAsync(A_out, Aws, (size_t)tokens * h * e, hipMemcpyDeviceToDevice,
                                    stream));
  char *out = reinterpret_cast<char *>(a.out);
  const char *x = reinterpret_cast<const char *>(a.x);
  // y = x + A·Woᵀ + bo for every token at once (position-wise, so the same
  // result as per group, with four times the tiles per launch), into out
  {
    GemmEpilogue e1;
    e1.bias = a.bo;
    e1.resid = x;
    e1.ld_resid = h;
    e1.out = out;
    e1.ld_out = h;
    const int epi1 = branch_epi(drop, 0, 0, e1);
    if (p.dtype == BPT_BF16)
      BPT_TRY(launch_gemm_bf16(epi1, Aws, h, a.Wo, h, tokens, h, h, e1, stream));
    else
      BPT_TRY(launch_gemm_f32(epi1, (const float *)Aws, h, (const float *)a.Wo, h, tokens, h, h,
                              e1, stream));
    if (y_out) BPT_TRY(hipMemcpyAsync(y_out, out, (size_t)tokens * h * e, hipMemcpyDeviceToDevice,
                                      stream));
  }
  // the FFN per group of rows: H = max(0, y·W1ᵀ + b1) in the bounded scratch,
  // then out = y + H·W2ᵀ + b2 in place
  for (int64_t r0 = 0; r0 < tokens; r0 += p.rows_per_group) {
    const int64_t rows = (tokens - r0 < p.rows_per_group) ? tokens - r0 : p.rows_per_group;
    const size_t row_off = (size_t)r0 * h * e;
    GemmEpilogue e2;
    e2.bias = a.b1;
    e2.out = Hws;
    e2.ld_out = f;
    GemmEpilogue e3;
    e3.bias = a.b2;
    e3.resid = out + row_off;
    e3.ld_resid = h;
    e3.out = out + row_off;
    e3.ld_out = h;
    const int epi3 = branch_epi(drop, 1, r0, e3);
    if (p.dtype == BPT_BF16) {
      BPT_TRY(launch_gemm_bf16(EPI_RELU, out + row_off, h, a.W1, h, rows, f, h, e2, stream));
      BPT_TRY(launch_gemm_bf16(epi3, Hws, f, a.W2, f, rows, h, f, e3, stream));
    } else {
      BPT_TRY(launch_gemm_f32(EPI_RELU, (const float *)(out + row_off), h, (const float *)a.W1, h,
                              rows, f, h, e2, stream));
      BPT_TRY(launch_gemm_f32(epi3, (const float *)Hws, f, (const float *)a.W2, f, rows, h, f, e3,
                              stream));
    }
    if (H_out && r0 + rows == tokens)
      BPT_TRY(hipMemcpyAsync(H_out, Hws, (size_t)rows * f * e, hipMemcpyDeviceToDevice, stream));
  }
  return BPT_OK;
}

// rows of the last FFN group (the ones H_out receives)
int64_t last_group_rows(const Plan &p) {
  const int64_t T = p.b * p.s, G = p.rows_per_group;
  return T - G * ((T - 1) / G);
}

int layer_entry(const bpt_shape *shape, const LayerArgs &a, int64_t B_q, int64_t B_kv, int causal,
                void *A_out, void *y_out, void *workspace, size_t ws_bytes, bpt_stream_t stream,
                int64_t ffn_rows = 0, const Dropout *drop = nullptr, void *H_out = nullptr) {
  Plan p;
  int st = make_plan(shape, B_q, B_kv, &p, ffn_rows);
  if (st) return st;
  if ((st = check_pointers(p, a, true, workspace, ws_bytes, nullptr))) return st;
  if (A_out && (st = check_pointers(p, a, true, workspace, ws_bytes, A_out))) return st;
  if (y_out && (st = check_pointers(p, a, true, workspace, ws_bytes, y_out))) return st;
  const size_t bytes = (size_t)(p.b * p.s) * p.h * p.esize;
  const size_t hbytes = (size_t)last_group_rows(p) * (size_t)p.f * p.esize;
  if (H_out) {
    if (reinterpret_cast<uintptr_t>(H_out) & 15u) return BPT_ERR_ALIGN;
    // H_out is checked like the other outputs: no overlap with an input,
    // the workspace, out, A_out or y_out
    const uintptr_t lo = (uintptr_t)H_out;
    const Range hr{lo, lo + hbytes};
    auto R = [](const void *q, size_t n) {
      return Range{(uintptr_t)q, (uintptr_t)q + n};
    };
    const size_t e = p.esize, h = p.h, f = p.f;
    const Range others[] = {R(a.x, bytes),       R(a.Wqkv, 3 * h * h * e), R(a.bqkv, 3 * h * e),
                            R(a.Wo, h * h * e),  R(a.bo, h * e),           R(a.W1, h * f * e),
                            R(a.b1, f * e),      R(a.W2, f * h * e),       R(a.b2, h * e),
                            R(a.out, bytes),     R(workspace, p.total)};
    for (const Range &o : others)
      if (overlap(hr, o)) return BPT_ERR_ALIAS;
    if ((A_out && overlap(hr, R(A_out, bytes))) || (y_out && overlap(hr, R(y_out, bytes))))
      return BPT_ERR_ALIAS;
  }
  if (A_out && y_out) {
    const uintptr_t lo1 = (uintptr_t)A_out, lo2 = (uintptr_t)y_out;
    if (lo1 < lo2 + bytes && lo2 < lo1 + bytes) return BPT_ERR_ALIAS;
  }
  if ((st = check_device())) return st;
  return run_layer(p, a, causal ? 1 : 0, A_out, y_out, reinterpret_cast<char *>(workspace),
                   reinterpret_cast<hipStream_t>(stream), drop, H_out);
}

// ---------------------------------------------------------------- backward
// Gradients of the inference forward (dropout off) for an upstream gradient
// G = dL/d out, with the forward recomputed block by block rather than
// stored (the BPT review, section 三: memory of the blockwise layer, and its
// remark that the method composes with rematerialisation): the attention
// keeps only each row's log-sum-exp, and the FFN's hidden activations exist
// for one group of rows at a time, as in the forward. The chain rule, in the
// [out, in] weight layout (y = x + A·Woᵀ + bo, H = relu(y·W1ᵀ + b1),
// out = y + H·W2ᵀ + b2):
//   per FFN group:  dH = (G·W2) ∘ [H > 0],  dy = G + dH·W1,
//                   dW2 += Gᵀ·H,  dW1 += dHᵀ·y,  db2 += Σ G,  db1 += Σ dH
//   then            dWo = dyᵀ·A,  dbo = Σ dy,  dO = dy·Wo (per head),
//                   attention backward -> dQKV = [dQ | dK | dV],
//                   dWqkv = dQKVᵀ·x,  dbqkv = Σ dQKV,  dx = dy + dQKV·Wqkv.
// Every product runs on the forward's MFMA GEMM; the contractions over
// tokens (the weight gradients) read their token-major operands transposed
// in LDS, so no transposed copy of an activation is made.
struct BwdPlan {
  Plan f;          // the forward's shape and FFN group size
  int64_t sp;      // dO's key-permuted transpose: positions per row (s rounded up to 64)
  int64_t Tp, cp;  // tokens and FFN group rows rounded up to 32
  size_t off_qs, off_k, off_v, off_vt, off_a, off_y, off_lse, off_dq, off_do, off_dot, off_dy, off_dqkv, off_h,
      off_dh, off_w2t, off_w1t, off_wot, off_wqkvt, off_zero, off_part, off_kpart;
  size_t kpart_elems; // room for the K-split partial products of the fp32 weight gradients
  size_t total;
};

// K splits for a fp32 weight-gradient product of M×N outputs over K: the
// smallest modelled time ceil(tiles·ns / 256 CUs)·(10.5 µs + 0.0247 µs·K/ns),
// the measured cost of one round of 256×256-tile GEMM workgroups on MI355X,
// over ns in {1, 2, 4, 8} with K % (32·ns) == 0. Few output tiles over a long
// K (dWo at h = 2048: 64 tiles, K = all tokens) otherwise leave most CUs idle.
int acc32_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  int best = 1;
  double best_t = 0.0;
  for (int ns = 1; ns <= 8; ns *= 2) {
    if (K % (32 * (int64_t)ns) != 0) continue;
    const double rounds = (double)((tiles * ns + 255) / 256);
    const double t = rounds * (10.5 + 0.0247 * (double)(K / ns));
    if (ns == 1 || t < best_t) {
      best = ns;
      best_t = t;
    }
  }
  return best;
}

int make_bwd_plan(const bpt_shape *sh, int64_t B_q, int64_t B_kv, int64_t ffn_rows, BwdPlan *bp) {
  int st = make_plan(sh, B_q, B_kv, &bp->f, ffn_rows);
  if (st) return st;
  if (sh->dtype != BPT_BF16) return BPT_ERR_DTYPE;
  const Plan &p = bp->f;
  const int64_t T = p.b * p.s;
  bp->sp = (p.s + 63) / 64 * 64;
  bp->Tp = (T + 31) / 32 * 32;
  bp->cp = (p.rows_per_group + 31) / 32 * 32;
  const size_t e = 2, h = p.h, f = p.f;
  size_t off = 0, sz;
  bool ok = true;
  auto region = [&](size_t elems, size_t esz, size_t *o) {
    if (!ok) return;
    if (!mul_ok(elems, esz, &sz) || sz > SIZE_MAX - off - kAlign) {
      ok = false;
      return;
    }
    *o = off;
    off = align_up(off + sz);
  };
  const size_t th = (size_t)T * h, c = p.rows_per_group, cp = bp->cp;
  region(th, e, &bp->off_qs);
  region(th, e, &bp->off_k);
  region(th, e, &bp->off_v);
  region(th, e, &bp->off_vt);
  region(th, e, &bp->off_a);
  region(th, e, &bp->off_y);
  region((size_t)p.b * p.nh * p.s, 4, &bp->off_lse);
  region((size_t)p.b * p.nh * p.s, 4, &bp->off_dq);
  region(th, e, &bp->off_do);
  region((size_t)p.b * p.nh * p.d * bp->sp, e, &bp->off_dot);
  region(th, e, &bp->off_dy);
  region(3 * th, e, &bp->off_dqkv);
  region(c * f, e, &bp->off_h);
  region(c * f, e, &bp->off_dh);
  region(f * h, e, &bp->off_w2t);
  region(f * h, e, &bp->off_w1t);
  region(h * h, e, &bp->off_wot);
  region(3 * h * h, e, &bp->off_wqkvt);
  const size_t wide = 3 * h > f ? 3 * h : f;
  region(wide, e, &bp->off_zero);
  // column-sum partials, one row per 64-row tile: over all tokens only the
  // 3h and h columns of dbqkv and dbo are summed, the f columns of db1 over
  // one FFN group's rows, so no (tokens / 64) x f array is needed
  const size_t part_t = (size_t)transpose_row_tiles(bp->Tp) * 3 * h;
  const size_t part_c = (size_t)transpose_row_tiles((int64_t)cp) * (f > h ? f : h);
  region(part_t > part_c ? part_t : part_c, 4, &bp->off_part);
  size_t kpart = 0;
  auto need = [&](int ks, size_t mn) {
    if (ks > 1 && (size_t)ks * mn > kpart) kpart = (size_t)ks * mn;
  };
  need(acc32_splits(p.h, p.f, cp), h * f);
  need(acc32_splits(p.f, p.h, cp), f * h);
  need(acc32_splits(p.h, p.h, bp->Tp), h * h);
  need(acc32_splits(3 * p.h, p.h, bp->Tp), 3 * h * h);
  region(kpart, 4, &bp->off_kpart);
  bp->kpart_elems = kpart;
  if (!ok) return BPT_ERR_SIZE;
  bp->total = off;
  return BPT_OK;
}

struct BwdArgs {
  const void *dout;
  void *dx;
  float *dWqkv, *dbqkv, *dWo, *dbo, *dW1, *db1, *dW2, *db2;
};

// The head split of the Q|K projection (Q scaled for the attention's exp2):
// the epilogue the forward part below uses, and the template of the
// backward's head split of dO (with unit scale).
GemmEpilogue qk_epilogue(const Plan &p, const void *bqkv, void *Qs, void *Kh) {
  GemmEpilogue eq;
  eq.bias = bqkv;
  eq.q = Qs;
  eq.k = Kh;
  eq.seq = p.s;
  eq.heads = p.nh;
  eq.head_dim = p.d;
  eq.hidden = p.h;
  eq.q_scale = attention_q_scale(p.d);
  return eq;
}

// The forward up to y, into the backward's workspace: Q (scaled) and K
// head-major, V transposed, A with each row's negated log-sum-exp (the
// attention at its 256-row, 64-key tile, the one with that output), and
// y = x + A·Woᵀ + bo (training mode: the branch through its dropout mask).
int bwd_forward_part(const BwdPlan &bp, const LayerArgs &a, int causal, char *ws, hipStream_t stream,
                     const Dropout *drop) {
  const Plan &p = bp.f;
  const int64_t T = p.b * p.s, h = p.h;
  typedef __bf16 bf;
  bf *Qs = reinterpret_cast<bf *>(ws + bp.off_qs), *Kh = reinterpret_cast<bf *>(ws + bp.off_k),
     *Vt = reinterpret_cast<bf *>(ws + bp.off_vt), *A = reinterpret_cast<bf *>(ws + bp.off_a),
     *y = reinterpret_cast<bf *>(ws + bp.off_y);
  float *nlse = reinterpret_cast<float *>(ws + bp.off_lse);
  const bf *x = reinterpret_cast<const bf *>(a.x), *Wqkv = reinterpret_cast<const bf *>(a.Wqkv),
           *bqkv = reinterpret_cast<const bf *>(a.bqkv);
  const GemmEpilogue eq = qk_epilogue(p, bqkv, Qs, Kh);
  BPT_TRY(launch_gemm_bf16(EPI_QK, x, h, Wqkv, h, T, 2 * h, h, eq, stream));
  GemmEpilogue ev = eq;
  ev.bias = bqkv + 2 * h;
  ev.v = Vt;
  BPT_TRY(launch_gemm_bf16(EPI_VT, x, h, Wqkv + 2 * h * h, h, T, h, h, ev, stream));
  BPT_TRY(launch_attention_bf16(Qs, Kh, Vt, A, p.b, p.s, p.nh, p.d, causal, stream, nlse));
  GemmEpilogue e1;
  e1.bias = a.bo;
  e1.resid = x;
  e1.ld_resid = h;
  e1.out = y;
  e1.ld_out = h;
  const int epi1 = branch_epi(drop, 0, 0, e1);
  BPT_TRY(launch_gemm_bf16(epi1, A, h, a.Wo, h, T, h, h, e1, stream));
  return BPT_OK;
}

// recompute: run the forward part first (false: bpt_layer_fwd_for_bwd left
// it in the workspace)
int run_layer_bwd(const BwdPlan &bp, const LayerArgs &a, const BwdArgs &g, int causal, char *ws,
                  hipStream_t stream, const Dropout *drop = nullptr, bool recompute = true) {
  const Plan &p = bp.f;
  const int64_t T = p.b * p.s, h = p.h, f = p.f;
  typedef __bf16 bf;
  auto W = [&](size_t off) { return reinterpret_cast<bf *>(ws + off); };
  bf *Qs = W(bp.off_qs), *Kh = W(bp.off_k), *Vh = W(bp.off_v), *A = W(bp.off_a), *y = W(bp.off_y),
     *dO = W(bp.off_do), *dOT = W(bp.off_dot), *dy = W(bp.off_dy), *dQKV = W(bp.off_dqkv), *H = W(bp.off_h),
     *dH = W(bp.off_dh), *W2T = W(bp.off_w2t), *W1T = W(bp.off_w1t), *WoT = W(bp.off_wot),
     *WqkvT = W(bp.off_wqkvt), *zero = W(bp.off_zero);
  float *nlse = reinterpret_cast<float *>(ws + bp.off_lse);
  float *nDq = reinterpret_cast<float *>(ws + bp.off_dq);
  float *part = reinterpret_cast<float *>(ws + bp.off_part);
  float *kpart = reinterpret_cast<float *>(ws + bp.off_kpart);
  // fp32 weight gradient out (+)= Xᵀ·Y over K token rows, X [K, M] and Y [K, N]
  // token-major (row strides M and N), read transposed in LDS, no copies;
  // the K range split when few output tiles would leave CUs idle (as many
  // splits as the partial-product room holds)
  auto wgrad = [&](const void *X, const void *Y, int64_t M, int64_t N, int64_t K, float *out,
                   int acc) {
    int ks = acc32_splits(M, N, (K + 31) / 32 * 32);
    while (ks > 1 && (size_t)ks * (size_t)M * (size_t)N > bp.kpart_elems) ks /= 2;
    return launch_gemm_acc32_tok(X, M, Y, N, M, N, K, ks, kpart, out, acc, zero, stream);
  };
  const bf *x = reinterpret_cast<const bf *>(a.x), *G = reinterpret_cast<const bf *>(g.dout);
  const bf *bqkv = reinterpret_cast<const bf *>(a.bqkv);
  const size_t wide = 3 * h > f ? 3 * h : f;

  // zero bias (for products that have none); the weights transposed
  BPT_TRY(launch_fill_u32(zero, (int64_t)(wide / 2), 0u, stream));
  BPT_TRY(launch_transpose_bf16(a.W2, f, W2T, h, f, h, stream));
  BPT_TRY(launch_transpose_bf16(a.W1, h, W1T, f, h, f, stream));
  BPT_TRY(launch_transpose_bf16(a.Wo, h, WoT, h, h, h, stream));
  BPT_TRY(launch_transpose_bf16(a.Wqkv, h, WqkvT, 3 * h, h, 3 * h, stream));

  // ---- the forward up to y (Q, K, V^T, A, the log-sum-exp), recomputed or
  // kept from bpt_layer_fwd_for_bwd; V head-major for the attention
  // backward, transposed back from V^T (a copy, not another product)
  if (recompute) {
    const int st = bwd_forward_part(bp, a, causal, ws, stream, drop);
    if (st) return st;
  }
  const GemmEpilogue eq = qk_epilogue(p, bqkv, Qs, Kh);
  BPT_TRY(launch_untranspose_perm(W(bp.off_vt), Vh, p.b * p.nh, p.s, p.d, stream));
  // training mode: a dropped branch's upstream gradient is the gradient of
  // its sum times the branch's mask and scale
  const bool dropping = drop && drop->threshold != 0;

  // ---- the FFN per group of rows
  for (int64_t r0 = 0; r0 < T; r0 += p.rows_per_group) {
    const int64_t rows = (T - r0 < p.rows_per_group) ? T - r0 : p.rows_per_group;
    const bf *Gg = G + r0 * h, *yg = y + r0 * h;
    const bf *Gb = Gg; // the FFN branch's upstream gradient
    if (dropping) {
      // into dO's buffer, free until the output projection below
      BPT_TRY(launch_dropout_scale_bf16(Gg, dO, rows, h, h, r0, drop->seed, 1, drop->threshold,
                                        drop->scale, stream));
      Gb = dO;
    }
    GemmEpilogue e2; // H = relu(y·W1ᵀ + b1)
    e2.bias = a.b1;
    e2.out = H;
    e2.ld_out = f;
    BPT_TRY(launch_gemm_bf16(EPI_RELU, yg, h, a.W1, h, rows, f, h, e2, stream));
    GemmEpilogue em; // dH = (G·W2) ∘ [H > 0]
    em.bias = zero;
    em.resid = H;
    em.ld_resid = f;
    em.out = dH;
    em.ld_out = f;
    BPT_TRY(launch_gemm_bf16(EPI_MASK, Gb, h, W2T, h, rows, f, h, em, stream));
    GemmEpilogue ed; // dy = G + dH·W1
    ed.bias = zero;
    ed.resid = Gg;
    ed.ld_resid = h;
    ed.out = dy + r0 * h;
    ed.ld_out = h;
    BPT_TRY(launch_gemm_bf16(EPI_RESID, dH, f, W1T, f, rows, h, f, ed, stream));
    // dW2 (+)= Gᵀ·H, dW1 (+)= dHᵀ·y over the group's rows
    BPT_TRY(launch_colsum(Gb, h, rows, h, part, g.db2, r0 > 0, stream));
    BPT_TRY(launch_colsum(dH, f, rows, f, part, g.db1, r0 > 0, stream));
    BPT_TRY(wgrad(Gb, H, h, f, rows, g.dW2, r0 > 0));
    BPT_TRY(wgrad(dH, yg, f, h, rows, g.dW1, r0 > 0));
  }

  // ---- output projection: dWo = daᵀ·A, dbo = Σ da, dO = da·Wo per head, with
  // da = dy (training mode: dy through the attention branch's mask)
  const bf *da = dy;
  if (dropping) {
    // into y's buffer: y is not read again
    BPT_TRY(launch_dropout_scale_bf16(dy, y, T, h, h, 0, drop->seed, 0, drop->threshold,
                                      drop->scale, stream));
    da = y;
  }
  BPT_TRY(launch_colsum(da, h, T, h, part, g.dbo, 0, stream));
  BPT_TRY(wgrad(da, A, h, h, T, g.dWo, 0));
  GemmEpilogue eo = eq; // the head split with unit scale, no bias
  eo.bias = zero;
  eo.q = dO;
  eo.q_scale = 1.f;
  BPT_TRY(launch_gemm_bf16(EPI_QK, da, h, WoT, h, T, h, h, eo, stream));
  BPT_TRY(launch_transpose_perm(dO, dOT, p.b * p.nh, p.s, bp.sp, p.d, stream));
  BPT_TRY(launch_attention_delta(dO, A, nDq, p.b, p.s, p.nh, p.d, stream));

  // ---- attention
  BPT_TRY(launch_attention_bwd_bf16(Qs, Kh, Vh, dO, dOT, nlse, nDq, dQKV, p.b, p.s, bp.sp, p.nh, p.d,
                                    causal, stream));

  // ---- projection: dWqkv = dQKVᵀ·x, dbqkv = Σ dQKV, dx = dy + dQKV·Wqkv
  BPT_TRY(launch_colsum(dQKV, 3 * h, T, 3 * h, part, g.dbqkv, 0, stream));
  BPT_TRY(wgrad(dQKV, x, 3 * h, h, T, g.dWqkv, 0));
  GemmEpilogue ex;
  ex.bias = zero;
  ex.resid = dy;
  ex.ld_resid = h;
  ex.out = g.dx;
  ex.ld_out = h;
  BPT_TRY(launch_gemm_bf16(EPI_RESID, dQKV, 3 * h, WqkvT, 3 * h, T, h, 3 * h, ex, stream));
  return BPT_OK;
}

// bpt_layer_fwd_for_bwd: the forward part into the backward's workspace, then
// the FFN per group as in the forward (H in the backward's H buffer),
// out = y + H·W2ᵀ + b2 with y read from the workspace.
int run_layer_fwd_for_bwd(const BwdPlan &bp, const LayerArgs &a, int causal, char *ws,
                          hipStream_t stream, const Dropout *drop) {
  int st = bwd_forward_part(bp, a, causal, ws, stream, drop);
  if (st) return st;
  const Plan &p = bp.f;
  const int64_t T = p.b * p.s, h = p.h, f = p.f;
  typedef __bf16 bf;
  const bf *y = reinterpret_cast<const bf *>(ws + bp.off_y);
  bf *H = reinterpret_cast<bf *>(ws + bp.off_h), *out = reinterpret_cast<bf *>(a.out);
  for (int64_t r0 = 0; r0 < T; r0 += p.rows_per_group) {
    const int64_t rows = (T - r0 < p.rows_per_group) ? T - r0 : p.rows_per_group;
    GemmEpilogue e2;
    e2.bias = a.b1;
    e2.out = H;
    e2.ld_out = f;
    BPT_TRY(launch_gemm_bf16(EPI_RELU, y + r0 * h, h, a.W1, h, rows, f, h, e2, stream));
    GemmEpilogue e3;
    e3.bias = a.b2;
    e3.resid = y + r0 * h;
    e3.ld_resid = h;
    e3.out = out + r0 * h;
    e3.ld_out = h;
    const int epi3 = branch_epi(drop, 1, r0, e3);
    BPT_TRY(launch_gemm_bf16(epi3, H, f, a.W2, f, rows, h, f, e3, stream));
  }
  return BPT_OK;
}

// the pointer, alignment and overlap checks of bpt_layer_fwd_for_bwd: x,
// the weights, out and the workspace, none overlapping another (out may not
// be x: the backward reads x again)
int fwd_for_bwd_checks(const BwdPlan &bp, const LayerArgs &a, const void *workspace,
                       size_t ws_bytes) {
  const Plan &p = bp.f;
  if (!a.x || !a.Wqkv || !a.bqkv || !a.Wo || !a.bo || !a.W1 || !a.b1 || !a.W2 || !a.b2 || !a.out ||
      !workspace)
    return BPT_ERR_NULL;
  const void *ptrs[] = {a.x, a.Wqkv, a.bqkv, a.Wo, a.bo, a.W1, a.b1, a.W2, a.b2, a.out, workspace};
  for (const void *q : ptrs)
    if (reinterpret_cast<uintptr_t>(q) & 15u) return BPT_ERR_ALIGN;
  if (ws_bytes < bp.total) return BPT_ERR_WORKSPACE;
  const size_t h = p.h, f = p.f, bsh = (size_t)(p.b * p.s) * h;
  auto R = [](const void *q, size_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(q);
    return Range{lo, lo + bytes};
  };
  const Range rs[11] = {R(a.x, bsh * 2),   R(a.Wqkv, 3 * h * h * 2), R(a.bqkv, 3 * h * 2),
                        R(a.Wo, h * h * 2), R(a.bo, h * 2),         R(a.W1, h * f * 2),
                        R(a.b1, f * 2),     R(a.W2, f * h * 2),     R(a.b2, h * 2),
                        R(a.out, bsh * 2),  R(workspace, bp.total)};
  // out and the workspace are written: neither may overlap anything else
  for (int i = 9; i < 11; ++i)
    for (int j = 0; j < 11; ++j)
      if (j != i && overlap(rs[i], rs[j])) return BPT_ERR_ALIAS;
  return BPT_OK;
}

int layer_bwd_entry(const bpt_shape *sh, const LayerArgs &a, const BwdArgs &g, int64_t B_q,
                    int64_t B_kv, int causal, int64_t ffn_rows, void *workspace, size_t ws_bytes,
                    bpt_stream_t stream, const Dropout *drop = nullptr, bool recompute = true) {
  BwdPlan bp;
  int st = make_bwd_plan(sh, B_q, B_kv, ffn_rows, &bp);
  if (st) return st;
  const Plan &p = bp.f;
  if (!a.x || !a.Wqkv || !a.bqkv || !a.Wo || !a.bo || !a.W1 || !a.b1 || !a.W2 || !a.b2 ||
      !g.dout || !g.dx || !g.dWqkv || !g.dbqkv || !g.dWo || !g.dbo || !g.dW1 || !g.db1 ||
      !g.dW2 || !g.db2 || !workspace)
    return BPT_ERR_NULL;
  const void *ptrs[] = {a.x,     a.Wqkv,  a.bqkv, a.Wo,   a.bo,  a.W1,  a.b1,
                        a.W2,    a.b2,    g.dout, g.dx,   g.dWqkv, g.dbqkv, g.dWo,
                        g.dbo,   g.dW1,   g.db1,  g.dW2,  g.db2, workspace};
  for (const void *q : ptrs)
    if (reinterpret_cast<uintptr_t>(q) & 15u) return BPT_ERR_ALIGN;
  if (ws_bytes < bp.total) return BPT_ERR_WORKSPACE;
  // outputs may overlap neither each other nor an input nor the workspace
  const size_t h = p.h, f = p.f, bsh = (size_t)(p.b * p.s) * h;
  auto R = [](const void *q, size_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(q);
    return Range{lo, lo + bytes};
  };
  const Range ins[11] = {R(a.x, bsh * 2),  R(a.Wqkv, 3 * h * h * 2), R(a.bqkv, 3 * h * 2),
                         R(a.Wo, h * h * 2), R(a.bo, h * 2),         R(a.W1, h * f * 2),
                         R(a.b1, f * 2),     R(a.W2, f * h * 2),     R(a.b2, h * 2),
                         R(g.dout, bsh * 2), R(workspace, bp.total)};
  const Range outs[9] = {R(g.dx, bsh * 2),       R(g.dWqkv, 3 * h * h * 4), R(g.dbqkv, 3 * h * 4),
                         R(g.dWo, h * h * 4),    R(g.dbo, h * 4),           R(g.dW1, f * h * 4),
                         R(g.db1, f * 4),        R(g.dW2, h * f * 4),       R(g.db2, h * 4)};
  for (int i = 0; i < 9; ++i) {
    for (int j = 0; j < 11; ++j)
      if (overlap(outs[i], ins[j])) return BPT_ERR_ALIAS;
    for (int j = i + 1; j < 9; ++j)
      if (overlap(outs[i], outs[j])) return BPT_ERR_ALIAS;
  }
  for (int j = 0; j < 10; ++j)
    if (overlap(ins[10], ins[j])) return BPT_ERR_ALIAS;
  if ((st = check_device())) return st;
  return run_layer_bwd(bp, a, g, causal ? 1 : 0, reinterpret_cast<char *>(workspace),
                       reinterpret_cast<hipStream_t>(stream), drop, recompute);
}

} // namespace

extern "C" {

int bpt_layer_workspace_bytes(const bpt_shape *shape, int64_t B_q, int64_t B_kv, int causal,
                              size_t *bytes) {
  (void)causal;
  if (!bytes) return BPT_ERR_NULL;
  Plan p;
  const int st = make_plan(shape, B_q, B_kv, &p);
  if (st) return st;
  *bytes = p.total;
  return BPT_OK;
}

int bpt_layer_workspace_bytes_ex(const bpt_shape *shape, int64_t B_q, int64_t B_kv, int causal,
                                 int64_t ffn_rows, size_t *bytes) {
  (void)causal;
  if (!bytes) return BPT_ERR_NULL;
  Plan p;
  const int st = make_plan(shape, B_q, B_kv, &p, ffn_rows);
  if (st) return st;
  *bytes = p.total;
  return BPT_OK;
}

int bpt_layer_fwd_ex(const bpt_shape *shape, const void *x, const void *Wqkv, const void *bqkv,
                     const void *Wo, const void *bo, const void *W1, const void *b1,
                     const void *W2, const void *b2, int64_t B_q, int64_t B_kv, int causal,
                     int64_t ffn_rows, void *out, void *workspace, size_t workspace_bytes,
                     bpt_stream_t stream) {
  const LayerArgs a{x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, out};
  return layer_entry(shape, a, B_q, B_kv, causal, nullptr, nullptr, workspace, workspace_bytes,
                     stream, ffn_rows);
}

int bpt_layer_fwd_train(const bpt_shape *shape, const void *x, const void *Wqkv,
                        const void *bqkv, const void *Wo, const void *bo, const void *W1,
                        const void *b1, const void *W2, const void *b2, int64_t B_q,
                        int64_t B_kv, int causal, int64_t ffn_rows, double dropout_p,
                        uint64_t seed, void *out, void *workspace, size_t workspace_bytes,
                        bpt_stream_t stream) {
  Dropout d;
  if (!dropout_threshold(dropout_p, &d.threshold)) return BPT_ERR_DROPOUT;
  d.seed = seed;
  d.scale = (float)(65536.0 / (65536.0 - (double)d.threshold));
  const LayerArgs a{x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, out};
  return layer_entry(shape, a, B_q, B_kv, causal, nullptr, nullptr, workspace, workspace_bytes,
                     stream, ffn_rows, &d);
}

int bpt_debug_dropout_keep(int64_t tokens, int64_t channels, int64_t token0, double dropout_p,
                           uint64_t seed, int site, void *keep, bpt_stream_t stream) {
  uint32_t threshold;
  if (!dropout_threshold(dropout_p, &threshold) || channels % 16 != 0) return BPT_ERR_DROPOUT;
  if (tokens < 0 || channels < 0 || token0 < 0 || (site != 0 && site != 1)) return BPT_ERR_SHAPE;
  if (tokens == 0 || channels == 0) return BPT_OK;
  if (!keep) return BPT_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(keep) & 15u) return BPT_ERR_ALIGN;
  if (tokens > INT64_MAX / channels) return BPT_ERR_SIZE;
  int st;
  if ((st = check_device())) return st;
  if (launch_dropout_keep(reinterpret_cast<uint8_t *>(keep), tokens, channels, token0, seed,
                          (uint32_t)site, threshold,
                          reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return BPT_ERR_HIP;
  return BPT_OK;
}

int bpt_layer_attention_tile(const bpt_shape *shape, int64_t B_q, int64_t B_kv, int64_t *rows,
                             int64_t *keys) {
  if (!rows || !keys) return BPT_ERR_NULL;
  Plan p;
  const int st = make_plan(shape, B_q, B_kv, &p);
  if (st) return st;
  *rows = p.attn_rows;
  *keys = p.attn_keys;
  return BPT_OK;
}

int bpt_layer_epilogue_rows(const bpt_shape *shape, int64_t B_q, int64_t *rows) {
  if (!rows) return BPT_ERR_NULL;
  Plan p;
  const int st = make_plan(shape, B_q, B_q, &p);
  if (st) return st;
  *rows = p.rows_per_group;
  return BPT_OK;
}

int bpt_layer_fwd(const bpt_shape *shape, const void *x, const void *Wqkv, const void *bqkv,
                  const void *Wo, const void *bo, const void *W1, const void *b1, const void *W2,
                  const void *b2, int64_t B_q, int64_t B_kv, int causal, void *out,
                  void *workspace, size_t workspace_bytes, bpt_stream_t stream) {
  const LayerArgs a{x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, out};
  return layer_entry(shape, a, B_q, B_kv, causal, nullptr, nullptr, workspace, workspace_bytes,
                     stream);
}

int bpt_debug_intermediates(const bpt_shape *shape, const void *x, const void *Wqkv,
                            const void *bqkv, const void *Wo, const void *bo, const void *W1,
                            const void *b1, const void *W2, const void *b2, int64_t B_q,
                            int64_t B_kv, int causal, int64_t ffn_rows, void *out, void *A_out,
                            void *y_out, void *H_out, void *workspace, size_t workspace_bytes,
                            bpt_stream_t stream) {
  const LayerArgs a{x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, out};
  return layer_entry(shape, a, B_q, B_kv, causal, A_out, y_out, workspace, workspace_bytes,
                     stream, ffn_rows, nullptr, H_out);
}

int bpt_debug_attention(const bpt_shape *shape, const void *x, const void *Wqkv,
                        const void *bqkv, int64_t B_q, int64_t B_kv, int causal, int run_qkv,
                        void *A_out, void *workspace, size_t workspace_bytes,
                        bpt_stream_t stream) {
  Plan p;
  int st = make_plan(shape, B_q, B_kv, &p);
  if (st) return st;
  const LayerArgs a{x, Wqkv, bqkv, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  if ((st = check_pointers(p, a, false, workspace, workspace_bytes, A_out))) return st;
  if ((st = check_device())) return st;
  return run_attention_part(p, a, causal ? 1 : 0, run_qkv != 0, A_out,
                            reinterpret_cast<char *>(workspace),
                            reinterpret_cast<hipStream_t>(stream));
}

int bpt_layer_bwd_workspace_bytes(const bpt_shape *shape, int64_t B_q, int64_t B_kv, int causal,
                                  int64_t ffn_rows, size_t *bytes) {
  (void)causal;
  if (!bytes) return BPT_ERR_NULL;
  BwdPlan bp;
  const int st = make_bwd_plan(shape, B_q, B_kv, ffn_rows, &bp);
  if (st) return st;
  *bytes = bp.total;
  return BPT_OK;
}

int bpt_layer_bwd(const bpt_shape *shape, const void *x, const void *Wqkv, const void *bqkv,
                  const void *Wo, const void *bo, const void *W1, const void *b1, const void *W2,
                  const void *b2, int64_t B_q, int64_t B_kv, int causal, int64_t ffn_rows,
                  const void *dout, void *dx, float *dWqkv, float *dbqkv, float *dWo, float *dbo,
                  float *dW1, float *db1, float *dW2, float *db2, void *workspace,
                  size_t workspace_bytes, bpt_stream_t stream) {
  const LayerArgs a{x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, nullptr};
  const BwdArgs g{dout, dx, dWqkv, dbqkv, dWo, dbo, dW1, db1, dW2, db2};
  return layer_bwd_entry(shape, a, g, B_q, B_kv, causal, ffn_rows, workspace, workspace_bytes,
                         stream);
}

int bpt_layer_bwd_train(const bpt_shape *shape, const void *x, const void *Wqkv,
                        const void *bqkv, const void *Wo, const void *bo, const void *W1,
                        const void *b1, const void *W2, const void *b2, int64_t B_q,
                        int64_t B_kv, int causal, int64_t ffn_rows, double dropout_p,
                        uint64_t seed, const void *dout, void *dx, float *dWqkv, float *dbqkv,
                        float *dWo, float *dbo, float *dW1, float *db1, float *dW2, float *db2,
                        void *workspace, size_t workspace_bytes, bpt_stream_t stream) {
  Dropout d;
  if (!dropout_threshold(dropout_p, &d.threshold)) return BPT_ERR_DROPOUT;
  d.seed = seed;
  d.scale = (float)(65536.0 / (65536.0 - (double)d.threshold));
  const LayerArgs a{x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, nullptr};
  const BwdArgs g{dout, dx, dWqkv, dbqkv, dWo, dbo, dW1, db1, dW2, db2};
  return layer_bwd_entry(shape, a, g, B_q, B_kv, causal, ffn_rows, workspace, workspace_bytes,
                         stream, &d);
}

int bpt_layer_fwd_for_bwd(const bpt_shape *shape, const void *x, const void *Wqkv,
                          const void *bqkv, const void *Wo, const void *bo, const void *W1,
                          const void *b1, const void *W2, const void *b2, int64_t B_q,
                          int64_t B_kv, int causal, int64_t ffn_rows, double dropout_p,
                          uint64_t seed, void *out, void *workspace, size_t workspace_bytes,
                          bpt_stream_t stream) {
  Dropout d;
  if (!dropout_threshold(dropout_p, &d.threshold)) return BPT_ERR_DROPOUT;
  d.seed = seed;
  d.scale = (float)(65536.0 / (65536.0 - (double)d.threshold));
  BwdPlan bp;
  int st = make_bwd_plan(shape, B_q, B_kv, ffn_rows, &bp);
  if (st) return st;
  const LayerArgs a{x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, out};
  if ((st = fwd_for_bwd_checks(bp, a, workspace, workspace_bytes))) return st;
  if ((st = check_device())) return st;
  return run_layer_fwd_for_bwd(bp, a, causal ? 1 : 0, reinterpret_cast<char *>(workspace),
                               reinterpret_cast<hipStream_t>(stream), &d);
}

int bpt_layer_bwd_from_fwd(const bpt_shape *shape, const void *x, const void *Wqkv,
                           const void *bqkv, const void *Wo, const void *bo, const void *W1,
                           const void *b1, const void *W2, const void *b2, int64_t B_q,
                           int64_t B_kv, int causal, int64_t ffn_rows, double dropout_p,
                           uint64_t seed, const void *dout, void *dx, float *dWqkv,
                           float *dbqkv, float *dWo, float *dbo, float *dW1, float *db1,
                           float *dW2, float *db2, void *workspace, size_t workspace_bytes,
                           bpt_stream_t stream) {
  Dropout d;
  if (!dropout_threshold(dropout_p, &d.threshold)) return BPT_ERR_DROPOUT;
  d.seed = seed;
  d.scale = (float)(65536.0 / (65536.0 - (double)d.threshold));
  const LayerArgs a{x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, nullptr};
  const BwdArgs g{dout, dx, dWqkv, dbqkv, dWo, dbo, dW1, db1, dW2, db2};
  return layer_bwd_entry(shape, a, g, B_q, B_kv, causal, ffn_rows, workspace, workspace_bytes,
                         stream, &d, false);
}

double bpt_layer_algorithmic_flops(const bpt_shape *shape, int causal) {
  if (check_shape(shape) != BPT_OK) return -1.0;
  const double b = (double)shape->batch, s = (double)shape->seq, h = (double)shape->hidden,
               f = (double)shape->ffn;
  const double dense = 6.0 * b * s * h * h + 2.0 * b * s * h * h + 4.0 * b * s * h * f;
  const double attn = causal ? 2.0 * b * h * s * (s + 1.0) : 4.0 * b * s * s * h;
  return dense + attn;
}

const char *bpt_status_string(int status) {
  switch (status) {
  case BPT_OK: return "ok";
  case BPT_ERR_NULL: return "a required pointer is NULL";
  case BPT_ERR_SHAPE: return "unsupported shape (h % heads, head dim in {32,64,128}, h and f multiples of 64, seq a multiple of 16)";
  case BPT_ERR_BLOCK: return "block size must be a multiple of 16 in [16, seq] that divides seq";
  case BPT_ERR_DTYPE: return "unsupported dtype";
  case BPT_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
  case BPT_ERR_ALIAS: return "an output overlaps an input, a weight or the workspace";
  case BPT_ERR_WORKSPACE: return "workspace too small";
  case BPT_ERR_DEVICE: return "the current device is not gfx950 or cannot be queried";
  case BPT_ERR_HIP: return "a HIP launch or copy failed";
  case BPT_ERR_SIZE: return "size computation overflows";
  case BPT_ERR_DROPOUT: return "dropout rate must lie in [0, 1) and mask channels be a multiple of 16";
  case BPT_ERR_SCRATCH: return "the call needs more workspace than bpt_layer_fwd_noalloc's fixed scratch (BPT_NOALLOC_SCRATCH_BYTES); use bpt_layer_fwd_ex or a smaller ffn_rows";
  default: return "unknown status";
  }
}

const char *bpt_version(void) { return "bpt-gfx950 0.1"; }

} // extern "C"
