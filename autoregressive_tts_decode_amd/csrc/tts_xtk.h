// Persistent, XCD-tensor-parallel Talker step kernel (CDNA4, gfx950).
//
// One batch-1 Talker decoder step ("Running Qwen3-TTS on an AMD R9700", section "Running
// Qwen3-TTS": the per-frame Talker pass that emits the semantic token) runs as ONE kernel of 256
// workgroups x 512 threads: all decoder layers, the final norm and the semantic head for the
// position held in the device counters. The layer split is the one of the CodePredictor kernel:
// XCD g (the one the workgroup runs on) owns KV head g (its query heads, their output-projection
// columns) and FFN rows [F/8 * g, +F/8); rank r = blockIdx / 8 owns 1/32 of each of those row sets. The
// exchanges are the same tagged-value hand-offs. What differs:
//   * attention reads the fp32 KV cache in HBM: the positions 0..p are split into 32 contiguous
//     chunks, one per rank of the XCD; each rank produces a partial softmax state per head, and
//     two exchanges combine them (rank r combines 8 of the 2 x 128 outputs, then an all-gather);
//   * the waves of a workgroup split by role: four front waves poll the exchanges and run the
//     attention, four back waves stream the weight rows (the loads of one wave return in order, so
//     a poll never waits behind weight rows in flight);
//   * the weight slices are large (up to 192 KB per workgroup and phase): the q/k/v and output
//     rows, the gate/up rows past the first 32 and the semantic head go through two 32-register
//     buffers of the back waves, each chunk issued as soon as the one before it has been
//     consumed, while the first gate/up rows and later the down rows are copied straight into
//     LDS (up to 128 KB) in parts spread over the layer;
//   * the row dots run on the matrix cores: a 16-row tile of weight rows is the B operand of
//     v_mfma_f32_16x16x32_bf16 (registers hold B fragments: lane l row l % 16, columns 32 s +
//     8 (l / 16) of K step s; LDS rows are padded by 16 bytes so a fragment's 16 rows fall on
//     different banks), the A operand the input row cut into two bf16 parts, hi (the fp32
//     pattern with its low 16 bits cleared) and mid (x - hi rounded to bf16): hi + mid is x to
//     within 2^-17 |x|, and the products are exact in fp32. The K range of a tile is split over
//     waves, whose partial sums are added in wave order;
//   * E4M3 weights (WT = uint8_t): a 16-byte lane load carries two K steps of codes (the input
//     fragments use the same column order), widened exactly to bf16 before each MFMA; each row's
//     sum is multiplied by its fp32 scale where the row is emitted.
#pragma once

#include "tts_trace.h"
#include "tts_xtp.h"

namespace tts {
namespace xtp {

constexpr int TMAXL = 32;      // Talker layers supported
constexpr int THMAX = 2048;    // Talker hidden size supported
constexpr int TFXMAX = 768;    // FFN rows per XCD supported (F / 8)
constexpr int ATS = 264;       // attention partial slot of one rank: 2 heads x (max, sum, 128 outputs), padded
constexpr int WB = 8;          // 16-byte units per lane in one weight buffer

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct TkDesc {
  LayerW layer[TMAXL];
  LayerS scale[TMAXL];               // per-row fp32 scales of E4M3 matrices (unused for bf16 rows)
  const float* head_scale;           // [V] of the E4M3 semantic head
  int32_t n_layers, H, F, V, nq, nkv, d, cap;
  float eps;
  const void *final_norm, *lm_head;
  const float *rope_cos, *rope_sin;  // [cap][d/2]
  float *kc, *vc;                    // fp32 KV cache, stream 0: layer l, head h, position t at ((l * ls) + h * cap + t) * d
  long long ls;                      // layer stride of the cache in (head, position) rows
  const float* x_in;                 // [H] the step's input row
  float *logits, *hT;                // [V] semantic logits, [H] final-normed hidden
  u64 *xin, *xcr, *att;
  DevState* st;
  uint32_t* err;
};

struct TkCall {
  const TkDesc* desc;
  int32_t bump_pos, bump_frame;
};

// Wave roles. The front waves poll every exchange and run the attention; the back waves stream
// the weight rows and do the row dots. A poll is a load, and the loads of one wave return in
// order, so a front wave never waits behind weight rows in flight.
constexpr int NF = 4;                        // front waves
constexpr int NB = NW - NF;                  // back waves
constexpr int PF = NF * 64;                  // polling threads
constexpr int TLWB = 2 * (65536 + 256);      // LDS weight rows of a workgroup (bytes): 32 padded bf16 rows of 2048
constexpr int LPADB = 16;                    // LDS row padding of the weight rows (bytes)
constexpr int XST = THMAX + 16;              // row stride of the split normed residual row (bf16 elements)
constexpr int OST = 256 + 16;                // ... of the split attention output of the XCD
constexpr int HST = TFXMAX + 16;             // ... of the split SwiGLU slice

// One weight chunk in the back waves' registers: rows (wave - NF) + NB * j (j < RR) of the chunk,
// 16-byte units lane + 64 * k (k < KK) of each row, RR * KK <= WB.
struct WBuf {
  u32x4 b[WB];
};

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

// Bytes per weight element (bf16 rows or E4M3 codes) and K steps per 16-byte unit of a lane.
template <typename WT>
struct TkW {
  static constexpr int ES = (int)sizeof(WT);
  static constexpr int KE = 2 / ES;
  static constexpr int KPB = KE * WB;  // K steps in one weight buffer
};
// Column (element) of K step ks that lane group q = lane / 16 starts at. For bf16 rows a lane's
// 8 columns of a step are 32 ks + 8 q; for E4M3 rows two steps share a 16-byte unit, so the pair
// (2 m, 2 m + 1) takes columns 64 m + 16 q (+ 8 for the odd step). The input fragments use the
// same columns, so every MFMA still pairs each weight with its own input element.
template <int KE>
__device__ __forceinline__ int kcol(int ks, int q) {
  return 32 * KE * (ks / KE) + 8 * KE * q + 8 * (ks % KE);
}

// x at element k of a two-part split buffer (parts at sp[k], sp[st + k])
__device__ __forceinline__ void put2(uint16_t* sp, int st, int k, float x) {
  const uint32_t u = __float_as_uint(x);
  const __bf16 mid = (__bf16)(x - __uint_as_float(u & 0xffff0000u));
  sp[k] = (uint16_t)(u >> 16);
  sp[st + k] = __builtin_bit_cast(uint16_t, mid);
}
// A fragment of K step ks: lane l supplies row l % 16 = part (rows 0, 1) or zeros, the 8 columns
// of kcol(ks, l / 16).
template <int KE>
__device__ __forceinline__ bf16x8v a_frag2(const uint16_t* sp, int st, int ks, const uint16_t* zero) {
  const int lane = fresh_tid() & 63, row = lane & 15;
  const uint16_t* p = row < 2 ? sp + row * st + kcol<KE>(ks, lane >> 4) : zero;
  return *reinterpret_cast<const bf16x8v*>(p);
}
// The tile's dot for the lane's C column (lanes < 16): the two parts' rows of C.
__device__ __forceinline__ float parts2(const f32x4& acc) { return acc[0] + acc[1]; }

// 8 E4M3 codes (two dwords) as a bf16 B fragment: the conversion widens two codes to fp32
// exactly, and every E4M3 value is a bf16 value, so the upper half of each fp32 is the code's
// bf16 pattern.
__device__ __forceinline__ bf16x8v e4m3x8_bf16(uint32_t w0, uint32_t w1) {
  const uint32_t w[2] = {w0, w1};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
    o[2 * i] = (__float_as_uint(lo.x) >> 16) | (__float_as_uint(lo.y) & 0xffff0000u);
    o[2 * i + 1] = (__float_as_uint(hi.x) >> 16) | (__float_as_uint(hi.y) & 0xffff0000u);
  }
  const u32x4 v = {o[0], o[1], o[2], o[3]};
  return __builtin_bit_cast(bf16x8v, v);
}
// The B fragment of step s of a buffer (bf16: entry s; E4M3: half s % 2 of entry s / 2)
template <int KE>
__device__ __forceinline__ bf16x8v b_frag(const WBuf& B, int s) {
  if constexpr (KE == 1) {
    return __builtin_bit_cast(bf16x8v, B.b[s]);
  } else {
    const u32x4 v = B.b[s / 2];
    return s % 2 ? e4m3x8_bf16(v[2], v[3]) : e4m3x8_bf16(v[0], v[1]);
  }
}

// B fragments of one 16-row weight tile into a back wave's buffer: K steps s0 .. s0 + n - 1
// (n <= KPB, s0 a multiple of KE) of tile row l % 16; rowptr(i) is the byte address of row i's
// first column (rows i >= nrows read as zeros). An odd E4M3 count also loads the step after the
// last, which lies in the same row.
// Zeros in every entry of a buffer. Paths that issue no tile (the front waves, a buffer a shape
// leaves unused) clear it instead, so every path writes the whole buffer: the earlier contents are
// dead at each issue point and the compiler keeps no copy of them (a copy would wait for the
// loads in flight).
__device__ __forceinline__ void wb_clear(WBuf& B) {
#pragma unroll
  for (int s = 0; s < WB; ++s) B.b[s] = (u32x4){0u, 0u, 0u, 0u};
}
template <typename WT, typename RowFn>
__device__ __forceinline__ void wb_issue_tile(WBuf& B, int nrows, int s0, int n, RowFn rowptr) {
  constexpr int ES = TkW<WT>::ES, KE = TkW<WT>::KE;
  if (wave_id() < NF) return wb_clear(B);
  const int lane = fresh_tid() & 63, i = lane & 15;
  const bool live = i < nrows;
  const uint8_t* row = rowptr(live ? i : 0) + ES * kcol<KE>(s0, lane >> 4);
  const int ne = (n + KE - 1) / KE;
#pragma unroll
  for (int s = 0; s < WB; ++s) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (s < ne && live) v = *glb(reinterpret_cast<const u32x4*>(row + 64 * s));
    B.b[s] = v;
  }
}
// acc += the tile in B (K steps s0 .. s0 + n - 1) against the split input sp
template <typename WT>
__device__ __forceinline__ f32x4 mfma_regs(const WBuf& B, int n, const uint16_t* sp, int st, int s0, const uint16_t* zero,
                                           f32x4 acc) {
  constexpr int KE = TkW<WT>::KE;
#pragma unroll
  for (int s = 0; s < KE * WB; ++s)
    if (s < n)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_frag2<KE>(sp, st, s0 + s, zero), b_frag<KE>(B, s), acc, 0, 0, 0);
  return acc;
}
// The 16-row tile at rows t0 .. t0 + 15 of the LDS rows w (row stride ws bytes; rows >= nrows
// read row t0), K steps s0 .. s0 + n - 1 (n >= 1), against the split input sp. For bf16 rows step
// s + 1's fragments are read before step s's MFMA issues, so the LDS reads overlap the MFMA chain.
template <typename WT>
struct LdsB {
  typedef u32x4 T;
};
template <>
struct LdsB<uint8_t> {
  typedef uint2 T;
};
template <typename WT>
__device__ __forceinline__ typename LdsB<WT>::T lds_braw(const uint8_t* wr, int s, int q) {
  constexpr int ES = TkW<WT>::ES, KE = TkW<WT>::KE;
  return *reinterpret_cast<const typename LdsB<WT>::T*>(wr + ES * kcol<KE>(s, q));
}
__device__ __forceinline__ bf16x8v lds_bwiden(const u32x4& r) { return __builtin_bit_cast(bf16x8v, r); }
__device__ __forceinline__ bf16x8v lds_bwiden(const uint2& r) { return e4m3x8_bf16(r.x, r.y); }
template <typename WT>
__device__ __forceinline__ f32x4 mfma_lds(const uint8_t* w, int ws, int t0, int nrows, int s0, int n, const uint16_t* sp,
                                          int st, const uint16_t* zero) {
  constexpr int KE = TkW<WT>::KE;
  const int lane = fresh_tid() & 63, q = lane >> 4;
  const int row = t0 + (lane & 15) < nrows ? t0 + (lane & 15) : t0;
  const uint8_t* wr = w + row * ws;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (KE == 2) {
    // (pipelined E4M3 steps measured slower: the plain loop, scheduled by the compiler)
#pragma unroll 4
    for (int s = s0; s < s0 + n; ++s) {
      const uint2 c = *reinterpret_cast<const uint2*>(wr + kcol<KE>(s, q));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_frag2<KE>(sp, st, s, zero), e4m3x8_bf16(c.x, c.y), acc, 0, 0, 0);
    }
    return acc;
  }
  bf16x8v a = a_frag2<KE>(sp, st, s0, zero);
  typename LdsB<WT>::T b = lds_braw<WT>(wr, s0, q);
  for (int s = s0; s < s0 + n - 1; ++s) {
    const bf16x8v an = a_frag2<KE>(sp, st, s + 1, zero);
    const typename LdsB<WT>::T bn = lds_braw<WT>(wr, s + 1, q);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, lds_bwiden(b), acc, 0, 0, 0);
    a = an;
    b = bn;
  }
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, lds_bwiden(b), acc, 0, 0, 0);
}

// The weight rows of a layer, per workgroup (H in {512, 1024, 2048}, 8 KV heads of dimension 128
// and 2 query heads per KV head), as 16-row MFMA tiles. Register tiles live in the back waves' two
// buffers; back wave b = wave - NF takes a share of each tile's K steps:
//   A0, A1   the 16 q/k/v rows x H: K steps [H/128 b, + H/128), the first KPB in A0     regs
//   C        output projection: the H/32 rows x 256 of the XCD's heads, H/512 tiles
//            split over the 4 back waves, 8 K steps each tile                        regs (buffer 0)
//   DL       the first nl gate/up rows (gate rows first, then up rows) x H               LDS
//   D0, D1   the remaining gate/up rows (at most one tile) x H, as A0, A1                regs
//   E        down projection: H/32 rows x F/8                                             LDS
// and after the last layer F0, F1, the semantic head's V/256 <= 16 rows x H, as A0, A1.
// Row addresses are in bytes (ES per element).
template <typename WT>
__device__ __forceinline__ void tk_issue_a(WBuf& B, const KCONST TkDesc& D, const KCONST LayerW& W, int half, int g, int r) {
  constexpr int ES = TkW<WT>::ES, KPB = TkW<WT>::KPB;
  const int H = D.H, d = D.d, G = D.nq / D.nkv, qper = (G + 2) * d / NR, spw = H / 128;
  const int b = wave_id() - NF;
  if (KPB * half >= spw) return wb_clear(B);
  wb_issue_tile<WT>(B, qper, spw * b + KPB * half, min(KPB, spw - KPB * half), [&](int i) -> const uint8_t* {
    const int q = qper * r + i;
    if (q < G * d) return reinterpret_cast<const uint8_t*>(W.wq) + (size_t)ES * (G * d * g + q) * H;
    if (q < (G + 1) * d) return reinterpret_cast<const uint8_t*>(W.wk) + (size_t)ES * (d * g + q - G * d) * H;
    return reinterpret_cast<const uint8_t*>(W.wv) + (size_t)ES * (d * g + q - (G + 1) * d) * H;
  });
}
template <typename WT>
__device__ __forceinline__ void tk_issue_c(WBuf& B, const KCONST TkDesc& D, const KCONST LayerW& W, int half, int g, int r) {
  constexpr int ES = TkW<WT>::ES;
  if (half) return wb_clear(B);  // one buffer holds the whole output projection
  const int hper = D.H / NR, Gd = D.nq / D.nkv * D.d, T = hper / 16, wpt = NB / T, spw = (Gd / 32) / wpt;
  const int b = wave_id() - NF, t = b / wpt;
  wb_issue_tile<WT>(B, 16, spw * (b % wpt), spw, [&](int i) -> const uint8_t* {
    return reinterpret_cast<const uint8_t*>(W.wo) + (size_t)ES * ((size_t)(hper * r + 16 * t + i) * (D.nq * D.d) + Gd * g);
  });
}
// gate/up row q of the rank (gate rows 0 .. fper, then up rows fper .. 2 fper), as a byte address
template <typename WT>
__device__ __forceinline__ const uint8_t* tk_gu_row(const KCONST TkDesc& D, const KCONST LayerW& W, int q, int g, int r) {
  const int fx = D.F / NX, fper = fx / NR;
  const int f = fx * g + fper * r + (q < fper ? q : q - fper);
  return reinterpret_cast<const uint8_t*>(q < fper ? W.wg : W.wu) + (size_t)TkW<WT>::ES * f * D.H;
}
// A descriptor pointer as a wave-uniform value (each 32-bit half through readfirstlane, kept
// unsigned so the low half never sign-extends into the high one).
__device__ __forceinline__ const uint8_t* tk_uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

// half c of the register tile of gate/up rows nl .. nd - 1 (past the nl rows held in LDS)
template <typename WT>
__device__ __forceinline__ void tk_issue_d(WBuf& B, const KCONST TkDesc& D, const KCONST LayerW& W, int nl, int c, int g,
                                           int r) {
  constexpr int ES = TkW<WT>::ES, KPB = TkW<WT>::KPB;
  const int nd = 2 * (D.F / NX / NR), spw = D.H / 128;
  const int b = wave_id() - NF;
  if (nd <= nl || KPB * c >= spw) return wb_clear(B);
  // the gate and up matrices are read through scalar loads first (a per-lane choice between two
  // descriptor pointers would otherwise become a per-lane descriptor read)
  const uint8_t *wg = tk_uniform_ptr(W.wg), *wu = tk_uniform_ptr(W.wu);
  const int fx = D.F / NX, fper = fx / NR;
  wb_issue_tile<WT>(B, nd - nl, spw * b + KPB * c, min(KPB, spw - KPB * c), [&](int i) -> const uint8_t* {
    const int q = nl + i;
    const int f = fx * g + fper * r + (q < fper ? q : q - fper);
    return (q < fper ? wg : wu) + (size_t)ES * f * D.H;
  });
}
template <typename WT>
__device__ __forceinline__ void tk_issue_f(WBuf& B, const KCONST TkDesc& D, int half) {
  constexpr int ES = TkW<WT>::ES, KPB = TkW<WT>::KPB;
  const int vper = D.V / NWG, spw = D.H / 128;
  const int b = wave_id() - NF;
  if (KPB * half >= spw) return wb_clear(B);
  wb_issue_tile<WT>(B, vper, spw * b + KPB * half, min(KPB, spw - KPB * half), [&](int i) -> const uint8_t* {
    return reinterpret_cast<const uint8_t*>(D.lm_head) + (size_t)ES * (vper * blockIdx.x + i) * D.H;
  });
}

struct TkSmem {
  float xs[THMAX + 64];       // residual row, then the per-rank sums of squares
  __align__(16) uint16_t xnp[2 * XST];  // normed row in two parts; (as floats) cross-reduce partials
  float qkv[512];             // this XCD's q/k/v slice
  float q[2][128];            // normed + rotated q of the XCD's two heads
  float kp[128], vp[128];     // the step's k (normed + rotated) and v
  float wm[NF][2], wl[NF][2]; // per-wave softmax max and sum per head
  float wo[NF][2][128];       // per-wave unnormalised attention output per head
  float cmb[NR * 10];         // gathered partials of this rank's 8 outputs; per-wave dot partials
  __align__(16) uint16_t obp[2 * OST];  // attention output of the XCD's heads, in two parts
  __align__(16) uint16_t hbp[2 * HST];  // SwiGLU slice of the XCD, in two parts
  __align__(16) uint16_t zero[8];
  float red[64];
  __align__(16) uint8_t lw[TLWB];  // weight rows copied by LDS-direct loads (gate/up rows, then down rows), padded
};
static_assert(NR * 10 >= NW * 2 * 16, "per-wave dot partials fit the combine buffer");
// per-wave dot partials: [wave][set][row of the tile]
__device__ __forceinline__ float* tk_pt(TkSmem& S, int wave, int set) { return S.cmb + (wave * 2 + set) * 16; }

// Per-thread constants of one layer: norm gains of elements tid, tid + NT, tid + 2 NT, tid + 3 NT
// (H <= 4 NT), and for the q/k waves the q- or k-norm gains of lanes lane, lane + 64. With E4M3
// rows also the row scales of the rank's rows that thread tid emits: q/k/v row tid (sq), output
// row tid (so), gate and up row tid (sg, su), down row tid (sd), and after the last layer the
// semantic head row tid (sh); sg, su, sd are loaded one layer ahead into sgn, sun, sdn (the
// current ones are still needed when the next layer's constants arrive). The gains are kept as
// raw bf16 patterns and widened where they are used: widening them at the load would make the
// loading wave wait there for the load, and with it for every row it issued before. For the same
// reason every load here is unconditional, from a valid index (a thread whose element or row does
// not exist never uses the value).
struct TkConsts {
  uint32_t an[4], mn[4], qk[2];
  float sq, so, sg, su, sd, sh, sgn, sun, sdn;
};
__device__ __forceinline__ float gain_f32(uint32_t raw) { return __uint_as_float(raw << 16); }

template <typename WT>
__device__ __forceinline__ void tk_load_consts(TkConsts& c, const KCONST TkDesc& D, int l, int g, int r) {
  const KCONST LayerW& W = D.layer[l];
  const uint16_t* an = reinterpret_cast<const uint16_t*>(W.attn_norm);  // gains are bf16 for every weight type
  const uint16_t* mn = reinterpret_cast<const uint16_t*>(W.mlp_norm);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = min((int)threadIdx.x + k * NT, D.H - 1);
    c.an[k] = glb(an)[i];
    c.mn[k] = glb(mn)[i];
  }
  // q-norm gains for waves 0, 1, k-norm gains for the others (used by wave 2 only)
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const uint16_t* gn = reinterpret_cast<const uint16_t*>(wave < 2 ? W.q_norm : W.k_norm);
  c.qk[0] = glb(gn)[lane];
  c.qk[1] = glb(gn)[lane + 64];
  c.sq = c.so = c.sgn = c.sun = c.sdn = c.sh = 1.f;
  if constexpr (TkW<WT>::ES == 1) {
    const KCONST LayerS& Sc = D.scale[l];
    const int tid = threadIdx.x, d = D.d, G = D.nq / D.nkv, qper = (G + 2) * d / NR, hper = D.H / NR;
    const int fx = D.F / NX, fper = fx / NR;
    // the rank's qper q/k/v rows lie in one of the three matrices (qper divides d)
    const int q0 = qper * r, qi = min(tid, qper - 1);
    const float* sqm = q0 < G * d ? Sc.wq + G * d * g + q0 : q0 < (G + 1) * d ? Sc.wk + d * g + q0 - G * d : Sc.wv + d * g + q0 - (G + 1) * d;
    c.sq = glb(sqm)[qi];
    c.so = glb(Sc.wo)[hper * r + min(tid, hper - 1)];
    c.sdn = glb(Sc.wd)[hper * r + min(tid, hper - 1)];
    c.sgn = glb(Sc.wg)[fx * g + fper * r + min(tid, fper - 1)];
    c.sun = glb(Sc.wu)[fx * g + fper * r + min(tid, fper - 1)];
  }
}

// A block of weight rows copied into LDS in parts, by the front (FRONT) or back waves, with
// LDS-direct loads: row i (at b0 + i * stride for i < split, else b1 + (i - split) * stride, upr
// 16-byte units) lands at dst[i * ldst ..], ldst = 16 upr + LPADB bytes, so the rows of an MFMA
// fragment fall on different LDS banks. One instruction moves up to 64 consecutive units of one
// row (cpr instructions a row; lanes past the row's end are off). part(n) issues at most n more
// instructions per wave: a wave that issues more than its share of the CU's memory queue holds
// stalls until the queue drains, so large copies go in parts spread over the barrier intervals of
// a layer. A copy has landed once the issuing wave's vector-memory counter has passed it.
template <bool FRONT>
struct RowCopy {
  const uint8_t *b0, *b1;
  long long stride;
  int split, upr, cpr, ninst, ldst, j;

  // b0, b1: byte addresses of rows 0 and split; stride: bytes between rows; upr: 16-byte units a row
  __device__ __forceinline__ void begin(const void* b0_, const void* b1_, int split_, long long stride_, int nrows, int upr_) {
    b0 = reinterpret_cast<const uint8_t*>(b0_);
    b1 = reinterpret_cast<const uint8_t*>(b1_);
    split = split_;
    stride = stride_;
    upr = upr_;
    cpr = (upr_ + 63) / 64;
    ninst = nrows * cpr;
    ldst = 16 * upr_ + LPADB;
    j = FRONT ? wave_id() : wave_id() - NF;
  }
  __device__ __forceinline__ void part(uint8_t* dst, int n) {
    static_assert(NF == NB, "front and back wave sets of one size");
    if ((wave_id() < NF) != FRONT) return;
    const int lane = threadIdx.x & 63;
    for (int c = 0; c < n && j < ninst; ++c, j += NF) {
      const int row = j / cpr, ch = j - row * cpr;
      const int u = 64 * ch + lane;
      const uint8_t* src = (row < split ? b0 + row * stride : b1 + (row - split) * stride) + 16 * (u < upr ? u : 0);
      if (u < upr)
        __builtin_amdgcn_global_load_lds((const GLB void*)src, (__attribute__((address_space(3))) void*)&dst[row * ldst + 1024 * ch],
                                         16, 0, 0);
    }
  }
};

// Wait until every load this wave issued has landed (the LDS-direct rows included).
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0); }

// x * rsqrt(mean(x^2) + eps) * gain (raw bf16 gains gr) over n <= 4 NT elements, in two parts into sp (row stride
// XST); with out, also as fp32 (to global memory). ss: NR per-rank partial sums of squares (from
// reduce_gather) or nullptr to reduce here.
__device__ __forceinline__ void tk_rmsnorm(const float* x, int n, const uint32_t* gr, float eps, uint16_t* sp, float* red,
                                           const float* ss, float* out = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float tot = 0.f;
  if (ss) {
#pragma unroll
    for (int q = 0; q < NR; q += 4) {
      const float4 f = *reinterpret_cast<const float4*>(ss + q);
      tot += (f.x + f.y) + (f.z + f.w);
    }
  } else {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = tid + k * NT;
      if (i < n) s += x[i] * x[i];
    }
    s = wave_sum(s);
    if (lane == 0) red[wave] = s;
    lds_barrier();
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += red[w];
  }
  const float sc = 1.0f / sqrtf(tot / (float)n + eps);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid + k * NT;
    if (i < n) {
      const float y = x[i] * sc * gain_f32(gr[k]);
      put2(sp, XST, i, y);
      if (out) glb(out)[i] = y;
    }
  }
  lds_barrier();
}

// Attention of this XCD's two query heads over positions 0..p of KV head g, this rank's chunk of
// positions, then the two combining exchanges; the XCD's 256 outputs land in S.obp, in two parts. Only the front
// waves compute; the back waves meet them at the barriers, running bg(k) (k = 0 .. 3) in the four
// intervals before them. rc, rs: RoPE factors of position p at lane (q/k waves).
template <typename WT, typename Bg>
__device__ __forceinline__ bool tk_attention(const KCONST TkDesc& D, const Xch& X, int layer, int p, const TkConsts& cn,
                                             float rc, float rs, TkSmem& S, uint32_t& tag, int& iring, int& apar, int g,
                                             int r, Bg bg) {
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63, d = D.d;
  const float* kg = D.kc + ((size_t)layer * D.ls + (size_t)g * D.cap) * d;
  const float* vg = D.vc + ((size_t)layer * D.ls + (size_t)g * D.cap) * d;
  // the step's q (two heads) and k: per-head RMSNorm + RoPE at position p; v as is
  if (wave < 3) {
    const float* src = S.qkv + wave * d;
    float v0 = src[lane], v1 = src[lane + 64];
    const float sc = 1.0f / sqrtf(wave_sum(v0 * v0 + v1 * v1) / (float)d + D.eps);
    v0 *= sc * gain_f32(cn.qk[0]);
    v1 *= sc * gain_f32(cn.qk[1]);
    float* dst = wave < 2 ? S.q[wave] : S.kp;
    const float a = v0 * rc - v1 * rs, b = v1 * rc + v0 * rs;
    dst[lane] = a;
    dst[lane + 64] = b;
    if (wave == 2 && r == 0) {  // append k to the cache (read by later steps only)
      float* kd = D.kc + ((size_t)layer * D.ls + (size_t)g * D.cap + p) * d;
      glb(kd)[lane] = a;
      glb(kd)[lane + 64] = b;
    }
  } else if (wave == 3) {
    const float v0 = S.qkv[3 * d + lane], v1 = S.qkv[3 * d + lane + 64];
    S.vp[lane] = v0;
    S.vp[lane + 64] = v1;
    if (r == 0) {
      float* vd = D.vc + ((size_t)layer * D.ls + (size_t)g * D.cap + p) * d;
      glb(vd)[lane] = v0;
      glb(vd)[lane + 64] = v1;
    }
  } else {
    bg(0);
  }
  lds_barrier();
  TTS_STAMP(53);
  // this rank's chunk [t0, t1) of positions 0..p; each front wave takes 16 positions per pass
  const int n = p + 1, C = (n + NR - 1) / NR;
  const int t0 = r * C, t1 = min(t0 + C, n);
  const int tq = lane >> 2, e = lane & 3;  // lane = 4 * (position in pass) + quarter of the head dimension
  const float scale = 1.0f / sqrtf((float)d);
  if (wave < NF) {
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f}, o[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
    for (int base = t0 + wave * 16; base < t1; base += NF * 16) {
      const int t = base + tq;
      const bool valid = t < t1;
      const bool cur = t == p;  // the step's own k is in LDS (the cache write is for later steps)
      const GLB f32x4* kr = reinterpret_cast<const GLB f32x4*>(glb(kg + (size_t)(valid && !cur ? t : t0) * d + 32 * e));
      const f32x4* kl = reinterpret_cast<const f32x4*>(S.kp + 32 * e);
      float s[2] = {0.f, 0.f};
#pragma unroll 4
      for (int i = 0; i < 8; ++i) {
        f32x4 kv4 = kr[i];
        if (cur) kv4 = kl[i];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float4 q4 = *reinterpret_cast<const float4*>(&S.q[h][32 * e + 4 * i]);
          s[h] = fmaf(q4.x, kv4.x, s[h]); s[h] = fmaf(q4.y, kv4.y, s[h]);
          s[h] = fmaf(q4.z, kv4.z, s[h]); s[h] = fmaf(q4.w, kv4.w, s[h]);
        }
      }
      // quarter sums within each group of 4 lanes (DPP), then the pass's max and weight sum over
      // the positions from the lanes 4 t read as scalars: no cross-lane step goes through LDS
      const int npass = min(16, t1 - base);
      float w[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        s[h] += TTS_DPP(s[h], 0xB1);  // quad_perm [1,0,3,2]
        s[h] += TTS_DPP(s[h], 0x4E);  // quad_perm [2,3,0,1]
        s[h] = valid ? s[h] * scale : -INFINITY;
        float mx = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) mx = fmaxf(mx, readlane_f(s[h], 4 * tt));
        const float mn = fmaxf(m[h], mx);  // finite: the pass holds at least one valid position
        const float corr = m[h] == -INFINITY ? 0.f : expf(m[h] - mn);
        w[h] = valid ? expf(s[h] - mn) : 0.f;
        float ws = 0.f;
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) ws += readlane_f(w[h], 4 * tt);
        l[h] = l[h] * corr + ws;
        o[h][0] *= corr;
        o[h][1] *= corr;
        m[h] = mn;
      }
      // outputs: lane owns dimensions lane, lane + 64 of both heads. The pass's v rows are loaded
      // in batches of 8, all of a batch's loads in flight together; rows past the pass are not
      // loaded (their weight is 0). The step's own row, not yet in the cache, comes from LDS.
#pragma unroll
      for (int h8 = 0; h8 < 16; h8 += 8) {
        if (h8 < npass) {
          float va[8], vb[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            va[k] = 0.f;
            vb[k] = 0.f;
            if (h8 + k < npass) {
              const int tp = base + h8 + k;
              va[k] = glb(vg)[(size_t)tp * d + lane];
              vb[k] = glb(vg)[(size_t)tp * d + lane + 64];
            }
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int tt = h8 + k;
            const bool own = base + tt == p;
            const float v0 = own ? S.vp[lane] : va[k], v1 = own ? S.vp[lane + 64] : vb[k];
            const float w0 = readlane_f(w[0], 4 * tt), w1 = readlane_f(w[1], 4 * tt);
            o[0][0] = fmaf(w0, v0, o[0][0]); o[0][1] = fmaf(w0, v1, o[0][1]);
            o[1][0] = fmaf(w1, v0, o[1][0]); o[1][1] = fmaf(w1, v1, o[1][1]);
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (lane == 0) { S.wm[wave][h] = m[h]; S.wl[wave][h] = l[h]; }
      S.wo[wave][h][lane] = o[h][0];
      S.wo[wave][h][lane + 64] = o[h][1];
    }
  } else {
    bg(1);
  }
  lds_barrier();
  TTS_STAMP(54);
  // this rank's partial: combine the front waves; publish (max, sum, 128 outputs) per head
  ++tag;
  u64* slot = D.att + (((size_t)g * 2 + (apar & 1)) * NR + r) * ATS;
  if (tid < 256) {
    const int h = tid >> 7, i = tid & 127;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NF; ++w) mx = fmaxf(mx, S.wm[w][h]);
    float ls = 0.f, os = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NF; ++w) {
        const float f = S.wm[w][h] == -INFINITY ? 0.f : expf(S.wm[w][h] - mx);
        ls += S.wl[w][h] * f;
        os += S.wo[w][h][i] * f;
      }
    }
    st_l(slot + h * 130 + 2 + i, pack(os, tag));
    if (i == 0) {
      st_l(slot + h * 130, pack(mx, tag));
      st_l(slot + h * 130 + 1, pack(ls, tag));
    }
  } else {
    bg(2);
  }
  TTS_STAMP(55);
  // rank r combines outputs [8 * (r % 16), +8) of head r / 16 from the 32 ranks' partials
  const int hb = r >> 4, db = 8 * (r & 15);
  const u64* base = D.att + ((size_t)g * 2 + (apar & 1)) * NR * ATS;
  if (!get_at<(NR * 10 + PF - 1) / PF, PF>(NR * 10, tag, S.cmb, X.err, [&](int i) -> const u64* {
        const int s = i / 10, k = i % 10;
        return base + (size_t)s * ATS + hb * 130 + (k < 2 ? k : 2 + db + (k - 2));
      }))
    return false;
  TTS_STAMP(56);
  ++apar;
  if (!slice_gather_pe<1, 1, PF>(X, 8, 256, [&](auto emit) {
        if (threadIdx.x >= 8) return;
        const int k = threadIdx.x;
        float mx = -INFINITY;
        for (int s2 = 0; s2 < NR; ++s2) mx = fmaxf(mx, S.cmb[s2 * 10]);
        float ls = 0.f, os = 0.f;
        for (int s2 = 0; s2 < NR; ++s2) {
          const float ms = S.cmb[s2 * 10];
          const float f = ms == -INFINITY ? 0.f : expf(ms - mx);
          ls += S.cmb[s2 * 10 + 1] * f;
          os += S.cmb[s2 * 10 + 2 + k] * f;
        }
        emit(k, 0, os / ls);
      }, [&](int i, float v) { put2(S.obp, OST, i, v); }, tag, iring, g, r, [&] { if (wave >= NF) bg(3); }))
    return false;
  return true;
}

// The constants the layer after l needs (the final-norm gains in c.an after the last layer).
template <typename WT>
__device__ __forceinline__ void tk_next_consts(TkConsts& c, const KCONST TkDesc& D, int l, int tid, int g, int r) {
  if (l + 1 < D.n_layers) {
    tk_load_consts<WT>(c, D, l + 1, g, r);
  } else {
    const uint16_t* f = reinterpret_cast<const uint16_t*>(D.final_norm);
#pragma unroll
    for (int k = 0; k < 4; ++k) c.an[k] = glb(f)[min(tid + k * NT, D.H - 1)];
    if constexpr (TkW<WT>::ES == 1) {
      const int vper = D.V / NWG;
      c.sh = glb(D.head_scale)[vper * blockIdx.x + min(tid, vper - 1)];
    }
  }
}

template <typename WT>
__global__ __launch_bounds__(NT) void k_talker_step(TkCall C) {
  const KCONST TkDesc& D = *(const KCONST TkDesc*)C.desc;
  __shared__ TkSmem S;
  TTS_TRACE_BEGIN(2048);
  TTS_STAMP(49);
  const Xch X{D.xin, D.xcr, D.err};
  constexpr int KT = (THMAX + NR + PF - 1) / PF;  // intra gather of a residual row + sums of squares
  constexpr int KQ = (512 + PF - 1) / PF;         // intra gather of the q/k/v slices
  constexpr int KH = (TFXMAX + PF - 1) / PF;      // intra gather of the SwiGLU slices
  const int g = xcd_id(), r = blockIdx.x / NX, tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int H = D.H, d = D.d, G = D.nq / D.nkv;
  const int qrows = (G + 2) * d, qper = qrows / NR, hper = H / NR, fx = D.F / NX, fper = fx / NR;
  constexpr int ES = TkW<WT>::ES, KPB = TkW<WT>::KPB;
  // an E4M3 row's sum times its scale (bf16 rows have none)
  auto scl = [](float v, float s) { return ES == 1 ? v * s : v; };
  TkConsts c;
  tk_load_consts<WT>(c, D, 0, g, r);
  const int nd = 2 * fper;                                // gate + up rows of the rank
  const int nl = min(min(nd, TLWB / (ES * H + LPADB)), 32);  // gate/up rows held in LDS (at most 2 tiles)
  const int b = wave - NF;                                // back wave index (register tiles)
  // K split of the tiles: register tiles over the 4 back waves, LDS tiles over all 8 waves
  const int ksh = H / 32;                                 // K steps of a hidden-wide row
  const int spq = ksh / NB;                               // per back wave, hidden-wide register tiles
  const int tc = hper / 16, wpc = NB / tc, spc = (G * d / 32) / wpc;  // output projection tiles
  const int tgl = (nl + 15) / 16, wpg = NW / tgl, spg = ksh / wpg;    // LDS gate/up tiles
  const int tdn = hper / 16, wpd = NW / tdn, spd = (fx / 32) / wpd;   // down tiles
  const int gld = ES * H + LPADB, dld = ES * fx + LPADB;  // LDS row strides (bytes) of the gate/up and down rows
  // The LDS gate/up block of a layer goes in parts (instructions per back wave, 32 for the largest
  // block): 4 while the previous layer's down exchange runs, 4 after the q/k/v rows, 6 during the
  // q/k/v exchange, 4 + 6 + 4 in the attention and the rest during its last exchange.
  RowCopy<false> gu;
  auto gu_begin = [&](const KCONST LayerW& W) {
    gu.begin(tk_gu_row<WT>(D, W, 0, g, r), tk_gu_row<WT>(D, W, fper, g, r), fper, (long long)ES * H, nl, ES * H / 16);
  };
  RowCopy<true> dn;  // the down rows, by the front waves, in two parts
  WBuf X0, X1;
  // the step's input row before the weight tiles (a wave's loads return in order: issued behind
  // the tiles it would wait for them), four elements per thread
  static_assert(THMAX <= 4 * NT, "one 16-byte load per thread holds the input row");
  f32x4 xin = {0.f, 0.f, 0.f, 0.f};
  if (4 * tid < H) xin = *reinterpret_cast<const GLB f32x4*>(glb(D.x_in) + 4 * tid);
  tk_issue_a<WT>(X0, D, D.layer[0], 0, g, r);
  tk_issue_a<WT>(X1, D, D.layer[0], 1, g, r);
  gu_begin(D.layer[0]);
  gu.part(S.lw, 4);
  uint32_t tag = glb(D.st)->epoch;
  const int p = glb(D.st)->pos;
  float rc = 1.f, rs = 0.f;  // RoPE factors of position p (the same in every layer)
  if (wave < 3) {
    rc = glb(D.rope_cos)[(size_t)p * 64 + lane];
    rs = glb(D.rope_sin)[(size_t)p * 64 + lane];
  }
  int iring = 0, cpar = 0, apar = 0;
  if (4 * tid < H) *reinterpret_cast<f32x4*>(&S.xs[4 * tid]) = xin;
  if (tid < 8) S.zero[tid] = 0;
  lds_barrier();
  float* xn = reinterpret_cast<float*>(S.xnp);  // cross-reduce partials (the split row is dead by then)
  // the sum over a tile's waves (tile t of wpt waves from wave w0) of row i of their partials
  auto tile_sum = [&](int w0, int wpt, int set, int t, int i) {
    float v = 0.f;
    for (int k = 0; k < wpt; ++k) v += tk_pt(S, w0 + t * wpt + k, set)[i];
    return v;
  };
  bool ok = true;
  for (int l = 0; ok && l < D.n_layers; ++l) {
    const KCONST LayerW& W = D.layer[l];
    const bool last = l + 1 == D.n_layers;
    TTS_STAMP(50);
    c.sg = c.sgn;  // this layer's gate/up/down row scales (E4M3)
    c.su = c.sun;
    c.sd = c.sdn;
    // q/k/v tile (A0: X0, A1: X1); the output projection tiles (C) follow in buffer 0
    tk_rmsnorm(S.xs, H, c.an, D.eps, S.xnp, S.red, l > 0 ? S.xs + H : nullptr);
    if (wave >= NF) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma_regs<WT>(X0, min(KPB, spq), S.xnp, XST, spq * b, S.zero, acc);
      acc = mfma_regs<WT>(X1, spq - KPB, S.xnp, XST, spq * b + KPB, S.zero, acc);
      if (lane < 16) tk_pt(S, wave, 0)[lane] = parts2(acc);
    }
    tk_issue_c<WT>(X0, D, W, 0, g, r);
    gu.part(S.lw, 4);
    lds_barrier();
    TTS_STAMP(51);
    if (!slice_gather<1, KQ, PF>(X, qper, qrows, [&](int e, int) { return scl(tile_sum(NF, NB, 0, 0, e), c.sq); }, S.qkv, tag, iring, g, r,
                                 [&] { gu.part(S.lw, 6); })) {
      ok = false;
      break;
    }
    TTS_STAMP(52);
    if (!tk_attention<WT>(D, X, l, p, c, rc, rs, S, tag, iring, apar, g, r, [&](int k) {
          if (k == 3) gu.part(S.lw, 1 << 20);
          else gu.part(S.lw, k == 1 ? 6 : 4);
        })) {
      ok = false;
      break;
    }
    TTS_STAMP(57);
    // output projection tiles (C: X0), residual; the register gate/up tile follows (D0 now, D1
    // during the exchange)
    if (wave >= NF) {
      const f32x4 acc = mfma_regs<WT>(X0, spc, S.obp, OST, spc * (b % wpc), S.zero, (f32x4){0.f, 0.f, 0.f, 0.f});
      if (lane < 16) tk_pt(S, wave, 0)[lane] = parts2(acc);
    }
    tk_issue_d<WT>(X0, D, W, nl, 0, g, r);
    lds_barrier();
    TTS_STAMP(58);
    if (!reduce_gather_p<1, THMAX, KT, PF>(
            X,
            [&](auto emit) {
              for (int i = fresh_tid(); i < hper; i += NT) emit(i, 0, scl(tile_sum(NF, wpc, 0, i / 16, i % 16), c.so));
            },
            S.xs, xn, H, true, tag, iring, cpar, g, r, [&] { tk_issue_d<WT>(X1, D, W, nl, 1, g, r); })) {
      ok = false;
      break;
    }
    TTS_STAMP(59);
    // gate and up rows (LDS tiles, then the register tile D0: X0, D1: X1), SwiGLU. Once the LDS
    // block is read the front waves copy the down rows in its place (half now, half during the
    // SwiGLU exchange) and the back waves, their registers free, start on the next layer's q/k/v
    // rows (or the semantic head). Each wave loads its own next-layer constants behind its other
    // loads.
    tk_rmsnorm(S.xs, H, c.mn, D.eps, S.xnp, S.red, S.xs + H);
    if (wave >= NF) wait_loads();
    lds_barrier();
    {
      const int t = wave / wpg;
      const f32x4 acc = mfma_lds<WT>(S.lw, gld, 16 * t, nl, spg * (wave % wpg), spg, S.xnp, XST, S.zero);
      if (lane < 16) tk_pt(S, wave, 0)[lane] = parts2(acc);
    }
    lds_barrier();
    const int dparts = (hper * ((ES * fx / 16 + 63) / 64) + 2 * NF - 1) / (2 * NF);  // first half, per front wave
    if (wave < NF) {
      dn.begin(reinterpret_cast<const uint8_t*>(W.wd) + (size_t)ES * ((size_t)(hper * r) * D.F + fx * g), nullptr, hper,
               (long long)ES * D.F, hper, ES * fx / 16);
      dn.part(S.lw, dparts);
    } else {
      if (nd > nl) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma_regs<WT>(X0, min(KPB, spq), S.xnp, XST, spq * b, S.zero, acc);
        acc = mfma_regs<WT>(X1, spq - KPB, S.xnp, XST, spq * b + KPB, S.zero, acc);
        if (lane < 16) tk_pt(S, wave, 1)[lane] = parts2(acc);
      }
      if (!last) tk_issue_a<WT>(X0, D, D.layer[l + 1], 0, g, r);
      else tk_issue_f<WT>(X0, D, 0);
    }
    // one load site for both roles (after each wave's own issue), so the constants need no copy
    // where the two paths meet
    tk_next_consts<WT>(c, D, l, tid, g, r);
    lds_barrier();
    TTS_STAMP(61);
    // gate/up row q: an LDS tile row below nl, else a row of the register tile
    auto gu_val = [&](int q) { return q < nl ? tile_sum(0, wpg, 0, q / 16, q % 16) : tile_sum(NF, NB, 1, 0, q - nl); };
    if (!slice_gather_pe<1, KH, PF>(
            X, fper, fx,
            [&](auto emit) {
              for (int i = fresh_tid(); i < fper; i += NT) emit(i, 0, silu(scl(gu_val(i), c.sg)) * scl(gu_val(fper + i), c.su));
            },
            [&](int i, float v) { put2(S.hbp, HST, i, v); }, tag, iring, g, r, [&] {
              if (wave < NF) {
                dn.part(S.lw, 1 << 20);
              } else {
                if (!last) tk_issue_a<WT>(X1, D, D.layer[l + 1], 1, g, r);
                else tk_issue_f<WT>(X1, D, 1);
              }
            })) {
      ok = false;
      break;
    }
    // down projection tiles from LDS, residual; the next layer's LDS gate/up block starts during
    // the exchange
    TTS_STAMP(62);
    if (wave < NF) wait_loads();
    lds_barrier();
    {
      const int t = wave / wpd;
      const f32x4 acc = mfma_lds<WT>(S.lw, dld, 16 * t, hper, spd * (wave % wpd), spd, S.hbp, HST, S.zero);
      if (lane < 16) tk_pt(S, wave, 0)[lane] = parts2(acc);
    }
    lds_barrier();
    TTS_STAMP(63);
    if (!reduce_gather_p<1, THMAX, KT, PF>(
            X,
            [&](auto emit) {
              for (int i = fresh_tid(); i < hper; i += NT) emit(i, 0, scl(tile_sum(0, wpd, 0, i / 16, i % 16), c.sd));
            },
            S.xs, xn, H, true, tag, iring, cpar, g, r, [&] {
              if (!last) {
                gu_begin(D.layer[l + 1]);
                gu.part(S.lw, 4);
              }
            })) {
      ok = false;
      break;
    }
  }
  TTS_STAMP(64);
  if (ok) {
    // final norm (gains in c.an; workgroup 0 also writes the normed row, h_T), semantic head tile
    // (F0: X0, F1: X1)
    tk_rmsnorm(S.xs, H, c.an, D.eps, S.xnp, S.red, S.xs + H, blockIdx.x == 0 ? D.hT : nullptr);
    const int vper = D.V / NWG;
    if (wave >= NF) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma_regs<WT>(X0, min(KPB, spq), S.xnp, XST, spq * b, S.zero, acc);
      acc = mfma_regs<WT>(X1, spq - KPB, S.xnp, XST, spq * b + KPB, S.zero, acc);
      if (lane < 16) tk_pt(S, wave, 0)[lane] = parts2(acc);
    }
    lds_barrier();
    for (int i = tid; i < vper; i += NT) glb(D.logits)[vper * blockIdx.x + i] = scl(tile_sum(NF, NB, 0, 0, i), c.sh);
  }
  TTS_STAMP(65);
  if (blockIdx.x == 0 && tid == 0) {
    // every workgroup has read the counters: all took part in the last exchange
    GLB DevState* st = glb(D.st);
    st->epoch = tag + 1;
    if (C.bump_pos) st->pos = p + 1;
    if (C.bump_frame) st->frame = st->frame + 1;
  }
}

}  // namespace xtp
}  // namespace tts
