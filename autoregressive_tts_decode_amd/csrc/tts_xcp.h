// Persistent CodePredictor frame kernel, lean form (CDNA4, gfx950; bf16 or E4M3 weights).
//
// The 15 sequential CodePredictor steps of a frame ("Running Qwen3-TTS on an AMD R9700", section
// "Running Qwen3-TTS": the small decoder runs once per acoustic codebook after the Talker step)
// run in ONE kernel of 256 workgroups x 512 threads, one per CU, with the layer split of the
// exchange protocol in tts_xtp.h: XCD g (its XCC_ID) owns KV head g, its two query heads, their
// output-projection columns and FFN units [384 g, 384 g + 384); rank r = blockIdx / 8 owns 1/32
// of each of those row sets. Per layer six dependent exchanges of tagged fp32 values (q/k/v slice
// gather, output-projection reduce-scatter across XCDs, residual all-gather, SwiGLU slice gather,
// down-projection reduce-scatter, residual all-gather) carry the data between the workgroups.
//
// The kernel is specialised to the CodePredictor shape both synthetic models share (hidden 1024,
// FFN 3072, 16 query and 8 KV heads of dimension 128, codebook vocabulary 2048, at most five
// layers; an input projection from a Talker hidden of 2048, or none), so every loop is static.
// A frame is bound by the exchange chain, and what sits between two exchanges is issued by eight
// waves sharing four SIMDs: every instruction on that path counts. Hence:
//   * the projections run on the matrix cores. A 16 x 32 weight tile (16 rows of the workgroup's
//     slice, 32 columns) is the B operand of one v_mfma_f32_16x16x32_bf16, one weight row per
//     column of B; the A operand holds the input row cut into three bf16 parts: hi is x with the
//     low 16 bits of its fp32 pattern cleared, mid the same of x - hi, lo = x - hi - mid. Each
//     remainder is exact in fp32 and lo has at most 8 significant bits, so the parts sum to x
//     exactly; products of bf16 values are exact in fp32, so a row dot is an fp32 dot up to the
//     order of its sums. The parts are rows 0..2 of A (4..6 for a second input row): the lane
//     holding a weight row's C column gets its dot as the sum of three C values, with no
//     cross-lane reduction. The K range is split across the eight waves, whose partial sums are
//     added in wave order (a fixed order: the result does not depend on timing);
//   * inputs are cut into their parts where they arrive: by the exchange polls (residual rows,
//     times the next RMSNorm gain; the SwiGLU slice) and by the attention waves;
//   * a workgroup keeps only its own 32 elements of each residual row (the reduce that makes them
//     runs there) and the per-rank sums of squares, double buffered, so the all-gather of the new
//     residual needs no barrier behind the reduce that reads the old one;
//   * the input projection's tiles (the same every step) stay in registers for the whole frame;
//   * a phase's weight tiles for the next layer are issued a layer ahead of their use, in pieces of
//     at most 32 KB per CU spread over the layer's six polls: a CU holds its waves at the issue once about
//     16 KB are in flight, and a poll waits behind the loads issued before it.
#pragma once

#include "tts_trace.h"
#include "tts_xtp.h"

namespace tts {
namespace xcp {

using xtp::CpCall;
using xtp::CpDesc;
using xtp::LayerW;
using xtp::NR;
using xtp::NT;
using xtp::NW;
using xtp::NWG;
using xtp::NX;
using xtp::u64;

constexpr int H = 1024;          // CodePredictor hidden size
constexpr int D = 128;           // head dimension
constexpr int G = 2;             // query heads per KV head
constexpr int F = 3072;          // FFN size
constexpr int V = 2048;          // codebook vocabulary (rows of one head)
constexpr int QR = (G + 2) * D;  // q/k/v rows of one XCD: 512
constexpr int QPER = QR / NR;    // 16 per rank: one tile
constexpr int HPER = H / NR;     // 32 residual rows per rank: two tiles
constexpr int FX = F / NX;       // 384 FFN units per XCD
constexpr int FPER = FX / NR;    // 12 per rank: 24 gate/up rows, a tile and a half
constexpr int VPER = V / NWG;    // 8 head rows per workgroup: half a tile
constexpr int KX = 256;          // input-projection columns per XCD (Talker hidden 2048 / 8)
constexpr int MAXL = 5;          // CodePredictor layers supported
constexpr int P = 16;            // CodePredictor positions per frame
constexpr int KVS = 132;         // LDS row stride of the K/V rows (padded against bank conflicts)
// Row scales of the E4M3 matrices a workgroup uses, in LDS: per layer its q/k/v rows (16), output
// rows (32), gate and up rows (12 each) and down rows (32); then the 15 heads' 8 rows; then the
// input projection's 32 rows.
constexpr int SCQ = 0, SCO = SCQ + QPER, SCG = SCO + HPER, SCU = SCG + FPER, SCD = SCU + FPER, SCL = SCD + HPER;
constexpr int SCH = MAXL * SCL, SCP = SCH + 15 * VPER, SCN = SCP + HPER;
// LDS row strides (bf16 elements) of the split inputs: 64 bytes past the row, so the parts of one
// input row fall on different banks
constexpr int SH = H + 32;
constexpr int SO = G * D + 32;
constexpr int SF = FX + 32;

static_assert(QPER == 16 && HPER == 32 && 2 * FPER == 24 && VPER == 8, "row tiles");
static_assert(H / 32 == 4 * NW && G * D / 32 == NW && KX == G * D && 2 * (FX / 32) == 3 * NW, "K split");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Weight tiles of one layer in registers. A tile's B fragment: lane l holds its row l % 16 at
// columns 32 s + 8 (l / 16) .. + 8 of K step s.
//   q    the rank's 16 q/k/v rows, K steps 4 w .. 4 w + 3 (of 32)
//   o    output-projection rows 0..15 (o[0]) and 16..31 (o[1]) of the rank, K step w (of 8)
//   ga   gate/up rows 0..15, K steps 4 w, 4 w + 1; gb the same at K steps 4 w + 2, 4 w + 3
//   gc   gate/up rows 16..23 (lanes l % 16 < 8), K steps 4 w .. 4 w + 3; in a step's last layer
//        lanes l % 16 >= 8 take the step's head rows, used after that layer
//   dn   down rows 16 (w / 4) .. + 15 of the rank, K steps 3 (w % 4) .. + 2 (of 12)
// (Each piece that is issued on its own is a variable of its own: a partial update of one array
// would make the compiler copy the whole array.)
// One K step's fragment of a lane: 8 bf16 weights (16 bytes) or 8 E4M3 codes (8 bytes, widened to
// bf16 before the MFMA).
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
template <typename WT>
struct Frag {
  typedef u32x4 T;
};
template <>
struct Frag<uint8_t> {
  typedef u32x2 T;
};
template <typename WT>
struct Wl {
  typedef typename Frag<WT>::T F;
  F q[4];
  F o[2];
  F ga[2], gb[2];
  F gc[4];
  F dn[3];
};

// The lane index from a fresh thread index: what is computed from it is recomputed where it is
// used instead of being kept live across the layer loop (registers are the scarce resource here:
// the weight tiles of a whole layer stay in them).
__device__ __forceinline__ int lane_id() { return xtp::fresh_tid() & 63; }
// bf16 gains of elements lane and lane + 64 of a head-dimension vector in LDS
__device__ __forceinline__ void unpack_pair(const uint16_t* gv, int lane, float (&o)[2]) {
  o[0] = to_f32(gv[lane]);
  o[1] = to_f32(gv[lane + 64]);
}
__device__ __forceinline__ float rl(float v, int i) { return xtp::readlane_f(v, i); }

// x into its parts at element k of input row m of a split buffer sp [M][3][stride]
__device__ __forceinline__ void put_split(uint16_t* sp, int stride, int m, int k, float x) {
  const uint32_t u = __float_as_uint(x);
  const float r1 = x - __uint_as_float(u & 0xffff0000u);
  const uint32_t u1 = __float_as_uint(r1);
  const float r2 = r1 - __uint_as_float(u1 & 0xffff0000u);
  uint16_t* d = sp + 3 * m * stride + k;
  d[0] = (uint16_t)(u >> 16);
  d[stride] = (uint16_t)(u1 >> 16);
  d[2 * stride] = (uint16_t)(__float_as_uint(r2) >> 16);
}

// ---------------------------------------------------------------------------- weight tiles

template <typename T>
__device__ __forceinline__ const GLB u32x4* units(const T* p) {
  return xtp::glb(reinterpret_cast<const u32x4*>(p));
}
// A lane's tile fragment: the 8 elements at row0 (a uniform row base) + (l % 16) ld + 8 (l / 16) + c
// of a matrix of WT elements with ld columns (16 bytes of bf16, 8 of E4M3). The lane offset comes
// from a fresh thread index, so it is recomputed at each issue instead of being kept live across
// the layer loop for every site.
template <typename WT>
__device__ __forceinline__ typename Frag<WT>::T ld_frag(const void* m, int ld, int row0, int c) {
  const int l = xtp::fresh_tid() & 63;
  const WT* base = reinterpret_cast<const WT*>(m) + (size_t)row0 * ld + c;
  return *xtp::glb(reinterpret_cast<const typename Frag<WT>::T*>(base + ((l & 15) * ld + 8 * (l >> 4))));
}

// the rank's q/k/v rows QPER r + l % 16 of XCD g's (query heads | key | value) rows; the 16 rows
// lie in one of the three matrices (QPER divides D)
template <typename WT>
__device__ __forceinline__ void issue_q(Wl<WT>& R, const KCONST CpDesc& Dd, int l, int g, int r) {
  const KCONST LayerW& W = Dd.layer[l];
  const int w = xtp::wave_id(), q0 = QPER * r;
  const void* m = q0 < G * D ? W.wq : q0 < (G + 1) * D ? W.wk : W.wv;
  const int row0 = q0 < G * D ? G * D * g + q0 : q0 < (G + 1) * D ? D * g + q0 - G * D : D * g + q0 - (G + 1) * D;
#pragma unroll
  for (int s = 0; s < 4; ++s) R.q[s] = ld_frag<WT>(m, H, row0, 32 * (4 * w + s));
}
// rows HPER r + 16 t + l % 16 (t = 0, 1), K step w of the 256 columns from c0, of a matrix with
// ld columns (output projection; input projection)
template <typename WT>
__device__ __forceinline__ void issue_narrow(typename Frag<WT>::T (&o)[2], const void* m, int ld, int c0, int r) {
  const int w = xtp::wave_id();
#pragma unroll
  for (int t = 0; t < 2; ++t) o[t] = ld_frag<WT>(m, ld, HPER * r + 16 * t, c0 + 32 * w);
}
template <typename WT>
__device__ __forceinline__ void issue_o(Wl<WT>& R, const KCONST CpDesc& Dd, int l, int g, int r) {
  issue_narrow<WT>(R.o, Dd.layer[l].wo, Dd.nq * D, G * D * g, r);
}
// A descriptor pointer as a wave-uniform value. Selecting per lane between two pointers read from
// the descriptor would otherwise become a per-lane read of the descriptor (a vector load whose wait
// drains every weight load in flight); read each with a scalar load first.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

// gate/up rows q = l % 16 of the rank's gate rows 0..FPER-1, then up rows, of FFN units
// [FX g + FPER r, +FPER) (lanes 12..15: up rows 0..3), K steps 4 w + s0, 4 w + s0 + 1
template <typename WT>
__device__ __forceinline__ void issue_gu0(typename Frag<WT>::T (&t)[2], const KCONST CpDesc& Dd, int l, int g, int r, int s0) {
  const KCONST LayerW& W = Dd.layer[l];
  const void *wg = uniform_ptr(W.wg), *wu = uniform_ptr(W.wu);
  const int w = xtp::wave_id(), f0 = FX * g + FPER * r;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const bool gate = (xtp::fresh_tid() & 15) < FPER;
    t[s] = ld_frag<WT>(gate ? wg : wu, H, gate ? f0 : f0 - FPER, 32 * (4 * w + s0 + s));
  }
}
// Lanes l % 16 < 8: gate/up rows 16..23 (up rows 4..11). Lanes l % 16 >= 8: with head j >= 1,
// that head's rows VPER blockIdx + l % 16 - 8 (the head tile of the step's last layer, used after
// it); else the up rows again (columns of C that are never used). K steps 4 w .. 4 w + 3.
template <typename WT>
__device__ __forceinline__ void issue_gu1(Wl<WT>& R, const KCONST CpDesc& Dd, int l, int g, int r, int j) {
  const int w = xtp::wave_id(), f0 = FX * g + FPER * r;
  const void *wu = uniform_ptr(Dd.layer[l].wu), *hd = uniform_ptr(Dd.heads);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bool head = j > 0 && (xtp::fresh_tid() & 8);
    R.gc[s] = ld_frag<WT>(head ? hd : wu, H, head ? (j - 1) * V + VPER * (int)blockIdx.x - 8 : f0 + (16 - FPER) - 8 * ((xtp::fresh_tid() >> 3) & 1),
                      32 * (4 * w + s));
  }
}
// down rows HPER r + 16 (w / 4) + l % 16, K steps 3 (w % 4) .. + 2 of XCD g's FFN columns
template <typename WT>
__device__ __forceinline__ void issue_dn(Wl<WT>& R, const KCONST CpDesc& Dd, int l, int g, int r) {
  const int w = xtp::wave_id();
#pragma unroll
  for (int s = 0; s < 3; ++s) R.dn[s] = ld_frag<WT>(Dd.layer[l].wd, F, HPER * r + 16 * (w >> 2), FX * g + 32 * (3 * (w & 3) + s));
}
// ---------------------------------------------------------------------------- matrix-core dots

// NS K steps from ks0 of one weight tile against the split input sp (row stride st): lane l
// supplies A row l % 16 = 4 m + p, part p of input row m (rows past the parts: zeros).
// A K step's B fragment: the bf16 weights as they are, or 8 E4M3 codes widened to bf16 (exactly:
// every E4M3 value is a bf16 value, the upper half of its fp32 widening)
__device__ __forceinline__ bf16x8 bfrag(const u32x4& f) { return __builtin_bit_cast(bf16x8, f); }
__device__ __forceinline__ bf16x8 bfrag(const u32x2& f) {
  const uint32_t w[2] = {f.x, f.y};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
    o[2 * i] = (__float_as_uint(lo.x) >> 16) | (__float_as_uint(lo.y) & 0xffff0000u);
    o[2 * i + 1] = (__float_as_uint(hi.x) >> 16) | (__float_as_uint(hi.y) & 0xffff0000u);
  }
  const u32x4 v = {o[0], o[1], o[2], o[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <int M, int NS, typename FT>
__device__ __forceinline__ f32x4 mfma_steps(const FT* wt, const uint16_t* sp, int st, int ks0, const uint16_t* zero,
                                            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f}) {
  const int row = lane_id() & 15, m = row >> 2, p = row & 3;
  const bool live = p < 3 && m < M;
  const uint16_t* base = sp + (3 * m + p) * st;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(live ? base + 32 * (ks0 + s) + 8 * (lane_id() >> 4) : zero);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bfrag(wt[s]), acc, 0, 0, 0);
  }
  return acc;
}
// Lane 16 m + i (m < M) gets the dot of weight row i with input row m: C rows 4 m .. 4 m + 2.
__device__ __forceinline__ float parts_sum(const f32x4& acc) { return (acc[0] + acc[1]) + acc[2]; }

// 1 / sqrt(mean(x^2) + eps) of a residual row from its NR per-rank sums of squares (whole wave)
__device__ __forceinline__ float norm_scale(const float* ss, float eps) {
  const int lane = lane_id();
  float v = lane < NR ? ss[lane] : 0.f;
  v = row16_sum(v);
  return 1.0f / sqrtf((rl(v, 0) + rl(v, 16)) / (float)H + eps);
}

// ---------------------------------------------------------------------------- shared memory

struct Smem {
  float xo[2][2][HPER];          // this rank's elements of the residual rows [buffer][row]
  float ss[2][2 * NR];           // per-rank sums of squares of the residual rows [buffer][row NR + rank]
  union {
    struct {
      float xn[NX * 2 * HPER];   // reduce-scatter partials: partner x, row m at (x M + m) HPER
      float qkv[2 * QR];         // this XCD's q/k/v rows (row m at m QR)
      float kq[4][D];            // normed, rotated q of each attention wave
    };
    __align__(16) float sv[V];   // sampled ids: the step's logits over the temperature (after the last layer)
  };
  float part[NW][2][32];         // per-wave partial dots [wave][tile][16 m + row]
  float cand[2 * NWG];           // argmax candidates (value, id bits)
  float rope[P][2][D / 2];       // cos, sin of positions 0..15
  float kvc[MAXL][2][P][KVS];    // this frame's K/V rows of KV head g, per layer
  __align__(16) uint16_t xsp[2 * 3 * SH];  // residual rows times the next RMSNorm gain, in parts
  __align__(16) uint16_t osp[2 * 3 * SO];  // attention output (or input-projection slice), in parts
  __align__(16) uint16_t hsp[2 * 3 * SF];  // SwiGLU slice of the XCD, in parts
  __align__(16) uint16_t zero[8];
  __align__(16) uint16_t gn[2 * MAXL + 1][H];  // RMSNorm gains: layer l attention 2 l, MLP 2 l + 1, final 2 MAXL
  __align__(16) uint16_t gqk[MAXL][2][D];      // q-norm, k-norm gains per layer
  float scl[SCN];                              // E4M3 row scales (unused for bf16 weights)
  __align__(16) uint32_t bins[4][256];         // sampled ids: radix-select histograms, one per key byte
  u64 ckey[64];                                // sampled ids: the kept keys
  int ncand;                                   // sampled ids: kept keys so far
  int wsum[NW];                                // sampled ids: per-wave counts of keys tied at the cut
};
static_assert(sizeof(float) * (NX * 2 * HPER + 2 * QR + 4 * D) == sizeof(float) * V, "sampled logits fill the layer temporaries");

// ---------------------------------------------------------------------------- exchanges

struct Ctx {
  const KCONST CpDesc* Dd;
  Smem* S;
  int g, r;
  uint32_t tag;
  int iring, cpar, apar, xb;
  const xtp::Xch X;
  __device__ __forceinline__ u64* intra_buf() { return X.xin + ((size_t)g * xtp::RING + (iring++ & (xtp::RING - 1))) * xtp::ISZ; }
};

// Cross reduce-scatter of the partial rows published by produce() (rows [HPER r, +HPER) of this
// rank for M input rows), plus the residual when given, then the intra all-gather of the full new
// rows: this rank's elements into xo and the sums of squares into ss of the other buffer, and
// every element, times the gain gn (the next RMSNorm's), in parts into xsp. after_put runs between
// publish and poll.
template <int M, typename Produce, typename AfterPut>
__device__ __forceinline__ bool reduce_gather(Ctx& c, bool residual, const uint16_t* gn, Produce produce, AfterPut after_put) {
  const int tid = xtp::fresh_tid();
  Smem& S = *c.S;
  ++c.tag;
  const uint32_t t = c.tag;
  u64* mine = c.X.xcr + ((size_t)(c.r * NX + c.g) * 2 + (c.cpar & 1)) * xtp::CSZ;
  produce([&](int e, int m, float v) { xtp::st_c(mine + m * 64 + e, xtp::pack(v, t)); });
  TTS_STAMP(20);
  after_put();
  TTS_STAMP(21);
  const u64* base = c.X.xcr + ((size_t)(c.r * NX) * 2 + (c.cpar & 1)) * xtp::CSZ;
  if (!xtp::get_at<(NX * M * HPER + NT - 1) / NT>(NX * M * HPER, t, S.xn, c.X.err, [&](int i) -> const u64* {
        const int sg = i >> 5, e = i & 31;  // segment (partner x, row m) = sg -> x = sg / M, m = sg % M
        return base + (size_t)(sg / M) * (2 * xtp::CSZ) + (sg % M) * 64 + e;
      }))
    return false;
  TTS_STAMP(22);
  ++c.cpar;
  ++c.tag;
  u64* buf = c.intra_buf();
  const int nb = c.xb ^ 1;
  if (tid < 64) {  // wave 0: lane 32 m + e reduces element HPER r + e of input row m
    const int m = tid >> 5, e = tid & 31;
    float v = 0.f;
    if (m < M) {
      if (residual) v = S.xo[c.xb][m][e];
#pragma unroll
      for (int x = 0; x < NX; ++x) v += S.xn[(x * M + m) * HPER + e];
      S.xo[nb][m][e] = v;
      xtp::st_l(buf + m * H + HPER * c.r + e, xtp::pack(v, c.tag));
    }
    const float s = row16_sum(v * v);
    const float sq[2] = {rl(s, 0) + rl(s, 16), rl(s, 32) + rl(s, 48)};
    if (tid < M) xtp::st_l(buf + M * H + tid * NR + c.r, xtp::pack(tid == 0 ? sq[0] : sq[1], c.tag));
  }
  c.xb = nb;
  TTS_STAMP(23);
  const bool ok = xtp::get_each<(M * (H + NR) + NT - 1) / NT>(
      M * (H + NR), c.tag, c.X.err, [&](int i) -> const u64* { return buf + i; },
      [&](int i, float v) {
        if (i < M * H)
          put_split(S.xsp, SH, i / H, i % H, v * to_f32(gn[i % H]));
        else
          S.ss[nb][i - M * H] = v;
      });
  TTS_STAMP(24);
  return ok;
}

// ---------------------------------------------------------------------------- the layer

// next layer (or the next step's first layer) whose tiles a phase issues after consuming its own
struct Next {
  int l;      // -1: none
  bool head;  // load head j's rows with the gc tiles (last layer of a step)
};

template <typename WT, int M>
__device__ __forceinline__ bool cp_layer(Ctx& c, Wl<WT>& R, int l, int j, int p0, Next nx) {
  const KCONST CpDesc& Dd = *c.Dd;
  Smem& S = *c.S;
  constexpr bool E8 = sizeof(WT) == 1;  // E4M3 rows: each row sum times its scale
  const float* sc = S.scl + l * SCL;
  const int lane = lane_id(), w = xtp::wave_id(), g = c.g, r = c.r;
  const float eps = Dd.eps;
  const uint16_t* gn_mlp = S.gn[2 * l + 1];
  const uint16_t* gn_next = l + 1 < Dd.n_layers ? S.gn[2 * (l + 1)] : S.gn[2 * MAXL];

  // --- q/k/v tile against RMSNorm(x): the parts in xsp carry the gain, the reducer the scale
  TTS_STAMP(10);
  {
    const f32x4 a = mfma_steps<M, 4>(R.q, S.xsp, SH, 4 * w, S.zero);
    if (lane < 16 * M) S.part[w][0][lane] = parts_sum(a);
  }
  xtp::lds_barrier();
  {
    ++c.tag;
    const uint32_t t = c.tag;
    u64* buf = c.intra_buf();
    if (w == 0) {
      const float sc0 = norm_scale(S.ss[c.xb], eps);
      const float sc1 = M == 2 ? norm_scale(S.ss[c.xb] + NR, eps) : 0.f;
      if (lane < 16 * M) {  // row lane % 16 of input row lane / 16, the waves' partials in wave order
        float v = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) v += S.part[ww][0][lane];
        if (E8) v *= sc[SCQ + (lane & 15)];
        xtp::st_l(buf + (lane >> 4) * QR + QPER * r + (lane & 15), xtp::pack(v * (lane < 16 ? sc0 : sc1), t));
      }
    }
    TTS_STAMP(11);
    if (!xtp::get_flat<(M * QR + NT - 1) / NT>(buf, M * QR, t, S.qkv, c.X.err)) return false;
    TTS_STAMP(13);
  }
  // the next q/k/v tiles: the waves that run no attention now, the attention waves after it
  if (nx.l >= 0 && w >= G * M) issue_q(R, Dd, nx.l, g, r);

  // --- attention of this XCD's heads over positions 0 .. p0 + M - 1: one wave per (head, row)
  if (w < G * M) {
    const int h = w / M, m = w % M, p = p0 + m;
    float (*kc)[KVS] = S.kvc[l][0];
    float (*vc)[KVS] = S.kvc[l][1];
    float qg[2], kg[2];
    unpack_pair(S.gqk[l][0], lane, qg);
    unpack_pair(S.gqk[l][1], lane, kg);
    // every attention wave appends the step's k/v rows itself (identical values), so no barrier
    // separates the append from its scores
#pragma unroll
    for (int mm = 0; mm < M; ++mm) {
      const float* kr = S.qkv + mm * QR + G * D;
      float k0 = kr[lane], k1 = kr[lane + 64];
      const float s = 1.0f / sqrtf(wave_sum(k0 * k0 + k1 * k1) / (float)D + eps);
      k0 *= s * kg[0];
      k1 *= s * kg[1];
      const float cs = S.rope[p0 + mm][0][lane], sn = S.rope[p0 + mm][1][lane];
      kc[p0 + mm][lane] = k0 * cs - k1 * sn;
      kc[p0 + mm][lane + 64] = k1 * cs + k0 * sn;
      vc[p0 + mm][lane] = kr[D + lane];
      vc[p0 + mm][lane + 64] = kr[D + lane + 64];
    }
    {
      const float* qr = S.qkv + m * QR + h * D;
      float q0 = qr[lane], q1 = qr[lane + 64];
      const float s = 1.0f / sqrtf(wave_sum(q0 * q0 + q1 * q1) / (float)D + eps);
      q0 *= s * qg[0];
      q1 *= s * qg[1];
      const float cs = S.rope[p][0][lane], sn = S.rope[p][1][lane];
      S.kq[w][lane] = q0 * cs - q1 * sn;
      S.kq[w][lane + 64] = q1 * cs + q0 * sn;
    }
    // scores: lane = 4 t + e holds position t (0..15), quarter e of the head dimension
    const int t = lane >> 2, e = lane & 3;
    float sc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 a = *reinterpret_cast<const float4*>(&S.kq[w][32 * e + 4 * i]);
      const float4 b = *reinterpret_cast<const float4*>(&kc[t][32 * e + 4 * i]);
      sc = fmaf(a.x, b.x, sc); sc = fmaf(a.y, b.y, sc); sc = fmaf(a.z, b.z, sc); sc = fmaf(a.w, b.w, sc);
    }
    sc += TTS_DPP(sc, 0xB1);  // quad_perm [1,0,3,2]
    sc += TTS_DPP(sc, 0x4E);  // quad_perm [2,3,0,1]
    sc = t <= p ? sc * (1.0f / sqrtf((float)D)) : -INFINITY;  // rows past p hold stale values
    float mx = fmaxf(sc, TTS_DPP(sc, 0x124));                  // row_ror:4
    mx = fmaxf(mx, TTS_DPP(mx, 0x128));                        // row_ror:8
    mx = fmaxf(fmaxf(rl(mx, 0), rl(mx, 16)), fmaxf(rl(mx, 32), rl(mx, 48)));
    const float wt = t <= p ? expf(sc - mx) : 0.f;
    const float ws = row16_sum(e == 0 ? wt : 0.f);
    const float ls = (rl(ws, 0) + rl(ws, 16)) + (rl(ws, 32) + rl(ws, 48));
    // all P rows in one unrolled pass, so their LDS reads go out together; rows past p (stale,
    // possibly never written) are replaced by row p, whose weight there is 0
    float o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int tt = 0; tt < P; ++tt) {
      const int tr = min(tt, p);
      const float wv = rl(wt, 4 * tt);
      o0 = fmaf(wv, vc[tr][lane], o0);
      o1 = fmaf(wv, vc[tr][lane + 64], o1);
    }
    put_split(S.osp, SO, m, h * D + lane, o0 / ls);
    put_split(S.osp, SO, m, h * D + lane + 64, o1 / ls);
    if (nx.l >= 0) issue_q(R, Dd, nx.l, g, r);
  }
  xtp::lds_barrier();
  TTS_STAMP(14);

  // --- output-projection partials of the rank's 32 rows (this XCD's head columns), residual
  {
    const f32x4 a0 = mfma_steps<M, 1>(&R.o[0], S.osp, SO, w, S.zero);
    const f32x4 a1 = mfma_steps<M, 1>(&R.o[1], S.osp, SO, w, S.zero);
    if (lane < 16 * M) {
      S.part[w][0][lane] = parts_sum(a0);
      S.part[w][1][lane] = parts_sum(a1);
    }
  }
  xtp::lds_barrier();
  if (!reduce_gather<M>(
          c, true, gn_mlp,
          [&](auto emit) {
            const int tid = xtp::fresh_tid();
            if (tid < 32 * M) {  // element e = 16 tile + i of input row m: tid = 32 m + e
              const int m = tid >> 5, e = tid & 31;
              float v = 0.f;
#pragma unroll
              for (int ww = 0; ww < NW; ++ww) v += S.part[ww][e >> 4][16 * m + (e & 15)];
              emit(e, m, E8 ? v * sc[SCO + e] : v);
            }
          },
          [&] {
            if (nx.l >= 0) issue_o(R, Dd, nx.l, g, r);
          }))
    return false;

  // --- gate/up tiles against RMSNorm(x), SwiGLU of the rank's FFN units
  {
    const f32x4 a0 = mfma_steps<M, 2>(R.gb, S.xsp, SH, 4 * w + 2, S.zero, mfma_steps<M, 2>(R.ga, S.xsp, SH, 4 * w, S.zero));
    const f32x4 a1 = mfma_steps<M, 4>(R.gc, S.xsp, SH, 4 * w, S.zero);
    if (lane < 16 * M) {
      S.part[w][0][lane] = parts_sum(a0);
      S.part[w][1][lane] = parts_sum(a1);
    }
  }
  // the gate/up registers are free: the next layer's tiles go out in two pieces, here and after
  // the SwiGLU gather
  if (nx.l >= 0 || nx.head) issue_gu1(R, Dd, nx.l >= 0 ? nx.l : l, g, r, nx.head ? j : 0);
  xtp::lds_barrier();
  {
    ++c.tag;
    const uint32_t t = c.tag;
    u64* buf = c.intra_buf();
    if (w == 0) {
      const float sc0 = norm_scale(S.ss[c.xb], eps);
      const float sc1 = M == 2 ? norm_scale(S.ss[c.xb] + NR, eps) : 0.f;
      if (lane < FPER * M) {  // FFN unit f of input row m: lane = FPER m + f
        const int m = lane / FPER, f = lane % FPER, qu = FPER + f;  // qu: its up row
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
          gs += S.part[ww][0][16 * m + f];
          us += S.part[ww][qu >> 4][16 * m + (qu & 15)];
        }
        if (E8) {
          gs *= sc[SCG + f];
          us *= sc[SCU + f];
        }
        const float sc = m == 0 ? sc0 : sc1;
        xtp::st_l(buf + m * FX + FPER * r + f, xtp::pack(silu(gs * sc) * (us * sc), t));
      }
    }
    TTS_STAMP(15);
    if (!xtp::get_each<(M * FX + NT - 1) / NT>(M * FX, t, c.X.err, [&](int i) -> const u64* { return buf + i; },
                                               [&](int i, float v) { put_split(S.hsp, SF, i / FX, i % FX, v); }))
      return false;
  }
  if (nx.l >= 0) issue_gu0<WT>(R.ga, Dd, nx.l, g, r, 0);
  if (nx.l >= 0) issue_gu0<WT>(R.gb, Dd, nx.l, g, r, 2);
  TTS_STAMP(16);

  // --- down-projection partials of the rank's 32 rows (this XCD's FFN columns), residual
  {
    const f32x4 a = mfma_steps<M, 3>(R.dn, S.hsp, SF, 3 * (w & 3), S.zero);
    if (lane < 16 * M) S.part[w][0][lane] = parts_sum(a);
  }
  xtp::lds_barrier();
  if (!reduce_gather<M>(
          c, true, gn_next,
          [&](auto emit) {
            const int tid = xtp::fresh_tid();
            if (tid < 32 * M) {  // tile e / 16 is the sum of waves 4 (e / 16) .. + 3
              const int m = tid >> 5, e = tid & 31, w0 = 4 * (e >> 4);
              float v = 0.f;
#pragma unroll
              for (int ww = 0; ww < 4; ++ww) v += S.part[w0 + ww][0][16 * m + (e & 15)];
              emit(e, m, E8 ? v * sc[SCD + e] : v);
            }
          },
          [&] {
            if (nx.l >= 0) issue_dn(R, Dd, nx.l, g, r);
          }))
    return false;
  return true;
}

// ---------------------------------------------------------------------------- the step

// Minimum of an int over the wave (DPP within 16-lane rows, then the four row results).
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
  v = min(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
  v = min(v, __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, true));  // row_ror:4
  v = min(v, __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true));  // row_ror:8
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// The best (value, id) of this workgroup's VPER logits (lanes 0..VPER-1 of wave 0 hold them),
// published to every workgroup; every wave then takes the argmax of all NWG candidates. Ties go to
// the lowest id: the maximum value first, then the lowest id among the lanes that hold it.
// Returns the id, or -1 on failure.
__device__ __forceinline__ int argmax_exchange(Ctx& c, float logit) {
  const int lane = lane_id(), w = xtp::wave_id();
  Smem& S = *c.S;
  ++c.tag;
  u64* cb = c.Dd->cand + (size_t)(c.apar & 1) * NWG * xtp::CAND;
  if (w == 0) {
    const float v = lane < VPER ? logit : -INFINITY;
    const float mx = wave_max(v);
    const int id = wave_min_i(lane < VPER && v == mx ? lane : 0x7fffffff);
    const int best = VPER * (int)blockIdx.x + (id < VPER ? id : 0);  // no lane equal: NaN logits
    if (lane < 2) xtp::st_c(cb + blockIdx.x * xtp::CAND + lane, xtp::pack(lane == 0 ? mx : __int_as_float(best), c.tag));
  }
  if (!xtp::get_at<1>(2 * NWG, c.tag, S.cand, c.X.err,
                      [&](int i) -> const u64* { return cb + (i >> 1) * xtp::CAND + (i & 1); }))
    return -1;
  ++c.apar;
  // every wave: lane l takes candidates l, l + 64, l + 128, l + 192 (ids increase with the index,
  // so a later candidate replaces an earlier one only when strictly larger)
  float v = S.cand[2 * lane];
  int id = __float_as_int(S.cand[2 * lane + 1]);
#pragma unroll
  for (int k = 1; k < NWG / 64; ++k) {
    const float v2 = S.cand[2 * (lane + 64 * k)];
    const int id2 = __float_as_int(S.cand[2 * (lane + 64 * k) + 1]);
    if (v2 > v) { v = v2; id = id2; }
  }
  const float mx = wave_max(v);
  const int best = wave_min_i(v == mx ? id : 0x7fffffff);
  return best < V ? best : 0;
}

// ---------------------------------------------------------------------------- sampled ids

constexpr int KS = 64;  // largest top_k of the in-kernel sampler: the kept ids fit one wave

// v shifted n lanes up within its row of 16 lanes (0 below the row's first lane), by DPP row_shr.
template <int N>
__device__ __forceinline__ int shr_i(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x110 + N, 0xF, 0xF, false); }
template <int N>
__device__ __forceinline__ float shr_f(float v) { return __int_as_float(shr_i<N>(__float_as_int(v))); }

// Inclusive prefix sums over the wave in lane order: within each row of 16 lanes by DPP row
// shifts, then the totals of the earlier rows added (a fixed order, the same in every wave).
__device__ __forceinline__ int wave_scan_i(int v) {
  v += shr_i<1>(v); v += shr_i<2>(v); v += shr_i<4>(v); v += shr_i<8>(v);
  const int lane = lane_id();
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31), r2 = __builtin_amdgcn_readlane(v, 47);
  return v + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}
__device__ __forceinline__ float wave_scan_f(float v) {
  v += shr_f<1>(v); v += shr_f<2>(v); v += shr_f<4>(v); v += shr_f<8>(v);
  const int lane = lane_id();
  const float r0 = rl(v, 15), r1 = rl(v, 31), r2 = rl(v, 47);
  if (lane >= 16) v += r0;
  if (lane >= 32) v += r1;
  if (lane >= 48) v += r2;
  return v;
}

// The float whose orderable key is o (the inverse of tts::orderable).
__device__ __forceinline__ float from_orderable(uint32_t o) { return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o); }

// Radix-select step, in every wave: from the histogram h of one key byte over the keys that match
// the bytes chosen so far, the byte value holding the need-th largest of them; need becomes its
// rank among the keys with that byte. Lane l reads bytes 255 - 4 l down to 252 - 4 l.
__device__ __forceinline__ uint32_t select_byte(const uint32_t* h, int& need) {
  const int lane = lane_id();
  const uint4 b = *reinterpret_cast<const uint4*>(h + 252 - 4 * lane);
  const int c[4] = {(int)b.w, (int)b.z, (int)b.y, (int)b.x};
  const int tot = c[0] + c[1] + c[2] + c[3];
  const int incl = wave_scan_i(tot), excl = incl - tot;
  const unsigned long long hit = __ballot(excl < need && need <= incl);
  const int L = hit ? __builtin_ctzll(hit) : 63;  // need never exceeds the keys counted
  int e = excl, q = 3;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    if (q == 3 && e + c[i] >= need) q = i;
    if (q == 3) e += c[i];
  }
  need -= __builtin_amdgcn_readlane(e, L);
  return (uint32_t)(255 - 4 * L - __builtin_amdgcn_readlane(q, L));
}

// Sampled id of a step from the logits of every workgroup's VPER head rows (lanes 0..VPER-1 of
// wave 0 hold this workgroup's). The acoustic sampler has no repetition penalty: the logits are
// divided by the temperature; top-k keeps the k largest in the order (logit descending, id
// ascending), found by a radix select over the orderable 32-bit keys; top-p keeps the shortest
// prefix of that order whose probability mass reaches top_p; the id is the first whose running sum
// of exp(l - l_max) exceeds u times the sum, else the last kept. Each workgroup gathers all V
// logits and every wave computes the same id from them, so no further exchange follows.
// Returns the id, or -1 on failure.
__device__ __forceinline__ int sample_exchange(Ctx& c, const CpCall& C, float logit, float u) {
  const int lane = lane_id(), w = xtp::wave_id(), tid = xtp::fresh_tid();
  Smem& S = *c.S;
  ++c.tag;
  static_assert(xtp::CAND == VPER && V == 4 * NT, "one candidate line per workgroup; four logits per thread");
  u64* cb = c.Dd->cand + (size_t)(c.apar & 1) * NWG * xtp::CAND;
  if (w == 0 && lane < VPER) xtp::st_c(cb + blockIdx.x * VPER + lane, xtp::pack(logit, c.tag));
  // histograms and the kept count start at zero (ordered before their use by the gather's barrier)
  for (int i = tid; i < 4 * 256; i += NT) (&S.bins[0][0])[i] = 0u;
  if (tid == 0) S.ncand = 0;
  const float temp = C.temperature;
  if (!xtp::get_each<V / NT>(V, c.tag, c.X.err, [&](int i) -> const u64* { return cb + i; },
                             [&](int i, float v) { S.sv[i] = v / temp; }))
    return -1;
  ++c.apar;
  TTS_STAMP(44);
  // thread t holds ids 4 t .. 4 t + 3
  const float4 x4 = *reinterpret_cast<const float4*>(&S.sv[4 * tid]);
  const uint32_t o[4] = {orderable(x4.x), orderable(x4.y), orderable(x4.z), orderable(x4.w)};
  const int k = C.top_k;
  uint32_t T = 0, mask = 0;
  int need = k;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int shift = 24 - 8 * q;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if ((o[i] & mask) == T) atomicAdd(&S.bins[q][(o[i] >> shift) & 255u], 1u);
    xtp::lds_barrier();
    T |= select_byte(S.bins[q], need) << shift;
    mask |= 0xffu << shift;
  }
  TTS_STAMP(45);
  // T: the k-th largest key; every key above it is kept, and the need lowest ids of those equal to it
  int before = 0;  // keys equal to T at lower ids than this thread's
  if (need < (int)S.bins[3][T & 255u]) {  // a tie at the cut (the same branch in every wave)
    const int e = (o[0] == T) + (o[1] == T) + (o[2] == T) + (o[3] == T);
    const int incl = wave_scan_i(e);
    if (lane == 63) S.wsum[w] = incl;
    xtp::lds_barrier();
    before = incl - e;
    for (int ww = 0; ww < w; ++ww) before += S.wsum[ww];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bool take = o[i] > T;
    if (o[i] == T) take = before++ < need;
    if (take) {
      const int slot = atomicAdd(&S.ncand, 1);
      if (slot < KS) S.ckey[slot] = ((u64)(~o[i]) << 32) | (uint32_t)(4 * tid + i);
    }
  }
  xtp::lds_barrier();
  TTS_STAMP(46);
  // every wave: the kept keys sorted ascending over its lanes (bitonic), i.e. logit descending
  u64 key = lane < k ? S.ckey[lane] : ~0ull;
#pragma unroll
  for (int kk = 2; kk <= 64; kk <<= 1) {
#pragma unroll
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)key, jj), hi = __shfl_xor((uint32_t)(key >> 32), jj);
      const u64 other = ((u64)hi << 32) | lo;
      const bool keep_min = ((lane & jj) == 0) == ((lane & kk) == 0);
      key = keep_min ? (other < key ? other : key) : (other > key ? other : key);
    }
  }
  const float v = from_orderable(~(uint32_t)(key >> 32));
  const int id = (int)(uint32_t)key;
  const float l0 = rl(v, 0);
  float wt = lane < k ? expf(v - l0) : 0.f;
  int kept = k;
  if (C.top_p < 1.0f) {
    const float tot = rl(wave_scan_f(wt), 63);
    const float cp = wave_scan_f(wt / tot);
    const unsigned long long m = __ballot(lane < k && cp >= C.top_p);
    kept = m ? __builtin_ctzll(m) + 1 : k;
    if (lane >= kept) wt = 0.f;
  }
  const float cum = wave_scan_f(wt);
  const float target = u * rl(cum, kept - 1);
  const unsigned long long hit = __ballot(lane < kept && cum > target);
  const int pick = hit ? __builtin_ctzll(hit) : kept - 1;
  const int best = __builtin_amdgcn_readlane(id, pick);
  return (unsigned)best < (unsigned)V ? best : 0;
}

// Step j's input rows: this rank's elements into xo[xb], the sums of squares into ss[xb], and the
// rows times the first layer's attention gain, in parts, into xsp. M = 2 at step 1 (h_T and
// E_sem[tok]), else E_ac[j - 1][tok]. With an input projection P, step 1 splits its K across the
// XCDs (the resident tiles pj), then a reduce-scatter + all-gather; steps 2..15 read the row
// P E_ac[j - 1][tok] of the projected table (a linear map of a table row is that row of the mapped
// table), which saves that exchange. Without a projection the rows are read as they are.
template <typename WT, int M>
__device__ __forceinline__ bool step_input(Ctx& c, const typename Frag<WT>::T (&pj)[2], int j, int tok) {
  const KCONST CpDesc& Dd = *c.Dd;
  Smem& S = *c.S;
  const int tid = xtp::fresh_tid(), lane = lane_id(), w = xtp::wave_id();
  const int Ht = Dd.Ht;
  const uint16_t* tab = j == 1 ? reinterpret_cast<const uint16_t*>(Dd.embed_sem)
                               : reinterpret_cast<const uint16_t*>(Dd.embed_ac) + (size_t)(j - 2) * V * Ht;
  const uint16_t* erow = tab + (size_t)tok * Ht;
  const uint16_t* gn0 = S.gn[0];
  // steps 2..15 with a projection: the projected codebook row P E_ac[j - 2][tok] from the table
  const float* trow = M == 1 && Dd.ptab ? Dd.ptab + ((size_t)(j - 2) * V + tok) * H : nullptr;
  if (Dd.proj && !trow) {
    // this XCD's 256 columns of each input row, in parts
    if (tid < KX) {
      const int c0 = KX * c.g + tid;
      if (M == 2) put_split(S.osp, SO, 0, tid, xtp::glb(Dd.hT)[c0]);
      put_split(S.osp, SO, M - 1, tid, to_f32(xtp::glb(erow)[c0]));
    }
    xtp::lds_barrier();
    const f32x4 a0 = mfma_steps<M, 1>(&pj[0], S.osp, SO, w, S.zero);
    const f32x4 a1 = mfma_steps<M, 1>(&pj[1], S.osp, SO, w, S.zero);
    if (lane < 16 * M) {
      S.part[w][0][lane] = parts_sum(a0);
      S.part[w][1][lane] = parts_sum(a1);
    }
    xtp::lds_barrier();
    return reduce_gather<M>(
        c, false, gn0,
        [&](auto emit) {
          if (tid < 32 * M) {
            const int m = tid >> 5, e = tid & 31;
            float v = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) v += S.part[ww][e >> 4][16 * m + (e & 15)];
            emit(e, m, sizeof(WT) == 1 ? v * S.scl[SCP + e] : v);
          }
        },
        [] {});
  }
  // no projection (Talker hidden = CodePredictor hidden), or a projected table row: the rows as
  // they are; the sums of squares in the layout an all-gather leaves them (one per wave here, the
  // other slots zero)
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float q = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = 128 * w + 64 * k + lane;
      const float x = (M == 2 && m == 0) ? xtp::glb(Dd.hT)[i] : trow ? xtp::glb(trow)[i] : to_f32(xtp::glb(erow)[i]);
      put_split(S.xsp, SH, m, i, x * to_f32(gn0[i]));
      if ((unsigned)(i - HPER * c.r) < (unsigned)HPER) S.xo[c.xb][m][i - HPER * c.r] = x;
      q = fmaf(x, x, q);
    }
    q = wave_sum(q);
    if (lane < NR / NW) S.ss[c.xb][m * NR + w + NW * lane] = lane == 0 ? q : 0.f;
  }
  xtp::lds_barrier();
  return true;
}

template <typename WT, int M>
__device__ __forceinline__ bool cp_step(Ctx& c, const CpCall& C, Wl<WT>& R, const typename Frag<WT>::T (&pj)[2], int j, int& tok,
                                        int frame) {
  const KCONST CpDesc& Dd = *c.Dd;
  Smem& S = *c.S;
  const int lane = lane_id(), w = xtp::wave_id();
  const int nl = Dd.n_layers;
  TTS_STAMP(40);
  if (!step_input<WT, M>(c, pj, j, tok)) return false;
  TTS_STAMP(41);
  const int p0 = (j == 1) ? 0 : j;
  for (int l = 0; l < nl; ++l) {
    Next nx;
    nx.l = l + 1 < nl ? l + 1 : (j < Dd.n_ac ? 0 : -1);
    nx.head = l + 1 == nl;
    if (!cp_layer<WT, M>(c, R, l, j, p0, nx)) return false;
  }
  // final RMSNorm of the last row (its parts times the final gain are in xsp), head j rows
  // VPER blockIdx + i (columns 8..15 of the gc tiles), argmax
  {
    const f32x4 a = mfma_steps<M, 4>(R.gc, S.xsp, SH, 4 * w, S.zero);
    if (lane < 16 * M) S.part[w][0][lane] = parts_sum(a);
  }
  xtp::lds_barrier();
  float logit = 0.f;
  if (w == 0) {  // lane i < VPER: head row VPER blockIdx + i (C column VPER + i) on the last input row
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) v += S.part[ww][0][16 * (M - 1) + VPER + (lane & (VPER - 1))];
    if (sizeof(WT) == 1) v *= S.scl[SCH + (j - 1) * VPER + (lane & (VPER - 1))];
    logit = v * norm_scale(S.ss[c.xb] + (M - 1) * NR, Dd.eps);
    if (C.logits && lane < VPER) xtp::glb(C.logits)[(size_t)(j - 1) * V + VPER * blockIdx.x + lane] = logit;
  }
  TTS_STAMP(42);
  const int best = C.do_sample ? sample_exchange(c, C, logit, xtp::glb(C.u)[C.u_offset + (C.use_frame ? frame * C.u_f_stride : 0) + j - 1])
                               : argmax_exchange(c, logit);
  TTS_STAMP(43);
  if (best < 0) return false;
  if (blockIdx.x == 0 && threadIdx.x == 0) xtp::glb(C.codes)[(C.use_frame ? (long)frame * C.f_stride : 0) + j - 1] = best;
  tok = C.forced ? xtp::glb(C.forced)[j - 1] : best;
  if (tok < 0) tok = 0;
  if (tok >= V) tok = V - 1;
  return true;
}

template <typename WT>
__global__ __launch_bounds__(NT) void k_cp_frame(CpCall C) {
  const KCONST CpDesc& Dd = *(const KCONST CpDesc*)C.desc;
  __shared__ Smem S;
  TTS_TRACE_BEGIN(0);
  TTS_STAMP(1);
  const int g = xtp::xcd_id(), r = blockIdx.x / NX, tid = threadIdx.x;
  Wl<WT> R;
  typename Frag<WT>::T pj[2];
  // RMSNorm gains, q/k-norm gains, the RoPE factors (and the E4M3 row scales) into LDS. Each wave
  // copies whole vectors, so the pointers it reads from the descriptor are wave-uniform (scalar
  // loads; a per-lane read of the descriptor is a vector load that waits for every load before
  // it), and every load is issued before the first store, so they are in flight together.
  {
    const int nl = Dd.n_layers, w = xtp::wave_id(), lane = lane_id();
    static_assert(H / 8 == 128 && D / 8 == 16 && P * (D / 2) == 2 * NT && SCL <= 128 && 15 * VPER <= 128 && HPER <= 64,
                  "prologue copy shapes");
    // norm gains: vector v (layer v / 2's attention or MLP gain, the final gain at v = 2 nl) on wave v % NW
    constexpr int NGV = (2 * MAXL + 1 + NW - 1) / NW;
    u32x4 gv[NGV][2];
#pragma unroll
    for (int k = 0; k < NGV; ++k) {
      const int v = w + NW * k;
      if (v <= 2 * nl) {
        const uint16_t* src = reinterpret_cast<const uint16_t*>(
            v == 2 * nl ? Dd.final_norm : (v & 1) ? Dd.layer[v >> 1].mlp_norm : Dd.layer[v >> 1].attn_norm);
        gv[k][0] = units(src)[lane];
        gv[k][1] = units(src)[lane + 64];
      }
    }
    // q/k-norm gains: vector 2 l + k (k = 1: the k-norm) on wave (2 l + k) % NW, lanes 0..15
    constexpr int NQV = (2 * MAXL + NW - 1) / NW;
    u32x4 qv[NQV];
#pragma unroll
    for (int k = 0; k < NQV; ++k) {
      const int v = w + NW * k;
      if (v < 2 * nl && lane < D / 8) {
        const uint16_t* src = reinterpret_cast<const uint16_t*>((v & 1) ? Dd.layer[v >> 1].k_norm : Dd.layer[v >> 1].q_norm);
        qv[k] = units(src)[lane];
      }
    }
    float rcs[2], rsn[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      rcs[k] = xtp::glb(Dd.rope_cos)[tid + NT * k];
      rsn[k] = xtp::glb(Dd.rope_sin)[tid + NT * k];
    }
    // E4M3 row scales of this workgroup's rows (1 where a layer or the projection is absent): wave
    // l < MAXL the layer's SCL, wave MAXL the 15 heads' VPER each, wave MAXL + 1 the projection's
    float sv2[2] = {1.f, 1.f};
    if constexpr (sizeof(WT) == 1) {
      if (w < MAXL) {
        if (w < nl) {
          const KCONST xtp::LayerS& Sc = Dd.scale[w];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int k = lane + 64 * h;
            if (k < SCO) {
              const int q0 = QPER * r + k;
              sv2[h] = q0 < G * D ? xtp::glb(Sc.wq)[G * D * g + q0]
                                  : q0 < (G + 1) * D ? xtp::glb(Sc.wk)[D * g + q0 - G * D] : xtp::glb(Sc.wv)[D * g + q0 - (G + 1) * D];
            } else if (k < SCG) {
              sv2[h] = xtp::glb(Sc.wo)[HPER * r + k - SCO];
            } else if (k < SCU) {
              sv2[h] = xtp::glb(Sc.wg)[FX * g + FPER * r + k - SCG];
            } else if (k < SCD) {
              sv2[h] = xtp::glb(Sc.wu)[FX * g + FPER * r + k - SCU];
            } else if (k < SCL) {
              sv2[h] = xtp::glb(Sc.wd)[HPER * r + k - SCD];
            }
          }
        }
      } else if (w == MAXL) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int e = lane + 64 * h;
          if (e < 15 * VPER) sv2[h] = xtp::glb(Dd.head_scale)[(size_t)(e / VPER) * V + VPER * blockIdx.x + e % VPER];
        }
      } else if (w == MAXL + 1 && Dd.proj_scale && lane < HPER) {
        sv2[0] = xtp::glb(Dd.proj_scale)[HPER * r + lane];
      }
    }
    // the stores
#pragma unroll
    for (int k = 0; k < NGV; ++k) {
      const int v = w + NW * k;
      if (v <= 2 * nl) {
        uint16_t* dst = S.gn[v == 2 * nl ? 2 * MAXL : v];
        *reinterpret_cast<u32x4*>(&dst[8 * lane]) = gv[k][0];
        *reinterpret_cast<u32x4*>(&dst[8 * (lane + 64)]) = gv[k][1];
      }
    }
#pragma unroll
    for (int k = 0; k < NQV; ++k) {
      const int v = w + NW * k;
      if (v < 2 * nl && lane < D / 8) *reinterpret_cast<u32x4*>(&S.gqk[v >> 1][v & 1][8 * lane]) = qv[k];
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = tid + NT * k;
      S.rope[i / (D / 2)][0][i % (D / 2)] = rcs[k];
      S.rope[i / (D / 2)][1][i % (D / 2)] = rsn[k];
    }
    if constexpr (sizeof(WT) == 1) {
      if (w < MAXL) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (lane + 64 * h < SCL) S.scl[w * SCL + lane + 64 * h] = sv2[h];
      } else if (w == MAXL) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (lane + 64 * h < 15 * VPER) S.scl[SCH + lane + 64 * h] = sv2[h];
      } else if (w == MAXL + 1 && lane < HPER) {
        S.scl[SCP + lane] = sv2[0];
      }
    }
    if (tid < 8) S.zero[tid] = 0;
  }
  // the first layer's weight tiles (and the resident input-projection tiles) after the small
  // loads above, which would otherwise wait behind them
  if (Dd.proj) issue_narrow<WT>(pj, Dd.proj, Dd.Ht, KX * g, r);
  issue_q(R, Dd, 0, g, r);
  issue_o(R, Dd, 0, g, r);
  issue_gu0<WT>(R.ga, Dd, 0, g, r, 0);
  issue_gu0<WT>(R.gb, Dd, 0, g, r, 2);
  issue_gu1(R, Dd, 0, g, r, 0);
  issue_dn(R, Dd, 0, g, r);
  Ctx c{&Dd, &S, g, r, xtp::glb(Dd.st)->epoch, 0, 0, 0, 0, xtp::Xch{Dd.xin, Dd.xcr, Dd.err}};
  const int frame = xtp::glb(Dd.st)->frame;
  int tok = xtp::glb(C.semantic)[0];
  if (tok < 0) tok = 0;
  if (tok >= Dd.Vs) tok = Dd.Vs - 1;
  xtp::lds_barrier();
  TTS_STAMP(2);
  bool ok = cp_step<WT, 2>(c, C, R, pj, 1, tok, frame);
  for (int j = 2; ok && j <= Dd.n_ac; ++j) ok = cp_step<WT, 1>(c, C, R, pj, j, tok, frame);
  TTS_STAMP(3);
  if (blockIdx.x == 0 && tid == 0) {
    xtp::glb(Dd.st)->epoch = c.tag + 1;  // every workgroup has read the epoch: all took part in the last exchange
    if (C.next_tok) xtp::glb(C.next_tok)[0] = tok;
  }
}

}  // namespace xcp
}  // namespace tts
