// Persistent CodePredictor frame kernel, lean form (CDNA4, gfx950; bf16 weights).
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
//   * row sums of two to four weight rows are reduced together (two cross-half lane swaps and one
//     16-lane DPP reduction instead of one full wave reduction per row);
//   * the residual rows are double buffered, so the all-gather of the new residual needs no
//     barrier behind the reduce that reads the old one;
//   * the input projection's rows (the same every step) stay in registers for the whole frame;
//   * a phase's weight rows for the next layer are issued after the first poll that follows the
//     phase (a poll waits behind the loads issued before it), a full layer ahead of their use.
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
constexpr int QPER = QR / NR;    // 16 per rank
constexpr int HPER = H / NR;     // 32 residual rows per rank
constexpr int FX = F / NX;       // 384 FFN units per XCD
constexpr int FPER = FX / NR;    // 12 per rank
constexpr int VPER = V / NWG;    // 8 head rows per workgroup, one per wave
constexpr int KX = 256;          // input-projection columns per XCD (Talker hidden 2048 / 8)
constexpr int MAXL = 5;          // CodePredictor layers supported
constexpr int P = 16;            // CodePredictor positions per frame
constexpr int KVS = 132;         // LDS row stride of the K/V rows (padded against bank conflicts)
constexpr int E = 8;             // bf16 elements per 16-byte unit
constexpr int KQ = H / E / 64;   // units per lane of a hidden-wide row: 2
constexpr int UO = G * D / E;    // units of an output-projection (or input-projection) row: 32
constexpr int UD = FX / E;       // units of a down-projection row: 48
constexpr int XW = H + NR;       // residual row plus the per-rank sums of squares

static_assert(QPER == 2 * NW && HPER == 4 * NW && 2 * FPER == 3 * NW && VPER == NW, "row split");
static_assert(UO == 32 && UD <= 64 && KX / E == UO, "unit split");

// Weight rows of one layer in registers (this workgroup's slices, bf16):
//   q   q/k/v rows 2 w, 2 w + 1 of the rank's 16; units lane, lane + 64
//   o   output projection: unit lane & 31 of rows 4 w + (lane >> 5) (o[0]) and 4 w + 2 + (lane >> 5) (o[1])
//   gu  gate/up rows 3 w .. 3 w + 2 of the rank's 24 (gate rows 0..11, then up rows 0..11)
//   dn  down projection rows 4 w .. 4 w + 3, unit lane (lanes < 48)
struct Wl {
  u32x4 q[2][KQ];
  u32x4 o[2];
  u32x4 gu[3][KQ];
  u32x4 dn[4];
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// bf16 gains of elements lane and lane + 64 of a head-dimension vector in LDS
__device__ __forceinline__ void unpack_pair(const uint16_t* gv, int lane, float (&o)[2]) {
  o[0] = to_f32(gv[lane]);
  o[1] = to_f32(gv[lane + 64]);
}

// ---------------------------------------------------------------------------- lane reductions

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
// a + b with the upper half of a exchanged for the lower half of b: lanes 0..31 hold
// a[l] + a[l + 32], lanes 32..63 hold b[l - 32] + b[l].
__device__ __forceinline__ float fold32(float a, float b) {
  const u32x2v s = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(s.x) + __uint_as_float(s.y);
}
// The same on 16-lane rows: row 0 <- a r0 + a r1, row 1 <- b r0 + b r1, row 2 <- a r2 + a r3,
// row 3 <- b r2 + b r3.
__device__ __forceinline__ float fold16(float a, float b) {
  const u32x2v s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(s.x) + __uint_as_float(s.y);
}
__device__ __forceinline__ float rl(float v, int i) { return xtp::readlane_f(v, i); }

// N (<= 4) values, each to be summed over the whole wave: on return v[i] is that sum (uniform).
template <int N>
__device__ __forceinline__ void sum_rows(float (&v)[N]) {
  static_assert(N >= 1 && N <= 4, "one to four rows");
  if constexpr (N == 1) {
    v[0] = wave_sum(v[0]);
  } else if constexpr (N == 2) {
    const float s = row16_sum(fold32(v[0], v[1]));
    v[0] = rl(s, 0) + rl(s, 16);
    v[1] = rl(s, 32) + rl(s, 48);
  } else {
    const float s = row16_sum(fold16(fold32(v[0], v[1]), fold32(v[2], N == 4 ? v[3] : 0.f)));
    v[0] = rl(s, 0);
    v[1] = rl(s, 32);
    v[2] = rl(s, 16);
    if constexpr (N == 4) v[3] = rl(s, 48);
  }
}

// ---------------------------------------------------------------------------- weight rows

template <typename T>
__device__ __forceinline__ const GLB u32x4* units(const T* p) {
  return xtp::glb(reinterpret_cast<const u32x4*>(p));
}

// q/k/v rows 2 w + i of rank r's slice of XCD g's (query heads | key | value) rows
__device__ __forceinline__ void issue_q(Wl& R, const KCONST CpDesc& Dd, int l, int g, int r) {
  const KCONST LayerW& W = Dd.layer[l];
  const int lane = lane_id(), w = xtp::wave_id();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = QPER * r + 2 * w + i;
    const uint16_t* row = q < G * D ? reinterpret_cast<const uint16_t*>(W.wq) + (size_t)(G * D * g + q) * H
                        : q < (G + 1) * D ? reinterpret_cast<const uint16_t*>(W.wk) + (size_t)(D * g + q - G * D) * H
                                          : reinterpret_cast<const uint16_t*>(W.wv) + (size_t)(D * g + q - (G + 1) * D) * H;
    const GLB u32x4* p = units(row);
#pragma unroll
    for (int k = 0; k < KQ; ++k) R.q[i][k] = p[lane + 64 * k];
  }
}
// rows [HPER r, +HPER) x columns [c0, c0 + 256) of a matrix with ld columns, in the o layout
__device__ __forceinline__ void issue_narrow(u32x4 (&o)[2], const void* m, int ld, int c0, int r) {
  const int lane = lane_id(), w = xtp::wave_id();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int row = HPER * r + 4 * w + 2 * k + (lane >> 5);
    o[k] = units(reinterpret_cast<const uint16_t*>(m) + (size_t)row * ld + c0)[lane & 31];
  }
}
__device__ __forceinline__ void issue_o(Wl& R, const KCONST CpDesc& Dd, int l, int g, int r) {
  issue_narrow(R.o, Dd.layer[l].wo, Dd.nq * D, G * D * g, r);
}
// gate/up row 3 w + i: gate rows 0..FPER-1, then up rows, of FFN units [FX g + FPER r, +FPER)
__device__ __forceinline__ void issue_gu(Wl& R, const KCONST CpDesc& Dd, int l, int g, int r) {
  const KCONST LayerW& W = Dd.layer[l];
  const int lane = lane_id(), w = xtp::wave_id();
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int q = 3 * w + i;
    const int f = FX * g + FPER * r + (q < FPER ? q : q - FPER);
    const GLB u32x4* p = units(reinterpret_cast<const uint16_t*>(q < FPER ? W.wg : W.wu) + (size_t)f * H);
#pragma unroll
    for (int k = 0; k < KQ; ++k) R.gu[i][k] = p[lane + 64 * k];
  }
}
// down rows HPER r + 4 w + i, columns of XCD g's FFN units, unit lane
__device__ __forceinline__ void issue_dn(Wl& R, const KCONST CpDesc& Dd, int l, int g, int r) {
  const int lane = lane_id(), w = xtp::wave_id();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = HPER * r + 4 * w + i;
    if (lane < UD) R.dn[i] = units(reinterpret_cast<const uint16_t*>(Dd.layer[l].wd) + (size_t)row * F + FX * g)[lane];
  }
}
// head j row VPER blockIdx + w
__device__ __forceinline__ void issue_hd(u32x4 (&hd)[1][KQ], const KCONST CpDesc& Dd, int j) {
  const int lane = lane_id(), w = xtp::wave_id();
  const GLB u32x4* p = units(reinterpret_cast<const uint16_t*>(Dd.heads) + ((size_t)(j - 1) * V + VPER * blockIdx.x + w) * H);
#pragma unroll
  for (int k = 0; k < KQ; ++k) hd[0][k] = p[lane + 64 * k];
}

// ---------------------------------------------------------------------------- row dots

// x[m][8 u .. 8 u + 8) from LDS, times the bf16 gains gn[8 u ..] when given
template <int M>
__device__ __forceinline__ void load_x(const float* x, int ldx, int u, const uint16_t* gn, float (&xv)[M][8]) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const float4 a = *reinterpret_cast<const float4*>(x + m * ldx + 8 * u);
    const float4 b = *reinterpret_cast<const float4*>(x + m * ldx + 8 * u + 4);
    xv[m][0] = a.x; xv[m][1] = a.y; xv[m][2] = a.z; xv[m][3] = a.w;
    xv[m][4] = b.x; xv[m][5] = b.y; xv[m][6] = b.z; xv[m][7] = b.w;
  }
  if (gn) {
    float gf[8];
    unpack(*reinterpret_cast<const u32x4*>(gn + 8 * u), gf, (uint16_t*)nullptr);
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[m][e] *= gf[e];
  }
}
template <int M>
__device__ __forceinline__ void fma_unit(const u32x4& w, const float (&xv)[M][8], float (&acc)[M]) {
  float wf[8];
  unpack(w, wf, (uint16_t*)nullptr);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float s = acc[m];
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(wf[e], xv[m][e], s);
    acc[m] = s;
  }
}
// R hidden-wide rows (units lane + 64 k) against M rows of x (stride ldx), gains gn (or null):
// per-lane partial sums acc[i][m].
template <int R, int M>
__device__ __forceinline__ void dot_wide(const u32x4 (&w)[R][KQ], const float* x, int ldx, const uint16_t* gn,
                                         float (&acc)[R][M]) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[i][m] = 0.f;
#pragma unroll
  for (int k = 0; k < KQ; ++k) {
    float xv[M][8];
    load_x<M>(x, ldx, lane + 64 * k, gn, xv);
#pragma unroll
    for (int i = 0; i < R; ++i) fma_unit<M>(w[i][k], xv, acc[i]);
  }
}
// The four narrow rows of the o layout against M rows of x (256 wide, stride ldx): out[i][m] is the
// sum of row 4 w + i (uniform).
template <int M>
__device__ __forceinline__ void dot_narrow(const u32x4 (&o)[2], const float* x, int ldx, float (&out)[4][M]) {
  const int lane = lane_id();
  float xv[M][8];
  load_x<M>(x, ldx, lane & 31, nullptr, xv);
  float a[2][M];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
#pragma unroll
    for (int m = 0; m < M; ++m) a[k][m] = 0.f;
    fma_unit<M>(o[k], xv, a[k]);
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    // rows: lanes 0-15 row 0, 16-31 row 2, 32-47 row 1, 48-63 row 3
    const float s = row16_sum(fold16(a[0][m], a[1][m]));
    out[0][m] = rl(s, 0);
    out[2][m] = rl(s, 16);
    out[1][m] = rl(s, 32);
    out[3][m] = rl(s, 48);
  }
}
// The four down rows against M rows of the SwiGLU slice (384 wide, stride FX).
template <int M>
__device__ __forceinline__ void dot_down(const u32x4 (&dn)[4], const float* x, float (&out)[4][M]) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) out[i][m] = 0.f;
  if (lane < UD) {
    float xv[M][8];
    load_x<M>(x, FX, lane, nullptr, xv);
#pragma unroll
    for (int i = 0; i < 4; ++i) fma_unit<M>(dn[i], xv, out[i]);
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float v[4] = {out[0][m], out[1][m], out[2][m], out[3][m]};
    sum_rows<4>(v);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i][m] = v[i];
  }
}

// 1 / sqrt(mean(x^2) + eps) of a residual row from its NR per-rank sums of squares
__device__ __forceinline__ float norm_scale(const float* ss, float eps) {
  const int lane = lane_id();
  float v = lane < NR ? ss[lane] : 0.f;
  v = row16_sum(v);
  return 1.0f / sqrtf((rl(v, 0) + rl(v, 16)) / (float)H + eps);
}

// Lane 0 stores entry idx(t) = vals[t] for t < N (wave-uniform values).
template <int N, typename Idx, typename St>
__device__ __forceinline__ void put_lanes(const float (&vals)[N], Idx idx, St store) {
  if (lane_id() == 0) {
#pragma unroll
    for (int t = 0; t < N; ++t) store(idx(t), vals[t]);
  }
}

// ---------------------------------------------------------------------------- shared memory

struct Smem {
  float xs[2][2 * XW];           // residual rows (double buffered): row m at m H, sums of squares at M H + m NR
  float xn[NX * 2 * HPER];       // reduce-scatter partials: partner x, row m at (x M + m) HPER
  float xp[2 * KX];              // input-projection input slice (row m at m KX)
  float qkv[2 * QR];             // this XCD's q/k/v rows (row m at m QR)
  float kq[4][D];                // normed, rotated q of each attention wave
  float ob[2 * G * D];           // attention output of this XCD's heads (row m at m G D)
  float gus[2 * FPER * 2];       // gate/up row sums: row q, input row m at q M + m
  float hb[2 * FX];              // SwiGLU slice of the XCD (row m at m FX)
  float cand[2 * NWG];           // argmax candidates (value, id bits)
  float red[2 * NW];
  float rope[P][2][D / 2];       // cos, sin of positions 0..15
  float kvc[MAXL][2][P][KVS];    // this frame's K/V rows of KV head g, per layer
  __align__(16) uint16_t gn[2 * MAXL + 1][H];  // RMSNorm gains: layer l attention 2 l, MLP 2 l + 1, final 2 MAXL
  __align__(16) uint16_t gqk[MAXL][2][D];      // q-norm, k-norm gains per layer
};

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
// rank for M input rows), plus the residual xs[cur] when given, then the intra all-gather of the
// full new rows into xs[cur ^ 1] (the other buffer). after_put runs between publish and poll.
template <int M, typename Produce, typename AfterPut>
__device__ __forceinline__ bool reduce_gather(Ctx& c, bool residual, Produce produce, AfterPut after_put) {
  const int tid = threadIdx.x;
  ++c.tag;
  const uint32_t t = c.tag;
  u64* mine = c.X.xcr + ((size_t)(c.r * NX + c.g) * 2 + (c.cpar & 1)) * xtp::CSZ;
  produce([&](int e, int m, float v) { xtp::st_c(mine + m * 64 + e, xtp::pack(v, t)); });
  TTS_STAMP(20);
  after_put();
  TTS_STAMP(21);
  const u64* base = c.X.xcr + ((size_t)(c.r * NX) * 2 + (c.cpar & 1)) * xtp::CSZ;
  if (!xtp::get_at<(NX * M * HPER + NT - 1) / NT>(NX * M * HPER, t, c.S->xn, c.X.err, [&](int i) -> const u64* {
        const int sg = i >> 5, e = i & 31;  // segment (partner x, row m) = sg -> x = sg / M, m = sg % M
        return base + (size_t)(sg / M) * (2 * xtp::CSZ) + (sg % M) * 64 + e;
      }))
    return false;
  TTS_STAMP(22);
  ++c.cpar;
  ++c.tag;
  u64* buf = c.intra_buf();
  const float* xs = c.S->xs[c.xb];
  if (tid < 64) {  // wave 0: lane m * 32 + e reduces row HPER r + e of input row m
    const int m = tid >> 5, e = tid & 31;
    float v = 0.f;
    if (m < M) {
      if (residual) v = xs[m * H + HPER * c.r + e];
#pragma unroll
      for (int x = 0; x < NX; ++x) v += c.S->xn[(x * M + m) * HPER + e];
      xtp::st_l(buf + m * H + HPER * c.r + e, xtp::pack(v, c.tag));
    }
    const float s = row16_sum(v * v);
    const float ss[2] = {rl(s, 0) + rl(s, 16), rl(s, 32) + rl(s, 48)};
    if (tid < M) xtp::st_l(buf + M * H + tid * NR + c.r, xtp::pack(tid == 0 ? ss[0] : ss[1], c.tag));
  }
  c.xb ^= 1;
  TTS_STAMP(23);
  const bool ok = xtp::get_flat<(2 * XW + NT - 1) / NT>(buf, M * XW, c.tag, c.S->xs[c.xb], c.X.err);
  TTS_STAMP(24);
  return ok;
}

// Intra gather of a slice: this rank's n values per input row (published by produce at row
// offset n r of a w-wide row) into dst (row m at m w) for every rank of the XCD.
template <int M, int KMAX, typename Produce>
__device__ __forceinline__ bool slice_gather(Ctx& c, int n, int w, Produce produce, float* dst) {
  ++c.tag;
  const uint32_t t = c.tag;
  u64* buf = c.intra_buf();
  produce([&](int e, int m, float v) { xtp::st_l(buf + m * w + n * c.r + e, xtp::pack(v, t)); });
  TTS_STAMP(11);
  const bool ok = xtp::get_flat<KMAX>(buf, M * w, t, dst, c.X.err);
  TTS_STAMP(13);
  return ok;
}

// ---------------------------------------------------------------------------- the layer

// next layer (or the next step's first layer) whose rows a phase issues after consuming its own
struct Next {
  int l;      // -1: none
  bool head;  // issue head j with the output-projection rows (last layer of a step)
};

template <int M>
__device__ __forceinline__ bool cp_layer(Ctx& c, Wl& R, u32x4 (&hd)[1][KQ], int l, int j, int p0, Next nx) {
  const KCONST CpDesc& Dd = *c.Dd;
  Smem& S = *c.S;
  const int lane = lane_id(), w = xtp::wave_id(), g = c.g, r = c.r;
  const float eps = Dd.eps;

  // --- q/k/v slice: rows 2 w, 2 w + 1 against RMSNorm(x), published straight from the dot
  TTS_STAMP(10);
  {
    const float* xs = S.xs[c.xb];
    float sc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) sc[m] = norm_scale(xs + M * H + m * NR, eps);
    float a[2][M];
    dot_wide<2, M>(R.q, xs, H, S.gn[2 * l], a);
    float v[2 * M];
#pragma unroll
    for (int m = 0; m < M; ++m) { v[2 * m] = a[0][m]; v[2 * m + 1] = a[1][m]; }
    sum_rows<2 * M>(v);
#pragma unroll
    for (int m = 0; m < M; ++m) { v[2 * m] *= sc[m]; v[2 * m + 1] *= sc[m]; }
    if (!slice_gather<M, (2 * QR + NT - 1) / NT>(
            c, QPER, QR,
            [&](auto emit) { put_lanes<2 * M>(v, [](int t) { return t; }, [&](int t, float x) { emit(2 * w + (t & 1), t >> 1, x); }); },
            S.qkv))
      return false;
  }
  if (nx.l >= 0) issue_q(R, Dd, nx.l, g, r);
  TTS_STAMP(12);

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
    float o0 = 0.f, o1 = 0.f;
    for (int tt = 0; tt <= p; ++tt) {
      const float wv = rl(wt, 4 * tt);
      o0 = fmaf(wv, vc[tt][lane], o0);
      o1 = fmaf(wv, vc[tt][lane + 64], o1);
    }
    S.ob[m * G * D + h * D + lane] = o0 / ls;
    S.ob[m * G * D + h * D + lane + 64] = o1 / ls;
  }
  xtp::lds_barrier();
  TTS_STAMP(14);

  // --- output projection partial of rows HPER r + 4 w + i (this XCD's head columns), residual
  {
    float o[4][M];
    dot_narrow<M>(R.o, S.ob, G * D, o);
    if (!reduce_gather<M>(
            c, true,
            [&](auto emit) {
              float v[4 * M];
#pragma unroll
              for (int m = 0; m < M; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) v[4 * m + i] = o[i][m];
              put_lanes<4 * M>(v, [](int t) { return t; }, [&](int t, float x) { emit(4 * w + (t & 3), t >> 2, x); });
            },
            [&] {
              if (nx.l >= 0) issue_o(R, Dd, nx.l, g, r);
              if (nx.head) issue_hd(hd, Dd, j);
            }))
      return false;
  }

  // --- gate/up rows 3 w + i against RMSNorm(x), SwiGLU of the rank's FFN units
  {
    const float* xs = S.xs[c.xb];
    float sc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) sc[m] = norm_scale(xs + M * H + m * NR, eps);
    float a[3][M];
    dot_wide<3, M>(R.gu, xs, H, S.gn[2 * l + 1], a);
    if constexpr (M == 1) {
      float v[3] = {a[0][0], a[1][0], a[2][0]};
      sum_rows<3>(v);
      const float vs[3] = {v[0] * sc[0], v[1] * sc[0], v[2] * sc[0]};
      put_lanes<3>(vs, [](int t) { return t; }, [&](int t, float x) { S.gus[3 * w + t] = x; });
    } else {
      float v0[4] = {a[0][0], a[0][1], a[1][0], a[1][1]};
      float v1[2] = {a[2][0], a[2][1]};
      sum_rows<4>(v0);
      sum_rows<2>(v1);
      const float vs[6] = {v0[0] * sc[0], v0[1] * sc[1], v0[2] * sc[0], v0[3] * sc[1], v1[0] * sc[0], v1[1] * sc[1]};
      put_lanes<6>(vs, [](int t) { return t; }, [&](int t, float x) { S.gus[6 * w + t] = x; });
    }
    xtp::lds_barrier();
    TTS_STAMP(15);
    if (!slice_gather<M, (2 * FX + NT - 1) / NT>(
            c, FPER, FX,
            [&](auto emit) {
              const int tid = threadIdx.x;
              if (tid < FPER * M) {
                const int f = tid % FPER, m = tid / FPER;
                emit(f, m, silu(S.gus[f * M + m]) * S.gus[(FPER + f) * M + m]);
              }
            },
            S.hb))
      return false;
  }
  if (nx.l >= 0) issue_gu(R, Dd, nx.l, g, r);
  TTS_STAMP(16);

  // --- down projection partial of rows HPER r + 4 w + i (this XCD's FFN columns), residual
  float dv[4][M];
  dot_down<M>(R.dn, S.hb, dv);
  return reduce_gather<M>(
      c, true,
      [&](auto emit) {
        float v[4 * M];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[4 * m + i] = dv[i][m];
        put_lanes<4 * M>(v, [](int t) { return t; }, [&](int t, float x) { emit(4 * w + (t & 3), t >> 2, x); });
      },
      [&] {
        if (nx.l >= 0) issue_dn(R, Dd, nx.l, g, r);
      });
}

// ---------------------------------------------------------------------------- the step

// The best (value, id) of this workgroup's VPER logits (one per wave, in S.red), published to
// every workgroup; every wave then takes the argmax of all NWG candidates (ties: the lower id).
// Returns the id, or -1 on failure.
__device__ __forceinline__ int argmax_exchange(Ctx& c, float logit) {
  const int lane = lane_id(), w = xtp::wave_id(), tid = threadIdx.x;
  Smem& S = *c.S;
  if (lane == 0) S.red[w] = logit;
  xtp::lds_barrier();
  ++c.tag;
  u64* cb = c.Dd->cand + (size_t)(c.apar & 1) * NWG * xtp::CAND;
  if (w == 0) {
    // lanes 0..7: the wave logits; the lowest index wins ties
    float v = lane < NW ? S.red[lane] : -INFINITY;
    int id = lane;
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) {
      const float v2 = __shfl_xor(v, o);
      const int id2 = __shfl_xor(id, o);
      if (v2 > v || (v2 == v && id2 < id)) { v = v2; id = id2; }
    }
    const float vals[2] = {v, __int_as_float(VPER * (int)blockIdx.x + id)};
    put_lanes<2>(vals, [](int t) { return t; },
                 [&](int t, float x) { xtp::st_c(cb + blockIdx.x * xtp::CAND + t, xtp::pack(x, c.tag)); });
  }
  if (!xtp::get_at<1>(2 * NWG, c.tag, S.cand, c.X.err,
                      [&](int i) -> const u64* { return cb + (i >> 1) * xtp::CAND + (i & 1); }))
    return -1;
  ++c.apar;
  (void)tid;
  // every wave: lane l takes candidates l, l + 64, l + 128, l + 192 (lower ids first), then the wave
  float v = S.cand[2 * lane];
  int id = __float_as_int(S.cand[2 * lane + 1]);
#pragma unroll
  for (int k = 1; k < NWG / 64; ++k) {
    const float v2 = S.cand[2 * (lane + 64 * k)];
    const int id2 = __float_as_int(S.cand[2 * (lane + 64 * k) + 1]);
    if (v2 > v) { v = v2; id = id2; }  // ids of later candidates are higher
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float v2 = __shfl_xor(v, o);
    const int id2 = __shfl_xor(id, o);
    if (v2 > v || (v2 == v && id2 < id)) { v = v2; id = id2; }
  }
  return __builtin_amdgcn_readfirstlane(id);
}

// Step j's input rows into xs[xb] (rows and per-rank sums of squares): with an input projection
// its K split across the XCDs (rows of the resident pj) and a reduce-scatter + all-gather;
// without one the rows themselves. M = 2 at step 1 (h_T and E_sem[tok]), else E_ac[j - 1][tok].
template <int M>
__device__ __forceinline__ bool step_input(Ctx& c, const u32x4 (&pj)[2], int j, int tok) {
  const KCONST CpDesc& Dd = *c.Dd;
  Smem& S = *c.S;
  const int tid = threadIdx.x, lane = lane_id(), w = xtp::wave_id();
  const int Ht = Dd.Ht;
  const uint16_t* tab = j == 1 ? reinterpret_cast<const uint16_t*>(Dd.embed_sem)
                               : reinterpret_cast<const uint16_t*>(Dd.embed_ac) + (size_t)(j - 2) * V * Ht;
  const uint16_t* erow = tab + (size_t)tok * Ht;
  if (Dd.proj) {
    // this XCD's 256 columns of each input row
    if (tid < KX / 4) {
      const int c0 = KX * c.g + 4 * tid;
      if (M == 2) {
        const u32x4 hv = *reinterpret_cast<const GLB u32x4*>(xtp::glb(Dd.hT) + c0);
        *reinterpret_cast<u32x4*>(&S.xp[4 * tid]) = hv;
      }
      const u32x2v ev = *reinterpret_cast<const GLB u32x2v*>(xtp::glb(erow) + c0);
      float* dst = &S.xp[(M - 1) * KX + 4 * tid];
      dst[0] = bf16_lo(ev.x); dst[1] = bf16_hi(ev.x); dst[2] = bf16_lo(ev.y); dst[3] = bf16_hi(ev.y);
    }
    xtp::lds_barrier();
    float o[4][M];
    dot_narrow<M>(pj, S.xp, KX, o);
    return reduce_gather<M>(
        c, false,
        [&](auto emit) {
          float v[4 * M];
#pragma unroll
          for (int m = 0; m < M; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[4 * m + i] = o[i][m];
          put_lanes<4 * M>(v, [](int t) { return t; }, [&](int t, float x) { emit(4 * w + (t & 3), t >> 2, x); });
        },
        [] {});
  }
  // no projection (Talker hidden = CodePredictor hidden): the rows as they are; the sums of
  // squares in the layout an all-gather leaves them (one per wave here, the other slots zero)
  float* xs = S.xs[c.xb];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float x0, x1;
    const int i0 = 128 * w + lane, i1 = i0 + 64;
    if (M == 2 && m == 0) {
      x0 = xtp::glb(Dd.hT)[i0];
      x1 = xtp::glb(Dd.hT)[i1];
    } else {
      x0 = to_f32(xtp::glb(erow)[i0]);
      x1 = to_f32(xtp::glb(erow)[i1]);
    }
    xs[m * H + i0] = x0;
    xs[m * H + i1] = x1;
    const float q = wave_sum(x0 * x0 + x1 * x1);
    if (lane < NR / NW) xs[M * H + m * NR + w + NW * lane] = lane == 0 ? q : 0.f;
  }
  xtp::lds_barrier();
  return true;
}

template <int M>
__device__ __forceinline__ bool cp_step(Ctx& c, const CpCall& C, Wl& R, u32x4 (&hd)[1][KQ], const u32x4 (&pj)[2], int j, int& tok,
                                        int frame) {
  const KCONST CpDesc& Dd = *c.Dd;
  Smem& S = *c.S;
  const int lane = lane_id(), w = xtp::wave_id();
  const int nl = Dd.n_layers;
  TTS_STAMP(40);
  if (!step_input<M>(c, pj, j, tok)) return false;
  TTS_STAMP(41);
  const int p0 = (j == 1) ? 0 : j;
  for (int l = 0; l < nl; ++l) {
    Next nx;
    nx.l = l + 1 < nl ? l + 1 : (j < Dd.n_ac ? 0 : -1);
    nx.head = l + 1 == nl;
    if (!cp_layer<M>(c, R, hd, l, j, p0, nx)) return false;
  }
  // final RMSNorm of the last row, head j row VPER blockIdx + w, argmax
  const float* xs = S.xs[c.xb];
  const float sc = norm_scale(xs + M * H + (M - 1) * NR, Dd.eps);
  float a[1][1];
  dot_wide<1, 1>(hd, xs + (M - 1) * H, H, S.gn[2 * MAXL], a);
  const float logit = wave_sum(a[0][0]) * sc;
  if (C.logits && lane == 0) xtp::glb(C.logits)[(size_t)(j - 1) * V + VPER * blockIdx.x + w] = logit;
  TTS_STAMP(42);
  const int best = argmax_exchange(c, logit);
  TTS_STAMP(43);
  if (best < 0) return false;
  if (blockIdx.x == 0 && threadIdx.x == 0) xtp::glb(C.codes)[(C.use_frame ? (long)frame * C.f_stride : 0) + j - 1] = best;
  tok = C.forced ? xtp::glb(C.forced)[j - 1] : best;
  if (tok < 0) tok = 0;
  if (tok >= V) tok = V - 1;
  return true;
}

__global__ __launch_bounds__(NT) void k_cp_frame(CpCall C) {
  const KCONST CpDesc& Dd = *(const KCONST CpDesc*)C.desc;
  __shared__ Smem S;
  TTS_TRACE_BEGIN(0);
  TTS_STAMP(1);
  const int g = xtp::xcd_id(), r = blockIdx.x / NX, tid = threadIdx.x;
  Wl R;
  u32x4 hd[1][KQ];
  u32x4 pj[2];
  // RMSNorm gains, q/k-norm gains and the RoPE factors into LDS
  {
    const int nl = Dd.n_layers;
    for (int i = tid; i < (2 * nl + 1) * (H / 8); i += NT) {
      const int v = i / (H / 8), u = i % (H / 8);
      const void* src = v == 2 * nl ? Dd.final_norm : (v & 1) ? Dd.layer[v >> 1].mlp_norm : Dd.layer[v >> 1].attn_norm;
      *reinterpret_cast<u32x4*>(&S.gn[v == 2 * nl ? 2 * MAXL : v][8 * u]) = units(reinterpret_cast<const uint16_t*>(src))[u];
    }
    for (int i = tid; i < nl * 2 * (D / 8); i += NT) {
      const int l = i / (2 * (D / 8)), k = (i / (D / 8)) & 1, u = i % (D / 8);
      const void* src = k ? Dd.layer[l].k_norm : Dd.layer[l].q_norm;
      *reinterpret_cast<u32x4*>(&S.gqk[l][k][8 * u]) = units(reinterpret_cast<const uint16_t*>(src))[u];
    }
    for (int i = tid; i < P * (D / 2); i += NT) {
      S.rope[i / (D / 2)][0][i % (D / 2)] = xtp::glb(Dd.rope_cos)[i];
      S.rope[i / (D / 2)][1][i % (D / 2)] = xtp::glb(Dd.rope_sin)[i];
    }
  }
  // the first layer's weight rows (and the resident input-projection rows) after the small
  // loads above, which would otherwise wait behind them
  if (Dd.proj) issue_narrow(pj, Dd.proj, Dd.Ht, KX * g, r);
  issue_q(R, Dd, 0, g, r);
  issue_o(R, Dd, 0, g, r);
  issue_gu(R, Dd, 0, g, r);
  issue_dn(R, Dd, 0, g, r);
  Ctx c{&Dd, &S, g, r, xtp::glb(Dd.st)->epoch, 0, 0, 0, 0, xtp::Xch{Dd.xin, Dd.xcr, Dd.err}};
  const int frame = xtp::glb(Dd.st)->frame;
  int tok = xtp::glb(C.semantic)[0];
  if (tok < 0) tok = 0;
  if (tok >= Dd.Vs) tok = Dd.Vs - 1;
  xtp::lds_barrier();
  TTS_STAMP(2);
  bool ok = cp_step<2>(c, C, R, hd, pj, 1, tok, frame);
  for (int j = 2; ok && j <= Dd.n_ac; ++j) ok = cp_step<1>(c, C, R, hd, pj, j, tok, frame);
  TTS_STAMP(3);
  if (blockIdx.x == 0 && tid == 0) {
    xtp::glb(Dd.st)->epoch = c.tag + 1;  // every workgroup has read the epoch: all took part in the last exchange
    if (C.next_tok) xtp::glb(C.next_tok)[0] = tok;
  }
}

}  // namespace xcp
}  // namespace tts
