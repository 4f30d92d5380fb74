// Device code of the frame decode: CDNA4 (gfx950, wave64) kernels.
//
// Ops (Qwen3-style decoder block; the block internals are a reading, the
// per-frame schedule is from "Running Qwen3-TTS on an AMD R9700", section
// "Running Qwen3-TTS"):
//   gemv      y = W x for M input rows, W bf16/fp32 [out, in] streamed once
//             with 16-byte loads per lane; optional RMSNorm prologue on x,
//             residual-add or SwiGLU epilogue; x may be gathered from an
//             embedding table by token.
//   embed_sum x = E_sem[c0] + sum_j E_ac[j][cj] (Talker input of a frame).
//   attn      decode attention over a contiguous GQA KV cache with the
//             per-head q/k RMSNorm, rotate-half RoPE and the KV append fused
//             in; positions split across blocks, merged by attn_merge.
//   sample    greedy argmax, or penalty -> temperature -> top-k -> top-p ->
//             inverse CDF at a given uniform.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tts {

constexpr int kMaxSeg = 3;

enum Epi : int { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2 };
enum Src : int { SRC_VEC = 0, SRC_TABLE = 1, SRC_VEC_THEN_TABLE = 2 };

// Decode-time counters kept on the device so that a captured frame graph can
// be replayed: pos = next Talker position to write, frame = frames since prefill.
struct DevState {
  int32_t pos;
  int32_t frame;
  uint32_t epoch;   // running exchange tag of the persistent kernels; never reset
  int32_t pad[61];
};

// Token / uniform addressing that may depend on the device frame counter:
// element(b) = base[b * b_stride + (use_frame ? frame * f_stride : 0) + offset]
struct TokRef {
  const int32_t* base;
  int32_t b_stride, f_stride, offset, use_frame;
};
struct URef {
  const float* base;
  int32_t b_stride, f_stride, offset, use_frame;
};

__device__ __forceinline__ int tok_at(const TokRef& r, const DevState* st, int b) {
  long i = (long)b * r.b_stride + r.offset + (r.use_frame ? (long)st->frame * r.f_stride : 0);
  return r.base[i];
}
// Token ids index embedding tables; ids outside [0, rows) are clamped so that a
// bad caller-supplied id cannot read outside the table.
__device__ __forceinline__ int clamp_tok(int t, int rows) { return t < 0 ? 0 : (t >= rows ? rows - 1 : t); }
__device__ __forceinline__ float u_at(const URef& r, const DevState* st, int b) {
  long i = (long)b * r.b_stride + r.offset + (r.use_frame ? (long)st->frame * r.f_stride : 0);
  return r.base[i];
}

// ---------------------------------------------------------------------------- element types

// bf16 weights are carried as their 16-bit patterns; a bf16 is the top half of an fp32.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ float to_f32(float v) { return v; }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ void store_elem(uint16_t* p, float v) { *p = f32_to_bf16(v); }
__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Matrix element types: float (fp32), uint16_t (bf16 bit patterns), uint8_t (E4M3 codes with a
// per-row fp32 scale). GT is the type of the gains and embedding tables next to them: E4M3
// matrices come with bf16 gains and tables.
template <typename WT> struct WTraits;
template <> struct WTraits<float> { static constexpr int E = 4; using GT = float; };     // elements per 16-byte lane load
template <> struct WTraits<uint16_t> { static constexpr int E = 8; using GT = uint16_t; };
template <> struct WTraits<uint8_t> { static constexpr int E = 16; using GT = uint16_t; };

// Unpack one 16-byte weight chunk into E floats.
__device__ __forceinline__ void unpack(const u32x4& w, float (&f)[8], uint16_t*) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void unpack(const u32x4& w, float (&f)[8], float*) {
  f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y); f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
}
// E4M3 (OCP) codes, byte i of the chunk -> f[i]: the CDNA4 conversion widens two bytes per
// instruction (the low or the high half of a dword), exactly.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void unpack(const u32x4& w, float (&f)[16], uint8_t*) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)d[i], false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)d[i], true);
    f[4 * i] = lo.x; f[4 * i + 1] = lo.y; f[4 * i + 2] = hi.x; f[4 * i + 3] = hi.y;
  }
}

// E consecutive elements of type T (fp32 or bf16) at p, as fp32, in 16-byte loads.
template <typename T, int E>
__device__ __forceinline__ void load_vals(const T* p, float (&f)[E]) {
  constexpr int PER = 16 / (int)sizeof(T);
  static_assert(E % PER == 0, "whole 16-byte loads");
#pragma unroll
  for (int i = 0; i < E / PER; ++i) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p + i * PER);
    float g[8];
    unpack(w, g, (T*)nullptr);
#pragma unroll
    for (int e = 0; e < PER; ++e) f[i * PER + e] = g[e];
  }
}

// ---------------------------------------------------------------------------- wave reductions (DPP)

#define TTS_DPP(v, ctrl) __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, (v)), (ctrl), 0xF, 0xF, true))

// Sum across the 16 lanes of each DPP row; every lane of the row gets the row sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += TTS_DPP(v, 0xB1);   // quad_perm [1,0,3,2]
  v += TTS_DPP(v, 0x4E);   // quad_perm [2,3,0,1]
  v += TTS_DPP(v, 0x124);  // row_ror:4
  v += TTS_DPP(v, 0x128);  // row_ror:8
  return v;
}
// Full wave64 sum, result uniform across the wave.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  int b = __builtin_bit_cast(int, v);
  float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, TTS_DPP(v, 0xB1));
  v = fmaxf(v, TTS_DPP(v, 0x4E));
  v = fmaxf(v, TTS_DPP(v, 0x124));
  v = fmaxf(v, TTS_DPP(v, 0x128));
  int b = __builtin_bit_cast(int, v);
  float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------------------- GEMV

struct GemvArgs {
  const void* w[kMaxSeg];   // segments share K; their rows are concatenated
  const float* wscale[kMaxSeg];  // E4M3 weights: per-row scales of each segment (else unused)
  int32_t seg_rows[kMaxSeg];
  int32_t nseg;
  int32_t N;                // total output rows (SwiGLU: rows per branch)
  int32_t K;
  int32_t M;                // input rows (streams x positions)
  int32_t src;              // enum Src
  const float* x;           // fp32 input rows
  int32_t x_stride;
  const void* table;        // embedding table [table_rows, K] (WTraits<WT>::GT) for gathered rows
  int32_t table_rows;
  TokRef tok;               // token of gathered row (indexed by stream)
  const void* gain;         // RMSNorm gain [K] (WTraits<WT>::GT); used by the NORM variants
  float eps;
  float* y;
  int32_t y_stride;
  const float* res;         // residual rows (EPI_RESID); may alias y
  int32_t res_stride;
  int32_t epi;              // enum Epi
  float* xn_out;            // optional: wave 0 writes the normalised input rows here
  int32_t xn_stride;
  int32_t nontemporal;      // stream the weights past the caches (read once per frame)
  int32_t ssq_out;          // EPI_RESID GEMM: also leave the new rows' chunk sums of squares
  int32_t ssq_in;           // RMSNorm GEMM whose input rows are the last ssq_out rows, unchanged
  int32_t defer_reduce;     // EPI_STORE split-K GEMM: leave the slices for the reader to add (no pass)
  int32_t bump_pos, bump_frame;  // added to the device counters by block 0 (it reads no counter)
  DevState* st;
};

// Rows each wave streams, by units per row U (a unit = one 16-byte load per lane).
template <int U, bool PAIR> struct GemvShape {
  static constexpr int RW0 = PAIR ? (8 / U) : (16 / U);
  static constexpr int RW = RW0 < 1 ? 1 : (RW0 > 4 ? 4 : RW0);
};

// E consecutive input elements of row m at element k0, as fp32.
template <typename WT, int E>
__device__ __forceinline__ void gemv_load_x(const GemvArgs& a, int m, int k0, float (&f)[E]) {
  const int stream = (a.src == SRC_VEC_THEN_TABLE) ? (m >> 1) : m;
  const bool from_table = (a.src == SRC_TABLE) || (a.src == SRC_VEC_THEN_TABLE && (m & 1));
  if (from_table) {
    using GT = typename WTraits<WT>::GT;
    const int t = clamp_tok(tok_at(a.tok, a.st, stream), a.table_rows);
    load_vals<GT, E>(reinterpret_cast<const GT*>(a.table) + (size_t)t * a.K + k0, f);
  } else {
    const float* xp = a.x + (size_t)((a.src == SRC_VEC_THEN_TABLE) ? stream : m) * a.x_stride + k0;
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(xp + e);
      f[e] = v.x; f[e + 1] = v.y; f[e + 2] = v.z; f[e + 3] = v.w;
    }
  }
}

template <typename WT>
__device__ __forceinline__ const WT* gemv_row_ptr(const GemvArgs& a, int row, const float** scale = nullptr) {
  int s = 0, off = 0;
#pragma unroll
  for (int i = 0; i < kMaxSeg - 1; ++i) {
    if (s < a.nseg - 1 && row >= off + a.seg_rows[s]) { off += a.seg_rows[s]; ++s; }
  }
  if (scale) *scale = a.wscale[s] + (row - off);
  return reinterpret_cast<const WT*>(a.w[s]) + (size_t)(row - off) * a.K;
}

// y = W x for M input rows. Every wave is independent: it loads its lanes'
// slice of each input row (and of the norm gain), then streams RW weight rows
// (PAIR: RW gate rows and RW up rows) with all loads in flight, reduces each
// row across the wave with DPP and applies the epilogue. No LDS, no barriers.
// E4M3 weights (WT = uint8_t) are widened in registers and each row's sum is
// multiplied by its scale before the epilogue.
template <typename WT, int U, int M, bool PAIR, bool NORM>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
  using GT = typename WTraits<WT>::GT;
  constexpr bool Q8 = sizeof(WT) == 1;
  constexpr int E = WTraits<WT>::E;
  constexpr int EU = E < 8 ? 8 : E;  // unpack buffer (fp32 fills 4 of 8)
  constexpr int CH = 64 * E;
  constexpr int RW = GemvShape<U, PAIR>::RW;
  constexpr int NR = PAIR ? 2 * RW : RW;
  const int lane = threadIdx.x & 63;
  const int wave_id = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int r0 = wave_id * RW;
  if (r0 >= a.N) return;

  // 1. input slices first, so that waiting for them does not queue behind the weights
  float xv[M][U][E];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int c = 0; c < U; ++c) gemv_load_x<WT, E>(a, m, c * CH + lane * E, xv[m][c]);
  float gv[NORM ? U : 1][E];
  if constexpr (NORM) {
#pragma unroll
    for (int c = 0; c < U; ++c) load_vals<GT, E>(reinterpret_cast<const GT*>(a.gain) + c * CH + lane * E, gv[c]);
  }

  // 2. every weight load of this wave (and the rows' scales)
  u32x4 wb[NR][U];
  float wsc[Q8 ? NR : 1];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    int row = r0 + (PAIR ? (r % RW) : r);
    if (row > a.N - 1) row = a.N - 1;
    const float* sp = nullptr;
    const WT* wp = PAIR ? reinterpret_cast<const WT*>(a.w[r / RW]) + (size_t)row * a.K : gemv_row_ptr<WT>(a, row, &sp);
    if constexpr (Q8) wsc[r] = PAIR ? a.wscale[r / RW][row] : *sp;
    const u32x4* p = reinterpret_cast<const u32x4*>(wp) + lane;
    if (a.nontemporal) {
#pragma unroll
      for (int c = 0; c < U; ++c) wb[r][c] = __builtin_nontemporal_load(p + c * 64);
    } else {
#pragma unroll
      for (int c = 0; c < U; ++c) wb[r][c] = p[c * 64];
    }
  }

  // 3. RMSNorm of the input rows (wave-local)
  if constexpr (NORM) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < U; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e) ss += xv[m][c][e] * xv[m][c][e];
      ss = wave_sum(ss);
      const float sc = 1.0f / sqrtf(ss / (float)a.K + a.eps);
#pragma unroll
      for (int c = 0; c < U; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e) xv[m][c][e] = xv[m][c][e] * sc * gv[c][e];
      if (a.xn_out && wave_id == 0) {
#pragma unroll
        for (int c = 0; c < U; ++c)
#pragma unroll
          for (int e = 0; e < E; ++e) a.xn_out[(size_t)m * a.xn_stride + c * CH + lane * E + e] = xv[m][c][e];
      }
    }
  }

  // 4. dot products
  float acc[NR][M];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
#pragma unroll
  for (int c = 0; c < U; ++c) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      float wf[EU];
      unpack(wb[r][c], wf, (WT*)nullptr);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float s = acc[r][m];
#pragma unroll
        for (int e = 0; e < E; ++e) s = fmaf(wf[e], xv[m][c][e], s);
        acc[r][m] = s;
      }
    }
  }

  // 5. reduce and write
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = r0 + r;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v = wave_sum(acc[r][m]);
      if constexpr (Q8) v *= wsc[r];
      if (PAIR) {
        float u = wave_sum(acc[RW + r][m]);
        if constexpr (Q8) u *= wsc[RW + r];
        v = silu(v) * u;
      }
      if (lane == 0 && row < a.N) {
        float* yp = a.y + (size_t)m * a.y_stride + row;
        if (a.epi == EPI_RESID) v += a.res[(size_t)m * a.res_stride + row];
        *yp = v;
      }
    }
  }
  if ((a.bump_pos | a.bump_frame) && wave_id == 0 && lane == 0) {
    a.st->pos += a.bump_pos;
    a.st->frame += a.bump_frame;
  }
}

// ---------------------------------------------------------------------------- embeddings

// x[b] = sum over t of table_t[tok_t(b)], summed in table order (t = 0 first).
struct EmbedArgs {
  const void* table[16];
  int32_t rows[16];
  TokRef tok[16];
  int32_t ntab;
  int32_t H;
  float* x;
  int32_t x_stride;
  const DevState* st;
  // Streaming text term ("Running Qwen3-TTS on an AMD R9700": the streaming mode feeds the text
  // one token per frame): when text.base is set, stream b adds the row E_text[id] of
  // id = text.base[b * text.b_stride + j], j = text.offset (+ frame * text.f_stride with
  // use_frame), provided j < text_n and id >= 0; otherwise nothing.
  const void* text_table;
  TokRef text;
  int32_t text_rows, text_n;
};

template <typename WT>
__global__ __launch_bounds__(256) void k_embed_sum(EmbedArgs a) {
  const int b = blockIdx.y;
  __shared__ int toks[17];
  if (threadIdx.x < a.ntab) toks[threadIdx.x] = clamp_tok(tok_at(a.tok[threadIdx.x], a.st, b), a.rows[threadIdx.x]);
  if (threadIdx.x == 16) {
    int id = -1;
    if (a.text.base) {
      const long j = a.text.offset + (a.text.use_frame ? (long)a.st->frame * a.text.f_stride : 0);
      if (j < a.text_n) id = a.text.base[(long)b * a.text.b_stride + j];
    }
    toks[16] = id < 0 ? -1 : clamp_tok(id, a.text_rows);
  }
  __syncthreads();
  const int ttok = toks[16];
  for (int k = blockIdx.x * 256 + threadIdx.x; k < a.H; k += gridDim.x * 256) {
    // every table's element loaded together (table index clamped to the last, a text row read
    // from row 0 when there is none), then summed in table order
    WT e[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int tt = min(t, a.ntab - 1);
      e[t] = reinterpret_cast<const WT*>(a.table[tt])[(size_t)toks[tt] * a.H + k];
    }
    const WT et = a.text_table ? reinterpret_cast<const WT*>(a.text_table)[(size_t)max(ttok, 0) * a.H + k] : e[0];
    float s = to_f32(e[0]);
#pragma unroll
    for (int t = 1; t < 16; ++t)
      if (t < a.ntab) s += to_f32(e[t]);
    if (ttok >= 0) s += to_f32(et);
    a.x[(size_t)b * a.x_stride + k] = s;
  }
}

// Rows m of the CodePredictor input when no projection applies:
// src VEC: x[m] <- vec row; TABLE: x[m] <- table[tok(m)]; VEC_THEN_TABLE: even m <- vec[m/2], odd m <- table[tok(m/2)].
struct GatherArgs {
  int32_t src, M, H;
  const float* vec;
  int32_t vec_stride;
  const void* table;
  int32_t table_rows;
  TokRef tok;
  float* x;
  int32_t x_stride;
  const DevState* st;
  // optional: the sums of squares of each row's 256-column chunks, ssq[m * gridDim.x + chunk] (the
  // grid then covers H with one column per thread), for the RMSNorm of the GEMM that reads x
  float* ssq;
};

template <typename WT>
__global__ __launch_bounds__(256) void k_gather(GatherArgs a) {
  const int m = blockIdx.y;
  const int stream = (a.src == SRC_VEC_THEN_TABLE) ? (m >> 1) : m;
  const bool from_table = (a.src == SRC_TABLE) || (a.src == SRC_VEC_THEN_TABLE && (m & 1));
  const int t = from_table ? clamp_tok(tok_at(a.tok, a.st, stream), a.table_rows) : 0;
  float q = 0.f;
  for (int k = blockIdx.x * 256 + threadIdx.x; k < a.H; k += gridDim.x * 256) {
    float v = from_table ? to_f32(reinterpret_cast<const WT*>(a.table)[(size_t)t * a.H + k])
                         : a.vec[(size_t)stream * a.vec_stride + k];
    a.x[(size_t)m * a.x_stride + k] = v;
    q += v * v;
  }
  if (a.ssq) {  // the same fixed order as the split-K reduction's sums of squares
    __shared__ float wsum[4];
    const float s = wave_sum(q);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) a.ssq[(size_t)m * gridDim.x + blockIdx.x] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  }
}

// ---------------------------------------------------------------------------- attention

struct AttnArgs {
  const float* qkv;         // rows (stream-major, M per stream) of [q (nq*d) | k (nkv*d) | v (nkv*d)]
  int32_t qkv_stride;
  // or, when qkv_part is set, those rows as qkv_ks split-K slices [slice][qkv_rows][qkv_n], added
  // here in slice order
  const float* qkv_part;
  int32_t qkv_ks, qkv_rows, qkv_n;
  int32_t M;                // new positions per stream
  int32_t nq, nkv, d;
  const void* q_norm;       // [d] weight dtype
  const void* k_norm;
  float eps;
  const float* rope_cos;    // [positions][d/2]
  const float* rope_sin;
  int32_t pos_const;        // position of row 0 when pos_from_state == 0
  int32_t pos_from_state;
  void* kc;                 // cache [B][nkv][cap][d] (KT)
  void* vc;
  int32_t cap;
  int32_t chunk;            // positions per split
  int32_t nsplit;
  float* out;               // nsplit == 1: [rows][nq*d]
  int32_t out_stride;
  float* part;              // nsplit > 1: [rows][nq][nsplit][d + 2] = (o[d], m, l)
  int32_t* counters;        // nsplit > 1: [B][nkv] arrival counters, zero between uses
  const DevState* st;
  const int32_t* kvstart;   // [B] first visible cache position of each stream (ragged prompts), or nullptr (0)
};

// Cache element loads of EPL contiguous elements into floats.
template <int EPL>
__device__ __forceinline__ void load_row(const uint16_t* p, float (&f)[EPL]) {
  if constexpr (EPL % 8 == 0) {
#pragma unroll
    for (int c = 0; c < EPL / 8; ++c) {
      const u32x4 w = reinterpret_cast<const u32x4*>(p)[c];
      f[8 * c + 0] = bf16_lo(w.x); f[8 * c + 1] = bf16_hi(w.x); f[8 * c + 2] = bf16_lo(w.y); f[8 * c + 3] = bf16_hi(w.y);
      f[8 * c + 4] = bf16_lo(w.z); f[8 * c + 5] = bf16_hi(w.z); f[8 * c + 6] = bf16_lo(w.w); f[8 * c + 7] = bf16_hi(w.w);
    }
  } else {
    static_assert(EPL == 4, "bf16 rows load 4 or a multiple of 8 elements");
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  }
}
template <int EPL>
__device__ __forceinline__ void load_row(const float* p, float (&f)[EPL]) {
  static_assert(EPL % 4 == 0, "fp32 rows load 4 elements per 16 bytes");
#pragma unroll
  for (int c = 0; c < EPL / 4; ++c) {
    const float4 w = reinterpret_cast<const float4*>(p)[c];
    f[4 * c + 0] = w.x; f[4 * c + 1] = w.y; f[4 * c + 2] = w.z; f[4 * c + 3] = w.w;
  }
}

// grid (nsplit, nkv, B), 256 threads. G query heads share a KV head; M new
// positions per stream; D = head_dim; each 16-lane group holds D/16
// elements per lane and walks positions s0+grp, s0+grp+16, ... of its split.
// With several splits, every block writes an unnormalised partial
// (o, max, sum) and the last block to arrive for a (stream, KV head) merges
// them (device-scope fences around an arrival counter), so no merge kernel.
// While the context fits kAttnOneSplit positions, one block per (stream, KV
// head) attends over all of it and writes the output itself: at short
// contexts the partial and merge pass cost more than the longer walk.
constexpr int kAttnOneSplit = 128;
template <typename WT, typename KT, int G, int M, int D>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
  constexpr int EPL = D / 16;
  constexpr int PL = D / 64;  // elements per lane in the norm/RoPE stage
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p0 = a.pos_from_state ? a.st->pos : a.pos_const;
  const int plast = p0 + M - 1;
  // positions per split for this launch's context (the same in every block of the grid)
  const int chunk = (a.nsplit > 1 && plast < kAttnOneSplit) ? kAttnOneSplit : a.chunk;
  const int s0 = split * chunk;
  if (s0 > plast) return;  // nothing to attend in this split; not counted by the merge
  const int s1 = min(s0 + chunk, plast + 1);
  const int used = min(a.nsplit, plast / chunk + 1);
  const int row0 = b * M;
  const int st0 = a.kvstart ? a.kvstart[b] : 0;  // positions before it are another stream's padding

  __shared__ float qs[M][G][D];
  KT* kcache = reinterpret_cast<KT*>(a.kc) + ((size_t)b * a.nkv + g) * a.cap * D;
  KT* vcache = reinterpret_cast<KT*>(a.vc) + ((size_t)b * a.nkv + g) * a.cap * D;

  // 1. per-head RMSNorm + RoPE of q and k, then k/v appended at their
  //    positions by the split that holds them. One wave per vector.
  for (int vi = wave; vi < M * (G + 2); vi += 4) {
    const int m = vi / (G + 2), j = vi % (G + 2);  // j < G: q head; G: k; G + 1: v
    const int p = p0 + m;
    const size_t col0 = (j < G) ? (size_t)(g * G + j) * D
                      : (j == G) ? (size_t)a.nq * D + (size_t)g * D : (size_t)(a.nq + a.nkv) * D + (size_t)g * D;
    float v[PL];
    if (a.qkv_part) {  // the projection's K slices, added in slice order (as the reduction pass would)
#pragma unroll
      for (int i = 0; i < PL; ++i) v[i] = 0.f;
      for (int z = 0; z < a.qkv_ks; ++z) {
        const float* sp = a.qkv_part + ((size_t)z * a.qkv_rows + row0 + m) * a.qkv_n + col0;
#pragma unroll
        for (int i = 0; i < PL; ++i) v[i] += sp[lane + 64 * i];
      }
    } else {
      const float* src = a.qkv + (size_t)(row0 + m) * a.qkv_stride + col0;
#pragma unroll
      for (int i = 0; i < PL; ++i) v[i] = src[lane + 64 * i];
    }
    if (j <= G) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < PL; ++i) ss += v[i] * v[i];
      ss = wave_sum(ss);
      const float sc = 1.0f / sqrtf(ss / (float)D + a.eps);
      const WT* gn = reinterpret_cast<const WT*>(j < G ? a.q_norm : a.k_norm);
#pragma unroll
      for (int i = 0; i < PL; ++i) v[i] = v[i] * sc * to_f32(gn[lane + 64 * i]);
      constexpr int HALF = D / 2;
      const float* cs = a.rope_cos + (size_t)p * HALF;
      const float* sn = a.rope_sin + (size_t)p * HALF;
      float r[PL];
      if constexpr (PL == 1) {
        const float other = __shfl_xor(v[0], 32);
        const int ii = lane & (HALF - 1);
        const float c = cs[ii], s = sn[ii];
        r[0] = (lane < HALF) ? (v[0] * c - other * s) : (v[0] * c + other * s);
      } else {
        constexpr int HP = PL / 2;
#pragma unroll
        for (int i = 0; i < PL; ++i) {
          const int ii = (lane + 64 * i) & (HALF - 1);
          const float c = cs[ii], s = sn[ii];
          r[i] = (i < HP) ? (v[i] * c - v[i + HP] * s) : (v[i] * c + v[i - HP] * s);
        }
      }
#pragma unroll
      for (int i = 0; i < PL; ++i) v[i] = r[i];
    }
    if (j < G) {
#pragma unroll
      for (int i = 0; i < PL; ++i) qs[m][j][lane + 64 * i] = v[i];
    } else if (p >= s0 && p < s0 + chunk) {
      KT* dst = (j == G ? kcache : vcache) + (size_t)p * D;
#pragma unroll
      for (int i = 0; i < PL; ++i) store_elem(dst + lane + 64 * i, v[i]);
    }
  }
  __syncthreads();

  // 2. online softmax over this split's positions
  const int grp = tid >> 4, gl16 = tid & 15;
  const float scale = 1.0f / sqrtf((float)D);
  float mrun[M][G], lrun[M][G], o[M][G][EPL], qv[M][G][EPL];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mrun[m][h] = -INFINITY;
      lrun[m][h] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) { o[m][h][e] = 0.f; qv[m][h][e] = qs[m][h][gl16 * EPL + e]; }
    }
  for (int t = s0 + grp; t < s1; t += 16) {
    float kf[EPL], vf[EPL];
    load_row<EPL>(kcache + (size_t)t * D + gl16 * EPL, kf);
    load_row<EPL>(vcache + (size_t)t * D + gl16 * EPL, vf);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const bool visible = t <= p0 + m && t >= st0;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) s = fmaf(qv[m][h][e], kf[e], s);
        s = row16_sum(s) * scale;
        if (visible) {
          const float mn = fmaxf(mrun[m][h], s);
          const float corr = expf(mrun[m][h] - mn);
          const float pw = expf(s - mn);
          lrun[m][h] = lrun[m][h] * corr + pw;
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[m][h][e] = o[m][h][e] * corr + pw * vf[e];
          mrun[m][h] = mn;
        }
      }
    }
  }

  // 3. combine: the 4 groups of a wave through lane exchanges (fixed order),
  //    then the 4 waves through LDS.
  __shared__ float wo[4][M][G][D];
  __shared__ float wm[4][M][G], wl[4][M][G];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m1 = fmaxf(mrun[m][h], __shfl_xor(mrun[m][h], 16));
      const float mw = fmaxf(m1, __shfl_xor(m1, 32));
      const float w = (mrun[m][h] == -INFINITY) ? 0.f : expf(mrun[m][h] - mw);
      float l = lrun[m][h] * w;
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float x = o[m][h][e] * w;
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        if (lane < 16) wo[wave][m][h][gl16 * EPL + e] = x;
      }
      if (lane == 0) { wm[wave][m][h] = mw; wl[wave][m][h] = l; }
    }
  __syncthreads();
  for (int i = tid; i < M * G * D; i += 256) {
    const int m = i / (G * D), h = (i / D) % G, e = i % D;
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) mx = fmaxf(mx, wm[q][m][h]);
    float l = 0.f, acc = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float w = (wm[q][m][h] == -INFINITY) ? 0.f : expf(wm[q][m][h] - mx);
      l += wl[q][m][h] * w;
      acc += wo[q][m][h][e] * w;
    }
    const int qh = g * G + h;
    const int row = row0 + m;
    if (used == 1) {
      a.out[(size_t)row * a.out_stride + (size_t)qh * D + e] = l > 0.f ? acc / l : 0.f;
    } else {
      float* pp = a.part + (((size_t)row * a.nq + qh) * a.nsplit + split) * (D + 2);
      pp[e] = acc;
      if (e == 0) { pp[D] = mx; pp[D + 1] = l; }
    }
  }
  if (used == 1) return;

  // 4. the last split block of this (stream, KV head) merges the partials
  __shared__ int last;
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    int* cnt = a.counters + (size_t)b * a.nkv + g;
    const int old = atomicAdd(cnt, 1);
    last = (old == used - 1);
    if (last) *cnt = 0;  // every arrival has been counted; ready for the next use
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  for (int i = tid; i < M * G * D; i += 256) {
    const int m = i / (G * D), h = (i / D) % G, e = i % D;
    const int qh = g * G + h;
    const int row = row0 + m;
    const int usedm = min(a.nsplit, (p0 + m) / chunk + 1);
    const float* pp = a.part + ((size_t)row * a.nq + qh) * a.nsplit * (D + 2);
    float mx = -INFINITY;
    for (int sp = 0; sp < usedm; ++sp) mx = fmaxf(mx, pp[sp * (D + 2) + D]);
    float l = 0.f, acc = 0.f;
    for (int sp = 0; sp < usedm; ++sp) {
      const float ms = pp[sp * (D + 2) + D];
      const float w = (ms == -INFINITY) ? 0.f : expf(ms - mx);
      l += w * pp[sp * (D + 2) + D + 1];
      acc += w * pp[sp * (D + 2) + e];
    }
    a.out[(size_t)row * a.out_stride + (size_t)qh * D + e] = l > 0.f ? acc / l : 0.f;
  }
}

// ---------------------------------------------------------------------------- sampling

struct SampleArgs {
  const float* logits;
  int32_t l_stride;
  int32_t V;
  int32_t do_sample, top_k;
  float top_p, temperature, penalty;
  URef u;
  uint8_t* history;         // [B][V] or nullptr
  int32_t h_stride;
  int32_t mark_history;
  int32_t* out;             // token (stream b at out[b * out_b_stride + frame * out_f_stride + out_offset])
  int32_t out_b_stride, out_f_stride, out_offset, out_use_frame;
  int32_t* next;            // optional: token fed to the next step (forced override)
  const int32_t* forced;    // optional [B][forced_stride]
  int32_t forced_stride, forced_offset;
  const DevState* st;
};

constexpr int kSortMax = 4096;

__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopKMax = 256;  // top_k up to this selects its candidates instead of sorting all V

// Inclusive prefix sum of v over the 256 threads of a block (ws: 4 ints of LDS). Every thread must
// call it.
__device__ __forceinline__ int block_incl_scan256(int v, int* ws) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  if (lane == 63) ws[w] = v;
  __syncthreads();
  int add = 0;
  for (int i = 0; i < w; ++i) add += ws[i];
  __syncthreads();  // ws is free again
  return v + add;
}

// Inclusive prefix sum of v over the 64 lanes of a wave, in lane order (Hillis-Steele steps).
__device__ __forceinline__ float wave_incl_sum(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// The draw from k <= 64 kept keys ((~orderable value) << 32 | id, in any order; vals[id] the
// scaled logit), by one whole wave with no block barrier: the keys sorted ascending across its
// lanes (logit descending, then id ascending) by a bitonic network on lane exchanges; top-p keeps
// the shortest prefix whose probability mass reaches top_p; the id is the first whose running sum
// of exp(l - l_max) exceeds u times the sum, else the last kept. The sums are prefix sums over the
// lanes (a fixed order). Returns the id in every lane.
__device__ __forceinline__ int draw_wave(const unsigned long long* cand, int k, const float* vals, float top_p, float u) {
  const int lane = threadIdx.x & 63;
  unsigned long long key = lane < k ? cand[lane] : ~0ull;
#pragma unroll
  for (int kk = 2; kk <= 64; kk <<= 1) {
#pragma unroll
    for (int j = kk >> 1; j > 0; j >>= 1) {
      const unsigned lo = __shfl_xor((unsigned)key, j), hi = __shfl_xor((unsigned)(key >> 32), j);
      const unsigned long long other = ((unsigned long long)hi << 32) | lo;
      const bool keep_min = ((lane & j) == 0) == ((lane & kk) == 0);
      key = keep_min ? (other < key ? other : key) : (other > key ? other : key);
    }
  }
  const int id = (int)(uint32_t)key;
  const float v = lane < k ? vals[id] : 0.f;
  const float l0 = __shfl(v, 0);
  float w = lane < k ? expf(v - l0) : 0.f;
  int kept = k;
  if (top_p < 1.0f) {
    const float tot = __shfl(wave_incl_sum(w), 63);
    const float cp = wave_incl_sum(w / tot);
    const unsigned long long m = __ballot(lane < k && cp >= top_p);
    kept = m ? __builtin_ctzll(m) + 1 : k;
    if (lane >= kept) w = 0.f;
  }
  const float cum = wave_incl_sum(w);
  const float target = u * __shfl(cum, kept - 1);
  const unsigned long long hit = __ballot(lane < kept && cum > target);
  return __shfl(id, hit ? __builtin_ctzll(hit) : kept - 1);
}

// One block (256 threads) per stream.
__global__ __launch_bounds__(256) void k_sample(SampleArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const float* l = a.logits + (size_t)b * a.l_stride;
  __shared__ float red_v[256];
  __shared__ int red_i[256];
  __shared__ int chosen;
  if (!a.do_sample) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    // up to LB logits per thread loaded together (indices clamped), then compared in id order
    constexpr int LB = 16;
    for (int i0 = tid; i0 < a.V; i0 += 256 * LB) {
      float lv[LB];
#pragma unroll
      for (int c = 0; c < LB; ++c) lv[c] = l[min(i0 + 256 * c, a.V - 1)];
#pragma unroll
      for (int c = 0; c < LB; ++c) {
        const int i = i0 + 256 * c;
        if (i < a.V && (bi == 0x7fffffff || lv[c] > bv)) { bv = lv[c]; bi = i; }
      }
    }
    red_v[tid] = bv; red_i[tid] = bi;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (tid < s) {
        const float v2 = red_v[tid + s];
        const int i2 = red_i[tid + s];
        if (v2 > red_v[tid] || (v2 == red_v[tid] && i2 < red_i[tid])) { red_v[tid] = v2; red_i[tid] = i2; }
      }
      __syncthreads();
    }
    if (tid == 0) chosen = red_i[0];
  } else {
    __shared__ unsigned long long keys[kSortMax];
    __shared__ float vals[kSortMax];
    bool drawn = false;  // the draw was made by one wave (top_k <= 64)
    const uint8_t* hist = a.history ? a.history + (size_t)b * a.h_stride : nullptr;
    if (a.top_k >= 1 && a.top_k <= kTopKMax && a.top_k <= a.V) {
      // Top-k without sorting all V: the order wanted is (logit desc, id asc), i.e. ascending
      // keys (~orderable(v) << 32 | id). A radix select over the 32-bit orderable values finds
      // the k-th largest value T; the candidates are every id above T and the lowest ids equal to
      // T up to k; only those k are sorted. Thread t handles the contiguous ids [t C, t C + C).
      __shared__ uint32_t okey[kSortMax];
      __shared__ unsigned long long cand[kTopKMax];
      __shared__ int bins[256], ws[4], sel_d, sel_need, ncand;
      const int k = a.top_k, C = (a.V + 255) / 256, i0 = tid * C, i1 = min(i0 + C, a.V);
      for (int i = i0; i < i1; ++i) {
        float v = l[i];
        if (hist && a.penalty != 1.0f && hist[i]) v = (v > 0.f) ? v / a.penalty : v * a.penalty;
        v = v / a.temperature;
        vals[i] = v;
        okey[i] = orderable(v);
      }
      uint32_t prefix = 0, pmask = 0;
      int need = k;  // how many of the values matching prefix are still to be taken
      for (int shift = 24; shift >= 0; shift -= 8) {
        bins[tid] = 0;
        __syncthreads();
        for (int i = i0; i < i1; ++i) {
          const uint32_t o = okey[i];
          if ((o & pmask) == prefix) atomicAdd(&bins[(o >> shift) & 255], 1);
        }
        __syncthreads();
        // digits from the top: thread t holds digit 255 - t; the digit whose running count first
        // reaches need holds the k-th largest value
        const int h = bins[255 - tid];
        const int incl = block_incl_scan256(h, ws);
        if (incl - h < need && need <= incl) {
          sel_d = 255 - tid;
          sel_need = need - (incl - h);
        }
        __syncthreads();
        prefix |= (uint32_t)sel_d << shift;
        pmask |= 0xffu << shift;
        need = sel_need;
        __syncthreads();
      }
      const uint32_t T = prefix;
      int eq = 0;
      for (int i = i0; i < i1; ++i) eq += okey[i] == T;
      if (tid == 0) ncand = 0;
      int rank = block_incl_scan256(eq, ws) - eq;  // ids equal to T before this thread's range
      for (int i = i0; i < i1; ++i) {
        const uint32_t o = okey[i];
        bool take = o > T;
        if (o == T) take = rank++ < need;
        if (take) cand[atomicAdd(&ncand, 1)] = ((unsigned long long)(~o) << 32) | (uint32_t)i;
      }
      __syncthreads();
      if (k <= 64) {
        // the kept keys fit one wave: it orders them and draws (no block barrier per sort stage)
        if (tid < 64) {
          const int t = draw_wave(cand, k, vals, a.top_p, u_at(a.u, a.st, b));
          if (tid == 0) chosen = t;
        }
        drawn = true;
      } else {
        int n2k = 1;
        while (n2k < k) n2k <<= 1;
        for (int i = k + tid; i < n2k; i += 256) cand[i] = ~0ull;
        __syncthreads();
        for (int kk = 2; kk <= n2k; kk <<= 1) {
          for (int j = kk >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < n2k; i += 256) {
              const int ixj = i ^ j;
              if (ixj > i) {
                const unsigned long long x = cand[i], y = cand[ixj];
                const bool up = (i & kk) == 0;
                if ((x > y) == up) { cand[i] = y; cand[ixj] = x; }
              }
            }
            __syncthreads();
          }
        }
        for (int i = tid; i < k; i += 256) keys[i] = cand[i];
        __syncthreads();
      }
    } else {
    int n2 = 1;
    while (n2 < a.V) n2 <<= 1;
    for (int i = tid; i < n2; i += 256) {
      if (i < a.V) {
        float v = l[i];
        if (hist && a.penalty != 1.0f && hist[i]) v = (v > 0.f) ? v / a.penalty : v * a.penalty;
        v = v / a.temperature;
        vals[i] = v;
        keys[i] = ((unsigned long long)(~orderable(v)) << 32) | (uint32_t)i;
      } else {
        keys[i] = ~0ull;
      }
    }
    __syncthreads();
    // bitonic sort, ascending
    for (int k = 2; k <= n2; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < n2; i += 256) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const unsigned long long x = keys[i], y = keys[ixj];
            const bool up = (i & k) == 0;
            if ((x > y) == up) { keys[i] = y; keys[ixj] = x; }
          }
        }
        __syncthreads();
      }
    }
    }
    if (tid == 0 && !drawn) {
      int kk = (a.top_k <= 0 || a.top_k > a.V) ? a.V : a.top_k;
      const float l0 = vals[(uint32_t)keys[0]];
      if (a.top_p < 1.0f) {
        float tot = 0.f;
        for (int i = 0; i < kk; ++i) tot += expf(vals[(uint32_t)keys[i]] - l0);
        float cum = 0.f;
        int m = kk - 1;
        for (int i = 0; i < kk; ++i) {
          cum += expf(vals[(uint32_t)keys[i]] - l0) / tot;
          if (cum >= a.top_p) { m = i; break; }
        }
        kk = m + 1;
      }
      float tot = 0.f;
      for (int i = 0; i < kk; ++i) tot += expf(vals[(uint32_t)keys[i]] - l0);
      const float target = u_at(a.u, a.st, b) * tot;
      int pick = kk - 1;
      float cum = 0.f;
      for (int i = 0; i < kk; ++i) {
        cum += expf(vals[(uint32_t)keys[i]] - l0);
        if (cum > target) { pick = i; break; }
      }
      chosen = (int)(uint32_t)keys[pick];
    }
  }
  __syncthreads();
  if (tid == 0) {
    const int t = chosen;
    const long fo = a.out_use_frame ? (long)a.st->frame * a.out_f_stride : 0;
    a.out[(long)b * a.out_b_stride + fo + a.out_offset] = t;
    if (a.history && a.mark_history) a.history[(size_t)b * a.h_stride + t] = 1;
    if (a.next) a.next[b] = a.forced ? a.forced[(size_t)b * a.forced_stride + a.forced_offset] : t;
  }
}

// ---------------------------------------------------------------------------- counters

__global__ void k_set_state(DevState* st, int pos, int frame) {
  if (threadIdx.x == 0 && blockIdx.x == 0) { st->pos = pos; st->frame = frame; }
}
__global__ void k_fill_u8(uint8_t* p, size_t n, uint8_t v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

// Per-stream stop on a designated semantic id (row f2 of the method's next steps; the pages leave
// the stop unfinished). Frame t of stream b, after its codes are written and consumed by the next
// Talker input: if the stream is running and its semantic token is eos, the stream stops at frame
// t (stop[b] = t) and the frame's 15 acoustic codes are masked to -1; a stream stopped at an
// earlier frame gets all 16 codes of frame t masked. The decode itself runs on in lockstep.
__global__ void k_eos_mask(int32_t* codes, int b_stride, const DevState* st, int eos, int32_t* stop, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int t = st->frame;
  int32_t* c = codes + (size_t)b * b_stride + (size_t)t * 16;
  if (stop[b] < 0) {
    if (c[0] == eos) {
      stop[b] = t;
      for (int j = 1; j < 16; ++j) c[j] = -1;
    }
  } else if (t > stop[b]) {
    for (int j = 0; j < 16; ++j) c[j] = -1;
  }
}

__global__ void k_fill_i32(int32_t* p, int n, int32_t v) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = v;
}

// Ragged prompts, right-aligned: out[b][p] = ids[b][p - start[b]] for p >= start[b], else 0 (a
// padding id whose positions every attention masks).
__global__ void k_align_ids(const int32_t* ids, int n, const int32_t* start, int B, int32_t* out) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < B * n; i += gridDim.x * blockDim.x) {
    const int b = i / n, p = i % n, s = start[b];
    out[i] = p >= s ? ids[(size_t)b * n + p - s] : 0;
  }
}

}  // namespace tts
