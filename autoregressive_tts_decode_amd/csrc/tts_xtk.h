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
//   * the weight slices are large (up to 192 KB per workgroup and phase): the q/k/v, output and
//     gate/up rows stream in chunks of at most 32 KB through two 32-register buffers of the back
//     waves, each chunk issued as soon as the one two back has been consumed, while the down rows
//     (up to 96 KB) are copied straight into LDS during the attention.
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
constexpr int TLW = 65536;                   // LDS weight rows of a workgroup (bf16 elements, 128 KB)

// One weight chunk in the back waves' registers: rows (wave - NF) + NB * j (j < RR) of the chunk,
// 16-byte units lane + 64 * k (k < KK) of each row, RR * KK <= WB.
struct WBuf {
  u32x4 b[WB];
};

template <typename WT, int RR, int KK, typename RowFn>
__device__ __forceinline__ void wb_issue(WBuf& B, int nrows, int ncols, RowFn rowptr) {
  static_assert(RR * KK <= WB, "chunk exceeds the weight buffer");
  constexpr int E = WTraits<WT>::E;
  const int lane = threadIdx.x & 63, wave = wave_id();
  if (wave < NF) return;
  const int units = ncols / E;
#pragma unroll
  for (int j = 0; j < RR; ++j) {
    const int i = (wave - NF) + NB * j;
    if (i < nrows) {
      const GLB u32x4* p = glb(reinterpret_cast<const u32x4*>(rowptr(i)));
#pragma unroll
      for (int k = 0; k < KK; ++k) {
        const int u = lane + 64 * k;
        if (u < units) B.b[j * KK + k] = p[u];
      }
    }
  }
}

// out[i] = dot(row i, x[0 .. ncols)) for this back wave's rows of the chunk (x and out in LDS).
template <typename WT, int RR, int KK>
__device__ __forceinline__ void wb_dot(const WBuf& B, int nrows, int ncols, const float* x, float* out) {
  constexpr int E = WTraits<WT>::E;
  const int lane = threadIdx.x & 63, wave = wave_id();
  if (wave < NF) return;
  const int units = ncols / E;
  float acc[RR];
#pragma unroll
  for (int j = 0; j < RR; ++j) acc[j] = 0.f;
#pragma unroll
  for (int k = 0; k < KK; ++k) {
    const int u = lane + 64 * k;
    if (u < units) {
      float xv[8];
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        const float4 f = *reinterpret_cast<const float4*>(x + u * E + e);
        xv[e] = f.x; xv[e + 1] = f.y; xv[e + 2] = f.z; xv[e + 3] = f.w;
      }
#pragma unroll
      for (int j = 0; j < RR; ++j) {
        if ((wave - NF) + NB * j < nrows) {
          float wf[8];
          unpack(B.b[j * KK + k], wf, (WT*)nullptr);
          float s = acc[j];
#pragma unroll
          for (int e = 0; e < E; ++e) s = fmaf(wf[e], xv[e], s);
          acc[j] = s;
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < RR; ++j) {
    const int i = (wave - NF) + NB * j;
    if (i < nrows) {
      const float v = wave_sum(acc[j]);
      if (lane == 0) out[i] = v;
    }
  }
}

// The weight rows of a layer, per workgroup, for H <= 2048, F / 8 <= 768, 8 KV heads of dimension
// 128 and 2 query heads per KV head. Register chunks (rows per back wave RR x 16-byte units per
// lane KK) and LDS blocks:
//   A0, A1   q/k/v slice rows [0, 8) and [8, 16) x H                          regs 2 x 4
//   C0, C1   output projection: halves of the H/32 rows x 256                  regs 8 x 1
//   DL       the first nL = min(2 F/256, TLW / H) gate/up rows (gate rows
//            first, then up rows) x H                                          LDS, during attention
//   D0, D1   the remaining gate/up rows, 8 a chunk                             regs 2 x 4
//   E        down projection: H/32 rows x F/8                                  LDS, after DL is read
// and after the last layer F0, F1, the semantic head: V/256 <= 16 rows x H, 8 a chunk -> regs 2 x 4.
template <typename WT>
__device__ __forceinline__ void tk_issue_a(WBuf& B, const KCONST TkDesc& D, const KCONST LayerW& W, int half, int g, int r) {
  const int H = D.H, d = D.d, G = D.nq / D.nkv, qper = (G + 2) * d / NR;
  wb_issue<WT, 2, 4>(B, qper / 2, H, [&](int i) -> const WT* {
    const int q = qper * r + (qper / 2) * half + i;
    if (q < G * d) return reinterpret_cast<const WT*>(W.wq) + (size_t)(G * d * g + q) * H;
    if (q < (G + 1) * d) return reinterpret_cast<const WT*>(W.wk) + (size_t)(d * g + q - G * d) * H;
    return reinterpret_cast<const WT*>(W.wv) + (size_t)(d * g + q - (G + 1) * d) * H;
  });
}
template <typename WT>
__device__ __forceinline__ void tk_issue_c(WBuf& B, const KCONST TkDesc& D, const KCONST LayerW& W, int half, int g, int r) {
  const int hper = D.H / NR, hh = hper / 2, Gd = D.nq / D.nkv * D.d;
  wb_issue<WT, 8, 1>(B, hh, Gd, [&](int i) -> const WT* {
    return reinterpret_cast<const WT*>(W.wo) + (size_t)(hper * r + hh * half + i) * (D.nq * D.d) + Gd * g;
  });
}
// gate/up row q of the rank: gate rows 0 .. fper, then up rows fper .. 2 fper
template <typename WT>
__device__ __forceinline__ const WT* tk_gu_row(const KCONST TkDesc& D, const KCONST LayerW& W, int q, int g, int r) {
  const int fx = D.F / NX, fper = fx / NR;
  const int f = fx * g + fper * r + (q < fper ? q : q - fper);
  return reinterpret_cast<const WT*>(q < fper ? W.wg : W.wu) + (size_t)f * D.H;
}
// register chunk c (8 rows) of the gate/up rows past the nl rows held in LDS
template <typename WT>
__device__ __forceinline__ void tk_issue_d(WBuf& B, const KCONST TkDesc& D, const KCONST LayerW& W, int nl, int c, int g,
                                           int r) {
  const int nd = 2 * (D.F / NX / NR);
  wb_issue<WT, 2, 4>(B, min(8, max(0, nd - nl - 8 * c)), D.H,
                     [&](int i) -> const WT* { return tk_gu_row<WT>(D, W, nl + 8 * c + i, g, r); });
}
template <typename WT>
__device__ __forceinline__ void tk_issue_f(WBuf& B, const KCONST TkDesc& D, int half) {
  const int vper = D.V / NWG;
  wb_issue<WT, 2, 4>(B, min(8, max(0, vper - 8 * half)), D.H, [&](int i) -> const WT* {
    return reinterpret_cast<const WT*>(D.lm_head) + (size_t)(vper * blockIdx.x + 8 * half + i) * D.H;
  });
}

struct TkSmem {
  float xs[THMAX + 64];       // residual row, then the per-rank sums of squares
  float xn[THMAX];            // normed row; cross-reduce partials
  float qkv[512];             // this XCD's q/k/v slice
  float q[2][128];            // normed + rotated q of the XCD's two heads
  float kp[128], vp[128];     // the step's k (normed + rotated) and v
  float wm[NF][2], wl[NF][2]; // per-wave softmax max and sum per head
  float wo[NF][2][128];       // per-wave unnormalised attention output per head
  float cmb[NR * 10];         // gathered partials of this rank's 8 outputs
  float ob[256];              // attention output of the XCD's heads
  float hb[TFXMAX];           // SwiGLU slice of the XCD
  float out[128];             // row results of this workgroup
  float red[64];
  __align__(16) uint16_t lw[TLW];  // weight rows copied by LDS-direct loads (gate/up rows, then down rows)
};

// Per-thread constants of one layer: norm gains of elements tid, tid + NT, tid + 2 NT, tid + 3 NT
// (H <= 4 NT), and for the q/k waves the q- or k-norm gains of lanes lane, lane + 64.
struct TkConsts {
  float an[4], mn[4], qk[2];
};

template <typename WT>
__device__ __forceinline__ void tk_load_consts(TkConsts& c, const KCONST TkDesc& D, const KCONST LayerW& W) {
  const WT* an = reinterpret_cast<const WT*>(W.attn_norm);
  const WT* mn = reinterpret_cast<const WT*>(W.mlp_norm);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = threadIdx.x + k * NT;
    c.an[k] = i < D.H ? to_f32(glb(an)[i]) : 0.f;
    c.mn[k] = i < D.H ? to_f32(glb(mn)[i]) : 0.f;
  }
  const int wave = wave_id(), lane = threadIdx.x & 63;
  c.qk[0] = c.qk[1] = 1.f;
  if (wave < 3) {
    const WT* gn = reinterpret_cast<const WT*>(wave < 2 ? W.q_norm : W.k_norm);
    c.qk[0] = to_f32(glb(gn)[lane]);
    c.qk[1] = to_f32(glb(gn)[lane + 64]);
  }
}

// A block of weight rows copied into LDS in parts, by the front (FRONT) or back waves, with
// LDS-direct loads: unit u of the block (row u / upr, unit u % upr of the row, upr 16-byte units
// a row) lands at dst[8 u], one instruction moving 64 consecutive units. Row i starts at
// b0 + i * stride for i < split, else at b1 + (i - split) * stride. part(n) issues at most n more
// instructions per wave: a wave that issues more than its share of the CU's memory queue holds
// stalls until the queue drains, so large copies go in parts spread over the barrier intervals of
// a layer. A copy has landed once the issuing wave's vector-memory counter has passed it.
template <typename WT, bool FRONT>
struct RowCopy {
  const WT *b0, *b1;
  long long stride;
  int split, upr, units, j;

  __device__ __forceinline__ void begin(const WT* b0_, const WT* b1_, int split_, long long stride_, int nrows, int upr_) {
    b0 = b0_;
    b1 = b1_;
    split = split_;
    stride = stride_;
    upr = upr_;
    units = nrows * upr_;
    j = FRONT ? wave_id() : wave_id() - NF;
  }
  __device__ __forceinline__ void part(uint16_t* dst, int n) {
    constexpr int E = WTraits<WT>::E;
    static_assert(E == 8, "LDS-direct rows are bf16");
    static_assert(NF == NB, "front and back wave sets of one size");
    if ((wave_id() < NF) != FRONT) return;
    const int lane = threadIdx.x & 63;
    for (int c = 0; c < n && 64 * j < units; ++c, j += NF) {
      const int u = 64 * j + lane;
      const int row = u / upr, col = u - row * upr;
      // lanes past the last unit re-read unit 0 and land in the 64-unit tail of the instruction
      const int rr = u < units ? row : 0;
      const WT* src = (rr < split ? b0 + rr * stride : b1 + (rr - split) * stride) + (u < units ? col * E : 0);
      __builtin_amdgcn_global_load_lds((const GLB void*)src, (__attribute__((address_space(3))) void*)&dst[64 * E * j], 16, 0, 0);
    }
  }
};

// Wait until every load this wave issued has landed (the LDS-direct rows included).
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0); }

// out[i] = dot(row i of w, x[0 .. ncols)) for nrows rows of ncols bf16 weights in LDS (row-major),
// all waves: wave w takes rows w, w + NW, ... (at most RM), lane the 16-byte units lane + 64 k
// (k < KK, ncols <= 512 KK). Rows go in groups of 4 so the cross-lane sums of a group overlap.
template <typename WT, int KK, int RM>
__device__ __forceinline__ void tk_dot_lds(const uint16_t* w, int nrows, int ncols, const float* x, float* out) {
  constexpr int E = WTraits<WT>::E;
  const int wave = wave_id(), lane = threadIdx.x & 63, upr = ncols / E;
  float xv[KK][8];
#pragma unroll
  for (int k = 0; k < KK; ++k) {
    const int u = lane + 64 * k;
#pragma unroll
    for (int e = 0; e < 8; e += 4) {
      const float4 f = u < upr ? *reinterpret_cast<const float4*>(x + u * E + e) : make_float4(0.f, 0.f, 0.f, 0.f);
      xv[k][e] = f.x; xv[k][e + 1] = f.y; xv[k][e + 2] = f.z; xv[k][e + 3] = f.w;
    }
  }
#pragma unroll
  for (int j0 = 0; j0 < RM; j0 += 4) {
    float acc[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int i = wave + NW * (j0 + jj);
      float s = 0.f;
      if (j0 + jj < RM && i < nrows) {
#pragma unroll
        for (int k = 0; k < KK; ++k) {
          const int u = lane + 64 * k;
          if (u < upr) {
            float wf[8];
            unpack(*reinterpret_cast<const u32x4*>(&w[(i * upr + u) * E]), wf, (WT*)nullptr);
#pragma unroll
            for (int e = 0; e < 8; ++e) s = fmaf(wf[e], xv[k][e], s);
          }
        }
      }
      acc[jj] = s;
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int i = wave + NW * (j0 + jj);
      const float v = wave_sum(acc[jj]);
      if (j0 + jj < RM && i < nrows && lane == 0) out[i] = v;
    }
  }
}

// y = x * rsqrt(mean(x^2) + eps) * gain over n <= 4 NT elements; ss: NR per-rank partial sums
// of squares (from reduce_gather) or nullptr to reduce here.
__device__ __forceinline__ void tk_rmsnorm(const float* x, int n, const float* gr, float eps, float* y, float* red,
                                           const float* ss) {
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
    if (i < n) y[i] = x[i] * sc * gr[k];
  }
  lds_barrier();
}

// Attention of this XCD's two query heads over positions 0..p of KV head g, this rank's chunk of
// positions, then the two combining exchanges; the XCD's 256 outputs land in S.ob. Only the front
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
    v0 *= sc * cn.qk[0];
    v1 *= sc * cn.qk[1];
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
      // outputs: lane owns dimensions lane, lane + 64 of both heads
      for (int tt = 0; tt < npass; ++tt) {
        const int tp = base + tt;
        const float w0 = readlane_f(w[0], 4 * tt), w1 = readlane_f(w[1], 4 * tt);
        float v0, v1;
        if (tp == p) { v0 = S.vp[lane]; v1 = S.vp[lane + 64]; }
        else { v0 = glb(vg)[(size_t)tp * d + lane]; v1 = glb(vg)[(size_t)tp * d + lane + 64]; }
        o[0][0] = fmaf(w0, v0, o[0][0]); o[0][1] = fmaf(w0, v1, o[0][1]);
        o[1][0] = fmaf(w1, v0, o[1][0]); o[1][1] = fmaf(w1, v1, o[1][1]);
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
  if (!slice_gather<1, 1, PF>(X, 8, 256, [&](int k, int) {
        float mx = -INFINITY;
        for (int s2 = 0; s2 < NR; ++s2) mx = fmaxf(mx, S.cmb[s2 * 10]);
        float ls = 0.f, os = 0.f;
        for (int s2 = 0; s2 < NR; ++s2) {
          const float ms = S.cmb[s2 * 10];
          const float f = ms == -INFINITY ? 0.f : expf(ms - mx);
          ls += S.cmb[s2 * 10 + 1] * f;
          os += S.cmb[s2 * 10 + 2 + k] * f;
        }
        return os / ls;
      }, S.ob, tag, iring, g, r, [&] { if (wave >= NF) bg(3); }))
    return false;
  return true;
}

// The constants the layer after l needs (the final-norm gains in c.an after the last layer).
template <typename WT>
__device__ __forceinline__ void tk_next_consts(TkConsts& c, const KCONST TkDesc& D, int l, int tid) {
  if (l + 1 < D.n_layers) {
    tk_load_consts<WT>(c, D, D.layer[l + 1]);
  } else {
    const WT* f = reinterpret_cast<const WT*>(D.final_norm);
#pragma unroll
    for (int k = 0; k < 4; ++k) c.an[k] = tid + k * NT < D.H ? to_f32(glb(f)[tid + k * NT]) : 0.f;
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
  TkConsts c;
  tk_load_consts<WT>(c, D, D.layer[0]);
  const int qh = qper / 2, hh = hper / 2, nd = 2 * fper;  // rows of A0/A1, C0/C1; gate + up rows
  const int nl = min(min(nd, TLW / H), 4 * NW);            // gate/up rows held in LDS (4 per wave)
  // The LDS gate/up block of a layer goes in parts (instructions per back wave, 32 for the largest
  // block): 4 while the previous layer's down exchange runs, 4 after the q/k/v rows, 6 during the
  // q/k/v exchange, 4 + 6 + 4 in the attention and the rest during its last exchange.
  RowCopy<WT, false> gu;
  auto gu_begin = [&](const KCONST LayerW& W) {
    gu.begin(tk_gu_row<WT>(D, W, 0, g, r), tk_gu_row<WT>(D, W, fper, g, r), fper, H, nl, H / 8);
  };
  RowCopy<WT, true> dn;  // the down rows, by the front waves, in two parts
  WBuf X0, X1;
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
  for (int i = tid; i < H; i += NT) S.xs[i] = glb(D.x_in)[i];
  lds_barrier();
  bool ok = true;
  for (int l = 0; ok && l < D.n_layers; ++l) {
    const KCONST LayerW& W = D.layer[l];
    const bool last = l + 1 == D.n_layers;
    TTS_STAMP(50);
    // q/k/v slice (A0: X0, A1: X1); the output projection rows (C0, C1) follow in their place
    tk_rmsnorm(S.xs, H, c.an, D.eps, S.xn, S.red, l > 0 ? S.xs + H : nullptr);
    wb_dot<WT, 2, 4>(X0, qh, H, S.xn, S.out);
    tk_issue_c<WT>(X0, D, W, 0, g, r);
    wb_dot<WT, 2, 4>(X1, qh, H, S.xn, S.out + qh);
    tk_issue_c<WT>(X1, D, W, 1, g, r);
    gu.part(S.lw, 4);
    lds_barrier();
    TTS_STAMP(51);
    if (!slice_gather<1, KQ, PF>(X, qper, qrows, [&](int e, int) { return S.out[e]; }, S.qkv, tag, iring, g, r,
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
    // output projection partial (C0: X0, C1: X1), residual; the register gate/up chunks follow
    // (D0 now, D1 during the exchange)
    wb_dot<WT, 8, 1>(X0, hh, G * d, S.ob, S.out);
    tk_issue_d<WT>(X0, D, W, nl, 0, g, r);
    wb_dot<WT, 8, 1>(X1, hh, G * d, S.ob, S.out + hh);
    lds_barrier();
    TTS_STAMP(58);
    if (!reduce_gather<1, THMAX, KT, PF>(X, S.out, S.xs, S.xn, H, true, tag, iring, cpar, g, r,
                                         [&] { tk_issue_d<WT>(X1, D, W, nl, 1, g, r); })) {
      ok = false;
      break;
    }
    TTS_STAMP(59);
    // gate and up rows (LDS block, then D0: X0, D1: X1), SwiGLU. Once the LDS block is read the
    // front waves copy the down rows in its place (half now, half during the SwiGLU exchange)
    // and the back waves, their registers free, start on the next layer's q/k/v rows (or the
    // semantic head). Each wave loads its own next-layer constants behind its other loads.
    tk_rmsnorm(S.xs, H, c.mn, D.eps, S.xn, S.red, S.xs + H);
    if (wave >= NF) wait_loads();
    lds_barrier();
    tk_dot_lds<WT, 4, 4>(S.lw, nl, H, S.xn, S.out);
    lds_barrier();
    TTS_STAMP(60);
    const int dparts = (hper * (fx / 8) / 64 + 2 * NF - 1) / (2 * NF);  // first half, per front wave
    if (wave < NF) {
      dn.begin(reinterpret_cast<const WT*>(W.wd) + (size_t)(hper * r) * D.F + fx * g, nullptr, hper, D.F, hper, fx / 8);
      dn.part(S.lw, dparts);
      tk_next_consts<WT>(c, D, l, tid);
    } else {
      wb_dot<WT, 2, 4>(X0, min(8, max(0, nd - nl)), H, S.xn, S.out + nl);
      if (!last) tk_issue_a<WT>(X0, D, D.layer[l + 1], 0, g, r);
      else tk_issue_f<WT>(X0, D, 0);
      wb_dot<WT, 2, 4>(X1, min(8, max(0, nd - nl - 8)), H, S.xn, S.out + nl + 8);
      tk_next_consts<WT>(c, D, l, tid);
    }
    lds_barrier();
    TTS_STAMP(61);
    if (!slice_gather<1, KH, PF>(X, fper, fx, [&](int e, int) { return silu(S.out[e]) * S.out[fper + e]; }, S.hb, tag,
                                 iring, g, r, [&] {
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
    // down projection partial from LDS, residual; the next layer's LDS gate/up block starts
    // during the exchange
    TTS_STAMP(62);
    if (wave < NF) wait_loads();
    lds_barrier();
    tk_dot_lds<WT, 2, 8>(S.lw, hper, fx, S.hb, S.out);
    lds_barrier();
    TTS_STAMP(63);
    if (!reduce_gather<1, THMAX, KT, PF>(X, S.out, S.xs, S.xn, H, true, tag, iring, cpar, g, r, [&] {
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
    // final norm (gains in c.an), semantic head slice (F0: X0, F1: X1)
    tk_rmsnorm(S.xs, H, c.an, D.eps, S.xn, S.red, S.xs + H);
    const int vper = D.V / NWG;
    wb_dot<WT, 2, 4>(X0, min(8, vper), H, S.xn, S.out);
    wb_dot<WT, 2, 4>(X1, max(0, vper - 8), H, S.xn, S.out + 8);
    lds_barrier();
    for (int i = tid; i < vper; i += NT) glb(D.logits)[vper * blockIdx.x + i] = S.out[i];
    if (blockIdx.x == 0)
      for (int i = tid; i < H; i += NT) glb(D.hT)[i] = S.xn[i];
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
