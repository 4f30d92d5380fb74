// Persistent, XCD-tensor-parallel CodePredictor frame kernel (CDNA4, gfx950).
//
// The 15 sequential CodePredictor steps of a frame ("Running Qwen3-TTS on an
// AMD R9700", section "Running Qwen3-TTS") run inside ONE kernel of 256
// workgroups x 512 threads -- one workgroup per CU, rank r on XCD g where
// g is the XCD the workgroup runs on (its XCC_ID) and r = blockIdx / 8. Each
// decoder layer is split across
// the 8 XCDs tensor-parallel: XCD g owns KV head g (query heads G*g ..
// G*g+G-1), the matching columns of the output projection and 1/8 of the
// FFN. Dependencies between phases are exchanges of tagged fp32 values
// ((tag << 32) | bits, read with device-scope relaxed atomic loads, so no
// cache maintenance or fences are needed):
//   intra: the 32 ranks of one XCD gather each other's slices
//          (q/k/v slice -> attention; reduced residual -> full residual;
//           SwiGLU slice -> down projection);
//   cross: rank r of every XCD reduce-scatters the partial sums of the output
//          and down projections (8 partners, rank-r rows).
// Cross values are written with device-scope stores, which write through to
// memory. Intra values are written with plain stores, which stay in the XCD's
// L2 as dirty lines; a device-scope load from a CU of the same XCD is served
// by that line (measured: an all-gather hop among the 32 ranks of an XCD takes
// ~0.35 us this way against ~0.95 us through memory). The group of a
// workgroup is therefore the XCD it runs on, read from the hardware, not a
// function of blockIdx: the dispatcher deals workgroups to the XCDs round
// robin, but from an XCD that depends on earlier launches. Round robin puts
// the 32 workgroups blockIdx = 8 k + c (k < 32) on one XCD, so r = blockIdx / 8
// numbers them 0..31. Were the deal ever uneven, a (g, r) slot would go
// unwritten and its readers time out; a tag never matches a stale value, so
// the failure is a time-out reported in the error word, never a wrong value.
// A consumer polls until every value it needs carries the expected tag; tags
// are unique per exchange (a running epoch kept on the device), and every
// exchange buffer is reused only after an exchange that all its readers must
// have passed, so a value is never overwritten while it may still be read.
// Each phase's weight loads are issued before it waits for its input, at a point where no poll
// follows within about a microsecond (a poll waits behind the loads its wave issued before it).
#pragma once

#include "tts_device.h"

namespace tts {
namespace xtp {

constexpr int NX = 8;       // XCDs
constexpr int NR = 32;      // ranks per XCD
constexpr int NWG = NX * NR;
constexpr int NT = 512;     // threads per workgroup
constexpr int NW = NT / 64; // waves per workgroup
constexpr int MAXL = 6;     // CodePredictor layers supported (K/V rows live in LDS)
constexpr int kCpPos = 16;  // CodePredictor positions per frame
constexpr int HMAX = 1024;  // CodePredictor hidden size supported
constexpr int KVS = 132;    // LDS row stride of the K/V rows (padded against bank conflicts)
// Weight-row register buffers, per wave: A holds hidden-wide rows (q/k/v, the first RA_R * NW
// gate/up rows, head: at most RA_R rows per wave of at most 64 * RA_K 16-byte units), C the
// gate/up rows past those (RC_R rows per wave), B narrow rows (output and down projections, input
// projection: RB_R rows of at most 64 * RB_K units). A wave holds its loads' issue once it has
// more than about 4 KB in flight (measured), so no exchange issues more than 4 KB per wave: the
// gate/up rows are split between A (issued right after the q/k/v exchange) and C (issued with the
// attention, when most waves are idle and the next poll is an attention and a dot away). The next layer's q/k/v rows go into A
// between the two gate/up dots.
constexpr int RA_R = 2, RA_K = 2;
constexpr int RC_R = 1;
constexpr int RB_R = 4, RB_K = 1;
constexpr int RING = 4;     // intra exchange buffers per XCD
constexpr int ISZ = 2 * HMAX + 128;  // intra buffer entries (2 rows x HMAX, sums of squares)
constexpr int CSZ = 2 * 64;    // cross slot entries (2 rows x 64)
constexpr int CAND = 8;        // candidate slot entries (one 64-byte line)
constexpr long long kSpin = 4000000;

typedef unsigned long long u64;

struct LayerW {
  const void *attn_norm, *wq, *wk, *wv, *q_norm, *k_norm, *wo, *mlp_norm, *wg, *wu, *wd;
};

// Exchange buffers (shared by the persistent kernels of a context, which never run concurrently:
// their tags come from one running counter) and the error word.
struct Xch {
  unsigned long long *xin, *xcr;
  uint32_t* err;
};

// Everything the kernel reads; built on the host once per weight binding and
// kept in device memory.
// Per-row fp32 scales of E4M3 matrices (null for bf16 weights): row i of a matrix is
// scale[i] * codes[i].
struct LayerS {
  const float *wq, *wk, *wv, *wo, *wg, *wu, *wd;
};

struct CpDesc {
  LayerW layer[MAXL];
  LayerS scale[MAXL];
  const float *head_scale, *proj_scale;  // [15 * V], [H]
  int32_t n_layers, H, Ht, F, V, Vs, nq, nkv, d, n_ac;
  float eps;
  const void *final_norm, *heads, *proj, *embed_ac, *embed_sem;
  const float* ptab;                 // [n_ac][V][H] projected codebook rows P E_ac[j][a], or null
  const float *rope_cos, *rope_sin;  // [16][d/2]
  const float* hT;                   // [Ht] pending Talker hidden (final-normed)
  u64 *xin, *xcr, *cand;
  DevState* st;
  uint32_t* err;                     // nonzero after a failed exchange (time-out)
};

// Per-launch arguments (pointers may differ between calls).
struct CpCall {
  const CpDesc* desc;
  const int32_t* semantic;  // [1]: the frame's semantic id
  const int32_t* forced;    // [15] or nullptr
  int32_t* codes;           // acoustic ids land at codes[(use_frame ? frame * f_stride : 0) + j - 1]
  int32_t f_stride, use_frame;
  float* logits;            // [15][V] or nullptr
  int32_t* next_tok;        // optional: last token fed forward (unused by the frame loop)
  // sampled acoustic ids (the hidden-1024 CodePredictor kernel only; 0 = greedy): top_k in
  // 1..64, top_p, temperature; step j draws at u[u_offset + (use_frame ? frame * u_f_stride : 0) + j - 1]
  int32_t do_sample, top_k;
  float top_p, temperature;
  const float* u;
  int32_t u_f_stride, u_offset;
};

// Wave index as a wave-uniform (scalar) value, so row addresses derived from it stay scalar.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
// threadIdx.x behind an empty asm statement: what is computed from it is recomputed where it is
// used instead of being hoisted out of the layer loop (hoisted per-thread offsets of every
// exchange would stay live in registers across the whole loop).
__device__ __forceinline__ int fresh_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Lane i's value, read into a scalar register (wave-uniform).
__device__ __forceinline__ float readlane_f(float v, int i) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), i));
}

__device__ __forceinline__ u64 pack(float v, uint32_t tag) { return ((u64)tag << 32) | __float_as_uint(v); }
__device__ __forceinline__ uint32_t tagof(u64 v) { return (uint32_t)(v >> 32); }
__device__ __forceinline__ float valof(u64 v) { return __uint_as_float((uint32_t)v); }
// Every pointer the kernel follows comes out of the descriptor in device memory, so the compiler
// cannot tell it is global and would emit flat instructions, which also count against the LDS
// counter: each LDS wait before a barrier would then wait for all weight rows in flight. All
// global accesses therefore go through explicitly global (address space 1) pointers.
#define GLB __attribute__((address_space(1)))
// Descriptors (weight pointers, shapes) sit in device memory that the host fills before a launch
// and no kernel writes. Read through the constant address space, they load with scalar
// instructions, which do not count against the vector-load counter: a descriptor read then never
// waits for the weight rows in flight (a generic read would be a vector load, and its wait would
// drain every load issued before it).
#define KCONST __attribute__((address_space(4)))
template <typename T>
__device__ __forceinline__ GLB T* glb(T* p) { return (GLB T*)p; }
template <typename T>
__device__ __forceinline__ const GLB T* glb(const T* p) { return (const GLB T*)p; }

// Cross-XCD value: device-scope store (written through to memory).
__device__ __forceinline__ void st_c(u64* p, u64 v) { __hip_atomic_store(glb(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// Intra-XCD value: plain 64-bit store, kept in this XCD's L2 where its readers' loads find it.
__device__ __forceinline__ void st_l(u64* p, u64 v) { __hip_atomic_store(glb(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT); }
// Every exchange read: device-scope load (misses the CU's L1; served by a dirty line of this
// XCD's L2, else by memory).
__device__ __forceinline__ u64 ld_c(const u64* p) { return __hip_atomic_load(glb(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// Error-word bit: an exchange timed out, or another workgroup failed.
constexpr uint32_t kErrTimeout = 1u;

// The XCD (0..7) this workgroup runs on, from the hardware register XCC_ID: the group that shares
// an L2 and so the intra-XCD exchange buffers.
__device__ __forceinline__ int xcd_id() {
  uint32_t xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  return (int)(xcc & (NX - 1));
}

// Workgroup barrier for LDS data: waits for this wave's LDS accesses, then meets the other waves.
// It is no memory-model fence, so vector loads in flight (weight rows, LDS-direct copies) are not
// waited for; a __syncthreads fence drains them whenever an LDS-direct copy is pending. The memory
// clobber keeps the compiler from moving memory accesses across it. Waves that read data another
// wave copied into LDS with LDS-direct loads need that wave to wait for its loads first.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// lds_barrier that also returns whether any thread passed fail = true. Each wave posts one vote,
// (tag << 1) | any-fail, in its own slot; a slot holding a later call's tag belongs to a wave that
// went on, which it does only when it saw no failure, so only this call's failing votes count.
__device__ __forceinline__ bool barrier_any(bool fail, uint32_t tag) {
  __shared__ uint32_t votes[NW];
  const uint32_t mine = (tag << 1) | (__any(fail) ? 1u : 0u);
  if ((threadIdx.x & 63) == 0) votes[wave_id()] = mine;
  lds_barrier();
  bool any = false;
#pragma unroll
  for (int w = 0; w < NW; ++w) any |= votes[w] == ((tag << 1) | 1u);
  return any;
}

// Gather n tagged entries, entry i read from at(i), into lds[0 .. n), polling until every entry
// carries tag; an entry already received is not read again. Each wave polls its own entries
// and the workgroup meets once, at the end, so one slow load does not hold back the other waves'
// next polls. n <= KMAX * NT. Returns false (and flags err) on time-out or when another
// workgroup failed.
// NPOLL: the first NPOLL threads (whole waves) poll, entry i on thread i % NPOLL; the others only
// meet the pollers at the final barrier (waves that must not wait behind their own outstanding
// weight loads). n <= KMAX * NPOLL.
// get_each hands each value to store(i, value) as it arrives instead.
template <int KMAX, int NPOLL = NT, typename At, typename Store>
__device__ __forceinline__ bool get_each(int n, uint32_t tag, uint32_t* err, At at, Store store) {
  const int tid = fresh_tid();
  unsigned pend = 0;
  if (NPOLL == NT || tid < NPOLL) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (tid + k * NPOLL < n) pend |= 1u << k;
  }
  bool fail = false;
  for (long long s = 0; NPOLL == NT || tid < NPOLL; ++s) {
    u64 v[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (pend & (1u << k)) v[k] = ld_c(at(tid + k * NPOLL));
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if ((pend & (1u << k)) && tagof(v[k]) == tag) {
        store(tid + k * NPOLL, valof(v[k]));
        pend &= ~(1u << k);
      }
    if (!__any(pend != 0)) break;
    if ((s & 255) == 255) {
      const uint32_t e = __hip_atomic_load(glb(err), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (e != 0 || s > kSpin) {
        fail = true;
        break;
      }
    }
  }
  if (barrier_any(fail, tag)) {
    if (tid == 0) __hip_atomic_fetch_or(glb(err), kErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
  }
  return true;
}

template <int KMAX, int NPOLL = NT, typename At>
__device__ __forceinline__ bool get_at(int n, uint32_t tag, float* lds, uint32_t* err, At at) {
  return get_each<KMAX, NPOLL>(n, tag, err, at, [&](int i, float v) { lds[i] = v; });
}

// Gather the n contiguous entries src[0 .. n) (see get_at).
template <int KMAX, int NPOLL = NT>
__device__ __forceinline__ bool get_flat(const u64* src, int n, uint32_t tag, float* lds, uint32_t* err) {
  return get_at<KMAX, NPOLL>(n, tag, lds, err, [&](int i) -> const u64* { return src + i; });
}

// ---------------------------------------------------------------------------- weight rows

// Rows of one phase: wave w streams rows row0 + w + NW j (j < MAXR), each row's 16-byte units
// spread over the lanes (unit u = lane + 64 k, k < MAXK).
template <typename WT, int RR, int KK>
struct Rows {
  static constexpr int MAXR = RR, MAXK = KK;
  u32x4 b[RR][KK];
  float s[RR];  // row scales (E4M3 weights; 1 for bf16)
};

// rowptr(i) -> const WT* of row i (0 <= i < nrows); ncols elements per row.
// rowscale(i) -> const float* of row i's scale (E4M3 weights only; read with the row).
template <typename WT, int RR, int KK, typename RowFn, typename ScaleFn>
__device__ __forceinline__ void rows_issue(Rows<WT, RR, KK>& R, int nrows, int ncols, RowFn rowptr, ScaleFn rowscale, bool nt,
                                           int row0 = 0) {
  constexpr int E = WTraits<WT>::E, MAXR = RR, MAXK = KK;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int units = ncols / E;
#pragma unroll
  for (int j = 0; j < MAXR; ++j) {
    const int i = row0 + wave + NW * j;
    if constexpr (E == 16) R.s[j] = i < nrows ? *glb(rowscale(i)) : 0.f;
    if (i < nrows) {
      const GLB u32x4* p = glb(reinterpret_cast<const u32x4*>(rowptr(i)));
#pragma unroll
      for (int k = 0; k < MAXK; ++k) {
        const int u = lane + 64 * k;
        if (u < units) R.b[j][k] = nt ? __builtin_nontemporal_load(p + u) : p[u];
      }
    }
  }
}

// out[i * M + m] = dot(row i, x[m * ldx .. + ncols]) for this wave's rows (LDS in/out).
// NG: the dot is taken with RMSNorm(x row m) instead: every element times its bf16 gain gn[k]
// (LDS), the row sum times 1 / sqrt(mean(x^2) + eps), with sum(x^2) the sum of the NR per-rank
// sums of squares at ss[m * NR ..]. The norm is then one scale per row sum and needs no pass
// (and no barrier) of its own.
// emit(i, m, v) takes each row sum (lane 0 of the row's wave).
template <typename WT, int M, int RR, int KK, bool NG, typename Emit>
__device__ __forceinline__ void rows_dot_impl(const Rows<WT, RR, KK>& R, int nrows, int ncols, const float* x, int ldx, Emit emit,
                                              int row0, const uint16_t* gn, const float* ss, float eps) {
  constexpr int E = WTraits<WT>::E, MAXR = RR, MAXK = KK;
  const int lane = threadIdx.x & 63, wave = row0 + wave_id();
  const int units = ncols / E;
  float acc[MAXR][M];
#pragma unroll
  for (int j = 0; j < MAXR; ++j)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[j][m] = 0.f;
#pragma unroll
  for (int k = 0; k < MAXK; ++k) {
    const int u = lane + 64 * k;
    if (u < units) {
      float xv[M][E];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float* xp = x + m * ldx + u * E;
#pragma unroll
        for (int e = 0; e < E; e += 4) {
          const float4 f = *reinterpret_cast<const float4*>(xp + e);
          xv[m][e] = f.x; xv[m][e + 1] = f.y; xv[m][e + 2] = f.z; xv[m][e + 3] = f.w;
        }
      }
      if constexpr (NG) {
#pragma unroll
        for (int h = 0; h < E; h += 8) {
          float gf[8];
          unpack(*reinterpret_cast<const u32x4*>(gn + u * E + h), gf, (uint16_t*)nullptr);
#pragma unroll
          for (int m = 0; m < M; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) xv[m][h + e] *= gf[e];
        }
      }
#pragma unroll
      for (int j = 0; j < MAXR; ++j) {
        if (wave + NW * j < nrows) {
          float wf[E];
          unpack(R.b[j][k], wf, (WT*)nullptr);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            float s = acc[j][m];
#pragma unroll
            for (int e = 0; e < E; ++e) s = fmaf(wf[e], xv[m][e], s);
            acc[j][m] = s;
          }
        }
      }
    }
  }
  // the norm scales after the dots (their LDS reads would otherwise hold registers through them)
  float sc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    sc[m] = 1.f;
    if constexpr (NG) {
      float t = 0.f;
#pragma unroll
      for (int q = 0; q < NR; q += 4) {
        const float4 f = *reinterpret_cast<const float4*>(ss + m * NR + q);
        t += (f.x + f.y) + (f.z + f.w);
      }
      sc[m] = 1.0f / sqrtf(t / (float)ncols + eps);
    }
  }
#pragma unroll
  for (int j = 0; j < MAXR; ++j) {
    const int i = wave + NW * j;
    if (i < nrows) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float v = wave_sum(acc[j][m]);
        if constexpr (E == 16) v *= R.s[j];
        if constexpr (NG) v *= sc[m];
        if (lane == 0) emit(i, m, v);
      }
    }
  }
}

template <typename WT, int M, int RR, int KK>
__device__ __forceinline__ void rows_dot(const Rows<WT, RR, KK>& R, int nrows, int ncols, const float* x, int ldx, float* out,
                                         int row0 = 0) {
  rows_dot_impl<WT, M, RR, KK, false>(R, nrows, ncols, x, ldx, [&](int i, int m, float v) { out[i * M + m] = v; }, row0, nullptr,
                                      nullptr, 0.f);
}

// The row sums to emit(i, m, v) instead of LDS.
template <typename WT, int M, int RR, int KK, typename Emit>
__device__ __forceinline__ void rows_dot_to(const Rows<WT, RR, KK>& R, int nrows, int ncols, const float* x, int ldx, Emit emit) {
  rows_dot_impl<WT, M, RR, KK, false>(R, nrows, ncols, x, ldx, emit, 0, nullptr, nullptr, 0.f);
}

// The same with RMSNorm(x) as the input (x: the residual rows, row stride ncols).
template <typename WT, int M, int RR, int KK>
__device__ __forceinline__ void rows_dot_norm(const Rows<WT, RR, KK>& R, int nrows, int ncols, const float* x, const uint16_t* gn,
                                              const float* ss, float eps, float* out, int row0 = 0) {
  rows_dot_impl<WT, M, RR, KK, true>(R, nrows, ncols, x, ncols, [&](int i, int m, float v) { out[i * M + m] = v; }, row0, gn, ss,
                                     eps);
}

template <typename WT, int M, int RR, int KK, typename Emit>
__device__ __forceinline__ void rows_dot_norm_to(const Rows<WT, RR, KK>& R, int nrows, int ncols, const float* x, const uint16_t* gn,
                                                 const float* ss, float eps, Emit emit) {
  rows_dot_impl<WT, M, RR, KK, true>(R, nrows, ncols, x, ncols, emit, 0, gn, ss, eps);
}

// ---------------------------------------------------------------------------- block helpers

// ---------------------------------------------------------------------------- the kernel

// Shared memory layout (floats). Row m of a residual-width array starts at m * H.
struct Smem {
  float xs[2 * HMAX + 2 * NR];  // residual rows (full), then per-rank sums of squares per row
  float xn[2 * HMAX];   // normed / staged input rows; reduce-scatter partials
  float qkv[2 * 512];   // this XCD's q/k/v slice
  float ob[2 * 256];    // attention output of this XCD's heads
  float hb[2 * 768];    // SwiGLU slice
  float out[2 * 128];   // row results of this workgroup
  float red[64];
  float kq[4][128];     // normed + rotated q of each attention wave
  float cand[2 * NWG];  // argmax candidates of every workgroup
  float kvc[MAXL][2][kCpPos][KVS];  // this frame's K/V rows of KV head g, per layer
  __align__(16) uint16_t gn[2 * MAXL + 1][HMAX];  // bf16 norm gains: layer l attention 2 l, MLP 2 l + 1; final 2 MAXL
};

// ---------------------------------------------------------------------------- weight phases
// A phase's rows are issued into one of two register buffers as soon as the phase two back has
// consumed it, so their HBM latency overlaps the two exchanges before the phase.

template <typename WT>
using RowsA = Rows<WT, RA_R, RA_K>;
template <typename WT>
using RowsC = Rows<WT, RC_R, RA_K>;
template <typename WT>
using RowsB = Rows<WT, RB_R, RB_K>;

// The issue functions take the layer index: its weight pointers and, for E4M3 matrices, its row
// scales (an E4M3 matrix row carries one fp32 scale; sc(ptr, i) is row i's, or null for bf16).
__device__ __forceinline__ const float* sc(const float* p, size_t i) { return p ? p + i : nullptr; }

// q/k/v rows [qper*r, +qper) of this XCD's (G q heads | k | v)
template <typename WT>
__device__ __forceinline__ void issue_qkv(RowsA<WT>& R, const KCONST CpDesc& D, int l, int g, int r) {
  const KCONST LayerW& W = D.layer[l];
  const KCONST LayerS& Sc = D.scale[l];
  const int H = D.H, d = D.d, G = D.nq / D.nkv, qper = (G + 2) * d / NR;
  rows_issue(R, qper, H, [&](int i) -> const WT* {
    const int q = qper * r + i;
    if (q < G * d) return reinterpret_cast<const WT*>(W.wq) + (size_t)(G * d * g + q) * H;
    if (q < (G + 1) * d) return reinterpret_cast<const WT*>(W.wk) + (size_t)(d * g + q - G * d) * H;
    return reinterpret_cast<const WT*>(W.wv) + (size_t)(d * g + q - (G + 1) * d) * H;
  }, [&](int i) -> const float* {
    const int q = qper * r + i;
    if (q < G * d) return sc(Sc.wq, G * d * g + q);
    if (q < (G + 1) * d) return sc(Sc.wk, d * g + q - G * d);
    return sc(Sc.wv, d * g + q - (G + 1) * d);
  }, false);
}
// output projection rows [hper*r, +hper), columns of this XCD's heads
template <typename WT>
__device__ __forceinline__ void issue_o(RowsB<WT>& R, const KCONST CpDesc& D, int l, int g, int r) {
  const KCONST LayerW& W = D.layer[l];
  const float* so = D.scale[l].wo;
  const int hper = D.H / NR, Gd = D.nq / D.nkv * D.d;
  rows_issue(R, hper, Gd, [&](int i) -> const WT* {
    return reinterpret_cast<const WT*>(W.wo) + (size_t)(hper * r + i) * (D.nq * D.d) + Gd * g;
  }, [&](int i) { return sc(so, hper * r + i); }, false);
}
// gate rows then up rows [fper*r, +fper) of this XCD's FFN slice: rows [row0, row0 + RR NW)
template <typename WT, int RR>
__device__ __forceinline__ void issue_gu(Rows<WT, RR, RA_K>& R, int row0, const KCONST CpDesc& D, int l, int g, int r) {
  const KCONST LayerW& W = D.layer[l];
  const KCONST LayerS& Sc = D.scale[l];
  const int fx = D.F / NX, fper = fx / NR;
  rows_issue(R, 2 * fper, D.H, [&](int i) -> const WT* {
    const int f = fx * g + fper * r + (i % fper);
    return reinterpret_cast<const WT*>(i < fper ? W.wg : W.wu) + (size_t)f * D.H;
  }, [&](int i) { return sc(i < fper ? Sc.wg : Sc.wu, fx * g + fper * r + (i % fper)); }, false, row0);
}
// down projection rows [hper*r, +hper), columns of this XCD's FFN slice
template <typename WT>
__device__ __forceinline__ void issue_down(RowsB<WT>& R, const KCONST CpDesc& D, int l, int g, int r) {
  const KCONST LayerW& W = D.layer[l];
  const float* sd = D.scale[l].wd;
  const int hper = D.H / NR, fx = D.F / NX;
  rows_issue(R, hper, fx, [&](int i) -> const WT* {
    return reinterpret_cast<const WT*>(W.wd) + (size_t)(hper * r + i) * D.F + fx * g;
  }, [&](int i) { return sc(sd, hper * r + i); }, false);
}
// head j rows [vper*blockIdx, +vper)
template <typename WT>
__device__ __forceinline__ void issue_head(RowsA<WT>& R, const KCONST CpDesc& D, int j) {
  const int vper = D.V / NWG;
  const WT* head = reinterpret_cast<const WT*>(D.heads) + (size_t)(j - 1) * D.V * D.H;
  const float* sh = D.head_scale;
  rows_issue(R, vper, D.H, [&](int i) -> const WT* { return head + (size_t)(vper * blockIdx.x + i) * D.H; },
             [&](int i) { return sc(sh, (size_t)(j - 1) * D.V + vper * blockIdx.x + i); }, false);
}
// input projection rows (K split: XCD g takes columns [Ht/8 * g, +Ht/8), rank r rows [hper*r, +hper))
template <typename WT>
__device__ __forceinline__ void issue_proj(RowsB<WT>& R, const KCONST CpDesc& D, int g, int r) {
  const int kx = D.Ht / NX, hper = D.H / NR;
  const float* sp = D.proj_scale;
  rows_issue(R, hper, kx, [&](int i) -> const WT* {
    return reinterpret_cast<const WT*>(D.proj) + (size_t)(hper * r + i) * D.Ht + kx * g;
  }, [&](int i) { return sc(sp, hper * r + i); }, false);
}

// ---------------------------------------------------------------------------- exchanges
// Each exchange publishes this workgroup's values first and only then runs after_put (which
// issues the next weight rows): issuing loads can stall while the memory pipeline is busy, and
// other workgroups are waiting for the values, not for this workgroup's weights.

// Cross reduce-scatter of this workgroup's hper x M partial rows (S.out, row-major [row][m]) with
// rank r of every XCD, plus an optional residual (S.xs), then the intra gather of the full rows into
// S.xs[0 .. M*H). With the rows each rank also publishes the sum of squares of its reduced rows,
// gathered into S.xs[M*H + m*NR + rank], so the next RMSNorm needs no reduction of its own.
// cpar alternates the cross slot so a rank one exchange ahead never overwrites unread values.
// HMX: the largest H the caller supports (sizes the cross gather); KMAX: loads per thread of the
// intra gather (M * (H + NR) entries).
// produce(emit): makes the partial rows, calling emit(row, m, value) once for every row < hper and
// m < M (from any thread; reduce_gather: all threads from S.out).
template <int M, int HMX, int KMAX, int NPOLL = NT, typename Produce, typename AfterPut>
__device__ __forceinline__ bool reduce_gather_p(const Xch& X, Produce produce, float* xs, float* xn, int H, bool residual,
                                                uint32_t& tag, int& iring, int& cpar, int g, int r, AfterPut after_put) {
  const int tid = fresh_tid(), hper = H / NR;
  ++tag;
  u64* mine = X.xcr + ((size_t)(r * NX + g) * 2 + (cpar & 1)) * CSZ;
  const uint32_t t = tag;
  produce([&](int e, int m, float v) { st_c(mine + m * 64 + e, pack(v, t)); });
  after_put();
  // partners: rank r on every XCD x, slot r * NX + x; their slots are 2 * CSZ apart.
  // Segment (x, m) -> xn[(x * M + m) * hper ..]
  // (hper is a power of two: entry i -> element i & (hper - 1) of segment i >> lh)
  const u64* base = X.xcr + ((size_t)(r * NX) * 2 + (cpar & 1)) * CSZ;
  const int lh = __builtin_ctz(hper);
  if (!get_at<(NX * M * (HMX / NR) + NPOLL - 1) / NPOLL, NPOLL>(NX * M * hper, tag, xn, X.err, [&](int i) -> const u64* {
        const int sg = i >> lh, e = i & (hper - 1);
        return base + (size_t)(sg / M) * (2 * CSZ) + (sg % M) * 64 + e;
      }))
    return false;
  ++cpar;
  ++tag;
  u64* buf = X.xin + ((size_t)g * RING + (iring++ & (RING - 1))) * ISZ;
  if (tid < 64) {  // hper * M <= 64: wave 0 reduces and publishes this rank's rows
    const int e = tid / M, m = tid % M;
    const int row = hper * r + e;
    const bool live = tid < hper * M;
    float v = 0.f;
    if (live) {
      v = residual ? xs[m * H + row] : 0.f;
#pragma unroll
      for (int x = 0; x < NX; ++x) v += xn[(x * M + m) * hper + e];
      st_l(buf + m * H + row, pack(v, tag));
    }
#pragma unroll
    for (int mm = 0; mm < M; ++mm) {
      const float ss = wave_sum(live && m == mm ? v * v : 0.f);
      if (tid == 0) st_l(buf + M * H + mm * NR + r, pack(ss, tag));
    }
  }
  lds_barrier();  // the gather below overwrites the residual rows read above
  return get_flat<KMAX, NPOLL>(buf, M * (H + NR), tag, xs, X.err);
}

template <int M, int HMX, int KMAX, int NPOLL = NT, typename AfterPut>
__device__ __forceinline__ bool reduce_gather(const Xch& X, const float* out, float* xs, float* xn, int H, bool residual,
                                              uint32_t& tag, int& iring, int& cpar, int g, int r, AfterPut after_put) {
  const int hper = H / NR;
  return reduce_gather_p<M, HMX, KMAX, NPOLL>(
      X,
      [&](auto emit) {
        for (int i = fresh_tid(); i < hper * M; i += NT) emit(i / M, i % M, out[i]);
      },
      xs, xn, H, residual, tag, iring, cpar, g, r, after_put);
}

// Intra gather of a slice: this workgroup's n values per row (vals(e, m)) land at row offset
// n * r of every rank's copy; the full rows (width w) of all ranks go to dst.
// produce(emit): calls emit(e, m, value) once for every e < n and m < M (from any thread).
template <int M, int KMAX, int NPOLL = NT, typename Produce, typename AfterPut>
__device__ __forceinline__ bool slice_gather_p(const Xch& X, int n, int w, Produce produce, float* dst, uint32_t& tag, int& iring,
                                               int g, int r, AfterPut after_put) {
  ++tag;
  u64* buf = X.xin + ((size_t)g * RING + (iring++ & (RING - 1))) * ISZ;
  const uint32_t t = tag;
  produce([&](int e, int m, float v) { st_l(buf + m * w + n * r + e, pack(v, t)); });
  after_put();
  return get_flat<KMAX, NPOLL>(buf, M * w, tag, dst, X.err);
}

// slice_gather_p handing each gathered value to store(i, value) instead of an fp32 row.
template <int M, int KMAX, int NPOLL = NT, typename Produce, typename Store, typename AfterPut>
__device__ __forceinline__ bool slice_gather_pe(const Xch& X, int n, int w, Produce produce, Store store, uint32_t& tag, int& iring,
                                                int g, int r, AfterPut after_put) {
  ++tag;
  u64* buf = X.xin + ((size_t)g * RING + (iring++ & (RING - 1))) * ISZ;
  const uint32_t t = tag;
  produce([&](int e, int m, float v) { st_l(buf + m * w + n * r + e, pack(v, t)); });
  after_put();
  return get_each<KMAX, NPOLL>(M * w, tag, X.err, [&](int i) -> const u64* { return buf + i; }, store);
}

template <int M, int KMAX, int NPOLL = NT, typename ValFn, typename AfterPut>
__device__ __forceinline__ bool slice_gather(const Xch& X, int n, int w, ValFn vals, float* dst, uint32_t& tag, int& iring,
                                             int g, int r, AfterPut after_put) {
  return slice_gather_p<M, KMAX, NPOLL>(
      X, n, w,
      [&](auto emit) {
        for (int i = fresh_tid(); i < n * M; i += NT) emit(i / M, i % M, vals(i / M, i % M));
      },
      dst, tag, iring, g, r, after_put);
}

// ---------------------------------------------------------------------------- per-thread constants

// Per-head norm gains and RoPE factors a layer needs, held in registers so no global load sits on
// the critical path: for the attention waves the q- and k-norm gains of lanes lane, lane + 64 and
// the RoPE cos/sin of positions p0 .. p0 + M - 1 at lane. (The residual-norm gains sit in LDS.)
struct LayerConsts {
  float qg[2], kg[2], rc[2], rs[2];
};

template <typename WT, int M>
__device__ __forceinline__ void load_consts(LayerConsts& c, const KCONST CpDesc& D, const KCONST LayerW& W, int p0) {
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63, G = D.nq / D.nkv;
  using GT = typename WTraits<WT>::GT;  // gains stay bf16 next to E4M3 matrices
#pragma unroll
  for (int k = 0; k < 2; ++k) { c.qg[k] = c.kg[k] = c.rc[k] = 1.f; c.rs[k] = 0.f; }
  if (wave < G * M) {
    const GT* qn = reinterpret_cast<const GT*>(W.q_norm);
    const GT* kn = reinterpret_cast<const GT*>(W.k_norm);
    c.qg[0] = to_f32(glb(qn)[lane]);
    c.qg[1] = to_f32(glb(qn)[lane + 64]);
    c.kg[0] = to_f32(glb(kn)[lane]);
    c.kg[1] = to_f32(glb(kn)[lane + 64]);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      c.rc[m] = glb(D.rope_cos)[(p0 + m) * 64 + lane];
      c.rs[m] = glb(D.rope_sin)[(p0 + m) * 64 + lane];
    }
  }
}

// ---------------------------------------------------------------------------- the layer

// One decoder layer for M rows at positions p0 .. p0 + M - 1. Weight phases alternate between two
// register buffers and are issued two phases ahead of their use. On entry R1 holds this layer's
// q/k/v rows, R0 its output-projection rows and c its constants; on exit R1 holds the next layer's
// q/k/v rows (or head j), R0 the next layer's output-projection rows (or the next step's input
// projection) and c the next layer's constants. S.xs holds the input rows and, after them, their
// NR sums of squares per row (the RMSNorms take those; gains in S.gn).
template <typename WT, int M>
__device__ __forceinline__ bool cp_layer(const KCONST CpDesc& D, const CpCall& C, int layer, int j, int p0, Smem& S,
                                         RowsB<WT>& R0, RowsA<WT>& R1, RowsC<WT>& R2, LayerConsts& c, uint32_t& tag, int& iring,
                                         int& cpar, int g, int r) {
  const KCONST LayerW& W = D.layer[layer];
  const int H = D.H, d = D.d, G = D.nq / D.nkv;
  const int qrows = (G + 2) * d;          // q/k/v rows owned by one XCD
  const int qper = qrows / NR;            // rows per rank
  const int hper = H / NR;                // residual rows per rank (reduce-scatter slice)
  const int fx = D.F / NX, fper = fx / NR;  // FFN slice per XCD / per rank
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const bool last = layer + 1 == D.n_layers;
  const Xch X{D.xin, D.xcr, D.err};
  constexpr int KCP = (M * (HMAX + NR) + NT - 1) / NT;

  // --- q/k/v slice (R1). Here and in the output and down projections every wave publishes its row
  // sums as it makes them (no LDS staging, no barrier before the exchange).
  if (!slice_gather_p<M, M>(
          X, qper, qrows,
          [&](auto emit) { rows_dot_norm_to<WT, M>(R1, qper, H, S.xs, S.gn[2 * layer], S.xs + M * H, D.eps, emit); }, S.qkv,
          tag, iring, g, r, [] {}))
    return false;
  // The first gate/up rows go out after this exchange, not before its poll: the poll would wait
  // behind them (a wave's loads return in order), while the attention leaves most waves idle.
  issue_gu(R1, 0, D, layer, g, r);

  // --- attention for this XCD's heads over positions 0 .. p0 + M - 1 (d = 128): one wave per
  // (head h, row m). Every rank of the XCD computes it redundantly from the same gathered q/k/v
  // and keeps its own copy of the frame's K/V rows of KV head g in LDS (positions are written in
  // order, so rows 0 .. p are this frame's). Each attention wave normalises and rotates the step's
  // k rows itself and appends them (the waves write identical values), so no barrier separates
  // the append from the scores.
  if (wave < G * M) {
    float (*kc)[KVS] = S.kvc[layer][0];
    float (*vc)[KVS] = S.kvc[layer][1];
    const int h = wave / M, m = wave % M, p = p0 + m;
#pragma unroll
    for (int mm = 0; mm < M; ++mm) {
      const float* kr = S.qkv + mm * qrows + G * d;
      float k0 = kr[lane], k1 = kr[lane + 64];
      const float sc = 1.0f / sqrtf(wave_sum(k0 * k0 + k1 * k1) / (float)d + D.eps);
      k0 *= sc * c.kg[0];
      k1 *= sc * c.kg[1];
      kc[p0 + mm][lane] = k0 * c.rc[mm] - k1 * c.rs[mm];
      kc[p0 + mm][lane + 64] = k1 * c.rc[mm] + k0 * c.rs[mm];
      vc[p0 + mm][lane] = kr[d + lane];
      vc[p0 + mm][lane + 64] = kr[d + lane + 64];
    }
    {
      const float* qr = S.qkv + m * qrows + h * d;
      float q0 = qr[lane], q1 = qr[lane + 64];
      const float sc = 1.0f / sqrtf(wave_sum(q0 * q0 + q1 * q1) / (float)d + D.eps);
      q0 *= sc * c.qg[0];
      q1 *= sc * c.qg[1];
      // (select, not index: a dynamic index would move c out of registers)
      const float rc = (M == 2 && m == 1) ? c.rc[1] : c.rc[0], rs = (M == 2 && m == 1) ? c.rs[1] : c.rs[0];
      S.kq[wave][lane] = q0 * rc - q1 * rs;
      S.kq[wave][lane + 64] = q1 * rc + q0 * rs;
    }
    // scores: lane = 4 t + e, position t (0..15) and quarter e of the head dimension
    const int t = lane >> 2, e = lane & 3;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 a = *reinterpret_cast<const float4*>(&S.kq[wave][32 * e + 4 * i]);
      const float4 b = *reinterpret_cast<const float4*>(&kc[t][32 * e + 4 * i]);
      s = fmaf(a.x, b.x, s); s = fmaf(a.y, b.y, s); s = fmaf(a.z, b.z, s); s = fmaf(a.w, b.w, s);
    }
    // the quarters' sums within each group of 4 lanes (DPP quad permutes), then the max, the
    // weights' sum and the output over the 16 positions from the lanes 4 t read as scalars: no
    // cross-lane step goes through LDS
    s += TTS_DPP(s, 0xB1);  // quad_perm [1,0,3,2]
    s += TTS_DPP(s, 0x4E);  // quad_perm [2,3,0,1]
    s = t <= p ? s * (1.0f / sqrtf((float)d)) : -INFINITY;  // rows past p hold stale values
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < kCpPos; ++tt) mx = fmaxf(mx, readlane_f(s, 4 * tt));
    const float w = t <= p ? expf(s - mx) : 0.f;
    float l = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int tt = 0; tt < kCpPos; ++tt) {
      if (tt <= p) {
        const float wt = readlane_f(w, 4 * tt);
        l += wt;
        o0 = fmaf(wt, vc[tt][lane], o0);
        o1 = fmaf(wt, vc[tt][lane + 64], o1);
      }
    }
    S.ob[m * G * d + h * d + lane] = o0 / l;
    S.ob[m * G * d + h * d + lane + 64] = o1 / l;
  }
  issue_gu(R2, RA_R * NW, D, layer, g, r);  // the gate/up rows past R1's
  lds_barrier();

  // --- output projection partial (R0: rows [hper*r, +hper), this XCD's head columns), residual
  if (!reduce_gather_p<M, HMAX, KCP>(
          X, [&](auto emit) { rows_dot_to<WT, M>(R0, hper, G * d, S.ob, G * d, emit); }, S.xs, S.xn, H, true, tag, iring, cpar, g,
          r, [&] { issue_down(R0, D, layer, g, r); }))
    return false;

  // --- gate/up slice (R1) + SwiGLU
  rows_dot_norm<WT, M>(R1, 2 * fper, H, S.xs, S.gn[2 * layer + 1], S.xs + M * H, D.eps, S.out);
  // R1 is free: the next phase's rows go out before the second part's dot, so they are further
  // along when the SwiGLU exchange polls behind them
  if (!last) {
    load_consts<WT, M>(c, D, D.layer[layer + 1], p0);
    issue_qkv(R1, D, layer + 1, g, r);
  } else {
    issue_head(R1, D, j);
  }
  rows_dot_norm<WT, M>(R2, 2 * fper, H, S.xs, S.gn[2 * layer + 1], S.xs + M * H, D.eps, S.out, RA_R * NW);
  lds_barrier();
  if (!slice_gather<M, M>(X, fper, fx, [&](int e, int m) { return silu(S.out[e * M + m]) * S.out[(fper + e) * M + m]; }, S.hb,
                          tag, iring, g, r, [] {}))
    return false;

  // --- down projection partial (R0: rows [hper*r, +hper), this XCD's FFN columns), residual
  return reduce_gather_p<M, HMAX, KCP>(
      X, [&](auto emit) { rows_dot_to<WT, M>(R0, hper, fx, S.hb, fx, emit); }, S.xs, S.xn, H, true, tag, iring, cpar, g, r, [&] {
        if (!last) issue_o(R0, D, layer + 1, g, r);
        else if (j < D.n_ac && D.proj) issue_proj(R0, D, g, r);
      });
}

// Argmax over the head rows: each workgroup holds nrows logits of rows [row0, row0 + nrows) in
// S.out (M = 1). Every workgroup publishes its best (value, id) and reads all NWG candidates.
// Ties go to the lower id. Returns the id (or -1 on failure).
__device__ __forceinline__ int argmax_exchange(const KCONST CpDesc& D, Smem& S, int nrows, int row0, uint32_t& tag, int& apar) {
  const int tid = threadIdx.x;
  ++tag;
  u64* cb = D.cand + (size_t)(apar & 1) * NWG * CAND;
  if (tid == 0) {
    float bv = S.out[0];
    int bi = row0;
    for (int i = 1; i < nrows; ++i)
      if (S.out[i] > bv) { bv = S.out[i]; bi = row0 + i; }
    st_c(cb + blockIdx.x * CAND, pack(bv, tag));
    st_c(cb + blockIdx.x * CAND + 1, pack(__int_as_float(bi), tag));
  }
  if (!get_at<1>(2 * NWG, tag, S.cand, D.err, [&](int i) -> const u64* { return cb + (i >> 1) * CAND + (i & 1); })) return -1;
  ++apar;
  __shared__ int best;
  if (tid < NWG) {
    float v = S.cand[2 * tid];
    int id = __float_as_int(S.cand[2 * tid + 1]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float v2 = __shfl_xor(v, o);
      const int id2 = __shfl_xor(id, o);
      if (v2 > v || (v2 == v && id2 < id)) { v = v2; id = id2; }
    }
    if ((tid & 63) == 0) { S.red[tid >> 6] = v; S.red[8 + (tid >> 6)] = __int_as_float(id); }
  }
  lds_barrier();
  if (tid == 0) {
    float bv = S.red[0];
    int bi = __float_as_int(S.red[8]);
    for (int w = 1; w < NWG / 64; ++w) {
      const float v = S.red[w];
      const int id = __float_as_int(S.red[8 + w]);
      if (v > bv || (v == bv && id < bi)) { bv = v; bi = id; }
    }
    best = bi;
  }
  lds_barrier();
  return best;
}

// One CodePredictor step j (1..15) with M input rows; tok = its input token. On entry R0 holds the
// input projection's rows (when the model has one), R1 layer 0's q/k/v rows and c layer 0's
// constants; on exit they hold the next step's.
template <typename WT, int M>
__device__ __forceinline__ bool cp_step(const KCONST CpDesc& D, const CpCall& C, int j, int& tok, Smem& S, RowsB<WT>& R0,
                                        RowsA<WT>& R1, RowsC<WT>& R2, LayerConsts& c, uint32_t& tag, int& iring,
                                        int& cpar, int& apar, int frame, int g, int r) {
  const int H = D.H, Ht = D.Ht, V = D.V, tid = threadIdx.x;
  const Xch X{D.xin, D.xcr, D.err};
  constexpr int KCP = (M * (HMAX + NR) + NT - 1) / NT;
  using GT = typename WTraits<WT>::GT;  // embedding tables stay bf16 next to E4M3 matrices
  const GT* tab = (j == 1) ? reinterpret_cast<const GT*>(D.embed_sem)
                           : reinterpret_cast<const GT*>(D.embed_ac) + (size_t)(j - 2) * V * Ht;
  const GT* erow = tab + (size_t)tok * Ht;
  if (D.proj) {
    const int kx = Ht / NX, hper = H / NR;
    for (int i = tid; i < kx; i += NT) {
      if (M == 2) {
        S.xn[i] = glb(D.hT)[kx * g + i];
        S.xn[kx + i] = to_f32(glb(erow)[kx * g + i]);
      } else {
        S.xn[i] = to_f32(glb(erow)[kx * g + i]);
      }
    }
    lds_barrier();
    rows_dot<WT, M>(R0, hper, kx, S.xn, kx, S.out);
    lds_barrier();
    if (!reduce_gather<M, HMAX, KCP>(X, S.out, S.xs, S.xn, H, false, tag, iring, cpar, g, r, [&] { issue_o(R0, D, 0, g, r); }))
      return false;
  } else {
    issue_o(R0, D, 0, g, r);
    for (int i = tid; i < H; i += NT) {
      if (M == 2) {
        S.xs[i] = glb(D.hT)[i];
        S.xs[H + i] = to_f32(glb(erow)[i]);
      } else {
        S.xs[i] = to_f32(glb(erow)[i]);
      }
    }
    lds_barrier();
    // the rows' sums of squares in the layout an exchange leaves them: NR per row (one per wave
    // here, the rest zero)
    {
      const int wave = wave_id(), lane = tid & 63;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float q = 0.f;
        for (int i = wave * 64 + lane; i < H; i += NT) q += S.xs[m * H + i] * S.xs[m * H + i];
        q = wave_sum(q);
        if (lane < NR / NW) S.xs[M * H + m * NR + wave + NW * lane] = lane == 0 ? q : 0.f;
      }
    }
    lds_barrier();
  }
  const int p0 = (j == 1) ? 0 : j;
  for (int l = 0; l < D.n_layers; ++l)
    if (!cp_layer<WT, M>(D, C, l, j, p0, S, R0, R1, R2, c, tag, iring, cpar, g, r)) return false;
  // final norm on the last row, head j (R1), argmax
  const int vper = V / NWG;
  rows_dot_norm<WT, 1>(R1, vper, H, S.xs + (M - 1) * H, S.gn[2 * MAXL], S.xs + M * H + (M - 1) * NR, D.eps, S.out);
  lds_barrier();
  if (j < D.n_ac) {
    load_consts<WT, 1>(c, D, D.layer[0], j + 1);
    issue_qkv(R1, D, 0, g, r);
  }
  if (C.logits)
    for (int i = tid; i < vper; i += NT) glb(C.logits)[(size_t)(j - 1) * V + vper * blockIdx.x + i] = S.out[i];
  const int a = argmax_exchange(D, S, vper, vper * blockIdx.x, tag, apar);
  if (a < 0) return false;
  if (blockIdx.x == 0 && tid == 0) glb(C.codes)[(C.use_frame ? (long)frame * C.f_stride : 0) + j - 1] = a;
  tok = C.forced ? glb(C.forced)[j - 1] : a;
  if (tok < 0) tok = 0;
  if (tok >= V) tok = V - 1;
  return true;
}

template <typename WT>
__global__ __launch_bounds__(NT) void k_cp_frame(CpCall C) {
  const KCONST CpDesc& D = *(const KCONST CpDesc*)C.desc;
  __shared__ Smem S;
  const int g = xcd_id(), r = blockIdx.x / NX;
  // constants first (they are needed first), then the first two weight phases
  LayerConsts c;
  load_consts<WT, 2>(c, D, D.layer[0], 0);
  // every RMSNorm gain of the frame into LDS (bf16, as stored; the first barrier of the frame
  // comes before their first use)
  {
    static_assert(sizeof(typename WTraits<WT>::GT) == 2, "norm gains are bf16");
    const int nv = D.H / 8;  // 16-byte units per gain vector
    for (int i = threadIdx.x; i < (2 * D.n_layers + 1) * nv; i += NT) {
      const int v = i / nv, u = i % nv;
      const void* src = v == 2 * D.n_layers ? D.final_norm : (v & 1) ? D.layer[v >> 1].mlp_norm : D.layer[v >> 1].attn_norm;
      *reinterpret_cast<u32x4*>(&S.gn[v == 2 * D.n_layers ? 2 * MAXL : v][8 * u]) = glb(reinterpret_cast<const u32x4*>(src))[u];
    }
  }
  RowsB<WT> R0;
  RowsA<WT> R1;
  RowsC<WT> R2;
  if (D.proj) issue_proj(R0, D, g, r);
  issue_qkv(R1, D, 0, g, r);
  uint32_t tag = glb(D.st)->epoch;
  const int frame = glb(D.st)->frame;
  int iring = 0, cpar = 0, apar = 0;
  int tok = glb(C.semantic)[0];
  if (tok < 0) tok = 0;
  if (tok >= D.Vs) tok = D.Vs - 1;
  bool ok = cp_step<WT, 2>(D, C, 1, tok, S, R0, R1, R2, c, tag, iring, cpar, apar, frame, g, r);
  for (int j = 2; ok && j <= D.n_ac; ++j)
    ok = cp_step<WT, 1>(D, C, j, tok, S, R0, R1, R2, c, tag, iring, cpar, apar, frame, g, r);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    glb(D.st)->epoch = tag + 1;  // every workgroup has read the epoch: all took part in the last exchange
    if (C.next_tok) glb(C.next_tok)[0] = tok;
  }
}

}  // namespace xtp
}  // namespace tts
