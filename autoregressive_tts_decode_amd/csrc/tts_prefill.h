// Prefill: the Talker over a prompt of n text positions for B lockstep streams as dense GEMMs on
// the matrix cores ("Running Qwen3-TTS on an AMD R9700", section "Running Qwen3-TTS": the prompt
// pass before the frame loop). Positions are processed in chunks of at most kPrefillChunk per
// stream, M = B x chunk rows per GEMM; causal attention of a chunk reads the KV cache, which holds
// every earlier position. The same GEMM serves batched decode steps (many streams' rows).
// Activations stay fp32: the tiled GEMM (k_gemm_bf16) splits its fp32 input a into three bf16
// parts, hi = bf16(a), mid = bf16(a - hi), lo = bf16(a - hi - mid), whose sum is a exactly for
// normal values (each remainder is exact in fp32 and the last fits 8 mantissa bits), and
// accumulates W hi + W mid + W lo in fp32 (W is bf16 already): the product is the fp32 one up to
// accumulation order. The decode GEMM (k_gemm_dec, at most 64 rows) keeps two parts, hi and
// bf16(a - hi), about 17 significant bits of a, as the persistent Talker kernel does.
#pragma once

#include "tts_device.h"

namespace tts {

constexpr int kPrefillChunk = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// C[M, N] (+)= (rs[m] * gain[k] * A[m, k]) W^T, W: bf16 [N, K] rows in up to 3 segments (each a
// multiple of 64 rows), A fp32 [M, lda], C fp32 [M, ldc].
struct GemmArgs {
  const float* A;
  int lda;
  const float* rs;    // [M] row scale or nullptr
  const void* gain;   // [K] bf16 or nullptr
  const void* w[3];   // bf16 rows, or E4M3 codes (Q8) with per-row fp32 scales in wscale
  const float* wscale[3];
  int seg_rows[3], nseg;
  float* C;
  int ldc;
  int M, N, K;
  int add;            // 1: C += result (residual), 0: C = result
  int kslice;         // K columns per workgroup (blockIdx.z selects the slice); kslice < K: every
                      // workgroup writes its partial tile to part (slice z at part + z M N, row
                      // stride N) and k_splitk_reduce adds the slices into C in slice order, so the
                      // sum is the same on every run
  float* part;
  const float* ssq;   // or: the row scales come from per-chunk sums of squares of A's rows,
  int nchunk;         // ssq[m * nchunk + c] for 256-column chunks c (added in chunk order)
  float eps;
};

constexpr int kGBM = 64, kGBN = 64, kGBK = 64, kGLD = kGBK + 8;  // tile, LDS row stride (bf16)

// One 64 x 64 tile of C per workgroup (4 waves, each 32 x 32 = 2 x 2 MFMA 16x16x32 blocks).
// Q8: the weights are E4M3 codes; every code is a bf16 value exactly, so the B tile is widened to
// bf16 as it is staged and each output column (weight row) is multiplied by its scale at the end.
template <bool Q8>
__global__ __launch_bounds__(256) void k_gemm_bf16(GemmArgs a) {
  __shared__ __align__(16) __bf16 Ahi[kGBM][kGLD];
  __shared__ __align__(16) __bf16 Amid[kGBM][kGLD];
  __shared__ __align__(16) __bf16 Alo[kGBM][kGLD];
  __shared__ __align__(16) __bf16 Bs[kGBN][kGLD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * kGBN, m0 = blockIdx.y * kGBM;
  int seg = 0, nrel = n0;
  while (seg + 1 < a.nseg && nrel >= a.seg_rows[seg]) { nrel -= a.seg_rows[seg]; ++seg; }
  constexpr int WB = Q8 ? 1 : 2;  // bytes per weight element
  const char* W = reinterpret_cast<const char*>(a.w[seg]) + (size_t)nrel * a.K * WB;
  const int kbeg = blockIdx.z * a.kslice, kend = min(kbeg + a.kslice, a.K);
  const bool split = a.kslice < a.K;
  const int lr = tid >> 2, lk = (tid & 3) * 16;  // loader: row lr of the tile, 16 k from lk
  const bool arow = m0 + lr < a.M;
  float rsc = (a.rs && arow) ? a.rs[m0 + lr] : 1.f;
  if (a.ssq && arow) {
    float q = 0.f;
    for (int c = 0; c < a.nchunk; ++c) q += a.ssq[(size_t)(m0 + lr) * a.nchunk + c];
    rsc = 1.0f / sqrtf(q / (float)a.K + a.eps);
  }
  const float* Ap = a.A + (size_t)(m0 + lr) * a.lda + lk;
  const char* Wp = W + ((size_t)lr * a.K + lk) * WB;
  const uint16_t* gp = reinterpret_cast<const uint16_t*>(a.gain);
  const int wm = wave >> 1, wn = wave & 1, lq = lane >> 4, lc = lane & 15;
  f32x4v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x4v){0.f, 0.f, 0.f, 0.f};
  // A, W and gain operands of a K step go to registers one step ahead: the next step's loads are
  // in flight while this step's tile is staged and multiplied.
  float4 an[4];
  u32x4 bn0, bn1, gn0, gn1;
  auto load_step = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) an[q] = arow ? *reinterpret_cast<const float4*>(Ap + k0 + 4 * q) : make_float4(0.f, 0.f, 0.f, 0.f);
    bn0 = *reinterpret_cast<const u32x4*>(Wp + (size_t)k0 * WB);
    if constexpr (!Q8) bn1 = *reinterpret_cast<const u32x4*>(Wp + (size_t)k0 * WB + 16);
    if (gp) {
      gn0 = *reinterpret_cast<const u32x4*>(gp + k0 + lk);
      gn1 = *reinterpret_cast<const u32x4*>(gp + k0 + lk + 8);
    }
  };
  if (kbeg < kend) load_step(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += kGBK) {
    float av[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      av[4 * q] = an[q].x; av[4 * q + 1] = an[q].y; av[4 * q + 2] = an[q].z; av[4 * q + 3] = an[q].w;
    }
    const u32x4 b0 = bn0, b1 = bn1, g0 = gn0, g1 = gn1;
    if (k0 + kGBK < kend) load_step(k0 + kGBK);
    if (gp) {
      float gf0[8], gf1[8];
      unpack(g0, gf0, (uint16_t*)nullptr);
      unpack(g1, gf1, (uint16_t*)nullptr);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        av[e] = av[e] * rsc * gf0[e];
        av[e + 8] = av[e + 8] * rsc * gf1[e];
      }
    } else if (a.rs) {
#pragma unroll
      for (int e = 0; e < 16; ++e) av[e] *= rsc;
    }
    __syncthreads();  // the previous step's operand reads are done
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const __bf16 hi = (__bf16)av[e];
      const float r1 = av[e] - (float)hi;
      const __bf16 mid = (__bf16)r1;
      Ahi[lr][lk + e] = hi;
      Amid[lr][lk + e] = mid;
      Alo[lr][lk + e] = (__bf16)(r1 - (float)mid);
    }
    if constexpr (Q8) {
      float wf[16];
      unpack(b0, wf, (uint8_t*)nullptr);
      uint32_t pk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pk[e] = (__float_as_uint(wf[2 * e]) >> 16) | (__float_as_uint(wf[2 * e + 1]) & 0xffff0000u);
      *reinterpret_cast<u32x4*>(&Bs[lr][lk]) = (u32x4){pk[0], pk[1], pk[2], pk[3]};
      *reinterpret_cast<u32x4*>(&Bs[lr][lk + 8]) = (u32x4){pk[4], pk[5], pk[6], pk[7]};
    } else {
      *reinterpret_cast<u32x4*>(&Bs[lr][lk]) = b0;
      *reinterpret_cast<u32x4*>(&Bs[lr][lk + 8]) = b1;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kGBK; kk += 32) {
      bf16x8 ah[2], am[2], al[2], bw[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ah[i] = *reinterpret_cast<const bf16x8*>(&Ahi[wm * 32 + i * 16 + lc][kk + 8 * lq]);
        am[i] = *reinterpret_cast<const bf16x8*>(&Amid[wm * 32 + i * 16 + lc][kk + 8 * lq]);
        al[i] = *reinterpret_cast<const bf16x8*>(&Alo[wm * 32 + i * 16 + lc][kk + 8 * lq]);
        bw[i] = *reinterpret_cast<const bf16x8*>(&Bs[wn * 32 + i * 16 + lc][kk + 8 * lq]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // smallest part first, so the large products are added to the small ones' sum
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], bw[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am[i], bw[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bw[j], acc[i][j], 0, 0, 0);
        }
    }
  }
  // lane holds C[4 lq + r][lc] of each 16 x 16 block
  float csc[2] = {1.f, 1.f};
  if constexpr (Q8) {
#pragma unroll
    for (int j = 0; j < 2; ++j) csc[j] = a.wscale[seg][nrel + wn * 32 + j * 16 + lc];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 32 + i * 16 + 4 * lq + r, n = n0 + wn * 32 + j * 16 + lc;
        if (m < a.M) {
          float* c = a.C + (size_t)m * a.ldc + n;
          const float v = Q8 ? acc[i][j][r] * csc[j] : acc[i][j][r];
          if (split) a.part[((size_t)blockIdx.z * a.M + m) * a.N + n] = v;
          else *c = a.add ? *c + v : v;
        }
      }
}

// Decode GEMM for few rows (M <= 16 MT; bf16 weights): C = RMSNorm-scaled A [M][K] times the
// weight rows W [N][K]^T. A workgroup (4 waves) owns 64 RW weight rows (all in one segment) and one
// K slice of at most KSM columns: wave w loads the B fragments of rows 64 t + 16 w + l % 16
// (t < RW) for the whole slice into registers at once (lane l: columns 32 s + 8 (l / 16) of K
// step s), while the workgroup stages the slice of the A rows (times the row scale and the gain) in
// LDS as two bf16 parts (hi = bf16(x), lo = bf16(x - hi): their sum holds x to about 17
// significant bits, a relative error near 2^-17, as the persistent Talker kernel's activations;
// the products with bf16 weights are exact in the fp32 accumulator); each K step is then
// MT x RW x 2 MFMAs per wave, the smaller part first, every A fragment read once for the RW tiles. With several slices each writes its partial tile to part (slice z at
// part + z M N) and a pass of its own adds them in slice order.
template <int MT, int KSM, int RW>
__global__ __launch_bounds__(256) void k_gemm_dec(GemmArgs a) {
  constexpr int MR = 16 * MT;
  constexpr int LD = KSM + 8;  // LDS row stride (bf16)
  __shared__ __align__(16) __bf16 As[2][MR][LD];
  __shared__ float srs[MR];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 64 * RW;
  int seg = 0, nrel = n0;
  while (seg + 1 < a.nseg && nrel >= a.seg_rows[seg]) { nrel -= a.seg_rows[seg]; ++seg; }
  const int kbeg = blockIdx.z * a.kslice, kn = min(a.kslice, a.K - kbeg), nks = kn / 32;
  // Every load is issued before any is waited on, in the order of use: the row sums of squares
  // (or row scales), the A slice and its gains, then the weight fragments. Addresses are clamped
  // into range instead of predicated (a predicated load leaves a branch whose join waits for it);
  // what a clamped load brings in past the slice or the rows is never used.
  constexpr int Q4 = KSM / 4, AI = MR * Q4 / 256, CB = 24;  // A float4 per thread; chunk sums
  static_assert(AI * 256 == MR * Q4 && 256 % Q4 == 0, "A slice share");
  const int mr = min(tid & (MR - 1), a.M - 1);
  const int nch = a.ssq ? a.nchunk : 1;
  const float* sq = a.ssq ? a.ssq + (size_t)mr * nch : (a.rs ? a.rs + mr : a.A);
  const int ca = 4 * (tid % Q4), ma = tid / Q4, cl = min(ca, kn - 4);  // thread's columns (all its rows)
  float4 xa[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i)
    xa[i] = *reinterpret_cast<const float4*>(a.A + (size_t)min(ma + i * (256 / Q4), a.M - 1) * a.lda + kbeg + cl);
  const uint16_t* gp = reinterpret_cast<const uint16_t*>(a.gain);
  const uint16_t* gq = gp ? gp + kbeg + cl : reinterpret_cast<const uint16_t*>(a.A);
  uint16_t graw[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) graw[k] = gq[k];
  const uint16_t* wrow = reinterpret_cast<const uint16_t*>(a.w[seg]) + (size_t)(nrel + 16 * wave + (lane & 15)) * a.K + kbeg +
                         8 * (lane >> 4);
  u32x4 b[RW][KSM / 32];
#pragma unroll
  for (int t2 = 0; t2 < RW; ++t2)
#pragma unroll
    for (int s = 0; s < KSM / 32; ++s) b[t2][s] = *reinterpret_cast<const u32x4*>(wrow + (size_t)64 * t2 * a.K + 32 * min(s, nks - 1));
  static_assert(MR <= 64, "row scales from wave 0");
  if (wave == 0) {  // the row scales: only wave 0's lanes load the chunk sums
    float qv[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) qv[c] = sq[min(c, nch - 1)];
   if (tid < MR) {
    float sc = 1.f;
    if (tid < a.M) {
      if (a.ssq) {  // chunk sums added in chunk order
        float q = 0.f;
#pragma unroll
        for (int c = 0; c < CB; ++c)
          if (c < nch) q += qv[c];
        for (int c = CB; c < nch; ++c) q += sq[c];
        sc = 1.0f / sqrtf(q / (float)a.K + a.eps);
      } else if (a.rs) {
        sc = qv[0];
      }
    }
    srs[tid] = sc;
   }
  }
  __syncthreads();
  if (ca < kn) {
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int m = ma + i * (256 / Q4);
      float x[4] = {0.f, 0.f, 0.f, 0.f};
      if (m < a.M) {
        const float sc = srs[m];
        x[0] = xa[i].x * sc; x[1] = xa[i].y * sc; x[2] = xa[i].z * sc; x[3] = xa[i].w * sc;
        if (gp) {
#pragma unroll
          for (int k = 0; k < 4; ++k) x[k] *= to_f32(graw[k]);
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const __bf16 hi = (__bf16)x[k];
        As[0][m][ca + k] = hi;
        As[1][m][ca + k] = (__bf16)(x[k] - (float)hi);
      }
    }
  }
  __syncthreads();
  f32x4v acc[RW][MT];
#pragma unroll
  for (int t2 = 0; t2 < RW; ++t2)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t2][t] = (f32x4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KSM / 32; ++s) {
    if (s < nks) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int p = 1; p >= 0; --p) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(&As[p][16 * t + (lane & 15)][32 * s + 8 * (lane >> 4)]);
#pragma unroll
          for (int t2 = 0; t2 < RW; ++t2)
            acc[t2][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, b[t2][s]), acc[t2][t], 0, 0, 0);
        }
    }
  }
  const bool split = a.kslice < a.K;
#pragma unroll
  for (int t2 = 0; t2 < RW; ++t2) {
    const int n = n0 + 64 * t2 + 16 * wave + (lane & 15);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * t + 4 * (lane >> 4) + r;
        if (m < a.M) {
          if (split) {
            a.part[((size_t)blockIdx.z * a.M + m) * a.N + n] = acc[t2][t][r];
          } else {
            float* c = a.C + (size_t)m * a.ldc + n;
            *c = a.add ? *c + acc[t2][t][r] : acc[t2][t][r];
          }
        }
      }
  }
}

// Rows of a bf16 table E [R][K] through a bias-free bf16 projection P [N][K]: T[a][i] =
// sum_k E[a][k] P[i][k] in fp32 (T [R][N]). A product of two bf16 values is exact in fp32 and k
// runs in order, so T holds P E[a] up to the order of its sums, the same on every run. One 64 x 64
// tile of T per workgroup (16 x 16 threads, 4 x 4 outputs each); K % 32 == 0. Weight preparation,
// run once per weight binding. With E4M3 codes for P (PT = uint8_t), row i of P is pscale[i] times
// its codes: the codes are widened exactly and T[a][i] is the code sum times pscale[i].
__device__ __forceinline__ float proj_val(uint16_t v) { return to_f32(v); }
__device__ __forceinline__ float proj_val(uint8_t v) { return __builtin_amdgcn_cvt_pk_f32_fp8((int)v, false)[0]; }
template <typename PT>
__global__ __launch_bounds__(256) void k_proj_table(const uint16_t* E, const PT* P, const float* pscale, float* T, int R, int N,
                                                    int K) {
  __shared__ float Es[32][65];  // [k][row of the tile]
  __shared__ float Ps[32][65];  // [k][column of the tile]
  const int tid = threadIdx.x, tr = tid / 16, tc = tid % 16;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  float acc[4][4];
  for (int i = 0; i < 4; ++i)
    for (int q = 0; q < 4; ++q) acc[i][q] = 0.f;
  for (int k0 = 0; k0 < K; k0 += 32) {
    for (int e = tid; e < 64 * 32; e += 256) {
      const int rr = e / 32, kk = e % 32;
      Es[kk][rr] = r0 + rr < R ? to_f32(E[(size_t)(r0 + rr) * K + k0 + kk]) : 0.f;
      Ps[kk][rr] = c0 + rr < N ? proj_val(P[(size_t)(c0 + rr) * K + k0 + kk]) : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < 32; ++kk) {
      float a[4], b[4];
      for (int i = 0; i < 4; ++i) {
        a[i] = Es[kk][tr + 16 * i];
        b[i] = Ps[kk][tc + 16 * i];
      }
      for (int i = 0; i < 4; ++i)
        for (int q = 0; q < 4; ++q) acc[i][q] = fmaf(a[i], b[q], acc[i][q]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i)
    for (int q = 0; q < 4; ++q) {
      const int row = r0 + tr + 16 * i, col = c0 + tc + 16 * q;
      if (row < R && col < N) T[(size_t)row * N + col] = pscale ? acc[i][q] * pscale[col] : acc[i][q];
    }
}

// C[m][n] = (add ? C[m][n] : 0) + part[0][m][n] + part[1][m][n] + ... + part[ks - 1][m][n], the
// slices added in that order; one row chunk of 256 columns per workgroup (grid: chunks x M). With
// ssq, also the chunk's sum of squares of the new row, ssq[m * gridDim.x + chunk] (a fixed-order
// reduction), which the next RMSNorm reads instead of a pass of its own over the row.
__global__ __launch_bounds__(256) void k_splitk_reduce(float* C, int ldc, const float* part, int M, int N, int ks, int add,
                                                       float* ssq) {
  __shared__ float wsum[4];
  const int m = blockIdx.y, n = blockIdx.x * 256 + threadIdx.x;
  float v = 0.f;
  if (n < N) {
    const float* pp = part + (size_t)m * N + n;
    const size_t zs = (size_t)M * N;
    if (ks > 0) {
      // C and the slices loaded together (indices clamped, not predicated, so no load waits on
      // another), then added in slice order
      const float c0 = C[(size_t)m * ldc + n];
      constexpr int ZB = 16;
      float t[ZB];
#pragma unroll
      for (int z = 0; z < ZB; ++z) t[z] = pp[min(z, ks - 1) * zs];
      v = add ? c0 : 0.f;
#pragma unroll
      for (int z = 0; z < ZB; ++z)
        if (z < ks) v += t[z];
      for (int z = ZB; z < ks; ++z) v += pp[z * zs];
    } else {
      v = add ? C[(size_t)m * ldc + n] : 0.f;
    }
    C[(size_t)m * ldc + n] = v;
  }
  if (ssq) {
    const float q = wave_sum(v * v);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = q;
    __syncthreads();
    if (threadIdx.x == 0) ssq[(size_t)m * gridDim.x + blockIdx.x] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  }
}

// h[m][f] = silu(sum_z part[z][m][f]) * sum_z part[z][m][F + f] (slices in order; part rows hold
// the F gate columns, then the F up columns).
__global__ __launch_bounds__(256) void k_splitk_swiglu(const float* part, int M, int F, int ks, float* h, int ldh) {
  const size_t n = (size_t)M * F;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < n; idx += (size_t)gridDim.x * blockDim.x) {
    const size_t m = idx / F, f = idx % F;
    float g = 0.f, u = 0.f;
    const float* row = part + m * 2 * F + f;
    const size_t zs = (size_t)M * 2 * F;
    constexpr int ZB = 8;  // slices loaded together (indices clamped), then added in slice order
    float tg[ZB], tu[ZB];
#pragma unroll
    for (int z = 0; z < ZB; ++z) {
      tg[z] = row[min(z, ks - 1) * zs];
      tu[z] = row[min(z, ks - 1) * zs + F];
    }
#pragma unroll
    for (int z = 0; z < ZB; ++z)
      if (z < ks) { g += tg[z]; u += tu[z]; }
    for (int z = ZB; z < ks; ++z) {
      g += row[z * zs];
      u += row[z * zs + F];
    }
    h[m * ldh + f] = silu(g) * u;
  }
}

// rs[m] = 1 / sqrt(mean(x[m]^2) + eps) over K; one wave per row.
__global__ __launch_bounds__(256) void k_rowscale(const float* x, int ldx, int M, int K, float eps, float* rs) {
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (m >= M) return;
  const float* row = x + (size_t)m * ldx;
  float s = 0.f;
  if ((K & 3) == 0 && (ldx & 3) == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0) {
    for (int k = 4 * lane; k < K; k += 256) {
      const float4 v = *reinterpret_cast<const float4*>(row + k);
      s += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
    }
  } else {
    for (int k = lane; k < K; k += 64) s += row[k] * row[k];
  }
  s = wave_sum(s);
  if (lane == 0) rs[m] = 1.0f / sqrtf(s / (float)K + eps);
}

// out[m] = x[m] * rs[m] * gain (the normalised rows a GEMM with a row scale consumed), one
// block per row.
template <typename WT>
__global__ void k_norm_rows(const float* x, int ldx, const float* rs, const void* gain, int K, float* out, int ldo) {
  const int m = blockIdx.x;
  const WT* g = reinterpret_cast<const WT*>(gain);
  for (int k = threadIdx.x; k < K; k += blockDim.x) out[(size_t)m * ldo + k] = x[(size_t)m * ldx + k] * rs[m] * to_f32(g[k]);
}

// The device counters' advance that a GEMV epilogue does when a GEMM replaces it.
__global__ void k_bump_state(DevState* st, int dpos, int dframe) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    st->pos += dpos;
    st->frame += dframe;
  }
}

// Rows b * P + i of X = E_text[ids[b * n + p0 + i]] (i < P), fp32.
template <typename WT>
__global__ void k_embed_rows(const int32_t* ids, int n, int p0, int P, int vocab, const void* table, int H, float* X) {
  const int row = blockIdx.x, b = row / P, i = row % P;
  int tok = ids[(size_t)b * n + p0 + i];
  tok = tok < 0 ? 0 : (tok >= vocab ? vocab - 1 : tok);
  const WT* e = reinterpret_cast<const WT*>(table) + (size_t)tok * H;
  for (int k = threadIdx.x; k < H; k += blockDim.x) X[(size_t)row * H + k] = to_f32(e[k]);
}

struct QkArgs {
  const float* qkv;   // [M, (nq + 2 nkv) d]
  float* q;           // [M, nq d] normed + rotated q
  void *kc, *vc;      // cache of this layer: [B][nkv][cap][d]
  const void *q_norm, *k_norm;
  const float *rope_cos, *rope_sin;  // [cap][d / 2]
  int M, P, p0, nq, nkv, cap;
  float eps;
};

// One wave per (row, head): q heads -> per-head RMSNorm + RoPE into q; k heads -> the same into the
// cache at the row's position; v heads -> copied into the cache. d = 128.
template <typename WT, typename KT>
__global__ __launch_bounds__(256) void k_qk_rope_kv(QkArgs a) {
  const int nh = a.nq + 2 * a.nkv;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (item >= a.M * nh) return;
  const int row = item / nh, j = item % nh, b = row / a.P, pos = a.p0 + row % a.P;
  constexpr int d = 128;
  const float* src = a.qkv + (size_t)row * nh * d + (size_t)j * d;
  float v0 = src[lane], v1 = src[lane + 64];
  if (j < a.nq + a.nkv) {
    const WT* gn = reinterpret_cast<const WT*>(j < a.nq ? a.q_norm : a.k_norm);
    const float sc = 1.0f / sqrtf(wave_sum(v0 * v0 + v1 * v1) / (float)d + a.eps);
    v0 *= sc * to_f32(gn[lane]);
    v1 *= sc * to_f32(gn[lane + 64]);
    const float c = a.rope_cos[(size_t)pos * 64 + lane], s = a.rope_sin[(size_t)pos * 64 + lane];
    const float r0 = v0 * c - v1 * s, r1 = v1 * c + v0 * s;
    v0 = r0;
    v1 = r1;
  }
  if (j < a.nq) {
    float* q = a.q + (size_t)row * a.nq * d + (size_t)j * d;
    q[lane] = v0;
    q[lane + 64] = v1;
  } else {
    const int g = j < a.nq + a.nkv ? j - a.nq : j - a.nq - a.nkv;
    KT* dst = reinterpret_cast<KT*>(j < a.nq + a.nkv ? a.kc : a.vc) + (((size_t)b * a.nkv + g) * a.cap + pos) * d;
    store_elem(dst + lane, v0);
    store_elem(dst + lane + 64, v1);
  }
}

struct PAttnArgs {
  const float* q;     // [M, nq d]
  const void *kc, *vc;
  float* out;         // [M, nq d]
  int P, p0, nq, nkv, cap;
  const int32_t* kvstart;  // [B] first visible position of each stream (ragged prompts), or nullptr (0)
};

// Causal attention of prefill rows: one wave per (row i of stream b, q head h) over cached
// positions 0 .. p0 + i; lanes 4 t + e cover 16 positions per pass (quarter e of d = 128).
template <typename KT>
__global__ __launch_bounds__(256) void k_prefill_attn(PAttnArgs a) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6), h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x & 63;
  if (i >= a.P) return;
  constexpr int d = 128;
  const int row = b * a.P + i, pos = a.p0 + i, g = h / (a.nq / a.nkv);
  const KT* kc = reinterpret_cast<const KT*>(a.kc) + ((size_t)b * a.nkv + g) * a.cap * d;
  const KT* vc = reinterpret_cast<const KT*>(a.vc) + ((size_t)b * a.nkv + g) * a.cap * d;
  const float* q = a.q + (size_t)row * a.nq * d + (size_t)h * d;
  const int tq = lane >> 2, e = lane & 3;
  float qv[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) qv[k] = q[32 * e + k];
  const float scale = 1.0f / sqrtf((float)d);
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  // positions before the stream's start are padding (a row of the padding itself attends to
  // nothing and gives 0)
  for (int base = a.kvstart ? a.kvstart[b] : 0; base <= pos; base += 16) {
    const int t = base + tq;
    const bool valid = t <= pos;
    const KT* kr = kc + (size_t)(valid ? t : 0) * d + 32 * e;
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) s = fmaf(qv[k], to_f32(kr[k]), s);
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s = valid ? s * scale : -INFINITY;
    float mx = s;
#pragma unroll
    for (int o = 4; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float mn = fmaxf(m, mx);
    const float corr = m == -INFINITY ? 0.f : expf(m - mn);
    const float w = valid ? expf(s - mn) : 0.f;
    float ws = w;
#pragma unroll
    for (int o = 4; o < 64; o <<= 1) ws += __shfl_xor(ws, o);
    l = l * corr + ws;
    o0 *= corr;
    o1 *= corr;
    m = mn;
    // the pass's v rows, all loads in flight together (rows past the pass are not loaded; their
    // weight is 0), then the sums in position order
    const int np = min(16, pos + 1 - base);
    float va[16], vb[16];
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      va[tt] = 0.f;
      vb[tt] = 0.f;
      if (tt < np) {
        va[tt] = to_f32(vc[(size_t)(base + tt) * d + lane]);
        vb[tt] = to_f32(vc[(size_t)(base + tt) * d + lane + 64]);
      }
    }
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      const float wt = __shfl(w, 4 * tt);
      o0 = fmaf(wt, va[tt], o0);
      o1 = fmaf(wt, vb[tt], o1);
    }
  }
  float* o = a.out + (size_t)row * a.nq * d + (size_t)h * d;
  o[lane] = l > 0.f ? o0 / l : 0.f;
  o[lane + 64] = l > 0.f ? o1 / l : 0.f;
}

// h[m, f] = silu(gu[m, f]) * gu[m, F + f]
__global__ void k_swiglu_rows(const float* gu, int M, int F, float* h) {
  const size_t n = (size_t)M * F;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < n; idx += (size_t)gridDim.x * blockDim.x) {
    const size_t m = idx / F, f = idx % F;
    h[idx] = silu(gu[m * 2 * F + f]) * gu[m * 2 * F + F + f];
  }
}

// x[b] = X[b * P + P - 1] (the last prompt row of each stream)
__global__ void k_last_rows(const float* X, int P, int H, float* x) {
  const int b = blockIdx.x;
  for (int k = threadIdx.x; k < H; k += blockDim.x) x[(size_t)b * H + k] = X[((size_t)b * P + P - 1) * H + k];
}

}  // namespace tts
