// Optional phase timeline of the persistent kernels: with TTS_PHASE_TRACE defined at build time,
// thread 0 of every workgroup records (label << 48 | wall clock) at each TTS_STAMP(label) into
// g_trace[blockIdx][..] while g_trace_on is set; otherwise TTS_STAMP compiles to nothing. The
// wall clock is the 100 MHz constant-rate counter shared by all CUs, so stamps of different
// workgroups compare directly.
#pragma once

#include <hip/hip_runtime.h>

namespace tts {

constexpr int kTraceWg = 256;     // workgroups recorded
constexpr int kTracePer = 4096;   // stamps per workgroup

#ifdef TTS_PHASE_TRACE
__device__ long long g_trace[kTraceWg * kTracePer];
__device__ int g_trace_on;
__shared__ int g_trace_n;
// base: first slot of this kernel's stamps (kernels of one frame write disjoint ranges). The
// switch is read once here: while tracing is off the slot counter starts past the end, so a stamp
// costs one LDS compare and no global load.
#define TTS_TRACE_BEGIN(base) \
  do { if (threadIdx.x == 0) g_trace_n = g_trace_on && blockIdx.x < kTraceWg ? (base) : kTracePer; } while (0)
#define TTS_STAMP(lbl)                                                                                        \
  do {                                                                                                        \
    if (threadIdx.x == 0 && g_trace_n < kTracePer)                                                            \
      g_trace[blockIdx.x * kTracePer + g_trace_n++] = ((long long)(lbl) << 48) | (long long)wall_clock64();   \
  } while (0)
#else
#define TTS_TRACE_BEGIN(base) do { } while (0)
#define TTS_STAMP(lbl) do { } while (0)
#endif

}  // namespace tts
