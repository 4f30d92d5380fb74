// Host side of the C ABI in include/tts.h: validation, weight binding,
// workspace layout, launch sequences of the Talker step / CodePredictor frame
// / samplers, and the captured per-frame HIP graph.
//
// Per frame ("Running Qwen3-TTS on an AMD R9700", section "Running
// Qwen3-TTS"): the Talker runs once and emits the semantic token, then the
// CodePredictor runs 15 sequential steps for acoustic tokens 1..15. Here a
// replayed frame is: draw the semantic token from the pending Talker output,
// run the 15 CodePredictor steps, write the 16 codes, run the Talker step that
// consumes them (which leaves the next frame's Talker output pending).
#include "tts.h"
#include "tts_device.h"
#include "tts_prefill.h"
#include "tts_xcp.h"
#include "tts_xtk.h"
#include "tts_xtp.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

using namespace tts;

namespace {

constexpr int kCpPositions = 16;   // CodePredictor positions 0..15 per frame
constexpr int kAttnChunk = 32;     // Talker positions per attention split (the partial buffer's unit)

// Positions per attention block for B streams of nkv KV heads and a cache of cap positions:
// kAttnChunk while the (stream, head) pairs alone give the chip few blocks, 2 kAttnChunk at 128
// pairs, and the whole cache (one block per pair, no split) once the pairs alone fill the chip
// (256). A block pays a fixed q/k norm and combine cost, and split blocks the merge: its
// device-scope fences write back the XCD's L2 (32 streams x 8 heads at ~270 positions: a frame
// of 14.0 ms with 128-position splits, 8.8 ms with one block per pair). A multiple of kAttnChunk
// keeps the partial buffer's layout: split i of the larger chunk is its slot i, and the slots past
// the last used split are never written or read.
int attn_chunk(int B, int nkv, int cap) {
  const int pairs = B * nkv;
  if (pairs >= 256) return (cap + kAttnChunk - 1) / kAttnChunk * kAttnChunk;
  return pairs >= 128 ? 2 * kAttnChunk : kAttnChunk;
}
constexpr int kMaxGemvM = 8;       // input rows per GEMV launch
constexpr int kGemmMinRows = 16;   // batched projections with at least this many rows run as MFMA GEMMs
constexpr int kGemmWgs = 512;      // workgroups a split-K decode GEMM aims for
constexpr int kGemvXRegs = 96;     // per-lane registers a GEMV spends on its input rows (M * U * E)

struct Layer {
  const void *attn_norm = nullptr, *wq = nullptr, *wk = nullptr, *wv = nullptr, *q_norm = nullptr, *k_norm = nullptr;
  const void *wo = nullptr, *mlp_norm = nullptr, *wg = nullptr, *wu = nullptr, *wd = nullptr;
};

struct StackW {
  tts_stack_cfg c;
  std::vector<Layer> layers;
  const void* final_norm = nullptr;
};

struct GraphKey {
  tts_sampling sem, ac;
  const float* u;
  int32_t* codes;
  int batch;
  bool operator==(const GraphKey& o) const {
    return std::memcmp(&sem, &o.sem, sizeof sem) == 0 && std::memcmp(&ac, &o.ac, sizeof ac) == 0 && u == o.u &&
           codes == o.codes && batch == o.batch;
  }
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace layout, computed identically by tts_workspace_bytes and tts_create.
struct Layout {
  size_t st, tk, tv, ck, cv, tcos, tsin, ccos, csin, x, qkv, attn, h, part, counters, logits, hT, cx, clog, next_tok,
      sem_tok, ac_codes, history, kvstart, aids, ptab, cpdesc, tkdesc, cpdesc_s, tkdesc_s, px, pqkv, pq, po, pgu, ph, ps, pks, ssq, xin, xcr, cand, att, xerr, xzero_begin, xzero_end, total;
  int nsplit;
};

// Bytes per element of the projection matrices and of the gains / embedding tables.
size_t mat_bytes(const tts_config& c) { return c.weight_dtype == TTS_DTYPE_F32 ? 4 : (c.weight_dtype == TTS_DTYPE_BF16 ? 2 : 1); }
size_t tab_bytes(const tts_config& c) { return c.weight_dtype == TTS_DTYPE_F32 ? 4 : 2; }
// Elements per 16-byte lane load of the matrices.
int mat_per_unit(const tts_config& c) { return (int)(16 / mat_bytes(c)); }
size_t kv_bytes(const tts_config&) { return 4; }

bool xcp_capable(const tts_config& c);

// Weight row tiles of 64 per decode-GEMM workgroup: 4 past 32 input rows (the staged A slice then
// serves 256 weight rows) when every segment is a whole number of 256-row blocks, else 1.
int dec_rw(int M, const int* seg_rows, int nseg) {
  if (M <= 32) return 1;
  for (int s = 0; s < nseg; ++s)
    if (seg_rows[s] % 256) return 1;
  return 4;
}

// K split of the decode GEMM (k_gemm_dec) for N output rows, K columns, M input rows and rw row
// tiles per workgroup: slices of at most 256 columns (128 past 32 rows, which measured faster for
// 64-row prompt chunks), more of them only while the grid has fewer than 64 workgroups (each slice
// adds a partial tile that the following pass reads back; with every load of a workgroup issued at
// once, fewer and longer slices measured faster than filling all 256 compute units); returns the
// slice count.
int dec_split(int N, int K, int M, int rw, int* kslice) {
  const int kmax = M <= 32 ? 256 : 128, tiles = N / (64 * rw);
  const int ks_min = (K + kmax - 1) / kmax;
  const int want = std::max(1, (64 + tiles - 1) / tiles);
  int ks = std::max(ks_min, std::min(want, K / 64));
  const int ksl = ((K / 64 + ks - 1) / ks) * 64;
  *kslice = ksl;
  return (K + ksl - 1) / ksl;
}
// The lean CodePredictor kernel with an input projection P reads step j >= 2's input row from the
// table of projected codebook rows P E_ac[j - 2][a] (fp32), formed once per weight binding.
bool wants_proj_table(const tts_config& c) { return xcp_capable(c) && c.talker.hidden != c.codepred.hidden; }

Layout make_layout(const tts_config& c) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  const auto &t = c.talker, &p = c.codepred;
  const size_t B = c.max_batch, eb = kv_bytes(c);
  const size_t cap = c.max_cache_steps;
  L.nsplit = (int)((cap + kAttnChunk - 1) / kAttnChunk);
  L.st = take(sizeof(DevState));
  L.tk = take((size_t)t.n_layers * B * t.n_kv_heads * cap * t.head_dim * eb);
  L.tv = take((size_t)t.n_layers * B * t.n_kv_heads * cap * t.head_dim * eb);
  L.ck = take((size_t)p.n_layers * B * p.n_kv_heads * kCpPositions * p.head_dim * eb);
  L.cv = take((size_t)p.n_layers * B * p.n_kv_heads * kCpPositions * p.head_dim * eb);
  L.tcos = take(cap * (t.head_dim / 2) * 4);
  L.tsin = take(cap * (t.head_dim / 2) * 4);
  L.ccos = take(kCpPositions * (p.head_dim / 2) * 4);
  L.csin = take(kCpPositions * (p.head_dim / 2) * 4);
  const size_t rows = 2 * B;  // CodePredictor step 1 runs two positions per stream
  const size_t hmax = std::max(t.hidden, p.hidden);
  const size_t qkv_t = (size_t)(t.n_q_heads + 2 * t.n_kv_heads) * t.head_dim;
  const size_t qkv_c = (size_t)(p.n_q_heads + 2 * p.n_kv_heads) * p.head_dim;
  L.x = take(B * t.hidden * 4);
  L.qkv = take(rows * std::max(qkv_t, qkv_c) * 4);
  L.attn = take(rows * std::max((size_t)t.n_q_heads * t.head_dim, (size_t)p.n_q_heads * p.head_dim) * 4);
  L.h = take(rows * std::max(t.ffn, p.ffn) * 4);
  L.part = take(B * t.n_q_heads * (size_t)L.nsplit * (t.head_dim + 2) * 4);
  L.counters = take(B * t.n_kv_heads * 4);
  L.logits = take(B * t.vocab * 4);
  L.hT = take(B * t.hidden * 4);
  L.cx = take(rows * hmax * 4);
  L.clog = take(B * p.vocab * 4);
  L.next_tok = take(B * 4);
  L.sem_tok = take(B * 4);
  L.ac_codes = take(B * c.n_acoustic * 4);
  L.history = take(B * t.vocab);
  L.kvstart = take(B * 4);
  L.aids = take((size_t)B * cap * 4);
  L.ptab = take(wants_proj_table(c) ? (size_t)c.n_acoustic * p.vocab * p.hidden * 4 : 0);
  // GEMM prefill: one chunk of up to kPrefillChunk positions per stream
  {
    const size_t Mp = B * kPrefillChunk;
    const size_t qd = (size_t)t.n_q_heads * t.head_dim;
    L.px = take(Mp * t.hidden * 4);
    L.pqkv = take(Mp * qkv_t * 4);
    L.pq = take(Mp * qd * 4);
    L.po = take(Mp * qd * 4);
    L.pgu = take(Mp * 2 * t.ffn * 4);
    L.ph = take(Mp * t.ffn * 4);
    L.ps = take(Mp * 4);
    // split-K partial tiles: a split GEMM has at most kGemmWgs (row tile, column tile, K slice)
    // workgroups, each writing one 64 x 64 fp32 tile; the decode GEMM (rows <= 64: decode steps and
    // prompt chunks of few streams) writes slices x rows x N
    size_t pks = (size_t)kGemmWgs * kGBM * kGBN * 4;
    const int mdec = (int)std::min<size_t>(std::max(rows, Mp), 64);  // decode rows, or a prompt chunk of <= 64 rows
    const size_t qkvt = (size_t)(t.n_q_heads + 2 * t.n_kv_heads) * t.head_dim, qkvc = (size_t)(p.n_q_heads + 2 * p.n_kv_heads) * p.head_dim;
    const size_t shapes[][2] = {{qkvt, (size_t)t.hidden}, {(size_t)t.hidden, (size_t)t.n_q_heads * t.head_dim},
                                {2 * (size_t)t.ffn, (size_t)t.hidden}, {(size_t)t.hidden, (size_t)t.ffn}, {(size_t)t.vocab, (size_t)t.hidden},
                                {qkvc, (size_t)p.hidden}, {(size_t)p.hidden, (size_t)p.n_q_heads * p.head_dim},
                                {2 * (size_t)p.ffn, (size_t)p.hidden}, {(size_t)p.hidden, (size_t)p.ffn}, {(size_t)p.vocab, (size_t)p.hidden},
                                {(size_t)p.hidden, (size_t)t.hidden}};
    for (const auto& sh : shapes) {
      if (sh[0] % 64 || sh[1] % 64) continue;
      for (const int rw : {1, 4}) {  // either row-tile choice (segments decide it at launch)
        int ksl = 0;
        const int ks = dec_split((int)sh[0], (int)sh[1], mdec, rw, &ksl);
        pks = std::max(pks, (size_t)ks * mdec * sh[0] * 4);
      }
    }
    L.pks = take(pks);
    // per-row, per-256-column chunk sums of squares a residual GEMM leaves for the next RMSNorm
    L.ssq = take(Mp * ((hmax + 255) / 256) * 4);
  }
  // persistent kernels: descriptors and exchange buffers (the CodePredictor's K/V rows stay in LDS)
  L.cpdesc = take(sizeof(xtp::CpDesc));
  L.tkdesc = take(sizeof(xtp::TkDesc));
  // the same descriptors with the exchange buffers in the device's static scratch array
  // (tts_run_frames_noalloc)
  L.cpdesc_s = take(sizeof(xtp::CpDesc));
  L.tkdesc_s = take(sizeof(xtp::TkDesc));
  L.xzero_begin = off;
  L.xin = take((size_t)xtp::NX * xtp::RING * xtp::ISZ * 8);
  L.xcr = take((size_t)xtp::NWG * 2 * xtp::CSZ * 8);
  L.cand = take((size_t)2 * xtp::NWG * xtp::CAND * 8);
  L.att = take((size_t)xtp::NX * 2 * xtp::NR * xtp::ATS * 8);
  L.xerr = take(256);
  L.xzero_end = off;
  L.total = off;
  return L;
}

bool units_ok(int K, int E, int* U) {
  if (K <= 0 || K % (64 * E)) return false;
  const int u = K / (64 * E);
  if (!(u == 1 || u == 2 || u == 3 || u == 4 || u == 6 || u == 8 || u == 12 || u == 16)) return false;
  if (U) *U = u;
  return true;
}

// Returns an error text or "" when the config is one the kernels accept.
std::string check_config(const tts_config* c) {
  if (!c) return "config is NULL";
  if (c->weight_dtype != TTS_DTYPE_F32 && c->weight_dtype != TTS_DTYPE_BF16 && c->weight_dtype != TTS_DTYPE_FP8_E4M3)
    return "weight_dtype must be TTS_DTYPE_F32, TTS_DTYPE_BF16 or TTS_DTYPE_FP8_E4M3";
  // a bf16 cache alone puts the 1.7B acoustic logits just over the 1e-2 parity bar, so the caches stay fp32
  if (c->kv_dtype != TTS_DTYPE_F32) return "kv_dtype must be TTS_DTYPE_F32";
  if (c->n_acoustic != 15) return "n_acoustic must be 15";
  if (c->max_batch < 1 || c->max_batch > 64) return "max_batch must be in [1, 64]";
  if (c->max_cache_steps < 2 || c->max_cache_steps > 65536) return "max_cache_steps must be in [2, 65536]";
  if (c->max_frames < 1) return "max_frames must be >= 1";
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 1.f)) return "rms_eps must be > 0 and rope_theta > 1";
  if (c->text_vocab < 1) return "text_vocab must be >= 1";
  const int E = mat_per_unit(*c);
  const tts_stack_cfg* ss[2] = {&c->talker, &c->codepred};
  for (int i = 0; i < 2; ++i) {
    const tts_stack_cfg& s = *ss[i];
    const char* nm = i ? "codepred" : "talker";
    char buf[256];
    if (s.n_layers < 1 || s.vocab < 1 || s.n_q_heads < 1 || s.n_kv_heads < 1) {
      snprintf(buf, sizeof buf, "%s: n_layers, vocab and head counts must be >= 1", nm);
      return buf;
    }
    if (s.head_dim != 64 && s.head_dim != 128) { snprintf(buf, sizeof buf, "%s: head_dim must be 64 or 128", nm); return buf; }
    if (s.n_q_heads % s.n_kv_heads) { snprintf(buf, sizeof buf, "%s: n_q_heads must be a multiple of n_kv_heads", nm); return buf; }
    const int G = s.n_q_heads / s.n_kv_heads;
    if (G != 1 && G != 2 && G != 4) { snprintf(buf, sizeof buf, "%s: n_q_heads / n_kv_heads must be 1, 2 or 4", nm); return buf; }
    const int ks[3] = {s.hidden, s.n_q_heads * s.head_dim, s.ffn};
    for (int k : ks)
      if (!units_ok(k, E, nullptr)) {
        snprintf(buf, sizeof buf, "%s: hidden, n_q_heads*head_dim and ffn must be %d x {1,2,3,4,6,8,12,16} (got %d)", nm, 64 * E, k);
        return buf;
      }
  }
  return "";
}

// Whether the persistent XCD-tensor-parallel CodePredictor kernel handles this config: bf16 or E4M3 weights,
// 8 KV heads of dimension 128 (one per XCD), and per-workgroup weight slices that fit its two
// register buffers (rows per wave and 16-byte units per lane).
bool xtp_capable(const tts_config& c) {
  const tts_stack_cfg& p = c.codepred;
  // bf16 weights: 8 per 16-byte unit; E4M3 codes: 16 (with one fp32 scale per row)
  const int E = c.weight_dtype == TTS_DTYPE_FP8_E4M3 ? 16 : 8;
  const int Ht = c.talker.hidden;
  const int ra_rows = xtp::RA_R * xtp::NW, ra_units = 64 * xtp::RA_K;
  const int rb_rows = xtp::RB_R * xtp::NW, rb_units = 64 * xtp::RB_K;
  if (c.weight_dtype != TTS_DTYPE_BF16 && c.weight_dtype != TTS_DTYPE_FP8_E4M3) return false;
  if (p.n_kv_heads != xtp::NX || p.head_dim != 128) return false;
  const int G = p.n_q_heads / p.n_kv_heads;
  if (G < 1 || G > 2 || p.n_q_heads != G * p.n_kv_heads || ((G + 2) * p.head_dim) % xtp::NR) return false;
  if (p.hidden % xtp::NR || p.hidden > xtp::HMAX || p.hidden % E || p.hidden / E > ra_units) return false;
  // A rows: q/k/v slice, gate/up slice, head slice
  if ((G + 2) * p.head_dim / xtp::NR > ra_rows) return false;
  // gate/up rows: the A buffer's rows, then the C buffer's
  if (p.ffn % (xtp::NX * xtp::NR) || 2 * (p.ffn / (xtp::NX * xtp::NR)) > ra_rows + xtp::RC_R * xtp::NW) return false;
  if (p.vocab % xtp::NWG || p.vocab / xtp::NWG > ra_rows) return false;
  // B rows: output projection, down projection, input projection (hidden / 32 rows each)
  if (p.hidden / xtp::NR > rb_rows || G * p.head_dim / E > rb_units) return false;
  if (p.ffn / xtp::NX > 768 || (p.ffn / xtp::NX) % E || (p.ffn / xtp::NX) / E > rb_units) return false;
  if (Ht != p.hidden && (Ht > 2048 || Ht % (xtp::NX * E) || (Ht / xtp::NX) / E > rb_units)) return false;
  if (p.n_layers > xtp::MAXL || c.n_acoustic != 15) return false;
  return true;
}

// Whether the lean persistent CodePredictor kernel (tts_xcp.h) handles this config: bf16 or E4M3 weights
// and the CodePredictor shape it is specialised to (hidden 1024, FFN 3072, 16 query and 8 KV heads
// of 128, vocabulary 2048, at most 5 layers, 15 codebooks), with no input projection or one from a
// Talker hidden of 2048.
bool xcp_capable(const tts_config& c) {
  const tts_stack_cfg& p = c.codepred;
  if (c.weight_dtype != TTS_DTYPE_BF16 && c.weight_dtype != TTS_DTYPE_FP8_E4M3) return false;
  if (p.hidden != xcp::H || p.ffn != xcp::F || p.n_q_heads != xcp::G * xcp::NX || p.n_kv_heads != xcp::NX ||
      p.head_dim != xcp::D || p.vocab != xcp::V)
    return false;
  if (p.n_layers < 1 || p.n_layers > xcp::MAXL || c.n_acoustic != 15) return false;
  return c.talker.hidden == xcp::H || c.talker.hidden == xcp::NX * xcp::KX;
}

// Whether the persistent Talker step kernel handles this config: bf16 or E4M3 weights, an fp32 KV cache,
// 8 KV heads of dimension 128 with 2 query heads each, and weight slices that fit its chunk shapes
// (see tts_xtk.h).
bool xtk_capable(const tts_config& c) {
  const tts_stack_cfg& t = c.talker;
  if ((c.weight_dtype != TTS_DTYPE_BF16 && c.weight_dtype != TTS_DTYPE_FP8_E4M3) || c.kv_dtype != TTS_DTYPE_F32) return false;
  if (t.n_kv_heads != xtp::NX || t.head_dim != 128 || t.n_q_heads != 2 * t.n_kv_heads) return false;
  // MFMA tiles of 16 rows: H / 32 output rows per rank in 1, 2 or 4 tiles (H in {512, 1024, 2048});
  // F / 256 gate + up rows per rank, at most 32 in LDS and one more tile in registers; the down
  // tiles' K steps (F / 256) split evenly over the waves that share a tile
  if (t.hidden != 512 && t.hidden != 1024 && t.hidden != 2048) return false;
  if (t.hidden > xtp::THMAX || t.hidden + xtp::NR > xtp::ISZ) return false;
  if (t.ffn % 256 || t.ffn / xtp::NX > xtp::TFXMAX || 2 * (t.ffn / 256) > 48) return false;
  if ((t.ffn / 256) % (xtp::NW / (t.hidden / 512))) return false;
  if (t.vocab % xtp::NWG || t.vocab / xtp::NWG > 16) return false;
  if (t.n_layers > xtp::TMAXL) return false;
  return true;
}

}  // namespace

// Whether the GEMM prefill handles this config: bf16 or E4M3 weights, head dimension 128 and every GEMM
// dimension of the Talker a multiple of the 64 x 64 x 64 tile.
bool prefill_gemm_capable(const tts_config& c) {
  const tts_stack_cfg& t = c.talker;
  if ((c.weight_dtype != TTS_DTYPE_BF16 && c.weight_dtype != TTS_DTYPE_FP8_E4M3) || t.head_dim != 128) return false;
  const int qd = t.n_q_heads * t.head_dim, kd = t.n_kv_heads * t.head_dim;
  return t.hidden % 64 == 0 && qd % 64 == 0 && kd % 64 == 0 && t.ffn % 64 == 0;
}

struct tts_ctx {
  tts_config cfg{};
  hipStream_t stream = nullptr;
  char* ws = nullptr;
  Layout L{};
  int device = 0;
  // workspace views
  DevState* st = nullptr;
  float *x = nullptr, *qkv = nullptr, *attn = nullptr, *h = nullptr, *part = nullptr, *logits = nullptr, *hT = nullptr;
  int32_t* counters = nullptr;
  float *cx = nullptr, *clog = nullptr;
  float *tcos = nullptr, *tsin = nullptr, *ccos = nullptr, *csin = nullptr;
  int32_t *next_tok = nullptr, *sem_tok = nullptr, *ac_codes = nullptr;
  uint8_t* history = nullptr;
  // weights
  StackW talker, cp;
  const void *embed_text = nullptr, *embed_sem = nullptr, *lm_head = nullptr, *proj = nullptr, *embed_ac = nullptr,
             *heads = nullptr;
  bool weights_ok = false;
  const float* ptab = nullptr;  // projected codebook rows P E_ac[j][a] (fp32), when formed
  // rows whose chunk sums of squares sit in the ssq buffer (the last ssq_out GEMM's output), or null
  const float* ssq_x = nullptr;
  int ssq_stride = 0, ssq_rows = 0, ssq_K = 0;
  // the split-K slices of the last defer_reduce GEMM, left for its reader to add, or null
  const float* dpart = nullptr;
  int dks = 0, drows = 0, dn = 0;
  // streaming text of the frame loop (tts_set_text_stream): ids [B, text_n], borrowed
  const int32_t* text_ids = nullptr;
  int text_n = 0, text_next = 0;
  // ragged prompts: per-stream first visible Talker position, right-aligned ids
  int32_t *kvstart = nullptr, *aids = nullptr;
  std::vector<int32_t> starts_host;  // source of the last start upload (kept alive for the copy)
  // per-stream stop (tts_set_stop): eos id (-1: none) and the caller's stop-frame array
  int eos_id = -1;
  int32_t* stop = nullptr;
  // host mirror of the device counters
  bool prefilled = false;
  int batch = 0, pos = 0, frames = 0;
  // captured frame graph
  bool have_graph = false;
  GraphKey gkey{};
  hipGraph_t graph = nullptr;
  hipGraphExec_t gexec = nullptr;
  hipStream_t cap_stream = nullptr;  // private stream used only to record the frame graph
  // persistent CodePredictor kernel
  bool xtp_ok = false;   // config supported
  int exec_mode = TTS_EXEC_PERSISTENT;  // persistent CodePredictor when supported (batch 1, greedy)
  xtp::CpDesc* cpdesc = nullptr;
  xtp::CpDesc* cpdesc_s = nullptr;  // exchange buffers in the static scratch array
  xtp::TkDesc* tkdesc_s = nullptr;
  char* scratch = nullptr;          // this device's static scratch array (device address)
  bool use_scratch = false;         // persistent launches take the *_s descriptors
  bool xtk_ok = false;   // persistent Talker step supported
  bool xcp_ok = false;   // the lean CodePredictor kernel supports the config (bf16 or E4M3)
  int32_t dev_mask = 0;  // persistent kernels the device allows (tts_persistent_allowed)
  // exchange error word seen from the host without blocking (device_err_check)
  uint32_t* errh = nullptr;  // pinned host copy
  hipEvent_t err_ev = nullptr;
  bool err_pending = false;
  bool pgemm_ok = false;  // GEMM prefill supported
  int prefill_mode = TTS_PREFILL_GEMM;
  xtp::TkDesc* tkdesc = nullptr;
  uint32_t* xerr = nullptr;
  std::string err;

  int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    err = buf;
    return code;
  }
  bool bf16() const { return cfg.weight_dtype == TTS_DTYPE_BF16; }
  bool fp8() const { return cfg.weight_dtype == TTS_DTYPE_FP8_E4M3; }
  bool tab16() const { return cfg.weight_dtype != TTS_DTYPE_F32; }  // gains and embedding tables are bf16
  size_t meb() const { return mat_bytes(cfg); }
  size_t teb() const { return tab_bytes(cfg); }
  // E4M3 matrices and their per-row scales, for the scale of a row pointer into any of them
  struct QTensor { uintptr_t base; size_t bytes; int K; const float* scale; };
  std::vector<QTensor> qtensors;
  const float* scale_of(const void* w, int K) const {
    const uintptr_t p = (uintptr_t)w;
    for (const QTensor& q : qtensors)
      if (p >= q.base && p < q.base + q.bytes && q.K == K && (p - q.base) % (size_t)K == 0) return q.scale + (p - q.base) / K;
    return nullptr;
  }
  size_t kvb() const { return kv_bytes(cfg); }
};

#define HIP_TRY(call)                                                                          \
  do {                                                                                         \
    hipError_t e_ = (call);                                                                    \
    if (e_ != hipSuccess) return ctx->fail(TTS_E_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

#define HIP_LAUNCH_CHECK()                                                                          \
  do {                                                                                              \
    hipError_t e_ = hipGetLastError();                                                              \
    if (e_ != hipSuccess) return ctx->fail(TTS_E_HIP, "kernel launch: %s", hipGetErrorString(e_)); \
  } while (0)

// Static scratch of tts_run_frames_noalloc: the persistent kernels' exchange buffers (intra-XCD
// rings, cross-XCD slots, argmax candidates, the Talker's attention partials) for callers that
// cannot allocate. Each GPU the library runs on holds one copy for the life of the process; every
// call on that GPU shares it.
constexpr size_t align256(size_t v) { return (v + 255) / 256 * 256; }
struct ScratchLayout {
  static constexpr size_t xin = 0;
  static constexpr size_t xcr = align256(xin + (size_t)xtp::NX * xtp::RING * xtp::ISZ * 8);
  static constexpr size_t cand = align256(xcr + (size_t)xtp::NWG * 2 * xtp::CSZ * 8);
  static constexpr size_t att = align256(cand + (size_t)2 * xtp::NWG * xtp::CAND * 8);
  static constexpr size_t total = align256(att + (size_t)xtp::NX * 2 * xtp::NR * xtp::ATS * 8);
};
constexpr size_t kScratchBytes = ScratchLayout::total;  // 2.1 MiB
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of this device's scratch array, looked up once per device (the array's
// name is a host-side stand-in in host code, not a device address). Call with the device current.
char* scratch_device_ptr(int device, hipError_t* err) {
  static std::mutex mu;
  static std::vector<char*> table;
  std::lock_guard<std::mutex> lock(mu);
  if (device < 0) return nullptr;
  if ((int)table.size() <= device) table.resize(device + 1, nullptr);
  if (!table[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e;
      return nullptr;
    }
    table[device] = (char*)p;
  }
  return table[device];
}

namespace {

// The persistent kernels' exchange error word, seen from the host without blocking: every call
// that may launch them queues a copy of the word into pinned host memory and an event behind its
// work (device_err_probe); the next such call reads that copy once the event has completed and
// fails with TTS_E_DEVICE, enqueueing nothing, when the word was set. The word stays set until
// tts_reset, so every later call reports it again.
int device_err_check(tts_ctx* ctx) {
  if (!ctx->err_pending) return TTS_OK;
  const hipError_t q = hipEventQuery(ctx->err_ev);
  if (q == hipErrorNotReady) return TTS_OK;
  ctx->err_pending = false;
  if (q != hipSuccess) return ctx->fail(TTS_E_HIP, "hipEventQuery: %s", hipGetErrorString(q));
  if (*ctx->errh)
    return ctx->fail(TTS_E_DEVICE,
                     "a persistent kernel timed out in an exchange (error word %u): outputs since the last clean call are "
                     "invalid; tts_reset clears the state",
                     *ctx->errh);
  return TTS_OK;
}
int device_err_probe(tts_ctx* ctx) {
  if (!(ctx->xtp_ok || ctx->xtk_ok) || ctx->exec_mode != TTS_EXEC_PERSISTENT) return TTS_OK;
  HIP_TRY(hipMemcpyAsync(ctx->errh, ctx->xerr, 4, hipMemcpyDeviceToHost, ctx->stream));
  HIP_TRY(hipEventRecord(ctx->err_ev, ctx->stream));
  ctx->err_pending = true;
  return TTS_OK;
}

// ---------------------------------------------------------------------------- GEMV dispatch

template <typename WT, int U, int M, bool PAIR, bool NORM>
int launch_gemv_t(tts_ctx* ctx, const GemvArgs& a) {
  // only instantiate row counts whose input slices fit the register budget
  if constexpr (M * U * WTraits<WT>::E > kGemvXRegs) {
    return ctx->fail(TTS_E_UNSUPPORTED, "gemv: M=%d with K=%d exceeds the register budget", M, a.K);
  } else {
    constexpr int RW = GemvShape<U, PAIR>::RW;
    const int rows_per_block = 4 * RW;
    const int blocks = (a.N + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((k_gemv<WT, U, M, PAIR, NORM>), dim3(blocks), dim3(256), 0, ctx->stream, a);
    HIP_LAUNCH_CHECK();
    return TTS_OK;
  }
}

template <typename WT, int U, bool PAIR, bool NORM>
int launch_gemv_m(tts_ctx* ctx, const GemvArgs& a) {
  switch (a.M) {
    case 1: return launch_gemv_t<WT, U, 1, PAIR, NORM>(ctx, a);
    case 2: return launch_gemv_t<WT, U, 2, PAIR, NORM>(ctx, a);
    case 4: return launch_gemv_t<WT, U, 4, PAIR, NORM>(ctx, a);
    case 8: return launch_gemv_t<WT, U, 8, PAIR, NORM>(ctx, a);
    default: return ctx->fail(TTS_E_UNSUPPORTED, "gemv: M=%d", a.M);
  }
}

template <typename WT, bool PAIR, bool NORM>
int launch_gemv_u(tts_ctx* ctx, const GemvArgs& a) {
  int U = 0;
  if (!units_ok(a.K, WTraits<WT>::E, &U)) return ctx->fail(TTS_E_SHAPE, "gemv: K=%d", a.K);
  switch (U) {
    case 1: return launch_gemv_m<WT, 1, PAIR, NORM>(ctx, a);
    case 2: return launch_gemv_m<WT, 2, PAIR, NORM>(ctx, a);
    case 3: return launch_gemv_m<WT, 3, PAIR, NORM>(ctx, a);
    case 4: return launch_gemv_m<WT, 4, PAIR, NORM>(ctx, a);
    case 6: return launch_gemv_m<WT, 6, PAIR, NORM>(ctx, a);
    case 8: return launch_gemv_m<WT, 8, PAIR, NORM>(ctx, a);
    case 12: return launch_gemv_m<WT, 12, PAIR, NORM>(ctx, a);
    case 16: return launch_gemv_m<WT, 16, PAIR, NORM>(ctx, a);
  }
  return ctx->fail(TTS_E_SHAPE, "gemv: K=%d", a.K);
}

template <typename WT>
int launch_gemv_w(tts_ctx* ctx, const GemvArgs& a) {
  const bool pair = a.epi == EPI_SWIGLU, norm = a.gain != nullptr;
  if (pair) return norm ? launch_gemv_u<WT, true, true>(ctx, a) : launch_gemv_u<WT, true, false>(ctx, a);
  return norm ? launch_gemv_u<WT, false, true>(ctx, a) : launch_gemv_u<WT, false, false>(ctx, a);
}

// Launch a GEMV over M input rows, chunked so that each launch holds at most
// kGemvXRegs input elements per lane. Chunks re-stream the weights.
int gemv(tts_ctx* ctx, GemvArgs a) {
  const int Mtot = a.M;
  const int E = mat_per_unit(ctx->cfg);
  const int U = a.K / (64 * E);
  if (ctx->fp8()) {
    for (int s = 0; s < kMaxSeg; ++s) {
      if (!a.w[s]) continue;
      a.wscale[s] = ctx->scale_of(a.w[s], a.K);
      if (!a.wscale[s]) return ctx->fail(TTS_E_STATE, "gemv: no E4M3 scale for a weight segment");
    }
  }
  int chunk = kMaxGemvM;
  while (chunk > 1 && chunk * U * E > kGemvXRegs) chunk >>= 1;
  if (a.src == SRC_VEC_THEN_TABLE && chunk < 2) return ctx->fail(TTS_E_SHAPE, "gemv: K=%d too large for paired rows", a.K);
  for (int m0 = 0; m0 < Mtot;) {
    int mc = std::min(chunk, Mtot - m0);
    while (mc & (mc - 1)) mc &= mc - 1;  // power of two rows per launch
    GemvArgs c = a;
    c.M = mc;
    if (a.src == SRC_VEC_THEN_TABLE) {
      c.x = a.x + (size_t)(m0 / 2) * a.x_stride;
      c.tok.offset = a.tok.offset + (m0 / 2) * a.tok.b_stride;
    } else if (a.src == SRC_TABLE) {
      c.tok.offset = a.tok.offset + m0 * a.tok.b_stride;
    } else {
      c.x = a.x + (size_t)m0 * a.x_stride;
    }
    c.y = a.y + (size_t)m0 * a.y_stride;
    if (a.res) c.res = a.res + (size_t)m0 * a.res_stride;
    if (a.xn_out) c.xn_out = a.xn_out + (size_t)m0 * a.xn_stride;
    if (m0 + mc < Mtot) c.bump_pos = c.bump_frame = 0;  // counters advance once, with the last chunk
    const int rc = ctx->fp8() ? launch_gemv_w<uint8_t>(ctx, c)
                   : (ctx->bf16() ? launch_gemv_w<uint16_t>(ctx, c) : launch_gemv_w<float>(ctx, c));
    if (rc) return rc;
    m0 += mc;
  }
  return TTS_OK;
}

// A projection of M >= kGemmMinRows rows (batched decode) as one MFMA GEMM instead of GEMV
// launches of at most kMaxGemvM rows: the GEMV keeps its input rows in registers, so at large K it
// takes 2 rows per launch and re-streams the weights for every pair, while the GEMM reads each
// weight tile once per 64 rows. Same operands and epilogues as the GEMV (RMSNorm via a row scale
// and the gain applied while A is loaded; the residual as C += result; SwiGLU through a staging
// buffer; gathered input rows staged first). Needs bf16 weights and 64-multiple row segments.
int gather(tts_ctx* ctx, int src, int M, int H, const float* vec, int vec_stride, const void* table, int table_rows, TokRef tok,
           float* out, int out_stride, bool f32_table = false, bool want_ssq = false);

bool gemm_routes(const tts_ctx* ctx, const GemvArgs& a) {
  if (!ctx->pgemm_ok || !(ctx->bf16() || ctx->fp8()) || a.M < kGemmMinRows || a.K % kGBK) return false;
  for (int s = 0; s < a.nseg; ++s)
    if (a.seg_rows[s] % kGBN) return false;
  if (a.epi == EPI_RESID && (a.res != a.y || a.res_stride != a.y_stride)) return false;
  if (a.epi == EPI_SWIGLU && (a.nseg != 2 || a.y_stride != a.N)) return false;
  return a.M <= ctx->cfg.max_batch * kPrefillChunk;  // the staging buffers' rows
}

// The MFMA GEMM on the context's weight type (E4M3: the segments' row scales looked up here).
int launch_gemm(tts_ctx* ctx, GemmArgs g, dim3 grid) {
  if (ctx->fp8()) {
    for (int s = 0; s < g.nseg; ++s) {
      g.wscale[s] = ctx->scale_of(g.w[s], g.K);
      if (!g.wscale[s]) return ctx->fail(TTS_E_STATE, "gemm: no E4M3 scale for a weight segment");
    }
    hipLaunchKernelGGL(k_gemm_bf16<true>, grid, dim3(256), 0, ctx->stream, g);
  } else {
    hipLaunchKernelGGL(k_gemm_bf16<false>, grid, dim3(256), 0, ctx->stream, g);
  }
  HIP_LAUNCH_CHECK();
  return TTS_OK;
}

int proj_gemm(tts_ctx* ctx, const GemvArgs& a) {
  char* w = ctx->ws;
  float *X = (float*)(w + ctx->L.px), *GU = (float*)(w + ctx->L.pgu), *RS = (float*)(w + ctx->L.ps),
        *SSQ = (float*)(w + ctx->L.ssq);
  // RMSNorm scales from the sums of squares the residual GEMM that wrote these rows left behind
  const bool use_ssq = a.gain && a.ssq_in && a.src == SRC_VEC && !a.xn_out && ctx->ssq_x == a.x &&
                       ctx->ssq_stride == a.x_stride && ctx->ssq_rows == a.M && ctx->ssq_K == a.K;
  const float* A = a.x;
  int lda = a.x_stride;
  if (a.src != SRC_VEC) {
    if (int rc = gather(ctx, a.src, a.M, a.K, a.x, a.x_stride, a.table, a.table_rows, a.tok, X, a.K)) return rc;
    A = X;
    lda = a.K;
  }
  GemmArgs g;
  std::memset(&g, 0, sizeof g);
  g.A = A; g.lda = lda; g.rs = a.gain ? RS : nullptr; g.gain = a.gain; g.M = a.M; g.K = a.K;
  int N = 0;
  for (int s = 0; s < a.nseg; ++s) { g.w[s] = a.w[s]; g.seg_rows[s] = a.seg_rows[s]; N += a.seg_rows[s]; }
  g.nseg = a.nseg; g.N = N;
  if (a.epi == EPI_SWIGLU) { g.C = GU; g.ldc = N; g.add = 0; }
  else { g.C = a.y; g.ldc = a.y_stride; g.add = a.epi == EPI_RESID ? 1 : 0; }
  // Split K so that about kGemmWgs workgroups stream the weights (a decode GEMM has few row tiles:
  // unsplit, N/64 workgroups would each walk all of K with one load in flight). Each slice writes
  // its partial tile; k_splitk_reduce then adds them into C in slice order (with the residual
  // first for a residual epilogue), so results do not depend on workgroup timing.
  // Few rows (decode): k_gemm_dec, each workgroup's weight fragments loaded straight to registers.
  const bool dec = ctx->bf16() && a.M <= 64;
  const int rw = dec ? dec_rw(a.M, a.seg_rows, a.nseg) : 1;
  const int tiles = (N / kGBN) * ((a.M + kGBM - 1) / kGBM);
  int ks = 1, kslice = a.K;
  if (dec) {
    ks = dec_split(N, a.K, a.M, rw, &kslice);
  } else {
    ks = std::max(1, std::min(a.K / kGBK, kGemmWgs / tiles));
    kslice = ((a.K / kGBK + ks - 1) / ks) * kGBK;
    ks = (a.K + kslice - 1) / kslice;
    if (ks > 1 && (size_t)ks * tiles > (size_t)kGemmWgs)
      return ctx->fail(TTS_E_STATE, "gemm: %d K slices of %d tiles exceed the partial-tile buffer", ks, tiles);
  }
  g.kslice = kslice;
  g.part = (float*)(w + ctx->L.pks);
  if (dec && ks > 1 && (size_t)ks * a.M * N * 4 > ctx->L.ssq - ctx->L.pks)
    return ctx->fail(TTS_E_STATE, "gemm: %d K slices of %d x %d rows exceed the partial buffer", ks, a.M, N);
  if (use_ssq) {
    g.rs = nullptr; g.ssq = SSQ; g.nchunk = (a.K + 255) / 256; g.eps = ctx->cfg.rms_eps;
  } else if (a.gain) {
    hipLaunchKernelGGL(k_rowscale, dim3((a.M + 3) / 4), dim3(256), 0, ctx->stream, A, lda, a.M, a.K, ctx->cfg.rms_eps, RS);
    HIP_LAUNCH_CHECK();
    if (a.xn_out) {
      hipLaunchKernelGGL(k_norm_rows<uint16_t>, dim3(a.M), dim3(256), 0, ctx->stream, A, lda, RS, a.gain, a.K, a.xn_out, a.xn_stride);
      HIP_LAUNCH_CHECK();
    }
  }
  if (dec) {
    if (a.M <= 16) hipLaunchKernelGGL((k_gemm_dec<1, 256, 1>), dim3(N / 64, 1, ks), dim3(256), 0, ctx->stream, g);
    else if (a.M <= 32) hipLaunchKernelGGL((k_gemm_dec<2, 256, 1>), dim3(N / 64, 1, ks), dim3(256), 0, ctx->stream, g);
    else if (rw == 4) hipLaunchKernelGGL((k_gemm_dec<4, 128, 4>), dim3(N / 256, 1, ks), dim3(256), 0, ctx->stream, g);
    else hipLaunchKernelGGL((k_gemm_dec<4, 128, 1>), dim3(N / 64, 1, ks), dim3(256), 0, ctx->stream, g);
  } else if (int rc = launch_gemm(ctx, g, dim3(N / kGBN, (a.M + kGBM - 1) / kGBM, ks))) {
    return rc;
  }
  HIP_LAUNCH_CHECK();
  // ssq_out: a residual GEMM, or a plain store (the CodePredictor's input projection), also leaves
  // the written rows' 256-column chunk sums of squares
  const bool ssq_out = a.ssq_out && (a.epi == EPI_RESID || a.epi == EPI_STORE) && N % 256 == 0;
  if (a.epi == EPI_SWIGLU) {
    // the slices' gate and up sums meet in the SwiGLU pass (no separate reduction)
    if (ks > 1)
      hipLaunchKernelGGL(k_splitk_swiglu, dim3(std::min((a.M * a.N + 255) / 256, 4096)), dim3(256), 0, ctx->stream, g.part, a.M,
                         a.N, ks, a.y, a.y_stride);
    else
      hipLaunchKernelGGL(k_swiglu_rows, dim3(std::min((a.M * a.N + 255) / 256, 4096)), dim3(256), 0, ctx->stream, GU, a.M, a.N, a.y);
    HIP_LAUNCH_CHECK();
  } else if (ks > 1 && a.defer_reduce && a.epi == EPI_STORE && !ssq_out) {
    // the reader adds the slices itself (in the same order)
    ctx->dpart = g.part; ctx->dks = ks; ctx->drows = a.M; ctx->dn = N;
  } else if (ks > 1 || ssq_out) {
    // slices added in order (with the residual first); a residual GEMM also leaves the new rows'
    // sums of squares for the RMSNorm of the GEMM that reads them next
    hipLaunchKernelGGL(k_splitk_reduce, dim3((N + 255) / 256, a.M), dim3(256), 0, ctx->stream, g.C, g.ldc, g.part, a.M, N,
                       ks > 1 ? ks : 0, ks > 1 ? g.add : 1, ssq_out ? SSQ : nullptr);
    HIP_LAUNCH_CHECK();
  }
  if (ssq_out) {
    ctx->ssq_x = a.y; ctx->ssq_stride = a.y_stride; ctx->ssq_rows = a.M; ctx->ssq_K = N;
  } else if (a.y == ctx->ssq_x) {
    ctx->ssq_x = nullptr;
  }
  if (a.bump_pos || a.bump_frame) {
    hipLaunchKernelGGL(k_bump_state, dim3(1), dim3(64), 0, ctx->stream, ctx->st, a.bump_pos, a.bump_frame);
    HIP_LAUNCH_CHECK();
  }
  return TTS_OK;
}

int proj(tts_ctx* ctx, GemvArgs a) {
  if (gemm_routes(ctx, a)) return proj_gemm(ctx, a);
  ctx->ssq_x = nullptr;  // the GEMV leaves no sums of squares
  return gemv(ctx, a);
}

// ---------------------------------------------------------------------------- attention dispatch

template <typename WT, typename KT, int G, int M, int D>
int launch_attn_t(tts_ctx* ctx, const AttnArgs& a, int B) {
  hipLaunchKernelGGL((k_attn<WT, KT, G, M, D>), dim3(a.nsplit, a.nkv, B), dim3(256), 0, ctx->stream, a);
  HIP_LAUNCH_CHECK();
  return TTS_OK;
}

template <typename WT, typename KT, int G, int M>
int launch_attn_d(tts_ctx* ctx, const AttnArgs& a, int B) {
  if (a.d == 64) return launch_attn_t<WT, KT, G, M, 64>(ctx, a, B);
  if (a.d == 128) return launch_attn_t<WT, KT, G, M, 128>(ctx, a, B);
  return ctx->fail(TTS_E_SHAPE, "attention: head_dim %d", a.d);
}

template <typename WT, typename KT, int G>
int launch_attn_m(tts_ctx* ctx, const AttnArgs& a, int B) {
  if (a.M == 1) return launch_attn_d<WT, KT, G, 1>(ctx, a, B);
  if (a.M == 2) return launch_attn_d<WT, KT, G, 2>(ctx, a, B);
  return ctx->fail(TTS_E_SHAPE, "attention: %d new positions", a.M);
}

template <typename WT, typename KT>
int launch_attn_g(tts_ctx* ctx, const AttnArgs& a, int B) {
  const int G = a.nq / a.nkv;
  if (G == 1) return launch_attn_m<WT, KT, 1>(ctx, a, B);
  if (G == 2) return launch_attn_m<WT, KT, 2>(ctx, a, B);
  if (G == 4) return launch_attn_m<WT, KT, 4>(ctx, a, B);
  return ctx->fail(TTS_E_SHAPE, "attention: %d query heads per KV head", G);
}

int attention(tts_ctx* ctx, const AttnArgs& a, int B) {
  if (ctx->tab16()) return launch_attn_g<uint16_t, float>(ctx, a, B);
  return launch_attn_g<float, float>(ctx, a, B);
}

// ---------------------------------------------------------------------------- building blocks

TokRef tokref(const int32_t* base, int b_stride, int f_stride, int offset, int use_frame) {
  TokRef r;
  r.base = base; r.b_stride = b_stride; r.f_stride = f_stride; r.offset = offset; r.use_frame = use_frame;
  return r;
}
URef uref(const float* base, int b_stride, int f_stride, int offset, int use_frame) {
  URef r;
  r.base = base; r.b_stride = b_stride; r.f_stride = f_stride; r.offset = offset; r.use_frame = use_frame;
  return r;
}

GemvArgs gemv_args(tts_ctx* ctx) {
  GemvArgs a;
  std::memset(&a, 0, sizeof a);
  a.nseg = 1;
  a.eps = ctx->cfg.rms_eps;
  a.st = ctx->st;
  return a;
}

// One pass of a decoder stack over Mp new positions per stream (rows b*Mp+m
// of x, hidden H). Position of row m: pos_const + m, or the device Talker
// position when pos_from_state. KV caches [layers][B][nkv][cap][d].
// kvstart: per-stream first visible cache position (ragged Talker prompts), or nullptr.
int stack_step(tts_ctx* ctx, const StackW& S, float* x, int B, int Mp, int pos_const, int pos_from_state, void* kc,
               void* vc, int cap, int nsplit, const float* rc, const float* rs, bool nontemporal,
               const int32_t* kvstart = nullptr, bool in_ssq = false) {
  const tts_stack_cfg& c = S.c;
  const int rows = B * Mp;
  const int qd = c.n_q_heads * c.head_dim, kd = c.n_kv_heads * c.head_dim;
  const int qkv_n = qd + 2 * kd;
  // per-layer cache stride uses the allocated stream capacity, not the live batch
  const size_t layer_cache = (size_t)ctx->cfg.max_batch * c.n_kv_heads * cap * c.head_dim * ctx->kvb();
  // x was written outside this stack; in_ssq: by a gather that left its rows' sums of squares
  // (proj_gemm still checks that they describe these rows)
  if (!in_ssq) ctx->ssq_x = nullptr;
  for (int l = 0; l < c.n_layers; ++l) {
    const Layer& W = S.layers[l];
    // RMSNorm + QKV (after layer 0 the previous down projection left x's sums of squares)
    GemvArgs a = gemv_args(ctx);
    a.ssq_in = l > 0 || in_ssq;
    a.w[0] = W.wq; a.w[1] = W.wk; a.w[2] = W.wv;
    a.seg_rows[0] = qd; a.seg_rows[1] = kd; a.seg_rows[2] = kd;
    a.nseg = 3; a.N = qkv_n; a.K = c.hidden; a.M = rows;
    a.src = SRC_VEC; a.x = x; a.x_stride = c.hidden;
    a.gain = W.attn_norm;
    a.y = ctx->qkv; a.y_stride = qkv_n; a.epi = EPI_STORE; a.nontemporal = nontemporal;
    a.defer_reduce = 1;  // the attention adds a split GEMM's slices itself
    ctx->dpart = nullptr;
    if (int rc_ = proj(ctx, a)) return rc_;
    // q/k norm + RoPE + KV append + attention
    AttnArgs t;
    std::memset(&t, 0, sizeof t);
    t.qkv = ctx->qkv; t.qkv_stride = qkv_n; t.M = Mp;
    if (ctx->dpart) {
      t.qkv_part = ctx->dpart; t.qkv_ks = ctx->dks; t.qkv_rows = ctx->drows; t.qkv_n = ctx->dn;
      ctx->dpart = nullptr;
    }
    t.nq = c.n_q_heads; t.nkv = c.n_kv_heads; t.d = c.head_dim;
    t.q_norm = W.q_norm; t.k_norm = W.k_norm; t.eps = ctx->cfg.rms_eps;
    t.rope_cos = rc; t.rope_sin = rs;
    t.pos_const = pos_const; t.pos_from_state = pos_from_state;
    t.kc = (char*)kc + l * layer_cache; t.vc = (char*)vc + l * layer_cache;
    t.cap = cap; t.chunk = nsplit == 1 ? cap : attn_chunk(B, c.n_kv_heads, cap); t.nsplit = nsplit;
    t.out = ctx->attn; t.out_stride = qd; t.part = ctx->part; t.counters = ctx->counters; t.st = ctx->st;
    t.kvstart = kvstart;
    if (int rc_ = attention(ctx, t, B)) return rc_;
    // O projection + residual
    a = gemv_args(ctx);
    a.w[0] = W.wo; a.seg_rows[0] = c.hidden; a.N = c.hidden; a.K = qd; a.M = rows;
    a.src = SRC_VEC; a.x = ctx->attn; a.x_stride = qd;
    a.y = x; a.y_stride = c.hidden; a.res = x; a.res_stride = c.hidden; a.epi = EPI_RESID; a.nontemporal = nontemporal;
    a.ssq_out = 1;
    if (int rc_ = proj(ctx, a)) return rc_;
    // RMSNorm + gate/up + SwiGLU
    a = gemv_args(ctx);
    a.ssq_in = 1;
    a.w[0] = W.wg; a.w[1] = W.wu; a.seg_rows[0] = c.ffn; a.seg_rows[1] = c.ffn; a.nseg = 2;
    a.N = c.ffn; a.K = c.hidden; a.M = rows;
    a.src = SRC_VEC; a.x = x; a.x_stride = c.hidden; a.gain = W.mlp_norm;
    a.y = ctx->h; a.y_stride = c.ffn; a.epi = EPI_SWIGLU; a.nontemporal = nontemporal;
    if (int rc_ = proj(ctx, a)) return rc_;
    // down projection + residual
    a = gemv_args(ctx);
    a.w[0] = W.wd; a.seg_rows[0] = c.hidden; a.N = c.hidden; a.K = c.ffn; a.M = rows;
    a.src = SRC_VEC; a.x = ctx->h; a.x_stride = c.ffn;
    a.y = x; a.y_stride = c.hidden; a.res = x; a.res_stride = c.hidden; a.epi = EPI_RESID; a.nontemporal = nontemporal;
    a.ssq_out = 1;
    if (int rc_ = proj(ctx, a)) return rc_;
  }
  return TTS_OK;
}

// Talker final norm + semantic head: logits = W_lm RMSNorm(x); the normed
// hidden (h_T, which conditions the CodePredictor) is written as well.
int talker_head(tts_ctx* ctx, int B, int bump_pos, int bump_frame) {
  const auto& t = ctx->cfg.talker;
  GemvArgs a = gemv_args(ctx);
  a.bump_pos = bump_pos; a.bump_frame = bump_frame;
  a.w[0] = ctx->lm_head; a.seg_rows[0] = t.vocab; a.N = t.vocab; a.K = t.hidden; a.M = B;
  a.src = SRC_VEC; a.x = ctx->x; a.x_stride = t.hidden; a.gain = ctx->talker.final_norm;
  a.y = ctx->logits; a.y_stride = t.vocab; a.epi = EPI_STORE;
  a.xn_out = ctx->hT; a.xn_stride = t.hidden; a.nontemporal = 1;
  return proj(ctx, a);
}

// Talker prompt pass as GEMMs: chunks of up to kPrefillChunk positions per stream, M = B x chunk
// rows per GEMM; the last chunk's last row per stream goes to ctx->x for the head.
int prefill_gemm(tts_ctx* ctx, const int32_t* ids, int B, int n) {
  const auto& c = ctx->cfg;
  const tts_stack_cfg& t = c.talker;
  const int H = t.hidden, d = t.head_dim, qd = t.n_q_heads * d, kd = t.n_kv_heads * d, nqkv = qd + 2 * kd, F = t.ffn;
  const size_t layer_cache = (size_t)c.max_batch * t.n_kv_heads * c.max_cache_steps * d * ctx->kvb();
  char* w = ctx->ws;
  float *X = (float*)(w + ctx->L.px), *QKV = (float*)(w + ctx->L.pqkv), *Q = (float*)(w + ctx->L.pq),
        *O = (float*)(w + ctx->L.po), *GU = (float*)(w + ctx->L.pgu), *Hh = (float*)(w + ctx->L.ph),
        *RS = (float*)(w + ctx->L.ps);
  auto gemm = [&](const float* A, int lda, const float* rs, const void* gain, std::initializer_list<std::pair<const void*, int>> segs,
                  float* C, int N, int K, int M, int add) -> int {
    GemmArgs a;
    std::memset(&a, 0, sizeof a);
    a.A = A; a.lda = lda; a.rs = rs; a.gain = gain; a.C = C; a.ldc = N; a.M = M; a.N = N; a.K = K; a.add = add; a.kslice = K;
    for (auto& sg : segs) { a.w[a.nseg] = sg.first; a.seg_rows[a.nseg] = sg.second; ++a.nseg; }
    return launch_gemm(ctx, a, dim3(N / kGBN, (M + kGBM - 1) / kGBM));
  };
  for (int p0 = 0; p0 < n; p0 += kPrefillChunk) {
    const int P = std::min(kPrefillChunk, n - p0), M = B * P;
    // A chunk of 16..64 rows (a prompt of one or a few streams) takes the batched decode's split-K
    // route (proj_gemm): one 64-row tile per 64 weight rows would leave most CUs idle, while K
    // slices let about 256 workgroups stream each matrix, and the slices are added in order.
    // Wider chunks fill the chip with row tiles.
    const bool split = M >= kGemmMinRows && M <= 64;
    hipLaunchKernelGGL(k_embed_rows<uint16_t>, dim3(M), dim3(256), 0, ctx->stream, ids, n, p0, P, c.text_vocab, ctx->embed_text, H, X);
    HIP_LAUNCH_CHECK();
    ctx->ssq_x = nullptr;  // X holds fresh rows: no sums of squares are known for them
    for (int l = 0; l < t.n_layers; ++l) {
      const Layer& W = ctx->talker.layers[l];
      char* kc = w + ctx->L.tk + l * layer_cache;
      char* vc = w + ctx->L.tv + l * layer_cache;
      if (split) {
        GemvArgs a = gemv_args(ctx);
        a.ssq_in = l > 0;  // the previous layer's down projection left X's sums of squares
        a.w[0] = W.wq; a.w[1] = W.wk; a.w[2] = W.wv;
        a.seg_rows[0] = qd; a.seg_rows[1] = kd; a.seg_rows[2] = kd;
        a.nseg = 3; a.N = nqkv; a.K = H; a.M = M;
        a.src = SRC_VEC; a.x = X; a.x_stride = H; a.gain = W.attn_norm;
        a.y = QKV; a.y_stride = nqkv; a.epi = EPI_STORE;
        if (int rc = proj_gemm(ctx, a)) return rc;
      } else {
        hipLaunchKernelGGL(k_rowscale, dim3((M + 3) / 4), dim3(256), 0, ctx->stream, X, H, M, H, c.rms_eps, RS);
        HIP_LAUNCH_CHECK();
        if (int rc = gemm(X, H, RS, W.attn_norm, {{W.wq, qd}, {W.wk, kd}, {W.wv, kd}}, QKV, nqkv, H, M, 0)) return rc;
      }
      QkArgs q;
      std::memset(&q, 0, sizeof q);
      q.qkv = QKV; q.q = Q; q.kc = kc; q.vc = vc; q.q_norm = W.q_norm; q.k_norm = W.k_norm;
      q.rope_cos = ctx->tcos; q.rope_sin = ctx->tsin;
      q.M = M; q.P = P; q.p0 = p0; q.nq = t.n_q_heads; q.nkv = t.n_kv_heads; q.cap = c.max_cache_steps; q.eps = c.rms_eps;
      const int items = M * (t.n_q_heads + 2 * t.n_kv_heads);
      hipLaunchKernelGGL((k_qk_rope_kv<uint16_t, float>), dim3((items + 3) / 4), dim3(256), 0, ctx->stream, q);
      HIP_LAUNCH_CHECK();
      PAttnArgs pa;
      std::memset(&pa, 0, sizeof pa);
      pa.q = Q; pa.kc = kc; pa.vc = vc; pa.out = O; pa.P = P; pa.p0 = p0; pa.nq = t.n_q_heads; pa.nkv = t.n_kv_heads;
      pa.cap = c.max_cache_steps;
      pa.kvstart = ctx->kvstart;
      hipLaunchKernelGGL(k_prefill_attn<float>, dim3((P + 3) / 4, t.n_q_heads, B), dim3(256), 0, ctx->stream, pa);
      HIP_LAUNCH_CHECK();
      if (split) {
        // output projection + residual (leaves X's sums of squares), RMSNorm + gate/up + SwiGLU,
        // down projection + residual (leaves them again)
        GemvArgs a = gemv_args(ctx);
        a.w[0] = W.wo; a.seg_rows[0] = H; a.N = H; a.K = qd; a.M = M;
        a.src = SRC_VEC; a.x = O; a.x_stride = qd;
        a.y = X; a.y_stride = H; a.res = X; a.res_stride = H; a.epi = EPI_RESID; a.ssq_out = 1;
        if (int rc = proj_gemm(ctx, a)) return rc;
        a = gemv_args(ctx);
        a.ssq_in = 1;
        a.w[0] = W.wg; a.w[1] = W.wu; a.seg_rows[0] = F; a.seg_rows[1] = F; a.nseg = 2;
        a.N = F; a.K = H; a.M = M;
        a.src = SRC_VEC; a.x = X; a.x_stride = H; a.gain = W.mlp_norm;
        a.y = Hh; a.y_stride = F; a.epi = EPI_SWIGLU;
        if (int rc = proj_gemm(ctx, a)) return rc;
        a = gemv_args(ctx);
        a.w[0] = W.wd; a.seg_rows[0] = H; a.N = H; a.K = F; a.M = M;
        a.src = SRC_VEC; a.x = Hh; a.x_stride = F;
        a.y = X; a.y_stride = H; a.res = X; a.res_stride = H; a.epi = EPI_RESID; a.ssq_out = 1;
        if (int rc = proj_gemm(ctx, a)) return rc;
      } else {
        if (int rc = gemm(O, qd, nullptr, nullptr, {{W.wo, H}}, X, H, qd, M, 1)) return rc;
        hipLaunchKernelGGL(k_rowscale, dim3((M + 3) / 4), dim3(256), 0, ctx->stream, X, H, M, H, c.rms_eps, RS);
        HIP_LAUNCH_CHECK();
        if (int rc = gemm(X, H, RS, W.mlp_norm, {{W.wg, F}, {W.wu, F}}, GU, 2 * F, H, M, 0)) return rc;
        hipLaunchKernelGGL(k_swiglu_rows, dim3(std::min((M * F + 255) / 256, 4096)), dim3(256), 0, ctx->stream, GU, M, F, Hh);
        HIP_LAUNCH_CHECK();
        if (int rc = gemm(Hh, F, nullptr, nullptr, {{W.wd, H}}, X, H, F, M, 1)) return rc;
      }
    }
    if (p0 + P == n) {
      hipLaunchKernelGGL(k_last_rows, dim3(B), dim3(256), 0, ctx->stream, X, P, H, ctx->x);
      HIP_LAUNCH_CHECK();
    }
  }
  ctx->ssq_x = nullptr;  // the staging rows' sums of squares are of no later GEMM's input
  return TTS_OK;
}

int talker_stack(tts_ctx* ctx, int B, int pos_const, int pos_from_state) {
  const auto& c = ctx->cfg;
  return stack_step(ctx, ctx->talker, ctx->x, B, 1, pos_const, pos_from_state, ctx->ws + ctx->L.tk, ctx->ws + ctx->L.tv,
                    c.max_cache_steps, ctx->L.nsplit, ctx->tcos, ctx->tsin, true, ctx->kvstart);
}

// Talker input from a frame's 16 codes (codebook t of stream b at tok refs).
// text: the streaming text term (see EmbedArgs), or nullptr for none; text_n: its index bound.
int embed_sum(tts_ctx* ctx, int B, const TokRef* refs, const TokRef* text = nullptr, int text_n = 0) {
  const auto& c = ctx->cfg;
  EmbedArgs e;
  std::memset(&e, 0, sizeof e);
  e.ntab = 1 + c.n_acoustic;
  e.H = c.talker.hidden;
  const size_t ac_table = (size_t)c.codepred.vocab * c.talker.hidden * ctx->teb();
  e.table[0] = ctx->embed_sem;
  e.rows[0] = c.talker.vocab;
  e.tok[0] = refs[0];
  for (int j = 1; j <= c.n_acoustic; ++j) {
    e.table[j] = (const char*)ctx->embed_ac + (j - 1) * ac_table;
    e.rows[j] = c.codepred.vocab;
    e.tok[j] = refs[j];
  }
  e.x = ctx->x; e.x_stride = c.talker.hidden; e.st = ctx->st;
  if (text) {
    e.text_table = ctx->embed_text;
    e.text = *text;
    e.text_rows = c.text_vocab;
    e.text_n = text_n;
  }
  const int gx = (c.talker.hidden + 255) / 256;
  if (ctx->tab16()) hipLaunchKernelGGL(k_embed_sum<uint16_t>, dim3(gx, B), dim3(256), 0, ctx->stream, e);
  else hipLaunchKernelGGL(k_embed_sum<float>, dim3(gx, B), dim3(256), 0, ctx->stream, e);
  HIP_LAUNCH_CHECK();
  return TTS_OK;
}

int gather(tts_ctx* ctx, int src, int M, int H, const float* vec, int vec_stride, const void* table, int table_rows, TokRef tok,
           float* out, int out_stride, bool f32_table, bool want_ssq) {
  GatherArgs g;
  std::memset(&g, 0, sizeof g);
  g.src = src; g.M = M; g.H = H; g.vec = vec; g.vec_stride = vec_stride; g.table = table; g.table_rows = table_rows; g.tok = tok;
  g.x = out; g.x_stride = out_stride; g.st = ctx->st;
  if (out == ctx->ssq_x) ctx->ssq_x = nullptr;
  const int gx = (H + 255) / 256;
  // the rows' chunk sums of squares (into the buffer sized for max_batch x kPrefillChunk rows of
  // the widest hidden size), for the RMSNorm of the GEMM that reads them next
  if (want_ssq && H % 256 == 0 && (size_t)M <= (size_t)ctx->cfg.max_batch * kPrefillChunk) g.ssq = (float*)(ctx->ws + ctx->L.ssq);
  if (ctx->tab16() && !f32_table) hipLaunchKernelGGL(k_gather<uint16_t>, dim3(gx, M), dim3(256), 0, ctx->stream, g);
  else hipLaunchKernelGGL(k_gather<float>, dim3(gx, M), dim3(256), 0, ctx->stream, g);
  HIP_LAUNCH_CHECK();
  if (g.ssq) {
    ctx->ssq_x = out; ctx->ssq_stride = out_stride; ctx->ssq_rows = M; ctx->ssq_K = H;
  }
  return TTS_OK;
}

int sample(tts_ctx* ctx, const float* logits, int l_stride, int B, int V, const tts_sampling& s, URef u, uint8_t* hist,
           int h_stride, int mark, int32_t* out, int ob, int of, int oo, int ouf, int32_t* next, const int32_t* forced,
           int fs, int fo) {
  SampleArgs a;
  std::memset(&a, 0, sizeof a);
  a.logits = logits; a.l_stride = l_stride; a.V = V;
  a.do_sample = s.do_sample; a.top_k = s.top_k; a.top_p = s.top_p; a.temperature = s.temperature;
  a.penalty = s.repetition_penalty;
  a.u = u; a.history = hist; a.h_stride = h_stride; a.mark_history = mark;
  a.out = out; a.out_b_stride = ob; a.out_f_stride = of; a.out_offset = oo; a.out_use_frame = ouf;
  a.next = next; a.forced = forced; a.forced_stride = fs; a.forced_offset = fo; a.st = ctx->st;
  hipLaunchKernelGGL(k_sample, dim3(B), dim3(256), 0, ctx->stream, a);
  HIP_LAUNCH_CHECK();
  return TTS_OK;
}

// The 15 CodePredictor steps. semantic: token ref of the semantic id per
// stream. Acoustic token j of stream b goes to out (refs with offset j-1);
// logits (optional) to logits_out + b*15*Va + (j-1)*Va. u: uniform refs with
// offset of acoustic 1 (incremented per step). forced: [B][15] or nullptr.
// The persistent CodePredictor kernels handle batch 1 with greedy acoustic tokens; the hidden-1024
// one also draws sampled acoustic tokens in-kernel for top_k in 1..64 (others: per-op kernels).
bool use_xtp(tts_ctx* ctx, int B, const tts_sampling& ac) {
  if (!ctx->xtp_ok || ctx->exec_mode != TTS_EXEC_PERSISTENT || B != 1) return false;
  return !ac.do_sample || (ctx->xcp_ok && ac.top_k >= 1 && ac.top_k <= xcp::KS);
}

// u: the uniforms of acoustic 1 of the frame at u[u_offset + (use_frame ? frame * u_f_stride : 0)],
// then one per step (read only when ac samples).
int codepred_frame_xtp(tts_ctx* ctx, const int32_t* semantic, const int32_t* forced, int32_t* codes, int f_stride, int use_frame,
                       float* logits_out, const tts_sampling& ac, const float* u, int u_f_stride, int u_offset) {
  xtp::CpCall call;
  call.do_sample = ac.do_sample ? 1 : 0;
  call.top_k = ac.top_k;
  call.top_p = ac.top_p;
  call.temperature = ac.temperature;
  call.u = u;
  call.u_f_stride = u_f_stride;
  call.u_offset = u_offset;
  call.desc = ctx->use_scratch ? ctx->cpdesc_s : ctx->cpdesc;
  call.semantic = semantic;
  call.forced = forced;
  call.codes = codes;
  call.f_stride = f_stride;
  call.use_frame = use_frame;
  call.logits = logits_out;
  call.next_tok = nullptr;
  if (ctx->xcp_ok && ctx->fp8()) hipLaunchKernelGGL(xcp::k_cp_frame<uint8_t>, dim3(xtp::NWG), dim3(xtp::NT), 0, ctx->stream, call);
  else if (ctx->xcp_ok) hipLaunchKernelGGL(xcp::k_cp_frame<uint16_t>, dim3(xtp::NWG), dim3(xtp::NT), 0, ctx->stream, call);
  else if (ctx->fp8()) hipLaunchKernelGGL(xtp::k_cp_frame<uint8_t>, dim3(xtp::NWG), dim3(xtp::NT), 0, ctx->stream, call);
  else hipLaunchKernelGGL(xtp::k_cp_frame<uint16_t>, dim3(xtp::NWG), dim3(xtp::NT), 0, ctx->stream, call);
  HIP_LAUNCH_CHECK();
  return TTS_OK;
}

// The persistent Talker step (batch 1): all layers, final norm and semantic head for the position
// in the device counters; bumps the position (and the frame) at its end.
bool use_xtk(tts_ctx* ctx, int B) { return ctx->xtk_ok && ctx->exec_mode == TTS_EXEC_PERSISTENT && B == 1; }

int talker_step_xtk(tts_ctx* ctx, int bump_pos, int bump_frame) {
  xtp::TkCall call;
  call.desc = ctx->use_scratch ? ctx->tkdesc_s : ctx->tkdesc;
  call.bump_pos = bump_pos;
  call.bump_frame = bump_frame;
  if (ctx->fp8()) hipLaunchKernelGGL(xtp::k_talker_step<uint8_t>, dim3(xtp::NWG), dim3(xtp::NT), 0, ctx->stream, call);
  else hipLaunchKernelGGL(xtp::k_talker_step<uint16_t>, dim3(xtp::NWG), dim3(xtp::NT), 0, ctx->stream, call);
  HIP_LAUNCH_CHECK();
  return TTS_OK;
}

int codepred_frame(tts_ctx* ctx, int B, TokRef semantic, const tts_sampling& ac, URef u, const int32_t* forced,
                   int32_t* out, int ob, int of, int oo, int ouf, float* logits_out) {
  const auto& c = ctx->cfg;
  const int Hc = c.codepred.hidden, Ht = c.talker.hidden, Va = c.codepred.vocab;
  const size_t ac_table = (size_t)Va * Ht * ctx->teb();
  const size_t head_sz = (size_t)Va * Hc * ctx->meb();
  void* kc = ctx->ws + ctx->L.ck;
  void* vc = ctx->ws + ctx->L.cv;
  for (int j = 1; j <= c.n_acoustic; ++j) {
    const int Mp = (j == 1) ? 2 : 1;
    bool gathered = false;  // the input rows came from a gather that left their sums of squares
    // CodePredictor input rows
    if (j == 1) {
      if (ctx->proj) {
        GemvArgs a = gemv_args(ctx);
        a.w[0] = ctx->proj; a.seg_rows[0] = Hc; a.N = Hc; a.K = Ht; a.M = 2 * B;
        a.src = SRC_VEC_THEN_TABLE; a.x = ctx->hT; a.x_stride = Ht; a.table = ctx->embed_sem; a.table_rows = c.talker.vocab;
        a.tok = semantic;
        a.y = ctx->cx; a.y_stride = Hc; a.epi = EPI_STORE;
        a.ssq_out = 1;  // the rows' sums of squares for the first RMSNorm (on the GEMM route)
        if (int rc = proj(ctx, a)) return rc;
        gathered = true;
      } else {
        if (int rc = gather(ctx, SRC_VEC_THEN_TABLE, 2 * B, Hc, ctx->hT, Ht, ctx->embed_sem, c.talker.vocab, semantic, ctx->cx, Hc,
                            false, true))
          return rc;
        gathered = true;
      }
    } else {
      const void* table = (const char*)ctx->embed_ac + (size_t)(j - 2) * ac_table;
      TokRef prev = tokref(ctx->next_tok, 1, 0, 0, 0);
      if (ctx->ptab) {
        // the projected row P E_ac[j - 2][a] from the table (a linear map of a row is that row of
        // the mapped table)
        if (int rc = gather(ctx, SRC_TABLE, B, Hc, nullptr, 0, ctx->ptab + (size_t)(j - 2) * Va * Hc, Va, prev, ctx->cx, Hc, true,
                            true))
          return rc;
        gathered = true;
      } else if (ctx->proj) {
        GemvArgs a = gemv_args(ctx);
        a.w[0] = ctx->proj; a.seg_rows[0] = Hc; a.N = Hc; a.K = Ht; a.M = B;
        a.src = SRC_TABLE; a.table = table; a.table_rows = Va; a.tok = prev;
        a.y = ctx->cx; a.y_stride = Hc; a.epi = EPI_STORE;
        if (int rc = proj(ctx, a)) return rc;
      } else {
        if (int rc = gather(ctx, SRC_TABLE, B, Hc, nullptr, 0, table, Va, prev, ctx->cx, Hc, false, true)) return rc;
        gathered = true;
      }
    }
    if (int rc = stack_step(ctx, ctx->cp, ctx->cx, B, Mp, j == 1 ? 0 : j, 0, kc, vc, kCpPositions, 1, ctx->ccos, ctx->csin,
                            false, nullptr, gathered))
      return rc;
    // final norm + head j on the last position of each stream
    GemvArgs a = gemv_args(ctx);
    a.w[0] = (const char*)ctx->heads + (size_t)(j - 1) * head_sz; a.seg_rows[0] = Va; a.N = Va; a.K = Hc; a.M = B;
    a.src = SRC_VEC; a.x = ctx->cx + (size_t)(Mp - 1) * Hc; a.x_stride = Mp * Hc; a.gain = ctx->cp.final_norm;
    a.ssq_in = 1;  // used when these are the rows the last down projection wrote (Mp = 1)
    float* lg = logits_out ? logits_out + (size_t)(j - 1) * Va : ctx->clog;
    a.y = lg; a.y_stride = logits_out ? c.n_acoustic * Va : Va; a.epi = EPI_STORE;
    if (int rc = proj(ctx, a)) return rc;
    URef uj = u;
    uj.offset += j - 1;
    if (int rc = sample(ctx, lg, a.y_stride, B, Va, ac, uj, nullptr, 0, 0, out, ob, of, oo + j - 1, ouf, ctx->next_tok, forced,
                        c.n_acoustic, j - 1))
      return rc;
  }
  return TTS_OK;
}

void fill_rope(const tts_config& c, int d, int npos, std::vector<float>& cs, std::vector<float>& sn) {
  const int half = d / 2;
  cs.resize((size_t)npos * half);
  sn.resize((size_t)npos * half);
  for (int p = 0; p < npos; ++p)
    for (int i = 0; i < half; ++i) {
      const double inv = std::pow((double)c.rope_theta, -2.0 * i / d);
      const double ang = (double)p * inv;
      cs[(size_t)p * half + i] = (float)std::cos(ang);
      sn[(size_t)p * half + i] = (float)std::sin(ang);
    }
}

int check_sampling(tts_ctx* ctx, const tts_sampling* s, int V, const char* what) {
  if (!s) return ctx->fail(TTS_E_ARG, "%s sampling is NULL", what);
  if (s->do_sample) {
    if (!(s->temperature > 0.f)) return ctx->fail(TTS_E_ARG, "%s temperature must be > 0", what);
    if (!(s->repetition_penalty > 0.f)) return ctx->fail(TTS_E_ARG, "%s repetition_penalty must be > 0", what);
    if (!(s->top_p > 0.f)) return ctx->fail(TTS_E_ARG, "%s top_p must be > 0", what);
    if (V > kSortMax) return ctx->fail(TTS_E_UNSUPPORTED, "%s: sampling supports vocab <= %d (got %d)", what, kSortMax, V);
  }
  return TTS_OK;
}

int enqueue_frame(tts_ctx* ctx, const tts_sampling& sem, const tts_sampling& ac, const float* u, int32_t* codes) {
  const auto& c = ctx->cfg;
  const int B = ctx->batch;
  const int fs = c.max_frames * 16;
  // greedy never reads u; keep its strides at zero then so no address depends on it
  const int ub = u ? fs : 0, uf = u ? 16 : 0;
  if (!u) u = ctx->hT;
  // semantic token of frame t from the pending Talker logits
  if (int rc = sample(ctx, ctx->logits, c.talker.vocab, B, c.talker.vocab, sem, uref(u, ub, uf, 0, 1), ctx->history,
                      c.talker.vocab, 1, codes, fs, 16, 0, 1, ctx->sem_tok, nullptr, 0, 0))
    return rc;
  if (use_xtp(ctx, B, ac)) {
    if (int rc = codepred_frame_xtp(ctx, ctx->sem_tok, nullptr, codes + 1, 16, 1, nullptr, ac, u, uf, 1)) return rc;
  } else if (int rc = codepred_frame(ctx, B, tokref(ctx->sem_tok, 1, 0, 0, 0), ac, uref(u, ub, uf, u == ctx->hT ? 0 : 1, 1), nullptr,
                                     codes, fs, 16, 1, 1, nullptr)) {
    return rc;
  }
  TokRef refs[16];
  for (int j = 0; j < 16; ++j) refs[j] = tokref(codes, fs, 16, j, 1);
  // streaming text: the step on frame t's codes adds text id [b][next + t] while it exists
  const TokRef text = tokref(ctx->text_ids, ctx->text_n, 1, ctx->text_next, 1);
  if (int rc = embed_sum(ctx, B, refs, ctx->text_ids ? &text : nullptr, ctx->text_n)) return rc;
  // per-stream stop: the next Talker input holds the codes as drawn; the reported codes are masked
  if (ctx->eos_id >= 0) {
    hipLaunchKernelGGL(k_eos_mask, dim3((B + 63) / 64), dim3(64), 0, ctx->stream, codes, fs, ctx->st, ctx->eos_id, ctx->stop, B);
    HIP_LAUNCH_CHECK();
  }
  // the frame's last kernel also advances the device position and frame counters
  if (use_xtk(ctx, B)) return talker_step_xtk(ctx, 1, 1);
  if (int rc = talker_stack(ctx, B, 0, 1)) return rc;
  return talker_head(ctx, B, 1, 1);
}

void drop_graph(tts_ctx* ctx) {
  if (ctx->gexec) (void)hipGraphExecDestroy(ctx->gexec);
  if (ctx->graph) (void)hipGraphDestroy(ctx->graph);
  ctx->gexec = nullptr;
  ctx->graph = nullptr;
  ctx->have_graph = false;
}

}  // namespace

// ============================================================================ C ABI

extern "C" {

int32_t tts_persistent_allowed(const tts_device_desc* d) {
  if (!d) return 0;
  // gfx950 itself, with or without feature suffixes ("gfx950:sramecc+:xnack-")
  if (std::strncmp(d->arch, "gfx950", 6) != 0 || (d->arch[6] != '\0' && d->arch[6] != ':')) return 0;
  if (d->compute_units != xtp::NWG || d->xccs != xtp::NX) return 0;
  int32_t m = 0;
  if (d->codepred_wg_per_cu >= 1) m |= TTS_PERSISTENT_CODEPRED;
  if (d->talker_wg_per_cu >= 1) m |= TTS_PERSISTENT_TALKER;
  return m;
}

int tts_workspace_bytes(const tts_config* cfg, size_t* bytes) {
  if (!bytes) return TTS_E_ARG;
  std::string e = check_config(cfg);
  if (!e.empty()) return cfg ? TTS_E_SHAPE : TTS_E_ARG;
  *bytes = make_layout(*cfg).total;
  return TTS_OK;
}

int tts_create(const tts_config* cfg, void* hip_stream, void* workspace, size_t workspace_bytes, tts_ctx** out) {
  if (!out) return TTS_E_ARG;
  *out = nullptr;
  if (!cfg || !workspace) return TTS_E_ARG;
  if (!check_config(cfg).empty()) return TTS_E_SHAPE;
  if (((uintptr_t)workspace) & 255) return TTS_E_ARG;
  Layout L = make_layout(*cfg);
  if (workspace_bytes < L.total) return TTS_E_CAPACITY;
  tts_ctx* ctx = new tts_ctx();
  ctx->cfg = *cfg;
  ctx->stream = (hipStream_t)hip_stream;
  ctx->ws = (char*)workspace;
  ctx->L = L;
  if (hipGetDevice(&ctx->device) != hipSuccess) { delete ctx; return TTS_E_HIP; }
  char* w = ctx->ws;
  ctx->st = (DevState*)(w + L.st);
  ctx->x = (float*)(w + L.x); ctx->qkv = (float*)(w + L.qkv); ctx->attn = (float*)(w + L.attn); ctx->h = (float*)(w + L.h);
  ctx->part = (float*)(w + L.part); ctx->logits = (float*)(w + L.logits); ctx->hT = (float*)(w + L.hT);
  ctx->counters = (int32_t*)(w + L.counters);
  ctx->cx = (float*)(w + L.cx); ctx->clog = (float*)(w + L.clog);
  ctx->tcos = (float*)(w + L.tcos); ctx->tsin = (float*)(w + L.tsin); ctx->ccos = (float*)(w + L.ccos); ctx->csin = (float*)(w + L.csin);
  ctx->next_tok = (int32_t*)(w + L.next_tok); ctx->sem_tok = (int32_t*)(w + L.sem_tok); ctx->ac_codes = (int32_t*)(w + L.ac_codes);
  ctx->history = (uint8_t*)(w + L.history);
  ctx->kvstart = (int32_t*)(w + L.kvstart);
  ctx->aids = (int32_t*)(w + L.aids);
  ctx->cpdesc = (xtp::CpDesc*)(w + L.cpdesc);
  ctx->tkdesc = (xtp::TkDesc*)(w + L.tkdesc);
  ctx->cpdesc_s = (xtp::CpDesc*)(w + L.cpdesc_s);
  ctx->tkdesc_s = (xtp::TkDesc*)(w + L.tkdesc_s);
  // this device's static scratch array (tts_run_frames_noalloc), looked up once per device here
  {
    hipError_t se = hipSuccess;
    ctx->scratch = scratch_device_ptr(ctx->device, &se);
    if (!ctx->scratch) { delete ctx; return TTS_E_HIP; }
  }
  ctx->xerr = (uint32_t*)(w + L.xerr);
  ctx->xtp_ok = xtp_capable(*cfg);
  ctx->xtk_ok = xtk_capable(*cfg);
  ctx->xcp_ok = ctx->xtp_ok && xcp_capable(*cfg);
  // The persistent kernels need every one of their 256 workgroups resident at once, 32 on each of
  // the 8 XCDs: gate them on the device (elsewhere the per-op kernels run).
  {
    tts_device_desc dd;
    std::memset(&dd, 0, sizeof dd);
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, ctx->device) != hipSuccess) { delete ctx; return TTS_E_HIP; }
    std::snprintf(dd.arch, sizeof dd.arch, "%s", prop.gcnArchName);
    dd.compute_units = prop.multiProcessorCount;
    int xccs = 0;
    if (hipDeviceGetAttribute(&xccs, hipDeviceAttributeNumberOfXccs, ctx->device) != hipSuccess) xccs = 0;
    dd.xccs = xccs;
    int occ = 0;
    const bool e8 = cfg->weight_dtype == TTS_DTYPE_FP8_E4M3;
    const void* cpk = ctx->xcp_ok ? (e8 ? reinterpret_cast<const void*>(xcp::k_cp_frame<uint8_t>)
                                        : reinterpret_cast<const void*>(xcp::k_cp_frame<uint16_t>))
                                  : (e8 ? reinterpret_cast<const void*>(xtp::k_cp_frame<uint8_t>)
                                        : reinterpret_cast<const void*>(xtp::k_cp_frame<uint16_t>));
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, cpk, xtp::NT, 0) != hipSuccess) occ = 0;
    dd.codepred_wg_per_cu = occ;
    occ = 0;
    const void* tkk = cfg->weight_dtype == TTS_DTYPE_FP8_E4M3 ? reinterpret_cast<const void*>(xtp::k_talker_step<uint8_t>)
                                                              : reinterpret_cast<const void*>(xtp::k_talker_step<uint16_t>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, tkk, xtp::NT, 0) != hipSuccess) occ = 0;
    dd.talker_wg_per_cu = occ;
    (void)hipGetLastError();
    ctx->dev_mask = tts_persistent_allowed(&dd);
    ctx->xtp_ok = ctx->xtp_ok && (ctx->dev_mask & TTS_PERSISTENT_CODEPRED);
    ctx->xcp_ok = ctx->xcp_ok && ctx->xtp_ok;
    ctx->xtk_ok = ctx->xtk_ok && (ctx->dev_mask & TTS_PERSISTENT_TALKER);
  }
  if (hipHostMalloc((void**)&ctx->errh, sizeof(uint32_t), hipHostMallocDefault) != hipSuccess) { delete ctx; return TTS_E_HIP; }
  *ctx->errh = 0;
  if (hipEventCreateWithFlags(&ctx->err_ev, hipEventDisableTiming) != hipSuccess) {
    (void)hipHostFree(ctx->errh);
    delete ctx;
    return TTS_E_HIP;
  }
  ctx->pgemm_ok = prefill_gemm_capable(*cfg);
  ctx->talker.c = cfg->talker;
  ctx->cp.c = cfg->codepred;
  // RoPE tables: angles p * theta^(-2i/d) in double, rounded to fp32.
  std::vector<float> cs, sn;
  fill_rope(*cfg, cfg->talker.head_dim, cfg->max_cache_steps, cs, sn);
  hipError_t e1 = hipMemcpy(ctx->tcos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice);
  hipError_t e2 = hipMemcpy(ctx->tsin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice);
  fill_rope(*cfg, cfg->codepred.head_dim, kCpPositions, cs, sn);
  hipError_t e3 = hipMemcpy(ctx->ccos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice);
  hipError_t e4 = hipMemcpy(ctx->csin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice);
  if (e1 || e2 || e3 || e4) { delete ctx; return TTS_E_HIP; }
  hipLaunchKernelGGL(k_set_state, dim3(1), dim3(64), 0, ctx->stream, ctx->st, 0, 0);
  hipLaunchKernelGGL(k_fill_u8, dim3(1), dim3(256), 0, ctx->stream, (uint8_t*)ctx->counters,
                     (size_t)cfg->max_batch * cfg->talker.n_kv_heads * 4, (uint8_t)0);
  hipLaunchKernelGGL(k_fill_u8, dim3(1), dim3(64), 0, ctx->stream, (uint8_t*)ctx->st, sizeof(DevState), (uint8_t)0);
  hipLaunchKernelGGL(k_fill_u8, dim3(256), dim3(256), 0, ctx->stream, (uint8_t*)(w + L.xzero_begin),
                     L.xzero_end - L.xzero_begin, (uint8_t)0);
  if (hipGetLastError() != hipSuccess) { delete ctx; return TTS_E_HIP; }
  *out = ctx;
  return TTS_OK;
}

int tts_load_weights(tts_ctx* ctx, int32_t n, const char* const* names, void* const* dev_ptrs, const int64_t* shapes,
                     const int32_t* ranks, const int32_t* dtypes) {
  if (!ctx) return TTS_E_ARG;
  if (n < 0 || !names || !dev_ptrs || !shapes || !ranks || !dtypes) return ctx->fail(TTS_E_ARG, "load_weights: NULL argument");
  const tts_config& c = ctx->cfg;
  // dtype -1: the config's weight dtype for matrices; -2: its gain / table dtype (bf16 for FP8)
  struct Want { std::vector<int64_t> shape; const void** slot; int dtype = -1; };
  std::unordered_map<std::string, Want> want;
  StackW talker, cp;
  talker.c = c.talker; cp.c = c.codepred;
  talker.layers.resize(c.talker.n_layers);
  cp.layers.resize(c.codepred.n_layers);
  const void *embed_text = nullptr, *embed_sem = nullptr, *lm_head = nullptr, *proj = nullptr, *embed_ac = nullptr, *heads = nullptr;
  auto add_stack = [&](const char* prefix, StackW& S) {
    const tts_stack_cfg& s = S.c;
    const int64_t H = s.hidden, qd = (int64_t)s.n_q_heads * s.head_dim, kd = (int64_t)s.n_kv_heads * s.head_dim;
    for (int i = 0; i < s.n_layers; ++i) {
      std::string p = std::string(prefix) + ".layers." + std::to_string(i) + ".";
      Layer& L = S.layers[i];
      want[p + "attn_norm"] = {{H}, &L.attn_norm, -2};
      want[p + "wq"] = {{qd, H}, &L.wq};
      want[p + "wk"] = {{kd, H}, &L.wk};
      want[p + "wv"] = {{kd, H}, &L.wv};
      want[p + "q_norm"] = {{s.head_dim}, &L.q_norm, -2};
      want[p + "k_norm"] = {{s.head_dim}, &L.k_norm, -2};
      want[p + "wo"] = {{H, qd}, &L.wo};
      want[p + "mlp_norm"] = {{H}, &L.mlp_norm, -2};
      want[p + "wg"] = {{s.ffn, H}, &L.wg};
      want[p + "wu"] = {{s.ffn, H}, &L.wu};
      want[p + "wd"] = {{H, s.ffn}, &L.wd};
    }
    want[std::string(prefix) + ".final_norm"] = {{H}, &S.final_norm, -2};
  };
  add_stack("talker", talker);
  add_stack("cp", cp);
  const int64_t Ht = c.talker.hidden, Hc = c.codepred.hidden;
  want["talker.embed_text"] = {{c.text_vocab, Ht}, &embed_text, -2};
  want["talker.embed_sem"] = {{c.talker.vocab, Ht}, &embed_sem, -2};
  want["talker.lm_head"] = {{c.talker.vocab, Ht}, &lm_head};
  if (Ht != Hc) want["cp.proj"] = {{Hc, Ht}, &proj};
  want["cp.embed_ac"] = {{c.n_acoustic, c.codepred.vocab, Ht}, &embed_ac, -2};
  want["cp.heads"] = {{c.n_acoustic, c.codepred.vocab, Hc}, &heads};
  // E4M3 matrices: one fp32 scale per row ("<name>.scale", the matrix shape without its last dim)
  std::vector<std::string> mats;
  std::unordered_map<std::string, const void*> scale_ptr;
  if (c.weight_dtype == TTS_DTYPE_FP8_E4M3) {
    for (auto& kv : want)
      if (kv.second.dtype == -1) mats.push_back(kv.first);
    for (const std::string& m : mats) {
      std::vector<int64_t> sh = want[m].shape;
      sh.pop_back();
      scale_ptr[m] = nullptr;
      want[m + ".scale"] = {sh, &scale_ptr[m], TTS_DTYPE_F32};
    }
  }
  std::unordered_map<std::string, bool> seen;
  for (int i = 0; i < n; ++i) {
    if (!names[i]) return ctx->fail(TTS_E_ARG, "load_weights: name %d is NULL", i);
    auto it = want.find(names[i]);
    if (it == want.end()) return ctx->fail(TTS_E_SHAPE, "load_weights: unexpected tensor '%s'", names[i]);
    if (seen.count(names[i])) return ctx->fail(TTS_E_ARG, "load_weights: tensor '%s' given twice", names[i]);
    seen[names[i]] = true;
    const auto& shp = it->second.shape;
    if (ranks[i] != (int)shp.size()) return ctx->fail(TTS_E_SHAPE, "load_weights: '%s' has rank %d, expected %zu", names[i], ranks[i], shp.size());
    for (size_t k = 0; k < shp.size(); ++k)
      if (shapes[i * 4 + k] != shp[k])
        return ctx->fail(TTS_E_SHAPE, "load_weights: '%s' dim %zu is %lld, expected %lld", names[i], k, (long long)shapes[i * 4 + k],
                         (long long)shp[k]);
    const int wdt = it->second.dtype == -1 ? c.weight_dtype
                    : (it->second.dtype == -2 ? (c.weight_dtype == TTS_DTYPE_F32 ? TTS_DTYPE_F32 : TTS_DTYPE_BF16) : it->second.dtype);
    if (dtypes[i] != wdt) return ctx->fail(TTS_E_SHAPE, "load_weights: '%s' dtype %d, expected %d", names[i], dtypes[i], wdt);
    if (!dev_ptrs[i]) return ctx->fail(TTS_E_ARG, "load_weights: '%s' pointer is NULL", names[i]);
    if (((uintptr_t)dev_ptrs[i]) & 15) return ctx->fail(TTS_E_ARG, "load_weights: '%s' is not 16-byte aligned", names[i]);
    *it->second.slot = dev_ptrs[i];
  }
  for (auto& kv : want)
    if (!seen.count(kv.first)) return ctx->fail(TTS_E_SHAPE, "load_weights: tensor '%s' missing", kv.first.c_str());
  ctx->talker = talker;
  ctx->cp = cp;
  ctx->embed_text = embed_text; ctx->embed_sem = embed_sem; ctx->lm_head = lm_head; ctx->proj = proj;
  ctx->embed_ac = embed_ac; ctx->heads = heads;
  ctx->qtensors.clear();
  for (const std::string& m : mats) {
    const auto& sh = want[m].shape;
    size_t bytes = 1;
    for (int64_t d : sh) bytes *= (size_t)d;
    ctx->qtensors.push_back({(uintptr_t)*want[m].slot, bytes, (int)sh.back(), (const float*)scale_ptr[m]});
  }
  ctx->weights_ok = true;
  ctx->prefilled = false;
  ctx->ptab = nullptr;
  drop_graph(ctx);
  if (ctx->xtp_ok) {
    xtp::CpDesc D;
    std::memset(&D, 0, sizeof D);
    const tts_stack_cfg& p = c.codepred;
    for (int l = 0; l < p.n_layers; ++l) {
      const Layer& L = ctx->cp.layers[l];
      D.layer[l] = {L.attn_norm, L.wq, L.wk, L.wv, L.q_norm, L.k_norm, L.wo, L.mlp_norm, L.wg, L.wu, L.wd};
      if (ctx->fp8()) {
        const int H = p.hidden, qd = p.n_q_heads * p.head_dim;
        D.scale[l] = {ctx->scale_of(L.wq, H), ctx->scale_of(L.wk, H), ctx->scale_of(L.wv, H), ctx->scale_of(L.wo, qd),
                      ctx->scale_of(L.wg, H), ctx->scale_of(L.wu, H), ctx->scale_of(L.wd, p.ffn)};
        const xtp::LayerS& q = D.scale[l];
        if (!q.wq || !q.wk || !q.wv || !q.wo || !q.wg || !q.wu || !q.wd)
          return ctx->fail(TTS_E_STATE, "load_weights: no E4M3 scale for a CodePredictor layer %d matrix", l);
      }
    }
    if (ctx->fp8()) {
      D.head_scale = ctx->scale_of(ctx->heads, p.hidden);
      D.proj_scale = ctx->proj ? ctx->scale_of(ctx->proj, c.talker.hidden) : nullptr;
      if (!D.head_scale || (ctx->proj && !D.proj_scale))
        return ctx->fail(TTS_E_STATE, "load_weights: no E4M3 scale for the CodePredictor heads or input projection");
    }
    D.n_layers = p.n_layers; D.H = p.hidden; D.Ht = c.talker.hidden; D.F = p.ffn; D.V = p.vocab; D.Vs = c.talker.vocab;
    D.nq = p.n_q_heads; D.nkv = p.n_kv_heads; D.d = p.head_dim; D.n_ac = c.n_acoustic; D.eps = c.rms_eps;
    D.final_norm = ctx->cp.final_norm; D.heads = ctx->heads; D.proj = ctx->proj; D.embed_ac = ctx->embed_ac;
    D.embed_sem = ctx->embed_sem;
    D.ptab = nullptr;
    if (ctx->xcp_ok && ctx->proj && wants_proj_table(c)) {
      // projected codebook rows P E_ac[j][a] for steps 2..15 of the lean CodePredictor kernel
      float* T = (float*)(ctx->ws + ctx->L.ptab);
      const int R = c.n_acoustic * p.vocab, N = p.hidden, K = c.talker.hidden;
      if (ctx->fp8())
        hipLaunchKernelGGL(k_proj_table<uint8_t>, dim3(N / 64, (R + 63) / 64), dim3(256), 0, ctx->stream,
                           (const uint16_t*)ctx->embed_ac, (const uint8_t*)ctx->proj, D.proj_scale, T, R, N, K);
      else
        hipLaunchKernelGGL(k_proj_table<uint16_t>, dim3(N / 64, (R + 63) / 64), dim3(256), 0, ctx->stream,
                           (const uint16_t*)ctx->embed_ac, (const uint16_t*)ctx->proj, (const float*)nullptr, T, R, N, K);
      HIP_LAUNCH_CHECK();
      D.ptab = T;
    }
    ctx->ptab = D.ptab;
    D.rope_cos = ctx->ccos; D.rope_sin = ctx->csin;
    D.hT = ctx->hT;
    D.xin = (xtp::u64*)(ctx->ws + ctx->L.xin); D.xcr = (xtp::u64*)(ctx->ws + ctx->L.xcr);
    D.cand = (xtp::u64*)(ctx->ws + ctx->L.cand);
    D.st = ctx->st; D.err = ctx->xerr;
    HIP_TRY(hipMemcpyAsync(ctx->cpdesc, &D, sizeof D, hipMemcpyHostToDevice, ctx->stream));
    ScratchLayout SL;
    D.xin = (xtp::u64*)(ctx->scratch + SL.xin); D.xcr = (xtp::u64*)(ctx->scratch + SL.xcr);
    D.cand = (xtp::u64*)(ctx->scratch + SL.cand);
    HIP_TRY(hipMemcpyAsync(ctx->cpdesc_s, &D, sizeof D, hipMemcpyHostToDevice, ctx->stream));
    HIP_TRY(hipStreamSynchronize(ctx->stream));
  }
  if (ctx->xtk_ok) {
    xtp::TkDesc D;
    std::memset(&D, 0, sizeof D);
    const tts_stack_cfg& t = c.talker;
    for (int l = 0; l < t.n_layers; ++l) {
      const Layer& L = ctx->talker.layers[l];
      D.layer[l] = {L.attn_norm, L.wq, L.wk, L.wv, L.q_norm, L.k_norm, L.wo, L.mlp_norm, L.wg, L.wu, L.wd};
      if (ctx->fp8()) {
        const int H = t.hidden, qd = t.n_q_heads * t.head_dim;
        D.scale[l] = {ctx->scale_of(L.wq, H), ctx->scale_of(L.wk, H), ctx->scale_of(L.wv, H), ctx->scale_of(L.wo, qd),
                      ctx->scale_of(L.wg, H), ctx->scale_of(L.wu, H), ctx->scale_of(L.wd, t.ffn)};
        const xtp::LayerS& q = D.scale[l];
        if (!q.wq || !q.wk || !q.wv || !q.wo || !q.wg || !q.wu || !q.wd)
          return ctx->fail(TTS_E_STATE, "load_weights: no E4M3 scale for a Talker layer %d matrix", l);
      }
    }
    if (ctx->fp8()) {
      D.head_scale = ctx->scale_of(ctx->lm_head, t.hidden);
      if (!D.head_scale) return ctx->fail(TTS_E_STATE, "load_weights: no E4M3 scale for the semantic head");
    }
    D.n_layers = t.n_layers; D.H = t.hidden; D.F = t.ffn; D.V = t.vocab; D.nq = t.n_q_heads; D.nkv = t.n_kv_heads;
    D.d = t.head_dim; D.cap = c.max_cache_steps; D.eps = c.rms_eps;
    D.final_norm = ctx->talker.final_norm; D.lm_head = ctx->lm_head;
    D.rope_cos = ctx->tcos; D.rope_sin = ctx->tsin;
    D.kc = (float*)(ctx->ws + ctx->L.tk); D.vc = (float*)(ctx->ws + ctx->L.tv);
    D.ls = (long long)c.max_batch * t.n_kv_heads * c.max_cache_steps;
    D.x_in = ctx->x; D.logits = ctx->logits; D.hT = ctx->hT;
    D.xin = (xtp::u64*)(ctx->ws + ctx->L.xin); D.xcr = (xtp::u64*)(ctx->ws + ctx->L.xcr);
    D.att = (xtp::u64*)(ctx->ws + ctx->L.att);
    D.st = ctx->st; D.err = ctx->xerr;
    HIP_TRY(hipMemcpyAsync(ctx->tkdesc, &D, sizeof D, hipMemcpyHostToDevice, ctx->stream));
    ScratchLayout SL;
    D.xin = (xtp::u64*)(ctx->scratch + SL.xin); D.xcr = (xtp::u64*)(ctx->scratch + SL.xcr);
    D.att = (xtp::u64*)(ctx->scratch + SL.att);
    HIP_TRY(hipMemcpyAsync(ctx->tkdesc_s, &D, sizeof D, hipMemcpyHostToDevice, ctx->stream));
    HIP_TRY(hipStreamSynchronize(ctx->stream));
  }
  ctx->err.clear();
  return TTS_OK;
}

}  // extern "C"

namespace {

// The prompt pass of tts_prefill / tts_prefill_ragged after validation. starts: per-stream first
// prompt position (host, B entries) or nullptr for all 0; with starts, ids are the caller's
// left-aligned rows and are right-aligned into the workspace first.
int prefill_body(tts_ctx* ctx, const int32_t* ids, int32_t batch, int32_t n, const int32_t* starts, float* sem_logits) {
  const auto& c = ctx->cfg;
  drop_graph(ctx);
  hipLaunchKernelGGL(k_set_state, dim3(1), dim3(64), 0, ctx->stream, ctx->st, 0, 0);
  HIP_LAUNCH_CHECK();
  if (starts) {
    ctx->starts_host.assign(starts, starts + batch);
    HIP_TRY(hipMemcpyAsync(ctx->kvstart, ctx->starts_host.data(), (size_t)batch * 4, hipMemcpyHostToDevice, ctx->stream));
    hipLaunchKernelGGL(k_align_ids, dim3(std::min((batch * n + 255) / 256, 1024)), dim3(256), 0, ctx->stream, ids, n, ctx->kvstart,
                       batch, ctx->aids);
    HIP_LAUNCH_CHECK();
    ids = ctx->aids;
  } else {
    hipLaunchKernelGGL(k_fill_i32, dim3(1), dim3(256), 0, ctx->stream, ctx->kvstart, batch, 0);
    HIP_LAUNCH_CHECK();
  }
  if (ctx->stop) {
    hipLaunchKernelGGL(k_fill_i32, dim3(1), dim3(256), 0, ctx->stream, ctx->stop, c.max_batch, -1);
    HIP_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(k_fill_u8, dim3(64), dim3(256), 0, ctx->stream, ctx->history, (size_t)batch * c.talker.vocab, (uint8_t)0);
  HIP_LAUNCH_CHECK();
  if (ctx->pgemm_ok && ctx->prefill_mode == TTS_PREFILL_GEMM) {
    if (int rc = prefill_gemm(ctx, ids, batch, n)) return rc;
  } else {
    for (int p = 0; p < n; ++p) {
      if (int rc = gather(ctx, SRC_TABLE, batch, c.talker.hidden, nullptr, 0, ctx->embed_text, c.text_vocab, tokref(ids, n, 0, p, 0),
                          ctx->x, c.talker.hidden))
        return rc;
      if (int rc = talker_stack(ctx, batch, p, 0)) return rc;
    }
  }
  if (int rc = talker_head(ctx, batch, 0, 0)) return rc;
  hipLaunchKernelGGL(k_set_state, dim3(1), dim3(64), 0, ctx->stream, ctx->st, n, 0);
  HIP_LAUNCH_CHECK();
  if (sem_logits)
    HIP_TRY(hipMemcpyAsync(sem_logits, ctx->logits, (size_t)batch * c.talker.vocab * 4, hipMemcpyDeviceToDevice, ctx->stream));
  ctx->batch = batch;
  ctx->pos = n;
  ctx->frames = 0;
  ctx->prefilled = true;
  ctx->err.clear();
  return TTS_OK;
}

int check_prefill(tts_ctx* ctx, const int32_t* ids, int32_t batch, int32_t n) {
  if (!ctx->weights_ok) return ctx->fail(TTS_E_STATE, "prefill: weights not loaded");
  if (!ids) return ctx->fail(TTS_E_ARG, "prefill: ids is NULL");
  if (batch < 1 || batch > ctx->cfg.max_batch) return ctx->fail(TTS_E_ARG, "prefill: batch %d outside [1, %d]", batch, ctx->cfg.max_batch);
  if (n < 1) return ctx->fail(TTS_E_ARG, "prefill: n must be >= 1");
  if (n > ctx->cfg.max_cache_steps) return ctx->fail(TTS_E_CAPACITY, "prefill: %d positions exceed max_cache_steps %d", n, ctx->cfg.max_cache_steps);
  return TTS_OK;
}

}  // namespace

extern "C" {

int tts_prefill(tts_ctx* ctx, const int32_t* ids, int32_t batch, int32_t n, float* sem_logits) {
  if (!ctx) return TTS_E_ARG;
  if (int rc = check_prefill(ctx, ids, batch, n)) return rc;
  return prefill_body(ctx, ids, batch, n, nullptr, sem_logits);
}

int tts_prefill_ragged(tts_ctx* ctx, const int32_t* ids, const int32_t* lengths, int32_t batch, int32_t n, float* sem_logits) {
  if (!ctx) return TTS_E_ARG;
  if (!lengths) return ctx->fail(TTS_E_ARG, "prefill_ragged: lengths is NULL");
  if (int rc = check_prefill(ctx, ids, batch, n)) return rc;
  std::vector<int32_t> starts(batch);
  for (int b = 0; b < batch; ++b) {
    if (lengths[b] < 1 || lengths[b] > n) return ctx->fail(TTS_E_SHAPE, "prefill_ragged: lengths[%d] = %d outside [1, %d]", b, lengths[b], n);
    starts[b] = n - lengths[b];
  }
  // one stream needs no padding: its prompt is simply shorter
  if (batch == 1) return prefill_body(ctx, ids, 1, lengths[0], nullptr, sem_logits);
  return prefill_body(ctx, ids, batch, n, starts.data(), sem_logits);
}

int tts_set_stop(tts_ctx* ctx, int32_t eos_id, int32_t* stop_frames) {
  if (!ctx) return TTS_E_ARG;
  if (eos_id >= ctx->cfg.talker.vocab) return ctx->fail(TTS_E_ARG, "set_stop: eos_id %d outside the semantic vocabulary", eos_id);
  if (eos_id >= 0 && !stop_frames) return ctx->fail(TTS_E_ARG, "set_stop: stop_frames is NULL");
  drop_graph(ctx);  // the frame graph holds the stop kernel (or its absence)
  ctx->eos_id = eos_id < 0 ? -1 : eos_id;
  ctx->stop = eos_id < 0 ? nullptr : stop_frames;
  if (ctx->stop) {
    hipLaunchKernelGGL(k_fill_i32, dim3(1), dim3(256), 0, ctx->stream, ctx->stop, ctx->cfg.max_batch, -1);
    HIP_LAUNCH_CHECK();
  }
  ctx->err.clear();
  return TTS_OK;
}

int tts_talker_step(tts_ctx* ctx, const int32_t* prev_codes, float* sem_logits) {
  return tts_talker_step_text(ctx, prev_codes, nullptr, sem_logits);
}

int tts_talker_step_text(tts_ctx* ctx, const int32_t* prev_codes, const int32_t* text_ids, float* sem_logits) {
  if (!ctx) return TTS_E_ARG;
  if (!ctx->prefilled) return ctx->fail(TTS_E_STATE, "talker_step: call tts_prefill first");
  if (!prev_codes) return ctx->fail(TTS_E_ARG, "talker_step: prev_codes is NULL");
  if (ctx->pos + 1 > ctx->cfg.max_cache_steps) return ctx->fail(TTS_E_CAPACITY, "talker_step: KV cache full (%d positions)", ctx->pos);
  if (int rc = device_err_check(ctx)) return rc;
  const int B = ctx->batch;
  TokRef refs[16];
  for (int j = 0; j < 16; ++j) refs[j] = tokref(prev_codes, 16, 0, j, 0);
  const TokRef text = tokref(text_ids, 1, 0, 0, 0);
  if (int rc = embed_sum(ctx, B, refs, text_ids ? &text : nullptr, 1)) return rc;
  if (use_xtk(ctx, B)) {
    if (int rc = talker_step_xtk(ctx, 1, 0)) return rc;
  } else {
    if (int rc = talker_stack(ctx, B, 0, 1)) return rc;
    if (int rc = talker_head(ctx, B, 1, 0)) return rc;
  }
  if (sem_logits)
    HIP_TRY(hipMemcpyAsync(sem_logits, ctx->logits, (size_t)B * ctx->cfg.talker.vocab * 4, hipMemcpyDeviceToDevice, ctx->stream));
  ctx->pos += 1;
  if (int rc = device_err_probe(ctx)) return rc;
  ctx->err.clear();
  return TTS_OK;
}

int tts_codepred_frame(tts_ctx* ctx, const int32_t* semantic, const tts_sampling* ac, const float* u, const int32_t* forced,
                       int32_t* codes, float* logits) {
  if (!ctx) return TTS_E_ARG;
  if (!ctx->prefilled) return ctx->fail(TTS_E_STATE, "codepred_frame: call tts_prefill first");
  if (!semantic || !codes) return ctx->fail(TTS_E_ARG, "codepred_frame: semantic and codes must not be NULL");
  if (int rc = check_sampling(ctx, ac, ctx->cfg.codepred.vocab, "acoustic")) return rc;
  if (ac->do_sample && !u) return ctx->fail(TTS_E_ARG, "codepred_frame: u is NULL with do_sample");
  if (int rc = device_err_check(ctx)) return rc;
  const int B = ctx->batch;
  URef ur = uref(u ? u : ctx->hT, u ? 15 : 0, 0, 0, 0);
  if (use_xtp(ctx, B, *ac)) {
    if (int rc = codepred_frame_xtp(ctx, semantic, forced, codes, 0, 0, logits, *ac, u, 0, 0)) return rc;
  } else if (int rc = codepred_frame(ctx, B, tokref(semantic, 1, 0, 0, 0), *ac, ur, forced, codes, 15, 0, 0, 0, logits)) {
    return rc;
  }
  if (int rc = device_err_probe(ctx)) return rc;
  ctx->err.clear();
  return TTS_OK;
}

int tts_sample(tts_ctx* ctx, const float* logits, int32_t batch, int32_t vocab, const tts_sampling* s, const float* u,
               uint8_t* history, int32_t* out) {
  if (!ctx) return TTS_E_ARG;
  if (!logits || !out) return ctx->fail(TTS_E_ARG, "sample: logits and out must not be NULL");
  if (batch < 1 || vocab < 1 || vocab > 65536) return ctx->fail(TTS_E_ARG, "sample: batch %d / vocab %d out of range", batch, vocab);
  if (int rc = check_sampling(ctx, s, vocab, "sample")) return rc;
  if (s->do_sample && !u) return ctx->fail(TTS_E_ARG, "sample: u is NULL with do_sample");
  URef ur = uref(u ? u : logits, u ? 1 : 0, 0, 0, 0);
  if (int rc = sample(ctx, logits, vocab, batch, vocab, *s, ur, history, vocab, history ? 1 : 0, out, 1, 0, 0, 0, nullptr, nullptr,
                      0, 0))
    return rc;
  ctx->err.clear();
  return TTS_OK;
}

int tts_run_frames(tts_ctx* ctx, int32_t n, const tts_sampling* sem, const tts_sampling* ac, const float* u, int32_t* codes) {
  if (!ctx) return TTS_E_ARG;
  if (!ctx->prefilled) return ctx->fail(TTS_E_STATE, "run_frames: call tts_prefill first");
  if (n < 0) return ctx->fail(TTS_E_ARG, "run_frames: n must be >= 0");
  if (!codes) return ctx->fail(TTS_E_ARG, "run_frames: codes is NULL");
  if (int rc = check_sampling(ctx, sem, ctx->cfg.talker.vocab, "semantic")) return rc;
  if (int rc = check_sampling(ctx, ac, ctx->cfg.codepred.vocab, "acoustic")) return rc;
  if ((sem->do_sample || ac->do_sample) && !u) return ctx->fail(TTS_E_ARG, "run_frames: u is NULL with sampling");
  if (ctx->frames + n > ctx->cfg.max_frames)
    return ctx->fail(TTS_E_CAPACITY, "run_frames: %d + %d frames exceed max_frames %d", ctx->frames, n, ctx->cfg.max_frames);
  if (ctx->pos + n > ctx->cfg.max_cache_steps)
    return ctx->fail(TTS_E_CAPACITY, "run_frames: %d + %d positions exceed max_cache_steps %d", ctx->pos, n, ctx->cfg.max_cache_steps);
  if (n == 0) return TTS_OK;
  if (int rc = device_err_check(ctx)) return rc;
  GraphKey key{*sem, *ac, u, codes, ctx->batch};
  if (!ctx->have_graph || !(ctx->gkey == key)) {
    drop_graph(ctx);
    // Record on a private stream (the caller's may be the null stream, which
    // cannot be captured); nothing executes during capture. The graph is
    // then launched on the caller's stream.
    if (!ctx->cap_stream) HIP_TRY(hipStreamCreateWithFlags(&ctx->cap_stream, hipStreamNonBlocking));
    HIP_TRY(hipStreamBeginCapture(ctx->cap_stream, hipStreamCaptureModeThreadLocal));
    hipStream_t user = ctx->stream;
    ctx->stream = ctx->cap_stream;
    int rc = enqueue_frame(ctx, *sem, *ac, u, codes);
    ctx->stream = user;
    hipGraph_t g = nullptr;
    hipError_t ec = hipStreamEndCapture(ctx->cap_stream, &g);
    if (rc) { if (g) (void)hipGraphDestroy(g); return rc; }
    if (ec != hipSuccess) return ctx->fail(TTS_E_HIP, "hipStreamEndCapture: %s", hipGetErrorString(ec));
    ctx->graph = g;
    HIP_TRY(hipGraphInstantiate(&ctx->gexec, ctx->graph, nullptr, nullptr, 0));
    ctx->have_graph = true;
    ctx->gkey = key;
  }
  for (int i = 0; i < n; ++i) HIP_TRY(hipGraphLaunch(ctx->gexec, ctx->stream));
  ctx->frames += n;
  ctx->pos += n;
  if (int rc = device_err_probe(ctx)) return rc;
  ctx->err.clear();
  return TTS_OK;
}

int tts_run_frames_noalloc(tts_ctx* ctx, int32_t n, const tts_sampling* sem, const tts_sampling* ac, const float* u,
                           int32_t* codes) {
  if (!ctx) return TTS_E_ARG;
  if (!ctx->prefilled) return ctx->fail(TTS_E_STATE, "run_frames_noalloc: call tts_prefill first");
  if (n < 0) return ctx->fail(TTS_E_ARG, "run_frames_noalloc: n must be >= 0");
  if (!codes) return ctx->fail(TTS_E_ARG, "run_frames_noalloc: codes is NULL");
  if (int rc = check_sampling(ctx, sem, ctx->cfg.talker.vocab, "semantic")) return rc;
  if (int rc = check_sampling(ctx, ac, ctx->cfg.codepred.vocab, "acoustic")) return rc;
  if ((sem->do_sample || ac->do_sample) && !u) return ctx->fail(TTS_E_ARG, "run_frames_noalloc: u is NULL with sampling");
  if (ctx->frames + n > ctx->cfg.max_frames)
    return ctx->fail(TTS_E_CAPACITY, "run_frames_noalloc: %d + %d frames exceed max_frames %d", ctx->frames, n, ctx->cfg.max_frames);
  if (ctx->pos + n > ctx->cfg.max_cache_steps)
    return ctx->fail(TTS_E_CAPACITY, "run_frames_noalloc: %d + %d positions exceed max_cache_steps %d", ctx->pos, n,
                     ctx->cfg.max_cache_steps);
  const int B = ctx->batch;
  if (ac->do_sample || !use_xtp(ctx, B, *ac) || !use_xtk(ctx, B))
    return ctx->fail(TTS_E_UNSUPPORTED,
                     "run_frames_noalloc: runs both persistent kernels only (batch 1, greedy acoustic tokens, bf16 or E4M3 weights, "
                     "persistent exec mode)");
  // the exchange buffers this call needs, against the array's fixed size
  if (ScratchLayout::total > kScratchBytes)
    return ctx->fail(TTS_E_CAPACITY, "run_frames_noalloc: %zu bytes of exchange buffers exceed the %zu-byte scratch array",
                     (size_t)ScratchLayout::total, kScratchBytes);
  if (n == 0) return TTS_OK;
  if (int rc = device_err_check(ctx)) return rc;
  // The array keeps the last call's values, possibly another context's, whose exchange tags may be
  // the ones this context expects next: clear it first (a fill kernel, so a caller's graph capture
  // holds no memset node).
  hipLaunchKernelGGL(k_fill_u8, dim3(256), dim3(256), 0, ctx->stream, (uint8_t*)ctx->scratch, kScratchBytes, (uint8_t)0);
  HIP_LAUNCH_CHECK();
  // the frames launched one by one (no graph to instantiate)
  ctx->use_scratch = true;
  for (int i = 0; i < n; ++i) {
    if (int rc = enqueue_frame(ctx, *sem, *ac, u, codes)) {
      ctx->use_scratch = false;
      return rc;
    }
  }
  ctx->use_scratch = false;
  ctx->frames += n;
  ctx->pos += n;
  if (int rc = device_err_probe(ctx)) return rc;
  ctx->err.clear();
  return TTS_OK;
}

int tts_get_progress(const tts_ctx* ctx, int32_t* talker_pos, int32_t* frames) {
  if (!ctx) return TTS_E_ARG;
  if (talker_pos) *talker_pos = ctx->pos;
  if (frames) *frames = ctx->frames;
  return TTS_OK;
}

int tts_reset(tts_ctx* ctx) {
  if (!ctx) return TTS_E_ARG;
  // Counters, the exchange tag and every exchange buffer start over, which also clears the
  // state a failed persistent launch may have left behind.
  hipLaunchKernelGGL(k_fill_u8, dim3(1), dim3(64), 0, ctx->stream, (uint8_t*)ctx->st, sizeof(DevState), (uint8_t)0);
  HIP_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_fill_u8, dim3(256), dim3(256), 0, ctx->stream, (uint8_t*)(ctx->ws + ctx->L.xzero_begin),
                     ctx->L.xzero_end - ctx->L.xzero_begin, (uint8_t)0);
  HIP_LAUNCH_CHECK();
  ctx->prefilled = false;
  ctx->pos = 0;
  ctx->frames = 0;
  ctx->batch = 0;
  if (ctx->text_ids) drop_graph(ctx);
  ctx->text_ids = nullptr;
  ctx->text_n = ctx->text_next = 0;
  // the error word is cleared above (it is part of the exchange state); the pending host copy is
  // of the old word
  ctx->err_pending = false;
  ctx->err.clear();
  return TTS_OK;
}

int tts_set_text_stream(tts_ctx* ctx, const int32_t* text_ids, int32_t n_text, int32_t next) {
  if (!ctx) return TTS_E_ARG;
  if (text_ids && (n_text < 1 || next < 0))
    return ctx->fail(TTS_E_ARG, "set_text_stream: n_text %d must be >= 1 and next %d >= 0", n_text, next);
  drop_graph(ctx);  // the frame graph holds the text term's addresses
  ctx->text_ids = text_ids;
  ctx->text_n = text_ids ? n_text : 0;
  ctx->text_next = text_ids ? next : 0;
  ctx->err.clear();
  return TTS_OK;
}

int tts_set_exec_mode(tts_ctx* ctx, int32_t mode) {
  if (!ctx) return TTS_E_ARG;
  if (mode != TTS_EXEC_KERNELS && mode != TTS_EXEC_PERSISTENT) return ctx->fail(TTS_E_ARG, "exec mode %d", mode);
  if (mode == TTS_EXEC_PERSISTENT && !ctx->xtp_ok && !ctx->xtk_ok)
    return ctx->fail(TTS_E_UNSUPPORTED, "no persistent kernel handles this config");
  if (mode != ctx->exec_mode) drop_graph(ctx);
  ctx->exec_mode = mode;
  ctx->err.clear();
  return TTS_OK;
}

int tts_get_exec_mode(const tts_ctx* ctx, int32_t* mode, int32_t* persistent_supported) {
  if (!ctx) return TTS_E_ARG;
  if (mode) *mode = ctx->exec_mode == TTS_EXEC_PERSISTENT && (ctx->xtp_ok || ctx->xtk_ok) ? TTS_EXEC_PERSISTENT : TTS_EXEC_KERNELS;
  if (persistent_supported) *persistent_supported = (ctx->xtp_ok ? TTS_PERSISTENT_CODEPRED : 0) | (ctx->xtk_ok ? TTS_PERSISTENT_TALKER : 0);
  return TTS_OK;
}

int tts_set_prefill_mode(tts_ctx* ctx, int32_t mode) {
  if (!ctx) return TTS_E_ARG;
  if (mode != TTS_PREFILL_STEPS && mode != TTS_PREFILL_GEMM) return ctx->fail(TTS_E_ARG, "prefill mode %d", mode);
  if (mode == TTS_PREFILL_GEMM && !ctx->pgemm_ok) return ctx->fail(TTS_E_UNSUPPORTED, "the GEMM prefill does not handle this config");
  ctx->prefill_mode = mode;
  ctx->err.clear();
  return TTS_OK;
}

int tts_get_prefill_mode(const tts_ctx* ctx, int32_t* mode) {
  if (!ctx || !mode) return TTS_E_ARG;
  *mode = ctx->pgemm_ok && ctx->prefill_mode == TTS_PREFILL_GEMM ? TTS_PREFILL_GEMM : TTS_PREFILL_STEPS;
  return TTS_OK;
}

int tts_device_status(tts_ctx* ctx, int32_t* status) {
  if (!ctx || !status) return TTS_E_ARG;
  HIP_TRY(hipStreamSynchronize(ctx->stream));
  uint32_t e = 0;
  HIP_TRY(hipMemcpy(&e, ctx->xerr, 4, hipMemcpyDeviceToHost));
  *status = (int32_t)e;
  return TTS_OK;
}

const char* tts_last_error(const tts_ctx* ctx) { return ctx ? ctx->err.c_str() : "context is NULL"; }

void tts_destroy(tts_ctx* ctx) {
  if (!ctx) return;
  drop_graph(ctx);
  if (ctx->cap_stream) (void)hipStreamDestroy(ctx->cap_stream);
  if (ctx->err_ev) (void)hipEventDestroy(ctx->err_ev);
  if (ctx->errh) (void)hipHostFree(ctx->errh);
  delete ctx;
}

}  // extern "C"

#ifdef TTS_PHASE_TRACE
// Phase-timeline build only: switch stamping on (on = 1, clears the record first) or off, and
// copy the record (kTraceWg x kTracePer stamps, 0 = none) to the host buffer out when given.
extern "C" int tts_trace_ctl(int on, long long* out) {
  if (out && hipMemcpyFromSymbol(out, HIP_SYMBOL(tts::g_trace), sizeof(long long) * tts::kTraceWg * tts::kTracePer) != hipSuccess)
    return TTS_E_HIP;
  if (on) {
    std::vector<long long> z((size_t)tts::kTraceWg * tts::kTracePer, 0);
    if (hipMemcpyToSymbol(HIP_SYMBOL(tts::g_trace), z.data(), z.size() * sizeof(long long)) != hipSuccess) return TTS_E_HIP;
  }
  if (hipMemcpyToSymbol(HIP_SYMBOL(tts::g_trace_on), &on, sizeof(int)) != hipSuccess) return TTS_E_HIP;
  return hipDeviceSynchronize() == hipSuccess ? TTS_OK : TTS_E_HIP;
}
#endif
