/*
 * tts.h -- C ABI of the MI355X per-frame Talker + CodePredictor decode.
 *
 * The method ("Running Qwen3-TTS on an AMD R9700", section "Running
 * Qwen3-TTS"): audio is generated one acoustic frame (80 ms, 16 codebook
 * tokens [semantic, acoustic 1..15]) at a time. Per frame the Talker decoder
 * runs one step and emits the semantic token; the CodePredictor decoder then
 * runs 15 sequential steps and emits acoustic tokens 1..15. Sampling controls
 * follow the "qwen3-tts-hip" README, section "Library Usage" (do_sample,
 * top_k, top_p, temperature, repetition_penalty; the acoustic set has no
 * repetition penalty); a fixed KV-cache capacity independent of a request's
 * frame count follows the same section (max_cache_steps).
 *
 * Conventions for every entry point:
 *  - All array arguments are DEVICE pointers (HIP device memory owned by the
 *    caller), except the config/sampling structs and the name/shape tables of
 *    tts_load_weights, which are host memory.
 *  - The library never allocates or frees device memory. The caller
 *    allocates the workspace (size from tts_workspace_bytes) and the weights;
 *    the context borrows them until tts_destroy.
 *  - Every call is asynchronous on the stream given to tts_create. Results
 *    are valid after the caller synchronises that stream. A context belongs to
 *    one host thread at a time.
 *  - Host-side validation happens before anything is enqueued: on an error
 *    return nothing was enqueued and the device state is unchanged. The text
 *    of the last error is available from tts_last_error.
 *  - Tokens are int32. Logits are fp32. Weights are row-major [out, in],
 *    all fp32 (TTS_DTYPE_F32), all bf16 (TTS_DTYPE_BF16), or FP8 projection
 *    matrices with bf16 gains and embeddings (TTS_DTYPE_FP8_E4M3, below).
 *  - B (batch) streams run in lockstep: same prefill length, same positions.
 */
#ifndef TTS_H
#define TTS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TTS_ABI_VERSION 1

typedef struct tts_ctx tts_ctx;

enum tts_status {
  TTS_OK = 0,
  TTS_E_ARG = -1,        /* null pointer, bad enum or out-of-range scalar */
  TTS_E_SHAPE = -2,      /* config or tensor shape the library does not accept */
  TTS_E_CAPACITY = -3,   /* KV positions or frames would exceed the configured capacity */
  TTS_E_STATE = -4,      /* call out of order (e.g. a step before weights or prefill) */
  TTS_E_HIP = -5,        /* a HIP runtime call failed; tts_last_error has its text */
  TTS_E_UNSUPPORTED = -6, /* valid request outside what the library implements */
  TTS_E_DEVICE = -7      /* a persistent kernel launched by an earlier call timed out in an exchange:
                            outputs since the last clean call are invalid; nothing was enqueued;
                            reported by every call that may launch them until tts_reset */
};

/* TTS_DTYPE_FP8_E4M3 (weight_dtype only): weight-only 8-bit quantisation
 * ("Benchmarking a TTS Model on Your Own GPU": an eight-bit copy of the
 * weights, widened on the fly, with FP8 done natively by newer hardware).
 * The projection matrices (wq wk wv wo wg wu wd, talker.lm_head, cp.proj,
 * cp.heads) are OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits; subnormals; 0x7f/0xff NaN, never produced), one byte per
 * element, and each comes with "<name>.scale": fp32, shape = the matrix's
 * shape without its last dimension. Element [.., r, k] stands for
 * scale[.., r] * decode(code[.., r, k]); products and sums are fp32.
 * Norm gains and the three embedding tables stay bf16. */
enum tts_dtype { TTS_DTYPE_F32 = 0, TTS_DTYPE_BF16 = 1, TTS_DTYPE_FP8_E4M3 = 2 };

/* One decoder stack (Talker or CodePredictor). vocab is the semantic vocab
 * for the Talker and the per-codebook acoustic vocab for the CodePredictor. */
typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
} tts_stack_cfg;

typedef struct {
  tts_stack_cfg talker, codepred;
  int32_t text_vocab;
  int32_t n_acoustic;      /* must be 15 */
  float rms_eps;           /* RMSNorm epsilon */
  float rope_theta;        /* RoPE base */
  int32_t weight_dtype;    /* enum tts_dtype of the weights (FP8: matrices only, see above) */
  int32_t kv_dtype;        /* must be TTS_DTYPE_F32: the KV caches hold k/v unrounded (a bf16 cache
                              alone puts the 1.7B-class acoustic logits over the 1e-2 parity bar) */
  int32_t max_batch;       /* streams per context */
  int32_t max_cache_steps; /* Talker KV capacity in positions (prefill + frames) */
  int32_t max_frames;      /* frame capacity of the u / codes arrays of tts_run_frames */
} tts_config;

/* Sampling controls. do_sample = 0 is greedy argmax (lowest id on ties).
 * Otherwise: repetition penalty over the history set (positive logits
 * divided by it, others multiplied), division by temperature, top_k
 * (<= 0: all ids; ids ordered by logit descending then id ascending), top_p
 * (>= 1: no-op), then inverse CDF of exp(l - l_max) at the given uniform:
 * the first kept id whose running sum exceeds u * sum, else the last. */
typedef struct {
  int32_t do_sample;
  int32_t top_k;
  float top_p;
  float temperature;
  float repetition_penalty;
} tts_sampling;

/* Bytes of device workspace (KV caches, activations, tables, counters) for a
 * config. Returns TTS_E_SHAPE for configs the kernels do not accept. */
int tts_workspace_bytes(const tts_config* cfg, size_t* bytes);

/* Create a context on the current HIP device. hip_stream: a hipStream_t (NULL
 * = the null stream). workspace: device memory of at least
 * tts_workspace_bytes, 256-byte aligned, borrowed until tts_destroy. */
int tts_create(const tts_config* cfg, void* hip_stream, void* workspace, size_t workspace_bytes, tts_ctx** out);

/* Bind weights ("qwen3-tts-hip" README, section "Library Usage": an engine is
 * loaded once from a model directory and then serves requests; section "Module
 * Layout": the Talker and CodePredictor decoder stacks, their weights and
 * config). n tensors named by the canonical names (talker.embed_text,
 * talker.embed_sem, talker.layers.<i>.{attn_norm,wq,wk,wv,q_norm,k_norm,wo,
 * mlp_norm,wg,wu,wd}, talker.final_norm, talker.lm_head, cp.proj (only when
 * the widths differ), cp.embed_ac [15,Va,Ht], cp.layers.<i>.{...},
 * cp.final_norm, cp.heads [15,Va,Hc]). shapes: n x 4 int64 (row-major, only
 * the first ranks[i] entries used); dtypes: enum tts_dtype per tensor. Every
 * tensor must be present with the exact shape, the config's dtype and
 * 16-byte alignment; FP8 configs add one "<matrix>.scale" per matrix (fp32)
 * and give gains and embeddings as bf16. Pointers are borrowed until
 * tts_destroy. FP8 configs run both persistent kernels (E4M3 tiles widened
 * to bf16 for the matrix cores, each row sum times its scale), the MFMA GEMM
 * routes and the per-op kernels. */
int tts_load_weights(tts_ctx* ctx, int32_t n, const char* const* names, void* const* dev_ptrs,
                     const int64_t* shapes, const int32_t* ranks, const int32_t* dtypes);

/* The prompt pass ("Running Qwen3-TTS on an AMD R9700", section "Running
 * Qwen3-TTS": the Talker reads the text conditioning before the frame loop;
 * "qwen3-tts-hip" README, section "Library Usage": a request's text, or its
 * first text_lookahead_tokens ids in streaming mode). Reset the streams and run
 * the Talker over text ids [B, n] (positions 0..n-1). Leaves frame 0's Talker output pending (semantic logits and the
 * final-normed hidden that conditions the CodePredictor). sem_logits
 * [B, Vs] receives those logits when non-NULL. */
int tts_prefill(tts_ctx* ctx, const int32_t* ids, int32_t batch, int32_t n, float* sem_logits);

/* tts_prefill for prompts of different lengths (ragged batch; row f2 of the
 * method's next steps: per-stream lengths in batched attention). ids [B, n]
 * (device): stream b's prompt is ids[b][0 .. lengths[b]), the rest of the row
 * is ignored. lengths: HOST array of B entries in [1, n]. With B > 1 the
 * prompts are right-aligned at positions n - lengths[b] .. n - 1 and every
 * Talker attention masks the positions before a stream's start; queries and
 * keys then differ from a prompt placed at position 0 only by a common
 * rotation, which leaves their products unchanged ("Running Qwen3-TTS on an
 * AMD R9700" fixes no positional scheme; rotate-half RoPE depends on position
 * differences only), so each stream decodes as if alone up to rounding. One
 * stream is simply a prompt of lengths[0] ids. TTS_E_SHAPE for a length
 * outside [1, n]; otherwise as tts_prefill. */
int tts_prefill_ragged(tts_ctx* ctx, const int32_t* ids, const int32_t* lengths, int32_t batch, int32_t n,
                       float* sem_logits);

/* Per-stream stop on a designated semantic id for tts_run_frames (row f2 of
 * the method's next steps; the pages leave the stop unfinished). eos_id in
 * [0, Vs), or -1 to switch it off. stop_frames: device int32 array of
 * max_batch entries, borrowed: set to -1 here and by every prefill; when
 * stream b draws eos_id as the semantic token of frame t, stop_frames[b] = t,
 * the frame's 15 acoustic codes are written as -1, and every later frame of
 * the stream is written as 16 x -1. The batch keeps decoding in lockstep (a
 * stopped stream's work continues and is discarded), so the caller may stop
 * calling tts_run_frames once every stream has stopped. Changing the setting
 * drops the captured frame graph. */
int tts_set_stop(tts_ctx* ctx, int32_t eos_id, int32_t* stop_frames);

/* One Talker step ("Running Qwen3-TTS on an AMD R9700", section "Running
 * Qwen3-TTS": per frame the Talker generates the first, semantic codebook
 * token; "qwen3-tts-hip" README, section "Python Parity Fixtures": the
 * embedding sum is a checked stage) fed with the previous frame's codes
 * [B, 16]: the input is E_sem[c0] + sum_j E_ac[j][cj]. Advances the Talker position by one and
 * replaces the pending output; sem_logits [B, Vs] receives it when non-NULL. */
int tts_talker_step(tts_ctx* ctx, const int32_t* prev_codes, float* sem_logits);

/* tts_talker_step with the streaming text term ("Running Qwen3-TTS on an AMD
 * R9700": the streaming mode feeds the text one token per frame; "qwen3-tts-hip"
 * README, section "Library Usage": text_lookahead_tokens text ids go into the
 * streaming prefill). text_ids [B] (device, or NULL for none): stream b's input
 * also gets the text embedding row E_text[text_ids[b]] added after the 16 codebook
 * rows; an id < 0 adds nothing (the text is used up). Ids past the text table are
 * clamped to its last row. Same errors as tts_talker_step. */
int tts_talker_step_text(tts_ctx* ctx, const int32_t* prev_codes, const int32_t* text_ids, float* sem_logits);

/* The 15 CodePredictor steps of one frame ("Running Qwen3-TTS on an AMD
 * R9700", section "Running Qwen3-TTS": the smaller transformer fills in the
 * remaining 15 acoustic tokens of the frame, one after the other, and the
 * per-frame cost counts it 15 times; "qwen3-tts-hip" README, section "Library
 * Usage": the subtalker sampling controls), conditioned on the pending Talker
 * hidden and on semantic [B]. ac: acoustic sampling; u [B, 15] uniforms
 * (ignored when greedy; may be NULL then; u[b][j-1] is step j's draw). forced [B, 15] or NULL: when given,
 * forced[b][j-1] replaces the drawn a_j as the input of step j+1 (teacher
 * forcing); the drawn tokens are still written to codes [B, 15] and the
 * logits to logits [B, 15, Va] when non-NULL. */
int tts_codepred_frame(tts_ctx* ctx, const int32_t* semantic, const tts_sampling* ac, const float* u,
                       const int32_t* forced, int32_t* codes, float* logits);

/* Standalone sampler ("qwen3-tts-hip" README, section "Library Usage":
 * do_sample, top_k, top_p, temperature and repetition_penalty for the semantic
 * token, the subtalker_* set for the acoustic tokens) over logits [B, V] with
 * uniforms u [B] (may be NULL when greedy). history [B, V] (uint8, 0/1) or
 * NULL: when given and the penalty is not 1 it selects the penalised ids, and
 * the drawn id is marked in it. out [B] receives the ids. Greedy: V <= 65536;
 * sampled: V <= 4096 (TTS_E_UNSUPPORTED above). */
int tts_sample(tts_ctx* ctx, const float* logits, int32_t batch, int32_t vocab, const tts_sampling* s,
               const float* u, uint8_t* history, int32_t* out);

/* Generate n frames after tts_prefill (or after earlier frames). Frame t
 * (t counts frames since prefill) draws the semantic token from the pending
 * Talker logits with u[b][t][0] and the semantic history, runs the
 * CodePredictor with u[b][t][1..15], writes codes[b][t][0..15], then runs the
 * Talker step on those codes. u and codes are [B, max_frames, 16]. The frame
 * loop replays one captured HIP graph per frame, with positions and the frame
 * index kept on the device. */
int tts_run_frames(tts_ctx* ctx, int32_t n, const tts_sampling* sem, const tts_sampling* ac, const float* u,
                   int32_t* codes);

/* tts_run_frames for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * frames, launched one by one with no graph to instantiate, and the persistent
 * kernels' exchange buffers (2.1 MiB: intra-XCD rings, cross-XCD slots, argmax
 * candidates, Talker attention partials) taken from a static array of this
 * size that each GPU the library runs on holds until the process ends, instead
 * of from the context's workspace. Same arguments, results and errors as
 * tts_run_frames, plus TTS_E_UNSUPPORTED unless both persistent kernels run
 * (batch 1, greedy acoustic tokens, bf16 or E4M3 weights, persistent exec mode) and
 * TTS_E_CAPACITY if their exchange buffers would not fit the array. Calls no
 * allocating routine. The array keeps the last call's contents and is cleared
 * (by a kernel) at the start of every call; calls that overlap on one GPU,
 * from any contexts or threads, race on it. */
int tts_run_frames_noalloc(tts_ctx* ctx, int32_t n, const tts_sampling* sem, const tts_sampling* ac, const float* u,
                           int32_t* codes);

/* Streaming text for tts_run_frames (see tts_talker_step_text). text_ids
 * [B, n_text] (device, int32, borrowed until replaced, cleared by tts_reset or
 * NULL): the Talker step run on frame t's codes (t counts frames since the
 * prefill) adds E_text[text_ids[b][next + t]] while next + t < n_text, nothing
 * after that (ids < 0 add nothing either). For a prefill of the first L ids of
 * an utterance, next = L. NULL switches the text term off. Replacing it drops
 * the captured frame graph. TTS_E_ARG when ids are given with n_text < 1 or
 * next < 0. */
int tts_set_text_stream(tts_ctx* ctx, const int32_t* text_ids, int32_t n_text, int32_t next);

/* Execution of the CodePredictor frame and of the batch-1 Talker step (same
 * results either way, up to floating-point summation order):
 *  TTS_EXEC_PERSISTENT (default where supported): persistent kernels, whose
 *    workgroups split each layer across the 8 XCDs tensor-parallel and
 *    exchange tagged values instead of ending kernels. One runs all 15
 *    CodePredictor steps of a frame (batch 1, greedy acoustic tokens, bf16 or
 *    E4M3 weights, a CodePredictor with 8 KV heads of dimension 128); for the
 *    pages' CodePredictor shape (hidden 1024, FFN 3072, 16 query heads,
 *    vocab 2048) it also draws sampled acoustic tokens itself when top_k is
 *    in 1..64 (the logits gathered by every workgroup; same controls and
 *    decision precision as tts_sample); one runs
 *    a whole Talker step (batch 1, bf16 or E4M3 weights, hidden 512, 1024 or
 *    2048, 8 KV heads of dimension 128 with 2 query heads each, an fp32 KV
 *    cache). Both need a device that keeps all their 256
 *    workgroups resident at once (tts_persistent_allowed). Other calls use the
 *    per-op kernels. The prompt pass never uses them (see tts_set_prefill_mode).
 *  TTS_EXEC_KERNELS: one kernel per op.
 * Switching drops the captured frame graph. TTS_E_UNSUPPORTED if neither
 * persistent kernel handles the config. tts_get_exec_mode reports the mode
 * and, in *persistent_supported, which persistent kernels the config allows
 * (TTS_PERSISTENT_CODEPRED | TTS_PERSISTENT_TALKER). */
enum tts_exec_mode { TTS_EXEC_KERNELS = 0, TTS_EXEC_PERSISTENT = 1 };
enum tts_persistent_kernels { TTS_PERSISTENT_CODEPRED = 1, TTS_PERSISTENT_TALKER = 2 };
int tts_set_exec_mode(tts_ctx* ctx, int32_t mode);
int tts_get_exec_mode(const tts_ctx* ctx, int32_t* mode, int32_t* persistent_supported);

/* How tts_prefill runs the prompt ("Running Qwen3-TTS on an AMD R9700",
 * section "Running Qwen3-TTS": the prompt pass before the frame loop):
 *  TTS_PREFILL_GEMM (default where supported: bf16 or E4M3 weights, head dimension
 *    128, Talker dimensions multiples of 64): chunks of up to 64 positions
 *    per stream as MFMA GEMMs over all streams' rows, causal attention over
 *    the KV cache. fp32 activations enter each GEMM as three bf16 parts
 *    (hi, mid, lo) whose sum is the fp32 value, so the results match the
 *    step path up to summation order.
 *  TTS_PREFILL_STEPS: one position at a time through the decode kernels.
 * TTS_E_UNSUPPORTED when GEMM is asked for and the config cannot use it. */
enum tts_prefill_mode { TTS_PREFILL_STEPS = 0, TTS_PREFILL_GEMM = 1 };
int tts_set_prefill_mode(tts_ctx* ctx, int32_t mode);
int tts_get_prefill_mode(const tts_ctx* ctx, int32_t* mode);

/* Synchronise the context's stream and report the persistent kernel's
 * exchange status: *status = 0 when every exchange completed, nonzero when a
 * workgroup timed out waiting (e.g. not all workgroups were resident); the
 * affected outputs are then invalid. Without this call the same state is
 * reported, one call late and without blocking, as TTS_E_DEVICE by the next
 * call that may launch a persistent kernel. */
int tts_device_status(tts_ctx* ctx, int32_t* status);

/* What the persistent kernels need from a device: gfx950 with 256 compute
 * units on 8 XCDs (each kernel deals its 256 workgroups to the XCDs round
 * robin, 32 to an XCD, and exchanges values through that XCD's L2), and room
 * for at least one of its workgroups (512 threads and its LDS) on a CU.
 * tts_create fills this from the current device and runs the persistent kernels
 * only where tts_persistent_allowed returns their bit; elsewhere the per-op
 * kernels run. arch: the device's gcnArchName ("gfx950:sramecc+:xnack-").
 * codepred_wg_per_cu / talker_wg_per_cu: resident workgroups per CU of the
 * CodePredictor and Talker kernels (hipOccupancyMaxActiveBlocksPerMultiprocessor).
 * Returns TTS_PERSISTENT_CODEPRED | TTS_PERSISTENT_TALKER bits; 0 for NULL. */
typedef struct {
  char arch[64];
  int32_t compute_units;
  int32_t xccs;
  int32_t codepred_wg_per_cu;
  int32_t talker_wg_per_cu;
} tts_device_desc;
int32_t tts_persistent_allowed(const tts_device_desc* d);

/* Host-side counters: Talker positions written so far and frames generated
 * since the last prefill. Either pointer may be NULL. */
int tts_get_progress(const tts_ctx* ctx, int32_t* talker_pos, int32_t* frames);

/* Forget the streams (positions, frames, histories) and clear the persistent
 * kernel's exchange state, including a failure reported by
 * tts_device_status. Weights stay bound. */
int tts_reset(tts_ctx* ctx);

/* Text of the last error on this context ("" if none). Valid until the next
 * call on the context. */
const char* tts_last_error(const tts_ctx* ctx);

/* Release host state and the captured graphs. The workspace and weights are
 * the caller's. Safe on NULL. */
void tts_destroy(tts_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* TTS_H */
