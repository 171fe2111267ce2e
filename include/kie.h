/*
 * kie.h -- C ABI of the batch-1 decode engine for one AMD MI355X (gfx950).
 *
 * What the engine computes. Batch-1 autoregressive decoding of a dense decoder-only transformer,
 * one token at a time, each token depending on the previous one (agentlenshq.com,
 * 《突破内存墙：在标准 GPU 上实现 3,000 tokens/s 的推理速度》, opening section; aikraft.ru
 * «3000 токенов в секунду: как ускорить LLM на обычных GPU», §01). Every active weight is read
 * from HBM once per generated token (same pages: "瓶颈：是内存带宽，而非计算" and §02), and the
 * whole decode path -- MatMul, attention, normalisation and sampling -- runs inside one
 * GPU-resident program that does not return control to the host between tokens ("The Monokernel
 * Runtime" section; §04 "Моноядро"), with sampling on the GPU (§04). The pages do not give the
 * decoder's equations; the engine implements the pre-RMSNorm, RoPE (rotate-half pairs),
 * grouped-query attention and SwiGLU decoder with bf16 weights, a bf16 KV cache, fp32
 * activations and fp32 accumulation.
 *
 * Conventions for every function below
 *   - C99 types only. bf16 values are passed as raw uint16_t bit patterns.
 *   - "device pointer" = memory on the GPU the context was created on (e.g. a torch tensor's
 *     data_ptr()); "host pointer" = ordinary CPU memory.
 *   - All device memory is owned by the caller. The library never allocates device memory.
 *   - Every call enqueues work on the context's stream and returns at once; outputs are valid
 *     after kie_sync() or any synchronisation of that stream.
 *   - Functions never abort and never throw. They return KIE_OK (0) or a negative status;
 *     argument, configuration and capacity errors are found on the host, before anything is
 *     enqueued, and leave the context unchanged. kie_last_error() gives a message.
 */
#ifndef KIE_H
#define KIE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kie_status;
enum {
  KIE_OK = 0,
  KIE_ERR_INVALID_ARG = -1, /* a NULL pointer, a negative size, a token id out of range */
  KIE_ERR_UNSUPPORTED = -2, /* a shape or device the kernels do not handle (see kie_create) */
  KIE_ERR_CAPACITY = -3,    /* position + tokens would exceed max_seq_len */
  KIE_ERR_HIP = -4,         /* a HIP runtime call failed */
  KIE_ERR_STATE = -5,       /* the context holds a device error; call kie_reset() */
  KIE_ERR_TIMEOUT = -6,     /* a device-side wait exceeded its time limit (reported by kie_sync) */
  KIE_ERR_ABORTED = -7      /* the device run stopped early (reported by kie_sync) */
};

/* Model shape. Requirements checked by kie_create: d_model, n_heads*head_dim and ffn_dim are
 * multiples of 256; head_dim is 64 or 128; n_heads is a multiple of n_kv_heads; vocab_size and
 * d_model are even; the number of compute units is a multiple of n_kv_heads.
 * n_experts == 0: dense decoder (the other two expert fields must be 0 too).
 * n_experts > 0: every feed-forward block is a mixture of experts (the pages: only the routed
 * experts' weights are read per token -- aikraft.ru «3000 токенов в секунду…», §02; agentlenshq.com,
 * 《突破内存墙…》, opening section). A router [n_experts][d_model] gives one logit per expert; the
 * n_experts_active experts with the largest logits (ties to the lower index) run, each a SwiGLU
 * block of width expert_ffn_dim, and their outputs are summed with the weights
 * softmax(logits) restricted to the chosen and renormalised to sum to 1. Then ffn_dim must be 0,
 * n_experts even and at most 512, 1 <= n_experts_active <= min(8, n_experts), expert_ffn_dim a
 * multiple of 256, and (kernel instantiation) n_heads / n_kv_heads == 8 with head_dim 128.
 * weight_format: KIE_WEIGHTS_BF16 (0), or KIE_WEIGHTS_FP8_E4M3 (1): the seven matrices of every
 * layer and the LM head are 8-bit codes, which halves the bytes read per token (the pages: 8-bit
 * weights halve the bytes and so about double a bandwidth-bound decoder's ceiling, at a cost in
 * accuracy -- aikraft.ru «3000 токенов в секунду…», §02; wink.run, 《GPU 算力越堆越高,生成 token
 * 为什么还是慢》, on what optimisations change; the engine they describe itself does not quantize,
 * zdabc.icu, 《Kog 推理引擎…》). The pages fix no 8-bit format; this one is the OCP E4M3 encoding
 * (e4m3fn: bias 7, subnormals, no infinities, 0x7F and 0xFF are NaN) with one fp32 scale per matrix
 * (kie_weights.weight_scales): a matrix is its scale times its decoded codes, and each output of
 * a product is the scale times the fp32 sum of code x activation products. Embedding, norm gains
 * and the KV cache stay bf16. Then d_model, n_heads*head_dim and ffn_dim must be multiples of 512,
 * n_experts must be 0, and (kernel instantiation) n_heads / n_kv_heads is 2 with head_dim 64 or
 * 128, or 4 with head_dim 128. A prompt of an 8-bit model runs through the decode program one
 * position after the other (see kie_prefill). */
enum { KIE_WEIGHTS_BF16 = 0, KIE_WEIGHTS_FP8_E4M3 = 1 };
typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab_size;
  float rms_eps, rope_theta;
  int32_t max_seq_len; /* KV capacity in positions: prompt + generated tokens */
  int32_t n_experts, n_experts_active, expert_ffn_dim;
  int32_t weight_format; /* KIE_WEIGHTS_BF16 or KIE_WEIGHTS_FP8_E4M3 */
} kie_config;

/* Source weights: device pointers to row-major [out][in] bf16 matrices, borrowed only until the
 * packing started by kie_create has finished (after the first kie_sync they may be freed).
 * The per-layer members are HOST arrays of n_layers device pointers.
 *   embed [V][d], final_norm [d], lm_head [V][d];
 *   attn_norm[l] [d], wq[l] [n_heads*hd][d], wk[l] and wv[l] [n_kv_heads*hd][d],
 *   wo[l] [d][n_heads*hd], ffn_norm[l] [d], w_gate[l] and w_up[l] [F][d], w_down[l] [d][F].
 * Mixture of experts (E experts of width Fe; w_gate, w_up, w_down are then unused and may be NULL):
 *   w_router[l] [E][d], moe_gate[l] and moe_up[l] [E][Fe][d] (experts stacked), moe_down[l]
 *   [E][d][Fe]. For a dense model these four may be NULL.
 * KIE_WEIGHTS_FP8_E4M3: wq, wk, wv, wo, w_gate, w_up, w_down and lm_head point at one-byte codes
 * in the same [out][in] layouts (read through the uint16_t pointer type as bytes; still 16-byte
 * aligned), and weight_scales is a HOST array of n_layers * 7 + 1 finite floats: per layer the
 * scales of wq, wk, wv, wo, w_gate, w_up, w_down, then the LM head's. It is copied during
 * kie_create (a blocking copy) and may be freed when kie_create returns. NULL for bf16. */
typedef struct {
  const uint16_t *embed, *final_norm, *lm_head;
  const uint16_t *const *attn_norm, *const *wq, *const *wk, *const *wv, *const *wo;
  const uint16_t *const *ffn_norm, *const *w_gate, *const *w_up, *const *w_down;
  const uint16_t *const *w_router, *const *moe_gate, *const *moe_up, *const *moe_down;
  const float* weight_scales;
} kie_weights;

/* Token choice after each step, made on the GPU (aikraft.ru «3000 токенов в секунду…», §04:
 * sampling is taken off the CPU). top_k <= 1: greedy argmax, ties to the lower id. top_k > 1:
 * z = logits / temperature, the top_k largest z (ties to the lower id), p = softmax over them in
 * fp64, u = (splitmix64(seed ^ splitmix64(pos)) >> 40) * 2^-24 with pos the position of the
 * token being processed, and the first candidate whose running sum of p exceeds u. */
typedef struct {
  int32_t top_k;
  float temperature;
  uint64_t seed;
} kie_sampling;

typedef struct kie_ctx kie_ctx;

/* Sizes of the three caller-owned device buffers for a configuration (0 if it is invalid). The
 * packed-weight image holds every weight in consumption order plus the embedding table; the KV
 * cache is [n_layers][2][n_kv_heads][max_seq_len][head_dim] bf16 (K plane then V plane); the
 * workspace holds the inter-workgroup exchange words, the RoPE table and small tables. The GPU
 * used is the current HIP device; the workspace size depends on its compute-unit count. */
size_t kie_packed_weight_bytes(const kie_config* cfg);
size_t kie_kv_cache_bytes(const kie_config* cfg);
size_t kie_workspace_bytes(const kie_config* cfg);

/* Create a context on the current HIP device and enqueue the packing of `src` into `packed`
 * (kie_packed_weight_bytes) on `hip_stream` (a hipStream_t, or NULL for the default stream).
 * The packing lays every weight out in the order in which each wave of each compute unit reads it
 * during one token, one contiguous slice per wave, so that the memory accesses follow the
 * chip's layout (aikraft.ru «3000 токенов в секунду…», §05 on the MI300X chiplet topology;
 * setupai.cc 《Monokernel 推論引擎在 MI300X 上達到每秒 3,300 token》, 技術深入: memory accesses
 * mapped to the physical chiplet topology). The workspace (kie_workspace_bytes) is initialised
 * here; kv_cache (kie_kv_cache_bytes) needs no initialisation. Alignment: packed 16 bytes,
 * kv_cache and workspace 256 bytes (every cache row then owns whole cache lines). Every buffer
 * stays owned by the caller. Position starts at 0. All work is enqueued on hip_stream in order;
 * the call returns before it completes, and `src` must stay valid until the first kie_sync.
 * Errors: KIE_ERR_INVALID_ARG (a NULL or misaligned pointer, bad weight scales), KIE_ERR_UNSUPPORTED
 * (shape, or a device that is not gfx950 / cannot co-schedule one workgroup per compute unit),
 * KIE_ERR_HIP. On error *out is NULL and nothing was enqueued. */
kie_status kie_create(const kie_config* cfg, const kie_weights* src, void* packed, void* kv_cache,
                      void* workspace, void* hip_stream, kie_ctx** out);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): kie_create without the workspace argument. The workspace lives
 * in a static device array of KIE_STATIC_WORKSPACE_MAX bytes inside the library, one per GPU,
 * which each GPU the library runs on holds until the process ends. The call allocates no device
 * memory: it clears the array with a kernel, fills its tables with kernels and device-to-device
 * copies, and packs `src` into `packed` on hip_stream, like kie_create. Such a context runs its
 * prompt through the decode program (kie_prefill), since the matrix-core prompt pass's scratch
 * does not fit the array; everything else behaves as with kie_create. The array keeps the last
 * call's contents and is shared by every context made this way on the GPU: the latest one owns
 * it, and calls that enqueue work on an earlier one (kie_prefill, kie_decode_step, kie_generate,
 * kie_reset) return KIE_ERR_STATE. Calls that overlap on one GPU race. Errors: as kie_create, and
 * KIE_ERR_CAPACITY when the configuration's workspace (without the prompt-pass scratch) exceeds
 * KIE_STATIC_WORKSPACE_MAX. */
#define KIE_STATIC_WORKSPACE_MAX (64u << 20)
kie_status kie_create_static(const kie_config* cfg, const kie_weights* src, void* packed, void* kv_cache,
                             void* hip_stream, kie_ctx** out);

/* The prompt pass: time to first token is a metric of its own, separate from the per-token decode
 * speed (aikraft.ru «3000 токенов в секунду…», §01), and processing a long prompt is bound by
 * arithmetic rather than by memory bandwidth (zdabc.icu, 《Kog 推理引擎：不砍精度，单请求冲到 3000
 * tokens/s》, "AMD vs NVIDIA：两个数字的读法"), so it runs on the matrix cores.
 * Process a prompt of n_tokens ids (device int32 [n_tokens]) at positions pos .. pos+n_tokens-1,
 * writing their K/V rows, then choose the next token (device int32 [1], first_token_dev) from the
 * logits of the last prompt position; those logits are written to last_logits_dev (device fp32
 * [V]) unless it is NULL. Advances the position by n_tokens. All but the last position run as
 * matrix-core GEMMs (8-bit codes are widened to bf16 as the GEMMs read them; in a mixture of
 * experts each position's choice is made as in the decode program and every expert's positions
 * form its own products); the last position runs through the decode program. A context created
 * with kie_create_static has no room for the GEMMs' scratch: there every position runs through
 * the decode program, one after the other, in one launch.
 * Errors: KIE_ERR_INVALID_ARG, KIE_ERR_CAPACITY, KIE_ERR_STATE, KIE_ERR_HIP. */
kie_status kie_prefill(kie_ctx* ctx, const int32_t* tokens_dev, int32_t n_tokens, int32_t* first_token_dev,
                       float* last_logits_dev, const kie_sampling* sampling);

/* One decode step as one kernel launch: the per-launch cost that the monokernel removes
 * (agentlenshq.com, 《突破内存墙…》, "微秒级的损失在哪里": ~4.5 us to launch and clean up a kernel;
 * aikraft.ru «3000 токенов в секунду…», §03) can be measured against kie_generate with it.
 * Process token_in_dev (device int32 [1]) at the current position, write the chosen next token to
 * token_out_dev (device int32 [1]) and, unless NULL, the logits to logits_dev (device fp32 [V]).
 * Identical in results to kie_generate with n_steps = 1. Errors: as kie_generate. */
kie_status kie_decode_step(kie_ctx* ctx, const int32_t* token_in_dev, const kie_sampling* sampling,
                           int32_t* token_out_dev, float* logits_dev);

/* The monokernel: n_steps decode steps in ONE kernel launch, the whole decode path (matrix
 * products, attention, normalisation and sampling) in one GPU-resident program that does not
 * return control to the host between tokens (agentlenshq.com, 《突破内存墙…》, "The Monokernel
 * Runtime"; aikraft.ru «3000 токенов в секунду…», §04 "Моноядро"; setupai.cc 《Monokernel
 * 推論引擎…》, 技術深入).
 * Step s processes token t_s at position pos+s, where t_0 = *first_token_dev and t_s is the token
 * chosen at step s-1, or forced_dev[s-1] when forced_dev (device int32 [n_steps-1 or more]) is
 * given (teacher forcing; the chosen tokens are still written). tokens_out_dev (device int32
 * [n_steps]) receives the chosen token of every step; logits_dev, unless NULL, receives the
 * logits of every step (device fp32 [n_steps][V]). Advances the position by n_steps. The random
 * draw of step s depends only on (seed, pos+s), so n calls of kie_decode_step produce the same
 * tokens as one kie_generate of n steps. Errors: KIE_ERR_INVALID_ARG, KIE_ERR_CAPACITY,
 * KIE_ERR_STATE, KIE_ERR_HIP. */
kie_status kie_generate(kie_ctx* ctx, const int32_t* first_token_dev, int32_t n_steps, const kie_sampling* sampling,
                        const int32_t* forced_dev, int32_t* tokens_out_dev, float* logits_dev);

/* The host's only synchronisation point: the launches run without host round trips (the host-side
 * scheduling and GPU-CPU communication the pages remove from the token loop: agentlenshq.com,
 * 《突破内存墙…》, "微秒级的损失在哪里"), so the host learns their outcome here. Waits for the
 * context's stream and reads the device error word. Returns KIE_OK, KIE_ERR_TIMEOUT (a bounded
 * device wait expired), KIE_ERR_ABORTED (the abort word of kie_set_abort_flag was set, or an
 * input token id was out of range) -- after either the context is in the error state until
 * kie_reset -- or KIE_ERR_HIP. */
kie_status kie_sync(kie_ctx* ctx);

/* Start a new sequence: an agent runs many requests one after the other, each a fresh prompt
 * (agentlenshq.com, 《突破内存墙…》, opening section; aikraft.ru «3000 токенов в секунду…», §01).
 * Position back to 0 and any device error cleared (the KV contents are simply overwritten by
 * later steps). Enqueued on the context's stream. Errors: KIE_ERR_INVALID_ARG, KIE_ERR_HIP. */
kie_status kie_reset(kie_ctx* ctx);

/* Reuse or supply cached context: an agent's loop re-runs from an earlier point of its sequence
 * (agentlenshq.com, 《突破内存墙…》, opening section; aikraft.ru «3000 токенов в секунду…», §01:
 * inspect, plan, edit, test, fix, each step depending on the previous).
 * Set the position to pos (0 <= pos <= max_seq_len). Below the current position it rewinds the
 * sequence so that steps resume at pos (e.g. to re-run a suffix). Above it, the caller states that
 * the K/V rows of positions < pos are already in its kv_cache buffer (written there directly, in
 * the documented layout): later steps attend over them as they are. KIE_ERR_INVALID_ARG
 * otherwise. */
kie_status kie_set_position(kie_ctx* ctx, int32_t pos);

/* Stream the chosen tokens to the host while a launch runs (agentlenshq.com, 《突破内存墙…》,
 * "The Monokernel Runtime", and aikraft.ru «3000 токенов в секунду…», §04: the whole sequence is
 * decoded on the GPU; an agent loop still wants each token as it is produced). ring_host is
 * caller-owned pinned host memory (hipHostMalloc, or a pinned torch tensor) of 1 + capacity int32:
 * ring_host[0] counts the tokens written since this call, and token c sits at ring_host[1 + c %
 * capacity]. Each decode step stores its token and then, with release ordering, the new count
 * (system scope), so a host that reads the count and then the tokens below it sees their values
 * (tokens older than capacity are overwritten). Prompt passes do not write to the ring.
 * ring_host == NULL stops streaming. Errors: KIE_ERR_INVALID_ARG (capacity <= 0, or memory the
 * device cannot write). */
kie_status kie_set_token_stream(kie_ctx* ctx, int32_t* ring_host, int32_t capacity);

/* Stop a running launch from the host. host_word is caller-owned pinned host memory (hipHostMalloc,
 * or a pinned torch tensor) holding one int32 that the library only reads. While it is nonzero,
 * every launch of this context stops at the end of the current decode step (each workgroup reads
 * the word once per step, and while it waits for another workgroup), kie_sync then returns
 * KIE_ERR_ABORTED and the context needs kie_reset. Clear the word before later launches.
 * host_word == NULL removes it (the default). The pages' engine leaves the token loop entirely to
 * the GPU (agentlenshq.com, 《突破内存墙…》, "The Monokernel Runtime"); this is the host's way back
 * in. Errors: KIE_ERR_INVALID_ARG (memory the device cannot read). */
kie_status kie_set_abort_flag(kie_ctx* ctx, int32_t* host_word);

/* Current position (number of tokens whose K/V rows are in the cache), or -1 for NULL. */
int32_t kie_position(const kie_ctx* ctx);

/* Static description of a status code. */
const char* kie_status_string(kie_status status);

/* Message of the last error on this context ("" if none); for NULL, the last kie_create error. */
const char* kie_last_error(const kie_ctx* ctx);

/* Release the host-side context (no device memory is owned). NULL is accepted. */
void kie_destroy(kie_ctx* ctx);

/* Number of workgroups (= compute units) of the persistent kernel on the current device, or a
 * negative status. */
int32_t kie_num_workgroups(void);

#ifdef __cplusplus
}
#endif
#endif /* KIE_H */
