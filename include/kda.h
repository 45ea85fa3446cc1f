/*
 * kda.h — C ABI of libkda.so: Kimi Delta Attention (KDA) on AMD Instinct MI355X
 * (gfx950, CDNA4).
 *
 * The operation. Per batch b and head h a fixed-size state S (dk x dv, fp32) is
 * carried along the sequence. For each token t, with log-decay g_t (one value
 * per key channel), write strength beta_t, key k_t, value v_t and query q_t:
 *
 *     g_t <- clamp(g_t, -5, 0)
 *     S_t  = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *     o_t  = S_t^T q_t                       (read after the write, no scaling)
 *
 * Sources: a recurrent state updated with a learned write strength and
 * channel-wise forgetting, with the log-decay floored at -5 so that reciprocal
 * decay scaling over a 16-token tile stays inside bf16 range and the diagonal
 * tiles run as dense matrix products ("K3 tech report" podcast transcript, the
 * exchanges on Kimi Delta Attention and on the decay bound); a delta rule with
 * channel-wise forget gates and a lower bound on retention ("177: Kimi K3 in
 * Detail", section 15); a fixed-size recurrent state with a floored,
 * lower-bounded decay and dense diagonal and off-diagonal tiles ("Kimi K3 goes
 * trillion-scale with sparse MoE efficiency" subtitles, cue 14); a state that
 * is overwritten and read again for every token during decoding ("177: Kimi K3
 * in Detail", sections 10 and 17).
 *
 * Conventions shared by every entry point:
 *  - Every buffer is owned by the caller. Tensor pointers are device pointers
 *    (hipMalloc'd or equivalent). The library allocates nothing and keeps no
 *    global state; calls are re-entrant and may run on any stream.
 *  - Tensors are dense, row-major, packed (no strides). Alignment: q, k, g
 *    to 4 elements (16 bytes for fp32, 8 bytes for bf16); the forward's v
 *    and o, the workspace and the decode and speculative states S to 16
 *    bytes; every other tensor to its element size.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = null stream).
 *    All argument checks happen on the host before anything is launched; on
 *    any error nothing is launched and no output is written.
 *  - Log-decays outside [-5, 0] are clamped to the bound; NaN and Inf in any
 *    input propagate to the outputs (there are no device-side error paths).
 *    With KDA_GATE_SIGMOID, g holds gate logits instead (see kda_gate).
 *  - in_dtype applies to q, k, v, g, beta alike. The state is always fp32.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 4

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,         /* a required pointer is NULL */
    KDA_ERR_SHAPE = 2,        /* a size is negative or inconsistent */
    KDA_ERR_UNSUPPORTED = 3,  /* a supported-size or dtype rule is broken */
    KDA_ERR_ALIAS = 4,        /* an output overlaps an input it must not */
    KDA_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than required */
    KDA_ERR_HIP = 6,          /* the HIP runtime reported an error on launch */
    KDA_ERR_ALIGNMENT = 7,    /* a tensor pointer breaks its alignment rule */
    KDA_ERR_TOO_LARGE = 8     /* more scratch than kda_chunk_fwd_noalloc holds */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/*
 * What the g input holds (the *_ex and kda_spec_* entry points take it; the
 * others use KDA_GATE_LOG_DECAY).
 *  KDA_GATE_LOG_DECAY  g is the per-channel log-decay, clamped to [-5, 0].
 *  KDA_GATE_SIGMOID    g is a raw gate logit x; the log-decay is
 *                      -5 / (1 + exp(-x)) = -5 sigmoid(x), in (-5, 0): a
 *                      lower-bounded sigmoid decay whose retention factor
 *                      never falls below e^-5 ("Kimi K3 goes trillion-scale
 *                      with sparse MoE efficiency" subtitles, cue 14; the
 *                      pages give the bound, not the formula: scaling the
 *                      sigmoid to the bound is this library's reading).
 */
typedef enum { KDA_GATE_LOG_DECAY = 0, KDA_GATE_SIGMOID = 1 } kda_gate;

/* ABI version of the loaded library (KDA_ABI_VERSION at build time). */
int kda_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* kda_status_str(int status);

/*
 * Failure injection, for testing callers' error handling without a failing
 * device: the next `count` calls that pass their argument checks return
 * KDA_ERR_HIP instead of launching, before any HIP call (count <= 0 clears
 * it). Process-wide; meant for tests, never needed in normal use.
 */
void kda_debug_inject_launch_failures(int count);

/*
 * Bytes of device workspace kda_chunk_fwd needs for these sizes and input
 * dtype (0 when T, B or H is 0). Returns 0 as well for unsupported sizes;
 * kda_chunk_fwd then reports the precise error.
 */
size_t kda_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t dk,
                                    int64_t dv, int in_dtype);

/*
 * Chunkwise forward (prefill) of the recurrence above over T tokens.
 *
 *   q, k, g  [B, T, H, dk]  in_dtype
 *   v        [B, T, H, dv]  in_dtype
 *   beta     [B, T, H]      in_dtype
 *   S0       [B, H, dk, dv] fp32, state before token 0; NULL means zeros
 *   o        [B, T, H, dv]  out_dtype, written for every token
 *   S_T      [B, H, dk, dv] fp32, state after token T-1; NULL means not wanted.
 *            S_T may be the very same pointer as S0 (update in place); any
 *            other overlap of outputs with inputs is KDA_ERR_ALIAS.
 *   workspace, workspace_bytes: device scratch of at least
 *            kda_chunk_fwd_workspace_size(...) bytes, owned by the caller,
 *            not read before it is written; contents after the call are
 *            unspecified. Must not overlap any tensor. Calls that run at
 *            the same time must not share a workspace.
 *
 * Supported: dk in {64, 128}; dv a multiple of 16 in [16, 512]; B, H >= 0
 * with H * dv <= 2^25;
 * T >= 0 (T = 0 copies S0, or zeros, into S_T). in_dtype KDA_F32 (all fp32
 * arithmetic, fp32 matrix-core products) or KDA_BF16 (bf16 inputs; bf16
 * split-precision chunk Gram products, fp16 state and update products, v
 * exact in bf16 products, fp32 accumulation and fp32 state); out_dtype
 * KDA_F32 or KDA_BF16.
 * The computation works in chunks of 16 tokens aligned at t = 0; a last
 * partial chunk is padded internally with tokens that leave S unchanged.
 * With KDA_BF16 inputs the sequential pass advances two chunks (32 tokens)
 * per step. Values of v, S0, the state and the per-chunk update have no
 * range limit beyond fp32's: a slice whose state would leave the fp16
 * operand range (or fall far below it) is recomputed with an exact
 * power-of-two scale. The precomputed per-chunk operands are held in fp16;
 * they are at most 1 in magnitude for queries and keys of norm at most 1
 * (the method's L2-normalised q and k) and beta in [0, 1].
 */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* S0, void* o, float* S_T,
                         int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                         int in_dtype, int out_dtype, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Host-only check of kda_chunk_fwd's arguments: returns exactly the status
 * kda_chunk_fwd would return before launching (KDA_OK when it would launch).
 * Touches no device memory and makes no HIP call.
 */
kda_status kda_chunk_fwd_check(const void* q, const void* k, const void* v,
                               const void* g, const void* beta, const float* S0,
                               const void* o, const float* S_T, int64_t B, int64_t T,
                               int64_t H, int64_t dk, int64_t dv, int in_dtype,
                               int out_dtype, const void* workspace,
                               size_t workspace_bytes);

/*
 * The two stages kda_chunk_fwd runs, exposed separately (same arguments and
 * rules as kda_chunk_fwd). kda_chunk_fwd(...) is exactly kda_chunk_prep then
 * kda_chunk_state_pass on the same stream.
 *
 * kda_chunk_prep: every 16-token chunk of every (b, h) independently — the
 * per-chunk cumulative log-decay, the decay-scaled query and key operands, the
 * chunk Gram tiles, (I + strictly_lower(diag(beta) Kt Kh^T))^-1 and the
 * products the state pass needs (with KDA_BF16 inputs, per pair of chunks,
 * including the two tiles that couple the pair's chunks) — written to
 * `workspace`. Reads q, k, g, beta
 * only; the workspace then depends on nothing else, so one prep can feed
 * several state passes (e.g. replays of the same tokens from different
 * initial states, where only S0 and v change).
 *
 * kda_chunk_state_pass: the sequential pass over the chunks of each (b, h)
 * from S0, reading v and the workspace written by kda_chunk_prep for the same
 * B, T, H, dk, dv and in_dtype; writes o and S_T. With KDA_BF16 inputs it
 * also writes a few bytes of the workspace past the prepared operands (one
 * flag per 16-column slice of the state), so two state passes over one
 * workspace must not run at the same time.
 */
kda_status kda_chunk_prep(const void* q, const void* k, const void* g, const void* beta,
                          int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                          int in_dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

kda_status kda_chunk_state_pass(const void* v, const void* workspace,
                                size_t workspace_bytes, const float* S0, void* o,
                                float* S_T, int64_t B, int64_t T, int64_t H, int64_t dk,
                                int64_t dv, int in_dtype, int out_dtype, void* stream);

/*
 * One decode step: one token for each of N independent requests, updating
 * each request's state in place.
 *
 *   q, k, g  [N, H, dk]      in_dtype
 *   v        [N, H, dv]      in_dtype
 *   beta     [N, H]          in_dtype
 *   S        [N, H, dk, dv]  fp32, read and overwritten with the new state
 *   o        [N, H, dv]      out_dtype, o = S_new^T q
 *
 * Supported: dk, dv in {64, 128}; N, H >= 0. o must not overlap any input
 * or S. Each state is read once and written once (memory-bound).
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* g,
                           const void* beta, float* S, void* o, int64_t N, int64_t H,
                           int64_t dk, int64_t dv, int in_dtype, int out_dtype,
                           void* stream);

/* Host-only check of kda_decode_step's arguments (see kda_chunk_fwd_check). */
kda_status kda_decode_step_check(const void* q, const void* k, const void* v,
                                 const void* g, const void* beta, const float* S,
                                 const void* o, int64_t N, int64_t H, int64_t dk,
                                 int64_t dv, int in_dtype, int out_dtype);

/*
 * kda_chunk_fwd with two options.
 *
 *   gate            a kda_gate value: how g is read (KDA_ERR_UNSUPPORTED
 *                   otherwise).
 *   snapshots,      state snapshots every `snapshot_every` tokens, for prefix
 *   snapshot_every  reuse: the state after tokens [0, (j+1) * snapshot_every)
 *                   of sequence b is written to snapshots[b, j] for
 *                   j = 0 .. T / snapshot_every - 1, with layout
 *                   [B, T / snapshot_every, H, dk, dv] fp32. snapshot_every
 *                   is 0 (none; snapshots ignored) or a positive multiple
 *                   of 32, the state pass's step (KDA_ERR_UNSUPPORTED
 *                   otherwise; negative is KDA_ERR_SHAPE); snapshots may be
 *                   NULL only when no
 *                   snapshot falls inside T. They must not overlap any
 *                   other tensor or the workspace. 4-byte aligned.
 *
 * Snapshots serve a prefix cache that hashes fixed blocks of 512 tokens and
 * shares the recurrent state of a hit across requests ("177: Kimi K3 in
 * Detail", sections 10 and 16). Since chunks and pairs of chunks align at
 * t = 0 and snapshot_every is a multiple of 32, a later kda_chunk_fwd over the tokens
 * after snapshot j with S0 = snapshots[b, j] (for B = 1 that block is
 * exactly an [H, dk, dv] state) performs the same arithmetic as the
 * uninterrupted run: its o and S_T are bit-identical to the full run's.
 */
kda_status kda_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* S0, void* o, float* S_T,
                            int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                            int in_dtype, int out_dtype, int gate, float* snapshots,
                            int64_t snapshot_every, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Host-only check of kda_chunk_fwd_ex's arguments (see kda_chunk_fwd_check). */
kda_status kda_chunk_fwd_ex_check(const void* q, const void* k, const void* v,
                                  const void* g, const void* beta, const float* S0,
                                  const void* o, const float* S_T, int64_t B, int64_t T,
                                  int64_t H, int64_t dk, int64_t dv, int in_dtype,
                                  int out_dtype, int gate, const float* snapshots,
                                  int64_t snapshot_every, const void* workspace,
                                  size_t workspace_bytes);

/* kda_decode_step with a kda_gate value for g (KDA_ERR_UNSUPPORTED otherwise). */
kda_status kda_decode_step_ex(const void* q, const void* k, const void* v, const void* g,
                              const void* beta, float* S, void* o, int64_t N, int64_t H,
                              int64_t dk, int64_t dv, int in_dtype, int out_dtype,
                              int gate, void* stream);

/*
 * Speculative decoding: verification from a checkpoint, then commit by
 * replay. The state is rewritten by every token, so a rejected draft cannot
 * be torn off afterwards; instead the state at the last accepted position is
 * kept, the draft tokens' inputs are logged (about 1 KiB per head and token
 * at d = 128), and the accepted prefix is replayed from the checkpoint
 * ("177: Kimi K3 in Detail", section 23; "Kimi K3 goes trillion-scale with
 * sparse MoE efficiency" subtitles, cue 28).
 *
 * kda_spec_verify: for N requests with T draft tokens each, the outputs of
 * all T tokens, stepping from the checkpoint S, which is only read. o[n, t]
 * equals what T successive kda_decode_step calls from S would return.
 *
 *   q, k, g  [N, T, H, dk]  in_dtype
 *   v        [N, T, H, dv]  in_dtype
 *   beta     [N, T, H]      in_dtype
 *   S        [N, H, dk, dv] fp32, the checkpoint (read only); 16-byte aligned
 *   o        [N, T, H, dv]  out_dtype; must not overlap any input or S
 *
 * kda_spec_commit: S advanced in place over the first accepted[n] tokens of
 * request n (values outside [0, T] are clamped to it; 0 leaves S unchanged).
 * The result equals accepted[n] successive kda_decode_step calls. q and o are
 * not involved.
 *
 *   k, g, v, beta   as for kda_spec_verify
 *   S               [N, H, dk, dv] fp32, in place; 16-byte aligned
 *   accepted        [N] int32 on the device, 4-byte aligned
 *
 * Supported: dk, dv in {64, 128}; N, T, H >= 0; gate a kda_gate value. A
 * verify + commit pair reads the state twice and writes it once whatever T
 * is, where T decode steps would read and write it T times each.
 */
kda_status kda_spec_verify(const void* q, const void* k, const void* v, const void* g,
                           const void* beta, const float* S, void* o, int64_t N, int64_t T,
                           int64_t H, int64_t dk, int64_t dv, int in_dtype, int out_dtype,
                           int gate, void* stream);

kda_status kda_spec_commit(const void* k, const void* v, const void* g, const void* beta,
                           float* S, const int32_t* accepted, int64_t N, int64_t T,
                           int64_t H, int64_t dk, int64_t dv, int in_dtype, int gate,
                           void* stream);

/* Host-only checks of the two calls above (see kda_chunk_fwd_check). */
kda_status kda_spec_verify_check(const void* q, const void* k, const void* v,
                                 const void* g, const void* beta, const float* S,
                                 const void* o, int64_t N, int64_t T, int64_t H,
                                 int64_t dk, int64_t dv, int in_dtype, int out_dtype,
                                 int gate);

kda_status kda_spec_commit_check(const void* k, const void* v, const void* g,
                                 const void* beta, const float* S,
                                 const int32_t* accepted, int64_t N, int64_t T, int64_t H,
                                 int64_t dk, int64_t dv, int in_dtype, int gate);

/*
 * kda_spec_commit_verify: the boundary between two speculative rounds in one
 * pass over the state (the replay of logged inputs from the checkpoint, as
 * above). S is first advanced in place over the first accepted[n] of the T1
 * tokens logged in the previous round (exactly as kda_spec_commit), and then
 * o[n, t] is formed for the T2 draft tokens of the next round, stepping from
 * the advanced state, which the drafts leave unchanged (as kda_spec_verify).
 * The result equals kda_spec_commit followed by kda_spec_verify, up to the
 * rounding order of the sums over dk; the state is read once and written
 * once, where the two calls read it twice and write it once.
 *
 *   k1, g1    [N, T1, H, dk]  in_dtype   logged tokens of the previous round
 *   v1        [N, T1, H, dv]  in_dtype
 *   beta1     [N, T1, H]      in_dtype
 *   accepted  [N] int32 on the device, 4-byte aligned; clamped to [0, T1]
 *   q2, k2, g2 [N, T2, H, dk] in_dtype   draft tokens of the next round
 *   v2        [N, T2, H, dv]  in_dtype
 *   beta2     [N, T2, H]      in_dtype
 *   S         [N, H, dk, dv] fp32, in place; 16-byte aligned
 *   o         [N, T2, H, dv]  out_dtype
 *
 * S and o must not overlap any input, nor each other. T1 = 0 leaves S as it
 * is (a plain verify); T2 = 0 writes no output (a plain commit). Pointers
 * need element alignment only; with q2, k2, g2, v2, k1, g1 and v1 all 16-byte
 * aligned the two steps run as one kernel, otherwise as the two calls'
 * kernels in order. Errors as for the two calls.
 */
kda_status kda_spec_commit_verify(const void* k1, const void* v1, const void* g1,
                                  const void* beta1, const int32_t* accepted, int64_t T1,
                                  const void* q2, const void* k2, const void* v2,
                                  const void* g2, const void* beta2, int64_t T2, float* S,
                                  void* o, int64_t N, int64_t H, int64_t dk, int64_t dv,
                                  int in_dtype, int out_dtype, int gate, void* stream);

/* Host-only check of kda_spec_commit_verify (see kda_chunk_fwd_check). */
kda_status kda_spec_commit_verify_check(const void* k1, const void* v1, const void* g1,
                                        const void* beta1, const int32_t* accepted, int64_t T1,
                                        const void* q2, const void* k2, const void* v2,
                                        const void* g2, const void* beta2, int64_t T2,
                                        const float* S, const void* o, int64_t N, int64_t H,
                                        int64_t dk, int64_t dv, int in_dtype, int out_dtype,
                                        int gate);

/*
 * Context-parallel prefill, the part one device runs: a sequence cut into
 * spans is prepared and passed span by span without knowing the state that
 * enters each span, and the spans are joined afterwards (KDA context
 * parallelism: "K3 tech report" podcast transcript, the exchange on
 * recreating the training efficiency; "Kimi K3 goes trillion-scale with
 * sparse MoE efficiency" subtitles, cue 22). The recurrence is affine in the
 * state: a span maps its entering state S_in to F S_in + E, with F its state
 * transition and E the state it reaches from zero.
 *
 * kda_chunk_transition: for the tokens of a workspace written by
 * kda_chunk_prep (same B, T, H, dk, dv, in_dtype), the transition
 *   F  [B, H, dk, dk] fp32, the state after the tokens from S_in = I with
 *      v = 0 (NULL: not wanted)
 * and the state from zero
 *   E  [B, H, dk, dv] fp32, the state after the tokens from S_in = 0
 *      (NULL: not wanted; v is then not read and may be NULL)
 *   v  [B, T, H, dv] in_dtype, 16-byte aligned (needed for E only).
 * F costs a state pass over dk columns that reads no v and writes no
 * outputs (cheaper than kda_chunk_state_pass over an identity state and zero
 * values, which writes T x H x dk outputs); E a state pass without outputs.
 * T = 0 gives F = I, E = 0. F and E must not overlap each other, v or the
 * workspace. Same sizes and rules as kda_chunk_fwd otherwise; the workspace
 * is written past the prepared operands as by kda_chunk_state_pass.
 *
 * kda_state_affine_scan: the entering state of every span,
 *   S[0] = S0,  S[r + 1] = F[r] S[r] + E[r],  r = 0 .. P-1,
 * for N independent units (N = B * H):
 *   F   [P, N, dk, dk] fp32, 16-byte aligned
 *   E   [P, N, dk, dv] fp32
 *   S0  [N, dk, dv]    fp32 (NULL means zeros)
 *   S   [P + 1, N, dk, dv] fp32 out; S[P] is the state after the last span.
 *       S must not overlap F, E or S0.
 * Products in fp32 on the matrix cores, fp32 accumulation. dk in {64, 128};
 * dv a multiple of 16 in [16, 512]; P, N >= 0.
 */
kda_status kda_chunk_transition(const void* v, const void* workspace, size_t workspace_bytes,
                                float* F, float* E, int64_t B, int64_t T, int64_t H, int64_t dk,
                                int64_t dv, int in_dtype, void* stream);

kda_status kda_state_affine_scan(const float* F, const float* E, const float* S0, float* S,
                                 int64_t P, int64_t N, int64_t dk, int64_t dv, void* stream);

/* Host-only checks of the two calls above (see kda_chunk_fwd_check). */
kda_status kda_chunk_transition_check(const void* v, const void* workspace,
                                      size_t workspace_bytes, const float* F, const float* E,
                                      int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                      int in_dtype);

kda_status kda_state_affine_scan_check(const float* F, const float* E, const float* S0,
                                       const float* S, int64_t P, int64_t N, int64_t dk,
                                       int64_t dv);

/*
 * kda_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same arguments, rules and results as
 * kda_chunk_fwd (bit for bit), minus workspace and workspace_bytes. It uses a
 * scratch array built into the library instead: KDA_NOALLOC_SCRATCH_BYTES per
 * device, held from the library's first use on a device until the process
 * ends. Calls whose kda_chunk_fwd_workspace_size(...) exceeds it return
 * KDA_ERR_TOO_LARGE before anything runs (at d = 128 with bf16 inputs that
 * is about 2,150 pairs of chunks over all (b, h), e.g. 32 heads of 2,048
 * tokens). It makes no allocation of its own (the first call on a device
 * only looks up the array's device address). Every call on a device shares
 * the one array: calls that overlap in time on the same device (on different
 * streams, or from different threads) race and must not be issued.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)

kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g,
                                 const void* beta, const float* S0, void* o, float* S_T,
                                 int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                 int in_dtype, int out_dtype, void* stream);

/* Host-only check of kda_chunk_fwd_noalloc's arguments (see kda_chunk_fwd_check). */
kda_status kda_chunk_fwd_noalloc_check(const void* q, const void* k, const void* v,
                                       const void* g, const void* beta, const float* S0,
                                       const void* o, const float* S_T, int64_t B, int64_t T,
                                       int64_t H, int64_t dk, int64_t dv, int in_dtype,
                                       int out_dtype);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
