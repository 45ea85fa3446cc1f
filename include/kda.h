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
 *    to 4 elements (16 bytes for fp32, 8 bytes for bf16); the forward's v,
 *    the workspace and the decode state S to 16 bytes; every other tensor to
 *    its element size.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = null stream).
 *    All argument checks happen on the host before anything is launched; on
 *    any error nothing is launched and no output is written.
 *  - Log-decays outside [-5, 0] are clamped to the bound; NaN and Inf in any
 *    input propagate to the outputs (there are no device-side error paths).
 *  - in_dtype applies to q, k, v, g, beta alike. The state is always fp32.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,         /* a required pointer is NULL */
    KDA_ERR_SHAPE = 2,        /* a size is negative or inconsistent */
    KDA_ERR_UNSUPPORTED = 3,  /* a supported-size or dtype rule is broken */
    KDA_ERR_ALIAS = 4,        /* an output overlaps an input it must not */
    KDA_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than required */
    KDA_ERR_HIP = 6,          /* the HIP runtime reported an error on launch */
    KDA_ERR_ALIGNMENT = 7     /* a tensor pointer breaks its alignment rule */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* ABI version of the loaded library (KDA_ABI_VERSION at build time). */
int kda_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* kda_status_str(int status);

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
 *            unspecified. Must not overlap any tensor.
 *
 * Supported: dk in {64, 128}; dv a multiple of 16 in [16, 512]; B, H >= 0
 * with H * dv <= 2^25;
 * T >= 0 (T = 0 copies S0, or zeros, into S_T). in_dtype KDA_F32 (all fp32
 * arithmetic, fp32 matrix-core products) or KDA_BF16 (bf16 inputs; bf16
 * split-precision chunk Gram products, fp16 state products, fp32
 * accumulation and fp32 state); out_dtype KDA_F32 or KDA_BF16.
 * The computation works in chunks of 16 tokens aligned at t = 0; a last
 * partial chunk is padded internally with tokens that leave S unchanged.
 * With KDA_BF16 inputs, entries of v, of the state and of the per-chunk
 * update (beta times prediction error) must stay below 65504 in magnitude.
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
 * products the state pass needs — written to `workspace`. Reads q, k, g, beta
 * only; the workspace then depends on nothing else, so one prep can feed
 * several state passes (e.g. replays of the same tokens from different
 * initial states, where only S0 and v change).
 *
 * kda_chunk_state_pass: the sequential pass over the chunks of each (b, h)
 * from S0, reading v and the workspace written by kda_chunk_prep for the same
 * B, T, H, dk, dv and in_dtype; writes o and S_T.
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

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
