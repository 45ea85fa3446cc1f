// Internal interface between the C-ABI host layer (kda_api.cpp) and the HIP
// kernel translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int64_t kChunkTokens = 16;

// Per-(batch, head, chunk) workspace record of the fp32-input path, written by
// the chunk-prep kernel and read by the state-pass kernel. Offsets in bytes;
// total is a multiple of 1024 (whole units of 64 lanes x 16 bytes, the state
// pass's load granule). All operands are fp32.
//   w     -W (16 x dk)          q    Qt (16 x dk)        kbar  Kb (16 x dk)
//   m     M (16 x 16)           tb   Tm diag(beta)       eg    e^gamma (dk)
struct RecordLayout {
  int64_t w, q, kbar, m, tb, eg, bytes;
};

inline RecordLayout record_layout(int64_t dk) {
  RecordLayout L;
  const int64_t tile = dk * kChunkTokens * 4;  // 16 tokens x dk, fp32
  L.w = 0;
  L.q = tile;
  L.kbar = 2 * tile;
  L.m = 3 * tile;
  L.tb = L.m + 1024;
  L.eg = L.tb + 1024;
  const int64_t end = L.eg + dk * 4;
  L.bytes = (end + 1023) / 1024 * 1024;  // whole 1 KiB units: 64 lanes x 16 bytes
  return L;
}

// Per-(batch, head, pair of chunks) workspace record of the bf16-input path:
// the state pass advances 32 tokens (two 16-token chunks c1, c2) per step.
// Operands in fragment order (see kda_chunk.hip). The tiles that multiply
// the state or the update are fp16; those that multiply v keep v exact in
// bf16 and are split into bf16 high and low parts:
//   w1, w2   -W of c1 and -W of c2 times Diag(e^gamma1)      (16 x dk each, fp16)
//   q1, q2   Qt of c1 and Qt of c2 times Diag(e^gamma1)      (fp16)
//   kb       [Kb of c1 times Diag(e^gamma2) | Kb of c2]      (dk x 32, fp16)
//   m1       [M of c1, high | low parts]                      (fp16)
//   m2h, m2l [M21 | M of c2], high and low parts, M21 = Qt2 Kb1^T
//   tb1, tb2 Tm beta of c1 and of c2, [high | low] (bf16)
//   c21      -C21, C21 = W2 Kb1^T                             (fp16)
//   eg       e^(gamma1 + gamma2) per channel, fp32
struct PairLayout {
  int64_t w1, w2, q1, q2, kb, m1, m2h, m2l, tb1, tb2, c21, eg, bytes;
};

inline PairLayout pair_layout(int64_t dk) {
  PairLayout L;
  const int64_t tile = dk * kChunkTokens * 2;  // 16 tokens x dk, fp16
  L.w1 = 0;
  L.w2 = tile;
  L.q1 = 2 * tile;
  L.q2 = 3 * tile;
  L.kb = 4 * tile;            // dk x 32 tokens
  L.m1 = 6 * tile;            // 64 lanes x 16 bytes each from here on
  L.m2h = L.m1 + 1024;
  L.m2l = L.m2h + 1024;
  L.tb1 = L.m2l + 1024;
  L.tb2 = L.tb1 + 1024;
  L.c21 = L.tb2 + 1024;       // 64 lanes x 8 bytes
  L.eg = L.c21 + 512;
  const int64_t end = L.eg + dk * 4;
  L.bytes = (end + 1023) / 1024 * 1024;  // whole 1 KiB units: 64 lanes x 16 bytes
  return L;
}

// How the g input becomes the per-channel log-decay (kda_gate values).
enum GateMode : int { kGateLogDecay = 0, kGateSigmoid = 1 };

struct ChunkFwdArgs {
  const void *q, *k, *v, *g, *beta;
  const float* S0;
  void* o;
  float* S_T;
  int64_t B, T, H, dk, dv;
  int in_dtype, out_dtype;  // kda_dtype values
  void* workspace;
  int gate = kGateLogDecay;
  float* snapshots = nullptr;     // [B, T / snapshot_every, H, dk, dv] or null
  int64_t snapshot_every = 0;     // tokens between snapshots, a multiple of 32
  float* E_out = nullptr;         // the transition's E beside F (one pass over dk + dv columns)
};

struct DecodeArgs {
  const void *q, *k, *v, *g, *beta;
  float* S;
  void* o;
  int64_t N, H, dk, dv;
  int in_dtype, out_dtype;
  int gate = kGateLogDecay;
};

// Speculative verification / commit over T logged tokens per request.
// verify: o for all T tokens from S, S unchanged; commit: S advanced in place
// by accepted[n] tokens (clamped to [0, T]), no output.
struct SpecArgs {
  const void *q, *k, *v, *g, *beta;
  float* S;
  void* o;
  const int32_t* accepted;
  int64_t N, T, H, dk, dv;
  int in_dtype, out_dtype;
  int gate = kGateLogDecay;
};

// The state transition F [B, H, dk, dk] of the prepared tokens and/or the
// state E [B, H, dk, dv] they reach from zero (either may be null), from a
// workspace written by launch_chunk_prep; `a` supplies v, the sizes, dtype and
// workspace.
hipError_t launch_chunk_transition(const ChunkFwdArgs& a, float* F, float* E, hipStream_t stream);

// S[r + 1] = F[r] S[r] + E[r] for r = 0 .. P-1 with S[0] = S0 (zeros when
// null), per unit n: F [P, N, dk, dk], E [P, N, dk, dv], S [P + 1, N, dk, dv].
hipError_t launch_affine_scan(const float* F, const float* E, const float* S0, float* S,
                              int64_t P, int64_t N, int64_t dk, int64_t dv, hipStream_t stream);

// Size of the built-in device scratch of the no-allocation forward (one copy
// per device, held until the process ends).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;

// This device's address of the built-in scratch (looked up once per device,
// with the device current); fails for devices beyond the supported count.
hipError_t noalloc_scratch(void** ptr);

// Launch the chunkwise forward (prep kernel then state pass) on `stream`.
hipError_t launch_chunk_fwd(const ChunkFwdArgs& a, hipStream_t stream);
// The two stages on their own (fields of `a` a stage does not use are ignored).
hipError_t launch_chunk_prep(const ChunkFwdArgs& a, hipStream_t stream);
hipError_t launch_chunk_state_pass(const ChunkFwdArgs& a, hipStream_t stream);

// Launch one decode step on `stream`.
hipError_t launch_decode_step(const DecodeArgs& a, hipStream_t stream);

// Launch a speculative verification (commit = false) or commit (commit = true).
hipError_t launch_spec(const SpecArgs& a, bool commit, hipStream_t stream);

// The previous round's logged tokens for kda_spec_commit_verify: k1, g1
// [N, T1, H, dk], v1 [N, T1, H, dv], beta1 [N, T1, H] and the accepted
// counts; the SpecArgs beside them describe the next round's drafts.
struct SpecPrefix {
  const void *k1, *v1, *g1, *beta1;
  const int32_t* accepted;
  int64_t T1;
};
hipError_t launch_spec_commit_verify(const SpecArgs& drafts, const SpecPrefix& pre,
                                     hipStream_t stream);

}  // namespace kda
