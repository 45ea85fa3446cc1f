// C-ABI host layer of libkda.so: argument checks, workspace sizing, dispatch
// to the HIP launchers. See include/kda.h for the contract.
#include "kda.h"

#include <hip/hip_runtime_api.h>

#include <atomic>

#include "kda_launch.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t elems, int64_t esize) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(elems) * static_cast<uintptr_t>(esize)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

bool dtype_ok(int d) { return d == KDA_F32 || d == KDA_BF16; }
int64_t dsize(int d) { return d == KDA_F32 ? 4 : 2; }

// Products of sizes must not overflow; every size here is bounded first.
constexpr int64_t kMaxElems = int64_t(1) << 46;

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_str(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "a size is negative or inconsistent";
    case KDA_ERR_UNSUPPORTED: return "unsupported size or dtype";
    case KDA_ERR_ALIAS: return "an output overlaps an input it must not";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_HIP: return "HIP runtime error on launch";
    case KDA_ERR_ALIGNMENT: return "a tensor pointer breaks its alignment rule";
    case KDA_ERR_TOO_LARGE:
      return "the call needs more workspace than the built-in scratch holds "
             "(KDA_NOALLOC_SCRATCH_BYTES); use kda_chunk_fwd with a workspace";
    default: return "unknown status";
  }
}

size_t kda_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                    int in_dtype) {
  if (B < 0 || T < 0 || H < 0 || (dk != 64 && dk != 128) || !dtype_ok(in_dtype)) return 0;
  if (dv < 16 || dv > 512 || dv % 16 != 0) return 0;
  if (B > kMaxElems || T > kMaxElems || H > kMaxElems) return 0;
  // fp32 inputs: one record per 16-token chunk; bf16 inputs: one per pair
  // of chunks, then one int per (b, h, 16-column slice) for the state pass
  // (whole KiB)
  const int64_t units = in_dtype == KDA_F32 ? (T + 15) / 16 : (T + 31) / 32;
  const int64_t bytes = in_dtype == KDA_F32 ? kda::record_layout(dk).bytes : kda::pair_layout(dk).bytes;
  const double total = static_cast<double>(B) * H * units * bytes;
  if (total > 9.0e18) return 0;
  if (units == 0 || B * H == 0) return 0;
  const int64_t cols = dk + dv;  // the transition's F and E run as one pass over dk + dv columns
  const int64_t flags = in_dtype == KDA_F32 ? 0 : (B * H * (cols / 16) * 4 + 1023) / 1024 * 1024;
  return static_cast<size_t>(B * H * units * bytes + flags);
}

}  // extern "C"

namespace {

enum : unsigned { kPrep = 1u, kPass = 2u };

struct ChunkPtrs {
  const void *q, *k, *v, *g, *beta;
  const float* S0;
  const void* o;
  const float* S_T;
  const void* ws;
  size_t ws_bytes;
  const float* snaps = nullptr;  // state snapshots (pass stage), or NULL
  int64_t snap_every = 0;
  bool builtin_ws = false;       // the library's own scratch: no workspace checks
};

// The argument rules of include/kda.h for the tensors a stage touches:
// kPrep reads q, k, g, beta and writes the workspace; kPass reads v, S0 and
// the workspace and writes o and S_T.
kda_status check_chunk(const ChunkPtrs& p, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                       int in_dtype, int out_dtype, unsigned stages) {
  if (B < 0 || T < 0 || H < 0 || dk < 0 || dv < 0) return KDA_ERR_SHAPE;
  if (B > kMaxElems || T > kMaxElems || H > kMaxElems) return KDA_ERR_SHAPE;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_UNSUPPORTED;
  if (dk != 64 && dk != 128) return KDA_ERR_UNSUPPORTED;
  if (dv < 16 || dv > 512 || dv % 16 != 0) return KDA_ERR_UNSUPPORTED;
  const double toks = static_cast<double>(B) * T * H;
  if (toks * (dk > dv ? dk : dv) > static_cast<double>(kMaxElems)) return KDA_ERR_SHAPE;
  // B * H first, in double: with T = 0 the token bound above admits any B, H
  if (static_cast<double>(B) * H > static_cast<double>(0x0fffffffLL)) return KDA_ERR_UNSUPPORTED;
  const int64_t NC = (T + 15) / 16;
  if (B * H * NC > 0x7fffffffLL) return KDA_ERR_UNSUPPORTED;
  if (H * dv > (int64_t(1) << 25)) return KDA_ERR_UNSUPPORTED;  // 32-bit per-lane offsets
  const int64_t BH = B * H, BTH = B * T * H;
  if (BH == 0) return KDA_OK;  // nothing to read or write
  const bool prep = stages & kPrep, pass = stages & kPass;
  if (T > 0 && prep && (!p.q || !p.k || !p.g || !p.beta)) return KDA_ERR_NULL;
  if (T > 0 && pass && (!p.v || !p.o)) return KDA_ERR_NULL;
  const size_t need = kda_chunk_fwd_workspace_size(B, T, H, dk, dv, in_dtype);
  const bool ws_checked = T > 0 && !p.builtin_ws;
  if (ws_checked && (!p.ws || p.ws_bytes < need)) return KDA_ERR_WORKSPACE;
  const int64_t es = dsize(in_dtype), eo = dsize(out_dtype);
  if (prep) {
    const void* vec4[] = {p.q, p.k, p.g};  // read as 4-element vectors
    for (const void* x : vec4)
      if (x && !aligned(x, 4 * es)) return KDA_ERR_ALIGNMENT;
    if (p.beta && !aligned(p.beta, es)) return KDA_ERR_ALIGNMENT;
  }
  if (pass) {
    // v is read and o written as vectors (16-byte units, 8 bytes for bf16 o)
    if ((p.v && !aligned(p.v, 16)) || (p.o && !aligned(p.o, 16))) return KDA_ERR_ALIGNMENT;
    if ((p.S0 && !aligned(p.S0, 4)) || (p.S_T && !aligned(p.S_T, 4))) return KDA_ERR_ALIGNMENT;
  }
  if (ws_checked && !aligned(p.ws, 16)) return KDA_ERR_ALIGNMENT;
  const Range none{0, 0};
  const Range rq = prep ? range_of(p.q, BTH * dk, es) : none;
  const Range rk = prep ? range_of(p.k, BTH * dk, es) : none;
  const Range rg = prep ? range_of(p.g, BTH * dk, es) : none;
  const Range rb = prep ? range_of(p.beta, BTH, es) : none;
  const Range rv = pass ? range_of(p.v, BTH * dv, es) : none;
  const Range rs0 = pass && p.S0 ? range_of(p.S0, BH * dk * dv, 4) : none;
  const Range ro = pass && T > 0 ? range_of(p.o, BTH * dv, eo) : none;
  const Range rst = pass && p.S_T ? range_of(p.S_T, BH * dk * dv, 4) : none;
  const Range rw = ws_checked ? range_of(p.ws, static_cast<int64_t>(need), 1) : none;
  const Range ins[] = {rq, rk, rv, rg, rb, rs0};
  for (const Range& x : ins) {
    if (overlap(ro, x) || overlap(rw, x)) return KDA_ERR_ALIAS;
    if (&x != &ins[5] && overlap(rst, x)) return KDA_ERR_ALIAS;
  }
  if (overlap(ro, rst) || overlap(ro, rw) || overlap(rw, rst)) return KDA_ERR_ALIAS;
  if (overlap(rst, rs0) && p.S_T != p.S0) return KDA_ERR_ALIAS;
  // snapshots: [B, T / every, H, dk, dv] fp32 written by the pass stage
  if (p.snap_every < 0) return KDA_ERR_SHAPE;
  if (p.snap_every % 32 != 0) return KDA_ERR_UNSUPPORTED;  // whole steps of the state pass
  const int64_t nsnap = p.snap_every > 0 ? T / p.snap_every : 0;
  if (pass && nsnap > 0) {
    if (!p.snaps) return KDA_ERR_NULL;
    if (!aligned(p.snaps, 4)) return KDA_ERR_ALIGNMENT;
    const Range rsn = range_of(p.snaps, B * nsnap * H * dk * dv, 4);
    const Range all[] = {rq, rk, rv, rg, rb, rs0, ro, rst, rw};
    for (const Range& x : all)
      if (overlap(rsn, x)) return KDA_ERR_ALIAS;
  }
  return KDA_OK;
}

bool gate_ok(int gate) { return gate == KDA_GATE_LOG_DECAY || gate == KDA_GATE_SIGMOID; }

kda_status launch_status(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// Launch failures to simulate (kda_debug_inject_launch_failures): each call
// that passed its checks and would launch takes one and returns KDA_ERR_HIP
// instead, before any HIP call.
std::atomic<int> g_injected_failures{0};

bool injected_failure() {
  int n = g_injected_failures.load(std::memory_order_relaxed);
  while (n > 0)
    if (g_injected_failures.compare_exchange_weak(n, n - 1, std::memory_order_relaxed)) return true;
  return false;
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd_check(const void* q, const void* k, const void* v, const void* g,
                               const void* beta, const float* S0, const void* o,
                               const float* S_T, int64_t B, int64_t T, int64_t H, int64_t dk,
                               int64_t dv, int in_dtype, int out_dtype, const void* workspace,
                               size_t workspace_bytes) {
  const ChunkPtrs p{q, k, v, g, beta, S0, o, S_T, workspace, workspace_bytes};
  return check_chunk(p, B, T, H, dk, dv, in_dtype, out_dtype, kPrep | kPass);
}

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* S0, void* o, float* S_T, int64_t B,
                         int64_t T, int64_t H, int64_t dk, int64_t dv, int in_dtype, int out_dtype,
                         void* workspace, size_t workspace_bytes, void* stream) {
  const ChunkPtrs p{q, k, v, g, beta, S0, o, S_T, workspace, workspace_bytes};
  const kda_status st = check_chunk(p, B, T, H, dk, dv, in_dtype, out_dtype, kPrep | kPass);
  if (st != KDA_OK) return st;
  if (B * H == 0) return KDA_OK;
  kda::ChunkFwdArgs a{q, k, v, g, beta, S0, o, S_T, B, T, H, dk, dv, in_dtype, out_dtype, workspace};
  if (injected_failure()) return KDA_ERR_HIP;
  return launch_status(kda::launch_chunk_fwd(a, static_cast<hipStream_t>(stream)));
}

kda_status kda_chunk_fwd_ex_check(const void* q, const void* k, const void* v, const void* g,
                                  const void* beta, const float* S0, const void* o,
                                  const float* S_T, int64_t B, int64_t T, int64_t H, int64_t dk,
                                  int64_t dv, int in_dtype, int out_dtype, int gate,
                                  const float* snapshots, int64_t snapshot_every,
                                  const void* workspace, size_t workspace_bytes) {
  if (!gate_ok(gate)) return KDA_ERR_UNSUPPORTED;
  ChunkPtrs p{q, k, v, g, beta, S0, o, S_T, workspace, workspace_bytes};
  p.snaps = snapshots;
  p.snap_every = snapshot_every;
  return check_chunk(p, B, T, H, dk, dv, in_dtype, out_dtype, kPrep | kPass);
}

kda_status kda_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* S0, void* o, float* S_T, int64_t B,
                            int64_t T, int64_t H, int64_t dk, int64_t dv, int in_dtype,
                            int out_dtype, int gate, float* snapshots, int64_t snapshot_every,
                            void* workspace, size_t workspace_bytes, void* stream) {
  const kda_status st =
      kda_chunk_fwd_ex_check(q, k, v, g, beta, S0, o, S_T, B, T, H, dk, dv, in_dtype, out_dtype,
                             gate, snapshots, snapshot_every, workspace, workspace_bytes);
  if (st != KDA_OK) return st;
  if (B * H == 0) return KDA_OK;
  kda::ChunkFwdArgs a{q, k, v, g, beta, S0, o, S_T, B, T, H, dk, dv, in_dtype, out_dtype, workspace};
  a.gate = gate;
  a.snapshots = snapshots;
  a.snapshot_every = snapshot_every;
  if (injected_failure()) return KDA_ERR_HIP;
  return launch_status(kda::launch_chunk_fwd(a, static_cast<hipStream_t>(stream)));
}

kda_status kda_chunk_prep(const void* q, const void* k, const void* g, const void* beta,
                          int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int in_dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
  const ChunkPtrs p{q, k, nullptr, g, beta, nullptr, nullptr, nullptr, workspace, workspace_bytes};
  const kda_status st = check_chunk(p, B, T, H, dk, dv, in_dtype, KDA_F32, kPrep);
  if (st != KDA_OK) return st;
  if (B * H == 0 || T == 0) return KDA_OK;
  kda::ChunkFwdArgs a{q, k, nullptr, g, beta, nullptr, nullptr, nullptr, B, T, H, dk, dv,
                      in_dtype, KDA_F32, workspace};
  if (injected_failure()) return KDA_ERR_HIP;
  return launch_status(kda::launch_chunk_prep(a, static_cast<hipStream_t>(stream)));
}

kda_status kda_chunk_state_pass(const void* v, const void* workspace, size_t workspace_bytes,
                                const float* S0, void* o, float* S_T, int64_t B, int64_t T,
                                int64_t H, int64_t dk, int64_t dv, int in_dtype, int out_dtype,
                                void* stream) {
  const ChunkPtrs p{nullptr, nullptr, v, nullptr, nullptr, S0, o, S_T, workspace, workspace_bytes};
  const kda_status st = check_chunk(p, B, T, H, dk, dv, in_dtype, out_dtype, kPass);
  if (st != KDA_OK) return st;
  if (B * H == 0) return KDA_OK;
  kda::ChunkFwdArgs a{nullptr, nullptr, v, nullptr, nullptr, S0, o, S_T, B, T, H, dk, dv,
                      in_dtype, out_dtype, const_cast<void*>(workspace)};
  if (injected_failure()) return KDA_ERR_HIP;
  return launch_status(kda::launch_chunk_state_pass(a, static_cast<hipStream_t>(stream)));
}

kda_status kda_decode_step_check(const void* q, const void* k, const void* v, const void* g,
                                 const void* beta, const float* S, const void* o, int64_t N,
                                 int64_t H, int64_t dk, int64_t dv, int in_dtype, int out_dtype) {
  if (N < 0 || H < 0 || dk < 0 || dv < 0) return KDA_ERR_SHAPE;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_UNSUPPORTED;
  if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return KDA_ERR_UNSUPPORTED;
  if (N > 0x7fffffffLL || H > 0x7fffffffLL || N * H > 0x7fffffffLL) return KDA_ERR_UNSUPPORTED;
  const int64_t NH = N * H;
  if (NH == 0) return KDA_OK;
  if (!q || !k || !v || !g || !beta || !S || !o) return KDA_ERR_NULL;
  const int64_t es = dsize(in_dtype);
  {
    const void* elem[] = {q, k, v, g, beta};
    for (const void* p : elem)
      if (!aligned(p, es)) return KDA_ERR_ALIGNMENT;
    if (!aligned(S, 16) || !aligned(o, dsize(out_dtype))) return KDA_ERR_ALIGNMENT;
  }
  const Range ro = range_of(o, NH * dv, dsize(out_dtype));
  const Range rs = range_of(S, NH * dk * dv, 4);
  const Range others[] = {range_of(q, NH * dk, es), range_of(k, NH * dk, es),
                          range_of(v, NH * dv, es), range_of(g, NH * dk, es),
                          range_of(beta, NH, es)};
  if (overlap(ro, rs)) return KDA_ERR_ALIAS;
  for (const Range& x : others)
    if (overlap(ro, x) || overlap(rs, x)) return KDA_ERR_ALIAS;
  return KDA_OK;
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* g,
                           const void* beta, float* S, void* o, int64_t N, int64_t H, int64_t dk,
                           int64_t dv, int in_dtype, int out_dtype, void* stream) {
  return kda_decode_step_ex(q, k, v, g, beta, S, o, N, H, dk, dv, in_dtype, out_dtype,
                            KDA_GATE_LOG_DECAY, stream);
}

kda_status kda_decode_step_ex(const void* q, const void* k, const void* v, const void* g,
                              const void* beta, float* S, void* o, int64_t N, int64_t H,
                              int64_t dk, int64_t dv, int in_dtype, int out_dtype, int gate,
                              void* stream) {
  if (!gate_ok(gate)) return KDA_ERR_UNSUPPORTED;
  const kda_status st =
      kda_decode_step_check(q, k, v, g, beta, S, o, N, H, dk, dv, in_dtype, out_dtype);
  if (st != KDA_OK) return st;
  if (N * H == 0) return KDA_OK;
  kda::DecodeArgs a{q, k, v, g, beta, S, o, N, H, dk, dv, in_dtype, out_dtype};
  a.gate = gate;
  if (injected_failure()) return KDA_ERR_HIP;
  return launch_status(kda::launch_decode_step(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Arguments of kda_spec_verify (commit = false) and kda_spec_commit (true).
kda_status check_spec(bool commit, const void* q, const void* k, const void* v, const void* g,
                      const void* beta, const float* S, const void* o, const int32_t* accepted,
                      int64_t N, int64_t T, int64_t H, int64_t dk, int64_t dv, int in_dtype,
                      int out_dtype, int gate) {
  if (N < 0 || T < 0 || H < 0 || dk < 0 || dv < 0) return KDA_ERR_SHAPE;
  if (!dtype_ok(in_dtype) || (!commit && !dtype_ok(out_dtype)) || !gate_ok(gate))
    return KDA_ERR_UNSUPPORTED;
  if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return KDA_ERR_UNSUPPORTED;
  if (N > 0x7fffffffLL || H > 0x7fffffffLL || N * H > 0x7fffffffLL) return KDA_ERR_UNSUPPORTED;
  if (T > kMaxElems || static_cast<double>(N) * H * T * 128 > static_cast<double>(kMaxElems))
    return KDA_ERR_SHAPE;
  const int64_t NH = N * H, NTH = N * T * H;
  if (NH == 0 || T == 0) return KDA_OK;
  if (!k || !v || !g || !beta || !S) return KDA_ERR_NULL;
  if (commit ? !accepted : (!q || !o)) return KDA_ERR_NULL;
  const int64_t es = dsize(in_dtype), eo = dsize(out_dtype);
  const void* elem[] = {commit ? k : q, k, v, g, beta};
  for (const void* p : elem)
    if (!aligned(p, es)) return KDA_ERR_ALIGNMENT;
  if (!aligned(S, 16)) return KDA_ERR_ALIGNMENT;
  if (commit ? !aligned(accepted, 4) : !aligned(o, eo)) return KDA_ERR_ALIGNMENT;
  const Range none{0, 0};
  const Range rs = range_of(S, NH * dk * dv, 4);
  const Range rout = commit ? rs : range_of(o, NTH * dv, eo);  // what the call writes
  const Range ins[] = {commit ? none : range_of(q, NTH * dk, es), range_of(k, NTH * dk, es),
                       range_of(v, NTH * dv, es), range_of(g, NTH * dk, es),
                       range_of(beta, NTH, es), commit ? range_of(accepted, N, 4) : rs};
  for (const Range& x : ins)
    if (overlap(rout, x)) return KDA_ERR_ALIAS;
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_spec_verify_check(const void* q, const void* k, const void* v, const void* g,
                                 const void* beta, const float* S, const void* o, int64_t N,
                                 int64_t T, int64_t H, int64_t dk, int64_t dv, int in_dtype,
                                 int out_dtype, int gate) {
  return check_spec(false, q, k, v, g, beta, S, o, nullptr, N, T, H, dk, dv, in_dtype, out_dtype,
                    gate);
}

kda_status kda_spec_verify(const void* q, const void* k, const void* v, const void* g,
                           const void* beta, const float* S, void* o, int64_t N, int64_t T,
                           int64_t H, int64_t dk, int64_t dv, int in_dtype, int out_dtype,
                           int gate, void* stream) {
  const kda_status st =
      kda_spec_verify_check(q, k, v, g, beta, S, o, N, T, H, dk, dv, in_dtype, out_dtype, gate);
  if (st != KDA_OK) return st;
  if (N * H == 0 || T == 0) return KDA_OK;
  kda::SpecArgs a{q, k, v, g, beta, const_cast<float*>(S), o, nullptr, N, T, H, dk, dv,
                  in_dtype, out_dtype};
  a.gate = gate;
  if (injected_failure()) return KDA_ERR_HIP;
  return launch_status(kda::launch_spec(a, false, static_cast<hipStream_t>(stream)));
}

kda_status kda_spec_commit_check(const void* k, const void* v, const void* g, const void* beta,
                                 const float* S, const int32_t* accepted, int64_t N, int64_t T,
                                 int64_t H, int64_t dk, int64_t dv, int in_dtype, int gate) {
  return check_spec(true, nullptr, k, v, g, beta, S, nullptr, accepted, N, T, H, dk, dv, in_dtype,
                    KDA_F32, gate);
}

kda_status kda_spec_commit(const void* k, const void* v, const void* g, const void* beta,
                           float* S, const int32_t* accepted, int64_t N, int64_t T, int64_t H,
                           int64_t dk, int64_t dv, int in_dtype, int gate, void* stream) {
  const kda_status st =
      kda_spec_commit_check(k, v, g, beta, S, accepted, N, T, H, dk, dv, in_dtype, gate);
  if (st != KDA_OK) return st;
  if (N * H == 0 || T == 0) return KDA_OK;
  kda::SpecArgs a{nullptr, k, v, g, beta, S, nullptr, accepted, N, T, H, dk, dv, in_dtype, KDA_F32};
  a.gate = gate;
  if (injected_failure()) return KDA_ERR_HIP;
  return launch_status(kda::launch_spec(a, true, static_cast<hipStream_t>(stream)));
}


kda_status kda_spec_commit_verify_check(const void* k1, const void* v1, const void* g1,
                                        const void* beta1, const int32_t* accepted, int64_t T1,
                                        const void* q2, const void* k2, const void* v2,
                                        const void* g2, const void* beta2, int64_t T2,
                                        const float* S, const void* o, int64_t N, int64_t H,
                                        int64_t dk, int64_t dv, int in_dtype, int out_dtype,
                                        int gate) {
  // each step's own rules, then those across the two token sets: S is
  // written (after the logged tokens are read) and must not overlap the
  // drafts; o must not overlap the logged tokens or the accepted counts
  kda_status st = check_spec(true, nullptr, k1, v1, g1, beta1, S, nullptr, accepted, N, T1, H, dk,
                             dv, in_dtype, KDA_F32, gate);
  if (st != KDA_OK) return st;
  st = check_spec(false, q2, k2, v2, g2, beta2, S, o, nullptr, N, T2, H, dk, dv, in_dtype,
                  out_dtype, gate);
  if (st != KDA_OK) return st;
  const int64_t NH = N * H;
  if (NH == 0 || T1 == 0 || T2 == 0) return KDA_OK;
  const int64_t es = dsize(in_dtype), eo = dsize(out_dtype);
  const Range rs = range_of(S, NH * dk * dv, 4);
  const Range ro = range_of(o, N * T2 * H * dv, eo);
  const Range drafts[] = {range_of(q2, N * T2 * H * dk, es), range_of(k2, N * T2 * H * dk, es),
                          range_of(v2, N * T2 * H * dv, es), range_of(g2, N * T2 * H * dk, es),
                          range_of(beta2, N * T2 * H, es)};
  for (const Range& x : drafts)
    if (overlap(rs, x)) return KDA_ERR_ALIAS;
  const Range logged[] = {range_of(k1, N * T1 * H * dk, es), range_of(v1, N * T1 * H * dv, es),
                          range_of(g1, N * T1 * H * dk, es), range_of(beta1, N * T1 * H, es),
                          range_of(accepted, N, 4)};
  for (const Range& x : logged)
    if (overlap(ro, x)) return KDA_ERR_ALIAS;
  return KDA_OK;
}

kda_status kda_spec_commit_verify(const void* k1, const void* v1, const void* g1,
                                  const void* beta1, const int32_t* accepted, int64_t T1,
                                  const void* q2, const void* k2, const void* v2,
                                  const void* g2, const void* beta2, int64_t T2, float* S,
                                  void* o, int64_t N, int64_t H, int64_t dk, int64_t dv,
                                  int in_dtype, int out_dtype, int gate, void* stream) {
  const kda_status st =
      kda_spec_commit_verify_check(k1, v1, g1, beta1, accepted, T1, q2, k2, v2, g2, beta2, T2, S,
                                   o, N, H, dk, dv, in_dtype, out_dtype, gate);
  if (st != KDA_OK) return st;
  if (N * H == 0 || (T1 == 0 && T2 == 0)) return KDA_OK;
  kda::SpecArgs a{q2, k2, v2, g2, beta2, S, o, nullptr, N, T2, H, dk, dv, in_dtype, out_dtype};
  a.gate = gate;
  const kda::SpecPrefix pre{k1, v1, g1, beta1, accepted, T1};
  if (injected_failure()) return KDA_ERR_HIP;
  return launch_status(kda::launch_spec_commit_verify(a, pre, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

kda_status check_transition(const void* v, const void* ws, size_t ws_bytes, const float* F,
                            const float* E, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                            int in_dtype) {
  if (B < 0 || T < 0 || H < 0 || dk < 0 || dv < 0) return KDA_ERR_SHAPE;
  if (B > kMaxElems || T > kMaxElems || H > kMaxElems) return KDA_ERR_SHAPE;
  if (!dtype_ok(in_dtype)) return KDA_ERR_UNSUPPORTED;
  if (dk != 64 && dk != 128) return KDA_ERR_UNSUPPORTED;
  if (dv < 16 || dv > 512 || dv % 16 != 0) return KDA_ERR_UNSUPPORTED;
  const double toks = static_cast<double>(B) * T * H;
  if (toks * (dk > dv ? dk : dv) > static_cast<double>(kMaxElems)) return KDA_ERR_SHAPE;
  // B * H first, in double: with T = 0 the token bound above admits any B, H
  if (static_cast<double>(B) * H > static_cast<double>(0x0fffffffLL)) return KDA_ERR_UNSUPPORTED;
  const int64_t NC = (T + 15) / 16;
  if (B * H * NC > 0x7fffffffLL) return KDA_ERR_UNSUPPORTED;
  if (H * (dk > dv ? dk : dv) > (int64_t(1) << 25)) return KDA_ERR_UNSUPPORTED;
  const int64_t BH = B * H;
  if (BH == 0) return KDA_OK;
  if (T > 0 && E && !v) return KDA_ERR_NULL;
  const size_t need = kda_chunk_fwd_workspace_size(B, T, H, dk, dv, in_dtype);
  if (T > 0 && (F || E) && (!ws || ws_bytes < need)) return KDA_ERR_WORKSPACE;
  if (T > 0 && E && !aligned(v, 16)) return KDA_ERR_ALIGNMENT;
  if ((F && !aligned(F, 4)) || (E && !aligned(E, 4))) return KDA_ERR_ALIGNMENT;
  if (T > 0 && (F || E) && !aligned(ws, 16)) return KDA_ERR_ALIGNMENT;
  const Range none{0, 0};
  const Range rv = T > 0 && E ? range_of(v, B * T * H * dv, dsize(in_dtype)) : none;
  const Range rw = T > 0 && (F || E) ? range_of(ws, static_cast<int64_t>(need), 1) : none;
  const Range rf = F ? range_of(F, BH * dk * dk, 4) : none;
  const Range re = E ? range_of(E, BH * dk * dv, 4) : none;
  if (overlap(rf, re) || overlap(rf, rv) || overlap(rf, rw) || overlap(re, rv) || overlap(re, rw))
    return KDA_ERR_ALIAS;
  return KDA_OK;
}

kda_status check_scan(const float* F, const float* E, const float* S0, const float* S, int64_t P,
                      int64_t N, int64_t dk, int64_t dv) {
  if (P < 0 || N < 0 || dk < 0 || dv < 0) return KDA_ERR_SHAPE;
  if (dk != 64 && dk != 128) return KDA_ERR_UNSUPPORTED;
  if (dv < 16 || dv > 512 || dv % 16 != 0) return KDA_ERR_UNSUPPORTED;
  if (N > 0x0fffffffLL || P > 0x0fffffffLL ||
      static_cast<double>(P + 1) * N * dk * (dk > dv ? dk : dv) > static_cast<double>(kMaxElems))
    return KDA_ERR_SHAPE;
  if (N == 0) return KDA_OK;
  if (!S || (P > 0 && (!F || !E))) return KDA_ERR_NULL;
  if (!aligned(S, 4) || (S0 && !aligned(S0, 4)) || (E && !aligned(E, 4))) return KDA_ERR_ALIGNMENT;
  if (F && !aligned(F, 16)) return KDA_ERR_ALIGNMENT;  // read as 4-float vectors
  const Range none{0, 0};
  const Range rs = range_of(S, (P + 1) * N * dk * dv, 4);
  const Range ins[] = {P > 0 ? range_of(F, P * N * dk * dk, 4) : none,
                       P > 0 ? range_of(E, P * N * dk * dv, 4) : none,
                       S0 ? range_of(S0, N * dk * dv, 4) : none};
  for (const Range& x : ins)
    if (overlap(rs, x)) return KDA_ERR_ALIAS;
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_chunk_transition_check(const void* v, const void* workspace, size_t workspace_bytes,
                                      const float* F, const float* E, int64_t B, int64_t T,
                                      int64_t H, int64_t dk, int64_t dv, int in_dtype) {
  return check_transition(v, workspace, workspace_bytes, F, E, B, T, H, dk, dv, in_dtype);
}

kda_status kda_chunk_transition(const void* v, const void* workspace, size_t workspace_bytes,
                                float* F, float* E, int64_t B, int64_t T, int64_t H, int64_t dk,
                                int64_t dv, int in_dtype, void* stream) {
  const kda_status st =
      check_transition(v, workspace, workspace_bytes, F, E, B, T, H, dk, dv, in_dtype);
  if (st != KDA_OK) return st;
  if (B * H == 0 || (!F && !E)) return KDA_OK;
  kda::ChunkFwdArgs a{nullptr, nullptr, v, nullptr, nullptr, nullptr, nullptr, nullptr, B, T, H,
                      dk, dv, in_dtype, KDA_F32, const_cast<void*>(workspace)};
  if (injected_failure()) return KDA_ERR_HIP;
  return launch_status(kda::launch_chunk_transition(a, F, E, static_cast<hipStream_t>(stream)));
}

kda_status kda_state_affine_scan_check(const float* F, const float* E, const float* S0,
                                       const float* S, int64_t P, int64_t N, int64_t dk,
                                       int64_t dv) {
  return check_scan(F, E, S0, S, P, N, dk, dv);
}

kda_status kda_state_affine_scan(const float* F, const float* E, const float* S0, float* S,
                                 int64_t P, int64_t N, int64_t dk, int64_t dv, void* stream) {
  const kda_status st = check_scan(F, E, S0, S, P, N, dk, dv);
  if (st != KDA_OK) return st;
  if (N == 0) return KDA_OK;
  if (injected_failure()) return KDA_ERR_HIP;
  return launch_status(
      kda::launch_affine_scan(F, E, S0, S, P, N, dk, dv, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

static_assert(KDA_NOALLOC_SCRATCH_BYTES == kda::kNoAllocScratchBytes,
              "header and library disagree on the built-in scratch size");

extern "C" {

kda_status kda_chunk_fwd_noalloc_check(const void* q, const void* k, const void* v,
                                       const void* g, const void* beta, const float* S0,
                                       const void* o, const float* S_T, int64_t B, int64_t T,
                                       int64_t H, int64_t dk, int64_t dv, int in_dtype,
                                       int out_dtype) {
  // the arguments as for kda_chunk_fwd; the workspace is the library's own
  ChunkPtrs p{q, k, v, g, beta, S0, o, S_T, nullptr, 0};
  p.builtin_ws = true;
  const kda_status st = check_chunk(p, B, T, H, dk, dv, in_dtype, out_dtype, kPrep | kPass);
  if (st != KDA_OK) return st;
  if (kda_chunk_fwd_workspace_size(B, T, H, dk, dv, in_dtype) > KDA_NOALLOC_SCRATCH_BYTES)
    return KDA_ERR_TOO_LARGE;
  return KDA_OK;
}

kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g,
                                 const void* beta, const float* S0, void* o, float* S_T,
                                 int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                 int in_dtype, int out_dtype, void* stream) {
  const kda_status st = kda_chunk_fwd_noalloc_check(q, k, v, g, beta, S0, o, S_T, B, T, H, dk, dv,
                                                    in_dtype, out_dtype);
  if (st != KDA_OK) return st;
  if (B * H == 0) return KDA_OK;
  if (injected_failure()) return KDA_ERR_HIP;
  void* ws = nullptr;
  if (kda::noalloc_scratch(&ws) != hipSuccess) return KDA_ERR_HIP;
  kda::ChunkFwdArgs a{q, k, v, g, beta, S0, o, S_T, B, T, H, dk, dv, in_dtype, out_dtype, ws};
  return launch_status(kda::launch_chunk_fwd(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

extern "C" {

void kda_debug_inject_launch_failures(int count) {
  g_injected_failures.store(count > 0 ? count : 0, std::memory_order_relaxed);
}

}  // extern "C"
