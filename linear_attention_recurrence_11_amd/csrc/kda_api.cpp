// C-ABI host layer of libkda.so: argument checks, workspace sizing, dispatch
// to the HIP launchers. See include/kda.h for the contract.
#include "kda.h"

#include <hip/hip_runtime.h>

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
    default: return "unknown status";
  }
}

size_t kda_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                    int in_dtype) {
  if (B < 0 || T < 0 || H < 0 || (dk != 64 && dk != 128) || !dtype_ok(in_dtype)) return 0;
  if (dv < 16 || dv > 512 || dv % 16 != 0) return 0;
  if (B > kMaxElems || T > kMaxElems || H > kMaxElems) return 0;
  const int64_t NC = (T + 15) / 16;
  const kda::RecordLayout L = kda::record_layout(dk, in_dtype == KDA_F32);
  const double total = static_cast<double>(B) * H * NC * L.bytes;
  if (total > 9.0e18) return 0;
  return static_cast<size_t>(B * H * NC * L.bytes);
}

kda_status kda_chunk_fwd_check(const void* q, const void* k, const void* v, const void* g,
                               const void* beta, const float* S0, const void* o,
                               const float* S_T, int64_t B, int64_t T, int64_t H, int64_t dk,
                               int64_t dv, int in_dtype, int out_dtype, const void* workspace,
                               size_t workspace_bytes) {
  if (B < 0 || T < 0 || H < 0 || dk < 0 || dv < 0) return KDA_ERR_SHAPE;
  if (B > kMaxElems || T > kMaxElems || H > kMaxElems) return KDA_ERR_SHAPE;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_UNSUPPORTED;
  if (dk != 64 && dk != 128) return KDA_ERR_UNSUPPORTED;
  if (dv < 16 || dv > 512 || dv % 16 != 0) return KDA_ERR_UNSUPPORTED;
  const double toks = static_cast<double>(B) * T * H;
  if (toks * (dk > dv ? dk : dv) > static_cast<double>(kMaxElems)) return KDA_ERR_SHAPE;
  const int64_t NC = (T + 15) / 16;
  if (B * H * NC > 0x7fffffffLL || B * H > 0x0fffffffLL) return KDA_ERR_UNSUPPORTED;
  const int64_t BH = B * H, BTH = B * T * H;
  if (BH == 0) return KDA_OK;  // nothing to read or write
  if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_NULL;
  const size_t need = kda_chunk_fwd_workspace_size(B, T, H, dk, dv, in_dtype);
  if (T > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
  const int64_t es = dsize(in_dtype);
  {
    const void* vec4[] = {q, k, g};  // read as 4-element vectors
    for (const void* p : vec4)
      if (p && !aligned(p, 4 * es)) return KDA_ERR_ALIGNMENT;
    const void* elem[] = {v, beta};
    for (const void* p : elem)
      if (p && !aligned(p, es)) return KDA_ERR_ALIGNMENT;
    if ((o && !aligned(o, dsize(out_dtype))) || (S0 && !aligned(S0, 4)) || (S_T && !aligned(S_T, 4)))
      return KDA_ERR_ALIGNMENT;
    if (T > 0 && workspace && !aligned(workspace, 16)) return KDA_ERR_ALIGNMENT;
  }
  const Range rq = range_of(q, BTH * dk, es), rk = range_of(k, BTH * dk, es);
  const Range rv = range_of(v, BTH * dv, es), rg = range_of(g, BTH * dk, es);
  const Range rb = range_of(beta, BTH, es);
  const Range rs0 = range_of(S0, S0 ? BH * dk * dv : 0, 4);
  const Range ro = range_of(o, BTH * dv, dsize(out_dtype));
  const Range rst = range_of(S_T, S_T ? BH * dk * dv : 0, 4);
  const Range rw = range_of(workspace, T > 0 && workspace ? static_cast<int64_t>(need) : 0, 1);
  const Range inputs[] = {rq, rk, rv, rg, rb};
  for (const Range& x : inputs) {
    if (T > 0 && overlap(ro, x)) return KDA_ERR_ALIAS;
    if (overlap(rst, x) || overlap(rw, x)) return KDA_ERR_ALIAS;
  }
  if (T > 0 && (overlap(ro, rs0) || overlap(ro, rst) || overlap(ro, rw))) return KDA_ERR_ALIAS;
  if (overlap(rw, rs0) || overlap(rw, rst)) return KDA_ERR_ALIAS;
  if (overlap(rst, rs0) && S_T != S0) return KDA_ERR_ALIAS;
  return KDA_OK;
}

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* S0, void* o, float* S_T, int64_t B,
                         int64_t T, int64_t H, int64_t dk, int64_t dv, int in_dtype, int out_dtype,
                         void* workspace, size_t workspace_bytes, void* stream) {
  const kda_status st = kda_chunk_fwd_check(q, k, v, g, beta, S0, o, S_T, B, T, H, dk, dv,
                                            in_dtype, out_dtype, workspace, workspace_bytes);
  if (st != KDA_OK) return st;
  if (B * H == 0) return KDA_OK;
  kda::ChunkFwdArgs a{q, k, v, g, beta, S0, o, S_T, B, T, H, dk, dv, in_dtype, out_dtype, workspace};
  const hipError_t e = kda::launch_chunk_fwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
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
  const kda_status st =
      kda_decode_step_check(q, k, v, g, beta, S, o, N, H, dk, dv, in_dtype, out_dtype);
  if (st != KDA_OK) return st;
  if (N * H == 0) return KDA_OK;
  kda::DecodeArgs a{q, k, v, g, beta, S, o, N, H, dk, dv, in_dtype, out_dtype};
  const hipError_t e = kda::launch_decode_step(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
