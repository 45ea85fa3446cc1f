// Speculative-decoding verification and commit for KDA on gfx950.
//
// The state is rewritten in place by every token, so rolling back after a
// rejected draft cannot drop tokens the way a KV cache can. Instead the state
// at the last accepted position is kept as the checkpoint, the per-token
// inputs (k, v, g, beta: about 1 KiB per head and token at d = 128) are
// logged, and the accepted prefix is replayed from the checkpoint
// ("177: Kimi K3 in Detail", section 23: record the moves and replay them
// instead of snapshotting the board every step; "Kimi K3 goes trillion-scale
// with sparse MoE efficiency" subtitles, cue 28). Two entry points:
//
//   verify  o_t for the T draft tokens of each request, starting from the
//           checkpoint S, which is only read (T decode steps in one pass).
//   commit  S advanced in place over the first accepted[n] of those tokens
//           (the replay; q and o play no part).
//
// Per token the step is the decode step's (decay rows, erase against the
// decayed state, write, read after the write). A verify + commit pair moves
// the 64 KiB fp32 state three times (read, read, write) whatever T is, where
// T single decode steps would move it 2T times.
//
// Verify runs one 256-thread workgroup per (request, head); commit runs up to
// 1024 persistent 1024-thread workgroups that take the units in turn and
// load the next unit's state while replaying the current one (spec_threads,
// kCommitGrid). Thread t owns float4 column group cg = t % (dv/4) of rows
// rg + RG*j, as in the decode step, and keeps its part of S in registers
// across all tokens. Per token three
// barriers: token inputs staged, partial reductions written, u published.
// The token inputs are double-buffered by token parity so that the next
// token's staging cannot overwrite what slower threads still read.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

// Threads per workgroup. Verify reads the state once and has three barriers
// per token, which favour small workgroups; commit also writes the state
// back, which favours more wavefronts streaming it (measured on 256 requests
// x 32 heads x 4 drafts: verify 141 us at 256 threads, 288 us at 1024;
// commit 231 us at 256, 207 us at 1024, 200 us with the persistent grid and
// its prefetch, which lowers verify's occupancy too far to pay there).
template <bool COMMIT>
constexpr int spec_threads() {
  return COMMIT ? 1024 : 256;
}
constexpr int64_t kCommitGrid = 1024;

template <typename InT, typename OutT, int DK, int DV, int GATE, bool COMMIT>
__global__ __launch_bounds__(spec_threads<COMMIT>()) void kda_spec_kernel(const InT* __restrict__ q,
                                                       const InT* __restrict__ k,
                                                       const InT* __restrict__ v,
                                                       const InT* __restrict__ g,
                                                       const InT* __restrict__ beta,
                                                       float* __restrict__ S,
                                                       OutT* __restrict__ o,
                                                       const int32_t* __restrict__ accepted,
                                                       int64_t T, int64_t H, int64_t units) {
  constexpr int CPR = DV / 4;
  constexpr int NT = spec_threads<COMMIT>();
  constexpr int RG = NT / CPR;
  constexpr int RPT = DK / RG;
  static_assert(RPT >= 1 && DK % RG == 0, "shape");
  __shared__ float s_q[2][DK], s_k[2][DK], s_e[2][DK];
  __shared__ float s_red[2][RG][DV + 4];
  __shared__ float s_u[DV];
  __shared__ float s_qk;

  const int t = threadIdx.x;
  const int cg = t % CPR, rg = t / CPR;
  const int64_t stride = gridDim.x;
  // Commit streams each state in and out once: non-temporal accesses, and the
  // next unit's state is loaded while the current one replays its tokens.
  // Verify only reads the state, one unit per workgroup.
  auto load_state = [&](int64_t u, f32x4 (&x)[RPT]) __attribute__((always_inline)) {
    const float* Su = S + static_cast<size_t>(u) * DK * DV;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const f32x4* src = reinterpret_cast<const f32x4*>(Su + static_cast<size_t>(rg + RG * j) * DV + 4 * cg);
      if constexpr (COMMIT)
        x[j] = __builtin_nontemporal_load(src);
      else
        x[j] = *src;
    }
  };
  f32x4 next[RPT];
  int64_t unit = blockIdx.x;  // the grid never exceeds the unit count
  if constexpr (COMMIT) load_state(unit, next);
  for (; unit < units; unit += stride) {  // uniform per workgroup
    const int64_t n = unit / H, h = unit % H;
    float* Su = S + static_cast<size_t>(unit) * DK * DV;
    if constexpr (!COMMIT) load_state(unit, next);
    float4 s[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) s[j] = make_float4(next[j][0], next[j][1], next[j][2], next[j][3]);
    if constexpr (COMMIT) {
      if (unit + stride < units) load_state(unit + stride, next);
    }

    int64_t ntok = T;
    if constexpr (COMMIT) {
      const int64_t a = accepted[n];
      ntok = a < 0 ? 0 : (a > T ? T : a);
    }
    __syncthreads();  // the previous unit's LDS readers are done
    for (int64_t tt = 0; tt < ntok; ++tt) {
      const int pb = static_cast<int>(tt & 1);
      const size_t tok = static_cast<size_t>((n * T + tt) * H + h);
      for (int i = t; i < DK; i += NT) {
        if constexpr (!COMMIT) s_q[pb][i] = load_in(q, tok * DK + i);
        s_k[pb][i] = load_in(k, tok * DK + i);
        s_e[pb][i] = expf(gate_decay<GATE>(load_in(g, tok * DK + i)));
      }
      __syncthreads();
      if constexpr (!COMMIT) {
        if (t < 64) {
          float acc = 0.f;
          for (int i = t; i < DK; i += 64) acc += s_q[pb][i] * s_k[pb][i];
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
          if (t == 0) s_qk = acc;
        }
      }
      float r4[4] = {0.f, 0.f, 0.f, 0.f}, p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const int row = rg + RG * j;
        const float e = s_e[pb][row], kr = s_k[pb][row];
        s[j].x *= e; s[j].y *= e; s[j].z *= e; s[j].w *= e;
        r4[0] += kr * s[j].x; r4[1] += kr * s[j].y; r4[2] += kr * s[j].z; r4[3] += kr * s[j].w;
        if constexpr (!COMMIT) {
          const float qr = s_q[pb][row];
          p4[0] += qr * s[j].x; p4[1] += qr * s[j].y; p4[2] += qr * s[j].z; p4[3] += qr * s[j].w;
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s_red[0][rg][4 * cg + c] = r4[c];
        if constexpr (!COMMIT) s_red[1][rg][4 * cg + c] = p4[c];
      }
      __syncthreads();
      if (t < DV) {
        float r = 0.f, p = 0.f;
#pragma unroll
        for (int x = 0; x < RG; ++x) {
          r += s_red[0][x][t];
          if constexpr (!COMMIT) p += s_red[1][x][t];
        }
        const float u = load_in(beta, tok) * (load_in(v, tok * DV + t) - r);
        s_u[t] = u;
        if constexpr (!COMMIT) store_out(o, tok * DV + t, p + s_qk * u);
      }
      __syncthreads();
      const float u0 = s_u[4 * cg], u1 = s_u[4 * cg + 1], u2 = s_u[4 * cg + 2], u3 = s_u[4 * cg + 3];
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const float kr = s_k[pb][rg + RG * j];
        s[j].x += kr * u0; s[j].y += kr * u1; s[j].z += kr * u2; s[j].w += kr * u3;
      }
    }
    if constexpr (COMMIT) {
      if (ntok > 0) {
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          const f32x4 x = {s[j].x, s[j].y, s[j].z, s[j].w};
          __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(Su + static_cast<size_t>(rg + RG * j) * DV + 4 * cg));
        }
      }
    }
  }
}

template <typename InT, typename OutT, int DK, int DV, int GATE, bool COMMIT>
hipError_t launch_typed(const SpecArgs& a, hipStream_t stream) {
  const int64_t units = a.N * a.H;
  // commit: persistent workgroups over the units; verify: one per unit
  const int64_t grid = COMMIT && units > kCommitGrid ? kCommitGrid : units;
  hipLaunchKernelGGL((kda_spec_kernel<InT, OutT, DK, DV, GATE, COMMIT>),
                     dim3(static_cast<uint32_t>(grid)), dim3(spec_threads<COMMIT>()), 0, stream,
                     static_cast<const InT*>(a.q), static_cast<const InT*>(a.k),
                     static_cast<const InT*>(a.v), static_cast<const InT*>(a.g),
                     static_cast<const InT*>(a.beta), a.S, static_cast<OutT*>(a.o), a.accepted,
                     a.T, a.H, units);
  return hipGetLastError();
}

template <typename InT, typename OutT, int DK, int DV, bool COMMIT>
hipError_t launch_gate(const SpecArgs& a, hipStream_t s) {
  return a.gate == kGateSigmoid ? launch_typed<InT, OutT, DK, DV, kGateSigmoid, COMMIT>(a, s)
                                : launch_typed<InT, OutT, DK, DV, kGateLogDecay, COMMIT>(a, s);
}

template <typename InT, typename OutT, bool COMMIT>
hipError_t launch_shape(const SpecArgs& a, hipStream_t s) {
  if (a.dk == 64)
    return a.dv == 64 ? launch_gate<InT, OutT, 64, 64, COMMIT>(a, s)
                      : launch_gate<InT, OutT, 64, 128, COMMIT>(a, s);
  return a.dv == 64 ? launch_gate<InT, OutT, 128, 64, COMMIT>(a, s)
                    : launch_gate<InT, OutT, 128, 128, COMMIT>(a, s);
}

}  // namespace

hipError_t launch_spec(const SpecArgs& a, bool commit, hipStream_t stream) {
  if (a.N * a.H == 0 || a.T == 0) return hipSuccess;
  const bool in32 = a.in_dtype == 0;
  if (commit)  // no output: the output type is immaterial
    return in32 ? launch_shape<float, float, true>(a, stream)
                : launch_shape<uint16_t, float, true>(a, stream);
  const bool out32 = a.out_dtype == 0;
  if (in32)
    return out32 ? launch_shape<float, float, false>(a, stream)
                 : launch_shape<float, uint16_t, false>(a, stream);
  return out32 ? launch_shape<uint16_t, float, false>(a, stream)
               : launch_shape<uint16_t, uint16_t, false>(a, stream);
}

}  // namespace kda
