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
// across all tokens. The inputs of up to kTokBlock tokens are staged in LDS
// at once (commit loads a unit's first block one unit ahead, beside that
// unit's state), so no token waits on a global load of its own. Per token two
// barriers: partial reductions written, u published.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

// Threads per workgroup. Verify reads the state once and synchronises every
// token, which favours small workgroups; commit also writes the state back,
// which favours more wavefronts streaming it (measured on 256 requests x 32
// heads x 4 drafts, with three barriers per token: verify 141 us at 256
// threads, 288 us at 1024; commit 231 us at 256, 207 us at 1024, 200 us with
// the persistent grid and its prefetch. Verify on that persistent grid, with
// the current two barriers: 101 us for one draft against 130, but 212 us for
// four against 168, its per-token reductions over 32 row groups no longer
// hidden by other resident workgroups).
template <bool COMMIT>
constexpr int spec_threads() {
  return COMMIT ? 1024 : 256;
}
constexpr int64_t kCommitGrid = 1024;
constexpr int kTokBlock = 8;  // tokens whose inputs are staged in LDS at once

// Wavefronts per SIMD the register allocation must leave room for: verify
// relies on several resident workgroups hiding each other's latency.
template <bool COMMIT>
constexpr int spec_waves_per_simd() {
  return COMMIT ? 1 : 4;
}

template <typename InT, typename OutT, int DK, int DV, int GATE, bool COMMIT>
__global__ __launch_bounds__(spec_threads<COMMIT>()) __attribute__((amdgpu_waves_per_eu(spec_waves_per_simd<COMMIT>())))
void kda_spec_kernel(const InT* __restrict__ q,
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
  constexpr int TB = kTokBlock, NW = NT / 64;
  __shared__ float s_q[COMMIT ? 1 : TB][DK], s_k[TB][DK], s_e[TB][DK], s_v[TB][DV];
  __shared__ float s_b[TB], s_qk[TB];
  __shared__ float s_red[COMMIT ? 1 : 2][RG][DV + 4];
  __shared__ float s_u[DV];

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
  // Commit: a block's token inputs as loaded (bf16 bits or floats): element
  // e of this thread is i = t + e * NT of the block's nb x dk (k, g) and
  // nb x dv (v) elements, and b is beta of token t (t < nb). Loads complete
  // in order, so the next unit's first block is loaded right after that
  // unit's state prefetch: loaded after the prefetch, the current unit's
  // inputs would make their first use wait for it. (Verify has no prefetch;
  // it stages straight from global memory, with few loads in flight, which
  // keeps it within its register budget.)
  constexpr int EK = (TB * DK + NT - 1) / NT, EV = (TB * DV + NT - 1) / NT;
  struct InBlock {
    InT q[COMMIT ? 1 : EK], k[EK], g[EK], v[EV], b;
  };
  auto stage_direct = [&](size_t tok0, int nb) __attribute__((always_inline)) {
    for (int i = t; i < nb * DK; i += NT) {
      const int j = i / DK, c = i % DK;
      const size_t x = (tok0 + static_cast<size_t>(j) * H) * DK + c;
      if constexpr (!COMMIT) s_q[j][c] = load_in(q, x);
      s_k[j][c] = load_in(k, x);
      s_e[j][c] = expf(gate_decay<GATE>(load_in(g, x)));
    }
    for (int i = t; i < nb * DV; i += NT) {
      const int j = i / DV, c = i % DV;
      s_v[j][c] = load_in(v, (tok0 + static_cast<size_t>(j) * H) * DV + c);
    }
    if (t < nb) s_b[t] = load_in(beta, tok0 + static_cast<size_t>(t) * H);
  };
  auto load_block = [&](InBlock& x, int64_t u, int64_t t0, int nb) __attribute__((always_inline)) {
    const int64_t n = u / H, h = u % H;
    const size_t tok0 = static_cast<size_t>((n * T + t0) * H + h);  // token j: tok0 + j * H
#pragma unroll
    for (int e = 0; e < EK; ++e) {
      const int i = t + e * NT;
      if (i < nb * DK) {
        const size_t idx = (tok0 + static_cast<size_t>(i / DK) * H) * DK + i % DK;
        if constexpr (!COMMIT) x.q[e] = q[idx];
        x.k[e] = k[idx];
        x.g[e] = g[idx];
      }
    }
#pragma unroll
    for (int e = 0; e < EV; ++e) {
      const int i = t + e * NT;
      if (i < nb * DV) x.v[e] = v[(tok0 + static_cast<size_t>(i / DV) * H) * DV + i % DV];
    }
    if (t < nb) x.b = beta[tok0 + static_cast<size_t>(t) * H];
  };
  auto stage_block = [&](const InBlock& x, int nb) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < EK; ++e) {
      const int i = t + e * NT;
      if (i < nb * DK) {
        const int j = i / DK, c = i % DK;
        if constexpr (!COMMIT) s_q[j][c] = to_f32(x.q[e]);
        s_k[j][c] = to_f32(x.k[e]);
        s_e[j][c] = expf(gate_decay<GATE>(to_f32(x.g[e])));
      }
    }
#pragma unroll
    for (int e = 0; e < EV; ++e) {
      const int i = t + e * NT;
      if (i < nb * DV) s_v[i / DV][i % DV] = to_f32(x.v[e]);
    }
    if (t < nb) s_b[t] = to_f32(x.b);
  };
  const int nb0 = static_cast<int>(T < TB ? T : TB);  // tokens of a first block, loaded ahead
  f32x4 next[RPT];
  InBlock ahead{};
  int64_t unit = blockIdx.x;  // the grid never exceeds the unit count
  if constexpr (COMMIT) {
    load_state(unit, next);
    load_block(ahead, unit, 0, nb0);
  }
  for (; unit < units; unit += stride) {  // uniform per workgroup
    const int64_t n = unit / H, h = unit % H;
    float* Su = S + static_cast<size_t>(unit) * DK * DV;
    if constexpr (!COMMIT) load_state(unit, next);
    float4 s[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) s[j] = make_float4(next[j][0], next[j][1], next[j][2], next[j][3]);
    const InBlock first = ahead;
    if constexpr (COMMIT) {
      if (unit + stride < units) {
        load_state(unit + stride, next);
        load_block(ahead, unit + stride, 0, nb0);
      }
    }

    int64_t ntok = T;
    if constexpr (COMMIT) {
      const int64_t a = accepted[n];
      ntok = a < 0 ? 0 : (a > T ? T : a);
    }
    for (int64_t t0 = 0; t0 < ntok; t0 += TB) {
      const int nb = static_cast<int>(ntok - t0 < TB ? ntok - t0 : TB);
      const size_t tok0 = static_cast<size_t>((n * T + t0) * H + h);  // token j: tok0 + j * H
      __syncthreads();  // the readers of the previous block (or unit) are done
      if constexpr (COMMIT) {
        if (t0 == 0) {
          stage_block(first, nb);
        } else {
          InBlock x;
          load_block(x, unit, t0, nb);
          stage_block(x, nb);
        }
      } else {
        stage_direct(tok0, nb);
      }
      __syncthreads();
      if constexpr (!COMMIT) {
        // q_t . k_t of each token, one wavefront per token; read after the
        // token's first barrier
        const int w = t >> 6, l = t & 63;
        for (int j = w; j < nb; j += NW) {
          float acc = 0.f;
          for (int c = l; c < DK; c += 64) acc += s_q[j][c] * s_k[j][c];
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
          if (l == 0) s_qk[j] = acc;
        }
      }
      for (int j = 0; j < nb; ++j) {
        float r4[4] = {0.f, 0.f, 0.f, 0.f}, p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < RPT; ++jj) {
          const int row = rg + RG * jj;
          const float e = s_e[j][row], kr = s_k[j][row];
          s[jj].x *= e; s[jj].y *= e; s[jj].z *= e; s[jj].w *= e;
          r4[0] += kr * s[jj].x; r4[1] += kr * s[jj].y; r4[2] += kr * s[jj].z; r4[3] += kr * s[jj].w;
          if constexpr (!COMMIT) {
            const float qr = s_q[j][row];
            p4[0] += qr * s[jj].x; p4[1] += qr * s[jj].y; p4[2] += qr * s[jj].z; p4[3] += qr * s[jj].w;
          }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          s_red[0][rg][4 * cg + c] = r4[c];
          if constexpr (!COMMIT) s_red[COMMIT ? 0 : 1][rg][4 * cg + c] = p4[c];
        }
        __syncthreads();
        if (t < DV) {
          float r = 0.f, p = 0.f;
#pragma unroll
          for (int x = 0; x < RG; ++x) {
            r += s_red[0][x][t];
            if constexpr (!COMMIT) p += s_red[COMMIT ? 0 : 1][x][t];
          }
          const float u = s_b[j] * (s_v[j][t] - r);
          s_u[t] = u;
          if constexpr (!COMMIT)
            store_out(o, (tok0 + static_cast<size_t>(j) * H) * DV + t, p + s_qk[j] * u);
        }
        __syncthreads();
        const float u0 = s_u[4 * cg], u1 = s_u[4 * cg + 1], u2 = s_u[4 * cg + 2], u3 = s_u[4 * cg + 3];
#pragma unroll
        for (int jj = 0; jj < RPT; ++jj) {
          const float kr = s_k[j][rg + RG * jj];
          s[jj].x += kr * u0; s[jj].y += kr * u1; s[jj].z += kr * u2; s[jj].w += kr * u3;
        }
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
