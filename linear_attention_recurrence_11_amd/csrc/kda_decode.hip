// One KDA decode step on gfx950: a single token for each of N requests.
//
// Per (request, head) with fp32 state S (dk x dv), in place:
//   S' = Diag(e^g) S;  r = S'^T k;  p = S'^T q;  u = beta (v - r);
//   S  = S' + k u^T;   o = S^T q = p + (q . k) u
// The step is the T = 1 case of the recurrence: the fixed-size state is read
// and overwritten for every token ("177: Kimi K3 in Detail", sections 10 and
// 17: decoding re-reads the whole recurrent state per token). Memory-bound:
// each state is streamed from HBM once and written back once, held in
// registers in between.
//
// Workgroups of 1024 threads, each taking (request, head) units in turn
// (unit = blockIdx.x + k * gridDim.x). Thread t owns the float4 column group
// cg = t % (dv/4) of rows rg + RG*j (RG = 1024/(dv/4)), so one load
// instruction of a wavefront covers whole 512-byte rows (coalesced). At d =
// 128 a thread holds four rows' float4: the 64 KiB state streams through
// sixteen wavefronts at once, and the next unit's state is loaded while the
// current one is reduced, updated and written back, together with that
// unit's token inputs. Measured on 256 requests x 32 heads: 181.6 us per
// step; 194 us with the inputs loaded after the next state's prefetch (their
// use then waited for it), 188.6 us with one workgroup per unit and no
// prefetch, 195 us with 128-, 256- or 512-thread workgroups.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kDecThreads = 1024;
constexpr int64_t kDecGrid = 1024;  // workgroups in flight over the units

template <typename InT, typename OutT, int DK, int DV, int GATE>
__global__ __launch_bounds__(kDecThreads) void kda_decode_kernel(const InT* __restrict__ q,
                                                                 const InT* __restrict__ k,
                                                                 const InT* __restrict__ v,
                                                                 const InT* __restrict__ g,
                                                                 const InT* __restrict__ beta,
                                                                 float* __restrict__ S,
                                                                 OutT* __restrict__ o, int64_t units) {
  constexpr int CPR = DV / 4;                   // threads per row
  constexpr int RG = kDecThreads / CPR;         // row groups
  constexpr int RPT = DK / RG;                  // rows per thread
  static_assert(RPT >= 1 && DK % RG == 0, "shape");
  __shared__ float s_q[DK], s_k[DK], s_e[DK];
  __shared__ float s_red[2][RG][DV + 4];
  __shared__ float s_u[DV];
  __shared__ float s_qk;

  const int t = threadIdx.x;
  const int cg = t % CPR, rg = t / CPR;
  const int64_t stride = gridDim.x;
  // The states are touched once per step and far exceed the caches:
  // non-temporal loads and stores keep them from displacing the per-token
  // inputs (measured: 201 us per step without either hint, 195 with one).
  auto load_state = [&](int64_t u, f32x4 (&x)[RPT]) __attribute__((always_inline)) {
    const float* Su = S + static_cast<size_t>(u) * DK * DV;
#pragma unroll
    for (int j = 0; j < RPT; ++j)
      x[j] = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(Su + static_cast<size_t>(rg + RG * j) * DV + 4 * cg));
  };
  // The token inputs travel with the state: each unit's q, k, g (thread t <
  // dk holds channel t) and v, beta (thread t < dv holds column t) are loaded
  // one unit ahead, beside its state, and kept as loaded (bf16 bits) until
  // used. Loads complete in order, so an input load issued after the next
  // state's prefetch would make its first use wait for that whole prefetch.
  static_assert(DK <= kDecThreads && DV <= kDecThreads, "one input element per thread");
  InT nq{}, nk{}, ng{}, nv{}, nb{};
  auto load_inputs = [&](int64_t u) __attribute__((always_inline)) {
    if (t < DK) {
      nq = q[u * DK + t];
      nk = k[u * DK + t];
      ng = g[u * DK + t];
    }
    if (t < DV) {
      nv = v[u * DV + t];
      nb = beta[u];
    }
  };
  f32x4 next[RPT];
  int64_t unit = blockIdx.x;  // the grid never exceeds the unit count
  load_state(unit, next);
  load_inputs(unit);
  for (; unit < units; unit += stride) {  // uniform per workgroup
    float* Su = S + static_cast<size_t>(unit) * DK * DV;
    float4 s[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) s[j] = make_float4(next[j][0], next[j][1], next[j][2], next[j][3]);
    const InT cq = nq, ck = nk, cgt = ng, cv = nv, cb = nb;
    if (unit + stride < units) {
      load_state(unit + stride, next);
      load_inputs(unit + stride);
    }

    __syncthreads();  // the previous unit's readers of s_q, s_k, s_e, s_u are done
    if (t < DK) {
      s_q[t] = to_f32(cq);
      s_k[t] = to_f32(ck);
      s_e[t] = expf(gate_decay<GATE>(to_f32(cgt)));
    }
    __syncthreads();
    if (t < 64) {  // q . k by one wavefront
      float acc = 0.f;
      for (int i = t; i < DK; i += 64) acc += s_q[i] * s_k[i];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
      if (t == 0) s_qk = acc;
    }

    // S' = Diag(e) S ; partial r and p over this thread's rows
    float r4[4] = {0.f, 0.f, 0.f, 0.f}, p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int row = rg + RG * j;
      const float e = s_e[row], kr = s_k[row], qr = s_q[row];
      s[j].x *= e; s[j].y *= e; s[j].z *= e; s[j].w *= e;
      r4[0] += kr * s[j].x; r4[1] += kr * s[j].y; r4[2] += kr * s[j].z; r4[3] += kr * s[j].w;
      p4[0] += qr * s[j].x; p4[1] += qr * s[j].y; p4[2] += qr * s[j].z; p4[3] += qr * s[j].w;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      s_red[0][rg][4 * cg + c] = r4[c];
      s_red[1][rg][4 * cg + c] = p4[c];
    }
    __syncthreads();
    if (t < DV) {
      float r = 0.f, p = 0.f;
#pragma unroll
      for (int x = 0; x < RG; ++x) {
        r += s_red[0][x][t];
        p += s_red[1][x][t];
      }
      const float u = to_f32(cb) * (to_f32(cv) - r);
      s_u[t] = u;
      store_out(o, unit * DV + t, p + s_qk * u);
    }
    __syncthreads();

    // S = S' + k u^T, written back
    const float u0 = s_u[4 * cg], u1 = s_u[4 * cg + 1], u2 = s_u[4 * cg + 2], u3 = s_u[4 * cg + 3];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int row = rg + RG * j;
      const float kr = s_k[row];
      const f32x4 x = {s[j].x + kr * u0, s[j].y + kr * u1, s[j].z + kr * u2, s[j].w + kr * u3};
      __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(Su + static_cast<size_t>(row) * DV + 4 * cg));
    }
  }
}

template <typename InT, typename OutT, int DK, int DV, int GATE>
hipError_t launch5(const DecodeArgs& a, hipStream_t stream) {
  const int64_t units = a.N * a.H;
  const int64_t grid = units < kDecGrid ? units : kDecGrid;
  hipLaunchKernelGGL((kda_decode_kernel<InT, OutT, DK, DV, GATE>), dim3(static_cast<uint32_t>(grid)),
                     dim3(kDecThreads), 0, stream, static_cast<const InT*>(a.q),
                     static_cast<const InT*>(a.k), static_cast<const InT*>(a.v),
                     static_cast<const InT*>(a.g), static_cast<const InT*>(a.beta), a.S,
                     static_cast<OutT*>(a.o), units);
  return hipGetLastError();
}

template <typename InT, typename OutT, int DK, int DV>
hipError_t launch4(const DecodeArgs& a, hipStream_t s) {
  return a.gate == kGateSigmoid ? launch5<InT, OutT, DK, DV, kGateSigmoid>(a, s)
                                : launch5<InT, OutT, DK, DV, kGateLogDecay>(a, s);
}

template <typename InT, typename OutT>
hipError_t launch2(const DecodeArgs& a, hipStream_t s) {
  if (a.dk == 64) return a.dv == 64 ? launch4<InT, OutT, 64, 64>(a, s) : launch4<InT, OutT, 64, 128>(a, s);
  return a.dv == 64 ? launch4<InT, OutT, 128, 64>(a, s) : launch4<InT, OutT, 128, 128>(a, s);
}

}  // namespace

hipError_t launch_decode_step(const DecodeArgs& a, hipStream_t stream) {
  if (a.N * a.H == 0) return hipSuccess;
  const bool in32 = a.in_dtype == 0, out32 = a.out_dtype == 0;
  if (in32) return out32 ? launch2<float, float>(a, stream) : launch2<float, uint16_t>(a, stream);
  return out32 ? launch2<uint16_t, float>(a, stream) : launch2<uint16_t, uint16_t>(a, stream);
}

}  // namespace kda
