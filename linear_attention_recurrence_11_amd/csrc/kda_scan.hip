// Affine scan of span transitions on gfx950: the step that joins the spans
// of a sequence split for context-parallel prefill.
//
// The recurrence is affine in the state, so a span of tokens maps its
// entering state S_in to S_out = F S_in + E, with F (dk x dk) its state
// transition and E (dk x dv) the state it reaches from zero. A sequence cut
// into spans r = 0 .. P-1, each prepared, passed and transitioned without
// knowing its entering state, gets every entering state from
//   S[0] = S0,  S[r + 1] = F[r] S[r] + E[r],
// after which each span reruns its state pass from S[r] (KDA context
// parallelism across devices: "K3 tech report" podcast transcript, the
// exchange on recreating the training efficiency; "Kimi K3 goes
// trillion-scale with sparse MoE efficiency" subtitles, cue 22).
//
// One wavefront per (unit n, 16-column slice of dv) keeps its dk x 16 slice
// of S in registers across the P spans, in the matrix-core output layout, and
// forms F[r] S as fp32 16x16x4 matrix-core products with fp32 accumulation
// (dk/16 x dk/4 products per span). Contraction slot gq of the k-step
// (m', i) is channel 16m' + 4gq + i, so each lane's own state values are the
// B operand and F is read as four consecutive floats per lane and row.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

template <int DK>
__global__ __launch_bounds__(64) void kda_affine_scan(const float* __restrict__ F,
                                                      const float* __restrict__ E,
                                                      const float* __restrict__ S0,
                                                      float* __restrict__ S, int64_t P, int64_t N,
                                                      int64_t DV) {
  constexpr int NM = DK / 16;
  const int l = threadIdx.x, c16 = l & 15, gq = l >> 4;
  const int64_t nslices = DV / 16;
  const int64_t n = blockIdx.x / nslices, slice = blockIdx.x % nslices;
  const int64_t col = slice * 16 + c16;
  const size_t state = static_cast<size_t>(DK) * DV;  // one unit's state
  // st[m][i] = S[16m + 4gq + i][col]
  f32x4 st[NM];
  const size_t lane = static_cast<size_t>(4 * gq) * DV + col;
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      st[m][i] = S0 ? S0[n * state + lane + static_cast<size_t>(16 * m + i) * DV] : 0.f;
  float* out = S + n * state + lane;
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) out[static_cast<size_t>(16 * m + i) * DV] = st[m][i];
  for (int64_t r = 0; r < P; ++r) {
    const float* Fr = F + (static_cast<size_t>(r) * N + n) * DK * DK;
    const float* Er = E + (static_cast<size_t>(r) * N + n) * state + lane;
    f32x4 acc[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][i] = Er[static_cast<size_t>(16 * m + i) * DV];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      // this lane's row of F for output rows 16m + c16, channels 16m' + 4gq + i
      const float* row = Fr + static_cast<size_t>(16 * m + c16) * DK + 4 * gq;
#pragma unroll
      for (int mk = 0; mk < NM; ++mk) {
        const float4 a = *reinterpret_cast<const float4*>(row + 16 * mk);
        acc[m] = mma_16x16x4_f32(a.x, st[mk][0], acc[m]);
        acc[m] = mma_16x16x4_f32(a.y, st[mk][1], acc[m]);
        acc[m] = mma_16x16x4_f32(a.z, st[mk][2], acc[m]);
        acc[m] = mma_16x16x4_f32(a.w, st[mk][3], acc[m]);
      }
    }
    out += static_cast<size_t>(N) * state;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      st[m] = acc[m];
#pragma unroll
      for (int i = 0; i < 4; ++i) out[static_cast<size_t>(16 * m + i) * DV] = st[m][i];
    }
  }
}

}  // namespace

hipError_t launch_affine_scan(const float* F, const float* E, const float* S0, float* S,
                              int64_t P, int64_t N, int64_t dk, int64_t dv, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int64_t blocks = N * (dv / 16);
  if (dk == 64)
    hipLaunchKernelGGL(kda_affine_scan<64>, dim3(static_cast<uint32_t>(blocks)), dim3(64), 0,
                       stream, F, E, S0, S, P, N, dv);
  else
    hipLaunchKernelGGL(kda_affine_scan<128>, dim3(static_cast<uint32_t>(blocks)), dim3(64), 0,
                       stream, F, E, S0, S, P, N, dv);
  return hipGetLastError();
}

}  // namespace kda
